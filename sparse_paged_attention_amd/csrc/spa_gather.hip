// Gather-metadata export: the per-query canonical list of physical KV rows,
// produced by the same translation code (spa_device.h) that the attention
// kernel uses to fetch its rows.  The counterpart of the top-k -> paged-offset
// translation step in the ATOM DeepSeek-V4 decode trace ("What this test
// actually drives"), exported so it can be compared bit-for-bit.

#include <hip/hip_runtime.h>

#include <cstdint>

#include "spa_device.h"

namespace spa {
namespace {

__global__ __launch_bounds__(256) void gather_kernel(const Params p, int32_t cap,
                                                     int64_t *__restrict__ rows_out,
                                                     int32_t *__restrict__ counts_out) {
  const int32_t nb = cap > 0 ? (cap + 255) / 256 : 1;
  const int32_t i = blockIdx.x / nb;
  const int32_t eb = blockIdx.x - i * nb;
  const int32_t e = eb * 256 + threadIdx.x;
  const QueryKV kv = query_kv(p, i);
  const int32_t N = kv.n_sel + kv.win_len;
  if (e < cap) {
    int64_t r = -1;
    if (e < N) {
      r = entry_row(p, kv, i, e);
      if (r < 0) r = -2;
    }
    rows_out[(int64_t)i * cap + e] = r;
  }
  if (eb == 0 && threadIdx.x == 0) {
    int32_t *c = counts_out + (int64_t)i * 4;
    c[0] = kv.win_lo;
    c[1] = kv.win_len;
    c[2] = kv.n_c;
    c[3] = kv.n_sel;
  }
}

}  // namespace

hipError_t launch_gather(const Params &p, int32_t cap, int64_t *rows_out, int32_t *counts_out,
                         hipStream_t stream) {
  if (p.num_queries == 0) return hipSuccess;
  const int64_t nb = cap > 0 ? (cap + 255) / 256 : 1;
  const dim3 grid((unsigned)(nb * p.num_queries));
  hipLaunchKernelGGL(gather_kernel, grid, dim3(256), 0, stream, p, cap, rows_out, counts_out);
  return hipGetLastError();
}

}  // namespace spa
