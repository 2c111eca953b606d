// Exact merge of sink-free split partials (O_s, LSE_s) plus the sink.
//
// RL-Kernel PR "[WS2] CP-aware Attention contract and dispatch metadata",
// Summary and Behavior: a deterministic (out, lse) reduction; tessera PR
// "Block AttnRes model": the attn-with-stats / softmax_merge primitive pair.
// For a row r:  M = max(max_s LSE_s, sink),  Z = sum_s e^(LSE_s - M) + e^(sink - M),
// LSE = M + ln Z,  O = sum_s e^(LSE_s - M) O_s / Z.  The sink acts as one more
// part with O = 0.  The order of the sums is fixed (s ascending), so the
// result is bitwise deterministic.
//
// HBM-bound: one wave per row, each lane owns D/64 consecutive floats.

#include <hip/hip_runtime.h>

#include <cstdint>

#include "spa_internal.h"

namespace spa {
namespace {

template <int D>
__global__ __launch_bounds__(256) void merge_kernel(const float *__restrict__ o_parts,
                                                    const float *__restrict__ lse_parts,
                                                    int32_t S, int64_t rows, int32_t hq,
                                                    const float *__restrict__ sink,
                                                    uint16_t *__restrict__ o_out,
                                                    float *__restrict__ lse_out) {
  constexpr int E = D / 64;   // floats per lane
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= rows) return;
  const float sk = sink ? sink[row % hq] : -INFINITY;
  // loads are issued 8 parts at a time so that they are in flight together
  float M = sk;
  for (int s0 = 0; s0 < S; s0 += 8) {
    float ls[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) ls[k] = s0 + k < S ? lse_parts[(int64_t)(s0 + k) * rows + row] : -INFINITY;
#pragma unroll
    for (int k = 0; k < 8; ++k) M = fmaxf(M, ls[k]);
  }
  float o[E];
#pragma unroll
  for (int e = 0; e < E; ++e) o[e] = 0.f;
  float lse = -INFINITY;
  if (M != -INFINITY) {
    float Z = sk == -INFINITY ? 0.f : __expf(sk - M);
    for (int s0 = 0; s0 < S; s0 += 8) {
      float ls[8];
      float v[8][E];
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const bool in = s0 + k < S;
        ls[k] = in ? lse_parts[(int64_t)(s0 + k) * rows + row] : -INFINITY;
        const float *src = o_parts + ((int64_t)(s0 + k) * rows + row) * D + lane * E;
        if constexpr (E == 2) {
          const float2 t = in ? *(const float2 *)src : make_float2(0.f, 0.f);
          v[k][0] = t.x;
          v[k][E - 1] = t.y;
        } else {
          v[k][0] = in ? src[0] : 0.f;
        }
      }
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const float w = ls[k] == -INFINITY ? 0.f : __expf(ls[k] - M);
        Z += w;
#pragma unroll
        for (int e = 0; e < E; ++e) o[e] += w * v[k][e];
      }
    }
    const float inv = 1.f / Z;
#pragma unroll
    for (int e = 0; e < E; ++e) o[e] *= inv;
    lse = M + __logf(Z);
  }
  uint16_t *dst = o_out + row * D + lane * E;
#pragma unroll
  for (int e = 0; e < E; ++e) dst[e] = __builtin_bit_cast(uint16_t, (__bf16)o[e]);
  if (lse_out && lane == 0) lse_out[row] = lse;
}

}  // namespace

hipError_t launch_merge(const float *o_parts, const float *lse_parts, int32_t num_parts,
                        int64_t rows, int32_t head_dim, int32_t num_q_heads, const float *sink,
                        uint16_t *o_out, float *lse_out, hipStream_t stream) {
  if (rows == 0) return hipSuccess;
  const dim3 grid((unsigned)((rows + 3) / 4));
  if (head_dim == 64)
    hipLaunchKernelGGL(merge_kernel<64>, grid, dim3(256), 0, stream, o_parts, lse_parts,
                       num_parts, rows, num_q_heads, sink, o_out, lse_out);
  else
    hipLaunchKernelGGL(merge_kernel<128>, grid, dim3(256), 0, stream, o_parts, lse_parts,
                       num_parts, rows, num_q_heads, sink, o_out, lse_out);
  return hipGetLastError();
}

}  // namespace spa
