// Top-k selection of compressed groups from per-token scores, for gfx950.
//
// On the pages, the step before the attention core scores every complete
// compressed group of a token, selects index_topk of them with a radix
// top-k and packs the selected ids into paged offsets (ATOM PR "test: add
// block-level DeepSeek-V4 attention test", sections "What this test
// actually drives" and "Validation").  This kernel is the selection; the
// offsets are the canonical rows attn_build_gather exports.
//
// Order (the pages fix none): descending score, ties by ascending id, -0.0
// below +0.0, a NaN score below every number.  Each float32 score maps to a
// uint32 key whose unsigned order is this order (non-negative: top bit set;
// negative: all bits inverted; NaN: 0), so the selection is unique.
//
// One workgroup per row.  The keys of a row of up to kTkCache entries are
// kept in LDS after one read of the scores.  A radix select over the key,
// 8 bits per pass from the top, finds the k-th largest key T and how many of
// the entries equal to T are taken: each pass builds the histogram of the
// entries still matching T's known high bits, and one workgroup scan over the
// 256 digits (highest first) finds the digit where the running count reaches
// the number still wanted.  The passes stop early once every entry under the
// known prefix is taken.  The entries above T are then collected in any
// order and those equal to T in ascending id order (a workgroup scan gives
// each its rank); the at most k selected (key, id) pairs are sorted by a
// bitonic network on (key << 32 | ~id), descending, held in registers.

#include <hip/hip_runtime.h>

#include <cstdint>

#include "spa_internal.h"
#include "spa_kernel_util.h"

namespace spa {
namespace {

constexpr int kTkThreads = 256;
constexpr int kTkCache = 4096;   // rows of up to this many entries keep their keys in LDS

__device__ __forceinline__ uint32_t score_key(uint32_t bits) {
  const bool nan = (bits & 0x7F800000u) == 0x7F800000u && (bits & 0x007FFFFFu) != 0u;
  if (nan) return 0u;
  return (bits & 0x80000000u) ? ~bits : (bits | 0x80000000u);
}


__device__ __forceinline__ unsigned long long shfl_xor_u64(unsigned long long v, int m) {
  const uint32_t lo = (uint32_t)__shfl_xor((int)(uint32_t)v, m);
  const uint32_t hi = (uint32_t)__shfl_xor((int)(uint32_t)(v >> 32), m);
  return ((unsigned long long)hi << 32) | lo;
}

// Sorts sel[0, kk) descending as a bitonic network over P = 256 * C entries
// held in registers (entry c * 256 + tid in v[c]; padding 0 sorts last, a
// selected pair is never 0 since ~id has its top bit set), then writes the
// ids of the first k positions (-1 past kk).  A stride below 64 pairs lanes
// of one wave (shuffles), a stride of 256 or more pairs registers of one
// thread, and only strides 64 and 128 exchange through LDS.  sel must be
// readable by every thread on entry.
template <int C>
__device__ __forceinline__ void sort_write(unsigned long long *sel, int32_t kk, int32_t k, int32_t *out) {
  const int tid = threadIdx.x;
  constexpr int P = kTkThreads * C;
  unsigned long long v[C];
#pragma unroll
  for (int c = 0; c < C; ++c) {
    const int i = c * kTkThreads + tid;
    v[c] = i < kk ? sel[i] : 0ull;
  }
  __syncthreads();                           // sel is the exchange buffer from here
#pragma unroll
  for (int size = 2; size <= P; size <<= 1) {
#pragma unroll
    for (int s = size >> 1; s > 0; s >>= 1) {
      if (s >= kTkThreads) {
#pragma unroll
        for (int c = 0; c < C; ++c) {
          const int cp = c ^ (s / kTkThreads);
          if (cp > c) {
            const bool desc = ((c * kTkThreads + tid) & size) == 0;
            const unsigned long long a = v[c], b = v[cp];
            if (desc ? (a < b) : (a > b)) {
              v[c] = b;
              v[cp] = a;
            }
          }
        }
      } else {
        unsigned long long w[C];
        if (s >= 64) {
#pragma unroll
          for (int c = 0; c < C; ++c) sel[c * kTkThreads + tid] = v[c];
          __syncthreads();
#pragma unroll
          for (int c = 0; c < C; ++c) w[c] = sel[c * kTkThreads + (tid ^ s)];
          __syncthreads();
        } else {
#pragma unroll
          for (int c = 0; c < C; ++c) w[c] = shfl_xor_u64(v[c], s);
        }
#pragma unroll
        for (int c = 0; c < C; ++c) {
          const bool desc = ((c * kTkThreads + tid) & size) == 0;
          const bool lower = (tid & s) == 0;
          const unsigned long long a = v[c], b = w[c];
          v[c] = (desc == lower) ? (a > b ? a : b) : (a < b ? a : b);
        }
      }
    }
  }
#pragma unroll
  for (int c = 0; c < C; ++c) {
    const int i = c * kTkThreads + tid;
    if (i < k) out[i] = i < kk ? (int32_t)(~(uint32_t)(v[c] & 0xFFFFFFFFull)) : -1;
  }
  for (int32_t i = P + tid; i < k; i += kTkThreads) out[i] = -1;
}

__global__ __launch_bounds__(kTkThreads) void topk_kernel(const float *scores, int64_t ld, const int32_t *n_valid,
                                                        int32_t k, int32_t *ids_out, int32_t *cnt_out) {
  __shared__ uint32_t hist[256];
  __shared__ uint32_t cache[kTkCache];
  __shared__ unsigned long long sel[kTopkMax];
  __shared__ int32_t wsum[kTkThreads / 64];
  __shared__ int32_t sh_digit, sh_krem, sh_done, sh_ngt;
  const int tid = threadIdx.x;
  const int64_t row = blockIdx.x;
  const uint32_t *src = reinterpret_cast<const uint32_t *>(scores + row * ld);
  int32_t n = n_valid[row];
  n = n < 0 ? 0 : (n > ld ? (int32_t)ld : n);
  const int32_t kk = n < k ? n : k;
  int32_t *out = ids_out + row * (int64_t)k;
  const bool cached = n <= kTkCache;
  // the key of entry j (from the LDS copy when the row fits)
  auto key = [&](int32_t j) -> uint32_t { return cached ? cache[j] : score_key(src[j]); };

  if (kk < n) {
    if (cached) {
      for (int32_t j = tid; j < n; j += kTkThreads) cache[j] = score_key(src[j]);
    }
    // -- radix select: the k-th largest key T's high bits (prefix under
    // mask) and how many of the entries matching them are taken (krem)
    uint32_t prefix = 0u, mask = 0u;
    int32_t krem = kk;
    for (int pass = 0; pass < 4; ++pass) {
      const int shift = 24 - 8 * pass;
      hist[tid] = 0u;
      __syncthreads();
      for (int32_t j = tid; j < n; j += kTkThreads) {
        const uint32_t u = key(j);
        if ((u & mask) == prefix) atomicAdd(&hist[(u >> shift) & 255u], 1u);
      }
      __syncthreads();
      // thread t owns digit 255 - t: the entries above it are the exclusive
      // prefix sum in this order
      const int32_t h = (int32_t)hist[255 - tid];
      int32_t tot;
      const int32_t above = block_excl_scan<kTkThreads>(h, tot, wsum);
      if (above < krem && above + h >= krem) {
        sh_digit = 255 - tid;
        sh_krem = krem - above;
        sh_done = (krem - above == h) ? 1 : 0;
      }
      __syncthreads();
      prefix |= (uint32_t)sh_digit << shift;
      mask |= 0xFFu << shift;
      krem = sh_krem;
      const bool done = sh_done != 0;
      __syncthreads();                       // sh_* and hist are rewritten in the next pass
      if (done) break;
    }
    // -- collect: every entry above the prefix, and the first krem entries
    // matching it in ascending id order
    const int32_t ngt = kk - krem;
    if (tid == 0) sh_ngt = 0;
    __syncthreads();
    int32_t eq_base = 0;
    for (int32_t c0 = 0; c0 < n; c0 += kTkThreads) {
      const int32_t j = c0 + tid;
      const uint32_t u = j < n ? key(j) : 0u;
      const bool gt = j < n && (u & mask) > prefix;
      const bool eq = j < n && (u & mask) == prefix;
      int32_t tot;
      const int32_t r = eq_base + block_excl_scan<kTkThreads>(eq ? 1 : 0, tot, wsum);
      const unsigned long long comp = ((unsigned long long)u << 32) | (uint32_t)(~(uint32_t)j);
      if (gt) {
        const int32_t slot = atomicAdd(&sh_ngt, 1);
        if (slot < ngt) sel[slot] = comp;
      }
      if (eq && r < krem) sel[ngt + r] = comp;
      eq_base += tot;
    }
  } else {
    // every valid entry is taken (n <= k <= kTopkMax)
    for (int32_t j = tid; j < n; j += kTkThreads)
      sel[j] = ((unsigned long long)score_key(src[j]) << 32) | (uint32_t)(~(uint32_t)j);
  }
  __syncthreads();
  // -- sort the kk selected pairs, descending, and write the ids
  if (kk <= 256) {
    sort_write<1>(sel, kk, k, out);
  } else if (kk <= 512) {
    sort_write<2>(sel, kk, k, out);
  } else if (kk <= 1024) {
    sort_write<4>(sel, kk, k, out);
  } else {
    sort_write<8>(sel, kk, k, out);
  }
  if (tid == 0) cnt_out[row] = kk;
}

}  // namespace

hipError_t launch_topk(const float *scores, int64_t ld, const int32_t *n_valid, int32_t rows, int32_t k,
                       int32_t *ids_out, int32_t *cnt_out, hipStream_t stream) {
  if (rows == 0) return hipSuccess;
  if (k < 1 || k > kTopkMax) return hipErrorInvalidValue;
  hipLaunchKernelGGL(topk_kernel, dim3((unsigned)rows), dim3(kTkThreads), 0, stream, scores, ld, n_valid, k, ids_out,
                     cnt_out);
  return hipGetLastError();
}

}  // namespace spa
