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
// HBM-bound: D/4 lanes per row, one float4 of O each (at D 512 a row spans
// two waves); up to 8 parts are
// loaded (LSE and O together) in one round trip, more in chunks of 8.

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
                                                    float *__restrict__ lse_out, int32_t unit_rows) {
  constexpr int LPR = D / 4;          // lanes per row
  constexpr int RPB = 256 / LPR;      // rows per block
  const int c = threadIdx.x % LPR;    // this lane's float4 of the row
  int64_t row;
  if (unit_rows > 0) {
    // Rows come in units of unit_rows (the heads of one query and KV head);
    // block b takes a piece of a unit u with u = b (mod 8), so that it runs
    // on the XCD whose L2 holds the partials the attention kernel wrote for
    // u.
    const int32_t bpu = (unit_rows + RPB - 1) / RPB;
    const int64_t i = blockIdx.x >> 3;
    const int64_t j = i / bpu;
    const int32_t r = (int32_t)(i - j * bpu) * RPB + (int32_t)(threadIdx.x / LPR);
    const int64_t u = (int64_t)(blockIdx.x & 7) + 8 * j;
    if (u * unit_rows >= rows || r >= unit_rows) return;
    row = u * unit_rows + r;
  } else {
    row = (int64_t)blockIdx.x * RPB + threadIdx.x / LPR;
  }
  if (row >= rows) return;
  const float sk = sink ? sink[row % hq] : -INFINITY;
  float M = sk;
  float4 o = make_float4(0.f, 0.f, 0.f, 0.f);
  float Z = 0.f;
  auto part = [&](int s) { return *(const float4 *)(o_parts + ((int64_t)s * rows + row) * D + 4 * c); };
  auto add = [&](float w, const float4 &v) {
    o.x += w * v.x;
    o.y += w * v.y;
    o.z += w * v.z;
    o.w += w * v.w;
  };
  if (S <= 8) {
    // one round trip: every part's LSE and O in flight together
    float ls[8];
    float4 v[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const bool in = k < S;
      ls[k] = in ? lse_parts[(int64_t)k * rows + row] : -INFINITY;
      v[k] = in ? part(k) : make_float4(0.f, 0.f, 0.f, 0.f);
    }
#pragma unroll
    for (int k = 0; k < 8; ++k) M = fmaxf(M, ls[k]);
    if (M != -INFINITY) {
      Z = sk == -INFINITY ? 0.f : __expf(sk - M);
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const float w = ls[k] == -INFINITY ? 0.f : __expf(ls[k] - M);
        Z += w;
        add(w, v[k]);
      }
    }
  } else {
    for (int s0 = 0; s0 < S; s0 += 8) {
      float ls[8];
#pragma unroll
      for (int k = 0; k < 8; ++k) ls[k] = s0 + k < S ? lse_parts[(int64_t)(s0 + k) * rows + row] : -INFINITY;
#pragma unroll
      for (int k = 0; k < 8; ++k) M = fmaxf(M, ls[k]);
    }
    if (M != -INFINITY) {
      Z = sk == -INFINITY ? 0.f : __expf(sk - M);
      for (int s0 = 0; s0 < S; s0 += 8) {
        float ls[8];
        float4 v[8];
#pragma unroll
        for (int k = 0; k < 8; ++k) {
          const bool in = s0 + k < S;
          ls[k] = in ? lse_parts[(int64_t)(s0 + k) * rows + row] : -INFINITY;
          v[k] = in ? part(s0 + k) : make_float4(0.f, 0.f, 0.f, 0.f);
        }
#pragma unroll
        for (int k = 0; k < 8; ++k) {
          const float w = ls[k] == -INFINITY ? 0.f : __expf(ls[k] - M);
          Z += w;
          add(w, v[k]);
        }
      }
    }
  }
  float lse = -INFINITY;
  if (M != -INFINITY) {
    const float inv = 1.f / Z;
    o.x *= inv;
    o.y *= inv;
    o.z *= inv;
    o.w *= inv;
    lse = M + __logf(Z);
  }
  uint2 w;
  w.x = (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)o.x) | ((uint32_t)__builtin_bit_cast(uint16_t, (__bf16)o.y) << 16);
  w.y = (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)o.z) | ((uint32_t)__builtin_bit_cast(uint16_t, (__bf16)o.w) << 16);
  *(uint2 *)(o_out + row * D + 4 * c) = w;
  if (lse_out && c == 0) lse_out[row] = lse;
}

}  // namespace

hipError_t launch_merge(const float *o_parts, const float *lse_parts, int32_t num_parts,
                        int64_t rows, int32_t head_dim, int32_t num_q_heads, const float *sink,
                        uint16_t *o_out, float *lse_out, int32_t unit_rows, hipStream_t stream) {
  if (rows == 0) return hipSuccess;
  const int64_t rpb = 256 / (head_dim / 4);
  int64_t blocks = (rows + rpb - 1) / rpb;
  if (unit_rows > 0) {
    if (rows % unit_rows != 0) return hipErrorInvalidValue;
    const int64_t units = rows / unit_rows;
    blocks = 8 * ((units + 7) / 8) * ((unit_rows + rpb - 1) / rpb);
  }
  if (blocks > 0x7FFFFFFFLL) return hipErrorInvalidConfiguration;
  const dim3 grid((unsigned)blocks);
  if (head_dim == 64)
    hipLaunchKernelGGL(merge_kernel<64>, grid, dim3(256), 0, stream, o_parts, lse_parts,
                       num_parts, rows, num_q_heads, sink, o_out, lse_out, unit_rows);
  else if (head_dim == 128)
    hipLaunchKernelGGL(merge_kernel<128>, grid, dim3(256), 0, stream, o_parts, lse_parts,
                       num_parts, rows, num_q_heads, sink, o_out, lse_out, unit_rows);
  else
    hipLaunchKernelGGL(merge_kernel<512>, grid, dim3(256), 0, stream, o_parts, lse_parts,
                       num_parts, rows, num_q_heads, sink, o_out, lse_out, unit_rows);
  return hipGetLastError();
}

}  // namespace spa
