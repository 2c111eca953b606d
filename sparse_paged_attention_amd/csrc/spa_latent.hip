// Sparse paged attention over a shared latent KV cache with 512-wide heads,
// for gfx950.
//
// The DeepSeek-V4 cache the pages decode keeps one latent row per token that
// serves as both key and value, 512 wide.  RL-Kernel PR "Roadmap item 24:
// joint compressed/window attention with sink", review comments on the
// joint-attention contract and on the model's packed-page gather: the plan
// holds a single bf16 `_kv` buffer of head_dim-wide rows, the contract
// admits head widths 128 and 512, and the gather turns packed pages into
// 512-wide bf16 rows.  The KV set, the sink and the outputs are those of
// the 128-wide path; only the head width and the K = V sharing differ, and
// the sharing lets one LDS tile serve as K and as V, so each gathered row is
// read once.
//
// One workgroup of eight waves per (query, KV head, block of 64 query heads,
// KV slice): wave w takes head group w / 4 (32 heads, the MFMA's N) and head
// dimensions 128 (w % 4) .. +127.  Per 32-row tile (1 KiB rows, three LDS
// stages filled by direct global->LDS loads, one 1 KiB load per row):
//   * each wave forms the partial S^T = K.Q^T over its 128 dimensions
//     (v_mfma_f32_32x32x16_bf16) and stores it in LDS;
//   * after a barrier, wave (g, q) sums float4 q of its group's four
//     partials in a fixed order and publishes it; after another barrier the
//     four waves of a group read the same sums (half the LDS reads of each
//     wave summing everything) and run identical online softmaxes (log2
//     domain, sink folded into (m, l), lazy rescale);
//   * O^T += V^T.P^T for the wave's 128 dimensions, V^T read from the same
//     tile by transposing LDS reads.
// A 1 KiB row is four 256-byte quarters, each laid out (and swizzled) like a
// 128-wide row, so the fragment reads have the 128-wide path's conflict
// behaviour.  With several slices the workgroup writes a sink-free partial
// (O_s in fp32, LSE_s) for the LSE merge.
//
// FP8: the compressed pool may hold e4m3 codes (OCP or FNUZ) with one fp32
// scale per latent row, shared by its key and value roles.  A slice then
// takes its compressed entries and its window entries as separate chunks,
// so every tile is all e4m3 or all bf16.  An e4m3 tile's 512-byte rows (two
// per 1 KiB direct load) land in the upper half of the tile's stage with
// their scales; after the tile's barrier every thread reads its codes, and
// after a second barrier widens them exactly to bf16 over the whole stage.
// The scale multiplies the summed fp32 scores and p before its bf16
// rounding, as on the 128-wide path.

#include <hip/hip_runtime.h>

#include <cstdint>

#include "spa_device.h"
#include "spa_kernel_util.h"

namespace spa {
namespace {

constexpr int kD = 512;
constexpr int kRowB = 2 * kD;              // 1 KiB rows
constexpr int kQB = 256;                   // bytes per 128-wide quarter
constexpr int kPT = 32;                    // rows per tile
constexpr int kTileB = kPT * kRowB;
constexpr int kLThreads = 512;             // eight waves
constexpr int kLRows = 512;                // rows translated per chunk (one per thread)
constexpr int kLStages = 3;               // two tiles in flight while one is computed
constexpr int64_t kCmpBit = int64_t(1) << 62;

template <bool FP8>
struct LatentSmem {
  alignas(16) uint8_t kv[kLStages][kTileB];
  alignas(16) float f8s[FP8 ? kLStages : 1][64];   // e4m3 tiles: row scales (32 used)
  alignas(16) float4 xs[2][4][4][64];      // partial S^T: [head group][quarter][float4][lane]
  alignas(16) float4 xf[2][4][64];         // summed S^T: [head group][float4][lane]
  alignas(16) int64_t row[kLRows];         // row * Hkv + g (bit 62: compressed), -1: masked
};

// byte offset of the 16-byte chunk holding dimensions 8c .. 8c+7 of tile row r
__device__ __forceinline__ int chunk_off(int r, int c) {
  return r * kRowB + (c >> 4) * kQB + (((c & 15) ^ swz<16>(r)) * 16);
}

template <bool FP8>
__global__ __launch_bounds__(kLThreads) void attn_latent_kernel(Params p) {
  __shared__ LatentSmem<FP8> sm;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int hg = wave >> 2;                  // head group
  const int dq = wave & 3;                   // dimension quarter
  const int hi = lane >> 5;
  const int S = p.num_splits;
  const int hblocks = (p.group + 63) / 64;
  const int64_t job = blockIdx.x;
  const int split = (int)(job % S);
  const int64_t u = job / S;
  const int hb = (int)(u % hblocks);
  const int64_t v = u / hblocks;
  const int g = (int)(v % p.hkv);
  const int i = (int)(v / p.hkv);
  const QueryKV kv = query_kv(p, i);
  const int32_t U = kv.n_sel + kv.win_len;
  // slice: canonical entries [e_lo, e_hi), ceil(U / S) rounded up to a tile
  const int32_t per = round_up((U + S - 1) / S, kPT);
  const int32_t e_lo = min(U, split * per);
  const int32_t e_hi = min(U, e_lo + per);

  const int hl = hb * 64 + hg * 32 + (lane & 31);
  const bool hvalid = hl < p.group;
  const int64_t qrow = (int64_t)i * p.hq + (int64_t)g * p.group + hl;
  bf16x8 qf[8];
  {
    const uint16_t *q = p.q + qrow * kD + 128 * dq + 8 * hi;
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) qf[kk] = hvalid ? *(const bf16x8 *)(q + 16 * kk) : bf16x8{};
  }
  const float sink = (hvalid && p.sink != nullptr && S == 1) ? p.sink[g * p.group + hl] : -INFINITY;
  float m = sink == -INFINITY ? -INFINITY : sink * kLog2e;
  float l = (sink != -INFINITY && hi == 0) ? 1.f : 0.f;
  f32x16 acc[4];
#pragma unroll
  for (int db = 0; db < 4; ++db) acc[db] = f32x16{};

  const uint8_t *const kraw = in_sgpr(p.k_raw), *const kcmp = in_sgpr(p.k_cmp);
  const float *const kscale = in_sgpr(p.k_cmp_scale);
  const bool fnuz = FP8 && p.cmp_fnuz != 0;
  constexpr int kF8Off = kTileB / 2;         // e4m3 codes staged in the upper half of a stage
  // tile loads: wave w moves rows 4w .. 4w+3, one 1 KiB load per row; lane
  // L's chunk is logical chunk 16 (L / 16) + ((L % 16) ^ swz(row))
  auto issue = [&](int j) {
    const int st = j % kLStages;
    // every row first: the loads' memory clobber keeps a later LDS read
    // from starting ahead of them
    int64_t ers[4];
#pragma unroll
    for (int n = 0; n < 4; ++n) ers[n] = sm.row[kPT * j + 4 * wave + n];
#pragma unroll
    for (int n = 0; n < 4; ++n) {
      const int r = 4 * wave + n;
      const int64_t er = ers[n];
      const int cs = (lane >> 4) * kQB + (((lane & 15) ^ swz<16>(r)) * 16);
      const bool cmp = (er & kCmpBit) != 0;
      dma16(er >= 0 ? (cmp ? kcmp : kraw) + (er & ~kCmpBit) * kRowB + cs : kZeroRow + (cs & (kQB - 1)),
            sm.kv[st] + r * kRowB);
    }
  };

  // an e4m3 tile: wave w moves rows 4w .. 4w+3, two 512-byte rows per
  // 1 KiB load (lane L: row 4w + 2n + L / 32, bytes 16 (L % 32) ..); wave 0
  // also loads the 32 scales
  auto issue_f8 = [&](int j) {
    const int st = j % kLStages;
    int64_t ers[2];
#pragma unroll
    for (int n = 0; n < 2; ++n) ers[n] = sm.row[kPT * j + 4 * wave + 2 * n + (lane >> 5)];
    const int64_t es = (wave == 0 && lane < kPT) ? sm.row[kPT * j + lane] : -1;
#pragma unroll
    for (int n = 0; n < 2; ++n) {
      const int64_t er = ers[n];
      dma16(er >= 0 ? kcmp + (er & ~kCmpBit) * kD + (lane & 31) * 16 : kZeroRow + (lane & 15) * 16,
            sm.kv[st] + kF8Off + (4 * wave + 2 * n) * kD);
    }
    if (wave == 0) {
      const int64_t er = es;
      dma4(er >= 0 ? (const void *)(kscale + (er & ~kCmpBit)) : (const void *)(kZeroRow + 4 * lane),
           sm.f8s[FP8 ? st : 0]);
    }
  };

  // one chunk: canonical entries c0 .. c0+n-1, all compressed when f8c
  auto run_chunk = [&](const int32_t c0, const int32_t n, const bool f8c) {
    const int32_t ntiles = (n + kPT - 1) / kPT;
    {
      const int32_t e = c0 + tid;
      int64_t er = -1;
      if (tid < n) {
        const bool cmp = e < kv.n_sel;
        const int64_t pr = logical_row(p, kv, cmp, entry_logical(p, kv, i, e));
        if (pr >= 0) er = (pr * p.hkv + g) | (cmp ? kCmpBit : 0);
      }
      if (tid < ntiles * kPT) sm.row[tid] = er;
    }
    __syncthreads();
    auto issue_tile = [&](int j) {
      if (FP8 && f8c) issue_f8(j);
      else issue(j);
    };
    issue_tile(0);
    if (ntiles > 1) issue_tile(1);
    for (int j = 0; j < ntiles; ++j) {
      // this wave's loads of tile j are complete (tile j+1's may still be in
      // flight: four loads, or two and wave 0's scales for an e4m3 tile),
      // then everyone's; every wave is done with tile j-1, whose stage tile
      // j+2 refills
      if (j + 1 < ntiles) {
        if (FP8 && f8c) {
          if (wave == 0) wait_vmcnt<3>();
          else wait_vmcnt<2>();
        } else {
          wait_vmcnt<4>();
        }
      } else {
        wait_vmcnt<0>();
      }
      block_sync();
      if (FP8 && f8c) {
        // widen the staged codes over the whole stage: every thread reads
        // its four 8-code pieces before any bf16 write lands on them
        uint8_t *W = sm.kv[j % kLStages];
        uint2 cw[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const int idx = tid + kLThreads * k;   // row idx / 64, piece idx % 64
          cw[k] = *(const uint2 *)(W + kF8Off + (idx >> 6) * kD + (idx & 63) * 8);
        }
        block_sync();
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const int idx = tid + kLThreads * k;
          *(uint4 *)(W + chunk_off(idx >> 6, idx & 63)) = widen8_e4m3(cw[k], fnuz);
        }
        block_sync();                        // the widened tile is in
      }
      if (j + 2 < ntiles) issue_tile(j + 2);
      const uint8_t *T = sm.kv[j % kLStages];
      const uint32_t tm = (uint32_t)__ballot(lane < 32 && sm.row[kPT * j + (lane & 31)] >= 0);
      // partial scores over this wave's 128 dimensions
      f32x16 s = f32x16{};
#pragma unroll
      for (int kk = 0; kk < 8; ++kk) {
        const int r = lane & 31;
        const bf16x8 kf = *(const bf16x8 *)(T + chunk_off(r, 16 * dq + 2 * kk + hi));
        s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[kk], s, 0, 0, 0);
      }
      // V^T fragments of the wave's dimensions (read while the partials
      // are exchanged)
      bf16x8 vf[4][2];
      {
        const int G = lane >> 4, L = lane & 15;
#pragma unroll
        for (int db = 0; db < 4; ++db)
#pragma unroll
          for (int k2 = 0; k2 < 2; ++k2) {
            i16x4 f[2];
#pragma unroll
            for (int rr = 0; rr < 2; ++rr) {
              const int row = 16 * k2 + 8 * rr + 4 * (G >> 1) + (L >> 2);
              const int d = 128 * dq + 32 * db + 16 * (G & 1) + 4 * (L & 3);
              f[rr] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                  (lds_i16x4_t *)(T + chunk_off(row, d >> 3) + (L & 1) * 8));
            }
            const i16x8 cat = {f[0][0], f[0][1], f[0][2], f[0][3], f[1][0], f[1][1], f[1][2], f[1][3]};
            vf[db][k2] = __builtin_bit_cast(bf16x8, cat);
          }
      }
#pragma unroll
      for (int c = 0; c < 4; ++c)
        sm.xs[hg][dq][c][lane] = make_float4(s[4 * c], s[4 * c + 1], s[4 * c + 2], s[4 * c + 3]);
      block_sync();
      // the group's full scores: wave (g, q) sums float4 q of the four
      // partials (quarter order) and publishes it; then every wave of the
      // group reads all four sums, so the four hold the same scores
      {
        float4 t = sm.xs[hg][0][dq][lane];
#pragma unroll
        for (int q = 1; q < 4; ++q) {
          const float4 x = sm.xs[hg][q][dq][lane];
          t.x += x.x;
          t.y += x.y;
          t.z += x.z;
          t.w += x.w;
        }
        sm.xf[hg][dq][lane] = t;
      }
      block_sync();
      float sc[16];
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const float4 t = sm.xf[hg][c][lane];
        sc[4 * c] = t.x;
        sc[4 * c + 1] = t.y;
        sc[4 * c + 2] = t.z;
        sc[4 * c + 3] = t.w;
      }
      // the row scale multiplies the summed scores of an e4m3 tile
      if (FP8 && f8c) {
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          const float4 k4 = *(const float4 *)(&sm.f8s[FP8 ? j % kLStages : 0][8 * q4 + 4 * hi]);
          sc[4 * q4 + 0] *= k4.x;
          sc[4 * q4 + 1] *= k4.y;
          sc[4 * q4 + 2] *= k4.z;
          sc[4 * q4 + 3] *= k4.w;
        }
      }
      // online softmax; lane rows of S^T: 8 (r / 4) + 4 hi + r % 4
      const uint32_t tmh = tm >> (4 * hi);
#pragma unroll
      for (int r = 0; r < 16; ++r) sc[r] = ((tmh >> (8 * (r >> 2) + (r & 3))) & 1u) ? sc[r] : -INFINITY;
      float smax = sc[0];
#pragma unroll
      for (int r = 1; r < 16; ++r) smax = fmaxf(smax, sc[r]);
      smax = max_lane_pair(smax);
      const float tmax = smax * p.scale_log2;
      const bool need = tmax > m + kTau;
      if (__any(need)) {
        const float alpha = need ? __builtin_amdgcn_exp2f(m - tmax) : 1.f;
        m = need ? tmax : m;
        l *= alpha;
#pragma unroll
        for (int db = 0; db < 4; ++db) acc[db] *= alpha;
      }
      const float negm = m == -INFINITY ? 0.f : -m;
      float psum = 0.f;
      bf16x8 pb[2];
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float pr = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[r], p.scale_log2, negm));
        psum += pr;
        // an e4m3 tile: the row scale multiplies p before its bf16 rounding
        const float pv = (FP8 && f8c) ? pr * sm.f8s[FP8 ? j % kLStages : 0][8 * (r >> 2) + 4 * hi + (r & 3)] : pr;
        pb[r >> 3][r & 7] = (__bf16)pv;
      }
      l += psum;
#pragma unroll
      for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int k2 = 0; k2 < 2; ++k2)
          acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf[db][k2], pb[k2], acc[db], 0, 0, 0);
    }
    wait_vmcnt<0>();
    __syncthreads();                         // the row list is rewritten by the next chunk
  };
  if (FP8) {
    const int32_t c_hi = min(e_hi, kv.n_sel);
    for (int32_t c0 = e_lo; c0 < c_hi; c0 += kLRows) run_chunk(c0, min(kLRows, c_hi - c0), true);
    for (int32_t c0 = max(e_lo, kv.n_sel); c0 < e_hi; c0 += kLRows) run_chunk(c0, min(kLRows, e_hi - c0), false);
  } else {
    for (int32_t c0 = e_lo; c0 < e_hi; c0 += kLRows) run_chunk(c0, min(kLRows, e_hi - c0), false);
  }

  // ---- epilogue: O = acc / l, LSE = (m + log2 l) ln 2; lane column = head,
  // value r = dimension 128 dq + 32 db + 8 (r / 4) + 4 hi + r % 4
  const float lt = l + __shfl_xor(l, 32);
  const float inv = lt > 0.f ? 1.f / lt : 0.f;
  const float lse2 = (m == -INFINITY || !(lt > 0.f)) ? -INFINITY : m + __builtin_amdgcn_logf(lt);
  const float lse = lse2 == -INFINITY ? -INFINITY : lse2 * kLn2;
  if (!hvalid) return;
  if (S > 1) {
    const int64_t prow = (int64_t)split * p.num_queries * p.hq + qrow;
    float *po = p.part_o + prow * kD + 128 * dq;
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int i4 = 0; i4 < 4; ++i4)
        *(float4 *)(po + 32 * db + 8 * i4 + 4 * hi) =
            make_float4(acc[db][4 * i4] * inv, acc[db][4 * i4 + 1] * inv, acc[db][4 * i4 + 2] * inv,
                        acc[db][4 * i4 + 3] * inv);
    if (dq == 0 && hi == 0) p.part_lse[prow] = lse;
    return;
  }
  uint16_t *orow = p.o + qrow * kD + 128 * dq;
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int i4 = 0; i4 < 4; ++i4) {
      uint2 w;
      w.x = bf16_bits(acc[db][4 * i4 + 0] * inv) | (bf16_bits(acc[db][4 * i4 + 1] * inv) << 16);
      w.y = bf16_bits(acc[db][4 * i4 + 2] * inv) | (bf16_bits(acc[db][4 * i4 + 3] * inv) << 16);
      *(uint2 *)(orow + 32 * db + 8 * i4 + 4 * hi) = w;
    }
  if (dq == 0 && hi == 0 && p.lse) p.lse[qrow] = lse;
}

}  // namespace

hipError_t launch_latent(const Params &p, hipStream_t stream) {
  if (p.head_dim != kD || p.k_raw != p.v_raw || (p.ratio > 0 && p.k_cmp != p.v_cmp)) return hipErrorInvalidValue;
  if (p.cmp_fp8 && p.k_cmp_scale != p.v_cmp_scale) return hipErrorInvalidValue;
  if (p.num_queries == 0) return hipSuccess;
  const int64_t grid = (int64_t)p.num_queries * p.hkv * ((p.group + 63) / 64) * p.num_splits;
  if (grid > 0x7FFFFFFFLL) return hipErrorInvalidConfiguration;
  if (p.cmp_fp8)
    hipLaunchKernelGGL(attn_latent_kernel<true>, dim3((unsigned)grid), dim3(kLThreads), 0, stream, p);
  else
    hipLaunchKernelGGL(attn_latent_kernel<false>, dim3((unsigned)grid), dim3(kLThreads), 0, stream, p);
  return hipGetLastError();
}

}  // namespace spa
