// Sparse paged attention forward with a sink, for gfx950 (CDNA4).
//
// Operation: RL-Kernel PR "Roadmap item 24: joint compressed/window attention
// with sink", section "Reuse and arithmetic" — the selected compressed KV, the
// full recent raw window and a per-head sink logit share one softmax
// denominator; the sink has no value row; P and O are bf16, LSE is fp32
// natural log.  The KV set and page translation live in spa_device.h.
//
// Work decomposition.  One workgroup owns one (query, KV slice, KV head,
// group of up to 128 query heads).  All query heads of a KV head read the same
// KV rows, so they share every KV tile the workgroup stages in LDS: each wave
// holds 32 query heads and the tile's 32 KV rows feed bf16 MFMAs for all of
// them.
//
//   S^T[kv, head]  = K[kv, :] . Q^T[:, head]        v_mfma_f32_32x32x16_bf16
//   O^T[d, head]  += V^T[d, kv] . P^T[kv, head]      v_mfma_f32_32x32x16_bf16
//
// With S^T and O^T in the MFMA accumulator layout every lane owns one query
// head (lane % 32), so the online-softmax state (m, l) is per lane; the
// row max needs one exchange with lane ^ 32, and P^T goes from the S^T
// accumulators straight into the B operand of the PV MFMA (the KV order inside
// a 16-row step is permuted identically on both operands).  V^T comes from
// the row-major V tile through the gfx950 LDS transpose read
// (ds_read_b64_tr_b16), so no transposition pass is needed.
//
// Data movement.  The KV rows of a slice are translated to 64-bit row
// offsets once per chunk of up to 16 tiles (the page-table walk), then every
// tile is fetched by direct global->LDS loads (global_load_lds_dwordx4,
// 16 B per lane, no VGPR staging) into a 3-deep ring of LDS buffers, so two
// tiles are in flight while the third is computed.  Masked rows (slice tail,
// invalid metadata) are fetched from a static zero row, so every thread issues
// the same number of loads per tile and one vmcnt immediate tracks the ring.
// LDS rows are XOR-swizzled in 16-byte chunks so that the K reads (one row per
// lane) and the transpose reads (4 rows x 32 B per 16 lanes) are free of bank
// conflicts.
//
// FP8 (OCP e4m3) compressed rows land in an LDS staging area and are widened
// to bf16 exactly (every e4m3 value is a bf16 value) by the hardware
// v_cvt_pk_f32_fp8; the per-token scales are applied in fp32 to the scores
// (k) and to P (v), so the MFMAs see the exact codes.
//
// Softmax runs in the log2 domain (scores pre-multiplied by scale*log2 e,
// sink by log2 e) with v_exp_f32; the running max starts at the sink and the
// running sum at exp(0) = 1, i.e. the sink is folded into (m, l) from the
// start.  With num_splits > 1 the workgroup writes a sink-free partial
// (O_s f32, LSE_s) and the merge kernel adds the sink exactly once.

#include <hip/hip_runtime.h>

#include <cstdint>

#include "spa_device.h"

namespace spa {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(3))) i16x4 lds_i16x4_t;

constexpr int kTile = 32;        // KV rows per tile
constexpr int kBufs = 3;         // LDS ring depth
constexpr int kChunkTiles = 16;  // tiles translated per page-table pass
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// Source of the 16-byte loads for masked rows.
__device__ __attribute__((aligned(16))) const uint8_t kZeroRow[256] = {};

// One wave-wide direct global->LDS load: lane L's 16 bytes from `src` land at
// lds_dst + 16 L (lds_dst is wave-uniform and goes through M0).  Written as
// inline asm so that the compiler does not guard every later LDS read with a
// wait for all outstanding loads; completion is tracked explicitly with
// wait_vmcnt<> below.  The instruction has no destination registers.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"   // M0 is reserved; only these loads use it here
__device__ __forceinline__ void dma16(const void *src, void *lds_dst) {
  const uint32_t lds = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(lds_void_t *)lds_dst);
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off"
               :
               : "v"(src), "s"(lds)
               : "memory", "m0");
}
#pragma clang diagnostic pop

// s_waitcnt with only the vector-memory counter constrained (gfx9 encoding:
// vmcnt[3:0] | expcnt[6:4] | lgkmcnt[11:8] | vmcnt[5:4] << 14).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

// Workgroup barrier that waits only for this wave's LDS operations.  The
// HIP __syncthreads() adds a workgroup release fence, which on gfx950 also
// waits for every outstanding global load and would drain the LDS ring;
// global->LDS loads are instead completed explicitly with wait_vmcnt<>.
// The "memory" clobber keeps the compiler from moving LDS accesses across it.
__device__ __forceinline__ void block_sync() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

__device__ __forceinline__ uint32_t pack_bf16_hi(float lo, float hi) {
  // exact narrowing for values that are bf16 already (widened e4m3 codes)
  return (__builtin_bit_cast(uint32_t, lo) >> 16) | (__builtin_bit_cast(uint32_t, hi) & 0xFFFF0000u);
}

template <int D, int NW, bool FP8>
struct Cfg {
  static constexpr int kThreads = NW * 64;
  static constexpr int kRowB = 2 * D;                 // bf16 row bytes
  static constexpr int kChunks = kRowB / 16;          // 16-byte chunks per row
  static constexpr int kTileB = kTile * kRowB;        // one K (or V) tile, bytes
  static constexpr int kKVInstr = 2 * kTileB / 1024;  // wave-wide 1 KiB loads per tile
  static constexpr int kOps = kKVInstr / NW;          // loads per thread per tile
  static constexpr int kF8TileB = kTile * D;          // one e4m3 K (or V) tile
  static constexpr int kF8Instr = 2 * kF8TileB / 1024;
  static_assert(kKVInstr % NW == 0 && kF8Instr % NW == 0, "load split");
  static_assert((kF8Instr / NW) <= kOps, "fp8 loads are padded to the bf16 count");
};

template <int D, int NW, bool FP8>
struct Smem {
  using C = Cfg<D, NW, FP8>;
  alignas(16) uint8_t kv[kBufs][2][C::kTileB];
  alignas(16) uint8_t stage[FP8 ? kBufs : 1][2][FP8 ? C::kF8TileB : 16];
  alignas(16) uint8_t dummy[FP8 ? 1024 : 16];
  alignas(16) int64_t erow[kChunkTiles * kTile];      // element row (row*Hkv+g), -1 = masked
  alignas(16) float ks[kChunkTiles * kTile];
  alignas(16) float vs[kChunkTiles * kTile];
};

// Tile j of a slice: compressed tiles cover [c_lo, c_hi), window tiles
// cover [w_lo, w_hi); a tile never mixes the two kinds.
struct SliceTiles {
  int c_lo, c_hi, w_lo, w_hi, nct, total;
  __device__ __forceinline__ void tile(int j, int &start, int &len, bool &cmp) const {
    if (j < nct) {
      start = c_lo + j * kTile;
      len = min(kTile, c_hi - start);
      cmp = true;
    } else {
      start = w_lo + (j - nct) * kTile;
      len = min(kTile, w_hi - start);
      cmp = false;
    }
  }
};

template <int D, int NW, bool FP8>
__global__ __launch_bounds__(NW * 64) void attn_fwd_kernel(const Params p) {
  using C = Cfg<D, NW, FP8>;
  __shared__ Smem<D, NW, FP8> sm;

  const int S = p.num_splits;
  const int qi = blockIdx.x / S;
  const int split = blockIdx.x - qi * S;
  const int g = blockIdx.y / p.head_groups;
  const int hgrp = blockIdx.y - g * p.head_groups;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int hi = lane >> 5;             // which half of the wave
  const int hl = hgrp * 128 + wave * 32 + (lane & 31);   // head within the KV group
  const bool head_ok = hl < p.group;
  const int h = g * p.group + hl;

  // ---- Q^T as the B operand: lane holds head (lane%32), d = 16kk + 8*hi ..+7
  bf16x8 qf[D / 16];
  {
    const uint16_t *qrow = p.q + ((int64_t)qi * p.hq + (head_ok ? h : 0)) * D;
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk) {
      uint4 v = head_ok ? *(const uint4 *)(qrow + 16 * kk + 8 * hi) : make_uint4(0, 0, 0, 0);
      qf[kk] = __builtin_bit_cast(bf16x8, v);
    }
    // Complete the Q loads here: a lazy wait at the first MFMA would also
    // wait for every global->LDS load in flight at that point.
    wait_vmcnt<0>();
  }

  // ---- KV set of the query and this workgroup's slice of it
  const QueryKV kv = query_kv(p, qi);
  const int N = kv.n_sel + kv.win_len;
  const int per = ((N + S - 1) / S + kTile - 1) / kTile * kTile;
  const int e0 = min(N, split * per);
  const int e1 = min(N, e0 + per);
  SliceTiles st;
  st.c_lo = e0;
  st.c_hi = min(e1, kv.n_sel);
  st.w_lo = max(e0, kv.n_sel);
  st.w_hi = e1;
  st.nct = st.c_hi > st.c_lo ? (st.c_hi - st.c_lo + kTile - 1) / kTile : 0;
  const int nwt = st.w_hi > st.w_lo ? (st.w_hi - st.w_lo + kTile - 1) / kTile : 0;
  st.total = st.nct + nwt;

  // ---- online softmax state (log2 domain); the sink is folded in up front
  float m = -INFINITY, l = 0.f;
  if (S == 1 && p.sink != nullptr && head_ok) {
    m = p.sink[h] * kLog2e;
    l = hi == 0 ? 1.f : 0.f;   // exp2(sink - m) = 1, counted once per head
  }
  f32x16 acc[D / 32];
#pragma unroll
  for (int db = 0; db < D / 32; ++db) acc[db] = f32x16{};

  const float *ksc = p.k_cmp_scale;
  const float *vsc = p.v_cmp_scale;

  for (int cbase = 0; cbase < st.total; cbase += kChunkTiles) {
    const int ct = min(kChunkTiles, st.total - cbase);
    block_sync();   // previous chunk is done with the row table
    // -- page-table walk for the chunk's tiles
    for (int idx = tid; idx < ct * kTile; idx += C::kThreads) {
      const int j = cbase + idx / kTile;
      const int r = idx % kTile;
      int start, len;
      bool cmp;
      st.tile(j, start, len, cmp);
      int64_t er = -1;
      float a = 1.f, b = 1.f;
      if (r < len) {
        const int64_t row = entry_row(p, kv, qi, start + r);
        if (row >= 0) {
          er = row * p.hkv + g;
          if (FP8 && cmp) {
            a = ksc[er];
            b = vsc[er];
          }
        }
      }
      sm.erow[idx] = er;
      sm.ks[idx] = a;
      sm.vs[idx] = b;
    }
    block_sync();

    // -- issue the loads of chunk tile jj into ring buffer jj % kBufs
    auto issue = [&](int jj) {
      int start, len;
      bool cmp;
      st.tile(cbase + jj, start, len, cmp);
      const int buf = jj % kBufs;
      const int64_t *er = &sm.erow[jj * kTile];
      if (!FP8 || !cmp) {
        const uint8_t *kb = cmp ? p.k_cmp : p.k_raw;
        const uint8_t *vb = cmp ? p.v_cmp : p.v_raw;
#pragma unroll
        for (int n0 = 0; n0 < C::kOps; ++n0) {
          const int n = wave + n0 * NW;
          const int which = n / (C::kKVInstr / 2);
          const int nn = n - which * (C::kKVInstr / 2);
          const int lin = nn * 1024 + lane * 16;
          const int r = lin / C::kRowB;
          const int cp = (lin % C::kRowB) / 16;
          const int c = cp ^ (r & (C::kChunks - 1));
          const int64_t e = er[r];
          const uint8_t *src = e >= 0 ? (which ? vb : kb) + e * C::kRowB + c * 16
                                      : kZeroRow + (lane & 15) * 16;
          dma16(src, &sm.kv[buf][which][nn * 1024]);
        }
      } else {
#pragma unroll
        for (int n0 = 0; n0 < C::kOps; ++n0) {
          const int n = wave + n0 * NW;
          if (n < C::kF8Instr) {
            const int which = n / (C::kF8Instr / 2);
            const int nn = n - which * (C::kF8Instr / 2);
            const int lin = nn * 1024 + lane * 16;
            const int r = lin / D;
            const int c = (lin % D) / 16;
            const int64_t e = er[r];
            const uint8_t *src = e >= 0 ? (which ? p.v_cmp : p.k_cmp) + e * D + c * 16
                                        : kZeroRow + (lane & 15) * 16;
            dma16(src, &sm.stage[FP8 ? buf : 0][which][nn * 1024]);
          } else {
            dma16(kZeroRow + (lane & 15) * 16, &sm.dummy[0]);   // keeps the count uniform
          }
        }
      }
    };

    const int pre = min(kBufs - 1, ct);
    for (int jj = 0; jj < pre; ++jj) issue(jj);

    for (int jj = 0; jj < ct; ++jj) {
      if (jj + kBufs - 1 < ct) issue(jj + kBufs - 1);
      const int ahead = min(kBufs - 1, ct - 1 - jj);   // tiles issued after jj
      if (ahead >= 2) wait_vmcnt<2 * C::kOps>();
      else if (ahead == 1) wait_vmcnt<C::kOps>();
      else wait_vmcnt<0>();
      block_sync();

      int start, len;
      bool cmp;
      st.tile(cbase + jj, start, len, cmp);
      const int buf = jj % kBufs;

      if (FP8 && cmp) {
        // widen the staged e4m3 rows to bf16 (exact) into the swizzled tile
        constexpr int kPieces = kTile * D / 8;   // 8-byte pieces per tile
        for (int idx = tid; idx < 2 * kPieces; idx += C::kThreads) {
          const int which = idx / kPieces;
          const int pidx = idx - which * kPieces;
          const int r = pidx / (D / 8);
          const int piece = pidx - r * (D / 8);
          const uint2 w = *(const uint2 *)&sm.stage[FP8 ? buf : 0][which][r * D + piece * 8];
          const f32x2 a0 = __builtin_amdgcn_cvt_pk_f32_fp8((int)w.x, false);
          const f32x2 a1 = __builtin_amdgcn_cvt_pk_f32_fp8((int)w.x, true);
          const f32x2 a2 = __builtin_amdgcn_cvt_pk_f32_fp8((int)w.y, false);
          const f32x2 a3 = __builtin_amdgcn_cvt_pk_f32_fp8((int)w.y, true);
          uint4 o;
          o.x = pack_bf16_hi(a0[0], a0[1]);
          o.y = pack_bf16_hi(a1[0], a1[1]);
          o.z = pack_bf16_hi(a2[0], a2[1]);
          o.w = pack_bf16_hi(a3[0], a3[1]);
          *(uint4 *)&sm.kv[buf][which][r * C::kRowB + ((piece ^ (r & (C::kChunks - 1))) * 16)] = o;
        }
        block_sync();
      }

      if (wave * 32 + hgrp * 128 < p.group) {
        const uint8_t *Kt = sm.kv[buf][0];
        const uint8_t *Vt = sm.kv[buf][1];
        // S^T = K . Q^T
        f32x16 s = f32x16{};
        {
          const int r = lane & 31;
#pragma unroll
          for (int kk = 0; kk < D / 16; ++kk) {
            const int c = 2 * kk + hi;
            const bf16x8 a = *(const bf16x8 *)(Kt + r * C::kRowB + ((c ^ (r & (C::kChunks - 1))) * 16));
            s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[kk], s, 0, 0, 0);
          }
        }
        // scale, mask, online softmax
        const float *tks = &sm.ks[jj * kTile];
        const float *tvs = &sm.vs[jj * kTile];
        float x[16];
        float tmax = -INFINITY;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int r = 8 * (i >> 2) + 4 * hi + (i & 3);
          float v = s[i] * p.scale_log2;
          if (FP8 && cmp) v *= tks[r];
          x[i] = r < len ? v : -INFINITY;
          tmax = fmaxf(tmax, x[i]);
        }
        tmax = fmaxf(tmax, __shfl_xor(tmax, 32));
        const float m_new = fmaxf(m, tmax);
        const bool live = m_new != -INFINITY;
        const float alpha = live ? __builtin_amdgcn_exp2f(m - m_new) : 1.f;
        float psum = 0.f;
        float pr[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          pr[i] = live ? __builtin_amdgcn_exp2f(x[i] - m_new) : 0.f;
          psum += pr[i];
        }
        l = l * alpha + psum;
        m = m_new;
#pragma unroll
        for (int db = 0; db < D / 32; ++db) acc[db] *= alpha;
        if (FP8 && cmp) {
#pragma unroll
          for (int i = 0; i < 16; ++i) pr[i] *= tvs[8 * (i >> 2) + 4 * hi + (i & 3)];
        }
        bf16x8 pb[2];
#pragma unroll
        for (int k2 = 0; k2 < 2; ++k2)
#pragma unroll
          for (int j = 0; j < 8; ++j) pb[k2][j] = (__bf16)pr[8 * k2 + j];

        // O^T += V^T . P^T ; V^T from the transpose read of the row-major tile
        const int G = lane >> 4;
        const int L = lane & 15;
#pragma unroll
        for (int db = 0; db < D / 32; ++db) {
#pragma unroll
          for (int k2 = 0; k2 < 2; ++k2) {
            i16x4 part[2];
#pragma unroll
            for (int rr = 0; rr < 2; ++rr) {
              const int row = 16 * k2 + 8 * rr + 4 * (G >> 1) + (L >> 2);
              const int d = 32 * db + 16 * (G & 1) + 4 * (L & 3);
              const int off = row * C::kRowB + (((d >> 3) ^ (row & (C::kChunks - 1))) * 16) + (L & 1) * 8;
              part[rr] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t *)(Vt + off));
            }
            typedef short i16x8 __attribute__((ext_vector_type(8)));
            const i16x8 cat = {part[0][0], part[0][1], part[0][2], part[0][3],
                               part[1][0], part[1][1], part[1][2], part[1][3]};
            acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, cat), pb[k2],
                                                              acc[db], 0, 0, 0);
          }
        }
      }
      block_sync();   // ring buffer jj % kBufs may be refilled next
    }
  }

  // ---- epilogue
  const float lt = l + __shfl_xor(l, 32);
  if (!head_ok) return;
  const float inv = lt > 0.f ? 1.f / lt : 0.f;
  const float lse2 = (m == -INFINITY || !(lt > 0.f)) ? -INFINITY : m + __builtin_amdgcn_logf(lt);
  const float lse = lse2 == -INFINITY ? -INFINITY : lse2 * kLn2;
  if (S == 1) {
    uint16_t *orow = p.o + ((int64_t)qi * p.hq + h) * D;
#pragma unroll
    for (int db = 0; db < D / 32; ++db) {
#pragma unroll
      for (int i4 = 0; i4 < 4; ++i4) {
        const int d0 = 32 * db + 8 * i4 + 4 * hi;
        uint2 w;
        const __bf16 b0 = (__bf16)(acc[db][4 * i4 + 0] * inv);
        const __bf16 b1 = (__bf16)(acc[db][4 * i4 + 1] * inv);
        const __bf16 b2 = (__bf16)(acc[db][4 * i4 + 2] * inv);
        const __bf16 b3 = (__bf16)(acc[db][4 * i4 + 3] * inv);
        w.x = (uint32_t)__builtin_bit_cast(uint16_t, b0) | ((uint32_t)__builtin_bit_cast(uint16_t, b1) << 16);
        w.y = (uint32_t)__builtin_bit_cast(uint16_t, b2) | ((uint32_t)__builtin_bit_cast(uint16_t, b3) << 16);
        *(uint2 *)(orow + d0) = w;
      }
    }
    if (hi == 0 && p.lse) p.lse[(int64_t)qi * p.hq + h] = lse;
  } else {
    const int64_t prow = ((int64_t)split * p.num_queries + qi) * p.hq + h;
    float *orow = p.part_o + prow * D;
#pragma unroll
    for (int db = 0; db < D / 32; ++db) {
#pragma unroll
      for (int i4 = 0; i4 < 4; ++i4) {
        const int d0 = 32 * db + 8 * i4 + 4 * hi;
        float4 w = make_float4(acc[db][4 * i4] * inv, acc[db][4 * i4 + 1] * inv,
                               acc[db][4 * i4 + 2] * inv, acc[db][4 * i4 + 3] * inv);
        *(float4 *)(orow + d0) = w;
      }
    }
    if (hi == 0) p.part_lse[prow] = lse;
  }
}

template <int D, int NW, bool FP8>
hipError_t launch_t(const Params &p, hipStream_t stream) {
  dim3 grid((unsigned)p.num_queries * (unsigned)p.num_splits, (unsigned)(p.hkv * p.head_groups));
  hipLaunchKernelGGL((attn_fwd_kernel<D, NW, FP8>), grid, dim3(NW * 64), 0, stream, p);
  return hipGetLastError();
}

template <int D, bool FP8>
hipError_t launch_d(const Params &p, hipStream_t stream) {
  const int heads = p.group < 128 ? p.group : 128;
  if (heads <= 32) return launch_t<D, 1, FP8>(p, stream);
  if (heads <= 64) return launch_t<D, 2, FP8>(p, stream);
  return launch_t<D, 4, FP8>(p, stream);
}

}  // namespace

hipError_t launch_attention(const Params &p, hipStream_t stream) {
  if (p.num_queries == 0) return hipSuccess;
  if (p.head_dim == 64) return p.cmp_fp8 ? launch_d<64, true>(p, stream) : launch_d<64, false>(p, stream);
  return p.cmp_fp8 ? launch_d<128, true>(p, stream) : launch_d<128, false>(p, stream);
}

}  // namespace spa
