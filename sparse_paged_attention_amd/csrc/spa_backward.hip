// Backward of sparse paged attention with a sink, for gfx950 (bf16 caches,
// D 128).
//
// The forward keeps its log-sum-exp for a backward pass (RL-Kernel PR
// "Roadmap item 24: joint compressed/window attention with sink", section
// "Reuse and arithmetic").  The pages give no formulas for it; these are
// the derivative of the forward definition.  For one query head with KV set
// rows j, scores s_j = scale <q, k_j>, p_j = exp(s_j - LSE) and upstream
// gradient dO:
//   dp_j = <dO, v_j>,  Delta = <dO, O>,  ds_j = p_j (dp_j - Delta)
//   dq = scale sum_j ds_j k_j,  dk_j += scale ds_j q,  dv_j += p_j dO
//   dsink += -exp(sink - LSE) Delta
// O and LSE are the forward's outputs; P is recomputed from LSE, so there
// is no running max.
//
// One workgroup per (query, KV head, block of 64 query heads) with two
// waves of 32 query heads, or, for a prefill call whose lists are short
// enough, per (query pair, KV head, 64-head block) with four waves (query x
// head half).  A pair streams the union of its two KV sets (per-query
// bitmaps of the listed groups, then the window positions from the lower
// window start to the higher query position), each row flagged with the
// queries that read it; pairs across sequences, or lists that name a group
// twice, stream the two lists one after the other.  Rows are translated
// through the page tables (the forward's device functions) into an LDS list
// and streamed as 32-row K and V tiles through two LDS stages with direct
// global->LDS loads.  Per tile and wave, on v_mfma_f32_32x32x16_bf16:
//   S^T = K.Q^T and dP^T = V.dO^T (a lane per head): P, dS per head column;
//   S = Q.K^T and dP = dO.V^T (a lane per KV row): P, dS per row column;
//   dQ^T += K^T.dS^T      (K^T by transposing LDS reads, as the forward's V^T)
//   dV = P.dO, dK = dS.Q  over every wave's heads (both queries of a pair),
//                          for a share of the head dimensions per wave (P
//                          and dS swapped through LDS; dO and Q are LDS
//                          tiles too, read transposed the same way)
// Computing the scores in both orientations costs two extra MFMA products per
// tile but puts each of P and dS in the register layout its consumer needs,
// with no LDS round trip.  dK and dV rows are added to the fp32 gradient
// caches with float atomics, once per workgroup and element (so a row both
// queries of a pair read is added once): a lane per head dimension, so each
// atomic instruction covers 128 contiguous bytes of two rows.  dQ is written once
// (fp32).  The sink gradient is written per (query, head) and summed over
// the queries by sink_reduce_kernel, in a fixed order.
//
// With a workspace for it, a prefill call instead forms dK and dV in the
// KV-block pass further down (rows summed over the queries that read them
// before one atomic add per block and query slice), and the kernel above
// runs without its dK and dV part.

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdint>

#include "spa_device.h"
#include "spa_kernel_util.h"

namespace spa {
namespace {

constexpr int kD = 128;
constexpr int kRowB = 2 * kD;              // bf16 row bytes
constexpr int kChunks = kRowB / 16;        // 16-byte chunks per row
constexpr int kPT = 32;                    // KV rows per tile
constexpr int kTileB = kPT * kRowB;
constexpr int kBRows = 512;                // rows translated per chunk (one query per workgroup)
constexpr int kPairRows = kPairRowsMax;    // rows of a query pair's list (one chunk)
constexpr int kBmWords = 1024;             // bitmap words per query: groups < 32768
// K and V tile stages: two with the dK and dV part (its atomics share the
// load counter); three without it, two tiles' loads in flight and two
// workgroups per CU, so one's setup runs under the other's tiles
template <bool DKV>
constexpr int kBStages = DKV ? 2 : 3;
constexpr int64_t kCmpBit = int64_t(1) << 62;

// NQ queries per workgroup (1, or 2 for a prefill query pair); 2 NQ waves,
// wave w = query (w / 2) x head half (w % 2).  DKV: the workgroup also forms
// dK and dV (Q, dO, P and dS exchanged through LDS); without it only dQ.
template <int NQ, bool DKV>
struct BwdSmem {
  static constexpr int kRows = NQ == 1 ? kBRows : kPairRows;
  union {
    struct {
      alignas(16) uint8_t k[kBStages<DKV>][kTileB];
      alignas(16) uint8_t v[kBStages<DKV>][kTileB];
    } t;
    uint32_t bm[2][kBmWords];              // query pair setup: each query's selected groups
  } u;
  static constexpr int kX = DKV ? 2 * NQ : 1;
  alignas(16) uint8_t q[kX][DKV ? kTileB : 16];   // wave w: its query's 32 heads as tile rows
  alignas(16) uint8_t dO[kX][DKV ? kTileB : 16];
  alignas(16) int64_t row[kRows];          // row * Hkv + g (bit 62: compressed), -1: masked
  uint8_t flg[NQ == 1 ? 1 : kRows];        // query pair: bit q = in query q's set
  alignas(16) bf16x8 xp[kX][2][DKV ? 64 : 1];   // P and dS of each wave's heads, A-fragment order
  alignas(16) bf16x8 xd[kX][2][DKV ? 64 : 1];
  alignas(16) float lse2[NQ * 64];         // LSE * log2(e); +inf: no softmax (no rows, not a head)
  alignas(16) float delta[NQ * 64];
  int32_t wsum[2 * NQ];
  int32_t dup;                             // a pair's list names a group twice
};
static_assert(sizeof(BwdSmem<2, true>::u) >= 2 * kBmWords * 4, "bitmaps fit the tile stages");

// A K^T, V^T, Q^T or dO^T fragment of a tile in LDS (transposing reads):
// as the A operand, lane L holds column d = 32 db + L % 32 and the tile rows
// of k-chunk k2 in the order the S^T accumulator lists its rows.
__device__ __forceinline__ bf16x8 tr_frag(const uint8_t *T, int lane, int db, int k2) {
  const int G = lane >> 4;
  const int L = lane & 15;
  i16x4 f[2];
#pragma unroll
  for (int rr = 0; rr < 2; ++rr) {
    const int row = 16 * k2 + 8 * rr + 4 * (G >> 1) + (L >> 2);
    const int d = 32 * db + 16 * (G & 1) + 4 * (L & 3);
    const int off = row * kRowB + (((d >> 3) ^ swz<kChunks>(row)) * 16) + (L & 1) * 8;
    f[rr] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t *)(T + off));
  }
  const i16x8 cat = {f[0][0], f[0][1], f[0][2], f[0][3], f[1][0], f[1][1], f[1][2], f[1][3]};
  return __builtin_bit_cast(bf16x8, cat);
}

// Row fragment (natural layout): lane L holds row L % 32, chunk 2 kk + L / 32.
__device__ __forceinline__ bf16x8 row_frag(const uint8_t *T, int lane, int kk) {
  const int r = lane & 31;
  const int c = 2 * kk + (lane >> 5);
  return *(const bf16x8 *)(T + r * kRowB + ((c ^ swz<kChunks>(r)) * 16));
}

// The row list of a query pair (queries i0, i1 of the same prefill call):
// the union of their KV sets when both sit in one sequence (compressed
// groups in ascending id order from per-query bitmaps, then the window
// positions from the lower window start to the higher query position),
// else their two canonical lists one after the other.  Each row carries
// bit q for membership in query q's set.  Returns the number of rows; the
// list is padded with masked rows to a whole tile.
template <int NT, class Smem>
__device__ int32_t pair_rows(const Params &p, Smem &sm, int32_t i0, int32_t i1, bool has1, const QueryKV &kv0,
                             const QueryKV &kv1, int32_t g) {
  const int tid = threadIdx.x;
  constexpr int kIters = Smem::kRows / NT;
  const int32_t U0 = kv0.n_sel + kv0.win_len, U1 = has1 ? kv1.n_sel + kv1.win_len : 0;
  const int32_t wlo = min(kv0.win_len > 0 ? kv0.win_lo : INT32_MAX, kv1.win_len > 0 ? kv1.win_lo : INT32_MAX);
  const int32_t whi = max(kv0.win_len > 0 ? kv0.t : -1, kv1.win_len > 0 ? kv1.t : -1);
  const int32_t wrange = whi >= wlo ? whi - wlo + 1 : 0;
  bool uni = has1 && U0 > 0 && U1 > 0 && kv0.b == kv1.b && kv0.n_c <= 32 * kBmWords && kv1.n_c <= 32 * kBmWords &&
             kv0.n_sel + kv1.n_sel + wrange <= Smem::kRows;
  int32_t U = 0, ncu = 0;
  if (uni) {
    // ---- bitmaps of the two lists (a repeated id falls back to the
    // concatenation, which counts it twice as the single-query path does)
    for (int w = tid; w < 2 * kBmWords; w += NT) sm.u.bm[w / kBmWords][w % kBmWords] = 0u;
    if (tid == 0) sm.dup = 0;
    __syncthreads();
    for (int32_t e = tid; e < kv0.n_sel + kv1.n_sel; e += NT) {
      const int q = e < kv0.n_sel ? 0 : 1;
      const QueryKV &kv = q ? kv1 : kv0;
      const int32_t c = check_cmp_id(p, kv, p.cmp_idx[(int64_t)(q ? i1 : i0) * p.topk + (q ? e - kv0.n_sel : e)]);
      if (c >= 0) {
        const uint32_t bit = 1u << (c & 31);
        if (atomicOr(&sm.u.bm[q][c >> 5], bit) & bit) sm.dup = 1;
      }
    }
    __syncthreads();
    uni = sm.dup == 0;
    if (uni) {
      // ---- ranks: four bitmap words per thread, in id order
      constexpr int kWpt = kBmWords / NT;
      uint32_t wd[kWpt];
      int32_t own = 0;
#pragma unroll
      for (int k = 0; k < kWpt; ++k) {
        wd[k] = sm.u.bm[0][tid * kWpt + k] | sm.u.bm[1][tid * kWpt + k];
        own += __popc(wd[k]);
      }
      int32_t pre = block_excl_scan<NT>(own, ncu, sm.wsum);
#pragma unroll
      for (int k = 0; k < kWpt; ++k) {
        const int w = tid * kWpt + k;
        uint32_t bits = wd[k];
        while (bits) {
          const int b = __ffs(bits) - 1;
          bits &= bits - 1;
          const int32_t c = 32 * w + b;
          sm.row[pre] = c;
          sm.flg[pre] = (uint8_t)(((sm.u.bm[0][w] >> b) & 1u) | (((sm.u.bm[1][w] >> b) & 1u) << 1));
          ++pre;
        }
      }
      U = ncu + wrange;
      __syncthreads();                       // every logical id and flag is in; the bitmaps are dead
      // ---- window positions and the translation of every row
#pragma unroll
      for (int it = 0; it < kIters; ++it) {
        const int32_t r = tid + it * NT;
        if (r < (U + kPT - 1) / kPT * kPT) {
          int64_t er = -1;
          uint8_t f = 0;
          if (r < ncu) {
            f = sm.flg[r];
            const int64_t pr = logical_row(p, kv0, true, (int32_t)sm.row[r]);
            if (pr >= 0) er = (pr * p.hkv + g) | kCmpBit;
          } else if (r < U) {
            const int32_t x = wlo + (r - ncu);
            f = (uint8_t)((kv0.win_len > 0 && x >= kv0.win_lo && x <= kv0.t ? 1u : 0u) |
                          (kv1.win_len > 0 && x >= kv1.win_lo && x <= kv1.t ? 2u : 0u));
            const int64_t pr = f ? logical_row(p, kv0, false, x) : -1;
            if (pr >= 0) er = pr * p.hkv + g;
          }
          sm.row[r] = er;
          sm.flg[r] = er >= 0 ? f : 0;
        }
      }
    }
  }
  if (!uni) {
    // ---- concatenation: query 0's canonical rows, then query 1's
    U = U0 + U1;
#pragma unroll
    for (int it = 0; it < kIters; ++it) {
      const int32_t r = tid + it * NT;
      if (r < (U + kPT - 1) / kPT * kPT) {
        int64_t er = -1;
        uint8_t f = 0;
        if (r < U) {
          const int q = r < U0 ? 0 : 1;
          const QueryKV &kv = q ? kv1 : kv0;
          const int32_t e = q ? r - U0 : r;
          const bool cmp = e < kv.n_sel;
          const int64_t pr = logical_row(p, kv, cmp, entry_logical(p, kv, q ? i1 : i0, e));
          if (pr >= 0) er = (pr * p.hkv + g) | (cmp ? kCmpBit : 0);
          f = (uint8_t)(1u << q);
        }
        sm.row[r] = er;
        sm.flg[r] = er >= 0 ? f : 0;
      }
    }
  }
  return U;
}

template <int NQ, bool DKV>
__global__ __launch_bounds__(128 * NQ, DKV ? 1 : 2) void attn_bwd_kernel(Params p, BwdParams b) {
  constexpr int NT = 128 * NQ;
  constexpr int NW = 2 * NQ;                 // waves
  constexpr int kRowsPerWave = kPT / NW;     // tile rows each wave loads
  __shared__ BwdSmem<NQ, DKV> sm;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int qw = wave >> 1;                  // the wave's query (0 with one query per workgroup)
  const int hw = wave & 1;                   // the wave's head half
  const int hi = lane >> 5;
  const int hblocks = (p.group + 63) / 64;
  // heaviest jobs (the last queries of a prefill) first
  const int64_t job = (int64_t)gridDim.x - 1 - blockIdx.x;
  const int hb = (int)(job % hblocks);
  const int64_t u = job / hblocks;
  const int g = (int)(u % p.hkv);
  const int32_t i0 = (int32_t)(u / p.hkv) * NQ;
  const int32_t i1 = i0 + 1;
  const bool has1 = NQ == 2 && i1 < p.num_queries;
  const QueryKV kv0 = query_kv(p, i0);
  const QueryKV kv1 = has1 ? query_kv(p, i1) : QueryKV{0, 0, 0, 0, 0, 0};
  const int32_t iq = qw ? i1 : i0;
  const bool qvalid = qw == 0 || has1;

  // ---- Q and dO of the wave's heads: LDS tiles (rows = heads) and the
  // natural B fragments in registers
  const int h0 = hb * 64 + hw * 32;                   // first head of the wave, within the group
  const int64_t qbase = (int64_t)iq * p.hq + (int64_t)g * p.group;
#pragma unroll
  for (int n = 0; n < 8; ++n) {
    const int idx = n * 64 + lane;
    const int r = idx >> 4, c = idx & 15;
    const bool ok = qvalid && h0 + r < p.group;
    const int64_t off = (qbase + h0 + r) * kD + c * 8;
    if constexpr (DKV) {
      const uint4 qv = ok ? *(const uint4 *)(p.q + off) : uint4{0, 0, 0, 0};
      const uint4 ov = ok ? *(const uint4 *)(b.d_o + off) : uint4{0, 0, 0, 0};
      const int dst = r * kRowB + ((c ^ swz<kChunks>(r)) * 16);
      *(uint4 *)(sm.q[wave] + dst) = qv;
      *(uint4 *)(sm.dO[wave] + dst) = ov;
    }
  }
  const int hl = h0 + (lane & 31);                    // this lane's head (head-column layouts)
  const bool hvalid = qvalid && hl < p.group;
  bf16x8 qf[kD / 16], dof[kD / 16];
  {
    const int64_t off = (qbase + hl) * kD + 8 * hi;
#pragma unroll
    for (int kk = 0; kk < kD / 16; ++kk) {
      qf[kk] = hvalid ? *(const bf16x8 *)(p.q + off + 16 * kk) : bf16x8{};
      dof[kk] = hvalid ? *(const bf16x8 *)(b.d_o + off + 16 * kk) : bf16x8{};
    }
  }
  // Delta = <dO, O> of the lane's head (each half of the wave sums 64 of
  // the D products) and the head's LSE
  const int hslot = qw * 64 + hw * 32 + (lane & 31);  // the head's slot in lse2 / delta
  {
    float dsum = 0.f;
    if (hvalid) {
      const int64_t off = (qbase + hl) * kD + 64 * hi;
#pragma unroll
      for (int c = 0; c < 8; ++c) {
        const uint4 ov = *(const uint4 *)(b.o + off + 8 * c);
        const uint4 gv = *(const uint4 *)(b.d_o + off + 8 * c);
        const uint32_t ow[4] = {ov.x, ov.y, ov.z, ov.w};
        const uint32_t gw[4] = {gv.x, gv.y, gv.z, gv.w};
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          dsum = __builtin_fmaf(__builtin_bit_cast(float, ow[w] << 16), __builtin_bit_cast(float, gw[w] << 16), dsum);
          dsum = __builtin_fmaf(__builtin_bit_cast(float, ow[w] & 0xFFFF0000u),
                                __builtin_bit_cast(float, gw[w] & 0xFFFF0000u), dsum);
        }
      }
    }
    dsum += __shfl_xor(dsum, 32);
    if (hi == 0) {
      const float lse = hvalid ? b.lse[qbase + hl] : INFINITY;
      const bool live = hvalid && lse != -INFINITY;
      sm.lse2[hslot] = live ? lse * kLog2e : INFINITY;
      sm.delta[hslot] = live ? dsum : 0.f;
      // for the KV-block pass: every head slot of the padded group, the
      // heads past the group as +inf / 0
      if (b.lse2_ws != nullptr && qvalid && hl < b.gp) {
        const int64_t wi = ((int64_t)iq * p.hkv + g) * b.gp + hl;
        b.lse2_ws[wi] = live ? lse * kLog2e : INFINITY;
        b.delta_ws[wi] = live ? dsum : 0.f;
      }
      if (hvalid && b.dsink_part != nullptr) {
        const float part = (live && p.sink != nullptr) ? -__expf(p.sink[g * p.group + hl] - lse) * dsum : 0.f;
        b.dsink_part[qbase + hl] = part;
      }
    }
  }
  __syncthreads();
  const float my_lse2 = sm.lse2[hslot];
  const float my_delta = sm.delta[hslot];

  f32x16 dqa[kD / 32];
#pragma unroll
  for (int db = 0; db < kD / 32; ++db) dqa[db] = f32x16{};

  const uint8_t *const kraw = in_sgpr(p.k_raw), *const vraw = in_sgpr(p.v_raw);
  const uint8_t *const kcmp = in_sgpr(p.k_cmp), *const vcmp = in_sgpr(p.v_cmp);
  float *const dk_raw = in_sgpr(b.dk_raw), *const dv_raw = in_sgpr(b.dv_raw);
  float *const dk_cmp = in_sgpr(b.dk_cmp), *const dv_cmp = in_sgpr(b.dv_cmp);
  const float sl2 = p.scale_log2;
  const float scale = b.scale;
  // tile loads: wave w moves rows kRowsPerWave w .. (four per direct load);
  // lane L's chunk in load n is logical chunk (L % 16) ^ swz(row), row =
  // kRowsPerWave w + 4n + L / 16
  int32_t csrc[kRowsPerWave / 4];
#pragma unroll
  for (int n = 0; n < kRowsPerWave / 4; ++n) {
    const int r = kRowsPerWave * wave + 4 * n + lane / kChunks;
    csrc[n] = ((lane % kChunks) ^ swz<kChunks>(r)) * 16;
  }

  // the list: one query's rows in chunks, or a query pair's rows at once
  const int32_t Utot = NQ == 1 ? kv0.n_sel + kv0.win_len : 0;
  int32_t c0 = 0;
  bool more = true;
  while (more) {
    int32_t n;
    if constexpr (NQ == 1) {
      n = min(kBRows, Utot - c0);
      more = c0 + n < Utot;
      if (n <= 0) break;
      constexpr int kIters = kBRows / NT;
      int32_t xs[kIters];
#pragma unroll
      for (int it = 0; it < kIters; ++it) {
        const int32_t e = c0 + tid + it * NT;
        xs[it] = e < c0 + n ? entry_logical(p, kv0, i0, e) : -1;
      }
#pragma unroll
      for (int it = 0; it < kIters; ++it) {
        const int32_t r = tid + it * NT;
        if (r < (n + kPT - 1) / kPT * kPT) {
          const int32_t e = c0 + r;
          int64_t er = -1;
          if (r < n) {
            const bool cmp = e < kv0.n_sel;
            const int64_t pr = logical_row(p, kv0, cmp, xs[it]);
            if (pr >= 0) er = (pr * p.hkv + g) | (cmp ? kCmpBit : 0);
          }
          sm.row[r] = er;
        }
      }
      c0 += n;
    } else {
      n = pair_rows<NT>(p, sm, i0, i1, has1, kv0, kv1, g);
      more = false;
      if (n <= 0) break;
    }
    __syncthreads();
    const int32_t ntiles = (n + kPT - 1) / kPT;

    auto issue = [&](int j) {
      const int st = j % kBStages<DKV>;
      // every row first: the loads' memory clobber keeps a later LDS read
      // from starting ahead of them
      int64_t ers[kRowsPerWave / 4];
#pragma unroll
      for (int q4 = 0; q4 < kRowsPerWave / 4; ++q4) ers[q4] = sm.row[kPT * j + kRowsPerWave * wave + 4 * q4 + lane / kChunks];
#pragma unroll
      for (int q4 = 0; q4 < kRowsPerWave / 4; ++q4) {
        const int rr = kRowsPerWave * wave + 4 * q4;
        const int64_t er = ers[q4];
        const bool cmp = (er & kCmpBit) != 0;
        const int64_t off = (er & ~kCmpBit) * kRowB + csrc[q4];
        dma16(er >= 0 ? (cmp ? kcmp : kraw) + off : kZeroRow + csrc[q4], sm.u.t.k[st] + rr * kRowB);
        dma16(er >= 0 ? (cmp ? vcmp : vraw) + off : kZeroRow + csrc[q4], sm.u.t.v[st] + rr * kRowB);
      }
    };
    // a row of the list is in this wave's query's set
    auto in_set = [&](int r) -> bool {
      if constexpr (NQ == 1) return sm.row[r] >= 0;
      else return ((sm.flg[r] >> qw) & 1u) != 0;
    };

    constexpr int NS = kBStages<DKV>;
    constexpr int kLoads = 2 * (kRowsPerWave / 4);   // this wave's direct loads per tile
    for (int t = 0; t < NS - 1 && t < ntiles; ++t) issue(t);
    for (int j = 0; j < ntiles; ++j) {
      // tile j is in (this wave's loads, then everyone's), and every wave is
      // done with tile j-1, whose stage the next loads refill.  With dK and
      // dV the wait also covers the previous tile's atomics; without, the
      // loads of the tiles after j stay in flight
      if constexpr (DKV) {
        wait_vmcnt<0>();
      } else {
        const int pending = min(NS - 2, ntiles - 1 - j);
        if (pending >= 4) wait_vmcnt<4 * kLoads>();
        else if (pending == 3) wait_vmcnt<3 * kLoads>();
        else if (pending == 2) wait_vmcnt<2 * kLoads>();
        else if (pending == 1) wait_vmcnt<kLoads>();
        else wait_vmcnt<0>();
      }
      block_sync();
      if (j + NS - 1 < ntiles) issue(j + NS - 1);
      const int st = j % NS;
      const uint8_t *Kt = sm.u.t.k[st];
      const uint8_t *Vt = sm.u.t.v[st];
      const bool lvalid = in_set(kPT * j + (lane & 31));
      const uint32_t tm = (uint32_t)__ballot(lane < 32 && lvalid);

      // scores and dP in both orientations (without dK and dV, the head-
      // column ones only)
      f32x16 s_rh = f32x16{}, s_hr = f32x16{}, dp_rh = f32x16{}, dp_hr = f32x16{};
      bf16x8 ktf[kD / 32][2];                // K^T fragments of dQ^T += K^T dS^T
      if constexpr (DKV) {
#pragma unroll
        for (int kk = 0; kk < kD / 16; ++kk) {
          const bf16x8 kf = row_frag(Kt, lane, kk);
          s_rh = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[kk], s_rh, 0, 0, 0);
          s_hr = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qf[kk], kf, s_hr, 0, 0, 0);
        }
#pragma unroll
        for (int kk = 0; kk < kD / 16; ++kk) {
          const bf16x8 vf = row_frag(Vt, lane, kk);
          dp_rh = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, dof[kk], dp_rh, 0, 0, 0);
          dp_hr = __builtin_amdgcn_mfma_f32_32x32x16_bf16(dof[kk], vf, dp_hr, 0, 0, 0);
        }
#pragma unroll
        for (int db = 0; db < kD / 32; ++db)
#pragma unroll
          for (int k2 = 0; k2 < 2; ++k2) ktf[db][k2] = tr_frag(Kt, lane, db, k2);
      } else {
        // two workgroups share each CU, so one's fragment reads run under
        // the other's products; S and dP alternate
#pragma unroll
        for (int kk = 0; kk < kD / 16; ++kk) {
          s_rh = __builtin_amdgcn_mfma_f32_32x32x16_bf16(row_frag(Kt, lane, kk), qf[kk], s_rh, 0, 0, 0);
          dp_rh = __builtin_amdgcn_mfma_f32_32x32x16_bf16(row_frag(Vt, lane, kk), dof[kk], dp_rh, 0, 0, 0);
        }
#pragma unroll
        for (int db = 0; db < kD / 32; ++db)
#pragma unroll
          for (int k2 = 0; k2 < 2; ++k2) ktf[db][k2] = tr_frag(Kt, lane, db, k2);
      }
      // head-column layout: value r is row 8(r/4) + 4hi + r%4 of the tile
      bf16x8 dsb[2];
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = 8 * (r >> 2) + 4 * hi + (r & 3);
        const float pr = ((tm >> row) & 1u) ? __builtin_amdgcn_exp2f(__builtin_fmaf(s_rh[r], sl2, -my_lse2)) : 0.f;
        dsb[r >> 3][r & 7] = (__bf16)(pr * (dp_rh[r] - my_delta));
      }
      // dQ^T += K^T . dS^T
#pragma unroll
      for (int db = 0; db < kD / 32; ++db)
#pragma unroll
        for (int k2 = 0; k2 < 2; ++k2)
          dqa[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ktf[db][k2], dsb[k2], dqa[db], 0, 0, 0);
      if constexpr (!DKV) continue;
      // row-column layout: value r is head 8(r/4) + 4hi + r%4 of the wave
      bf16x8 pb[2], dsh[2];
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const float4 l4 = *(const float4 *)(&sm.lse2[qw * 64 + hw * 32 + 8 * q4 + 4 * hi]);
        const float4 d4 = *(const float4 *)(&sm.delta[qw * 64 + hw * 32 + 8 * q4 + 4 * hi]);
        const float lv[4] = {l4.x, l4.y, l4.z, l4.w};
        const float dv[4] = {d4.x, d4.y, d4.z, d4.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int r = 4 * q4 + e;
          const float pr = lvalid ? __builtin_amdgcn_exp2f(__builtin_fmaf(s_hr[r], sl2, -lv[e])) : 0.f;
          pb[r >> 3][r & 7] = (__bf16)pr;
          dsh[r >> 3][r & 7] = (__bf16)(pr * (dp_hr[r] - dv[e]));
        }
      }
      // dV = P . dO and dK = scale dS . Q for the tile's rows over every
      // wave's heads (both queries of a pair): the waves swap their P and dS
      // fragments through LDS and split the head dimensions, so each gradient
      // element is added once per workgroup.  Value r is row 8(r/4) + 4hi +
      // r%4, lane column d.
#pragma unroll
      for (int k2 = 0; k2 < 2; ++k2) {
        sm.xp[wave][k2][lane] = pb[k2];
        sm.xd[wave][k2][lane] = dsh[k2];
      }
      int64_t er[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) er[r] = sm.row[kPT * j + 8 * (r >> 2) + 4 * hi + (r & 3)];
      block_sync();
#pragma unroll
      for (int dbi = 0; dbi < 4 / NW; ++dbi) {
        const int db = (4 / NW) * wave + dbi;
        f32x16 av = f32x16{}, ak = f32x16{};
#pragma unroll
        for (int kc = 0; kc < 2 * NW; ++kc) {
          const int w2 = kc >> 1, k2 = kc & 1;
          av = __builtin_amdgcn_mfma_f32_32x32x16_bf16(sm.xp[w2][k2][lane], tr_frag(sm.dO[w2], lane, db, k2), av, 0,
                                                       0, 0);
          ak = __builtin_amdgcn_mfma_f32_32x32x16_bf16(sm.xd[w2][k2][lane], tr_frag(sm.q[w2], lane, db, k2), ak, 0,
                                                       0, 0);
        }
        const int d = 32 * db + (lane & 31);
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          if (er[r] >= 0) {
            const bool cmp = (er[r] & kCmpBit) != 0;
            const int64_t off = (er[r] & ~kCmpBit) * kD + d;
            unsafeAtomicAdd((cmp ? dv_cmp : dv_raw) + off, av[r]);
            unsafeAtomicAdd((cmp ? dk_cmp : dk_raw) + off, ak[r] * scale);
          }
        }
      }
    }
    wait_vmcnt<0>();
    __syncthreads();                         // the row list is rewritten by the next chunk
  }

  // ---- dQ = scale dQ^T^T: lane column = head, value r = d 32db + 8(r/4) + 4hi + r%4
  if (hvalid) {
    float *dq = b.dq + (qbase + hl) * kD;
#pragma unroll
    for (int db = 0; db < kD / 32; ++db)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const float4 v = {dqa[db][4 * q4] * scale, dqa[db][4 * q4 + 1] * scale, dqa[db][4 * q4 + 2] * scale,
                          dqa[db][4 * q4 + 3] * scale};
        *(float4 *)(dq + 32 * db + 8 * q4 + 4 * hi) = v;
      }
  }
}

// dsink[h] += sum over queries of part[i, h], one workgroup per head, in a
// fixed order (strided partial sums, then a tree).
__global__ __launch_bounds__(256) void sink_reduce_kernel(const float *part, int32_t nq, int32_t hq, float *dsink) {
  __shared__ float red[256];
  const int h = blockIdx.x;
  float s = 0.f;
  for (int32_t i = threadIdx.x; i < nq; i += 256) s += part[(int64_t)i * hq + h];
  red[threadIdx.x] = s;
  __syncthreads();
  for (int w = 128; w > 0; w >>= 1) {
    if ((int)threadIdx.x < w) red[threadIdx.x] += red[threadIdx.x + w];
    __syncthreads();
  }
  if (threadIdx.x == 0) dsink[h] += red[0];
}


// ---------------------------------------------------------------------------
// KV-block pass: dK and dV for blocks of 32 rows of one sequence's raw or
// compressed rows, summed in registers over every (query, 64-head chunk)
// that reads them and added to the gradient caches once per workgroup.
// The query-centric kernel above, without its dK and dV part, gives dQ,
// the sink partials, and each head's LSE log2(e) and Delta.
//
// A workgroup takes four consecutive blocks (one per wave, its K and V rows
// held as B fragments in registers) and a slice of 32 consecutive queries.
// The slice's queries that read any of the four blocks become items, each
// with a row mask per block: the window's rows, computed from the query's
// position; for a top-k layer the bitmap words of its listed groups
// (written once per query by bwd_bitmap_kernel); for an all-groups layer
// its complete groups.  A group a query lists again is a further item of
// its own (the extras list), so it counts once per listing, as in the
// forward.  The four waves share each item's Q and dO rows (64 heads) in
// a ring of four LDS buffers, three items' loads in flight; per item and
// wave, on the wave's own block:
//   S = Q.K^T, dP = dO.V^T (a lane per row, the item's heads in registers)
//   P = exp2(S scale log2 e - LSE log2 e) on the item's rows, dS = P (dP - Delta)
//   dV += P^T.dO, dK += dS^T.Q   (dO, Q by transposing LDS reads)
// Each wave then adds its block's dK and dV rows with float atomics.

constexpr int kKvQ = 32;                   // queries per workgroup
constexpr int kKvRing = 4;                 // item buffers
constexpr int kKvAhead = kKvRing - 1;      // items whose loads are in flight
constexpr int kKvLoads = 9;                // direct loads per wave and item

__device__ __forceinline__ int64_t quiet_row(const Params &p, int32_t b, bool cmp, int32_t x) {
  const int32_t P = p.page_size;
  const int32_t col = x / P;
  const int32_t stride = cmp ? p.cmp_pt_stride : p.raw_pt_stride;
  if (col >= stride) return -1;
  const int32_t page = (cmp ? p.cmp_pt : p.raw_pt)[(int64_t)b * stride + col];
  if (page < 0 || (int64_t)page >= (cmp ? p.cmp_pages : p.raw_pages)) return -1;
  return (int64_t)page * P + (x - col * P);
}

__global__ __launch_bounds__(64) void bwd_extras_zero_kernel(int32_t *n) {
  if (threadIdx.x == 0) *n = 0;
}

// Per query of a top-k layer: the bitmap words of its listed groups, and an
// extras entry (query, group) for each repeated listing.
__global__ __launch_bounds__(256) void bwd_bitmap_kernel(Params p, BwdKvPlan pl) {
  __shared__ uint32_t bm[kBmWords];
  const int tid = threadIdx.x;
  const int32_t i = blockIdx.x;
  const QueryKV kv = query_kv(p, i);
  const int32_t nw = min((kv.n_c + 31) >> 5, pl.nb_cmp);
  for (int32_t w = tid; w < pl.nb_cmp; w += 256) bm[w] = 0u;
  __syncthreads();
  for (int32_t e = tid; e < kv.n_sel; e += 256) {
    const int32_t c = check_cmp_id(p, kv, p.cmp_idx[(int64_t)i * p.topk + e]);
    if (c >= 0 && (c >> 5) < nw) {
      const uint32_t bit = 1u << (c & 31);
      if (atomicOr(&bm[c >> 5], bit) & bit) {
        const int32_t slot = atomicAdd(pl.n_extra, 1);
        if (slot < pl.cap_extra) pl.extra[slot] = make_int2(i, c);
      }
    }
  }
  __syncthreads();
  uint32_t *const words = pl.bitmap + (int64_t)i * pl.nb_cmp;
  for (int32_t w = tid; w < pl.nb_cmp; w += 256) words[w] = bm[w];
}

struct KvItem {
  int32_t q;
  uint32_t m[4];                           // row mask of each wave's block
};

struct KvBuf {
  alignas(16) uint8_t q[2][kTileB];        // the item's 64 heads as two 32-row tiles
  alignas(16) uint8_t dO[2][kTileB];
  alignas(16) uint8_t meta[4][1024];       // wave w's direct load: LSE log2(e) in meta[0], Delta in meta[1]
};

struct KvSmem {
  KvBuf buf[kKvRing];
  KvItem item[64];
  int64_t row[4][kPT];                     // physical row * Hkv + g, -1: no row
  int32_t n_items;
};

// The row mask of block kb (rows 32 kb .. 32 kb + 31) within [lo, hi].
__device__ __forceinline__ uint32_t span_mask(int32_t kb, int32_t lo, int32_t hi) {
  const int32_t a = max(lo - 32 * kb, 0), z = min(hi - 32 * kb, 31);
  if (z < a) return 0u;
  const uint32_t upto = z == 31 ? 0xFFFFFFFFu : (1u << (z + 1)) - 1u;
  return upto & ~((1u << a) - 1u);
}

__global__ __launch_bounds__(256) void attn_bwd_kv_kernel(Params p, BwdParams b, BwdKvPlan pl) {
  __shared__ KvSmem sm;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int hi = lane >> 5;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  // (query slice, KV head, block group): workgroup x runs on XCD x % 8, so
  // slice ch's workgroups all run on XCD ch % 8, one after another, and
  // read its Q and dO rows from that XCD's L2; compressed groups (the
  // longer lists) first within a slice
  const int64_t x = blockIdx.x;
  const int64_t m = x >> 3;
  const int g = (int)(m % p.hkv);
  const int64_t y = m / p.hkv;
  const int32_t ngt = p.num_seqs * (pl.ng_cmp + pl.ng_raw);
  const int32_t grp = (int32_t)(y % ngt);
  const int32_t ch = (int32_t)(8 * (y / ngt) + (x & 7));
  if (ch >= pl.nch) return;
  const int32_t ncg = p.num_seqs * pl.ng_cmp;
  const bool cmp = grp < ncg;
  const int32_t gi = cmp ? grp : grp - ncg;
  const int32_t ngk = cmp ? pl.ng_cmp : pl.ng_raw;
  const int32_t nbk = cmp ? pl.nb_cmp : pl.nb_raw;
  const int32_t sb = gi / ngk;
  const int32_t kb0 = 4 * (gi % ngk);
  const int32_t q0 = ch * kKvQ;
  const bool topk_cmp = cmp && p.topk > 0;
  const int32_t n_extra = topk_cmp ? min(*pl.n_extra, pl.cap_extra) : 0;
  const int rounds = 1 + (n_extra + 63) / 64;

  // the wave's block: rows and their K and V B fragments (lane L: row L % 32,
  // dimensions 16 s + 8 (L / 32) .. + 8)
  const int32_t kb = kb0 + wave;
  if (lane < kPT) {
    const int64_t pr = kb < nbk ? quiet_row(p, sb, cmp, 32 * kb + lane) : -1;
    sm.row[wave][lane] = pr >= 0 ? pr * p.hkv + g : -1;
  }
  __syncthreads();
  const int64_t my_row = sm.row[wave][lane & 31];
  const bool rvalid = my_row >= 0;
  const uint8_t *const kbase = cmp ? p.k_cmp : p.k_raw;
  const uint8_t *const vbase = cmp ? p.v_cmp : p.v_raw;
  bf16x8 kf[kD / 16], vf[kD / 16];
#pragma unroll
  for (int s2 = 0; s2 < kD / 16; ++s2) {
    const int64_t off = my_row * kRowB + (16 * s2 + 8 * hi) * 2;
    kf[s2] = rvalid ? *(const bf16x8 *)(kbase + off) : bf16x8{};
    vf[s2] = rvalid ? *(const bf16x8 *)(vbase + off) : bf16x8{};
  }

  f32x16 av[kD / 32], ak[kD / 32];
#pragma unroll
  for (int db = 0; db < kD / 32; ++db) {
    av[db] = f32x16{};
    ak[db] = f32x16{};
  }
  const int nhc = (p.group + 63) / 64;
  const float sl2 = p.scale_log2;
  bool any = false;

  for (int round = 0; round < rounds; ++round) {
    // ---- the round's items: round 0 the slice's queries, later rounds
    // the extras list 64 at a time (wave 0 builds the list)
    if (wave == 0) {
      KvItem it{0, {0u, 0u, 0u, 0u}};
      bool use = false;
      if (round == 0) {
        const int32_t i = q0 + lane;
        if (lane < kKvQ && i < p.num_queries) {
          const QueryKV kv = query_kv(p, i);
          it.q = i;
          if (kv.b == sb && (cmp ? kv.n_sel > 0 : kv.win_len > 0)) {
#pragma unroll
            for (int w = 0; w < 4; ++w) {
              const int32_t k2 = kb0 + w;
              uint32_t m = 0u;
              if (k2 < nbk) {
                if (!cmp) m = span_mask(k2, kv.win_lo, kv.t);
                else if (p.topk > 0) m = pl.bitmap[(int64_t)i * pl.nb_cmp + k2];
                else m = span_mask(k2, 0, kv.n_sel - 1);
              }
              it.m[w] = m;
            }
            use = (it.m[0] | it.m[1] | it.m[2] | it.m[3]) != 0u;
          }
        }
      } else {
        const int32_t xe = 64 * (round - 1) + lane;
        if (xe < n_extra) {
          const int2 ex = pl.extra[xe];
          const int32_t w = (ex.y >> 5) - kb0;
          if (ex.x >= q0 && ex.x < q0 + kKvQ && w >= 0 && w < 4 && p.query_seq[ex.x] == sb) {
            it.q = ex.x;
            it.m[w] = 1u << (ex.y & 31);
            use = true;
          }
        }
      }
      const unsigned long long bal = __ballot(use);
      if (use) sm.item[__builtin_amdgcn_mbcnt_hi((uint32_t)(bal >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)bal, 0u))] = it;
      if (lane == 0) sm.n_items = __builtin_popcountll(bal);
    }
    __syncthreads();
    const int32_t nt = sm.n_items * nhc;
    if (nt == 0) {
      __syncthreads();                       // the list is rebuilt next round
      continue;
    }
    any = true;

    // item f -> slot f % 4: wave w moves tile rows 16 n + 4 w .. + 3 of Q
    // and dO (n = 0..3) and its meta row
    auto issue = [&](int32_t f) {
      const int32_t k = f / nhc;
      const int hc = f - k * nhc;
      const int32_t q = sm.item[k].q;
      KvBuf &B = sm.buf[f % kKvRing];
      const int64_t hrow0 = (int64_t)q * p.hq + (int64_t)g * p.group + 64 * hc;
#pragma unroll
      for (int n = 0; n < 4; ++n) {
        const int R = 16 * n + 4 * wave + (lane >> 4);
        const int cs = ((lane & 15) ^ swz<kChunks>(R & 31)) * 16;
        const bool hv = 64 * hc + R < p.group;
        const int64_t off = (hrow0 + R) * kRowB + cs;
        dma16(hv ? (const uint8_t *)p.q + off : kZeroRow + cs, &B.q[0][0] + (16 * n + 4 * wave) * kRowB);
        dma16(hv ? (const uint8_t *)b.d_o + off : kZeroRow + cs, &B.dO[0][0] + (16 * n + 4 * wave) * kRowB);
      }
      const int64_t mrow = ((int64_t)q * p.hkv + g) * b.gp + 64 * hc;
      dma16(((wave & 1) ? b.delta_ws : b.lse2_ws) + mrow + 4 * (lane & 15), B.meta[wave]);
    };
    const int32_t pro = min(nt, kKvAhead);
    for (int32_t f = 0; f < pro; ++f) issue(f);
    for (int32_t j = 0; j < nt; ++j) {
      const int32_t pending = min(nt - 1 - j, kKvAhead - 1);
      if (pending >= 2) wait_vmcnt<2 * kKvLoads>();
      else if (pending == 1) wait_vmcnt<kKvLoads>();
      else wait_vmcnt<0>();
      block_sync();                          // item j is in; every wave is done with item j - 1
      if (j + kKvAhead < nt) issue(j + kKvAhead);
      const int32_t k = j / nhc;
      const int hc = j - k * nhc;
      const uint32_t mask = sm.item[k].m[wave];
      if (mask == 0u) continue;
      const KvBuf &B = sm.buf[j % kKvRing];
      const bool rin = rvalid && ((mask >> (lane & 31)) & 1u) != 0u;
      const float *const lsev = (const float *)B.meta[0];
      const float *const delv = (const float *)B.meta[1];
#pragma unroll
      for (int hb = 0; hb < 2; ++hb) {
        if (64 * hc + 32 * hb >= p.group) break;
        const uint8_t *Qt = B.q[hb];
        const uint8_t *Ot = B.dO[hb];
        // every fragment read is issued ahead of the products that use it
        bf16x8 qa[kD / 16], oa[kD / 16];
#pragma unroll
        for (int kk = 0; kk < kD / 16; ++kk) {
          qa[kk] = row_frag(Qt, lane, kk);
          oa[kk] = row_frag(Ot, lane, kk);
        }
        f32x16 sc = f32x16{}, dp = f32x16{};
#pragma unroll
        for (int kk = 0; kk < kD / 16; ++kk) {
          sc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qa[kk], kf[kk], sc, 0, 0, 0);
          dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(oa[kk], vf[kk], dp, 0, 0, 0);
        }
        bf16x8 ot[kD / 32][2], qt[kD / 32][2];
#pragma unroll
        for (int db = 0; db < kD / 32; ++db)
#pragma unroll
          for (int k2 = 0; k2 < 2; ++k2) {
            ot[db][k2] = tr_frag(Ot, lane, db, k2);
            qt[db][k2] = tr_frag(Qt, lane, db, k2);
          }
        // a lane per row; value r is head 32 hb + 8(r/4) + 4hi + r%4 of the chunk
        bf16x8 pa[2], da[2];
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          const float4 l4 = *(const float4 *)(lsev + 32 * hb + 8 * q4 + 4 * hi);
          const float4 d4 = *(const float4 *)(delv + 32 * hb + 8 * q4 + 4 * hi);
          const float lv[4] = {l4.x, l4.y, l4.z, l4.w};
          const float dv[4] = {d4.x, d4.y, d4.z, d4.w};
#pragma unroll
          for (int c = 0; c < 4; ++c) {
            const int r = 4 * q4 + c;
            const float pr = rin ? __builtin_amdgcn_exp2f(__builtin_fmaf(sc[r], sl2, -lv[c])) : 0.f;
            pa[r >> 3][r & 7] = (__bf16)pr;
            da[r >> 3][r & 7] = (__bf16)(rin ? pr * (dp[r] - dv[c]) : 0.f);   // rows outside the set may hold NaN
          }
        }
#pragma unroll
        for (int db = 0; db < kD / 32; ++db)
#pragma unroll
          for (int k2 = 0; k2 < 2; ++k2) {
            av[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(pa[k2], ot[db][k2], av[db], 0, 0, 0);
            ak[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(da[k2], qt[db][k2], ak[db], 0, 0, 0);
          }
        // issue order: the 16 fragment reads, the S and dP products with
        // the 32 transposing reads between them, then the rest
        __builtin_amdgcn_sched_group_barrier(0x100, 16, 0);
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
        }
      }
    }
    __syncthreads();                         // the item list and the buffers are rewritten next round
  }
  if (!any) return;

  // ---- the wave's block: value r is row 8(r/4) + 4hi + r%4, lane column
  // d = 32 db + L % 32
  float *const dv_out = cmp ? b.dv_cmp : b.dv_raw;
  float *const dk_out = cmp ? b.dk_cmp : b.dk_raw;
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int64_t er = sm.row[wave][8 * (r >> 2) + 4 * hi + (r & 3)];
    if (er >= 0) {
#pragma unroll
      for (int db = 0; db < kD / 32; ++db) {
        const int d = 32 * db + (lane & 31);
        unsafeAtomicAdd(dv_out + er * kD + d, av[db][r]);
        unsafeAtomicAdd(dk_out + er * kD + d, ak[db][r] * b.scale);
      }
    }
  }
}

}  // namespace

bool backward_eligible(const Params &p) { return p.head_dim == kD && !p.cmp_fp8; }

// query pairs: a prefill call whose pair lists fit one chunk, with a top-k
// list or no compressed part (an all-groups layer's lists can be long)
bool backward_pairs_eligible(const Params &p) {
  return p.query_seq != nullptr && p.query_pos != nullptr && (p.ratio == 0 || p.topk > 0) &&
         2 * ((int64_t)p.topk + p.window) <= kPairRows;
}

namespace {
struct KvSizes {
  int32_t nb_raw, nb_cmp, ng_raw, ng_cmp, nch, gp;
  bool bitmap;
};
KvSizes kv_sizes(const Params &p) {
  KvSizes z;
  z.nb_raw = (int32_t)(((int64_t)p.raw_pt_stride * p.page_size + 31) / 32);
  z.nb_cmp = p.ratio > 0 ? (int32_t)(((int64_t)p.cmp_pt_stride * p.page_size + 31) / 32) : 0;
  z.ng_raw = (z.nb_raw + 3) / 4;
  z.ng_cmp = (z.nb_cmp + 3) / 4;
  z.nch = (p.num_queries + kKvQ - 1) / kKvQ;
  z.gp = (p.group + 63) / 64 * 64;
  z.bitmap = p.ratio > 0 && p.topk > 0;
  return z;
}
size_t up256(size_t x) { return (x + 255) / 256 * 256; }
}  // namespace

bool backward_kv_eligible(const Params &p) {
  if (!backward_eligible(p) || p.query_seq == nullptr || p.query_pos == nullptr) return false;
  const KvSizes z = kv_sizes(p);
  return (!z.bitmap || z.nb_cmp <= kBmWords) &&
         (int64_t)p.num_seqs * (z.ng_raw + z.ng_cmp) * p.hkv * ((z.nch + 7) / 8 * 8) <= 0x7FFFFFFFLL;
}

size_t backward_kv_workspace(const Params &p, void *base, BwdKvPlan *pl, BwdParams *b) {
  const KvSizes z = kv_sizes(p);
  const size_t heads = (size_t)p.num_queries * p.hkv * z.gp;
  const size_t n_bm = z.bitmap ? (size_t)p.num_queries * z.nb_cmp : 0;
  const size_t cap_extra = z.bitmap ? (size_t)p.num_queries * p.topk : 0;
  size_t at = up256((size_t)p.num_queries * p.hq * sizeof(float));  // the sink partials
  const size_t o_lse = at;
  at += up256(heads * sizeof(float));
  const size_t o_delta = at;
  at += up256(heads * sizeof(float));
  const size_t o_bm = at;
  at += up256(n_bm * sizeof(uint32_t));
  const size_t o_n = at;
  at += 256;
  const size_t o_extra = at;
  at += up256(cap_extra * sizeof(int2));
  if (base != nullptr) {
    uint8_t *w = static_cast<uint8_t *>(base);
    pl->nb_raw = z.nb_raw;
    pl->nb_cmp = z.nb_cmp;
    pl->ng_raw = z.ng_raw;
    pl->ng_cmp = z.ng_cmp;
    pl->nch = z.nch;
    pl->bitmap = reinterpret_cast<uint32_t *>(w + o_bm);
    pl->n_extra = reinterpret_cast<int32_t *>(w + o_n);
    pl->extra = reinterpret_cast<int2 *>(w + o_extra);
    pl->cap_extra = (int32_t)std::min<size_t>(cap_extra, 0x7FFFFFFF);
    b->lse2_ws = reinterpret_cast<float *>(w + o_lse);
    b->delta_ws = reinterpret_cast<float *>(w + o_delta);
    b->gp = z.gp;
  }
  return at;
}

hipError_t launch_backward(const Params &p, const BwdParams &b, bool pairs, const BwdKvPlan *kv,
                           hipStream_t stream) {
  if (!backward_eligible(p) || (pairs && !backward_pairs_eligible(p))) return hipErrorInvalidValue;
  if (kv != nullptr && (!backward_kv_eligible(p) || b.lse2_ws == nullptr)) return hipErrorInvalidValue;
  if (p.num_queries == 0) return hipSuccess;
  const int64_t hblocks = (p.group + 63) / 64;
  hipError_t e = hipSuccess;
  if (kv != nullptr && p.ratio > 0 && p.topk > 0) {
    // the listed groups' bitmaps and the extras list
    hipLaunchKernelGGL(bwd_extras_zero_kernel, dim3(1), dim3(64), 0, stream, kv->n_extra);
    hipLaunchKernelGGL(bwd_bitmap_kernel, dim3((unsigned)p.num_queries), dim3(256), 0, stream, p, *kv);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (pairs) {
    const int64_t blocks = (int64_t)((p.num_queries + 1) / 2) * p.hkv * hblocks;
    if (blocks > 0x7FFFFFFFLL) return hipErrorInvalidValue;
    if (kv != nullptr)
      hipLaunchKernelGGL((attn_bwd_kernel<2, false>), dim3((unsigned)blocks), dim3(256), 0, stream, p, b);
    else
      hipLaunchKernelGGL((attn_bwd_kernel<2, true>), dim3((unsigned)blocks), dim3(256), 0, stream, p, b);
  } else {
    const int64_t blocks = (int64_t)p.num_queries * p.hkv * hblocks;
    if (blocks > 0x7FFFFFFFLL) return hipErrorInvalidValue;
    if (kv != nullptr)
      hipLaunchKernelGGL((attn_bwd_kernel<1, false>), dim3((unsigned)blocks), dim3(128), 0, stream, p, b);
    else
      hipLaunchKernelGGL((attn_bwd_kernel<1, true>), dim3((unsigned)blocks), dim3(128), 0, stream, p, b);
  }
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (kv != nullptr && kv->ng_raw + kv->ng_cmp > 0) {
    const int64_t blocks = (int64_t)p.num_seqs * (kv->ng_raw + kv->ng_cmp) * p.hkv * ((kv->nch + 7) / 8 * 8);
    hipLaunchKernelGGL(attn_bwd_kv_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, p, b, *kv);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (b.dsink != nullptr && b.dsink_part != nullptr) {
    hipLaunchKernelGGL(sink_reduce_kernel, dim3((unsigned)p.hq), dim3(256), 0, stream, b.dsink_part, p.num_queries,
                       p.hq, b.dsink);
    e = hipGetLastError();
  }
  return e;
}

}  // namespace spa
