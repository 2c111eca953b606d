// Sparse paged attention for gfx950, prefill: query pairs that share KV
// tiles, every wave of a workgroup a compute wave.
//
// Operation: the same as spa_attention.hip (RL-Kernel PR "Roadmap item 24:
// joint compressed/window attention with sink", section "Reuse and
// arithmetic"; KV-set and translation rules in spa_device.h), for prefill
// calls with bf16 caches and D 128.
//
// In a prefill the KV sets of neighbouring tokens of a sequence overlap
// almost entirely: their windows differ by one row, and the compressed
// groups two neighbours select are mostly the same (all of them, while n_c
// is at most the top-k).  One workgroup serves two queries (a pair) of one
// KV head and 64 of its query heads.  It streams the UNION of the two KV
// sets once through LDS, and each of its four waves (query q of the pair,
// heads 32w .. 32w+31) masks the rows its own query does not select.  A tile
// of K and V then feeds 128 (query, head) columns instead of 64.  Two
// workgroups (eight waves) fit on a CU.
//
// Setup of a query pair (before the tile loop):
//   * the loads that need nothing else are issued together: the Q fragments,
//     both queries' metadata and both whole list rows; the KV sets are first
//     computed without the check of the positions against seq_lens, whose
//     loads are issued with the page-table slices below;
//   * union mode, when both queries are in one sequence, their windows touch,
//     their complete groups fit the bitmaps and the page-table columns they
//     need fit the LDS slices: the page-table slices are loaded into LDS,
//     each query's selected groups become a bitmap (a listed id that is not
//     a complete group of that query is flagged and left out), the OR of the
//     two is ranked word by word, and every union group and every window
//     position (from the lower window start to the higher query position)
//     is translated through the slices;
//   * otherwise (pair across sequences, far-apart positions, a list that
//     names a group twice) concatenation mode: query 0's rows, then query
//     1's, each in canonical order and selected by its own query only, with
//     the page-table entries read row by row;
//   * the result is one list of rows padded to whole tiles: the byte
//     addresses of each row's K and V (the static zero row when masked) and
//     a byte per row, bit q = selected by query q.
// The tile loop then needs no translation and almost no address arithmetic:
// tile j is rows 32j .. 32j+31 of that list.
//
// Pipeline: NST LDS stages of one K and one V tile, one barrier per step,
// and the scores one tile ahead of the softmax.  Step j waits for tile j+1
// (each wave for its own loads, then the barrier), issues the loads of tile
// j+2 into the stage of tile j-1 (every wave has passed the barrier, so none
// still reads it), and then runs S(j+1)^T = K(j+1).Q^T on the matrix cores
// while the vector ALUs take the online softmax of tile j, whose scores the
// previous step computed; O^T += V(j)^T.P(j)^T closes the step.  So each
// wave keeps its matrix cores and its vector ALUs busy at once, rather than
// in turn.
//
// The compute is that of spa_attention.hip's compute waves: S^T = K.Q^T and
// O^T += V^T.P^T on v_mfma_f32_32x32x16_bf16, Q^T in registers, the online
// softmax in the log2 domain with the sink folded into the running (m, l),
// and the lazy rescale of O.

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdint>
#include <type_traits>

#include "spa_device.h"
#include "spa_kernel_util.h"

namespace spa {
namespace {

constexpr int kD = 128;
constexpr int kRowB = 2 * kD;              // bf16 row bytes
constexpr int kChunks = kRowB / 16;        // 16-byte chunks per row
constexpr int kPT = 32;                    // KV rows per tile
constexpr int kPTileB = kPT * kRowB;       // one K (or V) tile, bytes
constexpr int kThreads = 256;              // four compute waves
constexpr int kUMax = kPairRowsMax;        // union rows a workgroup can hold
constexpr int kRowIters = (kUMax + kThreads - 1) / kThreads;
constexpr int kBmWords = 1024;             // bitmap words per query: groups < 32768

constexpr int kPtMax = 4096;               // page-table entries the LDS slices hold
constexpr int64_t kCmpBit = int64_t(1) << 62;   // setup: a compressed-pool row

template <int NST>
struct PairSmem {
  union {
    struct {
      alignas(16) uint8_t k[NST][kPTileB];
      alignas(16) uint8_t v[NST][kPTileB];
    } t;
    struct {                               // setup only (union mode)
      uint32_t bm[2][kBmWords];            // selected groups of each query
      alignas(16) int32_t pt[kPtMax];      // page-table slices: compressed, then raw
      int32_t wpre[kBmWords];              // union rank of each bitmap word's first group
    } s;
  } u;
  // the union rows, padded to a whole tile: byte addresses of K and V (the
  // zero row for a masked row) and the selecting queries
  alignas(16) uint64_t ka[kUMax];
  alignas(16) uint64_t va[kUMax];
  uint8_t flg[kUMax];                      // bit q: selected by query q
  int32_t wsum[4];
  int32_t dup;                             // a list names a group twice
};
static_assert(sizeof(PairSmem<3>::u.s) <= sizeof(PairSmem<3>::u.t), "setup arrays fit the tile stages");
static_assert(kBmWords == 4 * kThreads, "four bitmap words per thread in the rank scan");
static_assert(kUMax % kPT == 0, "padding to a whole tile stays within the row list");

// Wave = query * 2 + head half.
template <int NST>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2)))
void attn_pair_kernel(const Params p) {
  static_assert(NST == 3, "three LDS stages: tiles j and j+1 read, tile j+2 loading");
  __shared__ PairSmem<NST> sm;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int hi = lane >> 5;
  const int qw = wave >> 1;                  // this wave's query within the pair

  // workgroup -> item: (pair, KV head, 64-head block), the last pairs (the
  // longest KV sets in a causal prefill) first
  int32_t i0, i1, g, hb;
  {
    const int32_t hblocks = (p.group + 63) / 64;
    const int32_t per_pair = p.hkv * hblocks;
    const int32_t npairs = (p.num_queries + 1) / 2;
    // the first 2C items (C compute units, two resident workgroups each)
    // put the C longest with the C shortest, so that the two workgroups of
    // a CU finish at different times and the setups of later items overlap
    // the tile loops of others; the rest follow longest first
    const int32_t w = (int32_t)(blockIdx.x / per_pair);
    const int32_t C = p.num_cus;
    int32_t pr = npairs - 1 - w;
    if (C > 0 && npairs >= 2 * C) pr = w < C ? npairs - 1 - w : w < 2 * C ? w - C : npairs - 1 - (w - C);
    const int32_t rem = (int32_t)(blockIdx.x % per_pair);
    g = rem / hblocks;
    hb = rem - g * hblocks;
    i0 = 2 * pr;
    i1 = 2 * pr + 1;
  }
  const bool has1 = i1 < p.num_queries;
  const int32_t iq = qw == 0 ? i0 : i1;      // this wave's query
  const bool qvalid = qw == 0 || has1;

  // ---- phase A: the loads that need nothing else, issued together and
  // unconditionally (an invalid one reads a valid address and its value is
  // dropped), so that the first, the pair's metadata, can be waited for
  // alone: lane k of one load takes value k of (query_seq, query_pos) of
  // both queries and their list counts; then both whole list rows
  // (capacity topk each; entries past a count are not used) and the Q
  // fragments of this lane's head
  const int32_t topk_arg = p.topk;
  int32_t meta;
  {
    const int32_t *src = p.query_seq + i0;
    if (lane == 1) src = p.query_pos + i0;
    if (lane == 2 && has1) src = p.query_seq + i1;
    if (lane == 3 && has1) src = p.query_pos + i1;
    if (lane == 4 && topk_arg > 0) src = p.cmp_cnt + i0;
    if (lane == 5 && topk_arg > 0 && has1) src = p.cmp_cnt + i1;
    meta = *src;
  }
  int32_t ids[kRowIters];
#pragma unroll
  for (int it = 0; it < kRowIters; ++it) {
    const int e = tid + it * kThreads;
    const int q = e >= topk_arg ? 1 : 0;
    const bool ok = topk_arg > 0 && e < 2 * topk_arg && (q == 0 || has1);
    int32_t v = *(ok ? p.cmp_idx + (int64_t)(q ? i1 : i0) * topk_arg + (e - q * topk_arg) : p.query_seq + i0);
    ids[it] = ok ? v : -1;
  }
  const int hl = hb * 64 + (wave & 1) * 32 + (lane & 31);
  const bool hvalid = qvalid && hl < p.group;
  bf16x8 qf[kD / 16];
  {
    const uint16_t *qrow = p.q + ((int64_t)(hvalid ? iq : i0) * p.hq + (int64_t)g * p.group + (hvalid ? hl : 0)) * kD + 8 * hi;
#pragma unroll
    for (int kk = 0; kk < kD / 16; ++kk) {
      bf16x8 v = *(const bf16x8 *)(qrow + 16 * kk);
      qf[kk] = hvalid ? v : bf16x8{};
    }
  }
  wait_vmcnt<kRowIters + kD / 16>();         // the metadata is in; lists and Q in flight
  const int32_t topk = p.topk;                        // 0: no list
  const int32_t P = p.page_size;
  const int64_t hkv = p.hkv;
  int32_t U = 0;                                      // rows in the pair's list

  // a row of the list: pool row (row * Hkv + g, kCmpBit for the compressed
  // pool) or -1 (masked), stored as the byte addresses of its K and V
  const uint8_t *const kraw = in_sgpr(p.k_raw), *const vraw = in_sgpr(p.v_raw);
  const uint8_t *const kcmp = in_sgpr(p.k_cmp), *const vcmp = in_sgpr(p.v_cmp);
  auto put_row = [&](int r, int64_t er) {
    const uint8_t *ka = kZeroRow, *va = kZeroRow;
    if (er >= 0) {
      const bool cmp = (er & kCmpBit) != 0;
      const int64_t off = (er & ~kCmpBit) * kRowB;
      ka = (cmp ? kcmp : kraw) + off;
      va = (cmp ? vcmp : vraw) + off;
    }
    sm.ka[r] = (uint64_t)ka;
    sm.va[r] = (uint64_t)va;
  };

  const int32_t mb0 = __builtin_amdgcn_readlane(meta, 0), mt0 = __builtin_amdgcn_readlane(meta, 1);
  const int32_t mb1 = has1 ? __builtin_amdgcn_readlane(meta, 2) : -1;
  const int32_t mt1 = has1 ? __builtin_amdgcn_readlane(meta, 3) : -1;
  const int32_t mc0 = topk > 0 ? __builtin_amdgcn_readlane(meta, 4) : 0;
  const int32_t mc1 = (topk > 0 && has1) ? __builtin_amdgcn_readlane(meta, 5) : 0;

  // ---- the pair's KV sets, before the positions are checked against
  // seq_lens (those loads and the sink's are issued now and used after the
  // next wait)
  const bool bok0 = mb0 >= 0 && mb0 < p.num_seqs;
  const bool bok1 = has1 && mb1 >= 0 && mb1 < p.num_seqs;
  const QueryKV pk0 = bok0 ? query_kv_of(p, mb0, mt0, INT32_MAX, mc0, false) : QueryKV{0, 0, 0, 0, 0, 0};
  const QueryKV pk1 = bok1 ? query_kv_of(p, mb1, mt1, INT32_MAX, mc1, false) : QueryKV{0, 0, 0, 0, 0, 0};
  int32_t lens = 0;                                   // lane 0: seq_lens[mb0], lane 1: seq_lens[mb1]
  if ((lane == 0 && bok0) || (lane == 1 && bok1)) lens = p.seq_lens[lane == 0 ? mb0 : mb1];
  const float sink = (hvalid && p.sink != nullptr) ? p.sink[g * p.group + hl] : -INFINITY;

  // union mode: one sequence, touching windows, the groups within the
  // bitmaps and the page-table columns within the LDS slices
  const bool touch = pk0.win_len == 0 || pk1.win_len == 0 ||
                     (pk1.win_lo <= pk0.t + 1 && pk0.win_lo <= pk1.t + 1);
  const int32_t ncmax = max(pk0.n_c, pk1.n_c);
  int32_t wlo = 0, nwin = 0;                          // union window: positions wlo .. wlo+nwin-1
  if (pk0.win_len > 0 || pk1.win_len > 0) {
    wlo = pk0.win_len == 0 ? pk1.win_lo : pk1.win_len == 0 ? pk0.win_lo : min(pk0.win_lo, pk1.win_lo);
    const int32_t whi = pk0.win_len == 0 ? pk1.t : pk1.win_len == 0 ? pk0.t : max(pk0.t, pk1.t);
    nwin = whi - wlo + 1;
  }
  const int32_t ncol_c = p.ratio > 0 ? min((ncmax + P - 1) / P, p.cmp_pt_stride) : 0;
  const int32_t col_lo = wlo / P;
  const int32_t ncol_r = nwin > 0 ? max(0, min((wlo + nwin - 1) / P, p.raw_pt_stride - 1) - col_lo + 1) : 0;
  bool uni = bok0 && (!has1 || (bok1 && mb1 == mb0)) && touch && ncmax <= 32 * kBmWords &&
                   ncol_c + ncol_r <= kPtMax;

  QueryKV kv0{0, 0, 0, 0, 0, 0}, kv1{0, 0, 0, 0, 0, 0};
  if (uni) {
    const int32_t b = mb0;
    // -- page-table slices into LDS (direct loads): compressed columns
    // 0 .. ncol_c-1, then raw columns col_lo .. col_lo+ncol_r-1
    for (int c = wave; 64 * c < ncol_c + ncol_r; c += kThreads / 64) {
      const int k = 64 * c + lane;
      const void *src = kZeroRow;
      if (k < ncol_c) src = p.cmp_pt + (int64_t)b * p.cmp_pt_stride + k;
      else if (k < ncol_c + ncol_r) src = p.raw_pt + (int64_t)b * p.raw_pt_stride + col_lo + (k - ncol_c);
      dma4(src, &sm.u.s.pt[64 * c]);
    }
    for (int k = tid; k < 2 * kBmWords; k += kThreads) (&sm.u.s.bm[0][0])[k] = 0u;
    if (tid == 0) sm.dup = 0;
    wait_vmcnt<0>();                                  // slices, lists, Q
    __syncthreads();                                  // slices in, bitmaps cleared
    // -- the KV sets checked against seq_lens (a query past its sequence
    // has an empty set; the error bits are raised once); they are subsets
    // of the provisional ones, so the slices cover them
    const int32_t len0 = __builtin_amdgcn_readlane(lens, 0), len1 = __builtin_amdgcn_readlane(lens, 1);
    kv0 = query_kv_of(p, mb0, mt0, len0, mc0, tid == 0);
    if (bok1) kv1 = query_kv_of(p, mb1, mt1, len1, mc1, tid == 0);
    if (has1 && !bok1 && tid == 0) flag_error(p, kErrQuery);
    // -- selected groups: one bitmap per query
#pragma unroll
    for (int it = 0; it < kRowIters; ++it) {
      const int e = tid + it * kThreads;
      if (topk > 0 && e < 2 * topk) {
        const int q = e >= topk ? 1 : 0;
        const QueryKV &kv = q ? kv1 : kv0;
        if (e - q * topk < kv.n_sel) {
          const int32_t c = ids[it];
          if (c >= 0 && c < kv.n_c) {
            if (atomicOr(&sm.u.s.bm[q][c >> 5], 1u << (c & 31)) & (1u << (c & 31))) sm.dup = 1;
          } else {
            flag_error(p, kErrCmpId);
          }
        }
      }
    }
    __syncthreads();
    // a list that names a group twice counts it twice, as the canonical
    // order does: such a pair takes the concatenation below
    uni = sm.dup == 0;
  }
  if (uni) {
    // -- rank of every word's first group in the ascending union: thread t
    // sums words 4t .. 4t+3, one scan over the threads
    const int32_t nw = (ncmax + 31) / 32;             // <= kBmWords = 4 * kThreads
    int32_t wc[4];
    int32_t own = 0;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int k = 4 * tid + u;
      wc[u] = k < nw ? __popc(sm.u.s.bm[0][k] | sm.u.s.bm[1][k]) : 0;
      own += wc[u];
    }
    int32_t ncu;                                      // groups in the union
    int32_t pre = block_excl_scan<kThreads>(own, ncu, sm.wsum);
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int k = 4 * tid + u;
      if (k < nw) sm.u.s.wpre[k] = pre;
      pre += wc[u];
    }
    const int32_t wlo2 = kv0.win_len == 0 ? kv1.win_lo : kv1.win_len == 0 ? kv0.win_lo : min(kv0.win_lo, kv1.win_lo);
    const int32_t nwin2 = (kv0.win_len == 0 && kv1.win_len == 0) ? 0
                          : (kv0.win_len == 0 ? kv1.t : kv1.win_len == 0 ? kv0.t : max(kv0.t, kv1.t)) - wlo2 + 1;
    U = min(ncu + nwin2, kUMax);
    __syncthreads();                                  // word ranks in
    // -- translation from the slices: pool row (row * Hkv + g) with bit 62
    // set for a compressed row, or -1; one thread per group id, then per
    // window position; rows up to the next tile edge padded
    const bool pow2 = p.page_shift >= 0;
    auto pool_row = [&](int32_t x, bool cmp) -> int64_t {
      const int32_t col = pow2 ? x >> p.page_shift : x / P;
      const int32_t off = x - col * P;
      int32_t page = -1;
      if (cmp ? col < ncol_c : (col >= col_lo && col - col_lo < ncol_r)) page = sm.u.s.pt[cmp ? col : ncol_c + (col - col_lo)];
      if (page >= 0 && (int64_t)page < (cmp ? p.cmp_pages : p.raw_pages))
        return (((int64_t)page * P + off) * hkv + g) | (cmp ? kCmpBit : 0);
      flag_error(p, kErrPage);
      return -1;
    };
    for (int c = tid; c < 32 * nw; c += kThreads) {
      const uint32_t b0 = sm.u.s.bm[0][c >> 5], b1 = sm.u.s.bm[1][c >> 5];
      const uint32_t bit = 1u << (c & 31);
      if ((b0 | b1) & bit) {
        const int32_t r = sm.u.s.wpre[c >> 5] + __popc((b0 | b1) & (bit - 1u));
        if (r < kUMax) {
          const int64_t er = pool_row(c, true);
          put_row(r, er);
          sm.flg[r] = (uint8_t)(er >= 0 ? ((b0 & bit) ? 1u : 0u) | ((b1 & bit) ? 2u : 0u) : 0u);
        }
      }
    }
    for (int e = tid; e < (U + kPT - 1) / kPT * kPT - ncu; e += kThreads) {
      const int r = ncu + e;
      int64_t er = -1;
      uint32_t sel = 0;
      if (e < nwin2 && r < kUMax) {
        const int32_t x = wlo2 + e;
        sel = (kv0.win_len > 0 && x >= kv0.win_lo && x <= kv0.t ? 1u : 0u) |
              (kv1.win_len > 0 && x >= kv1.win_lo && x <= kv1.t ? 2u : 0u);
        if (sel != 0) er = pool_row(x, false);
      }
      if (r < kUMax) {
        put_row(r, er);
        sm.flg[r] = (uint8_t)(er >= 0 ? sel : 0u);
      }
    }
  } else {
    // -- concatenation: query 0's canonical rows, then query 1's (the
    // metadata is read again: this path is for the odd cases)
    kv0 = query_kv(p, i0);
    kv1 = has1 ? query_kv(p, i1) : QueryKV{0, 0, 0, 0, 0, 0};
    const int32_t U0 = kv0.n_sel + kv0.win_len;
    const int32_t U1 = has1 ? kv1.n_sel + kv1.win_len : 0;
    U = min(U0 + U1, kUMax);
    int32_t xs[kRowIters];
#pragma unroll
    for (int it = 0; it < kRowIters; ++it) {
      const int r = tid + it * kThreads;
      xs[it] = -1;
      if (r < U) {
        const int q = r < U0 ? 0 : 1;
        const QueryKV &kv = q ? kv1 : kv0;
        const int32_t e = q ? r - U0 : r;
        if (e < kv.n_sel) xs[it] = topk > 0 ? p.cmp_idx[(int64_t)(q ? i1 : i0) * topk + e] : e;
        else xs[it] = kv.win_lo + (e - kv.n_sel);
      }
    }
    int32_t pg[kRowIters];
#pragma unroll
    for (int it = 0; it < kRowIters; ++it) {
      const int r = tid + it * kThreads;
      pg[it] = -1;
      if (r < U) {
        const int q = r < U0 ? 0 : 1;
        const QueryKV &kv = q ? kv1 : kv0;
        const int32_t e = q ? r - U0 : r;
        const bool cmp = e < kv.n_sel;
        int32_t x = xs[it];
        if (cmp && (x < 0 || x >= kv.n_c)) {
          flag_error(p, kErrCmpId);
          x = -1;
        }
        if (x >= 0) {
          const int32_t col = x / P;
          if (col < (cmp ? p.cmp_pt_stride : p.raw_pt_stride))
            pg[it] = (cmp ? p.cmp_pt + (int64_t)kv.b * p.cmp_pt_stride : p.raw_pt + (int64_t)kv.b * p.raw_pt_stride)[col];
          else {
            flag_error(p, kErrPage);
            x = -1;
          }
        }
        xs[it] = x;
      }
    }
#pragma unroll
    for (int it = 0; it < kRowIters; ++it) {
      const int r = tid + it * kThreads;
      if (r < (U + kPT - 1) / kPT * kPT) {
        int64_t er = -1;
        uint32_t sel = 0;
        if (r < U) {
          const int q = r < U0 ? 0 : 1;
          const QueryKV &kv = q ? kv1 : kv0;
          const int32_t e = q ? r - U0 : r;
          const bool cmp = e < kv.n_sel;
          if (xs[it] >= 0) {
            if (pg[it] >= 0 && (int64_t)pg[it] < (cmp ? p.cmp_pages : p.raw_pages))
              er = (((int64_t)pg[it] * P + (xs[it] % P)) * hkv + g) | (cmp ? kCmpBit : 0);
            else
              flag_error(p, kErrPage);
          }
          sel = 1u << q;
        }
        put_row(r, er);
        sm.flg[r] = (uint8_t)(er >= 0 ? sel : 0u);
      }
    }
  }
  wait_vmcnt<0>();                           // Q fragments, sink and every setup load are in
  __syncthreads();                           // rows and flags complete; bitmaps and slices dead

  // ---- tile loads: wave w moves rows 8w .. 8w+7 of a side (two 1 KiB
  // direct loads, four rows each); the 16-byte chunk of lane L in load n is
  // logical chunk (L % 16) ^ swz(row), row = 8w + 4n + L / 16.  K of a tile
  // is needed one step before its V, so step j issues K of tile j+3 and V
  // of tile j+2: both two steps ahead.
  int32_t csrc[2];
#pragma unroll
  for (int n = 0; n < 2; ++n) {
    const int r = 8 * wave + 4 * n + lane / kChunks;
    csrc[n] = ((lane % kChunks) ^ swz<kChunks>(r)) * 16;
  }
  const int32_t ntiles = (U + kPT - 1) / kPT;
  uint64_t nka[2], nva[2];
  auto fetch_k = [&](int j) {
#pragma unroll
    for (int n = 0; n < 2; ++n) nka[n] = j < ntiles ? sm.ka[kPT * j + 8 * wave + 4 * n + lane / kChunks] : (uint64_t)kZeroRow;
  };
  auto fetch_v = [&](int j) {
#pragma unroll
    for (int n = 0; n < 2; ++n) nva[n] = j < ntiles ? sm.va[kPT * j + 8 * wave + 4 * n + lane / kChunks] : (uint64_t)kZeroRow;
  };
  // LDS offsets of this wave's rows in stage 0 (scalar)
  const uint32_t kdst = __builtin_amdgcn_readfirstlane(lds_offset(sm.u.t.k[0]) + 8 * wave * kRowB);
  const uint32_t vdst = __builtin_amdgcn_readfirstlane(lds_offset(sm.u.t.v[0]) + 8 * wave * kRowB);
  auto issue_k = [&](const int st) {
#pragma unroll
    for (int n = 0; n < 2; ++n) dma16_at((const void *)(nka[n] + csrc[n]), kdst + st * kPTileB + 4 * n * kRowB);
  };
  auto issue_v = [&](const int st) {
#pragma unroll
    for (int n = 0; n < 2; ++n) dma16_at((const void *)(nva[n] + csrc[n]), vdst + st * kPTileB + 4 * n * kRowB);
  };
  // wait until at most n (even, <= 8) of this wave's loads are in flight
  auto wait_loads = [](int n) {
    if (n >= 8) wait_vmcnt<8>();
    else if (n >= 6) wait_vmcnt<6>();
    else if (n >= 4) wait_vmcnt<4>();
    else if (n >= 2) wait_vmcnt<2>();
    else wait_vmcnt<0>();
  };
  // this wave's selection mask of tile j (rows its query selects)
  auto tile_mask = [&](int j) -> uint32_t {
    return (uint32_t)__ballot(lane < 32 && ((sm.flg[kPT * j + (lane & 31)] >> qw) & 1u));
  };
  // LDS byte addresses of this lane's fragments in stage 0: K (MFMA A
  // operand: row lane % 32, k = 16 kk + 8 hi ..) and V^T (the transpose
  // read: for (db, rr); k2 adds 16 rows).  A step adds its stage as an
  // immediate offset.
  uint32_t koff[kD / 16], voff[kD / 32][2];
  {
    const int r = lane & 31;
#pragma unroll
    for (int kk = 0; kk < kD / 16; ++kk)
      koff[kk] = lds_offset(sm.u.t.k[0]) + r * kRowB + (((2 * kk + hi) ^ swz<kChunks>(r)) * 16);
    const int G = lane >> 4;
    const int L = lane & 15;
#pragma unroll
    for (int db = 0; db < kD / 32; ++db)
#pragma unroll
      for (int rr = 0; rr < 2; ++rr) {
        const int row = 8 * rr + 4 * (G >> 1) + (L >> 2);
        const int d = 32 * db + 16 * (G & 1) + 4 * (L & 3);
        voff[db][rr] = lds_offset(sm.u.t.v[0]) + row * kRowB + (((d >> 3) ^ swz<kChunks>(row)) * 16) + (L & 1) * 8;
      }
  }
  auto read_k = [&](auto stage, bf16x8 (&kf)[kD / 16]) {
    constexpr int ST = decltype(stage)::value;
#pragma unroll
    for (int kk = 0; kk < kD / 16; ++kk) kf[kk] = *(const lds_bf16x8_t *)(uintptr_t)(koff[kk] + ST * kPTileB);
  };

  // ---- per-lane softmax state; the sink initialises (m, l)
  float m = sink == -INFINITY ? -INFINITY : sink * kLog2e;
  float l = (sink != -INFINITY && hi == 0) ? 1.f : 0.f;   // exp2(sink - m) = 1, counted once per head
  f32x16 acc[kD / 32];
#pragma unroll
  for (int db = 0; db < kD / 32; ++db) acc[db] = f32x16{};

  // ---- prologue: tile j's K and V go to stage j % NST; issued in the
  // order K0 V0 K1 K2 V1 (the last two as a step -1 would), then the scores
  // of tile 0
  fetch_k(0);
  fetch_v(0);
  if (ntiles > 0) {
    issue_k(0);
    issue_v(0);
  }
  fetch_k(1);
  if (ntiles > 1) issue_k(1);
  fetch_k(2);
  if (ntiles > 2) issue_k(2);
  fetch_v(1);
  if (ntiles > 1) issue_v(1);
  f32x16 s = f32x16{};                      // raw scores S^T of the tile the next step takes
  uint32_t tm = 0;
  if (ntiles > 0) {
    wait_loads(2 + (ntiles > 1 ? 4 : 0) + (ntiles > 2 ? 2 : 0));   // K0 in: V0 K1 K2 V1 may be in flight
    block_sync();                            // K of tile 0 is in LDS
    tm = tile_mask(0);
    bf16x8 kf[kD / 16];
    read_k(std::integral_constant<int, 0>{}, kf);
#pragma unroll
    for (int kk = 0; kk < kD / 16; ++kk) s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[kk], qf[kk], s, 0, 0, 0);
  }

  // ---- one step of the tile loop (tile j in stage ST, a compile-time
  // constant, so that every LDS address is a register plus an immediate).
  // Step j runs three independent pieces together: the scores of tile j+1
  // and O^T += V^T.P^T of tile j-1 on the matrix cores, the softmax of tile
  // j on the vector ALUs; it ends by reading V of tile j for the next step.
  // Lane rows of S^T: 8*(i/4) + 4*hi + i%4.
  i16x8 vprev[kD / 32][2];                  // V^T fragments of the previous tile
  bf16x8 pprev[2];                          // its P (bf16), relative to its m
#pragma unroll
  for (int db = 0; db < kD / 32; ++db) vprev[db][0] = vprev[db][1] = i16x8{};
  pprev[0] = pprev[1] = bf16x8{};
  auto pv_prev = [&]() {
#pragma unroll
    for (int db = 0; db < kD / 32; ++db)
#pragma unroll
      for (int k2 = 0; k2 < 2; ++k2)
        acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, vprev[db][k2]), pprev[k2], acc[db],
                                                          0, 0, 0);
  };
  auto step = [&](const int j, auto stage) {
    constexpr int ST = decltype(stage)::value;
    const bool more = j + 1 < ntiles;
    bf16x8 kf[kD / 16];
    uint32_t tm_next = 0;
    // K of tile j+1 and V of tile j are in (this wave's loads: only those
    // of step j-1 may still be in flight) ...
    wait_loads((j + 2 < ntiles ? 2 : 0) + (j + 1 < ntiles ? 2 : 0));
    block_sync();                            // ... for every wave, and every wave is past step j-1
    if (j + 3 < ntiles) {
      fetch_k(j + 3);
      issue_k(ST);                           // K of tile j+3 replaces K of tile j
    }
    if (j + 2 < ntiles) {
      fetch_v(j + 2);
      issue_v((ST + 2) % NST);               // V of tile j+2 replaces V of tile j-1
    }
    if (more) tm_next = tile_mask(j + 1);
    // (after the last tile the stage read holds stale rows: those scores
    // are not used).  The offsets are redefined opaquely at every step, so
    // that the compiler keeps one register each and folds the stage into the
    // instructions, instead of one register per stage.
#pragma unroll
    for (int kk = 0; kk < kD / 16; ++kk) asm volatile("" : "+v"(koff[kk]));
#pragma unroll
    for (int db = 0; db < kD / 32; ++db)
#pragma unroll
      for (int rr = 0; rr < 2; ++rr) asm volatile("" : "+v"(voff[db][rr]));
    read_k(std::integral_constant<int, (ST + 1) % NST>{}, kf);
    float sc[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) sc[i] = s[i];
    mask_tile_rows(sc, tm);
    f32x16 sn = f32x16{};
#pragma unroll
    for (int kk = 0; kk < kD / 16; ++kk) sn = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[kk], qf[kk], sn, 0, 0, 0);
    pv_prev();
    float smax = fmaxf(fmaxf(fmaxf(sc[0], sc[1]), fmaxf(sc[2], sc[3])), fmaxf(fmaxf(sc[4], sc[5]), fmaxf(sc[6], sc[7])));
    smax = fmaxf(smax, fmaxf(fmaxf(fmaxf(sc[8], sc[9]), fmaxf(sc[10], sc[11])),
                             fmaxf(fmaxf(sc[12], sc[13]), fmaxf(sc[14], sc[15]))));
    smax = max_lane_pair(smax);
    const float tmax = smax * p.scale_log2;
    const bool need = tmax > m + kTau;
    const bool rescale = __any(need);
    const float alpha = need ? __builtin_amdgcn_exp2f(m - tmax) : 1.f;
    m = need ? tmax : m;
    const float negm = m == -INFINITY ? 0.f : -m;
    float pr[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) pr[i] = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[i], p.scale_log2, negm));
    float psum = ((pr[0] + pr[1]) + (pr[2] + pr[3])) + ((pr[4] + pr[5]) + (pr[6] + pr[7]));
    psum += ((pr[8] + pr[9]) + (pr[10] + pr[11])) + ((pr[12] + pr[13]) + (pr[14] + pr[15]));
    l = l * alpha + psum;
#pragma unroll
    for (int k2 = 0; k2 < 2; ++k2)
#pragma unroll
      for (int jj = 0; jj < 8; ++jj) pprev[k2][jj] = (__bf16)pr[8 * k2 + jj];
    // P is complete here (not sunk past the rescale branch), and the region
    // issues one MFMA, then a share of the softmax's vector instructions, in
    // turn
    asm volatile("" ::"v"(pprev[0]), "v"(pprev[1]));
#pragma unroll
    for (int kk = 0; kk < kD / 8; ++kk) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x002, 5, 0);
    }
    // O (with tile j-1's PV in) to this tile's m, before tile j's PV
    if (rescale) {
#pragma unroll
      for (int db = 0; db < kD / 32; ++db) acc[db] *= alpha;
    }
    // the V^T fragments of tile j (MFMA A operand through the transpose
    // read), for the next step
#pragma unroll
    for (int db = 0; db < kD / 32; ++db)
#pragma unroll
      for (int k2 = 0; k2 < 2; ++k2) {
        i16x4 h[2];
#pragma unroll
        for (int rr = 0; rr < 2; ++rr)
          h[rr] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (lds_i16x4_t *)(uintptr_t)(voff[db][rr] + ST * kPTileB + 16 * k2 * kRowB));
        vprev[db][k2] = __builtin_shufflevector(h[0], h[1], 0, 1, 2, 3, 4, 5, 6, 7);
      }
    s = sn;
    tm = tm_next;
  };
  int32_t j = 0;
  for (; j + NST <= ntiles; j += NST) {
    step(j, std::integral_constant<int, 0>{});
    step(j + 1, std::integral_constant<int, 1>{});
    step(j + 2, std::integral_constant<int, 2>{});
  }
  if (j < ntiles) step(j, std::integral_constant<int, 0>{});
  if (j + 1 < ntiles) step(j + 1, std::integral_constant<int, 1>{});
  pv_prev();                                 // the last tile's PV

  // ---- epilogue: O = acc / l (bf16, RNE), LSE = (m + log2 l) ln 2; a query
  // that failed its checks has no rows and writes O = 0 and LSE = sink
  const float lt = l + __shfl_xor(l, 32);
  const float inv = lt > 0.f ? 1.f / lt : 0.f;
  const float lse2 = (m == -INFINITY || !(lt > 0.f)) ? -INFINITY : m + __builtin_amdgcn_logf(lt);
  const float lse = lse2 == -INFINITY ? -INFINITY : lse2 * kLn2;
  if (!hvalid) return;
  const int64_t h = (int64_t)g * p.group + hl;
  uint16_t *orow = p.o + ((int64_t)iq * p.hq + h) * kD;
#pragma unroll
  for (int db = 0; db < kD / 32; ++db) {
#pragma unroll
    for (int i4 = 0; i4 < 4; ++i4) {
      const int d0 = 32 * db + 8 * i4 + 4 * hi;
      uint2 w;
      w.x = bf16_bits(acc[db][4 * i4 + 0] * inv) | (bf16_bits(acc[db][4 * i4 + 1] * inv) << 16);
      w.y = bf16_bits(acc[db][4 * i4 + 2] * inv) | (bf16_bits(acc[db][4 * i4 + 3] * inv) << 16);
      *(uint2 *)(orow + d0) = w;
    }
  }
  if (hi == 0 && p.lse) p.lse[(int64_t)iq * p.hq + h] = lse;
}

}  // namespace

bool prefill_pairs_eligible(const Params &p) {
  return p.head_dim == kD && !p.cmp_fp8 && p.num_splits == 1 && p.query_seq != nullptr &&
         p.query_pos != nullptr && (p.ratio == 0 || p.topk > 0) &&
         2 * ((int64_t)p.topk + p.window) <= kUMax;
}

hipError_t launch_prefill_pairs(const Params &p, hipStream_t stream) {
  if (p.num_queries == 0) return hipSuccess;
  if (!prefill_pairs_eligible(p)) return hipErrorInvalidConfiguration;
  const int64_t npairs = (p.num_queries + 1) / 2;
  const int64_t grid = npairs * p.hkv * ((p.group + 63) / 64);
  if (grid > 0x7FFFFFFFLL) return hipErrorInvalidConfiguration;
  Params q = p;
  q.num_cus = (p.hkv * ((p.group + 63) / 64) == 1) ? device_cu_count() : 0;   // one item per pair
  hipLaunchKernelGGL((attn_pair_kernel<kPairStages>), dim3((unsigned)grid), dim3(kThreads), 0, stream, q);
  return hipGetLastError();
}

}  // namespace spa
