// Sparse paged attention for gfx950 with every wave of a workgroup a compute
// wave: prefill query pairs that share KV tiles, and decode KV slices.
//
// Operation: the same as spa_attention.hip (RL-Kernel PR "Roadmap item 24:
// joint compressed/window attention with sink", section "Reuse and
// arithmetic"; KV-set and translation rules in spa_device.h), for calls with
// bf16 caches and D 128.
//
// Prefill query pairs (DEC = false).  In a prefill the KV sets of
// neighbouring tokens of a sequence overlap almost entirely: their windows
// differ by one row, and the compressed groups two neighbours select are
// mostly the same (all of them, while n_c is at most the top-k).  One
// workgroup serves two queries (a pair) of one KV head and 64 of its query
// heads, with one KV slice.  It streams the UNION of the two KV sets once
// through LDS, and each of its four waves (query q of the pair, heads
// 32w .. 32w+31) masks the rows its own query does not select.  A tile of K
// and V then feeds 128 (query, head) columns instead of 64.
//
// Decode slices (DEC = true).  One workgroup serves one KV slice of one
// query, one KV head and 128 of its query heads (four waves of 32 heads).
// A slice's list slots are cut by capacity, not by the query's own counts
// (any partition of a set gives the same softmax), so they are loaded
// together with the metadata; with several slices it writes a sink-free
// partial (O_s, LSE_s) that the LSE merge kernel combines with the sink.
//
// Every wave issues a quarter of each tile's direct global->LDS loads and
// then runs its MFMAs; two workgroups (eight waves) fit on a CU.
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
//   * the result is one list of 64-bit pool rows (row * Hkv + g, bit 62 for
//     a compressed row, -1 when masked) padded to whole tiles, with a byte
//     per row: bit q = selected by query q.
// The tile loop then needs no translation: tile j is rows 32j .. 32j+31 of
// that list; masked rows load a static zero row.
//
// Pipeline: NST LDS stages of one K and one V tile, one barrier per step.
// Step j waits for tile j (each wave for its own loads, then the barrier),
// issues the loads of tile j+NST-1 into the stage of tile j-1 (every wave
// has passed the barrier, so none still reads it) and computes tile j.
//
// The compute of a tile is that of spa_attention.hip's compute waves:
// S^T = K.Q^T and O^T += V^T.P^T on v_mfma_f32_32x32x16_bf16, Q^T in
// registers, the online softmax in the log2 domain with the sink folded into
// the running (m, l), and the lazy rescale of O.

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
constexpr int64_t kCmpBit = int64_t(1) << 62;   // row list: a compressed-pool row

template <int NST, bool FP8>
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
  // union rows: logical id during setup, then row * Hkv + g (bit 62: a
  // compressed row; -1: masked), padded with -1 to a whole tile
  alignas(16) int64_t row[kUMax];
  uint8_t flg[kUMax];                      // bit q: selected by query q
  int32_t wsum[4];
  int32_t dup;                             // a list names a group twice
  // e4m3 compressed tiles (decode slices with FP8 pages): the staged codes
  // of both sides, 32 rows of D bytes, and their fp32 row scales
  alignas(16) uint8_t f8k[FP8 ? NST : 1][FP8 ? kPT * kD : 16];
  alignas(16) uint8_t f8v[FP8 ? NST : 1][FP8 ? kPT * kD : 16];
  alignas(16) float f8sk[FP8 ? NST : 1][64];
  alignas(16) float f8sv[FP8 ? NST : 1][64];
};
static_assert(sizeof(PairSmem<2, false>::u) == 2 * 2 * kPTileB, "setup arrays fit the tile stages");
static_assert(kBmWords == 4 * kThreads, "four bitmap words per thread in the rank scan");
static_assert(kUMax % kPT == 0, "padding to a whole tile stays within the row list");

// DEC = false: a prefill query pair (two queries, 64 heads: wave = query *
// 2 + head half).  DEC = true: one KV slice of a decode query (one query,
// 128 heads: wave = head quarter), whose sink-free partial the LSE merge
// combines when there are several slices.
//
// FP8 (decode slices only): the compressed pool holds OCP e4m3 codes with an
// fp32 scale per row.  The compressed rows of a slice fill whole tiles (the
// window starts at the next tile), an e4m3 tile is loaded into a staging
// area with its scales and widened to bf16 in LDS by all waves after its
// barrier (every e4m3 value is a bf16 value, so this is exact), and the k
// scale multiplies the fp32 scores, the v scale p before its bf16 rounding.
template <int NST, bool DEC, bool FP8>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2)))
void attn_pair_kernel(const Params p) {
  static_assert(NST >= 2 && NST <= 4, "two to four LDS stages");
  static_assert(!FP8 || (DEC && NST == 2), "e4m3 tiles: decode slices with two stages");
  __shared__ PairSmem<NST, FP8> sm;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int hi = lane >> 5;
  const int qw = DEC ? 0 : wave >> 1;        // this wave's query within the pair
  const int32_t S = DEC ? p.num_splits : 1;

  // workgroup -> item.  Pairs: (pair, KV head, 64-head block), the last pairs
  // (the longest KV sets in a causal prefill) first.  Decode: (query, KV
  // head, 128-head block, slice).
  int32_t i0, i1, g, hb, split = 0;
  if constexpr (DEC) {
    const int32_t hblocks = (p.group + 127) / 128;
    const int32_t per_q = p.hkv * hblocks * S;
    i0 = (int32_t)(blockIdx.x / per_q);
    const int32_t rem = (int32_t)(blockIdx.x % per_q);
    split = rem % S;
    g = rem / S / hblocks;
    hb = rem / S - g * hblocks;
    i1 = i0;
  } else {
    const int32_t hblocks = (p.group + 63) / 64;
    const int32_t per_pair = p.hkv * hblocks;
    const int32_t npairs = (p.num_queries + 1) / 2;
    const int32_t pr = npairs - 1 - (int32_t)(blockIdx.x / per_pair);
    const int32_t rem = (int32_t)(blockIdx.x % per_pair);
    g = rem / hblocks;
    hb = rem - g * hblocks;
    i0 = 2 * pr;
    i1 = 2 * pr + 1;
  }
  const bool has1 = !DEC && i1 < p.num_queries;
  const int32_t iq = qw == 0 ? i0 : i1;      // this wave's query
  const bool qvalid = qw == 0 || has1;

  // ---- phase A: the loads that need nothing else, issued together: the Q
  // fragments and sink of this lane's head, the metadata and the list
  // entries this item reads (for pairs both whole list rows, capacity topk
  // each; entries past a count are not used)
  const int hl = DEC ? hb * 128 + wave * 32 + (lane & 31) : hb * 64 + (wave & 1) * 32 + (lane & 31);
  const bool hvalid0 = qvalid && hl < p.group;       // before the query's own checks
  bf16x8 qf[kD / 16];
  {
    const uint16_t *qrow = p.q + ((int64_t)iq * p.hq + (int64_t)g * p.group + hl) * kD + 8 * hi;
#pragma unroll
    for (int kk = 0; kk < kD / 16; ++kk)
      qf[kk] = hvalid0 ? *(const bf16x8 *)(qrow + 16 * kk) : bf16x8{};
  }
  // with several slices the partials are sink-free; the merge adds the sink
  const float sink = (hvalid0 && p.sink != nullptr && S == 1) ? p.sink[g * p.group + hl] : -INFINITY;
  const int32_t topk = p.topk;                        // 0: no list
  const int32_t P = p.page_size;
  const int64_t hkv = p.hkv;
  int32_t U = 0;                                      // rows in the item's list
  int32_t wbase = 0;                                  // decode: first window row
  if constexpr (DEC) {
    // ---- a decode slice.  Slice s holds the compressed entries in list
    // slots [s*cper, (s+1)*cper) (cper = the list capacity, or the groups
    // the page table can hold for an all-groups layer, over S) and the
    // window entries [s*wper, (s+1)*wper) (wper = W over S), each cut at the
    // query's own counts; any partition gives the same result
    const int64_t cap = p.ratio == 0 ? 0 : topk > 0 ? topk : (int64_t)p.cmp_pt_stride * P;
    const int32_t cper = (int32_t)((cap + S - 1) / S);
    const int32_t wper = (p.window + S - 1) / S;
    const int32_t c0 = split * cper;
    int32_t ids[kRowIters];
#pragma unroll
    for (int it = 0; it < kRowIters; ++it) {
      const int e = tid + it * kThreads;
      ids[it] = (topk > 0 && e < cper && c0 + e < topk) ? p.cmp_idx[(int64_t)i0 * topk + c0 + e] : -1;
    }
    const QueryKV kv = query_kv(p, i0);
    if (topk == 0 && kv.n_sel > cap && split == 0 && tid == 0) flag_error(p, kErrPage);   // groups past the table
    const int32_t cs = min(c0, kv.n_sel), ce = min(c0 + cper, kv.n_sel);
    const int32_t ws = min(split * wper, kv.win_len), we = min(split * wper + wper, kv.win_len);
    const int32_t Uc = ce - cs;
    wbase = FP8 ? (Uc + kPT - 1) / kPT * kPT : Uc;   // first window row
    U = min(wbase + (we - ws), kUMax);
    const bool pow2 = p.page_shift >= 0;
    int32_t xs[kRowIters], pg[kRowIters];
#pragma unroll
    for (int it = 0; it < kRowIters; ++it) {
      const int r = tid + it * kThreads;
      int32_t x = -1;
      const int32_t *src = nullptr;
      if (r < U && (r < Uc || r >= wbase)) {
        const bool cmp = r < Uc;
        x = cmp ? (topk > 0 ? ids[it] : cs + r) : kv.win_lo + ws + (r - wbase);
        if (cmp && (x < 0 || x >= kv.n_c)) {
          flag_error(p, kErrCmpId);
          x = -1;
        }
        if (x >= 0) {
          const int32_t col = pow2 ? x >> p.page_shift : x / P;
          if (col < (cmp ? p.cmp_pt_stride : p.raw_pt_stride))
            src = cmp ? p.cmp_pt + (int64_t)kv.b * p.cmp_pt_stride + col : p.raw_pt + (int64_t)kv.b * p.raw_pt_stride + col;
          else {
            flag_error(p, kErrPage);
            x = -1;
          }
        }
      }
      xs[it] = x;
      pg[it] = src != nullptr ? *src : -1;
    }
#pragma unroll
    for (int it = 0; it < kRowIters; ++it) {
      const int r = tid + it * kThreads;
      if (r < (U + kPT - 1) / kPT * kPT) {
        const bool cmp = r < Uc;
        int64_t er = -1;
        if (r < U && xs[it] >= 0) {
          if (pg[it] >= 0 && (int64_t)pg[it] < (cmp ? p.cmp_pages : p.raw_pages)) {
            const int32_t col = pow2 ? xs[it] >> p.page_shift : xs[it] / P;
            er = (((int64_t)pg[it] * P + (xs[it] - col * P)) * hkv + g) | (cmp ? kCmpBit : 0);
          } else {
            flag_error(p, kErrPage);
          }
        }
        sm.row[r] = er;
        sm.flg[r] = (uint8_t)(er >= 0 ? 1u : 0u);
      }
    }
  } else {
    const int32_t mb0 = p.query_seq[i0], mt0 = p.query_pos[i0];
    const int32_t mb1 = has1 ? p.query_seq[i1] : -1, mt1 = has1 ? p.query_pos[i1] : -1;
    const int32_t mc0 = topk > 0 ? p.cmp_cnt[i0] : 0;
    const int32_t mc1 = (topk > 0 && has1) ? p.cmp_cnt[i1] : 0;
    int32_t ids[kRowIters];
#pragma unroll
    for (int it = 0; it < kRowIters; ++it) {
      const int e = tid + it * kThreads;
      const int q = e >= topk ? 1 : 0;
      ids[it] = (topk > 0 && e < 2 * topk && (q == 0 || has1))
                    ? p.cmp_idx[(int64_t)(q ? i1 : i0) * topk + (e - q * topk)] : -1;
    }

    // ---- the pair's KV sets, before the positions are checked against
    // seq_lens (those loads are issued now and checked after the build)
    const bool bok0 = mb0 >= 0 && mb0 < p.num_seqs;
    const bool bok1 = has1 && mb1 >= 0 && mb1 < p.num_seqs;
    const QueryKV pk0 = bok0 ? query_kv_of(p, mb0, mt0, INT32_MAX, mc0, false) : QueryKV{0, 0, 0, 0, 0, 0};
    const QueryKV pk1 = bok1 ? query_kv_of(p, mb1, mt1, INT32_MAX, mc1, false) : QueryKV{0, 0, 0, 0, 0, 0};
    const int32_t len0 = bok0 ? p.seq_lens[mb0] : 0;
    const int32_t len1 = bok1 ? p.seq_lens[mb1] : 0;

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
            sm.row[r] = er;
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
          sm.row[r] = er;
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
          sm.row[r] = er;
          sm.flg[r] = (uint8_t)(er >= 0 ? sel : 0u);
        }
      }
    }
  }   // pairs
  wait_vmcnt<0>();                           // Q fragments, sink and every setup load are in
  __syncthreads();                           // rows and flags complete; bitmaps and slices dead

  // a query that failed its checks computes nothing and writes O = 0 and
  // LSE = sink (its rows are all unselected); the lanes write only real heads
  const bool hvalid = hvalid0;

  // ---- tile loads: wave w moves rows 8w .. 8w+7 of both sides (two 1 KiB
  // direct loads per side, four rows each); the 16-byte chunk of lane L in
  // load n is logical chunk (L % 16) ^ swz(row), row = 8w + 4n + L / 16.
  // The pool rows of the next tile to issue are read one step ahead.
  const uint8_t *const kraw = in_sgpr(p.k_raw), *const vraw = in_sgpr(p.v_raw);
  const uint8_t *const kcmp = in_sgpr(p.k_cmp), *const vcmp = in_sgpr(p.v_cmp);
  int32_t csrc[2];
#pragma unroll
  for (int n = 0; n < 2; ++n) {
    const int r = 8 * wave + 4 * n + lane / kChunks;
    csrc[n] = ((lane % kChunks) ^ swz<kChunks>(r)) * 16;
  }
  const int32_t ntiles = (U + kPT - 1) / kPT;
  const int32_t nf8 = FP8 ? wbase / kPT : 0;         // tiles 0 .. nf8-1 hold e4m3 rows
  const bool fnuz = FP8 && p.cmp_fnuz != 0;          // e4m3 pages in the FNUZ variant
  int64_t nrow[2];
  // an e4m3 tile: wave w moves rows 8w .. 8w+7 of D bytes per side (one
  // 1 KiB load each, lane L: row 8w + L / 8, bytes 16 (L % 8) ..), into the
  // staging area; waves 0 and 1 also load the 32 k and v scales
  auto fetch_rows = [&](int j) {
    if (FP8 && j < nf8) {
      nrow[0] = sm.row[kPT * j + 8 * wave + lane / 8];
      nrow[1] = sm.row[kPT * j + (lane & 31)];
      return;
    }
#pragma unroll
    for (int n = 0; n < 2; ++n) nrow[n] = j < ntiles ? sm.row[kPT * j + 8 * wave + 4 * n + lane / kChunks] : -1;
  };
  auto issue = [&](int j) {
    const int st = j % NST;
    if (FP8 && j < nf8) {
      const int64_t er = nrow[0];
      const int64_t off = (er & ~kCmpBit) * kD + (lane % 8) * 16;
      dma16(er >= 0 ? kcmp + off : kZeroRow + (lane % 8) * 16, sm.f8k[FP8 ? st : 0] + 1024 * wave);
      dma16(er >= 0 ? vcmp + off : kZeroRow + (lane % 8) * 16, sm.f8v[FP8 ? st : 0] + 1024 * wave);
      if (wave < 2) {
        const int64_t es = nrow[1];
        const float *scl = wave == 0 ? p.k_cmp_scale : p.v_cmp_scale;
        dma4(lane < kPT && es >= 0 ? (const void *)(scl + (es & ~kCmpBit)) : (const void *)(kZeroRow + 4 * lane),
             wave == 0 ? sm.f8sk[FP8 ? st : 0] : sm.f8sv[FP8 ? st : 0]);
      }
      return;
    }
    const uint8_t *ks[2], *vs[2];
#pragma unroll
    for (int n = 0; n < 2; ++n) {
      const int64_t er = nrow[n];
      const bool cmp = (er & kCmpBit) != 0;
      const int64_t off = (er & ~kCmpBit) * kRowB + csrc[n];
      ks[n] = er >= 0 ? (cmp ? kcmp : kraw) + off : kZeroRow + csrc[n];
      vs[n] = er >= 0 ? (cmp ? vcmp : vraw) + off : kZeroRow + csrc[n];
    }
#pragma unroll
    for (int n = 0; n < 2; ++n) dma16(ks[n], sm.u.t.k[st] + (8 * wave + 4 * n) * kRowB);
#pragma unroll
    for (int n = 0; n < 2; ++n) dma16(vs[n], sm.u.t.v[st] + (8 * wave + 4 * n) * kRowB);
  };

  // ---- per-lane softmax state; the sink initialises (m, l)
  float m = sink == -INFINITY ? -INFINITY : sink * kLog2e;
  float l = (sink != -INFINITY && hi == 0) ? 1.f : 0.f;   // exp2(sink - m) = 1, counted once per head
  f32x16 acc[kD / 32];
#pragma unroll
  for (int db = 0; db < kD / 32; ++db) acc[db] = f32x16{};

  // One tile: every K and V fragment of the tile is read from LDS first (the
  // V transpose reads are in flight during the scores and the softmax), then
  // S^T = K . Q^T, the online softmax of the scores (rows not selected by
  // this wave's query masked to -inf) and O^T += V^T . P^T.  Lane rows of
  // S^T: 8*(i/4) + 4*hi + i%4.
  auto tile = [&](int st, uint32_t tm, bool f8) {
    const uint8_t *Kt = sm.u.t.k[st];
    const uint8_t *Vt = sm.u.t.v[st];
    bf16x8 kf[kD / 16];
    {
      const int r = lane & 31;
#pragma unroll
      for (int kk = 0; kk < kD / 16; ++kk) {
        const int c = 2 * kk + hi;
        kf[kk] = *(const bf16x8 *)(Kt + r * kRowB + ((c ^ swz<kChunks>(r)) * 16));
      }
    }
    i16x4 vf[kD / 32][2][2];
    {
      const int G = lane >> 4;
      const int L = lane & 15;
#pragma unroll
      for (int db = 0; db < kD / 32; ++db)
#pragma unroll
        for (int k2 = 0; k2 < 2; ++k2)
#pragma unroll
          for (int rr = 0; rr < 2; ++rr) {
            const int row = 16 * k2 + 8 * rr + 4 * (G >> 1) + (L >> 2);
            const int d = 32 * db + 16 * (G & 1) + 4 * (L & 3);
            const int off = row * kRowB + (((d >> 3) ^ swz<kChunks>(row)) * 16) + (L & 1) * 8;
            vf[db][k2][rr] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t *)(Vt + off));
          }
    }
    f32x16 s = f32x16{};
#pragma unroll
    for (int kk = 0; kk < kD / 16; ++kk) s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[kk], qf[kk], s, 0, 0, 0);

    float sc[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) sc[i] = s[i];
    if (FP8 && f8) {
      // the k scale of each row multiplies the fp32 score of its exact code
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const float4 k4 = *(const float4 *)(&sm.f8sk[FP8 ? st : 0][8 * q4 + 4 * hi]);
        sc[4 * q4 + 0] *= k4.x;
        sc[4 * q4 + 1] *= k4.y;
        sc[4 * q4 + 2] *= k4.z;
        sc[4 * q4 + 3] *= k4.w;
      }
    }
    const uint32_t tmh = tm >> (4 * hi);
#pragma unroll
    for (int i = 0; i < 16; ++i) sc[i] = ((tmh >> (8 * (i >> 2) + (i & 3))) & 1u) ? sc[i] : -INFINITY;
    float smax = fmaxf(fmaxf(fmaxf(sc[0], sc[1]), fmaxf(sc[2], sc[3])), fmaxf(fmaxf(sc[4], sc[5]), fmaxf(sc[6], sc[7])));
    smax = fmaxf(smax, fmaxf(fmaxf(fmaxf(sc[8], sc[9]), fmaxf(sc[10], sc[11])),
                             fmaxf(fmaxf(sc[12], sc[13]), fmaxf(sc[14], sc[15]))));
    smax = max_lane_pair(smax);
    const float tmax = smax * p.scale_log2;
    const bool need = tmax > m + kTau;
    if (__any(need)) {
      const float alpha = need ? __builtin_amdgcn_exp2f(m - tmax) : 1.f;
      m = need ? tmax : m;
      l *= alpha;
#pragma unroll
      for (int db = 0; db < kD / 32; ++db) acc[db] *= alpha;
    }
    const float negm = m == -INFINITY ? 0.f : -m;
    float pr[16];
    float psum = 0.f;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      pr[i] = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[i], p.scale_log2, negm));
      psum += pr[i];
    }
    l += psum;
    if (FP8 && f8) {
      // the v scale of each row multiplies p before its bf16 rounding
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const float4 v4 = *(const float4 *)(&sm.f8sv[FP8 ? st : 0][8 * q4 + 4 * hi]);
        pr[4 * q4 + 0] *= v4.x;
        pr[4 * q4 + 1] *= v4.y;
        pr[4 * q4 + 2] *= v4.z;
        pr[4 * q4 + 3] *= v4.w;
      }
    }
    bf16x8 pb[2];
#pragma unroll
    for (int k2 = 0; k2 < 2; ++k2)
#pragma unroll
      for (int j = 0; j < 8; ++j) pb[k2][j] = (__bf16)pr[8 * k2 + j];
#pragma unroll
    for (int db = 0; db < kD / 32; ++db)
#pragma unroll
      for (int k2 = 0; k2 < 2; ++k2) {
        const i16x8 cat = {vf[db][k2][0][0], vf[db][k2][0][1], vf[db][k2][0][2], vf[db][k2][0][3],
                           vf[db][k2][1][0], vf[db][k2][1][1], vf[db][k2][1][2], vf[db][k2][1][3]};
        acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, cat), pb[k2], acc[db], 0, 0, 0);
      }
  };

  // ---- the tile loop
  fetch_rows(0);
#pragma unroll
  for (int j = 0; j < NST - 1; ++j) {
    if (j < ntiles) issue(j);
    fetch_rows(j + 1);
  }
  for (int j = 0; j < ntiles; ++j) {
    // this wave's selection mask of tile j
    const uint32_t tm = (uint32_t)__ballot(lane < 32 && ((sm.flg[kPT * j + (lane & 31)] >> qw) & 1u));
    // this wave's loads of tile j are complete (those of the next NST-2
    // tiles may still be in flight; four loads per tile) ...
    const int ahead = min(NST - 2, ntiles - 1 - j);
    if (ahead >= 2) wait_vmcnt<8>();
    else if (ahead == 1) wait_vmcnt<4>();
    else wait_vmcnt<0>();
    // ... and, after the barrier, every wave's: tile j is in LDS, and every
    // wave is done with tile j-1, whose stage the next load refills
    block_sync();
    const bool f8 = FP8 && j < nf8;
    if (FP8 && f8) {
      // widen the staged e4m3 tile into the bf16 tile of its stage (exact),
      // in the swizzled layout of a bf16 tile: 8 codes per thread and step
      const int st = j % NST;
#pragma unroll
      for (int side = 0; side < 2; ++side) {
        const uint8_t *src = side ? sm.f8v[FP8 ? st : 0] : sm.f8k[FP8 ? st : 0];
        uint8_t *dst = side ? sm.u.t.v[st] : sm.u.t.k[st];
#pragma unroll
        for (int it = 0; it < kPT * kD / 8 / kThreads; ++it) {
          const int idx = tid + it * kThreads;
          const int r = idx / (kD / 8);
          const int piece = idx - r * (kD / 8);
          const uint2 w = *(const uint2 *)(src + r * kD + piece * 8);
          f32x2 a0 = __builtin_amdgcn_cvt_pk_f32_fp8((int)w.x, false);
          f32x2 a1 = __builtin_amdgcn_cvt_pk_f32_fp8((int)w.x, true);
          f32x2 a2 = __builtin_amdgcn_cvt_pk_f32_fp8((int)w.y, false);
          f32x2 a3 = __builtin_amdgcn_cvt_pk_f32_fp8((int)w.y, true);
          if (fnuz) {
            // FNUZ code c is OCP code c halved (bias 8 against 7), except
            // 0x7F / 0xFF (+-240; OCP NaN) and 0x80 (NaN; OCP -0)
            auto fix = [](float x, uint32_t word, int byte) {
              const uint32_t c = (word >> (8 * byte)) & 0xFFu;
              return (c & 0x7Fu) == 0x7Fu ? ((c & 0x80u) ? -240.f : 240.f)
                     : c == 0x80u          ? __builtin_bit_cast(float, 0x7FC00000u)
                                           : 0.5f * x;
            };
            a0 = f32x2{fix(a0[0], w.x, 0), fix(a0[1], w.x, 1)};
            a1 = f32x2{fix(a1[0], w.x, 2), fix(a1[1], w.x, 3)};
            a2 = f32x2{fix(a2[0], w.y, 0), fix(a2[1], w.y, 1)};
            a3 = f32x2{fix(a3[0], w.y, 2), fix(a3[1], w.y, 3)};
          }
          uint4 o;
          o.x = pack_bf16_hi(a0[0], a0[1]);
          o.y = pack_bf16_hi(a1[0], a1[1]);
          o.z = pack_bf16_hi(a2[0], a2[1]);
          o.w = pack_bf16_hi(a3[0], a3[1]);
          *(uint4 *)(dst + r * kRowB + ((piece ^ swz<kChunks>(r)) * 16)) = o;
        }
      }
      block_sync();                          // the widened tile is in
    }
    if (j + NST - 1 < ntiles) {
      issue(j + NST - 1);
      fetch_rows(j + NST);
    }
    tile(j % NST, tm, f8);
  }

  // ---- epilogue: O = acc / l (bf16, RNE), LSE = (m + log2 l) ln 2
  const float lt = l + __shfl_xor(l, 32);
  const float inv = lt > 0.f ? 1.f / lt : 0.f;
  const float lse2 = (m == -INFINITY || !(lt > 0.f)) ? -INFINITY : m + __builtin_amdgcn_logf(lt);
  const float lse = lse2 == -INFINITY ? -INFINITY : lse2 * kLn2;
  if (!hvalid) return;
  const int64_t h = (int64_t)g * p.group + hl;
  if (DEC && S > 1) {
    // a slice's sink-free partial: O_s = acc / l in fp32 and LSE_s (-inf
    // for an empty slice, whose weight in the merge is then 0)
    const int64_t prow = ((int64_t)split * p.num_queries + iq) * p.hq + h;
    float *prow_o = p.part_o + prow * kD;
#pragma unroll
    for (int db = 0; db < kD / 32; ++db) {
#pragma unroll
      for (int i4 = 0; i4 < 4; ++i4) {
        const int d0 = 32 * db + 8 * i4 + 4 * hi;
        *(float4 *)(prow_o + d0) = make_float4(acc[db][4 * i4] * inv, acc[db][4 * i4 + 1] * inv,
                                               acc[db][4 * i4 + 2] * inv, acc[db][4 * i4 + 3] * inv);
      }
    }
    if (hi == 0) p.part_lse[prow] = lse;
    return;
  }
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
  hipLaunchKernelGGL((attn_pair_kernel<kPairStages, false, false>), dim3((unsigned)grid), dim3(kThreads), 0, stream, p);
  return hipGetLastError();
}

bool decode_slices_eligible(const Params &p) {
  if (p.head_dim != kD || p.query_seq != nullptr || p.query_pos != nullptr || p.num_splits < 1) return false;
  const int64_t S = p.num_splits;
  const int64_t cap = p.ratio == 0 ? 0 : p.topk > 0 ? p.topk : (int64_t)p.cmp_pt_stride * p.page_size;
  int64_t cper = (cap + S - 1) / S;
  if (p.cmp_fp8) cper = (cper + kPT - 1) / kPT * kPT;   // e4m3 rows fill whole tiles
  return cper + (p.window + S - 1) / S <= kUMax;
}

hipError_t launch_decode_slices(const Params &p, hipStream_t stream) {
  if (p.num_queries == 0) return hipSuccess;
  if (!decode_slices_eligible(p)) return hipErrorInvalidConfiguration;
  const int64_t grid = (int64_t)p.num_queries * p.hkv * ((p.group + 127) / 128) * p.num_splits;
  if (grid > 0x7FFFFFFFLL) return hipErrorInvalidConfiguration;
  if (p.cmp_fp8)
    hipLaunchKernelGGL((attn_pair_kernel<2, true, true>), dim3((unsigned)grid), dim3(kThreads), 0, stream, p);
  else
    hipLaunchKernelGGL((attn_pair_kernel<kDecodeStages, true, false>), dim3((unsigned)grid), dim3(kThreads), 0, stream, p);
  return hipGetLastError();
}

}  // namespace spa
