// Decode (one query token per sequence) for gfx950.
//
// Operation: sparse paged attention with a sink (RL-Kernel PR "Roadmap item
// 24: joint compressed/window attention with sink", section "Reuse and
// arithmetic"; KV-set and translation rules in spa_device.h), D 128, bf16 raw
// pages and bf16 or e4m3 (OCP or FNUZ) compressed pages with a per-row fp32
// scale.  With several KV slices each slice writes a sink-free partial
// (O_s, LSE_s) that the LSE merge kernel combines with the sink (RL-Kernel
// "[WS2] CP-aware Attention contract", Behavior: a deterministic (out, lse)
// reduction).
//
// One workgroup of four waves per (query, KV head, block of 128 query heads,
// KV slice); wave w computes heads 32w .. 32w+31 of the block (the MFMA's N)
// on every tile of the slice, one wave per SIMD.
//
// Setup has two dependent round trips before the first score:
//   1. issued together: the query's metadata (sequence length, list count),
//      the slice's list slots and both page-table rows of the sequence
//      (direct loads into LDS, when the rows fit), and the Q fragments;
//   2. one thread per slice row forms its 64-bit pool row (row * Hkv + g,
//      bit 62 for the compressed pool, -1 when masked), then every wave
//      issues its share of every tile's direct global->LDS loads at once.
// A slice's tiles are all in flight together whenever they fit the LDS
// stages (NST of them); a longer slice refills the stages of the previous
// step's tiles after each barrier.  e4m3 tiles land in a staging area with
// their row scales and are widened to bf16 in LDS after their barrier (every
// e4m3 value is a bf16 value, so this is exact); the k scale multiplies the
// fp32 score of the exact code and the v scale multiplies p before its bf16
// rounding.
//
// The tiles are taken two at a time: the two score products S^T = K.Q^T
// (v_mfma_f32_32x32x16_bf16, Q^T in registers) are independent chains that
// the matrix core interleaves, one online-softmax update in the log2 domain
// covers both (the sink folded into the running (m, l), a lazy rescale of
// O), then O^T += V^T.P^T for both (V^T by the transposing LDS read).

#include <hip/hip_runtime.h>

#include <cstdint>
#include <type_traits>

#include "spa_device.h"
#include "spa_kernel_util.h"

namespace spa {
namespace {

constexpr int kD = 128;
constexpr int kRowB = 2 * kD;              // bf16 row bytes
constexpr int kChunks = kRowB / 16;        // 16-byte chunks per row
constexpr int kPT = 32;                    // rows per tile
constexpr int kTileB = kPT * kRowB;        // one K (or V) tile
constexpr int kF8TileB = kPT * kD;         // one e4m3 tile side
constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kHeads = 128;                // query heads per workgroup
constexpr int kRowsMax = kDecodeRowsMax;   // rows of one slice
constexpr int kPtLds = 2048;               // page-table entries staged in LDS
constexpr int64_t kCmpBit = int64_t(1) << 62;

template <bool FP8>
struct Stages {
  static constexpr int n = FP8 ? 5 : 8;
};

template <bool FP8>
struct DecodeSmem {
  static constexpr int NST = Stages<FP8>::n;
  alignas(16) uint8_t k[NST][kTileB];
  alignas(16) uint8_t v[NST][kTileB];
  alignas(16) uint8_t f8[FP8 ? NST : 1][FP8 ? 2 * kF8TileB : 16];   // e4m3 codes: K side, then V side
  alignas(16) float f8s[FP8 ? NST : 1][64];                         // 32 k scales, then 32 v scales
  alignas(16) int64_t row[kRowsMax];           // pool rows of the slice, padded to whole tiles
  alignas(16) int32_t ids[kRowsMax];           // the slice's list slots
  alignas(16) int32_t pt[kPtLds];              // raw page-table row, then the compressed one
};

// s_waitcnt vmcnt(n) for a run-time n (0 .. 32; a larger n waits for 32)
template <int N>
__device__ __forceinline__ void wait_vmcnt_le_rec(int n) {
  if constexpr (N == 32) {
    wait_vmcnt<32>();
  } else {
    if (n <= N) wait_vmcnt<N>();
    else wait_vmcnt_le_rec<N + 1>(n);
  }
}
__device__ __forceinline__ void wait_vmcnt_le(int n) { wait_vmcnt_le_rec<0>(n); }

template <bool FP8>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(1)))
void attn_decode_kernel(const Params p) {
  constexpr int NST = Stages<FP8>::n;
  static_assert(NST >= 4, "a step's two tiles are issued one step ahead");
  __shared__ DecodeSmem<FP8> sm;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int hi = lane >> 5;
  const int32_t S = p.num_splits;

  // workgroup -> (query i, KV head g, head block hb, slice)
  const uint32_t hblocks = (uint32_t)(p.group + kHeads - 1) / kHeads;
  uint32_t wg = blockIdx.x;                  // the grid is below 2^31
  const int32_t split = (int32_t)(wg % (uint32_t)S);
  wg /= (uint32_t)S;
  const int32_t hb = (int32_t)(wg % hblocks);
  wg /= hblocks;
  const int32_t g = (int32_t)(wg % (uint32_t)p.hkv);
  const int32_t i = (int32_t)(wg / (uint32_t)p.hkv);
  const int32_t b = i;                       // decode: query i is sequence i's last token

  // ---- round trip 1, everything issued together: the metadata (vector
  // loads: lane 0 the sequence length, lane 1 the list count), the slice's
  // list slots and the page-table rows (into LDS), the Q fragments of this
  // lane's head
  const int32_t topk = p.topk;
  const bool has_list = p.ratio > 0 && topk > 0;
  const int32_t meta = *((lane == 1 && has_list) ? p.cmp_cnt + i : p.seq_lens + b);
  const int32_t P = p.page_size;
  const int64_t cap = p.ratio == 0 ? 0 : topk > 0 ? topk : (int64_t)p.cmp_pt_stride * P;
  const int32_t cper = (int32_t)((cap + S - 1) / S);
  const int32_t wper = (p.window + S - 1) / S;
  const int32_t c0 = split * cper;
  if (topk > 0) {
    for (int c = wave; 64 * c < cper; c += kWaves) {
      const int e = 64 * c + lane;
      const void *src = (e < cper && c0 + e < topk) ? (const void *)(p.cmp_idx + (int64_t)i * topk + c0 + e)
                                                    : (const void *)kZeroRow;
      dma4(src, &sm.ids[64 * c]);
    }
  }
  const int32_t nr = p.raw_pt_stride;
  const int32_t nc = p.ratio > 0 ? p.cmp_pt_stride : 0;
  const bool stage_pt = nr + nc <= kPtLds;
  if (stage_pt) {
    for (int c = wave; 64 * c < nr + nc; c += kWaves) {
      const int k = 64 * c + lane;
      const void *src = k < nr        ? (const void *)(p.raw_pt + (int64_t)b * nr + k)
                        : k < nr + nc ? (const void *)(p.cmp_pt + (int64_t)b * nc + (k - nr))
                                      : (const void *)kZeroRow;
      dma4(src, &sm.pt[64 * c]);
    }
  }
  const int hl = hb * kHeads + wave * 32 + (lane & 31);   // head within the KV group
  const bool hvalid = hl < p.group;
  bf16x8 qf[kD / 16];
  {
    const uint16_t *qrow = p.q + ((int64_t)i * p.hq + (int64_t)g * p.group + hl) * kD + 8 * hi;
#pragma unroll
    for (int kk = 0; kk < kD / 16; ++kk) qf[kk] = hvalid ? *(const bf16x8 *)(qrow + 16 * kk) : bf16x8{};
  }
  // one slice: the sink initialises (m, l); several: the merge adds it
  const float sink = (hvalid && p.sink != nullptr && S == 1) ? p.sink[g * p.group + hl] : -INFINITY;
  wait_vmcnt<0>();
  block_sync();                              // list slots and page-table rows in LDS
  const int32_t len_b = __builtin_amdgcn_readfirstlane(meta);
  const int32_t cnt_i = has_list ? __builtin_amdgcn_readlane(meta, 1) : 0;
  const QueryKV kv = query_kv_of(p, b, len_b - 1, len_b, cnt_i, tid == 0);

  // ---- the slice: list slots [c0, c0 + cper) and window slots
  // [split * wper, ...), each cut at the query's own counts; with e4m3 pages
  // the window starts at the next tile edge
  if (topk == 0 && kv.n_sel > cap && split == 0 && tid == 0) flag_error(p, kErrPage);   // groups past the table
  const int32_t cs = min(c0, kv.n_sel), ce = min(c0 + cper, kv.n_sel);
  const int32_t ws = min(split * wper, kv.win_len), we = min(split * wper + wper, kv.win_len);
  const int32_t Uc = ce - cs;
  const int32_t wbase = FP8 ? round_up(Uc, kPT) : Uc;   // first window row
  const int32_t U = min(wbase + (we - ws), kRowsMax);
  const int32_t T = (U + kPT - 1) / kPT;
  const int32_t nf8 = FP8 ? wbase / kPT : 0;           // tiles 0 .. nf8-1 hold e4m3 rows

  // ---- translation: one thread per row; the page ids come from LDS, or
  // from the page tables when their rows did not fit
  {
    const bool pow2 = p.page_shift >= 0;
    for (int r = tid; r < T * kPT; r += kThreads) {
      const bool cmp = r < Uc;
      int32_t x = -1, col = -1;
      if (r < U && (r < Uc || r >= wbase)) {
        x = cmp ? (topk > 0 ? sm.ids[r] : cs + r) : kv.win_lo + ws + (r - wbase);
        if (cmp && (x < 0 || x >= kv.n_c)) {
          flag_error(p, kErrCmpId);
          x = -1;
        }
        if (x >= 0) {
          col = pow2 ? x >> p.page_shift : x / P;
          if (col >= (cmp ? nc : nr)) {
            flag_error(p, kErrPage);
            x = -1;
          }
        }
      }
      int64_t er = -1;
      if (x >= 0) {
        const int32_t page = stage_pt ? sm.pt[cmp ? nr + col : col]
                                      : (cmp ? p.cmp_pt + (int64_t)b * nc : p.raw_pt + (int64_t)b * nr)[col];
        if (page >= 0 && (int64_t)page < (cmp ? p.cmp_pages : p.raw_pages))
          er = (((int64_t)page * P + (x - col * P)) * p.hkv + g) | (cmp ? kCmpBit : 0);
        else
          flag_error(p, kErrPage);
      }
      sm.row[r] = er;
    }
  }
  block_sync();                              // rows in LDS

  // ---- tile loads.  A bf16 tile: wave w moves rows 8w .. 8w+7 of both
  // sides (two 1 KiB direct loads per side; lane L of load n: row 8w + 4n +
  // L / 16, logical chunk (L % 16) ^ swz(row), so the rows land
  // XOR-swizzled).  An e4m3 tile: wave w moves K rows 8w .. 8w+7 and the same
  // V rows (one 1 KiB load per side; lane L: row 8w + L / 8, bytes
  // 16 (L % 8) ..), and wave 0 also the 64 row scales (lanes 0-31 k, 32-63 v).
  const uint8_t *const kraw = in_sgpr(p.k_raw), *const vraw = in_sgpr(p.v_raw);
  const uint8_t *const kcmp = in_sgpr(p.k_cmp), *const vcmp = in_sgpr(p.v_cmp);
  int csrc[2];
#pragma unroll
  for (int n = 0; n < 2; ++n) csrc[n] = ((lane % kChunks) ^ swz<kChunks>(8 * wave + 4 * n + lane / kChunks)) * 16;
  auto nloads = [&](int j) { return (FP8 && j < nf8) ? (wave == 0 ? 3 : 2) : 4; };
  auto issue_bf16 = [&](int st, int64_t er0, int64_t er1) {
    const int64_t ers[2] = {er0, er1};
#pragma unroll
    for (int n = 0; n < 2; ++n) {
      const int64_t er = ers[n];
      const bool cmp = (er & kCmpBit) != 0;
      const int64_t off = (er & ~kCmpBit) * kRowB + csrc[n];
      dma16(er >= 0 ? (cmp ? kcmp : kraw) + off : kZeroRow + csrc[n], sm.k[st] + (8 * wave + 4 * n) * kRowB);
    }
#pragma unroll
    for (int n = 0; n < 2; ++n) {
      const int64_t er = ers[n];
      const bool cmp = (er & kCmpBit) != 0;
      const int64_t off = (er & ~kCmpBit) * kRowB + csrc[n];
      dma16(er >= 0 ? (cmp ? vcmp : vraw) + off : kZeroRow + csrc[n], sm.v[st] + (8 * wave + 4 * n) * kRowB);
    }
  };
  auto issue = [&](int j) {
    const int st = j % NST;
    if (FP8 && j < nf8) {
      // both rows first: the loads' memory clobber keeps a later LDS read
      // from starting ahead of them
      const int64_t er = sm.row[kPT * j + 8 * wave + lane / 8];
      const int64_t es = wave == 0 ? sm.row[kPT * j + (lane & 31)] : -1;
      const int64_t off = (er & ~kCmpBit) * kD + (lane % 8) * 16;
      uint8_t *dst = sm.f8[FP8 ? st : 0] + wave * 1024;
      dma16(er >= 0 ? kcmp + off : kZeroRow + (lane % 8) * 16, dst);
      dma16(er >= 0 ? vcmp + off : kZeroRow + (lane % 8) * 16, dst + kF8TileB);
      if (wave == 0) {
        const float *scl = lane < 32 ? p.k_cmp_scale : p.v_cmp_scale;
        dma4(es >= 0 ? (const void *)(scl + (es & ~kCmpBit)) : (const void *)(kZeroRow + 4 * (lane & 31)),
             sm.f8s[FP8 ? st : 0]);
      }
      return;
    }
    issue_bf16(st, sm.row[kPT * j + 8 * wave + lane / kChunks], sm.row[kPT * j + 8 * wave + 4 + lane / kChunks]);
  };

  // ---- per-lane softmax state; the sink initialises (m, l)
  float m = sink == -INFINITY ? -INFINITY : sink * kLog2e;
  float l = (sink != -INFINITY && hi == 0) ? 1.f : 0.f;   // exp2(sink - m) = 1, counted once per head
  f32x16 acc[kD / 32];
#pragma unroll
  for (int db = 0; db < kD / 32; ++db) acc[db] = f32x16{};

  // NT tiles (stages st[t], row masks tm[t], e4m3 flags f8[t]): the K
  // fragments of all of them, the NT score chains interleaved, the V^T
  // fragments (transposing reads, in flight during the softmax), one online
  // softmax update over the NT * 16 scores of each lane, O^T += V^T.P^T.
  // Lane rows of S^T: 8*(q/4) + 4*hi + q%4.
  auto tiles = [&](auto NTc, const int *st, const uint32_t *tm, const bool *f8) {
    constexpr int NT = decltype(NTc)::value;
    bf16x8 kf[NT][kD / 16];
    {
      const int r = lane & 31;
#pragma unroll
      for (int t = 0; t < NT; ++t)
#pragma unroll
        for (int kk = 0; kk < kD / 16; ++kk) {
          const int c = 2 * kk + hi;
          kf[t][kk] = *(const bf16x8 *)(sm.k[st[t]] + r * kRowB + ((c ^ swz<kChunks>(r)) * 16));
        }
    }
    f32x16 s[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t) s[t] = f32x16{};
#pragma unroll
    for (int kk = 0; kk < kD / 16; ++kk)
#pragma unroll
      for (int t = 0; t < NT; ++t) s[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[t][kk], qf[kk], s[t], 0, 0, 0);
    // V^T operands: two transposing reads (rows 8rw + ..) fill the two
    // halves of each 8-element operand
    i16x8 vf[NT][kD / 32][2];
    {
      const int G = lane >> 4;
      const int L = lane & 15;
#pragma unroll
      for (int t = 0; t < NT; ++t)
#pragma unroll
        for (int db = 0; db < kD / 32; ++db)
#pragma unroll
          for (int k2 = 0; k2 < 2; ++k2) {
            i16x4 h[2];
#pragma unroll
            for (int rw = 0; rw < 2; ++rw) {
              const int row = 16 * k2 + 8 * rw + 4 * (G >> 1) + (L >> 2);
              const int d = 32 * db + 16 * (G & 1) + 4 * (L & 3);
              const int off = row * kRowB + (((d >> 3) ^ swz<kChunks>(row)) * 16) + (L & 1) * 8;
              h[rw] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t *)(sm.v[st[t]] + off));
            }
            vf[t][db][k2] = __builtin_shufflevector(h[0], h[1], 0, 1, 2, 3, 4, 5, 6, 7);
          }
    }
    float sc[NT][16];
    float smax = -INFINITY;
#pragma unroll
    for (int t = 0; t < NT; ++t) {
#pragma unroll
      for (int q = 0; q < 16; ++q) sc[t][q] = s[t][q];
      if (FP8 && f8[t]) {
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          const float4 k4 = *(const float4 *)(&sm.f8s[FP8 ? st[t] : 0][8 * q4 + 4 * hi]);
          sc[t][4 * q4 + 0] *= k4.x;
          sc[t][4 * q4 + 1] *= k4.y;
          sc[t][4 * q4 + 2] *= k4.z;
          sc[t][4 * q4 + 3] *= k4.w;
        }
      }
      mask_tile_rows(sc[t], tm[t]);
#pragma unroll
      for (int q = 0; q < 16; ++q) smax = fmaxf(smax, sc[t][q]);
    }
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
    bf16x8 pb[NT][2];
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      float pr[16];
#pragma unroll
      for (int q = 0; q < 16; ++q) {
        pr[q] = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[t][q], p.scale_log2, negm));
        l += pr[q];
      }
      if (FP8 && f8[t]) {
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          const float4 v4 = *(const float4 *)(&sm.f8s[FP8 ? st[t] : 0][32 + 8 * q4 + 4 * hi]);
          pr[4 * q4 + 0] *= v4.x;
          pr[4 * q4 + 1] *= v4.y;
          pr[4 * q4 + 2] *= v4.z;
          pr[4 * q4 + 3] *= v4.w;
        }
      }
#pragma unroll
      for (int k2 = 0; k2 < 2; ++k2)
#pragma unroll
        for (int q = 0; q < 8; ++q) pb[t][k2][q] = (__bf16)pr[8 * k2 + q];
    }
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
      for (int db = 0; db < kD / 32; ++db)
#pragma unroll
        for (int k2 = 0; k2 < 2; ++k2)
          acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, vf[t][db][k2]), pb[t][k2],
                                                           acc[db], 0, 0, 0);
  };

  // ---- the tile loop, two tiles a step
  const bool fnuz = FP8 && p.cmp_fnuz != 0;
  int issued = min(T, NST);
  {
    // every tile that fits the stages, its rows read from LDS together
    int64_t er0[NST][2];
#pragma unroll
    for (int j = 0; j < NST; ++j)
#pragma unroll
      for (int n = 0; n < 2; ++n)
        er0[j][n] = (j < issued && !(FP8 && j < nf8)) ? sm.row[kPT * j + 8 * wave + 4 * n + lane / kChunks] : 0;
#pragma unroll
    for (int j = 0; j < NST; ++j) {
      if (j < issued) {
        if (FP8 && j < nf8) issue(j);
        else issue_bf16(j, er0[j][0], er0[j][1]);
      }
    }
  }
  // When every tile is in flight (the slice fits the stages), one wait and
  // one barrier cover all of them and the waves then run through the tiles
  // without meeting again, so that one wave's LDS reads overlap another's
  // matrix products; a longer slice waits and meets once per step to reuse
  // stages.
  const bool all_in = T <= NST;
  if (all_in) {
    wait_vmcnt<0>();
    block_sync();
  }
  for (int j = 0; j < T; j += 2) {
    const int nt = min(2, T - j);
    if (!all_in) {
      // this wave's loads of the step's tiles are complete (those of later
      // tiles may be in flight) ...
      int pend = 0;
      for (int t = j + nt; t < issued; ++t) pend += nloads(t);
      wait_vmcnt_le(pend);
      // ... and, after the barrier, every wave's; every wave is also done
      // with the previous step's tiles, whose stages take the next tiles
      block_sync();
      for (; issued < T && issued < j + NST; ++issued) issue(issued);
    }
    if (FP8 && (all_in ? j == 0 : j < nf8) && nf8 > 0) {
      // widen e4m3 tiles into their bf16 stages (exact), in the swizzled
      // layout, 8 codes per thread and pass: every e4m3 tile at once when
      // all are in, else the step's
      const int j0 = all_in ? 0 : j;
      const int nw = all_in ? nf8 : min(nf8, j + nt) - j;
      for (int idx = tid; idx < nw * 2 * kPT * (kD / 8); idx += kThreads) {
        const int jj = j0 + idx / (2 * kPT * (kD / 8));
        const int rem = idx % (2 * kPT * (kD / 8));
        const int side = rem / (kPT * (kD / 8));
        const int r = (rem / (kD / 8)) % kPT;
        const int piece = rem % (kD / 8);
        const int st = jj % NST;
        const uint2 w = *(const uint2 *)(sm.f8[FP8 ? st : 0] + side * kF8TileB + r * kD + piece * 8);
        const uint4 o = widen8_e4m3(w, fnuz);
        uint8_t *dst = side ? sm.v[st] : sm.k[st];
        *(uint4 *)(dst + r * kRowB + ((piece ^ swz<kChunks>(r)) * 16)) = o;
      }
      block_sync();                          // the widened tiles are in
    }
    const int st[2] = {j % NST, (j + 1) % NST};
    const uint32_t tm[2] = {(uint32_t)__ballot(lane < 32 && sm.row[kPT * j + (lane & 31)] >= 0),
                            nt > 1 ? (uint32_t)__ballot(lane < 32 && sm.row[kPT * (j + 1) + (lane & 31)] >= 0) : 0u};
    const bool f8[2] = {FP8 && j < nf8, FP8 && j + 1 < nf8};
    if (nt == 2) tiles(std::integral_constant<int, 2>{}, st, tm, f8);
    else tiles(std::integral_constant<int, 1>{}, st, tm, f8);
  }

  // ---- epilogue: O = acc / l (bf16, RNE), LSE = (m + log2 l) ln 2; with
  // several slices a sink-free partial O_s = acc / l (fp32) and LSE_s
  const float lt = l + __shfl_xor(l, 32);
  const float inv = lt > 0.f ? 1.f / lt : 0.f;
  const float lse2 = (m == -INFINITY || !(lt > 0.f)) ? -INFINITY : m + __builtin_amdgcn_logf(lt);
  const float lse = lse2 == -INFINITY ? -INFINITY : lse2 * kLn2;
  if (!hvalid) return;
  const int64_t orow = (int64_t)i * p.hq + (int64_t)g * p.group + hl;
  if (S > 1) {
    const int64_t prow = (int64_t)split * p.num_queries * p.hq + orow;
    float *po = p.part_o + prow * kD;
#pragma unroll
    for (int db = 0; db < kD / 32; ++db)
#pragma unroll
      for (int i4 = 0; i4 < 4; ++i4)
        *(float4 *)(po + 32 * db + 8 * i4 + 4 * hi) =
            make_float4(acc[db][4 * i4] * inv, acc[db][4 * i4 + 1] * inv, acc[db][4 * i4 + 2] * inv,
                        acc[db][4 * i4 + 3] * inv);
    if (hi == 0) p.part_lse[prow] = lse;
    return;
  }
  uint16_t *o = p.o + orow * kD;
#pragma unroll
  for (int db = 0; db < kD / 32; ++db)
#pragma unroll
    for (int i4 = 0; i4 < 4; ++i4) {
      uint2 w;
      w.x = bf16_bits(acc[db][4 * i4] * inv) | (bf16_bits(acc[db][4 * i4 + 1] * inv) << 16);
      w.y = bf16_bits(acc[db][4 * i4 + 2] * inv) | (bf16_bits(acc[db][4 * i4 + 3] * inv) << 16);
      *(uint2 *)(o + 32 * db + 8 * i4 + 4 * hi) = w;
    }
  if (hi == 0 && p.lse != nullptr) p.lse[orow] = lse;
}

}  // namespace

bool decode_eligible(const Params &p) {
  if (p.head_dim != kD || p.query_seq != nullptr || p.query_pos != nullptr) return false;
  if (p.num_splits < 1 || p.num_splits > kMaxSplits) return false;
  const int64_t S = p.num_splits;
  const int64_t cap = p.ratio == 0 ? 0 : p.topk > 0 ? p.topk : (int64_t)p.cmp_pt_stride * p.page_size;
  int64_t cper = (cap + S - 1) / S;
  if (p.cmp_fp8) cper = (cper + kPT - 1) / kPT * kPT;   // e4m3 rows fill whole tiles
  return cper + (p.window + S - 1) / S <= kRowsMax;
}

hipError_t launch_decode(const Params &p, hipStream_t stream) {
  if (p.num_queries == 0) return hipSuccess;
  if (!decode_eligible(p)) return hipErrorInvalidConfiguration;
  if (p.num_splits > 1 && (p.part_o == nullptr || p.part_lse == nullptr)) return hipErrorInvalidValue;
  const int64_t grid = (int64_t)p.num_queries * p.hkv * ((p.group + kHeads - 1) / kHeads) * p.num_splits;
  if (grid > 0x7FFFFFFFLL) return hipErrorInvalidConfiguration;
  if (p.cmp_fp8)
    hipLaunchKernelGGL(attn_decode_kernel<true>, dim3((unsigned)grid), dim3(kThreads), 0, stream, p);
  else
    hipLaunchKernelGGL(attn_decode_kernel<false>, dim3((unsigned)grid), dim3(kThreads), 0, stream, p);
  return hipGetLastError();
}

}  // namespace spa
