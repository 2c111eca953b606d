// Decode (one query token per sequence) for gfx950, one KV pass per query:
// the waves of a workgroup split the query's KV rows instead of its heads.
//
// Operation: sparse paged attention with a sink (RL-Kernel PR "Roadmap item
// 24: joint compressed/window attention with sink", section "Reuse and
// arithmetic"; KV-set and translation rules in spa_device.h), D 128, bf16 raw
// pages and bf16 or e4m3 (OCP or FNUZ) compressed pages with a per-row fp32
// scale, one slice.
//
// One workgroup of four waves per (query, KV head, block of 32 query heads,
// the MFMA's N).  Wave w takes the tiles w, w+4, w+8, .. of the query's rows
// and runs its own online softmax over them with its own two LDS stages and
// no barrier; at the end the four states (m, l, O^T) meet in LDS and wave w
// forms dimensions 32w .. 32w+31 of O by the exact log-sum-exp combination
// (the sink is folded into wave 0's state only).  So a query's set is read
// once per head block with no split partials and no merge kernel, and the
// head blocks of a query run on one XCD (workgroup w runs on XCD w mod 8),
// where its rows stay in the L2.
//
// Setup (the same as the sliced decode kernel's with one slice): issued
// together, the query's metadata, its list row and both page-table rows of
// the sequence (direct loads into LDS when they fit) and the Q fragments;
// then one thread per row forms its 64-bit pool row (bit 62 for the
// compressed pool, -1 when masked).  With e4m3 pages the window starts at
// the next tile edge, so every tile is all e4m3 or all bf16.
//
// A bf16 tile: 8 direct 1 KiB loads per side (lane L of load n: row
// 4n + L / 16, logical chunk (L % 16) ^ swz(row)).  An e4m3 tile: 4 loads
// per side of 8 rows of 128 codes each (lane L of load n: row 8n + L / 8,
// 16-byte piece (L % 8) ^ f8_swz(row)), and one load of the 32 k and 32 v
// scales.  The codes stay in LDS as they are: the wave reads each MFMA
// operand's 8 codes (V's through the 8-bit transpose read) and widens them
// exactly to bf16 in registers.  The k scale multiplies the fp32 scores and
// the v scale p before its bf16 rounding.

#include <hip/hip_runtime.h>

#include <cstdint>

#include "spa_device.h"
#include "spa_kernel_util.h"

namespace spa {
namespace {

constexpr int kD = 128;
constexpr int kRowB = 2 * kD;              // bf16 row bytes
constexpr int kChunks = kRowB / 16;        // 16-byte chunks per row
constexpr int kPT = 32;                    // rows per tile
constexpr int kTileB = kPT * kRowB;        // one side of a tile
constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;

// e4m3 tile rows (128 bytes): logical 16-byte piece c of row r sits at
// piece c ^ f8_swz(r), so the 8 rows that one 16-lane group of the V
// transpose read touches fall in distinct banks, and the 32 rows of a K
// operand read in 16 distinct bank groups instead of two.
__device__ __forceinline__ int f8_swz(int r) { return (r >> 1) & 7; }
// The same for the 64-byte half rows of V's codes that a workgroup forming
// half of O stages: the 16 rows of a transpose read's k block fall in
// distinct banks for each piece.
__device__ __forceinline__ int f8h_swz(int r) { return (r >> 2) & 3; }
constexpr int kHeads = 32;                 // query heads per workgroup
constexpr int kRowsMax = kDecodeRowsMax;
constexpr int kPtLds = 2048;               // page-table entries staged in LDS
constexpr int kWSt = 2;                    // LDS stages per wave
constexpr int64_t kCmpBit = int64_t(1) << 62;

// DH: the workgroup forms one half of O's dimensions and stages only that
// half of each V row (128 bytes).  The list and page-table rows, read only
// while the rows are formed, share the stages' memory.  Two stages per wave
// (one tile's loads in flight while the other computes): a third stage, with
// two tiles' loads in flight, was no faster and slowed the e4m3 pages.
template <bool DH>
struct RowsSmem {
  static constexpr int kVRowB = DH ? kRowB / 2 : kRowB;
  static constexpr int kOD = DH ? kD / 2 : kD;        // output dimensions of the workgroup
  static constexpr int kSt = kWSt;                    // LDS stages per wave
  union {
    struct {
      alignas(16) uint8_t k[kWaves][kSt][kTileB];
      alignas(16) uint8_t v[kWaves][kSt][kPT * kVRowB];
    } t;
    struct {
      alignas(16) int32_t ids[kRowsMax];    // the list row
      alignas(16) int32_t pt[kPtLds];       // raw page-table row, then the compressed one
    } s;
    alignas(16) float acc[kWaves][kOD / 32][16][64];   // the waves' O^T: [wave][d block][value][lane]
  } u;
  alignas(16) float f8s[kWaves][kSt][64];   // e4m3 tiles: 32 k scales, then 32 v scales
  alignas(16) int64_t row[kRowsMax];        // pool rows, padded to whole tiles
  float mw[kWaves][64];                     // the waves' m and l per lane
  float lw[kWaves][64];
};

template <bool FP8, bool DH, bool FNUZ>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(1)))
void attn_decode_rows_kernel(const Params p) {
  static_assert(FP8 || !FNUZ, "FNUZ is an e4m3 format");
  using Smem = RowsSmem<DH>;
  constexpr int kVRowB = Smem::kVRowB;
  constexpr int kVChunks = kVRowB / 16;
  constexpr int kOD = Smem::kOD;
  __shared__ Smem sm;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int hi = lane >> 5;

  // workgroup -> (unit u = query * Hkv + KV head, head block hb, dimension
  // half dh): the workgroups of a unit share the workgroup index mod 8,
  // hence the XCD
  const int32_t nhb = (p.group + kHeads - 1) / kHeads;
  const int32_t units = p.num_queries * p.hkv;
  const int32_t y0 = (int32_t)(blockIdx.x >> 3);
  const int32_t dh = DH ? (y0 & 1) : 0;
  const int32_t y = DH ? (y0 >> 1) : y0;
  const int32_t hb = y % nhb;
  const bool lead = hb == 0 && dh == 0;      // raises the error bits
  const int32_t u = (y / nhb) * 8 + (int32_t)(blockIdx.x & 7);
  if (u >= units) return;                    // padding of the grid to whole groups of 8
  const int32_t g = u % p.hkv;
  const int32_t i = u / p.hkv;
  const int32_t b = i;                       // decode: query i is sequence i's last token

  // ---- round trip 1, everything issued together
  const int32_t topk = p.topk;
  const bool has_list = p.ratio > 0 && topk > 0;
  const int32_t meta = *((lane == 1 && has_list) ? p.cmp_cnt + i : p.seq_lens + b);
  const int32_t P = p.page_size;
  const int64_t cap = p.ratio == 0 ? 0 : topk > 0 ? topk : (int64_t)p.cmp_pt_stride * P;
  if (topk > 0) {
    for (int c = wave; 64 * c < topk; c += kWaves) {
      const int e = 64 * c + lane;
      dma4(e < topk ? (const void *)(p.cmp_idx + (int64_t)i * topk + e) : (const void *)kZeroRow, &sm.u.s.ids[64 * c]);
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
      dma4(src, &sm.u.s.pt[64 * c]);
    }
  }
  const int hl = hb * kHeads + (lane & 31);  // head within the KV group
  const bool hvalid = hl < p.group;
  bf16x8 qf[kD / 16];
  {
    const uint16_t *qrow = p.q + ((int64_t)i * p.hq + (int64_t)g * p.group + (hvalid ? hl : 0)) * kD + 8 * hi;
#pragma unroll
    for (int kk = 0; kk < kD / 16; ++kk) {
      const bf16x8 v = *(const bf16x8 *)(qrow + 16 * kk);
      qf[kk] = hvalid ? v : bf16x8{};
    }
  }
  // the sink enters wave 0's state only
  const float sink = (wave == 0 && hvalid && p.sink != nullptr) ? p.sink[g * p.group + hl] : -INFINITY;
  wait_vmcnt<0>();
  block_sync();                              // list and page-table rows in LDS
  const int32_t len_b = __builtin_amdgcn_readfirstlane(meta);
  const int32_t cnt_i = has_list ? __builtin_amdgcn_readlane(meta, 1) : 0;
  const QueryKV kv = query_kv_of(p, b, len_b - 1, len_b, cnt_i, tid == 0 && lead);

  // ---- the rows: the selected groups, then (from the next tile edge with
  // e4m3 pages) the window
  if (topk == 0 && kv.n_sel > cap && tid == 0 && lead) flag_error(p, kErrPage);   // groups past the table
  const int32_t Uc = (int32_t)min((int64_t)kv.n_sel, cap);
  const int32_t wbase = FP8 ? round_up(Uc, kPT) : Uc;  // first window row
  const int32_t U = min(wbase + kv.win_len, kRowsMax);
  const int32_t T = (U + kPT - 1) / kPT;
  const int32_t nf8 = FP8 ? wbase / kPT : 0;           // tiles 0 .. nf8-1 hold e4m3 rows
  {
    const bool pow2 = p.page_shift >= 0;
    for (int r = tid; r < T * kPT; r += kThreads) {
      const bool cmp = r < Uc;
      int32_t x = -1, col = -1;
      if (r < U && (r < Uc || r >= wbase)) {
        x = cmp ? (topk > 0 ? sm.u.s.ids[r] : r) : kv.win_lo + (r - wbase);
        if (cmp && (x < 0 || x >= kv.n_c)) {
          if (lead) flag_error(p, kErrCmpId);
          x = -1;
        }
        if (x >= 0) {
          col = pow2 ? x >> p.page_shift : x / P;
          if (col >= (cmp ? nc : nr)) {
            if (lead) flag_error(p, kErrPage);
            x = -1;
          }
        }
      }
      int64_t er = -1;
      if (x >= 0) {
        const int32_t page = stage_pt ? sm.u.s.pt[cmp ? nr + col : col]
                                      : (cmp ? p.cmp_pt + (int64_t)b * nc : p.raw_pt + (int64_t)b * nr)[col];
        if (page >= 0 && (int64_t)page < (cmp ? p.cmp_pages : p.raw_pages))
          er = (((int64_t)page * P + (x - col * P)) * p.hkv + g) | (cmp ? kCmpBit : 0);
        else if (lead)
          flag_error(p, kErrPage);
      }
      {
        // the row's K byte address (bf16 rows kRowB bytes apart, e4m3 code
        // rows kD), its pool in the two low bits (rows are 16-byte aligned):
        // 0 raw, 1 compressed, 2 masked (the zero row)
        const bool cmpr = (er & kCmpBit) != 0;
        const uint64_t base = (uint64_t)(uintptr_t)(cmpr ? p.k_cmp : p.k_raw);
        const uint64_t stride = (FP8 && cmpr) ? kD : kRowB;
        sm.row[r] = er < 0 ? (int64_t)((uint64_t)(uintptr_t)kZeroRow | 2u)
                           : (int64_t)((base + (uint64_t)(er & ~kCmpBit) * stride) | (cmpr ? 1u : 0u));
      }
    }
  }
  block_sync();                              // rows in LDS; the list and page-table rows are dead

  // ---- this wave's tiles: j = wave + 4t, stage t % 2
  const uint8_t *const kraw = in_sgpr(p.k_raw), *const vraw = in_sgpr(p.v_raw);
  const uint8_t *const kcmp = in_sgpr(p.k_cmp), *const vcmp = in_sgpr(p.v_cmp);
  const int32_t ntw = T > wave ? (T - wave + kWaves - 1) / kWaves : 0;
  auto tile_of = [&](int t) { return wave + kWaves * t; };
  // V byte address of a row from its stored K address
  const int64_t dv_raw = vraw - kraw, dv_cmp = vcmp - kcmp;
  auto v_of = [&](uint64_t a) -> const uint8_t * {
    const uint32_t tag = (uint32_t)a & 3u;
    return (const uint8_t *)(uintptr_t)((a & ~(uint64_t)3) + (uint64_t)(tag == 0 ? dv_raw : tag == 1 ? dv_cmp : 0));
  };
  auto row_valid = [&](int64_t v) -> bool { return ((uint32_t)v & 3u) != 2u; };
  auto is_f8 = [&](int t) { return FP8 && tile_of(t) < nf8; };
  constexpr int NST = Smem::kSt;
  auto issue = [&](int t) {
    const int j = tile_of(t);
    const int st = t % NST;
    // every row of the tile is read before the first load: the loads' memory
    // clobber keeps a later LDS read from starting ahead of them
    if (FP8 && j < nf8) {
      // e4m3: 8 rows of 128 codes per load, pieces swizzled by f8_swz; with
      // DH, V's half rows: 16 rows of 64 codes per load, swizzled by f8h_swz
      int64_t e8[4], eh[2];
#pragma unroll
      for (int n = 0; n < 4; ++n) e8[n] = sm.row[kPT * j + 8 * n + lane / 8];
      if constexpr (DH) {
#pragma unroll
        for (int n = 0; n < 2; ++n) eh[n] = sm.row[kPT * j + 16 * n + lane / 4];
      }
      const int64_t es = sm.row[kPT * j + (lane & 31)];
      // an e4m3 tile's rows are compressed (K codes at the stored address,
      // V codes the pools' K-to-V distance on) or masked (the zero row, whose
      // first 128 bytes every piece below stays within)
#pragma unroll
      for (int n = 0; n < 4; ++n) {
        const uint64_t a = (uint64_t)e8[n];
        const uint8_t *src =
            (const uint8_t *)(uintptr_t)(a & ~(uint64_t)3) + (((lane % 8) ^ f8_swz(8 * n + lane / 8)) * 16);
        dma16(src, sm.u.t.k[wave][st] + 8 * n * kD);
        if constexpr (!DH) dma16(src + ((a & 3u) == 1u ? dv_cmp : 0), sm.u.t.v[wave][st] + 8 * n * kD);
      }
      if constexpr (DH) {
#pragma unroll
        for (int n = 0; n < 2; ++n) {
          const uint64_t a = (uint64_t)eh[n];
          const uint8_t *src = (const uint8_t *)(uintptr_t)(a & ~(uint64_t)3) + ((a & 3u) == 1u ? dv_cmp : 0) +
                               kD / 2 * dh + (((lane % 4) ^ f8h_swz(16 * n + lane / 4)) * 16);
          dma16(src, sm.u.t.v[wave][st] + 16 * n * (kD / 2));
        }
      }
      // the row's scale, its index from the code address
      const float *scl = lane < 32 ? p.k_cmp_scale : p.v_cmp_scale;
      const uint64_t row8 = (((uint64_t)es & ~(uint64_t)3) - (uint64_t)(uintptr_t)kcmp) / kD;
      dma4(((uint32_t)es & 3u) == 1u ? (const void *)(scl + row8) : (const void *)(kZeroRow + 4 * (lane & 31)),
           sm.f8s[wave][st]);
      return;
    }
    int64_t ek[8], ev[4];
#pragma unroll
    for (int n = 0; n < 8; ++n) ek[n] = sm.row[kPT * j + 4 * n + lane / kChunks];
    if constexpr (DH) {
#pragma unroll
      for (int n = 0; n < 4; ++n) ev[n] = sm.row[kPT * j + 8 * n + lane / kVChunks];
    }
#pragma unroll
    for (int n = 0; n < 8; ++n) {
      const int r = 4 * n + lane / kChunks;
      const int64_t er = ek[n];
      const int cs = ((lane % kChunks) ^ swz<kChunks>(r)) * 16;
      const uint64_t a = (uint64_t)er;
      dma16((const uint8_t *)(uintptr_t)(a & ~(uint64_t)3) + cs, sm.u.t.k[wave][st] + 4 * n * kRowB);
      if constexpr (!DH) dma16(v_of(a) + cs, sm.u.t.v[wave][st] + 4 * n * kRowB);
    }
    if constexpr (DH) {
      // the workgroup's half of each V row: 8 rows of 128 bytes per load
#pragma unroll
      for (int n = 0; n < 4; ++n) {
        const int r = 8 * n + lane / kVChunks;
        const int cs = ((lane % kVChunks) ^ swz<kVChunks>(r)) * 16;
        dma16(v_of((uint64_t)ev[n]) + kVRowB * dh + cs, sm.u.t.v[wave][st] + 8 * n * kVRowB);
      }
    }
  };
  constexpr int kLoads = DH ? 12 : 16;       // direct loads of a bf16 tile
  constexpr int kLoads8 = DH ? 7 : 9;        // and of an e4m3 tile

  float m = sink == -INFINITY ? -INFINITY : sink * kLog2e;
  float l = (sink != -INFINITY && hi == 0) ? 1.f : 0.f;   // exp2(sink - m) = 1, counted once per head
  f32x16 acc[kOD / 32];
#pragma unroll
  for (int db = 0; db < kOD / 32; ++db) acc[db] = f32x16{};

  if (ntw > 0) issue(0);
  if (ntw > 1) issue(1);
  for (int t = 0; t < ntw; ++t) {
    const int j = tile_of(t);
    const int st = t % NST;
    const bool f8 = is_f8(t);
    // this wave's loads of tile j are complete (those of its next tile may
    // still be in flight: kLoads, or kLoads8 for an e4m3 tile)
    if (t + 1 < ntw) {
      if (is_f8(t + 1)) wait_vmcnt<kLoads8>();
      else wait_vmcnt<kLoads>();
    } else {
      wait_vmcnt<0>();
    }
    uint8_t *Kt = sm.u.t.k[wave][st];
    uint8_t *Vt = sm.u.t.v[wave][st];
    const uint32_t tm = (uint32_t)__ballot(lane < 32 && row_valid(sm.row[kPT * j + (lane & 31)]));
    bf16x8 kf[kD / 16];
    i16x8 vf[kOD / 32][2];
    if (FP8 && f8) {
      // e4m3 codes straight into the MFMA operands: K's A fragment is 8
      // codes of one row; V's is one dimension over the 8 rows that P's
      // fragment holds (rows 4hi .. 4hi+3 and 8+4hi .. 8+4hi+3 of the 16),
      // which the 8-bit transpose read gathers: output lane L's byte b comes
      // from input lane 2b + L / 8, so input lanes 2b and 2b+1 point at the
      // codes of the b-th of those rows for the 16-lane group's 16 dimensions
      uint2 kc[kD / 16];
      v2i32 vc[kOD / 32][2];
      const int r = lane & 31;
#pragma unroll
      for (int kk = 0; kk < kD / 16; ++kk)
        kc[kk] = *(const uint2 *)(Kt + r * kD + ((kk ^ f8_swz(r)) * 16) + 8 * hi);
      const int G = lane >> 4;
      const int L = lane & 15;
#pragma unroll
      for (int db = 0; db < kOD / 32; ++db)
#pragma unroll
        for (int k2 = 0; k2 < 2; ++k2) {
          const int b8 = L >> 1;
          const int row = 16 * k2 + 4 * (G >> 1) + 8 * (b8 >> 2) + (b8 & 3);
          const int piece = 2 * db + (G & 1);
          // V's codes: whole rows, or with DH the workgroup's 64-code halves
          const int voff = DH ? row * (kD / 2) + ((piece ^ f8h_swz(row)) * 16)
                              : row * kD + ((piece ^ f8_swz(row)) * 16);
          vc[db][k2] = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_v2i32_t *)(Vt + voff + (L & 1) * 8));
        }
#pragma unroll
      for (int kk = 0; kk < kD / 16; ++kk) kf[kk] = __builtin_bit_cast(bf16x8, widen8_e4m3<FNUZ>(kc[kk]));
#pragma unroll
      for (int db = 0; db < kOD / 32; ++db)
#pragma unroll
        for (int k2 = 0; k2 < 2; ++k2)
          vf[db][k2] = __builtin_bit_cast(
              i16x8, widen8_e4m3<FNUZ>(make_uint2((uint32_t)vc[db][k2][0], (uint32_t)vc[db][k2][1])));
    } else {
      const int r = lane & 31;
#pragma unroll
      for (int kk = 0; kk < kD / 16; ++kk) {
        const int c = 2 * kk + hi;
        kf[kk] = *(const bf16x8 *)(Kt + r * kRowB + ((c ^ swz<kChunks>(r)) * 16));
      }
      const int G = lane >> 4;
      const int L = lane & 15;
#pragma unroll
      for (int db = 0; db < kOD / 32; ++db)
#pragma unroll
        for (int k2 = 0; k2 < 2; ++k2) {
          i16x4 h[2];
#pragma unroll
          for (int rw = 0; rw < 2; ++rw) {
            const int row = 16 * k2 + 8 * rw + 4 * (G >> 1) + (L >> 2);
            const int d = 32 * db + 16 * (G & 1) + 4 * (L & 3);
            const int off = row * kVRowB + (((d >> 3) ^ swz<kVChunks>(row)) * 16) + (L & 1) * 8;
            h[rw] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t *)(Vt + off));
          }
          vf[db][k2] = __builtin_shufflevector(h[0], h[1], 0, 1, 2, 3, 4, 5, 6, 7);
        }
    }
    float ks[16], vs[16];
    if (FP8 && f8) {
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const float4 k4 = *(const float4 *)(&sm.f8s[wave][st][8 * q4 + 4 * hi]);
        const float4 v4 = *(const float4 *)(&sm.f8s[wave][st][32 + 8 * q4 + 4 * hi]);
        ks[4 * q4] = k4.x, ks[4 * q4 + 1] = k4.y, ks[4 * q4 + 2] = k4.z, ks[4 * q4 + 3] = k4.w;
        vs[4 * q4] = v4.x, vs[4 * q4 + 1] = v4.y, vs[4 * q4 + 2] = v4.z, vs[4 * q4 + 3] = v4.w;
      }
    }
    // every LDS read of the stage is in (tile t+2 takes it once tile t's
    // products are issued, so that its loads do not hold them back)
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");

    f32x16 s = f32x16{};
#pragma unroll
    for (int kk = 0; kk < kD / 16; ++kk) s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[kk], qf[kk], s, 0, 0, 0);
    float sc[16];
#pragma unroll
    for (int q = 0; q < 16; ++q) sc[q] = (FP8 && f8) ? s[q] * ks[q] : s[q];
    mask_tile_rows(sc, tm);
    float smax = sc[0];
#pragma unroll
    for (int q = 1; q < 16; ++q) smax = fmaxf(smax, sc[q]);
    smax = max_lane_pair(smax);
    const float tmax = smax * p.scale_log2;
    const bool need = tmax > m + kTau;
    if (__any(need)) {
      const float alpha = need ? __builtin_amdgcn_exp2f(m - tmax) : 1.f;
      m = need ? tmax : m;
      l *= alpha;
#pragma unroll
      for (int db = 0; db < kOD / 32; ++db) acc[db] *= alpha;
    }
    const float negm = m == -INFINITY ? 0.f : -m;
    bf16x8 pb[2];
#pragma unroll
    for (int q = 0; q < 16; ++q) {
      const float pr = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[q], p.scale_log2, negm));
      l += pr;
      pb[q >> 3][q & 7] = (__bf16)((FP8 && f8) ? pr * vs[q] : pr);
    }
#pragma unroll
    for (int db = 0; db < kOD / 32; ++db)
#pragma unroll
      for (int k2 = 0; k2 < 2; ++k2)
        acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, vf[db][k2]), pb[k2], acc[db],
                                                         0, 0, 0);
    if (t + 2 < ntw) issue(t + 2);
  }

  // ---- the four states meet: wave w forms dimensions 32w .. 32w+31 of
  // the workgroup's (two waves with half of the dimensions),
  // O = sum_s 2^(m_s - M) acc_s / sum_s 2^(m_s - M) l_s, LSE = (M + log2 L) ln 2
  block_sync();                              // every wave is done with its stages
#pragma unroll
  for (int db = 0; db < kOD / 32; ++db)
#pragma unroll
    for (int q = 0; q < 16; ++q) sm.u.acc[wave][db][q][lane] = acc[db][q];
  sm.mw[wave][lane] = m;
  sm.lw[wave][lane] = l;
  block_sync();
  if (wave >= kOD / 32) return;
  float M = -INFINITY;
#pragma unroll
  for (int s = 0; s < kWaves; ++s) M = fmaxf(M, sm.mw[s][lane]);
  float L = 0.f, o[16];
#pragma unroll
  for (int q = 0; q < 16; ++q) o[q] = 0.f;
#pragma unroll
  for (int s = 0; s < kWaves; ++s) {
    const float ms = sm.mw[s][lane];
    const float wgt = ms == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(ms - M);
    L += wgt * (sm.lw[s][lane] + sm.lw[s][lane ^ 32]);
#pragma unroll
    for (int q = 0; q < 16; ++q) o[q] += wgt * sm.u.acc[s][wave][q][lane];
  }
  const float inv = L > 0.f ? 1.f / L : 0.f;
  const float lse2 = (M == -INFINITY || !(L > 0.f)) ? -INFINITY : M + __builtin_amdgcn_logf(L);
  const float lse = lse2 == -INFINITY ? -INFINITY : lse2 * kLn2;
  if (!hvalid) return;
  const int64_t orow = (int64_t)i * p.hq + (int64_t)g * p.group + hl;
  uint16_t *out = p.o + orow * kD + kOD * dh + 32 * wave;
#pragma unroll
  for (int i4 = 0; i4 < 4; ++i4) {
    uint2 w;
    w.x = bf16_bits(o[4 * i4] * inv) | (bf16_bits(o[4 * i4 + 1] * inv) << 16);
    w.y = bf16_bits(o[4 * i4 + 2] * inv) | (bf16_bits(o[4 * i4 + 3] * inv) << 16);
    *(uint2 *)(out + 8 * i4 + 4 * hi) = w;
  }
  if (wave == 0 && hi == 0 && dh == 0 && p.lse != nullptr) p.lse[orow] = lse;
}

}  // namespace

bool decode_rows_eligible(const Params &p) {
  if (p.head_dim != kD || p.query_seq != nullptr || p.query_pos != nullptr || p.num_splits != 1) return false;
  const int64_t cap = p.ratio == 0 ? 0 : p.topk > 0 ? p.topk : (int64_t)p.cmp_pt_stride * p.page_size;
  const int64_t crow = p.cmp_fp8 ? (cap + kPT - 1) / kPT * kPT : cap;   // e4m3 rows fill whole tiles
  return crow + p.window <= kRowsMax && (p.topk == 0 || p.topk <= kRowsMax);
}

hipError_t launch_decode_rows(const Params &p, bool halves, hipStream_t stream) {
  if (p.num_queries == 0) return hipSuccess;
  if (!decode_rows_eligible(p)) return hipErrorInvalidConfiguration;
  const int64_t units = (int64_t)p.num_queries * p.hkv;
  const int64_t grid = (units + 7) / 8 * 8 * ((p.group + kHeads - 1) / kHeads) * (halves ? 2 : 1);
  if (grid > 0x7FFFFFFFLL) return hipErrorInvalidConfiguration;
  auto kernel = p.cmp_fp8 ? (p.cmp_fnuz ? (halves ? attn_decode_rows_kernel<true, true, true>
                                                  : attn_decode_rows_kernel<true, false, true>)
                                        : (halves ? attn_decode_rows_kernel<true, true, false>
                                                  : attn_decode_rows_kernel<true, false, false>))
                : halves ? attn_decode_rows_kernel<false, true, false>
                         : attn_decode_rows_kernel<false, false, false>;
  hipLaunchKernelGGL(kernel, dim3((unsigned)grid), dim3(kThreads), 0, stream, p);
  return hipGetLastError();
}

}  // namespace spa
