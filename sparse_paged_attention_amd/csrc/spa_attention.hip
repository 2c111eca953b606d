// Sparse paged attention forward with a sink, for gfx950 (CDNA4).
//
// Operation: RL-Kernel PR "Roadmap item 24: joint compressed/window attention
// with sink", section "Reuse and arithmetic" — the selected compressed KV, the
// full recent raw window and a per-head sink logit share one softmax
// denominator; the sink has no value row; P and O are bf16, LSE is fp32
// natural log.  The KV set and page translation rules live in spa_device.h.
//
// Work decomposition.  A job is (query, KV head, KV slice, block of 32*NH
// query heads); all query heads of a KV head read the same KV rows, so one
// job streams its KV rows once through LDS and each compute wave feeds every
// tile to bf16 MFMAs for its 32 heads:
//
//   S^T[kv, head]  = K[kv, :] . Q^T[:, head]        v_mfma_f32_32x32x16_bf16
//   O^T[d, head]  += V^T[d, kv] . P^T[kv, head]      v_mfma_f32_32x32x16_bf16
//
// With S^T and O^T in the MFMA accumulator layout every lane owns one query
// head (lane % 32): the online-softmax state (m, l) is per lane, the row max
// needs one exchange with lane ^ 32, and P^T goes from the S^T accumulators
// straight into the B operand of the PV MFMA (the KV order inside a 16-row
// step is permuted identically on both operands).  V^T comes from the
// row-major V tile through the gfx950 LDS transpose read (ds_read_b64_tr_b16).
//
// Persistent workgroups.  The grid holds as many workgroups as are resident
// at once; each runs a static list of jobs.  Jobs are grouped in units (one
// query and KV head: its slices and head blocks read the same rows); units
// are dealt to the 8 XCDs round-robin (unit u to XCD u % 8, so every XCD gets
// a mix of short and long KV sets) and, within an XCD, consecutive jobs go to
// consecutive workgroups, so the jobs of one unit share that XCD's L2.  This
// affects speed only, never results.
//
// Job streams.  A workgroup runs NS streams (NS = 2 for 64-head bf16 jobs,
// else 1); job k of the workgroup goes to stream k % NS.  A stream is a
// sequence of 32-row tiles: per job a Q tile (its query's rows for the head
// block) and then its KV tiles (selected compressed rows, then the window;
// an empty set gets one fully masked tile).  Each stream has its compute
// waves, a K load wave, a V load wave, a translation wave and a row wave;
// the streams share the workgroup's barriers, one per step.  Step t of a stream (after
// barrier t): the compute waves take tile t (scores, softmax, PV product;
// a Q tile is copied into the Q fragments); the load waves issue the K and
// V sides of tile t+3 into rings of 4 LDS slots with direct global->LDS
// loads (global_load_lds_dwordx4: no VGPR staging; a Q tile puts heads 0-31
// in its K slot and 32-63 in its V slot); the row wave forms the pool row
// of every row of tile t+4; the translation wave loads the page-table
// entries of tile t+7 and the list entries of tile t+10 into small LDS
// rings, with direct loads as well.  Every helper wave issues the same number of loads each
// step (padding loads read a static zero row into a scratch area), so one
// vmcnt immediate tracks everything: before barrier t+1 each waits for its
// loads of steps <= t-2.  The per-job metadata is computed once, up front,
// one job per helper lane.  After a job's last KV tile the epilogue writes
// its output and the state is reset for the next job.
//
// Softmax runs in the log2 domain (scores pre-multiplied by scale*log2 e,
// sink by log2 e) with v_exp_f32; with one slice the running max starts at
// the sink and the running sum at exp(0) = 1, i.e. the sink is folded into
// (m, l) from the start.  With num_splits > 1 each slice writes a sink-free
// partial (O_s f32, LSE_s) to the workspace and the merge kernel
// (spa_merge.hip) combines them, adding the sink exactly once.
//
// FP8 (OCP e4m3) compressed rows land in an LDS staging area, together with
// their fp32 per-token scales, and are widened to bf16 exactly (every e4m3
// value is a bf16 value) by v_cvt_scalef32_pk_bf16_fp8 at scale 1 (FNUZ codes
// through v_cvt_pk_f32_fp8 and fix-ups); the scales are applied in fp32
// to the scores (k) and to P (v), so the MFMAs see the exact codes.
//
// Invalid metadata (a listed id that is not a complete group, a page id
// outside its pool, a page-table column past the table, a bad count or
// position) masks the entry, sets a bit in err_flag and is never loaded.

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdint>
#include <type_traits>

#include "spa_device.h"
#include "spa_kernel_util.h"

namespace spa {
namespace {

constexpr int kTile = 32;      // KV rows per tile
constexpr int kRing = 4;       // LDS tile slots
constexpr int kXRing = 8;      // translation ring slots (list, page-table and id entries)

// Tile descriptor flags.
enum : uint32_t { kTileQ = 1, kTileKV = 2, kTileCmp = 4, kTileLast = 8, kTileWiden = 16 };

// ---------------------------------------------------------------- job lists
// Job k of workgroup (XCD x, index y of Gx on that XCD): local index
// l = y + k Gx, unit unit_begin + x + 8 floor(l / R), job r = l % R of the
// unit (R = jobs_per_unit; r = split * head_groups + head block).
struct JobId {
  int32_t qi, g, split, hb;
  bool valid;
};

__device__ __forceinline__ JobId job_id(const Params &p, int32_t x, int32_t y, int32_t Gx, int32_t k) {
  const int32_t R = p.jobs_per_unit;
  const int32_t l = y + k * Gx;
  const int32_t m = l / R;
  const int32_t r = l - m * R;
  const int32_t u = p.unit_begin + x + 8 * m;
  JobId j;
  j.valid = u < p.unit_end;
  j.qi = u / p.hkv;
  j.g = u - j.qi * p.hkv;
  j.split = r / p.head_groups;
  j.hb = r - j.split * p.head_groups;
  return j;
}

template <int D, int NH, bool FP8>
struct Cfg {
  static constexpr int NC = NH;                        // compute waves
  static constexpr int kThreads = NC * 64;             // compute threads
  static constexpr int kBlock = kThreads + 256;        // + two load waves (K, V), the translation wave and the row wave
  static constexpr int kRowB = 2 * D;                  // bf16 row bytes
  static constexpr int kChunks = kRowB / 16;           // 16-byte chunks per row
  static constexpr int kTileB = kTile * kRowB;         // one K (or V) tile, bytes
  static constexpr int kHalfOps = kTileB / 1024;       // wave-wide 1 KiB loads per K (or V) tile
  static constexpr int kF8RowB = D;                    // e4m3 row bytes
  static constexpr int kF8TileB = kTile * D;           // one e4m3 K (or V) tile
  static constexpr int kF8HalfOps = kF8TileB / 1024;
  static constexpr int kLoadOps = kHalfOps;            // loads per stream step for one side (K or V) of a tile
  static constexpr int kMaxJobs = 64;                  // jobs per workgroup per launch
  static_assert(!FP8 || kF8HalfOps + 1 <= kLoadOps, "fp8 tile: data + scale loads fit the per-tile count");
  static_assert(2 * kLoadOps < 64, "vmcnt range");
};

template <int D, int NH, bool FP8>
struct Smem {
  using C = Cfg<D, NH, FP8>;
  alignas(16) uint8_t kr[kRing][C::kTileB];                       // K tiles (a Q tile: heads 0-31)
  alignas(16) uint8_t vr[kRing][C::kTileB];                       // V tiles (a Q tile: heads 32-63)
  alignas(16) uint8_t stk[FP8 ? kRing : 1][FP8 ? C::kF8TileB : 16];   // e4m3 K staging
  alignas(16) uint8_t stv[FP8 ? kRing : 1][FP8 ? C::kF8TileB : 16];   // e4m3 V staging
  alignas(16) float scl_k[FP8 ? kRing : 1][64];                   // k scales [0,32)
  alignas(16) float scl_v[FP8 ? kRing : 1][64];                   // v scales [0,32)
  alignas(16) int32_t lst[kXRing][64];                            // list entries (lanes 0-31)
  alignas(16) int32_t pg[kXRing][64];                             // page-table entries (lanes 0-31)
  alignas(16) int32_t xid[kXRing][32];                            // logical id per row, -1 = masked
  // pool row of every row of a tile (-1: masked), by tile slot, and the
  // mask of its valid rows
  alignas(16) int64_t erow[kRing][32];
  uint32_t emask[kRing];
  alignas(16) uint8_t dummy[1024];                                // destination of padding loads
  alignas(16) uint4 desc[kRing];                                  // tile descriptors
  int32_t ntiles;
};

template <int D, int NH, int NS, bool FP8>
__global__ __launch_bounds__(NS * (NH + 4) * 64) __attribute__((amdgpu_waves_per_eu(3)))  // <= 168 VGPRs
void attn_fwd_kernel(const Params p) {
  using C = Cfg<D, NH, FP8>;
  static_assert(NS == 1 || NS == 2, "one or two streams per workgroup");
  static_assert(!FP8 || NS == 1, "fp8 staging leaves LDS for one stream only");
  __shared__ Smem<D, NH, FP8> sm_all[NS];

  const int32_t x = (int32_t)(blockIdx.x & 7);
  const int32_t y = (int32_t)(blockIdx.x >> 3);
  const int32_t Gx = (int32_t)(gridDim.x >> 3);
  if (!job_id(p, x, y, Gx, 0).valid) return;   // no work for this workgroup

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int hi = lane >> 5;                    // which half of the wave
  const int S = p.num_splits;
  // NS independent streams (job sequences) share the workgroup and its
  // barriers: waves [0, NS*NC) compute (stream wave / NC), then the K and
  // V load waves of each stream, then each stream's translation wave, then
  // each stream's row wave.  A workgroup's waves 0-3 sit on four different
  // SIMDs and every further four on the same four, so with NS = 2 and
  // NC = 2 every SIMD runs one compute wave, one load wave and one of the
  // translation and row waves: a SIMD's wave issues its loads into LDS at a
  // bounded rate, which the load waves then share evenly.
  constexpr int NCW = NS * C::NC;
  const bool helper = wave >= NCW;
  const int hidx = wave - NCW;                 // helper index
  const int strm = !helper ? wave / C::NC : hidx < 2 * NS ? hidx >> 1 : hidx < 3 * NS ? hidx - 2 * NS : hidx - 3 * NS;
  Smem<D, NH, FP8> &sm = sm_all[strm];
  // stream strm's k-th job is the workgroup's job NS*k + strm
  auto jid = [&](int32_t k) { return job_id(p, x, y, Gx, NS * k + strm); };

  // =================================================================
  // Load waves (K, V and Q tiles), translation wave (page-table and list
  // entries) and row wave (pool rows)
  // =================================================================
  if (helper) {
    // the K load wave issues the K side of every tile (K rows, Q heads
    // 0-31) and its descriptor, the V load wave the V side (V rows, Q heads
    // 32-63), the translation wave the list and page-table entries and the
    // row wave the pool row of every tile row
    const bool loader = hidx < 2 * NS;
    const bool vload = loader && (hidx & 1) != 0;
    const bool roww = hidx >= 3 * NS;        // the row wave: pool rows of every tile
    const bool xlat = !loader && !roww;      // the translation wave: list and page-table entries
    const int64_t raw_np = in_sgpr(p.raw_pages), cmp_np = in_sgpr(p.cmp_pages);
    const int32_t raw_st = in_sgpr(p.raw_pt_stride), cmp_st = in_sgpr(p.cmp_pt_stride);
    const int32_t *const raw_pt = in_sgpr(p.raw_pt), *const cmp_pt = in_sgpr(p.cmp_pt);
    const uint8_t *const raw_b = vload ? in_sgpr(p.v_raw) : in_sgpr(p.k_raw);   // this load wave's side
    const uint8_t *const cmp_b = vload ? in_sgpr(p.v_cmp) : in_sgpr(p.k_cmp);
    const float *const cmp_sc = vload ? in_sgpr(p.v_cmp_scale) : in_sgpr(p.k_cmp_scale);
    // ---- per-job metadata, one job per lane (ordinary loads: nothing is in
    // flight yet); both waves compute the same records
    const JobId jl = jid(lane);
    const bool jvalid = lane < C::kMaxJobs && jl.valid;
    int32_t jnc = 0, jcs = 0, jncr = 0, jwb = 0, jnwr = 0, jnct = 0, jnkv = 1;
    int64_t jrpt = 0, jcpt = 0, jlst = 0;   // row bases: page tables, list
    const int64_t jq = ((int64_t)jl.qi * p.hq + jl.g * p.group + jl.hb * p.heads_per_block) * D;   // Q
    const int32_t jnh = jvalid ? min(32 * NH, p.group - jl.hb * p.heads_per_block) : 0;   // real heads
    const uint8_t *zero16 = kZeroRow + (lane & 15) * 16;
    const void *zero4 = kZeroRow + lane * 4;
    // Job 0's Q tile and (top-k layers) the list entries of its first
    // compressed tiles need no metadata: they are issued before it is read,
    // so that their loads overlap the metadata loads.  The list entries are
    // taken up to the slice's capacity; the page stage uses only the valid
    // ones.
    constexpr int kSpec = 6;                 // tiles 1..kSpec of the stream at most
    int32_t nspec = 0;
    if (xlat && p.topk > 0 && jid(0).valid) {   // (a stream may have no job at all)
      const JobId j0 = jid(0);
      const int cper = round_up((p.topk + S - 1) / S, kTile);
      const int cs0 = min(p.topk, j0.split * cper);
      const int cap0 = min(p.topk, cs0 + cper) - cs0;
      nspec = min(kSpec, (cap0 + kTile - 1) / kTile);
      for (int u = 1; u <= nspec; ++u) {
        const int32_t idx = (u - 1) * kTile + lane;
        dma4(lane < kTile && idx < cap0 ? (const void *)(p.cmp_idx + (int64_t)j0.qi * p.topk + cs0 + idx) : zero4,
             &sm.lst[u % kXRing][0]);
      }
    }
    // the 16-byte chunk each lane moves within its row in load n of a tile:
    // row 4n + lane/16 (D 128) or 8n + lane/8 (D 64), logical chunk
    // (lane % chunks) ^ swz(row), which depends on n mod (16 / rows per load)
    // only
    constexpr int kRowsPerOp = 1024 / C::kRowB;
    constexpr int kPeriod = 16 / kRowsPerOp;   // 4 (D 128) or 2 (D 64)
    int32_t cs16[kPeriod];
#pragma unroll
    for (int n = 0; n < kPeriod; ++n) {
      const int r = n * kRowsPerOp + lane / C::kChunks;
      cs16[n] = ((lane % C::kChunks) ^ swz<C::kChunks>(r)) * 16;
    }

    if (loader) {
      // job 0's Q tile: heads 0-31 into K slot 0 (K load wave), 32-63 into
      // V slot 0 (V load wave)
      const int64_t q0 = (int64_t)(((uint64_t)__builtin_amdgcn_readlane((uint32_t)(jq >> 32), 0) << 32) |
                                   __builtin_amdgcn_readlane((uint32_t)jq, 0));
      const int32_t nh0 = __builtin_amdgcn_readlane(jnh, 0);
      const int r0 = vload ? 32 : 0;
      const uint8_t *qb = (const uint8_t *)(p.q + q0) + (r0 + lane / C::kChunks) * C::kRowB;
      uint8_t *dst = vload ? sm.vr[0] : sm.kr[0];
#pragma unroll
      for (int n = 0; n < C::kHalfOps; ++n) {
        const int r = r0 + n * kRowsPerOp + lane / C::kChunks;
        dma16(r < nh0 ? qb + n * 1024 + cs16[n % kPeriod] : zero16, dst + n * 1024);
      }
      if (!vload && lane == 0) sm.desc[0] = make_uint4(0u, kTileQ, 0u, 0u);
    }
    if (jvalid) {
      const QueryKV kv = query_kv(p, jl.qi);
      // slices cut by capacity: list slots [cs, ce) of the compressed part
      // (the top-k list, or the n_c groups of an all-groups layer) and
      // window slots [ws, we)
      const int ccap = p.topk > 0 ? p.topk : kv.n_sel;
      const int cper = round_up((ccap + S - 1) / S, kTile);
      const int cs = min(ccap, jl.split * cper);
      const int ce = min(ccap, cs + cper);
      const int wper = round_up((p.window + S - 1) / S, kTile);
      const int ws = min(kv.win_len, jl.split * wper);
      const int we = min(kv.win_len, ws + wper);
      jnc = kv.n_c;
      jcs = cs;
      jncr = max(0, min(ce, kv.n_sel) - cs);
      jwb = kv.win_lo + ws;
      jnwr = we - ws;
      jnct = (jncr + kTile - 1) / kTile;
      jnkv = max(1, jnct + (jnwr + kTile - 1) / kTile);   // an empty set still gets one (masked) tile
      jrpt = (int64_t)kv.b * p.raw_pt_stride;
      jcpt = (int64_t)kv.b * p.cmp_pt_stride;
      jlst = (int64_t)jl.qi * p.topk + cs;
    }
    const int32_t jg = jl.g;
    const int32_t njobs = __popcll(__ballot(jvalid));
    // total stream length (a Q tile + the KV tiles per job)
    int32_t T = jvalid ? 1 + jnkv : 0;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) T += __shfl_xor(T, d);
    if (loader && lane == 0) sm.ntiles = T;

    int32_t errbits = 0;   // reported once at the end (an atomic now would add to the load count)

    // wave-uniform copy of job k's record, refreshed when a cursor moves on
    auto rd = [&](int32_t v, int32_t k) { return __builtin_amdgcn_readlane(v, k); };
    auto rd64 = [&](int64_t v, int32_t k) {
      const uint32_t lo = __builtin_amdgcn_readlane((uint32_t)v, k);
      const uint32_t hi32 = __builtin_amdgcn_readlane((uint32_t)(v >> 32), k);
      return (int64_t)(((uint64_t)hi32 << 32) | lo);
    };
    struct Job {
      int32_t nkv, nct, ncr, cs, wb, nwr, nc, nh, g;
      int64_t rpt, cpt, lst, q;
    };
    auto job = [&](int32_t k) {
      Job j{0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0};
      if (k < njobs) {
        j.nkv = rd(jnkv, k);
        j.nct = rd(jnct, k);
        j.ncr = rd(jncr, k);
        j.cs = rd(jcs, k);
        j.wb = rd(jwb, k);
        j.nwr = rd(jnwr, k);
        j.nc = rd(jnc, k);
        j.nh = rd(jnh, k);
        j.g = rd(jg, k);
        j.rpt = rd64(jrpt, k);
        j.cpt = rd64(jcpt, k);
        j.lst = rd64(jlst, k);
        j.q = rd64(jq, k);
      }
      return j;
    };
    // stream cursor: job k, position v (0 = Q tile, 1..nkv = KV tiles),
    // stream index u
    struct Cur {
      int32_t k, v, u;
      Job j;
    };
    auto advance = [&](Cur &c) {
      ++c.u;
      if (c.k < njobs && ++c.v > c.j.nkv) {
        ++c.k;
        c.v = 0;
        c.j = job(c.k);
      }
    };
    const bool pow2 = p.page_shift >= 0;
    const int32_t P = p.page_size;
    // ---------------- translation and row wave stages
    // -- list stage: list entries of a compressed KV tile of a top-k layer
    // (pad = false: a tile with nothing to load issues no padding load;
    // only where the wave then waits for all of its loads)
    auto stage_list = [&](const Cur &c, bool pad) {
      const void *src = zero4;
      void *dst = sm.dummy;
      if (c.k < njobs && c.v > 0 && p.topk > 0 && c.v - 1 < c.j.nct) {
        const int32_t idx = (c.v - 1) * kTile + lane;
        if (lane < kTile && idx < c.j.ncr) src = p.cmp_idx + c.j.lst + idx;
        dst = &sm.lst[c.u % kXRing][0];
      }
      if (pad || dst != (void *)sm.dummy) dma4(src, dst);
    };
    // -- page stage: logical id of every row of a KV tile (from its list
    // entry `le`, read by the caller), then its page-table entry
    auto stage_page = [&](const Cur &c, int32_t le, bool pad) {
      const void *src = zero4;
      void *dst = sm.dummy;
      if (c.k < njobs && c.v > 0) {
        const int32_t e0 = c.v - 1;
        const bool cmp = e0 < c.j.nct;
        if (lane < kTile) {
          int32_t xv = -1;
          if (cmp) {
            const int32_t idx = e0 * kTile + lane;
            if (idx < c.j.ncr) {
              if (p.topk > 0) {
                if (le >= 0 && le < c.j.nc) xv = le;
                else errbits |= kErrCmpId;
              } else {
                xv = c.j.cs + idx;   // all-groups layer: ids in order
              }
            }
          } else {
            const int32_t idx = (e0 - c.j.nct) * kTile + lane;
            if (idx < c.j.nwr) xv = c.j.wb + idx;
          }
          if (xv >= 0) {
            const int32_t col = pow2 ? (xv >> p.page_shift) : xv / P;
            if (col < (cmp ? cmp_st : raw_st)) {
              src = cmp ? (const void *)(cmp_pt + c.j.cpt + col) : (const void *)(raw_pt + c.j.rpt + col);
            } else {
              errbits |= kErrPage;
              xv = -1;
            }
          }
          sm.xid[c.u % kXRing][lane] = xv;
        }
        dst = &sm.pg[c.u % kXRing][0];
      }
      if (pad || dst != (void *)sm.dummy) dma4(src, dst);
    };
    auto list_entry = [&](const Cur &c) { return sm.lst[c.u % kXRing][lane & 31]; };
    // -- row stage: pool row of every row of a KV tile from its id and page
    // entry (read by the caller), and the mask of the valid rows
    auto stage_rows = [&](const Cur &c, int32_t xv, int32_t page) {
      if (c.k >= njobs || c.v == 0) return;
      const bool cmp = c.v - 1 < c.j.nct;
      int64_t er = -1;
      if (lane < kTile && xv >= 0) {
        if (page >= 0 && (int64_t)page < (cmp ? cmp_np : raw_np)) {
          const int32_t off = pow2 ? (xv & (P - 1)) : xv - (xv / P) * P;
          er = ((int64_t)page * P + off) * p.hkv + c.j.g;
        } else {
          errbits |= kErrPage;
        }
      }
      const uint32_t mask = (uint32_t)__ballot(er >= 0);
      if (lane < kTile) sm.erow[c.u % kRing][lane] = er;
      if (lane == 0) sm.emask[c.u % kRing] = mask;
    };

    // ---------------- tile loads
    // -- one side of a tile (K or V load wave).  The pool
    // rows each lane loads are read first, in one batch of LDS reads (a
    // load's asm orders every later LDS access behind it) ...
    struct Rows {
      int64_t r[C::kHalfOps];
      int64_t own;   // row `lane` (lanes 0-31), for the fp8 scales
    };
    auto side_rows = [&](const Cur &c) {
      Rows w;
      const int es = c.u % kRing;
      const bool f8 = FP8 && c.k < njobs && c.v > 0 && c.v - 1 < c.j.nct;
#pragma unroll
      for (int n = 0; n < C::kHalfOps; ++n) {
        const int r = f8 ? min((n * 1024 + lane * 16) / C::kF8RowB, kTile - 1) : n * kRowsPerOp + lane / C::kChunks;
        w.r[n] = sm.erow[es][r];
      }
      w.own = sm.erow[es][lane & 31];
      return w;
    };
    // ... then its loads: K or V rows (the zero row for a masked one), or
    // the matching head half of a Q tile, or padding past the last job
    auto side_loads = [&](const Cur &c, const Rows &w) {
      const int slot = c.u % kRing;
      uint8_t *dst = vload ? sm.vr[slot] : sm.kr[slot];
      if (c.k >= njobs) {
#pragma unroll
        for (int n = 0; n < C::kHalfOps; ++n) dma16(zero16, sm.dummy);
        return;
      }
      if (c.v == 0) {
        // Q rows of the block's heads, swizzled like a K tile: heads 0-31 in
        // the K slot, 32-63 in the V slot; heads past the KV group read zeros
        const int r0 = vload ? 32 : 0;
        const uint8_t *qb = (const uint8_t *)(p.q + c.j.q) + (r0 + lane / C::kChunks) * C::kRowB;
#pragma unroll
        for (int n = 0; n < C::kHalfOps; ++n) {
          const int r = r0 + n * kRowsPerOp + lane / C::kChunks;
          dma16(r < c.j.nh ? qb + n * 1024 + cs16[n % kPeriod] : zero16, dst + n * 1024);
        }
        return;
      }
      const bool cmp = c.v - 1 < c.j.nct;
      const uint8_t *const base = cmp ? cmp_b : raw_b;
      if (!(FP8 && cmp)) {
        const uint8_t *src[C::kHalfOps];
#pragma unroll
        for (int n = 0; n < C::kHalfOps; ++n)
          src[n] = (w.r[n] >= 0 ? base + w.r[n] * C::kRowB : kZeroRow) + cs16[n % kPeriod];
#pragma unroll
        for (int n = 0; n < C::kHalfOps; ++n) dma16(src[n], dst + n * 1024);
      } else {
        const uint8_t *src[C::kF8HalfOps];
#pragma unroll
        for (int n = 0; n < C::kF8HalfOps; ++n)
          src[n] = (w.r[n] >= 0 ? base + w.r[n] * C::kF8RowB : kZeroRow) + (n * 1024 + lane * 16) % C::kF8RowB;
        const void *ssrc = (lane < kTile && w.own >= 0) ? (const void *)(cmp_sc + w.own) : zero4;
        uint8_t *sdst = vload ? sm.stv[FP8 ? slot : 0] : sm.stk[FP8 ? slot : 0];
#pragma unroll
        for (int n = 0; n < C::kF8HalfOps; ++n) dma16(src[n], sdst + n * 1024);
        dma4(ssrc, vload ? sm.scl_v[FP8 ? slot : 0] : sm.scl_k[FP8 ? slot : 0]);
#pragma unroll
        for (int n = C::kF8HalfOps + 1; n < C::kHalfOps; ++n) dma16(zero16, sm.dummy);
      }
    };
    // -- descriptor of a tile (load wave)
    auto tile_desc = [&](const Cur &c, uint32_t mask) {
      if (c.k >= njobs) return make_uint4(0u, 0u, 0u, 0u);
      if (c.v == 0) return make_uint4(0u, kTileQ, (uint32_t)c.k, 0u);
      const bool cmp = c.v - 1 < c.j.nct;
      uint32_t f = kTileKV;
      if (cmp) f |= kTileCmp;
      if (FP8 && cmp) f |= kTileWiden;
      if (c.v == c.j.nkv) f |= kTileLast;
      return make_uint4(mask, f, (uint32_t)c.k, 0u);
    };
    auto load_step = [&](Cur &c) {
      const Rows w = side_rows(c);
      const uint32_t mask = sm.emask[c.u % kRing];
      side_loads(c, w);
      if (!vload && lane == 0) sm.desc[c.u % kRing] = tile_desc(c, mask);
      advance(c);
    };

    // ---- the stream.  Step t (after barrier t): the load waves issue the K
    // and V sides of tile t+3; the row wave forms the pool rows of tile t+4
    // and the translation wave issues the page entries of tile t+7 and the
    // list entries of tile t+10.  Each wave issues a fixed number of loads per step and,
    // before barrier t+1, waits for its own loads of steps <= t-2: tile t+1
    // for the compute waves, and every stage's input two steps before it is
    // read.
    //
    // Priming, before barrier 0: the translation wave issues the lists of
    // tiles 0-6 (those not loaded early), then their page entries and the
    // lists of tiles 7-9 (each phase complete before the next), and forms
    // the pool rows of tiles 0-3 (the row wave starts at tile 4); after a
    // barrier the load waves issue tiles
    // 1 and 2 (tile 0, job 0's Q tile, was issued at the start).
    Cur cv{0, 0, 0, job(0)};   // load waves: tiles; row wave: rows; translation wave: rows (priming), page entries, lists
    Cur cp = cv, cl = cv;
    if (loader) {
      advance(cv);
    } else if (roww) {
      for (int n = 0; n < 4; ++n) advance(cv);
    } else if (njobs == 0) {
      // a stream with no job: its stages pad
      for (int n = 0; n < 7; ++n) advance(cp);
      for (int n = 0; n < 10; ++n) advance(cl);
      for (int n = 0; n < 4; ++n) advance(cv);
    } else if (njobs == 1 || cv.j.nkv >= 6) {
      // Tiles 1-6 belong to job 0 (or lie past the last job), and the early
      // loads hold the lists of its compressed ones: their rows are resolved
      // lane-parallel, 64 entries (two tiles) per pass, with the page-table
      // loads of all three passes in flight together.  Same results as the
      // per-tile stages below.
      wait_vmcnt<0>();   // the early list loads
      const Job &j0 = cv.j;
      int32_t xr[3], pr[3];
#pragma unroll
      for (int it = 0; it < 3; ++it) {
        const int32_t v = 2 * it + 1 + (lane >> 5);   // tile (stream index) of this lane's entry
        const int32_t row = lane & 31;
        int32_t xv = -1;
        const int32_t *src = nullptr;
        if (v <= j0.nkv) {
          const bool cmp = v - 1 < j0.nct;
          if (cmp) {
            const int32_t idx = (v - 1) * kTile + row;
            if (idx < j0.ncr) {
              if (p.topk > 0) {
                const int32_t le = sm.lst[v % kXRing][row];
                if (le >= 0 && le < j0.nc) xv = le;
                else errbits |= kErrCmpId;
              } else {
                xv = j0.cs + idx;
              }
            }
          } else {
            const int32_t idx = (v - 1 - j0.nct) * kTile + row;
            if (idx < j0.nwr) xv = j0.wb + idx;
          }
          if (xv >= 0) {
            const int32_t col = pow2 ? (xv >> p.page_shift) : xv / P;
            if (col < (cmp ? cmp_st : raw_st)) {
              src = cmp ? cmp_pt + j0.cpt + col : raw_pt + j0.rpt + col;
            } else {
              errbits |= kErrPage;
              xv = -1;
            }
          }
        }
        xr[it] = xv;
        pr[it] = src != nullptr ? *src : 0;
      }
#pragma unroll
      for (int it = 0; it < 3; ++it) {
        const int32_t v = 2 * it + 1 + (lane >> 5);
        const int32_t row = lane & 31;
        sm.xid[v % kXRing][row] = xr[it];
        sm.pg[v % kXRing][row] = pr[it];
        // pool rows of tiles 1-3 (tile 0 is a Q tile)
        if (it < 2) {
          int64_t er = -1;
          if (xr[it] >= 0 && v <= j0.nkv) {
            const bool cmp = v - 1 < j0.nct;
            if (pr[it] >= 0 && (int64_t)pr[it] < (cmp ? cmp_np : raw_np)) {
              const int32_t off = pow2 ? (xr[it] & (P - 1)) : xr[it] - (xr[it] / P) * P;
              er = ((int64_t)pr[it] * P + off) * p.hkv + j0.g;
            } else {
              errbits |= kErrPage;
            }
          }
          const uint64_t m = __ballot(er >= 0);
          if (v <= 3) sm.erow[v % kRing][row] = er;
          if (lane == 0) sm.emask[(2 * it + 1) % kRing] = (uint32_t)m;
          if (lane == 0 && it == 0) sm.emask[2 % kRing] = (uint32_t)(m >> 32);
        }
      }
      for (int n = 0; n < 7; ++n) advance(cp);
      for (int n = 0; n < 7; ++n) advance(cl);
      for (int n = 0; n < 3; ++n) {
        stage_list(cl, false);
        advance(cl);
      }
      for (int n = 0; n < 4; ++n) advance(cv);
      wait_vmcnt<0>();
    } else {
      wait_vmcnt<0>();   // the early list loads land before any stage reuses their slots
      for (int n = 0; n < 7; ++n) {
        // the early loads hold the lists of job 0's first compressed tiles
        const bool early = cl.k == 0 && cl.v >= 1 && cl.v <= nspec && cl.v - 1 < cl.j.nct;
        if (!early) stage_list(cl, false);
        advance(cl);
      }
      wait_vmcnt<0>();
      for (int n = 0; n < 7; ++n) {
        stage_page(cp, list_entry(cp), false);
        advance(cp);
      }
      for (int n = 0; n < 3; ++n) {
        stage_list(cl, false);
        advance(cl);
      }
      wait_vmcnt<0>();
      for (int n = 0; n < 4; ++n) {
        stage_rows(cv, sm.xid[cv.u % kXRing][lane & 31], sm.pg[cv.u % kXRing][lane & 31]);
        advance(cv);
      }
    }
    block_sync();   // pool rows of tiles 0-3 are in
    // every stream takes as many steps as the longest (a finished one pads)
    if (NS > 1) T = max(sm_all[0].ntiles, sm_all[NS - 1].ntiles);
    if (loader) {
      load_step(cv);                   // tile 1; tile 2 waits for step 0 (the Q tile's short step)
      wait_vmcnt<C::kLoadOps>();       // tile 0 (its side)
    }
    for (int t = 0; t < T; ++t) {
      block_sync();   // barrier t
      if (FP8 && (sm.desc[t % kRing].y & kTileWiden)) block_sync();   // the compute waves widen tile t
      if (loader) {
        if (t == 0) load_step(cv);
        load_step(cv);
        wait_vmcnt<2 * C::kLoadOps>();
      } else if (roww) {
        stage_rows(cv, sm.xid[cv.u % kXRing][lane & 31], sm.pg[cv.u % kXRing][lane & 31]);
        advance(cv);
      } else {
        stage_page(cp, list_entry(cp), true);
        advance(cp);
        stage_list(cl, true);
        advance(cl);
        wait_vmcnt<2 * 2>();
      }
    }
    wait_vmcnt<0>();
    const int32_t eb = (__any(errbits & kErrCmpId) ? kErrCmpId : 0) | (__any(errbits & kErrPage) ? kErrPage : 0);
    if (lane == 0 && eb != 0 && p.err_flag != nullptr) atomicOr(p.err_flag, eb);
    return;
  }

  // =================================================================
  // Compute waves
  // =================================================================
  const int hw = wave % C::NC;                // this wave's 32-head block within the job's heads
  block_sync();                               // priming: the page entries of tiles 0-5 are in
  const int32_t T = NS == 1 ? sm.ntiles : max(sm_all[0].ntiles, sm_all[NS - 1].ntiles);
  block_sync();                               // barrier 0: tile 0 is in

  // per-job state
  bf16x8 qf[D / 16];                          // Q^T as the B operand: head lane%32, d = 16kk + 8hi ..+7
  float m = -INFINITY, l = 0.f;
  f32x16 acc[D / 32];
  // sink logit of this lane's head in job k (-inf: none), loaded one job
  // ahead so that its load is long complete when the job starts
  auto load_sink = [&](int32_t k) {
    const JobId j = jid(k);
    const int hl = j.hb * p.heads_per_block + hw * 32 + (lane & 31);
    return (j.valid && S == 1 && p.sink != nullptr && hl < p.group) ? p.sink[j.g * p.group + hl] : -INFINITY;
  };
  float sink_next = load_sink(0);
  auto init_job = [&](int32_t k) {
    m = sink_next == -INFINITY ? -INFINITY : sink_next * kLog2e;
    l = (sink_next != -INFINITY && hi == 0) ? 1.f : 0.f;   // exp2(sink - m) = 1, counted once per head
#pragma unroll
    for (int db = 0; db < D / 32; ++db) acc[db] = f32x16{};
    sink_next = load_sink(k + 1);
  };
  auto epilogue = [&](int32_t k) {
    const JobId j = jid(k);
    const int hl = j.hb * p.heads_per_block + hw * 32 + (lane & 31);
    const float lt = l + __shfl_xor(l, 32);
    const float inv = lt > 0.f ? 1.f / lt : 0.f;
    const float lse2 = (m == -INFINITY || !(lt > 0.f)) ? -INFINITY : m + __builtin_amdgcn_logf(lt);
    const float lse = lse2 == -INFINITY ? -INFINITY : lse2 * kLn2;
    if (hl >= p.group) return;
    const int h = j.g * p.group + hl;
    if (S == 1) {
      uint16_t *orow = p.o + ((int64_t)j.qi * p.hq + h) * D;
#pragma unroll
      for (int db = 0; db < D / 32; ++db) {
#pragma unroll
        for (int i4 = 0; i4 < 4; ++i4) {
          const int d0 = 32 * db + 8 * i4 + 4 * hi;
          uint2 w;
          w.x = bf16_bits(acc[db][4 * i4 + 0] * inv) | (bf16_bits(acc[db][4 * i4 + 1] * inv) << 16);
          w.y = bf16_bits(acc[db][4 * i4 + 2] * inv) | (bf16_bits(acc[db][4 * i4 + 3] * inv) << 16);
          *(uint2 *)(orow + d0) = w;
        }
      }
      if (hi == 0 && p.lse) p.lse[(int64_t)j.qi * p.hq + h] = lse;
    } else {
      // split: the sink-free partial; the merge kernel adds the sink
      const int64_t prow = ((int64_t)j.split * p.num_queries + j.qi) * p.hq + h;
      float *orow = p.part_o + prow * D;
#pragma unroll
      for (int db = 0; db < D / 32; ++db) {
#pragma unroll
        for (int i4 = 0; i4 < 4; ++i4) {
          const int d0 = 32 * db + 8 * i4 + 4 * hi;
          *(float4 *)(orow + d0) = make_float4(acc[db][4 * i4] * inv, acc[db][4 * i4 + 1] * inv,
                                               acc[db][4 * i4 + 2] * inv, acc[db][4 * i4 + 3] * inv);
        }
      }
      if (hi == 0) p.part_lse[prow] = lse;
    }
  };

  // Q fragments of this wave's heads from a Q tile in ring slot `slot`
  // (heads 0-31 in the K slot, 32-63 in the V slot, swizzled like a K tile)
  auto load_q = [&](int slot) {
    const uint8_t *Qt = hw == 0 ? sm.kr[slot] : sm.vr[slot];
    const int r = lane & 31;
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk) {
      const int c = 2 * kk + hi;
      qf[kk] = *(const bf16x8 *)(Qt + r * C::kRowB + ((c ^ swz<C::kChunks>(r)) * 16));
    }
  };

  // FP8: widen a staged e4m3 tile (OCP, or FNUZ) to bf16 (exact) into its
  // swizzled slot
  const bool fnuz = FP8 && p.cmp_fnuz != 0;
  auto widen = [&](const uint8_t *src, uint8_t *dst) {
    constexpr int kPieces = kTile * D / 8;   // 8-byte pieces per tile
    for (int idx = hw * 64 + lane; idx < kPieces; idx += C::kThreads) {
      const int r = idx / (D / 8);
      const int piece = idx - r * (D / 8);
      const uint2 w = *(const uint2 *)(src + r * D + piece * 8);
      const uint4 o = widen8_e4m3(w, fnuz);
      *(uint4 *)(dst + r * C::kRowB + ((piece ^ swz<C::kChunks>(r)) * 16)) = o;
    }
  };

  // S^T = K . Q^T for the tile in K slot `slot`
  auto scores = [&](int slot) {
    const uint8_t *Kt = sm.kr[slot];
    const int r = lane & 31;
    f32x16 s = f32x16{};
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk) {
      const int c = 2 * kk + hi;
      const bf16x8 a = *(const bf16x8 *)(Kt + r * C::kRowB + ((c ^ swz<C::kChunks>(r)) * 16));
      s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[kk], s, 0, 0, 0);
    }
    return s;
  };

  // Online softmax of a tile's scores, then O^T += V^T . P^T.  Lane rows:
  // 8*(i/4) + 4*hi + i%4.  The max is taken on the raw scores (the scale
  // c = scale*log2 e is positive), and p = exp2(s*c - m) is one FMA and one
  // exp per score.
  auto softmax_pv = [&](auto masked, const f32x16 &s, uint32_t tm, int slot, bool cmp) {
    float sc[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) sc[i] = s[i];
    if (FP8 && cmp) {
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const float4 kk4 = *(const float4 *)(&sm.scl_k[FP8 ? slot : 0][8 * q4 + 4 * hi]);
        sc[4 * q4 + 0] *= kk4.x;
        sc[4 * q4 + 1] *= kk4.y;
        sc[4 * q4 + 2] *= kk4.z;
        sc[4 * q4 + 3] *= kk4.w;
      }
    }
    if constexpr (decltype(masked)::value) {
      const uint32_t tmh = tm >> (4 * hi);   // row 8*(i/4) + 4*hi + i%4 is bit 8*(i/4) + i%4 of tmh
#pragma unroll
      for (int i = 0; i < 16; ++i) sc[i] = ((tmh >> (8 * (i >> 2) + (i & 3))) & 1u) ? sc[i] : -INFINITY;
    }
    float smax = fmaxf(fmaxf(fmaxf(sc[0], sc[1]), fmaxf(sc[2], sc[3])), fmaxf(fmaxf(sc[4], sc[5]), fmaxf(sc[6], sc[7])));
    smax = fmaxf(smax, fmaxf(fmaxf(fmaxf(sc[8], sc[9]), fmaxf(sc[10], sc[11])),
                             fmaxf(fmaxf(sc[12], sc[13]), fmaxf(sc[14], sc[15]))));
    smax = max_lane_pair(smax);
    const float tmax = smax * p.scale_log2;               // -inf stays -inf
    const bool need = tmax > m + kTau;                     // same on both lanes of a head
    if (__any(need)) {
      const float alpha = need ? __builtin_amdgcn_exp2f(m - tmax) : 1.f;   // m = -inf -> 0
      m = need ? tmax : m;
      l *= alpha;
#pragma unroll
      for (int db = 0; db < D / 32; ++db) acc[db] *= alpha;
    }
    const float negm = m == -INFINITY ? 0.f : -m;          // all scores are -inf then
    float pr[16];
    float psum = 0.f;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      pr[i] = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[i], p.scale_log2, negm));
      psum += pr[i];
    }
    l += psum;
    if (FP8 && cmp) {
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const float4 vv = *(const float4 *)(&sm.scl_v[FP8 ? slot : 0][8 * q4 + 4 * hi]);
        pr[4 * q4 + 0] *= vv.x;
        pr[4 * q4 + 1] *= vv.y;
        pr[4 * q4 + 2] *= vv.z;
        pr[4 * q4 + 3] *= vv.w;
      }
    }
    bf16x8 pb[2];
#pragma unroll
    for (int k2 = 0; k2 < 2; ++k2)
#pragma unroll
      for (int j = 0; j < 8; ++j) pb[k2][j] = (__bf16)pr[8 * k2 + j];

    // V^T from the transpose read of the row-major tile
    const uint8_t *Vt = sm.vr[slot];
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
          const int off = row * C::kRowB + (((d >> 3) ^ swz<C::kChunks>(row)) * 16) + (L & 1) * 8;
          part[rr] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t *)(Vt + off));
        }
        const i16x8 cat = {part[0][0], part[0][1], part[0][2], part[0][3],
                           part[1][0], part[1][1], part[1][2], part[1][3]};
        acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, cat), pb[k2], acc[db], 0, 0, 0);
      }
    }
  };

  // The stream: step t (after barrier t) consumes tile t, either a job's Q
  // tile (its fragments into registers) or one of its KV tiles (scores,
  // online softmax, PV product; the job's output after its last tile).  The
  // load wave refills tile t's slot only after barrier t+1.
  init_job(0);
  for (int t = 0; t < T; ++t) {
    if (t > 0) block_sync();                  // barrier t (barrier 0 was taken above)
    const int slot = t % kRing;
    const uint4 d = sm.desc[slot];
    if (d.y & kTileWiden) {
      if (FP8) {
        widen(sm.stk[FP8 ? slot : 0], sm.kr[slot]);
        widen(sm.stv[FP8 ? slot : 0], sm.vr[slot]);
      }
      block_sync();
    }
    if (d.y & kTileQ) {
      load_q(slot);
    } else if (d.y & kTileKV) {
      const bool cmp = (d.y & kTileCmp) != 0;
      const f32x16 s = scores(slot);
      if (d.x == 0xFFFFFFFFu) softmax_pv(std::false_type{}, s, d.x, slot, cmp);
      else softmax_pv(std::true_type{}, s, d.x, slot, cmp);
      if (d.y & kTileLast) {
        epilogue((int32_t)d.z);
        init_job((int32_t)d.z + 1);
      }
    }
  }
}

template <int D, int NH, int NS, bool FP8>
hipError_t launch_t(const Params &p0, hipStream_t stream) {
  using C = Cfg<D, NH, FP8>;
  constexpr int kBlock = NS * C::kBlock;
  static int resident[64] = {};   // workgroups resident at once, per device
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
  if (resident[dev] == 0) {
    int per_cu = 0, cus = 0;
    e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, attn_fwd_kernel<D, NH, NS, FP8>, kBlock, 0);
    if (e != hipSuccess) return e;
    e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return e;
    resident[dev] = std::max(8, per_cu * cus / 8 * 8);
  }
  const int64_t units = (int64_t)p0.num_queries * p0.hkv;
  const int64_t R = p0.jobs_per_unit;
  const int64_t G = std::min<int64_t>(resident[dev], (units * R + 7) / 8 * 8);
  const int64_t Gx = G / 8;
  // units per launch: 8 * floor(NS * kMaxJobs * Gx / R), so that no stream
  // gets more than kMaxJobs jobs (every XCD gets at most upl / 8 units)
  const int64_t upl = 8 * std::max<int64_t>(1, NS * C::kMaxJobs * Gx / R);
  if ((upl / 8) * R > NS * C::kMaxJobs * Gx) return hipErrorInvalidConfiguration;
  Params p = p0;
  for (int64_t u0 = 0; u0 < units; u0 += upl) {
    p.unit_begin = (int32_t)u0;
    p.unit_end = (int32_t)std::min(units, u0 + upl);
    hipLaunchKernelGGL((attn_fwd_kernel<D, NH, NS, FP8>), dim3((unsigned)G), dim3(kBlock), 0, stream, p);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

template <int D, bool FP8>
hipError_t launch_d(const Params &p, hipStream_t stream) {
  const int heads = p.group < p.heads_per_block ? p.group : p.heads_per_block;
  // 64-head jobs in bf16: two streams per workgroup (one workgroup per CU,
  // a compute wave on every SIMD); otherwise one stream (two workgroups per
  // CU)
  if (heads <= 32) return launch_t<D, 1, 1, FP8>(p, stream);
  if constexpr (FP8) return launch_t<D, 2, 1, FP8>(p, stream);
  else return launch_t<D, 2, 2, FP8>(p, stream);
}

}  // namespace

hipError_t launch_attention(const Params &p, hipStream_t stream) {
  if (p.num_queries == 0) return hipSuccess;
  if (p.head_dim == 64) return p.cmp_fp8 ? launch_d<64, true>(p, stream) : launch_d<64, false>(p, stream);
  return p.cmp_fp8 ? launch_d<128, true>(p, stream) : launch_d<128, false>(p, stream);
}

}  // namespace spa
