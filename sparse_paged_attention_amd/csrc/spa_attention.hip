// Sparse paged attention forward with a sink, for gfx950 (CDNA4).
//
// Operation: RL-Kernel PR "Roadmap item 24: joint compressed/window attention
// with sink", section "Reuse and arithmetic" — the selected compressed KV, the
// full recent raw window and a per-head sink logit share one softmax
// denominator; the sink has no value row; P and O are bf16, LSE is fp32
// natural log.  The KV set and page translation live in spa_device.h.
//
// Work decomposition.  A job is (query group, KV head, KV slice, block of
// query heads).  A query group is NQ queries (1 for decode; consecutive
// prefill tokens otherwise).  All query heads of a KV head read the same KV
// rows, and consecutive tokens of one sequence read mostly the same rows
// (overlapping windows, mostly shared compressed groups), so a workgroup
// streams one KV stream for the whole group through LDS and every compute
// wave feeds each tile to bf16 MFMAs for its (token, 32 query heads):
//
//   S^T[kv, head]  = K[kv, :] . Q^T[:, head]        v_mfma_f32_32x32x16_bf16
//   O^T[d, head]  += V^T[d, kv] . P^T[kv, head]      v_mfma_f32_32x32x16_bf16
//
// With S^T and O^T in the MFMA accumulator layout every lane owns one query
// head (lane % 32), so the online-softmax state (m, l) is per lane; the row
// max needs one exchange with lane ^ 32, and P^T goes from the S^T
// accumulators straight into the B operand of the PV MFMA (the KV order inside
// a 16-row step is permuted identically on both operands).  V^T comes from the
// row-major V tile through the gfx950 LDS transpose read (ds_read_b64_tr_b16),
// so no transposition pass is needed.
//
// The group's stream.  When the group's queries belong to one sequence, sit
// within one window span of each other and (for a listed layer) their group
// ids fit an LDS bitmap, the stream is the union of their KV sets: the union
// of the compressed lists (built in LDS: one bit per (id, token), then
// compacted in ascending id order), then the union of the windows; each row
// carries a token mask and every compute wave masks the rows its token does
// not see.  Otherwise the workgroup makes one pass per query over that
// query's own set.  Masked work is never counted as useful.
//
// Grid.  Jobs are numbered (group, KV head, slice, head block) with the head
// block fastest and dealt to the 8 XCDs in contiguous ranges (workgroup w runs
// job (w % 8) * ceil(jobs/8) + w / 8), so the head blocks that read the same
// KV rows land on one XCD and share its L2.  This affects speed only, never
// results.
//
// Data movement.  The rows of up to 16 tiles are translated first (list
// loads for the whole batch, then page-table loads), then every tile is
// fetched by direct global->LDS loads (global_load_lds_dwordx4, 16 B per
// lane, no VGPR staging) into a ring of NBUF LDS buffers.  One extra wave per
// workgroup is the producer: it issues all tile loads and waits for them, so
// the compute waves never stall on a full memory queue; one barrier per tile
// hands a filled buffer to the compute waves and returns the previous one.
// Masked rows are fetched from a static zero row and excluded through the
// per-tile row masks, so the producer issues the same number of loads per
// tile and one vmcnt immediate tracks the ring.  LDS rows are XOR-swizzled in
// 16-byte chunks so that the K reads (one row per lane) and the transpose
// reads (4 rows x 32 B per 16 lanes) are free of bank conflicts.
//
// FP8 (OCP e4m3) compressed rows land in an LDS staging area, together with
// their fp32 per-token scales (one 4-byte direct load per row), and are
// widened to bf16 exactly (every e4m3 value is a bf16 value) by the hardware
// v_cvt_pk_f32_fp8; the scales are applied in fp32 to the scores (k) and to
// P (v), so the MFMAs see the exact codes.
//
// Softmax runs in the log2 domain (scores pre-multiplied by scale*log2 e,
// sink by log2 e) with v_exp_f32; with one slice the running max starts at
// the sink and the running sum at exp(0) = 1, i.e. the sink is folded into
// (m, l) from the start.  With num_splits > 1 (decode) each slice writes a
// sink-free partial (O_s f32, LSE_s) to the workspace and the merge kernel
// (spa_merge.hip) combines them, adding the sink exactly once.

#include <hip/hip_runtime.h>

#include <cstdint>

#include "spa_device.h"

namespace spa {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef short i16x8 __attribute__((ext_vector_type(8)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4_t;

constexpr int kTile = 32;        // KV rows per tile
constexpr int kChunkTiles = 16;  // tiles translated per page-table pass
constexpr int kUnionCap = 4096;  // compressed ids a group union may span
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
// The running max used for the exponentials moves only when a tile's max
// exceeds it by more than kTau (log2 units), so P and the sums stay below
// 2^kTau and the O accumulators are rescaled only on such jumps.  Any
// reference value gives the same softmax; only the rounding differs.
constexpr float kTau = 8.f;

// Source of the 16-byte loads for masked rows (and of padding loads).
__device__ __attribute__((aligned(16))) const uint8_t kZeroRow[256] = {};

// LDS byte offset of a generic pointer into shared memory: the LDS aperture
// is 4 GiB aligned in the flat address space, so the low 32 bits are the
// offset (this avoids a checked generic->local address-space cast).
__device__ __forceinline__ uint32_t lds_offset(const void *p) { return (uint32_t)(uintptr_t)p; }

#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"   // M0 is reserved; only these loads use it here
// One wave-wide direct global->LDS load: lane L's 16 (or 4) bytes from `src`
// land at lds_dst + 16 L (or 4 L); lds_dst is wave-uniform and goes through
// M0.  Written as inline asm so that the compiler does not guard every later
// LDS read with a wait for all outstanding loads; completion is tracked
// explicitly with wait_vmcnt<>.  The instructions have no destination
// registers.
__device__ __forceinline__ void dma16(const void *src, void *lds_dst) {
  const uint32_t lds = __builtin_amdgcn_readfirstlane(lds_offset(lds_dst));
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off"
               :
               : "v"(src), "s"(lds)
               : "memory", "m0");
}
__device__ __forceinline__ void dma4(const void *src, void *lds_dst) {
  const uint32_t lds = __builtin_amdgcn_readfirstlane(lds_offset(lds_dst));
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dword %0, off"
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

// Wait until at most `ahead` tiles of OPS loads each are still in flight.
template <int OPS, int MAXA>
__device__ __forceinline__ void wait_tiles(int ahead) {
  static_assert(MAXA <= 5 && MAXA * OPS < 64, "ring depth");
  if (MAXA >= 5 && ahead >= 5) wait_vmcnt<(MAXA >= 5 ? 5 * OPS : 0)>();
  else if (MAXA >= 4 && ahead >= 4) wait_vmcnt<(MAXA >= 4 ? 4 * OPS : 0)>();
  else if (MAXA >= 3 && ahead >= 3) wait_vmcnt<(MAXA >= 3 ? 3 * OPS : 0)>();
  else if (MAXA >= 2 && ahead >= 2) wait_vmcnt<(MAXA >= 2 ? 2 * OPS : 0)>();
  else if (MAXA >= 1 && ahead >= 1) wait_vmcnt<OPS>();
  else wait_vmcnt<0>();
}

// Workgroup barrier that waits only for this wave's LDS operations.  The
// HIP __syncthreads() adds a workgroup release fence, which on gfx950 also
// waits for every outstanding global load and would drain the LDS ring;
// global->LDS loads are instead completed explicitly with wait_vmcnt<>.
// The "memory" clobber keeps the compiler from moving LDS accesses across it.
__device__ __forceinline__ void block_sync() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

__device__ __forceinline__ uint32_t pack_bf16_hi(float lo, float hi) {
  // exact narrowing for values that are bf16 already (widened e4m3 codes)
  return (__builtin_bit_cast(uint32_t, lo) >> 16) | (__builtin_bit_cast(uint32_t, hi) & 0xFFFF0000u);
}

__device__ __forceinline__ int round_up(int x, int m) { return (x + m - 1) / m * m; }

__device__ __forceinline__ uint32_t bf16_bits(float x) { return __builtin_bit_cast(uint16_t, (__bf16)x); }

template <int D, int NH, int NQ, bool FP8, int NBUF>
struct Cfg {
  static constexpr int NC = NH * NQ;                  // compute waves
  static constexpr int kThreads = NC * 64;            // compute threads
  static constexpr int kBlock = (NC + 1) * 64;        // + one producer wave
  static constexpr int kRowB = 2 * D;                 // bf16 row bytes
  static constexpr int kChunks = kRowB / 16;          // 16-byte chunks per row
  static constexpr int kTileB = kTile * kRowB;        // one K (or V) tile, bytes
  static constexpr int kKVInstr = 2 * kTileB / 1024;  // wave-wide 1 KiB loads per tile
  static constexpr int kOps = kKVInstr;               // producer loads per tile
  static constexpr int kF8TileB = kTile * D;          // one e4m3 K (or V) tile
  static constexpr int kF8Instr = 2 * kF8TileB / 1024;
  static constexpr int kSlots = kChunkTiles * kTile;
  static constexpr int kPer = kSlots / kThreads;      // translation slots per thread
  static_assert(NC <= 4, "compute waves (5 waves per workgroup keep 256 VGPRs per lane)");
  static_assert(!FP8 || kF8Instr + 1 <= kOps, "fp8 tiles: data + scale loads fit the per-tile count");
  static_assert((NBUF - 2) * kOps < 64, "vmcnt range");
  static_assert(kSlots % kThreads == 0, "slots");
};

template <int D, int NH, int NQ, bool FP8, int NBUF>
struct Smem {
  using C = Cfg<D, NH, NQ, FP8, NBUF>;
  static constexpr int kU = NQ > 1 ? kUnionCap : 4;
  alignas(16) uint8_t kv[NBUF][2][C::kTileB];
  alignas(16) uint8_t stage[FP8 ? NBUF : 1][2][FP8 ? C::kF8TileB : 16];
  alignas(16) float scl[FP8 ? NBUF : 1][64];          // k scales [0,32), v scales [32,64)
  alignas(16) uint8_t dummy[FP8 ? 1024 : 16];
  alignas(16) int64_t erow[C::kSlots];                 // element row (row*Hkv+g), -1 = masked
  uint32_t tmask[kChunkTiles][NQ];                     // bit r: row r of the tile is seen by token q
  // group union (NQ > 1): per-id token bits, then the compacted list
  alignas(16) uint32_t ubits[kU / 4];                  // byte c: tokens whose list holds id c
  alignas(16) int32_t uid[kU];                         // union ids, ascending
  uint8_t umask[kU];                                   // token bits of uid[k]
  int32_t scan[C::kThreads];
  QueryKV qkv[NQ];                                     // the group's queries
  int32_t gshared, gnq, gwlo, gnwr, gncmax, gnu;
};

// The KV stream of one pass: compressed rows [0, ncr) then window rows
// [0, nwr); compressed tiles first, window tiles start on a tile boundary.
struct Stream {
  int ncr, nwr, nct, total;
  __device__ __forceinline__ void tile(int j, int &k0, int &len, bool &cmp) const {
    if (j < nct) {
      k0 = j * kTile;
      len = min(kTile, ncr - k0);
      cmp = true;
    } else {
      k0 = (j - nct) * kTile;
      len = min(kTile, nwr - k0);
      cmp = false;
    }
  }
};

template <int D, int NH, int NQ, bool FP8, int NBUF>
__global__ __launch_bounds__((NH * NQ + 1) * 64) void attn_fwd_kernel(const Params p) {
  using C = Cfg<D, NH, NQ, FP8, NBUF>;
  __shared__ Smem<D, NH, NQ, FP8, NBUF> sm;

  // ---- job of this workgroup (XCD-contiguous numbering)
  const int job = (int)(blockIdx.x & 7) * p.jobs_per_xcd + (int)(blockIdx.x >> 3);
  if (job >= p.total_jobs) return;
  const int S = p.num_splits;
  int t = job;
  const int hgw = t % p.head_groups;
  t /= p.head_groups;
  const int split = t % S;
  t /= S;
  const int g = t % p.hkv;
  const int grp = t / p.hkv;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int hi = lane >> 5;                  // which half of the wave
  const bool producer = wave == C::NC;       // the last wave only moves data
  const int qt = producer ? 0 : wave / NH;   // this wave's token within the group
  const int hw = producer ? 0 : wave % NH;   // this wave's 32-head block within the workgroup's heads
  const int qi = grp * NQ + qt;              // this wave's query
  const bool q_ok = !producer && qi < p.num_queries;
  const int hl = hgw * p.heads_per_block + hw * 32 + (lane & 31);   // head within the KV group
  const bool head_ok = q_ok && hl < p.group;
  const bool wave_ok = q_ok && hgw * p.heads_per_block + hw * 32 < p.group;
  const int h = g * p.group + hl;

  // ---- Q^T as the B operand: lane holds head (lane%32), d = 16kk + 8*hi ..+7
  bf16x8 qf[D / 16];
  {
    const uint16_t *qrow = p.q + ((int64_t)(q_ok ? qi : 0) * p.hq + (head_ok ? h : 0)) * D;
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk) {
      uint4 v = head_ok ? *(const uint4 *)(qrow + 16 * kk + 8 * hi) : make_uint4(0, 0, 0, 0);
      qf[kk] = __builtin_bit_cast(bf16x8, v);
    }
  }

  // ---- decode (one query per group): the slice's list entries of the first
  // chunk are loaded right away, together with Q and the query's counts.
  // Slices are cut by capacity: list slots [cs, ce) of the compressed part
  // (the top-k list, or the n_c groups of an all-groups layer) and window
  // slots [ws, we).
  int32_t xl[C::kPer];
  const int lper = (NQ == 1 && p.topk > 0) ? round_up((p.topk + S - 1) / S, kTile) : 0;
  const int ls = min(p.topk, split * lper);
  const int le = NQ == 1 ? min(p.topk, ls + lper) : 0;
#pragma unroll
  for (int u = 0; u < C::kPer; ++u) {
    const int e = ls + tid + u * C::kThreads;   // slot idx -> tile idx/32, row idx%32
    xl[u] = (!producer && e < le) ? p.cmp_idx[(int64_t)grp * p.topk + e] : -1;
  }

  // ---- the group's queries, in LDS (computed once, read uniformly)
  if (tid < NQ) {
    const int i = grp * NQ + tid;
    sm.qkv[tid] = i < p.num_queries ? query_kv(p, i) : QueryKV{0, 0, 0, 0, 0, 0};
  }
  block_sync();
  if (tid == 0) {
    int nqv = 0;
    bool same = true;
    int tmax = -1, wlo = 0x7FFFFFFF, ncm = 0;
    for (int q = 0; q < NQ; ++q) {
      if (grp * NQ + q >= p.num_queries) break;
      const QueryKV k = sm.qkv[q];
      ++nqv;
      // a query whose metadata failed validation has an empty set
      same = same && k.b == sm.qkv[0].b && k.win_len + k.n_sel > 0;
      tmax = max(tmax, k.t);
      wlo = min(wlo, k.win_lo);
      ncm = max(ncm, k.n_c);
    }
    const int nwr = max(0, tmax - wlo + 1);
    sm.gnq = nqv;
    sm.gwlo = wlo;
    sm.gnwr = nwr;
    sm.gncmax = ncm;
    sm.gshared = NQ > 1 && nqv > 1 && same && S == 1 && nwr <= 2 * p.window + 2 * NQ &&
                 (p.topk == 0 || ncm <= kUnionCap);
  }
  block_sync();
  const bool shared = sm.gshared != 0;
  const int nq_valid = sm.gnq;

  // ---- online softmax state (log2 domain); the sink is folded in up front
  float m = -INFINITY, l = 0.f;
  if (S == 1 && p.sink != nullptr && head_ok) {
    m = p.sink[h] * kLog2e;
    l = hi == 0 ? 1.f : 0.f;   // exp2(sink - m) = 1, counted once per head
  }
  f32x16 acc[D / 32];
#pragma unroll
  for (int db = 0; db < D / 32; ++db) acc[db] = f32x16{};

  const int npass = shared ? 1 : (NQ == 1 ? 1 : nq_valid);
  for (int pass = 0; pass < npass; ++pass) {
    // ---- this pass's stream
    const int pq = shared ? 0 : pass;          // the query of a single-query pass
    const QueryKV pkv = sm.qkv[pq];
    const int pqi = grp * NQ + pq;
    Stream st;
    int c_base = 0, w_base = 0;                // first list entry / first window position
    int nu = 0;                                // union size (listed layers)
    if (shared) {
      if (p.topk > 0) {
        // union of the lists: token bits per id, then compaction in id order
        for (int w = producer ? kUnionCap : tid; w < kUnionCap / 4; w += C::kThreads) sm.ubits[w] = 0u;
        block_sync();
        if (!producer) {
#pragma unroll
          for (int q = 0; q < NQ; ++q) {
            if (q < nq_valid) {
              const int i = grp * NQ + q;
              const QueryKV kq = sm.qkv[q];
              for (int e = tid; e < kq.n_sel; e += C::kThreads) {
                const int c = check_cmp_id(p, kq, p.cmp_idx[(int64_t)i * p.topk + e]);
                if (c >= 0) atomicOr(&sm.ubits[c >> 2], 1u << (8 * (c & 3) + q));
              }
            }
          }
        }
        block_sync();
        // compaction: thread t owns ids [t*per, (t+1)*per)
        const int ncmax = sm.gncmax;
        const int per = (ncmax + C::kThreads - 1) / C::kThreads;
        int cnt = 0;
        if (!producer) {
          for (int c = tid * per; c < min(ncmax, (tid + 1) * per); ++c)
            cnt += ((sm.ubits[c >> 2] >> (8 * (c & 3))) & 0xFFu) != 0u;
          sm.scan[tid] = cnt;
        }
        block_sync();
        if (wave == 0) {   // exclusive scan of the per-thread counts
          constexpr int kPerLane = (C::kThreads + 63) / 64;
          int v[kPerLane];
          int sum = 0;
#pragma unroll
          for (int k = 0; k < kPerLane; ++k) {
            const int idx = lane * kPerLane + k;
            v[k] = idx < C::kThreads ? sm.scan[idx] : 0;
            sum += v[k];
          }
          int inc = sum;
#pragma unroll
          for (int d = 1; d < 64; d <<= 1) {
            const int o = __shfl_up(inc, d);
            if (lane >= d) inc += o;
          }
          int run = inc - sum;
#pragma unroll
          for (int k = 0; k < kPerLane; ++k) {
            const int idx = lane * kPerLane + k;
            if (idx < C::kThreads) sm.scan[idx] = run;
            run += v[k];
          }
        }
        block_sync();
        if (!producer) {
          int pos = sm.scan[tid];
          for (int c = tid * per; c < min(ncmax, (tid + 1) * per); ++c) {
            const uint32_t bits = (sm.ubits[c >> 2] >> (8 * (c & 3))) & 0xFFu;
            if (bits) {
              sm.uid[pos] = c;
              sm.umask[pos] = (uint8_t)bits;
              ++pos;
            }
          }
        }
        {
          // total = last thread's offset + its count
          block_sync();
          nu = sm.scan[C::kThreads - 1];
          int lastcnt = 0;
          const int tl = C::kThreads - 1;
          for (int c = tl * per; c < min(ncmax, (tl + 1) * per); ++c)
            lastcnt += ((sm.ubits[c >> 2] >> (8 * (c & 3))) & 0xFFu) != 0u;
          nu += lastcnt;
        }
        st.ncr = nu;
      } else {
        st.ncr = sm.gncmax;   // all-groups layer: ids [0, ncmax), token q sees ids < n_c(q)
      }
      st.nwr = sm.gnwr;
      w_base = sm.gwlo;
    } else {
      // one query: its own set, or its slice of it (decode splits)
      const int ccap = p.topk > 0 ? p.topk : pkv.n_sel;
      const int cper = round_up((ccap + S - 1) / S, kTile);
      const int cs = min(ccap, split * cper);
      const int ce = min(ccap, cs + cper);
      const int wper = round_up((p.window + S - 1) / S, kTile);
      const int ws = min(pkv.win_len, split * wper);
      const int we = min(pkv.win_len, ws + wper);
      c_base = cs;
      st.ncr = max(0, min(ce, pkv.n_sel) - cs);
      st.nwr = we - ws;
      w_base = pkv.win_lo + ws;
    }
    st.nct = (st.ncr + kTile - 1) / kTile;
    st.total = st.nct + (st.nwr + kTile - 1) / kTile;
    const bool use_xl = NQ == 1 && p.topk > 0;

    for (int cbase = 0; cbase < st.total; cbase += kChunkTiles) {
      const int ct = min(kChunkTiles, st.total - cbase);
      block_sync();   // the previous chunk (or pass) is done with the row table
      // -- translation (compute waves): all list loads of the batch, then all
      // page-table loads
      if (!producer) {
        int32_t x[C::kPer];
        bool cmpk[C::kPer];
        uint32_t tok[C::kPer];   // token bits of the row
#pragma unroll
        for (int u = 0; u < C::kPer; ++u) {
          const int idx = tid + u * C::kThreads;
          const int j = cbase + idx / kTile;
          const int r = idx % kTile;
          x[u] = -1;
          cmpk[u] = false;
          tok[u] = 0u;
          if (idx < ct * kTile) {
            int k0, len;
            bool cmp;
            st.tile(j, k0, len, cmp);
            cmpk[u] = cmp;
            const int k = k0 + r;
            if (r < len) {
              if (cmp) {
                if (shared) {
                  if (p.topk > 0) {
                    x[u] = sm.uid[k];
                    tok[u] = sm.umask[k];
                  } else {
                    x[u] = k;
#pragma unroll
                    for (int q = 0; q < NQ; ++q)
                      if (q < nq_valid && k < sm.qkv[q].n_c) tok[u] |= 1u << q;
                  }
                } else {
                  // chunk 0 of a decode list: the list entry was loaded up front
                  x[u] = (use_xl && cbase == 0) ? check_cmp_id(p, pkv, xl[u])
                                                : entry_logical(p, pkv, pqi, c_base + k);
                  tok[u] = 1u << pq;
                }
              } else {
                const int pos = w_base + k;
                x[u] = pos;
                if (shared) {
#pragma unroll
                  for (int q = 0; q < NQ; ++q)
                    if (q < nq_valid && pos >= sm.qkv[q].win_lo && pos <= sm.qkv[q].t) tok[u] |= 1u << q;
                } else {
                  tok[u] = 1u << pq;
                }
              }
            }
          }
        }
#pragma unroll
        for (int u = 0; u < C::kPer; ++u) {
          const int idx = tid + u * C::kThreads;
          const int64_t row = logical_row(p, pkv, cmpk[u], x[u]);
          sm.erow[idx] = row >= 0 ? row * p.hkv + g : -1;
          // a tile's 32 slots are 32 consecutive lanes of one wave
#pragma unroll
          for (int q = 0; q < NQ; ++q) {
            const uint64_t seen = __ballot(row >= 0 && ((tok[u] >> q) & 1u));
            if ((lane & 31) == 0 && idx / kTile < kChunkTiles) sm.tmask[idx / kTile][q] = (uint32_t)(seen >> (lane & 32));
          }
        }
      }
      // Q loads and the translation loads complete here, before the ring starts:
      // a wait placed lazily later would also wait for the tile loads in flight.
      wait_vmcnt<0>();
      block_sync();

      // -- producer: issue the loads of chunk tile jj into ring buffer jj % NBUF
      auto issue = [&](int jj) {
        int k0, len;
        bool cmp;
        st.tile(cbase + jj, k0, len, cmp);
        const int buf = jj % NBUF;
        const int64_t *er = &sm.erow[jj * kTile];
        if (!FP8 || !cmp) {
          const uint8_t *kb = cmp ? p.k_cmp : p.k_raw;
          const uint8_t *vb = cmp ? p.v_cmp : p.v_raw;
          int64_t off[C::kKVInstr / 2];
#pragma unroll
          for (int n = 0; n < C::kKVInstr / 2; ++n) {   // row lookups first; K and V share rows
            const int lin = n * 1024 + lane * 16;
            const int r = lin / C::kRowB;
            const int c = ((lin % C::kRowB) / 16) ^ (r & (C::kChunks - 1));
            const int64_t e = er[r];
            off[n] = e >= 0 ? e * C::kRowB + c * 16 : -1;
          }
#pragma unroll
          for (int n = 0; n < C::kKVInstr / 2; ++n)
            dma16(off[n] >= 0 ? kb + off[n] : kZeroRow + (lane & 15) * 16, &sm.kv[buf][0][n * 1024]);
#pragma unroll
          for (int n = 0; n < C::kKVInstr / 2; ++n)
            dma16(off[n] >= 0 ? vb + off[n] : kZeroRow + (lane & 15) * 16, &sm.kv[buf][1][n * 1024]);
        } else {
          int64_t off[C::kF8Instr / 2];
#pragma unroll
          for (int n = 0; n < C::kF8Instr / 2; ++n) {
            const int lin = n * 1024 + lane * 16;
            const int r = lin / D;
            const int c = (lin % D) / 16;
            const int64_t e = er[r];
            off[n] = e >= 0 ? e * D + c * 16 : -1;
          }
          const int64_t es = er[lane & 31];
#pragma unroll
          for (int n = 0; n < C::kF8Instr / 2; ++n)
            dma16(off[n] >= 0 ? p.k_cmp + off[n] : kZeroRow + (lane & 15) * 16, &sm.stage[FP8 ? buf : 0][0][n * 1024]);
#pragma unroll
          for (int n = 0; n < C::kF8Instr / 2; ++n)
            dma16(off[n] >= 0 ? p.v_cmp + off[n] : kZeroRow + (lane & 15) * 16, &sm.stage[FP8 ? buf : 0][1][n * 1024]);
          // the per-token scales: lanes 0-31 k, lanes 32-63 v
          const float *sc = hi ? p.v_cmp_scale : p.k_cmp_scale;
          dma4(es >= 0 ? (const void *)(sc + es) : (const void *)kZeroRow, &sm.scl[FP8 ? buf : 0][0]);
#pragma unroll
          for (int n = C::kF8Instr + 1; n < C::kKVInstr; ++n)
            dma4(kZeroRow + lane * 4, &sm.dummy[0]);   // keeps the per-tile count uniform
        }
      };

      if (producer) {
        const int pre = min(NBUF - 1, ct);
        for (int jj = 0; jj < pre; ++jj) issue(jj);
      }

      for (int jj = 0; jj < ct; ++jj) {
        // the producer waits for tile jj; the barrier then hands it to the compute
        // waves and tells the producer that tile jj-1's buffer is free
        if (producer) wait_tiles<C::kOps, NBUF - 2>(min(NBUF - 2, ct - 1 - jj));
        block_sync();
        if (producer && jj + NBUF - 1 < ct) issue(jj + NBUF - 1);

        int k0, len;
        bool cmp;
        st.tile(cbase + jj, k0, len, cmp);
        const int buf = jj % NBUF;

        if (FP8 && cmp) {
          // widen the staged e4m3 rows to bf16 (exact) into the swizzled tile
          constexpr int kPieces = kTile * D / 8;   // 8-byte pieces per tile
          for (int idx = producer ? 2 * kPieces : tid; idx < 2 * kPieces; idx += C::kThreads) {
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

        const uint32_t tm = sm.tmask[jj][qt];
        if (wave_ok && tm != 0u) {
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
          // online softmax.  Lane rows: 8*(i/4) + 4*hi + i%4.  The max is taken
          // on the raw scores (the scale c = scale*log2 e is positive), and
          // p = exp2(s*c - m) is one FMA and one exp per score.
          float sc[16];
#pragma unroll
          for (int i = 0; i < 16; ++i) sc[i] = s[i];
          if (FP8 && cmp) {
#pragma unroll
            for (int q4 = 0; q4 < 4; ++q4) {
              const float4 kk4 = *(const float4 *)(&sm.scl[FP8 ? buf : 0][8 * q4 + 4 * hi]);
              sc[4 * q4 + 0] *= kk4.x;
              sc[4 * q4 + 1] *= kk4.y;
              sc[4 * q4 + 2] *= kk4.z;
              sc[4 * q4 + 3] *= kk4.w;
            }
          }
          if (tm != 0xFFFFFFFFu) {
#pragma unroll
            for (int i = 0; i < 16; ++i) {
              const int r = 8 * (i >> 2) + 4 * hi + (i & 3);
              sc[i] = ((tm >> r) & 1u) ? sc[i] : -INFINITY;
            }
          }
          float smax = fmaxf(fmaxf(fmaxf(sc[0], sc[1]), fmaxf(sc[2], sc[3])),
                             fmaxf(fmaxf(sc[4], sc[5]), fmaxf(sc[6], sc[7])));
          smax = fmaxf(smax, fmaxf(fmaxf(fmaxf(sc[8], sc[9]), fmaxf(sc[10], sc[11])),
                                   fmaxf(fmaxf(sc[12], sc[13]), fmaxf(sc[14], sc[15]))));
          smax = fmaxf(smax, __shfl_xor(smax, 32));
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
              const float4 vv = *(const float4 *)(&sm.scl[FP8 ? buf : 0][32 + 8 * q4 + 4 * hi]);
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
              const i16x8 cat = {part[0][0], part[0][1], part[0][2], part[0][3],
                                 part[1][0], part[1][1], part[1][2], part[1][3]};
              acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, cat), pb[k2],
                                                                acc[db], 0, 0, 0);
            }
          }
        }
      }
    }
  }
  if (producer) return;

  // ---- epilogue
  const float lt = l + __shfl_xor(l, 32);
  const float inv = lt > 0.f ? 1.f / lt : 0.f;
  const float lse2 = (m == -INFINITY || !(lt > 0.f)) ? -INFINITY : m + __builtin_amdgcn_logf(lt);
  const float lse = lse2 == -INFINITY ? -INFINITY : lse2 * kLn2;
  if (!head_ok) return;
  if (S == 1) {
    uint16_t *orow = p.o + ((int64_t)qi * p.hq + h) * D;
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
    if (hi == 0 && p.lse) p.lse[(int64_t)qi * p.hq + h] = lse;
    return;
  }

  // split: write the sink-free partial; the merge kernel adds the sink
  const int64_t prow = ((int64_t)split * p.num_queries + qi) * p.hq + h;
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

template <int D, int NH, int NQ, bool FP8>
hipError_t launch_t(const Params &p, hipStream_t stream) {
  constexpr int NBUF = 4;   // 3 tiles in flight behind the one being computed
  const unsigned grid = (unsigned)p.jobs_per_xcd * 8u;
  hipLaunchKernelGGL((attn_fwd_kernel<D, NH, NQ, FP8, NBUF>), dim3(grid), dim3((NH * NQ + 1) * 64), 0, stream, p);
  return hipGetLastError();
}

template <int D, bool FP8>
hipError_t launch_d(const Params &p, hipStream_t stream) {
  const int heads = p.group < p.heads_per_block ? p.group : p.heads_per_block;
  const int nh = heads <= 32 ? 1 : (heads <= 64 ? 2 : 4);
  const int nq = p.queries_per_group;
  switch (nh * 16 + nq) {
    case 1 * 16 + 1: return launch_t<D, 1, 1, FP8>(p, stream);
    case 2 * 16 + 1: return launch_t<D, 2, 1, FP8>(p, stream);
    case 4 * 16 + 1: return launch_t<D, 4, 1, FP8>(p, stream);
    case 1 * 16 + 2: return launch_t<D, 1, 2, FP8>(p, stream);
    case 2 * 16 + 2: return launch_t<D, 2, 2, FP8>(p, stream);
    case 1 * 16 + 4: return launch_t<D, 1, 4, FP8>(p, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t launch_attention(const Params &p, hipStream_t stream) {
  if (p.num_queries == 0) return hipSuccess;
  if (p.head_dim == 64) return p.cmp_fp8 ? launch_d<64, true>(p, stream) : launch_d<64, false>(p, stream);
  return p.cmp_fp8 ? launch_d<128, true>(p, stream) : launch_d<128, false>(p, stream);
}

}  // namespace spa
