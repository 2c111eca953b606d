// Top-k selection of compressed groups from per-token scores, for gfx950.
//
// On the pages, the step before the attention core scores every complete
// compressed group of a token, selects index_topk of them with a radix
// top-k and packs the selected ids into paged offsets (ATOM PR "test: add
// block-level DeepSeek-V4 attention test", sections "What this test
// actually drives" and "Validation").  This kernel is the selection; the
// offsets are the canonical rows attn_build_gather exports.
//
// Order (the pages fix none): descending score, ties by ascending id, -0.0
// below +0.0, a NaN score below every number.  Each float32 score maps to a
// uint32 key whose unsigned order is this order (non-negative: top bit set;
// negative: all bits inverted; NaN: 0), so the selection is unique.  The ids
// are written in this order, or the same selection in ascending id order.
//
// One workgroup of four waves per row.  A row of up to 256 * R entries
// (R = 4 or 16, chosen from the row stride) keeps its keys in registers,
// entry i * 256 + t in thread t's i-th key, loaded before the row's count is
// known.  A radix select over the key, 8 bits per pass from the top, finds
// the k-th largest key T and how many of the entries equal to T are taken:
// each pass adds the entries still matching T's known high bits into that
// pass's own histogram (all four cleared at the start, so a pass needs one
// barrier), and every wave reads the whole histogram and finds the digit
// where the running count from the top reaches the number still wanted with
// a DPP prefix sum, so no wave waits for another's answer.  The passes stop
// early once every entry under the known prefix is taken.  The entries
// above T and the first ones equal to T are then ranked in ascending id
// order by ballots and one exchange of per-wave counts.  In id order each
// selected id is then written at its rank directly.  In score order the selected
// (key, id) pairs are ordered as (key << 32 | ~id), descending: up to 512,
// in a launch with at most as many rows as compute units, by one bitonic
// network over the workgroup (lanes exchange by DPP and swizzles, waves
// through LDS), the shortest chain; in a larger launch by a bitonic network
// within each wave over runs of 128 in registers, then each pair's position
// from binary searches of the other runs, the least work; more than 512 by
// one bitonic network over the workgroup.  Longer rows run the same select with
// histograms of the whole workgroup over the scores in memory.

#include <hip/hip_runtime.h>

#include <cstdint>

#include "spa_internal.h"
#include "spa_kernel_util.h"

namespace spa {
namespace {

constexpr int kTkThreads = 256;

__device__ __forceinline__ uint32_t score_key(uint32_t bits) {
  const bool nan = (bits & 0x7F800000u) == 0x7F800000u && (bits & 0x007FFFFFu) != 0u;
  if (nan) return 0u;
  return (bits & 0x80000000u) ? ~bits : (bits | 0x80000000u);
}


// The sort key of entry j with key u: (u << 32 | ~j) orders by descending
// score, ties by ascending id; (~j << 32 | ~j) by ascending id alone.  Both
// are nonzero, as ~j has its top bit set.
template <bool BY_ID>
__device__ __forceinline__ unsigned long long pair_code(uint32_t u, int32_t j) {
  const uint32_t nj = ~(uint32_t)j;
  return ((unsigned long long)(BY_ID ? nj : u) << 32) | nj;
}

__device__ __forceinline__ unsigned long long shfl_xor_u64(unsigned long long v, int m) {
  const uint32_t lo = (uint32_t)__shfl_xor((int)(uint32_t)v, m);
  const uint32_t hi = (uint32_t)__shfl_xor((int)(uint32_t)(v >> 32), m);
  return ((unsigned long long)hi << 32) | lo;
}

// Sorts sel[0, kk) descending as a bitonic network over P = 256 * C entries
// held in registers (entry c * 256 + tid in v[c]; padding 0 sorts last, a
// selected pair is never 0 since ~id has its top bit set), then writes the
// ids of the first k positions (-1 past kk).  A stride below 64 pairs lanes
// of one wave (shuffles), a stride of 256 or more pairs registers of one
// thread, and only strides 64 and 128 exchange through LDS.  sel must be
// readable by every thread on entry.
template <int C>
__device__ __forceinline__ void sort_write(unsigned long long *sel, int32_t kk, int32_t k, int32_t *out) {
  const int tid = threadIdx.x;
  constexpr int P = kTkThreads * C;
  unsigned long long v[C];
#pragma unroll
  for (int c = 0; c < C; ++c) {
    const int i = c * kTkThreads + tid;
    v[c] = i < kk ? sel[i] : 0ull;
  }
  __syncthreads();                           // sel is the exchange buffer from here
#pragma unroll
  for (int size = 2; size <= P; size <<= 1) {
#pragma unroll
    for (int s = size >> 1; s > 0; s >>= 1) {
      if (s >= kTkThreads) {
#pragma unroll
        for (int c = 0; c < C; ++c) {
          const int cp = c ^ (s / kTkThreads);
          if (cp > c) {
            const bool desc = ((c * kTkThreads + tid) & size) == 0;
            const unsigned long long a = v[c], b = v[cp];
            if (desc ? (a < b) : (a > b)) {
              v[c] = b;
              v[cp] = a;
            }
          }
        }
      } else {
        unsigned long long w[C];
        if (s >= 64) {
#pragma unroll
          for (int c = 0; c < C; ++c) sel[c * kTkThreads + tid] = v[c];
          __syncthreads();
#pragma unroll
          for (int c = 0; c < C; ++c) w[c] = sel[c * kTkThreads + (tid ^ s)];
          __syncthreads();
        } else {
#pragma unroll
          for (int c = 0; c < C; ++c) w[c] = shfl_xor_u64(v[c], s);
        }
#pragma unroll
        for (int c = 0; c < C; ++c) {
          const bool desc = ((c * kTkThreads + tid) & size) == 0;
          const bool lower = (tid & s) == 0;
          const unsigned long long a = v[c], b = w[c];
          v[c] = (desc == lower) ? (a > b ? a : b) : (a < b ? a : b);
        }
      }
    }
  }
#pragma unroll
  for (int c = 0; c < C; ++c) {
    const int i = c * kTkThreads + tid;
    if (i < k) out[i] = i < kk ? (int32_t)(~(uint32_t)(v[c] & 0xFFFFFFFFull)) : -1;
  }
  for (int32_t i = P + tid; i < k; i += kTkThreads) out[i] = -1;
}

// Inclusive prefix sum over the 64 lanes of a wave (DPP row shifts, then
// the row broadcasts of lanes 15 and 31).
__device__ __forceinline__ uint32_t wave_incl_scan(uint32_t x) {
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x111, 0xf, 0xf, false);  // row_shr:1
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x112, 0xf, 0xf, false);  // row_shr:2
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x114, 0xf, 0xf, false);  // row_shr:4
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x118, 0xf, 0xf, false);  // row_shr:8
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x142, 0xa, 0xf, false);  // row_bcast:15 to rows 1, 3
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x143, 0xc, 0xf, false);  // row_bcast:31 to rows 2, 3
  return x;
}

__device__ __forceinline__ uint32_t lanes_below(unsigned long long m) {
  return __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
}

struct TopkSmem {
  alignas(16) uint32_t hist[4][256];         // one histogram per radix pass
  unsigned long long sel[kTopkMax];          // the selected (key, ~id) pairs
  uint32_t cnt[2][64];                       // per (key register, wave): entries above T, equal to T
  int32_t wsum[kTkThreads / 64];
  int32_t sh_digit, sh_krem, sh_done, sh_ngt;
};

// Finds, from a pass's histogram (highest digit first), the digit where the
// count of entries above it first reaches krem; every wave computes it
// alone.  Lane l holds digits 255 - 4l ... 252 - 4l.
__device__ __forceinline__ void find_digit(const uint32_t *h, int32_t &krem, uint32_t &digit, bool &done) {
  const int lane = threadIdx.x & 63;
  const uint4 b = *reinterpret_cast<const uint4 *>(h + 252 - 4 * lane);
  const uint32_t hv[4] = {b.w, b.z, b.y, b.x};
  const uint32_t s = hv[0] + hv[1] + hv[2] + hv[3];
  uint32_t c = wave_incl_scan(s) - s;
  const uint32_t kr = (uint32_t)krem;
  int32_t at = -1;
  uint32_t rem = 0, full = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    if (at < 0 && c < kr && c + hv[i] >= kr) {
      at = i;
      rem = kr - c;
      full = rem == hv[i] ? 1u : 0u;
    }
    c += hv[i];
  }
  const unsigned long long m = __ballot(at >= 0);
  const int src = __builtin_ctzll(m);
  digit = (uint32_t)__builtin_amdgcn_readlane((int)(255 - 4 * lane - at), src);
  krem = __builtin_amdgcn_readlane((int)rem, src);
  done = __builtin_amdgcn_readlane((int)full, src) != 0;
}

// Radix select and collect over the keys in registers (entry i * 256 + tid
// in u[i]).  By score: writes the kk selected pairs to sm.sel, the entries
// above T in ascending id order, then those equal to T.  By id: writes the
// ids straight to out, entry j at the number of selected entries below it
// (those above T below j, plus those equal to T below j up to the number
// taken), and -1 past kk.
template <int R, bool BY_ID>
__device__ __forceinline__ void select_regs(const uint32_t (&u)[R], int32_t n, int32_t kk, int32_t k, TopkSmem &sm,
                                            int32_t *out) {
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  uint32_t prefix = 0u, mask = 0u;
  int32_t krem = kk;
#pragma unroll
  for (int pass = 0; pass < 4; ++pass) {
    const int shift = 24 - 8 * pass;
#pragma unroll
    for (int i = 0; i < R; ++i) {
      if (i * kTkThreads + tid < n && (u[i] & mask) == prefix) atomicAdd(&sm.hist[pass][(u[i] >> shift) & 255u], 1u);
    }
    __syncthreads();
    uint32_t digit;
    bool done;
    find_digit(sm.hist[pass], krem, digit, done);
    prefix |= digit << shift;
    mask |= 0xFFu << shift;
    if (done) break;
  }
  // ranks in ascending id order: entry i * 256 + 64 * wave + lane
  unsigned long long bg[R], be[R];
#pragma unroll
  for (int i = 0; i < R; ++i) {
    const bool valid = i * kTkThreads + tid < n;
    bg[i] = __ballot(valid && (u[i] & mask) > prefix);
    be[i] = __ballot(valid && (u[i] & mask) == prefix);
    if (lane == 0) {
      sm.cnt[0][i * 4 + wave] = (uint32_t)__builtin_popcountll(bg[i]);
      sm.cnt[1][i * 4 + wave] = (uint32_t)__builtin_popcountll(be[i]);
    }
  }
  __syncthreads();
  const uint32_t cg = lane < 4 * R ? sm.cnt[0][lane] : 0u;
  const uint32_t ce = lane < 4 * R ? sm.cnt[1][lane] : 0u;
  const uint32_t og = wave_incl_scan(cg) - cg, oe = wave_incl_scan(ce) - ce;
  const int32_t ngt = kk - krem;
#pragma unroll
  for (int i = 0; i < R; ++i) {
    const int j = i * kTkThreads + tid;
    const uint32_t bgi = (uint32_t)__builtin_amdgcn_readlane((int)og, i * 4 + wave);
    const uint32_t bei = (uint32_t)__builtin_amdgcn_readlane((int)oe, i * 4 + wave);
    const int32_t gpre = (int32_t)(bgi + lanes_below(bg[i]));
    const int32_t epre = (int32_t)(bei + lanes_below(be[i]));
    const bool is_gt = (bg[i] >> lane) & 1ull, is_eq = (be[i] >> lane) & 1ull;
    if constexpr (BY_ID) {
      if (is_gt || (is_eq && epre < krem)) out[gpre + (epre < krem ? epre : krem)] = j;
    } else {
      const unsigned long long comp = pair_code<false>(u[i], j);
      if (is_gt) sm.sel[gpre] = comp;
      if (is_eq && epre < krem) sm.sel[ngt + epre] = comp;
    }
  }
  if constexpr (BY_ID) {
    for (int32_t i = kk + tid; i < k; i += kTkThreads) out[i] = -1;
  }
}

// The same select for rows longer than the registers hold: histograms and
// ranks of the whole workgroup, the keys re-read from the scores each pass.
template <bool BY_ID>
__device__ void select_global(const uint32_t *src, int32_t n, int32_t kk, TopkSmem &sm) {
  const int tid = threadIdx.x;
  uint32_t prefix = 0u, mask = 0u;
  int32_t krem = kk;
  for (int pass = 0; pass < 4; ++pass) {
    const int shift = 24 - 8 * pass;
    for (int32_t j = tid; j < n; j += kTkThreads) {
      const uint32_t u = score_key(src[j]);
      if ((u & mask) == prefix) atomicAdd(&sm.hist[pass][(u >> shift) & 255u], 1u);
    }
    __syncthreads();
    // thread t owns digit 255 - t: the entries above it are the exclusive
    // prefix sum in this order
    const int32_t h = (int32_t)sm.hist[pass][255 - tid];
    int32_t tot;
    const int32_t above = block_excl_scan<kTkThreads>(h, tot, sm.wsum);
    if (above < krem && above + h >= krem) {
      sm.sh_digit = 255 - tid;
      sm.sh_krem = krem - above;
      sm.sh_done = (krem - above == h) ? 1 : 0;
    }
    __syncthreads();
    prefix |= (uint32_t)sm.sh_digit << shift;
    mask |= 0xFFu << shift;
    krem = sm.sh_krem;
    const bool done = sm.sh_done != 0;
    __syncthreads();                         // sh_* are rewritten in the next pass
    if (done) break;
  }
  // every entry above the prefix, and the first krem entries matching it
  // in ascending id order
  const int32_t ngt = kk - krem;
  if (tid == 0) sm.sh_ngt = 0;
  __syncthreads();
  int32_t eq_base = 0;
  for (int32_t c0 = 0; c0 < n; c0 += kTkThreads) {
    const int32_t j = c0 + tid;
    const uint32_t u = j < n ? score_key(src[j]) : 0u;
    const bool gt = j < n && (u & mask) > prefix;
    const bool eq = j < n && (u & mask) == prefix;
    int32_t tot;
    const int32_t r = eq_base + block_excl_scan<kTkThreads>(eq ? 1 : 0, tot, sm.wsum);
    const unsigned long long comp = pair_code<BY_ID>(u, j);
    if (gt) {
      const int32_t slot = atomicAdd(&sm.sh_ngt, 1);
      if (slot < ngt) sm.sel[slot] = comp;
    }
    if (eq && r < krem) sm.sel[ngt + r] = comp;
    eq_base += tot;
  }
}

// The value lane (lane ^ S) holds, for S < 64: DPP within rows of 16
// lanes for S 1, 2, 4 and 8, a swizzle within 32 lanes for 16, a permute
// for 32.
template <int S>
__device__ __forceinline__ uint32_t xor_lane(uint32_t x) {
  if constexpr (S == 1) {
    return (uint32_t)__builtin_amdgcn_mov_dpp((int)x, 0xB1, 0xf, 0xf, false);        // quad_perm [1,0,3,2]
  } else if constexpr (S == 2) {
    return (uint32_t)__builtin_amdgcn_mov_dpp((int)x, 0x4E, 0xf, 0xf, false);        // quad_perm [2,3,0,1]
  } else if constexpr (S == 4) {
    const int t = __builtin_amdgcn_update_dpp(0, (int)x, 0x104, 0xf, 0x5, false);    // row_shl:4 into lanes 0-3, 8-11
    return (uint32_t)__builtin_amdgcn_update_dpp(t, (int)x, 0x114, 0xf, 0xa, false);  // row_shr:4 into lanes 4-7, 12-15
  } else if constexpr (S == 8) {
    return (uint32_t)__builtin_amdgcn_mov_dpp((int)x, 0x128, 0xf, 0xf, false);       // row_ror:8
  } else if constexpr (S == 16) {
    return (uint32_t)__builtin_amdgcn_ds_swizzle((int)x, 0x401F);                    // xor 16 within 32 lanes
  } else {
    return (uint32_t)__shfl_xor((int)x, 32);
  }
}

// Lanes whose bit S is clear.
constexpr uint64_t lanes_bit_clear(int S) {
  uint64_t m = 0;
  for (int l = 0; l < 64; ++l)
    if ((l & S) == 0) m |= 1ull << l;
  return m;
}

// One compare-exchange step of the bitonic network over the 128 entries of
// a wave, entry 64 * r + lane in v[r]; a block of SIZE entries is ordered
// descending where (entry & SIZE) == 0, so the last step leaves the wave's
// entries descending.
template <int SIZE, int S>
__device__ __forceinline__ void wave_bitonic_step(unsigned long long (&v)[2]) {
  if constexpr (S == 64) {
    const unsigned long long a = v[0], b = v[1];
    const bool gt = a > b;
    v[0] = gt ? a : b;
    v[1] = gt ? b : a;
  } else {
#pragma unroll
    for (int r = 0; r < 2; ++r) {
      const uint64_t desc = SIZE <= 32 ? lanes_bit_clear(SIZE) : (SIZE == 64 && r == 1) ? 0ull : ~0ull;
      const uint64_t take_max = ~(lanes_bit_clear(S) ^ desc);
      const unsigned long long a = v[r];
      const unsigned long long b = ((unsigned long long)xor_lane<S>((uint32_t)(a >> 32)) << 32) |
                                   xor_lane<S>((uint32_t)a);
      const bool keep = (a > b) == __builtin_amdgcn_inverse_ballot_w64(take_max);
      v[r] = keep ? a : b;
    }
  }
  if constexpr (S > 1) wave_bitonic_step<SIZE, S / 2>(v);
}

template <int SIZE>
__device__ __forceinline__ void wave_bitonic_sort(unsigned long long (&v)[2]) {
  wave_bitonic_step<SIZE, SIZE / 2>(v);
  if constexpr (SIZE < 128) wave_bitonic_sort<SIZE * 2>(v);
}

// How many entries of a descending run of 128 exceed x.
__device__ __forceinline__ int32_t count_above(const unsigned long long *run, unsigned long long x) {
  int32_t c = 0;
#pragma unroll
  for (int step = 64; step >= 1; step >>= 1)
    if (run[c + step - 1] > x) c += step;
  if (c == 127 && run[127] > x) c = 128;
  return c;
}

// Orders up to 512 selected pairs (sel[0, kk)) and writes the ids of the
// first k positions (-1 past kk), with the least work (for launches with more
// rows than compute units): wave w sorts entries [128w, 128w + 128) in
// registers, and after one barrier each entry's position is its place in
// its own run plus the entries above it in the other runs, found by binary
// search; the id is written there directly.
__device__ __forceinline__ void rank_write_runs(unsigned long long *sel, int32_t kk, int32_t k, int32_t *out) {
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int32_t runs = (kk + 127) >> 7;
  unsigned long long v[2];
  if (wave < runs) {
#pragma unroll
    for (int r = 0; r < 2; ++r) {
      const int32_t i = 128 * wave + 64 * r + lane;
      v[r] = i < kk ? sel[i] : 0ull;
    }
    wave_bitonic_sort<2>(v);
#pragma unroll
    for (int r = 0; r < 2; ++r) sel[128 * wave + 64 * r + lane] = v[r];
  }
  __syncthreads();
  if (wave < runs) {
#pragma unroll
    for (int r = 0; r < 2; ++r) {
      const unsigned long long x = v[r];
      int32_t pos = 64 * r + lane;
      for (int c = 0; c < 4; ++c)
        if (c < runs && c != wave) pos += count_above(sel + 128 * c, x);
      if (x != 0ull) out[pos] = (int32_t)(~(uint32_t)(x & 0xFFFFFFFFull));
    }
  }
  for (int32_t i = kk + tid; i < k; i += kTkThreads) out[i] = -1;
}

// One compare-exchange step (block size SIZE, stride S) of the bitonic
// network over the 512 entries of a workgroup: entry i = 128 w + 64 r + lane
// is v[r] of wave w's lane.  A block of SIZE entries is ordered descending
// where (i & SIZE) == 0, so the last step leaves all 512 descending.  Strides
// below 64 pair lanes of a wave, 64 pairs the two registers of a lane, and
// 128 and 256 pair waves through LDS (buf: 512 entries).
template <int SIZE, int S>
__device__ __forceinline__ void bitonic512_step(unsigned long long (&v)[2], int wave, unsigned long long *buf) {
  const int lane = threadIdx.x & 63;
  if constexpr (S >= 128) {
    // pairs of waves: wave w's entries meet wave w ^ (S / 128)'s
#pragma unroll
    for (int r = 0; r < 2; ++r) buf[128 * wave + 64 * r + lane] = v[r];
    __syncthreads();
    unsigned long long w[2];
#pragma unroll
    for (int r = 0; r < 2; ++r) w[r] = buf[(128 * wave + 64 * r + lane) ^ S];
    __syncthreads();                         // the next exchange rewrites buf
    const bool desc = ((128 * wave) & SIZE) == 0;
    const bool lower = ((128 * wave) & S) == 0;
#pragma unroll
    for (int r = 0; r < 2; ++r) {
      const unsigned long long a = v[r], b = w[r];
      v[r] = (desc == lower) ? (a > b ? a : b) : (a < b ? a : b);
    }
  } else if constexpr (S == 64) {
    // SIZE >= 128: the direction is the wave's
    const bool desc = ((128 * wave) & SIZE) == 0;
    const unsigned long long a = v[0], b = v[1];
    const bool gt = a > b;
    v[0] = (gt == desc) ? a : b;
    v[1] = (gt == desc) ? b : a;
  } else {
#pragma unroll
    for (int r = 0; r < 2; ++r) {
      uint64_t desc;
      if constexpr (SIZE <= 32) desc = lanes_bit_clear(SIZE);
      else desc = (((128 * wave + 64 * r) & SIZE) == 0) ? ~0ull : 0ull;
      const uint64_t take_max = ~(lanes_bit_clear(S) ^ desc);
      const unsigned long long a = v[r];
      const unsigned long long b = ((unsigned long long)xor_lane<S>((uint32_t)(a >> 32)) << 32) |
                                   xor_lane<S>((uint32_t)a);
      const bool keep = (a > b) == __builtin_amdgcn_inverse_ballot_w64(take_max);
      v[r] = keep ? a : b;
    }
  }
  if constexpr (S > 1) bitonic512_step<SIZE, S / 2>(v, wave, buf);
}

template <int SIZE>
__device__ __forceinline__ void bitonic512_sort(unsigned long long (&v)[2], int wave, unsigned long long *buf) {
  bitonic512_step<SIZE, SIZE / 2>(v, wave, buf);
  if constexpr (SIZE < 512) bitonic512_sort<SIZE * 2>(v, wave, buf);
}

// The same, with the shortest chain (for launches with at most as many rows
// as compute units, where each row's latency is the call's): one bitonic
// network over the workgroup's 512 entries, padding 0 (below every selected
// pair, as ~id has its top bit set) sorting last; position i is then entry i.
__device__ __forceinline__ void rank_write_net(unsigned long long *sel, int32_t kk, int32_t k, int32_t *out) {
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  unsigned long long v[2];
#pragma unroll
  for (int r = 0; r < 2; ++r) {
    const int32_t i = 128 * wave + 64 * r + lane;
    v[r] = i < kk ? sel[i] : 0ull;
  }
  __syncthreads();                           // sel is the exchange buffer from here
  bitonic512_sort<2>(v, wave, sel);
#pragma unroll
  for (int r = 0; r < 2; ++r) {
    const int32_t i = 128 * wave + 64 * r + lane;
    if (i < kk) out[i] = (int32_t)(~(uint32_t)(v[r] & 0xFFFFFFFFull));
  }
  for (int32_t i = kk + tid; i < k; i += kTkThreads) out[i] = -1;
}

template <int R, bool BY_ID>
__global__ __launch_bounds__(kTkThreads) void topk_kernel(const float *scores, int64_t ld, const int32_t *n_valid,
                                                        int32_t k, int32_t *ids_out, int32_t *cnt_out,
                                                        int32_t few_rows) {
  __shared__ TopkSmem sm;
  const int tid = threadIdx.x;
  const int64_t row = blockIdx.x;
  const uint32_t *src = reinterpret_cast<const uint32_t *>(scores + row * ld);
  // the keys of the first 256 * R entries (within the row's stride) are
  // loaded before the count arrives
  uint32_t u[R];
#pragma unroll
  for (int i = 0; i < R; ++i) {
    const int32_t j = i * kTkThreads + tid;
    u[i] = j < ld ? src[j] : 0u;
  }
  int32_t n = n_valid[row];
#pragma unroll
  for (int i = 0; i < 4; ++i) sm.hist[i][tid] = 0u;
  n = n < 0 ? 0 : (n > ld ? (int32_t)ld : n);
  const int32_t kk = n < k ? n : k;
  int32_t *out = ids_out + row * (int64_t)k;
#pragma unroll
  for (int i = 0; i < R; ++i) u[i] = score_key(u[i]);

  if (kk < n) {
    __syncthreads();                         // the histograms are clear
    if (n <= R * kTkThreads) {
      select_regs<R, BY_ID>(u, n, kk, k, sm, out);
      if (BY_ID) {                           // the ids are written
        if (tid == 0) cnt_out[row] = kk;
        return;
      }
    } else {
      select_global<BY_ID>(src, n, kk, sm);
    }
  } else if (BY_ID) {
    // every valid entry is taken (n <= k), already in id order
    for (int32_t j = tid; j < k; j += kTkThreads) out[j] = j < n ? j : -1;
    if (tid == 0) cnt_out[row] = kk;
    return;
  } else if (n <= R * kTkThreads) {
    // every valid entry is taken (n <= k)
#pragma unroll
    for (int i = 0; i < R; ++i) {
      const int32_t j = i * kTkThreads + tid;
      if (j < n) sm.sel[j] = pair_code<false>(u[i], j);
    }
  } else {
    for (int32_t j = tid; j < n; j += kTkThreads) sm.sel[j] = pair_code<false>(score_key(src[j]), j);
  }
  __syncthreads();
  // -- sort the kk selected pairs, descending, and write the ids
  if (kk <= 512) {
    if (few_rows) rank_write_net(sm.sel, kk, k, out);
    else rank_write_runs(sm.sel, kk, k, out);
  } else if (kk <= 1024) {
    sort_write<4>(sm.sel, kk, k, out);
  } else {
    sort_write<8>(sm.sel, kk, k, out);
  }
  if (tid == 0) cnt_out[row] = kk;
}

}  // namespace

hipError_t launch_topk(const float *scores, int64_t ld, const int32_t *n_valid, int32_t rows, int32_t k,
                       int32_t *ids_out, int32_t *cnt_out, bool by_id, hipStream_t stream) {
  if (rows == 0) return hipSuccess;
  if (k < 1 || k > kTopkMax) return hipErrorInvalidValue;
  auto kernel = ld <= 4 * kTkThreads ? (by_id ? topk_kernel<4, true> : topk_kernel<4, false>)
                                     : (by_id ? topk_kernel<16, true> : topk_kernel<16, false>);
  // rows that leave compute units idle: the shortest sort chain; more rows:
  // the sort with the least work
  const int32_t cus = device_cu_count();
  const int32_t few_rows = (cus > 0 && rows <= cus) ? 1 : 0;
  hipLaunchKernelGGL(kernel, dim3((unsigned)rows), dim3(kTkThreads), 0, stream, scores, ld, n_valid, k, ids_out,
                     cnt_out, few_rows);
  return hipGetLastError();
}

}  // namespace spa
