// Device helpers shared by the attention kernels: vector types, direct
// global->LDS loads, wait and barrier primitives, the lane-pair max, a
// workgroup prefix sum and the XOR swizzle of LDS tile rows.  Device code
// only.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

namespace spa {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef short i16x8 __attribute__((ext_vector_type(8)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef int v2i32 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4_t;
typedef __attribute__((address_space(3))) v2i32 lds_v2i32_t;
typedef __attribute__((address_space(3))) const bf16x8 lds_bf16x8_t;

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
// The running max used for the exponentials moves only when a tile's max
// exceeds it by more than kTau (log2 units), so P and the sums stay below
// 2^kTau and the O accumulators are rescaled only on such jumps.  Any
// reference value gives the same softmax; only the rounding differs.
constexpr float kTau = 8.f;

// A kernel argument held in scalar registers.  Without it, a select between
// two argument fields (raw or compressed pool, K or V side) can become one
// vector load from the argument block, and the wait for that load would also
// drain every tile load in flight.
template <typename T>
__device__ __forceinline__ T in_sgpr(T v) {
  asm volatile("" : "+s"(v));
  return v;
}

// Source of the padding loads and of the loads for masked rows.
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
// The same with the LDS destination given as a byte offset (wave-uniform).
__device__ __forceinline__ void dma16_at(const void *src, uint32_t lds) {
  lds = __builtin_amdgcn_readfirstlane(lds);
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

// Workgroup barrier that waits only for this wave's LDS operations.  The
// HIP __syncthreads() adds a workgroup release fence, which on gfx950 also
// waits for every outstanding global load and would drain the LDS ring;
// global->LDS loads are instead completed explicitly with wait_vmcnt<>.
// The "memory" clobber keeps the compiler from moving LDS accesses across it.
__device__ __forceinline__ void block_sync() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// max(v, v of lane ^ 32): v_permlane32_swap exchanges the upper half of its
// first operand with the lower half of its second, so with both holding v
// each lane ends up with its own value in one register and its partner's in
// the other.  (Written as asm: the builtin is folded wrongly when both
// operands are the same value.)
__device__ __forceinline__ float max_lane_pair(float v) {
  float a = v, b = v;
  asm volatile("s_nop 1\n\tv_permlane32_swap_b32 %0, %1" : "+v"(a), "+v"(b));
  return fmaxf(a, b);
}

// Masks the scores of a 32-row tile held in the MFMA accumulator layout
// (lane l holds rows 8*(q/4) + 4*(l/32) + q%4, q = 0..15, of column l%32):
// a row whose bit in the wave-uniform mask tm is clear gets -inf.  The lane
// mask of each score (two bits of tm: one for lanes 0-31, one for 32-63) is
// formed in scalar registers and applied by one v_cndmask (inverse ballot),
// so the compiler still sees the scores' dependence on the MFMA that wrote
// them; a full mask costs nothing.
__device__ __forceinline__ void mask_tile_rows(float (&sc)[16], uint32_t tm) {
  tm = __builtin_amdgcn_readfirstlane(tm);
  if (tm == 0xFFFFFFFFu) return;
#pragma unroll
  for (int q = 0; q < 16; ++q) {
    const int r0 = 8 * (q >> 2) + (q & 3);
    // all ones where the row bit is set: bit r0 (lanes 0-31), bit r0+4 (32-63)
    const uint32_t lo = (uint32_t)((int32_t)(tm << (31 - r0)) >> 31);
    const uint32_t hi = (uint32_t)((int32_t)(tm << (27 - r0)) >> 31);
    const uint64_t m = (uint64_t)lo | ((uint64_t)hi << 32);
    sc[q] = __builtin_amdgcn_inverse_ballot_w64(m) ? sc[q] : -INFINITY;
  }
}

__device__ __forceinline__ uint32_t pack_bf16_hi(float lo, float hi) {
  // exact narrowing for values that are bf16 already (widened e4m3 codes)
  return (__builtin_bit_cast(uint32_t, lo) >> 16) | (__builtin_bit_cast(uint32_t, hi) & 0xFFFF0000u);
}

// Eight e4m3 codes (little-endian in w) widened exactly to bf16, packed two
// per word.  OCP: the scaled conversion with scale 1 (gfx950) turns two codes
// into two bf16 values in one instruction; every OCP e4m3 value is a bf16
// value, so nothing rounds.  FNUZ (bias 8, no infinities, one NaN): code c is
// the OCP value of c halved, except 0x7F / 0xFF (+-240, OCP NaN) and 0x80
// (NaN, OCP -0), fixed by selects on the OCP values widened to fp32 by
// v_cvt_pk_f32_fp8.  Every such value is a bf16 value.
template <bool FNUZ>
__device__ __forceinline__ uint4 widen8_e4m3(uint2 w) {
  if constexpr (!FNUZ) {
    typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
    const bf16x2_t a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)w.x, 1.0f, false);
    const bf16x2_t b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)w.x, 1.0f, true);
    const bf16x2_t c = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)w.y, 1.0f, false);
    const bf16x2_t d = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)w.y, 1.0f, true);
    return make_uint4(__builtin_bit_cast(uint32_t, a), __builtin_bit_cast(uint32_t, b), __builtin_bit_cast(uint32_t, c),
                      __builtin_bit_cast(uint32_t, d));
  } else {
    const f32x2 a0 = __builtin_amdgcn_cvt_pk_f32_fp8((int)w.x, false);
    const f32x2 a1 = __builtin_amdgcn_cvt_pk_f32_fp8((int)w.x, true);
    const f32x2 a2 = __builtin_amdgcn_cvt_pk_f32_fp8((int)w.y, false);
    const f32x2 a3 = __builtin_amdgcn_cvt_pk_f32_fp8((int)w.y, true);
    float f[8] = {a0[0], a0[1], a1[0], a1[1], a2[0], a2[1], a3[0], a3[1]};
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const uint32_t c = ((i < 4 ? w.x : w.y) >> (8 * (i & 3))) & 0xFFu;
      const float s240 = __builtin_bit_cast(float, 0x43700000u | ((c & 0x80u) << 24));   // +-240
      const float h = 0.5f * f[i];
      f[i] = (c & 0x7Fu) == 0x7Fu ? s240 : h;
      f[i] = c == 0x80u ? __builtin_bit_cast(float, 0x7FC00000u) : f[i];
    }
    uint4 o;
    o.x = (__builtin_bit_cast(uint32_t, f[0]) >> 16) | (__builtin_bit_cast(uint32_t, f[1]) & 0xFFFF0000u);
    o.y = (__builtin_bit_cast(uint32_t, f[2]) >> 16) | (__builtin_bit_cast(uint32_t, f[3]) & 0xFFFF0000u);
    o.z = (__builtin_bit_cast(uint32_t, f[4]) >> 16) | (__builtin_bit_cast(uint32_t, f[5]) & 0xFFFF0000u);
    o.w = (__builtin_bit_cast(uint32_t, f[6]) >> 16) | (__builtin_bit_cast(uint32_t, f[7]) & 0xFFFF0000u);
    return o;
  }
}

__device__ __forceinline__ uint4 widen8_e4m3(uint2 w, bool fnuz) {
  return fnuz ? widen8_e4m3<true>(w) : widen8_e4m3<false>(w);
}

__device__ __forceinline__ int round_up(int x, int m) { return (x + m - 1) / m * m; }

__device__ __forceinline__ uint32_t bf16_bits(float x) { return __builtin_bit_cast(uint16_t, (__bf16)x); }

// LDS layout of a tile: row r (2D bytes) holds logical 16-byte chunk c at
// physical chunk c ^ swz(r).  For D 128 (16 chunks) the permutation makes
// both access patterns conflict-free: the K (and Q) reads, where 16 lanes
// read one chunk of 16 consecutive rows, and the V transpose reads, where 16
// lanes read 2 adjacent chunks of 4 consecutive rows.  For D 64 (8 chunks,
// two rows per bank sweep) the K reads are conflict-free.
// Exclusive prefix sum of v over a workgroup of NT threads; `total` gets
// the sum.  wsum holds NT / 64 ints of LDS.  Every thread must call it.
template <int NT>
__device__ __forceinline__ int32_t block_excl_scan(int32_t v, int32_t &total, int32_t *wsum) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int32_t x = v;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int32_t y = __shfl_up(x, d);
    if (lane >= d) x += y;
  }
  if (lane == 63) wsum[wave] = x;
  __syncthreads();
  int32_t before = 0;
  total = 0;
#pragma unroll
  for (int w = 0; w < NT / 64; ++w) {
    const int32_t s = wsum[w];
    if (w < wave) before += s;
    total += s;
  }
  __syncthreads();
  return before + x - v;
}

template <int CH>
__device__ __forceinline__ int swz(int r) {
  if constexpr (CH == 16) return ((r & 7) << 1) | ((r >> 3) & 1);
  else return (r >> 1) & 7;
}

}  // namespace
}  // namespace spa
