// Device helpers shared by the decode-attention kernels (gfx950 / CDNA4,
// wave64). Lane-exchange semantics used below, as measured on gfx950:
//   permlane16_swap(a, b) -> (A, B) with rows of 16 lanes
//       A = [a.r0, b.r0, a.r2, b.r2],  B = [a.r1, b.r1, a.r3, b.r3]
//   permlane32_swap(a, b) -> (A, B) with halves of 32 lanes
//       A = [a.lo, b.lo],  B = [a.hi, b.hi]
//   DPP row_ror:8, row_half_mirror and quad_perm act inside a 16-lane row.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace da {

constexpr int kPage = 16;       // tokens per page
constexpr int kWave = 64;       // lanes per wavefront
constexpr float kLog2e = 1.4426950408889634f;

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef short s16x4 __attribute__((ext_vector_type(4)));

// ---------------------------------------------------------------- lane moves
template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false));
}
constexpr int kDppRowRor8 = 0x128;       // lane i <- lane i^8 (inside a row)
constexpr int kDppRowHalfMirror = 0x141; // lane i <- lane i^7 (inside a row)
constexpr int kDppQuadXor2 = 0x4E;       // quad_perm [2,3,0,1]: lane i <- i^2
constexpr int kDppQuadXor1 = 0xB1;       // quad_perm [1,0,3,2]: lane i <- i^1

// Butterfly over the 16 lanes of a row with xor partners 8, 7, 2, 1 (a basis
// of the 4 lane bits). Each step adds a value and its partner's, which is
// symmetric, so every lane of the row ends with a bitwise-identical total.
__device__ __forceinline__ float row_sum16(float x) {
  x += dpp<kDppRowRor8>(x);
  x += dpp<kDppRowHalfMirror>(x);
  x += dpp<kDppQuadXor2>(x);
  x += dpp<kDppQuadXor1>(x);
  return x;
}
__device__ __forceinline__ float row_max16(float x) {
  x = fmaxf(x, dpp<kDppRowRor8>(x));
  x = fmaxf(x, dpp<kDppRowHalfMirror>(x));
  x = fmaxf(x, dpp<kDppQuadXor2>(x));
  x = fmaxf(x, dpp<kDppQuadXor1>(x));
  return x;
}

struct f2 { float a, b; };

__device__ __forceinline__ f2 swap16(float a, float b) {
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(a), __float_as_uint(b), false, false);
  return {__uint_as_float(r[0]), __uint_as_float(r[1])};
}
__device__ __forceinline__ f2 swap32(float a, float b) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(a), __float_as_uint(b), false, false);
  return {__uint_as_float(r[0]), __uint_as_float(r[1])};
}
// Value of lane i^32 (the other half of the wave).
__device__ __forceinline__ float xor32(float x) {
  f2 r = swap32(x, x);
  return (threadIdx.x & 32) ? r.a : r.b;
}
// Value of lane i^16 (the neighbouring row).
__device__ __forceinline__ float xor16(float x) {
  f2 r = swap16(x, x);
  return (threadIdx.x & 16) ? r.a : r.b;
}

// ---------------------------------------------------------------- numerics
__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

// bf16 bit patterns packed two per dword -> fp32 (exact).
__device__ __forceinline__ float bf16_lo(uint32_t u) { return __uint_as_float(u << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t u) { return __uint_as_float(u & 0xFFFF0000u); }

__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float acc) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a), __builtin_bit_cast(bf16x2, b),
                                         acc, false);
}

// sigmoid(x) = 1 / (1 + exp(-x)); exp(-x) = inf for very negative x gives 0.
__device__ __forceinline__ float sigmoidf(float x) { return 1.f / (1.f + expf(-x)); }

// ---------------------------------------------------------------- memory
__device__ __forceinline__ uint4 ld16(const void* p) { return *reinterpret_cast<const uint4*>(p); }

// 16-byte load with the non-temporal hint (global_load_dwordx4 ... nt): for
// the KV page stream, which is read once per call. Measured on gfx950, random
// 16 KB pages stream at ~6.97 TB/s with it against ~6.15 TB/s without.
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

// 16 KB of zeros in device memory. Software pipelines that issue the same
// loads on every pass point the slots they will not use (past the end of a
// walk, pairs without a page) here: the lines stay in L2, where re-reading
// the last real page with the non-temporal hint would go to HBM again.
// A pointer select, not a branch, so the compiler's load counting is kept.
static __device__ uint4 g_zero_page[1024];

__device__ __forceinline__ uint4 ld16_stream(const void* p) {
  const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}

// s_waitcnt vmcnt(0) (expcnt and lgkmcnt left unconstrained). Used at the end
// of rarely taken branches that issue vector loads, so that the loads do not
// stay pending across the join: otherwise the wait the compiler places before
// the next use of any prefetched register becomes vmcnt(0) on every pass.
__device__ __forceinline__ void wait_vmem_all() { __builtin_amdgcn_s_waitcnt(0x0F70); }

}  // namespace da
