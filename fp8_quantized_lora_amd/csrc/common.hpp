// Device helpers shared by the gfx950 kernels of the melded FP8 LoRA step.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace falq {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef int v4i __attribute__((ext_vector_type(4)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef int v2i __attribute__((ext_vector_type(2)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));

constexpr float kE4M3Max = 448.0f;
constexpr float kE5M2Max = 57344.0f;      // OCP E5M2: 1.75 * 2^15 (0x7B)
constexpr float kE2M1Max = 6.0f;          // OCP FP4 E2M1: 1.5 * 2^2

// ---------------------------------------------------------------------------
// E4M3 (OCP e4m3fn) conversions on the gfx950 conversion unit.
//
// v_cvt_pk_fp8_f32 rounds to nearest even.  Inputs are clamped to +-448 first
// so that overflow saturates whatever the instruction does past the largest
// finite value; NaN lanes are patched to 0x7F | sign afterwards (fmin/fmax
// would turn NaN into a finite bound).  Signed zero passes through.
// ---------------------------------------------------------------------------
__device__ __forceinline__ float clamp448(float v) {
  return fminf(fmaxf(v, -kE4M3Max), kE4M3Max);
}

__device__ __forceinline__ uint32_t nan_patch(uint32_t codes, float a, float b, float c, float d) {
  if (__builtin_expect(__builtin_isnan(a) | __builtin_isnan(b) | __builtin_isnan(c) |
                       __builtin_isnan(d), 0)) {
    float v[4] = {a, b, c, d};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if (__builtin_isnan(v[i])) {
        uint32_t sgn = (__float_as_uint(v[i]) >> 31) << 7;
        codes = (codes & ~(0xFFu << (8 * i))) | ((0x7Fu | sgn) << (8 * i));
      }
    }
  }
  return codes;
}

// four floats -> four E4M3 codes packed little-endian (a in the low byte)
__device__ __forceinline__ uint32_t enc4(float a, float b, float c, float d) {
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(clamp448(a), clamp448(b), 0, false);
  w = __builtin_amdgcn_cvt_pk_fp8_f32(clamp448(c), clamp448(d), w, true);
  return nan_patch((uint32_t)w, a, b, c, d);
}

// enc4 without the NaN patch, converting over `old` (both halves are
// rewritten; passing a live register saves zeroing one)
__device__ __forceinline__ uint32_t enc4_nonan(float a, float b, float c, float d, uint32_t old) {
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(clamp448(a), clamp448(b), (int)old, false);
  w = __builtin_amdgcn_cvt_pk_fp8_f32(clamp448(c), clamp448(d), w, true);
  return (uint32_t)w;
}

// one float -> one FP4 E2M1 code (0..15): nearest, ties to the even code,
// |v| > 6 and infinities saturate to 6, NaN (every comparison false) gives a
// zero; the sign bit is kept.  The seven midpoints of the magnitudes
// 0, .5, 1, 1.5, 2, 3, 4, 6 are exact: a tie goes to the code with mantissa
// bit 0, hence > at 0.25, 1.25, 2.5, 5 and >= at 0.75, 1.75, 3.5
__device__ __forceinline__ uint32_t enc1_e2m1(float v) {
  const float a = fabsf(v);
  const uint32_t c = (uint32_t)(a > 0.25f) + (uint32_t)(a >= 0.75f) + (uint32_t)(a > 1.25f) +
                     (uint32_t)(a >= 1.75f) + (uint32_t)(a > 2.5f) + (uint32_t)(a >= 3.5f) +
                     (uint32_t)(a > 5.0f);
  return c | ((__float_as_uint(v) >> 31) << 3);
}

// one float -> one E4M3 code
__device__ __forceinline__ uint32_t enc1(float a) {
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(clamp448(a), 0.0f, 0, false);
  uint32_t c = (uint32_t)w & 0xFFu;
  if (__builtin_isnan(a)) c = 0x7Fu | ((__float_as_uint(a) >> 31) << 7);
  return c;
}

// E5M2 casts, the same scheme: v_cvt_pk_bf8_f32 rounds to nearest even; the
// clamp to +-57344 saturates finite overflow and infinities (so no code
// reaches the infinity pattern 0x7C); NaN lanes become 0x7F | sign
__device__ __forceinline__ float clamp_e5(float v) {
  return fminf(fmaxf(v, -kE5M2Max), kE5M2Max);
}

__device__ __forceinline__ uint32_t enc4_e5m2(float a, float b, float c, float d) {
  int w = __builtin_amdgcn_cvt_pk_bf8_f32(clamp_e5(a), clamp_e5(b), 0, false);
  w = __builtin_amdgcn_cvt_pk_bf8_f32(clamp_e5(c), clamp_e5(d), w, true);
  return nan_patch((uint32_t)w, a, b, c, d);
}

__device__ __forceinline__ uint32_t enc1_e5m2(float a) {
  int w = __builtin_amdgcn_cvt_pk_bf8_f32(clamp_e5(a), 0.0f, 0, false);
  uint32_t c = (uint32_t)w & 0xFFu;
  if (__builtin_isnan(a)) c = 0x7Fu | ((__float_as_uint(a) >> 31) << 7);
  return c;
}

// E5M2 bytes 0,1 (hi = false) or 2,3 (hi = true) of a dword -> two floats (exact)
__device__ __forceinline__ float2 dec2_e5m2(uint32_t w, bool hi) {
  typedef float v2f __attribute__((ext_vector_type(2)));
  v2f r = hi ? __builtin_amdgcn_cvt_pk_f32_bf8((int)w, true)
             : __builtin_amdgcn_cvt_pk_f32_bf8((int)w, false);
  return make_float2(r.x, r.y);
}

// E4M3 bytes 0,1 (hi = false) or 2,3 (hi = true) of a dword -> two floats (exact)
__device__ __forceinline__ float2 dec2(uint32_t w, bool hi) {
  typedef float v2f __attribute__((ext_vector_type(2)));
  v2f r = hi ? __builtin_amdgcn_cvt_pk_f32_fp8((int)w, true)
             : __builtin_amdgcn_cvt_pk_f32_fp8((int)w, false);
  return make_float2(r.x, r.y);
}

// ---------------------------------------------------------------------------
// Direct global -> LDS loads (global_load_lds_dwordx4): each lane moves 16
// bytes from its own global address to LDS byte m0 + 16 * lane, without
// passing through VGPRs.  Written as inline asm with no outputs, so the
// compiler tracks nothing: completion is waited for with wait_vmem (vmcnt
// counts these loads), and a workgroup barrier then makes every wave's data
// visible.  The LDS address must be wave-uniform (m0).
// ---------------------------------------------------------------------------
typedef __attribute__((address_space(3))) uint8_t lds_u8;

__device__ __forceinline__ void load16_to_lds(const void* g, uint32_t lds_addr) {
  // "{m0}": the compiler itself places the LDS address in m0 (a register
  // it reserves, so it may not be named as a clobber)
  asm volatile("global_load_lds_dwordx4 %0, off" ::"v"(g), "{m0}"(lds_addr) : "memory");
}
__device__ __forceinline__ uint32_t lds_offset(const void* p) {
  return (uint32_t)(uintptr_t)(const lds_u8*)p;
}
// wait until at most n vector-memory instructions of this wave are in flight
// (n in {0, 2, 4, 5, 8, 9, 10, 16, 24}; other values wait for all)
__device__ __forceinline__ void wait_vmem(int n) {
#define FALQ_WVM(k) \
  case k: __builtin_amdgcn_s_waitcnt(((k) & 0xF) | (((k) >> 4) << 14) | (0x7 << 4) | (0xF << 8)); break;
  switch (n) {
    FALQ_WVM(0) FALQ_WVM(2) FALQ_WVM(4) FALQ_WVM(5) FALQ_WVM(8) FALQ_WVM(9) FALQ_WVM(10)
    FALQ_WVM(16) FALQ_WVM(24)
    default: __builtin_amdgcn_s_waitcnt((0x7 << 4) | (0xF << 8)); break;
  }
#undef FALQ_WVM
}
// workgroup barrier that does not wait for outstanding memory operations
// (__syncthreads would drain vmcnt first and serialise the direct loads)
__device__ __forceinline__ void barrier_no_drain() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// ---------------------------------------------------------------------------
// Wavefront (64 lanes) reductions.
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) {
    uint32_t o = __shfl_xor(v, off, 64);
    v = v > o ? v : o;
  }
  return v;
}

__device__ __forceinline__ int wave_sum_i32(int v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, 64);
  return v;
}

__device__ __forceinline__ float wave_max_f32(float v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v = fmaxf(v, __shfl_xor(v, off, 64));
  return v;
}

}  // namespace falq
