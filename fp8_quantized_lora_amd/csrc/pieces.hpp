// A float operand as three E4M3 pieces with one scale per row, for the FP8
// matrix cores (the adapter factors A, B^T and the rank-r products U, V).
//
// Row j of F, elements f[k * cs] for k < K, gets the scale
// s_j = 448 / max_k |f[k]| (1 for an all-zero row), and each element v the
// codes q0 = E4M3(v s_j), q1 = E4M3(v s_j - dec(q0)), q2 = E4M3(v s_j -
// dec(q0) - dec(q1)): dec(q0) + dec(q1) + dec(q2) equals v s_j to within
// about 2^-12 of it (3 significant bits per piece, each piece the rounding of
// what the earlier ones left).  Positions K <= k < Kp get zero codes.
#pragma once
#include "common.hpp"

namespace falq {

__device__ __forceinline__ void piece_codes3(float v, float sc, uint8_t* p, int64_t plane) {
  v *= sc;
  const uint32_t q0 = enc1(v);
  const float r1 = v - dec2(q0, false).x;
  const uint32_t q1 = enc1(r1);
  const float r2 = r1 - dec2(q1, false).x;
  p[0] = (uint8_t)q0;
  p[plane] = (uint8_t)q1;
  p[2 * plane] = (uint8_t)enc1(r2);
}

// One row by one workgroup of NT threads.  Rows of up to NT * HOLD elements
// are read once, all loads of a thread in flight together, and kept in
// registers between the row's amax and its pieces; longer rows are read
// twice.  P receives the pieces at P[k], P[plane + k], P[2 plane + k]; *sp
// the scale.
template <int NT, int HOLD>
__device__ __forceinline__ void piece_row(const float* __restrict__ f, int64_t cs, int64_t K,
                                          int64_t Kp, uint8_t* __restrict__ P, int64_t plane,
                                          float* __restrict__ sp) {
  __shared__ uint32_t red[NT / 64];
  __shared__ float s_sc;
  const int t = threadIdx.x;
  const bool held = K <= (int64_t)NT * HOLD;
  float v[HOLD];
  uint32_t m = 0;
  if (held) {
#pragma unroll
    for (int i = 0; i < HOLD; ++i) {
      const int64_t k = t + (int64_t)i * NT;
      v[i] = k < K ? f[k * cs] : 0.0f;
    }
#pragma unroll
    for (int i = 0; i < HOLD; ++i) {
      const uint32_t a = __float_as_uint(v[i]) & 0x7FFFFFFFu;
      if (a < 0x7F800000u && a > m) m = a;
    }
  } else {
    for (int64_t k = t; k < K; k += NT) {
      const uint32_t a = __float_as_uint(f[k * cs]) & 0x7FFFFFFFu;
      if (a < 0x7F800000u && a > m) m = a;
    }
  }
  m = wave_max_u32(m);
  if ((t & 63) == 0) red[t >> 6] = m;
  __syncthreads();
  if (t == 0) {
    uint32_t mm = red[0];
    for (int w = 1; w < NT / 64; ++w) mm = red[w] > mm ? red[w] : mm;
    const float amax = __uint_as_float(mm);
    float sc = amax == 0.0f ? 1.0f : kE4M3Max / amax;
    if (__builtin_isinf(sc)) sc = 3.402823466e38f;
    s_sc = sc;
    *sp = sc;
  }
  __syncthreads();
  const float sc = s_sc;
  if (held) {
#pragma unroll
    for (int i = 0; i < HOLD; ++i) {
      const int64_t k = t + (int64_t)i * NT;
      if (k < Kp) piece_codes3(v[i], sc, P + k, plane);
    }
    for (int64_t k = t + (int64_t)HOLD * NT; k < Kp; k += NT) P[k] = P[plane + k] = P[2 * plane + k] = 0;
  } else {
    for (int64_t k = t; k < Kp; k += NT) piece_codes3(k < K ? f[k * cs] : 0.0f, sc, P + k, plane);
  }
}

// a row of zero pieces (padding ranks), scale 1
template <int NT>
__device__ __forceinline__ void piece_row_zero(int64_t Kp, uint8_t* __restrict__ P, int64_t plane,
                                               float* __restrict__ sp) {
  for (int64_t k = threadIdx.x; k < Kp; k += NT) P[k] = P[plane + k] = P[2 * plane + k] = 0;
  if (threadIdx.x == 0) *sp = 1.0f;
}

}  // namespace falq
