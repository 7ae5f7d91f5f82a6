// A float operand F (rows j: ranks; columns k: the contraction index) as
// three E4M3 "pieces" per element for the FP8 matrix cores, with one
// power-of-two scale per row and 32-element block that the matrix core
// applies itself, as the operand's E8M0 block scale of
// v_mfma_scale_f32_16x16x128_f8f6f4 (the adapter factors A and B^T, and the
// rank-r products U = X^ A^T and V = G^ B).
//
// Blocks.  The FP8 kernels hold a 128-wide K step of an operand row with lane
// group g (lanes 16 g .. 16 g + 15) taking K positions 32 g .. 32 g + 31 in
// its eight registers.  The matrix core splits a K step into four scale
// blocks by register half and lane-group pair (lane 16 s + i supplies the
// scale of row i's block s), which in that layout puts position d of the
// step (0 <= d < 128) in block 2 bit4(d) + bit6(d): block s holds
// d = 64 (s & 1) + 16 (s >> 1) + 32 b + i, b in {0, 1}, i < 16.
//
// Encoding.  With m the block's largest finite magnitude, e is the largest
// integer with m 2^e <= 448 (0 for a block of zeros; clamped to
// [-127, 127]), and each element v gets q0 = E4M3(v 2^e),
// q1 = E4M3(v 2^e - dec(q0)), q2 = E4M3(v 2^e - dec(q0) - dec(q1)): each
// piece rounds what the earlier ones left, so the three decode to v 2^e
// within about 2^-12 of it (the subtractions are exact).  The block's scale
// byte is the E8M0 code 127 - e: the matrix core multiplies the products of
// the block by 2^-e.
//
// Layout.  Pieces P[p][j][k] at P + p * plane + j * Kp + k, scale bytes
// E[c][j][s] at E + (c * Rp + j) * 4 + s for K step c: the scale bytes of
// 16 consecutive rows in one step are 64 contiguous bytes.  Rows past R and
// columns past K hold zero codes (scale byte 127).
#pragma once
#include "common.hpp"

namespace falq {

// the block of position d of a 128-wide K step
__host__ __device__ constexpr int piece_block(int d) { return 2 * ((d >> 4) & 1) + ((d >> 6) & 1); }

// e for a block whose largest finite magnitude is m
__device__ __forceinline__ int piece_exp(float m) {
  if (!(m > 0.0f)) return 0;
  // m = f 2^E with 0.5 <= f < 1, and 448 = 0.875 * 2^9
  const int E = __builtin_amdgcn_frexp_expf(m);
  const float f = __builtin_amdgcn_frexp_mantf(m);
  const int e = (f <= 0.875f ? 9 : 8) - E;
  return e < -127 ? -127 : (e > 127 ? 127 : e);
}

// finite magnitude of v as an ordered integer (0 for NaN and infinities)
__device__ __forceinline__ uint32_t finite_mag(float v) {
  const uint32_t a = __float_as_uint(v) & 0x7FFFFFFFu;
  return a < 0x7F800000u ? a : 0u;
}

// four values already multiplied by 2^e -> the three pieces' codes, four per
// dword (value 0 in the low byte)
__device__ __forceinline__ void pieces4(float a, float b, float c, float d, uint32_t& q0,
                                        uint32_t& q1, uint32_t& q2) {
  q0 = enc4(a, b, c, d);
  float2 lo = dec2(q0, false), hi = dec2(q0, true);
  a -= lo.x;
  b -= lo.y;
  c -= hi.x;
  d -= hi.y;
  q1 = enc4(a, b, c, d);
  lo = dec2(q1, false);
  hi = dec2(q1, true);
  q2 = enc4(a - lo.x, b - lo.y, c - hi.x, d - hi.y);
}

// pieces of F [R x K] (element (j, k) at f[j * rs + k * cs]) into P, E as
// laid out above; Rp a multiple of 16, Kp of 128.  Every lane of a wave
// takes part (the block maxima are wave shuffles): a job's lane count is a
// multiple of 256.
struct PieceJob {
  const float* f;
  int64_t rs, cs, R, K;
  uint8_t* P;
  uint8_t* E;
  int64_t Rp, Kp;
};

// lanes of a job: KC (k contiguous in F, cs = 1): 8 lanes per block, four
// consecutive k each, so that 32 adjacent lanes read one 512-byte row step;
// otherwise (rs = 1): 16 rows side by side, 4 lanes per block (16 apart),
// eight consecutive k each, so that 16 adjacent lanes read 16 consecutive
// floats of one k
template <bool KC>
__host__ __device__ constexpr int64_t piece_job_lanes(int64_t Rp, int64_t Kp) {
  return Rp * Kp / (KC ? 4 : 8);
}

// where lane gid of a job sits: row j, K step c, block s, its first
// position d in the step, and t (the lane's index within its block)
template <bool KC>
__device__ __forceinline__ void piece_lane_pos(int64_t Rp, int64_t gid, int64_t& j, int64_t& c,
                                               int& s, int& d, int& t) {
  if constexpr (KC) {
    t = (int)(gid & 7);
    s = (int)((gid >> 3) & 3);
    const int64_t jc = gid >> 5;
    j = jc % Rp;
    c = jc / Rp;
    d = 64 * (s & 1) + 16 * (s >> 1) + 32 * (t >> 2) + 4 * (t & 3);
  } else {
    const int jl = (int)(gid & 15);
    t = (int)((gid >> 4) & 3);
    s = (int)((gid >> 6) & 3);
    const int64_t jc = gid >> 8, nj = Rp / 16;
    j = (jc % nj) * 16 + jl;
    c = jc / nj;
    d = 64 * (s & 1) + 16 * (s >> 1) + 32 * (t >> 1) + 8 * (t & 1);
  }
}

// the pieces of a lane's N consecutive values v (row j, positions c * 128 +
// d ..): the block maximum over the block's lanes (wave shuffles), the
// block's exponent, the codes, the scale byte (by the block's lane t = 0)
template <bool KC, int N>
__device__ __forceinline__ void piece_lane_store(const float (&v)[N], uint8_t* __restrict__ P,
                                                 uint8_t* __restrict__ E, int64_t Rp, int64_t Kp,
                                                 int64_t j, int64_t c, int s, int d, int t) {
  uint32_t m = 0;
#pragma unroll
  for (int i = 0; i < N; ++i) m = max(m, finite_mag(v[i]));
  if constexpr (KC) {
#pragma unroll
    for (int o = 1; o < 8; o <<= 1) m = max(m, (uint32_t)__shfl_xor((int)m, o, 64));
  } else {
    m = max(m, (uint32_t)__shfl_xor((int)m, 16, 64));
    m = max(m, (uint32_t)__shfl_xor((int)m, 32, 64));
  }
  const int e = piece_exp(__uint_as_float(m));
  uint32_t q0[N / 4], q1[N / 4], q2[N / 4];
#pragma unroll
  for (int h = 0; h < N / 4; ++h)
    pieces4(ldexpf(v[4 * h], e), ldexpf(v[4 * h + 1], e), ldexpf(v[4 * h + 2], e),
            ldexpf(v[4 * h + 3], e), q0[h], q1[h], q2[h]);
  uint8_t* p = P + j * Kp + c * 128 + d;
  const int64_t plane = Rp * Kp;
  if constexpr (N == 4) {
    *reinterpret_cast<uint32_t*>(p) = q0[0];
    *reinterpret_cast<uint32_t*>(p + plane) = q1[0];
    *reinterpret_cast<uint32_t*>(p + 2 * plane) = q2[0];
  } else {
    *reinterpret_cast<uint2*>(p) = make_uint2(q0[0], q0[1]);
    *reinterpret_cast<uint2*>(p + plane) = make_uint2(q1[0], q1[1]);
    *reinterpret_cast<uint2*>(p + 2 * plane) = make_uint2(q2[0], q2[1]);
  }
  if (t == 0) E[(c * Rp + j) * 4 + s] = (uint8_t)(127 - e);
}

template <bool KC>
__device__ __forceinline__ void piece_job_lane(const PieceJob& q, int64_t gid) {
  constexpr int N = KC ? 4 : 8;
  int64_t j, c;
  int s, d, t;
  piece_lane_pos<KC>(q.Rp, gid, j, c, s, d, t);
  const int64_t k = c * 128 + d;
  float v[N];
  const bool row = j < q.R;
  const float* src = q.f + (row ? j * q.rs + k * q.cs : 0);
  if (KC && row && k + 3 < q.K && ((uintptr_t)src & 15) == 0) {
    const float4 x = *reinterpret_cast<const float4*>(src);
    v[0] = x.x;
    v[1] = x.y;
    v[2] = x.z;
    v[3] = x.w;
  } else {
#pragma unroll
    for (int i = 0; i < N; ++i) v[i] = row && k + i < q.K ? src[i * q.cs] : 0.0f;
  }
  piece_lane_store<KC, N>(v, q.P, q.E, q.Rp, q.Kp, j, c, s, d, t);
}

}  // namespace falq
