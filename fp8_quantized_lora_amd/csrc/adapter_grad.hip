// Rank-r adapter gradients of the melded layer on gfx950 matrix cores.
//
// With X^ = dec(X~)/s_x and G^ = dec(G~)/s_g (the FP8 tensors the forward and
// the dX product already hold: no second quantized LoRA path), the FALQON
// rebuttal (thread 4, reply Q1) gives dL/dA = B^T (dL/dO) x^T, and dL/dB uses
// the factor x A^T.  In row-major form:
//     U  = X^ A^T   [T x r]        V  = G^ B   [T x r]
//     dB = G^^T U   [d_out x r]    dA = V^T X^ [r x d_in]
//
// All four are "skinny" contractions: one operand is FP8 codes (T x d), the
// other a rank-r float operand.  One kernel does all of them:
//     P[s][m][n] = sum_{k in split s} dec(Q)[m][k] * H[n][k]
// where Q is read either row-wise (Q[m][k] = codes[m*ld + k]: U, V) or
// column-wise (Q[m][k] = codes[k*ld + m]: dB, dA, contracting over tokens),
// on v_mfma_f32_32x32x16_bf16.  Precision:
//  * an E4M3 code decodes exactly to bf16 (3 mantissa bits, fp32 exponent
//    range), so the FP8 operand is exact;
//  * the float operand H is split as H = hi + lo with hi = bf16(H),
//    lo = bf16(H - hi); two MFMAs per block, fp32 accumulation.  The relative
//    error per product is about 2^-17, far inside the 1e-3 parity bound;
//  * U and V are stored as hi/lo bf16 pairs as well (transposed to [r x T],
//    tokens padded with zeros to a multiple of 64) for the second pass.
// Work is split over K (d for U/V, T for dB/dA) so that every shape launches
// a few hundred workgroups; the partial sums are added in a fixed order by
// a reduction kernel (no atomics: the result is the same on every run).
// U and V are T x r: a few MiB, consumed at once, cache resident.
#include "common.hpp"
#include "kernels.hpp"
#include "pieces.hpp"
#include "transpose_u8.hpp"

#include <algorithm>

namespace falq {
namespace {

constexpr int TM = 256, TN = 64, TK = 128;     // skinny tile: M x N outputs, K step
constexpr int kSkThreads = 512;                // skinny kernel: 8 waves, 64 x 32 outputs each

__device__ __forceinline__ uint16_t bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}
__device__ __forceinline__ float bf16_to_f32(uint16_t h) { return __uint_as_float((uint32_t)h << 16); }

// two floats that hold E4M3 values (<= 4 significant bits) -> packed bf16x2 (exact)
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return __builtin_amdgcn_perm(__float_as_uint(hi), __float_as_uint(lo), 0x07060302u);
}

// 4 E4M3 codes in a dword -> 4 bf16 in two dwords (element order preserved)
__device__ __forceinline__ uint2 dec4_bf16(uint32_t w) {
  float2 a = dec2(w, false), b = dec2(w, true);
  return make_uint2(pack_bf16x2(a.x, a.y), pack_bf16x2(b.x, b.y));
}

// the same for E5M2 codes (2 mantissa bits, exponents 2^-16 .. 2^15: exact in bf16)
__device__ __forceinline__ uint2 dec4_bf16_e5m2(uint32_t w) {
  float2 a = dec2_e5m2(w, false), b = dec2_e5m2(w, true);
  return make_uint2(pack_bf16x2(a.x, a.y), pack_bf16x2(b.x, b.y));
}

// 16-byte chunk slot of chunk c in an LDS row of 128 bytes: the XOR by
// swz(row) makes the 16-row fragment reads conflict-free (same geometry as
// the FP8 GEMM's stages)
__device__ __forceinline__ int swz(int row) { return (row ^ ((row >> 3) & 1)) & 7; }

struct Prob {
  const uint8_t* Q;      // FP8 codes
  int64_t ldq;           // row stride of Q in bytes
  const uint16_t* Hhi;   // [N x ldh] bf16 bits, K contiguous
  const uint16_t* Hlo;
  int64_t ldh;
  float* P;              // [S][M][N] partial sums
  int M, N, K;           // contraction over K
  int kchunk;            // K range of split s: [s*kchunk, min(K, (s+1)*kchunk)), a multiple of TK
  int tilesM, tilesN;
};

// One K step of the skinny kernel, staged in registers between the global
// loads and the LDS stores (two steps are in flight).
struct Stage {
  uint4 q[4];            // FP8 operand: 64 bytes per thread
  uint4 h[4];            // bf16 hi/lo operand: 64 bytes per thread
  uint32_t ok;           // in-range bits: q (0..3, or 0..15 column-wise), h (16..19)
};

// P[s][m][n] = sum over k in split s of dec(Q)[m][k] * (Hhi + Hlo)[n][k]
// (NPL = 2), or of dec(Q)[m][k] * Hhi[n][k] alone (NPL = 1: H exact in bf16,
// e.g. decoded E4M3 codes).
// Q is read row-wise (Q[m][k] = codes[m * ldq + k]) or, with TRANS,
// column-wise (Q[m][k] = codes[k * ldq + m]: contraction over tokens, the
// 4 x 16-byte transpose done in registers).  LDS holds the FP8 codes
// ([256 rows][128 k], 32 KB) and H ([hi/lo][k half][64 n][64 k], 32 KB) per
// stage; the codes are decoded to bf16 when a fragment is read.
//
// The grid is 1-D over (problem, split, tile) with the tile fastest.  The
// dispatcher deals consecutive workgroup ids round-robin to the 8 XCDs; the
// id is remapped so that each XCD gets a run of consecutive logical ids, i.e.
// whole (problem, split) groups, whose tiles all read the same K chunk of H:
// that chunk then comes from HBM into one XCD's L2 once, not once per tile.
typedef uint8_t SkQ[TM * TK];             // one stage of FP8 codes
typedef uint8_t SkH[2][2][TN * 128];      // one stage of H: [hi/lo][k half][64 n x 64 k]

// One workgroup: tile `tile` of problem p over K split s.  QF is the format
// of p's codes (0 E4M3, 1 E5M2: both decode exactly to bf16).
template <bool TRANS, int NPL, int QF>
__device__ __forceinline__ void skinny_tile(const Prob& p, int tile, int s, SkQ* sQ, SkH* sH) {
  static_assert(NPL == 1 || NPL == 2, "one or two bf16 planes of H");
  const int m0 = (tile % p.tilesM) * TM;
  const int n0 = (tile / p.tilesM) * TN;
  const int kb = s * p.kchunk;
  const int ke = min(p.K, kb + p.kchunk);

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int wm = w >> 1, wn = w & 1;             // wave tile: rows wm*64.., cols wn*32..
  v16f acc[2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int v = 0; v < 16; ++v) acc[i][v] = 0.0f;

  // Every load is issued unconditionally from a clamped in-bounds address;
  // the out-of-range parts are zeroed only when the stage is written to LDS,
  // so nothing waits for a stage's loads before the step that stores it.
  auto gload = [&](int k0, Stage& R) {
    uint32_t ok = 0;
    if (!TRANS) {
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int c = tid + u * kSkThreads;                  // 2048 chunks of 16 codes
        const int row = c >> 3, col = (c & 7) * 16;
        const int gm = m0 + row, gk = k0 + col;
        R.q[u] = *reinterpret_cast<const uint4*>(p.Q + (int64_t)min(gm, p.M - 1) * p.ldq +
                                                 min(gk, p.K - 16));
        ok |= (gm < p.M && gk < ke) ? 1u << u : 0u;
      }
    } else {
      const int m4 = (tid & 63) * 4, tg = tid >> 6;         // 4 columns x 16 tokens
      const int gm = m0 + m4;
      uint32_t d[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int gk = k0 + tg * 16 + i;
        d[i] = *reinterpret_cast<const uint32_t*>(p.Q + (int64_t)min(gk, p.K - 1) * p.ldq +
                                                  min(gm, p.M - 4));
        ok |= (gm < p.M && gk < ke) ? 1u << i : 0u;
      }
#pragma unroll
      for (int u = 0; u < 4; ++u) R.q[u] = make_uint4(d[4 * u], d[4 * u + 1], d[4 * u + 2], d[4 * u + 3]);
    }
#pragma unroll
    for (int u = 0; u < 2 * NPL; ++u) {
      const int c = tid + u * kSkThreads;                    // [hi/lo][64 n][16 chunks of 8]
      const int h = c >> 10, rem = c & 1023;
      const int n = rem >> 4, k8 = (rem & 15) * 8;
      const int gn = n0 + n, gk = k0 + k8;
      // H rows may be padded past K; out-of-range lanes read row 0
      const bool in = gn < p.N && gk < ke;
      const int64_t off = in ? (int64_t)gn * p.ldh + gk : 0;
      R.h[u] = *reinterpret_cast<const uint4*>((h ? p.Hlo : p.Hhi) + off);
      ok |= in ? 1u << (16 + u) : 0u;
    }
    R.ok = ok;
  };
  auto keep = [](uint4 v, uint32_t ok, int bit) {
    const uint32_t m = 0u - ((ok >> bit) & 1u);
    return make_uint4(v.x & m, v.y & m, v.z & m, v.w & m);
  };

  auto sstore = [&](int buf, const Stage& R) {
    if (!TRANS) {
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int c = tid + u * kSkThreads;
        const int row = c >> 3, ch = c & 7;
        *reinterpret_cast<uint4*>(sQ[buf] + row * TK + ((ch ^ swz(row)) * 16)) = keep(R.q[u], R.ok, u);
      }
    } else {
      const int m4 = (tid & 63) * 4, tg = tid >> 6;
      uint32_t out[4][4];                                    // [column][4 tokens]
#pragma unroll
      for (int g = 0; g < 4; ++g) {                          // tokens 4g .. 4g+3
        uint4 v = R.q[g];
        v.x &= 0u - ((R.ok >> (4 * g)) & 1u);
        v.y &= 0u - ((R.ok >> (4 * g + 1)) & 1u);
        v.z &= 0u - ((R.ok >> (4 * g + 2)) & 1u);
        v.w &= 0u - ((R.ok >> (4 * g + 3)) & 1u);
        const uint32_t t01a = __builtin_amdgcn_perm(v.y, v.x, 0x05010400u);
        const uint32_t t01b = __builtin_amdgcn_perm(v.y, v.x, 0x07030602u);
        const uint32_t t23a = __builtin_amdgcn_perm(v.w, v.z, 0x05010400u);
        const uint32_t t23b = __builtin_amdgcn_perm(v.w, v.z, 0x07030602u);
        out[0][g] = __builtin_amdgcn_perm(t23a, t01a, 0x05040100u);
        out[1][g] = __builtin_amdgcn_perm(t23a, t01a, 0x07060302u);
        out[2][g] = __builtin_amdgcn_perm(t23b, t01b, 0x05040100u);
        out[3][g] = __builtin_amdgcn_perm(t23b, t01b, 0x07060302u);
      }
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const int row = m4 + c;
        *reinterpret_cast<uint4*>(sQ[buf] + row * TK + ((tg ^ swz(row)) * 16)) =
            make_uint4(out[c][0], out[c][1], out[c][2], out[c][3]);
      }
    }
#pragma unroll
    for (int u = 0; u < 2 * NPL; ++u) {
      const int c = tid + u * kSkThreads;
      const int h = c >> 10, rem = c & 1023;
      const int n = rem >> 4, k8 = rem & 15;
      *reinterpret_cast<uint4*>(sH[buf][h][k8 >> 3] + n * 128 + (((k8 & 7) ^ swz(n)) * 16)) =
          keep(R.h[u], R.ok, 16 + u);
    }
  };

  // fragments: 32x32x16 bf16 MFMA, lane l: row/col l % 32, K half l / 32.
  // A 16-byte LDS chunk holds the codes of two consecutive MFMA steps: step
  // 2*q2 + sub of the stage uses k = q2*32 + half*16 + sub*8 + 0..7 for both
  // operands (a fixed permutation of the stage's 128 k).
  const int r32 = lane & 31, half = lane >> 5;
  auto compute = [&](int buf) {
#pragma unroll
    for (int q2 = 0; q2 < TK / 32; ++q2) {
      v8bf a[2][2];                                          // [m block][sub]
#pragma unroll
      for (int mb = 0; mb < 2; ++mb) {
        const int row = wm * 64 + mb * 32 + r32;
        const uint4 c = *reinterpret_cast<const uint4*>(sQ[buf] + row * TK +
                                                        (((q2 * 2 + half) ^ swz(row)) * 16));
        uint2 c0, c1, c2, c3;
        if (QF == 0) {
          c0 = dec4_bf16(c.x); c1 = dec4_bf16(c.y); c2 = dec4_bf16(c.z); c3 = dec4_bf16(c.w);
        } else {
          c0 = dec4_bf16_e5m2(c.x); c1 = dec4_bf16_e5m2(c.y);
          c2 = dec4_bf16_e5m2(c.z); c3 = dec4_bf16_e5m2(c.w);
        }
        a[mb][0] = __builtin_bit_cast(v8bf, make_uint4(c0.x, c0.y, c1.x, c1.y));
        a[mb][1] = __builtin_bit_cast(v8bf, make_uint4(c2.x, c2.y, c3.x, c3.y));
      }
      const int n = wn * 32 + r32;
#pragma unroll
      for (int sub = 0; sub < 2; ++sub) {
        const int ch = ((q2 & 1) * 4 + half * 2 + sub) ^ swz(n);
        const v8bf bh = __builtin_bit_cast(
            v8bf, *reinterpret_cast<const uint4*>(sH[buf][0][q2 >> 1] + n * 128 + ch * 16));
#pragma unroll
        for (int mb = 0; mb < 2; ++mb)
          acc[mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[mb][sub], bh, acc[mb], 0, 0, 0);
        if (NPL == 2) {
          const v8bf bl = __builtin_bit_cast(
              v8bf, *reinterpret_cast<const uint4*>(sH[buf][1][q2 >> 1] + n * 128 + ch * 16));
#pragma unroll
          for (int mb = 0; mb < 2; ++mb)
            acc[mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[mb][sub], bl, acc[mb], 0, 0, 0);
        }
      }
    }
  };
  // LDS stores of this wave complete, then a barrier that does not wait for
  // the global loads still in flight
  auto sync = [] {
    __builtin_amdgcn_s_waitcnt(0xC07F);                     // lgkmcnt(0)
    barrier_no_drain();
  };

  const int nk = ke > kb ? (ke - kb + TK - 1) / TK : 0;
  Stage R0, R1;
  gload(kb, R0);
  gload(kb + TK, R1);
  if (nk > 0) sstore(0, R0);
  sync();
  // step it: stage it is in LDS buffer it & 1, stage it+1 in registers; the
  // loads of stage it+2 go into the register set that stage it came from
  // (the loads of stage it+2 are issued even past the last stage, from
  // clamped addresses and never stored: a fixed number of loads in flight
  // lets the compiler wait for exactly one stage)
  auto step = [&](int it, Stage& Rcur, Stage& Rnext) {
    gload(kb + (it + 2) * TK, Rcur);
    __builtin_amdgcn_sched_barrier(0);
    compute(it & 1);
    __builtin_amdgcn_sched_barrier(0);
    if (it + 1 < nk) sstore((it + 1) & 1, Rnext);
    sync();
  };
  int it = 0;
  for (; it + 1 < nk; it += 2) {
    step(it, R0, R1);
    step(it + 1, R1, R0);
  }
  if (it < nk) step(it, R0, R1);

  float* P = p.P + (int64_t)s * p.M * p.N;
  const int n = n0 + wn * 32 + r32;
  if (n < p.N) {
#pragma unroll
    for (int mb = 0; mb < 2; ++mb) {
      const int rbase = m0 + wm * 64 + mb * 32 + 4 * half;
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int m = rbase + 8 * (v >> 2) + (v & 3);
        if (m < p.M) P[(int64_t)m * p.N + n] = acc[mb][v];
      }
    }
  }
}

// Grid: (problem, split, tile) with the tile fastest; problem 0 uses codes of
// format QF0, problem 1 of format QF1.
template <bool TRANS, int NPL, int QF0, int QF1>
__global__ __launch_bounds__(kSkThreads, 1) void skinny_kernel(Prob p0, Prob p1, int tiles_max,
                                                               int splits) {
  __shared__ __attribute__((aligned(16))) SkQ sQ[2];     // 64 KB
  __shared__ __attribute__((aligned(16))) SkH sH[2];     // 64 KB
  const int nblk = gridDim.x, per = nblk / 8, b = blockIdx.x;
  const int lid = b < per * 8 ? (b % 8) * per + b / 8 : b;
  const int tile = lid % tiles_max, rest = lid / tiles_max;
  const int s = rest % splits;
  if constexpr (QF0 == QF1) {
    const Prob p = rest / splits == 0 ? p0 : p1;           // a copy: selected in SGPRs
    if (tile >= p.tilesM * p.tilesN) return;
    skinny_tile<TRANS, NPL, QF0>(p, tile, s, sQ, sH);
  } else if (rest / splits == 0) {
    if (tile >= p0.tilesM * p0.tilesN) return;
    skinny_tile<TRANS, NPL, QF0>(p0, tile, s, sQ, sH);
  } else {
    if (tile >= p1.tilesM * p1.tilesN) return;
    skinny_tile<TRANS, NPL, QF1>(p1, tile, s, sQ, sH);
  }
}

// fp32 [rows x cols] -> bf16 hi/lo, optionally transposed ([cols x ld_out]).
// Two problems per launch (blockIdx.z), 32 x 32 tiles.
struct Split {
  const float* src;
  int rows, cols;
  bool transpose;
  int64_t ld_out;
  uint16_t* hi;
  uint16_t* lo;
  int tx, ty;          // tiles along cols, rows
};

// one 32 x 32 tile of a Split (256 threads; t: 32 x 33 floats of LDS)
__device__ __forceinline__ void split_tile(const Split& p, int tile, float (*t)[33]) {
  const int r0 = (tile / p.tx) * 32, c0 = (tile % p.tx) * 32;
  const int tx = threadIdx.x & 31, ty = threadIdx.x >> 5;   // 32 x 8
  if (!p.transpose) {
    for (int rr = ty; rr < 32; rr += 8) {
      const int r = r0 + rr, c = c0 + tx;
      if (r < p.rows && c < p.cols) {
        const float x = p.src[(int64_t)r * p.cols + c];
        const uint16_t h = bf16_rne(x);
        p.hi[(int64_t)r * p.ld_out + c] = h;
        p.lo[(int64_t)r * p.ld_out + c] = bf16_rne(x - bf16_to_f32(h));
      }
    }
    return;
  }
  for (int rr = ty; rr < 32; rr += 8) {
    const int r = r0 + rr, c = c0 + tx;
    t[rr][tx] = (r < p.rows && c < p.cols) ? p.src[(int64_t)r * p.cols + c] : 0.0f;
  }
  __syncthreads();
  for (int cc = ty; cc < 32; cc += 8) {
    const int c = c0 + cc, r = r0 + tx;
    if (c < p.cols && r < p.rows) {
      const float x = t[tx][cc];
      const uint16_t h = bf16_rne(x);
      p.hi[(int64_t)c * p.ld_out + r] = h;
      p.lo[(int64_t)c * p.ld_out + r] = bf16_rne(x - bf16_to_f32(h));
    }
  }
}

__global__ __launch_bounds__(256) void split_bf16_kernel(Split p0, Split p1) {
  const Split p = blockIdx.z == 0 ? p0 : p1;
  if ((int)blockIdx.x >= p.tx * p.ty) return;
  __shared__ float t[32][33];
  split_tile(p, (int)blockIdx.x, t);
}

// The backward's preparation in one launch (each part alone is too small to
// fill the GPU, and every launch costs a few microseconds of ramp): workgroups
// [0, n_tr) transpose W~ for the dX product (128 x 128 tiles, tr_tx per tile
// row), the next sa.tx * sa.ty split A, the rest split B (transposed).
__global__ __launch_bounds__(256) void bwd_prep_kernel(const uint8_t* __restrict__ wq,
                                                       int64_t d_out, int64_t d_in,
                                                       uint8_t* __restrict__ wt, int n_tr,
                                                       int tr_tx, Split sa, Split sb) {
  __shared__ float t[32][33];
  const int b = blockIdx.x;
  if (b < n_tr) {
    transpose_u8_tile(wq, d_out, d_in, wt, b % tr_tx, b / tr_tx);
    return;
  }
  const int na = sa.tx * sa.ty;
  if (b - n_tr < na)
    split_tile(sa, b - n_tr, t);
  else
    split_tile(sb, b - n_tr - na, t);
}

// out = sum_s P[s] / (*sc * *sc2) with P[s] of shape [M x N] (a null sc or
// sc2 stands for 1), folded in split
// order s = 0, 1, ... (deterministic).  A workgroup owns a 16 (m) x 64 (n)
// tile, one float4 of it per thread, transposed through LDS when the output
// is n-major.  Two problems per launch (blockIdx.z).
//   mode 0: out_f32[m * ldo + n]           (dB)
//   mode 1: out_f32[n * ldo + m]           (dA)
//   mode 2: hi/lo bf16 [n * ldo + m], and zeros for M <= m < Mpad   (U^T, V^T)
struct Red {
  const float* P;
  int S, M, N, Mpad;
  const float* sc;
  const float* sc2;
  int mode;
  float* out;
  int64_t ldo;
  uint16_t* ohi;
  uint16_t* olo;
  int tilesM, tilesN;
};

constexpr int RM = 16;   // rows of a reduction tile

__global__ __launch_bounds__(256) void reduce_kernel(Red r0, Red r1) {
  const Red R = blockIdx.z == 0 ? r0 : r1;
  const int tile = blockIdx.x;
  if (tile >= R.tilesM * R.tilesN) return;
  const int m0 = (tile % R.tilesM) * RM, n0 = (tile / R.tilesM) * 64;
  __shared__ float t[64][RM + 1];
  const int tid = threadIdx.x;
  const float scale = 1.0f / ((R.sc ? R.sc[0] : 1.0f) * (R.sc2 ? R.sc2[0] : 1.0f));
  const int64_t plane = (int64_t)R.M * R.N;
  const bool vec = (R.N % 4) == 0;
  const int mm = tid >> 4, nn = (tid & 15) * 4;
  const int m = m0 + mm, n = n0 + nn;
  float v[4] = {0.f, 0.f, 0.f, 0.f};
  if (m < R.M && n < R.N) {
    const int64_t off = (int64_t)m * R.N + n;
    if (vec) {
      // eight planes' loads in flight, added in plane order
      for (int s0 = 0; s0 < R.S; s0 += 8) {
        float4 x[8];
#pragma unroll
        for (int u = 0; u < 8; ++u)
          x[u] = s0 + u < R.S ? *reinterpret_cast<const float4*>(R.P + (s0 + u) * plane + off)
                              : make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
        for (int u = 0; u < 8; ++u)
          if (s0 + u < R.S) { v[0] += x[u].x; v[1] += x[u].y; v[2] += x[u].z; v[3] += x[u].w; }
      }
    } else {
      for (int s = 0; s < R.S; ++s)
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if (n + e < R.N) v[e] += R.P[s * plane + off + e];
    }
  }
#pragma unroll
  for (int e = 0; e < 4; ++e) v[e] *= scale;
  if (R.mode == 0) {
    if (m < R.M) {
      if (vec && n < R.N && (R.ldo % 4) == 0) {
        *reinterpret_cast<float4*>(R.out + (int64_t)m * R.ldo + n) = make_float4(v[0], v[1], v[2], v[3]);
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if (n + e < R.N) R.out[(int64_t)m * R.ldo + n + e] = v[e];
      }
    }
    return;
  }
#pragma unroll
  for (int e = 0; e < 4; ++e) t[nn + e][mm] = v[e];
  __syncthreads();
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int idx = tid + u * 256;            // 64 rows (n) x 16 m
    const int tn = idx >> 4, tm = idx & 15;
    const int nn2 = n0 + tn, mm2 = m0 + tm;
    if (nn2 >= R.N) continue;
    const float x = t[tn][tm];
    if (R.mode == 1) {
      if (mm2 < R.M) R.out[(int64_t)nn2 * R.ldo + mm2] = x;
    } else if (mm2 < R.Mpad) {
      const uint16_t h = bf16_rne(x);
      R.ohi[(int64_t)nn2 * R.ldo + mm2] = h;
      R.olo[(int64_t)nn2 * R.ldo + mm2] = bf16_rne(x - bf16_to_f32(h));
    }
  }
}

Red red(const float* P, int S, int64_t M, int64_t N, int64_t Mpad, const float* sc, int mode,
        float* out, int64_t ldo, uint16_t* ohi, uint16_t* olo) {
  Red r;
  r.P = P; r.S = S; r.M = (int)M; r.N = (int)N; r.Mpad = (int)Mpad; r.sc = sc; r.sc2 = nullptr;
  r.mode = mode;
  r.out = out; r.ldo = ldo; r.ohi = ohi; r.olo = olo;
  r.tilesM = (int)((std::max(M, Mpad) + RM - 1) / RM);
  r.tilesN = (int)((N + 63) / 64);
  return r;
}

void launch_reduce(const Red& a, const Red* b, hipStream_t s) {
  const int tiles = std::max(a.tilesM * a.tilesN, b ? b->tilesM * b->tilesN : 0);
  reduce_kernel<<<dim3(tiles, 1, b ? 2 : 1), 256, 0, s>>>(a, b ? *b : a);
}

__global__ void fill_kernel(float* p, int64_t n, float v) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
       i += (int64_t)gridDim.x * blockDim.x)
    p[i] = v;
}

// E4M3 codes -> bf16 (exact: 3 mantissa bits), 16 codes per thread; n is a
// multiple of 16
__global__ __launch_bounds__(256) void decode_bf16_kernel(const uint8_t* __restrict__ q, int64_t n,
                                                          uint16_t* __restrict__ out) {
  const int64_t n16 = n / 16;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n16;
       i += (int64_t)gridDim.x * blockDim.x) {
    const uint4 c = reinterpret_cast<const uint4*>(q)[i];
    const uint2 a = dec4_bf16(c.x), b = dec4_bf16(c.y), d = dec4_bf16(c.z), e = dec4_bf16(c.w);
    reinterpret_cast<uint4*>(out)[2 * i] = make_uint4(a.x, a.y, b.x, b.y);
    reinterpret_cast<uint4*>(out)[2 * i + 1] = make_uint4(d.x, d.y, e.x, e.y);
  }
}

// ---------------------------------------------------------------------------
// Host-side plan: split counts and workspace layout (identical for the size
// query and the launch).
// ---------------------------------------------------------------------------
struct Plan {
  int64_t Tp;            // tokens padded to TK
  int S1, S2;            // K splits of pass 1 (U, V) and pass 2 (dB, dA)
  int kc1u, kc1v, kc2;   // K chunk per split
  size_t off_ahi, off_alo, off_bhi, off_blo, off_p1u, off_p1v, off_uhi, off_ulo, off_vhi, off_vlo,
      off_p2b, off_p2a, total;
};

int ceil_div(int64_t a, int64_t b) { return (int)((a + b - 1) / b); }

// splits of K so that about one skinny workgroup per CU (256) runs, each
// with at least two K steps
int pick_splits(int64_t tiles, int64_t K, int64_t per_split_bytes, int64_t cap_bytes) {
  int s = 1;
  while (tiles * s < 256 && K / (int64_t)(s * 2) >= 2 * TK && per_split_bytes * (s * 2) <= cap_bytes)
    s *= 2;
  return s;
}

int chunk_for(int64_t K, int S) { return ceil_div(ceil_div(K, S), TK) * TK; }

Plan make_plan(int64_t T, int64_t d_in, int64_t d_out, int64_t r) {
  Plan p{};
  p.Tp = (T + TK - 1) / TK * TK;
  const int64_t nT = ceil_div(r, TN);
  const int64_t tiles1 = (int64_t)ceil_div(T, TM) * nT * 2;
  const int64_t tiles2 = ((int64_t)ceil_div(d_in, TM) + ceil_div(d_out, TM)) * nT;
  const int64_t cap = 256ll << 20;
  p.S1 = pick_splits(tiles1, std::min(d_in, d_out), T * r * 4 * 2, cap);
  p.S2 = pick_splits(tiles2, T, (d_in + d_out) * r * 4, cap);
  p.kc1u = chunk_for(d_in, p.S1);
  p.kc1v = chunk_for(d_out, p.S1);
  p.kc2 = chunk_for(T, p.S2);
  size_t o = 0;
  auto take = [&](size_t bytes) { size_t at = o; o = align_up(o + bytes, 256); return at; };
  p.off_ahi = take((size_t)r * d_in * 2);
  p.off_alo = take((size_t)r * d_in * 2);
  p.off_bhi = take((size_t)r * d_out * 2);
  p.off_blo = take((size_t)r * d_out * 2);
  p.off_p1u = take((size_t)p.S1 * T * r * 4);
  p.off_p1v = take((size_t)p.S1 * T * r * 4);
  p.off_uhi = take((size_t)r * p.Tp * 2);
  p.off_ulo = take((size_t)r * p.Tp * 2);
  p.off_vhi = take((size_t)r * p.Tp * 2);
  p.off_vlo = take((size_t)r * p.Tp * 2);
  p.off_p2b = take((size_t)p.S2 * d_out * r * 4);
  p.off_p2a = take((size_t)p.S2 * d_in * r * 4);
  p.total = o;
  return p;
}

Prob prob(const uint8_t* Q, int64_t ldq, const uint16_t* hi, const uint16_t* lo, int64_t ldh,
          float* P, int64_t M, int64_t N, int64_t K, int kchunk) {
  Prob q;
  q.Q = Q; q.ldq = ldq; q.Hhi = hi; q.Hlo = lo; q.ldh = ldh; q.P = P;
  q.M = (int)M; q.N = (int)N; q.K = (int)K; q.kchunk = kchunk;
  q.tilesM = ceil_div(M, TM);
  q.tilesN = ceil_div(N, TN);
  return q;
}

// Frozen FP8 factor A~: U = dec(X~) dec(A~)^T (one skinny problem, H = the
// decoded codes, one bf16 plane) and dB = dec(G~)^T U (one problem, H = U^T
// as bf16 hi/lo).
struct FrozenPlan {
  int64_t Tp;
  int S;                 // K splits
  int kc;                // K chunk per split
  size_t off_h, off_lo, off_p, total;
};

FrozenPlan frozen_u_plan(int64_t T, int64_t d_in, int64_t r) {
  FrozenPlan p{};
  const int64_t tiles = (int64_t)ceil_div(T, TM) * ceil_div(r, TN);
  p.S = pick_splits(tiles, d_in, T * r * 4, 256ll << 20);
  p.kc = chunk_for(d_in, p.S);
  size_t o = 0;
  auto take = [&](size_t bytes) { size_t at = o; o = align_up(o + bytes, 256); return at; };
  p.off_h = take((size_t)r * d_in * 2);        // decoded A~ [r x d_in] bf16
  p.off_p = take((size_t)p.S * T * r * 4);     // partials [S][T][r]
  p.total = o;
  return p;
}

FrozenPlan frozen_db_plan(int64_t T, int64_t d_out, int64_t r) {
  FrozenPlan p{};
  p.Tp = (T + TK - 1) / TK * TK;
  const int64_t tiles = (int64_t)ceil_div(d_out, TM) * ceil_div(r, TN);
  p.S = pick_splits(tiles, T, d_out * r * 4, 256ll << 20);
  p.kc = chunk_for(T, p.S);
  size_t o = 0;
  auto take = [&](size_t bytes) { size_t at = o; o = align_up(o + bytes, 256); return at; };
  p.off_h = take((size_t)r * p.Tp * 2);        // U^T hi [r x Tp]
  p.off_lo = take((size_t)r * p.Tp * 2);       // U^T lo
  p.off_p = take((size_t)p.S * d_out * r * 4); // partials [S][d_out][r]
  p.total = o;
  return p;
}

}  // namespace

size_t frozen_u_ws_bytes(int64_t T, int64_t d_in, int64_t r) {
  if (r == 0 || T == 0) return 0;
  return frozen_u_plan(T, d_in, r).total;
}

size_t frozen_db_ws_bytes(int64_t T, int64_t d_out, int64_t r) {
  if (r == 0 || T == 0) return 0;
  return frozen_db_plan(T, d_out, r).total;
}

hipError_t launch_frozen_u(const uint8_t* xq, const float* s_x, const uint8_t* aq,
                           const float* s_a, int64_t T, int64_t d_in, int64_t r, float* u,
                           void* ws, hipStream_t s) {
  if (r == 0 || T == 0) return hipSuccess;
  if (d_in == 0) return launch_fill_f32(u, T * r, 0.0f, s);
  const FrozenPlan pl = frozen_u_plan(T, d_in, r);
  uint8_t* base = reinterpret_cast<uint8_t*>(ws);
  uint16_t* h = reinterpret_cast<uint16_t*>(base + pl.off_h);
  float* part = reinterpret_cast<float*>(base + pl.off_p);
  {
    const int64_t n16 = r * d_in / 16;
    const int blocks = (int)std::min<int64_t>((n16 + 255) / 256, 2048);
    decode_bf16_kernel<<<blocks, 256, 0, s>>>(aq, r * d_in, h);
  }
  const Prob pu = prob(xq, d_in, h, nullptr, d_in, part, T, r, d_in, pl.kc);
  const int tiles = pu.tilesM * pu.tilesN;
  skinny_kernel<false, 1, 0, 0><<<tiles * pl.S, kSkThreads, 0, s>>>(pu, pu, tiles, pl.S);
  Red ru = red(part, pl.S, T, r, T, s_x, 0, u, r, nullptr, nullptr);
  ru.sc2 = s_a;
  launch_reduce(ru, nullptr, s);
  return hipGetLastError();
}

hipError_t launch_frozen_db(const uint8_t* gq, const float* s_g, const float* u, int64_t T,
                            int64_t d_out, int64_t r, float* dB, void* ws, hipStream_t s,
                            int g_fmt) {
  if (r == 0 || d_out == 0) return hipSuccess;
  if (T == 0) return launch_fill_f32(dB, d_out * r, 0.0f, s);
  const FrozenPlan pl = frozen_db_plan(T, d_out, r);
  uint8_t* base = reinterpret_cast<uint8_t*>(ws);
  uint16_t* hi = reinterpret_cast<uint16_t*>(base + pl.off_h);
  uint16_t* lo = reinterpret_cast<uint16_t*>(base + pl.off_lo);
  float* part = reinterpret_cast<float*>(base + pl.off_p);
  // U [T x r] -> U^T as bf16 hi/lo [r x Tp], tokens T..Tp-1 zero (one plane, no scale)
  launch_reduce(red(u, 1, T, r, pl.Tp, nullptr, 2, nullptr, pl.Tp, hi, lo), nullptr, s);
  const Prob pb = prob(gq, d_out, hi, lo, pl.Tp, part, d_out, r, T, pl.kc);
  const int tiles = pb.tilesM * pb.tilesN;
  if (g_fmt == 0)
    skinny_kernel<true, 2, 0, 0><<<tiles * pl.S, kSkThreads, 0, s>>>(pb, pb, tiles, pl.S);
  else
    skinny_kernel<true, 2, 1, 1><<<tiles * pl.S, kSkThreads, 0, s>>>(pb, pb, tiles, pl.S);
  launch_reduce(red(part, pl.S, d_out, r, d_out, s_g, 0, dB, r, nullptr, nullptr), nullptr, s);
  return hipGetLastError();
}

size_t adapter_grad_ws_bytes(int64_t T, int64_t d_in, int64_t d_out, int64_t r) {
  if (r == 0 || T == 0) return 0;
  return make_plan(T, d_in, d_out, r).total;
}

hipError_t launch_fill_f32(float* p, int64_t n, float v, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  int blocks = (int)std::min<int64_t>((n + 255) / 256, 4096);
  fill_kernel<<<blocks, 256, 0, s>>>(p, n, v);
  return hipGetLastError();
}

// the two float-operand splits of the adapter gradients (A as is; B
// transposed, only when dA is wanted)
namespace {
void make_splits(const Plan& pl, uint8_t* base, const float* A, const float* B, int64_t d_in,
                 int64_t d_out, int64_t r, Split& sa, Split& sb) {
  auto u16 = [&](size_t off) { return reinterpret_cast<uint16_t*>(base + off); };
  sa = Split{A, (int)r, (int)d_in, false, d_in, u16(pl.off_ahi), u16(pl.off_alo),
             ceil_div(d_in, 32), ceil_div(r, 32)};
  sb = Split{B, (int)d_out, (int)r, true, d_out, u16(pl.off_bhi), u16(pl.off_blo),
             ceil_div(r, 32), ceil_div(d_out, 32)};
}
}  // namespace

hipError_t launch_bwd_prep(const uint8_t* wq, uint8_t* wt, const float* A, const float* B,
                           int64_t T, int64_t d_in, int64_t d_out, int64_t r, bool want_da,
                           void* ws, hipStream_t s) {
  const bool tr = wt != nullptr && d_in > 0 && d_out > 0;
  const bool sp = r > 0 && T > 0 && d_in > 0 && d_out > 0;
  if (!tr && !sp) return hipSuccess;
  if (tr && (d_in % 16 != 0 || d_out % 16 != 0)) return hipErrorInvalidValue;
  const int tr_tx = tr ? ceil_div(d_in, 128) : 1;
  const int n_tr = tr ? tr_tx * ceil_div(d_out, 128) : 0;
  Split sa{}, sb{};
  if (sp) {
    make_splits(make_plan(T, d_in, d_out, r), reinterpret_cast<uint8_t*>(ws), A, B, d_in, d_out,
                r, sa, sb);
    if (!want_da) sb.tx = sb.ty = 0;
  }
  const int grid = n_tr + sa.tx * sa.ty + sb.tx * sb.ty;
  bwd_prep_kernel<<<grid, 256, 0, s>>>(wq, d_out, d_in, wt, n_tr, tr_tx, sa, sb);
  return hipGetLastError();
}

hipError_t launch_adapter_grads(const uint8_t* gq, const float* s_g, const uint8_t* xq,
                                const float* s_x, const float* A, const float* B, int64_t T,
                                int64_t d_in, int64_t d_out, int64_t r, float* dA, float* dB,
                                void* ws, hipStream_t s, int g_fmt, bool presplit) {
  if (r == 0) return hipSuccess;
  if (T == 0) {
    hipError_t e = launch_fill_f32(dB, d_out * r, 0.0f, s);
    if (e == hipSuccess && dA) e = launch_fill_f32(dA, r * d_in, 0.0f, s);
    return e;
  }
  const Plan pl = make_plan(T, d_in, d_out, r);
  uint8_t* base = reinterpret_cast<uint8_t*>(ws);
  auto u16 = [&](size_t off) { return reinterpret_cast<uint16_t*>(base + off); };
  auto f32 = [&](size_t off) { return reinterpret_cast<float*>(base + off); };
  const bool want_da = dA != nullptr;

  // 0. float operands -> bf16 hi/lo: A as is [r x d_in]; B transposed [r x d_out]
  //    (done already by launch_bwd_prep when presplit)
  if (!presplit) {
    Split sa, sb;
    make_splits(pl, base, A, B, d_in, d_out, r, sa, sb);
    const int tiles = std::max(sa.tx * sa.ty, want_da ? sb.tx * sb.ty : 0);
    split_bf16_kernel<<<dim3(tiles, 1, want_da ? 2 : 1), 256, 0, s>>>(sa, sb);
  }

  // 1. U = dec(X~) A^T, V = dec(G~) B  (partials over d)
  Prob pu = prob(xq, d_in, u16(pl.off_ahi), u16(pl.off_alo), d_in, f32(pl.off_p1u), T, r, d_in,
                 pl.kc1u);
  Prob pv = prob(gq, d_out, u16(pl.off_bhi), u16(pl.off_blo), d_out, f32(pl.off_p1v), T, r, d_out,
                 pl.kc1v);
  {
    const int tiles = pu.tilesM * pu.tilesN;
    const int grid = tiles * pl.S1 * (want_da ? 2 : 1);
    if (g_fmt == 0)
      skinny_kernel<false, 2, 0, 0><<<grid, kSkThreads, 0, s>>>(pu, pv, tiles, pl.S1);
    else
      skinny_kernel<false, 2, 0, 1><<<grid, kSkThreads, 0, s>>>(pu, pv, tiles, pl.S1);
  }
  // reduce -> U^T, V^T as bf16 hi/lo [r x Tp], scaled by 1/s_x, 1/s_g
  {
    const Red ru = red(f32(pl.off_p1u), pl.S1, T, r, pl.Tp, s_x, 2, nullptr, pl.Tp,
                       u16(pl.off_uhi), u16(pl.off_ulo));
    const Red rv = red(f32(pl.off_p1v), pl.S1, T, r, pl.Tp, s_g, 2, nullptr, pl.Tp,
                       u16(pl.off_vhi), u16(pl.off_vlo));
    launch_reduce(ru, want_da ? &rv : nullptr, s);
  }

  // 2. dB = dec(G~)^T U, dA^T = dec(X~)^T V  (contract over tokens, partials over T)
  Prob pb = prob(gq, d_out, u16(pl.off_uhi), u16(pl.off_ulo), pl.Tp, f32(pl.off_p2b), d_out, r,
                 T, pl.kc2);
  Prob pa = prob(xq, d_in, u16(pl.off_vhi), u16(pl.off_vlo), pl.Tp, f32(pl.off_p2a), d_in, r, T,
                 pl.kc2);
  {
    const int tiles = std::max(pb.tilesM * pb.tilesN, want_da ? pa.tilesM * pa.tilesN : 0);
    const int grid = tiles * pl.S2 * (want_da ? 2 : 1);
    if (g_fmt == 0)
      skinny_kernel<true, 2, 0, 0><<<grid, kSkThreads, 0, s>>>(pb, pa, tiles, pl.S2);
    else
      skinny_kernel<true, 2, 1, 0><<<grid, kSkThreads, 0, s>>>(pb, pa, tiles, pl.S2);
  }
  {
    const Red rb = red(f32(pl.off_p2b), pl.S2, d_out, r, d_out, s_g, 0, dB, r, nullptr, nullptr);
    const Red ra = red(f32(pl.off_p2a), pl.S2, d_in, r, d_in, s_x, 1, dA, d_in, nullptr, nullptr);
    launch_reduce(rb, want_da ? &ra : nullptr, s);
  }
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// U = X^ A^T formed with the forward product, V = G^ B with the dX product
// (melded_linear_fwd_xa / melded_linear_bwd_xa): the float factor enters the
// FP8 matrix cores as three E4M3 pieces per element with a power-of-two
// scale per rank and 32-element block, which the matrix core applies itself
// (pieces.hpp; the residual after three pieces is about 2^-12 of the element
// or less).  The GEMM then adds three MFMAs per K step in the four waves that
// hold the tile's unit (gemm_fp8_kernel.hpp, SecondB), and the dX product
// writes V straight as the pieces the token-contracting kernel reads.  No
// piece needs more than its own block, so forming them is one pass over the
// factor with every lane busy.  Shapes whose tile grid has too few columns
// for the units (gemm_fp8_nt_fuses_second) form U or V with the skinny
// kernel instead.
// ---------------------------------------------------------------------------
namespace {

// pieces of A [r x K] (K contiguous) for the forward product
constexpr int kPieceThreads = 256;

__global__ __launch_bounds__(kPieceThreads) void pieces_kernel(PieceJob q) {
  const int64_t gid = (int64_t)blockIdx.x * kPieceThreads + threadIdx.x;
  // the job's lanes come in whole waves
  if (gid < piece_job_lanes<true>(q.Rp, q.Kp)) piece_job_lane<true>(q, gid);
}

constexpr int kPrepThreads = 1024;    // four 128 x 128 transpose tiles per workgroup

int64_t prep_blocks(const PieceJob& q) {
  return q.P == nullptr ? 0 : (piece_job_lanes<false>(q.Rp, q.Kp) + kPrepThreads - 1) / kPrepThreads;
}

// The fused backward's preparation in one launch (each part alone is too
// small to fill the GPU): the first nb workgroups form the pieces of B^T
// (read from B [d_out x r]) for the dX product that also forms G^ B, the
// next nu those of U = X^ A^T (xa [T x r]) for the token-contracting dB, the
// rest transpose W~ for the dX product (128 x 128 tiles, tr_tx per tile row,
// four per workgroup).
__global__ __launch_bounds__(kPrepThreads) void xa_prep_kernel(const uint8_t* __restrict__ wq,
                                                               int64_t d_out, int64_t d_in,
                                                               uint8_t* __restrict__ wt, int n_tr,
                                                               int tr_tx, PieceJob jb, int nb,
                                                               PieceJob ju, int nu) {
  // the piece jobs take the first workgroup ids, so that they are dispatched
  // first and their latency overlaps the streaming transpose
  int b = blockIdx.x;
  if (b < nb + nu) {
    const bool is_b = b < nb;
    const PieceJob& q = is_b ? jb : ju;
    const int64_t gid = (int64_t)(is_b ? b : b - nb) * kPrepThreads + threadIdx.x;
    // a job's lanes come in whole waves
    if (gid < piece_job_lanes<false>(q.Rp, q.Kp)) piece_job_lane<false>(q, gid);
    return;
  }
  b -= nb + nu;
  const int tile = b * (kPrepThreads / 256) + (int)(threadIdx.x >> 8);
  if (tile < n_tr)
    transpose_u8_tile(wq, d_out, d_in, wt, tile % tr_tx, tile / tr_tx, (int)(threadIdx.x & 255));
}

// one skinny product Out [M x R] = dec(Q) F^T / s_q with F [R x K] float,
// split into bf16 hi/lo (row-wise Q, K contiguous in both)
struct OnePlan {
  int S, kc;
  size_t hi, lo, p, total;
};

OnePlan one_plan(int64_t M, int64_t K, int64_t R) {
  OnePlan p{};
  const int64_t tiles = (int64_t)ceil_div(M, TM) * ceil_div(R, TN);
  p.S = pick_splits(tiles, K, M * R * 4, 256ll << 20);
  p.kc = chunk_for(K, p.S);
  size_t o = 0;
  auto take = [&](size_t bytes) { size_t at = o; o = align_up(o + bytes, 256); return at; };
  p.hi = take((size_t)(R * K * 2));
  p.lo = take((size_t)(R * K * 2));
  p.p = take((size_t)p.S * M * R * 4);
  p.total = o;
  return p;
}

// F = A [R x K] (trans = false) or B^T with B [K x R] (trans = true)
hipError_t launch_one_skinny(const uint8_t* q, int64_t ldq, int qf, const float* s_q,
                             const float* F, bool trans, int64_t M, int64_t K, int64_t R,
                             float* out, void* ws, hipStream_t s) {
  const OnePlan pl = one_plan(M, K, R);
  uint8_t* base = reinterpret_cast<uint8_t*>(ws);
  uint16_t* hi = reinterpret_cast<uint16_t*>(base + pl.hi);
  uint16_t* lo = reinterpret_cast<uint16_t*>(base + pl.lo);
  float* part = reinterpret_cast<float*>(base + pl.p);
  const Split sp = trans ? Split{F, (int)K, (int)R, true, K, hi, lo, ceil_div(R, 32), ceil_div(K, 32)}
                         : Split{F, (int)R, (int)K, false, K, hi, lo, ceil_div(K, 32), ceil_div(R, 32)};
  split_bf16_kernel<<<dim3(sp.tx * sp.ty, 1, 1), 256, 0, s>>>(sp, sp);
  const Prob pr = prob(q, ldq, hi, lo, K, part, M, R, K, pl.kc);
  const int tiles = pr.tilesM * pr.tilesN;
  if (qf == 0)
    skinny_kernel<false, 2, 0, 0><<<tiles * pl.S, kSkThreads, 0, s>>>(pr, pr, tiles, pl.S);
  else
    skinny_kernel<false, 2, 1, 1><<<tiles * pl.S, kSkThreads, 0, s>>>(pr, pr, tiles, pl.S);
  launch_reduce(red(part, pl.S, M, R, M, s_q, 0, out, R, nullptr, nullptr), nullptr, s);
  return hipGetLastError();
}

// the token-contracting half from U, V [T x r] (fp32, fully scaled):
// U^T, V^T as bf16 hi/lo [r x Tp], then dB = G^^T U, dA = (X^^T V)^T
struct UvPlan {
  int64_t Tp;
  int S2, kc2;
  size_t uhi, ulo, vhi, vlo, p2b, p2a, total;
};

UvPlan uv_plan(int64_t T, int64_t d_in, int64_t d_out, int64_t r) {
  UvPlan p{};
  p.Tp = (T + TK - 1) / TK * TK;
  const int64_t nT = ceil_div(r, TN);
  const int64_t tiles2 = ((int64_t)ceil_div(d_in, TM) + ceil_div(d_out, TM)) * nT;
  p.S2 = pick_splits(tiles2, T, (d_in + d_out) * r * 4, 256ll << 20);
  p.kc2 = chunk_for(T, p.S2);
  size_t o = 0;
  auto take = [&](size_t bytes) { size_t at = o; o = align_up(o + bytes, 256); return at; };
  p.uhi = take((size_t)r * p.Tp * 2);
  p.ulo = take((size_t)r * p.Tp * 2);
  p.vhi = take((size_t)r * p.Tp * 2);
  p.vlo = take((size_t)r * p.Tp * 2);
  p.p2b = take((size_t)p.S2 * d_out * r * 4);
  p.p2a = take((size_t)p.S2 * d_in * r * 4);
  p.total = o;
  return p;
}

hipError_t launch_grads_from_uv(const uint8_t* gq, int g_fmt, const float* s_g, const uint8_t* xq,
                                const float* s_x, const float* u, const float* v, int64_t T,
                                int64_t d_in, int64_t d_out, int64_t r, float* dA, float* dB,
                                void* ws, hipStream_t s) {
  const UvPlan pl = uv_plan(T, d_in, d_out, r);
  uint8_t* base = reinterpret_cast<uint8_t*>(ws);
  auto u16 = [&](size_t off) { return reinterpret_cast<uint16_t*>(base + off); };
  auto f32 = [&](size_t off) { return reinterpret_cast<float*>(base + off); };
  const bool want_da = dA != nullptr;
  {
    const Red ru = red(u, 1, T, r, pl.Tp, nullptr, 2, nullptr, pl.Tp, u16(pl.uhi), u16(pl.ulo));
    const Red rv = red(v, 1, T, r, pl.Tp, nullptr, 2, nullptr, pl.Tp, u16(pl.vhi), u16(pl.vlo));
    launch_reduce(ru, want_da ? &rv : nullptr, s);
  }
  Prob pb = prob(gq, d_out, u16(pl.uhi), u16(pl.ulo), pl.Tp, f32(pl.p2b), d_out, r, T, pl.kc2);
  Prob pa = prob(xq, d_in, u16(pl.vhi), u16(pl.vlo), pl.Tp, f32(pl.p2a), d_in, r, T, pl.kc2);
  {
    const int tiles = std::max(pb.tilesM * pb.tilesN, want_da ? pa.tilesM * pa.tilesN : 0);
    const int grid = tiles * pl.S2 * (want_da ? 2 : 1);
    if (g_fmt == 0)
      skinny_kernel<true, 2, 0, 0><<<grid, kSkThreads, 0, s>>>(pb, pa, tiles, pl.S2);
    else
      skinny_kernel<true, 2, 1, 0><<<grid, kSkThreads, 0, s>>>(pb, pa, tiles, pl.S2);
  }
  {
    const Red rb = red(f32(pl.p2b), pl.S2, d_out, r, d_out, s_g, 0, dB, r, nullptr, nullptr);
    const Red ra = red(f32(pl.p2a), pl.S2, d_in, r, d_in, s_x, 1, dA, d_in, nullptr, nullptr);
    launch_reduce(rb, want_da ? &ra : nullptr, s);
  }
  return hipGetLastError();
}

// pieces of a float operand with R rows and K columns (K a multiple of
// 128): rows padded to 16
struct PiecesPlan {
  int64_t Rp;
  size_t p, e, total;
};
PiecesPlan pieces_plan(int64_t R, int64_t K) {
  PiecesPlan q{};
  q.Rp = (R + 15) / 16 * 16;
  size_t o = 0;
  auto take = [&](size_t bytes) { size_t at = o; o = align_up(o + bytes, 256); return at; };
  q.p = take((size_t)(3 * q.Rp * K));
  q.e = take((size_t)(K / 128 * q.Rp * 4));
  q.total = o;
  return q;
}

// the part of the backward's workspace that forms V (pieces of B^T for the
// fused product, or the skinny product's splits and partials)
size_t v_region_bytes(int64_t T, int64_t d_out, int64_t r) {
  return std::max(pieces_plan(r, d_out).total, one_plan(T, d_out, r).total);
}

}  // namespace

size_t fwd_xa_ws_bytes(int64_t T, int64_t d_in, int64_t d_out, int64_t r) {
  if (r <= 0 || T <= 0 || d_in <= 0) return 0;
  if (gemm_fp8_nt_fuses_second(d_out, d_in, r)) return pieces_plan(r, d_in).total;
  return one_plan(T, d_in, r).total;
}

hipError_t launch_fwd_xa(const uint8_t* xq, const float* s_x, const uint8_t* wq, const float* s_w,
                         const float* A, int64_t T, int64_t d_in, int64_t d_out, int64_t r,
                         float* y, float* xa, void* ws, hipStream_t s) {
  if (T == 0) return hipSuccess;
  if (d_in == 0) {
    hipError_t e = d_out > 0 ? launch_fill_f32(y, T * d_out, 0.0f, s) : hipSuccess;
    return e == hipSuccess && r > 0 ? launch_fill_f32(xa, T * r, 0.0f, s) : e;
  }
  if (r > 0 && gemm_fp8_nt_fuses_second(d_out, d_in, r)) {
    const PiecesPlan pp = pieces_plan(r, d_in);
    uint8_t* base = reinterpret_cast<uint8_t*>(ws);
    const PieceJob q{A, d_in, 1, r, d_in, base + pp.p, base + pp.e, pp.Rp, d_in};
    const int64_t blocks = (piece_job_lanes<true>(pp.Rp, d_in) + kPieceThreads - 1) / kPieceThreads;
    pieces_kernel<<<(unsigned)blocks, kPieceThreads, 0, s>>>(q);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    return launch_gemm_fp8_nt_pieces(xq, d_in, wq, d_in, y, d_out, T, d_out, d_in, s_x, s_w,
                                     base + pp.p, base + pp.e, pp.Rp, r, xa, r, nullptr, nullptr,
                                     0, 0, s, 0);
  }
  hipError_t e = d_out > 0 ? launch_gemm_fp8_nt(xq, d_in, wq, d_in, y, d_out, T, d_out, d_in, s_x,
                                                s_w, s)
                           : hipSuccess;
  if (e != hipSuccess || r == 0) return e;
  return launch_one_skinny(xq, d_in, 0, s_x, A, false, T, d_in, r, xa, ws, s);
}

// ---------------------------------------------------------------------------
// A's pieces kept by the optimizer: A changes only in the adapter step, so
// the step that moves A can leave the pieces the next forward needs, and the
// forward then launches no pieces kernel.
// ---------------------------------------------------------------------------
namespace {

// blocks [0, na): SGD on A and the pieces of the new A (8 lanes per 32-element
// block, four consecutive elements each); blocks [na, na + nb): SGD on B.
// The update is the same as sgd_kernel's, p - lr * g with two roundings.
__global__ __launch_bounds__(kPieceThreads) void sgd_pieces_kernel(
    float* __restrict__ A, const float* __restrict__ dA, int64_t r, int64_t d_in,
    float* __restrict__ B, const float* __restrict__ dB, int64_t nbv, float lr, PieceJob q,
    int64_t na) {
  const int64_t b = blockIdx.x;
  if (b < na) {
    const int64_t gid = b * kPieceThreads + threadIdx.x;
    // the job's lanes come in whole waves
    if (gid >= piece_job_lanes<true>(q.Rp, q.Kp)) return;
    int64_t j, c;
    int s, d, t;
    piece_lane_pos<true>(q.Rp, gid, j, c, s, d, t);
    float v[4] = {0.0f, 0.0f, 0.0f, 0.0f};
    if (j < r) {
      float4* pa = reinterpret_cast<float4*>(A + j * d_in + c * 128 + d);
      float4 a = *pa;
      const float4 g = *reinterpret_cast<const float4*>(dA + j * d_in + c * 128 + d);
      a.x = a.x - lr * g.x;
      a.y = a.y - lr * g.y;
      a.z = a.z - lr * g.z;
      a.w = a.w - lr * g.w;
      *pa = a;
      v[0] = a.x;
      v[1] = a.y;
      v[2] = a.z;
      v[3] = a.w;
    }
    piece_lane_store<true, 4>(v, q.P, q.E, q.Rp, q.Kp, j, c, s, d, t);
    return;
  }
  const int64_t i = (b - na) * kPieceThreads + threadIdx.x;
  if (i < nbv / 4) {
    float4 x = reinterpret_cast<float4*>(B)[i];
    const float4 g = reinterpret_cast<const float4*>(dB)[i];
    x.x = x.x - lr * g.x;
    x.y = x.y - lr * g.y;
    x.z = x.z - lr * g.z;
    x.w = x.w - lr * g.w;
    reinterpret_cast<float4*>(B)[i] = x;
  }
  if (b == na) {
    for (int64_t k = nbv / 4 * 4 + threadIdx.x; k < nbv; k += kPieceThreads) B[k] = B[k] - lr * dB[k];
  }
}

}  // namespace

bool adapter_pieces_ok(int64_t r, int64_t d_in) {
  return r > 0 && d_in > 0 && d_in % 128 == 0 && r <= ((int64_t)1 << 20) &&
         d_in <= ((int64_t)1 << 31);
}

size_t adapter_pieces_bytes(int64_t r, int64_t d_in) {
  return adapter_pieces_ok(r, d_in) ? pieces_plan(r, d_in).total : 0;
}

hipError_t launch_adapter_pieces(const float* A, int64_t r, int64_t d_in, void* pieces,
                                 hipStream_t s) {
  const PiecesPlan pp = pieces_plan(r, d_in);
  uint8_t* base = reinterpret_cast<uint8_t*>(pieces);
  const PieceJob q{A, d_in, 1, r, d_in, base + pp.p, base + pp.e, pp.Rp, d_in};
  const int64_t blocks = (piece_job_lanes<true>(pp.Rp, d_in) + kPieceThreads - 1) / kPieceThreads;
  pieces_kernel<<<(unsigned)blocks, kPieceThreads, 0, s>>>(q);
  return hipGetLastError();
}

hipError_t launch_sgd_pieces(float* A, float* B, const float* dA, const float* dB, int64_t r,
                             int64_t d_in, int64_t d_out, float lr, void* pieces, hipStream_t s) {
  const PiecesPlan pp = pieces_plan(r, d_in);
  uint8_t* base = reinterpret_cast<uint8_t*>(pieces);
  const PieceJob q{A, d_in, 1, r, d_in, base + pp.p, base + pp.e, pp.Rp, d_in};
  const int64_t na = (piece_job_lanes<true>(pp.Rp, d_in) + kPieceThreads - 1) / kPieceThreads;
  const int64_t nbv = d_out * r;
  const int64_t nb = std::max<int64_t>(1, (nbv / 4 + kPieceThreads - 1) / kPieceThreads);
  sgd_pieces_kernel<<<(unsigned)(na + nb), kPieceThreads, 0, s>>>(A, dA, r, d_in, B, dB, nbv, lr,
                                                                    q, na);
  return hipGetLastError();
}

hipError_t launch_fwd_xa_pieces(const uint8_t* xq, const float* s_x, const uint8_t* wq,
                                const float* s_w, const void* pieces, int64_t T, int64_t d_in,
                                int64_t d_out, int64_t r, float* y, float* xa, hipStream_t s) {
  if (T == 0) return hipSuccess;
  const PiecesPlan pp = pieces_plan(r, d_in);
  const uint8_t* base = reinterpret_cast<const uint8_t*>(pieces);
  return launch_gemm_fp8_nt_pieces(xq, d_in, wq, d_in, y, d_out, T, d_out, d_in, s_x, s_w,
                                   base + pp.p, base + pp.e, pp.Rp, r, xa, r, nullptr, nullptr, 0,
                                   0, s, 0);
}

// V = G^ B [T x r] (row-major), when no kernel writes it straight as pieces
size_t bwd_xa_ws_bytes(int64_t T, int64_t d_in, int64_t d_out, int64_t r) {
  if (r <= 0 || T <= 0 || d_in <= 0 || d_out <= 0) return 0;
  size_t o = align_up((size_t)r * (size_t)T * 4, 256);   // V
  o += v_region_bytes(T, d_out, r);
  return o + (token_grads_ok(T, d_in, d_out, r) ? token_grads_ws_bytes(T, d_in, d_out, r)
                                                : uv_plan(T, d_in, d_out, r).total);
}

hipError_t launch_bwd_xa(const uint8_t* gq, int g_fmt, const float* s_g, const uint8_t* xq,
                         const float* s_x, const uint8_t* wq, uint8_t* wt, const float* s_w,
                         const float* B, const float* xa, int64_t T, int64_t d_in, int64_t d_out,
                         int64_t r, float* dx, float* dA, float* dB, void* ws, hipStream_t s,
                         const uint8_t* wt_given) {
  uint8_t* base = reinterpret_cast<uint8_t*>(ws);
  float* v = reinterpret_cast<float*>(base);
  uint8_t* vreg = base + align_up((size_t)r * (size_t)T * 4, 256);
  uint8_t* rest = vreg + v_region_bytes(T, d_out, r);
  const bool want_v = dA != nullptr && r > 0;
  const bool tr = dx != nullptr && d_in > 0 && d_out > 0;
  // the dX product with V formed in the same tiles when both are wanted and
  // the grid allows; the token-contracting kernel when the shape allows
  const bool fuse = want_v && tr && gemm_fp8_nt_fuses_second(d_in, d_out, r);
  const bool tok = r > 0 && token_grads_ok(T, d_in, d_out, r);
  if (tr && (d_in % 16 != 0 || d_out % 16 != 0)) return hipErrorInvalidValue;
  const PiecesPlan pp = pieces_plan(r, d_out);
  PieceJob jb{}, ju{};
  if (fuse) jb = PieceJob{B, 1, r, r, d_out, vreg + pp.p, vreg + pp.e, pp.Rp, d_out};
  uint8_t *vp = nullptr, *ve = nullptr;
  int64_t tRp = 0, tTp = 0;
  if (tok) {
    uint8_t *up, *ue;
    token_grads_pieces(rest, T, d_in, d_out, r, 0, &up, &ue, &tRp, &tTp);
    token_grads_pieces(rest, T, d_in, d_out, r, 1, &vp, &ve, &tRp, &tTp);
    ju = PieceJob{xa, 1, r, r, T, up, ue, tRp, tTp};
  }
  const int nb = (int)prep_blocks(jb), nu = (int)prep_blocks(ju);
  const bool do_tr = tr && wt_given == nullptr;
  const uint8_t* wtb = wt_given ? wt_given : wt;        // the dX product's W~^T
  const int tr_tx = do_tr ? ceil_div(d_in, 128) : 1;
  const int n_tr = do_tr ? tr_tx * ceil_div(d_out, 128) : 0;
  const int grid = ceil_div(n_tr, kPrepThreads / 256) + nb + nu;
  if (grid > 0) {
    xa_prep_kernel<<<grid, kPrepThreads, 0, s>>>(wq, d_out, d_in, wt, n_tr, tr_tx, jb, nb, ju, nu);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  hipError_t e = hipSuccess;
  if (fuse) {
    // with the token-contracting kernel, V goes straight into its pieces
    e = launch_gemm_fp8_nt_pieces(gq, d_out, wtb, d_out, dx, d_in, T, d_in, d_out, s_g, s_w,
                                  vreg + pp.p, vreg + pp.e, pp.Rp, r, v, r, tok ? vp : nullptr,
                                  tok ? ve : nullptr, tRp, tTp, s, g_fmt);
  } else {
    if (tr) e = launch_gemm_fp8_nt(gq, d_out, wtb, d_out, dx, d_in, T, d_in, d_out, s_g, s_w, s,
                                   g_fmt);
    if (e == hipSuccess && want_v)
      e = launch_one_skinny(gq, d_out, g_fmt, s_g, B, true, T, d_out, r, v, vreg, s);
  }
  if (e != hipSuccess || r == 0) return e;
  if (tok)
    return launch_token_grads(gq, g_fmt, s_g, xq, s_x, xa, true, v, fuse, T, d_in, d_out, r, dA,
                              dB, rest, s);
  return launch_grads_from_uv(gq, g_fmt, s_g, xq, s_x, xa, v, T, d_in, d_out, r, dA, dB, rest, s);
}

}  // namespace falq
