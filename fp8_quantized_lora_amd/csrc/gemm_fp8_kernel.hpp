// FP8 GEMM kernel template (C = A . B^T, both operands K-contiguous) for
// gfx950; instantiated by gemm_fp8.hip.  See that file for the design notes.
#pragma once

#include "common.hpp"
#include "pieces.hpp"

namespace falq {
namespace gemm {

template <int BM_, int BN_, int BK_, int WGM_, int WGN_>
struct Cfg {
  static constexpr int BM = BM_, BN = BN_, BK = BK_, WGM = WGM_, WGN = WGN_;
  static constexpr int kThreads = WGM * WGN * 64;
  static constexpr int WTM = BM / WGM, WTN = BN / WGN;
  static constexpr int MB = WTM / 32, NB = WTN / 32;
  static constexpr int ROW = BK + 16;                    // padded LDS row (bytes)
  static constexpr int CPR = BK / 16;                    // 16-byte chunks per row
  static constexpr int A_CH = BM * CPR / kThreads;
  static constexpr int B_CH = BN * CPR / kThreads;
  static constexpr int LDS_BYTES = 2 * (BM + BN) * ROW;
  static_assert(BM * CPR % kThreads == 0 && BN * CPR % kThreads == 0, "tile/threads");
  static_assert(WTM % 32 == 0 && WTN % 32 == 0 && BK % 64 == 0, "mfma shape");
};

__device__ __forceinline__ v8i join(uint4 lo, uint4 hi) {
  v8i r;
  r[0] = lo.x; r[1] = lo.y; r[2] = lo.z; r[3] = lo.w;
  r[4] = hi.x; r[5] = hi.y; r[6] = hi.z; r[7] = hi.w;
  return r;
}

// Logical tile order: groups of G tile rows, column by column inside a group,
// so that a run of consecutive logical tiles shares few A rows and B columns.
__host__ __device__ __forceinline__ void tile_of(int logical, int tilesM, int tilesN, int& tm,
                                                 int& tn) {
  constexpr int G = 8;                                       // tile rows per group
  const int gsz = G * tilesN;
  const int g = logical / gsz;
  const int first = g * G;
  const int gm = min(tilesM - first, G);
  const int rem = logical - g * gsz;
  tm = first + rem % gm;
  tn = rem / gm;
}

// The dispatcher deals consecutive workgroup ids round-robin to the 8 XCDs;
// of the first n ids, each XCD gets a contiguous run of logical ids (ids past
// the last multiple of 8 keep their own).
__device__ __forceinline__ int xcd_remap(int bid, int n) {
  const int per = n / 8;
  return bid < per * 8 ? (bid % 8) * per + bid / 8 : bid;
}

__device__ __forceinline__ void tile_coords(int tilesM, int tilesN, int& tm, int& tn) {
  tile_of(xcd_remap(blockIdx.x, tilesM * tilesN), tilesM, tilesN, tm, tn);
}

// FA: format of the A codes (0 = E4M3, 1 = E5M2: the MFMA's A-format field);
// B is E4M3.  acc_c != 0 adds the product onto C.
template <class C, int FA>
__global__ __launch_bounds__(C::kThreads, 1) void gemm_fp8_nt_kernel(
    const uint8_t* __restrict__ A, int64_t lda, const uint8_t* __restrict__ B, int64_t ldb,
    float* __restrict__ Cm, int64_t ldc, int M, int N, int K, const float* __restrict__ sa,
    const float* __restrict__ sb, int tilesM, int tilesN, int acc_c) {
  __shared__ __attribute__((aligned(16))) uint8_t smem[C::LDS_BYTES];
  uint8_t* sA = smem;
  uint8_t* sB = smem + 2 * C::BM * C::ROW;

  int tm, tn;
  tile_coords(tilesM, tilesN, tm, tn);
  const int m0 = tm * C::BM, n0 = tn * C::BN;
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int wm = wid / C::WGN, wn = wid % C::WGN;

  v16f acc[C::MB][C::NB];
#pragma unroll
  for (int i = 0; i < C::MB; ++i)
#pragma unroll
    for (int j = 0; j < C::NB; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;

  uint4 ra[C::A_CH], rb[C::B_CH];
  auto gload = [&](int k0) {
#pragma unroll
    for (int i = 0; i < C::A_CH; ++i) {
      const int c = tid + i * C::kThreads;
      const int row = c / C::CPR, col = (c % C::CPR) * 16;
      const int gr = m0 + row, gk = k0 + col;
      const bool ok = gr < M && gk < K;
      // branch-free edge handling: read a valid address, zero the value
      uint4 v = *reinterpret_cast<const uint4*>(A + (int64_t)min(gr, M - 1) * lda + min(gk, K - 16));
      ra[i] = ok ? v : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < C::B_CH; ++i) {
      const int c = tid + i * C::kThreads;
      const int row = c / C::CPR, col = (c % C::CPR) * 16;
      const int gr = n0 + row, gk = k0 + col;
      const bool ok = gr < N && gk < K;
      uint4 v = *reinterpret_cast<const uint4*>(B + (int64_t)min(gr, N - 1) * ldb + min(gk, K - 16));
      rb[i] = ok ? v : make_uint4(0, 0, 0, 0);
    }
  };
  auto sstore = [&](int buf) {
    uint8_t* a = sA + buf * C::BM * C::ROW;
    uint8_t* b = sB + buf * C::BN * C::ROW;
#pragma unroll
    for (int i = 0; i < C::A_CH; ++i) {
      const int c = tid + i * C::kThreads;
      *reinterpret_cast<uint4*>(a + (c / C::CPR) * C::ROW + (c % C::CPR) * 16) = ra[i];
    }
#pragma unroll
    for (int i = 0; i < C::B_CH; ++i) {
      const int c = tid + i * C::kThreads;
      *reinterpret_cast<uint4*>(b + (c / C::CPR) * C::ROW + (c % C::CPR) * 16) = rb[i];
    }
  };

  const int nk = (K + C::BK - 1) / C::BK;
  if (nk > 0) {
    gload(0);
    sstore(0);
  }
  __syncthreads();
  const int a_off = (wm * C::WTM + (lane & 31)) * C::ROW + (lane >> 5) * 32;
  const int b_off = (wn * C::WTN + (lane & 31)) * C::ROW + (lane >> 5) * 32;
  for (int kt = 0; kt < nk; ++kt) {
    const int cur = kt & 1;
    if (kt + 1 < nk) gload((kt + 1) * C::BK);
    const uint8_t* a_base = sA + cur * C::BM * C::ROW + a_off;
    const uint8_t* b_base = sB + cur * C::BN * C::ROW + b_off;
#pragma unroll
    for (int kk = 0; kk < C::BK; kk += 64) {
      v8i af[C::MB], bf[C::NB];
#pragma unroll
      for (int i = 0; i < C::MB; ++i) {
        const uint8_t* p = a_base + i * 32 * C::ROW + kk;
        af[i] = join(*reinterpret_cast<const uint4*>(p), *reinterpret_cast<const uint4*>(p + 16));
      }
#pragma unroll
      for (int j = 0; j < C::NB; ++j) {
        const uint8_t* p = b_base + j * 32 * C::ROW + kk;
        bf[j] = join(*reinterpret_cast<const uint4*>(p), *reinterpret_cast<const uint4*>(p + 16));
      }
#pragma unroll
      for (int i = 0; i < C::MB; ++i)
#pragma unroll
        for (int j = 0; j < C::NB; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(af[i], bf[j], acc[i][j], FA,
                                                                      0, 0, 0, 0, 0);
    }
    if (kt + 1 < nk) sstore(cur ^ 1);
    __syncthreads();
  }

  const float scale = 1.0f / (sa[0] * sb[0]);
  const int rbase = m0 + wm * C::WTM + 4 * (lane >> 5);
  const int cbase = n0 + wn * C::WTN + (lane & 31);
#pragma unroll
  for (int i = 0; i < C::MB; ++i)
#pragma unroll
    for (int j = 0; j < C::NB; ++j) {
      const int col = cbase + j * 32;
      if (col >= N) continue;
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int row = rbase + i * 32 + 8 * (v >> 2) + (v & 3);
        if (row < M) {
          float* c = Cm + (int64_t)row * ldc + col;
          *c = acc_c ? *c + acc[i][j][v] * scale : acc[i][j][v] * scale;
        }
      }
    }
}


// ---------------------------------------------------------------------------
// Fast path for K a multiple of 128: direct-to-LDS loads and a two-stage LDS
// ring, v_mfma_f32_16x16x128_f8f6f4, 8 waves (2 per SIMD) on a 256 x 256
// tile.
//
//  * global_load_lds_dwordx4 moves 16 bytes per lane from global memory
//    straight into LDS (no staging registers, no LDS write instructions);
//    it is issued from inline asm so that the compiler does not serialise it
//    with a full vmcnt wait before every LDS read: completion is tracked with
//    explicit vmcnt waits, then a bare s_barrier.
//  * one DMA instruction fills 1 KB = 8 rows of 128 K-bytes; within a row the
//    16-byte chunk c is stored at slot c ^ swz(row), swz(r) = (r ^ (r >> 3)) & 7
//    over the row's index within its 16-row fragment.  Of the XOR swizzles
//    measured with the LDS bank-conflict counter on gfx950 this is one of the
//    two with no conflicts for the 16 x 16-byte fragment reads (the plain
//    (r >> 1) & 7 pattern costs an extra cycle per ds_read_b128).
//  * each wave owns a 128 x 64 sub-tile: 8 x 4 blocks of 16 x 16, four fp32
//    accumulators per lane per block.  A fragment lane l holds row l % 16 and
//    32 bytes at K offset 32 * (l / 16) of the 128-byte K step; B the same.
// ---------------------------------------------------------------------------
namespace dma {

constexpr int BM = 256, BN = 256, BK = 128, WGM = 2, WGN = 4, S = 2;
__device__ __forceinline__ int swz(int row) { return (row ^ ((row >> 3) & 1)) & 7; }
constexpr int NW = WGM * WGN, kThreads = NW * 64;
constexpr int WTM = BM / WGM, WTN = BN / WGN, MB = WTM / 16, NB = WTN / 16;
constexpr int UR = 16;                                  // rank rows of the second B operand
constexpr int STAGE = (BM + BN) * BK;
constexpr int MAX_NU = 3;                               // pieces of the second B operand
static_assert(S * (STAGE + MAX_NU * UR * BK + UR * 4) + 4 * UR * 4 <= 160 * 1024, "LDS");
constexpr int AI = BM * BK / 1024 / NW, BI = BN * BK / 1024 / NW;   // DMA instructions / wave / stage
constexpr int LPS = AI + BI;

// Optional second product against a small second B operand of NU E4M3
// "pieces" summed on the matrix cores: the frozen adapter factor A~ in the
// forward (NU = 1: U = dec(X~) dec(A~)^T / (sa * sb)), or a float operand
// held as NU = 3 E4M3 pieces with a power-of-two scale per row and 32-element
// K block (pieces.hpp), which the matrix core applies as the operand's E8M0
// block scale (the trained A in the forward, B^T in the dX product:
// C2 = dec(A) F^T / sa to within the pieces' residual, about 2^-12 of each
// element).  Its 16-rank blocks times 64-row quarters of a tile are "units";
// the tile in column tn < 4 * ceil(R / 16) takes unit tn: block tn / 4,
// quarter tn % 4.  The quarter's rows are held by the four waves of row group
// wm = quarter / 2, so each of them issues NU more MFMAs per K step (on its
// fragment i = (quarter % 2) * 4 + wn), NU per SIMD.  The unit's scale bytes
// of a K step (16 rows x 4 blocks, 64 contiguous bytes) ride in the LDS
// stage, loaded by wave 2 NU.
//
// The second product goes to C ([M x R] floats), or (P != nullptr) straight
// into pieces of its transpose for a later contraction over the M rows:
// rows m of C become the K positions of the pieces (P[p][j][m], scale bytes
// E[c][j][s]: pieces.hpp's layout with Rp = prp rows and Kp = pkp columns,
// zero codes for m >= M).  A block of 32 rows spans two waves of the row
// group (positions 16 wn .. 16 wn + 15 and 16 (wn ^ 2) .. of the quarter),
// which trade their row maxima through LDS.
struct SecondB {
  const uint8_t* B;      // piece 0: [R x K] codes, row stride ldb
  int64_t ldb;
  int64_t plane;         // bytes from one piece to the next
  int R;
  const uint8_t* be;     // NU = 3: scale bytes of B (rows padded to brp, a multiple of 16)
  int64_t brp;
  const float* sb;       // NU = 1: one scale for all of B
  float* C;              // [M x R] fp32 output, row stride ldc
  int64_t ldc;
  uint8_t* P;            // or pieces of C^T (rows: prp, multiple of 16; columns: pkp >= M,
  uint8_t* E;            // a multiple of 128) and their scale bytes
  int64_t prp, pkp;
};

// FA: format of the A codes (0 = E4M3, 1 = E5M2; B and the second B are
// E4M3), or 4: both operands FP4 E2M1, two codes per byte, or 5: both
// operands bfloat16 (K counts bytes throughout; bf16 takes no scales: sa and
// sb are ignored).  acc != 0 adds the product onto C instead of overwriting
// it (whole tiles only).
// MODE 0: workgroup b takes the whole logical tile xcd_remap(b, tiles)
// (tiles = the number of workgroups).  MODE 1: workgroups 2j and 2j + 1
// take the two K halves of logical tile first + j and add them into C with
// float atomics (C zeroed beforehand): exactly two addends meet a zero per
// element, and the sum of two floats does not depend on their order, so the
// result is the same on every run.  MODE 2 (split K, for outputs with too few
// tiles to fill the GPU): workgroup b takes tile b % tiles over K steps
// [s * acc_c, (s + 1) * acc_c), s = b / tiles, and writes its unscaled partial
// sums to plane s of C (planes of M * ldc floats); a reduction adds the
// planes in a fixed order.
template <int NU, int FA, int MODE = 0>
__global__ __launch_bounds__(kThreads, 1) void gemm_fp8_nt_dma(
    const uint8_t* __restrict__ A, int64_t lda, const uint8_t* __restrict__ B, int64_t ldb,
    float* __restrict__ C, int64_t ldc, int M, int N, int K, const float* __restrict__ sa,
    const float* __restrict__ sb, int tilesM, int tilesN, int tiles_or_first, SecondB u,
    int acc_c) {
  constexpr bool FU = NU > 0;
  static_assert(NU >= 0 && NU <= MAX_NU, "pieces");
  static_assert(!(FU && MODE != 0), "the second product is not split");
  constexpr bool HALF = MODE == 1;
  static_assert(FA != 5 || !FU, "no second product with bf16 operands");
  constexpr bool BS = NU == 3;                             // block-scaled pieces
  constexpr int SE = BS ? UR * 4 : 0;                      // their scale bytes per stage
  constexpr int SB = STAGE + NU * UR * BK + SE;            // bytes per LDS stage
  __shared__ __attribute__((aligned(1024))) uint8_t smem[S * SB];
  int tm, tn, k_lo = 0, nk = K / BK;
  if constexpr (HALF) {
    const int j = blockIdx.x, h = j & 1;
    tile_of(tiles_or_first + (j >> 1), tilesM, tilesN, tm, tn);
    k_lo = h ? nk / 2 : 0;
    nk = h ? nk - nk / 2 : nk / 2;
  } else if constexpr (MODE == 2) {
    const int b = blockIdx.x, sp = b / tiles_or_first;
    tile_of(b % tiles_or_first, tilesM, tilesN, tm, tn);
    k_lo = sp * acc_c;
    nk = min(nk - k_lo, acc_c);
    C += (int64_t)sp * M * ldc;
  } else {
    tile_of(xcd_remap(blockIdx.x, tiles_or_first), tilesM, tilesN, tm, tn);
  }
  const int m0 = tm * BM, n0 = tn * BN;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, wm = w / WGN, wn = w % WGN;
  // second product: this tile's unit (block ub, quarter uq), if any
  const bool has_u = FU && tn < 4 * ((u.R + UR - 1) / UR);
  const int ub = tn >> 2, uq = tn & 3;
  // wave-uniform (read from lane 0), so the extra MFMA sits behind a scalar branch
  const bool wave_u = __builtin_amdgcn_readfirstlane((int)(has_u && wm == (uq >> 1))) != 0;
  const int iu = __builtin_amdgcn_readfirstlane((uq & 1) * 4 + wn);   // the wave's fragment

  v4f acc[MB][NB];
#pragma unroll
  for (int i = 0; i < MB; ++i)
#pragma unroll
    for (int j = 0; j < NB; ++j)
#pragma unroll
      for (int v = 0; v < 4; ++v) acc[i][j][v] = 0.0f;

  // per-lane source of each DMA instruction: row (clamped into the matrix;
  // rows past M or N are computed and discarded) and the swizzled chunk
  const int lrow = lane >> 3, lslot = lane & 7;
  const uint8_t* gA[AI];
  const uint8_t* gB[BI];
#pragma unroll
  for (int j = 0; j < AI; ++j) {
    const int row = (w * AI + j) * 8 + lrow;
    gA[j] = A + (int64_t)min(m0 + row, M - 1) * lda + k_lo * BK + ((lslot ^ swz(row)) * 16);
  }
#pragma unroll
  for (int j = 0; j < BI; ++j) {
    const int row = (w * BI + j) * 8 + lrow;
    gB[j] = B + (int64_t)min(n0 + row, N - 1) * ldb + k_lo * BK + ((lslot ^ swz(row)) * 16);
  }
  // the 16 rank rows of the unit's block in each piece: waves 2p and 2p + 1
  // load 8 rows each of piece p
  const bool load_u = __builtin_amdgcn_readfirstlane((int)(has_u && w < 2 * NU)) != 0;
  const uint8_t* gU = nullptr;
  if (FU && load_u) {
    const int row = (w & 1) * 8 + lrow;
    gU = u.B + (int64_t)(w >> 1) * u.plane + (int64_t)min(ub * UR + row, u.R - 1) * u.ldb +
         k_lo * BK + ((lslot ^ swz(row)) * 16);
  }
  // the unit's scale bytes: four lanes of wave 2 NU, 16 bytes each
  const bool load_e = BS && __builtin_amdgcn_readfirstlane((int)(has_u && w == 2 * NU)) != 0;
  const uint8_t* gE = nullptr;
  if (BS && load_e) gE = u.be + (int64_t)(k_lo * u.brp + ub * UR) * 4 + (lane & 3) * 16;
  auto issue = [&](int stage, int k0) {
    const uint32_t base = lds_offset(smem + stage * SB);
    const uint32_t la = __builtin_amdgcn_readfirstlane(base + w * AI * 1024);
    const uint32_t lb = __builtin_amdgcn_readfirstlane(base + BM * BK + w * BI * 1024);
#pragma unroll
    for (int j = 0; j < AI; ++j) load16_to_lds(gA[j] + k0, la + j * 1024);
#pragma unroll
    for (int j = 0; j < BI; ++j) load16_to_lds(gB[j] + k0, lb + j * 1024);
    if (FU && load_u)
      load16_to_lds(gU + k0, __builtin_amdgcn_readfirstlane(base + (BM + BN) * BK + w * 1024));
    if (BS && load_e && lane < 4)
      load16_to_lds(gE + (int64_t)(k0 / BK) * u.brp * 4,
                    __builtin_amdgcn_readfirstlane(base + (BM + BN + NU * UR) * BK));
  };

#pragma unroll
  for (int s = 0; s < S - 1; ++s)
    if (s < nk) issue(s, s * BK);

  const int r16 = lane & 15, g = lane >> 4;
  const int sw = swz(r16);
  const int o0 = ((2 * g) ^ sw) * 16, o1 = ((2 * g + 1) ^ sw) * 16;
  const int offA = (wm * WTM + r16) * BK, offB = BM * BK + (wn * WTN + r16) * BK;
  // FP4 (FA == 4): a 128-byte row holds 256 values, two MFMA K-halves of
  // 128; lane group g reads its 16 bytes of each half (chunks g and g + 4),
  // joined so that the register layout matches the FP8 path.  bf16 (FA == 5):
  // a row holds 64 values, two K-halves of the 16 x 16 x 32 bf16 MFMA, whose
  // lane group g takes elements 8g .. 8g + 7 of its half: chunks g and g + 4
  // again.
  constexpr bool HALVES = FA == 4 || FA == 5;
  const int p0 = HALVES ? (g ^ sw) * 16 : o0, p1 = HALVES ? ((g + 4) ^ sw) * 16 : o1;
  auto frag = [&](const uint8_t* p) {
    return join(*reinterpret_cast<const uint4*>(p + p0), *reinterpret_cast<const uint4*>(p + p1));
  };
  // The product is formed transposed, D = B A^T per 16 x 16 block (the
  // MFMA's rows are C's columns), so that each lane ends with four
  // consecutive columns of one row of C: one 16-byte store per block.
  auto mma = [&](const v8i& a, const v8i& b, v4f c) {
    if constexpr (FA == 4) {
      const v8i alo = {a[0], a[1], a[2], a[3], 0, 0, 0, 0}, ahi = {a[4], a[5], a[6], a[7], 0, 0, 0, 0};
      const v8i blo = {b[0], b[1], b[2], b[3], 0, 0, 0, 0}, bhi = {b[4], b[5], b[6], b[7], 0, 0, 0, 0};
      c = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(blo, alo, c, 4, 4, 0, 0, 0, 0);
      return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(bhi, ahi, c, 4, 4, 0, 0, 0, 0);
    } else if constexpr (FA == 5) {
      const v4i alo = {a[0], a[1], a[2], a[3]}, ahi = {a[4], a[5], a[6], a[7]};
      const v4i blo = {b[0], b[1], b[2], b[3]}, bhi = {b[4], b[5], b[6], b[7]};
      c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(v8bf, blo),
                                                  __builtin_bit_cast(v8bf, alo), c, 0, 0, 0);
      return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(v8bf, bhi),
                                                     __builtin_bit_cast(v8bf, ahi), c, 0, 0, 0);
    } else {
      return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(b, a, c, 0, FA, 0, 0, 0, 0);
    }
  };
  // No scalar load may be pending when the loop starts: the compiler then
  // treats each step's LDS reads as returning in order and waits only for the
  // fragments the next MFMA needs.
  const float scale = (FA == 5 || MODE == 2) ? 1.0f : 1.0f / (sa[0] * sb[0]);
  const float scale_u = BS ? 1.0f / sa[0] : (FU ? 1.0f / (sa[0] * u.sb[0]) : 0.0f);
  v4f accu;
#pragma unroll
  for (int v = 0; v < 4; ++v) accu[v] = 0.0f;
  const int offU = (BM + BN) * BK + r16 * BK;
  // the lane's scale byte: row r16 of the unit, block g of the step
  const int offE = (BM + BN + NU * UR) * BK + r16 * 4 + g;
  __builtin_amdgcn_s_waitcnt(0xC07F);                        // lgkmcnt(0)
  for (int kt = 0; kt < nk; ++kt) {
    // stage kt has landed once at most (stages issued after it) * LPS loads are in flight
    wait_vmem(min(S - 2, nk - 1 - kt) * LPS);
    barrier_no_drain();
    const uint8_t* st = smem + (kt % S) * SB;
    // Fragment reads in the order the MFMAs consume them (A0, B0..B3, then
    // A(i+1) ahead of the MFMAs on A(i)); scheduling barriers keep the
    // compiler from reordering them, so the first MFMA waits for 4 reads,
    // not 12.
    v8i bf[NB], af[2], bu[NU > 0 ? NU : 1];
    af[0] = frag(st + offA);
#pragma unroll
    for (int j = 0; j < NB; ++j) {
      bf[j] = frag(st + offB + j * 16 * BK);
      __builtin_amdgcn_sched_barrier(0);
    }
    int eu = 127;
    if (FU && wave_u) {
#pragma unroll
      for (int p = 0; p < NU; ++p) bu[p] = frag(st + offU + p * UR * BK);
      if constexpr (BS) eu = st[offE];
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int i = 0; i < MB; ++i) {
      if (i + 1 < MB) af[(i + 1) & 1] = frag(st + offA + (i + 1) * 16 * BK);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int j = 0; j < NB; ++j) acc[i][j] = mma(af[i & 1], bf[j], acc[i][j]);
      if (FU && wave_u && __builtin_expect(i == iu, 0)) {
#pragma unroll
        for (int p = 0; p < NU; ++p) {
          if constexpr (BS)
            accu = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(af[i & 1], bu[p], accu, FA, 0,
                                                                    0, 127, 0, eu);
          else
            accu = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(af[i & 1], bu[p], accu, FA, 0,
                                                                    0, 0, 0, 0);
        }
      }
      __builtin_amdgcn_sched_barrier(0);
      // the next stage's direct loads go out once this step's first
      // fragments are in registers (an inline-asm load ahead of the first
      // reads makes the compiler wait for all twelve of them)
      if (i == 0 && kt + S - 1 < nk) issue((kt + S - 1) % S, (kt + S - 1) * BK);
      __builtin_amdgcn_sched_barrier(0);
    }
  }

  // lane l holds row r16 = l % 16 of each 16 x 16 block and its columns
  // 4 (l / 16) .. 4 (l / 16) + 3
  const int row0 = m0 + wm * WTM + r16;
  const int col0 = n0 + wn * WTN + 4 * g;
#pragma unroll
  for (int i = 0; i < MB; ++i) {
    const int row = row0 + i * 16;
    if (row >= M) continue;
    float* crow = C + (int64_t)row * ldc;
#pragma unroll
    for (int j = 0; j < NB; ++j) {
      const int col = col0 + j * 16;
      if (col >= N) continue;                 // N is a multiple of 16: all four or none
      v4f v = acc[i][j] * scale;
      if constexpr (HALF) {
#pragma unroll
        for (int e = 0; e < 4; ++e) unsafeAtomicAdd(crow + col + e, v[e]);
      } else {
        if (MODE == 0 && acc_c) v = *reinterpret_cast<const v4f*>(crow + col) + v;
        *reinterpret_cast<v4f*>(crow + col) = v;
      }
    }
  }
  if constexpr (FU) {
    const int rank = ub * UR + r16;
    const int urow0 = m0 + uq * 64 + wn * 16 + 4 * g;      // the lane's four rows
    v4f x = accu * scale_u;
    if (BS && has_u && u.P != nullptr) {
      // pieces of the transpose: the block of rows (quarter bit 6, wave bit 4)
      // spans this wave and wave wn ^ 2 of the row group
      __shared__ uint32_t xmax[4][UR];
      uint32_t mx = 0;
      if (wave_u) {
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          if (urow0 + v >= M) x[v] = 0.0f;
          mx = max(mx, finite_mag(x[v]));
        }
        mx = max(mx, (uint32_t)__shfl_xor((int)mx, 16, 64));
        mx = max(mx, (uint32_t)__shfl_xor((int)mx, 32, 64));
        if (g == 0) xmax[wn][r16] = mx;
      }
      __syncthreads();
      if (wave_u && urow0 < u.pkp) {
        mx = max(mx, xmax[wn ^ 2][r16]);
        const int e = piece_exp(__uint_as_float(mx));
        uint32_t q0, q1, q2;
        pieces4(ldexpf(x[0], e), ldexpf(x[1], e), ldexpf(x[2], e), ldexpf(x[3], e), q0, q1, q2);
        const int64_t plane = u.prp * u.pkp;
        uint8_t* p = u.P + (int64_t)rank * u.pkp + urow0;
        *reinterpret_cast<uint32_t*>(p) = q0;
        *reinterpret_cast<uint32_t*>(p + plane) = q1;
        *reinterpret_cast<uint32_t*>(p + 2 * plane) = q2;
        if (g == 0 && wn < 2) {
          const int64_t c = (m0 + uq * 64) / 128;
          u.E[(c * u.prp + rank) * 4 + 2 * (wn & 1) + (uq & 1)] = (uint8_t)(127 - e);
        }
      }
    } else if (wave_u && rank < u.R) {
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int row = urow0 + v;
        if (row < M) u.C[(int64_t)row * u.ldc + rank] = x[v];
      }
    }
  }
}

}  // namespace dma
}  // namespace gemm
}  // namespace falq
