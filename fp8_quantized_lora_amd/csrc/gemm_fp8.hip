// FP8 (OCP E4M3) GEMMs of the melded linear layer on gfx950 matrix cores.
//
// Forward  (FALQON introduction, method paragraph: one FP8 product, no LoRA
//          branch):      Y[T x d_out]  = X~ [T x d_in]  . W~[d_out x d_in]^T
// Backward dX:           dX[T x d_in]  = G~ [T x d_out] . W~[d_out x d_in]
//          (the dX path passes W~^T, built by launch_transpose_u8)
// Both are C = A . B^T with A and B K-contiguous ("NT"), fp32 accumulation,
// and the per-tensor scales folded into the epilogue: C *= 1 / (sa * sb).
//
// Two kernels.  K a multiple of 128 (every shape of the workloads) takes the
// direct-to-LDS kernel described in gemm_fp8_kernel.hpp (namespace dma).
// One 256 x 256 tile occupies a CU, so a tile count just past a multiple of
// the CU count leaves most CUs idle in the last round (4096 x 5120 outputs:
// 320 tiles, 64 in the second round of 256).  When the last round holds at
// most half the CUs and K is long, its tiles are split into two K halves,
// one workgroup each, in a second launch; the halves add into C (zeroed
// first by zero_tiles_kernel).
// Other K take the general kernel below:
//  * workgroup tile BM x BN x BK = 256 x 256 x 128 bytes, 4 waves in 2 x 2,
//    each wave a 128 x 128 sub-tile of 4 x 4 blocks of
//    v_mfma_f32_32x32x64_f8f6f4 (16 fp32 accumulators per lane per block);
//  * A and B tiles double-buffered in LDS (2 x 2 x 256 x 144 B = 144 KiB of
//    the 160 KiB per CU); rows padded to 144 B so that the 32 lanes reading
//    one fragment column hit distinct banks;
//  * the next K tile is loaded from global memory into registers before the
//    MFMAs of the current tile are issued, and written to the other LDS
//    buffer after them: one barrier per K step;
//  * tiles are ordered so that consecutive hardware workgroup ids, which the
//    dispatcher deals round-robin to the 8 XCDs, map to one compact block of
//    tiles per XCD (shared A rows / B columns stay in that XCD's L2).
//
// Operand layout in the MFMA: lane l of the A operand holds row (l % 32) and
// 32 consecutive K bytes starting at 32 * (l / 32) of the current 64-byte K
// slice; B is loaded the same way, so whatever order the matrix core pairs K
// elements in, both operands present the same K index in the same slot.
#include "common.hpp"
#include <algorithm>
#include <cstdint>
#include "gemm_fp8_kernel.hpp"
#include "kernels.hpp"
#include "transpose_u8.hpp"

namespace falq {
namespace {

// out[cols x rows] = in[rows x cols]^T for byte matrices whose sizes are
// multiples of 16: one 128 x 128 tile per workgroup (transpose_u8.hpp)
__global__ __launch_bounds__(256) void transpose_u8_kernel(const uint8_t* __restrict__ in,
                                                           int64_t rows, int64_t cols,
                                                           uint8_t* __restrict__ out) {
  transpose_u8_tile(in, rows, cols, out, (int)blockIdx.x, (int)blockIdx.y);
}

// zero the C blocks of logical tiles [first, first + count): block b clears
// 16 rows of tile first + b / 16, one 1 KB row segment per 256 threads
__global__ __launch_bounds__(256) void zero_tiles_kernel(float* __restrict__ C, int64_t ldc, int M,
                                                         int N, int tilesM, int tilesN, int first) {
  int tm, tn;
  gemm::tile_of(first + (int)blockIdx.x / 16, tilesM, tilesN, tm, tn);
  const int col = tn * gemm::dma::BN + (int)threadIdx.x;
  const int r0 = tm * gemm::dma::BM + ((int)blockIdx.x % 16) * 16;
  if (col >= N) return;
#pragma unroll 4
  for (int r = r0; r < r0 + 16 && r < M; ++r) C[(int64_t)r * ldc + col] = 0.0f;
}

// Number of workgroups that take whole tiles: all nt tiles, or, when the last
// round (nt mod CUs tiles) fills at most half the CUs and K has at least 64
// steps of 128, the tiles before that round.  With shorter K the zero fill
// and the atomic adds cost what the split saves (measured: 4096 x 5120 x 5120
// and 8192 x 11008 x 4096 take the same time either way; 4096 x 5120 x 13824
// 244 us split, 283 us whole).
int whole_tiles(int nt, int nk) {
  int dev = 0, ncu = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      ncu <= 0)
    return nt;
  const int rem = nt % ncu;
  if (rem == 0 || 2 * rem > ncu || nk < 64) return nt;
  return nt - rem;
}

// Tile columns for the fast kernel when an output's 256 x 256 tiles leave a
// short last round: the first c tile columns fill whole rounds of the CUs,
// and the remaining columns go to the generic kernel in 128 x 128 tiles
// (16 waves of 32 x 32, 256-byte K steps), which take about half of a large
// tile's time per round (4096 x 1024 x 5120: 33.8 us for 256 small tiles
// against 58.8 us for 64 large ones) — worth it when they fit in one round.  c >= min_cols keeps the tiles that carry a
// second product in the fast kernel.  0: no split.
int tail_split_cols(int64_t M, int64_t N, int min_cols) {
  int dev = 0, ncu = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      ncu <= 0)
    return 0;
  const int64_t tM = (M + gemm::dma::BM - 1) / gemm::dma::BM;
  const int64_t tN = (N + gemm::dma::BN - 1) / gemm::dma::BN;
  const int64_t nt = tM * tN, rounds = nt / ncu;
  if (rounds == 0 || nt % ncu == 0) return 0;
  const int64_t c = rounds * ncu / tM;
  if (c < std::max(min_cols, 1) || c >= tN) return 0;
  const int64_t nt_small = ((M + 127) / 128) * ((N - c * gemm::dma::BN + 127) / 128);
  return nt_small <= ncu ? (int)c : 0;
}

// the generic kernel in 128 x 128 tiles over output columns [n0, N) (lab,
// 4096 x 1024 x 5120: 4 waves and 128-byte K steps 44.7 us, 8 waves 41.4,
// 16 waves 39.0, 8 waves and 256-byte steps 36.3, 16 waves and 256-byte
// steps 33.8)
template <int FA>
hipError_t launch_tail(const uint8_t* A, int64_t lda, const uint8_t* B, int64_t ldb, float* C,
                       int64_t ldc, int64_t M, int64_t N, int64_t K, int64_t n0, const float* sa,
                       const float* sb, hipStream_t s) {
  using Cf = gemm::Cfg<128, 128, 256, 4, 4>;
  const int64_t Nt = N - n0;
  const int tilesM = (int)((M + Cf::BM - 1) / Cf::BM);
  const int tilesN = (int)((Nt + Cf::BN - 1) / Cf::BN);
  gemm::gemm_fp8_nt_kernel<Cf, FA><<<tilesM * tilesN, Cf::kThreads, 0, s>>>(
      A, lda, B + n0 * ldb, ldb, C + n0, ldc, (int)M, (int)Nt, (int)K, sa, sb, tilesM, tilesN, 0);
  return hipGetLastError();
}

// C (+)= scale * sum of the S partial planes P[s] (M x N, row stride ldp,
// plane stride M * ldp), added in plane order; scale = 1 / (sa * sb), or 1
// without scales
__global__ __launch_bounds__(256) void splitk_reduce_kernel(const float* __restrict__ P, int S,
                                                            int M, int N, int64_t ldp,
                                                            float* __restrict__ C, int64_t ldc,
                                                            const float* __restrict__ sa,
                                                            const float* __restrict__ sb,
                                                            int acc) {
  const float scale = sa ? 1.0f / (sa[0] * sb[0]) : 1.0f;
  const int64_t n4 = N / 4, total = (int64_t)M * n4;
  const int64_t plane = (int64_t)M * ldp;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total;
       i += (int64_t)gridDim.x * blockDim.x) {
    const int64_t m = i / n4, c = (i % n4) * 4;
    const float* p = P + m * ldp + c;
    v4f v = *reinterpret_cast<const v4f*>(p);
    for (int sp = 1; sp < S; ++sp) v = v + *reinterpret_cast<const v4f*>(p + sp * plane);
    v = v * scale;
    float* cp = C + m * ldc + c;
    if (acc) v = *reinterpret_cast<const v4f*>(cp) + v;
    *reinterpret_cast<v4f*>(cp) = v;
  }
}

// split-K plan of an output with nt tiles and nk K steps: the number of
// splits (1: none) so that about one workgroup per CU runs, each split at
// least 4 K steps
struct SplitK {
  int S, kc;
};
SplitK splitk_plan(int nt, int nk) {
  int S = 1;
  while (nt * S * 2 <= 256 && nk / (S * 2) >= 4) S *= 2;
  return {S, (nk + S - 1) / S};
}

}  // namespace

size_t gemm_splitk_ws_bytes(int64_t M, int64_t N, int64_t K_bytes) {
  if (M <= 0 || N <= 0 || K_bytes <= 0 || K_bytes % gemm::dma::BK != 0) return 0;
  const int nt = (int)(((M + gemm::dma::BM - 1) / gemm::dma::BM) *
                       ((N + gemm::dma::BN - 1) / gemm::dma::BN));
  const SplitK sk = splitk_plan(nt, (int)(K_bytes / gemm::dma::BK));
  if (sk.S == 1) return 0;
  return (size_t)sk.S * (size_t)M * (size_t)align_up((size_t)N, 4) * 4;
}

namespace {

// the direct-to-LDS kernel over tM x tN tiles, with the last round split, or
// (given a workspace of gemm_splitk_ws_bytes) split over K when the tiles
// alone would leave most CUs idle
template <int FA>
hipError_t launch_dma(const uint8_t* A, int64_t lda, const uint8_t* B, int64_t ldb, float* C,
                      int64_t ldc, int64_t M, int64_t N, int64_t K, const float* sa,
                      const float* sb, hipStream_t s, int acc = 0, float* splitk_ws = nullptr) {
  const int tM = (int)((M + gemm::dma::BM - 1) / gemm::dma::BM);
  const int tN = (int)((N + gemm::dma::BN - 1) / gemm::dma::BN);
  const int nt = tM * tN;
  if (splitk_ws) {
    const SplitK sk = splitk_plan(nt, (int)(K / gemm::dma::BK));
    if (sk.S > 1) {
      const int64_t ldp = (int64_t)align_up((size_t)N, 4);
      gemm::dma::gemm_fp8_nt_dma<0, FA, 2><<<nt * sk.S, gemm::dma::kThreads, 0, s>>>(
          A, lda, B, ldb, splitk_ws, ldp, (int)M, (int)N, (int)K, sa, sb, tM, tN, nt,
          gemm::dma::SecondB{}, sk.kc);
      hipError_t e = hipGetLastError();
      if (e != hipSuccess) return e;
      const int64_t items = M * (N / 4);
      const int blocks = (int)std::min<int64_t>((items + 255) / 256, 2048);
      splitk_reduce_kernel<<<blocks, 256, 0, s>>>(splitk_ws, sk.S, (int)M, (int)N, ldp, C, ldc,
                                                  FA == 5 ? nullptr : sa, sb, acc);
      return hipGetLastError();
    }
  }
  // an accumulating product keeps whole tiles (a split would add three terms)
  const int full = acc ? nt : whole_tiles(nt, (int)(K / gemm::dma::BK));
  if constexpr (FA == 0 || FA == 1) {
    // short K: the last round's columns as small tiles instead
    const int c = acc || full < nt ? 0 : tail_split_cols(M, N, 0);
    if (c > 0) {
      gemm::dma::gemm_fp8_nt_dma<0, FA><<<tM * c, gemm::dma::kThreads, 0, s>>>(
          A, lda, B, ldb, C, ldc, (int)M, c * gemm::dma::BN, (int)K, sa, sb, tM, c, tM * c,
          gemm::dma::SecondB{}, 0);
      const hipError_t e = hipGetLastError();
      if (e != hipSuccess) return e;
      return launch_tail<FA>(A, lda, B, ldb, C, ldc, M, N, K, (int64_t)c * gemm::dma::BN, sa, sb,
                             s);
    }
  }
  if (full < nt) {
    zero_tiles_kernel<<<(nt - full) * 16, 256, 0, s>>>(C, ldc, (int)M, (int)N, tM, tN, full);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (full > 0) {
    gemm::dma::gemm_fp8_nt_dma<0, FA><<<full, gemm::dma::kThreads, 0, s>>>(
        A, lda, B, ldb, C, ldc, (int)M, (int)N, (int)K, sa, sb, tM, tN, full,
        gemm::dma::SecondB{}, acc);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (full < nt)
    gemm::dma::gemm_fp8_nt_dma<0, FA, 1><<<2 * (nt - full), gemm::dma::kThreads, 0, s>>>(
        A, lda, B, ldb, C, ldc, (int)M, (int)N, (int)K, sa, sb, tM, tN, full,
        gemm::dma::SecondB{}, 0);
  return hipGetLastError();
}

}  // namespace

namespace {
template <int FA>
hipError_t gemm_nt(const uint8_t* A, int64_t lda, const uint8_t* B, int64_t ldb, float* C,
                   int64_t ldc, int64_t M, int64_t N, int64_t K, const float* sa, const float* sb,
                   hipStream_t s, int acc, float* splitk_ws) {
  if (K % gemm::dma::BK == 0)
    return launch_dma<FA>(A, lda, B, ldb, C, ldc, M, N, K, sa, sb, s, acc,
                          N % 4 == 0 ? splitk_ws : nullptr);
  using Cf = gemm::Cfg<256, 256, 128, 2, 2>;
  const int tilesM = (int)((M + Cf::BM - 1) / Cf::BM);
  const int tilesN = (int)((N + Cf::BN - 1) / Cf::BN);
  gemm::gemm_fp8_nt_kernel<Cf, FA><<<tilesM * tilesN, Cf::kThreads, 0, s>>>(
      A, lda, B, ldb, C, ldc, (int)M, (int)N, (int)K, sa, sb, tilesM, tilesN, acc);
  return hipGetLastError();
}
}  // namespace

// the kernels index tiles, rows and K with 32-bit ints and launch one
// workgroup per tile (or two per split tile) on a 1-D grid
static bool gemm_shape_ok(int64_t M, int64_t N, int64_t K) {
  const int64_t tiles = ((M + 255) / 256) * ((N + 255) / 256);
  return M <= INT32_MAX && N <= INT32_MAX && K <= INT32_MAX && 2 * tiles <= INT32_MAX;
}

hipError_t launch_gemm_fp8_nt(const uint8_t* A, int64_t lda, const uint8_t* B, int64_t ldb,
                              float* C, int64_t ldc, int64_t M, int64_t N, int64_t K,
                              const float* sa, const float* sb, hipStream_t s, int a_fmt,
                              int acc, float* splitk_ws) {
  if (M == 0 || N == 0) return hipSuccess;
  if (!gemm_shape_ok(M, N, K)) return hipErrorInvalidValue;
  return a_fmt == 0 ? gemm_nt<0>(A, lda, B, ldb, C, ldc, M, N, K, sa, sb, s, acc, splitk_ws)
                    : gemm_nt<1>(A, lda, B, ldb, C, ldc, M, N, K, sa, sb, s, acc, splitk_ws);
}

hipError_t launch_gemm_bf16_nt(const uint16_t* A, int64_t lda, const uint16_t* B, int64_t ldb,
                               float* C, int64_t ldc, int64_t M, int64_t N, int64_t K,
                               hipStream_t s, int acc, float* splitk_ws) {
  if (M == 0 || N == 0) return hipSuccess;
  // the direct-to-LDS kernel over K in bytes: 64 bf16 per 128-byte step
  if (K <= 0 || K % 64 != 0 || !gemm_shape_ok(M, N, 2 * K)) return hipErrorInvalidValue;
  return launch_dma<5>(reinterpret_cast<const uint8_t*>(A), 2 * lda,
                       reinterpret_cast<const uint8_t*>(B), 2 * ldb, C, ldc, M, N, 2 * K, nullptr,
                       nullptr, s, acc, N % 4 == 0 ? splitk_ws : nullptr);
}

hipError_t launch_gemm_fp4_nt(const uint8_t* A, int64_t lda, const uint8_t* B, int64_t ldb,
                              float* C, int64_t ldc, int64_t M, int64_t N, int64_t Kb,
                              const float* sa, const float* sb, hipStream_t s) {
  if (M == 0 || N == 0) return hipSuccess;
  if (Kb <= 0 || Kb % gemm::dma::BK != 0 || !gemm_shape_ok(M, N, Kb)) return hipErrorInvalidValue;
  return launch_dma<4>(A, lda, B, ldb, C, ldc, M, N, Kb, sa, sb, s);
}

bool gemm_fp8_nt_fuses_second(int64_t N, int64_t K, int64_t R) {
  if (R <= 0 || K <= 0 || K % gemm::dma::BK != 0) return false;
  const int64_t tN = (N + gemm::dma::BN - 1) / gemm::dma::BN;
  return 4 * ((R + gemm::dma::UR - 1) / gemm::dma::UR) <= tN;
}

hipError_t launch_gemm_fp8_nt_second(const uint8_t* A, int64_t lda, const uint8_t* B, int64_t ldb,
                                     float* C, int64_t ldc, int64_t M, int64_t N, int64_t K,
                                     const float* sa, const float* sb, const uint8_t* Bu,
                                     int64_t ldbu, int64_t R, float* Cu, int64_t ldcu,
                                     const float* sbu, hipStream_t s) {
  if (M == 0) return hipSuccess;
  if (!gemm_fp8_nt_fuses_second(N, K, R) || !gemm_shape_ok(M, N, K)) return hipErrorInvalidValue;
  const int tM = (int)((M + gemm::dma::BM - 1) / gemm::dma::BM);
  // the tile columns past the ones that carry the second product may go to
  // the small-tile kernel (tail_split_cols)
  const int c = tail_split_cols(M, N, 4 * (int)((R + gemm::dma::UR - 1) / gemm::dma::UR));
  const int tN = c > 0 ? c : (int)((N + gemm::dma::BN - 1) / gemm::dma::BN);
  const int64_t Nm = c > 0 ? (int64_t)c * gemm::dma::BN : N;
  gemm::dma::gemm_fp8_nt_dma<1, 0><<<tM * tN, gemm::dma::kThreads, 0, s>>>(
      A, lda, B, ldb, C, ldc, (int)M, (int)Nm, (int)K, sa, sb, tM, tN, tM * tN,
      gemm::dma::SecondB{Bu, ldbu, 0, (int)R, nullptr, 0, sbu, Cu, ldcu, nullptr, nullptr, 0, 0},
      0);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess || c == 0) return e;
  return launch_tail<0>(A, lda, B, ldb, C, ldc, M, N, K, Nm, sa, sb, s);
}

hipError_t launch_gemm_fp8_nt_pieces(const uint8_t* A, int64_t lda, const uint8_t* B,
                                     int64_t ldb, float* C, int64_t ldc, int64_t M, int64_t N,
                                     int64_t K, const float* sa, const float* sb,
                                     const uint8_t* P, const uint8_t* PE, int64_t prp, int64_t R,
                                     float* Cu, int64_t ldcu, uint8_t* Po, uint8_t* Eo,
                                     int64_t po_rp, int64_t po_kp, hipStream_t s, int a_fmt) {
  if (M == 0) return hipSuccess;
  if (!gemm_fp8_nt_fuses_second(N, K, R) || !gemm_shape_ok(M, N, K)) return hipErrorInvalidValue;
  const int64_t r16 = (R + gemm::dma::UR - 1) / gemm::dma::UR * gemm::dma::UR;
  if (prp < r16 || prp % 16 != 0) return hipErrorInvalidValue;
  if (Po != nullptr && (po_rp < r16 || po_rp % 16 != 0 || po_kp < M || po_kp % 128 != 0))
    return hipErrorInvalidValue;
  const int tM = (int)((M + gemm::dma::BM - 1) / gemm::dma::BM);
  // the tile columns past the ones that carry the pieces' product may go to
  // the small-tile kernel (tail_split_cols)
  const int c = tail_split_cols(M, N, (int)(4 * (r16 / gemm::dma::UR)));
  const int tN = c > 0 ? c : (int)((N + gemm::dma::BN - 1) / gemm::dma::BN);
  const int64_t Nm = c > 0 ? (int64_t)c * gemm::dma::BN : N;
  const gemm::dma::SecondB u{P,  K,  prp * K, (int)R, PE,    prp,   nullptr,
                             Cu, ldcu, Po,    Eo,     po_rp, po_kp};
  if (a_fmt == 0)
    gemm::dma::gemm_fp8_nt_dma<3, 0><<<tM * tN, gemm::dma::kThreads, 0, s>>>(
        A, lda, B, ldb, C, ldc, (int)M, (int)Nm, (int)K, sa, sb, tM, tN, tM * tN, u, 0);
  else
    gemm::dma::gemm_fp8_nt_dma<3, 1><<<tM * tN, gemm::dma::kThreads, 0, s>>>(
        A, lda, B, ldb, C, ldc, (int)M, (int)Nm, (int)K, sa, sb, tM, tN, tM * tN, u, 0);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess || c == 0) return e;
  return a_fmt == 0 ? launch_tail<0>(A, lda, B, ldb, C, ldc, M, N, K, Nm, sa, sb, s)
                    : launch_tail<1>(A, lda, B, ldb, C, ldc, M, N, K, Nm, sa, sb, s);
}

hipError_t launch_transpose_u8(const uint8_t* in, int64_t rows, int64_t cols, uint8_t* out,
                               hipStream_t s) {
  if (rows == 0 || cols == 0) return hipSuccess;
  if (rows % 16 != 0 || cols % 16 != 0) return hipErrorInvalidValue;
  dim3 grid((unsigned)((cols + 127) / 128), (unsigned)((rows + 127) / 128));
  transpose_u8_kernel<<<grid, 256, 0, s>>>(in, rows, cols, out);
  return hipGetLastError();
}

}  // namespace falq
