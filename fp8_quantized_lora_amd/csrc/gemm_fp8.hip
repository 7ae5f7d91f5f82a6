// FP8 (OCP E4M3) GEMMs of the melded linear layer on gfx950 matrix cores.
//
// Forward  (FALQON introduction, method paragraph: one FP8 product, no LoRA
//          branch):      Y[T x d_out]  = X~ [T x d_in]  . W~[d_out x d_in]^T
// Backward dX:           dX[T x d_in]  = G~ [T x d_out] . W~[d_out x d_in]
//          (the dX path passes W~^T, built by launch_transpose_u8)
// Both are C = A . B^T with A and B K-contiguous ("NT"), fp32 accumulation,
// and the per-tensor scales folded into the epilogue: C *= 1 / (sa * sb).
//
// Kernel shape (CDNA4):
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
#include "kernels.hpp"

namespace falq {
namespace {

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

using Big = Cfg<256, 256, 128, 2, 2>;

__device__ __forceinline__ v8i join(uint4 lo, uint4 hi) {
  v8i r;
  r[0] = lo.x; r[1] = lo.y; r[2] = lo.z; r[3] = lo.w;
  r[4] = hi.x; r[5] = hi.y; r[6] = hi.z; r[7] = hi.w;
  return r;
}

__device__ __forceinline__ void tile_coords(int tilesM, int tilesN, int& tm, int& tn) {
  const int nt = tilesM * tilesN;
  const int bid = blockIdx.x;
  const int per = nt / 8;
  int logical = bid;
  if (bid < per * 8) logical = (bid % 8) * per + bid / 8;   // 8 XCDs, round-robin dispatch
  constexpr int G = 8;                                       // tile rows per group
  const int gsz = G * tilesN;
  const int g = logical / gsz;
  const int first = g * G;
  const int gm = min(tilesM - first, G);
  const int rem = logical - g * gsz;
  tm = first + rem % gm;
  tn = rem / gm;
}

template <class C>
__global__ __launch_bounds__(C::kThreads, 1) void gemm_fp8_nt_kernel(
    const uint8_t* __restrict__ A, int64_t lda, const uint8_t* __restrict__ B, int64_t ldb,
    float* __restrict__ Cm, int64_t ldc, int M, int N, int K, const float* __restrict__ sa,
    const float* __restrict__ sb, int tilesM, int tilesN) {
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
          acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(af[i], bf[j], acc[i][j], 0, 0,
                                                                      0, 0, 0, 0);
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
        if (row < M) Cm[(int64_t)row * ldc + col] = acc[i][j][v] * scale;
      }
    }
}

// in [rows x cols] -> out [cols x rows], bytes; rows and cols multiples of 16
__global__ __launch_bounds__(256) void transpose_u8_kernel(const uint8_t* __restrict__ in,
                                                           int64_t rows, int64_t cols,
                                                           uint8_t* __restrict__ out) {
  __shared__ uint8_t t[64][64 + 4];
  const int64_t r0 = (int64_t)blockIdx.y * 64, c0 = (int64_t)blockIdx.x * 64;
  const int tid = threadIdx.x;
  {
    const int rr = tid >> 2, cc = (tid & 3) * 16;
    uint4 v = make_uint4(0, 0, 0, 0);
    if (r0 + rr < rows && c0 + cc < cols)
      v = *reinterpret_cast<const uint4*>(in + (r0 + rr) * cols + c0 + cc);
    uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int b = 0; b < 16; ++b) t[rr][cc + b] = (uint8_t)(w[b >> 2] >> (8 * (b & 3)));
  }
  __syncthreads();
  {
    const int oc = tid >> 2, orr = (tid & 3) * 16;  // output row = input column
    if (c0 + oc < cols && r0 + orr < rows) {
      uint32_t w[4] = {0, 0, 0, 0};
#pragma unroll
      for (int b = 0; b < 16; ++b) w[b >> 2] |= (uint32_t)t[orr + b][oc] << (8 * (b & 3));
      *reinterpret_cast<uint4*>(out + (c0 + oc) * rows + r0 + orr) = make_uint4(w[0], w[1], w[2], w[3]);
    }
  }
}

}  // namespace

hipError_t launch_gemm_fp8_nt(const uint8_t* A, int64_t lda, const uint8_t* B, int64_t ldb,
                              float* C, int64_t ldc, int64_t M, int64_t N, int64_t K,
                              const float* sa, const float* sb, hipStream_t s) {
  if (M == 0 || N == 0) return hipSuccess;
  using Cf = Big;
  const int tilesM = (int)((M + Cf::BM - 1) / Cf::BM);
  const int tilesN = (int)((N + Cf::BN - 1) / Cf::BN);
  gemm_fp8_nt_kernel<Cf><<<tilesM * tilesN, Cf::kThreads, 0, s>>>(
      A, lda, B, ldb, C, ldc, (int)M, (int)N, (int)K, sa, sb, tilesM, tilesN);
  return hipGetLastError();
}

hipError_t launch_transpose_u8(const uint8_t* in, int64_t rows, int64_t cols, uint8_t* out,
                               hipStream_t s) {
  if (rows == 0 || cols == 0) return hipSuccess;
  dim3 grid((unsigned)((cols + 63) / 64), (unsigned)((rows + 63) / 64));
  transpose_u8_kernel<<<grid, 256, 0, s>>>(in, rows, cols, out);
  return hipGetLastError();
}

}  // namespace falq
