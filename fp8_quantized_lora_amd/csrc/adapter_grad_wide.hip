// Rank-r adapter gradients for large r (the rank-sweep workload's 2048 and
// 8192): the grouping of the FALQON rebuttal (thread 4, reply Q1), where
// dL/dA = B^T (dL/dO) x^T, i.e. through the full weight gradient
//     M  = G^^T X^                 [d_out x d_in]   one FP8 product, K = T
//     dB = M A^T                   [d_out x r]      = G^^T (X^ A^T)
//     dA = B^T M                   [r x d_in]       = (G^ B)^T X^
// The sums are the same as the skinny kernels' (adapter_grad.hip); only the
// order of the two contractions differs.  Cost: 2 d_in d_out T FP8 flops for
// M, then 2 d_in d_out r per gradient, against 4 T r (d_in + d_out) for the
// skinny route; with T = 2 d and r in the thousands this is several times
// less work, and every product is a full-size GEMM.
//
// M comes out of the FP8 GEMM in float32 (G~^T and X~^T, transposed copies
// of the codes, are the K-contiguous operands); dB and dA run on the bf16
// matrix cores with both float operands split as hi + lo bfloat16 (hi =
// bf(v), lo = bf(v - hi)) and the three significant cross products
// hi*hi + hi*lo + lo*hi formed as ONE product over a K three times as long:
//     [M_hi | M_hi | M_lo] . [A_hi | A_lo | A_hi]^T
// (relative error about 2^-16 per product; the dropped lo*lo term is below
// 2^-16 too).
#include "common.hpp"
#include "kernels.hpp"

#include <algorithm>

namespace falq {
namespace {

__device__ __forceinline__ uint16_t bf16_nearest(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

constexpr int WT = 64;     // tile side

// dst [out_rows x 3 out_cols] bfloat16 (row stride 3 out_cols): segment s of
// row i holds the hi (plane bit 0) or lo (bit 1) half of v(i, c), where
// v(i, c) = src[i][c] or, with trans, src[c][i]; src is float32 [rows x cols]
// with row stride lds.  out_rows x out_cols = rows x cols, or cols x rows.
__global__ __launch_bounds__(256) void split_cat_kernel(const float* __restrict__ src, int64_t rows,
                                                        int64_t cols, int64_t lds,
                                                        uint16_t* __restrict__ dst, int trans,
                                                        int planes) {
  __shared__ float t[WT][WT + 1];
  const int64_t out_rows = trans ? cols : rows, out_cols = trans ? rows : cols;
  const int64_t o_r0 = (int64_t)blockIdx.y * WT, o_c0 = (int64_t)blockIdx.x * WT;
  const int64_t s_r0 = trans ? o_c0 : o_r0, s_c0 = trans ? o_r0 : o_c0;
  for (int e = threadIdx.x; e < WT * WT; e += 256) {
    const int r = e / WT, c = e % WT;
    const int64_t sr = s_r0 + r, sc = s_c0 + c;
    t[r][c] = (sr < rows && sc < cols) ? src[sr * lds + sc] : 0.0f;
  }
  __syncthreads();
  const int64_t ldd = 3 * out_cols;
  for (int e = threadIdx.x; e < WT * WT; e += 256) {
    const int r = e / WT, c = e % WT;
    const int64_t orr = o_r0 + r, oc = o_c0 + c;
    if (orr >= out_rows || oc >= out_cols) continue;
    const float v = trans ? t[c][r] : t[r][c];
    const uint16_t hi = bf16_nearest(v);
    const uint16_t lo = bf16_nearest(v - __uint_as_float((uint32_t)hi << 16));
    uint16_t* d = dst + orr * ldd + oc;
#pragma unroll
    for (int sgm = 0; sgm < 3; ++sgm) d[sgm * out_cols] = ((planes >> sgm) & 1) ? lo : hi;
  }
}

hipError_t split_cat(const float* src, int64_t rows, int64_t cols, int64_t lds, uint16_t* dst,
                     bool trans, int planes, hipStream_t s) {
  const int64_t out_rows = trans ? cols : rows, out_cols = trans ? rows : cols;
  if (out_rows == 0 || out_cols == 0) return hipSuccess;
  dim3 grid((unsigned)((out_cols + WT - 1) / WT), (unsigned)((out_rows + WT - 1) / WT));
  split_cat_kernel<<<grid, 256, 0, s>>>(src, rows, cols, lds, dst, trans ? 1 : 0, planes);
  return hipGetLastError();
}

constexpr int kHiHiLo = 0b100, kHiLoHi = 0b010;   // plane of each K segment (bit set: lo)

struct WidePlan {
  size_t gt, xt, m, mcat, mtcat, acat, btcat, sk, total;
};

WidePlan wide_plan(int64_t T, int64_t d_in, int64_t d_out, int64_t r) {
  WidePlan p{};
  size_t o = 0;
  auto take = [&](size_t bytes) { size_t at = o; o = align_up(o + bytes, 256); return at; };
  p.gt = take((size_t)(d_out * T));                    // G~^T
  p.xt = take((size_t)(d_in * T));                     // X~^T
  p.m = take((size_t)(d_out * d_in * 4));              // M (fp32)
  p.mcat = take((size_t)(d_out * 3 * d_in * 2));       // [M_hi | M_hi | M_lo]
  p.mtcat = take((size_t)(d_in * 3 * d_out * 2));      // [Mt_hi | Mt_hi | Mt_lo]
  p.acat = take((size_t)(r * 3 * d_in * 2));           // [A_hi | A_lo | A_hi]
  p.btcat = take((size_t)(r * 3 * d_out * 2));         // [Bt_hi | Bt_lo | Bt_hi]
  size_t sk = gemm_splitk_ws_bytes(d_out, d_in, T);
  sk = std::max(sk, gemm_splitk_ws_bytes(d_out, r, 2 * 3 * d_in));
  sk = std::max(sk, gemm_splitk_ws_bytes(r, d_in, 2 * 3 * d_out));
  p.sk = take(sk);
  p.total = o;
  return p;
}

}  // namespace

bool adapter_wide_route(int64_t T, int64_t d_in, int64_t d_out, int64_t r) {
  if (r <= 0 || r % 4 != 0 || T <= 0 || T % 16 != 0 || d_in % 64 != 0 || d_out % 64 != 0 ||
      d_in <= 0 || d_out <= 0)
    return false;
  // bf16-equivalent work: the skinny route's four products with the hi/lo
  // split, against M at the FP8 rate (half) plus the two 3-segment products
  const double skinny = 8.0 * (double)T * (double)r * (double)(d_in + d_out);
  const double wide = (double)d_in * (double)d_out * ((double)T + 12.0 * (double)r);
  return skinny > 1.5 * wide;
}

size_t adapter_wide_ws_bytes(int64_t T, int64_t d_in, int64_t d_out, int64_t r) {
  return wide_plan(T, d_in, d_out, r).total;
}

hipError_t launch_adapter_grads_wide(const uint8_t* gq, int g_fmt, const float* s_g,
                                     const uint8_t* xq, const float* s_x, const float* A,
                                     const float* B, int64_t T, int64_t d_in, int64_t d_out,
                                     int64_t r, float* dA, float* dB, void* ws, hipStream_t s) {
  const WidePlan p = wide_plan(T, d_in, d_out, r);
  uint8_t* base = reinterpret_cast<uint8_t*>(ws);
  auto b16 = [&](size_t off) { return reinterpret_cast<uint16_t*>(base + off); };
  float* sk = reinterpret_cast<float*>(base + p.sk);
  float* m = reinterpret_cast<float*>(base + p.m);
  hipError_t e = launch_transpose_u8(gq, T, d_out, base + p.gt, s);
  if (e == hipSuccess) e = launch_transpose_u8(xq, T, d_in, base + p.xt, s);
  // M = G^^T X^ [d_out x d_in]
  if (e == hipSuccess)
    e = launch_gemm_fp8_nt(base + p.gt, T, base + p.xt, T, m, d_in, d_out, d_in, T, s_g, s_x, s,
                           g_fmt, 0, sk);
  // dB = M A^T
  if (e == hipSuccess) e = split_cat(m, d_out, d_in, d_in, b16(p.mcat), false, kHiHiLo, s);
  if (e == hipSuccess) e = split_cat(A, r, d_in, d_in, b16(p.acat), false, kHiLoHi, s);
  if (e == hipSuccess)
    e = launch_gemm_bf16_nt(b16(p.mcat), 3 * d_in, b16(p.acat), 3 * d_in, dB, r, d_out, r,
                            3 * d_in, s, 0, sk);
  if (e != hipSuccess || dA == nullptr) return e;
  // dA = B^T M, as NT against M^T
  e = split_cat(m, d_out, d_in, d_in, b16(p.mtcat), true, kHiHiLo, s);
  if (e == hipSuccess) e = split_cat(B, d_out, r, r, b16(p.btcat), true, kHiLoHi, s);
  if (e == hipSuccess)
    e = launch_gemm_bf16_nt(b16(p.btcat), 3 * d_out, b16(p.mtcat), 3 * d_out, dA, d_in, r, d_in,
                            3 * d_out, s, 0, sk);
  return e;
}

}  // namespace falq
