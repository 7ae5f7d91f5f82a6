// The two LoRA layers the melded layer is measured against (FALQON abstract
// and introduction: the method removes the quantization overhead of a
// separate LoRA computational path; OpenReview rebuttal, thread 1, Q2 and
// Table R1: FP8 against FP16 LoRA adapter compute, with the turning point
// near rank 8192).  Both keep the FP8 backbone product of the melded layer
// and add the adapter as a separate branch, built from this library's own
// kernels:
//
//  * separate-path FP8 LoRA: the adapter factors and the rank-r
//    intermediates are quantized per tensor to E4M3 on every step, and every
//    product runs on the FP8 matrix cores:
//        A~ = Q(A), B~ = Q(B), U = X^ A^^T, U~ = Q(U), Y = X^ W^^T + U^ B^^T
//        V = G^ B^, V~ = Q(V), dX = G^ W^ + V^ A^, dB = G^^T U^, dA = V^^T X^
//    (^ = the dequantized value: code / scale);
//  * BF16 LoRA: the adapter branch in bfloat16 with fp32 accumulation,
//    from the unquantized X and dY:
//        U = bf(X) bf(A)^T, Y = X^ W^^T + bf(U) bf(B)^T
//        V = bf(dY) bf(B), dX = G^ W^ + bf(V) bf(A), dB = bf(dY)^T bf(U),
//        dA = bf(V)^T bf(X)
//    (bf = round to nearest even bfloat16).
// Every product is C = A B^T on the direct-to-LDS GEMM (K-contiguous
// operands: the T-contracting products take transposed copies) or, for K
// not a multiple of 128 bytes, the register-staged FP8 GEMM; rank-r outputs
// that leave most CUs idle run split over K.  Operands whose rank dimension is
// the contraction are zero-padded to a multiple of 16 (FP8) or 64 (bf16)
// ranks in the workspace.
#include "common.hpp"
#include "kernels.hpp"

#include <algorithm>

namespace falq {
namespace {

constexpr int CT = 64;                      // conversion tile (elements per side)

__device__ __forceinline__ float ld_elem(const float* p, int64_t i) { return p[i]; }
__device__ __forceinline__ float ld_elem(const uint16_t* p, int64_t i) {
  return __uint_as_float((uint32_t)p[i] << 16);
}
__device__ __forceinline__ float ld_elem(const uint8_t* p, int64_t i) {
  return __uint_as_float((uint32_t)p[i]);   // the code's bits travel unchanged
}
__device__ __forceinline__ void st_elem(uint16_t* p, int64_t i, float v) {
  uint32_t u = __float_as_uint(v);          // bfloat16, nearest even (NaN stays NaN)
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) {
    p[i] = (uint16_t)((u >> 16) | 0x40u);
    return;
  }
  u += 0x7FFFu + ((u >> 16) & 1u);
  p[i] = (uint16_t)(u >> 16);
}
__device__ __forceinline__ void st_elem(uint8_t* p, int64_t i, float v) {
  p[i] = (uint8_t)__float_as_uint(v);
}

// dst [out_rows x out_cols] (row stride ldd) = src [rows x cols] (row stride
// lds), or its transpose, converted element by element; positions past the
// source are written as zeros (padding).  One 64 x 64 tile of dst per
// workgroup, staged through LDS so that both sides are read and written
// along rows.
template <typename Tin, typename Tout>
__global__ __launch_bounds__(256) void convert_tile_kernel(const Tin* __restrict__ src, int64_t rows,
                                                           int64_t cols, int64_t lds,
                                                           Tout* __restrict__ dst,
                                                           int64_t out_rows, int64_t out_cols,
                                                           int64_t ldd, int trans) {
  __shared__ float t[CT][CT + 1];
  const int64_t o_r0 = (int64_t)blockIdx.y * CT, o_c0 = (int64_t)blockIdx.x * CT;
  // the source block this tile reads: rows/cols swapped when transposing
  const int64_t s_r0 = trans ? o_c0 : o_r0, s_c0 = trans ? o_r0 : o_c0;
  for (int e = threadIdx.x; e < CT * CT; e += 256) {
    const int r = e / CT, c = e % CT;
    const int64_t sr = s_r0 + r, sc = s_c0 + c;
    t[r][c] = (sr < rows && sc < cols) ? ld_elem(src, sr * lds + sc) : 0.0f;
  }
  __syncthreads();
  for (int e = threadIdx.x; e < CT * CT; e += 256) {
    const int r = e / CT, c = e % CT;
    const int64_t orr = o_r0 + r, oc = o_c0 + c;
    if (orr < out_rows && oc < out_cols) st_elem(dst, orr * ldd + oc, trans ? t[c][r] : t[r][c]);
  }
}

template <typename Tin, typename Tout>
hipError_t convert(const Tin* src, int64_t rows, int64_t cols, int64_t lds, Tout* dst,
                   int64_t out_rows, int64_t out_cols, int64_t ldd, bool trans, hipStream_t s) {
  if (out_rows == 0 || out_cols == 0) return hipSuccess;
  dim3 grid((unsigned)((out_cols + CT - 1) / CT), (unsigned)((out_rows + CT - 1) / CT));
  convert_tile_kernel<Tin, Tout><<<grid, 256, 0, s>>>(src, rows, cols, lds, dst, out_rows,
                                                      out_cols, ldd, trans ? 1 : 0);
  return hipGetLastError();
}

int64_t up(int64_t v, int64_t m) { return (v + m - 1) / m * m; }

// workspace carving (the same for the size query and the launch)
struct Carve {
  size_t o = 0;
  size_t take(size_t bytes) {
    const size_t at = o;
    o = align_up(o + bytes, 256);
    return at;
  }
};

// ---- separate-path FP8 -------------------------------------------------------
// saved: A~ [r x d_in], B~ [d_out x r], U~ [T x r16] and the scales s_a,
// s_b, s_u (written by the forward, read by the backward), then V~ [T x r16]
// and s_v (written by the backward)
struct SepSaved {
  size_t aq, bq, uq, sc, vq, total;
};
SepSaved sep_saved(int64_t T, int64_t d_in, int64_t d_out, int64_t r) {
  Carve c;
  SepSaved s;
  s.aq = c.take((size_t)(r * d_in));
  s.bq = c.take((size_t)(d_out * r));
  s.uq = c.take((size_t)(T * up(r, 16)));
  s.sc = c.take(16);
  s.vq = c.take((size_t)(T * up(r, 16)));
  s.total = c.o;
  return s;
}

struct SepWs {
  size_t qz, ap, bp, u32, sk, wt, btp, v32, atp, gt, ut, xt, vt, total;
};
SepWs sep_ws(int64_t T, int64_t d_in, int64_t d_out, int64_t r) {
  const int64_t r16 = up(r, 16);
  Carve c;
  SepWs w;
  w.qz = c.take(quantize_ws_bytes());
  w.ap = c.take((size_t)(r16 * d_in));                  // A~ padded to r16 rows
  w.bp = c.take((size_t)(d_out * r16));                 // B~ padded to r16 columns
  w.u32 = c.take((size_t)(T * r16 * 4));                // U (fp32)
  size_t sk = 0;                                        // split-K partials, largest product
  sk = std::max(sk, gemm_splitk_ws_bytes(T, r16, d_in));
  sk = std::max(sk, gemm_splitk_ws_bytes(T, r16, d_out));
  sk = std::max(sk, gemm_splitk_ws_bytes(d_out, r16, T));
  sk = std::max(sk, gemm_splitk_ws_bytes(r16, d_in, T));
  w.sk = c.take(sk);
  w.wt = c.take((size_t)(d_in * d_out));                // W~^T
  w.btp = c.take((size_t)(r16 * d_out));                // B~^T padded
  w.v32 = c.take((size_t)(T * r16 * 4));
  w.atp = c.take((size_t)(d_in * r16));                 // A~^T padded
  w.gt = c.take((size_t)(d_out * T));                   // G~^T
  w.ut = c.take((size_t)(r16 * T));                     // U~^T
  w.xt = c.take((size_t)(d_in * T));                    // X~^T
  w.vt = c.take((size_t)(r16 * T));                     // V~^T
  w.total = c.o;
  return w;
}

// ---- BF16 LoRA ---------------------------------------------------------------
struct BfWs {
  size_t xb, ab, u32, sk, bb, wt, gb, btb, v32, vb, atb, gtb, utb, xtb, vtb, total;
};
BfWs bf_ws(int64_t T, int64_t d_in, int64_t d_out, int64_t r) {
  const int64_t rb = up(r, 64);
  Carve c;
  BfWs w;
  w.xb = c.take((size_t)(T * d_in * 2));
  w.ab = c.take((size_t)(rb * d_in * 2));
  w.u32 = c.take((size_t)(T * rb * 4));
  size_t sk = 0;
  sk = std::max(sk, gemm_splitk_ws_bytes(T, rb, 2 * d_in));
  sk = std::max(sk, gemm_splitk_ws_bytes(T, rb, 2 * d_out));
  sk = std::max(sk, gemm_splitk_ws_bytes(d_out, rb, 2 * T));
  sk = std::max(sk, gemm_splitk_ws_bytes(rb, d_in, 2 * T));
  w.sk = c.take(sk);
  w.bb = c.take((size_t)(d_out * rb * 2));
  w.wt = c.take((size_t)(d_in * d_out));
  w.gb = c.take((size_t)(T * d_out * 2));
  w.btb = c.take((size_t)(rb * d_out * 2));
  w.v32 = c.take((size_t)(T * rb * 4));
  w.vb = c.take((size_t)(T * rb * 2));
  w.atb = c.take((size_t)(d_in * rb * 2));
  w.gtb = c.take((size_t)(d_out * T * 2));
  w.utb = c.take((size_t)(rb * T * 2));
  w.xtb = c.take((size_t)(d_in * T * 2));
  w.vtb = c.take((size_t)(rb * T * 2));
  w.total = c.o;
  return w;
}

#define FALQ_TRY(x)                         \
  do {                                      \
    const hipError_t e_ = (x);              \
    if (e_ != hipSuccess) return e_;        \
  } while (0)

}  // namespace

size_t lora_sep_saved_bytes(int64_t T, int64_t d_in, int64_t d_out, int64_t r) {
  return sep_saved(T, d_in, d_out, r).total;
}
size_t lora_sep_ws_bytes(int64_t T, int64_t d_in, int64_t d_out, int64_t r) {
  return sep_ws(T, d_in, d_out, r).total;
}
size_t lora_bf16_saved_bytes(int64_t T, int64_t r) { return (size_t)(T * up(r, 64) * 2); }
size_t lora_bf16_ws_bytes(int64_t T, int64_t d_in, int64_t d_out, int64_t r) {
  return bf_ws(T, d_in, d_out, r).total;
}

hipError_t launch_lora_sep_fwd(const uint8_t* xq, const float* s_x, const uint8_t* wq,
                               const float* s_w, const float* A, const float* B, int64_t T,
                               int64_t d_in, int64_t d_out, int64_t r, float* y, void* saved,
                               void* ws, hipStream_t s) {
  const int64_t r16 = up(r, 16);
  const SepSaved sv = sep_saved(T, d_in, d_out, r);
  const SepWs w = sep_ws(T, d_in, d_out, r);
  uint8_t* sb = reinterpret_cast<uint8_t*>(saved);
  uint8_t* wb = reinterpret_cast<uint8_t*>(ws);
  uint8_t* aq = sb + sv.aq;
  uint8_t* bq = sb + sv.bq;
  uint8_t* uq = sb + sv.uq;
  float* sc = reinterpret_cast<float*>(sb + sv.sc);     // s_a, s_b, s_u
  void* qz = wb + w.qz;
  float* sk = reinterpret_cast<float*>(wb + w.sk);
  // the backbone product
  FALQ_TRY(launch_gemm_fp8_nt(xq, d_in, wq, d_in, y, d_out, T, d_out, d_in, s_x, s_w, s));
  // A~ = Q(A), B~ = Q(B)
  FALQ_TRY(launch_quantize(A, 0, 0, r * d_in, nullptr, aq, sc + 0, nullptr, nullptr, qz, s));
  FALQ_TRY(launch_quantize(B, 0, 0, d_out * r, nullptr, bq, sc + 1, nullptr, nullptr, qz, s));
  // U = X^ A^^T  [T x r16] (A~ padded to r16 rows with zero codes)
  uint8_t* ap = wb + w.ap;
  FALQ_TRY(convert(aq, r, d_in, d_in, ap, r16, d_in, d_in, false, s));
  float* u32 = reinterpret_cast<float*>(wb + w.u32);
  FALQ_TRY(launch_gemm_fp8_nt(xq, d_in, ap, d_in, u32, r16, T, r16, d_in, s_x, sc + 0, s, 0, 0,
                              sk));
  // U~ = Q(U)
  FALQ_TRY(launch_quantize(u32, 0, 0, T * r16, nullptr, uq, sc + 2, nullptr, nullptr, qz, s));
  // Y += U^ B^^T (K = r16; B~ padded to r16 columns)
  uint8_t* bp = wb + w.bp;
  FALQ_TRY(convert(bq, d_out, r, r, bp, d_out, r16, r16, false, s));
  return launch_gemm_fp8_nt(uq, r16, bp, r16, y, d_out, T, d_out, r16, sc + 2, sc + 1, s, 0, 1);
}

hipError_t launch_lora_sep_bwd(const uint8_t* gq, const float* s_g, const uint8_t* xq,
                               const float* s_x, const uint8_t* wq, const float* s_w,
                               void* saved, int64_t T, int64_t d_in, int64_t d_out, int64_t r,
                               float* dx, float* dA, float* dB, void* ws, hipStream_t s) {
  const int64_t r16 = up(r, 16);
  const SepSaved sv = sep_saved(T, d_in, d_out, r);
  const SepWs w = sep_ws(T, d_in, d_out, r);
  uint8_t* sb = reinterpret_cast<uint8_t*>(saved);
  uint8_t* wb = reinterpret_cast<uint8_t*>(ws);
  const uint8_t* aq = sb + sv.aq;
  const uint8_t* bq = sb + sv.bq;
  const uint8_t* uq = sb + sv.uq;
  float* sc = reinterpret_cast<float*>(sb + sv.sc);
  void* qz = wb + w.qz;
  float* sk = reinterpret_cast<float*>(wb + w.sk);
  // the backbone product dX = G^ W^
  uint8_t* wt = wb + w.wt;
  FALQ_TRY(launch_transpose_u8(wq, d_out, d_in, wt, s));
  FALQ_TRY(launch_gemm_fp8_nt(gq, d_out, wt, d_out, dx, d_in, T, d_in, d_out, s_g, s_w, s));
  // V = G^ B^  [T x r16] against B~^T padded to r16 rows
  uint8_t* btp = wb + w.btp;
  FALQ_TRY(convert(bq, d_out, r, r, btp, r16, d_out, d_out, true, s));
  float* v32 = reinterpret_cast<float*>(wb + w.v32);
  FALQ_TRY(launch_gemm_fp8_nt(gq, d_out, btp, d_out, v32, r16, T, r16, d_out, s_g, sc + 1, s, 0,
                              0, sk));
  // V~ = Q(V), kept in `saved` beside the forward's factors
  uint8_t* vq = sb + sv.vq;
  float* s_v = sc + 3;
  FALQ_TRY(launch_quantize(v32, 0, 0, T * r16, nullptr, vq, s_v, nullptr, nullptr, qz, s));
  // dX += V^ A^ against A~^T padded to r16 columns
  uint8_t* atp = wb + w.atp;
  FALQ_TRY(convert(aq, r, d_in, d_in, atp, d_in, r16, r16, true, s));
  FALQ_TRY(launch_gemm_fp8_nt(vq, r16, atp, r16, dx, d_in, T, d_in, r16, s_v, sc + 0, s, 0, 1));
  // dB = G^^T U^ over tokens: G~^T [d_out x T], U~^T [r16 x T]
  uint8_t* gt = wb + w.gt;
  uint8_t* ut = wb + w.ut;
  FALQ_TRY(launch_transpose_u8(gq, T, d_out, gt, s));
  FALQ_TRY(launch_transpose_u8(uq, T, r16, ut, s));
  FALQ_TRY(launch_gemm_fp8_nt(gt, T, ut, T, dB, r, d_out, r, T, s_g, sc + 2, s, 0, 0, sk));
  // dA = V^^T X^ over tokens: V~^T [r16 x T], X~^T [d_in x T]
  uint8_t* vt = wb + w.vt;
  uint8_t* xt = wb + w.xt;
  FALQ_TRY(launch_transpose_u8(vq, T, r16, vt, s));
  FALQ_TRY(launch_transpose_u8(xq, T, d_in, xt, s));
  return launch_gemm_fp8_nt(vt, T, xt, T, dA, d_in, r, d_in, T, s_v, s_x, s, 0, 0, sk);
}

hipError_t launch_lora_bf16_fwd(const float* x, const uint8_t* xq, const float* s_x,
                                const uint8_t* wq, const float* s_w, const float* A,
                                const float* B, int64_t T, int64_t d_in, int64_t d_out, int64_t r,
                                float* y, void* saved, void* ws, hipStream_t s) {
  const int64_t rb = up(r, 64);
  const BfWs w = bf_ws(T, d_in, d_out, r);
  uint8_t* wb = reinterpret_cast<uint8_t*>(ws);
  uint16_t* ub = reinterpret_cast<uint16_t*>(saved);
  float* sk = reinterpret_cast<float*>(wb + w.sk);
  FALQ_TRY(launch_gemm_fp8_nt(xq, d_in, wq, d_in, y, d_out, T, d_out, d_in, s_x, s_w, s));
  uint16_t* xb = reinterpret_cast<uint16_t*>(wb + w.xb);
  uint16_t* ab = reinterpret_cast<uint16_t*>(wb + w.ab);
  FALQ_TRY(convert(x, T, d_in, d_in, xb, T, d_in, d_in, false, s));
  FALQ_TRY(convert(A, r, d_in, d_in, ab, rb, d_in, d_in, false, s));
  // U = bf(X) bf(A)^T [T x rb], then bf(U)
  float* u32 = reinterpret_cast<float*>(wb + w.u32);
  FALQ_TRY(launch_gemm_bf16_nt(xb, d_in, ab, d_in, u32, rb, T, rb, d_in, s, 0, sk));
  FALQ_TRY(convert(u32, T, rb, rb, ub, T, rb, rb, false, s));
  // Y += bf(U) bf(B)^T (K = rb)
  uint16_t* bb = reinterpret_cast<uint16_t*>(wb + w.bb);
  FALQ_TRY(convert(B, d_out, r, r, bb, d_out, rb, rb, false, s));
  return launch_gemm_bf16_nt(ub, rb, bb, rb, y, d_out, T, d_out, rb, s, 1);
}

hipError_t launch_lora_bf16_bwd(const float* dy, const uint8_t* gq, const float* s_g,
                                const float* x, const uint8_t* wq, const float* s_w,
                                const float* A, const float* B, const void* saved, int64_t T,
                                int64_t d_in, int64_t d_out, int64_t r, float* dx, float* dA,
                                float* dB, void* ws, hipStream_t s) {
  const int64_t rb = up(r, 64);
  const BfWs w = bf_ws(T, d_in, d_out, r);
  uint8_t* wb = reinterpret_cast<uint8_t*>(ws);
  const uint16_t* ub = reinterpret_cast<const uint16_t*>(saved);
  float* sk = reinterpret_cast<float*>(wb + w.sk);
  uint8_t* wt = wb + w.wt;
  FALQ_TRY(launch_transpose_u8(wq, d_out, d_in, wt, s));
  FALQ_TRY(launch_gemm_fp8_nt(gq, d_out, wt, d_out, dx, d_in, T, d_in, d_out, s_g, s_w, s));
  auto b16 = [&](size_t off) { return reinterpret_cast<uint16_t*>(wb + off); };
  // V = bf(dY) bf(B) [T x rb] against bf(B)^T padded to rb rows, then bf(V)
  FALQ_TRY(convert(dy, T, d_out, d_out, b16(w.gb), T, d_out, d_out, false, s));
  FALQ_TRY(convert(B, d_out, r, r, b16(w.btb), rb, d_out, d_out, true, s));
  float* v32 = reinterpret_cast<float*>(wb + w.v32);
  FALQ_TRY(launch_gemm_bf16_nt(b16(w.gb), d_out, b16(w.btb), d_out, v32, rb, T, rb, d_out, s, 0,
                               sk));
  FALQ_TRY(convert(v32, T, rb, rb, b16(w.vb), T, rb, rb, false, s));
  // dX += bf(V) bf(A) against bf(A)^T padded to rb columns
  FALQ_TRY(convert(A, r, d_in, d_in, b16(w.atb), d_in, rb, rb, true, s));
  FALQ_TRY(launch_gemm_bf16_nt(b16(w.vb), rb, b16(w.atb), rb, dx, d_in, T, d_in, rb, s, 1));
  // dB = bf(dY)^T bf(U) over tokens
  FALQ_TRY(convert(dy, T, d_out, d_out, b16(w.gtb), d_out, T, T, true, s));
  FALQ_TRY(convert(ub, T, rb, rb, b16(w.utb), rb, T, T, true, s));
  FALQ_TRY(launch_gemm_bf16_nt(b16(w.gtb), T, b16(w.utb), T, dB, r, d_out, r, T, s, 0, sk));
  // dA = bf(V)^T bf(X) over tokens
  FALQ_TRY(convert(x, T, d_in, d_in, b16(w.xtb), d_in, T, T, true, s));
  FALQ_TRY(convert(b16(w.vb), T, rb, rb, b16(w.vtb), rb, T, T, true, s));
  return launch_gemm_bf16_nt(b16(w.vtb), T, b16(w.xtb), T, dA, d_in, r, d_in, T, s, 0, sk);
}

}  // namespace falq
