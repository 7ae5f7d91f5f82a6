// C ABI of the melded FP8 LoRA step: argument validation and dispatch to the
// gfx950 kernels.  Every argument error is reported before anything is
// launched; launches are asynchronous on the caller's stream.
#include "../../include/falqon.h"
#include "kernels.hpp"

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdint>

namespace {

using falq::align_up;

inline bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

// a required device pointer: non-null and 16-byte aligned
inline bool need(const void* p) { return p != nullptr && aligned(p, 16); }
// an optional device pointer: null, or 16-byte aligned
inline bool opt(const void* p) { return p == nullptr || aligned(p, 16); }
// a device scalar (float / int32): non-null and 4-byte aligned
inline bool scalar(const void* p) { return p != nullptr && aligned(p, 4); }

inline bool dims_ok(int64_t d) { return d >= 0 && d % 16 == 0 && d <= (int64_t)1 << 30; }

// T, d_in, d_out of a melded linear layer: the GEMMs (T x d_out and T x d_in
// outputs) launch one workgroup per 256 x 256 tile, two per split tile, on a
// 32-bit grid
inline bool gemm_dims_ok(int64_t T, int64_t d_in, int64_t d_out) {
  if (T < 0 || T > ((int64_t)1 << 30) || !dims_ok(d_in) || !dims_ok(d_out)) return false;
  const int64_t tiles = ((T + 255) / 256) * ((std::max(d_in, d_out) + 255) / 256);
  return 2 * tiles <= INT32_MAX;
}

inline falq_status hip_status(hipError_t e) { return e == hipSuccess ? FALQ_OK : FALQ_EHIP; }

inline bool ws_ok(const void* ws, size_t have, size_t need_bytes) {
  if (need_bytes == 0) return true;
  return ws != nullptr && aligned(ws, 256) && have >= need_bytes;
}

// dX = dec(G~) dec(W~) / (s_g s_w) as an NT FP8 GEMM against W~^T, which is
// written to the first d_in * d_out bytes of the workspace
hipError_t run_dx(const uint8_t* gq, int g_fmt, const float* s_g, const uint8_t* wq,
                  const float* s_w, int64_t T, int64_t d_in, int64_t d_out, float* dx, uint8_t* wt,
                  hipStream_t s) {
  if (T * d_in == 0) return hipSuccess;
  if (d_out == 0) return falq::launch_fill_f32(dx, T * d_in, 0.0f, s);
  hipError_t e = falq::launch_transpose_u8(wq, d_out, d_in, wt, s);
  if (e != hipSuccess) return e;
  return falq::launch_gemm_fp8_nt(gq, d_out, wt, d_out, dx, d_in, T, d_in, d_out, s_g, s_w, s,
                                  g_fmt);
}

inline bool fmt_ok(int f) { return f == FALQ_E4M3 || f == FALQ_E5M2; }

static_assert(falq::kQuantizeScratchBytes == FALQ_QUANTIZE_SCRATCH_BYTES,
              "the scratch size the header states");

}  // namespace

extern "C" {

const char* falq_status_string(falq_status s) {
  switch (s) {
    case FALQ_OK: return "FALQ_OK";
    case FALQ_EINVAL: return "FALQ_EINVAL: invalid argument";
    case FALQ_EHIP: return "FALQ_EHIP: HIP launch or runtime error";
    case FALQ_EUNSUPPORTED: return "FALQ_EUNSUPPORTED: not supported by this library";
  }
  return "unknown falq_status";
}

const char* falq_version(void) { return "0.1.0"; }

size_t fp8_quantize_workspace_bytes(int64_t n) {
  (void)n;
  return falq::quantize_ws_bytes();
}

falq_status fp8_quantize(const void* x, int dtype, int64_t n, const float* scale_in, uint8_t* q,
                         float* scale, float* amax, int32_t* nonfinite, void* ws, size_t ws_bytes,
                         falq_stream stream) {
  return fp8_quantize_fmt(x, dtype, n, FALQ_E4M3, scale_in, q, scale, amax, nonfinite, ws,
                          ws_bytes, stream);
}

falq_status fp8_quantize_fmt(const void* x, int dtype, int64_t n, int fmt, const float* scale_in,
                             uint8_t* q, float* scale, float* amax, int32_t* nonfinite, void* ws,
                             size_t ws_bytes, falq_stream stream) {
  if (n < 0 || (dtype != FALQ_F32 && dtype != FALQ_BF16) || !fmt_ok(fmt)) return FALQ_EINVAL;
  if (n > 0 && (!need(x) || !need(q))) return FALQ_EINVAL;
  if (!scalar(scale) || (scale_in && !aligned(scale_in, 4)) || (amax && !aligned(amax, 4)) ||
      (nonfinite && !aligned(nonfinite, 4)))
    return FALQ_EINVAL;
  if (!ws_ok(ws, ws_bytes, falq::quantize_ws_bytes())) return FALQ_EINVAL;
  return hip_status(falq::launch_quantize(x, dtype, fmt, n, scale_in, q, scale, amax, nonfinite,
                                          ws, reinterpret_cast<hipStream_t>(stream)));
}

uint64_t fp8_quantize_wait_ticks(uint64_t ticks) { return falq::quantize_wait_ticks(ticks); }

falq_status fp8_quantize_noalloc(const void* x, int dtype, int64_t n, int fmt,
                                 const float* scale_in, uint8_t* q, float* scale, float* amax,
                                 int32_t* nonfinite, falq_stream stream) {
  if (n < 0 || (dtype != FALQ_F32 && dtype != FALQ_BF16) || !fmt_ok(fmt)) return FALQ_EINVAL;
  if (n > 0 && (!need(x) || !need(q))) return FALQ_EINVAL;
  if (!scalar(scale) || (scale_in && !aligned(scale_in, 4)) || (amax && !aligned(amax, 4)) ||
      (nonfinite && !aligned(nonfinite, 4)))
    return FALQ_EINVAL;
  // the scratch need does not grow with n (at most kQzMaxParts partials)
  if (falq::quantize_ws_bytes() > falq::quantize_scratch_bytes()) return FALQ_EUNSUPPORTED;
  void* ws = nullptr;
  if (falq::quantize_scratch(&ws) != hipSuccess || ws == nullptr) return FALQ_EHIP;
  return hip_status(falq::launch_quantize(x, dtype, fmt, n, scale_in, q, scale, amax, nonfinite,
                                          ws, reinterpret_cast<hipStream_t>(stream)));
}

falq_status fp4_quantize(const void* x, int dtype, int64_t n, const float* scale_in, uint8_t* q,
                         float* scale, float* amax, int32_t* nonfinite, void* ws, size_t ws_bytes,
                         falq_stream stream) {
  if (n < 0 || n % 2 != 0 || (dtype != FALQ_F32 && dtype != FALQ_BF16)) return FALQ_EINVAL;
  if (n > 0 && (!need(x) || !need(q))) return FALQ_EINVAL;
  if (!scalar(scale) || (scale_in && !aligned(scale_in, 4)) || (amax && !aligned(amax, 4)) ||
      (nonfinite && !aligned(nonfinite, 4)))
    return FALQ_EINVAL;
  if (!ws_ok(ws, ws_bytes, falq::quantize_ws_bytes())) return FALQ_EINVAL;
  return hip_status(falq::launch_quantize(x, dtype, 2, n, scale_in, q, scale, amax, nonfinite, ws,
                                          reinterpret_cast<hipStream_t>(stream)));
}

falq_status melded_linear_fwd_fp4(const uint8_t* xq, const float* s_x, const uint8_t* wq,
                                  const float* s_w, int64_t T, int64_t d_in, int64_t d_out,
                                  float* y, falq_stream stream) {
  if (!gemm_dims_ok(T, d_in, d_out) || d_in % 256 != 0)
    return FALQ_EINVAL;
  if (!scalar(s_x) || !scalar(s_w)) return FALQ_EINVAL;
  if (T * d_in > 0 && !need(xq)) return FALQ_EINVAL;
  if (d_out * d_in > 0 && !need(wq)) return FALQ_EINVAL;
  if (T * d_out > 0 && !need(y)) return FALQ_EINVAL;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  if (T == 0 || d_out == 0) return FALQ_OK;
  if (d_in == 0) return hip_status(falq::launch_fill_f32(y, T * d_out, 0.0f, s));
  return hip_status(falq::launch_gemm_fp4_nt(xq, d_in / 2, wq, d_in / 2, y, d_out, T, d_out,
                                             d_in / 2, s_x, s_w, s));
}

falq_status melded_linear_fwd(const uint8_t* xq, const float* s_x, const uint8_t* wq,
                              const float* s_w, int64_t T, int64_t d_in, int64_t d_out, float* y,
                              falq_stream stream) {
  if (!gemm_dims_ok(T, d_in, d_out)) return FALQ_EINVAL;
  if (!scalar(s_x) || !scalar(s_w)) return FALQ_EINVAL;
  if (T * d_in > 0 && !need(xq)) return FALQ_EINVAL;
  if (d_out * d_in > 0 && !need(wq)) return FALQ_EINVAL;
  if (T * d_out > 0 && !need(y)) return FALQ_EINVAL;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  if (T == 0 || d_out == 0) return FALQ_OK;
  if (d_in == 0) return hip_status(falq::launch_fill_f32(y, T * d_out, 0.0f, s));
  return hip_status(
      falq::launch_gemm_fp8_nt(xq, d_in, wq, d_in, y, d_out, T, d_out, d_in, s_x, s_w, s));
}

size_t melded_linear_bwd_workspace_bytes(int64_t T, int64_t d_in, int64_t d_out, int64_t r) {
  if (T < 0 || d_in < 0 || d_out < 0 || r < 0) return 0;
  const size_t wt = align_up((size_t)d_in * (size_t)d_out, 256);      // W~^T for dX
  return wt + (falq::adapter_wide_route(T, d_in, d_out, r)
                   ? falq::adapter_wide_ws_bytes(T, d_in, d_out, r)
                   : falq::adapter_grad_ws_bytes(T, d_in, d_out, r));
}

falq_status melded_linear_bwd(const uint8_t* gq, const float* s_g, const uint8_t* xq,
                              const float* s_x, const uint8_t* wq, const float* s_w,
                              const float* A, const float* B, int64_t T, int64_t d_in,
                              int64_t d_out, int64_t r, float* dx, float* dA, float* dB, void* ws,
                              size_t ws_bytes, falq_stream stream) {
  return melded_linear_bwd_fmt(gq, FALQ_E4M3, s_g, xq, s_x, wq, s_w, A, B, T, d_in, d_out, r, dx,
                               dA, dB, ws, ws_bytes, stream);
}

falq_status melded_linear_bwd_fmt(const uint8_t* gq, int g_fmt, const float* s_g,
                                  const uint8_t* xq, const float* s_x, const uint8_t* wq,
                                  const float* s_w, const float* A, const float* B, int64_t T,
                                  int64_t d_in, int64_t d_out, int64_t r, float* dx, float* dA,
                                  float* dB, void* ws, size_t ws_bytes, falq_stream stream) {
  if (!fmt_ok(g_fmt)) return FALQ_EINVAL;
  if (!gemm_dims_ok(T, d_in, d_out) || r < 0 ||
      r > ((int64_t)1 << 20))
    return FALQ_EINVAL;
  if (!scalar(s_g) || !scalar(s_x) || !scalar(s_w)) return FALQ_EINVAL;
  if (T * d_out > 0 && !need(gq)) return FALQ_EINVAL;
  if (T * d_in > 0 && !need(xq)) return FALQ_EINVAL;
  if (d_out * d_in > 0 && dx && !need(wq)) return FALQ_EINVAL;
  if (!opt(dx) || !opt(dA)) return FALQ_EINVAL;
  if (r * d_in > 0 && !need(A)) return FALQ_EINVAL;
  if (r * d_out > 0 && (!need(B) || !need(dB))) return FALQ_EINVAL;
  if (r * d_in > 0 && dA && !need(dA)) return FALQ_EINVAL;
  if (!ws_ok(ws, ws_bytes, melded_linear_bwd_workspace_bytes(T, d_in, d_out, r)))
    return FALQ_EINVAL;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  uint8_t* base = reinterpret_cast<uint8_t*>(ws);
  const size_t wt_bytes = align_up((size_t)d_in * (size_t)d_out, 256);
  // W~^T (for dX) and the adapter operands' bf16 splits in one launch
  const bool gemm_dx = dx && T * d_in > 0 && d_out > 0;
  const bool grads = r > 0 && T > 0 && d_in > 0 && d_out > 0;
  // large ranks contract through the full weight gradient instead
  const bool wide = grads && falq::adapter_wide_route(T, d_in, d_out, r);
  if (falq::launch_bwd_prep(wq, gemm_dx ? base : nullptr, A, B, T, d_in, d_out,
                            grads && !wide ? r : 0, dA != nullptr, base + wt_bytes,
                            s) != hipSuccess)
    return FALQ_EHIP;
  hipError_t e = hipSuccess;
  if (gemm_dx)
    e = falq::launch_gemm_fp8_nt(gq, d_out, base, d_out, dx, d_in, T, d_in, d_out, s_g, s_w, s,
                                 g_fmt);
  else if (dx && T * d_in > 0)                                 // d_out == 0
    e = falq::launch_fill_f32(dx, T * d_in, 0.0f, s);
  if (e != hipSuccess) return FALQ_EHIP;
  if (r > 0) {
    if (d_in == 0 || d_out == 0) {
      if (d_out > 0) e = falq::launch_fill_f32(dB, d_out * r, 0.0f, s);
      if (e == hipSuccess && dA && d_in > 0) e = falq::launch_fill_f32(dA, r * d_in, 0.0f, s);
    } else if (wide) {
      e = falq::launch_adapter_grads_wide(gq, g_fmt, s_g, xq, s_x, A, B, T, d_in, d_out, r, dA,
                                          dB, base + wt_bytes, s);
    } else {
      e = falq::launch_adapter_grads(gq, s_g, xq, s_x, A, B, T, d_in, d_out, r, dA, dB,
                                     base + wt_bytes, s, g_fmt, /*presplit=*/grads);
    }
  }
  return hip_status(e);
}

falq_status fp8_dequantize(const uint8_t* q, const float* scale, int64_t n, float* out,
                           falq_stream stream) {
  if (n < 0 || !scalar(scale)) return FALQ_EINVAL;
  if (n > 0 && (!need(q) || !need(out))) return FALQ_EINVAL;
  return hip_status(falq::launch_dequantize(q, n, scale, out, reinterpret_cast<hipStream_t>(stream)));
}

size_t melded_linear_fwd_frozen_a_workspace_bytes(int64_t T, int64_t d_in, int64_t r) {
  if (T < 0 || d_in < 0 || r < 0) return 0;
  return falq::frozen_u_ws_bytes(T, d_in, r);
}

falq_status melded_linear_fwd_frozen_a(const uint8_t* xq, const float* s_x, const uint8_t* wq,
                                       const float* s_w, const uint8_t* aq, const float* s_a,
                                       int64_t T, int64_t d_in, int64_t d_out, int64_t r,
                                       float* y, float* u, void* ws, size_t ws_bytes,
                                       falq_stream stream) {
  if (!gemm_dims_ok(T, d_in, d_out) || r < 0 ||
      r > ((int64_t)1 << 20))
    return FALQ_EINVAL;
  if (!scalar(s_a)) return FALQ_EINVAL;
  if (r * d_in > 0 && !need(aq)) return FALQ_EINVAL;
  if (T * r > 0 && !need(u)) return FALQ_EINVAL;
  if (!ws_ok(ws, ws_bytes, melded_linear_fwd_frozen_a_workspace_bytes(T, d_in, r)))
    return FALQ_EINVAL;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  if (T > 0 && d_in > 0 && falq::gemm_fp8_nt_fuses_second(d_out, d_in, r)) {
    // U from the forward GEMM's own X~ tiles (one launch)
    if (!scalar(s_x) || !scalar(s_w) || !need(xq) || !need(wq) || !need(y)) return FALQ_EINVAL;
    return hip_status(falq::launch_gemm_fp8_nt_second(xq, d_in, wq, d_in, y, d_out, T, d_out, d_in,
                                                      s_x, s_w, aq, d_in, r, u, r, s_a, s));
  }
  const falq_status st = melded_linear_fwd(xq, s_x, wq, s_w, T, d_in, d_out, y, stream);
  if (st != FALQ_OK) return st;
  return hip_status(falq::launch_frozen_u(xq, s_x, aq, s_a, T, d_in, r, u, ws, s));
}

size_t melded_linear_bwd_frozen_a_workspace_bytes(int64_t T, int64_t d_in, int64_t d_out,
                                                  int64_t r) {
  if (T < 0 || d_in < 0 || d_out < 0 || r < 0) return 0;
  const size_t wt = align_up((size_t)d_in * (size_t)d_out, 256);      // W~^T for dX
  return wt + falq::frozen_db_ws_bytes(T, d_out, r);
}

falq_status melded_linear_bwd_frozen_a(const uint8_t* gq, const float* s_g, const uint8_t* wq,
                                       const float* s_w, const float* u, int64_t T, int64_t d_in,
                                       int64_t d_out, int64_t r, float* dx, float* dB, void* ws,
                                       size_t ws_bytes, falq_stream stream) {
  return melded_linear_bwd_frozen_a_fmt(gq, FALQ_E4M3, s_g, wq, s_w, u, T, d_in, d_out, r, dx, dB,
                                        ws, ws_bytes, stream);
}

falq_status melded_linear_bwd_frozen_a_fmt(const uint8_t* gq, int g_fmt, const float* s_g,
                                           const uint8_t* wq, const float* s_w, const float* u,
                                           int64_t T, int64_t d_in, int64_t d_out, int64_t r,
                                           float* dx, float* dB, void* ws, size_t ws_bytes,
                                           falq_stream stream) {
  if (!fmt_ok(g_fmt)) return FALQ_EINVAL;
  if (!gemm_dims_ok(T, d_in, d_out) || r < 0 ||
      r > ((int64_t)1 << 20))
    return FALQ_EINVAL;
  if (!scalar(s_g) || !scalar(s_w)) return FALQ_EINVAL;
  if (T * d_out > 0 && !need(gq)) return FALQ_EINVAL;
  if (d_out * d_in > 0 && dx && !need(wq)) return FALQ_EINVAL;
  if (!opt(dx)) return FALQ_EINVAL;
  if (T * r > 0 && !need(u)) return FALQ_EINVAL;
  if (r * d_out > 0 && !need(dB)) return FALQ_EINVAL;
  if (!ws_ok(ws, ws_bytes, melded_linear_bwd_frozen_a_workspace_bytes(T, d_in, d_out, r)))
    return FALQ_EINVAL;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  uint8_t* base = reinterpret_cast<uint8_t*>(ws);
  const size_t wt_bytes = align_up((size_t)d_in * (size_t)d_out, 256);
  if (dx && run_dx(gq, g_fmt, s_g, wq, s_w, T, d_in, d_out, dx, base, s) != hipSuccess)
    return FALQ_EHIP;
  return hip_status(
      falq::launch_frozen_db(gq, s_g, u, T, d_out, r, dB, base + wt_bytes, s, g_fmt));
}

falq_status adapter_step(float* A, float* B, const float* dA, const float* dB, int64_t r,
                         int64_t d_in, int64_t d_out, float lr, falq_stream stream) {
  if (r < 0 || d_in < 0 || d_out < 0) return FALQ_EINVAL;
  if (r * d_in > 0 && (!need(A) || !opt(dA))) return FALQ_EINVAL;
  if (r * d_out > 0 && (!need(B) || !need(dB))) return FALQ_EINVAL;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const int64_t na = dA ? r * d_in : 0;
  return hip_status(falq::launch_sgd2(A, dA, na, B, dB, r * d_out, lr, s));
}

falq_status adapter_step_adamw(float* A, float* B, const float* dA, const float* dB, float* mA,
                               float* vA, float* mB, float* vB, int64_t r, int64_t d_in,
                               int64_t d_out, float lr, float beta1, float beta2, float eps,
                               float weight_decay, void* state, falq_stream stream) {
  if (r < 0 || d_in < 0 || d_out < 0) return FALQ_EINVAL;
  if (!std::isfinite(lr) || !std::isfinite(weight_decay) || !(beta1 >= 0.0f && beta1 < 1.0f) ||
      !(beta2 >= 0.0f && beta2 < 1.0f) || !(eps > 0.0f) || !std::isfinite(eps))
    return FALQ_EINVAL;
  if (state == nullptr || !aligned(state, 8)) return FALQ_EINVAL;
  const bool train_a = dA != nullptr && r * d_in > 0;
  if (train_a && (!need(A) || !need(dA) || !need(mA) || !need(vA))) return FALQ_EINVAL;
  if (r * d_in > 0 && !opt(dA)) return FALQ_EINVAL;
  if (r * d_out > 0 && (!need(B) || !need(dB) || !need(mB) || !need(vB))) return FALQ_EINVAL;
  const falq::AdamWTensor ta{A, dA, mA, vA, train_a ? r * d_in : 0};
  const falq::AdamWTensor tb{B, dB, mB, vB, r * d_out};
  return hip_status(falq::launch_adamw2(ta, tb, reinterpret_cast<falq::AdamWState*>(state), lr,
                                        beta1, beta2, eps, weight_decay,
                                        reinterpret_cast<hipStream_t>(stream)));
}

size_t rowwise_proxy_update_workspace_bytes(int64_t d_in, int64_t d_out, int64_t r) {
  if (d_in < 0 || d_out < 0 || r < 0) return 0;
  return falq::proxy_ws_bytes(d_in, d_out, r);
}

falq_status rowwise_proxy_update(uint8_t* wq, const float* s_w, const float* A, float* B,
                                 int64_t d_in, int64_t d_out, int64_t r, float tau, int64_t k_max,
                                 int32_t* sel_idx, int32_t* n_sel, float* rho, void* ws,
                                 size_t ws_bytes, falq_stream stream) {
  // rows are independent: only d_in needs 16-byte rows of codes
  if (!dims_ok(d_in) || d_out < 0 || d_out > ((int64_t)1 << 30) || r < 0 ||
      r > ((int64_t)1 << 20) || k_max < 0)
    return FALQ_EINVAL;
  if (!scalar(s_w) || !scalar(n_sel)) return FALQ_EINVAL;
  if (d_out * d_in > 0 && !need(wq)) return FALQ_EINVAL;
  if (r * d_in > 0 && !need(A)) return FALQ_EINVAL;
  if (r * d_out > 0 && !need(B)) return FALQ_EINVAL;
  if (d_out > 0 && !need(sel_idx)) return FALQ_EINVAL;
  if (!opt(rho)) return FALQ_EINVAL;
  if (!ws_ok(ws, ws_bytes, rowwise_proxy_update_workspace_bytes(d_in, d_out, r)))
    return FALQ_EINVAL;
  return hip_status(falq::launch_proxy_update(wq, s_w, A, B, d_in, d_out, r, tau, k_max, sel_idx,
                                              n_sel, rho, ws, reinterpret_cast<hipStream_t>(stream)));
}

falq_status rowwise_proxy_update_t(uint8_t* wq, uint8_t* wqT, const float* s_w, const float* A,
                                   float* B, int64_t d_in, int64_t d_out, int64_t r, float tau,
                                   int64_t k_max, int32_t* sel_idx, int32_t* n_sel, float* rho,
                                   void* ws, size_t ws_bytes, falq_stream stream) {
  // the transpose takes whole 16 x 16 byte blocks: d_out a multiple of 16 too
  if (!dims_ok(d_in) || !dims_ok(d_out) || r < 0 || r > ((int64_t)1 << 20) || k_max < 0)
    return FALQ_EINVAL;
  if (!scalar(s_w) || !scalar(n_sel)) return FALQ_EINVAL;
  if (d_out * d_in > 0 && (!need(wq) || !need(wqT) || wq == wqT)) return FALQ_EINVAL;
  if (r * d_in > 0 && !need(A)) return FALQ_EINVAL;
  if (r * d_out > 0 && !need(B)) return FALQ_EINVAL;
  if (d_out > 0 && !need(sel_idx)) return FALQ_EINVAL;
  if (!opt(rho)) return FALQ_EINVAL;
  if (!ws_ok(ws, ws_bytes, rowwise_proxy_update_workspace_bytes(d_in, d_out, r)))
    return FALQ_EINVAL;
  return hip_status(falq::launch_proxy_update_ranks(
      wq, s_w, A, B, d_in, d_out, r, r, nullptr, tau, k_max, sel_idx, n_sel, rho, ws,
      reinterpret_cast<hipStream_t>(stream), d_out * d_in > 0 ? wqT : nullptr));
}

size_t rowwise_proxy_update_topk_rank_workspace_bytes(int64_t d_in, int64_t d_out, int64_t r,
                                                      int64_t k_rank) {
  if (d_in < 0 || d_out < 0 || r < 0 || k_rank < 0 || k_rank > r) return 0;
  return falq::proxy_topk_rank_ws_bytes(d_in, d_out, r, k_rank);
}

falq_status rowwise_proxy_update_topk_rank(uint8_t* wq, const float* s_w, const float* A, float* B,
                                           int64_t d_in, int64_t d_out, int64_t r,
                                           int64_t k_rank, float tau, int64_t k_max,
                                           int32_t* sel_idx, int32_t* n_sel, float* rho,
                                           int32_t* comp_idx, void* ws, size_t ws_bytes,
                                           falq_stream stream) {
  if (!dims_ok(d_in) || d_out < 0 || d_out > ((int64_t)1 << 30) || r < 0 || r > 65536 ||
      k_rank < 0 || k_rank > r || k_max < 0)
    return FALQ_EINVAL;
  if (!scalar(s_w) || !scalar(n_sel)) return FALQ_EINVAL;
  if (d_out * d_in > 0 && !need(wq)) return FALQ_EINVAL;
  if (r * d_in > 0 && !need(A)) return FALQ_EINVAL;
  if (r * d_out > 0 && !need(B)) return FALQ_EINVAL;
  if (d_out > 0 && !need(sel_idx)) return FALQ_EINVAL;
  if (k_rank > 0 && (comp_idx == nullptr || !aligned(comp_idx, 4))) return FALQ_EINVAL;
  if (!opt(rho)) return FALQ_EINVAL;
  if (!ws_ok(ws, ws_bytes, rowwise_proxy_update_topk_rank_workspace_bytes(d_in, d_out, r, k_rank)))
    return FALQ_EINVAL;
  return hip_status(falq::launch_proxy_update_topk_rank(
      wq, s_w, A, B, d_in, d_out, r, k_rank, tau, k_max, sel_idx, n_sel, rho, comp_idx, ws,
      reinterpret_cast<hipStream_t>(stream)));
}

// ---- the baselines: LoRA with a separate adapter branch ----------------------

namespace {
bool sep_dims_ok(int64_t T, int64_t d_in, int64_t d_out, int64_t r) {
  const int64_t r16 = (r + 15) / 16 * 16;      // the rank padded to 16 in the products
  return gemm_dims_ok(T, d_in, d_out) && T % 16 == 0 && r >= 0 && r % 8 == 0 &&
         r <= ((int64_t)1 << 20) && gemm_dims_ok(T, d_in, r16) && gemm_dims_ok(T, r16, d_out);
}
bool bf16_dims_ok(int64_t T, int64_t d_in, int64_t d_out, int64_t r) {
  return sep_dims_ok(T, d_in, d_out, r) && T % 64 == 0 && d_in % 64 == 0 && d_out % 64 == 0;
}
}  // namespace

size_t lora_separate_fp8_saved_bytes(int64_t T, int64_t d_in, int64_t d_out, int64_t r) {
  if (!sep_dims_ok(T, d_in, d_out, r)) return 0;
  return falq::lora_sep_saved_bytes(T, d_in, d_out, r);
}

size_t lora_separate_fp8_workspace_bytes(int64_t T, int64_t d_in, int64_t d_out, int64_t r) {
  if (!sep_dims_ok(T, d_in, d_out, r)) return 0;
  return falq::lora_sep_ws_bytes(T, d_in, d_out, r);
}

falq_status lora_separate_fp8_fwd(const uint8_t* xq, const float* s_x, const uint8_t* wq,
                                  const float* s_w, const float* A, const float* B, int64_t T,
                                  int64_t d_in, int64_t d_out, int64_t r, float* y, void* saved,
                                  size_t saved_bytes, void* ws, size_t ws_bytes,
                                  falq_stream stream) {
  if (!sep_dims_ok(T, d_in, d_out, r)) return FALQ_EINVAL;
  if (!scalar(s_x) || !scalar(s_w)) return FALQ_EINVAL;
  if (T * d_in > 0 && !need(xq)) return FALQ_EINVAL;
  if (d_out * d_in > 0 && !need(wq)) return FALQ_EINVAL;
  if (T * d_out > 0 && !need(y)) return FALQ_EINVAL;
  if (r * d_in > 0 && !need(A)) return FALQ_EINVAL;
  if (r * d_out > 0 && !need(B)) return FALQ_EINVAL;
  if (!ws_ok(saved, saved_bytes, falq::lora_sep_saved_bytes(T, d_in, d_out, r)) ||
      !ws_ok(ws, ws_bytes, falq::lora_sep_ws_bytes(T, d_in, d_out, r)))
    return FALQ_EINVAL;
  if (T == 0 || d_out == 0 || d_in == 0) return melded_linear_fwd(xq, s_x, wq, s_w, T, d_in, d_out, y, stream);
  return hip_status(falq::launch_lora_sep_fwd(xq, s_x, wq, s_w, A, B, T, d_in, d_out, r, y,
                                              saved, ws, reinterpret_cast<hipStream_t>(stream)));
}

falq_status lora_separate_fp8_bwd(const uint8_t* gq, const float* s_g, const uint8_t* xq,
                                  const float* s_x, const uint8_t* wq, const float* s_w,
                                  void* saved, size_t saved_bytes, int64_t T, int64_t d_in,
                                  int64_t d_out, int64_t r, float* dx, float* dA, float* dB,
                                  void* ws, size_t ws_bytes, falq_stream stream) {
  if (!sep_dims_ok(T, d_in, d_out, r)) return FALQ_EINVAL;
  if (!scalar(s_g) || !scalar(s_x) || !scalar(s_w)) return FALQ_EINVAL;
  if (T * d_out > 0 && !need(gq)) return FALQ_EINVAL;
  if (T * d_in > 0 && (!need(xq) || !need(dx))) return FALQ_EINVAL;
  if (d_out * d_in > 0 && !need(wq)) return FALQ_EINVAL;
  if (r * d_in > 0 && !need(dA)) return FALQ_EINVAL;
  if (r * d_out > 0 && !need(dB)) return FALQ_EINVAL;
  if (!ws_ok(saved, saved_bytes, falq::lora_sep_saved_bytes(T, d_in, d_out, r)) ||
      !ws_ok(ws, ws_bytes, falq::lora_sep_ws_bytes(T, d_in, d_out, r)))
    return FALQ_EINVAL;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  if (T == 0 || d_in == 0 || d_out == 0) {
    hipError_t e = hipSuccess;
    if (T * d_in > 0) e = falq::launch_fill_f32(dx, T * d_in, 0.0f, s);
    if (e == hipSuccess) e = falq::launch_fill_f32(dA, r * d_in, 0.0f, s);
    if (e == hipSuccess) e = falq::launch_fill_f32(dB, d_out * r, 0.0f, s);
    return hip_status(e);
  }
  return hip_status(falq::launch_lora_sep_bwd(gq, s_g, xq, s_x, wq, s_w, saved, T, d_in, d_out, r,
                                              dx, dA, dB, ws, s));
}

size_t lora_bf16_saved_bytes(int64_t T, int64_t d_in, int64_t d_out, int64_t r) {
  if (!bf16_dims_ok(T, d_in, d_out, r)) return 0;
  return falq::lora_bf16_saved_bytes(T, r);
}

size_t lora_bf16_workspace_bytes(int64_t T, int64_t d_in, int64_t d_out, int64_t r) {
  if (!bf16_dims_ok(T, d_in, d_out, r)) return 0;
  return falq::lora_bf16_ws_bytes(T, d_in, d_out, r);
}

falq_status lora_bf16_fwd(const float* x, const uint8_t* xq, const float* s_x, const uint8_t* wq,
                          const float* s_w, const float* A, const float* B, int64_t T,
                          int64_t d_in, int64_t d_out, int64_t r, float* y, void* saved,
                          size_t saved_bytes, void* ws, size_t ws_bytes, falq_stream stream) {
  if (!bf16_dims_ok(T, d_in, d_out, r)) return FALQ_EINVAL;
  if (!scalar(s_x) || !scalar(s_w)) return FALQ_EINVAL;
  if (T * d_in > 0 && (!need(xq) || !need(x))) return FALQ_EINVAL;
  if (d_out * d_in > 0 && !need(wq)) return FALQ_EINVAL;
  if (T * d_out > 0 && !need(y)) return FALQ_EINVAL;
  if (r * d_in > 0 && !need(A)) return FALQ_EINVAL;
  if (r * d_out > 0 && !need(B)) return FALQ_EINVAL;
  if (!ws_ok(saved, saved_bytes, falq::lora_bf16_saved_bytes(T, r)) ||
      !ws_ok(ws, ws_bytes, falq::lora_bf16_ws_bytes(T, d_in, d_out, r)))
    return FALQ_EINVAL;
  if (T == 0 || d_out == 0 || d_in == 0) return melded_linear_fwd(xq, s_x, wq, s_w, T, d_in, d_out, y, stream);
  return hip_status(falq::launch_lora_bf16_fwd(x, xq, s_x, wq, s_w, A, B, T, d_in, d_out, r, y,
                                               saved, ws, reinterpret_cast<hipStream_t>(stream)));
}

falq_status lora_bf16_bwd(const float* dy, const uint8_t* gq, const float* s_g, const float* x,
                          const uint8_t* wq, const float* s_w, const float* A, const float* B,
                          const void* saved, size_t saved_bytes, int64_t T, int64_t d_in,
                          int64_t d_out, int64_t r, float* dx, float* dA, float* dB, void* ws,
                          size_t ws_bytes, falq_stream stream) {
  if (!bf16_dims_ok(T, d_in, d_out, r)) return FALQ_EINVAL;
  if (!scalar(s_g) || !scalar(s_w)) return FALQ_EINVAL;
  if (T * d_out > 0 && (!need(gq) || !need(dy))) return FALQ_EINVAL;
  if (T * d_in > 0 && (!need(x) || !need(dx))) return FALQ_EINVAL;
  if (d_out * d_in > 0 && !need(wq)) return FALQ_EINVAL;
  if (r * d_in > 0 && (!need(A) || !need(dA))) return FALQ_EINVAL;
  if (r * d_out > 0 && (!need(B) || !need(dB))) return FALQ_EINVAL;
  if (!ws_ok(saved, saved_bytes, falq::lora_bf16_saved_bytes(T, r)) ||
      !ws_ok(ws, ws_bytes, falq::lora_bf16_ws_bytes(T, d_in, d_out, r)))
    return FALQ_EINVAL;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  if (T == 0 || d_in == 0 || d_out == 0) {
    hipError_t e = hipSuccess;
    if (T * d_in > 0) e = falq::launch_fill_f32(dx, T * d_in, 0.0f, s);
    if (e == hipSuccess) e = falq::launch_fill_f32(dA, r * d_in, 0.0f, s);
    if (e == hipSuccess) e = falq::launch_fill_f32(dB, d_out * r, 0.0f, s);
    return hip_status(e);
  }
  return hip_status(falq::launch_lora_bf16_bwd(dy, gq, s_g, x, wq, s_w, A, B, saved, T, d_in,
                                               d_out, r, dx, dA, dB, ws, s));
}

// ---- U formed with the forward product, V with the dX product ----------------

int melded_linear_xa_fused(int64_t T, int64_t d_in, int64_t d_out, int64_t r) {
  if (!gemm_dims_ok(T, d_in, d_out) || T <= 0 || r <= 0 || r > ((int64_t)1 << 20)) return 0;
  return falq::gemm_fp8_nt_fuses_second(d_out, d_in, r) &&
         falq::gemm_fp8_nt_fuses_second(d_in, d_out, r) &&
         !falq::adapter_wide_route(T, d_in, d_out, r);
}

size_t melded_linear_fwd_xa_workspace_bytes(int64_t T, int64_t d_in, int64_t d_out, int64_t r) {
  if (T < 0 || d_in < 0 || d_out < 0 || r < 0) return 0;
  return falq::fwd_xa_ws_bytes(T, d_in, d_out, r);
}

falq_status melded_linear_fwd_xa(const uint8_t* xq, const float* s_x, const uint8_t* wq,
                                 const float* s_w, const float* A, int64_t T, int64_t d_in,
                                 int64_t d_out, int64_t r, float* y, float* xa, void* ws,
                                 size_t ws_bytes, falq_stream stream) {
  if (!gemm_dims_ok(T, d_in, d_out) || r < 0 || r > ((int64_t)1 << 20)) return FALQ_EINVAL;
  if (!scalar(s_x) || !scalar(s_w)) return FALQ_EINVAL;
  if (T * d_in > 0 && !need(xq)) return FALQ_EINVAL;
  if (d_out * d_in > 0 && !need(wq)) return FALQ_EINVAL;
  if (T * d_out > 0 && !need(y)) return FALQ_EINVAL;
  if (r * d_in > 0 && !need(A)) return FALQ_EINVAL;
  if (T * r > 0 && !need(xa)) return FALQ_EINVAL;
  if (!ws_ok(ws, ws_bytes, falq::fwd_xa_ws_bytes(T, d_in, d_out, r))) return FALQ_EINVAL;
  return hip_status(falq::launch_fwd_xa(xq, s_x, wq, s_w, A, T, d_in, d_out, r, y, xa, ws,
                                        reinterpret_cast<hipStream_t>(stream)));
}

size_t adapter_pieces_bytes(int64_t r, int64_t d_in) { return falq::adapter_pieces_bytes(r, d_in); }

falq_status adapter_pieces(const float* A, int64_t r, int64_t d_in, void* pieces,
                           size_t pieces_bytes, falq_stream stream) {
  if (!falq::adapter_pieces_ok(r, d_in) || !need(A)) return FALQ_EINVAL;
  if (!need(pieces) || pieces_bytes < falq::adapter_pieces_bytes(r, d_in)) return FALQ_EINVAL;
  return hip_status(
      falq::launch_adapter_pieces(A, r, d_in, pieces, reinterpret_cast<hipStream_t>(stream)));
}

falq_status adapter_step_pieces(float* A, float* B, const float* dA, const float* dB, int64_t r,
                                int64_t d_in, int64_t d_out, float lr, void* pieces,
                                size_t pieces_bytes, falq_stream stream) {
  if (!falq::adapter_pieces_ok(r, d_in) || d_out < 0 || d_out > ((int64_t)1 << 31))
    return FALQ_EINVAL;
  if (!need(A) || !need(dA)) return FALQ_EINVAL;
  if (d_out > 0 && (!need(B) || !need(dB))) return FALQ_EINVAL;
  if (!need(pieces) || pieces_bytes < falq::adapter_pieces_bytes(r, d_in)) return FALQ_EINVAL;
  return hip_status(falq::launch_sgd_pieces(A, B, dA, dB, r, d_in, d_out, lr, pieces,
                                            reinterpret_cast<hipStream_t>(stream)));
}

falq_status melded_linear_fwd_xa_pieces(const uint8_t* xq, const float* s_x, const uint8_t* wq,
                                        const float* s_w, const void* pieces, size_t pieces_bytes,
                                        int64_t T, int64_t d_in, int64_t d_out, int64_t r,
                                        float* y, float* xa, falq_stream stream) {
  if (!gemm_dims_ok(T, d_in, d_out) || T < 0 || !falq::adapter_pieces_ok(r, d_in))
    return FALQ_EINVAL;
  if (!falq::gemm_fp8_nt_fuses_second(d_out, d_in, r)) return FALQ_EINVAL;
  if (!scalar(s_x) || !scalar(s_w)) return FALQ_EINVAL;
  if (T > 0 && (!need(xq) || !need(y) || !need(xa))) return FALQ_EINVAL;
  if (!need(wq)) return FALQ_EINVAL;
  if (!need(pieces) || pieces_bytes < falq::adapter_pieces_bytes(r, d_in)) return FALQ_EINVAL;
  return hip_status(falq::launch_fwd_xa_pieces(xq, s_x, wq, s_w, pieces, T, d_in, d_out, r, y, xa,
                                               reinterpret_cast<hipStream_t>(stream)));
}

size_t melded_linear_bwd_xa_workspace_bytes(int64_t T, int64_t d_in, int64_t d_out, int64_t r) {
  if (T < 0 || d_in < 0 || d_out < 0 || r < 0) return 0;
  const size_t wt = align_up((size_t)d_in * (size_t)d_out, 256);      // W~^T for dX
  return wt + (falq::adapter_wide_route(T, d_in, d_out, r)
                   ? falq::adapter_wide_ws_bytes(T, d_in, d_out, r)
                   : falq::bwd_xa_ws_bytes(T, d_in, d_out, r));
}

}  // extern "C"

namespace {

// melded_linear_bwd_xa (wqT == nullptr: W~^T formed from wq in the workspace)
// and melded_linear_bwd_xa_t (wq == nullptr: the caller's W~^T)
falq_status bwd_xa_impl(const uint8_t* gq, int g_fmt, const float* s_g, const uint8_t* xq,
                        const float* s_x, const uint8_t* wq, const uint8_t* wqT, const float* s_w,
                        const float* A, const float* B, const float* xa, int64_t T, int64_t d_in,
                        int64_t d_out, int64_t r, float* dx, float* dA, float* dB, void* ws,
                        size_t ws_bytes, falq_stream stream) {
  if (!fmt_ok(g_fmt)) return FALQ_EINVAL;
  if (!gemm_dims_ok(T, d_in, d_out) || r < 0 || r > ((int64_t)1 << 20)) return FALQ_EINVAL;
  if (!scalar(s_g) || !scalar(s_x) || !scalar(s_w)) return FALQ_EINVAL;
  if (T * d_out > 0 && !need(gq)) return FALQ_EINVAL;
  if (T * d_in > 0 && !need(xq)) return FALQ_EINVAL;
  if (d_out * d_in > 0 && dx && !need(wqT ? wqT : wq)) return FALQ_EINVAL;
  if (!opt(dx) || !opt(dA)) return FALQ_EINVAL;
  if (r * d_in > 0 && !need(A)) return FALQ_EINVAL;
  if (r * d_out > 0 && (!need(B) || !need(dB))) return FALQ_EINVAL;
  if (T * r > 0 && !need(xa)) return FALQ_EINVAL;
  if (!ws_ok(ws, ws_bytes, melded_linear_bwd_xa_workspace_bytes(T, d_in, d_out, r)))
    return FALQ_EINVAL;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  uint8_t* base = reinterpret_cast<uint8_t*>(ws);
  const size_t wt_bytes = align_up((size_t)d_in * (size_t)d_out, 256);
  const bool grads = r > 0 && T > 0 && d_in > 0 && d_out > 0;
  const bool wide = grads && falq::adapter_wide_route(T, d_in, d_out, r);
  const bool gemm_dx = dx && T * d_in > 0 && d_out > 0;
  hipError_t e = hipSuccess;
  // the dX product's W~^T: the caller's, or formed in the workspace
  const uint8_t* wt = wqT ? wqT : base;
  if (gemm_dx && (!grads || wide) && !wqT) e = falq::launch_transpose_u8(wq, d_out, d_in, base, s);
  if (e != hipSuccess) return FALQ_EHIP;
  if (!grads) {
    if (gemm_dx) e = falq::launch_gemm_fp8_nt(gq, d_out, wt, d_out, dx, d_in, T, d_in, d_out,
                                              s_g, s_w, s, g_fmt);
    else if (dx && T * d_in > 0) e = falq::launch_fill_f32(dx, T * d_in, 0.0f, s);
    if (e == hipSuccess && r > 0) {
      if (d_out > 0) e = falq::launch_fill_f32(dB, d_out * r, 0.0f, s);
      if (e == hipSuccess && dA && d_in > 0) e = falq::launch_fill_f32(dA, r * d_in, 0.0f, s);
    }
    return hip_status(e);
  }
  if (wide) {
    if (gemm_dx) e = falq::launch_gemm_fp8_nt(gq, d_out, wt, d_out, dx, d_in, T, d_in, d_out,
                                              s_g, s_w, s, g_fmt);
    if (e == hipSuccess)
      e = falq::launch_adapter_grads_wide(gq, g_fmt, s_g, xq, s_x, A, B, T, d_in, d_out, r, dA,
                                          dB, base + wt_bytes, s);
    return hip_status(e);
  }
  // the transpose of W~ runs inside launch_bwd_xa's preparation launch
  return hip_status(falq::launch_bwd_xa(gq, g_fmt, s_g, xq, s_x, wq, base, s_w, B, xa, T, d_in,
                                        d_out, r, gemm_dx ? dx : nullptr, dA, dB,
                                        base + wt_bytes, s, wqT));
}

}  // namespace

extern "C" {

falq_status melded_linear_bwd_xa(const uint8_t* gq, int g_fmt, const float* s_g,
                                 const uint8_t* xq, const float* s_x, const uint8_t* wq,
                                 const float* s_w, const float* A, const float* B,
                                 const float* xa, int64_t T, int64_t d_in, int64_t d_out,
                                 int64_t r, float* dx, float* dA, float* dB, void* ws,
                                 size_t ws_bytes, falq_stream stream) {
  return bwd_xa_impl(gq, g_fmt, s_g, xq, s_x, wq, nullptr, s_w, A, B, xa, T, d_in, d_out, r, dx,
                     dA, dB, ws, ws_bytes, stream);
}

falq_status melded_linear_bwd_xa_t(const uint8_t* gq, int g_fmt, const float* s_g,
                                   const uint8_t* xq, const float* s_x, const uint8_t* wqT,
                                   const float* s_w, const float* A, const float* B,
                                   const float* xa, int64_t T, int64_t d_in, int64_t d_out,
                                   int64_t r, float* dx, float* dA, float* dB, void* ws,
                                   size_t ws_bytes, falq_stream stream) {
  if (d_out * d_in > 0 && dx && wqT == nullptr) return FALQ_EINVAL;
  return bwd_xa_impl(gq, g_fmt, s_g, xq, s_x, nullptr, wqT, s_w, A, B, xa, T, d_in, d_out, r, dx,
                     dA, dB, ws, ws_bytes, stream);
}

falq_status fp8_transpose(const uint8_t* q, int64_t rows, int64_t cols, uint8_t* qT,
                          falq_stream stream) {
  if (!dims_ok(rows) || !dims_ok(cols)) return FALQ_EINVAL;
  if (rows * cols == 0) return FALQ_OK;
  if (!need(q) || !need(qT) || q == qT) return FALQ_EINVAL;
  return hip_status(
      falq::launch_transpose_u8(q, rows, cols, qT, reinterpret_cast<hipStream_t>(stream)));
}

}  // extern "C"
