// Internal launchers of the gfx950 kernels (host side).  Each returns
// hipSuccess or the launch error; arguments are validated by api.cpp.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace falq {

// ---- fp8_quantize: amax partials + cast ---------------------------------
constexpr int kQzMaxParts = 2048;
size_t quantize_ws_bytes();
// fmt 0: E4M3 (s = 448 / amax), 1: E5M2 (s = 57344 / amax), 2: FP4 E2M1
// (s = 6 / amax; two codes per byte, the lower index in the low nibble; n even)
hipError_t launch_quantize(const void* x, int dtype, int fmt, int64_t n, const float* scale_in,
                           uint8_t* q, float* scale, float* amax, int32_t* nonfinite,
                           void* ws, hipStream_t s);

// out[i] = dec(q[i]) / *s (float32, correctly rounded division)
hipError_t launch_dequantize(const uint8_t* q, int64_t n, const float* s, float* out,
                             hipStream_t st);

// ---- FP8 GEMMs ------------------------------------------------------------
// C[M x N] (fp32, row stride ldc) = dec(A)[M x K] . dec(B)[N x K]^T / (sa * sb);
// A in E4M3 (a_fmt 0) or E5M2 (a_fmt 1), B in E4M3
hipError_t launch_gemm_fp8_nt(const uint8_t* A, int64_t lda, const uint8_t* B, int64_t ldb,
                              float* C, int64_t ldc, int64_t M, int64_t N, int64_t K,
                              const float* sa, const float* sb, hipStream_t s, int a_fmt = 0);
// FP4 E2M1 operands, two codes per byte: C = dec(A) . dec(B)^T / (sa * sb),
// Kb = bytes per row (a multiple of 128: 256 values)
hipError_t launch_gemm_fp4_nt(const uint8_t* A, int64_t lda, const uint8_t* B, int64_t ldb,
                              float* C, int64_t ldc, int64_t M, int64_t N, int64_t Kb,
                              const float* sa, const float* sb, hipStream_t s);
// The same product plus Cu[M x R] = dec(A) . dec(Bu)[R x K]^T / (sa * sbu) in
// the same launch (the DMA kernel's extra units); only where
// gemm_fp8_nt_fuses_second(N, K, R) holds
bool gemm_fp8_nt_fuses_second(int64_t N, int64_t K, int64_t R);
hipError_t launch_gemm_fp8_nt_second(const uint8_t* A, int64_t lda, const uint8_t* B, int64_t ldb,
                                     float* C, int64_t ldc, int64_t M, int64_t N, int64_t K,
                                     const float* sa, const float* sb, const uint8_t* Bu,
                                     int64_t ldbu, int64_t R, float* Cu, int64_t ldcu,
                                     const float* sbu, hipStream_t s);
// out[cols x rows] = in[rows x cols]^T (bytes; rows and cols multiples of 16)
hipError_t launch_transpose_u8(const uint8_t* in, int64_t rows, int64_t cols, uint8_t* out,
                               hipStream_t s);

// ---- adapter gradients ----------------------------------------------------
size_t adapter_grad_ws_bytes(int64_t T, int64_t d_in, int64_t d_out, int64_t r);
hipError_t launch_adapter_grads(const uint8_t* gq, const float* s_g, const uint8_t* xq,
                                const float* s_x, const float* A, const float* B,
                                int64_t T, int64_t d_in, int64_t d_out, int64_t r,
                                float* dA, float* dB, void* ws, hipStream_t s, int g_fmt = 0,
                                bool presplit = false);
// The backward's preparation in one launch: W~^T into wt (skipped when wt is
// null) and, when r, T, d_in and d_out are all positive, the adapter
// gradients' float-operand splits into their workspace ws (B's only with
// want_da); launch_adapter_grads with presplit then skips its own split.
hipError_t launch_bwd_prep(const uint8_t* wq, uint8_t* wt, const float* A, const float* B,
                           int64_t T, int64_t d_in, int64_t d_out, int64_t r, bool want_da,
                           void* ws, hipStream_t s);

// frozen FP8 factor A~: u [T x r] = dec(X~) dec(A~)^T / (s_x s_a)
size_t frozen_u_ws_bytes(int64_t T, int64_t d_in, int64_t r);
hipError_t launch_frozen_u(const uint8_t* xq, const float* s_x, const uint8_t* aq,
                           const float* s_a, int64_t T, int64_t d_in, int64_t r, float* u,
                           void* ws, hipStream_t s);
// dB [d_out x r] = dec(G~)^T u / s_g
size_t frozen_db_ws_bytes(int64_t T, int64_t d_out, int64_t r);
hipError_t launch_frozen_db(const uint8_t* gq, const float* s_g, const float* u, int64_t T,
                            int64_t d_out, int64_t r, float* dB, void* ws, hipStream_t s,
                            int g_fmt = 0);

// ---- SGD ------------------------------------------------------------------
// two tensors in one launch (either may be empty); 16-byte aligned pointers
hipError_t launch_sgd2(float* pa, const float* ga, int64_t na, float* pb, const float* gb,
                       int64_t nb, float lr, hipStream_t s);

// ---- AdamW ----------------------------------------------------------------
// float32 scalars of one AdamW step (derived on the host, see api.cpp)
struct AdamWScalars {
  float b1, b2, omb1, omb2, eps, decay, step_size, inv_bc2;
};
// one tensor: parameters, gradient, first and second moments (in place)
struct AdamWTensor {
  float* p;
  const float* g;
  float* m;
  float* v;
  int64_t n;
};
// optimizer state in device memory (64 bytes; all zero before the first step)
struct AdamWState {
  int64_t t;             // steps taken
  double pow1, pow2;     // beta1^t, beta2^t (running products)
  AdamWScalars sc;       // the float32 scalars of step t
  uint32_t pad[2];
};
static_assert(sizeof(AdamWState) == 64, "64-byte AdamW state");
// advance the state one step, then update the two tensors (either may be
// empty: n == 0); 16-byte aligned
hipError_t launch_adamw2(const AdamWTensor& a, const AdamWTensor& b, AdamWState* st, float lr,
                         float beta1, float beta2, float eps, float wd, hipStream_t s);

// ---- row-wise proxy update -------------------------------------------------
size_t proxy_ws_bytes(int64_t d_in, int64_t d_out, int64_t r);
hipError_t launch_proxy_update(uint8_t* wq, const float* s_w, const float* A, float* B,
                               int64_t d_in, int64_t d_out, int64_t r, float tau,
                               int64_t k_max, int32_t* sel_idx, int32_t* n_sel, float* rho,
                               void* ws, hipStream_t s);

// the same with the chain over ranks kidx[0..r) (ascending) of an adapter whose
// B rows hold rs values (A rows indexed by kidx too)
hipError_t launch_proxy_update_ranks(uint8_t* wq, const float* s_w, const float* A, float* B,
                                     int64_t d_in, int64_t d_out, int64_t r, int64_t rs,
                                     const int32_t* kidx, float tau, int64_t k_max,
                                     int32_t* sel_idx, int32_t* n_sel, float* rho, void* ws,
                                     hipStream_t s);
// proxy update over the top-k rank components (k <= r <= 65536): K [k] int32 output
size_t proxy_topk_rank_ws_bytes(int64_t d_in, int64_t d_out, int64_t r, int64_t k);
hipError_t launch_proxy_update_topk_rank(uint8_t* wq, const float* s_w, const float* A, float* B,
                                         int64_t d_in, int64_t d_out, int64_t r, int64_t k,
                                         float tau, int64_t k_max, int32_t* sel_idx,
                                         int32_t* n_sel, float* rho, int32_t* comp_idx,
                                         void* ws, hipStream_t s);

// ---- misc -----------------------------------------------------------------
hipError_t launch_fill_f32(float* p, int64_t n, float v, hipStream_t s);

inline size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

}  // namespace falq
