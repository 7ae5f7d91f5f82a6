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
// the device address of this device's file-scope scratch array (looked up once
// per device with hipGetSymbolAddress) and its size; quantize_ws_bytes() fits
constexpr size_t kQuantizeScratchBytes = (size_t)kQzMaxParts * 8;
size_t quantize_scratch_bytes();
// the one-launch route's wait for the exchange words, in ticks of the
// 100 MHz real-time counter; sets it, returns the previous value
uint64_t quantize_wait_ticks(uint64_t ticks);
hipError_t quantize_scratch(void** out);
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
                              const float* sa, const float* sb, hipStream_t s, int a_fmt = 0,
                              int acc = 0, float* splitk_ws = nullptr);
// bytes of split-K partials a product of M x N outputs over K_bytes needs
// (0: it runs unsplit); splitk_ws = nullptr never splits
size_t gemm_splitk_ws_bytes(int64_t M, int64_t N, int64_t K_bytes);
// C (+)= A B^T with bfloat16 operands (K-contiguous, strides and K in
// elements; K a multiple of 64), fp32 accumulation and output; acc != 0 adds
// onto C
hipError_t launch_gemm_bf16_nt(const uint16_t* A, int64_t lda, const uint16_t* B, int64_t ldb,
                               float* C, int64_t ldc, int64_t M, int64_t N, int64_t K,
                               hipStream_t s, int acc = 0, float* splitk_ws = nullptr);

// ---- LoRA layers with a separate adapter branch (the baselines) ------------
size_t lora_sep_saved_bytes(int64_t T, int64_t d_in, int64_t d_out, int64_t r);
size_t lora_sep_ws_bytes(int64_t T, int64_t d_in, int64_t d_out, int64_t r);
size_t lora_bf16_saved_bytes(int64_t T, int64_t r);
size_t lora_bf16_ws_bytes(int64_t T, int64_t d_in, int64_t d_out, int64_t r);
hipError_t launch_lora_sep_fwd(const uint8_t* xq, const float* s_x, const uint8_t* wq,
                               const float* s_w, const float* A, const float* B, int64_t T,
                               int64_t d_in, int64_t d_out, int64_t r, float* y, void* saved,
                               void* ws, hipStream_t s);
hipError_t launch_lora_sep_bwd(const uint8_t* gq, const float* s_g, const uint8_t* xq,
                               const float* s_x, const uint8_t* wq, const float* s_w,
                               void* saved, int64_t T, int64_t d_in, int64_t d_out, int64_t r,
                               float* dx, float* dA, float* dB, void* ws, hipStream_t s);
hipError_t launch_lora_bf16_fwd(const float* x, const uint8_t* xq, const float* s_x,
                                const uint8_t* wq, const float* s_w, const float* A,
                                const float* B, int64_t T, int64_t d_in, int64_t d_out, int64_t r,
                                float* y, void* saved, void* ws, hipStream_t s);
hipError_t launch_lora_bf16_bwd(const float* dy, const uint8_t* gq, const float* s_g,
                                const float* x, const uint8_t* wq, const float* s_w,
                                const float* A, const float* B, const void* saved, int64_t T,
                                int64_t d_in, int64_t d_out, int64_t r, float* dx, float* dA,
                                float* dB, void* ws, hipStream_t s);
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
// C = dec(A) dec(B)^T / (sa sb) as launch_gemm_fp8_nt, and in the same tiles
// Cu [M x R] = dec(A) F^T / sa for a float operand F [R x K] held as
// block-scaled E4M3 pieces (pieces.hpp: planes P [3][prp][K], scale bytes PE,
// prp >= R rounded up to 16, a multiple of 16).  With Po != nullptr the
// second product is written instead as pieces of Cu^T [R x M] (Po
// [3][po_rp][po_kp], scale bytes Eo; po_kp >= M a multiple of 128, zero codes
// past M).  Requires gemm_fp8_nt_fuses_second(N, K, R); a_fmt as
// launch_gemm_fp8_nt.
hipError_t launch_gemm_fp8_nt_pieces(const uint8_t* A, int64_t lda, const uint8_t* B,
                                     int64_t ldb, float* C, int64_t ldc, int64_t M, int64_t N,
                                     int64_t K, const float* sa, const float* sb,
                                     const uint8_t* P, const uint8_t* PE, int64_t prp, int64_t R,
                                     float* Cu, int64_t ldcu, uint8_t* Po, uint8_t* Eo,
                                     int64_t po_rp, int64_t po_kp, hipStream_t s, int a_fmt);
// out[cols x rows] = in[rows x cols]^T (bytes; rows and cols multiples of 16)
hipError_t launch_transpose_u8(const uint8_t* in, int64_t rows, int64_t cols, uint8_t* out,
                               hipStream_t s);

// ---- adapter gradients ----------------------------------------------------
size_t adapter_grad_ws_bytes(int64_t T, int64_t d_in, int64_t d_out, int64_t r);
// U = X^ A^T with the forward product, V = G^ B with the dX product
size_t fwd_xa_ws_bytes(int64_t T, int64_t d_in, int64_t d_out, int64_t r);
hipError_t launch_fwd_xa(const uint8_t* xq, const float* s_x, const uint8_t* wq, const float* s_w,
                         const float* A, int64_t T, int64_t d_in, int64_t d_out, int64_t r,
                         float* y, float* xa, void* ws, hipStream_t s);
// A's pieces (pieces.hpp layout, rows padded to 16) in a caller's buffer:
// formed from A, or left by an SGD step on A and B; the forward from them
bool adapter_pieces_ok(int64_t r, int64_t d_in);
size_t adapter_pieces_bytes(int64_t r, int64_t d_in);
hipError_t launch_adapter_pieces(const float* A, int64_t r, int64_t d_in, void* pieces,
                                 hipStream_t s);
hipError_t launch_sgd_pieces(float* A, float* B, const float* dA, const float* dB, int64_t r,
                             int64_t d_in, int64_t d_out, float lr, void* pieces, hipStream_t s);
hipError_t launch_fwd_xa_pieces(const uint8_t* xq, const float* s_x, const uint8_t* wq,
                                const float* s_w, const void* pieces, int64_t T, int64_t d_in,
                                int64_t d_out, int64_t r, float* y, float* xa, hipStream_t s);
// dB = G^^T U and dA = V^T X^ from U, V [T x r] (float32) on the FP8 matrix
// cores with the LDS transpose read (token_grad.hip); dA may be null.
// Needs d_in and d_out multiples of 128.
bool token_grads_ok(int64_t T, int64_t d_in, int64_t d_out, int64_t r);
size_t token_grads_ws_bytes(int64_t T, int64_t d_in, int64_t d_out, int64_t r);
// U, V [T x r] row-major floats; with u_ready (v_ready) their pieces are in
// place already (token_grads_pieces: where) and u (v) is not read.
hipError_t launch_token_grads(const uint8_t* gq, int g_fmt, const float* s_g, const uint8_t* xq,
                              const float* s_x, const float* u, bool u_ready, const float* v,
                              bool v_ready, int64_t T, int64_t d_in, int64_t d_out, int64_t r,
                              float* dA, float* dB, void* ws, hipStream_t s);
// the pieces' place in the workspace (which = 0: U, 1: V): planes
// [3][Rp][Tp] at *P, scale bytes [Tp / 128][Rp][4] at *E (pieces.hpp)
void token_grads_pieces(void* ws, int64_t T, int64_t d_in, int64_t d_out, int64_t r, int which,
                        uint8_t** P, uint8_t** E, int64_t* Rp, int64_t* Tp);
size_t bwd_xa_ws_bytes(int64_t T, int64_t d_in, int64_t d_out, int64_t r);
// wq is transposed into wt (d_in x d_out bytes) when dx is wanted, unless
// the caller hands the transpose in as wt_given (then wq and wt are unused)
hipError_t launch_bwd_xa(const uint8_t* gq, int g_fmt, const float* s_g, const uint8_t* xq,
                         const float* s_x, const uint8_t* wq, uint8_t* wt, const float* s_w,
                         const float* B, const float* xa, int64_t T, int64_t d_in, int64_t d_out,
                         int64_t r, float* dx, float* dA, float* dB, void* ws, hipStream_t s,
                         const uint8_t* wt_given = nullptr);
// large ranks: through the full weight gradient M = G^^T X^ (adapter_grad_wide.hip)
bool adapter_wide_route(int64_t T, int64_t d_in, int64_t d_out, int64_t r);
size_t adapter_wide_ws_bytes(int64_t T, int64_t d_in, int64_t d_out, int64_t r);
hipError_t launch_adapter_grads_wide(const uint8_t* gq, int g_fmt, const float* s_g,
                                     const uint8_t* xq, const float* s_x, const float* A,
                                     const float* B, int64_t T, int64_t d_in, int64_t d_out,
                                     int64_t r, float* dA, float* dB, void* ws, hipStream_t s);
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
  double pow1, pow2;     // beta1^t, beta2^t (leading double of each; informational)
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
// B rows hold rs values (A rows indexed by kidx too); with wt != nullptr the
// update also writes wt [d_in x d_out] = the updated wq^T (d_in, d_out
// multiples of 16)
hipError_t launch_proxy_update_ranks(uint8_t* wq, const float* s_w, const float* A, float* B,
                                     int64_t d_in, int64_t d_out, int64_t r, int64_t rs,
                                     const int32_t* kidx, float tau, int64_t k_max,
                                     int32_t* sel_idx, int32_t* n_sel, float* rho, void* ws,
                                     hipStream_t s, uint8_t* wt = nullptr);
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
