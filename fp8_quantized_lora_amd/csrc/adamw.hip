// 32-bit AdamW on the adapter factors (FALQON OpenReview rebuttal, thread 3,
// reply W3.1: the runs train with a 32-bit AdamW optimizer).  AdamW is Adam
// with decoupled weight decay (the decay multiplies the weights instead of
// being added to the gradient); weights and both moments are float32.
//
// Elementwise over A and B in one launch.  Every operation is rounded on its
// own (the library is built without fp contraction), in this order:
//     m'  = b1*m + omb1*g
//     v'  = b2*v + (omb2*g)*g
//     den = sqrt(v')*inv_bc2 + eps
//     p'  = decay*p - step_size*(m'/den)
// with sqrt and the division correctly rounded.  The step-dependent scalars
// come from a 64-byte optimizer state in device memory, advanced by a
// one-thread kernel before the update: step t, the running float64 products
// beta1^t and beta2^t, and the float32 scalars of the step (decay =
// 1 - lr*wd, step_size = lr / (1 - beta1^t), inv_bc2 = 1 / sqrt(1 -
// beta2^t), each computed in float64 and rounded once).  Nothing comes from
// the host per step, so a captured graph replays consecutive steps.
// Memory: 16 bytes read and 12 bytes written per element, float4 at a time.
#include "common.hpp"
#include "kernels.hpp"

#include <algorithm>

namespace falq {
namespace {

constexpr int kThreads = 256;

// the optimizer state (AdamWState in kernels.hpp): all zero = before step 1
__global__ void adamw_advance_kernel(AdamWState* st, float lr, float beta1, float beta2, float eps,
                                     float wd) {
  const bool first = st->t == 0;
  const double p1 = (first ? 1.0 : st->pow1) * (double)beta1;
  const double p2 = (first ? 1.0 : st->pow2) * (double)beta2;
  st->t += 1;
  st->pow1 = p1;
  st->pow2 = p2;
  AdamWScalars c;
  c.b1 = beta1;
  c.b2 = beta2;
  c.omb1 = (float)(1.0 - (double)beta1);
  c.omb2 = (float)(1.0 - (double)beta2);
  c.eps = eps;
  c.decay = (float)(1.0 - (double)lr * (double)wd);
  c.step_size = (float)((double)lr / (1.0 - p1));
  c.inv_bc2 = (float)(1.0 / sqrt(1.0 - p2));
  st->sc = c;
}

__device__ __forceinline__ void adam1(float& p, float g, float& m, float& v,
                                      const AdamWScalars& c) {
  m = c.b1 * m + c.omb1 * g;
  v = c.b2 * v + (c.omb2 * g) * g;
  // sqrtf and '/' are the correctly rounded operations in HIP device code
  // (no approximate-math flags are used in this library)
  const float den = sqrtf(v) * c.inv_bc2 + c.eps;
  p = c.decay * p - c.step_size * (m / den);
}

// grid-stride over the float4 items of a, then of b; the scalar tails (n % 4)
// are done by workgroup 0
__global__ __launch_bounds__(kThreads) void adamw_kernel(AdamWTensor a, AdamWTensor b,
                                                         const AdamWState* __restrict__ st) {
  const AdamWScalars c = st->sc;
  const int64_t na4 = a.n / 4, nb4 = b.n / 4;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < na4 + nb4; i += stride) {
    const AdamWTensor& t = i < na4 ? a : b;
    const int64_t j = i < na4 ? i : i - na4;
    float4 p = reinterpret_cast<const float4*>(t.p)[j];
    const float4 g = reinterpret_cast<const float4*>(t.g)[j];
    float4 m = reinterpret_cast<const float4*>(t.m)[j];
    float4 v = reinterpret_cast<const float4*>(t.v)[j];
    adam1(p.x, g.x, m.x, v.x, c);
    adam1(p.y, g.y, m.y, v.y, c);
    adam1(p.z, g.z, m.z, v.z, c);
    adam1(p.w, g.w, m.w, v.w, c);
    reinterpret_cast<float4*>(t.p)[j] = p;
    reinterpret_cast<float4*>(t.m)[j] = m;
    reinterpret_cast<float4*>(t.v)[j] = v;
  }
  if (blockIdx.x == 0) {
    for (int u = 0; u < 2; ++u) {
      const AdamWTensor& t = u == 0 ? a : b;
      for (int64_t i = t.n / 4 * 4 + threadIdx.x; i < t.n; i += blockDim.x)
        adam1(t.p[i], t.g[i], t.m[i], t.v[i], c);
    }
  }
}

}  // namespace

hipError_t launch_adamw2(const AdamWTensor& a, const AdamWTensor& b, AdamWState* st, float lr,
                         float beta1, float beta2, float eps, float wd, hipStream_t s) {
  adamw_advance_kernel<<<1, 1, 0, s>>>(st, lr, beta1, beta2, eps, wd);
  const AdamWTensor none{nullptr, nullptr, nullptr, nullptr, 0};
  const AdamWTensor ta = a.n > 0 ? a : none, tb = b.n > 0 ? b : none;
  if (ta.n + tb.n > 0) {
    const int64_t blocks =
        std::min<int64_t>((ta.n / 4 + tb.n / 4 + kThreads - 1) / kThreads + 1, 4096);
    adamw_kernel<<<(int)blocks, kThreads, 0, s>>>(ta, tb, st);
  }
  return hipGetLastError();
}

}  // namespace falq
