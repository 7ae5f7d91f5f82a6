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
// one-thread kernel before the update: step t, then the float32 scalars of
// step t (decay = 1 - lr*wd, step_size = lr / (1 - beta1^t), inv_bc2 =
// 1 / sqrt(1 - beta2^t), omb = 1 - beta), each the value of its formula
// rounded once to float32.  The formulas are evaluated in double-double
// arithmetic (about 104 significant bits; beta^t by repeated squaring from
// t), so the single rounding to float32 is the correct one unless the exact
// value lies within ~2^-95 of a float32 rounding boundary.  Nothing comes
// from the host per step, so a captured graph replays consecutive steps.
// Memory: 16 bytes read and 12 bytes written per element, float4 at a time.
#include "common.hpp"
#include "kernels.hpp"

#include <algorithm>

namespace falq {
namespace {

constexpr int kThreads = 256;

// ---- double-double arithmetic (value = hi + lo, |lo| <= ulp(hi) / 2) ------
// Error-free transformations: a + b = s + e exactly (Knuth's two-sum), and
// a * b = p + e exactly (the product's error from one fused multiply-add).
// The library is built without fp contraction, so the compiler neither fuses
// nor reassociates these sums.
struct dd {
  double hi, lo;
};
__device__ dd two_sum(double a, double b) {
  const double s = a + b, bb = s - a;
  return {s, (a - (s - bb)) + (b - bb)};
}
__device__ dd fast_two_sum(double a, double b) {      // |a| >= |b|
  const double s = a + b;
  return {s, b - (s - a)};
}
__device__ dd dd_add(dd a, dd b) {
  dd s = two_sum(a.hi, b.hi);
  const dd t = two_sum(a.lo, b.lo);
  s = fast_two_sum(s.hi, s.lo + t.hi);
  return fast_two_sum(s.hi, s.lo + t.lo);
}
__device__ dd dd_neg(dd a) { return {-a.hi, -a.lo}; }
__device__ dd dd_mul(dd a, dd b) {
  const double p = a.hi * b.hi, e = fma(a.hi, b.hi, -p);
  return fast_two_sum(p, e + (a.hi * b.lo + a.lo * b.hi));
}
// a / b by long division: three quotient digits, each from the remainder
__device__ dd dd_div(dd a, dd b) {
  const double q1 = a.hi / b.hi;
  dd r = dd_add(a, dd_neg(dd_mul(b, {q1, 0.0})));
  const double q2 = r.hi / b.hi;
  r = dd_add(r, dd_neg(dd_mul(b, {q2, 0.0})));
  const double q3 = r.hi / b.hi;
  return dd_add(fast_two_sum(q1, q2), {q3, 0.0});
}
// sqrt(a), a > 0: one Newton correction of the double square root
__device__ dd dd_sqrt(dd a) {
  const double x = sqrt(a.hi);
  const dd r = dd_add(a, dd_neg(dd_mul({x, 0.0}, {x, 0.0})));
  return fast_two_sum(x, r.hi / (2.0 * x));
}
// b^t, t >= 0, by repeated squaring
__device__ dd dd_pow(double b, int64_t t) {
  dd r{1.0, 0.0}, p{b, 0.0};
  while (t > 0) {
    if (t & 1) r = dd_mul(r, p);
    p = dd_mul(p, p);
    t >>= 1;
  }
  return r;
}
// hi + lo rounded once to float32.  (float)hi is the nearest float to hi; it
// can differ from the nearest float to hi + lo only when hi sits exactly on
// a midpoint between two floats (|lo| is below hi's double spacing), where
// the sign of lo decides.
__device__ float dd_to_f32(dd a) {
  const float f = (float)a.hi;
  if (a.lo != 0.0 && __builtin_isfinite(f)) {
    const float below = nextafterf(f, -__builtin_inff()), above = nextafterf(f, __builtin_inff());
    if (a.hi == 0.5 * ((double)below + (double)f) && a.lo < 0.0) return below;
    if (a.hi == 0.5 * ((double)f + (double)above) && a.lo > 0.0) return above;
  }
  return f;
}

// the optimizer state (AdamWState in kernels.hpp): all zero = before step 1
__global__ void adamw_advance_kernel(AdamWState* st, float lr, float beta1, float beta2, float eps,
                                     float wd) {
  const int64_t t = st->t + 1;
  const dd one{1.0, 0.0};
  const dd p1 = dd_pow((double)beta1, t), p2 = dd_pow((double)beta2, t);
  st->t = t;
  st->pow1 = p1.hi;
  st->pow2 = p2.hi;
  AdamWScalars c;
  c.b1 = beta1;
  c.b2 = beta2;
  c.omb1 = dd_to_f32(two_sum(1.0, -(double)beta1));
  c.omb2 = dd_to_f32(two_sum(1.0, -(double)beta2));
  c.eps = eps;
  // lr * wd is exact in double (two 24-bit significands)
  c.decay = dd_to_f32(two_sum(1.0, -((double)lr * (double)wd)));
  c.step_size = dd_to_f32(dd_div({(double)lr, 0.0}, dd_add(one, dd_neg(p1))));
  c.inv_bc2 = dd_to_f32(dd_div(one, dd_sqrt(dd_add(one, dd_neg(p2)))));
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
