// fp8_quantize: per-tensor current scaling to OCP E4M3 (or E5M2) on gfx950.
//
// The scale is s = 448 / max|x| (57344 / max|x| for E5M2; the per-tensor
// factor s_X of the FALQON rebuttal, thread 2 reply W2), so every cast
// depends on one global maximum.
//
// One launch where x fits the resident workgroups (up to 100 MiB): qz_one.
// Every workgroup loads its 64 KB of x once and keeps it in registers (for
// x above 64 MiB, 36 KB more in LDS by direct loads), reduces max |x| over
// its finite elements and counts its
// non-finite ones, and publishes both as 64-bit words tagged with the call's
// epoch (high half) in a small library-owned device array.  Workgroup 0
// gathers the words of all workgroups, folds them and publishes the result
// (tagged the same way); every workgroup then casts its registers.  Each
// word is written and read by one device-scope atomic, so a reader that sees
// the epoch sees the value that came with it: no fences, no counters to
// clear, nothing to reset between calls.  Every wait has a deadline (the
// 100 MHz real-time counter): a workgroup whose words have not arrived by
// then (not resident, or a concurrent call on another stream overwrote its
// slot) has its range read directly by the waiting workgroup instead, so
// the result is the same exact maximum in every case, only later.
// Otherwise (larger x, or a stream under graph capture, whose replays would
// repeat the epoch) two launches, both streaming and fully coalesced:
//   1. qz_amax   : max of |x| over finite elements, each workgroup over one
//                  contiguous range (as the ordered
//                  uint32 bit pattern of a non-negative float) and a count of
//                  non-finite elements, one partial per workgroup;
//   2. qz_cast   : every workgroup folds the <= 1024 partials (4 KB, L2
//                  resident) into amax and s, then casts its share of x with
//                  the hardware E4M3 converter.  Workgroup 0 writes s, amax
//                  and the non-finite count.
// Both forms give bit-identical results from run to run.
#include "common.hpp"
#include "kernels.hpp"

#include <float.h>

#include <algorithm>
#include <atomic>
#include <mutex>

namespace falq {
namespace {

constexpr int kThreads = 256;
constexpr int kUnroll = 8;
constexpr int kAmaxUnroll = 4;

// x is streamed with nontemporal loads: both passes read each byte once, and
// a load that allocates in the caches has to write back the dirty lines that
// earlier kernels' outputs left there first (measured on a bf16 4096 x 4096
// tensor after a large write: 20 us for the amax pass with ordinary loads,
// 10 us with nontemporal ones)
__device__ __forceinline__ uint4 stream16(const void* x, int64_t i) {
  const v4i t = __builtin_nontemporal_load(reinterpret_cast<const v4i*>(x) + i);
  return make_uint4((uint32_t)t[0], (uint32_t)t[1], (uint32_t)t[2], (uint32_t)t[3]);
}

template <int DT> struct Vec;
template <> struct Vec<0> {  // float32: 4 elements per 16-byte load
  static constexpr int N = 4;
  __device__ static void unpack(const uint4& u, float (&v)[8]) {
    v[0] = __uint_as_float(u.x); v[1] = __uint_as_float(u.y);
    v[2] = __uint_as_float(u.z); v[3] = __uint_as_float(u.w);
  }
  __device__ static void load(const void* x, int64_t i, float (&v)[8]) { unpack(stream16(x, i), v); }
  __device__ static float scalar(const void* x, int64_t i) {
    return reinterpret_cast<const float*>(x)[i];
  }
};
template <> struct Vec<1> {  // bfloat16: 8 elements per 16-byte load
  static constexpr int N = 8;
  __device__ static void unpack(const uint4& u, float (&v)[8]) {
    const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      v[2 * k] = __uint_as_float(w[k] << 16);
      v[2 * k + 1] = __uint_as_float(w[k] & 0xFFFF0000u);
    }
  }
  __device__ static void load(const void* x, int64_t i, float (&v)[8]) { unpack(stream16(x, i), v); }
  __device__ static float scalar(const void* x, int64_t i) {
    return __uint_as_float((uint32_t)reinterpret_cast<const uint16_t*>(x)[i] << 16);
  }
};

__device__ __forceinline__ void absorb(float f, uint32_t& m, int& bad) {
  uint32_t a = __float_as_uint(f) & 0x7FFFFFFFu;
  if (a >= 0x7F800000u) ++bad;
  else m = a > m ? a : m;
}

__device__ __forceinline__ float scale_of(float amax, float fmt_max,
                                          const float* __restrict__ scale_in) {
  if (scale_in) return *scale_in;
  if (amax == 0.0f) return 1.0f;
  const float sc = fmt_max / amax;        // IEEE-correct fp32 division
  return __builtin_isinf(sc) ? FLT_MAX : sc;
}

// every workgroup: fold the per-workgroup partials into amax and the scale;
// workgroup 0 publishes s, amax and the non-finite count
__device__ float fold_scale(const uint32_t* __restrict__ part_max, const int* __restrict__ part_bad,
                            int nparts, float fmt_max, const float* __restrict__ scale_in,
                            float* __restrict__ scale_out, float* __restrict__ amax_out,
                            int32_t* __restrict__ nonfinite_out) {
  __shared__ uint32_t sm[kThreads / 64];
  __shared__ int sb[kThreads / 64];
  __shared__ float s_scale;
  uint32_t m = 0;
  int bad = 0;
  for (int i = threadIdx.x; i < nparts; i += kThreads) {
    const uint32_t p = part_max[i];
    m = p > m ? p : m;
    bad += part_bad[i];
  }
  m = wave_max_u32(m);
  bad = wave_sum_i32(bad);
  if ((threadIdx.x & 63) == 0) { sm[threadIdx.x >> 6] = m; sb[threadIdx.x >> 6] = bad; }
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t mm = sm[0];
    int bb = sb[0];
#pragma unroll
    for (int k = 1; k < kThreads / 64; ++k) { mm = sm[k] > mm ? sm[k] : mm; bb += sb[k]; }
    const float amax = __uint_as_float(mm);
    const float sc = scale_of(amax, fmt_max, scale_in);
    s_scale = sc;
    if (blockIdx.x == 0) {
      *scale_out = sc;
      if (amax_out) *amax_out = amax;
      if (nonfinite_out) *nonfinite_out = bb;
    }
  }
  __syncthreads();
  return s_scale;
}

// F = 0: E4M3, F = 1: E5M2
template <int F>
__device__ __forceinline__ uint32_t enc4f(float a, float b, float c, float d) {
  return F == 0 ? enc4(a, b, c, d) : enc4_e5m2(a, b, c, d);
}

template <int DT, int F>
__device__ __forceinline__ void store_codes(uint8_t* __restrict__ q, int64_t i, const float (&v)[8],
                                            float s) {
  if (F == 2) {                          // FP4 E2M1: two codes per byte, low nibble first
    uint32_t w = 0;
#pragma unroll
    for (int e = 0; e < (DT == 0 ? 4 : 8); ++e) w |= enc1_e2m1(v[e] * s) << (4 * e);
    if (DT == 0) reinterpret_cast<uint16_t*>(q)[i] = (uint16_t)w;
    else reinterpret_cast<uint32_t*>(q)[i] = w;
    return;
  }
  if (DT == 0) {
    reinterpret_cast<uint32_t*>(q)[i] = enc4f<F>(v[0] * s, v[1] * s, v[2] * s, v[3] * s);
  } else {
    const uint32_t c0 = enc4f<F>(v[0] * s, v[1] * s, v[2] * s, v[3] * s);
    const uint32_t c1 = enc4f<F>(v[4] * s, v[5] * s, v[6] * s, v[7] * s);
    reinterpret_cast<uint2*>(q)[i] = make_uint2(c0, c1);
  }
}

__device__ __forceinline__ void block_partials(uint32_t m, int bad, uint32_t* __restrict__ part_max,
                                               int* __restrict__ part_bad) {
  __shared__ uint32_t sm[kThreads / 64];
  __shared__ int sb[kThreads / 64];
  m = wave_max_u32(m);
  bad = wave_sum_i32(bad);
  if ((threadIdx.x & 63) == 0) { sm[threadIdx.x >> 6] = m; sb[threadIdx.x >> 6] = bad; }
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t mm = sm[0];
    int bb = sb[0];
#pragma unroll
    for (int k = 1; k < kThreads / 64; ++k) { mm = sm[k] > mm ? sm[k] : mm; bb += sb[k]; }
    part_max[blockIdx.x] = mm;
    part_bad[blockIdx.x] = bb;
  }
}

template <int DT>
__global__ __launch_bounds__(kThreads) void qz_amax(const void* __restrict__ x, int64_t n,
                                                    uint32_t* __restrict__ part_max,
                                                    int* __restrict__ part_bad) {
  using V = Vec<DT>;
  const int64_t nvec = n / V::N;
  uint32_t m = 0;
  int bad = 0;
  // each workgroup streams one contiguous range, kAmaxUnroll 16-byte loads
  // in flight per lane per round (measured on 4096 x 4096 fp32 behind dirty
  // caches: 14.0 us against 16.6 us for a grid stride with 16 loads per lane)
  const int64_t per = (nvec + gridDim.x - 1) / gridDim.x;
  const int64_t b0 = (int64_t)blockIdx.x * per, b1 = min(nvec, b0 + per);
  for (int64_t i0 = b0 + threadIdx.x; i0 < b1; i0 += (int64_t)kThreads * kAmaxUnroll) {
    float v[kAmaxUnroll][8];
#pragma unroll
    for (int u = 0; u < kAmaxUnroll; ++u)
      if (i0 + u * kThreads < b1) V::load(x, i0 + u * kThreads, v[u]);
#pragma unroll
    for (int u = 0; u < kAmaxUnroll; ++u)
      if (i0 + u * kThreads < b1)
#pragma unroll
        for (int e = 0; e < V::N; ++e) absorb(v[u][e], m, bad);
  }
  if (blockIdx.x == 0)
    for (int64_t i = nvec * V::N + threadIdx.x; i < n; i += kThreads) absorb(V::scalar(x, i), m, bad);

  block_partials(m, bad, part_max, part_bad);
}

// the n % N elements past the last whole vector, by one workgroup
template <int DT, int F>
__device__ __forceinline__ void cast_tail(const void* __restrict__ x, int64_t n,
                                          uint8_t* __restrict__ q, float s) {
  using V = Vec<DT>;
  const int64_t nvec = n / V::N;
  if (F == 2) {                          // n is even: the tail in whole bytes
    for (int64_t i = nvec * V::N + 2 * threadIdx.x; i + 1 < n; i += 2 * kThreads)
      q[i / 2] = (uint8_t)(enc1_e2m1(V::scalar(x, i) * s) |
                           (enc1_e2m1(V::scalar(x, i + 1) * s) << 4));
  } else {
    for (int64_t i = nvec * V::N + threadIdx.x; i < n; i += kThreads)
      q[i] = (uint8_t)(F == 0 ? enc1(V::scalar(x, i) * s) : enc1_e5m2(V::scalar(x, i) * s));
  }
}

template <int DT, int F>
__global__ __launch_bounds__(kThreads) void qz_cast(const void* __restrict__ x, int64_t n,
                                                    const uint32_t* __restrict__ part_max,
                                                    const int* __restrict__ part_bad, int nparts,
                                                    const float* __restrict__ scale_in,
                                                    uint8_t* __restrict__ q,
                                                    float* __restrict__ scale_out,
                                                    float* __restrict__ amax_out,
                                                    int32_t* __restrict__ nonfinite_out) {
  using V = Vec<DT>;
  const int64_t nvec = n / V::N;
  // each workgroup casts one contiguous range (as the amax pass reads it:
  // 17.1 us against 20.4 us for a grid stride, 4096 x 4096 fp32)
  const int64_t per = (nvec + gridDim.x - 1) / gridDim.x;
  const int64_t b0 = (int64_t)blockIdx.x * per, b1 = min(nvec, b0 + per);
  int64_t i0 = b0 + threadIdx.x;
  // the first batch of x is requested before the partials are folded, so the
  // fold's latency overlaps the loads
  float v[kUnroll][8];
#pragma unroll
  for (int u = 0; u < kUnroll; ++u)
    if (i0 + u * kThreads < b1) V::load(x, i0 + u * kThreads, v[u]);
  const float s = fold_scale(part_max, part_bad, nparts,
                             F == 0 ? kE4M3Max : (F == 1 ? kE5M2Max : kE2M1Max), scale_in,
                             scale_out, amax_out, nonfinite_out);
  while (true) {
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int64_t i = i0 + u * kThreads;
      if (i < b1) store_codes<DT, F>(q, i, v[u], s);
    }
    i0 += (int64_t)kThreads * kUnroll;
    if (i0 >= b1) break;
#pragma unroll
    for (int u = 0; u < kUnroll; ++u)
      if (i0 + u * kThreads < b1) V::load(x, i0 + u * kThreads, v[u]);
  }
  if (blockIdx.x == 0) cast_tail<DT, F>(x, n, q, s);
}

// ---- one launch (qz_one) ----------------------------------------------------
constexpr int kOneR = 16;                                 // 16-byte vectors of x per lane
// ... plus kOneL more per lane staged in LDS for an x of 64 .. 100 MiB
// (36 KB per workgroup: four workgroups still fit a CU's 160 KB)
constexpr int kOneL = 9;
template <int L>
constexpr int64_t one_per() { return (int64_t)(kOneR + L) * kThreads; }   // vectors per workgroup
constexpr int kOneMaxWG = 1024;
constexpr int kOneSlots = kOneMaxWG / kThreads;           // words gathered per lane of workgroup 0
// exchange words: (max, non-finite count) of workgroup i at 2 i, 2 i + 1;
// the folded pair at 2 kOneMaxWG, 2 kOneMaxWG + 1
constexpr int kOneWords = 2 * kOneMaxWG + 2;

__device__ __forceinline__ uint64_t tagged(uint32_t epoch, uint32_t v) {
  return ((uint64_t)epoch << 32) | v;
}
__device__ __forceinline__ void put_word(uint64_t* p, uint64_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint64_t get_word(uint64_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// a direct global -> LDS load of 16 bytes per lane with the streaming hint
// (lane l's bytes land at lds_addr + 16 l; lds_addr wave-uniform)
__device__ __forceinline__ void stream16_to_lds(const void* g, uint32_t lds_addr) {
  asm volatile("global_load_lds_dwordx4 %0, off nt" ::"v"(g), "{m0}"(lds_addr) : "memory");
}

// max |x| and the non-finite count of workgroup b's range (and the scalar
// tail for b = 0), by one lane: the fallback for a range whose words have
// not arrived
template <int DT, int L>
__device__ void range_partial(const void* __restrict__ x, int64_t n, int b, uint32_t& m,
                              int& bad) {
  using V = Vec<DT>;
  const int64_t nvec = n / V::N;
  const int64_t b0 = (int64_t)b * one_per<L>(), b1 = min(nvec, b0 + one_per<L>());
  // one vector at a time: this runs beside the caller's 64 registers of x
#pragma unroll 1
  for (int64_t i = b0; i < b1; ++i) {
    float v[8];
    V::load(x, i, v);
#pragma unroll
    for (int e = 0; e < V::N; ++e) absorb(v[e], m, bad);
  }
  if (b == 0)
    for (int64_t i = nvec * V::N; i < n; ++i) absorb(V::scalar(x, i), m, bad);
}

// block reduction of (m, bad) to lane 0 of wave 0 (the other lanes' values
// are unspecified)
__device__ __forceinline__ void block_fold(uint32_t& m, int& bad) {
  __shared__ uint32_t sm[kThreads / 64];
  __shared__ int sb[kThreads / 64];
  m = wave_max_u32(m);
  bad = wave_sum_i32(bad);
  __syncthreads();
  if ((threadIdx.x & 63) == 0) { sm[threadIdx.x >> 6] = m; sb[threadIdx.x >> 6] = bad; }
  __syncthreads();
  if (threadIdx.x == 0) {
#pragma unroll
    for (int k = 1; k < kThreads / 64; ++k) { m = sm[k] > m ? sm[k] : m; bad += sb[k]; }
  }
}

// x [n] -> q, s with x held in registers (and, L > 0, L more vectors per
// lane in LDS): workgroup b owns vectors [b P, (b + 1) P), P = one_per<L>();
// gridDim.x <= kOneMaxWG workgroups, all of which the host has checked fit
// on the device at once.  `wait` bounds each wait for the exchange words, in
// ticks of the 100 MHz real-time counter.
template <int DT, int F, int L>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(4))) void qz_one(const void* __restrict__ x, int64_t n,
                                                   uint64_t* __restrict__ words, uint32_t epoch,
                                                   uint64_t wait,
                                                   const float* __restrict__ scale_in,
                                                   uint8_t* __restrict__ q,
                                                   float* __restrict__ scale_out,
                                                   float* __restrict__ amax_out,
                                                   int32_t* __restrict__ nonfinite_out) {
  using V = Vec<DT>;
  const int64_t nvec = n / V::N;
  const int tid = threadIdx.x, G = gridDim.x;
  const bool leader = blockIdx.x == 0;
  const int64_t i0 = (int64_t)blockIdx.x * one_per<L>() + tid;
  __shared__ __attribute__((aligned(16))) uint4 xs[L > 0 ? L * kThreads : 1];
  uint4 raw[kOneR];
#pragma unroll
  for (int u = 0; u < kOneR; ++u)
    if (i0 + u * kThreads < nvec) raw[u] = stream16(x, i0 + u * kThreads);
  // the LDS part: lane l of wave w puts vector kOneR + u at xs[u kThreads + 64 w + l]
  const int64_t j0 = i0 + (int64_t)kOneR * kThreads;
#pragma unroll
  for (int u = 0; u < L; ++u)
    if (j0 + u * kThreads < nvec)
      stream16_to_lds(reinterpret_cast<const uint4*>(x) + j0 + u * kThreads,
                      __builtin_amdgcn_readfirstlane(lds_offset(&xs[u * kThreads + (tid & ~63)])));
  uint32_t m = 0;
  int bad = 0;
#pragma unroll
  for (int u = 0; u < kOneR; ++u)
    if (i0 + u * kThreads < nvec) {
      float v[8];
      V::unpack(raw[u], v);
#pragma unroll
      for (int e = 0; e < V::N; ++e) absorb(v[e], m, bad);
    }
  if constexpr (L > 0) {
    wait_vmem(0);                        // this wave's own LDS slots have landed
#pragma unroll
    for (int u = 0; u < L; ++u)
      if (j0 + u * kThreads < nvec) {
        float v[8];
        V::unpack(xs[u * kThreads + tid], v);
#pragma unroll
        for (int e = 0; e < V::N; ++e) absorb(v[e], m, bad);
      }
  }
  if (leader)
    for (int64_t i = nvec * V::N + tid; i < n; i += kThreads) absorb(V::scalar(x, i), m, bad);
  // the floats are formed again from the held words for the cast: keeping
  // them (bf16: 128 per lane) would not fit the four waves per SIMD that
  // hold a 64 MiB x
#pragma unroll
  for (int u = 0; u < kOneR; ++u)
    asm volatile("" : "+v"(raw[u].x), "+v"(raw[u].y), "+v"(raw[u].z), "+v"(raw[u].w));
  block_fold(m, bad);
  if (tid == 0) {
    put_word(words + 2 * blockIdx.x, tagged(epoch, m));
    put_word(words + 2 * blockIdx.x + 1, tagged(epoch, (uint32_t)bad));
  }

  __shared__ uint32_t s_amax;
  __shared__ int s_bad, s_got;
  const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
  if (!leader) {
    // the folded pair from workgroup 0
    if (tid == 0) {
      int got = 0;
      while (true) {
        const uint64_t a = get_word(words + 2 * kOneMaxWG), c = get_word(words + 2 * kOneMaxWG + 1);
        if ((uint32_t)(a >> 32) == epoch && (uint32_t)(c >> 32) == epoch) {
          s_amax = (uint32_t)a;
          s_bad = (int)(uint32_t)c;
          got = 1;
          break;
        }
        if (__builtin_amdgcn_s_memrealtime() - t0 > wait) break;
        __builtin_amdgcn_s_sleep(2);
      }
      s_got = got;
    }
    __syncthreads();
  }
  if (leader || !s_got) {
    // gather every workgroup's pair (workgroup 0 waits for them; a
    // workgroup that gave up on workgroup 0 takes what has arrived), and
    // read the ranges of those that have not arrived
    uint32_t need = 0, got = 0;
#pragma unroll
    for (int k = 0; k < kOneSlots; ++k)
      if (tid + k * kThreads < G) need |= 1u << k;
    m = 0;
    bad = 0;
    while (true) {
#pragma unroll
      for (int k = 0; k < kOneSlots; ++k) {
        const int i = tid + k * kThreads;
        if (((need & ~got) >> k) & 1) {
          const uint64_t a = get_word(words + 2 * i), c = get_word(words + 2 * i + 1);
          if ((uint32_t)(a >> 32) == epoch && (uint32_t)(c >> 32) == epoch) {
            m = (uint32_t)a > m ? (uint32_t)a : m;
            bad += (int)(uint32_t)c;
            got |= 1u << k;
          }
        }
      }
      if (got == need || !leader || __builtin_amdgcn_s_memrealtime() - t0 > wait) break;
      __builtin_amdgcn_s_sleep(2);
    }
#pragma unroll 1
    for (int k = 0; k < kOneSlots; ++k)
      if (((need & ~got) >> k) & 1) range_partial<DT, L>(x, n, tid + k * kThreads, m, bad);
    block_fold(m, bad);
    if (tid == 0) {
      s_amax = m;
      s_bad = bad;
      if (leader) {
        put_word(words + 2 * kOneMaxWG, tagged(epoch, m));
        put_word(words + 2 * kOneMaxWG + 1, tagged(epoch, (uint32_t)bad));
      }
    }
    __syncthreads();
  }
  const float amax = __uint_as_float(s_amax);
  const float s = scale_of(amax, F == 0 ? kE4M3Max : (F == 1 ? kE5M2Max : kE2M1Max), scale_in);
  if (leader && tid == 0) {
    *scale_out = s;
    if (amax_out) *amax_out = amax;
    if (nonfinite_out) *nonfinite_out = s_bad;
  }
#pragma unroll
  for (int u = 0; u < kOneR; ++u) {
    const int64_t i = i0 + u * kThreads;
    if (i < nvec) {
      float v[8];
      V::unpack(raw[u], v);
      store_codes<DT, F>(q, i, v, s);
    }
  }
#pragma unroll
  for (int u = 0; u < L; ++u) {
    const int64_t i = j0 + u * kThreads;
    if (i < nvec) {
      float v[8];
      V::unpack(xs[u * kThreads + tid], v);
      store_codes<DT, F>(q, i, v, s);
    }
  }
  if (leader) cast_tail<DT, F>(x, n, q, s);
}

int blocks_for(int64_t nvec, int unroll, int cap) {
  int64_t b = (nvec + (int64_t)kThreads * unroll - 1) / ((int64_t)kThreads * unroll);
  if (b < 1) b = 1;
  if (b > cap) b = cap;
  return (int)b;
}

// out[i] = dec(q[i]) / s, the float32 division correctly rounded; 16 codes a
// thread, a scalar tail for n % 16
__global__ __launch_bounds__(kThreads) void dq_kernel(const uint8_t* __restrict__ q, int64_t n,
                                                      const float* __restrict__ scale,
                                                      float* __restrict__ out) {
  const float s = scale[0];
  const int64_t n16 = n / 16;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n16;
       i += (int64_t)gridDim.x * blockDim.x) {
    const uint4 c = reinterpret_cast<const uint4*>(q)[i];
    const uint32_t w[4] = {c.x, c.y, c.z, c.w};
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const float2 a = dec2(w[k], false), b = dec2(w[k], true);
      reinterpret_cast<float4*>(out)[4 * i + k] = make_float4(a.x / s, a.y / s, b.x / s, b.y / s);
    }
  }
  if (blockIdx.x == 0) {
    for (int64_t i = n16 * 16 + threadIdx.x; i < n; i += blockDim.x)
      out[i] = dec2(q[i], false).x / s;
  }
}

}  // namespace

hipError_t launch_dequantize(const uint8_t* q, int64_t n, const float* s, float* out,
                             hipStream_t st) {
  if (n <= 0) return hipSuccess;
  const int blocks = (int)std::min<int64_t>((n / 16 + kThreads - 1) / kThreads + 1, 2048);
  dq_kernel<<<blocks, kThreads, 0, st>>>(q, n, s, out);
  return hipGetLastError();
}

size_t quantize_ws_bytes() { return (size_t)kQzMaxParts * 8; }

// ---------------------------------------------------------------------------
// The one-launch route's exchange words: a file-scope device array, one copy
// per GPU for the life of the process, whose device address comes from
// hipGetSymbolAddress (once per device, with that device current).  Words
// are tagged with a per-call epoch, so the array never needs clearing; calls
// that overlap on one GPU (concurrent streams) may overwrite each other's
// words, which only sends the waiting workgroups to the fallback that reads
// the missing ranges themselves.
// ---------------------------------------------------------------------------
static __device__ __align__(256) uint64_t qz_words[kOneWords];

namespace {
constexpr int kOneDevices = 64;
std::mutex g_one_mu;
struct OneRoute {
  bool init = false;
  void* words = nullptr;
  int cap[2][3][2] = {};                    // resident workgroups of qz_one<DT, F, 0 / kOneL>
};
OneRoute g_one[kOneDevices];
std::atomic<uint32_t> g_epoch{0};
std::atomic<uint64_t> g_wait_ticks{50000};     // 500 us

template <int DT, int F, int L>
int resident(int ncu) {
  int per_cu = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(
          &per_cu, reinterpret_cast<const void*>(qz_one<DT, F, L>), kThreads, 0) != hipSuccess)
    return 0;
  return per_cu * ncu;
}

template <int L>
int64_t one_grid(int64_t nvec) { return std::max<int64_t>(1, (nvec + one_per<L>() - 1) / one_per<L>()); }

// The one-launch route for x [nvec vectors] on the current device: the
// exchange words, and in *lds whether the LDS-staged instance is needed
// (x larger than the registers of the resident workgroups hold); nullptr
// when x does not fit either instance or the stream is being captured
uint64_t* one_route(int dtype, int fmt, int64_t nvec, hipStream_t s, bool* lds) {
  if (one_grid<kOneL>(nvec) > kOneMaxWG) return nullptr;
  hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
  if (hipStreamIsCapturing(s, &cs) != hipSuccess || cs != hipStreamCaptureStatusNone)
    return nullptr;
  int dev = -1, ncu = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kOneDevices) return nullptr;
  std::lock_guard<std::mutex> lock(g_one_mu);
  OneRoute& r = g_one[dev];
  if (!r.init) {
    r.init = true;
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(qz_words)) != hipSuccess ||
        hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
      return nullptr;                       // r.words stays null: the two-launch route
    r.words = p;
#define FALQ_CAP(DT, F)                                  \
  r.cap[DT][F][0] = resident<DT, F, 0>(ncu);             \
  r.cap[DT][F][1] = resident<DT, F, kOneL>(ncu)
    FALQ_CAP(0, 0); FALQ_CAP(0, 1); FALQ_CAP(0, 2);
    FALQ_CAP(1, 0); FALQ_CAP(1, 1); FALQ_CAP(1, 2);
#undef FALQ_CAP
  }
  if (r.words == nullptr) return nullptr;
  const int* cap = r.cap[dtype != 0][fmt];
  const int64_t g0 = one_grid<0>(nvec), g1 = one_grid<kOneL>(nvec);
  if (g0 <= std::min(cap[0], kOneMaxWG)) *lds = false;
  else if (g1 <= std::min(cap[1], kOneMaxWG)) *lds = true;
  else return nullptr;
  return static_cast<uint64_t*>(r.words);
}
}  // namespace

uint64_t quantize_wait_ticks(uint64_t ticks) { return g_wait_ticks.exchange(ticks); }

hipError_t launch_quantize(const void* x, int dtype, int fmt, int64_t n, const float* scale_in,
                           uint8_t* q, float* scale, float* amax, int32_t* nonfinite,
                           void* ws, hipStream_t s) {
  bool lds = false;
  if (uint64_t* words = one_route(dtype, fmt, n / (dtype == 0 ? 4 : 8), s, &lds)) {
    uint32_t epoch = ++g_epoch;
    if (epoch == 0) epoch = ++g_epoch;      // 0 is the words' initial tag
    const int64_t nvec = n / (dtype == 0 ? 4 : 8);
    const int G = (int)(lds ? one_grid<kOneL>(nvec) : one_grid<0>(nvec));
    const uint64_t wait = g_wait_ticks.load(std::memory_order_relaxed);
#define FALQ_ONE(DT, F)                                                                        \
  do {                                                                                         \
    if (lds)                                                                                   \
      qz_one<DT, F, kOneL><<<G, kThreads, 0, s>>>(x, n, words, epoch, wait, scale_in, q, scale, \
                                                  amax, nonfinite);                            \
    else                                                                                       \
      qz_one<DT, F, 0><<<G, kThreads, 0, s>>>(x, n, words, epoch, wait, scale_in, q, scale,     \
                                              amax, nonfinite);                                \
  } while (0)
    if (dtype == 0 && fmt == 0) FALQ_ONE(0, 0);
    else if (dtype == 0 && fmt == 1) FALQ_ONE(0, 1);
    else if (dtype == 0) FALQ_ONE(0, 2);
    else if (fmt == 0) FALQ_ONE(1, 0);
    else if (fmt == 1) FALQ_ONE(1, 1);
    else FALQ_ONE(1, 2);
#undef FALQ_ONE
    return hipGetLastError();
  }
  uint32_t* part_max = reinterpret_cast<uint32_t*>(ws);
  int* part_bad = reinterpret_cast<int*>(part_max + kQzMaxParts);
  const int vecn = dtype == 0 ? 4 : 8;
  const int64_t nvec = n / vecn;
  const int g1 = blocks_for(nvec, 4 * kAmaxUnroll, 1024);   // every cast workgroup folds these partials
  const int g2 = blocks_for(nvec, kUnroll, 2048);
  if (dtype == 0)
    qz_amax<0><<<g1, kThreads, 0, s>>>(x, n, part_max, part_bad);
  else
    qz_amax<1><<<g1, kThreads, 0, s>>>(x, n, part_max, part_bad);
#define FALQ_CAST(DT, F)                                                                        \
  qz_cast<DT, F><<<g2, kThreads, 0, s>>>(x, n, part_max, part_bad, g1, scale_in, q, scale, amax, \
                                         nonfinite)
  if (dtype == 0 && fmt == 0) FALQ_CAST(0, 0);
  else if (dtype == 0 && fmt == 1) FALQ_CAST(0, 1);
  else if (dtype == 0) FALQ_CAST(0, 2);
  else if (fmt == 0) FALQ_CAST(1, 0);
  else if (fmt == 1) FALQ_CAST(1, 1);
  else FALQ_CAST(1, 2);
#undef FALQ_CAST
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Scratch for callers that cannot allocate (fp8_quantize_noalloc): the amax
// partials live in a file-scope device array instead of a caller workspace.
// Each GPU the library runs on holds its own copy (kQzMaxParts * 8 bytes) for
// the life of the process.  In host code `scratch` names a host-side stand-in,
// not device memory: its device address comes from hipGetSymbolAddress, once
// per device with that device current, and only that address is passed on.
// Every call on a GPU shares that GPU's array, so calls that overlap on one
// GPU (concurrent streams) race; stream-ordered calls do not.  Nothing in it
// needs to start at zero: every amax workgroup writes its partial before the
// cast launch reads it.
// ---------------------------------------------------------------------------
namespace {
static __device__ __align__(256) uint8_t scratch[kQuantizeScratchBytes];
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};
}  // namespace

size_t quantize_scratch_bytes() { return sizeof(scratch); }

hipError_t quantize_scratch(void** out) {
  *out = nullptr;
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return hipSuccess;
}

}  // namespace falq
