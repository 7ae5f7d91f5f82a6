// Row-wise proxy update of the FP8 backbone, and the adapter SGD step.
//
// FALQON keeps the adapter update in a row-wise proxy and merges only the
// rows whose update is large enough to survive FP8 rounding (summary page,
// key-design paragraph; introduction, method paragraph; rebuttal thread 2,
// reply W7: merge by top-k row selection).  The rows of B are the proxy: the
// pending delta of backbone row i is u_i = B_i . A.  Three launches:
//
//  proxy_score    every element once: the rank-r chain acc = fmaf(B[i,k],
//                 A[k,j], acc) for k = 0..r-1 from +0 (the fixed order makes
//                 the FP8 rounding below reproducible bit for bit), then
//                 t = fl(s_w * acc).  Each workgroup writes, per row, the max
//                 |t| and the largest code magnitude of its 512 columns, and
//                 it stages the candidate codes E4M3(fl(dec(q) + t)) for every
//                 element in a workspace copy of the backbone;
//  proxy_select   one workgroup: folds the per-column-block maxima (a max of
//                 non-negative bit patterns, order independent), then
//                 rho_i = max|t| / step_i (a power-of-two
//                 scaling), rho_i >= tau, optionally capped to the k_max
//                 largest (radix select on the float bits, equal scores to the
//                 lower row), compacted in row order;
//  proxy_apply    selected rows only: copy the staged codes into the backbone
//                 and zero the row of B.
// Without a cap on the number of merged rows (k_max = 0) the last two share
// one launch (proxy_select_apply): a row's merge depends on its own score.
//
// proxy_score runs the chain on the matrix cores: the fp32 MFMA with K = 1
// (v_mfma_f32_32x32x1_2b_f32) adds the outer product of a 64-lane column
// operand and a 64-lane row operand into two 32 x 32 accumulator blocks,
// each element with one rounding, i.e. exactly fmaf(b, a, acc).  Fed ranks
// in ascending order from +0 accumulators, a chain of these MFMAs gives the
// same bits as the scalar fmaf chain, at twice the rate of unpacked fp32 VALU
// fmas.  The product is formed transposed: the MFMA's rows are backbone
// columns (operand A[k, cols]) and its columns are backbone rows (operand
// B[rows, k]), so that one lane ends up holding 4 consecutive columns of one
// backbone row per accumulator group (a whole 4-byte code word).
//
// Workgroup tile 64 rows x 512 columns, 4 waves of 32 rows x 256 columns.
// Four MFMAs per rank cover a wave's tile: MFMA m takes column 4L + m of
// the wave's 256 at lane L (one ds_read_b128 per rank feeds all four) and
// row L % 32 of B.  Lane l then holds row l % 32 and, per block b and group
// g, the 16 columns 128b + 32g + 16(l / 32) + [0, 16): one 16-byte code
// load and one 16-byte staged store each.  A reaches LDS by direct
// global->LDS loads in stages of KC ranks; B's values (one per lane and rank)
// are loaded a stage ahead into registers.
#include "common.hpp"
#include "kernels.hpp"
#include "transpose_u8.hpp"

#include <algorithm>

namespace falq {
namespace {

typedef float f32x32 __attribute__((ext_vector_type(32)));

constexpr int kThreads = 256;
constexpr int kSelThreads = 1024;
constexpr int kSelRhoLds = 16384;  // rows whose scores proxy_select keeps in LDS
constexpr int PRB = 64;          // rows per score workgroup (two waves of 32)
constexpr int PCB = 512;         // columns per score workgroup (two waves of 256)
constexpr int KC = 8;            // ranks per LDS stage

// max(|x|, |y|, m) in one instruction: fmaxf on values the compiler cannot
// prove canonical costs a canonicalizing max per operand first.  NaN
// operands are skipped, as by fmaxf.  Only for VALU results (no MFMA result
// may be read here: the compiler does not see this operand's producer).
__device__ __forceinline__ float max3_abs(float x, float y, float m) {
  float r;
  asm("v_max3_f32 %0, |%1|, |%2|, %3" : "=v"(r) : "v"(x), "v"(y), "v"(m));
  return r;
}

// 1 / E4M3 spacing at magnitude m (the bits of a float >= 0, the largest
// |dec(code)| of a row): 2^9 below 2^-6 (exponent field 0 or 1), else
// 2^(3 - E) for m in [2^E, 2^(E+1))
__device__ __forceinline__ float inv_step_of_mag(uint32_t mbits) {
  if (mbits < 0x3C800000u) return 512.0f;
  const int e = (int)(mbits >> 23) - 127;
  return __uint_as_float((uint32_t)(127 + 3 - e) << 23);
}

// IDX: the chain runs over the r ranks kidx[0..r) (ascending) of an adapter
// whose B rows hold rs values; otherwise over ranks 0..r-1 and rs = r
template <bool IDX>
__global__ __launch_bounds__(kThreads, 2) void proxy_score(const uint8_t* __restrict__ wq,
                                                        const float* __restrict__ s_w_ptr,
                                                        const float* __restrict__ A,
                                                        const float* __restrict__ B, int d_in,
                                                        int d_out, int r, int rs,
                                                        const int32_t* __restrict__ kidx,
                                                        uint32_t* __restrict__ tmax_part,
                                                        uint32_t* __restrict__ cmax_part,
                                                        uint8_t* __restrict__ staged) {
  __shared__ __attribute__((aligned(1024))) float sA[2][KC][PCB];       // 32 KB
  __shared__ uint32_t red_t[4][32], red_c[4][32];
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6), wr = w >> 1, wc = w & 1;
  const int row0 = blockIdx.x * PRB + wr * 32;             // this wave's first row
  const int col0 = blockIdx.y * PCB;
  const int colw = col0 + wc * 256;                        // this wave's first column

  f32x32 acc[4];
#pragma unroll
  for (int m = 0; m < 4; ++m)
#pragma unroll
    for (int v = 0; v < 32; ++v) acc[m][v] = 0.0f;

  // this lane's B row (rows past d_out read the last row; their results are
  // discarded)
  const float* brow = B + (int64_t)min(row0 + (lane & 31), d_out - 1) * (IDX ? rs : r);
  auto rk = [&](int k) { return IDX ? kidx[k] : k; };      // rank of chain position k

  // stage `buf` <- A[k0 .. k0+KC) x [col0, col0+512): 16 half rows of 1 KB,
  // four per wave, by direct loads (columns past d_in are clamped into A).
  // Chain positions past r are padding: their LDS rows are written +0 and
  // their B operand is -0 (selected where it is used, so that the B loads
  // are not waited for early), so their MFMAs add fl(-0 * +0) = -0 to every
  // accumulator, which leaves each one (signed zeros included) unchanged.
  auto issue = [&](int buf, int k0) {
    const uint32_t lbase = lds_offset(&sA[buf][0][0]);
    if (k0 + KC <= r) {
      // a whole stage of real ranks: no test per load (branches in this
      // barrier-paced loop cost more than their instructions)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int c = w * 4 + j, kk = c >> 1, h = c & 1;
        const int gc = min(col0 + h * 256 + lane * 4, d_in - 4);
        load16_to_lds(A + (int64_t)rk(k0 + kk) * d_in + gc,
                      __builtin_amdgcn_readfirstlane(lbase + c * 1024));
      }
      return;
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int c = w * 4 + j, kk = c >> 1, h = c & 1;
      if (k0 + kk < r) {
        const int gc = min(col0 + h * 256 + lane * 4, d_in - 4);
        load16_to_lds(A + (int64_t)rk(k0 + kk) * d_in + gc,
                      __builtin_amdgcn_readfirstlane(lbase + c * 1024));
      } else {
        *reinterpret_cast<float4*>(&sA[buf][kk][h * 256 + lane * 4]) =
            make_float4(0.0f, 0.0f, 0.0f, 0.0f);
      }
    }
  };
  // a whole stage of consecutive ranks as two 16-byte loads (a lane's row
  // is 4 r bytes long, so r % 4 == 0 and an aligned B keep them aligned): the lanes of a
  // wave read 32 rows, and one 4-byte load per rank costs the memory path
  // 32 cache lines per instruction, eight times per stage (lab, 4096^2,
  // r = 64: 33.8 -> 32.5 us, the same bits)
  auto load_b = [&](float (&bv)[KC], int k0) {
    if (!IDX && k0 + KC <= r && (r & 3) == 0 && ((uintptr_t)B & 15) == 0) {
#pragma unroll
      for (int h = 0; h < KC / 4; ++h) {
        const float4 x = *reinterpret_cast<const float4*>(brow + k0 + 4 * h);
        bv[4 * h] = x.x;
        bv[4 * h + 1] = x.y;
        bv[4 * h + 2] = x.z;
        bv[4 * h + 3] = x.w;
      }
      return;
    }
#pragma unroll
    for (int u = 0; u < KC; ++u) bv[u] = brow[rk(min(k0 + u, r - 1))];
  };

  // one stage: wait for it, start the next one (A into the other LDS buffer,
  // its B values into `nxt`), then KC ranks of four MFMAs each
  // this lane's eight 16-byte code chunks (see the epilogue), loaded under
  // the last stage's MFMAs; addresses are clamped into the backbone and out
  // of range chunks are not used
  const int row = row0 + (lane & 31);
  const int64_t rbase = (int64_t)min(row, d_out - 1) * d_in;
  uint4 codes[8];
  auto load_codes = [&]() {
#pragma unroll
    for (int bg = 0; bg < 8; ++bg)
      codes[bg] = *reinterpret_cast<const uint4*>(
          wq + rbase + min(colw + 32 * bg + 16 * (lane >> 5), d_in - 16));
  };

  // stage s: wait until this wave's part of it landed (direct loads, padding
  // stores, B values), then the barrier: all of it landed, and stage s-1 is
  // no longer read, so its buffer can take stage s+1
  auto wait_stage = [&]() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(0x0070);                      // vmcnt(0) lgkmcnt(0)
    barrier_no_drain();
  };
  auto compute = [&](int s, const float (&cur)[KC]) {       // KC ranks, four MFMAs each
    const int buf = s & 1, k0 = s * KC;
#pragma unroll
    for (int kk = 0; kk < KC; ++kk) {
      const float4 a = *reinterpret_cast<const float4*>(&sA[buf][kk][wc * 256 + lane * 4]);
      const float b = k0 + kk < r ? cur[kk] : -0.0f;         // padding: -0
      acc[0] = __builtin_amdgcn_mfma_f32_32x32x1f32(a.x, b, acc[0], 0, 0, 0);
      acc[1] = __builtin_amdgcn_mfma_f32_32x32x1f32(a.y, b, acc[1], 0, 0, 0);
      acc[2] = __builtin_amdgcn_mfma_f32_32x32x1f32(a.z, b, acc[2], 0, 0, 0);
      acc[3] = __builtin_amdgcn_mfma_f32_32x32x1f32(a.w, b, acc[3], 0, 0, 0);
    }
  };
  // B values alternate between two register sets; the last stage is peeled
  // so that the prefetched codes are live only there
  const int nslab = (r + KC - 1) / KC, last = nslab - 1;
  float b0[KC], b1[KC];
  if (nslab > 0) {
    issue(0, 0);
    load_b(b0, 0);
  }
  int s = 0;
  for (; s + 1 < last; s += 2) {
    wait_stage();
    issue((s + 1) & 1, (s + 1) * KC);
    load_b(b1, (s + 1) * KC);
    compute(s, b0);
    wait_stage();
    issue(s & 1, (s + 2) * KC);
    load_b(b0, (s + 2) * KC);
    compute(s + 1, b1);
  }
  if (s < last) {
    wait_stage();
    issue((s + 1) & 1, (s + 1) * KC);
    load_b(b1, (s + 1) * KC);
    compute(s, b0);
#pragma unroll
    for (int u = 0; u < KC; ++u) b0[u] = b1[u];
    ++s;
  }
  if (nslab > 0) {
    wait_stage();
    load_codes();
    compute(s, b0);
  } else {
    load_codes();
  }

  // Epilogue.  Accumulator m, register v = 4bg + q of lane l holds column
  // colw + 32bg + 16(l / 32) + 4q + m of row row0 + l % 32 (bg = 0..7 spans
  // the two MFMA blocks and their four register groups): code chunk bg.
  const float s_w = *s_w_ptr;
  float tm = 0.0f, cmf = 0.0f;           // max |t| and max |dec(code)| of this lane's columns
#pragma unroll
  for (int bg = 0; bg < 8; ++bg) {
    const int c = colw + 32 * bg + 16 * (lane >> 5);
    if (row >= d_out || c >= d_in) continue;                 // d_in is a multiple of 16
    const uint32_t cw[4] = {codes[bg].x, codes[bg].y, codes[bg].z, codes[bg].w};
    float sum[4][4];
    uint32_t out[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int v = 4 * bg + q;
      const float t0 = s_w * acc[0][v], t1 = s_w * acc[1][v];
      const float t2 = s_w * acc[2][v], t3 = s_w * acc[3][v];
      tm = max3_abs(t2, t3, max3_abs(t0, t1, tm));
      const float2 lo = dec2(cw[q], false), hi = dec2(cw[q], true);
      cmf = max3_abs(hi.x, hi.y, max3_abs(lo.x, lo.y, cmf));
      sum[q][0] = lo.x + t0;
      sum[q][1] = lo.y + t1;
      sum[q][2] = hi.x + t2;
      sum[q][3] = hi.y + t3;
      out[q] = enc4_nonan(sum[q][0], sum[q][1], sum[q][2], sum[q][3], cw[q]);
    }
    bool nan = false;
#pragma unroll
    for (int q = 0; q < 4; ++q)
      nan |= __builtin_isnan(sum[q][0]) | __builtin_isnan(sum[q][1]) |
             __builtin_isnan(sum[q][2]) | __builtin_isnan(sum[q][3]);
    if (__builtin_expect(nan, 0)) {
#pragma unroll
      for (int q = 0; q < 4; ++q) out[q] = nan_patch(out[q], sum[q][0], sum[q][1], sum[q][2], sum[q][3]);
    }
    *reinterpret_cast<uint4*>(staged + (int64_t)row * d_in + c) =
        make_uint4(out[0], out[1], out[2], out[3]);
  }
  uint32_t cm = __float_as_uint(cmf);
  // row maxima: lanes l and l + 32 share a row; then the two waves of the
  // same rows meet in LDS (|t| >= 0: bit order = value order)
  uint32_t tb = __float_as_uint(tm);
  tb = max(tb, (uint32_t)__shfl_xor((int)tb, 32, 64));
  cm = max(cm, (uint32_t)__shfl_xor((int)cm, 32, 64));
  if (lane < 32) {
    red_t[w][lane] = tb;
    red_c[w][lane] = cm;
  }
  __syncthreads();
  if (tid < PRB) {
    const int half = tid >> 5, i = tid & 31, rr = blockIdx.x * PRB + tid;
    if (rr < d_out) {
      tmax_part[(int64_t)blockIdx.y * d_out + rr] = max(red_t[2 * half][i], red_t[2 * half + 1][i]);
      cmax_part[(int64_t)blockIdx.y * d_out + rr] = max(red_c[2 * half][i], red_c[2 * half + 1][i]);
    }
  }
}

// exclusive prefix sum over the 1024 threads of a workgroup; *total = sum
__device__ int block_excl_scan(int v, int* smem16, int* total) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  int x = v;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int y = __shfl_up(x, off, 64);
    if (lane >= off) x += y;
  }
  if (lane == 63) smem16[w] = x;
  __syncthreads();
  int base = 0, tot = 0;
  for (int k = 0; k < kSelThreads / 64; ++k) {
    const int t = smem16[k];
    if (k < w) base += t;
    tot += t;
  }
  __syncthreads();
  *total = tot;
  return base + x - v;
}

// rho_i from the per-column-block maxima, written to rho[] for every row;
// then the selection.  Thread t owns rows [t*R, t*R + R), R = ceil(d_out/1024),
// so one block-wide scan orders the uncapped selection.  (One workgroup of
// kSelThreads.)
__device__ __forceinline__ void select_rows(const uint32_t* __restrict__ tmax_part,
                                            const uint32_t* __restrict__ cmax_part, int ncb,
                                            float* __restrict__ rho, int d_out, float tau,
                                            int k_max, int32_t* __restrict__ sel,
                                            int32_t* __restrict__ n_sel) {
  __shared__ int hist[256];
  __shared__ int s16[kSelThreads / 64];
  __shared__ uint32_t s_prefix;
  __shared__ int s_need;
  __shared__ float s_rho[kSelRhoLds];  // rho read back from LDS when d_out fits
  const int tid = threadIdx.x;
  float* rv = d_out <= kSelRhoLds ? s_rho : rho;
  // fold the column-block maxima: rows strided over the threads (coalesced);
  // a thread folds four rows at once with the loads of eight column blocks
  // (64 loads) in flight, so the fold takes ncb / 8 round trips
  for (int i0 = tid; i0 < d_out; i0 += 4 * kSelThreads) {
    uint32_t tb[4] = {0, 0, 0, 0}, cb[4] = {0, 0, 0, 0};
    for (int b = 0; b < ncb; b += 8) {
      uint32_t x[8][4], y[8][4];
#pragma unroll
      for (int u = 0; u < 8; ++u)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int i = min(i0 + j * kSelThreads, d_out - 1), bb = min(b + u, ncb - 1);
          x[u][j] = tmax_part[(int64_t)bb * d_out + i];    // clamped repeats fold harmlessly
          y[u][j] = cmax_part[(int64_t)bb * d_out + i];
        }
#pragma unroll
      for (int u = 0; u < 8; ++u)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          tb[j] = x[u][j] > tb[j] ? x[u][j] : tb[j];
          cb[j] = y[u][j] > cb[j] ? y[u][j] : cb[j];
        }
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int i = i0 + j * kSelThreads;
      if (i < d_out) {
        const float x = __uint_as_float(tb[j]) * inv_step_of_mag(cb[j]);
        rho[i] = x;
        if (rv != rho) rv[i] = x;
      }
    }
  }
  __syncthreads();                     // every row's rho written, read back below

  const int R = (d_out + kSelThreads - 1) / kSelThreads;
  const int i0 = tid * R, i1 = min(d_out, i0 + R);
  int cnt = 0;
  for (int i = i0; i < i1; ++i) cnt += (rv[i] >= tau) ? 1 : 0;
  int total;
  const int base = block_excl_scan(cnt, s16, &total);
  const bool capped = k_max > 0 && total > k_max;
  if (!capped) {
    int pos = base;
    for (int i = i0; i < i1; ++i)
      if (rv[i] >= tau) sel[pos++] = i;
    if (tid == 0) *n_sel = total;
    return;
  }

  // k_max largest scores: radix select of the k-th largest key, then a
  // row-order compaction that keeps the lowest rows among equal scores
  if (tid == 0) { s_prefix = 0; s_need = k_max; }
  __syncthreads();
  for (int shift = 24; shift >= 0; shift -= 8) {
    for (int b = tid; b < 256; b += kSelThreads) hist[b] = 0;
    __syncthreads();
    const uint32_t prefix = s_prefix;
    const uint32_t hmask = shift == 24 ? 0u : (0xFFFFFFFFu << (shift + 8));
    for (int i = tid; i < d_out; i += kSelThreads) {
      const float x = rv[i];
      if (!(x >= tau)) continue;
      const uint32_t key = __float_as_uint(x);
      if ((key & hmask) == (prefix & hmask)) atomicAdd(&hist[(key >> shift) & 0xFF], 1);
    }
    __syncthreads();
    if (tid == 0) {
      int need = s_need, cum = 0, digit = 0;
      for (int b = 255; b >= 0; --b) {
        if (cum + hist[b] >= need) { digit = b; break; }
        cum += hist[b];
      }
      s_need = need - cum;
      s_prefix = prefix | ((uint32_t)digit << shift);
    }
    __syncthreads();
  }
  const uint32_t key_star = s_prefix;  // k-th largest score
  const int need_eq = s_need;          // rows with score == key_star to keep
  int n_eq = 0, n_gt = 0;
  for (int i = i0; i < i1; ++i) {
    const float x = rv[i];
    if (!(x >= tau)) continue;
    const uint32_t key = __float_as_uint(x);
    n_eq += key == key_star;
    n_gt += key > key_star;
  }
  int eq_total;
  int eq_rank = block_excl_scan(n_eq, s16, &eq_total);
  const int eq_take = max(0, min(n_eq, need_eq - eq_rank));   // lowest rows first
  int tk_total;
  int pos = block_excl_scan(n_gt + eq_take, s16, &tk_total);
  int eq_left = eq_take;
  for (int i = i0; i < i1; ++i) {
    const float x = rv[i];
    if (!(x >= tau)) continue;
    const uint32_t key = __float_as_uint(x);
    if (key > key_star || (key == key_star && eq_left-- > 0)) sel[pos++] = i;
  }
  if (tid == 0) *n_sel = tk_total;
}

__global__ __launch_bounds__(kSelThreads) void proxy_select(const uint32_t* __restrict__ tmax_part,
                                                            const uint32_t* __restrict__ cmax_part,
                                                            int ncb, float* __restrict__ rho,
                                                            int d_out, float tau, int k_max,
                                                            int32_t* __restrict__ sel,
                                                            int32_t* __restrict__ n_sel) {
  select_rows(tmax_part, cmax_part, ncb, rho, d_out, tau, k_max, sel, n_sel);
}

// The uncapped selection (k_max = 0: every row with rho_i >= tau) with the
// row copies in the same launch.  Whether row i is merged depends on rho_i
// alone, so the copies need not wait for the compacted list: workgroup 0
// computes rho and the list as proxy_select does, and every other workgroup
// takes kSelThreads / 64 rows, one per wave, folds that row's column-block
// maxima into rho_i with the same operations (the same bits), and when
// rho_i >= tau copies the staged codes into the backbone and zeroes the B
// row (B[row][kidx[k]] for k < r with IDX; B rows hold rs values).
template <bool IDX>
__global__ __launch_bounds__(kSelThreads) void proxy_select_apply(
    const uint32_t* __restrict__ tmax_part, const uint32_t* __restrict__ cmax_part, int ncb,
    float* __restrict__ rho, int d_out, float tau, int32_t* __restrict__ sel,
    int32_t* __restrict__ n_sel, uint8_t* __restrict__ wq, const uint8_t* __restrict__ staged,
    float* __restrict__ B, int d_in, int r, int rs, const int32_t* __restrict__ kidx) {
  if (blockIdx.x == 0) {
    select_rows(tmax_part, cmax_part, ncb, rho, d_out, tau, 0, sel, n_sel);
    return;
  }
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)(blockIdx.x - 1) * (kSelThreads / 64) + (threadIdx.x >> 6);
  if (row >= d_out) return;
  uint32_t tb = 0, cb = 0;
  for (int b = lane; b < ncb; b += 64) {
    const uint32_t x = tmax_part[(int64_t)b * d_out + row], y = cmax_part[(int64_t)b * d_out + row];
    tb = x > tb ? x : tb;
    cb = y > cb ? y : cb;
  }
  tb = wave_max_u32(tb);
  cb = wave_max_u32(cb);
  const float x = __uint_as_float(tb) * inv_step_of_mag(cb);
  if (!(x >= tau)) return;
  const uint4* src = reinterpret_cast<const uint4*>(staged + row * d_in);
  uint4* dst = reinterpret_cast<uint4*>(wq + row * d_in);
  for (int j = lane; j < d_in / 16; j += 64) dst[j] = src[j];
  for (int k = lane; k < r; k += 64) B[row * (IDX ? rs : r) + (IDX ? kidx[k] : k)] = 0.0f;
}

// proxy_select_apply that also leaves the transpose of the updated
// backbone, wt [d_in x d_out] = wq^T, for the next step's dX product.
// Workgroup 0 computes rho and the list as proxy_select does; every other
// workgroup takes four 128 x 128 tiles of the backbone, 256 threads each.
// A tile first decides its 128 rows from their column-block maxima (the
// same operations as select_rows, so the same bits), then each thread reads
// 16 rows x 4 bytes of the new backbone (the staged codes of a merged row,
// the backbone's own otherwise), writes the merged rows' bytes back, and
// stores the block's transpose (4 columns x 16 bytes) into wt; the tiles of
// the first tile column zero the merged rows of B.  Every byte of wq and wt
// is read or written by exactly one thread.  d_out and d_in are multiples
// of 16.
template <bool IDX>
__global__ __launch_bounds__(kSelThreads) void proxy_select_apply_t(
    const uint32_t* __restrict__ tmax_part, const uint32_t* __restrict__ cmax_part, int ncb,
    float* __restrict__ rho, int d_out, float tau, int32_t* __restrict__ sel,
    int32_t* __restrict__ n_sel, uint8_t* __restrict__ wq, const uint8_t* __restrict__ staged,
    float* __restrict__ B, int d_in, int r, int rs, const int32_t* __restrict__ kidx,
    uint8_t* __restrict__ wt, int n_tiles, int tiles_x) {
  if (blockIdx.x == 0) {
    select_rows(tmax_part, cmax_part, ncb, rho, d_out, tau, 0, sel, n_sel);
    return;
  }
  __shared__ uint8_t merge[4][128];
  const int q = threadIdx.x >> 8, t = threadIdx.x & 255;
  const int tile = (blockIdx.x - 1) * 4 + q;
  const bool live = tile < n_tiles;
  const int bx = live ? tile % tiles_x : 0, by = live ? tile / tiles_x : 0;
  if (live && t < 128) {
    const int64_t row = (int64_t)by * 128 + t;
    uint8_t m = 0;
    if (row < d_out) {
      uint32_t tb = 0, cb = 0;
      for (int b0 = 0; b0 < ncb; b0 += 8) {
        uint32_t x[8], y[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          const int b = min(b0 + u, ncb - 1);              // clamped repeats fold harmlessly
          x[u] = tmax_part[(int64_t)b * d_out + row];
          y[u] = cmax_part[(int64_t)b * d_out + row];
        }
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          tb = x[u] > tb ? x[u] : tb;
          cb = y[u] > cb ? y[u] : cb;
        }
      }
      m = __uint_as_float(tb) * inv_step_of_mag(cb) >= tau ? 1 : 0;
    }
    merge[q][t] = m;
  }
  __syncthreads();
  if (!live) return;
  if (bx == 0 && t < 128) {
    const int64_t row = (int64_t)by * 128 + t;
    if (row < d_out && merge[q][t])
      for (int k = 0; k < r; ++k) B[row * (IDX ? rs : r) + (IDX ? kidx[k] : k)] = 0.0f;
  }
  const int cg = t & 31, rg = t >> 5;
  const int64_t c = (int64_t)bx * 128 + cg * 4;             // 4 backbone columns
  const int64_t r0 = (int64_t)by * 128 + rg * 16;           // 16 backbone rows
  if (c >= d_in || r0 >= d_out) return;
  uint32_t d[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int64_t at = (r0 + i) * d_in + c;
    const bool mg = merge[q][rg * 16 + i] != 0;
    d[i] = *reinterpret_cast<const uint32_t*>((mg ? staged : wq) + at);
    if (mg) *reinterpret_cast<uint32_t*>(wq + at) = d[i];
  }
  uint32_t o[4][4];
  transpose_16x4(d, o);
#pragma unroll
  for (int k = 0; k < 4; ++k)
    *reinterpret_cast<uint4*>(wt + (c + k) * d_out + r0) = make_uint4(o[k][0], o[k][1], o[k][2], o[k][3]);
}

// one selected row per wave: copy the staged codes, zero the B row
// zeroes B[row][kidx[k]] for k < r (IDX; B rows hold rs values), else B[row][0..r)
template <bool IDX>
__global__ __launch_bounds__(kThreads) void proxy_apply(uint8_t* __restrict__ wq,
                                                        const uint8_t* __restrict__ staged,
                                                        float* __restrict__ B, int d_in, int r,
                                                        int rs, const int32_t* __restrict__ kidx,
                                                        const int32_t* __restrict__ sel,
                                                        const int32_t* __restrict__ n_sel) {
  const int n = *n_sel;
  const int lane = threadIdx.x & 63;
  const int e = blockIdx.x * (kThreads / 64) + (threadIdx.x >> 6);
  if (e >= n) return;
  const int64_t row = sel[e];
  const uint4* src = reinterpret_cast<const uint4*>(staged + row * d_in);
  uint4* dst = reinterpret_cast<uint4*>(wq + row * d_in);
  for (int j = lane; j < d_in / 16; j += 64) dst[j] = src[j];
  for (int k = lane; k < r; k += 64) B[row * (IDX ? rs : r) + (IDX ? kidx[k] : k)] = 0.0f;
}

// p <- fl(p - fl(lr * g)) for two tensors in one launch: float4 slots
// [0, na4) belong to the first, [na4, na4 + nb4) to the second; scalar tails
// are done by workgroup 0.
__global__ __launch_bounds__(256) void sgd_kernel(float* __restrict__ pa, const float* __restrict__ ga,
                                                  int64_t na, float* __restrict__ pb,
                                                  const float* __restrict__ gb, int64_t nb,
                                                  float lr) {
  const int64_t na4 = na / 4, nb4 = nb / 4;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < na4 + nb4; i += stride) {
    float* p = i < na4 ? pa : pb;
    const float* g = i < na4 ? ga : gb;
    const int64_t j = i < na4 ? i : i - na4;
    float4 a = reinterpret_cast<float4*>(p)[j];
    const float4 b = reinterpret_cast<const float4*>(g)[j];
    a.x = a.x - lr * b.x;     // two roundings: built without fp contraction
    a.y = a.y - lr * b.y;
    a.z = a.z - lr * b.z;
    a.w = a.w - lr * b.w;
    reinterpret_cast<float4*>(p)[j] = a;
  }
  if (blockIdx.x == 0) {
    for (int64_t i = na4 * 4 + threadIdx.x; i < na; i += blockDim.x) pa[i] = pa[i] - lr * ga[i];
    for (int64_t i = nb4 * 4 + threadIdx.x; i < nb; i += blockDim.x) pb[i] = pb[i] - lr * gb[i];
  }
}

struct ProxyWs {
  size_t off_tmax, off_cmax, off_rho, off_staged, total;
  int ncb;                                  // column blocks of the score kernel
};

ProxyWs proxy_layout(int64_t d_in, int64_t d_out) {
  ProxyWs p{};
  p.ncb = (int)((d_in + PCB - 1) / PCB);
  size_t o = 0;
  auto take = [&](size_t bytes) { size_t at = o; o = align_up(o + bytes, 256); return at; };
  p.off_tmax = take((size_t)p.ncb * d_out * 4);
  p.off_cmax = take((size_t)p.ncb * d_out * 4);
  p.off_rho = take((size_t)d_out * 4);
  p.off_staged = take((size_t)d_out * (size_t)d_in);
  p.total = o;
  return p;
}

}  // namespace

size_t proxy_ws_bytes(int64_t d_in, int64_t d_out, int64_t r) {
  (void)r;
  return proxy_layout(d_in, d_out).total;
}

hipError_t launch_proxy_update(uint8_t* wq, const float* s_w, const float* A, float* B,
                               int64_t d_in, int64_t d_out, int64_t r, float tau, int64_t k_max,
                               int32_t* sel_idx, int32_t* n_sel, float* rho, void* ws,
                               hipStream_t s) {
  return launch_proxy_update_ranks(wq, s_w, A, B, d_in, d_out, r, r, nullptr, tau, k_max, sel_idx,
                                   n_sel, rho, ws, s);
}

hipError_t launch_proxy_update_ranks(uint8_t* wq, const float* s_w, const float* A, float* B,
                                     int64_t d_in, int64_t d_out, int64_t r, int64_t rs,
                                     const int32_t* kidx, float tau, int64_t k_max,
                                     int32_t* sel_idx, int32_t* n_sel, float* rho, void* ws,
                                     hipStream_t s, uint8_t* wt) {
  const ProxyWs L = proxy_layout(d_in, d_out);
  uint8_t* base = reinterpret_cast<uint8_t*>(ws);
  uint32_t* tmax = reinterpret_cast<uint32_t*>(base + L.off_tmax);
  uint32_t* cmax = reinterpret_cast<uint32_t*>(base + L.off_cmax);
  float* rr = rho ? rho : reinterpret_cast<float*>(base + L.off_rho);
  uint8_t* staged = base + L.off_staged;
  if (d_out > 0 && d_in > 0) {
    dim3 grid((unsigned)((d_out + PRB - 1) / PRB), (unsigned)L.ncb);
    if (kidx)
      proxy_score<true><<<grid, kThreads, 0, s>>>(wq, s_w, A, B, (int)d_in, (int)d_out, (int)r,
                                                  (int)rs, kidx, tmax, cmax, staged);
    else
      proxy_score<false><<<grid, kThreads, 0, s>>>(wq, s_w, A, B, (int)d_in, (int)d_out, (int)r,
                                                   (int)rs, nullptr, tmax, cmax, staged);
  }
  if (wt != nullptr && k_max == 0 && d_out > 0 && d_in > 0) {
    const int tiles_x = (int)((d_in + 127) / 128);
    const int n_tiles = tiles_x * (int)((d_out + 127) / 128);
    const unsigned g = 1 + (unsigned)((n_tiles + 3) / 4);
    if (kidx)
      proxy_select_apply_t<true><<<g, kSelThreads, 0, s>>>(
          tmax, cmax, L.ncb, rr, (int)d_out, tau, sel_idx, n_sel, wq, staged, B, (int)d_in, (int)r,
          (int)rs, kidx, wt, n_tiles, tiles_x);
    else
      proxy_select_apply_t<false><<<g, kSelThreads, 0, s>>>(
          tmax, cmax, L.ncb, rr, (int)d_out, tau, sel_idx, n_sel, wq, staged, B, (int)d_in, (int)r,
          (int)rs, nullptr, wt, n_tiles, tiles_x);
    return hipGetLastError();
  }
  if (k_max == 0 && d_out > 0) {
    const unsigned g = 1 + (unsigned)((d_out + kSelThreads / 64 - 1) / (kSelThreads / 64));
    if (kidx)
      proxy_select_apply<true><<<g, kSelThreads, 0, s>>>(tmax, cmax, L.ncb, rr, (int)d_out, tau,
                                                         sel_idx, n_sel, wq, staged, B, (int)d_in,
                                                         (int)r, (int)rs, kidx);
    else
      proxy_select_apply<false><<<g, kSelThreads, 0, s>>>(tmax, cmax, L.ncb, rr, (int)d_out, tau,
                                                          sel_idx, n_sel, wq, staged, B,
                                                          (int)d_in, (int)r, (int)rs, nullptr);
    return hipGetLastError();
  }
  proxy_select<<<1, kSelThreads, 0, s>>>(tmax, cmax, L.ncb, rr, (int)d_out, tau, (int)k_max,
                                         sel_idx, n_sel);
  if (d_out > 0) {
    const int rows_per_block = kThreads / 64;
    const unsigned g = (unsigned)((d_out + rows_per_block - 1) / rows_per_block);
    if (kidx)
      proxy_apply<true><<<g, kThreads, 0, s>>>(wq, staged, B, (int)d_in, (int)r, (int)rs, kidx,
                                               sel_idx, n_sel);
    else
      proxy_apply<false><<<g, kThreads, 0, s>>>(wq, staged, B, (int)d_in, (int)r, (int)rs,
                                                nullptr, sel_idx, n_sel);
  }
  if (wt != nullptr && d_out > 0 && d_in > 0) {
    // the capped selection: the transpose after the merge, in a launch of its own
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    return launch_transpose_u8(wq, d_out, d_in, wt, s);
  }
  return hipGetLastError();
}

hipError_t launch_sgd2(float* pa, const float* ga, int64_t na, float* pb, const float* gb,
                       int64_t nb, float lr, hipStream_t s) {
  if (na <= 0) { pa = nullptr; ga = nullptr; na = 0; }
  if (nb <= 0) { pb = nullptr; gb = nullptr; nb = 0; }
  if (na + nb == 0) return hipSuccess;
  const int64_t blocks = std::min<int64_t>(((na + nb) / 4 + 255) / 256 + 1, 4096);
  sgd_kernel<<<(int)blocks, 256, 0, s>>>(pa, ga, na, pb, gb, nb, lr);
  return hipGetLastError();
}

}  // namespace falq
