// The token-contracting half of the adapter gradients on the FP8 matrix
// cores, from the rank-r factors U = X^ A^T and V = G^ B (FALQON rebuttal,
// thread 4, reply Q1: dL/dA = B^T (dL/dO) x^T, and dL/dB takes the x A^T
// factor computed ahead):
//     dB[n][j] = sum_t G^[t][n] U[t][j]        (problem 0, n over d_out)
//     dA[j][n] = sum_t V[t][j] X^[t][n]        (problem 1, n over d_in)
// Both contract over the tokens t, and the FP8 codes G~, X~ are stored token
// by token (row t holds the d codes of one token), so the contraction index
// is the row index.  The matrix core wants each lane to hold 32 consecutive
// contraction positions of one output row; gfx950's LDS transpose read
// (ds_read_b64_tr_b8) produces exactly that from the row-major tile:
//
//   within each group of 16 lanes, lane d receives byte (d % 8) of the
//   8-byte rows addressed by lanes 2e + d / 8, e = 0..7, as its bytes e.
//   So with source lane s pointing at tile row t0 + s / 2, columns
//   16 c + 8 (s % 2) .. +7, lane d receives rows t0 .. t0 + 7 of column
//   16 c + d: eight consecutive tokens of one output column.  Four reads
//   (t0 = 32 g + 8 i for the lane group g) fill the 32-byte operand.
//
// The float factor F (U or V) enters as three E4M3 pieces per element with a
// power-of-two scale per rank and 32-token block, applied by the matrix core
// as the operand's E8M0 block scale (pieces.hpp: planes [3][Rp][Tp] with the
// tokens contiguous, scale bytes [Tp / 128][Rp][4], zero codes beyond T).
// The pieces of V come from the dX product's epilogue, those of U (and of V
// when another kernel formed it) from the float factor (uv_pieces_kernel).
//
// Tile: 64 ranks x 64 output columns per workgroup over one split of the
// tokens, 8 waves (each 16 ranks x 32 columns: 2 blocks x 3 pieces = 6
// 16x16x128 MFMAs per 128-token step), a four-stage LDS ring filled by
// direct-to-LDS loads (the FP8 tile [128 t][64 n] and the pieces
// [3][64 j][128 t] per stage, 16-byte chunks XOR-swizzled by row so that
// both the transpose reads and the piece fragment reads are free of bank
// conflicts).  The kernel is bound by the number of direct-load instructions
// a CU issues, so the scale bytes (256 per step) come in windows of 16 steps
// (4 KB, one half-wave load per wave, double-buffered), not with every
// stage.  With too few tiles to fill half the GPU the tokens are split
// in two halves whose results are added with float atomics onto outputs
// zeroed beforehand: exactly two addends meet a zero, and a + b does not
// depend on which lands first, so the result is the same on every run.
#include "common.hpp"
#include "kernels.hpp"
#include "pieces.hpp"

#include <algorithm>

namespace falq {
namespace {

constexpr int TKR = 64, TKN = 64, TKK = 128, TKS = 4, TKW = 8;
constexpr int kTkThreads = TKW * 64;
constexpr int TQ_BYTES = TKK * TKN;                      // FP8 tile [128 t][64 n]
constexpr int TP_PLANE = TKR * TKK;                      // one piece [64 j][128 t]
constexpr int TSTAGE = TQ_BYTES + 3 * TP_PLANE;
constexpr int TEW = 16;                                  // steps per window of scale bytes
constexpr int TE_WIN = TEW * TKR * 4;                    // one window: [16 steps][64 j][4]
constexpr int TE_OFF = TKS * TSTAGE;                     // two windows after the ring
constexpr int TQ_I = TQ_BYTES / 1024 / TKW, TP_I = 3 * TP_PLANE / 1024 / TKW;
constexpr int TLPS = TQ_I + TP_I;                        // direct loads per wave per stage
static_assert(TQ_I * 1024 * TKW == TQ_BYTES && TP_I * 1024 * TKW == 3 * TP_PLANE, "loads");
static_assert(TE_WIN == TKW * 32 * 16, "one window: 32 lanes x 16 bytes per wave");
static_assert(TE_OFF + 2 * TE_WIN <= 160 * 1024, "LDS");
static_assert(TLPS == 4 && TKS == 4, "wait counts below assume four loads per stage, 4 stages");

// 128-byte piece rows: 16-byte chunk c of row r at slot c ^ swz8(r) (the
// FP8 GEMM's pattern: the 16-row fragment reads are conflict-free)
__device__ __forceinline__ int swz8(int row) { return (row ^ ((row >> 3) & 1)) & 7; }
// 64-byte FP8 rows: chunk c of token row t at slot c ^ swz4(t).  A transpose
// read serves 32 lanes at a time: two lane groups, each taking one chunk of 8
// consecutive rows, rows t0 .. t0 + 7 and t0 + 32 .. t0 + 39.  Row t's chunk
// lands in bank group 4 (t % 4) + slot, and bits 2 and 5 of t make the four
// rows that share t % 4 take four different slots: the 16 rows cover all 64
// banks (SQ_LDS_BANK_CONFLICT 0; with bits 2 and 3 alone, every read paid one
// conflict cycle, at the same kernel time)
__device__ __forceinline__ int swz4(int row) { return ((row >> 2) & 1) | (((row >> 5) & 1) << 1); }

__device__ __forceinline__ v8i join8(uint4 lo, uint4 hi) {
  v8i r;
  r[0] = lo.x; r[1] = lo.y; r[2] = lo.z; r[3] = lo.w;
  r[4] = hi.x; r[5] = hi.y; r[6] = hi.z; r[7] = hi.w;
  return r;
}

typedef __attribute__((address_space(3))) v2i lds_v2i;

constexpr int TNB = 2;                                   // 16-column blocks per wave

// acc[b] += Q block b (format QF) . piece p (E4M3, the lane's scale byte eb:
// rank r16, block g of the step), p = 0, 1, 2
template <int QF>
__device__ __forceinline__ void mma_pieces(const v8i (&qf)[TNB], const v8i (&pf)[3], int eb,
                                           v4f (&acc)[TNB]) {
#pragma unroll
  for (int p = 0; p < 3; ++p)
#pragma unroll
    for (int b = 0; b < TNB; ++b)
      acc[b] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(qf[b], pf[p], acc[b], QF, 0, 0,
                                                                127, 0, eb);
}

struct TokProb {
  const uint8_t* q;      // FP8 codes [T x N], row stride ldq
  int64_t ldq;
  const float* sq;       // their scale
  const uint8_t* P;      // pieces [3][Rp][Tp]
  const uint8_t* E;      // their scale bytes [Tp / 128][Rp][4]
  float* out;            // [N x r] (n_major) or [r x N]
  int N, n_major, tiles_n, blocks;
};

struct TokArgs {
  TokProb p[2];
  int T, Tp, r, Rp, S, kps;   // S = 1, or 2 (atomic adds onto zeroed outputs)
};

// The dispatcher deals consecutive workgroup ids round-robin to the 8 XCDs;
// the id is remapped so that each XCD takes a contiguous run of logical
// workgroups.  Two neighbouring 64-column tiles read the two halves of the
// same 128-byte lines of the codes, so on one XCD the second read is served
// by that XCD's L2 instead of HBM (ids past the last multiple of 8 keep
// their own).
__device__ __forceinline__ int tok_xcd_remap(int bid, int n) {
  const int per = n / 8;
  return bid < per * 8 ? (bid % 8) * per + bid / 8 : bid;
}

// logical workgroup: problem, then tile (rank tile, column tile), then split
// (fastest)
template <int QF0>
__global__ __launch_bounds__(kTkThreads, 1) void tok_kernel(TokArgs a) {
  __shared__ __attribute__((aligned(1024))) uint8_t smem[TE_OFF + 2 * TE_WIN];
  int b = tok_xcd_remap((int)blockIdx.x, (int)gridDim.x);
  const int pi = b >= a.p[0].blocks ? 1 : 0;
  if (pi) b -= a.p[0].blocks;
  // the problem's fields, selected one by one (no indexing of the argument
  // struct with a run-time value)
  TokProb pr;
  pr.q = pi ? a.p[1].q : a.p[0].q;
  pr.ldq = pi ? a.p[1].ldq : a.p[0].ldq;
  pr.sq = pi ? a.p[1].sq : a.p[0].sq;
  pr.P = pi ? a.p[1].P : a.p[0].P;
  pr.E = pi ? a.p[1].E : a.p[0].E;
  pr.out = pi ? a.p[1].out : a.p[0].out;
  pr.N = pi ? a.p[1].N : a.p[0].N;
  pr.n_major = pi ? a.p[1].n_major : a.p[0].n_major;
  pr.tiles_n = pi ? a.p[1].tiles_n : a.p[0].tiles_n;
  const int split = b % a.S, tile = b / a.S;
  const int rt = tile / pr.tiles_n, nt = tile % pr.tiles_n;
  const int nk_all = a.Tp / TKK;
  const int k_lo = split * a.kps;
  const int nk = max(0, min(nk_all - k_lo, a.kps));
  const int n0 = nt * TKN, j0 = rt * TKR;

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int rb = w & 3, nh = w >> 2;
  const int lrow = lane >> 3, lslot = lane & 7;          // piece rows: 8 x 128 bytes
  const int qrow = lane >> 2, qslot = lane & 3;          // FP8 rows: 16 x 64 bytes

  // direct-load sources: FP8 rows (tokens, clamped into [0, T): rows past T
  // meet zero pieces), piece rows (ranks of this tile, 3 planes)
  // (the lane's code row within a step, and its column offset)
  int qR[TQ_I];
  const uint8_t* gQ[TQ_I];
#pragma unroll
  for (int q = 0; q < TQ_I; ++q) {
    qR[q] = k_lo * TKK + (w * TQ_I + q) * 16 + qrow;
    gQ[q] = pr.q + n0 + ((qslot ^ swz4(qR[q])) * 16);
  }
  const uint8_t* gP[TP_I];
#pragma unroll
  for (int q = 0; q < TP_I; ++q) {
    const int R = (w * TP_I + q) * 8 + lrow;           // 0 .. 191: plane R / 64, rank row R % 64
    const int row = R & (TKR - 1);
    gP[q] = pr.P + (int64_t)(R >> 6) * a.Rp * a.Tp + (int64_t)(j0 + row) * a.Tp + k_lo * TKK +
            ((lslot ^ swz8(row)) * 16);
  }
  // scale bytes: in the window that opens at step kt, wave w brings steps
  // kt + 2 w, kt + 2 w + 1 (lanes 0 .. 15, 16 .. 31: 16 bytes each of the
  // step's 256; steps past the last are clamped to it and never read)
  const int e_step = 2 * w + ((lane >> 4) & 1);
  auto issue_e = [&](int kt) {
    const int64_t c = k_lo + min(kt + e_step, a.Tp / TKK - 1 - k_lo);
    const uint8_t* src = pr.E + (c * a.Rp + j0) * 4 + (lane & 15) * 16;
    const uint32_t dst = lds_offset(smem + TE_OFF + ((kt / TEW) & 1) * TE_WIN + w * 512);
    if (lane < 32) load16_to_lds(src, __builtin_amdgcn_readfirstlane(dst));
  };
  auto issue = [&](int stage, int kt) {
    // the next window rides ahead of the loads of the step that precedes it,
    // so that waiting for any step also covers its window (at the cost of
    // waiting for one load more in two steps of sixteen)
    if ((kt + 1) % TEW == 0) issue_e(kt + 1);
    const uint32_t base = lds_offset(smem + stage * TSTAGE);
    // token rows advance with kt; a row past T - 1 is clamped to it (the
    // swizzle depends on the row's position in the tile only: bits 2 and 5,
    // unchanged by whole steps)
#pragma unroll
    for (int q = 0; q < TQ_I; ++q) {
      const int t = min(qR[q] + kt * TKK, a.T - 1);
      load16_to_lds(gQ[q] + (int64_t)t * pr.ldq,
                    __builtin_amdgcn_readfirstlane(base + (w * TQ_I + q) * 1024));
    }
#pragma unroll
    for (int q = 0; q < TP_I; ++q)
      load16_to_lds(gP[q] + kt * TKK,
                    __builtin_amdgcn_readfirstlane(base + TQ_BYTES + (w * TP_I + q) * 1024));
  };

  v4f acc[TNB];
#pragma unroll
  for (int i = 0; i < TNB; ++i)
#pragma unroll
    for (int v = 0; v < 4; ++v) acc[i][v] = 0.0f;

  if (nk > 0) issue_e(0);
#pragma unroll
  for (int s = 0; s < TKS - 1; ++s)
    if (s < nk) issue(s, s);

  const int r16 = lane & 15, g = lane >> 4;
  const int sw = swz8(r16);
  const int offP = TQ_BYTES + (rb * 16 + r16) * TKK;
  const int p0 = ((2 * g) ^ sw) * 16, p1 = ((2 * g + 1) ^ sw) * 16;
  // transpose reads: lane (g, s = r16) reads row 32 g + 8 i + s / 2 of the
  // FP8 tile, bytes 8 (s % 2) .. +7 of its 16-byte column chunk
  const int trow = 32 * g + (r16 >> 1), thalf = 8 * (r16 & 1);
  // one step: stage kt has landed (with any window issued before it) once
  // the loads of the `after` stages issued after it are all that is left in
  // flight; then its operands, the loads of step kt + TKS - 1, the MFMAs
  auto step = [&](int kt, int after, bool refill) {
    if (after >= 2) wait_vmem(2 * TLPS); else if (after == 1) wait_vmem(TLPS); else wait_vmem(0);
    barrier_no_drain();
    const uint8_t* st = smem + (kt % TKS) * TSTAGE;
    v8i pf[3], qf[TNB];
    const int eb = smem[TE_OFF + ((kt / TEW) & 1) * TE_WIN + (kt % TEW) * (TKR * 4) +
                        (rb * 16 + r16) * 4 + g];
#pragma unroll
    for (int p = 0; p < 3; ++p) {
      const uint8_t* pp = st + offP + p * TP_PLANE;
      pf[p] = join8(*reinterpret_cast<const uint4*>(pp + p0), *reinterpret_cast<const uint4*>(pp + p1));
    }
#pragma unroll
    for (int bb = 0; bb < TNB; ++bb) {
      const int c = nh * TNB + bb;                                // 16-column chunk
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int t = trow + 8 * i;
        lds_u8* src = (lds_u8*)(st + t * TKN + ((c ^ swz4(t)) * 16) + thalf);
        const v2i x = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_v2i*)src);
        qf[bb][2 * i] = x[0];
        qf[bb][2 * i + 1] = x[1];
      }
    }
    if (refill) issue((kt + TKS - 1) % TKS, kt + TKS - 1);
    if (QF0 == 0 || pi)
      mma_pieces<0>(qf, pf, eb, acc);
    else
      mma_pieces<QF0>(qf, pf, eb, acc);
  };
  __builtin_amdgcn_s_waitcnt(0xC07F);                        // lgkmcnt(0)
  int kt = 0;
  // steady state: TKS - 2 stages behind each, and one to refill
  for (; kt + TKS - 1 < nk; ++kt) step(kt, TKS - 2, true);
  // the last TKS - 1 steps (or fewer)
  for (; kt < nk; ++kt) step(kt, min(TKS - 2, nk - 1 - kt), false);

  // lane: rank j0 + rb * 16 + r16, columns n0 + nh * 32 + 16 bb + 4 g .. +3
  const int j = j0 + rb * 16 + r16;
  if (j >= a.r) return;
  const float inv = 1.0f / pr.sq[0];
#pragma unroll
  for (int bb = 0; bb < TNB; ++bb) {
    const int n = n0 + nh * 32 + 16 * bb + 4 * g;
    const v4f v = acc[bb] * inv;
    if (a.S > 1) {
#pragma unroll
      for (int e = 0; e < 4; ++e)
        unsafeAtomicAdd(pr.out + (pr.n_major ? (int64_t)(n + e) * a.r + j : (int64_t)j * pr.N + n + e),
                        v[e]);
    } else if (pr.n_major) {
#pragma unroll
      for (int e = 0; e < 4; ++e) pr.out[(int64_t)(n + e) * a.r + j] = v[e];
    } else {
      *reinterpret_cast<v4f*>(pr.out + (int64_t)j * pr.N + n) = v;
    }
  }
}

// Pieces of the problems' float factors F [T x r] (element (t, j) at
// F[t * r + j]) where no earlier kernel formed them: blocks [0, ub) those of
// U, [ub, ub + vb) those of V, the rest clear the outputs (n0 floats of z0,
// n1 of z1) that the two token halves are added onto.
constexpr int kUvThreads = 1024, kUvZero = 16;

__global__ __launch_bounds__(kUvThreads) void uv_pieces_kernel(PieceJob u, int64_t ub, PieceJob v,
                                                               int64_t vb, float* z0, int64_t n0,
                                                               float* z1, int64_t n1) {
  int64_t b = blockIdx.x;
  if (b < ub + vb) {
    const bool is_u = b < ub;
    const PieceJob& q = is_u ? u : v;
    const int64_t gid = (is_u ? b : b - ub) * kUvThreads + threadIdx.x;
    // a job's lanes come in whole waves
    if (gid < piece_job_lanes<false>(q.Rp, q.Kp)) piece_job_lane<false>(q, gid);
    return;
  }
  b -= ub + vb;
#pragma unroll
  for (int i = 0; i < kUvZero; ++i) {
    const int64_t k = (b * kUvZero + i) * kUvThreads + threadIdx.x;
    if (k < n0) z0[k] = 0.0f;
    if (k < n1) z1[k] = 0.0f;
  }
}

struct TokPlan {
  int64_t Tp, Rp;
  int S, kps, tiles[2];
  size_t p[2], e[2], total;
};

TokPlan tok_plan(int64_t T, int64_t d_in, int64_t d_out, int64_t r, bool want_da) {
  TokPlan q{};
  q.Tp = (T + TKK - 1) / TKK * TKK;
  q.Rp = (r + TKR - 1) / TKR * TKR;
  const int64_t rtiles = q.Rp / TKR;
  q.tiles[0] = (int)(rtiles * (d_out / TKN));
  q.tiles[1] = want_da ? (int)(rtiles * (d_in / TKN)) : 0;
  const int64_t tiles = q.tiles[0] + q.tiles[1];
  const int64_t nk = q.Tp / TKK;
  // two token halves when the tiles alone fill less than half the GPU (128
  // of its 256 CUs) and each half has at least two steps (at 4096^2, r = 64:
  // 128 tiles, one split measured 18.4 us against 19.0 us for two halves
  // with their atomics and the clearing of the outputs)
  q.S = (tiles < 128 && nk >= 4) ? 2 : 1;
  q.kps = (int)((nk + q.S - 1) / q.S);
  size_t o = 0;
  auto take = [&](size_t bytes) { size_t at = o; o = align_up(o + bytes, 256); return at; };
  for (int i = 0; i < 2; ++i) {
    q.p[i] = take((size_t)(3 * q.Rp * q.Tp));
    q.e[i] = take((size_t)(q.Tp / TKK * q.Rp * 4));
  }
  q.total = o;
  return q;
}

}  // namespace

bool token_grads_ok(int64_t T, int64_t d_in, int64_t d_out, int64_t r) {
  return T > 0 && r > 0 && d_in > 0 && d_out > 0 && d_in % TKN == 0 && d_out % TKN == 0 &&
         T <= ((int64_t)1 << 30) && r <= ((int64_t)1 << 20);
}

size_t token_grads_ws_bytes(int64_t T, int64_t d_in, int64_t d_out, int64_t r) {
  if (!token_grads_ok(T, d_in, d_out, r)) return 0;
  return tok_plan(T, d_in, d_out, r, true).total;
}

void token_grads_pieces(void* ws, int64_t T, int64_t d_in, int64_t d_out, int64_t r, int which,
                        uint8_t** P, uint8_t** E, int64_t* Rp, int64_t* Tp) {
  const TokPlan q = tok_plan(T, d_in, d_out, r, true);
  uint8_t* base = reinterpret_cast<uint8_t*>(ws);
  *P = base + q.p[which];
  *E = base + q.e[which];
  *Rp = q.Rp;
  *Tp = q.Tp;
}

hipError_t launch_token_grads(const uint8_t* gq, int g_fmt, const float* s_g, const uint8_t* xq,
                              const float* s_x, const float* u, bool u_ready, const float* v,
                              bool v_ready, int64_t T, int64_t d_in, int64_t d_out, int64_t r,
                              float* dA, float* dB, void* ws, hipStream_t s) {
  const bool want_da = dA != nullptr;
  const TokPlan q = tok_plan(T, d_in, d_out, r, want_da);
  uint8_t* base = reinterpret_cast<uint8_t*>(ws);
  {
    const PieceJob ju{u, 1, r, r, T, base + q.p[0], base + q.e[0], q.Rp, q.Tp};
    const PieceJob jv{v, 1, r, r, T, base + q.p[1], base + q.e[1], q.Rp, q.Tp};
    const int64_t jobs = (piece_job_lanes<false>(q.Rp, q.Tp) + kUvThreads - 1) / kUvThreads;
    const int64_t ub = u_ready ? 0 : jobs, vb = v_ready || !want_da ? 0 : jobs;
    // clearing blocks (two token halves only): kUvThreads * kUvZero floats each
    const int64_t n0 = q.S > 1 ? d_out * r : 0, n1 = q.S > 1 && want_da ? r * d_in : 0;
    const int64_t per = (int64_t)kUvThreads * kUvZero;
    const int64_t zb = (std::max(n0, n1) + per - 1) / per;
    if (ub + vb + zb > 0) {
      uv_pieces_kernel<<<(unsigned)(ub + vb + zb), kUvThreads, 0, s>>>(ju, ub, jv, vb, dB, n0, dA,
                                                                       n1);
      hipError_t e = hipGetLastError();
      if (e != hipSuccess) return e;
    }
  }
  TokArgs a{};
  a.p[0] = TokProb{gq, d_out, s_g, base + q.p[0], base + q.e[0], dB, (int)d_out, 1,
                   (int)(d_out / TKN), q.tiles[0] * q.S};
  a.p[1] = TokProb{xq, d_in, s_x, base + q.p[1], base + q.e[1], dA, (int)d_in, 0,
                   (int)(d_in / TKN), q.tiles[1] * q.S};
  a.T = (int)T;
  a.Tp = (int)q.Tp;
  a.r = (int)r;
  a.Rp = (int)q.Rp;
  a.S = q.S;
  a.kps = q.kps;
  const int grid = (q.tiles[0] + q.tiles[1]) * q.S;
  if (g_fmt == 0)
    tok_kernel<0><<<grid, kTkThreads, 0, s>>>(a);
  else
    tok_kernel<1><<<grid, kTkThreads, 0, s>>>(a);
  return hipGetLastError();
}

}  // namespace falq
