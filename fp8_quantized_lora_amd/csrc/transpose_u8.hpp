// Byte-matrix transpose tile, shared by the stand-alone transpose launch and
// the backward's preparation kernel.
#pragma once

#include "common.hpp"

namespace falq {

// A 16 x 4 byte block (d[i] = 4 bytes of row i) as 4 x 16: o[k][g] holds
// bytes k of rows 4g .. 4g + 3, so that o[k][0..3] is column k's 16 bytes.
// Byte permutes only.
__device__ __forceinline__ void transpose_16x4(const uint32_t (&d)[16], uint32_t (&o)[4][4]) {
#pragma unroll
  for (int g = 0; g < 4; ++g) {                             // rows 4g .. 4g+3
    const uint32_t t01a = __builtin_amdgcn_perm(d[4 * g + 1], d[4 * g], 0x05010400u);
    const uint32_t t01b = __builtin_amdgcn_perm(d[4 * g + 1], d[4 * g], 0x07030602u);
    const uint32_t t23a = __builtin_amdgcn_perm(d[4 * g + 3], d[4 * g + 2], 0x05010400u);
    const uint32_t t23b = __builtin_amdgcn_perm(d[4 * g + 3], d[4 * g + 2], 0x07030602u);
    o[0][g] = __builtin_amdgcn_perm(t23a, t01a, 0x05040100u);
    o[1][g] = __builtin_amdgcn_perm(t23a, t01a, 0x07060302u);
    o[2][g] = __builtin_amdgcn_perm(t23b, t01b, 0x05040100u);
    o[3][g] = __builtin_amdgcn_perm(t23b, t01b, 0x07060302u);
  }
}

// out[cols x rows] = in[rows x cols]^T, the 128 x 128 tile (bx, by) of a
// matrix whose sizes are multiples of 16; 256 threads (tid 0 .. 255, by
// default the workgroup's own).  Each thread loads 16 rows x 4 bytes (a wave
// reads two 128-byte row segments per load), transposes them in registers
// with byte permutes, and stores 4 output rows x 16 bytes.  No LDS and no
// barrier: threads past the matrix return.
__device__ __forceinline__ void transpose_u8_tile(const uint8_t* __restrict__ in, int64_t rows,
                                                  int64_t cols, uint8_t* __restrict__ out, int bx,
                                                  int by, int tid = -1) {
  if (tid < 0) tid = threadIdx.x;
  const int cg = tid & 31, rg = tid >> 5;
  const int64_t c = (int64_t)bx * 128 + cg * 4;             // 4 input columns
  const int64_t r = (int64_t)by * 128 + rg * 16;            // 16 input rows
  if (c >= cols || r >= rows) return;                       // whole 16 x 4 blocks only
  uint32_t d[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) d[i] = *reinterpret_cast<const uint32_t*>(in + (r + i) * cols + c);
  uint32_t o[4][4];                                         // [column][4 rows]
  transpose_16x4(d, o);
#pragma unroll
  for (int k = 0; k < 4; ++k)
    *reinterpret_cast<uint4*>(out + (c + k) * rows + r) = make_uint4(o[k][0], o[k][1], o[k][2], o[k][3]);
}

}  // namespace falq
