// Packed forms of the D x D matrices (D = 128) that the three MFMA kernels
// exchange inside gdn_frame_fwd.  Each is laid out in the exact order the
// consuming kernel's waves read it, so every consumer load is one contiguous
// 1 KB (or 512 B) block per wave instruction.  All three are 64 KiB per
// (head, frame), the same as a float32 matrix.
//
// Notation: a "row block" rb is 16 consecutive rows, a "column block" cb is
// 16 consecutive columns; lane l = n + 16 g with n = l % 16, g = l / 16.
//
//  Gp  (G_t, bf16 hi/lo planes): 64 units of 1 KB, unit (cb, kb, plane) at
//      ((cb * 4 + kb) * 2 + plane) KiB; inside it lane l holds the 8 bf16 of
//      row 16 cb + n, columns 32 kb + 8 g .. +7.  G is symmetric, so these
//      are the MFMA A-operand rows of G^T as well.
//  Up  (U_t, float32): 64 units of 1 KB, unit (rb, cb) at (rb * 8 + cb) KiB;
//      lane l holds row 16 rb + n, columns 16 cb + 4 g .. +3.
//  Mp  (M_t, bf16 hi/lo planes): 128 units of 512 B, unit (rb, cb, plane)
//      at ((rb * 8 + cb) * 2 + plane) * 512 B; lane l holds the 4 bf16 of
//      row 16 rb + n, columns 16 cb + 4 g .. +3.
#pragma once

#include <stdint.h>

namespace gdn {
namespace packed {

constexpr int kD = 128;
constexpr int64_t kFrameBytes = int64_t{kD} * kD * 4;

// byte offset of the 16-byte chunk holding G[r][c .. c+7] (c % 8 == 0) in Gp
__host__ __device__ constexpr int g_chunk(int r, int c, int plane) {
  return ((((r >> 4) * 4 + (c >> 5)) * 2 + plane) << 10) + (((r & 15) + 16 * ((c & 31) >> 3)) << 4);
}
// byte offset of the 16-byte chunk holding U[r][c .. c+3] (c % 4 == 0) in Up
__host__ __device__ constexpr int u_chunk(int r, int c) {
  return (((r >> 4) * 8 + (c >> 4)) << 10) + (((r & 15) + 16 * ((c & 15) >> 2)) << 4);
}
// byte offset of the 8-byte chunk holding M[r][c .. c+3] (c % 4 == 0) in Mp
__host__ __device__ constexpr int m_chunk(int r, int c, int plane) {
  return ((((r >> 4) * 8 + (c >> 4)) * 2 + plane) << 9) + (((r & 15) + 16 * ((c & 15) >> 2)) << 3);
}

}  // namespace packed
}  // namespace gdn
