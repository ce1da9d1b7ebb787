// Transposition of 16-bit matrices through LDS, 64 x 64 tiles, 16-byte global
// accesses on both sides.
//
// One workgroup of 256 threads moves a strip of 64 source rows by 64 * ntile
// source columns, one 64 x 64 tile after another; the next tile's global loads
// are issued before the current tile goes through LDS, and the source row
// pointers (which may come from a gather map) are resolved once per strip.
#pragma once

#include "common.h"

namespace moe {

// src_row(r), r < 64: pointer to source row r of the strip (its column 0), or
// nullptr for a row of zeros.  dst_row(j, c): pointer to the 64 contiguous
// destination elements that receive column 64 j + c of the strip (source rows
// 0 .. 63 in order).  Must be called by all 256 threads of the workgroup.
template <typename SrcRow, typename DstRow>
__device__ __forceinline__ void transpose_strip16(int ntile, SrcRow src_row, DstRow dst_row) {
  // row stride 66 halves (132 bytes): the column-wise writes of a wavefront and the
  // row-wise reads land on different banks
  __shared__ uint16_t tile[64][66];
  const int t = threadIdx.x;
  const int r = t >> 2, q = (t & 3) * 16;   // load side: source row r, columns q .. q+15
  const int c = t >> 2, p = (t & 3) * 16;   // store side: destination row c, source rows p .. p+15
  const uint16_t* s = reinterpret_cast<const uint16_t*>(src_row(r));
  u32x4 a = {0u, 0u, 0u, 0u}, b = {0u, 0u, 0u, 0u};
  auto load = [&](int j) {
    if (s) {
      a = *reinterpret_cast<const u32x4*>(s + 64 * j + q);
      b = *reinterpret_cast<const u32x4*>(s + 64 * j + q + 8);
    }
  };
  load(0);
  for (int j = 0; j < ntile; ++j) {
    const u32x4 ca = a, cb = b;
    if (j + 1 < ntile) load(j + 1);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      tile[q + 2 * e][r] = (uint16_t)(ca[e] & 0xffffu);
      tile[q + 2 * e + 1][r] = (uint16_t)(ca[e] >> 16);
      tile[q + 8 + 2 * e][r] = (uint16_t)(cb[e] & 0xffffu);
      tile[q + 8 + 2 * e + 1][r] = (uint16_t)(cb[e] >> 16);
    }
    __syncthreads();
    const uint32_t* row = reinterpret_cast<const uint32_t*>(&tile[c][0]) + p / 2;
    u32x4 o0, o1;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      o0[e] = row[e];
      o1[e] = row[4 + e];
    }
    uint16_t* d = reinterpret_cast<uint16_t*>(dst_row(j, c));
    *reinterpret_cast<u32x4*>(d + p) = o0;
    *reinterpret_cast<u32x4*>(d + p + 8) = o1;
    __syncthreads();
  }
}

}  // namespace moe
