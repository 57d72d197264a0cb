// pass2_layout.h -- the W^T operand layout that the split plan's output passes read
// (forward pass 2, written by the forward's finalize and by the Nystrom solve; the
// backward's token pass), and their workgroup-to-(slice, chunk) mapping.
#pragma once
#include "device_common.h"
#include "tile_ops.h"

namespace aa {

// (anchor a, dim k) -> element of one slice's block of pass 2's W^T operands
// [dt2][jj][lane'][slot]: lane' (c', g') of [dt2][jj] holds dim out_dim_c(dt2, c') and
// anchors 32jj + 4g' + slot (slot < 4) and 32jj + 16 + 4g' + slot - 4 (slot >= 4).  With
// out_dim_c, lane group g of the output tiles 2h and 2h + 1 holds dims 32h + 8g .. + 7 of
// its token, so each 16-byte store of an output instruction lands in one contiguous
// 64-byte run per row.
__device__ __forceinline__ size_t w2_layout_index(int MP, int a, int k) {
  const int q = k & 31, dt2 = 2 * (k >> 5) + ((q & 7) >> 2), cc = 4 * (q >> 3) + (q & 3);
  const int jj = a >> 5, half = (a >> 4) & 1, gg = (a >> 2) & 3;
  return ((((size_t)dt2 * MP + jj) * kWave) + 16 * gg + cc) * 8 + 4 * half + (a & 3);
}

// Workgroup b of a grid of slices x chunks -> (slice, chunk).  Workgroups are dealt to the
// eight XCDs in turn (b to XCD b % 8); when the slices divide by eight, all chunks of a
// slice get ids on one XCD, so the slice's operands staged by every chunk are fetched into
// one L2 instead of eight.
__device__ __forceinline__ void slice_chunk_of(int b, int chunks, int& slice, int& chunk) {
  const int slices = (int)gridDim.x / chunks;
  if ((slices & 7) == 0) {
    const int k = b >> 3, ls = k / chunks;
    slice = 8 * ls + (b & 7);
    chunk = k - ls * chunks;
  } else {
    slice = b / chunks;
    chunk = b - slice * chunks;
  }
}

}  // namespace aa
