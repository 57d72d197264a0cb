// pass2_layout.h -- the W^T operand layout that pass 2 of the split plan reads (written by
// the forward's finalize and by the Nystrom solve).
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

}  // namespace aa
