// tile_ops.h -- bf16 tile building blocks shared by the fused kernel and the split passes:
// the transposed-logits softmax of one 16-token tile, transposing LDS reads and the
// phase-B tile accumulation built on them, and streaming row loads in MFMA operand layout.
#pragma once
#include "device_common.h"

namespace aa {

// With at most 64 anchors padding lies in the last two tiles: mask[h] is the initial
// accumulator of anchor tile 2MP - 2 + h.
template <int MP>
__device__ __forceinline__ void pad_mask(int g, int m, f32x4* mask) {
  static_assert(pad_tiles(2 * MP) == 2, "tile_softmax masks the last two tiles");
  pad_mask_tiles<2 * MP, 2>(g, m, mask);
}

// UOP: U's left operands, uop(j, kk) for anchor tile j and dim chunk kk (from LDS or
// registers).
template <int D, int MP, typename UOP>
__device__ __forceinline__ void tile_softmax_op(UOP uop, const u32x4* q, const f32x4* mask,
                                                bool token_ok, float c2, bf16x8* ab) {
  constexpr int KS = D / 32, AT = 2 * MP;
  f32x4 s[AT];
#pragma unroll
  for (int j = 0; j < AT; ++j) {
    f32x4 acc = (j >= AT - 2) ? mask[j - (AT - 2)] : zero4();
#pragma unroll
    for (int kk = 0; kk < KS; ++kk) acc = mfma_bf16(uop(j, kk), as_bf16x8(q[kk]), acc);
    s[j] = acc;
  }
  float mx = s[0][0];
#pragma unroll
  for (int j = 0; j < AT; ++j)
#pragma unroll
    for (int r = 0; r < 4; ++r) mx = fmaxf(mx, s[j][r]);
  mx = xor32_max(xor16_max(mx));
  const float mneg = -mx * c2;
  float z = 0.f;
#pragma unroll
  for (int j = 0; j < AT; ++j)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const float e = exp2_fast(fmaf(s[j][r], c2, mneg));
      s[j][r] = e;
      z += e;
    }
  z = xor32_sum(xor16_sum(z));
  const float inv = token_ok ? __builtin_amdgcn_rcpf(z) : 0.f;   // z >= 1 (the maximum adds 1)
#pragma unroll
  for (int jj = 0; jj < MP; ++jj) ab[jj] = pack_bf16(s[2 * jj] * inv, s[2 * jj + 1] * inv);
}

template <int D, int MP>
__device__ __forceinline__ void tile_softmax(const u32x4 (*u_lds)[D / 32][kWave], const u32x4* q,
                                             int lane, const f32x4* mask, bool token_ok, float c2,
                                             bf16x8* ab) {
  tile_softmax_op<D, MP>([&](int j, int kk) { return as_bf16x8(u_lds[j][kk][lane]); }, q, mask,
                         token_ok, c2, ab);
}

// Unnormalised weights exp(c (u_j . q) - c M_j) of one 16-token tile against the anchor
// rows in u_lds, with mneg[j] = -c M_j (c = c2, log2 units) for a bound M_j >= every
// logit of anchor j; zero for tokens past the end and for padded anchors (their logits
// start from -inf).  Same lane layout as tile_softmax.
template <int D, int MP>
__device__ __forceinline__ void tile_exp(const u32x4 (*u_lds)[D / 32][kWave], const u32x4* q,
                                         int lane, const f32x4* mask, bool token_ok, float c2,
                                         const float* mneg, int g, bf16x8* ab) {
  constexpr int KS = D / 32, AT = 2 * MP;
  f32x4 s[AT];
#pragma unroll
  for (int j = 0; j < AT; ++j) {
    f32x4 acc = (j >= AT - 2) ? mask[j - (AT - 2)] : zero4();
#pragma unroll
    for (int kk = 0; kk < KS; ++kk) acc = mfma_bf16(as_bf16x8(u_lds[j][kk][lane]), as_bf16x8(q[kk]), acc);
    s[j] = acc;
  }
  // keeps the loop-invariant reads of mneg from being hoisted out of the caller's loop
  asm volatile("" ::: "memory");
#pragma unroll
  for (int j = 0; j < AT; ++j) {
    const f32x4 mn = *(const f32x4*)(mneg + 16 * j + 4 * g);
#pragma unroll
    for (int r = 0; r < 4; ++r) s[j][r] = token_ok ? exp2_fast(fmaf(s[j][r], c2, mn[r])) : 0.f;
  }
#pragma unroll
  for (int jj = 0; jj < MP; ++jj) ab[jj] = pack_bf16(s[2 * jj], s[2 * jj + 1]);
}

// ---- transposing LDS reads (gfx950 ds_read_b64_tr_b16) ----------------------------------
// Within each 16-lane group every lane reads 8 bytes (4 x 16-bit) at its own address;
// lane i receives, in slot k, element i % 4 of what lane 4k + i / 4 read.
typedef short s16x4 __attribute__((__vector_size__(4 * sizeof(short))));
typedef short s16x8 __attribute__((__vector_size__(8 * sizeof(short))));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

__device__ __forceinline__ s16x4 lds_read_tr(const __bf16* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (lds_s16x4*)(__attribute__((address_space(3))) char*)(p));
}

// Row stride (bf16 elements) of a row-major LDS block with rows of L = 32 or 64 values:
// 16 values of padding put the eight rows that one transposing read serves per pass on
// distinct banks.
template <int L>
constexpr int tr_stride() { return L + 16; }

// MFMA operand whose contraction axis runs over the 32 rows of a row-major bf16 LDS
// block: lane (c, g) gets column col0 + c of rows 4g + s (slot s < 4) and 16 + 4g + s - 4
// (s >= 4).  Lane 4k + q of group g points at row 4g + k, columns col0 + 4q .. + 3.
__device__ __forceinline__ bf16x8 lds_operand_tr(const __bf16* blk, int stride, int col0, int c,
                                                 int g) {
  const __bf16* p = blk + (4 * g + (c >> 2)) * stride + col0 + 4 * (c & 3);
  const s16x4 lo = lds_read_tr(p);
  const s16x4 hi = lds_read_tr(p + 16 * stride);
  const s16x8 v = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  return __builtin_bit_cast(bf16x8, v);
}

// Phase B of a wave that owns the TPW contiguous tiles t0 .. t0 + TPW - 1 (t0 a multiple
// of TPW) of an (anchor tile, dim tile) grid with DT dim tiles per anchor tile (tile t:
// anchor tile t / DT, dim tile t % DT): accumulates P += A^T V for each tile (pacc[k])
// and, for a tile in dim tile 0, Delta += A^T 1 of its anchor tile (dacc[k / DT]), over
// `pairs` 32-row blocks of the row-major LDS copies of A (stride AS) and V (stride VS).
// When TPW is a multiple or a divisor of DT each distinct operand is read once per block;
// otherwise every tile reads its own two operands.  DELTA = false skips the column sums.
template <int TPW, int DT, int AS, int VS, bool DELTA = true>
__device__ __forceinline__ void accumulate_tiles(const __bf16* a_lds, const __bf16* v_lds, int t0,
                                                 int pairs, int c, int g, bf16x8 ones,
                                                 f32x4* pacc, f32x4* dacc) {
  if constexpr (TPW % DT == 0 || DT % TPW == 0) {
    constexpr bool BYROW = TPW % DT == 0;          // whole anchor tiles per wave
    constexpr int NJ = BYROW ? TPW / DT : 1;       // anchor tiles of the wave
    constexpr int NY = BYROW ? DT : TPW;           // dim tiles of the wave
    const int ja0 = t0 / DT, dt0 = t0 - ja0 * DT;  // dt0 == 0 when BYROW
    for (int ps = 0; ps < pairs; ++ps) {
      bf16x8 xs[NJ], ys[NY];
#pragma unroll
      for (int jl = 0; jl < NJ; ++jl)
        xs[jl] = lds_operand_tr(a_lds + 32 * ps * AS, AS, 16 * (ja0 + jl), c, g);
#pragma unroll
      for (int iy = 0; iy < NY; ++iy)
        ys[iy] = lds_operand_tr(v_lds + 32 * ps * VS, VS, 16 * (dt0 + iy), c, g);
#pragma unroll
      for (int k = 0; k < TPW; ++k) {
        const int jl = BYROW ? k / DT : 0, iy = BYROW ? k % DT : k;
        pacc[k] = mfma_bf16(xs[jl], ys[iy], pacc[k]);
        if (DELTA && dt0 + iy == 0) dacc[k / DT] = mfma_bf16(xs[jl], ones, dacc[k / DT]);
      }
    }
  } else {
    for (int ps = 0; ps < pairs; ++ps) {
#pragma unroll
      for (int k = 0; k < TPW; ++k) {
        const int t = t0 + k, ja = t / DT, dt = t - ja * DT;
        const bf16x8 x = lds_operand_tr(a_lds + 32 * ps * AS, AS, 16 * ja, c, g);
        const bf16x8 y = lds_operand_tr(v_lds + 32 * ps * VS, VS, 16 * dt, c, g);
        pacc[k] = mfma_bf16(x, y, pacc[k]);
        if (DELTA && dt == 0) dacc[k / DT] = mfma_bf16(x, ones, dacc[k / DT]);
      }
    }
  }
}

// Loads rows of Q or V in operand layout (lane (c,g): dims 8*KS*g ..), streaming (each
// byte is read once, so the loads are marked non-temporal).  Row r starts at element
// base + r * st.  Rows past the
// slice's end read its last row instead; their softmax weights are zeroed, so they add
// nothing (and a non-finite value there belongs to the same slice anyway).
template <int D>
__device__ __forceinline__ void load_rows(const __bf16* __restrict__ X, size_t base, long long st,
                                          int row, int n, int g, u32x4* out) {
  constexpr int KS = D / 32;
  const size_t off = base + (size_t)((long long)min(row, n - 1) * st) + 8 * KS * g;
#pragma unroll
  for (int kk = 0; kk < KS; ++kk) out[kk] = __builtin_nontemporal_load((const u32x4*)(X + off + 8 * kk));
}

// Rows of Q or V, DW dims from d0, with lane (c,g) holding dims d0 + 32kk + 8g .. + 7 in
// chunk kk: each load instruction reads one contiguous 64-byte run per row (a whole row
// when d = 32).  Rows past the slice's end read its last row, as in load_rows.
template <int D, int DW>
__device__ __forceinline__ void load_rows_c(const __bf16* __restrict__ X, size_t base, long long st,
                                            int row, int n, int g, int d0, u32x4* out) {
  const size_t off = base + (size_t)((long long)min(row, n - 1) * st) + d0 + 8 * g;
#pragma unroll
  for (int kk = 0; kk < DW / 32; ++kk)
    out[kk] = __builtin_nontemporal_load((const u32x4*)(X + off + 32 * kk));
}

// Output dim of accumulator row i (= 4g + r) of output dim tile dt2, chosen so that lane
// group g owns dims 32h + 8g .. + 7 for h = dt2 / 2: two adjacent tiles pack into one
// 16-byte store, and each store instruction covers a contiguous 64-byte run per row.
__host__ __device__ constexpr int out_dim_c(int dt2, int i) {
  return 32 * (dt2 >> 1) + 8 * (i >> 2) + 4 * (dt2 & 1) + (i & 3);
}

}  // namespace aa
