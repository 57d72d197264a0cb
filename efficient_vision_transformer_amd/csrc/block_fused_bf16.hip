// block_fused_bf16.hip -- the attention block's Q|V projection fused in front of the anchor
// attention: one workgroup per (batch b, head j) slice projects its own tokens and runs the
// layer on the result, so the projection never goes to HBM.
//
// The block (the layer dropped into a ViT block in place of self-attention: Pith verdict
// page on AnchorFormer, the DeiT / LeViT backbones among its supporting citations; the
// pages print no projections, so the plain multi-head reading), for X [B, n, C], C = h*d:
//   [Q | V] = X Wqv + bqv           head j: columns j*d .. of Q and C + j*d .. of V
//   H       = A (Delta^-1 (A^T V))  per slice, A = rowsoftmax(Q U^T / sqrt(d))
// with Q and V rounded to bf16 before the layer (as when they are stored).  This kernel
// writes H into [B, n, C] (head-major columns); the output projection follows separately.
//
// Per round of one 32-token pair per wave:
//   Projection: [Q|V]^T = Wqv_j^T X^T on the MFMA, features (the head's d query and d value
//     columns) on the M axis and the pair's tokens on N, the C-long contraction in chunks of
//     32 rows of Wqv staged in LDS (three buffers; read with the transposing LDS read, the
//     rows stored in the order that read hands them to each lane group) and X read from
//     global memory in 16-byte pieces (L2-resident: the heads of one image run on one XCD).
//     The accumulators start from the bias.
//   Q^T's accumulators are already the right operand of the logits S^T = U Q^T once
//     rounded to bf16 (their dims follow the same numbering, and U is staged with it), and
//     V^T's go to the LDS rows of V as 8-byte runs.
//   Then the fused kernel's phases: softmax in registers (A kept), A^T V and Delta over the
//   round's pairs from the LDS row copies, W = Delta^-1 P, H^T = W^T A^T stored.
#include <type_traits>

#include "device_common.h"
#include "kernels.h"
#include "tile_ops.h"

namespace aa {

template <int D, int MP, int NW>
struct BlockLds {
  static constexpr int AT = 2 * MP, KS = D / 32, DT = D / 16, F = 2 * D;
  static constexpr int AS = tr_stride<32 * MP>(), VS = tr_stride<D>();
  static constexpr int WS = F + 16;   // row stride of a staged chunk of Wqv (bank spread)
  u32x4 u[AT][KS][kWave];             // U as left operands, dims numbered as Q's operand
  union {
    struct {
      __attribute__((aligned(16))) __bf16 a[NW * 32 * AS];   // rows of A (after projection)
      __attribute__((aligned(16))) __bf16 v[NW * 32 * VS];   // rows of V, this round
    } av;
    __attribute__((aligned(16))) __bf16 wc[3][32 * WS];      // chunks of Wqv_j (projection)
  } x;
  u32x4 w[DT][MP][kWave];                                  // W^T left operands
  float dl[AT][16];                                        // Delta per anchor tile
};

// X row `tok` (clamped to the slice) of image b: lane group g's piece of chunk kc of the right
// operand, contraction rows 8g .. 8g + 7 of the chunk (one 16-byte load).
__device__ __forceinline__ bf16x8 x_operand(const __bf16* __restrict__ xrow, int kc, int g) {
  return as_bf16x8(*(const u32x4*)(xrow + 32 * kc + 8 * g));
}

// LDS row of contraction row k (0 .. 31) of a staged chunk of Wqv.  The transposing read
// hands lane group g rows 4g + s (s < 4) and 16 + 4g + s - 4 (s >= 4) of the block; storing
// row 8g + s there makes that the chunk's rows 8g .. 8g + 7, the rows X's operand holds.
__device__ __forceinline__ int w_lds_row(int k) { return ((k & 4) << 2) + 4 * (k >> 3) + (k & 3); }

// Workgroup -> slice: when the batch divides by eight, the h heads of an image get
// consecutive local ids on one XCD (workgroup k runs on XCD k % 8), so X's rows are
// fetched into one L2 and read there by all heads.
__device__ __forceinline__ int block_slice_of(int k, int B, int h) {
  if ((B & 7) != 0) return k;
  const int xcd = k & 7, local = k >> 3;
  return (xcd + 8 * (local / h)) * h + local % h;
}

template <int D, int MP, int NW, int ROUNDS, int MINW>
__global__ __launch_bounds__(NW * kWave, MINW)
void block_fused_bf16(const __bf16* __restrict__ X, const __bf16* __restrict__ Wqv,
                      const __bf16* __restrict__ bqv, const __bf16* __restrict__ U,
                      __bf16* __restrict__ H, int B, int h, int n, int m, float c2) {
  using L_t = BlockLds<D, MP, NW>;
  constexpr int KS = D / 32, DT = D / 16, AT = 2 * MP, FT = 2 * DT;   // FT feature tiles
  constexpr int AS = L_t::AS, VS = L_t::VS, WS = L_t::WS;
  constexpr int TILES = AT * DT, TPW = (TILES + NW - 1) / NW;
  constexpr int NDA = (TPW + DT - 1) / DT;
  static_assert(TILES % NW == 0 || NW % TILES == 0, "tiles split evenly over the waves");
  __shared__ L_t L;
  const int C = h * D;
  const int slice = block_slice_of((int)blockIdx.x, B, h);
  const int b = slice / h, head = slice - b * h;
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int c = lane & 15, g = lane >> 4;
  const int npairs = (n + 31) >> 5;
  const int nkc = C / 32;                       // contraction chunks of 32 rows
  const __bf16* Xb = X + (size_t)b * n * C;

  // U as left operands of S^T = U Q^T: lane (c,g) of tile j, chunk kk holds anchor 16j + c
  // at dims 32kk + 4g + s (s < 4) and 32kk + 16 + 4g + s - 4 (s >= 4), the numbering of the
  // projected Q operand.  Padded anchors are zero rows (their logits start from -inf).
  const __bf16* Uh = U + (size_t)head * m * D;
  for (int idx = threadIdx.x; idx < AT * KS * kWave; idx += NW * kWave) {
    const int j = idx / (KS * kWave), kk = (idx / kWave) % KS, l = idx & 63;
    const int a = 16 * j + (l & 15), gg = l >> 4;
    u32x4 v = {0u, 0u, 0u, 0u};
    if (a < m) {
      const u32x2 lo = *(const u32x2*)(Uh + (size_t)a * D + 32 * kk + 4 * gg);
      const u32x2 hi = *(const u32x2*)(Uh + (size_t)a * D + 32 * kk + 16 + 4 * gg);
      v = u32x4{lo[0], lo[1], hi[0], hi[1]};
    }
    L.u[j][kk][l] = v;
  }
  // Bias of this lane's accumulator rows: feature tile ft < DT is Q dims 16ft + 4g + r,
  // ft >= DT is V dims 16(ft - DT) + 4g + r.
  f32x4 bias[FT];
  u32x2 bb[FT] = {};
  if (bqv) {   // one branch around all of the loads (one wait for them)
#pragma unroll
    for (int ft = 0; ft < FT; ++ft)
      bb[ft] = *(const u32x2*)(bqv + (ft < DT ? head * D + 16 * ft : C + head * D + 16 * (ft - DT)) + 4 * g);
  }
#pragma unroll
  for (int ft = 0; ft < FT; ++ft) {
    const __bf16* bv = (const __bf16*)&bb[ft];
#pragma unroll
    for (int r = 0; r < 4; ++r) bias[ft][r] = (float)bv[r];
  }
  // Staging of chunk kc of Wqv_j: rows 32kc .. + 31, the head's D query columns then its D
  // value columns, as [row][feature] with row stride WS; F * 32 / 8 16-byte pieces.
  constexpr int WPIECES = 2 * D * 32 / 8;
  constexpr int WPT = (WPIECES + NW * kWave - 1) / (NW * kWave);
  auto wload = [&](int kc, u32x4* st) {
#pragma unroll
    for (int i = 0; i < WPT; ++i) {
      const int idx = (int)threadIdx.x + i * NW * kWave;
      if (WPIECES % (NW * kWave) == 0 || idx < WPIECES) {
        const int row = idx / (2 * D / 8), f8 = idx - row * (2 * D / 8);
        const int f = 8 * f8;
        const int col = f < D ? head * D + f : C + head * D + (f - D);
        st[i] = *(const u32x4*)(Wqv + (size_t)(32 * kc + row) * (2 * C) + col);
      }
    }
  };
  auto wstore = [&](int buf, const u32x4* st) {
#pragma unroll
    for (int i = 0; i < WPT; ++i) {
      const int idx = (int)threadIdx.x + i * NW * kWave;
      if (WPIECES % (NW * kWave) == 0 || idx < WPIECES) {
        const int row = idx / (2 * D / 8), f8 = idx - row * (2 * D / 8);
        *(u32x4*)(&L.x.wc[buf][w_lds_row(row) * WS + 8 * f8]) = st[i];
      }
    }
  };

  const bf16x8 ones = splat_bf16(1.f);
  f32x4 mask[2];
  pad_mask<MP>(g, m, mask);
  f32x4 pacc[TPW], dacc[NDA];
#pragma unroll
  for (int k = 0; k < TPW; ++k) pacc[k] = zero4();
#pragma unroll
  for (int k = 0; k < NDA; ++k) dacc[k] = zero4();
  bf16x8 keep[ROUNDS][2][MP];

#pragma unroll
  for (int r = 0; r < ROUNDS; ++r) {
    const int pairs_here = min(NW, npairs - r * NW);   // uniform over the workgroup
    if (pairs_here <= 0) break;
    const int p = r * NW + w;
    const __bf16* xrow[2];
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) xrow[tt] = Xb + (size_t)min(32 * p + 16 * tt + c, n - 1) * C;

    // ---- projection of this wave's pair: acc[ft][tt] = [Q|V]^T tile (features x tokens)
    f32x4 acc[FT][2];
#pragma unroll
    for (int ft = 0; ft < FT; ++ft)
#pragma unroll
      for (int tt = 0; tt < 2; ++tt) acc[ft][tt] = bias[ft];
    {
      // Three slots: chunk kc's X operands and staged W rows live in slot kc % 3 (in
      // registers, then W in LDS buffer kc % 3).  Chunk kc + 2 is requested while chunk kc
      // is multiplied, and W rows that arrived one chunk earlier go to LDS, so each load
      // has a chunk of products to land behind; slot indices are compile-time after the
      // loop is unrolled by three.
      u32x4 st[3][WPT];
      bf16x8 xo[3][2];
      // Loads are unconditional (a chunk past the end repeats the last one and is never
      // multiplied): loads under branches would make the compiler wait for every load in
      // flight wherever the paths join.
      auto request = [&](int kc, auto slot) {
        constexpr int S = decltype(slot)::value;
        const int k = min(kc, nkc - 1);
        wload(k, st[S]);
#pragma unroll
        for (int tt = 0; tt < 2; ++tt) xo[S][tt] = x_operand(xrow[tt], k, g);
      };
      auto stage = [&](int, auto slot) {
        constexpr int S = decltype(slot)::value;
        wstore(S, st[S]);
      };
      auto multiply = [&](int kc, auto slot) {
        constexpr int S = decltype(slot)::value;
        if (kc < nkc && p < npairs) {
#pragma unroll
          for (int ft = 0; ft < FT; ++ft) {
            const bf16x8 wo = lds_operand_tr(L.x.wc[S], WS, 16 * ft, c, g);
#pragma unroll
            for (int tt = 0; tt < 2; ++tt) acc[ft][tt] = mfma_bf16(wo, xo[S][tt], acc[ft][tt]);
          }
        }
      };
      using S0 = std::integral_constant<int, 0>;
      using S1 = std::integral_constant<int, 1>;
      using S2 = std::integral_constant<int, 2>;
      request(0, S0{});
      request(1, S1{});
      __syncthreads();   // the previous round's phase B no longer reads the A and V rows
      stage(0, S0{});
      __syncthreads();
      for (int kc = 0; kc < nkc; kc += 3) {
        request(kc + 2, S2{});
        stage(kc + 1, S1{});
        multiply(kc, S0{});
        __syncthreads();
        request(kc + 3, S0{});
        stage(kc + 2, S2{});
        multiply(kc + 1, S1{});
        __syncthreads();
        request(kc + 4, S1{});
        stage(kc + 3, S0{});
        multiply(kc + 2, S2{});
        __syncthreads();
      }
    }

    // ---- phase A: Q operands from the projection, softmax, A kept; rows of A and V to LDS
    if (p < npairs) {
#pragma unroll
      for (int tt = 0; tt < 2; ++tt) {
        const int row = 32 * w + 16 * tt + c;
        // V^T tile t: lane (c,g) holds V[token c][16t + 4g + r] -> one 8-byte run of the row
#pragma unroll
        for (int t = 0; t < DT; ++t)
          *(u32x2*)(L.x.av.v + row * VS + 16 * t + 4 * g) = pack4_bf16(acc[DT + t][tt]);
        u32x4 q[KS];
#pragma unroll
        for (int kk = 0; kk < KS; ++kk) q[kk] = as_u32x4(pack_bf16(acc[2 * kk][tt], acc[2 * kk + 1][tt]));
        bf16x8 ab[MP];
        tile_softmax<D, MP>(L.u, q, lane, mask, 32 * p + 16 * tt + c < n, c2, ab);
#pragma unroll
        for (int jj = 0; jj < MP; ++jj) keep[r][tt][jj] = ab[jj];
        __bf16* arow = L.x.av.a + row * AS + 4 * g;
#pragma unroll
        for (int jj = 0; jj < MP; ++jj) {
          const u32x4 v = as_u32x4(ab[jj]);
          *(u32x2*)(arow + 32 * jj) = u32x2{v[0], v[1]};
          *(u32x2*)(arow + 32 * jj + 16) = u32x2{v[2], v[3]};
        }
      }
    }
    __syncthreads();
    // ---- phase B: this wave's (anchor tile, dim tile) tiles of A^T V and Delta
    if (w * TPW < TILES)
      accumulate_tiles<TPW, DT, AS, VS>(L.x.av.a, L.x.av.v, w * TPW, pairs_here, c, g, ones, pacc, dacc);
  }

  // ---- W = P / Delta as bf16 left operands of H^T = W^T A^T (as in the fused kernel)
#pragma unroll
  for (int k = 0; k < TPW; ++k) {
    const int t = w * TPW + k;
    const int ja = t / DT, dt = t - (t / DT) * DT;
    if (t < TILES && dt == 0 && c == 0) {
#pragma unroll
      for (int r = 0; r < 4; ++r) L.dl[ja][4 * g + r] = dacc[k / DT][r];
    }
  }
  __syncthreads();
  {
    __bf16* wl = (__bf16*)&L.w[0][0][0];
#pragma unroll
    for (int k = 0; k < TPW; ++k) {
      const int t = w * TPW + k;
      if (t >= TILES) break;
      const int ja = t / DT, dt = t - (t / DT) * DT;
      const int dim = 16 * dt + c;
      const int q = dim & 31, dt2 = 2 * (dim >> 5) + ((q & 7) >> 2), cc = 4 * (q >> 3) + (q & 3);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int anchor = 16 * ja + 4 * g + r;
        const float delta = L.dl[ja][4 * g + r];
        const float wv = (delta > 0.f) ? pacc[k][r] * __builtin_amdgcn_rcpf(delta) : 0.f;
        const int jj = anchor >> 5, hf = (anchor >> 4) & 1, gg = (anchor >> 2) & 3;
        wl[(((dt2 * MP + jj) * 64) + 16 * gg + cc) * 8 + 4 * hf + (anchor & 3)] = (__bf16)wv;
      }
    }
  }
  __syncthreads();
  bf16x8 wop[DT][MP];
#pragma unroll
  for (int dt2 = 0; dt2 < DT; ++dt2)
#pragma unroll
    for (int jj = 0; jj < MP; ++jj) wop[dt2][jj] = as_bf16x8(L.w[dt2][jj][lane]);

  // ---- output: H [B, n, C] with head j's dims at columns j*D ..
#pragma unroll
  for (int r = 0; r < ROUNDS; ++r) {
    const int p = r * NW + w;
    if (p < npairs) {
#pragma unroll
      for (int tt = 0; tt < 2; ++tt) {
        const int row = 32 * p + 16 * tt + c;
        f32x4 hacc[DT];
#pragma unroll
        for (int dt2 = 0; dt2 < DT; ++dt2) {
          f32x4 a4 = zero4();
#pragma unroll
          for (int jj = 0; jj < MP; ++jj) a4 = mfma_bf16(wop[dt2][jj], keep[r][tt][jj], a4);
          hacc[dt2] = a4;
        }
        if (row < n) {
          __bf16* dst = H + ((size_t)b * n + row) * C + head * D + 8 * g;
#pragma unroll
          for (int hh = 0; hh < DT / 2; ++hh)
            __builtin_nontemporal_store(as_u32x4(pack_bf16(hacc[2 * hh], hacc[2 * hh + 1])),
                                        (u32x4*)(dst + 32 * hh));
        }
      }
    }
  }
}

// Plan: one round of eight waves (m <= 32, n <= 256; A kept in registers), d = 32 or 64.
// Measured at the ViT-B/16-384 block shape (m = 64, n = 576, C = 768: five rounds of four
// waves), projecting in the kernel was slower than the library projection followed by the
// attention kernels (each round streams the head's 2C x 2d weight columns again), so longer
// slices and more anchors keep the unfused path.
bool block_fused_supported(const Geometry& g) {
  if (g.d != 32 && g.d != 64) return false;
  return g.m_pad == 32 && (g.n + 31) / 32 <= 8;
}

template <int D, int MP, int NW, int ROUNDS, int MINW>
static hipError_t go_block(const Geometry& g, const void* X, const void* Wqv, const void* bqv,
                           const void* U, void* H, hipStream_t s) {
  if (g.slices > 0x7fffffffLL) return hipErrorInvalidValue;
  block_fused_bf16<D, MP, NW, ROUNDS, MINW><<<dim3((unsigned)g.slices), dim3(NW * kWave), 0, s>>>(
      (const __bf16*)X, (const __bf16*)Wqv, (const __bf16*)bqv, (const __bf16*)U, (__bf16*)H,
      g.B, g.h, g.n, g.m, g.c2);
  return hipGetLastError();
}

template <int D>
static hipError_t dispatch_block(const Geometry& g, const void* X, const void* Wqv,
                                 const void* bqv, const void* U, void* H, hipStream_t s) {
  // 128 registers: two workgroups of eight waves per CU
  return go_block<D, 1, 8, 1, 4>(g, X, Wqv, bqv, U, H, s);
}

hipError_t launch_block_fused_bf16(const Geometry& g, const void* X, const void* Wqv,
                                   const void* bqv, const void* U, void* H, hipStream_t s) {
  if (!block_fused_supported(g)) return hipErrorInvalidValue;
  if (g.d == 64) return dispatch_block<64>(g, X, Wqv, bqv, U, H, s);
  return dispatch_block<32>(g, X, Wqv, bqv, U, H, s);
}

}  // namespace aa
