// backward_fused_bf16.hip -- gradients of anchor attention for short sequences: one
// workgroup per (batch, head) slice computes dQ and dV of the slice and its share of dU.
//
// With c = 1/sqrt(d) and G = dL/dH (chain rule through the forward steps of Eq. (11) in
// the Eq. (12) order, Pith verdict page; the anchors are learnable weights, AnchorFormer
// abstract):
//   P = A^T V, PG = A^T G, Delta = column sums of A,
//   W = P / Delta, dP = PG / Delta, dDelta = -rowsum(PG * W) / Delta   (0 where Delta = 0)
//   dA = G W^T + V dP^T + 1 dDelta^T,  dS = A * (dA - rowsum(A * dA))
//   dQ = c dS U,  dV = A dP,  dU = c * sum over the batch of dS^T Q.
// Phase 1 (rounds of one 32-token pair per wave): A from the logits as in the forward;
//   rows of A, V and G to LDS; each wave accumulates its (16-anchor, 16-dim) tiles of P
//   (with Delta) and of PG through transposing LDS reads.
// Phase 2: W, dP and dDelta from the tiles, stored in LDS as MFMA operands.
// Phase 3 (rounds again): per 16-token tile, dA^T = dDelta + W G^T + dP V^T on the MFMA
//   (lanes = tokens), dS in registers, dQ^T = c U^T dS^T and dV^T = dP^T A^T written
//   out; rows of dS and Q go to LDS and each wave accumulates its tiles of dS^T Q.
// The slice's dS^T Q tiles go to a workspace; a second kernel sums them over the batch
// in a fixed order (deterministic, no atomics).
// Rows of Q, V and G stay in registers between the phases when every wave has at most
// two pairs (KEEP); otherwise phase 3 reads them again (one round ahead, like phase 1)
// and recomputes A.
#include <algorithm>

#include "device_common.h"
#include "kernels.h"
#include "tile_ops.h"

namespace aa {

template <int D, int MP, int NW>
struct BwdLds {
  static constexpr int AT = 2 * MP, KS = D / 32, DT = D / 16;
  static constexpr int AS = tr_stride<32 * MP>(), VS = tr_stride<D>();
  u32x4 u[AT][KS][kWave];       // U: left operands of the logits (lane (c,g), chunk kk:
  u32x4 wu[AT][KS][kWave];      //   anchor 16j + c, dims 32kk + 8g .. + 7); W and dP alike
  u32x4 dpu[AT][KS][kWave];
  u32x4 ut[DT][MP][kWave];      // U^T and dP^T: left operands of output-like products
  u32x4 dpw[DT][MP][kWave];
  __attribute__((aligned(16))) __bf16 a[NW * 32 * AS];   // rows of A (phase 1), dS (phase 3)
  __attribute__((aligned(16))) __bf16 v[NW * 32 * VS];   // rows of V (phase 1), Q (phase 3)
  __attribute__((aligned(16))) __bf16 g[NW * 32 * VS];   // rows of G (phase 1)
  __attribute__((aligned(16))) float dl[AT][16];         // Delta
  __attribute__((aligned(16))) float dd[AT][16];         // dDelta
  float dot[AT][DT][16];                                 // rowsum(PG * W) per dim tile
};

// (anchor a, dim k) -> element of a logits-layout operand block [AT][KS][lane][8].
__device__ __forceinline__ int logits_pos(int a, int k, int KS) {
  return ((((a >> 4) * KS + (k >> 5)) * kWave) + 16 * ((k >> 3) & 3) + (a & 15)) * 8 + (k & 7);
}
// (anchor a, dim k) -> element of an output-layout operand block [DT][MP][lane][8]: lane
// (c,g) of [dt2][jj] holds dim out_dim_c(dt2, c) and anchors 32jj + 4g + s (s < 4) and
// 32jj + 16 + 4g + s - 4 (s >= 4).
__device__ __forceinline__ int output_pos(int a, int k, int MP) {
  const int q = k & 31, dt2 = 2 * (k >> 5) + ((q & 7) >> 2), cc = 4 * (q >> 3) + (q & 3);
  return ((((dt2 * MP + (a >> 5)) * kWave) + 16 * ((a >> 2) & 3) + cc) * 8 +
          4 * ((a >> 4) & 1) + (a & 3));
}

// Rows of one 16-token tile in operand layout (lane (c,g): dims 32kk + 8g .. + 7).
template <int D>
struct TileRows {
  u32x4 q[D / 32], v[D / 32], g[D / 32];
};

// Start of the slice's rows in Q, V, G and their token strides.
struct SliceRows {
  size_t q, v, g;
  long long qs, vs, gs;
};

template <int D>
__device__ __forceinline__ void load_tile_rows(const __bf16* Q, const __bf16* V, const __bf16* G,
                                               const SliceRows& sr, int row, int n, int g,
                                               TileRows<D>& t) {
  load_rows_c<D, D>(Q, sr.q, sr.qs, row, n, g, 0, t.q);
  load_rows_c<D, D>(V, sr.v, sr.vs, row, n, g, 0, t.v);
  load_rows_c<D, D>(G, sr.g, sr.gs, row, n, g, 0, t.g);
}

// Row-major copies of a tile's rows ([token][anchor] for A or dS, [token][dim] for the
// others) at LDS row 32w + 16tt + c.
template <int MP, int AS>
__device__ __forceinline__ void put_anchor_row(__bf16* blk, int row, int g, const bf16x8* x) {
  __bf16* p = blk + row * AS + 4 * g;
#pragma unroll
  for (int jj = 0; jj < MP; ++jj) {
    const u32x4 v = as_u32x4(x[jj]);
    *(u32x2*)(p + 32 * jj) = u32x2{v[0], v[1]};
    *(u32x2*)(p + 32 * jj + 16) = u32x2{v[2], v[3]};
  }
}
template <int D, int VS>
__device__ __forceinline__ void put_dim_row(__bf16* blk, int row, int g, const u32x4* x) {
  __bf16* p = blk + row * VS + 8 * g;
#pragma unroll
  for (int kk = 0; kk < D / 32; ++kk) *(u32x4*)(p + 32 * kk) = x[kk];
}

// ROUNDS > 0: compile-time number of rounds with the rows kept in registers (KEEP);
// ROUNDS == 0: rounds from n, rows read again in phase 3.
template <int D, int MP, int NW, int ROUNDS>
__global__ __launch_bounds__(NW * kWave, 1)
void bwd_fused(const __bf16* __restrict__ Q, const __bf16* __restrict__ U,
               const __bf16* __restrict__ V, const __bf16* __restrict__ G,
               __bf16* __restrict__ dQ, __bf16* __restrict__ dV, float* __restrict__ partU,
               BwdViews bv, int h, int n, int m, float c2, float cs) {
  using L_t = BwdLds<D, MP, NW>;
  constexpr int AT = 2 * MP, KS = D / 32, DT = D / 16;
  constexpr int AS = L_t::AS, VS = L_t::VS;
  constexpr int TILES = AT * DT, TPW = TILES / NW;
  constexpr bool KEEP = ROUNDS > 0;
  constexpr int RK = KEEP ? ROUNDS : 1;
  static_assert(TILES % NW == 0 && TPW >= 1, "tiles split evenly over the waves");
  __shared__ L_t L;
  const int slice = blockIdx.x;
  const int head = slice % h;
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int c = lane & 15, g = lane >> 4;
  const SliceRows sr{view_base(bv.q, slice, h), view_base(bv.v, slice, h),
                     view_base(bv.g, slice, h), bv.q.st, bv.v.st, bv.g.st};
  const size_t dqb = view_base(bv.dq, slice, h), dvb = view_base(bv.dv, slice, h);
  const int npairs = (n + 31) >> 5;
  const int rounds = KEEP ? ROUNDS : (npairs + NW - 1) / NW;

  // Rows: all rounds up front (KEEP), else the first round (the next one is fetched
  // while the current one is processed).
  TileRows<D> rows[RK][2];
#pragma unroll
  for (int r = 0; r < RK; ++r)
#pragma unroll
    for (int tt = 0; tt < 2; ++tt)
      load_tile_rows<D>(Q, V, G, sr, 32 * (r * NW + w) + 16 * tt + c, n, g, rows[r][tt]);

  // U twice: as the logits' left operands and transposed for dQ; every load is issued
  // before the first LDS write.
  const __bf16* Uh = U + (size_t)head * m * D;
  Stage<AT * KS * kWave, NW * kWave> ust;
  stage_load(ust, [&](int idx) {
    const int j = idx / (KS * kWave), kk = (idx / kWave) % KS, l = idx & 63;
    const int a = 16 * j + (l & 15);
    u32x4 v = {0u, 0u, 0u, 0u};
    if (a < m) v = *(const u32x4*)(Uh + (size_t)a * D + 8 * (l >> 4) + 32 * kk);
    return v;
  });
  // rows of U (padded anchors zero) as chunks of 8 dims: chunk i = anchor i / (D/8)
  constexpr int UTC = 16 * AT * D / 8;
  Stage<UTC, NW * kWave> utst;
  stage_load(utst, [&](int idx) {
    const int a = idx / (D / 8), k = 8 * (idx - a * (D / 8));
    u32x4 v = {0u, 0u, 0u, 0u};
    if (a < m) v = *(const u32x4*)(Uh + (size_t)a * D + k);
    return v;
  });
  stage_store(ust, &L.u[0][0][0]);
  {
    __bf16* ut = (__bf16*)&L.ut[0][0][0];
#pragma unroll
    for (int i = 0; i < Stage<UTC, NW * kWave>::kPer; ++i) {
      const int idx = (int)threadIdx.x + i * NW * kWave;
      if (UTC % (NW * kWave) == 0 || idx < UTC) {
        const int a = idx / (D / 8), k = 8 * (idx - a * (D / 8));
        const bf16x8 v = as_bf16x8(utst.r[i]);
#pragma unroll
        for (int e = 0; e < 8; ++e) ut[output_pos(a, k + e, MP)] = v[e];
      }
    }
  }
  const bf16x8 ones = splat_bf16(1.f);
  f32x4 mask[2];
  pad_mask<MP>(g, m, mask);
  __syncthreads();

  // ---- phase 1: P = A^T V with Delta, PG = A^T G ----------------------------------------
  f32x4 pacc[TPW], gacc[TPW], uacc[TPW], dacc[TPW], dummy[TPW];
#pragma unroll
  for (int k = 0; k < TPW; ++k) { pacc[k] = zero4(); gacc[k] = zero4(); uacc[k] = zero4(); dacc[k] = zero4(); }
  bf16x8 keep[RK][2][MP];

#pragma unroll (KEEP ? RK : 1)
  for (int r = 0; r < rounds; ++r) {
    const int pairs_here = min(NW, npairs - r * NW);  // uniform over the workgroup
    if (pairs_here <= 0) break;
    const int p = r * NW + w;
    const int ri = KEEP ? r : 0;
    TileRows<D> nxt[KEEP ? 1 : 2];
    // the next round's rows, unconditionally (rows past the slice read its last row; a
    // pair past the end is never used): a load under a branch would make the wait for
    // this round's rows at the join a wait for everything
    constexpr bool more = !KEEP;
    if constexpr (more) {
#pragma unroll
      for (int tt = 0; tt < 2; ++tt) load_tile_rows<D>(Q, V, G, sr, 32 * (p + NW) + 16 * tt + c, n, g, nxt[tt]);
    }
    if (p < npairs) {
#pragma unroll
      for (int tt = 0; tt < 2; ++tt) {
        const int lrow = 32 * w + 16 * tt + c;
        bf16x8 ab[MP];
        tile_softmax<D, MP>(L.u, rows[ri][tt].q, lane, mask, 32 * p + 16 * tt + c < n, c2, ab);
        if constexpr (KEEP) {
#pragma unroll
          for (int jj = 0; jj < MP; ++jj) keep[ri][tt][jj] = ab[jj];
        }
        put_anchor_row<MP, AS>(L.a, lrow, g, ab);
        put_dim_row<D, VS>(L.v, lrow, g, rows[ri][tt].v);
        put_dim_row<D, VS>(L.g, lrow, g, rows[ri][tt].g);
      }
    }
    __syncthreads();
    accumulate_tiles<TPW, DT, AS, VS, true>(L.a, L.v, w * TPW, pairs_here, c, g, ones, pacc, dacc);
    accumulate_tiles<TPW, DT, AS, VS, false>(L.a, L.g, w * TPW, pairs_here, c, g, ones, gacc, dummy);
    __syncthreads();
    if constexpr (!KEEP) {
      rows[0][0] = nxt[0];
      rows[0][1] = nxt[1];
    }
  }

  // ---- phase 2: W, dP, dDelta as operands ------------------------------------------------
  // Tile t (anchor tile t / DT, dim tile t % DT) holds rows 16ja + 4g + r, dim 16dt + c;
  // Delta of an anchor tile comes from the wave that owns its dim tile 0.
#pragma unroll
  for (int k = 0; k < TPW; ++k) {
    const int t = w * TPW + k, ja = t / DT, dt = t - (t / DT) * DT;
    if (dt == 0 && c == 0) {
#pragma unroll
      for (int r = 0; r < 4; ++r) L.dl[ja][4 * g + r] = dacc[k / DT][r];
    }
  }
  __syncthreads();
  {
    __bf16* wu = (__bf16*)&L.wu[0][0][0];
    __bf16* dpu = (__bf16*)&L.dpu[0][0][0];
    __bf16* dpw = (__bf16*)&L.dpw[0][0][0];
#pragma unroll
    for (int k = 0; k < TPW; ++k) {
      const int t = w * TPW + k, ja = t / DT, dt = t - (t / DT) * DT;
      const int dim = 16 * dt + c;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int anchor = 16 * ja + 4 * g + r;
        const float delta = L.dl[ja][4 * g + r];
        const float rinv = (delta > 0.f) ? 1.f / delta : 0.f;
        const float wv = pacc[k][r] * rinv, dpv = gacc[k][r] * rinv;
        const float part = row16_sum(gacc[k][r] * wv);   // this tile's 16 dims
        if (c == 0) L.dot[ja][dt][4 * g + r] = part;
        wu[logits_pos(anchor, dim, KS)] = (__bf16)wv;
        dpu[logits_pos(anchor, dim, KS)] = (__bf16)dpv;
        dpw[output_pos(anchor, dim, MP)] = (__bf16)dpv;
      }
    }
  }
  __syncthreads();
  for (int e = threadIdx.x; e < 16 * AT; e += NW * kWave) {
    const int ja = e >> 4, i = e & 15;
    float s = 0.f;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) s += L.dot[ja][dt][i];
    const float delta = L.dl[ja][i];
    L.dd[ja][i] = (delta > 0.f) ? -s / delta : 0.f;
  }
  __syncthreads();

  // ---- phase 3: dQ, dV and the dS^T Q tiles ---------------------------------------------
  if constexpr (!KEEP) {
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) load_tile_rows<D>(Q, V, G, sr, 32 * w + 16 * tt + c, n, g, rows[0][tt]);
  }
#pragma unroll (KEEP ? RK : 1)
  for (int r = 0; r < rounds; ++r) {
    const int pairs_here = min(NW, npairs - r * NW);
    if (pairs_here <= 0) break;
    const int p = r * NW + w;
    const int ri = KEEP ? r : 0;
    TileRows<D> nxt[KEEP ? 1 : 2];
    // the next round's rows, unconditionally (rows past the slice read its last row; a
    // pair past the end is never used): a load under a branch would make the wait for
    // this round's rows at the join a wait for everything
    constexpr bool more = !KEEP;
    if constexpr (more) {
#pragma unroll
      for (int tt = 0; tt < 2; ++tt) load_tile_rows<D>(Q, V, G, sr, 32 * (p + NW) + 16 * tt + c, n, g, nxt[tt]);
    }
    if (p < npairs) {
#pragma unroll
      for (int tt = 0; tt < 2; ++tt) {
        const int row = 32 * p + 16 * tt + c;
        const int lrow = 32 * w + 16 * tt + c;
        const TileRows<D>& tr = rows[ri][tt];
        bf16x8 ab[MP];
        if constexpr (KEEP) {
#pragma unroll
          for (int jj = 0; jj < MP; ++jj) ab[jj] = keep[ri][tt][jj];
        } else {
          tile_softmax<D, MP>(L.u, tr.q, lane, mask, row < n, c2, ab);
        }
        // A in accumulator layout: anchor tile j, rows 4g + r' of token c.
        f32x4 av[AT], da[AT];
        float rs = 0.f;
#pragma unroll
        for (int j = 0; j < AT; ++j) {
#pragma unroll
          for (int q = 0; q < 4; ++q) av[j][q] = (float)ab[j >> 1][4 * (j & 1) + q];
          f32x4 acc = *(const f32x4*)&L.dd[j][4 * g];
#pragma unroll
          for (int kk = 0; kk < KS; ++kk) {
            acc = mfma_bf16(as_bf16x8(L.wu[j][kk][lane]), as_bf16x8(tr.g[kk]), acc);
            acc = mfma_bf16(as_bf16x8(L.dpu[j][kk][lane]), as_bf16x8(tr.v[kk]), acc);
          }
          da[j] = acc;
#pragma unroll
          for (int q = 0; q < 4; ++q) rs = fmaf(av[j][q], acc[q], rs);
        }
        rs = xor32_sum(xor16_sum(rs));
        bf16x8 dsb[MP];
#pragma unroll
        for (int jj = 0; jj < MP; ++jj)
          dsb[jj] = pack_bf16(av[2 * jj] * (da[2 * jj] - rs), av[2 * jj + 1] * (da[2 * jj + 1] - rs));
        f32x4 hq[DT], hv[DT];
#pragma unroll
        for (int dt2 = 0; dt2 < DT; ++dt2) {
          f32x4 aq = zero4(), avv = zero4();
#pragma unroll
          for (int jj = 0; jj < MP; ++jj) {
            aq = mfma_bf16(as_bf16x8(L.ut[dt2][jj][lane]), dsb[jj], aq);
            avv = mfma_bf16(as_bf16x8(L.dpw[dt2][jj][lane]), ab[jj], avv);
          }
          hq[dt2] = aq * cs;
          hv[dt2] = avv;
        }
        // Lane group g holds dims 32hh + 8g .. + 7 in tiles 2hh and 2hh + 1.  With d = 64
        // lanes c and c + 8 trade one 16-byte chunk (DPP row rotate by 8) so that each store
        // instruction writes whole 128-byte rows: tokens 0-7 of the tile, then 8-15.  Half
        // rows written by separate non-temporal stores cost extra HBM writes (measured:
        // 30.1 MB instead of 22.4 MB per step at B = 64, h = 6, n = 196, m = 30).
        if constexpr (DT == 4) {
          const bool lo = c < 8;
          const int ta = row - c + (c & 7), tb = ta + 8;
          const int o2 = (lo ? 0 : 32) + 8 * g;
          auto put = [&](const f32x4* hx, __bf16* X, size_t xb, const View& xw) {
            const u32x4 x0 = as_u32x4(pack_bf16(hx[0], hx[1]));
            const u32x4 x1 = as_u32x4(pack_bf16(hx[2], hx[3]));
            const u32x4 y = lo ? x1 : x0;
            u32x4 sw;
#pragma unroll
            for (int i = 0; i < 4; ++i) sw[i] = __builtin_amdgcn_update_dpp(0u, y[i], 0x128, 0xF, 0xF, false);
            if (ta < n) __builtin_nontemporal_store(lo ? x0 : sw, (u32x4*)(X + xb + view_row(xw, ta) + o2));
            if (tb < n) __builtin_nontemporal_store(lo ? sw : x1, (u32x4*)(X + xb + view_row(xw, tb) + o2));
          };
          put(hq, dQ, dqb, bv.dq);
          put(hv, dV, dvb, bv.dv);
        } else if (row < n) {
          const size_t oq = dqb + view_row(bv.dq, row) + 8 * g, ov = dvb + view_row(bv.dv, row) + 8 * g;
#pragma unroll
          for (int hh = 0; hh < DT / 2; ++hh) {
            __builtin_nontemporal_store(as_u32x4(pack_bf16(hq[2 * hh], hq[2 * hh + 1])), (u32x4*)(dQ + oq + 32 * hh));
            __builtin_nontemporal_store(as_u32x4(pack_bf16(hv[2 * hh], hv[2 * hh + 1])), (u32x4*)(dV + ov + 32 * hh));
          }
        }
        put_anchor_row<MP, AS>(L.a, lrow, g, dsb);
        put_dim_row<D, VS>(L.v, lrow, g, tr.q);
      }
    }
    __syncthreads();
    accumulate_tiles<TPW, DT, AS, VS, false>(L.a, L.v, w * TPW, pairs_here, c, g, ones, uacc, dummy);
    __syncthreads();
    if constexpr (!KEEP) {
      rows[0][0] = nxt[0];
      rows[0][1] = nxt[1];
    }
  }

  // dS^T Q tiles of this slice: [slice][ja][dt][r][lane].
#pragma unroll
  for (int k = 0; k < TPW; ++k) {
    const int t = w * TPW + k, ja = t / DT, dt = t - (t / DT) * DT;
    float* dst = partU + (((size_t)slice * AT + ja) * DT + dt) * 256;
#pragma unroll
    for (int q = 0; q < 4; ++q) dst[q * 64 + lane] = uacc[k][q];
  }
}

// Plans: n <= 1024 (32 pairs), m <= 64, d = 32 or 64; the rows stay in registers when
// every wave has at most two pairs.
bool bwd_fused_supported(const Geometry& g) {
  return (g.d == 32 || g.d == 64) && g.m_pad <= 64 && (g.n + 31) / 32 <= 32;
}

// Waves per workgroup: four for m <= 32; two for m <= 64, where four waves would need
// more than half of the LDS and leave one workgroup per CU (measured: 87 instead of
// 107 us at B = 32, h = 12, n = 576, m = 64, d = 64).
template <int D, int MP>
constexpr int bwd_waves() { return MP == 2 ? 2 : 4; }

template <int D, int MP, int ROUNDS>
static hipError_t go_fused(const Geometry& g, const BwdViews& bv, const void* Q, const void* U,
                           const void* V, const void* G, void* dQ, void* dV, float* partU,
                           hipStream_t s) {
  constexpr int NW = bwd_waves<D, MP>();
  if (g.slices > 0x7fffffffLL) return hipErrorInvalidValue;
  bwd_fused<D, MP, NW, ROUNDS><<<dim3((unsigned)g.slices), dim3(NW * kWave), 0, s>>>(
      (const __bf16*)Q, (const __bf16*)U, (const __bf16*)V, (const __bf16*)G, (__bf16*)dQ,
      (__bf16*)dV, partU, bv, g.h, g.n, g.m, g.c2, 1.0f / sqrtf((float)D));
  return hipGetLastError();
}

template <int D, int MP>
static hipError_t fused_rounds(const Geometry& g, const BwdViews& bv, const void* Q, const void* U,
                               const void* V, const void* G, void* dQ, void* dV, float* partU,
                               hipStream_t s) {
  constexpr int NW = bwd_waves<D, MP>();
  const int rounds = ((g.n + 31) / 32 + NW - 1) / NW;
  if (rounds <= 1) return go_fused<D, MP, 1>(g, bv, Q, U, V, G, dQ, dV, partU, s);
  if (rounds == 2) return go_fused<D, MP, 2>(g, bv, Q, U, V, G, dQ, dV, partU, s);
  return go_fused<D, MP, 0>(g, bv, Q, U, V, G, dQ, dV, partU, s);
}

hipError_t launch_backward_fused_bf16(const Geometry& g, const BwdViews& bv, const void* Q,
                                      const void* U, const void* V, const void* G, void* dQ,
                                      void* dU, void* dV, float* partU, hipStream_t s) {
  if (!bwd_fused_supported(g)) return hipErrorInvalidValue;
  hipError_t e;
  if (g.d == 64)
    e = (g.m_pad == 32) ? fused_rounds<64, 1>(g, bv, Q, U, V, G, dQ, dV, partU, s)
                        : fused_rounds<64, 2>(g, bv, Q, U, V, G, dQ, dV, partU, s);
  else
    e = (g.m_pad == 32) ? fused_rounds<32, 1>(g, bv, Q, U, V, G, dQ, dV, partU, s)
                        : fused_rounds<32, 2>(g, bv, Q, U, V, G, dQ, dV, partU, s);
  if (e != hipSuccess) return e;
  return launch_du_reduce_bf16(g, partU, 1, dU, s);
}

}  // namespace aa
