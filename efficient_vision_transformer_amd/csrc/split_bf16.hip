// split_bf16.hip -- anchor attention for long token sequences, bf16 in / bf16 out.
//
// Per (batch, head) slice (AnchorFormer, Pith verdict page: referee summary, Eq. (11)
// evaluated in the Eq. (12) order; desk-editor letter: A row-stochastic, Delta its
// column sums):
//   A = rowsoftmax(Q U^T / sqrt(d)),  Delta = 1^T A,  W = Delta^-1 (A^T V),  H = A W.
// The tokens of a slice are split into chunks so that the whole chip is busy:
//   pass 1  (one workgroup per chunk): logits, softmax, column sums and A^T V of the
//           chunk -> fp32 partials in the workspace;
//   finalize (one workgroup per 16 anchors of a slice): sums the partials over chunks
//           in chunk order (deterministic), W = P / Delta (0 where Delta == 0), written
//           as bf16 MFMA operands;
//   pass 2  (one workgroup per chunk): recomputes A from Q and writes H = A W.
// All products run on v_mfma_f32_16x16x32_bf16 with fp32 accumulation.
#include <type_traits>

#include "device_common.h"
#include "kernels.h"
#include "pass2_layout.h"
#include "tile_ops.h"

namespace aa {

// ---------------------------------------------------------------------------------------
// Pass 1 for more than 128 anchors (AT = 12 or 16 tiles on four waves, 24 or 32 tiles on
// eight).  The NW waves split the anchors into groups of J = AT / NW tiles.  Blocks of
// 32 NW tokens are staged through LDS:
// every wave loads one 32-token pair of Q (kept in its MFMA operand layout) and of V (kept
// as rows); the next block's rows are in flight while the current block is computed.
// For each pair, every wave forms S^T = U_group Q^T (lanes = tokens, registers = its
// anchors), reduces the maximum and then the sum over its anchors in registers plus two
// permlane swaps, and the NW groups' partial maxima and sums of every token are
// combined through LDS.  The wave writes the pair's rows of A for its anchors to its own
// LDS block and accumulates its (16-anchor, 16-dim) tiles of A^T V and Delta, reading
// both operands (tokens on the contraction axis) with the transposing LDS read.
// Partials leave in accumulator layout with dim tile dt holding dims 16dt .. 16dt + 15.
// DUAL (the backward): G ([token][dim], view gw) is staged beside V and A^T G accumulated
// into partG from the same A (no Delta), so Q is read and A formed once for both.
template <int D, int AT, int NW = 4, bool DUAL = false>
__global__ __launch_bounds__(NW * kWave, DUAL ? 1 : 2)
void pass1a_bf16(const __bf16* __restrict__ Q, const __bf16* __restrict__ U,
                 const __bf16* __restrict__ V, float* __restrict__ part,
                 float* __restrict__ dpart, View qw, View xw, int h, int n, int m, int chunks,
                 int chunk_len, float c2, float* __restrict__ lse,
                 const __bf16* __restrict__ G = nullptr, View gw = View{0, 0, 0},
                 float* __restrict__ partG = nullptr) {
  constexpr int J = AT / NW, KS = D / 32, DT = D / 16;
  constexpr int AS = 80;                     // A row stride (16J + padding, bank-spread)
  constexpr int VS = tr_stride<D>();
  static_assert(AT % NW == 0 && J >= 2 && J <= 4 && NW % 4 == 0,
                "four or eight anchor groups of 2 to 4 tiles");
  const int slice = blockIdx.x / chunks;
  const int chunk = blockIdx.x - slice * chunks;
  const int head = slice % h;
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // anchor group
  const int c = lane & 15, g = lane >> 4;
  const size_t qb = view_base(qw, slice, h), xb = view_base(xw, slice, h);
  const size_t gb = DUAL ? view_base(gw, slice, h) : 0;
  const int t_begin = chunk * chunk_len;
  const int t_end = min(n, t_begin + chunk_len);

  __shared__ __attribute__((aligned(16))) __bf16 g_lds[DUAL ? NW * 32 * VS : 8];   // G rows
  __shared__ u32x4 q_lds[NW][2][KS][kWave];
  __shared__ __attribute__((aligned(16))) __bf16 v_lds[NW * 32 * VS];   // V rows, this block
  __shared__ __attribute__((aligned(16))) __bf16 a_lds[NW][32 * AS];    // A rows, per wave
  __shared__ __attribute__((aligned(16))) float st_max[32 * NW][NW];    // per token, per group
  __shared__ __attribute__((aligned(16))) float st_sum[32 * NW][NW];

  auto load_pair = [&](int blk, u32x4 (*qv)[KS], u32x4 (*vv)[KS], u32x4 (*gv)[KS]) {
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) {
      load_rows<D>(Q, qb, qw.st, blk + 32 * w + 16 * tt + c, n, g, qv[tt]);
      load_rows<D>(V, xb, xw.st, blk + 32 * w + 16 * tt + c, n, g, vv[tt]);
      if constexpr (DUAL) load_rows<D>(G, gb, gw.st, blk + 32 * w + 16 * tt + c, n, g, gv[tt]);
    }
  };
  u32x4 qv[2][KS], vv[2][KS], gv[DUAL ? 2 : 1][KS];
  load_pair(t_begin, qv, vv, gv);

  // This group's anchors as left operands of S^T = U Q^T: lane (c,g) of tile jl holds
  // anchor 16(wJ + jl) + c (zero rows past m).  mask[jl]: initial accumulators, -inf on
  // padded anchors.
  bf16x8 uop[J][KS];
  f32x4 mask[J];
  const __bf16* Uh = U + (size_t)head * m * D;
#pragma unroll
  for (int jl = 0; jl < J; ++jl) {
    const int a = 16 * (w * J + jl) + c;
#pragma unroll
    for (int kk = 0; kk < KS; ++kk) {
      u32x4 v = {0u, 0u, 0u, 0u};
      if (a < m) v = *(const u32x4*)(Uh + (size_t)a * D + 8 * KS * g + 8 * kk);
      uop[jl][kk] = as_bf16x8(v);
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) mask[jl][r] = (16 * (w * J + jl) + 4 * g + r < m) ? 0.f : -INFINITY;
  }
  const bf16x8 ones = splat_bf16(1.f);
  f32x4 pacc[J][DT], dacc[J], gacc[DUAL ? J : 1][DT];
#pragma unroll
  for (int jl = 0; jl < J; ++jl) {
    dacc[jl] = zero4();
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) pacc[jl][dt] = zero4();
  }
#pragma unroll
  for (int jl = 0; jl < (DUAL ? J : 1); ++jl)
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) gacc[jl][dt] = zero4();

  for (int blk = t_begin; blk < t_end; blk += 32 * NW) {
    {  // stage pair w of this block, then request the next block's rows
#pragma unroll
      for (int tt = 0; tt < 2; ++tt) {
#pragma unroll
        for (int kk = 0; kk < KS; ++kk) q_lds[w][tt][kk][lane] = qv[tt][kk];
        __bf16* vrow = v_lds + (32 * w + 16 * tt + c) * VS + 8 * KS * g;
#pragma unroll
        for (int kk = 0; kk < KS; ++kk) *(u32x4*)(vrow + 8 * kk) = vv[tt][kk];
        if constexpr (DUAL) {
          __bf16* grow = g_lds + (32 * w + 16 * tt + c) * VS + 8 * KS * g;
#pragma unroll
          for (int kk = 0; kk < KS; ++kk) *(u32x4*)(grow + 8 * kk) = gv[tt][kk];
        }
      }
      if (blk + 32 * NW < t_end) load_pair(blk + 32 * NW, qv, vv, gv);
    }
    __syncthreads();

    for (int ps = 0; ps < NW; ++ps) {
      if (blk + 32 * ps >= t_end) break;  // uniform over the workgroup
      // a1: s[tt][jl] lane (c,g): token c of tile tt, anchors 16(wJ + jl) + 4g + r.
      f32x4 s[2][J];
#pragma unroll
      for (int tt = 0; tt < 2; ++tt)
#pragma unroll
        for (int jl = 0; jl < J; ++jl) {
          f32x4 acc = mask[jl];
#pragma unroll
          for (int kk = 0; kk < KS; ++kk) acc = mfma_bf16(uop[jl][kk], as_bf16x8(q_lds[ps][tt][kk][lane]), acc);
          s[tt][jl] = acc;
        }
      // a2: this group's maximum per token, combined over the groups through LDS.
#pragma unroll
      for (int tt = 0; tt < 2; ++tt) {
        float mx = s[tt][0][0];
#pragma unroll
        for (int jl = 0; jl < J; ++jl)
#pragma unroll
          for (int r = 0; r < 4; ++r) mx = fmaxf(mx, s[tt][jl][r]);
        mx = xor32_max(xor16_max(mx));
        if (g == 0) st_max[32 * ps + 16 * tt + c][w] = mx;
      }
      __syncthreads();
      float zp[2], mneg2[2];
#pragma unroll
      for (int tt = 0; tt < 2; ++tt) {
        const float* mrow = &st_max[32 * ps + 16 * tt + c][0];
        f32x4 mg = *(const f32x4*)mrow;
        float M = fmaxf(fmaxf(mg[0], mg[1]), fmaxf(mg[2], mg[3]));
#pragma unroll
        for (int q4 = 4; q4 < NW; q4 += 4) {
          mg = *(const f32x4*)(mrow + q4);
          M = fmaxf(M, fmaxf(fmaxf(mg[0], mg[1]), fmaxf(mg[2], mg[3])));
        }
        const float mneg = -M * c2;
        mneg2[tt] = mneg;
        f32x4 zt = zero4();
#pragma unroll
        for (int jl = 0; jl < J; ++jl) {
#pragma unroll
          for (int r = 0; r < 4; ++r) s[tt][jl][r] = exp2_fast(fmaf(s[tt][jl][r], c2, mneg));
          zt += s[tt][jl];
        }
        zp[tt] = xor32_sum(xor16_sum((zt[0] + zt[1]) + (zt[2] + zt[3])));
        if (g == 0) st_sum[32 * ps + 16 * tt + c][w] = zp[tt];
      }
      __syncthreads();
      // a3: normalised A rows of this group's anchors -> this wave's LDS block.
#pragma unroll
      for (int tt = 0; tt < 2; ++tt) {
        const int tok = 32 * ps + 16 * tt + c;
        f32x4 zg = *(const f32x4*)&st_sum[tok][0];
        float Z = (zg[0] + zg[1]) + (zg[2] + zg[3]);
#pragma unroll
        for (int q4 = 4; q4 < NW; q4 += 4) {   // groups summed in a fixed order
          zg = *(const f32x4*)&st_sum[tok][q4];
          Z += (zg[0] + zg[1]) + (zg[2] + zg[3]);
        }
        const float inv = (blk + tok < t_end) ? __builtin_amdgcn_rcpf(Z) : 0.f;   // Z >= 1
        // the token's log-sum-exp (base 2) for pass 2: every group holds it, group 0 writes
        if (lse && w == 0 && g == 0 && blk + tok < t_end)
          lse[(size_t)slice * n + blk + tok] = __builtin_amdgcn_logf(Z) - mneg2[tt];
        __bf16* arow = a_lds[w] + (16 * tt + c) * AS + 4 * g;
#pragma unroll
        for (int jl = 0; jl < J; ++jl) {
          *(u32x2*)(arow + 16 * jl) = pack4_bf16(s[tt][jl] * inv);
        }
      }
      // A^T V and Delta for this group's tiles over the pair's 32 tokens (the wave reads
      // back only its own A rows, so no barrier is needed here).
      bf16x8 xs[J], ys[DT];
#pragma unroll
      for (int jl = 0; jl < J; ++jl) xs[jl] = lds_operand_tr(a_lds[w], AS, 16 * jl, c, g);
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) ys[dt] = lds_operand_tr(v_lds + 32 * ps * VS, VS, 16 * dt, c, g);
#pragma unroll
      for (int jl = 0; jl < J; ++jl) {
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) pacc[jl][dt] = mfma_bf16(xs[jl], ys[dt], pacc[jl][dt]);
        dacc[jl] = mfma_bf16(xs[jl], ones, dacc[jl]);
      }
      if constexpr (DUAL) {
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) ys[dt] = lds_operand_tr(g_lds + 32 * ps * VS, VS, 16 * dt, c, g);
#pragma unroll
        for (int jl = 0; jl < J; ++jl)
#pragma unroll
          for (int dt = 0; dt < DT; ++dt) gacc[jl][dt] = mfma_bf16(xs[jl], ys[dt], gacc[jl][dt]);
      }
    }
    __syncthreads();   // q_lds / v_lds are restaged for the next block
  }

  // Partials: [slice][chunk][jt][dt][r][lane] holds P[16jt + 4g + r][16dt + c];
  // Delta as [slice][chunk][anchor].
  const size_t sc = (size_t)slice * chunks + chunk;
#pragma unroll
  for (int jl = 0; jl < J; ++jl) {
    const int jt = w * J + jl;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
      float* dst = part + ((sc * AT + jt) * DT + dt) * 256;
#pragma unroll
      for (int r = 0; r < 4; ++r) dst[r * 64 + lane] = pacc[jl][dt][r];
      if constexpr (DUAL) {
        float* dg = partG + ((sc * AT + jt) * DT + dt) * 256;
#pragma unroll
        for (int r = 0; r < 4; ++r) dg[r * 64 + lane] = gacc[jl][dt][r];
      }
    }
    if (c == 0) {
#pragma unroll
      for (int r = 0; r < 4; ++r) dpart[sc * (16 * AT) + 16 * jt + 4 * g + r] = dacc[jl][r];
    }
  }
}

// ---------------------------------------------------------------------------------------
// Pass 1 for up to 128 anchors.  The waves split the chunk's tokens in rounds of one
// 32-token pair per wave.  Phase A (per wave, its pair): S^T = U Q^T (lanes = tokens), the
// softmax over all anchors in registers plus two permlane swaps; the pair's rows of A
// ([token][anchor]) and V ([token][dim]) go to LDS as they are.  Phase B (after one
// barrier): each wave owns distinct (16-anchor, 16-dim) tiles of A^T V and of Delta and
// accumulates them over the round's pairs, reading both operands (tokens on the
// contraction axis) from the row copies with the transposing LDS read.  Partials leave in
// accumulator layout with dim tile dt holding dims 16dt .. 16dt + 15.
//
// DUAL (the backward): a second operand G ([token][dim], view gw) is accumulated beside V
// from the same A, A^T G into partG (no Delta); Q is read and A formed once for both.
// NYS (Nystrom attention, landmark pass): the anchors are the slice's landmark query rows,
// gathered from U (the queries, view uw) through the landmark indices lidx ([B][m]); Q
// holds the keys; and the weights are exp(c q.k - c M_a) with M_a landmark a's largest
// logit over this chunk's tokens (a first sweep over the chunk finds it, and it is written
// to cmax for the solve, which rescales the chunks to the overall maximum) instead of a
// softmax over anchors; phase B then accumulates F3 V and the row sums of F3 unnormalised.
template <int D, int MP, int NW, bool NYS = false, bool DUAL = false>
__global__ __launch_bounds__(NW * kWave, DUAL ? 1 : 2)
void pass1x_bf16(const __bf16* __restrict__ Q, const __bf16* __restrict__ U,
                 const __bf16* __restrict__ V, float* __restrict__ part,
                 float* __restrict__ dpart, View qw, View xw, int h, int n, int m, int chunks,
                 int chunk_len, float c2, float* __restrict__ cmax = nullptr,
                 const int* __restrict__ lidx = nullptr, View uw = View{0, 0, 0},
                 const __bf16* __restrict__ G = nullptr, View gw = View{0, 0, 0},
                 float* __restrict__ partG = nullptr) {
  static_assert(!(NYS && DUAL), "one mode at a time");
  constexpr int KS = D / 32, DT = D / 16, AT = 2 * MP;
  constexpr int TILES = AT * DT, TPW = (TILES + NW - 1) / NW;
  constexpr int NDA = (TPW + DT - 1) / DT;   // anchor tiles per wave needing a Delta
  static_assert(TILES % NW == 0, "tiles split evenly over the waves");
  const int slice = blockIdx.x / chunks;
  const int chunk = blockIdx.x - slice * chunks;
  const int head = slice % h;
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // uniform per wave
  const int c = lane & 15, g = lane >> 4;
  const size_t qb = view_base(qw, slice, h), xb = view_base(xw, slice, h);
  const size_t gb = DUAL ? view_base(gw, slice, h) : 0;
  const int t_begin = chunk * chunk_len;
  const int t_end = min(n, t_begin + chunk_len);
  const int npairs = (t_end - t_begin + 31) >> 5;

  constexpr int AS = tr_stride<32 * MP>(), VS = tr_stride<D>();
  __shared__ __attribute__((aligned(16))) __bf16 g_lds[DUAL ? NW * 32 * VS : 8];   // rows of G
  __shared__ u32x4 u_lds[AT][KS][kWave];
  __shared__ __attribute__((aligned(16))) __bf16 a_lds[NW * 32 * AS];   // rows of A, this round
  __shared__ __attribute__((aligned(16))) __bf16 v_lds[NW * 32 * VS];   // rows of V, this round

  // U first (L2-resident after the first workgroups), then this wave's first pair.
  constexpr int UCH = AT * KS * kWave;
  constexpr int UPT = (UCH + NW * kWave - 1) / (NW * kWave);
  u32x4 ust[UPT];
  // anchor a's row: U[head][a] (NYS: the query row of landmark token lidx[b][a])
  auto urow = [&](int a) -> const __bf16* {
    if constexpr (NYS) {
      const int tok = min(max(lidx[(size_t)(slice / h) * m + a], 0), n - 1);
      return U + view_base(uw, slice, h) + (size_t)((long long)tok * uw.st);
    } else {
      return U + ((size_t)head * m + a) * D;
    }
  };
#pragma unroll
  for (int i = 0; i < UPT; ++i) {
    const int idx = threadIdx.x + i * NW * kWave;
    if (idx < UCH) {
      const int j = idx / (KS * kWave), kk = (idx / kWave) % KS, l = idx & 63;
      const int a = min(16 * j + (l & 15), m - 1);   // padded anchors are masked
      ust[i] = *(const u32x4*)(urow(a) + 8 * KS * (l >> 4) + 8 * kk);
    }
  }
  // Rows of the wave's pair in each round; rows past the chunk read its last row (their
  // weights are zeroed), so every load is unconditional and the waits are exact counts.
  // Two register sets alternate between rounds: the next round's rows are requested at
  // the start of a round and first waited for at the start of the next one.
  auto load_pair = [&](int p, u32x4 (*qv)[KS], u32x4 (*vv)[KS], u32x4 (*gv)[KS]) {
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) {
      const int row = min(t_begin + 32 * p + 16 * tt + c, t_end - 1);
      load_rows<D>(Q, qb, qw.st, row, n, g, qv[tt]);
      load_rows<D>(V, xb, xw.st, row, n, g, vv[tt]);
      if constexpr (DUAL) load_rows<D>(G, gb, gw.st, row, n, g, gv[tt]);
    }
  };
  constexpr int GR = DUAL ? 2 : 1;
  u32x4 qa[2][KS], va[2][KS], qz[2][KS], vz[2][KS], ga[GR][KS], gz[GR][KS];
  load_pair(w, qa, va, ga);
#pragma unroll
  for (int i = 0; i < UPT; ++i) {
    const int idx = threadIdx.x + i * NW * kWave;
    if (idx < UCH) (&u_lds[0][0][0])[idx] = ust[i];
  }
  const bf16x8 ones = splat_bf16(1.f);
  f32x4 mask[2];
  pad_mask<MP>(g, m, mask);
  // NYS: mneg[a] = -c2 * (landmark a's largest logit over this chunk's tokens), 0 for
  // padding; the logits are formed exactly as tile_exp forms them below, so no exponent
  // there is positive
  __shared__ __attribute__((aligned(16))) float mneg[NYS ? 16 * AT : 4];
  __shared__ float cred[NYS ? NW : 1][NYS ? 16 * AT : 1];
  __syncthreads();
  if constexpr (NYS) {
    static_assert(16 * AT <= NW * kWave, "one landmark per thread");
    f32x4 mx[AT];
#pragma unroll
    for (int j = 0; j < AT; ++j) mx[j] = f32x4{-INFINITY, -INFINITY, -INFINITY, -INFINITY};
    for (int p = w; p < npairs; p += NW) {
#pragma unroll
      for (int tt = 0; tt < 2; ++tt) {
        const int row = t_begin + 32 * p + 16 * tt + c;
        u32x4 kr[KS];
        load_rows<D>(Q, qb, qw.st, min(row, t_end - 1), n, g, kr);
        const bool ok = row < t_end;
#pragma unroll
        for (int j = 0; j < AT; ++j) {
          f32x4 acc = (j >= AT - 2) ? mask[j - (AT - 2)] : zero4();
#pragma unroll
          for (int kk = 0; kk < KS; ++kk) acc = mfma_bf16(as_bf16x8(u_lds[j][kk][lane]), as_bf16x8(kr[kk]), acc);
#pragma unroll
          for (int r = 0; r < 4; ++r) mx[j][r] = ok ? fmaxf(mx[j][r], acc[r]) : mx[j][r];
        }
      }
    }
    // lane (c, g) holds landmarks 16j + 4g + r over its tokens: reduce over the lanes c,
    // then over the waves
#pragma unroll
    for (int j = 0; j < AT; ++j)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float v = row16_max(mx[j][r]);
        if (c == 0) cred[w][16 * j + 4 * g + r] = v;
      }
    __syncthreads();
    const int a = threadIdx.x;
    if (a < 16 * AT) {
      float M = cred[0][a];
#pragma unroll
      for (int ww = 1; ww < NW; ++ww) M = fmaxf(M, cred[ww][a]);
      mneg[a] = (a < m) ? -M * c2 : 0.f;
      cmax[((size_t)slice * chunks + chunk) * 16 * AT + a] = M;
    }
    __syncthreads();
  }

  // Wave w owns the contiguous tiles w*TPW .. w*TPW + TPW - 1 (tile t: anchor tile t / DT,
  // dim tile t % DT); the Delta of anchor tile ja is accumulated with its dim tile 0.
  f32x4 pacc[TPW], dacc[NDA], gacc[DUAL ? TPW : 1];
#pragma unroll
  for (int k = 0; k < TPW; ++k) pacc[k] = zero4();
#pragma unroll
  for (int k = 0; k < NDA; ++k) dacc[k] = zero4();
#pragma unroll
  for (int k = 0; k < (DUAL ? TPW : 1); ++k) gacc[k] = zero4();

  const int rounds = (npairs + NW - 1) / NW;
  auto round = [&](int r, u32x4 (*qc)[KS], u32x4 (*vc)[KS], u32x4 (*gc)[KS], u32x4 (*qn)[KS],
                   u32x4 (*vn)[KS], u32x4 (*gn)[KS]) {
    const int pairs_here = min(NW, npairs - r * NW);  // uniform over the workgroup
    const int p = r * NW + w;
    load_pair(p + NW, qn, vn, gn);
    // Phase A: rows 32w .. 32w + 31 of the round's LDS blocks hold this wave's pair.
    if (p < npairs) {
#pragma unroll
      for (int tt = 0; tt < 2; ++tt) {
        bf16x8 ab[MP];
        const bool token_ok = t_begin + 32 * p + 16 * tt + c < t_end;
        if constexpr (NYS)
          tile_exp<D, MP>(u_lds, qc[tt], lane, mask, token_ok, c2, mneg, g, ab);
        else
          tile_softmax<D, MP>(u_lds, qc[tt], lane, mask, token_ok, c2, ab);
        // ab[jj] holds anchors 32jj + 4g .. + 3 and 32jj + 16 + 4g .. + 3 of token c.
        __bf16* arow = a_lds + (32 * w + 16 * tt + c) * AS + 4 * g;
#pragma unroll
        for (int jj = 0; jj < MP; ++jj) {
          const u32x4 v = as_u32x4(ab[jj]);
          *(u32x2*)(arow + 32 * jj) = u32x2{v[0], v[1]};
          *(u32x2*)(arow + 32 * jj + 16) = u32x2{v[2], v[3]};
        }
        __bf16* vrow = v_lds + (32 * w + 16 * tt + c) * VS + 8 * KS * g;
#pragma unroll
        for (int kk = 0; kk < KS; ++kk) *(u32x4*)(vrow + 8 * kk) = vc[tt][kk];
        if constexpr (DUAL) {
          __bf16* grow = g_lds + (32 * w + 16 * tt + c) * VS + 8 * KS * g;
#pragma unroll
          for (int kk = 0; kk < KS; ++kk) *(u32x4*)(grow + 8 * kk) = gc[tt][kk];
        }
      }
    }
    __syncthreads();
    accumulate_tiles<TPW, DT, AS, VS>(a_lds, v_lds, w * TPW, pairs_here, c, g, ones, pacc, dacc);
    if constexpr (DUAL)
      accumulate_tiles<TPW, DT, AS, VS, false>(a_lds, g_lds, w * TPW, pairs_here, c, g, ones, gacc, dacc);
    __syncthreads();
  };
  for (int r = 0; r < rounds; r += 2) {
    round(r, qa, va, ga, qz, vz, gz);
    if (r + 1 < rounds) round(r + 1, qz, vz, gz, qa, va, ga);
  }

  // Partials: [slice][chunk][jt][dt][r][lane] holds P[16jt + 4g + r][16dt + c];
  // Delta as [slice][chunk][anchor] (from the dt == 0 tile of each anchor tile).
  const size_t sc = (size_t)slice * chunks + chunk;
#pragma unroll
  for (int k = 0; k < TPW; ++k) {
    const int t = w * TPW + k;
    const int ja = t / DT, dt = t - (t / DT) * DT;
    float* dst = part + ((sc * AT + ja) * DT + dt) * 256;
#pragma unroll
    for (int r = 0; r < 4; ++r) dst[r * 64 + lane] = pacc[k][r];
    if constexpr (DUAL) {
      float* dg = partG + ((sc * AT + ja) * DT + dt) * 256;
#pragma unroll
      for (int r = 0; r < 4; ++r) dg[r * 64 + lane] = gacc[k][r];
    }
    if (dt == 0 && c == 0) {
#pragma unroll
      for (int r = 0; r < 4; ++r) dpart[sc * (16 * AT) + 16 * ja + 4 * g + r] = dacc[k / DT][r];
    }
  }
}

// ---------------------------------------------------------------------------------------
// Finalize: W = Delta^-1 (sum over chunks of P), chunk order fixed.  One workgroup per
// (slice, 16-anchor tile).  Output layout = the left operand of pass 2's H^T = W^T A^T
// (w2_layout_index, per slice).  Column c of a partial's dim tile dt is dim 16dt + c.
template <int D>
__global__ __launch_bounds__(256)
void finalize_bf16(const float* __restrict__ part, const float* __restrict__ dpart,
                   __bf16* __restrict__ Wop, int chunks, int AT) {
  constexpr int DT = D / 16, U = 8;
  const int MP = AT / 2;
  const int slice = blockIdx.x / AT;
  const int jt = blockIdx.x - slice * AT;
  // Thread t owns accumulator slot (r, lane) of every dim tile: element dt*256 + t.
  const int r = (threadIdx.x >> 6) & 3, lane = threadIdx.x & 63;
  const int c = lane & 15, g = lane >> 4;
  const int anchor = 16 * jt + 4 * g + r;
  float p[DT], delta = 0.f;
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) p[dt] = 0.f;
  for (int ch0 = 0; ch0 < chunks; ch0 += U) {
    // all loads of U chunks first, then the adds in chunk order
    float pv[U][DT], dv[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int ch = min(ch0 + u, chunks - 1);
      const size_t sc = (size_t)slice * chunks + ch;
      dv[u] = dpart[sc * (16 * AT) + anchor];
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) pv[u][dt] = part[((sc * AT + jt) * DT + dt) * 256 + r * 64 + lane];
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (ch0 + u < chunks) {
        delta += dv[u];
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) p[dt] += pv[u][dt];
      }
    }
  }
  const float rinv = (delta > 0.f) ? 1.f / delta : 0.f;
  __bf16* Ws = Wop + (size_t)slice * DT * MP * 64 * 8;
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) {
    const float wv = (delta > 0.f) ? p[dt] * rinv : 0.f;
    Ws[w2_layout_index(MP, anchor, 16 * dt + c)] = (__bf16)wv;
  }
}

// ---------------------------------------------------------------------------------------
// Q tiles in flight per wave in pass 2 (1, 2 and 4 measured: one ahead is fastest at the
// dense and long shapes; more slots cost registers and occupancy)
constexpr int kPass2Ahead = 1;

// Waves per pass-2 workgroup: eight from 384 anchors up (U and W fill 96-128 KB of LDS,
// one workgroup per CU), else four.
template <int AT>
constexpr int pass2_waves() { return AT >= 24 ? 8 : kPass2Waves; }

// Tiles per pass-2 step: above 128 anchors (up to 256, d <= 64) two 16-token tiles share
// every U and W operand read from LDS.  At 128 anchors that was not faster (dense 56.7 us
// against 58.6 at three waves per SIMD and 57.3 when held to four); at d = 128 or beyond
// 256 anchors the second tile's registers would spill.
template <int D, int AT>
constexpr int pass2_tiles() { return (D <= 64 && AT > 8 && AT <= 16) ? 2 : 1; }

// Pass 2.  Each wave takes steps of TT consecutive 16-token tiles.  Logits are formed
// transposed, S^T = U Q^T (lanes = tokens, registers = anchors), so the softmax is an
// in-register reduction plus two permlane swaps and the normalised A is directly the right
// operand of H^T = W^T A^T.  U and W stay in LDS for the whole chunk; each operand read
// from it serves the step's TT tiles.  Each wave keeps kPass2Ahead of its steps' Q rows in
// flight (a register ring refilled as soon as a step's logits are formed); the first ones
// are requested before U and W are staged.
template <int D, int AT, bool LSE, int NW = pass2_waves<AT>(), int TT = pass2_tiles<D, AT>()>
__global__ __launch_bounds__(NW * kWave, 2)
void pass2_bf16(const __bf16* __restrict__ Q, const __bf16* __restrict__ U,
                const u32x4* __restrict__ Wop, __bf16* __restrict__ H, View qw, View ow, int h,
                int n, int m, int chunks, int chunk_len, float c2, int u_per_slice,
                const float* __restrict__ lse) {
  constexpr int KS = D / 32, DT = D / 16, MP = AT / 2;
  int slice, chunk;
  slice_chunk_of(blockIdx.x, chunks, slice, chunk);   // a slice's chunks on one XCD
  const int head = slice % h;
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // uniform per wave
  const int c = lane & 15, g = lane >> 4;
  const size_t qb = view_base(qw, slice, h), ob = view_base(ow, slice, h);
  const int t_begin = chunk * chunk_len;
  const int t_end = min(n, t_begin + chunk_len);

  // U and W (L2-resident after the first workgroups) are requested first, then the wave's
  // first Q tiles, so that writing U and W to LDS does not wait for Q.
  __shared__ u32x4 u_lds[AT][KS][kWave];
  __shared__ u32x4 w_lds[DT][MP][kWave];
  const __bf16* Uh = U + (size_t)(u_per_slice ? slice : head) * m * D;
  Stage<AT * KS * kWave, NW * kWave> ust;
  stage_load(ust, [&](int idx) {
    const int j = idx / (KS * kWave), kk = (idx / kWave) % KS, l = idx & 63;
    const int a = 16 * j + (l & 15);
    u32x4 v = {0u, 0u, 0u, 0u};
    if (a < m) v = *(const u32x4*)(Uh + (size_t)a * D + 8 * KS * (l >> 4) + 8 * kk);
    return v;
  });
  const u32x4* Ws = Wop + (size_t)slice * DT * MP * kWave;
  Stage<DT * MP * kWave, NW * kWave> wst;
  stage_load(wst, [&](int idx) { return Ws[idx]; });

  // Tiles past the chunk read the chunk's last row (clamped) and are not stored; loads
  // are unconditional so the wait before each step is an exact count.
  // LSE: the token's log-sum-exp from pass 1 comes with its Q row.
  const float* lse_s = LSE ? lse + (size_t)slice * n : nullptr;
  auto load_q = [&](int t0, u32x4 (*q)[KS], float* L) {
#pragma unroll
    for (int tt = 0; tt < TT; ++tt) {
      const int row = min(t0 + 16 * tt + c, t_end - 1);
      const size_t off = qb + view_row(qw, row) + 8 * KS * g;
#pragma unroll
      for (int kk = 0; kk < KS; ++kk)
        q[tt][kk] = __builtin_nontemporal_load((const u32x4*)(Q + off + 8 * kk));
      if constexpr (LSE) L[tt] = __builtin_nontemporal_load(lse_s + row);
    }
  };
  // Wave w takes the steps t_begin + 16 TT w + step*i; step i lives in ring slot i % PF.
  constexpr int PF = kPass2Ahead, step = 16 * TT * NW;
  u32x4 q[PF][TT][KS];
  float lq[PF][TT];
#pragma unroll
  for (int p = 0; p < PF; ++p) load_q(t_begin + 16 * TT * w + step * p, q[p], lq[p]);
  stage_store(ust, &u_lds[0][0][0]);
  stage_store(wst, &w_lds[0][0][0]);
  // above 256 anchors m is padded to a multiple of 128: up to eight padded tiles
  constexpr int NPAD = AT > 16 ? 8 : pad_tiles(AT);
  f32x4 mask[NPAD];
  pad_mask_tiles<AT, NPAD>(g, m, mask);
  __syncthreads();

  for (int tb = t_begin + 16 * TT * w; tb < t_end; tb += step * PF) {
#pragma unroll
  for (int p = 0; p < PF; ++p) {
    const int t0 = tb + step * p;
    if (t0 >= t_end) break;   // uniform per wave
    // a1 (transposed): s[tt][j] lane (c,g): token t0 + 16tt + c, anchors 16j + 4g + r.
    f32x4 s[TT][AT];
#pragma unroll
    for (int j = 0; j < AT; ++j) {
      // keeps the LDS operand loads of later tiles from being hoisted (register budget)
      if (AT >= 8 && j % 4 == 0) asm volatile("" ::: "memory");
      // padded anchors (>= m) lie in the last NPAD tiles and start from -inf
      const f32x4 a0 = (j >= AT - NPAD) ? mask[j - (AT - NPAD)] : zero4();
#pragma unroll
      for (int tt = 0; tt < TT; ++tt) s[tt][j] = a0;
#pragma unroll
      for (int kk = 0; kk < KS; ++kk) {
        const bf16x8 u = as_bf16x8(u_lds[j][kk][lane]);
#pragma unroll
        for (int tt = 0; tt < TT; ++tt) s[tt][j] = mfma_bf16(u, as_bf16x8(q[p][tt][kk]), s[tt][j]);
      }
    }
    bf16x8 abf[TT][MP];
    float nl[TT];
    if constexpr (LSE) {
#pragma unroll
      for (int tt = 0; tt < TT; ++tt) nl[tt] = -lq[p][tt];
    }
    // the slot is free: request the wave's step PF steps ahead into it
    load_q(t0 + step * PF, q[p], lq[p]);
#pragma unroll
    for (int tt = 0; tt < TT; ++tt) {
      if constexpr (LSE) {
        // a2 with the token's log-sum-exp L from pass 1: A = exp2(c2 s - L), already
        // normalised (padded anchors start from -inf and give 0)
#pragma unroll
        for (int j = 0; j < AT; ++j)
#pragma unroll
          for (int r = 0; r < 4; ++r) s[tt][j][r] = exp2_fast(fmaf(s[tt][j][r], c2, nl[tt]));
#pragma unroll
        for (int jj = 0; jj < MP; ++jj) abf[tt][jj] = pack_bf16(s[tt][2 * jj], s[tt][2 * jj + 1]);
      } else {
        // a2
        float mx = s[tt][0][0];
#pragma unroll
        for (int j = 0; j < AT; ++j)
#pragma unroll
          for (int r = 0; r < 4; ++r) mx = fmaxf(mx, s[tt][j][r]);
        mx = xor32_max(xor16_max(mx));
        const float mneg = -mx * c2;
        float z = 0.f;
#pragma unroll
        for (int j = 0; j < AT; ++j)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const float e = exp2_fast(fmaf(s[tt][j][r], c2, mneg));
            s[tt][j][r] = e;
            z += e;
          }
        z = xor32_sum(xor16_sum(z));
        const float inv = __builtin_amdgcn_rcpf(z);   // z >= 1 (the maximum adds 1)
#pragma unroll
        for (int jj = 0; jj < MP; ++jj)
          abf[tt][jj] = pack_bf16(s[tt][2 * jj] * inv, s[tt][2 * jj + 1] * inv);
      }
    }
    // a5: H^T = W^T A^T; lane (c,g) ends with token c, dims out_dim_c(dt2, 4g + r), i.e.
    // 32h + 8g .. + 7 in tiles 2h and 2h + 1.
    f32x4 hacc[TT][DT];
#pragma unroll
    for (int dt2 = 0; dt2 < DT; ++dt2) {
      if (AT >= 8) asm volatile("" ::: "memory");
#pragma unroll
      for (int tt = 0; tt < TT; ++tt) hacc[tt][dt2] = zero4();
#pragma unroll
      for (int jj = 0; jj < MP; ++jj) {
        const bf16x8 wv = as_bf16x8(w_lds[dt2][jj][lane]);
#pragma unroll
        for (int tt = 0; tt < TT; ++tt) hacc[tt][dt2] = mfma_bf16(wv, abf[tt][jj], hacc[tt][dt2]);
      }
    }
#pragma unroll
    for (int tt = 0; tt < TT; ++tt) {
      const int row = t0 + 16 * tt + c;
      if (row < t_end) {
        __bf16* dst = H + ob + view_row(ow, row) + 8 * g;
#pragma unroll
        for (int hh = 0; hh < DT / 2; ++hh)
          __builtin_nontemporal_store(as_u32x4(pack_bf16(hacc[tt][2 * hh], hacc[tt][2 * hh + 1])),
                                      (u32x4*)(dst + 32 * hh));
      }
    }
  }
  }
}

// ---------------------------------------------------------------------------------------
// Pass 1 above 128 anchors also writes each token's log-sum-exp in base 2 to lse
// ([slice][n], when lse is not null) for pass 2.
template <int D, int AT>
static void launch_pass1_t(const Geometry& geo, const SplitPlan& p, const void* Q, const void* U,
                           const void* X, float* part, float* dpart, float* lse,
                           hipStream_t stream) {
  const long long g1 = geo.slices * p.chunks1;
  if constexpr (AT <= 8) {
    pass1x_bf16<D, AT / 2, kPass1Waves><<<dim3((unsigned)g1), dim3(kPass1Waves * kWave), 0, stream>>>(
        (const __bf16*)Q, (const __bf16*)U, (const __bf16*)X, part, dpart, geo.vw.q, geo.vw.v,
        geo.h, geo.n, geo.m, p.chunks1, p.chunk_len1, geo.c2);
  } else if constexpr (AT >= 24) {
    pass1a_bf16<D, AT, 8><<<dim3((unsigned)g1), dim3(8 * kWave), 0, stream>>>(
        (const __bf16*)Q, (const __bf16*)U, (const __bf16*)X, part, dpart, geo.vw.q, geo.vw.v,
        geo.h, geo.n, geo.m, p.chunks1, p.chunk_len1, geo.c2, lse);
  } else {
    pass1a_bf16<D, AT><<<dim3((unsigned)g1), dim3(4 * kWave), 0, stream>>>(
        (const __bf16*)Q, (const __bf16*)U, (const __bf16*)X, part, dpart, geo.vw.q, geo.vw.v,
        geo.h, geo.n, geo.m, p.chunks1, p.chunk_len1, geo.c2, lse);
  }
}

template <int D, int AT>
static hipError_t launch_split_bf16_t(const Geometry& geo, const SplitPlan& p, const void* Q,
                                      const void* U, const void* V, void* H, void* ws,
                                      hipStream_t stream) {
  char* wsb = (char*)ws;
  float* part = (float*)wsb;
  float* dpart = (float*)(wsb + p.part_bytes);
  void* Wop = (void*)(wsb + p.part_bytes + p.dpart_bytes);
  // above 128 anchors pass 2 takes each token's log-sum-exp from pass 1 instead of forming
  // the softmax again (measured: the long workload 2 us faster, 128 anchors 1 us slower)
  constexpr bool kLse = AT > 8;
  float* lse = kLse ? (float*)(wsb + p.part_bytes + p.dpart_bytes + p.w_bytes) : nullptr;
  launch_pass1_t<D, AT>(geo, p, Q, U, V, part, dpart, lse, stream);
  finalize_bf16<D><<<dim3((unsigned)(geo.slices * AT)), dim3(256), 0, stream>>>(
      part, dpart, (__bf16*)Wop, p.chunks1, AT);
  const long long g2 = geo.slices * p.chunks2;
  pass2_bf16<D, AT, kLse><<<dim3((unsigned)g2), dim3(pass2_waves<AT>() * kWave), 0, stream>>>(
      (const __bf16*)Q, (const __bf16*)U, (const u32x4*)Wop, (__bf16*)H, geo.vw.q, geo.vw.o,
      geo.h, geo.n, geo.m, p.chunks2, p.chunk_len2, geo.c2, 0, lse);
  return hipGetLastError();
}

template <int D>
static hipError_t dispatch_at(const Geometry& g, const SplitPlan& p, const void* Q, const void* U,
                              const void* V, void* H, void* ws, hipStream_t s) {
  switch (g.at) {
    case 2: return launch_split_bf16_t<D, 2>(g, p, Q, U, V, H, ws, s);
    case 4: return launch_split_bf16_t<D, 4>(g, p, Q, U, V, H, ws, s);
    case 6: return launch_split_bf16_t<D, 6>(g, p, Q, U, V, H, ws, s);
    case 8: return launch_split_bf16_t<D, 8>(g, p, Q, U, V, H, ws, s);
    case 12: return launch_split_bf16_t<D, 12>(g, p, Q, U, V, H, ws, s);
    case 16: return launch_split_bf16_t<D, 16>(g, p, Q, U, V, H, ws, s);
    case 24:
    case 32:
      if constexpr (D <= 64) {
        return g.at == 24 ? launch_split_bf16_t<D, 24>(g, p, Q, U, V, H, ws, s)
                          : launch_split_bf16_t<D, 32>(g, p, Q, U, V, H, ws, s);
      }
      return hipErrorInvalidValue;
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_split_bf16(const Geometry& g, const SplitPlan& p, const void* Q, const void* U,
                             const void* V, void* H, void* ws, hipStream_t stream) {
  if (g.d == 64) return dispatch_at<64>(g, p, Q, U, V, H, ws, stream);
  if (g.d == 32) return dispatch_at<32>(g, p, Q, U, V, H, ws, stream);
  if (g.d == 128) return dispatch_at<128>(g, p, Q, U, V, H, ws, stream);
  return hipErrorInvalidValue;
}

hipError_t launch_pass1_bf16(const Geometry& g, const SplitPlan& p, const void* Q, const void* U,
                             const void* X, float* part, float* dpart, hipStream_t s) {
  auto at = [&](auto D) -> hipError_t {
    constexpr int d = decltype(D)::value;
    switch (g.at) {
      case 2: launch_pass1_t<d, 2>(g, p, Q, U, X, part, dpart, nullptr, s); break;
      case 4: launch_pass1_t<d, 4>(g, p, Q, U, X, part, dpart, nullptr, s); break;
      case 6: launch_pass1_t<d, 6>(g, p, Q, U, X, part, dpart, nullptr, s); break;
      case 8: launch_pass1_t<d, 8>(g, p, Q, U, X, part, dpart, nullptr, s); break;
      case 12: launch_pass1_t<d, 12>(g, p, Q, U, X, part, dpart, nullptr, s); break;
      case 16: launch_pass1_t<d, 16>(g, p, Q, U, X, part, dpart, nullptr, s); break;
      default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
  };
  if (g.d == 64) return at(std::integral_constant<int, 64>{});
  if (g.d == 32) return at(std::integral_constant<int, 32>{});
  if (g.d == 128) return at(std::integral_constant<int, 128>{});
  return hipErrorInvalidValue;
}

// The backward's pass 1 on V and on G in one launch (up to 256 anchors at d <= 64, 96 at
// d = 128): A^T V with Delta into part and dpart, A^T G into partG, partials as
// launch_pass1_bf16's.  Above 128 anchors each token's log-sum-exp (base 2) also goes to
// lse ([slice][n]) when it is not null.
hipError_t launch_pass1_dual_bf16(const Geometry& g, const SplitPlan& p, const void* Q,
                                  const void* U, const void* V, const View& vw, const void* G,
                                  const View& gw, float* part, float* partG, float* dpart,
                                  float* lse, hipStream_t s) {
  const long long g1 = g.slices * p.chunks1;
  auto at = [&](auto D) -> hipError_t {
    constexpr int d = decltype(D)::value;
#define AA_DUAL(MP)                                                                          \
  pass1x_bf16<d, MP, kPass1Waves, false, true><<<dim3((unsigned)g1), dim3(kPass1Waves * kWave), 0, s>>>( \
      (const __bf16*)Q, (const __bf16*)U, (const __bf16*)V, part, dpart, g.vw.q, vw, g.h, g.n, g.m, \
      p.chunks1, p.chunk_len1, g.c2, nullptr, nullptr, View{0, 0, 0}, (const __bf16*)G, gw, partG)
#define AA_DUALA(AT)                                                                         \
  pass1a_bf16<d, AT, 4, true><<<dim3((unsigned)g1), dim3(4 * kWave), 0, s>>>(                  \
      (const __bf16*)Q, (const __bf16*)U, (const __bf16*)V, part, dpart, g.vw.q, vw, g.h, g.n, g.m, \
      p.chunks1, p.chunk_len1, g.c2, lse, (const __bf16*)G, gw, partG)
    switch (g.at) {
      case 2: AA_DUAL(1); break;
      case 4: AA_DUAL(2); break;
      case 6: AA_DUAL(3); break;
      case 8:
        if constexpr (d <= 64) { AA_DUAL(4); break; }
        return hipErrorInvalidValue;
      case 12:
        if constexpr (d <= 64) { AA_DUALA(12); break; }
        return hipErrorInvalidValue;
      case 16:
        if constexpr (d <= 64) { AA_DUALA(16); break; }
        return hipErrorInvalidValue;
      default: return hipErrorInvalidValue;
    }
#undef AA_DUAL
#undef AA_DUALA
    return hipGetLastError();
  };
  if (g.d == 64) return at(std::integral_constant<int, 64>{});
  if (g.d == 32) return at(std::integral_constant<int, 32>{});
  if (g.d == 128 && g.at <= 6) return at(std::integral_constant<int, 128>{});
  return hipErrorInvalidValue;
}

// Nystrom attention: pass 1 in landmark mode (the keys K streamed as the tokens, the
// landmark query rows gathered from Q through idx as the anchors, the per-chunk landmark
// maxima written to cmax) and pass 2 with the per-slice landmark key rows kt as the
// anchors.
hipError_t launch_nystrom_pass1_bf16(const Geometry& g, const SplitPlan& p, const void* K,
                                     const View& kw, const void* Q, const View& qw,
                                     const int* idx, const void* V, const View& vw, float* part,
                                     float* dpart, float* cmax, hipStream_t s) {
  const long long g1 = g.slices * p.chunks1;
  auto at = [&](auto D) -> hipError_t {
    constexpr int d = decltype(D)::value;
#define AA_NYS1(MP)                                                                          \
  pass1x_bf16<d, MP, kPass1Waves, true><<<dim3((unsigned)g1), dim3(kPass1Waves * kWave), 0, s>>>( \
      (const __bf16*)K, (const __bf16*)Q, (const __bf16*)V, part, dpart, kw, vw, g.h, g.n, g.m, \
      p.chunks1, p.chunk_len1, g.c2, cmax, idx, qw)
    switch (g.at) {
      case 2: AA_NYS1(1); break;
      case 4: AA_NYS1(2); break;
      case 6: AA_NYS1(3); break;
      case 8:
        if constexpr (d <= 64) { AA_NYS1(4); break; }
        return hipErrorInvalidValue;
      default: return hipErrorInvalidValue;
    }
#undef AA_NYS1
    return hipGetLastError();
  };
  if (g.d == 64) return at(std::integral_constant<int, 64>{});
  if (g.d == 32) return at(std::integral_constant<int, 32>{});
  if (g.d == 128) return at(std::integral_constant<int, 128>{});   // up to 96 landmarks
  return hipErrorInvalidValue;
}

hipError_t launch_nystrom_pass2_bf16(const Geometry& g, const SplitPlan& p, const void* Q,
                                     const View& qw, const void* kt, const void* Wop, void* H,
                                     const View& ow, hipStream_t s) {
  const long long g2 = g.slices * p.chunks2;
  auto at = [&](auto D) -> hipError_t {
    constexpr int d = decltype(D)::value;
#define AA_NYS2(AT)                                                                           \
  pass2_bf16<d, AT, false><<<dim3((unsigned)g2), dim3(pass2_waves<AT>() * kWave), 0, s>>>(    \
      (const __bf16*)Q, (const __bf16*)kt, (const u32x4*)Wop, (__bf16*)H, qw, ow, g.h, g.n, g.m, \
      p.chunks2, p.chunk_len2, g.c2, 1, nullptr)
    switch (g.at) {
      case 2: AA_NYS2(2); break;
      case 4: AA_NYS2(4); break;
      case 6: AA_NYS2(6); break;
      case 8:
        if constexpr (d <= 64) { AA_NYS2(8); break; }
        return hipErrorInvalidValue;
      default: return hipErrorInvalidValue;
    }
#undef AA_NYS2
    return hipGetLastError();
  };
  if (g.d == 64) return at(std::integral_constant<int, 64>{});
  if (g.d == 32) return at(std::integral_constant<int, 32>{});
  if (g.d == 128) return at(std::integral_constant<int, 128>{});   // up to 96 landmarks
  return hipErrorInvalidValue;
}

}  // namespace aa
