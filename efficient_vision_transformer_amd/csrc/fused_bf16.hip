// fused_bf16.hip -- one workgroup per (batch, head) slice for short token sequences.
//
// Computes, per slice (AnchorFormer, Pith verdict page: referee summary, Eq. (11) in the
// Eq. (12) order; desk-editor letter: A row-stochastic, Delta its column sums):
//   A = rowsoftmax(Q U^T / sqrt(d)),  W = Delta^-1 (A^T V),  H = A W
// with Q and V read from HBM once and H written once.
//
// The slice's tokens are taken in rounds of one 32-token pair per wave.
//   Phase A (per wave, its pair): S^T = U Q^T on the MFMA (lanes = tokens, registers =
//     anchors), softmax over anchors in registers plus two permlane swaps, A rounded to
//     bf16.  The pair's rows of A ([token][anchor]) and of V ([token][dim]) go to LDS as
//     they are.
//   Phase B (after one barrier): every wave owns distinct (16-anchor, 16-dim) tiles of
//     A^T V and accumulates them, and the matching column sums Delta (A^T times ones),
//     over all pairs of the round.  Both operands need the tokens on the contraction
//     axis; the transposing LDS read delivers them in that layout straight from the row
//     copies.  No partial sums are ever added across waves, so the result does not
//     depend on scheduling.
// After the last round each wave turns its tiles into W = P / Delta (0 where Delta == 0)
// and stores them as bf16 MFMA operands in LDS; then every wave writes H^T = W^T A^T for
// its tokens, with A kept in registers (KEEP_A) or recomputed from Q.
#include "device_common.h"
#include "kernels.h"
#include "tile_ops.h"

namespace aa {

// NW waves per workgroup, ROUNDS rounds of NW pairs (compile-time bound; the loop stops
// at the slice's last pair).  MINW: waves per SIMD the registers must allow (two
// workgroups per CU).
template <int D, int MP, int NW, int ROUNDS, bool KEEP_A, int MINW>
__global__ __launch_bounds__(NW * kWave, MINW)
void fused_bf16(const __bf16* __restrict__ Q, const __bf16* __restrict__ U,
                const __bf16* __restrict__ V, __bf16* __restrict__ H, int h, int n, int m,
                float c2) {
  constexpr int KS = D / 32, DT = D / 16, AT = 2 * MP;
  constexpr int TILES = AT * DT, TPW = (TILES + NW - 1) / NW;
  constexpr int NDA = (TPW + DT - 1) / DT;   // anchor tiles per wave that need a Delta
  constexpr int AS = tr_stride<32 * MP>(), VS = tr_stride<D>();
  static_assert(TILES % NW == 0 || NW % TILES == 0, "tiles split evenly over the waves");
  const int slice = blockIdx.x;
  const int head = slice % h;
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // uniform per wave
  const int c = lane & 15, g = lane >> 4;
  const size_t base = (size_t)slice * (size_t)n * D;
  const int npairs = (n + 31) >> 5;

  __shared__ u32x4 u_lds[AT][KS][kWave];
  __shared__ __attribute__((aligned(16))) __bf16 a_lds[NW * 32 * AS];   // rows of A, this round
  __shared__ __attribute__((aligned(16))) __bf16 v_lds[NW * 32 * VS];   // rows of V, this round
  __shared__ u32x4 w_lds[DT][MP][kWave];    // W^T left operands

  // This wave's first pair goes out to memory before anything else.
  u32x4 qc[2][KS], vc[2][KS];
#pragma unroll
  for (int tt = 0; tt < 2; ++tt) {
    load_rows<D>(Q, base, 32 * w + 16 * tt + c, n, g, qc[tt]);
    load_rows<D>(V, base, 32 * w + 16 * tt + c, n, g, vc[tt]);
  }
  // U as left operands of S^T = U Q^T: lane (c,g) of tile j holds anchor 16j + c.
  const __bf16* Uh = U + (size_t)head * m * D;
  for (int idx = threadIdx.x; idx < AT * KS * kWave; idx += NW * kWave) {
    const int j = idx / (KS * kWave), kk = (idx / kWave) % KS, l = idx & 63;
    const int a = 16 * j + (l & 15);
    u32x4 v = {0u, 0u, 0u, 0u};
    if (a < m) v = *(const u32x4*)(Uh + (size_t)a * D + 8 * KS * (l >> 4) + 8 * kk);
    u_lds[j][kk][l] = v;
  }
  const bf16x8 ones = splat_bf16(1.f);
  f32x4 mask[2];
  pad_mask<MP>(g, m, mask);
  __syncthreads();

  // Wave w owns the contiguous tiles w*TPW .. w*TPW + TPW - 1 (tile t: anchor tile t / DT,
  // dim tile t % DT); the Delta of an anchor tile is accumulated with its dim tile 0.
  f32x4 pacc[TPW], dacc[NDA];
#pragma unroll
  for (int k = 0; k < TPW; ++k) pacc[k] = zero4();
#pragma unroll
  for (int k = 0; k < NDA; ++k) dacc[k] = zero4();
  bf16x8 keep[KEEP_A ? ROUNDS : 1][2][MP];

#pragma unroll (KEEP_A ? ROUNDS : 1)
  for (int r = 0; r < ROUNDS; ++r) {
    const int pairs_here = min(NW, npairs - r * NW);  // uniform over the workgroup
    if (pairs_here <= 0) break;
    const int p = r * NW + w;
    const bool more = (r + 1 < ROUNDS) && (p + NW < npairs);
    u32x4 qn[2][KS], vn[2][KS];
    if (more) {
#pragma unroll
      for (int tt = 0; tt < 2; ++tt) {
        load_rows<D>(Q, base, 32 * (p + NW) + 16 * tt + c, n, g, qn[tt]);
        load_rows<D>(V, base, 32 * (p + NW) + 16 * tt + c, n, g, vn[tt]);
      }
    }
    // Phase A: rows 32w .. 32w + 31 of the round's LDS blocks hold this wave's pair.
    if (p < npairs) {
#pragma unroll
      for (int tt = 0; tt < 2; ++tt) {
        bf16x8 ab[MP];
        tile_softmax<D, MP>(u_lds, qc[tt], lane, mask, 32 * p + 16 * tt + c < n, c2, ab);
        if constexpr (KEEP_A) {
#pragma unroll
          for (int jj = 0; jj < MP; ++jj) keep[r][tt][jj] = ab[jj];
        }
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
      }
    }
    __syncthreads();
    // Phase B: this wave's tiles, accumulated over the round's pairs.
#pragma unroll
    for (int k = 0; k < TPW; ++k) {
      const int t = w * TPW + k;
      if (t >= TILES) break;   // uniform per wave
      const int ja = t / DT, dt = t - (t / DT) * DT;
      f32x4 pa = pacc[k], da = dacc[k / DT];
#pragma unroll
      for (int ps = 0; ps < NW; ++ps) {
        if (ps < pairs_here) {
          const bf16x8 x = lds_operand_tr(a_lds + 32 * ps * AS, AS, 16 * ja, c, g);
          const bf16x8 y = lds_operand_tr(v_lds + 32 * ps * VS, VS, 16 * dt, c, g);
          pa = mfma_bf16(x, y, pa);
          if (dt == 0) da = mfma_bf16(x, ones, da);
        }
      }
      pacc[k] = pa;
      if (dt == 0) dacc[k / DT] = da;
    }
    __syncthreads();
    if (more) {
#pragma unroll
      for (int tt = 0; tt < 2; ++tt)
#pragma unroll
        for (int kk = 0; kk < KS; ++kk) { qc[tt][kk] = qn[tt][kk]; vc[tt][kk] = vn[tt][kk]; }
    }
  }

  // Tile (ja, dt) of P holds P[16ja + 4g + r][16dt + c] in lane (c,g), register r.
  // W = P / Delta for this wave's tiles, stored as bf16 left operands of H^T = W^T A^T:
  // [dt2][jj][lane'][slot] with lane' (c', g') holding dim out_dim(dt2, c') and anchors
  // {32jj + 4g' + s, 32jj + 16 + 4g' + s - 4}.  The Delta of each anchor tile goes
  // through LDS from the wave that accumulated it.
  __shared__ float dl_lds[AT][16];
#pragma unroll
  for (int k = 0; k < TPW; ++k) {
    const int t = w * TPW + k;
    const int ja = t / DT, dt = t - (t / DT) * DT;
    if (t < TILES && dt == 0 && c == 0) {
#pragma unroll
      for (int r = 0; r < 4; ++r) dl_lds[ja][4 * g + r] = dacc[k / DT][r];
    }
  }
  __syncthreads();
  {
    __bf16* wl = (__bf16*)&w_lds[0][0][0];
#pragma unroll
    for (int k = 0; k < TPW; ++k) {
      const int t = w * TPW + k;
      if (t >= TILES) break;
      const int ja = t / DT, dt = t - (t / DT) * DT;
      const int dim = 16 * dt + c;
      const int rem = dim % (D / 4);
      const int dt2 = rem >> 2, cc = 4 * (dim / (D / 4)) + (rem & 3);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int anchor = 16 * ja + 4 * g + r;
        const float delta = dl_lds[ja][4 * g + r];
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
    for (int jj = 0; jj < MP; ++jj) wop[dt2][jj] = as_bf16x8(w_lds[dt2][jj][lane]);

#pragma unroll (KEEP_A ? ROUNDS : 1)
  for (int r = 0; r < ROUNDS; ++r) {
    const int p = r * NW + w;
    if (p < npairs) {
      u32x4 qr[2][KS];
      if constexpr (!KEEP_A) {
#pragma unroll
        for (int tt = 0; tt < 2; ++tt) load_rows<D>(Q, base, 32 * p + 16 * tt + c, n, g, qr[tt]);
      }
#pragma unroll
      for (int tt = 0; tt < 2; ++tt) {
        const int row = 32 * p + 16 * tt + c;
        bf16x8 ab[MP];
        if constexpr (KEEP_A) {
#pragma unroll
          for (int jj = 0; jj < MP; ++jj) ab[jj] = keep[r][tt][jj];
        } else {
          tile_softmax<D, MP>(u_lds, qr[tt], lane, mask, row < n, c2, ab);
        }
        f32x4 hacc[DT];
#pragma unroll
        for (int dt2 = 0; dt2 < DT; ++dt2) {
          f32x4 acc = zero4();
#pragma unroll
          for (int jj = 0; jj < MP; ++jj) acc = mfma_bf16(wop[dt2][jj], ab[jj], acc);
          hacc[dt2] = acc;
        }
        if (row < n) {
          __bf16* dst = H + base + (size_t)row * D + (D / 4) * g;
#pragma unroll
          for (int hh = 0; hh < DT / 2; ++hh)
            __builtin_nontemporal_store(as_u32x4(pack_bf16(hacc[2 * hh], hacc[2 * hh + 1])),
                                        (u32x4*)(dst + 8 * hh));
        }
      }
    }
  }
}

// Plans (n <= 1024, m <= 64):
//   m <= 32: eight waves, A kept for up to two rounds (n <= 512), else recomputed;
//   m <= 64: four waves, A kept for up to five rounds (n <= 640), else recomputed.
// Both keep two workgroups per CU within the register and LDS budgets.
static bool fused_choose(const Geometry& g, FusedPlan* plan) {
  if (g.d != 32 && g.d != 64) return false;
  const int npairs = (g.n + 31) / 32;
  FusedPlan p{};
  if (g.m_pad == 32 && npairs <= 32) {
    p.waves = 8;
    p.pairs_per_wave = (npairs + 7) / 8;
    p.keep_a = p.pairs_per_wave <= 2;
  } else if (g.m_pad == 64 && npairs <= 32) {
    p.waves = 4;
    p.pairs_per_wave = (npairs + 3) / 4;
    p.keep_a = p.pairs_per_wave <= 5;
  } else {
    return false;
  }
  if (plan) *plan = p;
  return true;
}

bool fused_supported(const Geometry& g, FusedPlan* plan) { return fused_choose(g, plan); }

template <int D, int MP, int NW, int ROUNDS, bool KEEP, int MINW>
static hipError_t go(const Geometry& g, const void* Q, const void* U, const void* V, void* H,
                     hipStream_t s) {
  fused_bf16<D, MP, NW, ROUNDS, KEEP, MINW><<<dim3((unsigned)g.slices), dim3(NW * kWave), 0, s>>>(
      (const __bf16*)Q, (const __bf16*)U, (const __bf16*)V, (__bf16*)H, g.h, g.n, g.m, g.c2);
  return hipGetLastError();
}

template <int D>
static hipError_t dispatch(const Geometry& g, const FusedPlan& p, const void* Q, const void* U,
                           const void* V, void* H, hipStream_t s) {
  const int r = p.pairs_per_wave;
  if (g.m_pad == 32) {
    if (r == 1) return go<D, 1, 8, 1, true, 4>(g, Q, U, V, H, s);
    if (r == 2) return go<D, 1, 8, 2, true, 2>(g, Q, U, V, H, s);
    if (r <= 4) return go<D, 1, 8, 4, false, 2>(g, Q, U, V, H, s);
    return hipErrorInvalidValue;
  }
  if (r <= 2) return go<D, 2, 4, 2, true, 2>(g, Q, U, V, H, s);
  if (r <= 3) return go<D, 2, 4, 3, true, 2>(g, Q, U, V, H, s);
  if (r <= 5) return go<D, 2, 4, 5, true, 2>(g, Q, U, V, H, s);
  if (r <= 8) return go<D, 2, 4, 8, false, 2>(g, Q, U, V, H, s);
  return hipErrorInvalidValue;
}

hipError_t launch_fused_bf16(const Geometry& g, const FusedPlan& p, const void* Q, const void* U,
                             const void* V, void* H, hipStream_t s) {
  FusedPlan chk{};
  if (!fused_choose(g, &chk) || chk.waves != p.waves || chk.pairs_per_wave != p.pairs_per_wave ||
      chk.keep_a != p.keep_a)
    return hipErrorInvalidValue;
  if (g.d == 64) return dispatch<64>(g, p, Q, U, V, H, s);
  if (g.d == 32) return dispatch<32>(g, p, Q, U, V, H, s);
  return hipErrorInvalidValue;
}

}  // namespace aa
