// fused_bf16.hip -- one or two workgroups per (batch, head) slice for short sequences.
//
// Computes, per slice (AnchorFormer, Pith verdict page: referee summary, Eq. (11) in the
// Eq. (12) order; desk-editor letter: A row-stochastic, Delta its column sums):
//   A = rowsoftmax(Q U^T / sqrt(d)),  W = Delta^-1 (A^T V),  H = A W
// with Q and V read from HBM once and H written once (a slice shared by two workgroups,
// one per half of the output dims, reads Q twice; the second read is meant to hit L2).
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
#include <algorithm>

#include "device_common.h"
#include "kernels.h"
#include "tile_ops.h"

namespace aa {

// LDS of one workgroup, sized for a workgroup that handles DL of the D dims of V and H:
// all of them, or half at d = 128, where every slice is shared by two workgroups (a whole
// d = 128 slice's V rows would leave room for one workgroup per CU).
template <int D, int MP, int NW>
struct FusedLds {
  static constexpr int DL = (D == 128) ? D / 2 : D;
  static constexpr int AT = 2 * MP, KS = D / 32, DT = DL / 16;
  static constexpr int AS = tr_stride<32 * MP>(), VS = tr_stride<DL>();
  u32x4 u[AT][KS][kWave];                                   // U as left operands of S^T
  __attribute__((aligned(16))) __bf16 a[NW * 32 * AS];      // rows of A, this round
  __attribute__((aligned(16))) __bf16 v[NW * 32 * VS];      // rows of V, this round
  u32x4 w[DT][MP][kWave];                                   // W^T left operands
  float dl[AT][16];                                         // Delta per anchor tile
};

// One workgroup's share of a slice: all of its tokens and the DW output dims starting at
// d0 (DW = D, or D / 2 when two workgroups share the slice).  Both workgroups of a shared
// slice compute the same A (the logits need all of Q), each reads only its half of V and
// writes only its half of H.  NW waves, ROUNDS rounds of NW pairs (compile-time bound;
// the loop stops at the slice's last pair).
template <int D, int DW, int MP, int NW, int ROUNDS, bool KEEP_A>
__device__ __forceinline__ void fused_part(FusedLds<D, MP, NW>& L, const __bf16* __restrict__ Q,
                                           const __bf16* __restrict__ U,
                                           const __bf16* __restrict__ V, __bf16* __restrict__ H,
                                           const Views& vw, int slice, int d0, int h, int n, int m,
                                           float c2) {
  constexpr int KS = D / 32, KV = DW / 32, DTW = DW / 16, AT = 2 * MP;
  constexpr int TILES = AT * DTW, TPW = (TILES + NW - 1) / NW;
  constexpr int NDA = (TPW + DTW - 1) / DTW;   // anchor tiles per wave that need a Delta
  constexpr int AS = FusedLds<D, MP, NW>::AS, VS = tr_stride<DW>();
  static_assert(TILES % NW == 0 || NW % TILES == 0, "tiles split evenly over the waves");
  static_assert(DW <= FusedLds<D, MP, NW>::DL, "the LDS holds this part's dims");
  const int head = slice % h;
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // uniform per wave
  const int c = lane & 15, g = lane >> 4;
  const size_t qb = view_base(vw.q, slice, h), vb = view_base(vw.v, slice, h);
  const size_t ob = view_base(vw.o, slice, h);
  const long long qs = vw.q.st, vs = vw.v.st;
  const int npairs = (n + 31) >> 5;

  // This wave's first pair goes out to memory before anything else.  Lane (c,g) holds
  // dims 32kk + 8g .. + 7 of its token in chunk kk (of Q: all dims; of V: this part's).
  u32x4 qc[2][KS], vc[2][KV];
#pragma unroll
  for (int tt = 0; tt < 2; ++tt) {
    load_rows_c<D, D>(Q, qb, qs, 32 * w + 16 * tt + c, n, g, 0, qc[tt]);
    load_rows_c<D, DW>(V, vb, vs, 32 * w + 16 * tt + c, n, g, d0, vc[tt]);
  }
  // U as left operands of S^T = U Q^T: lane (c,g) of tile j holds anchor 16j + c with
  // the dims of Q's chunk layout.
  const __bf16* Uh = U + (size_t)head * m * D;
  for (int idx = threadIdx.x; idx < AT * KS * kWave; idx += NW * kWave) {
    const int j = idx / (KS * kWave), kk = (idx / kWave) % KS, l = idx & 63;
    const int a = 16 * j + (l & 15);
    u32x4 v = {0u, 0u, 0u, 0u};
    if (a < m) v = *(const u32x4*)(Uh + (size_t)a * D + 8 * (l >> 4) + 32 * kk);
    L.u[j][kk][l] = v;
  }
  const bf16x8 ones = splat_bf16(1.f);
  f32x4 mask[2];
  pad_mask<MP>(g, m, mask);
  __syncthreads();
  // With several rounds U's operands stay in registers instead of being read from LDS
  // every round.  At d = 128 those registers go to the kept A instead, and with more than
  // three kept rounds the next pair's V is requested at the end of a round rather than a
  // round ahead (registers again).
  constexpr bool UREG = KEEP_A && ROUNDS > 2 && D != 128;
  constexpr bool VAHEAD = !(D == 128 && KEEP_A && ROUNDS > 3);
  bf16x8 ureg[UREG ? AT : 1][KS];
  if constexpr (UREG) {
#pragma unroll
    for (int j = 0; j < AT; ++j)
#pragma unroll
      for (int kk = 0; kk < KS; ++kk) ureg[j][kk] = as_bf16x8(L.u[j][kk][lane]);
  }

  // Wave w owns the contiguous tiles w*TPW .. w*TPW + TPW - 1 (tile t: anchor tile t / DTW,
  // dim tile t % DTW of this part); the Delta of an anchor tile is accumulated with its
  // dim tile 0.
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
    // The next round's rows are requested unconditionally (rows past the slice read its
    // last row; a pair past the end is never used): a load under a branch would make the
    // wait for this round's rows at the join an unconditional vmcnt(0).
    const bool more = r + 1 < ROUNDS;
    u32x4 qn[2][KS], vn[VAHEAD ? 2 : 1][KV];
    if (more) {
#pragma unroll
      for (int tt = 0; tt < 2; ++tt) {
        load_rows_c<D, D>(Q, qb, qs, 32 * (p + NW) + 16 * tt + c, n, g, 0, qn[tt]);
        if constexpr (VAHEAD)
          load_rows_c<D, DW>(V, vb, vs, 32 * (p + NW) + 16 * tt + c, n, g, d0, vn[tt]);
      }
    }
    // Phase A: rows 32w .. 32w + 31 of the round's LDS blocks hold this wave's pair.
    if (p < npairs) {
#pragma unroll
      for (int tt = 0; tt < 2; ++tt) {
        bf16x8 ab[MP];
        if constexpr (UREG)
          tile_softmax_op<D, MP>([&](int j, int kk) { return ureg[j][kk]; }, qc[tt], mask,
                                 32 * p + 16 * tt + c < n, c2, ab);
        else
          tile_softmax<D, MP>(L.u, qc[tt], lane, mask, 32 * p + 16 * tt + c < n, c2, ab);
        if constexpr (KEEP_A) {
#pragma unroll
          for (int jj = 0; jj < MP; ++jj) keep[r][tt][jj] = ab[jj];
        }
        // ab[jj] holds anchors 32jj + 4g .. + 3 and 32jj + 16 + 4g .. + 3 of token c.
        __bf16* arow = L.a + (32 * w + 16 * tt + c) * AS + 4 * g;
#pragma unroll
        for (int jj = 0; jj < MP; ++jj) {
          const u32x4 v = as_u32x4(ab[jj]);
          *(u32x2*)(arow + 32 * jj) = u32x2{v[0], v[1]};
          *(u32x2*)(arow + 32 * jj + 16) = u32x2{v[2], v[3]};
        }
        __bf16* vrow = L.v + (32 * w + 16 * tt + c) * VS + 8 * g;
#pragma unroll
        for (int kk = 0; kk < KV; ++kk) *(u32x4*)(vrow + 32 * kk) = vc[tt][kk];
      }
    }
    __syncthreads();
    // Phase B: this wave's tiles (all TPW of them, or none when there are fewer tiles
    // than waves), accumulated over the round's pairs.
    if (w * TPW < TILES)
      accumulate_tiles<TPW, DTW, AS, VS>(L.a, L.v, w * TPW, pairs_here, c, g, ones, pacc, dacc);
    __syncthreads();
    if (more) {
#pragma unroll
      for (int tt = 0; tt < 2; ++tt) {
#pragma unroll
        for (int kk = 0; kk < KS; ++kk) qc[tt][kk] = qn[tt][kk];
        if constexpr (VAHEAD) {
#pragma unroll
          for (int kk = 0; kk < KV; ++kk) vc[tt][kk] = vn[tt][kk];
        } else {
          load_rows_c<D, DW>(V, vb, vs, 32 * (p + NW) + 16 * tt + c, n, g, d0, vc[tt]);
        }
      }
    }
  }

  // Tile (ja, dt) of P holds P[16ja + 4g + r][d0 + 16dt + c] in lane (c,g), register r.
  // W = P / Delta for this wave's tiles, stored as bf16 left operands of H^T = W^T A^T:
  // [dt2][jj][lane'][slot] with lane' (c', g') holding local dim out_dim_c(dt2, c') and
  // anchors {32jj + 4g' + s, 32jj + 16 + 4g' + s - 4}.  The Delta of each anchor tile
  // goes through LDS from the wave that accumulated it.
#pragma unroll
  for (int k = 0; k < TPW; ++k) {
    const int t = w * TPW + k;
    const int ja = t / DTW, dt = t - (t / DTW) * DTW;
    if (t < TILES && dt == 0 && c == 0) {
#pragma unroll
      for (int r = 0; r < 4; ++r) L.dl[ja][4 * g + r] = dacc[k / DTW][r];
    }
  }
  __syncthreads();
  {
    __bf16* wl = (__bf16*)&L.w[0][0][0];
#pragma unroll
    for (int k = 0; k < TPW; ++k) {
      const int t = w * TPW + k;
      if (t >= TILES) break;
      const int ja = t / DTW, dt = t - (t / DTW) * DTW;
      const int dim = 16 * dt + c;   // local dim; inverse of out_dim_c
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

  bf16x8 wop[DTW][MP];
#pragma unroll
  for (int dt2 = 0; dt2 < DTW; ++dt2)
#pragma unroll
    for (int jj = 0; jj < MP; ++jj) wop[dt2][jj] = as_bf16x8(L.w[dt2][jj][lane]);

#pragma unroll (KEEP_A ? ROUNDS : 1)
  for (int r = 0; r < ROUNDS; ++r) {
    const int p = r * NW + w;
    if (p < npairs) {
      u32x4 qr[2][KS];
      if constexpr (!KEEP_A) {
#pragma unroll
        for (int tt = 0; tt < 2; ++tt) load_rows_c<D, D>(Q, qb, qs, 32 * p + 16 * tt + c, n, g, 0, qr[tt]);
      }
#pragma unroll
      for (int tt = 0; tt < 2; ++tt) {
        const int row = 32 * p + 16 * tt + c;
        bf16x8 ab[MP];
        if constexpr (KEEP_A) {
#pragma unroll
          for (int jj = 0; jj < MP; ++jj) ab[jj] = keep[r][tt][jj];
        } else {
          tile_softmax<D, MP>(L.u, qr[tt], lane, mask, row < n, c2, ab);
        }
        f32x4 hacc[DTW];
#pragma unroll
        for (int dt2 = 0; dt2 < DTW; ++dt2) {
          f32x4 acc = zero4();
#pragma unroll
          for (int jj = 0; jj < MP; ++jj) acc = mfma_bf16(wop[dt2][jj], ab[jj], acc);
          hacc[dt2] = acc;
        }
        // Lane group g holds local dims 32hh + 8g .. + 7 in tiles 2hh and 2hh + 1.
        if (row < n) {
          __bf16* dst = H + ob + view_row(vw.o, row) + d0 + 8 * g;
#pragma unroll
          for (int hh = 0; hh < DTW / 2; ++hh)
            __builtin_nontemporal_store(as_u32x4(pack_bf16(hacc[2 * hh], hacc[2 * hh + 1])),
                                        (u32x4*)(dst + 32 * hh));
        }
      }
    }
  }
}

// Workgroups 0 .. full - 1 take slices 0 .. full - 1 whole; the remaining slices are
// shared by two workgroups each, one per half of the output dims, so that a grid with
// between one and two slices per CU still gives every CU about the same work.
// MINW: waves per SIMD the registers must allow (two workgroups per CU).
template <int D, int MP, int NW, int ROUNDS, bool KEEP_A, int MINW>
__global__ __launch_bounds__(NW * kWave, MINW)
void fused_bf16(const __bf16* __restrict__ Q, const __bf16* __restrict__ U,
                const __bf16* __restrict__ V, __bf16* __restrict__ H, Views vw, int h, int n,
                int m, float c2, int full) {
  __shared__ FusedLds<D, MP, NW> L;
  const int b = blockIdx.x;
  if (b < full) {
    if constexpr (D != 128)   // at d = 128 every slice is shared (full == 0)
      fused_part<D, D, MP, NW, ROUNDS, KEEP_A>(L, Q, U, V, H, vw, b, 0, h, n, m, c2);
  } else if constexpr (D >= 64) {
    // Within each run of 16 shared workgroups, ids i and i + 8 take the two halves of one
    // slice: workgroups are dealt to the XCDs in turn, so both halves (which read the
    // same Q) usually sit on one XCD and the second read of Q hits its L2.  A last
    // incomplete run pairs neighbouring ids.
    const int k = b - full;
    const int nsh = (int)(gridDim.x - full);   // twice the number of shared slices
    int sl, hf;
    if ((k | 15) < (nsh & ~15)) {
      sl = ((k >> 4) << 3) + (k & 7);
      hf = (k >> 3) & 1;
    } else {
      sl = k >> 1;
      hf = k & 1;
    }
    fused_part<D, D / 2, MP, NW, ROUNDS, KEEP_A>(L, Q, U, V, H, vw, full + sl, hf * (D / 2), h, n,
                                                 m, c2);
  }
}

// Plans (n <= 1024, m <= 64; d = 128 and m <= 32: n <= 256):
//   m <= 32: eight waves, A kept for up to two rounds (n <= 512), else recomputed; at
//            d = 128 four waves of up to two rounds, A kept;
//   m <= 64: four waves, A kept for up to five rounds (n <= 640), else recomputed.
// Registers and LDS allow two workgroups per CU (three for the d = 128, m <= 32 plan:
// 45 KB of LDS, four waves).  With d = 64 and
// fewer than two slices per CU, 2 * CUs - slices slices are shared by two workgroups so
// that every CU gets about one and a half slices' worth of loads, stores and products.
// With d = 128 every slice is shared (each workgroup holds 64 dims of V in LDS).
static bool fused_choose(const Geometry& g, int num_cus, FusedPlan* plan) {
  if (g.d != 32 && g.d != 64 && g.d != 128) return false;
  const int npairs = (g.n + 31) / 32;
  FusedPlan p{};
  // d = 128 with up to 32 anchors: n <= 256 (longer slices take the split plan)
  if (g.m_pad == 32 && g.d == 128 && npairs <= 8) {
    // four waves of up to two pairs: 45 KB of LDS, three workgroups per CU
    p.waves = 4;
    p.pairs_per_wave = (npairs + 3) / 4;
    p.keep_a = true;
  } else if (g.m_pad == 32 && npairs <= 32 && g.d != 128) {
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
  p.shared = 0;
  if (g.d == 64) p.shared = std::min<long long>(g.slices, std::max<long long>(0, 2LL * num_cus - g.slices));
  if (g.d == 128) p.shared = g.slices;
  if (plan) *plan = p;
  return true;
}

bool fused_supported(const Geometry& g, int num_cus, FusedPlan* plan) {
  return fused_choose(g, num_cus, plan);
}

template <int D, int MP, int NW, int ROUNDS, bool KEEP, int MINW>
static hipError_t go(const Geometry& g, const FusedPlan& p, const void* Q, const void* U,
                     const void* V, void* H, hipStream_t s) {
  const long long full = g.slices - p.shared;
  const long long grid = full + 2 * p.shared;
  if (grid > 0x7fffffffLL) return hipErrorInvalidValue;
  fused_bf16<D, MP, NW, ROUNDS, KEEP, MINW><<<dim3((unsigned)grid), dim3(NW * kWave), 0, s>>>(
      (const __bf16*)Q, (const __bf16*)U, (const __bf16*)V, (__bf16*)H, g.vw, g.h, g.n, g.m,
      g.c2, (int)full);
  return hipGetLastError();
}

template <int D>
static hipError_t dispatch(const Geometry& g, const FusedPlan& p, const void* Q, const void* U,
                           const void* V, void* H, hipStream_t s) {
  const int r = p.pairs_per_wave;
  if (g.m_pad == 32) {
    if constexpr (D == 128) {
      if (r <= 2) return go<D, 1, 4, 2, true, 3>(g, p, Q, U, V, H, s);
      return hipErrorInvalidValue;
    }
    if (r == 1) return go<D, 1, 8, 1, true, 4>(g, p, Q, U, V, H, s);
    if constexpr (D != 128) {
      if (r == 2) return go<D, 1, 8, 2, true, 2>(g, p, Q, U, V, H, s);
      if (r <= 4) return go<D, 1, 8, 4, false, 2>(g, p, Q, U, V, H, s);
    }
    return hipErrorInvalidValue;
  }
  if (r <= 2) return go<D, 2, 4, 2, true, 2>(g, p, Q, U, V, H, s);
  if (r <= 3) return go<D, 2, 4, 3, true, 2>(g, p, Q, U, V, H, s);
  if (r <= 5) return go<D, 2, 4, 5, true, 2>(g, p, Q, U, V, H, s);
  if (r <= 8) return go<D, 2, 4, 8, false, 2>(g, p, Q, U, V, H, s);
  return hipErrorInvalidValue;
}

hipError_t launch_fused_bf16(const Geometry& g, const FusedPlan& p, const void* Q, const void* U,
                             const void* V, void* H, hipStream_t s) {
  FusedPlan chk{};
  if (!fused_choose(g, 1, &chk) || chk.waves != p.waves || chk.pairs_per_wave != p.pairs_per_wave ||
      chk.keep_a != p.keep_a || p.shared < 0 || p.shared > g.slices || (p.shared > 0 && g.d == 32) ||
      (g.d == 128 && p.shared != g.slices))
    return hipErrorInvalidValue;
  if (g.d == 128) return dispatch<128>(g, p, Q, U, V, H, s);
  if (g.d == 64) return dispatch<64>(g, p, Q, U, V, H, s);
  if (g.d == 32) return dispatch<32>(g, p, Q, U, V, H, s);
  return hipErrorInvalidValue;
}

}  // namespace aa
