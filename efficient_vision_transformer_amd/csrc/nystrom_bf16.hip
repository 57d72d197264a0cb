// nystrom_bf16.hip -- Nystrom attention with given landmark tokens (bf16 in and out, fp32
// accumulation).
//
// Fast Nystrom Attention page (key machinery): the attention matrix is approximated by three
// row softmaxes through s landmark rows q = Q[idx], k = K[idx], the middle one inverted.  Per
// (batch, head) slice, with c = 1/sqrt(d):
//   F1 = rowsoftmax(Q k^T c) (n x s),  F2 = rowsoftmax(q k^T c) (s x s),
//   F3 = rowsoftmax(q K^T c) (s x n),  H = F1 (F2^-1 (F3 V)).
// Four launches:
//   nys_max     per (slice, token chunk): each landmark's largest logit q_a . k_t over the
//               chunk (MFMA, tokens in lanes); the chunk-0 workgroup of each slice also
//               copies the landmark rows of Q and K (token indices per batch element).
//   pass 1      (split plan, landmark mode): exp(c q_a . k_t - c M_a) with M_a the maximum
//               over all chunks, accumulated against V and against ones: F3 V and F3's row
//               sums, unnormalised, per chunk.
//   nys_solve   per slice: chunk sums -> F3 V; F2 in fp32 from the landmark rows; Z = F2^-1
//               (F3 V) by Gauss-Jordan elimination with partial pivoting, the augmented
//               matrix spread over the waves' registers; Z stored as pass 2's W operands.
//   pass 2      (split plan, per-slice anchors = the landmark keys): H = rowsoftmax(Q k^T c) Z.
#include <algorithm>

#include "device_common.h"
#include "kernels.h"
#include "pass2_layout.h"
#include "tile_ops.h"

namespace aa {

// Per (slice, chunk): cmax[slice][chunk][a] = max over the chunk's tokens t of q_a . k_t
// (raw logits, fp32 accumulation of bf16 products in the same MFMA order as pass 1's, so
// pass 1's exponents are never positive), with the landmark query rows q_a read from Q
// through the indices.  The slice's chunk-0 workgroup also writes the landmark rows of Q
// and K (qt, kt) for the later launches.  Four waves; each takes 16-token tiles with the
// next tile's rows in flight.  Entries of padded landmarks (a >= m) repeat landmark m - 1.
// Q and K contiguous [B, h, n, d]; landmark indices clamped to [0, n).
template <int D, int AT>
__global__ __launch_bounds__(256)
void nys_max(const __bf16* __restrict__ Q, const __bf16* __restrict__ K,
             const int* __restrict__ idx, __bf16* __restrict__ qt, __bf16* __restrict__ kt,
             float* __restrict__ cmax, View kw, int h, int n, int m, int chunks, int chunk_len) {
  constexpr int KS = D / 32, NW = 4, CH = D / 8;
  const int slice = blockIdx.x / chunks;
  const int chunk = blockIdx.x - slice * chunks;
  const int b = slice / h;
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int c = lane & 15, g = lane >> 4;
  const size_t kb = view_base(kw, slice, h);
  const int t_begin = chunk * chunk_len;
  const int t_end = min(n, t_begin + chunk_len);
  const int* ib = idx + (size_t)b * m;
  auto token = [&](int a) { return min(max(ib[a], 0), n - 1); };

  __shared__ u32x4 u_lds[AT][KS][kWave];
  __shared__ float red[NW][16 * AT];
  Stage<AT * KS * kWave, NW * kWave> ust;
  stage_load(ust, [&](int i) {
    const int j = i / (KS * kWave), kk = (i / kWave) % KS, l = i & 63;
    const int a = min(16 * j + (l & 15), m - 1);
    return *(const u32x4*)(Q + kb + (size_t)token(a) * D + 8 * KS * (l >> 4) + 8 * kk);
  });
  if (chunk == 0) {
    const size_t ob = (size_t)slice * m * D;
    for (int i = threadIdx.x; i < m * CH; i += NW * kWave) {
      const int a = i / CH, ch = i - a * CH;
      const size_t src = kb + (size_t)token(a) * D + 8 * ch;
      const u32x4 vq = *(const u32x4*)(Q + src), vk = *(const u32x4*)(K + src);
      *(u32x4*)(qt + ob + (size_t)a * D + 8 * ch) = vq;
      *(u32x4*)(kt + ob + (size_t)a * D + 8 * ch) = vk;
    }
  }
  u32x4 kr[KS];
  load_rows<D>(K, kb, kw.st, t_begin + 16 * w + c, n, g, kr);
  stage_store(ust, &u_lds[0][0][0]);
  __syncthreads();

  float mx[AT][4];
#pragma unroll
  for (int j = 0; j < AT; ++j)
#pragma unroll
    for (int r = 0; r < 4; ++r) mx[j][r] = -INFINITY;
  for (int t0 = t_begin + 16 * w; t0 < t_end; t0 += 16 * NW) {
    u32x4 kn[KS];
    load_rows<D>(K, kb, kw.st, t0 + 16 * NW + c, n, g, kn);   // rows clamped to the slice
    const bool ok = t0 + c < t_end;
#pragma unroll
    for (int j = 0; j < AT; ++j) {
      f32x4 acc = zero4();
#pragma unroll
      for (int kk = 0; kk < KS; ++kk) acc = mfma_bf16(as_bf16x8(u_lds[j][kk][lane]), as_bf16x8(kr[kk]), acc);
#pragma unroll
      for (int r = 0; r < 4; ++r) mx[j][r] = ok ? fmaxf(mx[j][r], acc[r]) : mx[j][r];
    }
#pragma unroll
    for (int kk = 0; kk < KS; ++kk) kr[kk] = kn[kk];
  }
  // lane (c, g) holds landmarks 16j + 4g + r over its tokens; reduce over the 16 lanes c
#pragma unroll
  for (int j = 0; j < AT; ++j)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const float v = row16_max(mx[j][r]);
      if (c == 0) red[w][16 * j + 4 * g + r] = v;
    }
  __syncthreads();
  if ((int)threadIdx.x < 16 * AT) {
    float M = red[0][threadIdx.x];
#pragma unroll
    for (int ww = 1; ww < NW; ++ww) M = fmaxf(M, red[ww][threadIdx.x]);
    cmax[((size_t)slice * chunks + chunk) * 16 * AT + threadIdx.x] = M;
  }
}

// Per slice: F3 V from the chunk partials, F2 from the landmark rows, Z = F2^-1 (F3 V) by
// Gauss-Jordan elimination with partial pivoting (fp32), Z written as pass 2's W operands.
// Partials: part[slice][chunk][jt][dt][r][lane] = sum_t e_(16jt+4g+r, t) v_(t, 16dt+c) and
// dpart[slice][chunk][a] = sum_t e_(a, t), as pass 1 leaves them.
//
// The system is padded to MPAD = 16 AT unknowns with identity rows (zero right-hand
// sides), so the elimination runs a compile-time number of steps.  The augmented matrix
// [F2 | F3 V] (MPAD x (MPAD + D)) lives in registers: wave w owns CW consecutive columns
// (32 up to 64 unknowns, else 16), lane l rows l and l + 64.  Rows are never swapped: the
// row chosen as pivot at step col ends holding unknown col (see the elimination loop).
template <int D, int AT>
constexpr int nys_solve_cw() { return 16 * AT <= 64 ? 32 : 16; }   // columns per wave
template <int D, int AT>
constexpr int nys_solve_waves() { return (16 * AT + D) / nys_solve_cw<D, AT>(); }

template <int D, int AT>
__global__ __launch_bounds__((nys_solve_waves<D, AT>() * kWave), 1)
void nys_solve(const float* __restrict__ part, const float* __restrict__ dpart,
               const __bf16* __restrict__ qt, const __bf16* __restrict__ kt,
               __bf16* __restrict__ Wop, int m, int chunks, float c2) {
  constexpr int MPAD = 16 * AT, DT = D / 16, MP = AT / 2, NC = MPAD + D, LD = NC + 1;
  constexpr int NG = nys_solve_waves<D, AT>(), T = NG * kWave, RPL = (MPAD + 63) / 64;
  constexpr int CW = nys_solve_cw<D, AT>();
  static_assert(MPAD % CW == 0 && D % CW == 0, "column groups of CW");
  const int slice = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  __shared__ float Mx[MPAD * LD];                         // set-up only
  // landmark rows with a row stride of D + 8 bf16 (144 or 80 bytes), so that the rows read
  // together by neighbouring threads fall on different LDS banks
  constexpr int RS = D + 8;
  __shared__ __attribute__((aligned(16))) __bf16 ql[MPAD * RS], kl[MPAD * RS];
  __shared__ float zl[MPAD];
  __shared__ float fbuf[2][MPAD];
  __shared__ int pbuf[2];
  __shared__ float pvbuf[2];

  // landmark rows (rows >= m zero)
  {
    const u32x4* qs = (const u32x4*)(qt + (size_t)slice * m * D);
    const u32x4* ks = (const u32x4*)(kt + (size_t)slice * m * D);
    Stage<MPAD * D / 8, T> qst, kst;
    stage_load(qst, [&](int i) { return (i < m * D / 8) ? qs[i] : u32x4{0u, 0u, 0u, 0u}; });
    stage_load(kst, [&](int i) { return (i < m * D / 8) ? ks[i] : u32x4{0u, 0u, 0u, 0u}; });
#pragma unroll
    for (int i = 0; i < Stage<MPAD * D / 8, T>::kPer; ++i) {
      const int c = tid + i * T;
      if ((MPAD * D / 8) % T == 0 || c < MPAD * D / 8) {
        const int a = c / (D / 8), k8 = c - a * (D / 8);
        *(u32x4*)(ql + a * RS + 8 * k8) = qst.r[i];
        *(u32x4*)(kl + a * RS + 8 * k8) = kst.r[i];
      }
    }
  }
  // chunk sums in chunk order into the right-hand side columns (element f of a chunk's
  // partial block: tile f / 256 = (jt, dt), slot r * 64 + l); every load of a chunk is in
  // flight at once
  {
    constexpr int EPT = (MPAD * D + T - 1) / T;
    float acc[EPT], z = 0.f;
#pragma unroll
    for (int e = 0; e < EPT; ++e) acc[e] = 0.f;
#pragma unroll 2
    for (int ch = 0; ch < chunks; ++ch) {
      const size_t sc = (size_t)slice * chunks + ch;
      const float* src = part + sc * MPAD * D;
      float v[EPT];
#pragma unroll
      for (int e = 0; e < EPT; ++e) {
        const int f = tid + e * T;
        v[e] = (f < MPAD * D) ? src[f] : 0.f;
      }
      const float dz = (tid < MPAD) ? dpart[sc * MPAD + tid] : 0.f;
#pragma unroll
      for (int e = 0; e < EPT; ++e) acc[e] += v[e];
      z += dz;
    }
#pragma unroll
    for (int e = 0; e < EPT; ++e) {
      const int f = tid + e * T;
      if (f < MPAD * D) {
        const int tile = f >> 8, slot = f & 255, jt = tile / DT, dt = tile - jt * DT;
        const int l = slot & 63, a = 16 * jt + 4 * (l >> 4) + (slot >> 6), k = 16 * dt + (l & 15);
        Mx[a * LD + MPAD + k] = acc[e];
      }
    }
    if (tid < MPAD) zl[tid] = z;
  }
  // F2 logits (fp32 sums of the bf16 products), identity rows and zero columns for padding
  for (int e = tid; e < MPAD * MPAD; e += T) {
    const int a = e / MPAD, l = e - a * MPAD;
    float v;
    if (a < m && l < m) {
      const u32x4* qa = (const u32x4*)(ql + a * RS);
      const u32x4* kb = (const u32x4*)(kl + l * RS);
      v = 0.f;
#pragma unroll
      for (int k8 = 0; k8 < D / 8; ++k8) {
        const bf16x8 x = as_bf16x8(qa[k8]), y = as_bf16x8(kb[k8]);
#pragma unroll
        for (int u = 0; u < 8; ++u) v = fmaf((float)x[u], (float)y[u], v);
      }
    } else {
      v = (a == l && a >= m) ? 1.f : 0.f;
    }
    Mx[a * LD + l] = v;
  }
  __syncthreads();
  // F3 V = P / z (z >= 1: each landmark's largest weight is exp(0)); zero rows for padding
  for (int e = tid; e < MPAD * D; e += T) {
    const int a = e / D, k = e - a * D;
    Mx[a * LD + MPAD + k] = (a < m) ? Mx[a * LD + MPAD + k] / zl[a] : 0.f;
  }
  // row softmax of F2 over the m landmark keys: one wave per row, lanes over the keys
  for (int a = w; a < m; a += NG) {
    float* row = Mx + a * LD;
    float e[RPL], mx = -INFINITY;
#pragma unroll
    for (int i = 0; i < RPL; ++i) {
      const int l = lane + 64 * i;
      e[i] = (l < m) ? row[l] : -INFINITY;
      mx = fmaxf(mx, e[i]);
    }
    mx = xor32_max(xor16_max(row16_max(mx)));
    float z = 0.f;
#pragma unroll
    for (int i = 0; i < RPL; ++i) {
      e[i] = exp2_fast((e[i] - mx) * c2);   // 0 for l >= m
      z += e[i];
    }
    z = xor32_sum(xor16_sum(row16_sum(z)));
    const float iz = 1.f / z;
#pragma unroll
    for (int i = 0; i < RPL; ++i)
      if (lane + 64 * i < m) row[lane + 64 * i] = e[i] * iz;
  }
  __syncthreads();

  float x[RPL][CW];
  bool used[RPL];
  int var[RPL];
#pragma unroll
  for (int i = 0; i < RPL; ++i) {
    const int r = lane + 64 * i;
    used[i] = r >= MPAD;   // lanes past the padded system never pivot
    var[i] = 0;
#pragma unroll
    for (int jj = 0; jj < CW; ++jj) x[i][jj] = (r < MPAD) ? Mx[r * LD + CW * w + jj] : 0.f;
  }

  // Step col: the wave owning column col picks the pivot among the unused rows (largest
  // |value|, smallest row on ties: wave maximum with DPP and permlane swaps, the row from a
  // ballot) and publishes the column, the pivot row and its value through LDS; after one
  // barrier every wave still holding columns >= col takes the pivot row from that lane of
  // its own registers (readlane) and subtracts (x_r[col] / pivot) times it from every other
  // row.  The pivot row is left unscaled (its own factor is zero); unknown col is its
  // right-hand side over the pivot, divided out at the end.  Steps run in groups of CW
  // (the column group W, uniform), unrolled within a group so that register indices are
  // static.
  float pvr[RPL];
#pragma unroll
  for (int i = 0; i < RPL; ++i) pvr[i] = 1.f;
  for (int W = 0; W < MPAD / CW; ++W) {
#pragma unroll
  for (int jc = 0; jc < CW; ++jc) {
    const int col = CW * W + jc, b = jc & 1;
    if (w == W) {
      float v[RPL], best = -1.f;
#pragma unroll
      for (int i = 0; i < RPL; ++i) {
        v[i] = used[i] ? -1.f : fabsf(x[i][jc]);
        best = fmaxf(best, v[i]);
      }
      best = xor32_max(xor16_max(row16_max(best)));
      int bi = MPAD;
#pragma unroll
      for (int i = RPL - 1; i >= 0; --i) {
        const unsigned long long bal = __ballot(v[i] == best);
        if (bal) bi = 64 * i + __builtin_ctzll(bal);
      }
#pragma unroll
      for (int i = 0; i < RPL; ++i) {
        const int r = lane + 64 * i;
        if (r < MPAD) fbuf[b][r] = x[i][jc];
        if (r == bi) pvbuf[b] = x[i][jc];
      }
      if (lane == 0) pbuf[b] = bi;
    }
    __syncthreads();
    if (CW * w + CW - 1 < col) continue;   // this wave's columns are all eliminated
    const int p = __builtin_amdgcn_readfirstlane(pbuf[b]);
    const float pv = pvbuf[b];
    float ipv = __builtin_amdgcn_rcpf(pv);
    ipv = ipv * fmaf(-pv, ipv, 2.f);   // one Newton step
    const int ip = p >> 6, lp = p & 63;
    float f[RPL];
#pragma unroll
    for (int i = 0; i < RPL; ++i) {
      const int r = lane + 64 * i;
      const bool piv = (r == p);
      if (piv) { used[i] = true; var[i] = col; pvr[i] = pv; }
      f[i] = (piv || r >= MPAD) ? 0.f : fbuf[b][r] * ipv;
    }
#pragma unroll
    for (int jj = 0; jj < CW; ++jj) {
      float xv = x[0][jj];
#pragma unroll
      for (int i = 1; i < RPL; ++i) xv = (ip == i) ? x[i][jj] : xv;
      const float pr = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(xv), lp));
#pragma unroll
      for (int i = 0; i < RPL; ++i) x[i][jj] = fmaf(-f[i], pr, x[i][jj]);
    }
  }
  }
  // Z[var][k]: the right-hand-side waves hold unknown var[i] in row lane + 64 i
  if (CW * w >= MPAD) {
    __bf16* dst = Wop + (size_t)slice * MPAD * D;
#pragma unroll
    for (int i = 0; i < RPL; ++i) {
      if (lane + 64 * i >= MPAD) continue;
      const int a = var[i];
#pragma unroll
      for (int jj = 0; jj < CW; ++jj) {
        const int k = CW * w - MPAD + jj;
        dst[w2_layout_index(MP, a, k)] = (__bf16)((a < m) ? x[i][jj] / pvr[i] : 0.f);
      }
    }
  }
}

// ---------------------------------------------------------------------------------------
template <int D, int AT>
static void launch_nys_kernels_t(const Geometry& g, const SplitPlan& p, const NystromBuffers& nb,
                                 const void* Q, const void* K, const int* idx, hipStream_t s,
                                 bool solve) {
  if (!solve) {
    nys_max<D, AT><<<dim3((unsigned)(g.slices * p.chunks1)), dim3(256), 0, s>>>(
        (const __bf16*)Q, (const __bf16*)K, idx, nb.qt, nb.kt, nb.cmax, g.vw.q, g.h, g.n, g.m,
        p.chunks1, p.chunk_len1);
  } else {
    nys_solve<D, AT><<<dim3((unsigned)g.slices), dim3(nys_solve_waves<D, AT>() * kWave), 0, s>>>(
        nb.part, nb.dpart, nb.qt, nb.kt, nb.wop, g.m, p.chunks1, g.c2);
  }
}

template <int D>
static hipError_t launch_nys_t(const Geometry& g, const SplitPlan& p, const NystromBuffers& nb,
                               const void* Q, const void* K, const int* idx, hipStream_t s,
                               bool solve) {
  switch (g.at) {
    case 2: launch_nys_kernels_t<D, 2>(g, p, nb, Q, K, idx, s, solve); break;
    case 4: launch_nys_kernels_t<D, 4>(g, p, nb, Q, K, idx, s, solve); break;
    case 6: launch_nys_kernels_t<D, 6>(g, p, nb, Q, K, idx, s, solve); break;
    case 8: launch_nys_kernels_t<D, 8>(g, p, nb, Q, K, idx, s, solve); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_nystrom_bf16(const Geometry& g, const SplitPlan& p, const void* Q, const void* K,
                               const void* V, const int* idx, void* H, const NystromBuffers& nb,
                               hipStream_t stream) {
  if (g.d != 32 && g.d != 64) return hipErrorInvalidValue;
  auto step = [&](bool solve) {
    return g.d == 64 ? launch_nys_t<64>(g, p, nb, Q, K, idx, stream, solve)
                     : launch_nys_t<32>(g, p, nb, Q, K, idx, stream, solve);
  };
  hipError_t e;
  if ((e = step(false)) != hipSuccess) return e;
  e = launch_nystrom_pass1_bf16(g, p, K, g.vw.q, nb.qt, V, g.vw.v, nb.part, nb.dpart, nb.cmax,
                                stream);
  if (e != hipSuccess) return e;
  if ((e = step(true)) != hipSuccess) return e;
  return launch_nystrom_pass2_bf16(g, p, Q, g.vw.q, nb.kt, nb.wop, H, g.vw.o, stream);
}

}  // namespace aa
