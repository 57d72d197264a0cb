// kernels.h -- internal launch interface between the C ABI and the HIP kernels.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>

#include "geometry.h"

namespace aa {

hipError_t launch_split_bf16(const Geometry& g, const SplitPlan& p, const void* Q,
                             const void* U, const void* V, void* H, void* workspace,
                             hipStream_t stream);
// Split pass 1 alone on (Q, U, X): per-chunk partials of A^T X and of the column sums of
// A, in the layout the finalize kernels read (used by the backward with X = V and
// X = dH).
hipError_t launch_pass1_bf16(const Geometry& g, const SplitPlan& p, const void* Q, const void* U,
                             const void* X, float* part, float* dpart, hipStream_t stream);
// The backward's pass 1 on V (view vw) and on G (view gw) in one launch, up to 256 anchors
// at d <= 64 and 96 at d = 128: A formed once, A^T V and Delta into part / dpart, A^T G
// into partG.
hipError_t launch_pass1_dual_bf16(const Geometry& g, const SplitPlan& p, const void* Q,
                                  const void* U, const void* V, const View& vw, const void* G,
                                  const View& gw, float* part, float* partG, float* dpart,
                                  float* lse, hipStream_t s);
// Workspace sections of the backward (see bwd_finalize / bwd_tokens).
struct BackwardBuffers {
  float* partP;   // pass-1 partials of A^T V      [slice][chunk][AT][DT][256]
  float* partG;   // pass-1 partials of A^T dH     [slice][chunk][AT][DT][256]
  float* dpart;   // pass-1 partials of Delta      [slice][chunk][16 AT]
  void* wu;       // W, logits-layout operands     [slice][AT][KS][64] x 16 B
  void* dprm;     // dP, row-major bf16            [slice][m_pad][d]
  float* dd;      // dDelta                        [slice][16 AT]
  float* partU;   // partials of dS^T Q            [slice][chunk_t][AT][DT][256]
  float* lse;     // log-sum-exp (base 2) per token [slice][n], above 128 anchors
  int chunks_t, chunk_len_t;   // the token pass's chunks (at most pass 1's)
};
// Views of the backward's tensors: Q, V, dH (inputs) and dQ, dV (outputs).
struct BwdViews {
  View q, v, g, dq, dv;
};
// Zeroes `bytes` (a multiple of 4) with a fill kernel (safe under stream capture).
hipError_t launch_zero(void* p, size_t bytes, hipStream_t stream);
// Domain of the split backward: up to 256 anchors at d = 32 or 64, up to 128 at d = 128.
bool bwd_split_supported(const Geometry& g);
hipError_t launch_backward_bf16(const Geometry& g, const SplitPlan& p, const BackwardBuffers& wb,
                                const BwdViews& bv, const void* Q, const void* U, const void* V,
                                const void* G, void* dQ, void* dU, void* dV, hipStream_t stream);
// fp32 split pass 1 alone on (Q, U, X), partials as launch_pass1_bf16's.
hipError_t launch_pass1_fp32(const Geometry& g, const SplitPlan& p, const void* Q, const void* U,
                             const void* X, float* part, float* dpart, hipStream_t stream);
// The fp32 backward's pass 1 on V and on G in one launch (d <= 64): A formed once.
hipError_t launch_pass1_dual_fp32(const Geometry& g, const SplitPlan& p, const void* Q,
                                  const void* U, const void* V, const View& vw, const void* G,
                                  const View& gw, float* part, float* partG, float* dpart,
                                  hipStream_t s);
// Workspace sections of the fp32 backward (see backward_fp32.hip).
struct BackwardBuffersF32 {
  float* partP;   // pass-1 partials of A^T V      [slice][chunk][AT][DT][256]
  float* partG;   // pass-1 partials of A^T dH     [slice][chunk][AT][DT][256]
  float* dpart;   // pass-1 partials of Delta      [slice][chunk][16 AT]
  float* wrm;     // W, row-major                  [slice][m_pad][d]
  float* dprm;    // dP, row-major                 [slice][m_pad][d]
  float* dd;      // dDelta                        [slice][m_pad]
  float* ds;      // dS rows                       [slice][n][m_pad]
  float* partU;   // partials of dS^T Q            [slice][chunk][AT][DT][256]
};
// Domain of the fp32 backward: d = 32 or 64, up to 256 anchors.
bool bwd_fp32_supported(const Geometry& g);
hipError_t launch_backward_fp32(const Geometry& g, const SplitPlan& p,
                                const BackwardBuffersF32& wb, const BwdViews& bv, const void* Q,
                                const void* U, const void* V, const void* G, void* dQ, void* dU,
                                void* dV, hipStream_t stream);
// dU = (1/sqrt(d)) x the sum over batch and chunks of per-(slice, chunk) partial tiles
// [slice][chunk][AT][DT][256] of dS^T Q.
hipError_t launch_du_reduce_bf16(const Geometry& g, const float* partU, int chunks, void* dU,
                                 hipStream_t stream);
// Short-sequence backward: one workgroup per slice (n <= 1024, m <= 64, d = 32 or 64),
// then the dU reduction; partU holds slices x m_pad x d floats.
bool bwd_fused_supported(const Geometry& g);
hipError_t launch_backward_fused_bf16(const Geometry& g, const BwdViews& bv, const void* Q,
                                      const void* U, const void* V, const void* G, void* dQ,
                                      void* dU, void* dV, float* partU, hipStream_t stream);
// Projections of the attention block (hipBLASLt): D[T, N] = X[T, K] W[K, N] + bias[N],
// row-major bf16, fp32 accumulation; bias may be null.  gemm_prepare finds descriptors
// and an algorithm for a shape (false: none), gemm_run enqueues with a workspace of
// kGemmWorkspaceBytes.
constexpr size_t kGemmWorkspaceBytes = size_t(32) << 20;
struct GemmCache;
GemmCache* gemm_cache_create();
void gemm_cache_destroy(GemmCache* c);
bool gemm_prepare(GemmCache* c, long long T, int K, int N, bool bias);
hipError_t gemm_run(GemmCache* c, const void* X, const void* W, const void* bias, void* D,
                    long long T, int K, int N, void* ws, hipStream_t stream);
// The attention block with the Q|V projection fused in front of the layer (bf16): one
// workgroup per slice projects X [B, n, C] with its head's columns of Wqv [C, 2C] (+ bqv,
// may be null) and writes H [B, n, C] (head-major columns).  d = 32 or 64 with A kept in
// registers, one round of eight waves: m <= 32 and n <= 256.
bool block_fused_supported(const Geometry& g);
hipError_t launch_block_fused_bf16(const Geometry& g, const void* X, const void* Wqv,
                                   const void* bqv, const void* U, void* H, hipStream_t stream);
// ReLU kernel linear attention, one workgroup per slice (bf16, d = 32 or 64): out =
// phi(Q) (phi(K)^T V) / max(phi(Q) phi(K)^T 1, cmin) on strided views.
hipError_t launch_relu_linear_bf16(const Geometry& g, const void* Q, const View& qw, const void* K,
                                   const View& kw, const void* V, const View& vw, void* O,
                                   const View& ow, float cmin, int num_cus, hipStream_t stream);
// Split plan of the linear attention: pass 1 over chunks1 chunks of chunk_len1 tokens
// writes partial S tiles and z; finalize sums them; pass 2 applies over chunks2 chunks.
struct LinearSplitPlan {
  int chunks1, chunk_len1, chunks2, chunk_len2;
  size_t part_bytes, zpart_bytes, sop_bytes, z_bytes;
  size_t workspace_bytes() const { return part_bytes + zpart_bytes + sop_bytes + z_bytes; }
};
hipError_t launch_relu_linear_split_bf16(const Geometry& g, const LinearSplitPlan& p, const void* Q,
                                         const View& qw, const void* K, const View& kw,
                                         const void* V, const View& vw, void* O, const View& ow,
                                         float cmin, void* workspace, hipStream_t stream);
hipError_t launch_split_fp32(const Geometry& g, const SplitPlan& p, const void* Q,
                             const void* U, const void* V, void* H, void* workspace,
                             hipStream_t stream);
bool fused_supported(const Geometry& g, int num_cus, FusedPlan* plan);
hipError_t launch_fused_bf16(const Geometry& g, const FusedPlan& p, const void* Q,
                             const void* U, const void* V, void* H, hipStream_t stream);

// Nystrom attention (bf16, landmarks s = Geometry::m <= 128): workspace pieces.
struct NystromBuffers {
  float* part;    // pass-1 partials of F3 V (unnormalised)  [slice][chunk][AT][DT][256]
  float* dpart;   // pass-1 partials of F3's row sums        [slice][chunk][16 AT]
  __bf16* wop;    // Z = F2^-1 F3 V as pass-2 W operands      [slice][DT][MP][64][8]
  __bf16* kt;     // landmark rows of K (written by the solve) [slice][s][d]
  float* cmax;    // per-chunk landmark maxima of q.k         [slice][chunk][16 AT]
};
hipError_t launch_nystrom_bf16(const Geometry& g, const SplitPlan& p, const void* Q, const void* K,
                               const void* V, const int* idx, void* H, const NystromBuffers& nb,
                               hipStream_t stream);
hipError_t launch_nystrom_pass1_bf16(const Geometry& g, const SplitPlan& p, const void* K,
                                     const View& kw, const void* Q, const View& qw,
                                     const int* idx, const void* V, const View& vw, float* part,
                                     float* dpart, float* cmax, hipStream_t s);
hipError_t launch_nystrom_pass2_bf16(const Geometry& g, const SplitPlan& p, const void* Q,
                                     const View& qw, const void* kt, const void* Wop, void* H,
                                     const View& ow, hipStream_t s);

}  // namespace aa
