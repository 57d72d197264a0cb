// geometry.h -- the problem geometry, tensor views and launch plans shared by the C ABI
// and the kernels (the parts of the launch interface that kernel code reads).
#pragma once
#include <stddef.h>

namespace aa {

// Element strides (batch, head, token) of a [B, h, n, d] view whose d values per token are
// contiguous; the contiguous layout is (h*n*d, n*d, d).  Strides are non-negative
// multiples of 16 bytes, so every row is a whole number of 16-byte vectors.
struct View {
  long long sb, sh, st;
};
// The views of one forward call: Q and V (inputs) and H (output).
struct Views {
  View q, v, o;
};

// Problem geometry of one call.  Q, V, H: [B, h, n, d] views; U: [h, m, d] contiguous.
struct Geometry {
  int B, h, n, m, d;
  int m_pad;          // m rounded up to a multiple of 32
  int at;             // anchor tiles of 16: m_pad / 16
  long long slices;   // B * h
  float c2;           // log2(e) / sqrt(d): logits are kept in base-2 units
  Views vw;           // strides of Q, V, H (contiguous unless the caller gives others)
};

// Split plan: pass 1 over chunks1 chunks of chunk_len1 tokens per slice writes
// partials (and each token's log-sum-exp); finalize reduces them; pass 2 over chunks2
// chunks writes H.
struct SplitPlan {
  int chunks1, chunk_len1;
  int chunks2, chunk_len2;
  size_t part_bytes, dpart_bytes, w_bytes, lse_bytes;   // workspace sections, in order
  size_t workspace_bytes() const { return part_bytes + dpart_bytes + w_bytes + lse_bytes; }
};

// Fused plan: one workgroup per slice, everything on chip.
struct FusedPlan {
  int waves;          // waves per workgroup
  int pairs_per_wave; // 32-token pairs handled by each wave
  bool keep_a;        // A kept in registers (else recomputed from Q for the output)
  long long shared;   // slices handled by two workgroups (one per half of the output dims)
};

constexpr int kPass1Waves = 4;    // pass 1 block = 4 pairs = 128 tokens
constexpr int kPass1Block = 128;
constexpr int kPass2Waves = 4;    // pass 2 block = 4 tiles = 64 tokens
constexpr int kPass2Block = 64;

}  // namespace aa
