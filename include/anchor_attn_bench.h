/* anchor_attn_bench.h -- a measurement helper shipped with the library; not part of the
 * method's interface.
 *
 * anchor_attn_stream_reference: c[i] = a[i] ^ b[i] over `bytes_each` bytes of each of
 * three device buffers (two read, one written): the anchor-attention forward's byte
 * pattern (Q and V read, H written) with no arithmetic, as a streaming kernel of one
 * 16-byte chunk per thread.  Timed over the forward's buffer sizes it gives the practical
 * bandwidth floor of one launch moving those bytes.  Enqueued on `stream` (a hipStream_t,
 * NULL = default stream); returns without waiting.
 * Arguments: device pointers, 16-byte aligned, c not overlapping a or b; bytes_each a
 * multiple of 16 (0 is a no-op).  Returns 0 on success, 1 for invalid arguments (nothing
 * enqueued), 4 when the launch fails. */
#ifndef ANCHOR_ATTN_BENCH_H
#define ANCHOR_ATTN_BENCH_H

#ifdef __cplusplus
extern "C" {
#endif

int anchor_attn_stream_reference(const void* a, const void* b, void* c, long long bytes_each,
                                 void* stream);

#ifdef __cplusplus
}
#endif

#endif /* ANCHOR_ATTN_BENCH_H */
