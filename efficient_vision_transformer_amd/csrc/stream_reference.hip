// stream_reference.hip -- a measurement helper, not part of the method: the forward's byte
// pattern (two equal buffers read, one written) with no arithmetic beyond an xor, as a
// streaming kernel of many short workgroups (one 16-byte chunk of each buffer per thread,
// non-temporal loads and stores).  Its launch time over the forward's buffers is the
// practical floor for one launch moving those bytes.
#include <hip/hip_runtime.h>

#include "anchor_attn_bench.h"

namespace {

typedef __attribute__((__vector_size__(4 * sizeof(unsigned)))) unsigned u32x4;

__global__ __launch_bounds__(256) void stream_xor(const u32x4* __restrict__ a,
                                                  const u32x4* __restrict__ b,
                                                  u32x4* __restrict__ c, long long n16) {
  const long long i = (long long)blockIdx.x * 256 + threadIdx.x;
  if (i < n16) {
    const u32x4 x = __builtin_nontemporal_load(a + i), y = __builtin_nontemporal_load(b + i);
    __builtin_nontemporal_store(x ^ y, c + i);
  }
}

}  // namespace

extern "C" int anchor_attn_stream_reference(const void* a, const void* b, void* c,
                                            long long bytes_each, void* stream) {
  if (bytes_each < 0 || bytes_each % 16 != 0) return 1;
  if (bytes_each == 0) return 0;
  if (!a || !b || !c || (((uintptr_t)a | (uintptr_t)b | (uintptr_t)c) & 15u)) return 1;
  const long long n16 = bytes_each / 16;
  const long long grid = (n16 + 255) / 256;
  if (grid > 0x7fffffffLL) return 1;
  stream_xor<<<dim3((unsigned)grid), dim3(256), 0, (hipStream_t)stream>>>(
      (const u32x4*)a, (const u32x4*)b, (u32x4*)c, n16);
  return hipGetLastError() == hipSuccess ? 0 : 4;
}
