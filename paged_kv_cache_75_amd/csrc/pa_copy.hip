// Whole-block copy for copy-on-write ("vLLM Framework and Inference Engine
// Design", section "What operations can cause memory fragmentation, and how
// does vLLM avoid it?": a shared block is copied only when a sequence must
// write into it).  A block of one pool is block_bytes contiguous bytes, so a
// pair is a plain contiguous copy; one launch covers up to kCopyMaxPools
// pools (grid y), whose pointers travel in the kernel arguments.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "pa_kernels.h"
#include "pa_launch.h"

namespace pa {

namespace {

constexpr int kCopyThreads = 256;
constexpr int kCopyVecs = int(kCopyChunkBytes / (16 * kCopyThreads));

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

// Workgroup (x, y) moves chunk x % chunks of pair x / chunks in pool y.  In a
// whole chunk each thread issues its four 16-byte loads before its stores, so
// a workgroup keeps 16 KiB in flight; the last, partial chunk of a block
// copies one vector at a time.  Loads and stores are non-temporal: every byte
// is touched once, and streaming it past the caches measured faster (the
// copy runs at the speed of a device-to-device memcpy of the same size).
__global__ __launch_bounds__(kCopyThreads) void copy_blocks_kernel(CopyArgs a) {
  const int pair = blockIdx.x / a.chunks;
  const int chunk = blockIdx.x - pair * a.chunks;
  const int32_t src = a.mapping[2 * pair];
  const int32_t dst = a.mapping[2 * pair + 1];
  if (src < 0 || src >= a.num_blocks || dst < 0 || dst >= a.num_blocks) return;
  char* pool = a.pools[blockIdx.y];
  const u32x4* from = reinterpret_cast<const u32x4*>(pool + int64_t(src) * a.block_bytes);
  u32x4* to = reinterpret_cast<u32x4*>(pool + int64_t(dst) * a.block_bytes);
  const int64_t vecs = a.block_bytes / 16;
  const int64_t first = int64_t(chunk) * (kCopyThreads * kCopyVecs);
  if (first + kCopyThreads * kCopyVecs <= vecs) {
    // a whole chunk (the same branch for the whole workgroup); four named
    // registers: an array here is turned into LDS by the compiler
    static_assert(kCopyVecs == 4, "one register per vector below");
    const int64_t i = first + threadIdx.x;
    const u32x4 v0 = __builtin_nontemporal_load(from + i);
    const u32x4 v1 = __builtin_nontemporal_load(from + i + kCopyThreads);
    const u32x4 v2 = __builtin_nontemporal_load(from + i + 2 * kCopyThreads);
    const u32x4 v3 = __builtin_nontemporal_load(from + i + 3 * kCopyThreads);
    __builtin_nontemporal_store(v0, to + i);
    __builtin_nontemporal_store(v1, to + i + kCopyThreads);
    __builtin_nontemporal_store(v2, to + i + 2 * kCopyThreads);
    __builtin_nontemporal_store(v3, to + i + 3 * kCopyThreads);
  } else {
    for (int64_t i = first + threadIdx.x; i < vecs; i += kCopyThreads)
      __builtin_nontemporal_store(__builtin_nontemporal_load(from + i), to + i);
  }
}

}  // namespace

hipError_t launch_copy_blocks(const CopyArgs& a, int32_t num_pairs, int32_t num_pools,
                              hipStream_t stream) {
  if (num_pairs == 0 || num_pools == 0) return hipSuccess;
  launch_timed(copy_blocks_kernel, dim3(num_pairs * a.chunks, num_pools), dim3(kCopyThreads),
               stream, a);
  return hipGetLastError();
}

}  // namespace pa
