// Device-side contract check of the arrays a write or decode call reads
// (pa_check_inputs).  The attention and write kernels stay inside the pools
// whatever the slot mapping, block tables and lengths hold -- they skip or
// clamp -- but silently; these kernels report.  They read the arrays only,
// never the pools, and check every index they form before using it.
//
// Report: report[0] counts violations; while the kernels run, report[2..3]
// hold the 64-bit key (kind << 40 | index) of the first one, kept by atomic
// minimum; the last kernel turns the key into kind, index and value.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdint>

#include "pa_kernels.h"

namespace pa {

namespace {

constexpr int kCheckThreads = 256;
constexpr int kKindShift = 40;

__device__ inline void record(const CheckArgs& a, int kind, int64_t index) {
  atomicAdd(a.report, 1);
  atomicMin(reinterpret_cast<unsigned long long*>(a.report + 2),
            (static_cast<unsigned long long>(kind) << kKindShift) |
                static_cast<unsigned long long>(index));
}

__global__ __launch_bounds__(kCheckThreads) void check_clear_kernel(CheckArgs a) {
  const int64_t i = int64_t(blockIdx.x) * kCheckThreads + threadIdx.x;
  if (i == 0) {
    a.report[0] = 0;
    a.report[1] = 0;
    *reinterpret_cast<unsigned long long*>(a.report + 2) = ~0ull;
  }
  if (a.seen)
    for (int64_t w = i; w < a.bitmap_words; w += int64_t(gridDim.x) * kCheckThreads) {
      a.seen[w] = 0;
      a.dup[w] = 0;
    }
}

// slots: out of range, or (with the bitmaps) seen before: mark the slot as
// duplicated; the tokens of a duplicated slot are all flagged by the next pass
__global__ __launch_bounds__(kCheckThreads) void check_slots_kernel(CheckArgs a) {
  const int64_t n = int64_t(blockIdx.x) * kCheckThreads + threadIdx.x;
  if (n >= a.num_tokens) return;
  const int32_t s = a.slots[n];
  if (s < 0) return;
  if (int64_t(s) >= a.num_slots) {
    record(a, PA_CHECK_SLOT_RANGE, n);
    return;
  }
  if (a.seen) {
    const uint32_t bit = 1u << (s & 31);
    if (atomicOr(a.seen + (s >> 5), bit) & bit) atomicOr(a.dup + (s >> 5), bit);
  }
}

__global__ __launch_bounds__(kCheckThreads) void check_dups_kernel(CheckArgs a) {
  const int64_t n = int64_t(blockIdx.x) * kCheckThreads + threadIdx.x;
  if (n >= a.num_tokens) return;
  const int32_t s = a.slots[n];
  if (s < 0 || int64_t(s) >= a.num_slots) return;
  if (a.dup[s >> 5] & (1u << (s & 31))) record(a, PA_CHECK_SLOT_DUP, n);
}

// one workgroup per sequence: its length, then the table entries the
// kernels would read for the clamped length
__global__ __launch_bounds__(kCheckThreads) void check_tables_kernel(CheckArgs a) {
  const int i = blockIdx.x;
  const int32_t T = a.lens[i];
  if (threadIdx.x == 0 && (T < 0 || T > a.max_len)) record(a, PA_CHECK_LENGTH, i);
  const int32_t Tc = T < 0 ? 0 : (T > a.max_len ? a.max_len : T);
  const int nb = min(a.max_blocks, (Tc + (1 << a.log2_block) - 1) >> a.log2_block);
  for (int j = threadIdx.x; j < nb; j += kCheckThreads) {
    const int64_t at = int64_t(i) * a.max_blocks + j;
    const int32_t e = a.tables[at];
    if (e < 0 || e >= a.num_blocks) record(a, PA_CHECK_TABLE, at);
  }
}

__global__ void check_finish_kernel(CheckArgs a) {
  const unsigned long long key = *reinterpret_cast<unsigned long long*>(a.report + 2);
  if (a.report[0] == 0) {
    a.report[1] = 0;
    a.report[2] = 0;
    a.report[3] = 0;
    return;
  }
  const int kind = int(key >> kKindShift);
  const int64_t index = int64_t(key & ((1ull << kKindShift) - 1));
  const int32_t value = kind == PA_CHECK_LENGTH  ? a.lens[index]
                        : kind == PA_CHECK_TABLE ? a.tables[index]
                                                 : a.slots[index];
  a.report[1] = kind;
  a.report[2] = int32_t(index);
  a.report[3] = value;
}

}  // namespace

hipError_t launch_check(const CheckArgs& a, hipStream_t stream) {
  const int64_t clear_blocks =
      a.seen ? std::min<int64_t>((a.bitmap_words + kCheckThreads - 1) / kCheckThreads, 4096) : 1;
  hipLaunchKernelGGL(check_clear_kernel, dim3(uint32_t(std::max<int64_t>(clear_blocks, 1))),
                     dim3(kCheckThreads), 0, stream, a);
  if (a.slots && a.num_tokens > 0) {
    const dim3 grid(uint32_t((int64_t(a.num_tokens) + kCheckThreads - 1) / kCheckThreads));
    hipLaunchKernelGGL(check_slots_kernel, grid, dim3(kCheckThreads), 0, stream, a);
    if (a.seen) hipLaunchKernelGGL(check_dups_kernel, grid, dim3(kCheckThreads), 0, stream, a);
  }
  if (a.tables && a.lens && a.num_seqs > 0)
    hipLaunchKernelGGL(check_tables_kernel, dim3(uint32_t(a.num_seqs)), dim3(kCheckThreads), 0,
                       stream, a);
  hipLaunchKernelGGL(check_finish_kernel, dim3(1), dim3(1), 0, stream, a);
  return hipGetLastError();
}

}  // namespace pa
