// progress.hip -- completion counters: one-thread kernels that advance a
// plan's replay counter and publish it into host-visible words once the work
// ahead of them on their stream has finished ("RDMA point-to-point
// communication for LLM systems": memory words updated by GPU kernels and
// polled by the CPU, so a transfer starts as soon as its data exists).
#include <hip/hip_runtime.h>

#include <cstdint>

namespace wt {
namespace {

// Replay counter in device memory: +1 at the start of every replay.
__global__ void __launch_bounds__(64) progress_begin_kernel(uint64_t *epoch) {
  if (threadIdx.x == 0) __hip_atomic_fetch_add(epoch, 1ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Publishes the current replay number. Stream order puts this behind the
// unit's kernels and copies; the release store at system scope makes their
// results visible to the host no later than the word itself.
__global__ void __launch_bounds__(64) progress_mark_kernel(const uint64_t *epoch, uint64_t *word) {
  if (threadIdx.x == 0) {
    const uint64_t v = __hip_atomic_load(epoch, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_store(word, v, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_SYSTEM);
  }
}

}  // namespace

hipError_t launch_progress_begin(uint64_t *epoch, hipStream_t stream) {
  hipLaunchKernelGGL(progress_begin_kernel, dim3(1), dim3(64), 0, stream, epoch);
  return hipGetLastError();
}

hipError_t launch_progress_mark(const uint64_t *epoch, uint64_t *word, hipStream_t stream) {
  hipLaunchKernelGGL(progress_mark_kernel, dim3(1), dim3(64), 0, stream, epoch, word);
  return hipGetLastError();
}

}  // namespace wt
