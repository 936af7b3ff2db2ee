// progress.hip -- completion counters: a one-thread kernel that publishes a
// plan's replay counter (advancing it at the first unit of a replay) into a
// host-visible word once the work ahead of it on its stream has finished ("RDMA point-to-point
// communication for LLM systems": memory words updated by GPU kernels and
// polled by the CPU, so a transfer starts as soon as its data exists).
#include <hip/hip_runtime.h>

#include <cstdint>

namespace wt {
namespace {

// Publishes the replay number. Stream order puts this behind the unit's
// kernels and copies; the release store at system scope makes their results
// visible to the host no later than the word itself. The first mark of a
// replay also advances the plan's replay counter (device memory); every
// later mark of the replay runs after it on the same stream, or behind it
// through the stage events.
__global__ void __launch_bounds__(64) progress_mark_kernel(uint64_t *epoch, uint64_t *word, int first) {
  if (threadIdx.x == 0) {
    const uint64_t v = first ? __hip_atomic_fetch_add(epoch, 1ull, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT) + 1
                             : __hip_atomic_load(epoch, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_store(word, v, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_SYSTEM);
  }
}

}  // namespace

hipError_t launch_progress_mark(uint64_t *epoch, uint64_t *word, bool first, hipStream_t stream) {
  hipLaunchKernelGGL(progress_mark_kernel, dim3(1), dim3(64), 0, stream, epoch, word, first ? 1 : 0);
  return hipGetLastError();
}

}  // namespace wt
