// Work queues of the persistent kernels (forward, query-major and KV-major
// backward): eight counters per kernel launch, one per XCD, cleared by a
// kernel on the launch stream (no memset, so a captured graph can replay the
// sequence).  The device side, queue_take, is in msa_device.h.
#include "msa_device.h"
#include "msa_internal.h"

namespace msa {
namespace {

__global__ void queue_reset_kernel(int32_t* queue) {
  if (threadIdx.x < kQueues) queue[threadIdx.x * kQueueStride] = 0;
}

}  // namespace

hipError_t launch_queue_reset(int32_t* queue, hipStream_t s) {
  hipLaunchKernelGGL(queue_reset_kernel, dim3(1), dim3(64), 0, s, queue);
  return hipGetLastError();
}

}  // namespace msa
