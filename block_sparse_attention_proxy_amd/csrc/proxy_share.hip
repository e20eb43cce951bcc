// One proxy head shared by every KV group (msa_config.proxy_heads = 1).
//
// The pages let the block pattern and the proxy be configured (keelcrux
// "Flash-MSA: Ein Training mit einer Million Tokens", Under the hood); with
// one proxy head its block choice serves every query head, and the proxy
// gradient's target T is the mean of the main probabilities over all query
// heads.  Scoring and selection run once, for the one head; the forward and
// backward kernels of every KV group read the one head's inputs, block lists
// and log-sum-exp directly.  Each group writes its own proxy gradient, in
// which only group 0 carries the proxy-softmax term Q (with weight Hkv) and
// every group its -T_g; the mean over the groups below is then the gradient
// of the shared head: the all-heads T is the mean of the group means, and
// the proxy gradients are linear in T.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "msa_internal.h"
#include "msa_profile.h"

namespace msa {

// dst[r][w] = scale * sum over c (in order) of src[r][c][w]
__global__ __launch_bounds__(256) void group_mean_kernel(const float* __restrict__ src,
                                                         float* __restrict__ dst, int64_t rows,
                                                         int copies, int64_t words, float scale) {
  const int64_t n = rows * words;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
       i += (int64_t)gridDim.x * blockDim.x) {
    const int64_t r = i / words, w = i % words;
    const float* p = src + r * copies * words + w;
    float acc = 0.f;
    for (int c = 0; c < copies; ++c) acc += p[c * words];
    dst[i] = acc * scale;
  }
}

static unsigned grid_for(int64_t n) {
  int64_t b = (n + 255) / 256;
  return (unsigned)(b < 1 ? 1 : (b > 65536 ? 65536 : b));
}

hipError_t launch_group_mean(const float* src, float* dst, int64_t rows, int copies, int64_t words,
                             hipStream_t s) {
  if (rows <= 0 || words <= 0) return hipSuccess;
  { ProfScope _ps("share_mean", s);
  hipLaunchKernelGGL(group_mean_kernel, dim3(grid_for(rows * words)), dim3(256), 0, s, src, dst, rows,
                     copies, words, 1.f / (float)copies); }
  return hipGetLastError();
}

int share_kernels(KernelEntry* out, int max) {
  const KernelEntry all[] = {
      {"share_mean", (const void*)group_mean_kernel, 256, 0},
  };
  int n = (int)(sizeof(all) / sizeof(all[0]));
  for (int i = 0; i < n && i < max; ++i) out[i] = all[i];
  return n;
}

}  // namespace msa
