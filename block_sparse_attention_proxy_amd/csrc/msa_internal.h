// Internal interface between the C-ABI layer (msa_api.cpp) and the kernel
// launchers (*.hip).  Not installed; not part of the public header.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>
#include <initializer_list>
#include <utility>

namespace msa {

// Raises the dynamic-LDS limit of a set of kernels once per device (the first
// launch on each device does it; later launches skip it).  Thread-safe: a
// race only repeats the idempotent attribute call.  Devices past the table
// size are handled on every call.
struct LdsLimitOnce {
  static constexpr int MAX_DEV = 64;
  std::atomic<unsigned char> done[MAX_DEV] = {};
  hipError_t ensure(std::initializer_list<std::pair<const void*, int>> kernels) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    const bool cached = dev >= 0 && dev < MAX_DEV;
    if (cached && done[dev].load(std::memory_order_acquire)) return hipSuccess;
    for (const auto& k : kernels) {
      e = hipFuncSetAttribute(k.first, hipFuncAttributeMaxDynamicSharedMemorySize, k.second);
      if (e != hipSuccess) return e;
    }
    if (cached) done[dev].store(1, std::memory_order_release);
    return hipSuccess;
  }
};

// Compute units of the current device, read once per device.
inline hipError_t device_cu_count(int* n) {
  static constexpr int MAX_DEV = 64;
  static std::atomic<int> cache[MAX_DEV] = {};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  const bool cached = dev >= 0 && dev < MAX_DEV;
  if (cached && (*n = cache[dev].load(std::memory_order_relaxed)) > 0) return hipSuccess;
  e = hipDeviceGetAttribute(n, hipDeviceAttributeMultiprocessorCount, dev);
  if (e != hipSuccess) return e;
  if (*n < 1) return hipErrorInvalidDevice;
  if (cached) cache[dev].store(*n, std::memory_order_relaxed);
  return hipSuccess;
}

// Geometry of one call, resolved on the host and passed to every kernel by value.
struct Geo {
  int32_t Hq, Hkv, G, D, DP;
  int32_t Bq, topk, lw, stride;      // stride = topk + local_window
  int32_t dil, span;                 // window dilation, span = lw * dil
  int32_t B, T, nqb, nkb;            // documents, tokens, total query / KV blocks
  int32_t max_nq;                    // largest per-document query-block count
  int64_t cap;                       // k2q capacity per group = nqb * stride
  int64_t score_elems;               // per group
  int32_t n_units;                   // proxy-scoring units (pairs of 128-row tiles)
  int32_t nslab;                     // column slabs (K2Q_SLAB blocks) of the inverted index, per group
  int32_t k2q_chunks;                // 256-row chunks per slab (the most any slab needs)
  int32_t Hp;                        // proxy heads of qp, kp, lse_p and the block lists: Hkv, or 1
                                     // for one head shared by every KV group
  float scale, pscale, lam;          // softmax scale, proxy scale, proxy loss weight
  float scale_log2, pscale_log2;     // scale * log2(e), pscale * log2(e)
  const int32_t* cu;                 // device cu_seqlens [B + 1]
  // per-document tables written by the metadata kernel into the workspace
  int32_t* qb0;                      // [B + 1] first global query block
  int32_t* kb0;                      // [B + 1] first global KV block
  int64_t* s0;                       // [B + 1] score-rectangle offset
  int32_t* order;                    // [B]     documents by length, longest first
  int32_t* unit0;                    // [B + 1] first scoring unit, in that order
  int32_t* qdoc;                     // [nqb] document of each global query block
  int32_t* kdoc;                     // [nkb] document of each global KV block
  int32_t* slab0;                    // [B + 1] first column slab of each document
};

// The proxy head a KV group reads (its own, or the one shared head), and the
// weight of the proxy-softmax term Q in that group's proxy gradient.  With a
// shared head the per-group gradients lam (Q - T_g) are averaged over the
// groups afterwards, so Q is taken once, in group 0, with weight Hkv, and the
// other groups contribute only their -T_g.
__host__ __device__ __forceinline__ int proxy_head(const Geo& g, int grp) { return g.Hp == 1 ? 0 : grp; }
__host__ __device__ __forceinline__ float proxy_qweight(const Geo& g, int grp) {
  // an integer first, converted once: the float then depends on grp and is
  // formed where it is used
  return (float)(g.Hp == g.Hkv ? 1 : (grp == 0 ? g.Hkv : 0));
}

// The contiguous range of n items that XCD x (or its queue) serves: n / 8
// items, one more for the first n % 8 XCDs; xcd_first(x, n) is its start.
constexpr int kXcds = 8;
__host__ __device__ __forceinline__ int xcd_first(int x, int n) {
  const int per = n / kXcds, rem = n % kXcds;
  return x * per + (x < rem ? x : rem);
}

// Work queues of the persistent kernels: one set of counters per kernel,
// kQueues of them (one per XCD) kQueueStride words (64 bytes) apart; the
// workspace holds kQueueSets sets.
constexpr int kQueues = kXcds, kQueueStride = 16, kQueueWords = kQueues * kQueueStride;
constexpr int kQueueSets = 3;                       // query-major, KV-major, forward
// Work queues of the persistent kernels: kQueues counters, one per XCD,
// kQueueStride words (64 bytes) apart; queue x serves a contiguous range of
// the n items (the first n % kQueues queues one item more).  The calling
// thread takes the next item of queue `home` (its workgroup's XCD) and, once
// that is empty, of the others in turn; `drained` counts the queues it has
// found empty and is kept by the caller between calls.  Returns -1 once every
// queue is empty, so a loop over queue_take ends on every workgroup.
__device__ __forceinline__ int queue_take(int32_t* queue, int n, int home, int& drained) {
  while (drained < kQueues) {
    const int x = (home + drained) % kQueues;
    const int first = xcd_first(x, n), size = xcd_first(x + 1, n) - first;
    if (size > 0) {
      const int c = atomicAdd(queue + x * kQueueStride, 1);
      if (c < size) return first + c;
    }
    ++drained;
  }
  return -1;
}

// Logical id of workgroup i of an n-workgroup grid launched one per item:
// workgroups are dealt round-robin to the XCDs, so XCD i mod kQueues gets the
// contiguous range of ids that queue would serve (neighbours share its L2).
__device__ __forceinline__ int xcd_remap(int i, int n) { return xcd_first(i % kQueues, n) + i / kQueues; }

// Workspace regions (byte offsets are computed by the host layout routine).
struct Work {
  int32_t* counts;                   // [Hkv * nslab * k2q_chunks * 64] selections per (slab, chunk, block)
  int32_t* totals;                   // [Hkv * nkb] selections per KV block
  float* delta;                      // [Hq * T]       rowsum(dO * O)
  float* lse2;                       // [Hq * T]       main LSE in log2 units
  float* lsep2;                      // [Hkv * T]      proxy LSE in log2 units
  float* cpart;                      // [Hkv * nhg * T * DP] proxy-gradient partials (G > 4)
  int32_t* queue;                    // [kQueueSets][kQueueWords] work-queue counters of the
                                     // query-major pass, the KV-major pass and the forward
};

// Inverted-index build: KV blocks of a document are taken in slabs of this
// many, the rows that can select a slab in chunks of 256.
constexpr int K2Q_SLAB = 256;
constexpr int K2Q_CHUNK = 256;

// Scratch of the allocation-free selection entry point: a file-scope device
// array of this many bytes per GPU.  noalloc_scratch() returns the current
// device's address of it (looked up once per device).
constexpr size_t kNoAllocScratchBytes = size_t(16) << 20;
hipError_t noalloc_scratch(void** ptr);

hipError_t launch_meta(const Geo& g, hipStream_t s);
// clears one set of work-queue counters (kQueues of them, 64 bytes apart)
hipError_t launch_queue_reset(int32_t* queue, hipStream_t s);
// shared proxy head: the in-order average over copies of fp32 rows
hipError_t launch_group_mean(const float* src, float* dst, int64_t rows, int copies, int64_t words,
                             hipStream_t s);
hipError_t launch_proxy_scores(const Geo& g, int is_bf16, const void* qp, const void* kp,
                               float* scores, hipStream_t s);
hipError_t launch_select(const Geo& g, const float* scores, int32_t* q2k_idx, int32_t* q2k_cnt,
                         int32_t* k2q_ptr, int32_t* k2q_idx, const Work& w, hipStream_t s);
// (gp: the proxy heads' geometry, Hkv = Hp, for the proxy log-sum-exp)
hipError_t launch_fwd(const Geo& g, const Geo& gp, int is_bf16, const void* q, const void* k, const void* v,
                      const void* qp, const void* kp, const int32_t* q2k_idx,
                      const int32_t* q2k_cnt, void* o, float* lse, float* lse_p, int32_t* queue,
                      hipStream_t s);
hipError_t launch_bwd(const Geo& g, int is_bf16, const void* q, const void* k, const void* v,
                      const void* qp, const void* kp, const void* o, const float* lse,
                      const float* lse_p, const void* dout, const int32_t* q2k_idx,
                      const int32_t* q2k_cnt, const int32_t* k2q_ptr, const int32_t* k2q_idx,
                      float* dq, float* dk, float* dv, float* dqp, float* dkp, const Work& w,
                      hipStream_t s);

// KV-major backward for bf16, d = 128, dp = 64 and 2, 4 or 8 heads per group
// (the software-pipelined kernel); other shapes use the generic kernel.
bool dkdv128_supported(const Geo& g);
hipError_t launch_dkdv128(const Geo& g, const void* q, const void* k, const void* v,
                          const void* qp, const void* kp, const float* lse2, const float* lsep2,
                          const void* dout, const float* delta, const int32_t* k2q_ptr,
                          const int32_t* k2q_idx, float* dk, float* dv, float* dkp, int32_t* queue,
                          hipStream_t s);

// Query-major backward for bf16, d = 128, dp = 64 and 1, 2, 4 or 8 heads per
// group (eight waves of 32 queries, two per SIMD); other shapes use the
// generic kernel.  Writes D and both LSEs in log2 units for the KV-major pass.
bool dq128_supported(const Geo& g);
hipError_t launch_dq128(const Geo& g, const void* q, const void* k, const void* v, const void* qp,
                        const void* kp, const void* o, const float* lse, const float* lse_p,
                        const void* dout, float* delta, float* lse2, float* lsep2,
                        const int32_t* q2k_idx, const int32_t* q2k_cnt, float* dq, float* dqp,
                        int32_t* queue, hipStream_t s);

// Kernel registry for the resource report: each translation unit lists the
// kernels it instantiates, with the block size and dynamic LDS of its launch.
struct KernelEntry {
  const char* name;
  const void* fn;
  int block;
  int dyn_lds;
};
int select_kernels(KernelEntry* out, int max);
int share_kernels(KernelEntry* out, int max);
int fwd_kernels(KernelEntry* out, int max);
int bwd_kernels(KernelEntry* out, int max);
int bwd_kv_kernels(KernelEntry* out, int max);
int bwd_q_kernels(KernelEntry* out, int max);

}  // namespace msa
