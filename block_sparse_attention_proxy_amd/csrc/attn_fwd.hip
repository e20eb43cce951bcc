// Sparse GQA forward over the selected KV blocks, with the proxy head's
// log-sum-exp over the same keys.
//
// Method: GQA attention restricted to the 128-token KV blocks chosen for each
// query block (ai-minor "Dramatically Speeding Up Million-Token Training!",
// News Overview: block-level sparsity, GQA instead of MLA; socker-news
// Flash-MSA summary 要約).  The attended set of query token i is every key
// u <= i inside the blocks selected for i's query block; the proxy softmax is
// taken over the same set and only its log-sum-exp is kept.
//
// Work split: a workgroup (4 waves) serves one (KV group, query block) and
// stages each selected KV block through LDS in two 64-key halves (K and V
// rows), double-buffered with a register prefetch of the next half; V^T
// fragments come from the row-major V tile through LDS transpose reads.
// A wave owns QT x 32 queries of one head and computes S^T = K Q^T on bf16
// MFMA so that each lane holds one query column; the probabilities then feed
// O^T += V^T P^T without leaving registers.  The proxy log-sum-exp over the
// same keys is a separate light kernel (one proxy head per group, dp-deep
// contractions), which keeps the main kernel's registers for attention.
#include "msa_device.h"
#include "msa_internal.h"
#include "msa_profile.h"

#include <type_traits>

namespace msa {

__device__ __forceinline__ int xcd_remap(int i, int n) {
  // Workgroups are dealt round-robin to the 8 XCDs; give each XCD a
  // contiguous range of logical ids so neighbours share that XCD's L2.
  const int per = n / 8, rem = n % 8;
  const int x = i % 8, k = i / 8;
  return x * per + (x < rem ? x : rem) + k;
}

template <typename T>
__device__ __forceinline__ void store4(T* dst, float a, float b, float c, float d);
template <>
__device__ __forceinline__ void store4<bf16>(bf16* dst, float a, float b, float c, float d) {
  bf16x4 r;
  r[0] = (bf16)a; r[1] = (bf16)b; r[2] = (bf16)c; r[3] = (bf16)d;
  *reinterpret_cast<bf16x4*>(dst) = r;
}
template <>
__device__ __forceinline__ void store4<float>(float* dst, float a, float b, float c, float d) {
  f32x4 r;
  r[0] = a; r[1] = b; r[2] = c; r[3] = d;
  *reinterpret_cast<f32x4*>(dst) = r;
}

template <typename T, int D, int DP, int QT>
struct FwdCfg {
  static constexpr int KC = 64;                         // keys per stage
  static constexpr int EPC = 16 / (int)sizeof(T);        // elements per 16-byte chunk
  static constexpr int PAD = 8;
  static constexpr int LDK = D + PAD;                    // K and V rows [KC][LDK]
  static constexpr int KS = KC * LDK;
  static constexpr int STAGE = 2 * KS;
  static constexpr int LDS_BYTES = 2 * STAGE * (int)sizeof(T);
  static constexpr int CPR = D / EPC;                    // chunks per row
  static constexpr int NK = KC * CPR / 256;              // chunks per thread per tensor
};

template <typename T, int D, int DP, int QT>
__global__ __launch_bounds__(256) void fwd_kernel(
    const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ v,
    const int32_t* __restrict__ q2k_idx, const int32_t* __restrict__ q2k_cnt,
    T* __restrict__ o, float* __restrict__ lse, Geo g) {
  typedef FwdCfg<T, D, DP, QT> C;
  extern __shared__ __align__(16) unsigned char smem_raw[];
  T* smem = reinterpret_cast<T*>(smem_raw);
  static_assert(C::NK >= 1, "tile split");

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int col = lane & 31, hi = lane >> 5;
  const int NU = g.G * (g.Bq / (32 * QT));
  const int nwg = (NU + 3) >> 2;
  const int bid = xcd_remap(blockIdx.x, gridDim.x);
  const int64_t item = bid / nwg;
  const int wgi = bid % nwg;
  const int grp = (int)(item / g.nqb);
  const int QB = (int)(item % g.nqb);
  const int u = wgi * 4 + wave;
  const bool active = u < NU;
  const int hl = u % g.G, chunk = u / g.G;
  const int h = grp * g.G + hl;

  int b;
  {
    int lo = 0, hi_ = g.B;
    while (hi_ - lo > 1) { int mid = (lo + hi_) >> 1; if (g.qb0[mid] <= QB) lo = mid; else hi_ = mid; }
    b = lo;
  }
  const int I = QB - g.qb0[b];
  const int t0 = g.cu[b];
  const int L = g.cu[b + 1] - t0;
  const int kb0 = g.kb0[b];
  const int diag = (I * g.Bq) >> 7;
  const int qbase = I * g.Bq + chunk * 32 * QT;
  const int64_t rowi = (int64_t)grp * g.nqb + QB;
  const int cnt = q2k_cnt[rowi];
  const int32_t* sel = q2k_idx + rowi * g.stride;

  frag_t<T> Qf[QT][D / 16];
  if (active) {
#pragma unroll
    for (int qt = 0; qt < QT; ++qt) {
      int row = qbase + qt * 32 + col;
      row = row < L ? row : L - 1;
      const T* src = q + ((int64_t)(t0 + row) * g.Hq + h) * D + hi * 8;
#pragma unroll
      for (int ks = 0; ks < D / 16; ++ks) Qf[qt][ks] = ld8(src + ks * 16);
    }
  }

  f32x16 O[D / 32][QT];
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
    for (int qt = 0; qt < QT; ++qt) O[dt][qt] = zero16();
  float m[QT], l[QT];
#pragma unroll
  for (int qt = 0; qt < QT; ++qt) { m[qt] = NEG_BIG; l[qt] = 0.f; }

  // stages: two 64-key halves per selected block; the second half of the
  // diagonal block is dropped when every query of the block precedes it.
  int nst = 2 * cnt;
  if (cnt > 0 && diag * 128 + 64 > I * g.Bq + g.Bq - 1) nst -= 1;

  uint4 Kr[C::NK], Vr[C::NK];
  auto load_stage = [&](int s) {
    const int J = sel[s >> 1] - kb0;
    const int key0 = J * 128 + (s & 1) * C::KC;
#pragma unroll
    for (int i = 0; i < C::NK; ++i) {
      const int c = tid + 256 * i, r = c / C::CPR, cc = c % C::CPR, key = key0 + r;
      const int64_t off = ((int64_t)(t0 + key) * g.Hkv + grp) * D + cc * C::EPC;
      Kr[i] = key < L ? *reinterpret_cast<const uint4*>(k + off) : make_uint4(0, 0, 0, 0);
      Vr[i] = key < L ? *reinterpret_cast<const uint4*>(v + off) : make_uint4(0, 0, 0, 0);
    }
  };
  auto store_stage = [&](int buf) {
    T* Ks = smem + buf * C::STAGE;
    T* Vs = Ks + C::KS;
#pragma unroll
    for (int i = 0; i < C::NK; ++i) {
      const int c = tid + 256 * i, r = c / C::CPR, cc = c % C::CPR;
      *reinterpret_cast<uint4*>(Ks + r * C::LDK + cc * C::EPC) = Kr[i];
      *reinterpret_cast<uint4*>(Vs + r * C::LDK + cc * C::EPC) = Vr[i];
    }
  };

  // One 32-key step: S^T = K Q^T, online softmax, O^T += V^T P^T.
  // lim: key row r of the tile is visible to query column qt iff r <= lim[qt]
  // (a large value when nothing is masked).  The running maximum m used for
  // the exponentials is only raised when a row's true maximum exceeds it by
  // more than RESCALE_GAP (base 2): P then stays below 2^RESCALE_GAP, the
  // result is the same after the final division by l, and the accumulator
  // rescale (VALU work on O) is rare.
  constexpr float RESCALE_GAP = 8.f;
  auto step = [&](const T* Ks, const T* Vs, int kt, const int (&lim)[QT]) {
    f32x16 S[QT];
#pragma unroll
    for (int qt = 0; qt < QT; ++qt) S[qt] = zero16();
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) {
      const frag_t<T> a = ld8(Ks + (kt * 32 + col) * C::LDK + ks * 16 + hi * 8);
#pragma unroll
      for (int qt = 0; qt < QT; ++qt) mma(S[qt], a, Qf[qt][ks]);
    }
    bool grow = false;
    float mnew[QT];
#pragma unroll
    for (int qt = 0; qt < QT; ++qt) {
      float mx = NEG_BIG;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const float x = acc_row(i, lane) <= lim[qt] ? S[qt][i] : -INFINITY;
        S[qt][i] = x;
        mx = fmaxf(mx, x);
      }
      mx = fmaxf(mx, __shfl_xor(mx, 32, 64)) * g.scale_log2;
      mnew[qt] = mx;
      grow |= mx > m[qt] + RESCALE_GAP;
    }
    if (__ballot(grow)) {
#pragma unroll
      for (int qt = 0; qt < QT; ++qt) {
        const float mn = fmaxf(m[qt], mnew[qt]);
        const float alpha = __builtin_amdgcn_exp2f(m[qt] - mn);
        m[qt] = mn;
        l[qt] *= alpha;
#pragma unroll
        for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
          for (int i = 0; i < 16; ++i) O[dt][qt][i] *= alpha;
      }
    }
#pragma unroll
    for (int qt = 0; qt < QT; ++qt) {
      float ls = 0.f;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const float p = __builtin_amdgcn_exp2f(fmaf(S[qt][i], g.scale_log2, -m[qt]));
        S[qt][i] = p;
        ls += p;
      }
      l[qt] += ls;
    }
    frag_t<T> Pf[2][QT];
#pragma unroll
    for (int kk = 0; kk < 2; ++kk)
#pragma unroll
      for (int qt = 0; qt < QT; ++qt) Pf[kk][qt] = acc_frag<T>(S[qt], kk);
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt) {
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        const frag_t<T> a = lds_col_frag<T>(Vs, C::LDK, kt * 32 + kk * 16, dt * 32, lane);
#pragma unroll
        for (int qt = 0; qt < QT; ++qt) mma(O[dt][qt], a, Pf[kk][qt]);
      }
    }
  };

  if (nst > 0) { load_stage(0); store_stage(0); }
  __syncthreads();

  // The loop body is straight-line: the stage after the last re-reads the
  // last stage (valid memory) into the unused buffer, and fully masked tiles
  // of the diagonal block are computed with every key masked.
  for (int s = 0; s < nst; ++s) {
    const int buf = s & 1;
    load_stage(s + 1 < nst ? s + 1 : s);
    const int J = sel[s >> 1] - kb0;
    const int kpos0 = J * 128 + (s & 1) * C::KC;
    const T* Ks = smem + buf * C::STAGE;
    const T* Vs = Ks + C::KS;
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
      int lim[QT];
#pragma unroll
      for (int qt = 0; qt < QT; ++qt)
        lim[qt] = (J == diag) ? qbase + qt * 32 + col - (kpos0 + kt * 32) : 1024;
      if (active) step(Ks, Vs, kt, lim);
    }
    store_stage(buf ^ 1);
    __syncthreads();
  }

  if (!active) return;
#pragma unroll
  for (int qt = 0; qt < QT; ++qt) {
    const float lt = l[qt] + __shfl_xor(l[qt], 32, 64);
    const int qpos = qbase + qt * 32 + col;
    if (qpos < L) {
      const int64_t t = t0 + qpos;
      const float inv = 1.f / lt;
      T* dst = o + (t * g.Hq + h) * D;
#pragma unroll
      for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
        for (int i4 = 0; i4 < 4; ++i4) {
          const int d0 = dt * 32 + acc_row(i4 * 4, lane);
          store4<T>(dst + d0, O[dt][qt][i4 * 4 + 0] * inv, O[dt][qt][i4 * 4 + 1] * inv,
                    O[dt][qt][i4 * 4 + 2] * inv, O[dt][qt][i4 * 4 + 3] * inv);
        }
      if (hi == 0) lse[(int64_t)h * g.T + t] = (m[qt] + log2f(lt)) * LN2;
    }
  }
}

// Proxy log-sum-exp over each query's selected keys: one wave per 32 queries
// of a (group, query block); kp tiles are read as A fragments straight from
// global memory (the waves of a workgroup walk the same blocks).
template <typename T, int DP>
__global__ __launch_bounds__(256) void proxy_lse_kernel(const T* __restrict__ qp,
                                                        const T* __restrict__ kp,
                                                        const int32_t* __restrict__ q2k_idx,
                                                        const int32_t* __restrict__ q2k_cnt,
                                                        float* __restrict__ lse_p, Geo g) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int col = lane & 31, hi = lane >> 5;
  const int nwq = g.Bq / 32;                     // waves per query block
  const int per_wg = 4 / nwq;                    // query blocks per workgroup
  const int64_t item = (int64_t)xcd_remap(blockIdx.x, gridDim.x) * per_wg + wave / nwq;
  if (item >= (int64_t)g.Hkv * g.nqb) return;    // no barriers in this kernel
  const int c = wave % nwq;
  const int grp = (int)(item / g.nqb);
  const int QB = (int)(item % g.nqb);
  int lo = 0, hi_ = g.B;
  while (hi_ - lo > 1) { int mid = (lo + hi_) >> 1; if (g.qb0[mid] <= QB) lo = mid; else hi_ = mid; }
  const int b = lo;
  const int I = QB - g.qb0[b];
  const int t0 = g.cu[b];
  const int L = g.cu[b + 1] - t0;
  const int kb0 = g.kb0[b];
  const int diag = (I * g.Bq) >> 7;
  const int q0 = I * g.Bq + c * 32;
  if (q0 >= L) return;
  const int qpos = q0 + col;
  const int qrow = qpos < L ? qpos : L - 1;
  frag_t<T> QPf[DP / 16];
  {
    const T* sp = qp + ((int64_t)(t0 + qrow) * g.Hkv + grp) * DP + hi * 8;
#pragma unroll
    for (int ks = 0; ks < DP / 16; ++ks) QPf[ks] = ld8(sp + ks * 16);
  }
  const int64_t rowi = (int64_t)grp * g.nqb + QB;
  const int cnt = q2k_cnt[rowi];
  const int32_t* sel = q2k_idx + rowi * g.stride;
  float mp = NEG_BIG, lp = 0.f;
  for (int si = 0; si < cnt; ++si) {
    const int J = sel[si] - kb0;
    const bool need_mask = (J == diag);
#pragma unroll
    for (int kt = 0; kt < 4; ++kt) {
      const int kpos = J * 128 + kt * 32;
      if (kpos > q0 + 31) break;
      int key = kpos + col;
      key = key < L ? key : L - 1;               // rows past the end are masked below
      const T* sk = kp + ((int64_t)(t0 + key) * g.Hkv + grp) * DP + hi * 8;
      f32x16 Y = zero16();
#pragma unroll
      for (int ks = 0; ks < DP / 16; ++ks) mma(Y, ld8(sk + ks * 16), QPf[ks]);
      float mx = NEG_BIG;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        float x = Y[i] * g.pscale_log2;
        if (need_mask && kpos + acc_row(i, lane) > qpos) x = -INFINITY;
        Y[i] = x;
        mx = fmaxf(mx, x);
      }
      mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
      const float mnew = fmaxf(mp, mx);
      float ls = 0.f;
#pragma unroll
      for (int i = 0; i < 16; ++i) ls += __builtin_amdgcn_exp2f(Y[i] - mnew);
      lp = lp * __builtin_amdgcn_exp2f(mp - mnew) + ls;
      mp = mnew;
    }
  }
  const float lt = lp + __shfl_xor(lp, 32, 64);
  if (hi == 0 && qpos < L) lse_p[(int64_t)grp * g.T + t0 + qpos] = (mp + log2f(lt)) * LN2;
}

template <typename T, int D, int DP>
static hipError_t fwd_dispatch(const Geo& g, const void* q, const void* k, const void* v,
                               const void* qp, const void* kp, const int32_t* q2k_idx,
                               const int32_t* q2k_cnt, void* o, float* lse, float* lse_p,
                               hipStream_t s) {
  constexpr int QT = 2;
  typedef FwdCfg<T, D, DP, QT> C;
  auto fn = fwd_kernel<T, D, DP, QT>;
  static bool attr = false;
  if (!attr) {
    hipError_t e = hipFuncSetAttribute((const void*)fn, hipFuncAttributeMaxDynamicSharedMemorySize,
                                       C::LDS_BYTES);
    if (e != hipSuccess) return e;
    attr = true;
  }
  const int NU = g.G * (g.Bq / (32 * QT));
  const int64_t nblk = (int64_t)g.Hkv * g.nqb * ((NU + 3) / 4);
  if (nblk == 0) return hipSuccess;
  { ProfScope _ps("fwd", s);
  hipLaunchKernelGGL(fn, dim3((unsigned)nblk), dim3(256), C::LDS_BYTES, s, (const T*)q, (const T*)k,
                     (const T*)v, q2k_idx, q2k_cnt, (T*)o, lse, g); }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int per_wg = 4 / (g.Bq / 32);
  const int64_t nrow = (int64_t)g.Hkv * g.nqb;
  { ProfScope _ps("proxy_lse", s);
  hipLaunchKernelGGL((proxy_lse_kernel<T, DP>), dim3((unsigned)((nrow + per_wg - 1) / per_wg)), dim3(256),
                     0, s, (const T*)qp, (const T*)kp, q2k_idx, q2k_cnt, lse_p, g); }
  return hipGetLastError();
}

hipError_t launch_fwd(const Geo& g, int is_bf16, const void* q, const void* k, const void* v,
                      const void* qp, const void* kp, const int32_t* q2k_idx,
                      const int32_t* q2k_cnt, void* o, float* lse, float* lse_p, hipStream_t s) {
  if (is_bf16) {
    if (g.D == 128) return fwd_dispatch<bf16, 128, 64>(g, q, k, v, qp, kp, q2k_idx, q2k_cnt, o, lse, lse_p, s);
    return fwd_dispatch<bf16, 64, 32>(g, q, k, v, qp, kp, q2k_idx, q2k_cnt, o, lse, lse_p, s);
  }
  return fwd_dispatch<float, 64, 32>(g, q, k, v, qp, kp, q2k_idx, q2k_cnt, o, lse, lse_p, s);
}

}  // namespace msa

namespace msa {
int fwd_kernels(KernelEntry* out, int max) {
  const KernelEntry all[] = {
      {"fwd<bf16,d128,dp64>", (const void*)fwd_kernel<bf16, 128, 64, 2>, 256, FwdCfg<bf16, 128, 64, 2>::LDS_BYTES},
      {"fwd<bf16,d64,dp32>", (const void*)fwd_kernel<bf16, 64, 32, 2>, 256, FwdCfg<bf16, 64, 32, 2>::LDS_BYTES},
      {"fwd<f32,d64,dp32>", (const void*)fwd_kernel<float, 64, 32, 2>, 256, FwdCfg<float, 64, 32, 2>::LDS_BYTES},
      {"proxy_lse<bf16,dp64>", (const void*)proxy_lse_kernel<bf16, 64>, 256, 0},
      {"proxy_lse<bf16,dp32>", (const void*)proxy_lse_kernel<bf16, 32>, 256, 0},
      {"proxy_lse<f32,dp32>", (const void*)proxy_lse_kernel<float, 32>, 256, 0},
  };
  int n = (int)(sizeof(all) / sizeof(all[0]));
  for (int i = 0; i < n && i < max; ++i) out[i] = all[i];
  return n;
}
}  // namespace msa
