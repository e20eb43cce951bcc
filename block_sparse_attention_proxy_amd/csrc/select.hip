// Proxy block scoring, top-k block selection and the KV-major inverted index.
//
// Method (pages: ai-minor "Dramatically Speeding Up Million-Token Training!",
// News Overview and Terminology; socker-news Flash-MSA summary 要約):
// a proxy head scores query-key pairs, the scores are max-pooled over
// 128-token KV blocks, and each query block keeps its best KV blocks.
// Readings used here: the pooled tile is (query block x KV block), the raw
// dot product <qp, kp> is pooled (a positive scale cannot change a ranking),
// candidates are the blocks strictly before the forced diagonal + window, and
// an exact score tie goes to the lower block index.
#include "msa_device.h"
#include "msa_internal.h"
#include "msa_profile.h"

#include <mutex>

namespace msa {

// ---------------------------------------------------------------------------
// Static scratch of the allocation-free selection entry point: the
// per-document tables and the inverted-index counters live here instead of
// in a caller's workspace.  Every GPU the library runs on holds its own copy
// until the process ends.  In host code the array's name is only a stand-in:
// its device address comes from hipGetSymbolAddress, taken once per device
// with that device current, and only that address is handed to kernels.
// ---------------------------------------------------------------------------
__device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

hipError_t noalloc_scratch(void** ptr) {
  constexpr int MAX_DEV = 64;
  static std::mutex mu;
  static void* addr[MAX_DEV] = {};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= MAX_DEV) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (!addr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    addr[dev] = p;
  }
  *ptr = addr[dev];
  return hipSuccess;
}

// Index b in [0, n) with a[b] <= x < a[b + 1] (a has n + 1 non-decreasing entries).
template <typename I>
__device__ __forceinline__ int find_segment(const I* a, int n, I x) {
  int lo = 0, hi = n;  // invariant: a[lo] <= x, answer < hi
  while (hi - lo > 1) {
    int mid = (lo + hi) >> 1;
    if (a[mid] <= x) lo = mid; else hi = mid;
  }
  return lo;
}

// ---------------------------------------------------------------------------
// metadata: per-document block offsets and a longest-first document order
// ---------------------------------------------------------------------------

// Block-wide exclusive scan of int64 values (256 threads); returns the
// exclusive prefix of this thread's value and adds the chunk total to *carry.
__device__ int64_t block_exscan256(int64_t v, int64_t* sh, int64_t& carry) {
  const int t = threadIdx.x;
  sh[t] = v;
  __syncthreads();
  for (int o = 1; o < 256; o <<= 1) {
    int64_t add = (t >= o) ? sh[t - o] : 0;
    __syncthreads();
    sh[t] += add;
    __syncthreads();
  }
  int64_t incl = sh[t];
  int64_t total = sh[255];
  __syncthreads();
  int64_t r = carry + incl - v;
  carry += total;
  return r;
}

__global__ __launch_bounds__(256) void meta_kernel(Geo g) {
  __shared__ int64_t sh[256];
  const int B = g.B;
  int64_t cq = 0, ck = 0, cs = 0, cu_ = 0;
  for (int base = 0; base < B + 1; base += 256) {
    int b = base + threadIdx.x;
    int64_t nq = 0, nk = 0;
    if (b < B) {
      int64_t L = g.cu[b + 1] - g.cu[b];
      nq = (L + g.Bq - 1) / g.Bq;
      nk = (L + 127) / 128;
    }
    int64_t eq = block_exscan256(nq, sh, cq);
    int64_t ek = block_exscan256(nk, sh, ck);
    int64_t es = block_exscan256(nq * nk, sh, cs);
    if (b <= B) {
      g.qb0[b] = (int32_t)eq;
      g.kb0[b] = (int32_t)ek;
      g.s0[b] = es;
    }
  }
  // rank documents by length (longest first, index breaks ties)
  for (int b = threadIdx.x; b < B; b += 256) {
    int Lb = g.cu[b + 1] - g.cu[b];
    int r = 0;
    for (int c = 0; c < B; ++c) {
      int Lc = g.cu[c + 1] - g.cu[c];
      r += (Lc > Lb) || (Lc == Lb && c < b);
    }
    g.order[r] = b;
  }
  __syncthreads();
  for (int base = 0; base < B + 1; base += 256) {
    int r = base + threadIdx.x;
    int64_t n = 0;
    if (r < B) {
      int b = g.order[r];
      int64_t L = g.cu[b + 1] - g.cu[b];
      int64_t tiles = (L + 127) / 128;
      n = (tiles + 1) / 2;
    }
    int64_t e = block_exscan256(n, sh, cu_);
    if (r <= B) g.unit0[r] = (int32_t)e;
  }
  // column slabs of the inverted index (K2Q_SLAB blocks each), in document order
  int64_t cs_ = 0;
  for (int base = 0; base < B + 1; base += 256) {
    int bb = base + threadIdx.x;
    int64_t n = 0;
    if (bb < B) n = ((g.cu[bb + 1] - g.cu[bb] + 127) / 128 + K2Q_SLAB - 1) / K2Q_SLAB;
    int64_t e = block_exscan256(n, sh, cs_);
    if (bb <= B) g.slab0[bb] = (int32_t)e;
  }
}

// Document of every global query block and KV block, so that kernels find
// their document with one load instead of a search over the document table.
__global__ __launch_bounds__(256) void docmap_kernel(Geo g) {
  const int64_t n = (int64_t)g.nqb + g.nkb;
  for (int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; e < n;
       e += (int64_t)gridDim.x * blockDim.x) {
    if (e < g.nqb) g.qdoc[e] = find_segment<int32_t>(g.qb0, g.B, (int32_t)e);
    else g.kdoc[e - g.nqb] = find_segment<int32_t>(g.kb0, g.B, (int32_t)(e - g.nqb));
  }
}

hipError_t launch_meta(const Geo& g, hipStream_t s) {
  { ProfScope _ps("meta", s);
  hipLaunchKernelGGL(meta_kernel, dim3(1), dim3(256), 0, s, g); }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t n = (int64_t)g.nqb + g.nkb;
  if (n > 0) {
    { ProfScope _ps("meta", s);
    hipLaunchKernelGGL(docmap_kernel, dim3((unsigned)((n + 255) / 256 < 4096 ? (n + 255) / 256 : 4096)),
                       dim3(256), 0, s, g); }
    e = hipGetLastError();
  }
  return e;
}

// ---------------------------------------------------------------------------
// proxy scores: S[g, I, J] = max over the tile of <qp, kp>
// ---------------------------------------------------------------------------
//
// One wave owns a unit = a pair of 128-row query tiles (p, nt - 1 - p) of one
// document, so every unit of a document costs about the same.  Per tile it
// keeps its 128 qp rows as A fragments and streams the candidate KV blocks of
// kp as B fragments straight from global memory (the waves of a workgroup
// walk the same KV blocks together and share them through the caches).
// Each KV block gives four 32x32 row tiles x four 32-key tiles; the maxima are
// folded per lane, reduced over the wave, and written 64 blocks at a time.

// Maximum over the 64 lanes, uniform result: row shifts within rows of 16
// lanes (DPP, no LDS round trips), then the four row maxima by readlane.
__device__ __forceinline__ float wave_max_dpp(float v) {
  const int ninf = (int)0xff800000u;
  int x = __float_as_int(v);
  x = __float_as_int(fmaxf(__int_as_float(x), __int_as_float(__builtin_amdgcn_update_dpp(ninf, x, 0x111, 0xf, 0xf, false))));
  x = __float_as_int(fmaxf(__int_as_float(x), __int_as_float(__builtin_amdgcn_update_dpp(ninf, x, 0x112, 0xf, 0xf, false))));
  x = __float_as_int(fmaxf(__int_as_float(x), __int_as_float(__builtin_amdgcn_update_dpp(ninf, x, 0x114, 0xf, 0xf, false))));
  x = __float_as_int(fmaxf(__int_as_float(x), __int_as_float(__builtin_amdgcn_update_dpp(ninf, x, 0x118, 0xf, 0xf, false))));
  const float r0 = __int_as_float(__builtin_amdgcn_readlane(x, 15));
  const float r1 = __int_as_float(__builtin_amdgcn_readlane(x, 31));
  const float r2 = __int_as_float(__builtin_amdgcn_readlane(x, 47));
  const float r3 = __int_as_float(__builtin_amdgcn_readlane(x, 63));
  return fmaxf(fmaxf(r0, r1), fmaxf(r2, r3));
}

template <typename T, int DP, int BQ>
__global__ __launch_bounds__(256, 2) void proxy_scores_kernel(const T* __restrict__ qp,
                                                           const T* __restrict__ kp,
                                                           float* __restrict__ scores, Geo g) {
  constexpr int KSL = DP / 16;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int grp = blockIdx.x % g.Hkv;
  const int unit = (blockIdx.x / g.Hkv) * 4 + wave;
  if (unit >= g.n_units) return;   // no barriers below
  const int r = find_segment<int32_t>(g.unit0, g.B, unit);
  const int b = g.order[r];
  const int p = unit - g.unit0[r];
  const int t0 = g.cu[b];
  const int L = g.cu[b + 1] - t0;
  const int nt = (L + 127) >> 7;
  const int nk = nt;
  const int nq = (L + BQ - 1) / BQ;
  const int64_t s0 = g.s0[b];
  const int Hp = g.Hkv;
  const int col = lane & 31;
  const int hi8 = (lane >> 5) * 8;

  for (int pass = 0; pass < 2; ++pass) {
    const int tile = pass == 0 ? p : nt - 1 - p;
    if (pass == 1 && tile == p) break;
    const int ncand = tile - g.span;              // blocks below the window's span
    if (ncand <= g.topk - 1) continue;            // all of them are taken; nothing to score

    frag_t<T> A[4][KSL];
#pragma unroll
    for (int rt = 0; rt < 4; ++rt) {
      int row = tile * 128 + rt * 32 + col;
      row = row < L ? row : L - 1;                // duplicate rows leave the max unchanged
      const T* src = qp + ((int64_t)(t0 + row) * Hp + grp) * DP + hi8;
#pragma unroll
      for (int ks = 0; ks < KSL; ++ks) A[rt][ks] = ld8(src + ks * 16);
    }
    const int I0 = (BQ == 128) ? tile : 2 * tile;
    const bool has1 = (BQ == 64) && (2 * tile + 1 < nq);
    float* out0 = scores + (int64_t)grp * g.score_elems + s0 + (int64_t)I0 * nk;
    float* out1 = out0 + nk;
    float stash0 = 0.f, stash1 = 0.f;

    // kp of one KV block as B fragments, in four 32-key slices.  Tiles run
    // slice by slice (kt outer), so slice kt is refilled with the next
    // block's keys as soon as its fourth tile has been issued: the load has
    // the other three slices' products to land in.
    frag_t<T> Bf[4][KSL];
    auto load_slice = [&](int J, int kt) __attribute__((always_inline)) {
      const T* src = kp + ((int64_t)(t0 + J * 128 + kt * 32 + col) * Hp + grp) * DP + hi8;
#pragma unroll
      for (int ks = 0; ks < KSL; ++ks) Bf[kt][ks] = ld8(src + ks * 16);
    };
    // maximum of a tile's 16 values folded into m: a tree of depth three
    auto fold = [](float m, const f32x16& a) __attribute__((always_inline)) {
      const float t0 = fmaxf(fmaxf(a[0], a[1]), a[2]), t1 = fmaxf(fmaxf(a[3], a[4]), a[5]);
      const float t2 = fmaxf(fmaxf(a[6], a[7]), a[8]), t3 = fmaxf(fmaxf(a[9], a[10]), a[11]);
      const float t4 = fmaxf(fmaxf(a[12], a[13]), a[14]);
      const float u0 = fmaxf(fmaxf(t0, t1), t2), u1 = fmaxf(fmaxf(t3, t4), a[15]);
      return fmaxf(fmaxf(m, u0), u1);
    };
    // slices issued in order (the loop waits for slice kt with the later
    // slices still in flight)
    static_for<4>([&](auto ktc) __attribute__((always_inline)) {
      load_slice(0, decltype(ktc)::value);
      __builtin_amdgcn_sched_barrier(0);
    });
    for (int J = 0; J < ncand; ++J) {
      const int Jn = J + 1 < ncand ? J + 1 : J;       // past the end: the last block again
      float m0 = NEG_BIG, m1 = NEG_BIG;
      // 16 tiles (4 key slices x 4 row tiles) of 4 products each, two tiles
      // at a time with their products alternating (no product waits for the
      // one before it), into four accumulators by turns: a pair's maxima are
      // taken after the next pair's products have been issued.
      f32x16 acc[4];
      auto fold_tile = [&](auto nc) __attribute__((always_inline)) {
        constexpr int n = decltype(nc)::value, rt = n % 4;
        if (BQ == 64 && rt >= 2) m1 = fold(m1, acc[n & 3]);
        else m0 = fold(m0, acc[n & 3]);
      };
      static_for<8>([&](auto pc) __attribute__((always_inline)) {
        constexpr int pr = decltype(pc)::value, n0 = 2 * pr, n1 = 2 * pr + 1;
        constexpr int kt = n0 / 4, rt0 = n0 % 4, rt1 = n1 % 4;
        acc[n0 & 3] = zero16();
        acc[n1 & 3] = zero16();
#pragma unroll
        for (int ks = 0; ks < KSL; ++ks) {
          mma(acc[n0 & 3], A[rt0][ks], Bf[kt][ks]);
          mma(acc[n1 & 3], A[rt1][ks], Bf[kt][ks]);
        }
        if constexpr (rt1 == 3) load_slice(Jn, kt);
        __builtin_amdgcn_sched_barrier(0);
        if constexpr (pr > 0) {
          fold_tile(std::integral_constant<int, n0 - 2>());
          fold_tile(std::integral_constant<int, n1 - 2>());
        }
        __builtin_amdgcn_sched_barrier(0);
      });
      fold_tile(std::integral_constant<int, 14>());
      fold_tile(std::integral_constant<int, 15>());
      // the wave maximum, stashed in lane J % 64 and stored 64 blocks at a time
      m0 = wave_max_dpp(m0);
      if (BQ == 64) m1 = wave_max_dpp(m1);
      if (lane == (J & 63)) { stash0 = m0; stash1 = m1; }
      if ((J & 63) == 63 || J == ncand - 1) {
        const int base = J & ~63;
        if (lane <= (J & 63)) {
          out0[base + lane] = stash0;
          if (has1) out1[base + lane] = stash1;
        }
      }
    }
  }
}

// bf16, dp = 64: the same units and tile order, with kp staged through LDS.
// Loading B fragments straight from global memory makes every 16-byte lane
// read touch its own 128-byte line (32 lines per instruction), which keeps
// the L1 tag lookups, not the matrix cores, the bound.  Here each wave copies
// its 32-key kp slices (4 KiB, 8 whole rows per instruction) into a private
// ring of SC_NS slots by DMA, SC_NS - 1 slices ahead, and reads the fragments
// back from the swizzled slot.  A wave reads only its own slots, so a count
// of its copies in flight (vmcnt) is the only synchronisation.
constexpr int SC_NS = 5;                            // slots per wave
constexpr int SC_SLICE = 32 * 64 * 2;               // bytes per slice
constexpr int SC_LDS = 4 * SC_NS * SC_SLICE;        // per workgroup: 80 KiB

template <int BQ>
__global__ __launch_bounds__(256, 2) void proxy_scores_lds_kernel(const bf16* __restrict__ qp,
                                                               const bf16* __restrict__ kp,
                                                               float* __restrict__ scores, Geo g) {
  constexpr int DP = 64, KSL = DP / 16;
  typedef Tile<bf16, DP> TP;
  extern __shared__ __align__(16) unsigned char smem_raw[];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int grp = blockIdx.x % g.Hkv;
  const int unit = (blockIdx.x / g.Hkv) * 4 + wave;
  if (unit >= g.n_units) return;   // no barriers below
  const int r = find_segment<int32_t>(g.unit0, g.B, unit);
  const int b = g.order[r];
  const int p = unit - g.unit0[r];
  const int t0 = g.cu[b];
  const int L = g.cu[b + 1] - t0;
  const int nt = (L + 127) >> 7;
  const int nk = nt;
  const int nq = (L + BQ - 1) / BQ;
  const int64_t s0 = g.s0[b];
  const int Hp = g.Hkv;
  const int col = lane & 31;
  const int hi8 = (lane >> 5) * 8;
  const uint32_t ring = lds_offset(smem_raw) + (uint32_t)wave * SC_NS * SC_SLICE;
  // copy side: lane l moves row 8 j + (l >> 3), 16-byte chunk l & 7 of a slice
  // (source chunk swizzled so that the slot holds the Tile layout)
  // through a buffer descriptor over the slice's 32 rows, with fixed per-lane
  // byte offsets (candidate blocks lie wholly inside the document)
  const int crow = lane >> 3;
  const uint32_t rsp = (uint32_t)Hp * DP * 2;
  uint32_t coff[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) coff[j] = (uint32_t)(8 * j + crow) * rsp + (uint32_t)swz<8>(8 * j + crow, lane & 7) * 16;
  // read side: fragment ks of this lane's key row in a slot
  const uint32_t rd0 = (uint32_t)TP::off(col, hi8) * 2;

  for (int pass = 0; pass < 2; ++pass) {
    const int tile = pass == 0 ? p : nt - 1 - p;
    if (pass == 1 && tile == p) break;
    const int ncand = tile - g.span;              // blocks below the window's span
    if (ncand <= g.topk - 1) continue;            // all of them are taken; nothing to score

    bf16x8 A[4][KSL];
#pragma unroll
    for (int rt = 0; rt < 4; ++rt) {
      int row = tile * 128 + rt * 32 + col;
      row = row < L ? row : L - 1;                // duplicate rows leave the max unchanged
      const bf16* src = qp + ((int64_t)(t0 + row) * Hp + grp) * DP + hi8;
#pragma unroll
      for (int ks = 0; ks < KSL; ++ks) A[rt][ks] = ld8(src + ks * 16);
    }
    const int I0 = (BQ == 128) ? tile : 2 * tile;
    const bool has1 = (BQ == 64) && (2 * tile + 1 < nq);
    float* out0 = scores + (int64_t)grp * g.score_elems + s0 + (int64_t)I0 * nk;
    float* out1 = out0 + nk;
    float stash0 = 0.f, stash1 = 0.f;
    // The register loads above complete before any copy is issued, so that
    // the copies are the only vector-memory operations the waits count.
    wait_vmcnt<0>();

    const int nsl = ncand * 4;                    // slices: block J, key slice kt -> 4 J + kt
    const bf16* kbase = kp + ((int64_t)t0 * Hp + grp) * DP;
    int i_q = 0;                                  // next slice to copy
    uint32_t i_slot = 0, c_slot = 0;              // byte offsets of the next copy's / read's slot
    auto copy_next = [&]() __attribute__((always_inline)) {
      const int q = i_q < nsl ? i_q : nsl - 1;    // past the end: the last slice again
      const i32x4 sd = make_srd(kbase + (int64_t)q * 32 * Hp * DP, 32u * rsp);
#pragma unroll
      for (int j = 0; j < 4; ++j) bdma16(sd, coff[j], ring + i_slot + j * 1024);
      ++i_q;
      i_slot = i_slot == (SC_NS - 1) * SC_SLICE ? 0u : i_slot + SC_SLICE;
    };
    auto read_slice = [&](bf16x8 (&Bf)[KSL]) __attribute__((always_inline)) {
      const uint32_t a = ring + c_slot + rd0;
#pragma unroll
      for (int ks = 0; ks < KSL; ++ks) Bf[ks] = lds_ld8<0>(a ^ (uint32_t)(ks << 5));
      c_slot = c_slot == (SC_NS - 1) * SC_SLICE ? 0u : c_slot + SC_SLICE;
    };
    auto fold = [](float m, const f32x16& a) __attribute__((always_inline)) {
      const float t0 = fmaxf(fmaxf(a[0], a[1]), a[2]), t1 = fmaxf(fmaxf(a[3], a[4]), a[5]);
      const float t2 = fmaxf(fmaxf(a[6], a[7]), a[8]), t3 = fmaxf(fmaxf(a[9], a[10]), a[11]);
      const float t4 = fmaxf(fmaxf(a[12], a[13]), a[14]);
      const float u0 = fmaxf(fmaxf(t0, t1), t2), u1 = fmaxf(fmaxf(t3, t4), a[15]);
      return fmaxf(fmaxf(m, u0), u1);
    };
#pragma unroll
    for (int j = 0; j < SC_NS - 1; ++j) copy_next();
    wait_vmcnt<4 * (SC_NS - 2)>();                // slice 0
    bf16x8 Bc[KSL], Bn[KSL];
    read_slice(Bc);
    f32x16 acc[4];
    for (int J = 0; J < ncand; ++J) {
      float m0 = NEG_BIG, m1 = NEG_BIG;
      static_for<4>([&](auto ktc) __attribute__((always_inline)) {
        constexpr int kt = decltype(ktc)::value;
        // the slot of the slice before this one is free: refill it, then
        // fetch the next slice's fragments once they have landed
        copy_next();
        wait_vmcnt<4 * (SC_NS - 2)>();
        static_for<2>([&](auto hc) __attribute__((always_inline)) {
          constexpr int h = decltype(hc)::value, rt0 = 2 * h, rt1 = 2 * h + 1;
          constexpr int a0 = h ? 2 : 0;                 // accumulator pair of this half
          acc[a0] = zero16();
          acc[a0 + 1] = zero16();
#pragma unroll
          for (int ks = 0; ks < KSL; ++ks) {
            mma(acc[a0], A[rt0][ks], Bc[ks]);
            mma(acc[a0 + 1], A[rt1][ks], Bc[ks]);
          }
          if constexpr (h == 0) read_slice(Bn);
          __builtin_amdgcn_sched_barrier(0);
          // maxima of the previous pair (the last pair of the block before
          // is folded at that block's end)
          if constexpr (kt > 0 || h > 0) {
            constexpr int pr0 = h == 0 ? 2 : 0;   // its first row tile
            const int pa = a0 ^ 2;
            if (BQ == 64 && pr0 >= 2) { m1 = fold(m1, acc[pa]); m1 = fold(m1, acc[pa + 1]); }
            else { m0 = fold(m0, acc[pa]); m0 = fold(m0, acc[pa + 1]); }
          }
          __builtin_amdgcn_sched_barrier(0);
        });
#pragma unroll
        for (int ks = 0; ks < KSL; ++ks) Bc[ks] = Bn[ks];
      });
      // last pair of the block: row tiles 2, 3 of key slice 3, accumulators 2, 3
      if (BQ == 64) { m1 = fold(m1, acc[2]); m1 = fold(m1, acc[3]); }
      else { m0 = fold(m0, acc[2]); m0 = fold(m0, acc[3]); }
      m0 = wave_max_dpp(m0);
      if (BQ == 64) m1 = wave_max_dpp(m1);
      if (lane == (J & 63)) { stash0 = m0; stash1 = m1; }
      if ((J & 63) == 63 || J == ncand - 1) {
        const int base = J & ~63;
        if (lane <= (J & 63)) {
          out0[base + lane] = stash0;
          if (has1) out1[base + lane] = stash1;
        }
      }
    }
    wait_vmcnt<0>();                              // copies past the end, before the ring is reused
  }
}

template <typename T, int DP>
static hipError_t scores_dispatch_bq(const Geo& g, const void* qp, const void* kp, float* scores,
                                     hipStream_t s) {
  int nblk = (g.n_units + 3) / 4 * g.Hkv;
  if (nblk == 0) return hipSuccess;
  if constexpr (sizeof(T) == 2 && DP == 64) {
    static LdsLimitOnce lds_limit;
    const hipError_t e = lds_limit.ensure({{(const void*)proxy_scores_lds_kernel<128>, SC_LDS},
                                           {(const void*)proxy_scores_lds_kernel<64>, SC_LDS}});
    if (e != hipSuccess) return e;
    { ProfScope _ps("proxy_scores", s);
    if (g.Bq == 128)
      hipLaunchKernelGGL((proxy_scores_lds_kernel<128>), dim3(nblk), dim3(256), SC_LDS, s,
                         (const bf16*)qp, (const bf16*)kp, scores, g);
    else
      hipLaunchKernelGGL((proxy_scores_lds_kernel<64>), dim3(nblk), dim3(256), SC_LDS, s,
                         (const bf16*)qp, (const bf16*)kp, scores, g); }
    return hipGetLastError();
  }
  if (g.Bq == 128)
    { ProfScope _ps("proxy_scores", s);
    hipLaunchKernelGGL((proxy_scores_kernel<T, DP, 128>), dim3(nblk), dim3(256), 0, s,
                       (const T*)qp, (const T*)kp, scores, g); }
  else
    { ProfScope _ps("proxy_scores", s);
    hipLaunchKernelGGL((proxy_scores_kernel<T, DP, 64>), dim3(nblk), dim3(256), 0, s,
                       (const T*)qp, (const T*)kp, scores, g); }
  return hipGetLastError();
}

hipError_t launch_proxy_scores(const Geo& g, int is_bf16, const void* qp, const void* kp,
                               float* scores, hipStream_t s) {
  if (is_bf16) {
    if (g.DP == 64) return scores_dispatch_bq<bf16, 64>(g, qp, kp, scores, s);
    return scores_dispatch_bq<bf16, 32>(g, qp, kp, scores, s);
  }
  return scores_dispatch_bq<float, 32>(g, qp, kp, scores, s);
}

// ---------------------------------------------------------------------------
// selection: one wave per (group, query block)
// ---------------------------------------------------------------------------
//
// The k - 1 best candidates are those at or above a cut in the order (score
// descending, block index ascending).  The cut is found on order-preserving
// integer keys by radix steps over 8-bit windows: the first window starts at
// the highest bit where the row's keys differ, a histogram of the window's
// digit locates the bin that holds the (k-1)-th key, and that bin is then
// resolved exactly: taken whole when all of it is needed, ranked member by
// member when it holds at most 64 keys, else split by the next window.  The
// pick is emitted in ascending block order with a ballot prefix count,
// followed by the forced window and diagonal blocks, then -1 padding.

__device__ __forceinline__ uint32_t order_key(float s) {
  uint32_t u = __float_as_uint(s);
  if (u == 0x80000000u) u = 0u;                   // -0 ties with +0
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ uint64_t lanes_below(int lane) {
  return lane == 0 ? 0ull : (~0ull >> (64 - lane));
}

// Orders LDS traffic inside one wave (each wave owns its LDS area, so no
// workgroup barrier is needed).
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
  __builtin_amdgcn_wave_barrier();
}

// Lane shifts within rows of 16 lanes; a lane whose source lies outside its
// row keeps `old`.
template <int SHIFT>
__device__ __forceinline__ uint32_t row_shr(uint32_t old, uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp((int)old, (int)v, 0x110 + SHIFT, 0xf, 0xf, false);
}
__device__ __forceinline__ uint32_t rd_lane(uint32_t v, int l) {
  return (uint32_t)__builtin_amdgcn_readlane((int)v, l);
}
__device__ __forceinline__ uint32_t wave_min(uint32_t v) {
  v = min(v, row_shr<1>(0xffffffffu, v));
  v = min(v, row_shr<2>(0xffffffffu, v));
  v = min(v, row_shr<4>(0xffffffffu, v));
  v = min(v, row_shr<8>(0xffffffffu, v));
  return min(min(rd_lane(v, 15), rd_lane(v, 31)), min(rd_lane(v, 47), rd_lane(v, 63)));
}
__device__ __forceinline__ uint32_t wave_max(uint32_t v) {
  v = max(v, row_shr<1>(0u, v));
  v = max(v, row_shr<2>(0u, v));
  v = max(v, row_shr<4>(0u, v));
  v = max(v, row_shr<8>(0u, v));
  return max(max(rd_lane(v, 15), rd_lane(v, 31)), max(rd_lane(v, 47), rd_lane(v, 63)));
}
// inclusive prefix sum over the 64 lanes
__device__ __forceinline__ uint32_t wave_incl_sum(uint32_t x, int lane) {
  x += row_shr<1>(0u, x);
  x += row_shr<2>(0u, x);
  x += row_shr<4>(0u, x);
  x += row_shr<8>(0u, x);
  const uint32_t r0 = rd_lane(x, 15), r1 = rd_lane(x, 31), r2 = rd_lane(x, 47);
  const int row = lane >> 4;
  return x + (row >= 1 ? r0 : 0u) + (row >= 2 ? r1 : 0u) + (row >= 3 ? r2 : 0u);
}

// Per-wave LDS: a 256-bin histogram (bin 255 - v counts digit v, so that lane
// l reads the four bins of digits 255 - 4l ... 252 - 4l, highest first) and
// room for the 64 members of a threshold bin.
struct SelLds {
  uint32_t hist[256];
  uint32_t mkey[64];
  int32_t mj[64];
};

__device__ __forceinline__ void hist_clear(SelLds& w, int lane) {
  reinterpret_cast<uint4*>(w.hist)[lane] = make_uint4(0u, 0u, 0u, 0u);
  wave_lds_sync();
}

// Given the histogram of one window's digit (over the keys that match the
// decided prefix), find the bin of the rem-th largest key: its digit, how
// many of its keys are still needed (rem, updated) and how many it holds.
__device__ __forceinline__ void radix_pick(SelLds& w, int lane, uint32_t& digit, int& rem, int& cnt) {
  wave_lds_sync();
  const uint4 hv = reinterpret_cast<const uint4*>(w.hist)[lane];
  const uint32_t hb[4] = {hv.x, hv.y, hv.z, hv.w};
  const uint32_t c = hv.x + hv.y + hv.z + hv.w;
  int above = (int)(wave_incl_sum(c, lane) - c);  // keys in the bins of lower lanes (higher digits)
  int found = -1, nrem = 0, fcnt = 0;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    if (found < 0 && above < rem && rem <= above + (int)hb[q]) { found = q; nrem = rem - above; fcnt = (int)hb[q]; }
    above += (int)hb[q];
  }
  const int src = __ffsll((unsigned long long)__ballot(found >= 0)) - 1;
  digit = 255u - (uint32_t)(4 * src + (int)rd_lane((uint32_t)found, src));
  rem = (int)rd_lane((uint32_t)nrem, src);
  cnt = (int)rd_lane((uint32_t)fcnt, src);
  wave_lds_sync();
}

// Float wave reductions (DPP within rows of 16 lanes, then the four row results).
template <int SHIFT>
__device__ __forceinline__ float row_shr_f(float old, float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(old), __float_as_int(v), 0x110 + SHIFT,
                                                    0xf, 0xf, false));
}
__device__ __forceinline__ float rd_lane_f(float v, int l) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), l));
}
__device__ __forceinline__ float wave_fmax(float v) {
  v = fmaxf(v, row_shr_f<1>(-INFINITY, v));
  v = fmaxf(v, row_shr_f<2>(-INFINITY, v));
  v = fmaxf(v, row_shr_f<4>(-INFINITY, v));
  v = fmaxf(v, row_shr_f<8>(-INFINITY, v));
  return fmaxf(fmaxf(rd_lane_f(v, 15), rd_lane_f(v, 31)), fmaxf(rd_lane_f(v, 47), rd_lane_f(v, 63)));
}
__device__ __forceinline__ float wave_fmin(float v) {
  v = fminf(v, row_shr_f<1>(INFINITY, v));
  v = fminf(v, row_shr_f<2>(INFINITY, v));
  v = fminf(v, row_shr_f<4>(INFINITY, v));
  v = fminf(v, row_shr_f<8>(INFINITY, v));
  return fminf(fminf(rd_lane_f(v, 15), rd_lane_f(v, 31)), fminf(rd_lane_f(v, 47), rd_lane_f(v, 63)));
}

// Emission modes of the register path.
enum SelMode { SEL_WHOLE = 0, SEL_CUT = 1, SEL_EQ = 2 };

// Selection: one wave per (group, query block).  Rows of up to 64 * SEL_REG
// candidates are read once into registers; longer rows re-read the scores in
// each of four fixed 8-bit steps.
constexpr int SEL_REG = 20;

// Rank the members of the cut bin (at most 64, collected in ascending block
// order into LDS) by (key descending, block ascending) and return the one of
// rank rem - 1: its key and block.
__device__ __forceinline__ void rank_members(SelLds& w, int lane, int cnt, int rem, uint32_t& cut_key,
                                             int& cut_j) {
  wave_lds_sync();
  const uint32_t K = lane < cnt ? w.mkey[lane] : 0u;
  const int J = lane < cnt ? w.mj[lane] : 0;
  int rank = 0;
  for (int m = 0; m < cnt; ++m) {
    const uint32_t Km = rd_lane(K, m);
    rank += (Km > K || (Km == K && m < lane)) ? 1 : 0;
  }
  const int src = __ffsll((unsigned long long)__ballot(lane < cnt && rank == rem - 1)) - 1;
  cut_key = rd_lane(K, src);
  cut_j = (int)rd_lane((uint32_t)J, src);
  wave_lds_sync();
}

// The first step on a row held in registers: 256 bins of equal width over
// [min, max] of the row's scores, bin(s) = min(255, (int)((max - s) * 256 /
// (max - min))).  Rounding is monotone, so bin(s) is non-increasing in s and a
// score in a lower bin is strictly larger than every score in a higher one:
// the bins refine the order (score descending, block ascending).  One
// histogram locates the bin of the (k-1)-th key; a bin holding at most 64
// keys is ranked exactly.  Rows whose range is not finite, or whose cut bin is
// larger, take the radix steps on order-preserving integer keys instead.
__global__ __launch_bounds__(256) void select_kernel(const float* __restrict__ scores,
                                                     int32_t* __restrict__ q2k_idx,
                                                     int32_t* __restrict__ q2k_cnt, Geo g) {
  __shared__ SelLds lds[4];
  const int lane = threadIdx.x & 63;
  // wave-uniform, so that every per-row value below lives in scalar registers
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t row = (int64_t)blockIdx.x * 4 + wave;
  if (row >= (int64_t)g.Hkv * g.nqb) return;      // no workgroup barriers in this kernel
  const int grp = (int)(row / g.nqb);
  const int QB = (int)(row % g.nqb);
  const int b = g.qdoc[QB];
  const int I = QB - g.qb0[b];
  const int L = g.cu[b + 1] - g.cu[b];
  const int nk = (L + 127) >> 7;
  const int kb0 = g.kb0[b];
  const int diag = (I * g.Bq) >> 7;
  int32_t* out = q2k_idx + ((int64_t)grp * g.nqb + QB) * g.stride;
  SelLds& w = lds[wave];
  int pos = 0;
  const int pool = diag - g.span;                 // candidates: blocks below the window's span
  if (pool <= g.topk - 1) {                       // all of them are taken
    for (int j = lane; j < pool; j += 64) out[j] = kb0 + j;
    pos = pool > 0 ? pool : 0;
  } else if (g.topk > 1) {
    const int ncand = pool;
    const float* srow = scores + (int64_t)grp * g.score_elems + g.s0[b] + (int64_t)I * nk;
    int rem = g.topk - 1;
    // emit the taken candidates in ascending block order (ballot prefix)
    auto emit = [&](int r, bool take) __attribute__((always_inline)) {
      const int j = r * 64 + lane;
      const uint64_t tm = __ballot(take);
      if (take) out[pos + __popcll(tm & lanes_below(lane))] = kb0 + j;
      pos += __popcll(tm);
    };
    if (ncand <= 64 * SEL_REG) {
      // the row through a buffer descriptor: lane offsets are immediates and
      // reads past the row's end return zero (and are marked invalid)
      const __amdgpu_buffer_rsrc_t rs =
          __builtin_amdgcn_make_buffer_rsrc((void*)srow, (short)0, ncand * 4, 0x00020000);
      // all of the row's loads are issued before the first is used
      uint32_t key[SEL_REG];
#pragma unroll
      for (int r = 0; r < SEL_REG; ++r)
        if (r * 64 < ncand) key[r] = __builtin_amdgcn_raw_buffer_load_b32(rs, lane * 4 + r * 256, 0, 0);
      float fhi = -INFINITY, flo = INFINITY;
#pragma unroll
      for (int r = 0; r < SEL_REG; ++r) {
        if (r * 64 >= ncand) break;
        const float sv = __builtin_bit_cast(float, key[r]);
        const bool valid = r * 64 + lane < ncand;
        fhi = fmaxf(fhi, valid ? sv : -INFINITY);
        flo = fminf(flo, valid ? sv : INFINITY);
      }
      fhi = wave_fmax(fhi);
      flo = wave_fmin(flo);
      const float inv = 256.f / (fhi - flo);
      bool done = false;
      if (fhi - flo <= 3.0e38f && inv <= 3.0e38f) {     // finite, non-zero range
        uint32_t bins[(SEL_REG + 3) / 4];                 // one byte per key
        hist_clear(w, lane);
#pragma unroll
        for (int r = 0; r < SEL_REG; ++r) {
          if (r * 64 >= ncand) break;
          const float sv = __builtin_bit_cast(float, key[r]);
          const int bn = min(255, max(0, (int)((fhi - sv) * inv)));
          if ((r & 3) == 0) bins[r >> 2] = 0u;
          bins[r >> 2] |= (uint32_t)bn << (8 * (r & 3));
          if (r * 64 + lane < ncand) atomicAdd(&w.hist[bn], 1u);
        }
        uint32_t digit;
        int cnt;
        int brem = rem;
        radix_pick(w, lane, digit, brem, cnt);        // hist[i] holds bin i: bin = 255 - digit
        const uint32_t bstar = 255u - digit;
        if (cnt == brem) {                            // the cut bin is taken whole
#pragma unroll
          for (int r = 0; r < SEL_REG; ++r) {
            if (r * 64 >= ncand) break;
            const uint32_t bn = (bins[r >> 2] >> (8 * (r & 3))) & 255u;
            emit(r, r * 64 + lane < ncand && bn <= bstar);
          }
          done = true;
        } else if (cnt <= 64) {
          int base = 0;
#pragma unroll
          for (int r = 0; r < SEL_REG; ++r) {
            if (r * 64 >= ncand) break;
            const int j = r * 64 + lane;
            const uint32_t bn = (bins[r >> 2] >> (8 * (r & 3))) & 255u;
            const bool in = j < ncand && bn == bstar;
            const uint64_t m = __ballot(in);
            if (in) {
              const int p = base + __popcll(m & lanes_below(lane));
              w.mkey[p] = order_key(__builtin_bit_cast(float, key[r]));
              w.mj[p] = j;
            }
            base += __popcll(m);
          }
          uint32_t cut_key;
          int cut_j;
          rank_members(w, lane, cnt, brem, cut_key, cut_j);
#pragma unroll
          for (int r = 0; r < SEL_REG; ++r) {
            if (r * 64 >= ncand) break;
            const int j = r * 64 + lane;
            const uint32_t bn = (bins[r >> 2] >> (8 * (r & 3))) & 255u;
            const uint32_t kv = order_key(__builtin_bit_cast(float, key[r]));
            emit(r, j < ncand && (bn < bstar || (bn == bstar && (kv > cut_key || (kv == cut_key && j <= cut_j)))));
          }
          done = true;
        }
      }
      if (!done) {
        // radix steps over 8-bit windows of order-preserving keys, the first
        // at the highest bit where the row's keys differ
#pragma unroll
        for (int r = 0; r < SEL_REG; ++r) {
          if (r * 64 >= ncand) break;
          key[r] = r * 64 + lane < ncand ? order_key(__builtin_bit_cast(float, key[r])) : 0u;
        }
        uint32_t kmin = 0xffffffffu, kmax = 0u;
#pragma unroll
        for (int r = 0; r < SEL_REG; ++r) {
          if (r * 64 >= ncand) break;
          kmin = min(kmin, r * 64 + lane < ncand ? key[r] : 0xffffffffu);
          kmax = max(kmax, key[r]);
        }
        kmin = wave_min(kmin);
        kmax = wave_max(kmax);
        int mode = SEL_EQ;
        uint32_t cut_key = 0, prefix = 0, pmask = 0;
        int cut_j = 0;
        if (kmin == kmax) {
          prefix = kmin;                            // all keys equal: lowest indices win
          pmask = 0xffffffffu;
        } else {
          int top = 31 - __clz(kmin ^ kmax);        // highest bit where the keys differ
          pmask = ~((2u << top) - 1u);              // 0 when top is 31
          prefix = kmin & pmask;
          for (;;) {
            const int lo = top >= 7 ? top - 7 : 0;
            const uint32_t wmask = ((2u << top) - 1u) & ~((1u << lo) - 1u);
            hist_clear(w, lane);
#pragma unroll
            for (int r = 0; r < SEL_REG; ++r) {
              if (r * 64 >= ncand) break;
              if (r * 64 + lane < ncand && (key[r] & pmask) == prefix)
                atomicAdd(&w.hist[255u - ((key[r] >> lo) & 255u)], 1u);
            }
            uint32_t digit;
            int cnt;
            radix_pick(w, lane, digit, rem, cnt);
            prefix |= (digit << lo) & wmask;
            pmask |= wmask;
            if (cnt == rem) { mode = SEL_WHOLE; break; }
            if (cnt <= 64) {
              // rank the bin's members (collected in ascending block order)
              int base = 0;
#pragma unroll
              for (int r = 0; r < SEL_REG; ++r) {
                if (r * 64 >= ncand) break;
                const int j = r * 64 + lane;
                const bool in = j < ncand && (key[r] & pmask) == prefix;
                const uint64_t m = __ballot(in);
                if (in) {
                  const int p = base + __popcll(m & lanes_below(lane));
                  w.mkey[p] = key[r];
                  w.mj[p] = j;
                }
                base += __popcll(m);
              }
              rank_members(w, lane, cnt, rem, cut_key, cut_j);
              mode = SEL_CUT;
              break;
            }
            if (lo == 0) break;                     // the whole key is decided: equal keys by index
            top = lo - 1;
          }
        }
        int eq_taken = 0;
#pragma unroll
        for (int r = 0; r < SEL_REG; ++r) {
          if (r * 64 >= ncand) break;
          const int j = r * 64 + lane;
          const bool valid = j < ncand;
          bool take;
          if (mode == SEL_WHOLE) {
            take = valid && (key[r] & pmask) >= prefix;
          } else if (mode == SEL_CUT) {
            take = valid && (key[r] > cut_key || (key[r] == cut_key && j <= cut_j));
          } else {
            const bool eq = valid && key[r] == prefix;
            const uint64_t eqm = __ballot(eq);
            const int eq_rank = eq_taken + __popcll(eqm & lanes_below(lane));
            take = (valid && key[r] > prefix) || (eq && eq_rank < rem);
            eq_taken += __popcll(eqm);
          }
          emit(r, take);
        }
      }
    } else {
      // rows too long for registers: the same bins, the row re-read for each
      // step (it stays in cache), the radix steps over the whole key only
      // when the cut bin holds more than 64 keys or the range is not finite
      float fhi = -INFINITY, flo = INFINITY;
      for (int j = lane; j < ncand; j += 64) {
        const float sv = srow[j];
        fhi = fmaxf(fhi, sv);
        flo = fminf(flo, sv);
      }
      fhi = wave_fmax(fhi);
      flo = wave_fmin(flo);
      const float inv = 256.f / (fhi - flo);
      auto bin_of = [&](float sv) __attribute__((always_inline)) {
        return (uint32_t)min(255, max(0, (int)((fhi - sv) * inv)));
      };
      bool done = false;
      if (fhi - flo <= 3.0e38f && inv <= 3.0e38f) {
        hist_clear(w, lane);
        for (int j = lane; j < ncand; j += 64) atomicAdd(&w.hist[bin_of(srow[j])], 1u);
        uint32_t digit;
        int cnt;
        int brem = rem;
        radix_pick(w, lane, digit, brem, cnt);
        const uint32_t bstar = 255u - digit;
        if (cnt == brem) {
          for (int base = 0; base < ncand; base += 64) {
            const int j = base + lane;
            emit(base >> 6, j < ncand && bin_of(srow[j < ncand ? j : 0]) <= bstar);
          }
          done = true;
        } else if (cnt <= 64) {
          int nb = 0;
          for (int base = 0; base < ncand; base += 64) {
            const int j = base + lane;
            const float sv = srow[j < ncand ? j : 0];
            const bool in = j < ncand && bin_of(sv) == bstar;
            const uint64_t m = __ballot(in);
            if (in) {
              const int p = nb + __popcll(m & lanes_below(lane));
              w.mkey[p] = order_key(sv);
              w.mj[p] = j;
            }
            nb += __popcll(m);
          }
          uint32_t cut_key;
          int cut_j;
          rank_members(w, lane, cnt, brem, cut_key, cut_j);
          for (int base = 0; base < ncand; base += 64) {
            const int j = base + lane;
            const float sv = srow[j < ncand ? j : 0];
            const uint32_t bn = bin_of(sv), kv = order_key(sv);
            emit(base >> 6, j < ncand && (bn < bstar || (bn == bstar && (kv > cut_key || (kv == cut_key && j <= cut_j)))));
          }
          done = true;
        }
      }
      if (!done) {
        uint32_t prefix = 0, pmask = 0;
        for (int shift = 24; shift >= 0; shift -= 8) {
          hist_clear(w, lane);
          for (int j = lane; j < ncand; j += 64) {
            const uint32_t key = order_key(srow[j]);
            if ((key & pmask) == prefix) atomicAdd(&w.hist[255u - ((key >> shift) & 255u)], 1u);
          }
          uint32_t digit;
          int cnt;
          radix_pick(w, lane, digit, rem, cnt);
          prefix |= digit << shift;
          pmask |= 255u << shift;
        }
        int eq_taken = 0;
        for (int base = 0; base < ncand; base += 64) {
          const int j = base + lane;
          const uint32_t key = j < ncand ? order_key(srow[j]) : 0u;
          const bool valid = j < ncand;
          const bool gt = valid && key > prefix;
          const bool eq = valid && key == prefix;
          const uint64_t eqm = __ballot(eq);
          const int eq_rank = eq_taken + __popcll(eqm & lanes_below(lane));
          emit(base >> 6, gt || (eq && eq_rank < rem));
          eq_taken += __popcll(eqm);
        }
      }
    }
  }
  // forced: the diagonal and the window's blocks diag - i * dil (i <= lw, >= 0),
  // ascending; every one lies above the candidates
  const int nf = (g.lw < diag / g.dil ? g.lw : diag / g.dil) + 1;
  for (int t = lane; t < nf; t += 64) out[pos + t] = kb0 + diag - (nf - 1 - t) * g.dil;
  pos += nf;
  for (int j = pos + lane; j < g.stride; j += 64) out[j] = -1;
  if (lane == 0) q2k_cnt[(int64_t)grp * g.nqb + QB] = pos;
}

// ---------------------------------------------------------------------------
// inverted index: counts -> exclusive scan -> emission, with no atomics
// outside LDS.  The KV blocks of each document are cut into slabs of 256, and
// the rows (query blocks) that can select a slab's blocks -- those whose
// diagonal block is at or past the slab's first block -- into chunks of 256
// consecutive rows.  A workgroup owns one (group, slab, chunk): it counts the
// chunk's selections per block into a table, the scan turns the table into
// k2q_ptr, and the emission places each row of the chunk, in ascending row
// order, after the rows of earlier chunks.  Every list therefore comes out
// ascending, and the result is the same on every run.
// ---------------------------------------------------------------------------

struct SlabView {
  int grp, slab, chunk, jlo, ncol, r0, r1, qb0;
  uint32_t glo;                      // global id of the slab's first KV block
};

// Workgroup wg -> (group, slab, chunk); r0 >= r1 when the chunk lies past the
// slab's rows.
__device__ __forceinline__ SlabView slab_view(const Geo& g, int64_t wg) {
  SlabView v;
  v.chunk = (int)(wg % g.k2q_chunks);
  const int64_t gs = wg / g.k2q_chunks;
  v.grp = (int)(gs / g.nslab);
  v.slab = (int)(gs % g.nslab);
  const int b = find_segment<int32_t>(g.slab0, g.B, v.slab);
  v.jlo = (v.slab - g.slab0[b]) * K2Q_SLAB;
  const int L = g.cu[b + 1] - g.cu[b];
  const int nk = (L + 127) >> 7;
  v.ncol = min(K2Q_SLAB, nk - v.jlo);
  const int nq = (L + g.Bq - 1) / g.Bq;
  const int imin = (v.jlo * 128 + g.Bq - 1) / g.Bq;   // first row whose diagonal reaches the slab
  v.r0 = imin + v.chunk * K2Q_CHUNK;
  v.r1 = min(nq, v.r0 + K2Q_CHUNK);
  v.qb0 = g.qb0[b];
  v.glo = (uint32_t)(g.kb0[b] + v.jlo);
  return v;
}

// Count, into cnt[c], the rows in [i0, i1) that selected block glo + c of
// the slab (LDS adds; a row never holds a block twice).
__device__ __forceinline__ void slab_count_rows(const Geo& g, const int32_t* rows0, const SlabView& v, int i0,
                                                int i1, uint32_t* cnt, int lane) {
  constexpr int U = 8;                              // rows in flight per wave
  for (int I = i0; I < i1; I += U) {
    int32_t e[U][2];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int32_t* row = rows0 + (int64_t)(I + u) * g.stride;
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int k = h * 64 + lane;
        e[u][h] = (I + u < i1 && k < g.stride) ? row[k] : -1;
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const uint32_t c = (uint32_t)e[u][h] - v.glo;
        if (c < (uint32_t)K2Q_SLAB) atomicAdd(&cnt[c], 1u);
      }
    }
    for (int k = 128 + lane; k < g.stride; k += 64) {   // rows longer than 128 entries
#pragma unroll
      for (int u = 0; u < U; ++u) {
        if (I + u >= i1) break;
        const uint32_t c = (uint32_t)rows0[(int64_t)(I + u) * g.stride + k] - v.glo;
        if (c < (uint32_t)K2Q_SLAB) atomicAdd(&cnt[c], 1u);
      }
    }
  }
}

// table[((grp * nslab + slab) * k2q_chunks + chunk) * 64 + c] = selections of
// the slab's block c by the chunk's rows.
__global__ __launch_bounds__(256) void k2q_count_kernel(const int32_t* __restrict__ q2k_idx,
                                                        int32_t* __restrict__ table, Geo g) {
  __shared__ uint32_t cnt[K2Q_SLAB];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const SlabView v = slab_view(g, blockIdx.x);
  for (int c = tid; c < K2Q_SLAB; c += 256) cnt[c] = 0u;
  __syncthreads();
  const int32_t* rows0 = q2k_idx + ((int64_t)v.grp * g.nqb + v.qb0) * g.stride;
  const int w0 = v.r0 + wave * (K2Q_CHUNK / 4);
  slab_count_rows(g, rows0, v, w0, min(v.r1, w0 + K2Q_CHUNK / 4), cnt, lane);
  __syncthreads();
  for (int c = tid; c < K2Q_SLAB; c += 256) table[(int64_t)blockIdx.x * K2Q_SLAB + c] = (int32_t)cnt[c];
}

// Each KV block's count: the sum of its chunks' counts (one thread per block).
__global__ __launch_bounds__(256) void k2q_total_kernel(const int32_t* __restrict__ table,
                                                        int32_t* __restrict__ totals, Geo g) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= (int64_t)g.Hkv * g.nkb) return;
  const int grp = (int)(i / g.nkb);
  const int KB = (int)(i % g.nkb);
  const int b = g.kdoc[KB];
  const int J = KB - g.kb0[b];
  const int slab = g.slab0[b] + J / K2Q_SLAB;
  const int32_t* tc = table + ((int64_t)grp * g.nslab + slab) * g.k2q_chunks * K2Q_SLAB + (J % K2Q_SLAB);
  int32_t c = 0;
  for (int ch = 0; ch < g.k2q_chunks; ++ch) c += tc[ch * K2Q_SLAB];
  totals[i] = c;
}

// Exclusive scan of one group's totals into k2q_ptr (nkb + 1 entries), one
// workgroup of 1024 threads per group: every thread sums a contiguous run,
// the run sums are scanned by DPP within waves and then over the 16 wave
// totals, and each run is written out; -1 fills the unused capacity.
__global__ __launch_bounds__(1024) void k2q_scan_kernel(const int32_t* __restrict__ totals,
                                                        int32_t* __restrict__ k2q_ptr,
                                                        int32_t* __restrict__ k2q_idx, Geo g) {
  __shared__ uint32_t wsum[16];
  __shared__ uint32_t total;
  const int grp = blockIdx.x;
  const int n = g.nkb;
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int per = (n + 1 + 1023) / 1024;
  const int lo = t * per, hi = min(lo + per, n);
  const int32_t* c = totals + (int64_t)grp * n;
  uint32_t local = 0;
  for (int i = lo; i < hi; ++i) local += (uint32_t)c[i];
  const uint32_t incl = wave_incl_sum(local, lane);
  if (lane == 63) wsum[wave] = incl;
  __syncthreads();
  uint32_t before = 0;
  for (int v = 0; v < wave; ++v) before += wsum[v];
  uint32_t run = before + incl - local;
  int32_t* p = k2q_ptr + (int64_t)grp * (n + 1);
  for (int i = lo; i < min(lo + per, n + 1); ++i) {
    p[i] = (int32_t)run;
    if (i == n) total = run;
    if (i < n) run += (uint32_t)c[i];
  }
  __syncthreads();
  int32_t* dst = k2q_idx + (int64_t)grp * g.cap;
  for (int64_t i = (int64_t)total + t; i < g.cap; i += 1024) dst[i] = -1;
}

// Emission for one (group, slab, chunk): wave w owns rows [r0 + 64 w, r0 +
// 64 w + 64); its place in each block's list starts after k2q_ptr, the earlier
// chunks (from the table) and the earlier waves (counted again here), and the
// wave walks its rows in ascending order, taking the next place of every slab
// block the row selected (an LDS add with return: one wave owns each counter).
__global__ __launch_bounds__(256) void k2q_emit_kernel(const int32_t* __restrict__ q2k_idx,
                                                       const int32_t* __restrict__ table,
                                                       const int32_t* __restrict__ k2q_ptr,
                                                       int32_t* __restrict__ k2q_idx, Geo g) {
  __shared__ uint32_t part[4][K2Q_SLAB];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const SlabView v = slab_view(g, blockIdx.x);
  if (v.r0 >= v.r1) return;                        // uniform over the workgroup
  const int w0 = v.r0 + wave * (K2Q_CHUNK / 4), w1 = min(v.r1, w0 + K2Q_CHUNK / 4);
#pragma unroll
  for (int m = 0; m < K2Q_SLAB / 64; ++m) part[wave][m * 64 + lane] = 0u;
  __syncthreads();
  const int32_t* rows0 = q2k_idx + ((int64_t)v.grp * g.nqb + v.qb0) * g.stride;
  slab_count_rows(g, rows0, v, w0, w1, part[wave], lane);
  __syncthreads();
  uint32_t start[K2Q_SLAB / 64];
#pragma unroll
  for (int m = 0; m < K2Q_SLAB / 64; ++m) {
    const int c = m * 64 + lane;
    start[m] = 0u;
    if (c < v.ncol) {
      uint32_t st = (uint32_t)k2q_ptr[(int64_t)v.grp * (g.nkb + 1) + v.glo + c];
      const int32_t* tc = table + ((int64_t)blockIdx.x - v.chunk) * K2Q_SLAB + c;
      for (int ch = 0; ch < v.chunk; ++ch) st += (uint32_t)tc[ch * K2Q_SLAB];
      for (int w = 0; w < wave; ++w) st += part[w][c];
      start[m] = st;
    }
  }
  __syncthreads();
#pragma unroll
  for (int m = 0; m < K2Q_SLAB / 64; ++m) part[wave][m * 64 + lane] = start[m];   // the wave's next places
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
  __builtin_amdgcn_wave_barrier();
  int32_t* dst = k2q_idx + (int64_t)v.grp * g.cap;
  constexpr int U = 8;
  for (int I = w0; I < w1; I += U) {
    int32_t e[U][2];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int32_t* row = rows0 + (int64_t)(I + u) * g.stride;
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int k = h * 64 + lane;
        e[u][h] = (I + u < w1 && k < g.stride) ? row[k] : -1;
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const uint32_t c = (uint32_t)e[u][h] - v.glo;
        if (c < (uint32_t)K2Q_SLAB) dst[atomicAdd(&part[wave][c], 1u)] = v.qb0 + I + u;
      }
    }
    for (int k = 128 + lane; k < g.stride; k += 64) {
#pragma unroll
      for (int u = 0; u < U; ++u) {
        if (I + u >= w1) break;
        const uint32_t c = (uint32_t)rows0[(int64_t)(I + u) * g.stride + k] - v.glo;
        if (c < (uint32_t)K2Q_SLAB) dst[atomicAdd(&part[wave][c], 1u)] = v.qb0 + I + u;
      }
    }
  }
}

static int grid_for(int64_t n, int threads) {
  int64_t b = (n + threads - 1) / threads;
  if (b < 1) b = 1;
  if (b > 65536) b = 65536;
  return (int)b;
}

hipError_t launch_select(const Geo& g, const float* scores, int32_t* q2k_idx, int32_t* q2k_cnt,
                         int32_t* k2q_ptr, int32_t* k2q_idx, const Work& w, hipStream_t s) {
  hipError_t e;
  const int64_t rows = (int64_t)g.Hkv * g.nqb;
  if (rows > 0) {
    { ProfScope _ps("select", s);
    hipLaunchKernelGGL(select_kernel, dim3((unsigned)((rows + 3) / 4)), dim3(256), 0, s, scores,
                       q2k_idx, q2k_cnt, g); }
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  const int64_t nwg = (int64_t)g.Hkv * g.nslab * g.k2q_chunks;
  if (nwg > 0) {
    { ProfScope _ps("k2q_count", s);
    hipLaunchKernelGGL(k2q_count_kernel, dim3((unsigned)nwg), dim3(256), 0, s, q2k_idx, w.counts, g); }
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  const int64_t nc = (int64_t)g.Hkv * g.nkb;
  if (nc > 0) {
    { ProfScope _ps("k2q_scan", s);
    hipLaunchKernelGGL(k2q_total_kernel, dim3((unsigned)((nc + 255) / 256)), dim3(256), 0, s, w.counts,
                       w.totals, g); }
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  { ProfScope _ps("k2q_scan", s);
  hipLaunchKernelGGL(k2q_scan_kernel, dim3(g.Hkv), dim3(1024), 0, s, w.totals, k2q_ptr, k2q_idx, g); }
  if ((e = hipGetLastError()) != hipSuccess) return e;
  if (nwg > 0) {
    { ProfScope _ps("k2q_emit", s);
    hipLaunchKernelGGL(k2q_emit_kernel, dim3((unsigned)nwg), dim3(256), 0, s, q2k_idx, w.counts, k2q_ptr,
                       k2q_idx, g); }
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace msa

namespace msa {
int select_kernels(KernelEntry* out, int max) {
  const KernelEntry all[] = {
      {"proxy_scores<bf16,dp64,bq128>", (const void*)proxy_scores_lds_kernel<128>, 256, SC_LDS},
      {"proxy_scores<bf16,dp64,bq64>", (const void*)proxy_scores_lds_kernel<64>, 256, SC_LDS},
      {"proxy_scores<bf16,dp32,bq64>", (const void*)proxy_scores_kernel<bf16, 32, 64>, 256, 0},
      {"proxy_scores<bf16,dp32,bq128>", (const void*)proxy_scores_kernel<bf16, 32, 128>, 256, 0},
      {"proxy_scores<f32,dp32,bq64>", (const void*)proxy_scores_kernel<float, 32, 64>, 256, 0},
      {"proxy_scores<f32,dp32,bq128>", (const void*)proxy_scores_kernel<float, 32, 128>, 256, 0},
      {"select", (const void*)select_kernel, 256, 0},
      {"k2q_count", (const void*)k2q_count_kernel, 256, 0},
      {"k2q_total", (const void*)k2q_total_kernel, 256, 0},
      {"k2q_scan", (const void*)k2q_scan_kernel, 1024, 0},
      {"k2q_emit", (const void*)k2q_emit_kernel, 256, 0},
  };
  int n = (int)(sizeof(all) / sizeof(all[0]));
  for (int i = 0; i < n && i < max; ++i) out[i] = all[i];
  return n;
}
}  // namespace msa
