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
// Work split: a work item is one (KV group, query block), or a half of one
// when it holds more than the workgroup's waves' worth of 32-query units.  For
// bf16 and d = 128 the grid is persistent (one workgroup of eight waves per
// CU, taking items from per-XCD work queues) and each selected KV block is
// staged through an LDS ring in two 64-key halves (K and V rows) by DMA; other
// shapes run one workgroup of four waves per item, double-buffered with a
// register prefetch.  V^T fragments come from the row-major V tile through
// LDS transpose reads.  A wave owns QT x 32 queries of one head and computes
// S^T = K Q^T on bf16 MFMA so that each lane holds one query column; the
// probabilities then feed O^T += V^T P^T without leaving registers.  The proxy log-sum-exp over the
// same keys is a separate light kernel (one proxy head per group, dp-deep
// contractions), which keeps the main kernel's registers for attention.
#include "msa_device.h"
#include "msa_internal.h"
#include "msa_profile.h"

#include <type_traits>

namespace msa {

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

template <typename T, int D, int DP, int QT, int NW>
struct FwdCfg {
  static constexpr int NT = 64 * NW;                     // threads per workgroup
  static constexpr int KC = 64;                          // keys per stage
  typedef Tile<T, D> TK;                                 // K and V rows, swizzled
  static constexpr int KS = KC * D;
  static constexpr int STAGE = 2 * KS;
  static constexpr int NBUF = 3;                         // LDS ring (two stages in flight)
  static constexpr int LDS_BYTES = NBUF * STAGE * (int)sizeof(T);
  static constexpr int EPC = TK::EPC, CPR = TK::CPR;
  static constexpr int NK = KC * CPR / NT;               // chunks per thread per tensor
};

template <typename U>
struct TypeTag { using type = U; };

template <typename T, int D, int DP, int QT, int NW>
__global__ __launch_bounds__(64 * NW) void fwd_kernel(
    const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ v,
    const int32_t* __restrict__ q2k_idx, const int32_t* __restrict__ q2k_cnt,
    T* __restrict__ o, float* __restrict__ lse, int32_t* __restrict__ queue, Geo g) {
  typedef FwdCfg<T, D, DP, QT, NW> C;
  typedef typename C::TK TK;
  extern __shared__ __align__(16) unsigned char smem_raw[];
  T* smem = reinterpret_cast<T*>(smem_raw);
  constexpr int NT = C::NT;
  static_assert(C::NK >= 1, "tile split");

  const int tid = threadIdx.x, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int NU = g.G * (g.Bq / (32 * QT));
  const int nwg = (NU + NW - 1) / NW;
  // bf16, d = 128: a persistent grid over a work queue (below); other shapes:
  // one workgroup per item
  constexpr bool PERSIST = sizeof(T) == 2 && D == 128;

  // One work item: a workgroup's share of one (KV group, query block).
  auto body = [&](const int bid) __attribute__((always_inline)) {
  // lane values from an opaque copy of the lane index in the persistent
  // kernel, so that they are formed per item rather than kept live across
  // items
  int lane = tid & 63;
  if constexpr (PERSIST) asm volatile("" : "+v"(lane));
  const int col = lane & 31, hi = lane >> 5;
  const int64_t item = bid / nwg;
  const int wgi = bid % nwg;
  const int grp = (int)(item / g.nqb);
  const int QB = (int)(item % g.nqb);
  const int u = wgi * NW + wave;
  const bool active = u < NU;
  const int hl = u % g.G, chunk = u / g.G;
  const int h = grp * g.G + hl;

  const int b = g.qdoc[QB];
  const int I = QB - g.qb0[b];
  const int t0 = g.cu[b];
  const int L = g.cu[b + 1] - t0;
  const int kb0 = g.kb0[b];
  const int diag = (I * g.Bq) >> 7;
  const int qbase = I * g.Bq + chunk * 32 * QT;
  const int64_t rowi = (int64_t)proxy_head(g, grp) * g.nqb + QB;   // the group's block list
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

  // Stages are 64-key halves of the selected blocks, ascending; the diagonal
  // block (always the last) needs the causal mask, the others never do.  Its
  // second half is dropped when every query of the block precedes it.
  int nst = 2 * cnt;
  if (diag * 128 + 64 > I * g.Bq + g.Bq - 1) nst -= 1;
  const int nst_plain = 2 * (cnt - 1);

  uint4 Kr[C::NK], Vr[C::NK];
  auto load_stage = [&](int s) __attribute__((always_inline)) {
    const int J = sel[s >> 1] - kb0;
    const int key0 = J * 128 + (s & 1) * C::KC;
#pragma unroll
    for (int i = 0; i < C::NK; ++i) {
      const int c = tid + NT * i, r = c / C::CPR, cc = c % C::CPR, key = key0 + r;
      const int64_t off = ((int64_t)(t0 + key) * g.Hkv + grp) * D + cc * C::EPC;
      Kr[i] = key < L ? *reinterpret_cast<const uint4*>(k + off) : make_uint4(0, 0, 0, 0);
      Vr[i] = key < L ? *reinterpret_cast<const uint4*>(v + off) : make_uint4(0, 0, 0, 0);
    }
  };
  auto store_stage = [&](int buf) __attribute__((always_inline)) {
    T* Ks = smem + buf * C::STAGE;
    T* Vs = Ks + C::KS;
#pragma unroll
    for (int i = 0; i < C::NK; ++i) {
      const int c = tid + NT * i, r = c / C::CPR, cc = c % C::CPR;
      *reinterpret_cast<uint4*>(Ks + TK::off(r, cc * C::EPC)) = Kr[i];
      *reinterpret_cast<uint4*>(Vs + TK::off(r, cc * C::EPC)) = Vr[i];
    }
  };

  // S^T = K Q^T for 32 keys (rows) of the stage in buffer Ks, masked if asked
  auto scores = [&](const T* Ks, int kt, int kpos, bool masked, f32x16 (&S)[QT]) __attribute__((always_inline)) {
#pragma unroll
    for (int qt = 0; qt < QT; ++qt) S[qt] = zero16();
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) {
      const frag_t<T> a = TK::row8(Ks, kt * 32 + col, ks * 16 + hi * 8);
#pragma unroll
      for (int qt = 0; qt < QT; ++qt) mma(S[qt], a, Qf[qt][ks]);
    }
    if (masked) {
#pragma unroll
      for (int qt = 0; qt < QT; ++qt) {
        const int lim = qbase + qt * 32 + col - kpos;    // key row r visible iff r <= lim
#pragma unroll
        for (int i = 0; i < 16; ++i) S[qt][i] = acc_row(i, lane) <= lim ? S[qt][i] : -INFINITY;
      }
    }
  };

  // Accumulation with a fixed reference maximum mref (base 2) per query
  // column: P = exp2(s * scale_log2 - mref), l += sum P, O^T += V^T P^T.  No
  // rescaling: with mref taken from real scores of the row, P stays finite
  // unless a later score exceeds it by ~128 (base 2); l is checked afterwards.
  f32x16 O[D / 32][QT];
  float l[QT], mref[QT], mtrue[QT];
  auto accumulate = [&](const T* Ks, const T* Vs, int kt, int kpos, bool masked) __attribute__((always_inline)) {
    f32x16 S[QT];
    scores(Ks, kt, kpos, masked, S);
#pragma unroll
    for (int qt = 0; qt < QT; ++qt) {
      float ls = 0.f;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const float p = __builtin_amdgcn_exp2f(fmaf(S[qt][i], g.scale_log2, -mref[qt]));
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
        const frag_t<T> a = TK::col(Vs, kt * 32 + kk * 16, dt * 32, lane);
#pragma unroll
        for (int qt = 0; qt < QT; ++qt) mma(O[dt][qt], a, Pf[kk][qt]);
      }
    }
  };
  auto row_max = [&](const f32x16 (&S)[QT], float (&mx)[QT]) __attribute__((always_inline)) {
#pragma unroll
    for (int qt = 0; qt < QT; ++qt) {
      float m = NEG_BIG;
#pragma unroll
      for (int i = 0; i < 16; ++i) m = fmaxf(m, S[qt][i]);
      mx[qt] = fmaxf(m, __shfl_xor(m, 32, 64)) * g.scale_log2;
    }
  };
  auto track_max = [&](const T* Ks, const T* Vs, int kt, int kpos, bool masked) __attribute__((always_inline)) {
    f32x16 S[QT];
    float mx[QT];
    scores(Ks, kt, kpos, masked, S);
    row_max(S, mx);
#pragma unroll
    for (int qt = 0; qt < QT; ++qt) mtrue[qt] = fmaxf(mtrue[qt], mx[qt]);
  };

  // The accumulation of one 64-key stage (bf16, d = 128) as a fixed sequence
  // of MFMAs, each pair (the two query tiles) sharing one operand read from
  // LDS: S of key tile 0 (K rows), S of tile 1, then P V of tile 0 (V^T
  // fragments), then of tile 1.  Every operand is read LOOK pairs ahead of
  // its use; tile 0's exponentials run between tile 1's S products and tile
  // 1's between tile 0's P V products; scheduling fences keep that order.
  constexpr bool FAST = sizeof(T) == 2 && D == 128;
  // This lane's LDS reads in a stage: the K row fragment of 16-column step
  // ks sits at oRow ^ (ks << 5), and the two transpose reads of the V^T
  // fragment of 32-column block dt at oColV ^ (dt << 6) and at that ^ 32 plus
  // 8 rows (the swizzle is an XOR of the chunk index with a function of the
  // row; rows 8 further down flip its bit 1).
  uint32_t oRow = 0, oColV = 0;
  if constexpr (FAST) {
    const int s16 = lane & 15, g4 = lane >> 4;
    const int tr_r = hi * 4 + (s16 >> 2), tr_c = 16 * (g4 & 1) + 4 * (s16 & 3);
    oRow = TK::off(col, hi * 8) * (int)sizeof(T);
    oColV = (C::KS + TK::off(tr_r, tr_c)) * (int)sizeof(T);
  }
  // (the element type comes in as a tag so that the body is type-checked only
  // where it is used, with bf16)
  auto stage_fast = [&](int buf, int kpos0, auto masked_c, auto tag) __attribute__((always_inline)) {
    using TT = typename decltype(tag)::type;
    constexpr bool MASKED = decltype(masked_c)::value;
    constexpr int NA = D / 16;                      // S operands per key tile
    constexpr int NB = 2 * (D / 32);                // P V operands per key tile
    constexpr int NO = 2 * NA + 2 * NB;
    constexpr int LOOK = 4;
    const uint32_t sb = (uint32_t)__builtin_amdgcn_readfirstlane(
        (int)(lds_offset(smem_raw) + buf * C::STAGE * (int)sizeof(T)));
    const uint32_t bRow = lds_base_add(sb, oRow), bCol = lds_base_add(sb, oColV);
    uint32_t aRow[D / 16], aCol[D / 32][2];
    static_for<D / 16>([&](auto kc) __attribute__((always_inline)) {
      constexpr int ks = decltype(kc)::value;
      aRow[ks] = xr<(uint32_t)(ks << 5)>(bRow);
    });
    static_for<D / 32>([&](auto dc) __attribute__((always_inline)) {
      constexpr int dt = decltype(dc)::value;
      aCol[dt][0] = xr<(uint32_t)(dt << 6)>(bCol);
      aCol[dt][1] = xr<(uint32_t)(dt << 6) ^ 32u>(bCol) + 8u * D * (uint32_t)sizeof(T);
    });
    f32x16 S[2][QT];
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int qt = 0; qt < QT; ++qt) S[kt][qt] = zero16();
    frag_t<TT> Pf[2][2][QT];
    frag_t<TT> opnd[NO];
    float ls[QT];
#pragma unroll
    for (int qt = 0; qt < QT; ++qt) ls[qt] = 0.f;
    int lim[QT];
#pragma unroll
    for (int qt = 0; qt < QT; ++qt) lim[qt] = qbase + qt * 32 + col - kpos0;
    auto operand = [&](auto mc) __attribute__((always_inline)) {
      constexpr int m = decltype(mc)::value;
      if constexpr (m < 2 * NA) {
        constexpr int kt = m / NA, ks = m % NA;
        opnd[m] = lds_ld8<kt * 32 * D * 2>(aRow[ks]);
      } else {
        constexpr int r = m - 2 * NA, kt = r / NB, dt = (r % NB) / 2, kk = (r % NB) % 2;
        opnd[m] = tr_pair_at<(kt * 32 + kk * 16) * D * 2>(aCol[dt][0], aCol[dt][1]);
      }
    };
    auto product = [&](auto mc) __attribute__((always_inline)) {
      constexpr int m = decltype(mc)::value;
      if constexpr (m < 2 * NA) {
        constexpr int kt = m / NA, ks = m % NA;
#pragma unroll
        for (int qt = 0; qt < QT; ++qt) mma(S[kt][qt], opnd[m], Qf[qt][ks]);
      } else {
        constexpr int r = m - 2 * NA, kt = r / NB, dt = (r % NB) / 2, kk = (r % NB) % 2;
#pragma unroll
        for (int qt = 0; qt < QT; ++qt) mma(O[dt][qt], opnd[m], Pf[kt][kk][qt]);
      }
    };
    // softmax element e (of 2 x 16) of key tile kt
    auto soft = [&](int kt, int e) __attribute__((always_inline)) {
      const int qt = e >> 4, i = e & 15;
      float p = __builtin_amdgcn_exp2f(fmaf(S[kt][qt][i], g.scale_log2, -mref[qt]));
      if (MASKED) p = acc_row(i, lane) <= lim[qt] - kt * 32 ? p : 0.f;
      S[kt][qt][i] = p;
      ls[qt] += p;
    };
    auto pack = [&](int kt) __attribute__((always_inline)) {
#pragma unroll
      for (int kk = 0; kk < 2; ++kk)
#pragma unroll
        for (int qt = 0; qt < QT; ++qt) Pf[kt][kk][qt] = acc_frag<TT>(S[kt][qt], kk);
    };
    static_for<LOOK>([&](auto mc) __attribute__((always_inline)) { operand(mc); });
    static_for<NO>([&](auto mc) __attribute__((always_inline)) {
      constexpr int m = decltype(mc)::value;
      product(mc);
      if constexpr (m + LOOK < NO) operand(std::integral_constant<int, m + LOOK>());
      if constexpr (m >= NA && m < 2 * NA) {
        constexpr int e0 = (m - NA) * QT * 16 / NA, e1 = (m - NA + 1) * QT * 16 / NA;
#pragma unroll
        for (int e = e0; e < e1; ++e) soft(0, e);
        if constexpr (m == 2 * NA - 1) pack(0);
      } else if constexpr (m >= 2 * NA && m < 2 * NA + NB) {
        constexpr int e0 = (m - 2 * NA) * QT * 16 / NB, e1 = (m - 2 * NA + 1) * QT * 16 / NB;
#pragma unroll
        for (int e = e0; e < e1; ++e) soft(1, e);
        if constexpr (m == 2 * NA + NB - 1) pack(1);
      }
      __builtin_amdgcn_sched_barrier(0);
    });
#pragma unroll
    for (int qt = 0; qt < QT; ++qt) l[qt] += ls[qt];
  };
  // The main pass with a DMA ring: stage s (64 keys of K and V) is copied
  // into slot s % 3 two stages ahead; every thread issues C::NK copies per
  // tensor per stage (past the last stage it re-copies the last one), which
  // the vmcnt waits count.  Keys past the document end (the last block only)
  // are clamped to its last key: they lie above every query of the block, so
  // the causal mask drops them.  The reference maxima come from stage 0.
  auto pass_ring = [&](auto tag) __attribute__((always_inline)) {   // built only where called
    const uint32_t lds0 = lds_offset(smem_raw);
    // copies through buffer descriptors over the stage's rows: each lane's
    // byte offset is fixed; a stage running past the document end has its rows
    // past the end clamped to the last one (a copy past a descriptor's bound
    // would leave its LDS row unwritten)
    const uint32_t rs = (uint32_t)g.Hkv * D * (uint32_t)sizeof(T);
    uint32_t vo[C::NK];
    int rr[C::NK];
#pragma unroll
    for (int i = 0; i < C::NK; ++i) {
      const int c = i * NT + tid, r = c / C::CPR, p = c % C::CPR;
      rr[i] = r;
      vo[i] = (uint32_t)r * rs + (uint32_t)(swz<C::CPR>(r, p) * 16);
    }
    auto issue = [&](int st) __attribute__((always_inline)) {
      const int sc = st < nst ? st : nst - 1;
      const int key0 = (sel[sc >> 1] - kb0) * 128 + (sc & 1) * C::KC;
      const uint32_t base = lds0 + (uint32_t)((st % C::NBUF) * C::STAGE * (int)sizeof(T));
      const int64_t row0 = (int64_t)(t0 + key0) * g.Hkv + grp;
      const int last = L - 1 - key0;
      const i32x4 sk = make_srd(k + row0 * D, (uint32_t)C::KC * rs);
      const i32x4 sv = make_srd(v + row0 * D, (uint32_t)C::KC * rs);
      uint32_t o[C::NK];
#pragma unroll
      for (int i = 0; i < C::NK; ++i) o[i] = vo[i];
      if (last < C::KC - 1) {
#pragma unroll
        for (int i = 0; i < C::NK; ++i)
          if (rr[i] > last) o[i] -= (uint32_t)(rr[i] - last) * rs;
      }
#pragma unroll
      for (int i = 0; i < C::NK; ++i) {
        const uint32_t dst = base + (uint32_t)((i * NT + wave * 64) * 16);
        bdma16(sk, o[i], dst);
        bdma16(sv, o[i], dst + (uint32_t)(C::KS * (int)sizeof(T)));
      }
    };
    wait_vmcnt<0>();                               // the Q fragments: the waits below count copies only
    issue(0);
    issue(1);
    wait_vmcnt<2 * C::NK>();
    __syncthreads();
    if (active) {
      f32x16 S0[QT];
      scores(smem, 0, (sel[0] - kb0) * 128, sel[0] - kb0 == diag, S0);
      row_max(S0, mref);
    }
    int s = 0;
    for (; s < nst_plain; ++s) {
      wait_vmcnt<2 * C::NK>();                     // stage s has landed
      __syncthreads();                             // everyone's, and slot (s + 2) % 3 is free
      issue(s + 2);
      if (active) stage_fast(s % C::NBUF, (sel[s >> 1] - kb0) * 128 + (s & 1) * C::KC, std::false_type(), tag);
    }
    for (; s < nst; ++s) {
      wait_vmcnt<2 * C::NK>();
      __syncthreads();
      issue(s + 2);
      if (active) stage_fast(s % C::NBUF, diag * 128 + (s & 1) * C::KC, std::true_type(), tag);
    }
    wait_vmcnt<0>();
    __syncthreads();
  };

  // One pass over every stage; stage 0 must already sit in buffer 0.  The
  // stage after the last re-reads the last one (valid memory) into the unused
  // buffer, so each loop body is straight-line.
  auto pass = [&](auto work) __attribute__((always_inline)) {
    int s = 0;
    for (; s < nst_plain; ++s) {
      const int buf = s & 1;
      load_stage(s + 1 < nst ? s + 1 : s);
      const T* Ks = smem + buf * C::STAGE;
      const T* Vs = Ks + C::KS;
      const int kpos0 = (sel[s >> 1] - kb0) * 128 + (s & 1) * C::KC;
      if (active) {
        work(Ks, Vs, 0, kpos0, false);
        work(Ks, Vs, 1, kpos0 + 32, false);
      }
      store_stage(buf ^ 1);
      __syncthreads();
    }
    for (; s < nst; ++s) {
      const int buf = s & 1;
      load_stage(s + 1 < nst ? s + 1 : s);
      const T* Ks = smem + buf * C::STAGE;
      const T* Vs = Ks + C::KS;
      const int kpos0 = diag * 128 + (s & 1) * C::KC;
      if (active) {
        work(Ks, Vs, 0, kpos0, true);
        work(Ks, Vs, 1, kpos0 + 32, true);
      }
      store_stage(buf ^ 1);
      __syncthreads();
    }
  };
  auto restage0 = [&]() __attribute__((always_inline)) {
    load_stage(0);
    store_stage(0);
    __syncthreads();
  };

#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
    for (int qt = 0; qt < QT; ++qt) O[dt][qt] = zero16();
#pragma unroll
  for (int qt = 0; qt < QT; ++qt) { l[qt] = 0.f; mref[qt] = NEG_BIG; mtrue[qt] = NEG_BIG; }

  // reference maximum: the first 32 keys of the list (never all masked for a
  // valid query: the list's lowest block starts at or before the query block)
  if constexpr (FAST) {
    pass_ring(TypeTag<T>());
  } else {
    restage0();
    if (active) {
      f32x16 S[QT];
      scores(smem, 0, (sel[0] - kb0) * 128, sel[0] - kb0 == diag, S);
      row_max(S, mref);
    }
    pass(accumulate);
  }

  // fallback when a later score exceeded the reference by too much (never for
  // ordinary inputs): find the true row maxima, then accumulate again
  bool bad = false;
  if (active) {
#pragma unroll
    for (int qt = 0; qt < QT; ++qt) {
      const float lt = l[qt] + __shfl_xor(l[qt], 32, 64);
      bad |= !(lt < 1.8446744e19f);                     // 2^64; also catches inf and nan
    }
  }
  if (__syncthreads_or(bad)) {
    restage0();
    pass(track_max);
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
      for (int qt = 0; qt < QT; ++qt) O[dt][qt] = zero16();
#pragma unroll
    for (int qt = 0; qt < QT; ++qt) { l[qt] = 0.f; mref[qt] = mtrue[qt]; }
    restage0();
    pass(accumulate);
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
      if (hi == 0) lse[(int64_t)h * g.T + t] = (mref[qt] + log2f(lt)) * LN2;
    }
  }
  };

  if constexpr (PERSIST) {
    // Items come from eight queues, one per XCD over a contiguous range of
    // items; a workgroup takes the next item of its own XCD's queue and, once
    // that is empty, of the others in turn (XCDs differ in speed by a few
    // percent, and a fixed split leaves the faster ones idle at the end).
    // Thread 0 takes it, a barrier hands it to every wave.  Every item ends
    // with a barrier after its last LDS read, so the next item's copies
    // cannot overwrite operands still in use.
    const uint32_t item_lds = lds_offset(smem_raw) + (uint32_t)C::LDS_BYTES;
    const int nitems = g.Hkv * g.nqb * nwg;
    int qi = 0;                                      // queues this workgroup has drained
    for (;;) {
      if (tid == 0)
        *reinterpret_cast<__attribute__((address_space(3))) int*>((uintptr_t)item_lds) =
            queue_take(queue, nitems, blockIdx.x % kQueues, qi);
      __syncthreads();
      const int bid = __builtin_amdgcn_readfirstlane(
          *reinterpret_cast<__attribute__((address_space(3))) const int*>((uintptr_t)item_lds));
      if (bid < 0) break;
      body(bid);
    }
  } else {
    body(xcd_remap(blockIdx.x, gridDim.x));
  }
}


// Proxy log-sum-exp over each query's selected keys: one wave per 32 queries
// of a (proxy head, query block), launched over the proxy heads' geometry
// (Hkv = Hp); kp tiles are read as A fragments straight from global memory
// (the waves of a workgroup walk the same blocks).
template <typename T, int DP>
__global__ __launch_bounds__(256, 4) void proxy_lse_kernel(const T* __restrict__ qp,
                                                        const T* __restrict__ kp,
                                                        const int32_t* __restrict__ q2k_idx,
                                                        const int32_t* __restrict__ q2k_cnt,
                                                        float* __restrict__ lse_p, Geo g) {
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int col = lane & 31, hi = lane >> 5;
  const int nwq = g.Bq / 32;                     // waves per query block
  const int per_wg = 4 / nwq;                    // query blocks per workgroup
  const int64_t item = (int64_t)xcd_remap(blockIdx.x, gridDim.x) * per_wg + wave / nwq;
  if (item >= (int64_t)g.Hkv * g.nqb) return;    // no barriers in this kernel
  const int c = wave % nwq;
  const int grp = (int)(item / g.nqb);
  const int QB = (int)(item % g.nqb);
  const int b = g.qdoc[QB];
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
    const T* sp = qp + ((int64_t)(t0 + qrow) * g.Hp + grp) * DP + hi * 8;
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
      const T* sk = kp + ((int64_t)(t0 + key) * g.Hp + grp) * DP + hi * 8;
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

// Proxy log-sum-exp for 128-row query blocks: a workgroup owns one (group,
// query block) and wave w its queries 32w .. 32w + 31, so all four waves walk
// the same list.  The kp rows of each selected block are copied once per
// workgroup into an LDS ring (three slots, two blocks in flight) and read as
// A fragments by every wave; one max and one rescale per block.
template <typename T, int DP>
struct LseCfg {
  typedef Tile<T, DP> TP;
  static constexpr int NBUF = 3, AHEAD = 2;
  static constexpr int SLOT = 128 * DP * (int)sizeof(T);          // one KV block of kp rows
  static constexpr int ROWS_PER_COPY = 64 / TP::CPR;               // rows one wave copy covers
  static constexpr int COPIES = 128 / (4 * ROWS_PER_COPY);         // per wave per block
  static constexpr int LDS_BYTES = NBUF * SLOT;
  static_assert(COPIES >= 1 && 128 % (4 * ROWS_PER_COPY) == 0, "copy split");
};

template <typename T, int DP>
__global__ __launch_bounds__(256, 3) void proxy_lse128_kernel(const T* __restrict__ qp,
                                                           const T* __restrict__ kp,
                                                           const int32_t* __restrict__ q2k_idx,
                                                           const int32_t* __restrict__ q2k_cnt,
                                                           float* __restrict__ lse_p, Geo g) {
  typedef LseCfg<T, DP> C;
  typedef typename C::TP TP;
  extern __shared__ __align__(16) unsigned char smem_raw[];
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int col = lane & 31, hi = lane >> 5;
  const int item = xcd_remap(blockIdx.x, gridDim.x);   // the grid is exactly Hkv * nqb
  const int grp = item / g.nqb;
  const int QB = item % g.nqb;
  const int b = g.qdoc[QB];
  const int I = QB - g.qb0[b];
  const int t0 = g.cu[b];
  const int L = g.cu[b + 1] - t0;
  const int kb0 = g.kb0[b];
  const int diag = (I * 128) >> 7;
  const int q0 = I * 128 + wave * 32;            // may lie past the document end: the wave
  const int qpos = q0 + col;                     // still copies and waits, its result is dropped
  const int qrow = qpos < L ? qpos : L - 1;
  frag_t<T> QPf[DP / 16];
  {
    const T* sp = qp + ((int64_t)(t0 + qrow) * g.Hp + grp) * DP + hi * 8;
#pragma unroll
    for (int ks = 0; ks < DP / 16; ++ks) QPf[ks] = ld8(sp + ks * 16);
  }
  const int64_t rowi = (int64_t)grp * g.nqb + QB;
  const int cnt = q2k_cnt[rowi];
  const int32_t* sel = q2k_idx + rowi * g.stride;
  // the register loads complete before the copies, so the waits count copies only
  wait_vmcnt<0>();
  const uint32_t lds0 = lds_offset(smem_raw);
  // kp rows of a block through a buffer descriptor with fixed per-lane byte
  // offsets; rows past the document end (diagonal block only, masked below)
  // clamped to its last row, since a copy past the bound leaves its LDS row
  // unwritten
  const uint32_t rs = (uint32_t)g.Hp * DP * (uint32_t)sizeof(T);
  uint32_t vo[C::COPIES];
  int rr[C::COPIES];
#pragma unroll
  for (int j = 0; j < C::COPIES; ++j) {
    const int r = (wave * C::COPIES + j) * C::ROWS_PER_COPY + lane / TP::CPR, p = lane % TP::CPR;
    rr[j] = r;
    vo[j] = (uint32_t)r * rs + (uint32_t)(swz<TP::CPR>(r, p) * 16);
  }
  auto issue = [&](int si) __attribute__((always_inline)) {
    const int J = sel[si < cnt ? si : cnt - 1] - kb0;    // past the end: the last block again
    const uint32_t base = lds0 + (uint32_t)((si % C::NBUF) * C::SLOT);
    const i32x4 sd = make_srd(kp + ((int64_t)(t0 + J * 128) * g.Hp + grp) * DP, 128u * rs);
    const int last = L - 1 - J * 128;
    uint32_t o[C::COPIES];
#pragma unroll
    for (int j = 0; j < C::COPIES; ++j) o[j] = vo[j];
    if (last < 127) {
#pragma unroll
      for (int j = 0; j < C::COPIES; ++j)
        if (rr[j] > last) o[j] -= (uint32_t)(rr[j] - last) * rs;
    }
#pragma unroll
    for (int j = 0; j < C::COPIES; ++j)
      bdma16(sd, o[j], base + (uint32_t)((wave * C::COPIES + j) * C::ROWS_PER_COPY * DP * (int)sizeof(T)));
  };
#pragma unroll
  for (int j = 0; j < C::AHEAD; ++j) issue(j);
  // running maximum and sum in base 2; the maximum is taken on the raw scores
  // (the scale is positive) and the scale folded into the exponent's fma
  const float psl2 = g.pscale_log2;
  float mp = NEG_BIG, lp = 0.f;
  for (int si = 0; si < cnt; ++si) {
    wait_vmcnt<(C::AHEAD - 1) * C::COPIES>();   // this block's copies have landed
    __syncthreads();                             // ... everyone's, and the slot refilled next is free
    issue(si + C::AHEAD);
    const T* KPs = reinterpret_cast<const T*>(smem_raw + (si % C::NBUF) * C::SLOT);
    const int J = sel[si] - kb0;
    const bool need_mask = J == diag;
    // key tiles that hold a key <= the wave's last query
    const int lim = q0 + 31 - J * 128;
    const int ntile = lim >= 96 ? 4 : (lim < 0 ? 0 : lim / 32 + 1);
    f32x16 Y[4];
    float mx = NEG_BIG;
#pragma unroll
    for (int kt = 0; kt < 4; ++kt) {
      if (kt >= ntile) break;
      Y[kt] = zero16();
#pragma unroll
      for (int ks = 0; ks < DP / 16; ++ks) mma(Y[kt], TP::row8(KPs, kt * 32 + col, ks * 16 + hi * 8), QPf[ks]);
      if (need_mask) {
#pragma unroll
        for (int i = 0; i < 16; ++i)
          if (J * 128 + kt * 32 + acc_row(i, lane) > qpos) Y[kt][i] = -INFINITY;
      }
#pragma unroll
      for (int i = 0; i < 16; ++i) mx = fmaxf(mx, Y[kt][i]);
    }
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64)) * psl2;
    const float mnew = fmaxf(mp, mx);
    float ls = 0.f;
#pragma unroll
    for (int kt = 0; kt < 4; ++kt) {
      if (kt >= ntile) break;
#pragma unroll
      for (int i = 0; i < 16; ++i) ls += __builtin_amdgcn_exp2f(fmaf(Y[kt][i], psl2, -mnew));
    }
    lp = lp * __builtin_amdgcn_exp2f(mp - mnew) + ls;
    mp = mnew;
  }
  wait_vmcnt<0>();                               // copies issued past the last block
  const float lt = lp + __shfl_xor(lp, 32, 64);
  if (hi == 0 && qpos < L) lse_p[(int64_t)grp * g.T + t0 + qpos] = (mp + log2f(lt)) * LN2;
}

template <typename T, int D, int DP>
static hipError_t fwd_dispatch(const Geo& g, const Geo& gp, const void* q, const void* k, const void* v,
                               const void* qp, const void* kp, const int32_t* q2k_idx,
                               const int32_t* q2k_cnt, void* o, float* lse, float* lse_p,
                               int32_t* queue, hipStream_t s) {
  // bf16, d = 128: eight waves of 32 queries (two waves per SIMD, each within
  // 256 registers); otherwise four waves of 64 queries
  constexpr bool W8 = sizeof(T) == 2 && D == 128;
  constexpr int QT = W8 ? 1 : 2, NW = W8 ? 8 : 4;
  typedef FwdCfg<T, D, DP, QT, NW> C;
  auto fn = fwd_kernel<T, D, DP, QT, NW>;
  // the persistent kernel keeps its work item in 256 bytes past the ring
  constexpr int lds_bytes = C::LDS_BYTES + (W8 ? 256 : 0);
  static LdsLimitOnce lds_limit;
  {
    const hipError_t e = lds_limit.ensure({{(const void*)fn, lds_bytes}});
    if (e != hipSuccess) return e;
  }
  const int NU = g.G * (g.Bq / (32 * QT));
  const int64_t nblk = (int64_t)g.Hkv * g.nqb * ((NU + NW - 1) / NW);
  if (nblk == 0) return hipSuccess;
  if (nblk > INT32_MAX / 2) return hipErrorInvalidValue;
  unsigned grid = (unsigned)nblk;
  hipError_t e;
  if constexpr (W8) {
    int ncu = 0;
    if ((e = device_cu_count(&ncu)) != hipSuccess) return e;
    grid = (unsigned)(nblk < ncu ? nblk : ncu);            // one workgroup per CU (LDS-bound)
    if ((e = launch_queue_reset(queue, s)) != hipSuccess) return e;
  }
  { ProfScope _ps("fwd", s);
  hipLaunchKernelGGL(fn, dim3(grid), dim3(C::NT), lds_bytes, s, (const T*)q, (const T*)k,
                     (const T*)v, q2k_idx, q2k_cnt, (T*)o, lse, queue, g); }
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  // the proxy log-sum-exp, once per proxy head
  const int64_t nrow = (int64_t)gp.Hkv * gp.nqb;
  if (gp.Bq == 128) {
    constexpr int lse_lds = LseCfg<T, DP>::LDS_BYTES;
    { ProfScope _ps("proxy_lse", s);
    hipLaunchKernelGGL((proxy_lse128_kernel<T, DP>), dim3((unsigned)nrow), dim3(256), lse_lds,
                       s, (const T*)qp, (const T*)kp, q2k_idx, q2k_cnt, lse_p, gp); }
    return hipGetLastError();
  }
  const int per_wg = 4 / (gp.Bq / 32);
  { ProfScope _ps("proxy_lse", s);
  hipLaunchKernelGGL((proxy_lse_kernel<T, DP>), dim3((unsigned)((nrow + per_wg - 1) / per_wg)), dim3(256),
                     0, s, (const T*)qp, (const T*)kp, q2k_idx, q2k_cnt, lse_p, gp); }
  return hipGetLastError();
}

hipError_t launch_fwd(const Geo& g, const Geo& gp, int is_bf16, const void* q, const void* k, const void* v,
                      const void* qp, const void* kp, const int32_t* q2k_idx,
                      const int32_t* q2k_cnt, void* o, float* lse, float* lse_p, int32_t* queue,
                      hipStream_t s) {
  if (is_bf16) {
    if (g.D == 128)
      return fwd_dispatch<bf16, 128, 64>(g, gp, q, k, v, qp, kp, q2k_idx, q2k_cnt, o, lse, lse_p, queue, s);
    return fwd_dispatch<bf16, 64, 32>(g, gp, q, k, v, qp, kp, q2k_idx, q2k_cnt, o, lse, lse_p, queue, s);
  }
  return fwd_dispatch<float, 64, 32>(g, gp, q, k, v, qp, kp, q2k_idx, q2k_cnt, o, lse, lse_p, queue, s);
}

}  // namespace msa

namespace msa {
int fwd_kernels(KernelEntry* out, int max) {
  const KernelEntry all[] = {
      {"fwd<bf16,d128,dp64>", (const void*)fwd_kernel<bf16, 128, 64, 1, 8>, 512, FwdCfg<bf16, 128, 64, 1, 8>::LDS_BYTES + 256},
      {"fwd<bf16,d64,dp32>", (const void*)fwd_kernel<bf16, 64, 32, 2, 4>, 256, FwdCfg<bf16, 64, 32, 2, 4>::LDS_BYTES},
      {"fwd<f32,d64,dp32>", (const void*)fwd_kernel<float, 64, 32, 2, 4>, 256, FwdCfg<float, 64, 32, 2, 4>::LDS_BYTES},
      {"proxy_lse<bf16,dp64>", (const void*)proxy_lse_kernel<bf16, 64>, 256, 0},
      {"proxy_lse<bf16,dp32>", (const void*)proxy_lse_kernel<bf16, 32>, 256, 0},
      {"proxy_lse<f32,dp32>", (const void*)proxy_lse_kernel<float, 32>, 256, 0},
      {"proxy_lse128<bf16,dp64>", (const void*)proxy_lse128_kernel<bf16, 64>, 256, LseCfg<bf16, 64>::LDS_BYTES},
      {"proxy_lse128<bf16,dp32>", (const void*)proxy_lse128_kernel<bf16, 32>, 256, LseCfg<bf16, 32>::LDS_BYTES},
      {"proxy_lse128<f32,dp32>", (const void*)proxy_lse128_kernel<float, 32>, 256, LseCfg<float, 32>::LDS_BYTES},
  };
  int n = (int)(sizeof(all) / sizeof(all[0]));
  for (int i = 0; i < n && i < max; ++i) out[i] = all[i];
  return n;
}
}  // namespace msa
