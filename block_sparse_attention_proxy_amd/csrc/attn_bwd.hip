// Fused backward of the sparse GQA attention and the proxy head.
//
// The pages fuse the proxy and main-attention backward passes (ai-minor
// "Dramatically Speeding Up Million-Token Training!", Why Does This Matter?:
// fused backward; keelcrux "Flash-MSA: Ein Training mit einer Million
// Tokens", Le fait) and keep every step except the proxy forward sparse.  The
// proxy gradient is read as a distillation KL over the selected keys: with
// T = mean over the group's heads of the main attention probabilities (held
// constant) and Q the proxy softmax, dY = lam (Q - T), dqp = s_p dY kp and
// dkp = s_p dY^T qp.
//
// Kernels, in launch order:
//   dq_kernel      query-major over the same block lists as the forward:
//                  D = rowsum(dO * O) (kept for the KV-major pass), dQ, and
//                  the proxy term sum_u (Q - P/G) kp per head
//   dqp_reduce     sums the per-head proxy terms when a group spans
//                  several workgroups (G > 4)
// For bf16, d = 128, dp = 64 the query-major pass is dq128_kernel
// (attn_bwd_q.hip) and the KV-major pass dkdv_ws_kernel (attn_bwd_kv.hip).
//   dkdv_kernel    KV-major over the inverted lists: dK, dV and dkp, each
//                  KV block owned by one workgroup, so no atomics
#include "msa_device.h"
#include "msa_internal.h"
#include "msa_profile.h"

#include <type_traits>

namespace msa {

// ---------------------------------------------------------------------------
// dQ kernel: a workgroup serves (group, query block, 4 units); a wave owns 32
// queries of one head.  Stages are 64-key halves of the selected blocks with
// K, V and kp rows copied global -> LDS by DMA one stage ahead; K^T and kp^T
// fragments come from the same tiles through LDS transpose reads.
// ---------------------------------------------------------------------------
template <typename T, int D, int DP>
struct DqCfg {
  static constexpr int KC = 64;                   // keys per stage
  static constexpr int NBUF = 3;                  // LDS ring of stages (one workgroup per CU)
  static constexpr int AHEAD = NBUF - 1;
  typedef Tile<T, D> TK;                          // K and V rows
  typedef Tile<T, DP> TP;                         // kp rows
  static constexpr int KS = KC * D, KPS = KC * DP;
  static constexpr int STAGE = 2 * KS + KPS;      // elements of T
  static constexpr int STAGE_BYTES = STAGE * (int)sizeof(T);
  static constexpr int LDS_BYTES = NBUF * STAGE_BYTES;
  static constexpr int EPC = TK::EPC;
  static constexpr int KROWS_PER_COPY = 64 / TK::CPR, PROWS_PER_COPY = 64 / TP::CPR;
  static constexpr int NKCOPY = KC / (4 * KROWS_PER_COPY);          // per tensor per wave
  static constexpr int NPCOPY = KC / (4 * PROWS_PER_COPY);
  static constexpr int COPIES = 2 * NKCOPY + NPCOPY;
  static_assert(NKCOPY >= 1 && NPCOPY >= 1, "copy split");
  static_assert(KC % (4 * KROWS_PER_COPY) == 0 && KC % (4 * PROWS_PER_COPY) == 0, "copy split");
  static_assert(4 * DP * 33 * 4 <= LDS_BYTES, "reduction scratch");
};

template <typename T, int D, int DP>
__global__ __launch_bounds__(256) void dq_kernel(
    const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ v,
    const T* __restrict__ qp, const T* __restrict__ kp, const T* __restrict__ o,
    const float* __restrict__ lse, const float* __restrict__ lse_p, const T* __restrict__ dout,
    float* __restrict__ delta, float* __restrict__ lse2_out, float* __restrict__ lsep2_out,
    const int32_t* __restrict__ q2k_idx, const int32_t* __restrict__ q2k_cnt,
    float* __restrict__ dq, float* __restrict__ dqp, float* __restrict__ cpart, Geo g) {
  typedef DqCfg<T, D, DP> C;
  typedef typename C::TK TK;
  typedef typename C::TP TP;
  extern __shared__ __align__(16) unsigned char smem_raw[];
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int col = lane & 31, hi = lane >> 5;
  const int NU = g.G * (g.Bq / 32);
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
  const int b = g.qdoc[QB];
  const int I = QB - g.qb0[b];
  const int t0 = g.cu[b];
  const int L = g.cu[b + 1] - t0;
  const int kb0 = g.kb0[b];
  const int diag = (I * g.Bq) >> 7;
  const int qbase = I * g.Bq + chunk * 32;
  const int pg = proxy_head(g, grp);                 // the proxy head this group reads
  const float qw = proxy_qweight(g, grp);            // weight of its proxy-softmax term
  const int64_t rowi = (int64_t)pg * g.nqb + QB;
  const int cnt = q2k_cnt[rowi];
  const int32_t* sel = q2k_idx + rowi * g.stride;
  const int qpos = qbase + col;
  const int qrow = qpos < L ? qpos : L - 1;
  const int64_t tq = t0 + qrow;

  // stages: 64-key halves of the selected blocks; the diagonal block is last
  int nst = 2 * cnt;
  if (diag * 128 + 64 > I * g.Bq + g.Bq - 1) nst -= 1;
  const int nst_plain = 2 * (cnt - 1);

  // Copy stage s (clamped to the last) into ring slot s % NBUF.  Key rows past
  // the document end are clamped to its last row; they only occur in the
  // diagonal block, where the causal mask removes them.
  auto issue = [&](int s, int slot) __attribute__((always_inline)) {
    const int ss = s < nst ? s : nst - 1;
    const uint32_t base = lds_offset(smem_raw) + slot * C::STAGE_BYTES;
    const int key0 = (sel[ss >> 1] - kb0) * 128 + (ss & 1) * C::KC;
#pragma unroll
    for (int j = 0; j < C::NKCOPY; ++j) {
      const int rfirst = (wave * C::NKCOPY + j) * C::KROWS_PER_COPY;
      const int r = rfirst + lane / TK::CPR, p = lane % TK::CPR;
      const int key = key0 + r < L ? key0 + r : L - 1;
      const int64_t off = ((int64_t)(t0 + key) * g.Hkv + grp) * D + swz<TK::CPR>(r, p) * C::EPC;
      dma16(k + off, base + rfirst * D * (int)sizeof(T));
      dma16(v + off, base + (C::KS + rfirst * D) * (int)sizeof(T));
    }
#pragma unroll
    for (int j = 0; j < C::NPCOPY; ++j) {
      const int rfirst = (wave * C::NPCOPY + j) * C::PROWS_PER_COPY;
      const int r = rfirst + lane / TP::CPR, p = lane % TP::CPR;
      const int key = key0 + r < L ? key0 + r : L - 1;
      const int64_t off = ((int64_t)(t0 + key) * g.Hp + pg) * DP + swz<TP::CPR>(r, p) * C::EPC;
      dma16(kp + off, base + (2 * C::KS + rfirst * DP) * (int)sizeof(T));
    }
  };
  frag_t<T> Qf[D / 16], dOf[D / 16], QPf[DP / 16];
  float lse2 = 0.f, dl = 0.f, lsep2 = 0.f;
  if (active) {
    const T* sq = q + (tq * g.Hq + h) * D + hi * 8;
    const T* sd = dout + (tq * g.Hq + h) * D + hi * 8;
    const T* so = o + (tq * g.Hq + h) * D + hi * 8;
    float part = 0.f;                               // this lane's half of rowsum(dO * O)
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) {
      Qf[ks] = ld8(sq + ks * 16);
      dOf[ks] = ld8(sd + ks * 16);
      const frag_t<T> of = ld8(so + ks * 16);
#pragma unroll
      for (int j = 0; j < 8; ++j) part = fmaf(to_f32(dOf[ks][j]), to_f32(of[j]), part);
    }
    dl = part + __shfl_xor(part, 32, 64);
    const T* sp = qp + (tq * g.Hp + pg) * DP + hi * 8;
#pragma unroll
    for (int ks = 0; ks < DP / 16; ++ks) QPf[ks] = ld8(sp + ks * 16);
    lse2 = lse[(int64_t)h * g.T + tq] * LOG2E;
    lsep2 = lse_p[(int64_t)pg * g.T + tq] * LOG2E;
    // per-query values the KV-major pass reads: D and both LSEs in log2 units
    if (hi == 0 && qpos < L) {
      delta[(int64_t)h * g.T + tq] = -dl;             // stored negated: -rowsum(dO * O)
      lse2_out[(int64_t)h * g.T + tq] = lse2;
      if (hl == 0) lsep2_out[(int64_t)grp * g.T + tq] = lsep2;
    }
  }
  // The register loads above complete before the first copies are issued, so
  // that the copies are the only vector-memory operations in flight in the
  // loop (the vmcnt waits there count only them).
  wait_vmcnt<0>();
#pragma unroll
  for (int j = 0; j < C::AHEAD; ++j) issue(j, j);

  // dQ^T, and the proxy terms kept apart: Cq^T += kp^T Q^T over the tiles this
  // head is assigned, Cp^T += kp^T P^T over every tile; the head's share of
  // the proxy gradient is Cq - Cp / G.
  f32x16 dQ[D / 32], Cq[DP / 32], Cp[DP / 32];
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt) dQ[dt] = zero16();
#pragma unroll
  for (int dt = 0; dt < DP / 32; ++dt) { Cq[dt] = zero16(); Cp[dt] = zero16(); }

  // One stage: two 32-key tiles.  Key row r of tile kt is visible to this
  // lane's query iff r <= qpos - (first key of the tile); only the diagonal
  // block's stages are masked.
  //
  // The main work of a stage is a fixed sequence of MFMAs, each with one
  // operand read from LDS: S and dP of tile 0 (NA products: K and V rows),
  // the same for tile 1, then dQ and the proxy term C_p of tile 0 (NB
  // products: K^T and kp^T fragments), then of tile 1.  It is issued in that
  // order with every LDS read LOOK products ahead of its use, tile 0's
  // softmax spread between tile 1's S/dP products and tile 1's between tile
  // 0's dQ products; scheduling fences keep that order.  The proxy term Q kp
  // of a tile is computed by the one head it is assigned to, at the end.
  // Byte offsets of this lane's LDS reads inside a stage, for the first tile
  // and half (the swizzle depends on the row modulo 16 only, so other tiles
  // and halves are constant offsets from these): row fragments of K/V (per
  // 16-column step), the two transpose reads of a K^T and a kp^T fragment
  // (per 32-column block), and row fragments of kp.
  uint32_t oRow[D / 16], oColK[D / 32][2], oColP[DP / 32][2];
  {
    const int s16 = lane & 15, g4 = lane >> 4;
    const int tr_r = hi * 4 + (s16 >> 2), tr_c = 16 * (g4 & 1) + 4 * (s16 & 3);
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) oRow[ks] = TK::off(col, ks * 16 + hi * 8) * (int)sizeof(T);
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt) {
      oColK[dt][0] = TK::off(tr_r, dt * 32 + tr_c) * (int)sizeof(T);
      oColK[dt][1] = TK::off(tr_r + 8, dt * 32 + tr_c) * (int)sizeof(T);
    }
#pragma unroll
    for (int dt = 0; dt < DP / 32; ++dt) {
      oColP[dt][0] = TP::off(tr_r, dt * 32 + tr_c) * (int)sizeof(T);
      oColP[dt][1] = TP::off(tr_r + 8, dt * 32 + tr_c) * (int)sizeof(T);
    }
  }
  constexpr int NA = 2 * (D / 16);                 // S and dP products per tile
  constexpr int NB = 2 * (D / 32 + DP / 32);       // dQ and C_p products per tile
  constexpr int NM = 2 * NA + 2 * NB;
  constexpr int LOOK = 4;
  auto stage_body = [&](int s, auto masked_c) __attribute__((always_inline)) {
    constexpr bool MASKED = decltype(masked_c)::value;
    wait_vmcnt<C::COPIES * (C::AHEAD - 1)>();
    __syncthreads();
    issue(s + C::AHEAD, (s + C::AHEAD) % C::NBUF);
    __builtin_amdgcn_sched_barrier(0);
    if (!active) return;
    const T* Ks = reinterpret_cast<const T*>(smem_raw + (s % C::NBUF) * C::STAGE_BYTES);
    const T* Vs = Ks + C::KS;
    const T* KPs = Vs + C::KS;
    const int lim0 = qpos - ((sel[s >> 1] - kb0) * 128 + (s & 1) * C::KC);
    f32x16 S[2], dP[2];
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) { S[kt] = zero16(); dP[kt] = zero16(); }
    frag_t<T> bs[2][2], bp[2][2];                  // [tile][half] softmax outputs as operands
    frag_t<T> opnd[NM];
    // this stage's read bases: slot base + lane offset, one add each
    uint32_t aRow[D / 16], aColK[D / 32][2], aColP[DP / 32][2];
    if constexpr (sizeof(T) == 2) {
      const uint32_t sb = (uint32_t)__builtin_amdgcn_readfirstlane(
          (int)(lds_offset(smem_raw) + (s % C::NBUF) * C::STAGE_BYTES));
#pragma unroll
      for (int ks = 0; ks < D / 16; ++ks) aRow[ks] = lds_base_add(sb, oRow[ks]);
#pragma unroll
      for (int dt = 0; dt < D / 32; ++dt) {
        aColK[dt][0] = lds_base_add(sb, oColK[dt][0]);
        aColK[dt][1] = lds_base_add(sb, oColK[dt][1]);
      }
#pragma unroll
      for (int dt = 0; dt < DP / 32; ++dt) {
        aColP[dt][0] = lds_base_add(sb, oColP[dt][0]);
        aColP[dt][1] = lds_base_add(sb, oColP[dt][1]);
      }
    }
    auto operand = [&](auto mc) __attribute__((always_inline)) {
      constexpr int m = decltype(mc)::value;
      if constexpr (sizeof(T) == 2) {
        // tile, half and tensor offsets are constants on the stage's bases
        if constexpr (m < 2 * NA) {
          constexpr int kt = m / NA, j = m % NA, ks = j / 2;
          constexpr int cst = ((j & 1) ? C::KS : 0) * 2 + kt * 32 * D * 2;
          opnd[m] = lds_ld8<cst>(aRow[ks]);
        } else {
          constexpr int r = m - 2 * NA, kt = r / NB, kk = (r % NB) / (NB / 2), c = (r % NB) % (NB / 2);
          if constexpr (c < D / 32) {
            constexpr int cst = (kt * 32 + kk * 16) * D * 2;
            opnd[m] = tr_pair_at<cst>(aColK[c][0], aColK[c][1]);
          } else {
            constexpr int cst = 2 * C::KS * 2 + (kt * 32 + kk * 16) * DP * 2;
            opnd[m] = tr_pair_at<cst>(aColP[c - D / 32][0], aColP[c - D / 32][1]);
          }
        }
      } else if constexpr (m < 2 * NA) {
        constexpr int kt = m / NA, j = m % NA, ks = j / 2;
        opnd[m] = TK::row8((j & 1) ? Vs : Ks, kt * 32 + col, ks * 16 + hi * 8);
      } else {
        constexpr int r = m - 2 * NA, kt = r / NB, kk = (r % NB) / (NB / 2), c = (r % NB) % (NB / 2);
        if constexpr (c < D / 32) opnd[m] = TK::col(Ks, kt * 32 + kk * 16, c * 32, lane);
        else opnd[m] = TP::col(KPs, kt * 32 + kk * 16, (c - D / 32) * 32, lane);
      }
    };
    auto product = [&](auto mc) __attribute__((always_inline)) {
      constexpr int m = decltype(mc)::value;
      if constexpr (m < 2 * NA) {
        constexpr int kt = m / NA, j = m % NA, ks = j / 2;
        if constexpr (j & 1) mma(dP[kt], opnd[m], dOf[ks]);
        else mma(S[kt], opnd[m], Qf[ks]);
      } else {
        constexpr int r = m - 2 * NA, kt = r / NB, kk = (r % NB) / (NB / 2), c = (r % NB) % (NB / 2);
        if constexpr (c < D / 32) mma(dQ[c], opnd[m], bs[kt][kk]);
        else mma(Cp[c - D / 32], opnd[m], bp[kt][kk]);
      }
    };
    auto soft = [&](int kt, int i) __attribute__((always_inline)) {
      float p = __builtin_amdgcn_exp2f(fmaf(S[kt][i], g.scale_log2, -lse2));
      if (MASKED) p = acc_row(i, lane) <= lim0 - kt * 32 ? p : 0.f;
      S[kt][i] = p;
      dP[kt][i] = p * (dP[kt][i] - dl);
    };
    auto pack = [&](int kt) __attribute__((always_inline)) {
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) { bs[kt][kk] = acc_frag<T>(dP[kt], kk); bp[kt][kk] = acc_frag<T>(S[kt], kk); }
    };
    static_for<LOOK>([&](auto mc) __attribute__((always_inline)) { operand(mc); });
    static_for<NM>([&](auto mc) __attribute__((always_inline)) {
      constexpr int m = decltype(mc)::value;
      product(mc);
      if constexpr (m + LOOK < NM) operand(std::integral_constant<int, m + LOOK>());
      // tile 0's 16 softmax elements over tile 1's S/dP products, tile 1's
      // over tile 0's dQ products
      if constexpr (m >= NA && m < 2 * NA) {
        constexpr int e0 = (m - NA) * 16 / NA, e1 = (m - NA + 1) * 16 / NA;
#pragma unroll
        for (int i = e0; i < e1; ++i) soft(0, i);
        if constexpr (m == 2 * NA - 1) pack(0);
      } else if constexpr (m >= 2 * NA && m < 2 * NA + NB) {
        constexpr int e0 = (m - 2 * NA) * 16 / NB, e1 = (m - 2 * NA + 1) * 16 / NB;
#pragma unroll
        for (int i = e0; i < e1; ++i) soft(1, i);
        if constexpr (m == 2 * NA + NB - 1) pack(1);
      }
      __builtin_amdgcn_sched_barrier(0);
    });
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
      if (((s * 2 + kt) % g.G) != hl || qw == 0.f) continue;
      f32x16 Y = zero16();
#pragma unroll
      for (int ks = 0; ks < DP / 16; ++ks) mma(Y, TP::row8(KPs, kt * 32 + col, ks * 16 + hi * 8), QPf[ks]);
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        float qv = __builtin_amdgcn_exp2f(fmaf(Y[i], g.pscale_log2, -lsep2));
        if (MASKED) qv = acc_row(i, lane) <= lim0 - kt * 32 ? qv : 0.f;
        Y[i] = qv;
      }
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        const frag_t<T> bq = acc_frag<T>(Y, kk);
#pragma unroll
        for (int dt = 0; dt < DP / 32; ++dt) mma(Cq[dt], TP::col(KPs, kt * 32 + kk * 16, dt * 32, lane), bq);
      }
    }
  };

  int s = 0;
  for (; s < nst_plain; ++s) stage_body(s, std::integral_constant<bool, false>());
  for (; s < nst; ++s) stage_body(s, std::integral_constant<bool, true>());
  wait_vmcnt<0>();
  __syncthreads();
  f32x16 Cd[DP / 32];
  const float invG = 1.f / (float)g.G;
#pragma unroll
  for (int dt = 0; dt < DP / 32; ++dt)
#pragma unroll
    for (int i = 0; i < 16; ++i) Cd[dt][i] = (qw == 1.f ? Cq[dt][i] : qw * Cq[dt][i]) - Cp[dt][i] * invG;

  // dQ out (fp32)
  if (active && qpos < L) {
    float* dst = dq + ((int64_t)(t0 + qpos) * g.Hq + h) * D;
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
      for (int i4 = 0; i4 < 4; ++i4) {
        f32x4 r;
#pragma unroll
        for (int j = 0; j < 4; ++j) r[j] = dQ[dt][i4 * 4 + j] * g.scale;
        *reinterpret_cast<f32x4*>(dst + dt * 32 + acc_row(i4 * 4, lane)) = r;
      }
  }
  // proxy term: sum over the heads of this workgroup that share a chunk.
  // Rows of 33 floats: the reads below walk the proxy dimension across lanes,
  // and a stride of 33 words puts every lane in its own bank.
  constexpr int RS = 33;
  float* red = reinterpret_cast<float*>(smem_raw);          // [4][DP][RS]
  if (active) {
#pragma unroll
    for (int dt = 0; dt < DP / 32; ++dt)
#pragma unroll
      for (int i = 0; i < 16; ++i) red[(wave * DP + dt * 32 + acc_row(i, lane)) * RS + col] = Cd[dt][i];
  }
  __syncthreads();
  const int u_lo = wgi * 4;
  const int u_hi = (u_lo + 4 < NU ? u_lo + 4 : NU) - 1;
  const int c_lo = u_lo / g.G, c_hi = u_hi / g.G;
  const int nhg = g.G > 4 ? g.G / 4 : 1;
  const int hg = g.G > 4 ? (wgi % nhg) : 0;
  const int nel = (c_hi - c_lo + 1) * 32 * DP;
  for (int e = tid; e < nel; e += 256) {
    const int cidx = e / (32 * DP);
    const int rem = e % (32 * DP);
    const int qq = rem / DP, dpi = rem % DP;
    const int c = c_lo + cidx;
    float acc = 0.f;
    for (int w = 0; w < 4; ++w) {
      const int uw = u_lo + w;
      if (uw < NU && uw / g.G == c) acc += red[(w * DP + dpi) * RS + qq];
    }
    const int pos = I * g.Bq + c * 32 + qq;
    if (pos < L) {
      const int64_t t = t0 + pos;
      if (nhg == 1) dqp[(t * g.Hkv + grp) * DP + dpi] = acc * g.pscale * g.lam;
      else cpart[(((int64_t)grp * nhg + hg) * g.T + t) * DP + dpi] = acc;
    }
  }
}

template <int DP>
__global__ void dqp_reduce_kernel(const float* __restrict__ cpart, float* __restrict__ dqp, Geo g) {
  const int nhg = g.G / 4;
  const int64_t n = (int64_t)g.T * g.Hkv * DP;
  for (int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; e < n;
       e += (int64_t)gridDim.x * blockDim.x) {
    const int64_t t = e / (g.Hkv * DP);
    const int grp = (int)((e / DP) % g.Hkv);
    const int dpi = (int)(e % DP);
    float acc = 0.f;
    for (int hg = 0; hg < nhg; ++hg) acc += cpart[(((int64_t)grp * nhg + hg) * g.T + t) * DP + dpi];
    dqp[e] = acc * g.pscale * g.lam;
  }
}

// ---------------------------------------------------------------------------
// dK/dV kernel: a workgroup owns one KV block of one group; wave w owns keys
// [32w, 32w + 32) and keeps K, V, kp of them as B fragments.  Stages walk the
// inverted list: (query block, 32-query chunk, head), with Q and dO rows in
// LDS (their transposed fragments come through LDS transpose reads).  T (the
// group-mean probability) is accumulated over the heads of a chunk, and the
// proxy term is applied at the chunk's last head, whose stage also carries qp.
// ---------------------------------------------------------------------------
template <typename T, int D, int DP>
struct KvCfg {
  static constexpr int QC = 32;                   // queries per stage
  static constexpr int NBUF = 4;                  // LDS ring of stages
  static constexpr int AHEAD = NBUF - 1;          // stages in flight ahead of the one computed
  typedef Tile<T, D> TQ;                          // Q and dO rows
  typedef Tile<T, DP> TP;                         // qp rows, and the block's kp rows
  static constexpr int QS = QC * D, PS = QC * DP;
  static constexpr int STAGE_T = 2 * QS + PS;                        // elements of T
  static constexpr int FL_OFF = ((STAGE_T * (int)sizeof(T) + 15) / 16) * 16;
  static constexpr int STAGE_BYTES = FL_OFF + 4 * QC * 4;            // lse2, D, lsep2, spare
  static constexpr int KP_OFF = NBUF * STAGE_BYTES;                  // kp rows of the KV block
  static constexpr int LDS_BYTES = KP_OFF + 128 * DP * (int)sizeof(T);
  static constexpr int EPC = TQ::EPC;
  // copies per wave per stage: Q and dO rows, one vector of floats, and the
  // qp rows at the last head of a chunk
  static constexpr int QROWS_PER_COPY = 64 / TQ::CPR;                // rows one wave copy covers
  static constexpr int NQCOPY = QC / (4 * QROWS_PER_COPY);           // per tensor per wave
  static constexpr int PROWS_PER_COPY = 64 / TP::CPR;
  static constexpr int NPCOPY = (QC + 4 * PROWS_PER_COPY - 1) / (4 * PROWS_PER_COPY);
  static constexpr int NKPCOPY = 32 / PROWS_PER_COPY;                // a wave's 32 kp rows
  static_assert(QC % PROWS_PER_COPY == 0 && 32 % PROWS_PER_COPY == 0, "copy split");
  static constexpr int COPIES = 2 * NQCOPY + 1;
  static_assert(NQCOPY >= 1 && QC % (4 * QROWS_PER_COPY) == 0, "copy split");
};

template <typename T, int D, int DP, int G>
__global__ __launch_bounds__(256) void dkdv_kernel(
    const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ v,
    const T* __restrict__ qp, const T* __restrict__ kp, const float* __restrict__ lse2,
    const float* __restrict__ lsep2, const T* __restrict__ dout, const float* __restrict__ delta,
    const int32_t* __restrict__ k2q_ptr, const int32_t* __restrict__ k2q_idx,
    float* __restrict__ dk, float* __restrict__ dv, float* __restrict__ dkp, Geo g) {
  typedef KvCfg<T, D, DP> C;
  typedef typename C::TQ TQ;
  typedef typename C::TP TP;
  extern __shared__ __align__(16) unsigned char smem_raw[];
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int col = lane & 31, hi = lane >> 5;
  const int bid = xcd_remap(blockIdx.x, gridDim.x);
  const int grp = bid / g.nkb;
  const int KB = bid % g.nkb;
  const int b = g.kdoc[KB];
  const int J = KB - g.kb0[b];
  const int t0 = g.cu[b];
  const int L = g.cu[b + 1] - t0;
  const int qb0 = g.qb0[b];
  const int kpos = J * 128 + wave * 32 + col;               // this lane's key (B-fragment column)
  const int krow = kpos < L ? kpos : L - 1;
  const int64_t tk = t0 + krow;
  const int pg = proxy_head(g, grp);                        // the proxy head this group reads
  const float qw = proxy_qweight(g, grp);                   // weight of its proxy-softmax term
  const int32_t* ptr = k2q_ptr + (int64_t)pg * (g.nkb + 1);
  const int32_t* lst = k2q_idx + (int64_t)pg * g.cap + ptr[KB];
  const int len = ptr[KB + 1] - ptr[KB];
  const int nch = g.Bq / 32;
  const float invG = 1.f / (float)G;
  const T* KPs = reinterpret_cast<const T*>(smem_raw + C::KP_OFF);

  // K and V of this lane's key stay in registers as B fragments; the kp rows
  // of the wave's 32 keys go to LDS (read only at a chunk's last head).
  frag_t<T> Kf[D / 16], Vf[D / 16];
  {
    const T* sk = k + (tk * g.Hkv + grp) * D + hi * 8;
    const T* sv = v + (tk * g.Hkv + grp) * D + hi * 8;
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) { Kf[ks] = ld8(sk + ks * 16); Vf[ks] = ld8(sv + ks * 16); }
  }
  wait_vmcnt<0>();
#pragma unroll
  for (int j = 0; j < C::NKPCOPY; ++j) {
    const int rfirst = wave * 32 + j * C::PROWS_PER_COPY;
    const int r = rfirst + lane / TP::CPR, p = lane % TP::CPR;
    const int key = J * 128 + r < L ? J * 128 + r : L - 1;
    dma16(kp + ((int64_t)(t0 + key) * g.Hp + pg) * DP + swz<TP::CPR>(r, p) * C::EPC,
          lds_offset(smem_raw) + C::KP_OFF + rfirst * DP * (int)sizeof(T));
  }

  f32x16 dK[D / 32], dV[D / 32], dKp[DP / 32], Tacc = zero16();
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt) { dK[dt] = zero16(); dV[dt] = zero16(); }
#pragma unroll
  for (int dt = 0; dt < DP / 32; ++dt) dKp[dt] = zero16();

  // Copy the stage (list entry li, query chunk c, head hl) into ring slot buf.
  // Rows past the document end are clamped to its last row (valid memory);
  // such rows are masked in the compute.  Every wave issues the same number of
  // copies per stage (COPIES, + NPCOPY at a chunk's last head), which the
  // vmcnt waits below rely on.
  auto issue_stage = [&](int buf, int li, int c, int hl, auto with_qp_c) __attribute__((always_inline)) {
    constexpr bool with_qp = decltype(with_qp_c)::value;
    const uint32_t base = lds_offset(smem_raw) + buf * C::STAGE_BYTES;
    const int I = lst[li] - qb0;
    const int h = grp * G + hl;
    const int row0 = I * g.Bq + c * 32;
#pragma unroll
    for (int j = 0; j < C::NQCOPY; ++j) {
      const int rfirst = (wave * C::NQCOPY + j) * C::QROWS_PER_COPY;
      const int r = rfirst + lane / TQ::CPR;
      const int p = lane % TQ::CPR;
      const int pos = row0 + r < L ? row0 + r : L - 1;
      const int64_t off = ((int64_t)(t0 + pos) * g.Hq + h) * D + swz<TQ::CPR>(r, p) * C::EPC;
      dma16(q + off, base + rfirst * D * (int)sizeof(T));
      dma16(dout + off, base + (C::QS + rfirst * D) * (int)sizeof(T));
    }
    if constexpr (with_qp) {
#pragma unroll
      for (int j = 0; j < C::NPCOPY; ++j) {
        // with fewer rows than copies, the extra waves repeat the first rows
        const int rfirst = ((wave * C::NPCOPY + j) % (C::QC / C::PROWS_PER_COPY)) * C::PROWS_PER_COPY;
        const int r = rfirst + lane / TP::CPR;
        const int p = lane % TP::CPR;
        const int pos = row0 + r < L ? row0 + r : L - 1;
        const int64_t off = ((int64_t)(t0 + pos) * g.Hp + pg) * DP + swz<TP::CPR>(r, p) * C::EPC;
        dma16(qp + off, base + (2 * C::QS + rfirst * DP) * (int)sizeof(T));
      }
    }
    // one float vector per wave (lse2, D, lsep2, and lsep2 again into the
    // spare slot): 32 lanes x 4 bytes, the other lanes inactive so nothing
    // lands outside the wave's 128-byte slot
    if (lane < C::QC) {
      const int pos = row0 + lane < L ? row0 + lane : L - 1;
      const int64_t t = t0 + pos;
      const float* src = wave == 0 ? lse2 + (int64_t)h * g.T + t
                       : wave == 1 ? delta + (int64_t)h * g.T + t
                       : lsep2 + (int64_t)grp * g.T + t;
      dma4(src, base + C::FL_OFF + wave * C::QC * 4);
    }
  };
  // the 8 query rows held by accumulator elements [8kk, 8kk + 8)
  auto rows8 = [&](const float* f, int kk, float (&out)[8]) __attribute__((always_inline)) {
#pragma unroll
    for (int i4 = 0; i4 < 2; ++i4) {
      const f32x4 x = *reinterpret_cast<const f32x4*>(f + acc_row(kk * 8 + i4 * 4, lane));
#pragma unroll
      for (int j = 0; j < 4; ++j) out[i4 * 4 + j] = x[j];
    }
  };
  // masked: query row r counts iff lo <= r < hi_ (causal lower bound from
  // this lane's key, upper bound from the document end).  The softmax scale
  // of dK and lam * s_p of dkp are applied once, at the end.
  auto main_part = [&](const unsigned char* base, int lo, int hi_, bool masked) __attribute__((always_inline)) {
    const T* Qs = reinterpret_cast<const T*>(base);
    const T* dOs = Qs + C::QS;
    const float* fl = reinterpret_cast<const float*>(base + C::FL_OFF);
    f32x16 S = zero16(), dP = zero16();
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) {
      mma(S, TQ::row8(Qs, col, ks * 16 + hi * 8), Kf[ks]);
      mma(dP, TQ::row8(dOs, col, ks * 16 + hi * 8), Vf[ks]);
    }
    // Two halves (accumulator elements [8kk, 8kk + 8), 16 query rows each).
    // The operands of both halves are read early; the products of the first
    // half are interleaved with the exponentials of the second.
    float lr[2][8], dl[2][8];
    frag_t<T> bv[2][D / 32], bk[2][D / 32];
    auto read_half = [&](int kk) __attribute__((always_inline)) {
      rows8(fl, kk, lr[kk]);
      rows8(fl + C::QC, kk, dl[kk]);
#pragma unroll
      for (int dt = 0; dt < D / 32; ++dt) {
        bv[kk][dt] = TQ::col(dOs, kk * 16, dt * 32, lane);
        bk[kk][dt] = TQ::col(Qs, kk * 16, dt * 32, lane);
      }
    };
    frag_t<T> ap[2], as[2];
    auto softmax_half = [&](int kk) __attribute__((always_inline)) {
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int i = kk * 8 + j;
        float p = __builtin_amdgcn_exp2f(fmaf(S[i], g.scale_log2, -lr[kk][j]));
        if (masked) p = (acc_row(i, lane) >= lo && acc_row(i, lane) < hi_) ? p : 0.f;
        dP[i] = p * (dP[i] + dl[kk][j]);              // dl holds -D
        S[i] = p;
        Tacc[i] += p;
      }
      ap[kk] = acc_frag<T>(S, kk);
      as[kk] = acc_frag<T>(dP, kk);
    };
    read_half(0);
    softmax_half(0);
    read_half(1);
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt) {
      mma(dV[dt], ap[0], bv[0][dt]);
      mma(dK[dt], as[0], bk[0][dt]);
    }
    softmax_half(1);
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt) {
      mma(dV[dt], ap[1], bv[1][dt]);
      mma(dK[dt], as[1], bk[1][dt]);
    }
    if constexpr (D == 128 && sizeof(T) == 2) {
      // row reads 6 ahead of the S/dP products; the remaining reads (LSE and
      // D rows, transposed Q/dO fragments) behind the last of them; the
      // second half's exponentials between the first half's products
      __builtin_amdgcn_sched_group_barrier(0x100, 6, 1);
#pragma unroll
      for (int j = 0; j < 10; ++j) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 1);
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 1);
      }
#pragma unroll
      for (int j = 0; j < 6; ++j) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 1);
        __builtin_amdgcn_sched_group_barrier(0x100, 4, 1);
      }
      __builtin_amdgcn_sched_group_barrier(0x002, 48, 1);
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 1);
        __builtin_amdgcn_sched_group_barrier(0x100, 2, 1);
        __builtin_amdgcn_sched_group_barrier(0x002, 6, 1);
      }
      __builtin_amdgcn_sched_group_barrier(0x008, 8, 1);
    }
  };
  // dkp += dY^T qp over a chunk: dY / (lam s_p) = qw Q - T / G (only -T / G
  // where qw = 0, with no proxy scores taken)
  auto proxy_part = [&](const unsigned char* base, int lo, int hi_, bool masked) __attribute__((always_inline)) {
    const T* Ps = reinterpret_cast<const T*>(base) + 2 * C::QS;
    const float* fl = reinterpret_cast<const float*>(base + C::FL_OFF);
    __builtin_amdgcn_sched_barrier(0);
    frag_t<T> bp[2][DP / 32];
#pragma unroll
    for (int kk = 0; kk < 2; ++kk)
#pragma unroll
      for (int dt = 0; dt < DP / 32; ++dt) bp[kk][dt] = TP::col(Ps, kk * 16, dt * 32, lane);
    f32x16 Y = zero16();
    if (qw != 0.f) {
      frag_t<T> ya[DP / 16], yb[DP / 16];
      float lp[2][8];
#pragma unroll
      for (int ks = 0; ks < DP / 16; ++ks) {
        ya[ks] = TP::row8(Ps, col, ks * 16 + hi * 8);
        yb[ks] = TP::row8(KPs, wave * 32 + col, ks * 16 + hi * 8);
      }
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) rows8(fl + 2 * C::QC, kk, lp[kk]);
#pragma unroll
      for (int ks = 0; ks < DP / 16; ++ks) mma(Y, ya[ks], yb[ks]);
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const int i = kk * 8 + j;
          float qv = __builtin_amdgcn_exp2f(fmaf(Y[i], g.pscale_log2, -lp[kk][j]));
          if (masked) qv = (acc_row(i, lane) >= lo && acc_row(i, lane) < hi_) ? qv : 0.f;
          Y[i] = qv * qw;
        }
      }
    }
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int i = kk * 8 + j;
        Y[i] = fmaf(-invG, Tacc[i], Y[i]);                   // dY / (lam * s_p)
      }
      const frag_t<T> ay = acc_frag<T>(Y, kk);
#pragma unroll
      for (int dt = 0; dt < DP / 32; ++dt) mma(dKp[dt], ay, bp[kk][dt]);
    }
    __builtin_amdgcn_sched_barrier(0);
  };

  // Stages run in list order over chunks (list entry, 32-query chunk) with the
  // G heads of a chunk unrolled; the ring holds AHEAD stages in flight.
  // Masked chunks: the leading entries whose diagonal is this KV block (the
  // list is ascending) and chunks that reach past the document end (only the
  // last entry can).  The stage index after the last re-reads the last chunk.
  const int nchunk = len * nch;
  int nmask = 0;
  while (nmask < len && nmask < 2 && (((lst[nmask] - qb0) * g.Bq) >> 7) == J) ++nmask;
  const int nchunk_lead = nmask * nch;
  const bool tail = len > 0 && (lst[len - 1] - qb0 + 1) * g.Bq > L;
  const int nchunk_plain_end = tail ? (len - 1) * nch : nchunk;

  // stage s = ci * G + hl  ->  (li, c, hl); counters advance incrementally
  int fli = 0, fc = 0;                    // list entry and chunk of the next stage to issue
  int fs = 0;                             // its index
  const int nst = nchunk * G;
  // The head of the stage issued next is known at compile time (stages go
  // round the G heads in order); a stage past the end re-reads the last
  // chunk with the same head, so every wave issues the same copies.
  auto issue_next = [&](auto hl_c) __attribute__((always_inline)) {
    constexpr int hl = decltype(hl_c)::value;
    const bool past = fs >= nst;
    const int li = past ? len - 1 : fli;
    const int c = past ? nch - 1 : fc;
    issue_stage(fs % C::NBUF, li, c, hl, std::integral_constant<bool, hl == G - 1>());
    ++fs;
    if (hl == G - 1) { if (++fc == nch) { fc = 0; ++fli; } }
  };
  if (nst > 0) {
    static_for<C::AHEAD>([&](auto jc) __attribute__((always_inline)) {
      issue_next(std::integral_constant<int, decltype(jc)::value % G>());
    });
  }
  int li = 0, c = 0;
  auto chunk_body = [&](int ci, bool masked) __attribute__((always_inline)) {
    const int I = lst[li] - qb0;
    const int qpos0 = I * g.Bq + c * 32;
    const int lo = kpos - qpos0, hi_ = L - qpos0;
    static_for<G>([&](auto hlc) __attribute__((always_inline)) {
      constexpr int hl = decltype(hlc)::value;
      // stage ci*G + hl must have landed: the AHEAD - 1 later stages in
      // flight issued COPIES (+ NPCOPY at their chunk's last head) each.
      // The kp rows were issued before the first stage, so they have landed
      // by the first wait.
      constexpr int later = []() {
        int n = 0;
        for (int j = 1; j < C::AHEAD; ++j) n += C::COPIES + (((hl + j) % G == G - 1) ? C::NPCOPY : 0);
        return n;
      }();
      wait_vmcnt<later>();
      __syncthreads();
      issue_next(std::integral_constant<int, (hl + C::AHEAD) % G>());
      __builtin_amdgcn_sched_barrier(0);
      const int s = ci * G + hl;
      const unsigned char* base = smem_raw + (s % C::NBUF) * C::STAGE_BYTES;
      main_part(base, lo, hi_, masked);
      if constexpr (hl == G - 1) proxy_part(base, lo, hi_, masked);
    });
    Tacc = zero16();
    if (++c == nch) { c = 0; ++li; }
  };
  // More than 4 heads: the heads of a chunk go in quads through a loop that is
  // not unrolled, so the stage code exists once per ring slot (stage s sits in
  // slot s % 4 = its head % 4).  Only the last quad carries the chunk's last
  // head: its qp copy, the extra copies the waits of its neighbours allow for,
  // and the proxy term are taken on a uniform branch.
  auto issue_next_rt = [&](int hl, auto with_qp_c) __attribute__((always_inline)) {
    constexpr bool with_qp = decltype(with_qp_c)::value;
    const bool past = fs >= nst;
    const int li_ = past ? len - 1 : fli;
    const int c_ = past ? nch - 1 : fc;
    issue_stage(fs % C::NBUF, li_, c_, hl, with_qp_c);
    ++fs;
    if constexpr (with_qp) {                     // branch-free, so the counters stay in registers
      const bool wrap = fc + 1 == nch;
      fli += wrap ? 1 : 0;
      fc = wrap ? 0 : fc + 1;
    }
  };
  auto chunk_body_quads = [&](bool masked) __attribute__((always_inline)) {
    const int I = lst[li] - qb0;
    const int qpos0 = I * g.Bq + c * 32;
    const int lo = kpos - qpos0, hi_ = L - qpos0;
    constexpr int NQ = G / 4;
    constexpr int BASE_LATER = (C::AHEAD - 1) * C::COPIES;
#pragma unroll 1
    for (int hq = 0; hq < NQ; ++hq) {
      const bool lastq = hq == NQ - 1;
      static_for<4>([&](auto jc) __attribute__((always_inline)) {
        constexpr int j = decltype(jc)::value;
        // stages s + 1 and s + 2 are in flight; one of them is the chunk's
        // last head (with its qp copy) when j is 1 or 2 in the last quad
        if constexpr (j == 1 || j == 2) {
          if (lastq) wait_vmcnt<BASE_LATER + C::NPCOPY>();
          else wait_vmcnt<BASE_LATER>();
        } else {
          wait_vmcnt<BASE_LATER>();
        }
        __syncthreads();
        if constexpr (j == 0) {
          if (lastq) issue_next_rt(G - 1, std::true_type());
          else issue_next_rt(hq * 4 + 3, std::false_type());
        } else {
          const int hn = hq * 4 + j + 3;
          issue_next_rt(hn < G ? hn : hn - G, std::false_type());
        }
        __builtin_amdgcn_sched_barrier(0);
        const unsigned char* base = smem_raw + j * C::STAGE_BYTES;
        main_part(base, lo, hi_, masked);
        if constexpr (j == 3) {
          if (lastq) proxy_part(base, lo, hi_, masked);
        }
      });
    }
    Tacc = zero16();
    const bool wrap = c + 1 == nch;
    li += wrap ? 1 : 0;
    c = wrap ? 0 : c + 1;
  };
  auto run_chunk = [&](int ci, bool masked) __attribute__((always_inline)) {
    if constexpr (G > 4) chunk_body_quads(masked);
    else chunk_body(ci, masked);
  };
  static_assert(G <= 4 || (G % 4 == 0 && C::NBUF == 4 && C::AHEAD == 3), "head quads");
  int ci = 0;
  for (; ci < nchunk_lead && ci < nchunk; ++ci) run_chunk(ci, true);
  for (; ci < nchunk_plain_end; ++ci) run_chunk(ci, false);
  for (; ci < nchunk; ++ci) run_chunk(ci, true);
  // copies issued past the last stage must land before the workgroup ends
  wait_vmcnt<0>();

  // outputs: lane holds column d = dt*32 + col for 16 key rows
  const float lam_ps = g.lam * g.pscale;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int key = J * 128 + wave * 32 + acc_row(i, lane);
    if (key < L) {
      const int64_t t = t0 + key;
      float* pk = dk + (t * g.Hkv + grp) * D;
      float* pv = dv + (t * g.Hkv + grp) * D;
#pragma unroll
      for (int dt = 0; dt < D / 32; ++dt) {
        pk[dt * 32 + col] = dK[dt][i] * g.scale;
        pv[dt * 32 + col] = dV[dt][i];
      }
      float* pp = dkp + (t * g.Hkv + grp) * DP;
#pragma unroll
      for (int dt = 0; dt < DP / 32; ++dt) pp[dt * 32 + col] = dKp[dt][i] * lam_ps;
    }
  }
}

static int grid_for_b(int64_t n, int threads) {
  int64_t b = (n + threads - 1) / threads;
  if (b < 1) b = 1;
  if (b > 65536) b = 65536;
  return (int)b;
}

template <typename T, int D, int DP>
static hipError_t bwd_dispatch(const Geo& g, const void* q, const void* k, const void* v,
                               const void* qp, const void* kp, const void* o, const float* lse,
                               const float* lse_p, const void* dout, const int32_t* q2k_idx,
                               const int32_t* q2k_cnt, const int32_t* k2q_ptr,
                               const int32_t* k2q_idx, float* dq, float* dk, float* dv, float* dqp,
                               float* dkp, const Work& w, hipStream_t s) {
  typedef DqCfg<T, D, DP> CQ;
  typedef KvCfg<T, D, DP> CK;
  // bf16, d = 128, dp = 64: the query-major pass is dq128 for every group
  // size and the KV-major pass the two-role kernel for 2, 4 and 8 heads per
  // group, so the generic kernels are built for the other shapes (and, here,
  // the KV-major pass of one head per group) only
  constexpr bool FAST = std::is_same<T, bf16>::value && D == 128 && DP == 64;
  static LdsLimitOnce lds_limit;
  {
    hipError_t e;
    if constexpr (FAST) {
      e = lds_limit.ensure({{(const void*)dkdv_kernel<T, D, DP, 1>, CK::LDS_BYTES}});
    } else {
      e = lds_limit.ensure({{(const void*)dq_kernel<T, D, DP>, CQ::LDS_BYTES},
                            {(const void*)dkdv_kernel<T, D, DP, 1>, CK::LDS_BYTES},
                            {(const void*)dkdv_kernel<T, D, DP, 2>, CK::LDS_BYTES},
                            {(const void*)dkdv_kernel<T, D, DP, 4>, CK::LDS_BYTES},
                            {(const void*)dkdv_kernel<T, D, DP, 8>, CK::LDS_BYTES}});
    }
    if (e != hipSuccess) return e;
  }
  hipError_t e;
  const int NU = g.G * (g.Bq / 32);
  const int64_t nq = (int64_t)g.Hkv * g.nqb * ((NU + 3) / 4);
  if constexpr (FAST) {
    if (!dq128_supported(g)) return hipErrorInvalidValue;
    { ProfScope _ps("bwd_dq", s);
    e = launch_dq128(g, q, k, v, qp, kp, o, lse, lse_p, dout, w.delta, w.lse2, w.lsep2, q2k_idx,
                     q2k_cnt, dq, dqp, w.queue, s); }
    if (e != hipSuccess) return e;
  } else if (nq > 0) {
    { ProfScope _ps("bwd_dq", s);
    hipLaunchKernelGGL((dq_kernel<T, D, DP>), dim3((unsigned)nq), dim3(256), CQ::LDS_BYTES, s,
                       (const T*)q, (const T*)k, (const T*)v, (const T*)qp, (const T*)kp, (const T*)o,
                       lse, lse_p, (const T*)dout, w.delta, w.lse2, w.lsep2, q2k_idx, q2k_cnt, dq, dqp,
                       w.cpart, g); }
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  if (!FAST && g.G > 4 && g.T > 0) {
    { ProfScope _ps("bwd_dqp_reduce", s);
    hipLaunchKernelGGL((dqp_reduce_kernel<DP>), dim3(grid_for_b((int64_t)g.T * g.Hkv * DP, 256)),
                       dim3(256), 0, s, w.cpart, dqp, g); }
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  const int64_t nk = (int64_t)g.Hkv * g.nkb;
  if (nk > 0 && FAST && dkdv128_supported(g)) {
    { ProfScope _ps("bwd_dkdv", s);
    e = launch_dkdv128(g, q, k, v, qp, kp, w.lse2, w.lsep2, dout, w.delta, k2q_ptr, k2q_idx, dk, dv,
                       dkp, w.queue + kQueueWords, s); }
    if (e != hipSuccess) return e;
  } else if (nk > 0) {
    { ProfScope _ps("bwd_dkdv", s);
#define MSA_LAUNCH_DKDV(GG)                                                                          \
    hipLaunchKernelGGL((dkdv_kernel<T, D, DP, GG>), dim3((unsigned)nk), dim3(256), CK::LDS_BYTES, s, \
                       (const T*)q, (const T*)k, (const T*)v, (const T*)qp, (const T*)kp, w.lse2,      \
                       w.lsep2, (const T*)dout, w.delta, k2q_ptr, k2q_idx, dk, dv, dkp, g)
    if constexpr (FAST) {
      switch (g.G) {
        case 1: MSA_LAUNCH_DKDV(1); break;       // G = 2, 4, 8: the two-role kernel
        default: return hipErrorInvalidValue;
      }
    } else {
      switch (g.G) {
        case 1: MSA_LAUNCH_DKDV(1); break;
        case 2: MSA_LAUNCH_DKDV(2); break;
        case 4: MSA_LAUNCH_DKDV(4); break;
        default: MSA_LAUNCH_DKDV(8); break;
      }
    }
#undef MSA_LAUNCH_DKDV
    }
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  return hipSuccess;
}

hipError_t launch_bwd(const Geo& g, int is_bf16, const void* q, const void* k, const void* v,
                      const void* qp, const void* kp, const void* o, const float* lse,
                      const float* lse_p, const void* dout, const int32_t* q2k_idx,
                      const int32_t* q2k_cnt, const int32_t* k2q_ptr, const int32_t* k2q_idx,
                      float* dq, float* dk, float* dv, float* dqp, float* dkp, const Work& w,
                      hipStream_t s) {
  if (is_bf16) {
    if (g.D == 128)
      return bwd_dispatch<bf16, 128, 64>(g, q, k, v, qp, kp, o, lse, lse_p, dout, q2k_idx, q2k_cnt,
                                         k2q_ptr, k2q_idx, dq, dk, dv, dqp, dkp, w, s);
    return bwd_dispatch<bf16, 64, 32>(g, q, k, v, qp, kp, o, lse, lse_p, dout, q2k_idx, q2k_cnt,
                                      k2q_ptr, k2q_idx, dq, dk, dv, dqp, dkp, w, s);
  }
  return bwd_dispatch<float, 64, 32>(g, q, k, v, qp, kp, o, lse, lse_p, dout, q2k_idx, q2k_cnt,
                                     k2q_ptr, k2q_idx, dq, dk, dv, dqp, dkp, w, s);
}

}  // namespace msa

namespace msa {
int bwd_kernels(KernelEntry* out, int max) {
  const KernelEntry all[] = {
      {"bwd_dkdv<bf16,d128,dp64,g1>", (const void*)dkdv_kernel<bf16, 128, 64, 1>, 256, KvCfg<bf16, 128, 64>::LDS_BYTES},
      {"bwd_dq<bf16,d64,dp32>", (const void*)dq_kernel<bf16, 64, 32>, 256, DqCfg<bf16, 64, 32>::LDS_BYTES},
      {"bwd_dkdv<bf16,d64,dp32,g1>", (const void*)dkdv_kernel<bf16, 64, 32, 1>, 256, KvCfg<bf16, 64, 32>::LDS_BYTES},
      {"bwd_dkdv<bf16,d64,dp32,g2>", (const void*)dkdv_kernel<bf16, 64, 32, 2>, 256, KvCfg<bf16, 64, 32>::LDS_BYTES},
      {"bwd_dkdv<bf16,d64,dp32,g4>", (const void*)dkdv_kernel<bf16, 64, 32, 4>, 256, KvCfg<bf16, 64, 32>::LDS_BYTES},
      {"bwd_dkdv<bf16,d64,dp32,g8>", (const void*)dkdv_kernel<bf16, 64, 32, 8>, 256, KvCfg<bf16, 64, 32>::LDS_BYTES},
      {"bwd_dq<f32,d64,dp32>", (const void*)dq_kernel<float, 64, 32>, 256, DqCfg<float, 64, 32>::LDS_BYTES},
      {"bwd_dkdv<f32,d64,dp32,g1>", (const void*)dkdv_kernel<float, 64, 32, 1>, 256, KvCfg<float, 64, 32>::LDS_BYTES},
      {"bwd_dkdv<f32,d64,dp32,g2>", (const void*)dkdv_kernel<float, 64, 32, 2>, 256, KvCfg<float, 64, 32>::LDS_BYTES},
      {"bwd_dkdv<f32,d64,dp32,g4>", (const void*)dkdv_kernel<float, 64, 32, 4>, 256, KvCfg<float, 64, 32>::LDS_BYTES},
      {"bwd_dkdv<f32,d64,dp32,g8>", (const void*)dkdv_kernel<float, 64, 32, 8>, 256, KvCfg<float, 64, 32>::LDS_BYTES},
      {"bwd_dqp_reduce<dp64>", (const void*)dqp_reduce_kernel<64>, 256, 0},
      {"bwd_dqp_reduce<dp32>", (const void*)dqp_reduce_kernel<32>, 256, 0},
  };
  int n = (int)(sizeof(all) / sizeof(all[0]));
  for (int i = 0; i < n && i < max; ++i) out[i] = all[i];
  return n;
}
}  // namespace msa
