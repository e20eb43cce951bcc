// Query-major backward for bf16 inputs with d = 128 and dp = 64: rowsum(dO O),
// dQ and the proxy gradient dqp, at two waves per SIMD.
//
// The pages fuse the proxy backward into the main backward (ai-minor
// "Dramatically Speeding Up Million-Token Training!", Why Does This Matter?;
// keelcrux "Flash-MSA: Ein Training mit einer Million Tokens", Le fait).  As
// in the KV-major pass, the proxy gradient is read as a distillation KL over
// the selected keys: T = mean over the group's heads of the main
// probabilities (held constant), Q = proxy softmax, dY = lam (Q - T); here
// dqp = s_p dY kp, which splits over the heads of a group as
// sum over heads of (Q on the key tiles assigned to the head - P / G) kp.
//
// Work decomposition: a work item is one (KV group, query block) (or half of
// one when it has more than eight 32-query units); the grid is persistent, one
// workgroup per CU taking items from a queue, and a workgroup runs eight waves; wave u owns 32 queries of one head (head u mod G, query chunk
// u / G), so a workgroup holds whole chunks for G in {1, 2, 4, 8} and sums the
// proxy term over their heads itself.  Stages are 64-key halves of the
// selected blocks, K, V and kp rows copied global -> LDS by DMA into a ring
// of three slots, two stages ahead, and shared by the eight waves.  A wave
// keeps its Q, dO and qp fragments and its dQ and proxy accumulators in
// registers (at most 256, so two waves share each SIMD without accumulator
// moves) and walks a stage as two 32-key tiles: S and dP (K and V rows from
// LDS), the softmax, then dQ += dS K and C += (-P / G) kp (transposed K and kp
// fragments from LDS); on the tiles assigned to its head also the proxy
// scores and C += Q kp.
#include "msa_device.h"
#include "msa_internal.h"
#include "msa_profile.h"

namespace msa {
namespace {

constexpr int QD = 128, QDP = 64, QKC = 64;            // head dim, proxy dim, keys per stage
constexpr int Q_NW = 8, Q_NT = 64 * Q_NW;
constexpr int Q_NBUF = 3, Q_AHEAD = Q_NBUF - 1;        // ring slots, stages in flight
constexpr int Q_KS = QKC * QD * 2;                     // bytes of a stage's K (or V) rows: 16 KiB
constexpr int Q_PS = QKC * QDP * 2;                    // bytes of its kp rows: 8 KiB
constexpr int Q_STAGE = 2 * Q_KS + Q_PS;
constexpr int Q_RING = Q_NBUF * Q_STAGE;               // 120 KiB
constexpr int Q_ITEM = Q_RING;                         // the workgroup's current work item
constexpr int Q_LDS = Q_RING + 256;
constexpr int Q_KCOPY = QKC / (Q_NW * 4);              // K (and V) copies per wave per stage, 4 rows each
constexpr int Q_PCOPY = QKC / (Q_NW * 8);              // kp copies per wave per stage, 8 rows each
constexpr int Q_COPIES = 2 * Q_KCOPY + Q_PCOPY;
constexpr int Q_RS = 33;                               // row stride (floats) of the reduction buffer
static_assert(Q_KCOPY >= 1 && Q_PCOPY >= 1, "copy split");
static_assert(Q_NW * QDP * Q_RS * 4 <= Q_RING, "reduction buffer");

// Two transpose reads joined into one fragment: the first at a + OFF, the
// second (8 rows further down) at b + OFF + OFF2.
template <int OFF, int OFF2>
__device__ __forceinline__ bf16x8 tr_two(uint32_t a, uint32_t b) {
  const bf16x4 x = lds_tr4_at<OFF>(a), y = lds_tr4_at<OFF + OFF2>(b);
  bf16x8 r;
#pragma unroll
  for (int j = 0; j < 4; ++j) { r[j] = x[j]; r[j + 4] = y[j]; }
  return r;
}

__global__ __launch_bounds__(Q_NT) void dq128_kernel(
    const bf16* __restrict__ q, const bf16* __restrict__ k, const bf16* __restrict__ v,
    const bf16* __restrict__ qp, const bf16* __restrict__ kp, const bf16* __restrict__ o,
    const float* __restrict__ lse, const float* __restrict__ lse_p, const bf16* __restrict__ dout,
    float* __restrict__ delta, float* __restrict__ lse2_out, float* __restrict__ lsep2_out,
    const int32_t* __restrict__ q2k_idx, const int32_t* __restrict__ q2k_cnt,
    float* __restrict__ dq, float* __restrict__ dqp, int32_t* __restrict__ queue, Geo g) {
  typedef Tile<bf16, QD> TK;
  typedef Tile<bf16, QDP> TP;
  extern __shared__ __align__(16) unsigned char smem_raw[];
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int NU = g.G * (g.Bq / 32);
  const int nwg = (NU + Q_NW - 1) / Q_NW;
  const int nitems = g.Hkv * g.nqb * nwg;
  const uint32_t item_lds = lds_offset(smem_raw) + Q_ITEM;
  int qi = 0;                                      // queues this workgroup has drained
  // Work items (a workgroup's share of one (group, query block)) come from
  // eight queues, one per XCD over a contiguous range of items; a workgroup
  // takes the next item of its own XCD's queue and, once that is empty, of
  // the others in turn (XCDs differ in speed by a few percent, and a fixed
  // split leaves the faster ones idle at the end).  Thread 0 takes it, a
  // barrier hands it to every wave.
  auto next_item = [&]() __attribute__((always_inline)) {
    if (tid == 0)
      *reinterpret_cast<__attribute__((address_space(3))) int*>((uintptr_t)item_lds) =
          queue_take(queue, nitems, blockIdx.x % kQueues, qi);
    __syncthreads();
    return __builtin_amdgcn_readfirstlane(
        *reinterpret_cast<__attribute__((address_space(3))) const int*>((uintptr_t)item_lds));
  };
  for (int bid; (bid = next_item()) >= 0;) {
  // lane values from an opaque copy of the lane index, so that they are
  // formed per item rather than kept live across items
  int lane = tid & 63;
  asm volatile("" : "+v"(lane));
  const int col = lane & 31, hi = lane >> 5;
  const int64_t item = bid / nwg;
  const int wgi = bid % nwg;
  const int grp = (int)(item / g.nqb);
  const int QB = (int)(item % g.nqb);
  const int u = wgi * Q_NW + wave;
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
  // and the only one that needs the causal mask
  int nst = 2 * cnt;
  if (diag * 128 + 64 > I * g.Bq + g.Bq - 1) nst -= 1;
  const int nst_plain = 2 * (cnt - 1);

  // Copy stage s (clamped to the last) into ring slot s % Q_NBUF through
  // buffer descriptors over the stage's rows: each lane's byte offset is
  // fixed.  A stage that runs past the document end (only in the diagonal
  // block, where the causal mask removes those rows) has its rows past the
  // end clamped to the last one: a copy past a descriptor's bound would leave
  // its LDS row unwritten, holding whatever the slot held before.
  const uint32_t lds0 = lds_offset(smem_raw);
  const uint32_t rsK = (uint32_t)g.Hkv * QD * 2, rsP = (uint32_t)g.Hp * QDP * 2;
  uint32_t voK[Q_KCOPY], voP[Q_PCOPY];
  int rK[Q_KCOPY], rP[Q_PCOPY];
#pragma unroll
  for (int j = 0; j < Q_KCOPY; ++j) {
    const int r = (wave * Q_KCOPY + j) * 4 + (lane >> 4), p = lane & 15;
    rK[j] = r;
    voK[j] = (uint32_t)r * rsK + (uint32_t)swz<16>(r, p) * 16;
  }
#pragma unroll
  for (int j = 0; j < Q_PCOPY; ++j) {
    const int r = (wave * Q_PCOPY + j) * 8 + (lane >> 3), p = lane & 7;
    rP[j] = r;
    voP[j] = (uint32_t)r * rsP + (uint32_t)swz<8>(r, p) * 16;
  }
  auto issue = [&](int s) __attribute__((always_inline)) {
    const int ss = s < nst ? s : nst - 1;
    const uint32_t base = lds0 + (uint32_t)((s % Q_NBUF) * Q_STAGE);
    const int key0 = (sel[ss >> 1] - kb0) * 128 + (ss & 1) * QKC;
    const int64_t row0 = (int64_t)(t0 + key0) * g.Hkv + grp;
    const int64_t rowp = (int64_t)(t0 + key0) * g.Hp + pg;
    const int last = L - 1 - key0;                  // last row of the document in the stage
    const i32x4 sK = make_srd(k + row0 * QD, QKC * rsK);
    const i32x4 sV = make_srd(v + row0 * QD, QKC * rsK);
    const i32x4 sP = make_srd(kp + rowp * QDP, QKC * rsP);
    uint32_t oK[Q_KCOPY], oP[Q_PCOPY];
#pragma unroll
    for (int j = 0; j < Q_KCOPY; ++j) oK[j] = voK[j];
#pragma unroll
    for (int j = 0; j < Q_PCOPY; ++j) oP[j] = voP[j];
    if (last < QKC - 1) {
#pragma unroll
      for (int j = 0; j < Q_KCOPY; ++j)
        if (rK[j] > last) oK[j] -= (uint32_t)(rK[j] - last) * rsK;
#pragma unroll
      for (int j = 0; j < Q_PCOPY; ++j)
        if (rP[j] > last) oP[j] -= (uint32_t)(rP[j] - last) * rsP;
    }
#pragma unroll
    for (int j = 0; j < Q_KCOPY; ++j) {
      const uint32_t dst = base + (uint32_t)((wave * Q_KCOPY + j) * 4 * QD * 2);
      bdma16(sK, oK[j], dst);
      bdma16(sV, oK[j], dst + Q_KS);
    }
#pragma unroll
    for (int j = 0; j < Q_PCOPY; ++j)
      bdma16(sP, oP[j], base + (uint32_t)(2 * Q_KS + (wave * Q_PCOPY + j) * 8 * QDP * 2));
  };

  bf16x8 Qf[QD / 16], dOf[QD / 16], QPf[QDP / 16];
  float lse2 = 0.f, dl = 0.f, lsep2 = 0.f;
  if (active) {
    const bf16* sq = q + (tq * g.Hq + h) * QD + hi * 8;
    const bf16* sd = dout + (tq * g.Hq + h) * QD + hi * 8;
    const bf16* so = o + (tq * g.Hq + h) * QD + hi * 8;
    float part = 0.f;                               // this lane's half of rowsum(dO * O)
#pragma unroll
    for (int ks = 0; ks < QD / 16; ++ks) {
      Qf[ks] = ld8(sq + ks * 16);
      dOf[ks] = ld8(sd + ks * 16);
      const bf16x8 of = ld8(so + ks * 16);
#pragma unroll
      for (int j = 0; j < 8; ++j) part = fmaf((float)dOf[ks][j], (float)of[j], part);
    }
    dl = part + __shfl_xor(part, 32, 64);
    const bf16* sp = qp + (tq * g.Hp + pg) * QDP + hi * 8;
#pragma unroll
    for (int ks = 0; ks < QDP / 16; ++ks) QPf[ks] = ld8(sp + ks * 16);
    lse2 = lse[(int64_t)h * g.T + tq] * LOG2E;
    lsep2 = lse_p[(int64_t)pg * g.T + tq] * LOG2E;
    // per-query values the KV-major pass reads: -D and both LSEs in log2 units
    if (hi == 0 && qpos < L) {
      delta[(int64_t)h * g.T + tq] = -dl;             // stored negated: -rowsum(dO * O)
      lse2_out[(int64_t)h * g.T + tq] = lse2;
      if (hl == 0) lsep2_out[(int64_t)grp * g.T + tq] = lsep2;
    }
  }
  // The register loads above complete before the first copies are issued, so
  // that the copies are the only vector-memory operations the waits count.
  wait_vmcnt<0>();
#pragma unroll
  for (int j = 0; j < Q_AHEAD; ++j) issue(j);

  // dQ^T and the proxy term C^T (dp x queries), both as accumulators in
  // registers
  f32x16 dQ[QD / 32], Cc[QDP / 32];
#pragma unroll
  for (int dt = 0; dt < QD / 32; ++dt) dQ[dt] = zero16();
#pragma unroll
  for (int dt = 0; dt < QDP / 32; ++dt) Cc[dt] = zero16();

  // This lane's LDS reads in a slot, as offsets from the slot base: row
  // fragments of K / V and of kp (16-column step ks at ^ (ks << 5)), and the
  // first of the two transpose reads of a K^T / kp^T fragment (32-column
  // block dt at ^ (dt << 6); the second read is at that ^ 32, 8 rows down).
  const int s16 = lane & 15, g4 = lane >> 4;
  const int tr_r = hi * 4 + (s16 >> 2), tr_c = 16 * (g4 & 1) + 4 * (s16 & 3);
  const uint32_t oRowK = (uint32_t)TK::off(col, hi * 8) * 2;
  const uint32_t oColK = (uint32_t)TK::off(tr_r, tr_c) * 2;
  const uint32_t oRowP = (uint32_t)(2 * Q_KS + TP::off(col, hi * 8) * 2);
  const uint32_t oColP = (uint32_t)(2 * Q_KS + TP::off(tr_r, tr_c) * 2);
  const float sl2 = g.scale_log2, psl2 = g.pscale_log2;
  // the weight of the proxy-softmax term folded into its exponent: qw Q =
  // exp2(Y s_p log2e - (lsep2 - log2 qw)) (exact for the weights used: 1 and
  // a power-of-two group count)
  const float lsepq = qw > 1.f ? lsep2 - __builtin_log2f(qw) : lsep2;
  const float ninvG = -1.f / (float)g.G;

  auto stage = [&](int s, auto masked_c) __attribute__((always_inline)) {
    constexpr bool MASKED = decltype(masked_c)::value;
    wait_vmcnt<Q_COPIES * (Q_AHEAD - 1)>();         // stage s has landed (own copies)
    __syncthreads();                                // everyone's; slot (s + 2) % 3 is free
    issue(s + Q_AHEAD);
    if (!active) return;
    const uint32_t sb = (uint32_t)__builtin_amdgcn_readfirstlane(
        (int)(lds0 + (uint32_t)((s % Q_NBUF) * Q_STAGE)));
    const uint32_t bRowK = lds_base_add(sb, oRowK), bColK = lds_base_add(sb, oColK);
    const uint32_t bRowP = lds_base_add(sb, oRowP), bColP = lds_base_add(sb, oColP);
    // causal mask of the diagonal block's stages: key row r of tile kt is
    // visible iff r <= lim0 - 32 kt, i.e. acc_row(i) < mw - 32 kt
    const int lim0 = qpos - ((sel[s >> 1] - kb0) * 128 + (s & 1) * QKC);
    const uint32_t mx = (uint32_t)(hi * 4);
    static_for<2>([&](auto ktc) __attribute__((always_inline)) {
      constexpr int kt = decltype(ktc)::value;
      constexpr int LOOK = 4;
      const int lim = lim0 - kt * 32 + 1;
      const uint32_t mw = lim > 0 ? (uint32_t)lim : 0u;
      // S^T = K Q^T and dP^T = V dO^T of the tile's 32 keys: 16 products,
      // K and V row fragments read LOOK products ahead
      f32x16 S = zero16(), dP = zero16();
      {
        bf16x8 op[16];
        uint32_t ad = 0;
        auto rd = [&](auto mc) __attribute__((always_inline)) {
          constexpr int m = decltype(mc)::value, ks = m / 2;
          if constexpr ((m & 1) == 0) ad = xr<(uint32_t)(ks << 5)>(bRowK);
          op[m] = lds_ld8<kt * 32 * QD * 2 + (m & 1) * Q_KS>(ad);
        };
        static_for<LOOK>([&](auto mc) __attribute__((always_inline)) { rd(mc); });
        static_for<16>([&](auto mc) __attribute__((always_inline)) {
          constexpr int m = decltype(mc)::value, ks = m / 2;
          if constexpr (m & 1) dP = __builtin_amdgcn_mfma_f32_32x32x16_bf16(op[m], dOf[ks], dP, 0, 0, 0);
          else S = __builtin_amdgcn_mfma_f32_32x32x16_bf16(op[m], Qf[ks], S, 0, 0, 0);
          if constexpr (m + LOOK < 16) rd(std::integral_constant<int, m + LOOK>());
        });
      }
      // softmax: P = exp2(S s log2e - lse2), dS = P (dP - D); both as bf16
      // operands in accumulator slots, P scaled by -1/G for the proxy term
      bf16x8 bs[2], bp[2];
      static_for<16>([&](auto ic) __attribute__((always_inline)) {
        constexpr int i = decltype(ic)::value;
        float p = __builtin_amdgcn_exp2f(fmaf(S[i], sl2, -lse2));
        if constexpr (MASKED) p = keep_if<(uint32_t)(((i >> 2) << 3) + (i & 3))>(p, mx, mw);
        bs[i >> 3][i & 7] = (bf16)(p * (dP[i] - dl));
        bp[i >> 3][i & 7] = (bf16)(p * ninvG);
      });
      // dQ^T += K^T dS^T (8 products), C^T += kp^T (-P / G)^T (4 products)
      {
        constexpr int NB = 2 * (QD / 32) + 2 * (QDP / 32);
        bf16x8 op[NB];
        uint32_t a0[QD / 32], a1[QD / 32], p0[QDP / 32], p1[QDP / 32];
        auto rd = [&](auto mc) __attribute__((always_inline)) {
          constexpr int m = decltype(mc)::value, kk = m / (NB / 2), c = m % (NB / 2);
          if constexpr (c < QD / 32) {
            if constexpr (kk == 0) {
              a0[c] = xr<(uint32_t)(c << 6)>(bColK);
              a1[c] = xr<32u>(a0[c]);
            }
            op[m] = tr_two<(kt * 32 + kk * 16) * QD * 2, 8 * QD * 2>(a0[c], a1[c]);
          } else {
            constexpr int dt = c - QD / 32;
            if constexpr (kk == 0) {
              p0[dt] = xr<(uint32_t)(dt << 6)>(bColP);
              p1[dt] = xr<32u>(p0[dt]);
            }
            op[m] = tr_two<(kt * 32 + kk * 16) * QDP * 2, 8 * QDP * 2>(p0[dt], p1[dt]);
          }
        };
        static_for<LOOK>([&](auto mc) __attribute__((always_inline)) { rd(mc); });
        static_for<NB>([&](auto mc) __attribute__((always_inline)) {
          constexpr int m = decltype(mc)::value, kk = m / (NB / 2), c = m % (NB / 2);
          if constexpr (c < QD / 32) dQ[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(op[m], bs[kk], dQ[c], 0, 0, 0);
          else Cc[c - QD / 32] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(op[m], bp[kk], Cc[c - QD / 32], 0, 0, 0);
          if constexpr (m + LOOK < NB) rd(std::integral_constant<int, m + LOOK>());
        });
      }
      // the proxy term of the tiles assigned to this head: Y^T = kp qp^T,
      // qw Q = exp2(Y s_p log2e - lsepq), C^T += kp^T (qw Q)^T (none where qw = 0)
      if (((s * 2 + kt) % g.G) == hl && qw != 0.f) {
        f32x16 Y = zero16();
        static_for<QDP / 16>([&](auto ksc) __attribute__((always_inline)) {
          constexpr int ks = decltype(ksc)::value;
          Y = __builtin_amdgcn_mfma_f32_32x32x16_bf16(lds_ld8<kt * 32 * QDP * 2>(xr<(uint32_t)(ks << 5)>(bRowP)),
                                                      QPf[ks], Y, 0, 0, 0);
        });
        bf16x8 bq[2];
        static_for<16>([&](auto ic) __attribute__((always_inline)) {
          constexpr int i = decltype(ic)::value;
          float qv = __builtin_amdgcn_exp2f(fmaf(Y[i], psl2, -lsepq));
          if constexpr (MASKED) qv = keep_if<(uint32_t)(((i >> 2) << 3) + (i & 3))>(qv, mx, mw);
          bq[i >> 3][i & 7] = (bf16)qv;
        });
        static_for<2>([&](auto kkc) __attribute__((always_inline)) {
          constexpr int kk = decltype(kkc)::value;
          static_for<QDP / 32>([&](auto dtc) __attribute__((always_inline)) {
            constexpr int dt = decltype(dtc)::value;
            const uint32_t x0 = xr<(uint32_t)(dt << 6)>(bColP);
            const uint32_t x1 = xr<32u>(x0);
            Cc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                tr_two<(kt * 32 + kk * 16) * QDP * 2, 8 * QDP * 2>(x0, x1), bq[kk], Cc[dt], 0, 0, 0);
          });
        });
      }
    });
  };

  int s = 0;
  for (; s < nst_plain; ++s) stage(s, std::false_type());
  for (; s < nst; ++s) stage(s, std::true_type());
  wait_vmcnt<0>();
  __syncthreads();

  // dQ out (fp32): lane holds query col, rows d = dt * 32 + acc_row(i)
  if (active && qpos < L) {
    float* dst = dq + ((int64_t)(t0 + qpos) * g.Hq + h) * QD;
#pragma unroll
    for (int dt = 0; dt < QD / 32; ++dt)
#pragma unroll
      for (int i4 = 0; i4 < 4; ++i4) {
        f32x4 r;
#pragma unroll
        for (int j = 0; j < 4; ++j) r[j] = dQ[dt][i4 * 4 + j] * g.scale;
        *reinterpret_cast<f32x4*>(dst + dt * 32 + acc_row(i4 * 4, lane)) = r;
      }
  }
  // proxy term: summed over the heads of each chunk, which all sit in this
  // workgroup (rows of 33 floats: every lane of a read in its own bank)
  float* red = reinterpret_cast<float*>(smem_raw);          // [Q_NW][QDP][Q_RS]
  if (active) {
#pragma unroll
    for (int dt = 0; dt < QDP / 32; ++dt)
#pragma unroll
      for (int i = 0; i < 16; ++i) red[(wave * QDP + dt * 32 + acc_row(i, lane)) * Q_RS + col] = Cc[dt][i];
  }
  __syncthreads();
  const int u_lo = wgi * Q_NW;
  const int u_hi = (u_lo + Q_NW < NU ? u_lo + Q_NW : NU) - 1;
  const int c_lo = u_lo / g.G, c_hi = u_hi / g.G;
  const int nel = (c_hi - c_lo + 1) * 32 * QDP;
  const float out_scale = g.pscale * g.lam;
  for (int e = tid; e < nel; e += Q_NT) {
    const int cidx = e / (32 * QDP);
    const int rem = e % (32 * QDP);
    const int qq = rem / QDP, dpi = rem % QDP;
    const int c = c_lo + cidx;
    float acc = 0.f;
    for (int w = 0; w < Q_NW; ++w) {
      const int uw = u_lo + w;
      if (uw < NU && uw / g.G == c) acc += red[(w * QDP + dpi) * Q_RS + qq];
    }
    const int pos = I * g.Bq + c * 32 + qq;
    if (pos < L) dqp[((int64_t)(t0 + pos) * g.Hkv + grp) * QDP + dpi] = acc * out_scale;
  }
  }
}


}  // namespace

bool dq128_supported(const Geo& g) { return g.G == 1 || g.G == 2 || g.G == 4 || g.G == 8; }

hipError_t launch_dq128(const Geo& g, const void* q, const void* k, const void* v, const void* qp,
                        const void* kp, const void* o, const float* lse, const float* lse_p,
                        const void* dout, float* delta, float* lse2, float* lsep2,
                        const int32_t* q2k_idx, const int32_t* q2k_cnt, float* dq, float* dqp,
                        int32_t* queue, hipStream_t s) {
  static LdsLimitOnce lds_limit;
  hipError_t e = lds_limit.ensure({{(const void*)dq128_kernel, Q_LDS}});
  if (e != hipSuccess) return e;
  const int NU = g.G * (g.Bq / 32);
  const int64_t n = (int64_t)g.Hkv * g.nqb * ((NU + Q_NW - 1) / Q_NW);
  if (n == 0) return hipSuccess;
  if (n > INT32_MAX / 2) return hipErrorInvalidValue;
  int ncu = 0;
  if ((e = device_cu_count(&ncu)) != hipSuccess) return e;
  const unsigned grid = (unsigned)(n < ncu ? n : ncu);      // one workgroup per CU (LDS-bound)
  if ((e = launch_queue_reset(queue, s)) != hipSuccess) return e;
  hipLaunchKernelGGL(dq128_kernel, dim3(grid), dim3(Q_NT), Q_LDS, s, (const bf16*)q,
                     (const bf16*)k, (const bf16*)v, (const bf16*)qp, (const bf16*)kp, (const bf16*)o,
                     lse, lse_p, (const bf16*)dout, delta, lse2, lsep2, q2k_idx, q2k_cnt, dq, dqp, queue, g);
  return hipGetLastError();
}

int bwd_q_kernels(KernelEntry* out, int max) {
  const KernelEntry all[] = {
      {"bwd_dq8<bf16,d128,dp64>", (const void*)dq128_kernel, Q_NT, Q_LDS},
  };
  int n = (int)(sizeof(all) / sizeof(all[0]));
  for (int i = 0; i < n && i < max; ++i) out[i] = all[i];
  return n;
}

}  // namespace msa
