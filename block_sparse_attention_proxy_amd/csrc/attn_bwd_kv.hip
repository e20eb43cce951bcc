// KV-major backward for bf16 inputs with d = 128 and dp = 64: dK, dV and the
// proxy gradient dkp, each KV block computed whole by one workgroup (no
// atomics on the outputs).
//
// The pages fuse the proxy backward into the main backward (ai-minor
// "Dramatically Speeding Up Million-Token Training!", Why Does This Matter?;
// keelcrux "Flash-MSA: Ein Training mit einer Million Tokens", Le fait).  As
// in the query-major pass, the proxy gradient is read as a distillation KL
// over the selected keys: T = mean over the group's heads of the main
// probabilities (held constant), Q = proxy softmax, dY = lam (Q - T), and here
// dkp = s_p dY^T qp.
//
// Work decomposition: a work item is one KV block of one group (128 keys).
// The grid is persistent, one workgroup per compute unit, and each workgroup
// takes items from a queue (one atomic counter per XCD) until all are done.
// Items differ in cost by two orders of magnitude (the inverted lists run
// from one entry to several hundred), and with one workgroup per item the
// hardware's in-order dispatch, which hands workgroups to the shader engines
// in turn, left compute units idle behind long items: about 16% of CU time
// on a 1M-token packing.  A workgroup runs eight waves, two per SIMD; the waves of key group kg (keys
// [32 kg, 32 kg + 32)) split the work of each stage between them (see the
// kernel below).  A stage is (entry of the block's inverted list, 32-query
// chunk, head): the Q and dO rows of the chunk for that head plus its LSE and
// rowsum(dO O) vectors (and, at a chunk's last head, the proxy rows qp and
// the proxy LSE) are copied global -> LDS by DMA into a six-slot ring, up to
// four stages ahead of the stage being computed.
//
// The copies use buffer descriptors: each stage's base address and valid
// byte count are scalar values, every lane's offset inside a stage is fixed,
// and rows past the end of the token range read as zeros (the descriptor's
// bound).  Rows past a document's end that are still inside the tensor are
// read and masked in the softmax.
#include "msa_device.h"
#include "msa_internal.h"
#include "msa_profile.h"

namespace msa {
namespace {


constexpr int KD = 128, KDP = 64, KQC = 32;
constexpr int TILE_B = KQC * KD * 2;                // one Q or dO tile of a stage: 8 KiB
constexpr int FL_VEC = 256;                         // one float vector: 32 valid floats + 32 zeros
constexpr int FL_SLOT = 4 * FL_VEC;                 // lse2, delta, lsep2, lsep2 (spare)
constexpr int QP_TILE = KQC * KDP * 2;              // 4 KiB

template <int OFF>
__device__ __forceinline__ f32x4 lds_f4(uint32_t base) {
  typedef __attribute__((address_space(3))) const f32x4 lds_f32x4;
  return *reinterpret_cast<lds_f32x4*>(reinterpret_cast<lds_u8*>((uintptr_t)base) + OFF);
}

// Two transpose reads joined into one fragment: the first at a + OFF, the
// second (8 rows further down) at b + OFF + OFF2.
template <int OFF, int OFF2>
__device__ __forceinline__ bf16x8 tr_pair2(uint32_t a, uint32_t b) {
  const bf16x4 x = lds_tr4_at<OFF>(a), y = lds_tr4_at<OFF + OFF2>(b);
  bf16x8 r;
#pragma unroll
  for (int j = 0; j < 4; ++j) { r[j] = x[j]; r[j + 4] = y[j]; }
  return r;
}

// ---------------------------------------------------------------------------
// Warp-specialized variant: eight waves, two per SIMD.  For key group kg
// (keys [32 kg, 32 kg + 32)) wave kg is the softmax wave and wave 4 + kg the
// accumulation wave; the two sit on the same SIMD, so the softmax wave's
// vector work and the accumulation wave's products issue side by side.
//
//   softmax wave, stage s:  S, dP (16 MFMAs: Q / dO rows x K / V fragments
//       in registers), P = exp2(S s log2e - lse2), dS = P (dP - D), both as
//       bf16 fragments into an exchange buffer; T += P; at a chunk's last
//       head the proxy scores Y = qp kp^T and dY / (lam s_p) = Q - T / G
//       into a second exchange buffer.
//   accumulation wave, stage s - 1:  dV += P^T dO and dK += dS^T Q
//       (16 MFMAs, transposed Q / dO fragments from the ring); at a chunk's
//       last head dkp += dY^T qp.  It also issues every copy.
//
// One workgroup barrier per stage orders the two: the exchange buffers are
// double-buffered by stage parity, and the ring slot a stage occupies is
// refilled only after the accumulation wave has passed it.
// ---------------------------------------------------------------------------
constexpr int WS_NB = 6;                               // ring of stages
constexpr int WS_SLOT = 2 * TILE_B;                    // Q tile, then dO tile
constexpr int WS_FL = WS_NB * WS_SLOT;                 // float vectors, FL_SLOT per slot
constexpr int WS_QP = WS_FL + WS_NB * FL_SLOT;         // qp tiles of up to three chunks
constexpr int WS_XB = WS_QP + 3 * QP_TILE;             // P / dS fragments [parity][kg][4][64 x 16 B]
constexpr int WS_XB_KG = 4 * 1024;
constexpr int WS_DY = WS_XB + 2 * 4 * WS_XB_KG;        // dY fragments [kg][2][64 x 16 B]
constexpr int WS_DUMMY = WS_DY + 4 * 2 * 1024;         // target of the placeholder copy, 256 B per wave
constexpr int WS_ITEM = WS_DUMMY + 4 * 256;           // the workgroup's current work item
constexpr int WS_LDS = WS_ITEM + 256;
static_assert(WS_LDS <= 160 * 1024, "LDS budget");
constexpr int WS_COPIES = 6;                           // per accumulation wave per stage (uniform)
constexpr int WS_LATER = WS_COPIES * (WS_NB - 3);      // copies of stages s+1 .. s+NB-3

// The qp rows of a chunk are copied with the copies of the chunk's last stage
// (its last head), issued four stages ahead of it, and read at that stage by
// both roles (by the accumulation wave one stage later).  With G heads a chunk
// spans G stages.  A ring of N slots is safe when the copy of chunk c + N,
// issued four stages before that chunk's last stage, comes at least two
// stages after chunk c's last stage (the iteration after its last read): G N
// >= 6, so two slots for G >= 4 and three for G = 2.
template <int G>
__device__ __forceinline__ uint32_t next_qp(uint32_t o) {
  constexpr uint32_t N = G == 2 ? 3u : 2u;               // qp slots in the ring
  return o == (N - 1) * (uint32_t)QP_TILE ? 0u : o + (uint32_t)QP_TILE;
}

__device__ __forceinline__ void lds_st16(uint32_t addr, const bf16x8& v) {
  typedef __attribute__((address_space(3))) bf16x8 lds_v8;
  *reinterpret_cast<lds_v8*>((uintptr_t)addr) = v;
}

template <int G>
__global__ __launch_bounds__(512) void dkdv_ws_kernel(
    const bf16* __restrict__ q, const bf16* __restrict__ k, const bf16* __restrict__ v,
    const bf16* __restrict__ qp, const bf16* __restrict__ kp, const float* __restrict__ lse2,
    const float* __restrict__ lsep2, const bf16* __restrict__ dout, const float* __restrict__ delta,
    const int32_t* __restrict__ k2q_ptr, const int32_t* __restrict__ k2q_idx,
    float* __restrict__ dk, float* __restrict__ dv, float* __restrict__ dkp, int32_t* __restrict__ queue,
    Geo g) {
  typedef Tile<bf16, KD> TQ;
  typedef Tile<bf16, KDP> TP;
  extern __shared__ __align__(16) unsigned char smem_raw[];
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const bool soft_role = wave < 4;
  const int kg = wave & 3;

  // Rows the descriptors leave unwritten are masked, but still enter products
  // with a zero weight; clearing LDS once keeps them finite.
  {
    f32x4 z;
#pragma unroll
    for (int j = 0; j < 4; ++j) z[j] = 0.f;
    for (int o = tid * 16; o < WS_LDS; o += 512 * 16) *reinterpret_cast<f32x4*>(smem_raw + o) = z;
  }
  const uint32_t lb = lds_offset(smem_raw);
  const uint32_t item_lds = lb + WS_ITEM;
  const int nk = g.Hkv * g.nkb;
  int qi = 0;                                              // queues this workgroup has drained

  // Work items are (group, KV block) pairs taken from eight queues, one per
  // XCD, each holding a contiguous range of the pairs; a workgroup takes its
  // next item from its own XCD's queue and, once that is empty, from the
  // others in turn.  Thread 0 takes it; a barrier hands it to every wave
  // (each role runs its own loop, with the same barriers per item).
  auto next_item = [&]() __attribute__((always_inline)) {
    if (tid == 0)
      *reinterpret_cast<__attribute__((address_space(3))) int*>((uintptr_t)item_lds) =
          queue_take(queue, nk, blockIdx.x % kQueues, qi);
    __syncthreads();
    return __builtin_amdgcn_readfirstlane(
        *reinterpret_cast<__attribute__((address_space(3))) const int*>((uintptr_t)item_lds));
  };
  struct Item { int grp, J, t0, L, qb0, pg, len; const int32_t* lst; };
  auto item_of = [&](int bid) __attribute__((always_inline)) {
    Item it;
    it.grp = bid / g.nkb;
    const int KB = bid % g.nkb;
    const int b = g.kdoc[KB];
    it.J = KB - g.kb0[b];
    it.t0 = g.cu[b];
    it.L = g.cu[b + 1] - it.t0;
    it.qb0 = g.qb0[b];
    it.pg = proxy_head(g, it.grp);                         // the proxy head this group reads
    const int32_t* ptr = k2q_ptr + (int64_t)it.pg * (g.nkb + 1);
    it.lst = k2q_idx + (int64_t)it.pg * g.cap + ptr[KB];
    it.len = ptr[KB + 1] - ptr[KB];
    return it;
  };
  const int nch = g.Bq / 32;

  if (soft_role) {
    // ======================= softmax wave ===================================
    for (int bid; (bid = next_item()) >= 0;) {
      const Item it = item_of(bid);
      const int grp = it.grp, J = it.J, t0 = it.t0, L = it.L, qb0 = it.qb0, pg = it.pg, len = it.len;
      const int32_t* lst = it.lst;
      // Lane-dependent values are derived per item from an opaque copy of the
      // lane index, so that the compiler forms them inside the loop instead of
      // keeping them live across items (which would exceed 256 registers).
      int lane = tid & 63;
      asm volatile("" : "+v"(lane));
      const int col = lane & 31, hi = lane >> 5;
      const uint32_t xb_lane = lb + WS_XB + kg * WS_XB_KG + lane * 16;   // + parity * 4 * WS_XB_KG + f * 1024
      const uint32_t dy_lane = lb + WS_DY + kg * 2048 + lane * 16;       // + f * 1024
      const int kpos = J * 128 + kg * 32 + col;               // this lane's key (fragment column)
      const int nst = len * nch * G;
      const int krow = kpos < L ? kpos : L - 1;
      const int64_t tk = t0 + krow;
      bf16x8 Kf[KD / 16], Vf[KD / 16], KPf[KDP / 16];
      {
        const bf16* sk = k + (tk * g.Hkv + grp) * KD + hi * 8;
        const bf16* sv = v + (tk * g.Hkv + grp) * KD + hi * 8;
        const bf16* sp = kp + (tk * g.Hp + pg) * KDP + hi * 8;
#pragma unroll
        for (int ks = 0; ks < KD / 16; ++ks) { Kf[ks] = ld8(sk + ks * 16); Vf[ks] = ld8(sv + ks * 16); }
#pragma unroll
        for (int ks = 0; ks < KDP / 16; ++ks) KPf[ks] = ld8(sp + ks * 16);
      }
      wait_vmcnt<0>();
      __syncthreads();                                       // LDS cleared before any copy lands

      // reads: Q / dO rows of a slot (address(ks) = bR ^ (ks << 5)), float
      // vectors, qp rows of a chunk (address(ks) = bP ^ (ks << 5))
      const uint32_t bR = lb + TQ::off(col, hi * 8) * 2;
      const uint32_t oF = lb + WS_FL + hi * 16;
      const uint32_t bP = lb + WS_QP + TP::off(col, hi * 8) * 2;
      int nmask = 0;
      while (nmask < len && nmask < 2 && (((lst[nmask] - qb0) * g.Bq) >> 7) == J) ++nmask;
      const bool tail = len > 0 && (lst[len - 1] - qb0 + 1) * g.Bq > L;


      // compute side
      int c_li = 0, c_c = 0, c_hl = 0;
      int c_I = len > 0 ? lst[0] - qb0 : 0;
      int c_next = len > 1 ? lst[1] - qb0 : c_I;
      f32x16 Tacc = zero16();
      const float sl2 = g.scale_log2, psl2 = g.pscale_log2;
      const float invG = 1.f / (float)G;
      int qwi = (int)proxy_qweight(g, grp);                  // weight of the proxy-softmax term
      asm volatile("" : "+v"(qwi));                          // (converted per item, not kept live)
      qwi = __builtin_amdgcn_readfirstlane(qwi);
      const float qw = (float)qwi;
      const uint32_t mw = (uint32_t)(L - kpos);
      f32x16 S[2], dP[2];                                    // [stage parity]
      // S, dP of stage t (16 products, operand reads LOOK ahead) into S[PAR],
      // dP[PAR]; between(m) runs after product m
      uint32_t c_so = 0, c_fo = 0, c_qo = 0;                 // LDS: slot of stage s, its floats, qp slot
      auto next_slot = [](uint32_t o, uint32_t step) __attribute__((always_inline)) {
        return o == (WS_NB - 1) * step ? 0u : o + step;
      };
      // dP starts from -D (the delta vectors hold -rowsum(dO O)), so that the
      // products give dP - D directly.
      auto products = [&](uint32_t so, uint32_t fo, auto par_c, auto&& between) __attribute__((always_inline)) {
        constexpr int PAR = decltype(par_c)::value;
        constexpr int LOOK = 4;
        const uint32_t rb = bR + so;
        const uint32_t fd = oF + fo;
        const f32x4 n0 = lds_f4<FL_VEC>(fd), n1 = lds_f4<FL_VEC + 32>(fd);
        const f32x4 n2 = lds_f4<FL_VEC + 64>(fd), n3 = lds_f4<FL_VEC + 96>(fd);
        f32x16 nD;
#pragma unroll
        for (int j = 0; j < 4; ++j) { nD[j] = n0[j]; nD[4 + j] = n1[j]; nD[8 + j] = n2[j]; nD[12 + j] = n3[j]; }
        bf16x8 op[16];
        uint32_t ad = 0;
        auto rd = [&](auto mc) __attribute__((always_inline)) {
          constexpr int m = decltype(mc)::value, ks = m / 2;
          if constexpr ((m & 1) == 0) ad = xr<(uint32_t)(ks << 5)>(rb);
          op[m] = lds_ld8<(m & 1) * TILE_B>(ad);
        };
        static_for<LOOK>([&](auto mc) __attribute__((always_inline)) { rd(mc); });
        static_for<16>([&](auto mc) __attribute__((always_inline)) {
          constexpr int m = decltype(mc)::value, ks = m / 2;
          if constexpr (m & 1)
            dP[PAR] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(op[m], Vf[ks], m == 1 ? nD : dP[PAR], 0, 0, 0);
          else
            S[PAR] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(op[m], Kf[ks], m == 0 ? zero16() : S[PAR], 0, 0, 0);
          if constexpr (m + LOOK < 16) rd(std::integral_constant<int, m + LOOK>());
          between(mc);
          __builtin_amdgcn_sched_barrier(0);
        });
      };

      // prologue: stage 0 has landed at the second barrier; its products.
      __syncthreads();
      __builtin_amdgcn_sched_barrier(0);
      products(0u, 0u, std::integral_constant<int, 0>(), [&](auto) __attribute__((always_inline)) {});

      // Iteration s: the products of stage s + 1 with the softmax of stage s
      // between them (P, dS to the exchange buffer), then at a chunk's last head
      // the proxy term.
      auto iteration = [&](int s, auto par_c) __attribute__((always_inline)) {
        constexpr int PAR = decltype(par_c)::value;
        __syncthreads();                                     // stage s + 1 has landed
        __builtin_amdgcn_sched_barrier(0);
        const uint32_t fb = oF + c_fo;
        const int qpos0 = c_I * g.Bq + c_c * 32;
        const bool masked = c_li < nmask || (tail && c_li == len - 1);
        const uint32_t mx = (uint32_t)(hi * 4 - kpos + qpos0);
        const uint32_t xb = xb_lane + (uint32_t)(s & 1) * 4 * WS_XB_KG;
        auto run = [&](auto masked_c) __attribute__((always_inline)) {
          constexpr bool MASKED = decltype(masked_c)::value;
          f32x4 lv[4];
          bf16x8 ap[2], as[2];
          lv[0] = lds_f4<0>(fb);
          products(next_slot(c_so, WS_SLOT), next_slot(c_fo, FL_SLOT), std::integral_constant<int, PAR ^ 1>(),
                   [&](auto mc) __attribute__((always_inline)) {
            constexpr int i = decltype(mc)::value;
            if constexpr ((i & 3) == 1 && i < 13) lv[(i + 3) / 4] = lds_f4<((i + 3) / 4) * 32>(fb);
            float pv = __builtin_amdgcn_exp2f(fmaf(S[PAR][i], sl2, -lv[i >> 2][i & 3]));
            if constexpr (MASKED) pv = keep_if<(uint32_t)(((i >> 2) << 3) + (i & 3))>(pv, mx, mw);
            Tacc[i] += pv;
            ap[i >> 3][i & 7] = (bf16)pv;
            as[i >> 3][i & 7] = (bf16)(pv * dP[PAR][i]);
            if constexpr ((i & 7) == 7) {
              lds_st16(xb + (i >> 3) * 1024, ap[i >> 3]);
              lds_st16(xb + (2 + (i >> 3)) * 1024, as[i >> 3]);
            }
          });
        };
        if (masked) run(std::true_type());
        else run(std::false_type());

        if (c_hl == G - 1) {
          // proxy term of the chunk: Y = qp kp^T, dY / (lam s_p) = qw Q - T / G
          // (only -T / G where qw = 0)
          // Q_MODE: 0 no proxy-softmax term (qw = 0), 1 weight 1, 2 weight qw
          auto proxy_dy = [&](auto masked_c, auto q_mode_c) __attribute__((always_inline)) {
            constexpr bool MASKED = decltype(masked_c)::value;
            constexpr int Q_MODE = decltype(q_mode_c)::value;
            f32x16 Y;
            if constexpr (Q_MODE != 0) {
              const uint32_t pb = bP + c_qo;
              Y = zero16();
              static_for<KDP / 16>([&](auto ksc) __attribute__((always_inline)) {
                constexpr int ks = decltype(ksc)::value;
                Y = __builtin_amdgcn_mfma_f32_32x32x16_bf16(lds_ld8<0>(xr<(uint32_t)(ks << 5)>(pb)), KPf[ks], Y, 0, 0, 0);
              });
            }
            static_for<2>([&](auto hc) __attribute__((always_inline)) {
              constexpr int h8 = decltype(hc)::value;
              bf16x8 ay;
              if constexpr (Q_MODE != 0) {
                const f32x4 l0 = lds_f4<2 * FL_VEC + (2 * h8) * 32>(fb), l1 = lds_f4<2 * FL_VEC + (2 * h8 + 1) * 32>(fb);
                static_for<8>([&](auto ec) __attribute__((always_inline)) {
                  constexpr int e = decltype(ec)::value, i = h8 * 8 + e;
                  const float lpv = e < 4 ? l0[e & 3] : l1[e & 3];
                  float qv = __builtin_amdgcn_exp2f(fmaf(Y[i], psl2, -lpv));
                  if constexpr (MASKED) qv = keep_if<(uint32_t)(((i >> 2) << 3) + (i & 3))>(qv, mx, mw);
                  if constexpr (Q_MODE == 2) qv *= qw;
                  ay[e] = (bf16)fmaf(-invG, Tacc[i], qv);
                });
              } else {
                static_for<8>([&](auto ec) __attribute__((always_inline)) {
                  constexpr int e = decltype(ec)::value, i = h8 * 8 + e;
                  ay[e] = (bf16)(-invG * Tacc[i]);
                });
              }
              lds_st16(dy_lane + h8 * 1024, ay);
            });
          };
          using Q0 = std::integral_constant<int, 0>;
          using Q1 = std::integral_constant<int, 1>;
          using Q2 = std::integral_constant<int, 2>;
          if (qwi == 1) {
            if (masked) proxy_dy(std::true_type(), Q1());
            else proxy_dy(std::false_type(), Q1());
          } else if (qwi != 0) {
            if (masked) proxy_dy(std::true_type(), Q2());
            else proxy_dy(std::false_type(), Q2());
          } else {
            proxy_dy(std::false_type(), Q0());
          }
          Tacc = zero16();
          c_hl = 0;
          c_qo = next_qp<G>(c_qo);
          if (++c_c == nch) {
            c_c = 0;
            ++c_li;
            c_I = c_next;
            const int nx = c_li + 1 < len ? c_li + 1 : len - 1;
            if (nx >= 0) c_next = __builtin_amdgcn_readfirstlane(lst[nx]) - qb0;
          }
        } else {
          ++c_hl;
        }
        c_so = next_slot(c_so, WS_SLOT);
        c_fo = next_slot(c_fo, FL_SLOT);
        __builtin_amdgcn_sched_barrier(0);
      };
      for (int s = 0; s < nst; s += 2) {
        iteration(s, std::integral_constant<int, 0>());
        if (s + 1 < nst) iteration(s + 1, std::integral_constant<int, 1>());
      }
      __syncthreads();                                       // the last stage's P, dS are visible
    }
  } else {
    // ===================== accumulation wave ================================
    for (int bid; (bid = next_item()) >= 0;) {
      const Item it = item_of(bid);
      const int grp = it.grp, J = it.J, t0 = it.t0, L = it.L, qb0 = it.qb0, pg = it.pg, len = it.len;
      const int32_t* lst = it.lst;
      // Lane-dependent values are derived per item from an opaque copy of the
      // lane index, so that the compiler forms them inside the loop instead of
      // keeping them live across items (which would exceed 256 registers).
      int lane = tid & 63;
      asm volatile("" : "+v"(lane));
      const int col = lane & 31, hi = lane >> 5;
      const uint32_t xb_lane = lb + WS_XB + kg * WS_XB_KG + lane * 16;   // + parity * 4 * WS_XB_KG + f * 1024
      const uint32_t dy_lane = lb + WS_DY + kg * 2048 + lane * 16;       // + f * 1024
      const int kpos = J * 128 + kg * 32 + col;               // this lane's key (fragment column)
      const int nst = len * nch * G;
      __syncthreads();                                       // LDS cleared before any copy lands
      // The accumulation waves issue every copy (the softmax waves carry the
      // longer instruction stream).  Stages 0 .. 3 go first; before barrier s
      // stage s + 1 has landed (own copies by count, the others' by the
      // barrier), and after it stage s + 4 refills the slot of stage s - 2,
      // which this wave finished before the barrier.
      const uint32_t rs_q = (uint32_t)g.Hq * KD * 2;
      const uint32_t rs_p = (uint32_t)g.Hp * KDP * 2;
      uint32_t voQ[2], ldQ[2];
#pragma unroll
      for (int jj = 0; jj < 2; ++jj) {
        const int rfirst = (kg * 2 + jj) * 4;                // 4 rows of 256 B per copy
        const int r = rfirst + (lane >> 4), p = lane & 15;
        voQ[jj] = (uint32_t)r * rs_q + (uint32_t)swz<16>(r, p) * 16;
        ldQ[jj] = lb + rfirst * 256;
      }
      const uint32_t voF = lane * 4;
      const uint32_t ldF = lb + WS_FL + kg * FL_VEC;
      uint32_t voP, ldP;
      {
        const int rfirst = kg * 8;                           // 8 rows of 128 B per copy
        const int r = rfirst + (lane >> 3), p = lane & 7;
        voP = (uint32_t)r * rs_p + (uint32_t)swz<8>(r, p) * 16;
        ldP = lb + WS_QP + rfirst * 128;
      }
      const uint32_t ldD = lb + WS_DUMMY + kg * 256;
      const bf16* qh = q + (int64_t)grp * G * KD;
      const bf16* dh = dout + (int64_t)grp * G * KD;
      const bf16* qpg = qp + (int64_t)pg * KDP;
      const float* fw = kg == 0 ? lse2 + (int64_t)grp * G * g.T
                      : kg == 1 ? delta + (int64_t)grp * G * g.T
                      : lsep2 + (int64_t)grp * g.T;
      const int fhs = kg < 2 ? g.T : 0;

      // issue side: the next stage's source addresses and LDS offsets are
      // advanced incrementally (one head: +256 B of Q / dO rows, +T floats of
      // lse2 / delta; one chunk: new rows), so a copy costs few scalar steps
      int i_li = 0, i_c = 0, i_hl = 0;
      int i_next = len > 1 ? lst[1] - qb0 : 0;
      auto rows_of = [&](int tr, bool live) __attribute__((always_inline)) {
        const int left = g.T - tr;
        return live && left > 0 ? (uint32_t)(left < KQC ? left : KQC) : 0u;
      };
      const int64_t dq_off = (const char*)dh - (const char*)qh;   // dO rows = Q rows + this
      const int64_t fstep = (int64_t)fhs * 4;
      const char* i_qa;                                      // Q rows of the next stage's head
      const char* i_fa;                                      // its float vector
      const char* i_pa;                                      // qp rows of its chunk
      uint32_t i_nq, i_nf, i_np;                             // valid bytes of each
      auto set_chunk = [&](int tr, bool live) __attribute__((always_inline)) {
        const uint32_t rows = rows_of(tr, live);
        i_qa = (const char*)(qh + (int64_t)tr * g.Hq * KD);
        i_fa = (const char*)(fw + tr);
        i_pa = (const char*)(qpg + (int64_t)tr * g.Hp * KDP);
        i_nq = rows * rs_q;
        i_nf = rows * 4;
        i_np = rows * rs_p;
      };
      int i_tr = t0 + (len > 0 ? lst[0] - qb0 : 0) * g.Bq;
      set_chunk(i_tr, len > 0);
      uint32_t i_so = 0, i_fo = 0, i_qo = 0;                 // LDS: slot, float slot, qp slot
      // One stage's copies in six parts, so that the main loop can spread them
      // between its products: a part that waits for room in the memory
      // pipeline then stalls one product, not the whole batch.
      i32x4 i_sq, i_sd;
      auto issue_part = [&](auto kc) __attribute__((always_inline)) {
        constexpr int k = decltype(kc)::value;
        if constexpr (k == 0) {
          i_sq = make_srd(i_qa, i_nq);
          i_sd = make_srd(i_qa + dq_off, i_nq);
          bdma16(i_sq, voQ[0], ldQ[0] + i_so);
        } else if constexpr (k == 1) {
          bdma16(i_sd, voQ[0], ldQ[0] + i_so + TILE_B);
        } else if constexpr (k == 2) {
          bdma16(i_sq, voQ[1], ldQ[1] + i_so);
        } else if constexpr (k == 3) {
          bdma16(i_sd, voQ[1], ldQ[1] + i_so + TILE_B);
        } else if constexpr (k == 4) {
          bdma4(make_srd(i_fa, i_nf), voF, ldF + i_fo);
        } else {
          if (i_hl == G - 1) {
            bdma16(make_srd(i_pa, i_np), voP, ldP + i_qo);
            i_qo = next_qp<G>(i_qo);
            i_hl = 0;
            if (++i_c == nch) {
              i_c = 0;
              ++i_li;
              i_tr = t0 + i_next * g.Bq;
              const int nx = i_li + 1 < len ? i_li + 1 : len - 1;
              if (nx >= 0) i_next = __builtin_amdgcn_readfirstlane(lst[nx]) - qb0;
            } else {
              i_tr += 32;
            }
            set_chunk(i_tr, i_li < len);
          } else {
            bdma4(make_srd(fw, 0u), voF, ldD);             // placeholder: keeps the copy count uniform
            ++i_hl;
            i_qa += KD * 2;
            i_fa += fstep;
          }
          i_so = i_so == (WS_NB - 1) * WS_SLOT ? 0u : i_so + WS_SLOT;
          i_fo = i_fo == (WS_NB - 1) * FL_SLOT ? 0u : i_fo + FL_SLOT;
        }
      };
      auto issue = [&]() __attribute__((always_inline)) {
        static_for<WS_COPIES>([&](auto kc) __attribute__((always_inline)) { issue_part(kc); });
      };
      for (int j = 0; j < WS_NB - 2; ++j) issue();
      wait_vmcnt<WS_COPIES * (WS_NB - 3)>();               // stage 0
      __syncthreads();
      const uint32_t bC = lb + TQ::off(hi * 4 + ((lane & 15) >> 2), 16 * ((lane >> 4) & 1) + 4 * (lane & 3)) * 2;
      const uint32_t bPc = lb + WS_QP + TP::off(hi * 4 + ((lane & 15) >> 2), 16 * ((lane >> 4) & 1) + 4 * (lane & 3)) * 2;
      f32x16 dK[KD / 32], dV[KD / 32], dKp[KDP / 32];
#pragma unroll
      for (int dt = 0; dt < KD / 32; ++dt) { dK[dt] = zero16(); dV[dt] = zero16(); }
#pragma unroll
      for (int dt = 0; dt < KDP / 32; ++dt) dKp[dt] = zero16();
      int hl = 0;                                            // head of stage s - 1
      uint32_t a_so = 0, a_qo = 0;                           // LDS: its slot, its chunk's qp slot
      // Stage s - 1's products, with stage s + 4's copies between them when
      // ISSUE (every iteration but the last).
      auto accumulate = [&](int s, auto issue_c) __attribute__((always_inline)) {
        constexpr bool ISSUE = decltype(issue_c)::value;
        const int sp = s - 1;
        const uint32_t cb = bC + a_so;
        a_so = a_so == (WS_NB - 1) * WS_SLOT ? 0u : a_so + WS_SLOT;
        const uint32_t xb = xb_lane + (uint32_t)(sp & 1) * 4 * WS_XB_KG;
        const bf16x8 ap0 = lds_ld8<0>(xb), ap1 = lds_ld8<1024>(xb);
        const bf16x8 as0 = lds_ld8<2048>(xb), as1 = lds_ld8<3072>(xb);
        {
          constexpr int LOOK = 4;
          bf16x8 op[16];
          uint32_t a0[KD / 32], a1[KD / 32];                 // transpose-read addresses per dt
          auto rd = [&](auto mc) __attribute__((always_inline)) {
            constexpr int m = decltype(mc)::value;
            constexpr int kk = m / 8, dt = (m % 8) / 2;
            // odd products: Q^T (dK), even: dO^T (dV)
            constexpr int OFF = ((m & 1) ? 0 : TILE_B) + kk * 16 * KD * 2;
            if constexpr (kk == 0 && (m & 1) == 0) {
              a0[dt] = xr<(uint32_t)(dt << 6)>(cb);
              a1[dt] = xr<32u>(a0[dt]);
            }
            op[m] = tr_pair2<OFF, 2048>(a0[dt], a1[dt]);
          };
          static_for<LOOK>([&](auto mc) __attribute__((always_inline)) { rd(mc); });
          static_for<16>([&](auto mc) __attribute__((always_inline)) {
            constexpr int m = decltype(mc)::value;
            constexpr int kk = m / 8, dt = (m % 8) / 2;
            const bf16x8& A = (m & 1) ? (kk ? as1 : as0) : (kk ? ap1 : ap0);
            if constexpr (m & 1) dK[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A, op[m], dK[dt], 0, 0, 0);
            else dV[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A, op[m], dV[dt], 0, 0, 0);
            if constexpr (m + LOOK < 16) rd(std::integral_constant<int, m + LOOK>());
            if constexpr (ISSUE && (m & 1) && m / 2 < WS_COPIES) {
              __builtin_amdgcn_sched_barrier(0);
              issue_part(std::integral_constant<int, m / 2>());
              __builtin_amdgcn_sched_barrier(0);
            }
          });
        }
        if (hl == G - 1) {
          // dkp += dY^T qp over the chunk that ended at stage s - 1
          const uint32_t pb = bPc + a_qo;
          a_qo = next_qp<G>(a_qo);
          const bf16x8 ay0 = lds_ld8<0>(dy_lane), ay1 = lds_ld8<1024>(dy_lane);
          static_for<2>([&](auto kkc) __attribute__((always_inline)) {
            constexpr int kk = decltype(kkc)::value;
            static_for<KDP / 32>([&](auto dtc) __attribute__((always_inline)) {
              constexpr int dt = decltype(dtc)::value;
              const uint32_t p0 = xr<(uint32_t)(dt << 6)>(pb);
              const uint32_t p1 = xr<32u>(p0);
              const bf16x8 bp = tr_pair2<kk * 16 * KDP * 2, 1024>(p0, p1);
              dKp[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kk ? ay1 : ay0, bp, dKp[dt], 0, 0, 0);
            });
          });
          hl = 0;
        } else {
          ++hl;
        }
      };
      if (nst > 0) {
        // iteration 0: stage 0 has landed; stage 4's copies, no products
        wait_vmcnt<WS_COPIES * (WS_NB - 4)>();
        __syncthreads();
        issue();
        for (int s = 1; s < nst; ++s) {
          wait_vmcnt<WS_COPIES * (WS_NB - 4)>();             // stage s + 1
          __syncthreads();
          accumulate(s, std::true_type());
        }
      }
      __syncthreads();
      if (nst > 0) accumulate(nst, std::false_type());
      wait_vmcnt<0>();                                       // copies past the last stage
      // outputs: lane holds column d = dt * 32 + col for 16 key rows
      const float lam_ps = g.lam * g.pscale;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int key = J * 128 + kg * 32 + acc_row(i, lane);
        if (key < L) {
          const int64_t t = t0 + key;
          float* pk = dk + (t * g.Hkv + grp) * KD;
          float* pv = dv + (t * g.Hkv + grp) * KD;
#pragma unroll
          for (int dt = 0; dt < KD / 32; ++dt) {
            pk[dt * 32 + col] = dK[dt][i] * g.scale;
            pv[dt * 32 + col] = dV[dt][i];
          }
          float* pp = dkp + (t * g.Hkv + grp) * KDP;
#pragma unroll
          for (int dt = 0; dt < KDP / 32; ++dt) pp[dt * 32 + col] = dKp[dt][i] * lam_ps;
        }
      }
    }
  }
}

}  // namespace

bool dkdv128_supported(const Geo& g) { return g.G == 2 || g.G == 4 || g.G == 8; }

hipError_t launch_dkdv128(const Geo& g, const void* q, const void* k, const void* v,
                          const void* qp, const void* kp, const float* lse2, const float* lsep2,
                          const void* dout, const float* delta, const int32_t* k2q_ptr,
                          const int32_t* k2q_idx, float* dk, float* dv, float* dkp, int32_t* queue,
                          hipStream_t s) {
  static LdsLimitOnce lds_limit;
  hipError_t e = lds_limit.ensure({{(const void*)dkdv_ws_kernel<2>, WS_LDS},
                                   {(const void*)dkdv_ws_kernel<4>, WS_LDS},
                                   {(const void*)dkdv_ws_kernel<8>, WS_LDS}});
  if (e != hipSuccess) return e;
  const int64_t nk = (int64_t)g.Hkv * g.nkb;
  if (nk == 0) return hipSuccess;
  if (nk > INT32_MAX / 2) return hipErrorInvalidValue;
  int ncu = 0;
  if ((e = device_cu_count(&ncu)) != hipSuccess) return e;
  const unsigned grid = (unsigned)(nk < ncu ? nk : ncu);     // one workgroup per CU (LDS-bound)
  if ((e = launch_queue_reset(queue, s)) != hipSuccess) return e;
#define MSA_LAUNCH_KV(GG)                                                                            \
  hipLaunchKernelGGL((dkdv_ws_kernel<GG>), dim3(grid), dim3(512), WS_LDS, s,                         \
                     (const bf16*)q, (const bf16*)k, (const bf16*)v, (const bf16*)qp, (const bf16*)kp,  \
                     lse2, lsep2, (const bf16*)dout, delta, k2q_ptr, k2q_idx, dk, dv, dkp, queue, g)
  switch (g.G) {
    case 2: MSA_LAUNCH_KV(2); break;
    case 4: MSA_LAUNCH_KV(4); break;
    case 8: MSA_LAUNCH_KV(8); break;
    default: return hipErrorInvalidValue;
  }
#undef MSA_LAUNCH_KV
  return hipGetLastError();
}

int bwd_kv_kernels(KernelEntry* out, int max) {
  const KernelEntry all[] = {
      {"bwd_dkdv_ws<g2>", (const void*)dkdv_ws_kernel<2>, 512, WS_LDS},
      {"bwd_dkdv_ws<g4>", (const void*)dkdv_ws_kernel<4>, 512, WS_LDS},
      {"bwd_dkdv_ws<g8>", (const void*)dkdv_ws_kernel<8>, 512, WS_LDS},
  };
  int n = (int)(sizeof(all) / sizeof(all[0]));
  for (int i = 0; i < n && i < max; ++i) out[i] = all[i];
  return n;
}

}  // namespace msa
