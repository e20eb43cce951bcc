// C ABI of the MSA hot path: argument checks, buffer layout, workspace
// carving and launches.  Every check runs on the host before anything is
// enqueued; errors are returned as msa_status with a thread-local message.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <string>
#include <vector>

#include "../../include/msa.h"
#include "msa_internal.h"
#include "msa_profile.h"

namespace {

thread_local std::string g_last_error;

msa_status fail(msa_status s, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return s;
}

msa_status hip_fail(hipError_t e, const char* where) {
  return fail(MSA_ERR_HIP, "%s: %s", where, hipGetErrorString(e));
}

constexpr int64_t kAlign = 256;
int64_t align_up(int64_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

// Host view of one call: sizes plus workspace region offsets.
struct Plan {
  msa::Geo g{};
  msa_layout lay{};
  int64_t off_qb0, off_kb0, off_s0, off_order, off_unit0, off_slab0, off_qdoc, off_kdoc, off_counts, off_totals;
  int64_t off_delta, off_lse2, off_lsep2, off_cpart, off_queue;
  // one proxy head shared by every KV group: the kernels read the one head
  // for every group, and the backward writes per-group proxy gradients here
  // before they are averaged (used only when shared)
  bool shared = false;
  int32_t Hp = 0;                    // proxy heads: the group count of scoring and selection
  int64_t off_dqpb, off_dkpb;
};

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

msa_status plan(const msa_config* cfg, const msa_varlen* vl, Plan* P) {
  g_last_error.clear();
  if (!cfg || !vl) return fail(MSA_ERR_INVALID_ARG, "cfg and vl must be non-null");
  const msa_config& c = *cfg;
  if (c.heads_kv <= 0 || c.heads_q <= 0)
    return fail(MSA_ERR_INVALID_ARG, "heads_q (%d) and heads_kv (%d) must be positive", c.heads_q, c.heads_kv);
  if (c.heads_q % c.heads_kv != 0)
    return fail(MSA_ERR_INVALID_ARG, "heads_q (%d) must be a multiple of heads_kv (%d)", c.heads_q, c.heads_kv);
  const int G = c.heads_q / c.heads_kv;
  if (G != 1 && G != 2 && G != 4 && G != 8)
    return fail(MSA_ERR_UNSUPPORTED, "group size %d not built (heads_q / heads_kv must be 1, 2, 4 or 8)", G);
  if (c.dtype != MSA_BF16 && c.dtype != MSA_F32) return fail(MSA_ERR_INVALID_ARG, "unknown dtype %d", c.dtype);
  const bool dims_ok = (c.head_dim == 128 && c.proxy_dim == 64 && c.dtype == MSA_BF16) ||
                       (c.head_dim == 64 && c.proxy_dim == 32);
  if (!dims_ok)
    return fail(MSA_ERR_UNSUPPORTED, "(head_dim, proxy_dim, dtype) = (%d, %d, %s) not built; built: (128, 64, bf16), (64, 32, bf16|f32)",
                c.head_dim, c.proxy_dim, c.dtype == MSA_BF16 ? "bf16" : "f32");
  if (c.kv_block != 128) return fail(MSA_ERR_UNSUPPORTED, "kv_block must be 128 (got %d)", c.kv_block);
  if (c.q_block != 64 && c.q_block != 128)
    return fail(MSA_ERR_UNSUPPORTED, "q_block must be 64 or 128 (got %d)", c.q_block);
  if (c.topk < 1) return fail(MSA_ERR_INVALID_ARG, "topk must be >= 1 (got %d)", c.topk);
  if (c.local_window < 0) return fail(MSA_ERR_INVALID_ARG, "local_window must be >= 0 (got %d)", c.local_window);
  if ((int64_t)c.topk + c.local_window > (1 << 20))
    return fail(MSA_ERR_INVALID_ARG, "topk + local_window too large");
  if (c.dilation < 0) return fail(MSA_ERR_INVALID_ARG, "dilation must be >= 0 (got %d)", c.dilation);
  const int64_t dil = c.dilation > 1 ? c.dilation : 1;
  if ((int64_t)c.local_window * dil > (1 << 20))
    return fail(MSA_ERR_INVALID_ARG, "local_window * dilation too large");
  const int64_t span = (int64_t)c.local_window * dil;
  if (c.proxy_heads != 0 && c.proxy_heads != 1 && c.proxy_heads != c.heads_kv)
    return fail(MSA_ERR_INVALID_ARG, "proxy_heads must be 0, 1 or heads_kv (got %d)", c.proxy_heads);
  const int64_t Hp = c.proxy_heads == 1 ? 1 : c.heads_kv;
  if (!(c.softmax_scale >= 0.f) || !std::isfinite(c.softmax_scale) || !(c.proxy_scale >= 0.f) ||
      !std::isfinite(c.proxy_scale) || !std::isfinite(c.proxy_loss_weight))
    return fail(MSA_ERR_INVALID_ARG, "scales must be finite and >= 0, the loss weight finite");
  if (vl->batch < 1) return fail(MSA_ERR_INVALID_ARG, "batch must be >= 1 (got %d)", vl->batch);
  if (vl->total_tokens < 0) return fail(MSA_ERR_INVALID_ARG, "total_tokens must be >= 0");
  if (!vl->cu_seqlens_host) return fail(MSA_ERR_INVALID_ARG, "cu_seqlens_host must be non-null");
  const int32_t* cu = vl->cu_seqlens_host;
  if (cu[0] != 0) return fail(MSA_ERR_INVALID_ARG, "cu_seqlens[0] must be 0 (got %d)", cu[0]);
  int64_t nqb = 0, nkb = 0, se = 0, pairs = 0, max_nq = 0, units = 0, slabs = 0;
  for (int b = 0; b < vl->batch; ++b) {
    const int64_t L = (int64_t)cu[b + 1] - cu[b];
    if (L < 0) return fail(MSA_ERR_INVALID_ARG, "cu_seqlens decreases at index %d", b + 1);
    const int64_t nq = (L + c.q_block - 1) / c.q_block, nk = (L + 127) / 128;
    nqb += nq;
    nkb += nk;
    se += nq * nk;
    if (nq > max_nq) max_nq = nq;
    units += ((L + 127) / 128 + 1) / 2;
    slabs += (nk + msa::K2Q_SLAB - 1) / msa::K2Q_SLAB;
    for (int64_t I = 0; I < nq; ++I) {
      const int64_t diag = I * c.q_block / 128;
      const int64_t pool = diag - span;           // candidates: blocks below the window's span
      if (pool <= (int64_t)c.topk - 1) continue;  // all of them are taken, no score needed
      const int64_t rows = std::min<int64_t>(c.q_block, L - I * c.q_block);
      pairs += rows * pool * 128;
    }
  }
  if (cu[vl->batch] != vl->total_tokens)
    return fail(MSA_ERR_INVALID_ARG, "cu_seqlens[batch] (%d) != total_tokens (%d)", cu[vl->batch], vl->total_tokens);
  if (max_nq > 16384)
    return fail(MSA_ERR_UNSUPPORTED, "a document of %lld query blocks exceeds the 16384 supported",
                (long long)max_nq);
  if (nqb * ((int64_t)c.topk + c.local_window) > INT32_MAX || se * (int64_t)c.heads_kv > ((int64_t)1 << 40))
    return fail(MSA_ERR_UNSUPPORTED, "problem too large for 32-bit block indexing");

  msa::Geo& g = P->g;
  g.Hq = c.heads_q; g.Hkv = c.heads_kv; g.G = G; g.D = c.head_dim; g.DP = c.proxy_dim;
  g.Bq = c.q_block; g.topk = c.topk; g.lw = c.local_window; g.stride = c.topk + c.local_window;
  g.dil = (int32_t)dil; g.span = (int32_t)span;
  g.B = vl->batch; g.T = vl->total_tokens; g.nqb = (int32_t)nqb; g.nkb = (int32_t)nkb;
  g.max_nq = (int32_t)max_nq; g.cap = nqb * g.stride; g.score_elems = se; g.n_units = (int32_t)units;
  g.nslab = (int32_t)slabs;
  g.k2q_chunks = (int32_t)((max_nq + msa::K2Q_CHUNK - 1) / msa::K2Q_CHUNK);
  g.scale = c.softmax_scale > 0.f ? c.softmax_scale : 1.f / std::sqrt((float)c.head_dim);
  g.pscale = c.proxy_scale > 0.f ? c.proxy_scale : 1.f / std::sqrt((float)c.proxy_dim);
  g.lam = c.proxy_loss_weight;
  g.scale_log2 = g.scale * 1.4426950408889634f;
  g.pscale_log2 = g.pscale * 1.4426950408889634f;
  g.cu = vl->cu_seqlens;

  const int64_t B = vl->batch;
  int64_t off = 0;
  P->off_qb0 = off;    off = align_up(off + 4 * (B + 1));
  P->off_kb0 = off;    off = align_up(off + 4 * (B + 1));
  P->off_s0 = off;     off = align_up(off + 8 * (B + 1));
  P->off_order = off;  off = align_up(off + 4 * B);
  P->off_unit0 = off;  off = align_up(off + 4 * (B + 1));
  P->off_slab0 = off;  off = align_up(off + 4 * (B + 1));
  P->off_qdoc = off;   off = align_up(off + 4 * nqb);
  P->off_kdoc = off;   off = align_up(off + 4 * nkb);
  P->off_counts = off;
  off = align_up(off + 4 * (int64_t)c.heads_kv * slabs * ((max_nq + msa::K2Q_CHUNK - 1) / msa::K2Q_CHUNK) * msa::K2Q_SLAB);
  P->off_totals = off; off = align_up(off + 4 * (int64_t)c.heads_kv * nkb);
  P->off_delta = off;  off = align_up(off + 4 * (int64_t)c.heads_q * vl->total_tokens);
  P->off_lse2 = off;   off = align_up(off + 4 * (int64_t)c.heads_q * vl->total_tokens);
  P->off_lsep2 = off;  off = align_up(off + 4 * (int64_t)c.heads_kv * vl->total_tokens);
  P->off_cpart = off;
  if (G > 4) off = align_up(off + 4 * (int64_t)c.heads_kv * (G / 4) * vl->total_tokens * c.proxy_dim);
  P->off_queue = off;  off = align_up(off + 4 * msa::kQueueSets * msa::kQueueWords);
  P->shared = Hp == 1 && c.heads_kv > 1;
  P->Hp = (int32_t)Hp;
  g.Hp = (int32_t)Hp;
  if (P->shared) {
    const int64_t T = vl->total_tokens, Hkv = c.heads_kv;
    P->off_dqpb = off; off = align_up(off + 4 * T * Hkv * c.proxy_dim);
    P->off_dkpb = off; off = align_up(off + 4 * T * Hkv * c.proxy_dim);
  }

  msa_layout& l = P->lay;
  l.total_qblocks = nqb;
  l.total_kvblocks = nkb;
  l.score_elems = se;
  l.sel_stride = g.stride;
  l.k2q_capacity = g.cap;
  l.scored_pairs = pairs;
  l.max_qblocks_doc = max_nq;
  l.workspace_bytes = off;
  l.proxy_heads = Hp;
  return MSA_OK;
}

msa_status bind_workspace(Plan* P, void* ws, size_t ws_bytes, msa::Work* w) {
  if (!ws) return fail(MSA_ERR_INVALID_ARG, "workspace must be non-null");
  if (!aligned16(ws)) return fail(MSA_ERR_INVALID_ARG, "workspace must be 16-byte aligned");
  if ((int64_t)ws_bytes < P->lay.workspace_bytes)
    return fail(MSA_ERR_WORKSPACE, "workspace of %zu bytes; %lld needed", ws_bytes,
                (long long)P->lay.workspace_bytes);
  if (!P->g.cu) return fail(MSA_ERR_INVALID_ARG, "cu_seqlens (device) must be non-null");
  char* base = static_cast<char*>(ws);
  P->g.qb0 = reinterpret_cast<int32_t*>(base + P->off_qb0);
  P->g.kb0 = reinterpret_cast<int32_t*>(base + P->off_kb0);
  P->g.s0 = reinterpret_cast<int64_t*>(base + P->off_s0);
  P->g.order = reinterpret_cast<int32_t*>(base + P->off_order);
  P->g.unit0 = reinterpret_cast<int32_t*>(base + P->off_unit0);
  P->g.qdoc = reinterpret_cast<int32_t*>(base + P->off_qdoc);
  P->g.kdoc = reinterpret_cast<int32_t*>(base + P->off_kdoc);
  P->g.slab0 = reinterpret_cast<int32_t*>(base + P->off_slab0);
  if (w) {
    w->counts = reinterpret_cast<int32_t*>(base + P->off_counts);
    w->totals = reinterpret_cast<int32_t*>(base + P->off_totals);
    w->delta = reinterpret_cast<float*>(base + P->off_delta);
    w->lse2 = reinterpret_cast<float*>(base + P->off_lse2);
    w->lsep2 = reinterpret_cast<float*>(base + P->off_lsep2);
    w->cpart = reinterpret_cast<float*>(base + P->off_cpart);
    w->queue = reinterpret_cast<int32_t*>(base + P->off_queue);
  }
  return MSA_OK;
}

// Geometry of scoring and selection (one group per proxy head), taken from
// the plan after the workspace is bound.
msa::Geo proxy_geo(const Plan& P) {
  msa::Geo g = P.g;
  g.Hkv = P.Hp;
  return g;
}

// Every per-document table a kernel reads must point into a bound workspace.
msa_status check_bound(const msa::Geo& g) {
  if (!g.cu || !g.qb0 || !g.kb0 || !g.s0 || !g.order || !g.unit0 || !g.qdoc || !g.kdoc || !g.slab0)
    return fail(MSA_ERR_INVALID_ARG, "internal: workspace tables not bound");
  return MSA_OK;
}

msa_status check_ptrs(std::initializer_list<std::pair<const void*, const char*>> ps) {
  for (auto& p : ps) {
    if (!p.first) return fail(MSA_ERR_INVALID_ARG, "%s must be non-null", p.second);
    if (!aligned16(p.first)) return fail(MSA_ERR_INVALID_ARG, "%s must be 16-byte aligned", p.second);
  }
  return MSA_OK;
}

// ---- per-kernel timing -----------------------------------------------------
struct ProfRecord {
  const char* name;
  hipEvent_t start, stop;
};
struct ProfAgg {
  std::string name;
  double ms;
  int64_t launches;
};
thread_local bool t_prof_on = false;
thread_local std::vector<hipEvent_t> t_pool;
thread_local std::vector<ProfRecord> t_records;
thread_local std::vector<ProfAgg> t_agg;
thread_local const char* t_open_name = nullptr;
thread_local hipEvent_t t_open_start = nullptr;

hipEvent_t pool_get() {
  if (!t_pool.empty()) {
    hipEvent_t e = t_pool.back();
    t_pool.pop_back();
    return e;
  }
  hipEvent_t e = nullptr;
  if (hipEventCreate(&e) != hipSuccess) return nullptr;
  return e;
}

}  // namespace

namespace msa {
bool prof_enabled() { return t_prof_on; }
void prof_begin(const char* name, hipStream_t s) {
  t_open_name = name;
  t_open_start = pool_get();
  if (t_open_start) (void)hipEventRecord(t_open_start, s);
}
void prof_end(hipStream_t s) {
  hipEvent_t stop = pool_get();
  if (!t_open_start || !stop) return;
  (void)hipEventRecord(stop, s);
  t_records.push_back({t_open_name, t_open_start, stop});
  t_open_start = nullptr;
}
}  // namespace msa

namespace {

// Per-group proxy gradients of a shared head in a bound workspace.
struct SharedGrads {
  float *dqp, *dkp;
};

SharedGrads shared_grads(const Plan& P, void* ws) {
  char* base = static_cast<char*>(ws);
  SharedGrads b;
  b.dqp = reinterpret_cast<float*>(base + P.off_dqpb);
  b.dkp = reinterpret_cast<float*>(base + P.off_dkpb);
  return b;
}

}  // namespace

extern "C" {

msa_status msa_profile_enable(int32_t on) {
  g_last_error.clear();
  t_prof_on = on != 0;
  return MSA_OK;
}

int32_t msa_profile_collect(void) {
  t_agg.clear();
  for (const ProfRecord& r : t_records) {
    float ms = 0.f;
    if (hipEventSynchronize(r.stop) == hipSuccess && hipEventElapsedTime(&ms, r.start, r.stop) == hipSuccess) {
      bool found = false;
      for (ProfAgg& a : t_agg)
        if (a.name == r.name) { a.ms += ms; a.launches += 1; found = true; break; }
      if (!found) t_agg.push_back({r.name, (double)ms, 1});
    }
    t_pool.push_back(r.start);
    t_pool.push_back(r.stop);
  }
  t_records.clear();
  return (int32_t)t_agg.size();
}

msa_status msa_profile_entry(int32_t index, char* name, size_t name_len, double* total_ms,
                             int64_t* launches) {
  g_last_error.clear();
  if (index < 0 || index >= (int32_t)t_agg.size())
    return fail(MSA_ERR_INVALID_ARG, "profile entry %d out of range", index);
  if (name && name_len > 0) {
    std::strncpy(name, t_agg[index].name.c_str(), name_len - 1);
    name[name_len - 1] = '\0';
  }
  if (total_ms) *total_ms = t_agg[index].ms;
  if (launches) *launches = t_agg[index].launches;
  return MSA_OK;
}


int32_t msa_abi_version(void) { return MSA_ABI_VERSION; }

const char* msa_status_string(msa_status s) {
  switch (s) {
    case MSA_OK: return "ok";
    case MSA_ERR_INVALID_ARG: return "invalid argument";
    case MSA_ERR_UNSUPPORTED: return "unsupported configuration";
    case MSA_ERR_HIP: return "HIP error";
    case MSA_ERR_WORKSPACE: return "workspace too small";
  }
  return "unknown status";
}

const char* msa_last_error(void) { return g_last_error.c_str(); }

msa_status msa_get_layout(const msa_config* cfg, const msa_varlen* vl, msa_layout* out) {
  if (!out) return fail(MSA_ERR_INVALID_ARG, "out must be non-null");
  Plan P;
  msa_status s = plan(cfg, vl, &P);
  if (s != MSA_OK) return s;
  *out = P.lay;
  return MSA_OK;
}

msa_status msa_proxy_scores(const msa_config* cfg, const msa_varlen* vl, const void* qp,
                            const void* kp, float* block_scores, void* workspace,
                            size_t workspace_bytes, void* stream) {
  Plan P;
  msa_status s = plan(cfg, vl, &P);
  if (s != MSA_OK) return s;
  if (P.g.T == 0) return MSA_OK;
  if ((s = check_ptrs({{qp, "qp"}, {kp, "kp"}, {block_scores, "block_scores"}})) != MSA_OK) return s;
  if ((s = bind_workspace(&P, workspace, workspace_bytes, nullptr)) != MSA_OK) return s;
  if ((s = check_bound(P.g)) != MSA_OK) return s;
  hipStream_t st = static_cast<hipStream_t>(stream);
  hipError_t e = msa::launch_meta(P.g, st);
  if (e != hipSuccess) return hip_fail(e, "metadata");
  const msa::Geo gp = proxy_geo(P);
  if ((s = check_bound(gp)) != MSA_OK) return s;
  e = msa::launch_proxy_scores(gp, cfg->dtype == MSA_BF16, qp, kp, block_scores, st);
  if (e != hipSuccess) return hip_fail(e, "proxy_scores");
  return MSA_OK;
}

msa_status msa_select_blocks(const msa_config* cfg, const msa_varlen* vl, const float* block_scores,
                             int32_t* q2k_idx, int32_t* q2k_cnt, int32_t* k2q_ptr,
                             int32_t* k2q_idx, void* workspace, size_t workspace_bytes,
                             void* stream) {
  Plan P;
  msa_status s = plan(cfg, vl, &P);
  if (s != MSA_OK) return s;
  if (P.g.T == 0) return MSA_OK;
  if ((s = check_ptrs({{block_scores, "block_scores"}, {q2k_idx, "q2k_idx"}, {q2k_cnt, "q2k_cnt"},
                       {k2q_ptr, "k2q_ptr"}, {k2q_idx, "k2q_idx"}})) != MSA_OK)
    return s;
  msa::Work w;
  if ((s = bind_workspace(&P, workspace, workspace_bytes, &w)) != MSA_OK) return s;
  if ((s = check_bound(P.g)) != MSA_OK) return s;
  hipStream_t st = static_cast<hipStream_t>(stream);
  hipError_t e = msa::launch_meta(P.g, st);
  if (e != hipSuccess) return hip_fail(e, "metadata");
  const msa::Geo gp = proxy_geo(P);
  if ((s = check_bound(gp)) != MSA_OK) return s;
  e = msa::launch_select(gp, block_scores, q2k_idx, q2k_cnt, k2q_ptr, k2q_idx, w, st);
  if (e != hipSuccess) return hip_fail(e, "select_blocks");
  return MSA_OK;
}

msa_status msa_select_blocks_noalloc(const msa_config* cfg, const msa_varlen* vl,
                                     const float* block_scores, int32_t* q2k_idx, int32_t* q2k_cnt,
                                     int32_t* k2q_ptr, int32_t* k2q_idx, void* stream) {
  Plan P;
  msa_status s = plan(cfg, vl, &P);
  if (s != MSA_OK) return s;
  if (P.g.T == 0) return MSA_OK;
  if ((s = check_ptrs({{block_scores, "block_scores"}, {q2k_idx, "q2k_idx"}, {q2k_cnt, "q2k_cnt"},
                       {k2q_ptr, "k2q_ptr"}, {k2q_idx, "k2q_idx"}})) != MSA_OK)
    return s;
  if (!P.g.cu) return fail(MSA_ERR_INVALID_ARG, "cu_seqlens (device) must be non-null");
  // selection reads the workspace prefix only: the per-document tables and
  // the inverted-index counts, which end where the backward's vectors begin
  const int64_t need = P.off_delta;
  if (need > (int64_t)msa::kNoAllocScratchBytes)
    return fail(MSA_ERR_WORKSPACE,
                "msa_select_blocks_noalloc needs %lld bytes of scratch; its static scratch holds %lld "
                "(use msa_select_blocks with a workspace)",
                (long long)need, (long long)msa::kNoAllocScratchBytes);
  void* scr = nullptr;
  hipError_t e = msa::noalloc_scratch(&scr);
  if (e != hipSuccess) return hip_fail(e, "scratch address");
  char* base = static_cast<char*>(scr);
  P.g.qb0 = reinterpret_cast<int32_t*>(base + P.off_qb0);
  P.g.kb0 = reinterpret_cast<int32_t*>(base + P.off_kb0);
  P.g.s0 = reinterpret_cast<int64_t*>(base + P.off_s0);
  P.g.order = reinterpret_cast<int32_t*>(base + P.off_order);
  P.g.unit0 = reinterpret_cast<int32_t*>(base + P.off_unit0);
  P.g.qdoc = reinterpret_cast<int32_t*>(base + P.off_qdoc);
  P.g.kdoc = reinterpret_cast<int32_t*>(base + P.off_kdoc);
  P.g.slab0 = reinterpret_cast<int32_t*>(base + P.off_slab0);
  msa::Work w{};
  w.counts = reinterpret_cast<int32_t*>(base + P.off_counts);
  w.totals = reinterpret_cast<int32_t*>(base + P.off_totals);
  if ((s = check_bound(P.g)) != MSA_OK) return s;
  hipStream_t st = static_cast<hipStream_t>(stream);
  e = msa::launch_meta(P.g, st);
  if (e != hipSuccess) return hip_fail(e, "metadata");
  const msa::Geo gp = proxy_geo(P);
  if ((s = check_bound(gp)) != MSA_OK) return s;
  e = msa::launch_select(gp, block_scores, q2k_idx, q2k_cnt, k2q_ptr, k2q_idx, w, st);
  if (e != hipSuccess) return hip_fail(e, "select_blocks");
  return MSA_OK;
}

int64_t msa_select_blocks_noalloc_max_bytes(void) { return (int64_t)msa::kNoAllocScratchBytes; }

msa_status msa_fwd(const msa_config* cfg, const msa_varlen* vl, const void* q, const void* k,
                   const void* v, const void* qp, const void* kp, const int32_t* q2k_idx,
                   const int32_t* q2k_cnt, void* o, float* lse, float* lse_p, void* workspace,
                   size_t workspace_bytes, void* stream) {
  Plan P;
  msa_status s = plan(cfg, vl, &P);
  if (s != MSA_OK) return s;
  if (P.g.T == 0) return MSA_OK;
  if ((s = check_ptrs({{q, "q"}, {k, "k"}, {v, "v"}, {qp, "qp"}, {kp, "kp"}, {q2k_idx, "q2k_idx"},
                       {q2k_cnt, "q2k_cnt"}, {o, "o"}, {lse, "lse"}, {lse_p, "lse_p"}})) != MSA_OK)
    return s;
  if ((s = bind_workspace(&P, workspace, workspace_bytes, nullptr)) != MSA_OK) return s;
  if ((s = check_bound(P.g)) != MSA_OK) return s;
  hipStream_t st = static_cast<hipStream_t>(stream);
  hipError_t e = msa::launch_meta(P.g, st);
  if (e != hipSuccess) return hip_fail(e, "metadata");
  // every group reads the proxy head's block lists; the proxy log-sum-exp is
  // taken once per proxy head
  // the forward's work-queue counters: the third set in the workspace
  int32_t* queue = reinterpret_cast<int32_t*>(static_cast<char*>(workspace) + P.off_queue) + 2 * msa::kQueueWords;
  e = msa::launch_fwd(P.g, proxy_geo(P), cfg->dtype == MSA_BF16, q, k, v, qp, kp, q2k_idx, q2k_cnt, o, lse,
                      lse_p, queue, st);
  if (e != hipSuccess) return hip_fail(e, "fwd");
  return MSA_OK;
}

msa_status msa_bwd(const msa_config* cfg, const msa_varlen* vl, const void* q, const void* k,
                   const void* v, const void* qp, const void* kp, const void* o, const float* lse,
                   const float* lse_p, const void* dout, const int32_t* q2k_idx,
                   const int32_t* q2k_cnt, const int32_t* k2q_ptr, const int32_t* k2q_idx,
                   float* dq, float* dk, float* dv, float* dqp, float* dkp, void* workspace,
                   size_t workspace_bytes, void* stream) {
  Plan P;
  msa_status s = plan(cfg, vl, &P);
  if (s != MSA_OK) return s;
  if (P.g.T == 0) return MSA_OK;
  if ((s = check_ptrs({{q, "q"}, {k, "k"}, {v, "v"}, {qp, "qp"}, {kp, "kp"}, {o, "o"}, {lse, "lse"},
                       {lse_p, "lse_p"}, {dout, "dout"}, {q2k_idx, "q2k_idx"}, {q2k_cnt, "q2k_cnt"},
                       {k2q_ptr, "k2q_ptr"}, {k2q_idx, "k2q_idx"}, {dq, "dq"}, {dk, "dk"}, {dv, "dv"},
                       {dqp, "dqp"}, {dkp, "dkp"}})) != MSA_OK)
    return s;
  msa::Work w;
  if ((s = bind_workspace(&P, workspace, workspace_bytes, &w)) != MSA_OK) return s;
  if ((s = check_bound(P.g)) != MSA_OK) return s;
  hipStream_t st = static_cast<hipStream_t>(stream);
  hipError_t e = msa::launch_meta(P.g, st);
  if (e != hipSuccess) return hip_fail(e, "metadata");
  if (P.shared) {
    // every group reads the shared head; its proxy gradients, one per group
    // (the proxy-softmax term in group 0 only), are averaged over the groups
    SharedGrads b = shared_grads(P, workspace);
    const int64_t T = P.g.T, Hkv = P.g.Hkv, dp = P.g.DP;
    e = msa::launch_bwd(P.g, cfg->dtype == MSA_BF16, q, k, v, qp, kp, o, lse, lse_p, dout, q2k_idx,
                        q2k_cnt, k2q_ptr, k2q_idx, dq, dk, dv, b.dqp, b.dkp, w, st);
    if (e != hipSuccess) return hip_fail(e, "bwd");
    if ((e = msa::launch_group_mean(b.dqp, dqp, T, (int)Hkv, dp, st)) != hipSuccess)
      return hip_fail(e, "shared proxy gradients");
    if ((e = msa::launch_group_mean(b.dkp, dkp, T, (int)Hkv, dp, st)) != hipSuccess)
      return hip_fail(e, "shared proxy gradients");
    return MSA_OK;
  }
  e = msa::launch_bwd(P.g, cfg->dtype == MSA_BF16, q, k, v, qp, kp, o, lse, lse_p, dout, q2k_idx,
                      q2k_cnt, k2q_ptr, k2q_idx, dq, dk, dv, dqp, dkp, w, st);
  if (e != hipSuccess) return hip_fail(e, "bwd");
  return MSA_OK;
}

static std::vector<msa::KernelEntry> all_kernels() {
  constexpr int kMax = 128;
  std::vector<msa::KernelEntry> v(kMax);
  int n = 0;
  n += msa::select_kernels(v.data() + n, kMax - n);
  n += msa::fwd_kernels(v.data() + n, kMax - n);
  n += msa::bwd_kernels(v.data() + n, kMax - n);
  n += msa::bwd_kv_kernels(v.data() + n, kMax - n);
  n += msa::bwd_q_kernels(v.data() + n, kMax - n);
  n += msa::share_kernels(v.data() + n, kMax - n);
  v.resize(n);
  return v;
}

int32_t msa_kernel_count(void) { return (int32_t)all_kernels().size(); }

msa_status msa_kernel_info(int32_t index, char* name, size_t name_len, int32_t* regs,
                           int32_t* lds_bytes, int32_t* scratch_bytes, int32_t* wg_per_cu) {
  g_last_error.clear();
  auto ks = all_kernels();
  if (index < 0 || index >= (int32_t)ks.size()) return fail(MSA_ERR_INVALID_ARG, "kernel index %d out of range", index);
  const msa::KernelEntry& k = ks[index];
  if (name && name_len > 0) {
    std::strncpy(name, k.name, name_len - 1);
    name[name_len - 1] = '\0';
  }
  hipFuncAttributes a;
  hipError_t e = hipFuncGetAttributes(&a, k.fn);
  if (e != hipSuccess) return hip_fail(e, "hipFuncGetAttributes");
  if (k.dyn_lds > 65536) {
    e = hipFuncSetAttribute(k.fn, hipFuncAttributeMaxDynamicSharedMemorySize, k.dyn_lds);
    if (e != hipSuccess) return hip_fail(e, "hipFuncSetAttribute");
  }
  int nb = 0;
  e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, k.fn, k.block, k.dyn_lds);
  if (e != hipSuccess) return hip_fail(e, "hipOccupancyMaxActiveBlocksPerMultiprocessor");
  if (regs) *regs = a.numRegs;
  if (lds_bytes) *lds_bytes = (int32_t)a.sharedSizeBytes + k.dyn_lds;
  if (scratch_bytes) *scratch_bytes = (int32_t)a.localSizeBytes;
  if (wg_per_cu) *wg_per_cu = nb;
  return MSA_OK;
}

}  // extern "C"
