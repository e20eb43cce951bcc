/*
 * msa.h -- C ABI of the MiniMax Sparse Attention (MSA) training hot path for
 * AMD Instinct MI355X (gfx950).
 *
 * The method, as the pages describe it:
 *   - a proxy head scores query-key pairs and the scores are max-pooled into
 *     128-token KV blocks; KV is selected per query block in those blocks
 *     (ai-minor "Dramatically Speeding Up Million-Token Training!", News
 *     Overview and Terminology Explained; socker-news Flash-MSA summary, 要約);
 *   - the main attention is grouped-query attention (GQA) over the selected
 *     blocks only (same sections);
 *   - the backward passes of the proxy and of the main attention are fused
 *     (ai-minor, Why Does This Matter?; keelcrux "Flash-MSA: Ein Training mit
 *     einer Million Tokens", Le fait);
 *   - sequences are varlen-packed (socker-news summary, 要約);
 *   - the block pattern has a configurable window and dilation (keelcrux,
 *     Under the hood).
 * Where the pages give no formula, these readings are used: one proxy head per
 * KV group shared by the group's query heads; block score = max over the
 * (query block x KV block) tile of the raw dot product <qp, kp>; the diagonal
 * block and `local_window` blocks before it are always selected and `topk`
 * counts the diagonal; with a dilation delta > 1 the forced window blocks are
 * diag - delta, ..., diag - local_window * delta (those >= 0), candidates are
 * the blocks below diag - local_window * delta, and the other blocks inside
 * that span are never selected; exact score ties go to the lower block index; the
 * proxy gradient is that of lam * KL(T || Q) over the selected keys, with T the
 * group-mean main attention probabilities held constant and Q the proxy
 * softmax.
 *
 * Conventions for every entry point
 *   - Tokens-major packed layouts: q, o, dout [T, Hq, d]; k, v [T, Hkv, d];
 *     qp, kp [T, Hp, dp].  Gradients are fp32 in the same layouts.
 *     lse [Hq, T] and lse_p [Hp, T] are fp32 natural logarithms.  Hp, the
 *     number of proxy heads, is Hkv (one per KV group) or 1 (one proxy head
 *     shared by every group: its block choice serves every query head, and the
 *     proxy gradient's target is the mean main attention over all query heads);
 *     every per-proxy-head tensor below (block scores, block lists, lse_p) has
 *     Hp in place of Hkv.
 *   - cu_seqlens: int32 [batch + 1], cu_seqlens[0] = 0, non-decreasing,
 *     cu_seqlens[batch] = total_tokens.  Blocks start at each document start;
 *     selection never crosses a document.  Zero-length documents are allowed.
 *   - Block ids in q2k_idx / k2q_idx are global: document offset + local index.
 *   - Query head h uses KV group h / (Hq / Hkv).
 *   - All device pointers are caller-owned device memory, 16-byte aligned.
 *     The library allocates no device memory.  Its only state is a
 *     thread-local error message, a per-device record that the kernels' LDS
 *     limits were raised and of the device's compute-unit count (the
 *     persistent kernels launch one workgroup per compute unit), and (only
 *     after msa_profile_enable) a thread-local pool of timing events.
 *   - The workspace (msa_layout.workspace_bytes) holds a call's per-document
 *     tables, per-query intermediates of the backward and the work-queue
 *     counters of its persistent kernels, which each call clears on `stream`
 *     before use.  Calls that share one workspace must not overlap: issue
 *     them on one stream or order them.  Work is enqueued asynchronously on
 *     `stream` (a hipStream_t; NULL = default stream); the caller keeps every
 *     buffer alive until that work completes.  Outputs are overwritten.
 *   - Errors: every argument is checked on the host before anything is
 *     launched; a failure returns a non-zero msa_status and
 *     msa_last_error() describes it.  Nothing aborts and no exception crosses
 *     the ABI.  Launch failures return MSA_ERR_HIP.
 */
#ifndef MSA_H_
#define MSA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MSA_ABI_VERSION 4

typedef enum {
  MSA_OK = 0,
  MSA_ERR_INVALID_ARG = 1,   /* null pointer, bad size, bad cu_seqlens, misalignment */
  MSA_ERR_UNSUPPORTED = 2,   /* valid but not built: head/proxy dims, block sizes, dtype */
  MSA_ERR_HIP = 3,           /* a HIP runtime or launch error */
  MSA_ERR_WORKSPACE = 4      /* workspace too small */
} msa_status;

typedef enum { MSA_BF16 = 0, MSA_F32 = 1 } msa_dtype;

typedef struct {
  int32_t heads_q;           /* Hq, a multiple of heads_kv */
  int32_t heads_kv;          /* Hkv */
  int32_t head_dim;          /* d:  128 (bf16) or 64 (bf16, fp32) */
  int32_t proxy_dim;         /* dp: 64 with d = 128, 32 with d = 64 */
  int32_t kv_block;          /* must be 128 */
  int32_t q_block;           /* 64 or 128 */
  int32_t topk;              /* selected blocks per query block, counting the diagonal; >= 1 */
  int32_t local_window;      /* forced blocks before the diagonal; >= 0 */
  float softmax_scale;       /* 0 -> 1/sqrt(d) */
  float proxy_scale;         /* 0 -> 1/sqrt(dp) */
  float proxy_loss_weight;   /* lam; 0 is a valid weight */
  int32_t dtype;             /* msa_dtype of q, k, v, qp, kp, o, dout */
  int32_t dilation;          /* stride of the forced window blocks; 0 or 1 = contiguous */
  int32_t proxy_heads;       /* Hp: 0 or heads_kv = one proxy head per KV group; 1 = one
                                proxy head shared by every group */
} msa_config;

typedef struct {
  const int32_t* cu_seqlens;       /* device copy, [batch + 1] */
  const int32_t* cu_seqlens_host;  /* host copy,   [batch + 1] (read during the call only) */
  int32_t batch;                   /* number of documents, >= 1 */
  int32_t total_tokens;            /* T */
} msa_varlen;

typedef struct {
  int64_t total_qblocks;     /* NQB = sum over documents of ceil(L / q_block) */
  int64_t total_kvblocks;    /* NKB = sum over documents of ceil(L / 128) */
  int64_t score_elems;       /* per proxy head: sum over documents of nq * nk */
  int64_t sel_stride;        /* topk + local_window */
  int64_t k2q_capacity;      /* per proxy head: NQB * sel_stride */
  int64_t scored_pairs;      /* per proxy head: (query, key) pairs the scoring contracts */
  int64_t max_qblocks_doc;   /* largest per-document query-block count */
  int64_t workspace_bytes;   /* one workspace serves every entry point */
  int64_t proxy_heads;       /* Hp, the leading size of every per-proxy-head tensor */
} msa_layout;

int32_t msa_abi_version(void);
const char* msa_status_string(msa_status s);
/* Message for the last failing call on this thread ("" if none). */
const char* msa_last_error(void);

/*
 * Sizes of every buffer for a configuration and packing.  Host only: touches
 * no device memory and needs no GPU.
 */
msa_status msa_get_layout(const msa_config* cfg, const msa_varlen* vl, msa_layout* out);

/*
 * Proxy block scores (ai-minor, News Overview: the maximum of the proxy
 * score over 128-token KV blocks).
 * block_scores: fp32 [Hp, score_elems]; document b's nq x nk rectangle is
 * row-major at a per-document offset.  Only the candidate entries of query
 * blocks that have candidates are written (J < diag - local_window * delta,
 * where diag = floor(I * q_block / 128) and delta the dilation, and only when
 * there are more than topk - 1 such J); the rest are left untouched and never
 * read.
 */
msa_status msa_proxy_scores(const msa_config* cfg, const msa_varlen* vl, const void* qp,
                            const void* kp, float* block_scores, void* workspace,
                            size_t workspace_bytes, void* stream);

/*
 * Top-k block selection per (proxy head, query block) and the KV-major
 * inverted index (ai-minor, News Overview / Terminology: KV chosen in block
 * units).
 * q2k_idx int32 [Hp, NQB, sel_stride]: ascending global KV block ids, -1 padded.
 * q2k_cnt int32 [Hp, NQB]: min(topk - 1, candidates) + forced blocks; with
 *         delta = 1 this is min(topk + local_window, diag + 1).
 * k2q_ptr int32 [Hp, NKB + 1]: per-proxy-head CSR offsets into row p of k2q_idx.
 * k2q_idx int32 [Hp, k2q_capacity]: ascending query-block ids per KV block;
 *         the unused tail of each row is -1.
 */
msa_status msa_select_blocks(const msa_config* cfg, const msa_varlen* vl, const float* block_scores,
                             int32_t* q2k_idx, int32_t* q2k_cnt, int32_t* k2q_ptr,
                             int32_t* k2q_idx, void* workspace, size_t workspace_bytes,
                             void* stream);

/*
 * msa_select_blocks without a workspace, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc).  Same arguments as msa_select_blocks minus the
 * workspace, same outputs bit for bit, same kernels.  The per-document tables
 * and inverted-index counters live in a static device array of
 * msa_select_blocks_noalloc_max_bytes() bytes (16 MiB) that the library holds
 * on every GPU it runs on until the process ends; this call allocates
 * nothing.  Needed: the per-document tables (about 0.1 byte per token) and the
 * inverted-index counts, 4 bytes per (proxy head, KV block, 256 query blocks
 * of the longest document).  That is 2.5 MiB for 1M tokens packed as 14
 * documents of at most 207k tokens, about 2 bytes per token for documents of
 * 256k tokens (some 7M tokens fit), and 8.3 MiB for one 1M-token document (the
 * longest single document that fits is about 1.45M tokens, 8 proxy heads); a
 * larger problem returns MSA_ERR_WORKSPACE before anything is launched.  Every
 * call on a GPU shares that GPU's array: calls that overlap on one GPU (on
 * different streams, or from different threads) race and must be ordered by
 * the caller.  Every count is written by the call itself (no memset), so
 * nothing has to be zeroed between calls.
 */
msa_status msa_select_blocks_noalloc(const msa_config* cfg, const msa_varlen* vl,
                                     const float* block_scores, int32_t* q2k_idx, int32_t* q2k_cnt,
                                     int32_t* k2q_ptr, int32_t* k2q_idx, void* stream);
int64_t msa_select_blocks_noalloc_max_bytes(void);

/*
 * Sparse GQA forward over the selected blocks (socker-news summary 要約;
 * ai-minor News Overview).  o has the input dtype; lse [Hq, T] and
 * lse_p [Hp, T] (proxy softmax over the same selected keys) are fp32.
 */
msa_status msa_fwd(const msa_config* cfg, const msa_varlen* vl, const void* q, const void* k,
                   const void* v, const void* qp, const void* kp, const int32_t* q2k_idx,
                   const int32_t* q2k_cnt, void* o, float* lse, float* lse_p, void* workspace,
                   size_t workspace_bytes, void* stream);

/*
 * Fused backward of the main attention and the proxy head (ai-minor, Why
 * Does This Matter?: fused backward).  Takes the forward's o, lse, lse_p and
 * block lists plus the upstream gradient dout; writes fp32 dq [T, Hq, d],
 * dk, dv [T, Hkv, d], dqp, dkp [T, Hp, dp].
 */
msa_status msa_bwd(const msa_config* cfg, const msa_varlen* vl, const void* q, const void* k,
                   const void* v, const void* qp, const void* kp, const void* o, const float* lse,
                   const float* lse_p, const void* dout, const int32_t* q2k_idx,
                   const int32_t* q2k_cnt, const int32_t* k2q_ptr, const int32_t* k2q_idx,
                   float* dq, float* dk, float* dv, float* dqp, float* dkp, void* workspace,
                   size_t workspace_bytes, void* stream);

/*
 * Resource usage of the library's kernels, for the occupancy report.  Needs a
 * GPU.  index in [0, msa_kernel_count()).  Writes the kernel name (at most
 * name_len bytes, NUL-terminated), VGPRs/lane as reported by the runtime,
 * static + dynamic LDS bytes, private (scratch) bytes per lane and the
 * maximum resident workgroups per compute unit at the launch size used.
 */
int32_t msa_kernel_count(void);
msa_status msa_kernel_info(int32_t index, char* name, size_t name_len, int32_t* regs,
                           int32_t* lds_bytes, int32_t* scratch_bytes, int32_t* wg_per_cu);

/*
 * Per-kernel timing, for roofline figures.  While enabled (per calling
 * thread), every kernel launch the library makes is bracketed by two
 * hipEvents recorded on the launch stream; the events come from a pool the
 * library creates on first use and keeps until the process ends.
 * msa_profile_collect waits for the recorded events, sums the elapsed time
 * per kernel name, clears the record and returns the number of names;
 * msa_profile_entry(i, ...) reads name i, its total milliseconds and its
 * launch count.  Needs a GPU.
 */
msa_status msa_profile_enable(int32_t on);
int32_t msa_profile_collect(void);
msa_status msa_profile_entry(int32_t index, char* name, size_t name_len, double* total_ms,
                             int64_t* launches);

#ifdef __cplusplus
}
#endif
#endif /* MSA_H_ */
