"""CPU oracle for the MiniMax Sparse Attention (MSA) training hot path.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import it.  The product path (the HIP
library and its Python binding) never imports, calls or links it, and this
module imports nothing from the product package.

Plain, slow, obviously correct numpy in float64.  The inputs are the stored
(bf16- or fp32-valued) tensors upcast to float64.  Every step follows the
pages' description in the order they give it; where the pages are silent the
plainest reading is taken (each one is named below as "Reading").

Pages cited (by title and section):
  [HN-ja]  "Flash-MSA：スパースアテンション kernels を用いて..." (socker-news
           translation of the Hacker News item), section 要約 (summary).
  [AIM]    "Dramatically Speeding Up Million-Token Training! The World's First
           Open-Source 'Flash-MSA' ..." (ai-minor), sections "News Overview",
           "Why Does This Matter?", "Terminology Explained".
  [KC]     "Flash-MSA: Ein Training mit einer Million Tokens ohne hohe
           Rechenkosten" (keelcrux), sections "Le fait", "Under the hood".

What the pages fix:
  * KV is selected in 128-token blocks by the maximum of a proxy score
    (max-pooling) [AIM News Overview; HN-ja 要約; AIM Terminology "MSA"].
  * A proxy head picks the KV subset [HN-ja 要約].
  * The main attention is GQA [HN-ja 要約; AIM News Overview].
  * Everything except the proxy forward is linear or sparse in context
    length [AIM Why Does This Matter?]; so the proxy backward is sparse.
  * The proxy and main backward passes are fused [AIM Why Does This Matter?;
    KC Le fait].
  * Sequences are varlen-packed [HN-ja 要約, "varlen"].

Readings (the pages give no formulas):
  R1  One proxy head per KV group (Hp = Hkv); its block choice is shared by the
      G query heads of the group.  Query head h uses group h // G.
  R1s The shared-proxy variant (Hp = 1, proxy_heads = 1): one proxy head whose
      block choice every query head uses; in R8, T is then the mean of the main
      probabilities over all Hq heads (the heads that share the choice).
  R2  Proxy block score S[g, I, J] = max over valid query rows t of block I and
      keys u of block J of the raw dot product <qp[t, g], kp[u, g]> (unscaled:
      a positive scale does not change a ranking).
  R3  Candidates of query block I are the KV blocks J < diag(I) - w, where
      diag(I) = floor(I * Bq / Bk) and w is the forced local window.  The
      diagonal block and the w blocks before it are always selected.  Top-k
      counts the diagonal: k - 1 candidates are added.  Total selected
      K = min(k + w, diag(I) + 1); when K = diag(I) + 1 every block 0..diag is
      taken and no score is needed.
  R3d Dilation delta >= 1 [KC Under the hood names a configurable window and
      dilation, nothing more]: the forced blocks are diag, diag - delta, ...,
      diag - w*delta (those >= 0); the candidate pool is J < diag - w*delta
      (the window's span); blocks inside the span that are not on its stride
      are neither forced nor candidates.  When the pool holds at most k - 1
      blocks all of it is taken and nothing is scored.  delta = 1 is R3.
  R4  Ranking key: score descending, then block index ascending (lower index
      wins an exact tie).  Lists are emitted ascending, padded with -1.
  R5  Attention set A_i = {u : block(u) selected for block(i), u <= i}
      (causal, diagonal included, never empty).  Blocks never span documents.
  R6  Forward: z = s<q_h[i], k_g[u]>, LSE = logsumexp_u z, P = exp(z - LSE),
      O = sum_u P v_g[u].  Proxy: y = s_p<qp_g[i], kp_g[u]> over the same A_i,
      LSE_p = logsumexp_u y.  s = 1/sqrt(d), s_p = 1/sqrt(dp) by default.
  R7  Main backward (upstream dO): the standard softmax-attention gradients.
  R8  Proxy gradient ("training signal"): a sparse distillation KL over the
      selected keys.  T_iu = (1/G) sum_{h in g} P^(h)_iu (held constant),
      Q_iu = exp(y - LSE_p), dY = lam (Q - T), dqp = s_p dY kp,
      dkp = s_p dY^T qp.  Loss: L_aux = lam sum T (ln T - ln Q).
"""
from __future__ import annotations

import math
from dataclasses import dataclass
from typing import Dict, Iterable, List, Optional, Tuple

import numpy as np


# --------------------------------------------------------------------------
# configuration and per-document block grid
# --------------------------------------------------------------------------

@dataclass(frozen=True)
class Config:
    heads_q: int
    heads_kv: int
    head_dim: int
    proxy_dim: int
    q_block: int
    topk: int
    local_window: int = 0
    kv_block: int = 128
    softmax_scale: Optional[float] = None
    proxy_scale: Optional[float] = None
    proxy_loss_weight: float = 1.0
    dilation: int = 1
    proxy_heads: int = 0      # 0: one per KV group (R1); 1: one shared proxy head (R1s)

    @property
    def Hp(self) -> int:
        return 1 if self.proxy_heads == 1 else self.heads_kv

    def proxy_of(self, g: int) -> int:
        """Proxy head whose choice KV group g uses."""
        return 0 if self.proxy_heads == 1 else g

    def groups_of(self, p: int) -> List[int]:
        """KV groups that use proxy head p."""
        return list(range(self.heads_kv)) if self.proxy_heads == 1 else [p]

    @property
    def G(self) -> int:
        return self.heads_q // self.heads_kv

    @property
    def scale(self) -> float:
        return self.softmax_scale if self.softmax_scale else 1.0 / math.sqrt(self.head_dim)

    @property
    def pscale(self) -> float:
        return self.proxy_scale if self.proxy_scale else 1.0 / math.sqrt(self.proxy_dim)

    @property
    def sel_stride(self) -> int:
        return self.topk + self.local_window


@dataclass(frozen=True)
class Doc:
    start: int      # first token (global)
    length: int
    nq: int         # query blocks
    nk: int         # KV blocks
    qb0: int        # global id of its first query block
    kb0: int        # global id of its first KV block
    s0: int         # offset of its nq x nk score rectangle


def doc_grid(cu_seqlens, cfg: Config) -> List[Doc]:
    """Per-document block grids; blocks start at each document start and the
    last block of a document may be partial [HN-ja 要約, varlen packing]."""
    cu = [int(x) for x in cu_seqlens]
    docs, qb, kb, s = [], 0, 0, 0
    for b in range(len(cu) - 1):
        L = cu[b + 1] - cu[b]
        assert L >= 0, "cu_seqlens must be non-decreasing"
        nq = -(-L // cfg.q_block)
        nk = -(-L // cfg.kv_block)
        docs.append(Doc(cu[b], L, nq, nk, qb, kb, s))
        qb, kb, s = qb + nq, kb + nk, s + nq * nk
    return docs


def totals(docs: List[Doc]) -> Tuple[int, int, int]:
    return (sum(d.nq for d in docs), sum(d.nk for d in docs), sum(d.nq * d.nk for d in docs))


def diag_block(I: int, cfg: Config) -> int:
    """KV block holding the first query token of query block I (R3)."""
    return (I * cfg.q_block) // cfg.kv_block


def forced_blocks(I: int, cfg: Config) -> List[int]:
    """The diagonal block and the window's blocks before it, ascending (R3, R3d)."""
    dg = diag_block(I, cfg)
    return sorted(dg - i * cfg.dilation for i in range(cfg.local_window + 1) if dg - i * cfg.dilation >= 0)


def pool_size(I: int, cfg: Config) -> int:
    """Blocks before the window's span: J < diag - w * delta (R3, R3d)."""
    return max(0, diag_block(I, cfg) - cfg.local_window * cfg.dilation)


def n_selected(I: int, cfg: Config) -> int:
    """K = min(k - 1, pool) + forced; with delta = 1 this is min(k + w, diag + 1) (R3)."""
    return min(cfg.topk - 1, pool_size(I, cfg)) + len(forced_blocks(I, cfg))


def candidate_count(I: int, cfg: Config) -> int:
    """Number of scored candidate blocks of query block I (0 when the whole
    pool is taken, which needs no score)."""
    n = pool_size(I, cfg)
    return n if n > cfg.topk - 1 else 0


def _qrows(doc: Doc, I: int, cfg: Config) -> np.ndarray:
    lo = I * cfg.q_block
    hi = min(lo + cfg.q_block, doc.length)
    return np.arange(doc.start + lo, doc.start + hi)


def _krows(doc: Doc, J: int, cfg: Config) -> np.ndarray:
    lo = J * cfg.kv_block
    hi = min(lo + cfg.kv_block, doc.length)
    return np.arange(doc.start + lo, doc.start + hi)


# --------------------------------------------------------------------------
# step 1: proxy block scores (max-pooled), R2 / R3
# --------------------------------------------------------------------------

def proxy_row_scores(qp, kp, doc: Doc, g: int, I: int, cfg: Config) -> np.ndarray:
    """Scores of the candidate blocks J = 0..ncand-1 of query block I.

    Max-pooling of the proxy score over each (query block x 128-token KV block)
    tile [AIM News Overview: 'maximum value of the proxy score', 128-token
    blocks].  Candidates lie strictly before the diagonal, so no causal mask is
    needed; only the valid query rows of a partial last block are pooled."""
    ncand = candidate_count(I, cfg)
    if ncand == 0:
        return np.zeros(0)
    rows = _qrows(doc, I, cfg)
    keys = np.arange(doc.start, doc.start + ncand * cfg.kv_block)
    a = qp[rows, g, :].astype(np.float64)
    b = kp[keys, g, :].astype(np.float64)
    dots = a @ b.T                                      # [rows, ncand*Bk]
    return dots.reshape(len(rows), ncand, cfg.kv_block).max(axis=(0, 2))


def proxy_block_scores(qp, kp, cu_seqlens, cfg: Config) -> np.ndarray:
    """Block-score tensor [Hp, score_elems] (row-major nq x nk rectangle per
    document); entries that are not candidates are -inf."""
    docs = doc_grid(cu_seqlens, cfg)
    _, _, ns = totals(docs)
    S = np.full((cfg.Hp, ns), -np.inf)
    for g in range(cfg.Hp):
        for doc in docs:
            for I in range(doc.nq):
                r = proxy_row_scores(qp, kp, doc, g, I, cfg)
                S[g, doc.s0 + I * doc.nk: doc.s0 + I * doc.nk + len(r)] = r
    return S


# --------------------------------------------------------------------------
# step 2: block selection, R3 / R4
# --------------------------------------------------------------------------

def select_row(cand_scores: np.ndarray, I: int, cfg: Config) -> List[int]:
    """Local block indices selected for query block I, ascending.

    Forced: the diagonal block and the window's blocks (R3, R3d).  Then the
    k - 1 candidates of the pool with the highest score, an exact tie going to
    the lower block index.  When the pool holds at most k - 1 blocks, all of
    it (with delta = 1: every block up to the diagonal)."""
    forced = forced_blocks(I, cfg)
    n = pool_size(I, cfg)
    if n <= cfg.topk - 1:
        return list(range(n)) + forced
    cands = list(range(len(cand_scores)))
    assert len(cands) == n
    ranked = sorted(cands, key=lambda J: (-float(cand_scores[J]), J))
    picked = ranked[: cfg.topk - 1]
    return sorted(picked + forced)


def select_blocks(scores: np.ndarray, cu_seqlens, cfg: Config):
    """q2k_idx [Hp, NQB, k + w] (global KV block ids, ascending, -1 padded) and
    q2k_cnt [Hp, NQB]."""
    docs = doc_grid(cu_seqlens, cfg)
    nqb, _, _ = totals(docs)
    idx = np.full((cfg.Hp, nqb, cfg.sel_stride), -1, dtype=np.int32)
    cnt = np.zeros((cfg.Hp, nqb), dtype=np.int32)
    for g in range(cfg.Hp):
        for doc in docs:
            for I in range(doc.nq):
                nc = candidate_count(I, cfg)
                row = scores[g, doc.s0 + I * doc.nk: doc.s0 + I * doc.nk + nc]
                sel = select_row(row, I, cfg)
                idx[g, doc.qb0 + I, :len(sel)] = np.asarray(sel) + doc.kb0
                cnt[g, doc.qb0 + I] = len(sel)
    return idx, cnt


# --------------------------------------------------------------------------
# step 3: inverted (KV-major) index
# --------------------------------------------------------------------------

def invert_index(q2k_idx: np.ndarray, q2k_cnt: np.ndarray, nkb: int):
    """For each (g, KV block), the ascending list of query blocks that selected
    it, as CSR: k2q_ptr [Hp, NKB + 1], k2q_idx [Hp, NQB * (k + w)] (row g holds
    group g's lists, unused tail -1)."""
    Hp, nqb, stride = q2k_idx.shape
    ptr = np.zeros((Hp, nkb + 1), dtype=np.int32)
    out = np.full((Hp, nqb * stride), -1, dtype=np.int32)
    for g in range(Hp):
        lists: List[List[int]] = [[] for _ in range(nkb)]
        for QB in range(nqb):
            for s in range(q2k_cnt[g, QB]):
                lists[q2k_idx[g, QB, s]].append(QB)
        pos = 0
        for KB in range(nkb):
            ptr[g, KB] = pos
            for QB in sorted(lists[KB]):
                out[g, pos] = QB
                pos += 1
        ptr[g, nkb] = pos
    return ptr, out


# --------------------------------------------------------------------------
# steps 4-6: attention over the selected keys of one query block
# --------------------------------------------------------------------------

def _block_keys(doc: Doc, sel_global: Iterable[int], cfg: Config) -> np.ndarray:
    keys = [_krows(doc, int(KB) - doc.kb0, cfg) for KB in sel_global]
    return np.concatenate(keys) if keys else np.zeros(0, dtype=np.int64)


def _softmax_rows(z: np.ndarray):
    """Row logsumexp and probabilities; -inf entries are masked keys."""
    m = z.max(axis=1, keepdims=True)
    e = np.exp(z - m)
    ssum = e.sum(axis=1, keepdims=True)
    lse = (m + np.log(ssum))[:, 0]
    return lse, e / ssum


def qblock_forward(q, k, v, qp, kp, doc: Doc, g: int, I: int, sel_global, cfg: Config):
    """Forward quantities of query block I for the G heads of group g (R5, R6).

    Returns rows, keys, and per head P, O, LSE, plus the proxy y, Q, LSE_p."""
    rows = _qrows(doc, I, cfg)
    keys = _block_keys(doc, sel_global, cfg)
    causal = keys[None, :] <= rows[:, None]                     # u <= i
    out = {"rows": rows, "keys": keys, "mask": causal, "P": [], "O": [], "LSE": []}
    Kg = k[keys, g, :].astype(np.float64)
    Vg = v[keys, g, :].astype(np.float64)
    for h in range(g * cfg.G, (g + 1) * cfg.G):
        Qh = q[rows, h, :].astype(np.float64)
        z = np.where(causal, cfg.scale * (Qh @ Kg.T), -np.inf)
        lse, P = _softmax_rows(z)
        out["P"].append(P)
        out["O"].append(P @ Vg)
        out["LSE"].append(lse)
    Qp = qp[rows, cfg.proxy_of(g), :].astype(np.float64)
    Kp = kp[keys, cfg.proxy_of(g), :].astype(np.float64)
    y = np.where(causal, cfg.pscale * (Qp @ Kp.T), -np.inf)
    lse_p, Qprob = _softmax_rows(y)
    out.update(y=y, Q=Qprob, LSE_p=lse_p)
    return out


def qblock_backward(fw, q, k, v, qp, kp, dO, g: int, cfg: Config, O_for_D=None):
    """Backward of one query block of group g, given its forward quantities.

    Main (R7): D = <dO, O>, dP = dO v^T, dS = P (dP - D), dQ = s dS k,
    dK = s dS^T q, dV = P^T dO (summed over the group's heads).
    Proxy (R8): T = mean over the group's heads of P; dY = lam (Q - T);
    dqp = s_p dY kp; dkp = s_p dY^T qp (the per-group reading R1; with a
    shared proxy head the layer driver forms T over all heads instead).  Fused with the main backward in the
    sense of the pages [AIM Why Does This Matter?]: both use the same P."""
    rows, keys = fw["rows"], fw["keys"]
    Kg = k[keys, g, :].astype(np.float64)
    Vg = v[keys, g, :].astype(np.float64)
    res = {"dQ": [], "dK": np.zeros((len(keys), cfg.head_dim)),
           "dV": np.zeros((len(keys), cfg.head_dim))}
    for j, h in enumerate(range(g * cfg.G, (g + 1) * cfg.G)):
        P = fw["P"][j]
        Qh = q[rows, h, :].astype(np.float64)
        dOh = dO[rows, h, :].astype(np.float64)
        Oh = fw["O"][j] if O_for_D is None else O_for_D[j]
        D = (dOh * Oh).sum(axis=1, keepdims=True)
        dP = dOh @ Vg.T
        dS = P * (dP - D)
        res["dQ"].append(cfg.scale * (dS @ Kg))
        res["dK"] += cfg.scale * (dS.T @ Qh)
        res["dV"] += P.T @ dOh
    res.update(proxy_backward([fw], qp, kp, cfg.proxy_of(g), cfg))
    return res


def proxy_backward(fws, qp, kp, p: int, cfg: Config):
    """Proxy gradient of proxy head p for one query block (R8): T = mean of the
    main probabilities over every head that uses p's choice (the forward
    quantities of those heads' groups are in ``fws``, sharing rows and keys);
    dY = lam (Q - T); dqp = s_p dY kp; dkp = s_p dY^T qp."""
    rows, keys = fws[0]["rows"], fws[0]["keys"]
    P = [Ph for fw in fws for Ph in fw["P"]]
    T = sum(P) / len(P)
    dY = cfg.proxy_loss_weight * (fws[0]["Q"] - T)
    Qp = qp[rows, p, :].astype(np.float64)
    Kp = kp[keys, p, :].astype(np.float64)
    return {"dqp": cfg.pscale * (dY @ Kp), "dkp": cfg.pscale * (dY.T @ Qp), "T": T}


# --------------------------------------------------------------------------
# whole-layer drivers
# --------------------------------------------------------------------------

def _sel_of(q2k_idx, q2k_cnt, g, QB):
    return [int(x) for x in q2k_idx[g, QB, : q2k_cnt[g, QB]]]


def forward(q, k, v, qp, kp, cu_seqlens, q2k_idx, q2k_cnt, cfg: Config):
    """O [T, Hq, d], LSE [Hq, T], LSE_p [Hp, T] (natural log)."""
    T = q.shape[0]
    O = np.zeros((T, cfg.heads_q, cfg.head_dim))
    LSE = np.zeros((cfg.heads_q, T))
    LSEp = np.zeros((cfg.Hp, T))
    for doc in doc_grid(cu_seqlens, cfg):
        for g in range(cfg.heads_kv):
            for I in range(doc.nq):
                fw = qblock_forward(q, k, v, qp, kp, doc, g, I,
                                    _sel_of(q2k_idx, q2k_cnt, cfg.proxy_of(g), doc.qb0 + I), cfg)
                for j, h in enumerate(range(g * cfg.G, (g + 1) * cfg.G)):
                    O[fw["rows"], h, :] = fw["O"][j]
                    LSE[h, fw["rows"]] = fw["LSE"][j]
                LSEp[cfg.proxy_of(g), fw["rows"]] = fw["LSE_p"]
    return O, LSE, LSEp


def backward(q, k, v, qp, kp, dO, cu_seqlens, q2k_idx, q2k_cnt, cfg: Config, O_for_D=None):
    """dq, dk, dv, dqp, dkp (float64).  ``O_for_D`` optionally supplies the O
    used in D = <dO, O> (default: the oracle's own forward)."""
    T = q.shape[0]
    dq = np.zeros((T, cfg.heads_q, cfg.head_dim))
    dk = np.zeros((T, cfg.heads_kv, cfg.head_dim))
    dv = np.zeros((T, cfg.heads_kv, cfg.head_dim))
    dqp = np.zeros((T, cfg.Hp, cfg.proxy_dim))
    dkp = np.zeros((T, cfg.Hp, cfg.proxy_dim))
    for doc in doc_grid(cu_seqlens, cfg):
        for I in range(doc.nq):
            fws = {}
            for g in range(cfg.heads_kv):
                fw = qblock_forward(q, k, v, qp, kp, doc, g, I,
                                    _sel_of(q2k_idx, q2k_cnt, cfg.proxy_of(g), doc.qb0 + I), cfg)
                fws[g] = fw
                od = None
                if O_for_D is not None:
                    od = [O_for_D[fw["rows"], h, :].astype(np.float64)
                          for h in range(g * cfg.G, (g + 1) * cfg.G)]
                bw = qblock_backward(fw, q, k, v, qp, kp, dO, g, cfg, od)
                rows, keys = fw["rows"], fw["keys"]
                for j, h in enumerate(range(g * cfg.G, (g + 1) * cfg.G)):
                    dq[rows, h, :] = bw["dQ"][j]
                dk[keys, g, :] += bw["dK"]          # keys are distinct within a block
                dv[keys, g, :] += bw["dV"]
            for p in range(cfg.Hp):
                pb = proxy_backward([fws[g] for g in cfg.groups_of(p)], qp, kp, p, cfg)
                rows, keys = fws[cfg.groups_of(p)[0]]["rows"], fws[cfg.groups_of(p)[0]]["keys"]
                dqp[rows, p, :] = pb["dqp"]
                dkp[keys, p, :] += pb["dkp"]
    return dq, dk, dv, dqp, dkp


def losses(q, k, v, qp, kp, dO, cu_seqlens, q2k_idx, q2k_cnt, cfg: Config, T_fixed=None):
    """Scalar objectives whose gradients the backward returns (for finite
    differences).  L_main = sum <dO, O>.  L_aux = lam sum_{g,i} sum_u
    T (ln T - ln Q) with T held fixed (0 ln 0 = 0), one term per proxy head.
    ``T_fixed`` maps (doc index, proxy head, I) to the T matrix to hold; by
    default T comes from the given q, k."""
    Lm, La = 0.0, 0.0
    for bi, doc in enumerate(doc_grid(cu_seqlens, cfg)):
        for I in range(doc.nq):
            fws = {}
            for g in range(cfg.heads_kv):
                fw = qblock_forward(q, k, v, qp, kp, doc, g, I,
                                    _sel_of(q2k_idx, q2k_cnt, cfg.proxy_of(g), doc.qb0 + I), cfg)
                fws[g] = fw
                for j, h in enumerate(range(g * cfg.G, (g + 1) * cfg.G)):
                    Lm += float((dO[fw["rows"], h, :].astype(np.float64) * fw["O"][j]).sum())
            for p in range(cfg.Hp):
                P = [Ph for g in cfg.groups_of(p) for Ph in fws[g]["P"]]
                T = sum(P) / len(P) if T_fixed is None else T_fixed[(bi, p, I)]
                fw = fws[cfg.groups_of(p)[0]]
                lnQ = np.where(fw["mask"], fw["y"] - fw["LSE_p"][:, None], 0.0)
                lnT = np.log(np.where(T > 0, T, 1.0))
                La += cfg.proxy_loss_weight * float((T * (lnT - lnQ)).sum())
    return Lm, La


def group_mean_probs(q, k, v, qp, kp, cu_seqlens, q2k_idx, q2k_cnt, cfg: Config):
    """T for every (doc index, proxy head, I), for holding it fixed in L_aux."""
    out = {}
    for bi, doc in enumerate(doc_grid(cu_seqlens, cfg)):
        for I in range(doc.nq):
            for p in range(cfg.Hp):
                P = []
                for g in cfg.groups_of(p):
                    fw = qblock_forward(q, k, v, qp, kp, doc, g, I,
                                        _sel_of(q2k_idx, q2k_cnt, p, doc.qb0 + I), cfg)
                    P += fw["P"]
                out[(bi, p, I)] = sum(P) / len(P)
    return out


def run_all(q, k, v, qp, kp, dO, cu_seqlens, cfg: Config) -> Dict[str, np.ndarray]:
    """Every step of the path, in order."""
    docs = doc_grid(cu_seqlens, cfg)
    _, nkb, _ = totals(docs)
    S = proxy_block_scores(qp, kp, cu_seqlens, cfg)
    q2k_idx, q2k_cnt = select_blocks(S, cu_seqlens, cfg)
    k2q_ptr, k2q_idx = invert_index(q2k_idx, q2k_cnt, nkb)
    O, LSE, LSEp = forward(q, k, v, qp, kp, cu_seqlens, q2k_idx, q2k_cnt, cfg)
    dq, dk, dv, dqp, dkp = backward(q, k, v, qp, kp, dO, cu_seqlens, q2k_idx, q2k_cnt, cfg)
    return dict(scores=S, q2k_idx=q2k_idx, q2k_cnt=q2k_cnt, k2q_ptr=k2q_ptr, k2q_idx=k2q_idx,
                O=O, LSE=LSE, LSEp=LSEp, dq=dq, dk=dk, dv=dv, dqp=dqp, dkp=dkp)


# --------------------------------------------------------------------------
# sampled evaluation for large workloads
# --------------------------------------------------------------------------

def _doc_of_qb(docs: List[Doc], QB: int) -> Doc:
    for d in docs:
        if d.qb0 <= QB < d.qb0 + d.nq:
            return d
    raise IndexError(QB)


def _doc_of_kb(docs: List[Doc], KB: int) -> Doc:
    for d in docs:
        if d.kb0 <= KB < d.kb0 + d.nk:
            return d
    raise IndexError(KB)


def sampled_query_side(q, k, v, qp, kp, dO, cu_seqlens, q2k_idx, q2k_cnt, cfg: Config,
                       samples: List[Tuple[int, int]], O_for_D=None):
    """For sampled (g, global query block) pairs: O, LSE, LSE_p, dQ and dqp of
    that block's rows, computed from the definition.  dqp is the gradient of
    proxy head p = cfg.proxy_of(g) (returned as "p"); with a shared proxy head
    (R1s) it takes T over every group's heads, as the layer backward does."""
    docs = doc_grid(cu_seqlens, cfg)
    out = []
    for g, QB in samples:
        doc = _doc_of_qb(docs, QB)
        I = QB - doc.qb0
        p = cfg.proxy_of(g)
        sel = _sel_of(q2k_idx, q2k_cnt, p, QB)
        fw = qblock_forward(q, k, v, qp, kp, doc, g, I, sel, cfg)
        od = None
        if O_for_D is not None:
            od = [O_for_D[fw["rows"], h, :].astype(np.float64)
                  for h in range(g * cfg.G, (g + 1) * cfg.G)]
        bw = qblock_backward(fw, q, k, v, qp, kp, dO, g, cfg, od)
        dqp = bw["dqp"]
        if cfg.proxy_heads == 1:
            fws = [fw if gg == g else qblock_forward(q, k, v, qp, kp, doc, gg, I, sel, cfg)
                   for gg in cfg.groups_of(p)]
            dqp = proxy_backward(fws, qp, kp, p, cfg)["dqp"]
        out.append(dict(g=g, p=p, QB=QB, rows=fw["rows"], O=np.stack(fw["O"], 1),
                        LSE=np.stack(fw["LSE"], 0), LSE_p=fw["LSE_p"],
                        dQ=np.stack(bw["dQ"], 1), dqp=dqp))
    return out


def sampled_key_side(q, k, v, qp, kp, dO, cu_seqlens, q2k_idx, q2k_cnt, cfg: Config,
                     samples: List[Tuple[int, int]], O_for_D=None,
                     qblocks: Optional[Tuple[int, int]] = None):
    """For sampled (g, global KV block) pairs: dK, dV and dkp of that block's
    keys, summed over every query block whose selection holds it.  dK and dV
    are group g's; dkp is proxy head p = cfg.proxy_of(g)'s (returned as "p"),
    with T over every group's heads when the proxy head is shared (R1s).  With
    ``qblocks = (lo, hi)`` only the document's query blocks lo <= I < hi
    contribute (the full sums are the sums of such parts)."""
    docs = doc_grid(cu_seqlens, cfg)
    out = []
    for g, KB in samples:
        doc = _doc_of_kb(docs, KB)
        p = cfg.proxy_of(g)
        kr = _krows(doc, KB - doc.kb0, cfg)
        dK = np.zeros((len(kr), cfg.head_dim))
        dV = np.zeros((len(kr), cfg.head_dim))
        dKp = np.zeros((len(kr), cfg.proxy_dim))
        lo, hi = (0, doc.nq) if qblocks is None else (max(0, qblocks[0]), min(doc.nq, qblocks[1]))
        for I in range(lo, hi):
            sel = _sel_of(q2k_idx, q2k_cnt, p, doc.qb0 + I)
            if KB not in sel:
                continue
            fw = qblock_forward(q, k, v, qp, kp, doc, g, I, sel, cfg)
            od = None
            if O_for_D is not None:
                od = [O_for_D[fw["rows"], h, :].astype(np.float64)
                      for h in range(g * cfg.G, (g + 1) * cfg.G)]
            bw = qblock_backward(fw, q, k, v, qp, kp, dO, g, cfg, od)
            pos = np.searchsorted(fw["keys"], kr)
            dK += bw["dK"][pos]
            dV += bw["dV"][pos]
            if cfg.proxy_heads == 1:
                fws = [fw if gg == g else qblock_forward(q, k, v, qp, kp, doc, gg, I, sel, cfg)
                       for gg in cfg.groups_of(p)]
                dKp += proxy_backward(fws, qp, kp, p, cfg)["dkp"][pos]
            else:
                dKp += bw["dkp"][pos]
        out.append(dict(g=g, p=p, KB=KB, keys=kr, dK=dK, dV=dV, dkp=dKp))
    return out


# --------------------------------------------------------------------------
# independent dense routine (for the top-k >= all special case)
# --------------------------------------------------------------------------

def dense_causal_gqa(q, k, v, cu_seqlens, scale: float, G: int):
    """Textbook causal softmax attention per document, query head h reading KV
    head h // G.  Written without any block notion, for the dense pin."""
    T, Hq, d = q.shape
    O = np.zeros((T, Hq, d))
    LSE = np.zeros((Hq, T))
    cu = [int(x) for x in cu_seqlens]
    for b in range(len(cu) - 1):
        s, e = cu[b], cu[b + 1]
        if e == s:
            continue
        L = e - s
        mask = np.tril(np.ones((L, L), dtype=bool))
        for h in range(Hq):
            Qh = q[s:e, h, :].astype(np.float64)
            Kh = k[s:e, h // G, :].astype(np.float64)
            Vh = v[s:e, h // G, :].astype(np.float64)
            z = np.where(mask, scale * (Qh @ Kh.T), -np.inf)
            lse, P = _softmax_rows(z)
            O[s:e, h, :] = P @ Vh
            LSE[h, s:e] = lse
    return O, LSE
