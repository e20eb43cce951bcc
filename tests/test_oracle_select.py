"""Pins for the oracle's proxy scoring, block selection and inverted index.

The pages print no worked example; the pins are brute force written
independently of the oracle's code, designed ties, a hand-worked example
(tests/golden/select_example.json) and the invariants the pages fix: 128-token
KV blocks chosen by the maximum proxy score [ai-minor "Dramatically Speeding Up
Million-Token Training!", News Overview] and a forced diagonal block.
"""
import itertools
import json
import os

import numpy as np
import pytest

from oracle import msa_oracle as om

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _cfg(**kw):
    base = dict(heads_q=4, heads_kv=2, head_dim=8, proxy_dim=4, q_block=64, topk=3,
                local_window=0, kv_block=128)
    base.update(kw)
    return om.Config(**base)


def _half_ints(rng, shape):
    # multiples of 1/2 in [-2, 2]: fp64 dot products over few terms are exact
    return rng.integers(-4, 5, size=shape).astype(np.float64) / 2.0


def brute_scores(qp, kp, seqlens, cfg):
    """Explicit loops over every (query token, key token) pair of a document;
    tile (query block, KV block) maximum over pairs strictly before the
    query block's forced set."""
    out = {}
    start = 0
    for b, L in enumerate(seqlens):
        nq = -(-L // cfg.q_block)
        for g in range(cfg.heads_kv):
            for I in range(nq):
                first_tok = I * cfg.q_block
                # blocks before the window's span (w blocks, stride = dilation)
                forced_lo = first_tok // cfg.kv_block - cfg.local_window * cfg.dilation
                if max(0, forced_lo) <= cfg.topk - 1:
                    continue
                for J in range(forced_lo):
                    best = -np.inf
                    for t in range(first_tok, min(first_tok + cfg.q_block, L)):
                        for u in range(J * cfg.kv_block, (J + 1) * cfg.kv_block):
                            s = 0.0
                            for c in range(cfg.proxy_dim):
                                s += qp[start + t, g, c] * kp[start + u, g, c]
                            best = max(best, s)
                    out[(b, g, I, J)] = best
        start += L
    return out


@pytest.mark.parametrize("seqlens,q_block,w,dil", [((700,), 64, 0, 1), ((300, 0, 517), 128, 1, 1),
                                                   ((640,), 64, 1, 1), ((900,), 64, 1, 2)])
def test_scores_match_bruteforce(seqlens, q_block, w, dil):
    rng = np.random.default_rng(1)
    cfg = _cfg(q_block=q_block, local_window=w, topk=2, dilation=dil)
    T = sum(seqlens)
    qp = _half_ints(rng, (T, cfg.heads_kv, cfg.proxy_dim))
    kp = _half_ints(rng, (T, cfg.heads_kv, cfg.proxy_dim))
    cu = np.concatenate([[0], np.cumsum(seqlens)])
    S = om.proxy_block_scores(qp, kp, cu, cfg)
    bf = brute_scores(qp, kp, seqlens, cfg)
    docs = om.doc_grid(cu, cfg)
    seen = 0
    for (b, g, I, J), val in bf.items():
        d = docs[b]
        assert S[g, d.s0 + I * d.nk + J] == val
        seen += 1
    assert seen > 0
    # every other entry is a non-candidate
    assert np.isfinite(S).sum() == seen


def rank_select(scores, n_cand, n_pick):
    """J is picked iff fewer than n_pick candidates beat it, where J' beats J
    when its score is larger, or equal with a lower index."""
    picked = []
    for J in range(n_cand):
        beaten = sum(1 for Jp in range(n_cand)
                     if scores[Jp] > scores[J] or (scores[Jp] == scores[J] and Jp < J))
        if beaten < n_pick:
            picked.append(J)
    return picked


@pytest.mark.parametrize("topk,w,q_block", [(4, 0, 64), (3, 2, 128), (1, 0, 128), (5, 1, 64)])
def test_selection_rank_bruteforce(topk, w, q_block):
    rng = np.random.default_rng(7)
    cfg = _cfg(topk=topk, local_window=w, q_block=q_block)
    for trial in range(40):
        I = int(rng.integers(0, 40))
        dg = om.diag_block(I, cfg)
        nc = om.candidate_count(I, cfg)
        # coarse values force many exact ties
        sc = rng.integers(-3, 4, size=nc).astype(np.float64)
        sel = om.select_row(sc, I, cfg)
        if nc == 0:
            assert sel == list(range(dg + 1))
            continue
        expect = sorted(rank_select(sc, nc, topk - 1) + list(range(dg - w, dg + 1)))
        assert sel == expect


@pytest.mark.parametrize("topk,w,dil,q_block", [(3, 2, 3, 128), (4, 1, 2, 64), (2, 3, 2, 128), (1, 2, 4, 64)])
def test_selection_dilation_bruteforce(topk, w, dil, q_block):
    """Dilated window, written out independently: forced = diagonal minus
    multiples of the dilation (w of them, those >= 0); a block before the
    diagonal that is not forced is selectable only below the window's span
    diag - w * dilation; of those the k - 1 best by rank, or all of them when
    there are no more than k - 1."""
    rng = np.random.default_rng(17)
    cfg = _cfg(topk=topk, local_window=w, q_block=q_block, dilation=dil)
    for trial in range(60):
        I = int(rng.integers(0, 64))
        dg = I * q_block // 128
        forced = [J for J in range(dg + 1) if (dg - J) % dil == 0 and (dg - J) // dil <= w]
        below = [J for J in range(dg + 1) if J < dg - w * dil]
        gaps = [J for J in range(dg + 1) if J not in forced and J not in below]
        nc = om.candidate_count(I, cfg)
        sc = rng.integers(-3, 4, size=nc).astype(np.float64)
        sel = om.select_row(sc, I, cfg)
        if len(below) <= topk - 1:
            assert nc == 0 and sel == sorted(below + forced)
        else:
            assert nc == len(below)
            assert sel == sorted(rank_select(sc, nc, topk - 1) + forced)
        assert not set(gaps) & set(sel)
        assert om.n_selected(I, cfg) == len(sel)


def test_dilation_one_is_the_contiguous_window():
    for topk, w, q_block in [(3, 2, 128), (5, 0, 64), (2, 4, 64)]:
        a = _cfg(topk=topk, local_window=w, q_block=q_block)
        b = _cfg(topk=topk, local_window=w, q_block=q_block, dilation=1)
        for I in range(80):
            dg = om.diag_block(I, a)
            assert om.n_selected(I, b) == min(topk + w, dg + 1)
            assert om.candidate_count(I, b) == (0 if dg + 1 <= topk + w else dg - w)
            sc = np.arange(om.candidate_count(I, b), dtype=np.float64)[::-1].copy()
            assert om.select_row(sc, I, a) == om.select_row(sc, I, b)


def test_all_ties_pick_lowest():
    """kp constant for every token: every candidate block of a row has the same
    score, so the picks are blocks 0 .. k-2."""
    rng = np.random.default_rng(3)
    cfg = _cfg(topk=4, q_block=128, local_window=1)
    T = 128 * 12 + 37
    qp = rng.standard_normal((T, cfg.heads_kv, cfg.proxy_dim))
    kp = np.broadcast_to(rng.standard_normal((1, cfg.heads_kv, cfg.proxy_dim)),
                         (T, cfg.heads_kv, cfg.proxy_dim)).copy()
    cu = np.array([0, T])
    S = om.proxy_block_scores(qp, kp, cu, cfg)
    idx, cnt = om.select_blocks(S, cu, cfg)
    for g in range(cfg.heads_kv):
        for I in range(-(-T // 128)):
            dg = I
            sel = list(idx[g, I, :cnt[g, I]])
            if om.candidate_count(I, cfg) == 0:
                assert sel == list(range(dg + 1))
            else:
                assert sel == [0, 1, 2] + [dg - 1, dg]


@pytest.mark.parametrize("name", ["select_example.json", "select_dilation_example.json"])
def test_golden_hand_example(name):
    with open(os.path.join(GOLDEN, name)) as f:
        ex = json.load(f)
    cfg = _cfg(q_block=ex["q_block"], topk=ex["topk"], local_window=ex["local_window"],
               dilation=ex.get("dilation", 1))
    for row in ex["rows"]:
        sel = om.select_row(np.asarray(row["candidate_scores"], dtype=np.float64), row["I"], cfg)
        assert sel == row["expected"], row


def _invariants(idx, cnt, cu, cfg):
    docs = om.doc_grid(cu, cfg)
    for g in range(cfg.heads_kv):
        for d in docs:
            for I in range(d.nq):
                QB = d.qb0 + I
                sel = list(idx[g, QB, :cnt[g, QB]])
                dg = om.diag_block(I, cfg) + d.kb0
                pool = max(0, dg - d.kb0 - cfg.local_window * cfg.dilation)
                forced = [dg - i * cfg.dilation for i in range(cfg.local_window + 1)
                          if dg - i * cfg.dilation >= d.kb0]
                assert cnt[g, QB] == min(cfg.topk - 1, pool) + len(forced)
                if cfg.dilation == 1:
                    assert cnt[g, QB] == min(cfg.topk + cfg.local_window, dg - d.kb0 + 1)
                assert all(x == -1 for x in idx[g, QB, cnt[g, QB]:])
                assert sel == sorted(set(sel))                     # ascending, unique
                assert all(d.kb0 <= x < d.kb0 + d.nk for x in sel)  # inside the document
                assert all(x <= dg for x in sel)                   # causal
                for f in forced:
                    assert f in sel                                # diagonal + window
                assert all(x in forced or x < d.kb0 + pool for x in sel)


@pytest.mark.parametrize("seqlens,q_block,topk,w,dil", [((1000, 300, 2000), 64, 4, 0, 1),
                                                        ((3000, 129), 128, 3, 2, 1),
                                                        ((2600, 700), 64, 3, 2, 3)])
def test_selection_invariants_and_inverse(seqlens, q_block, topk, w, dil):
    rng = np.random.default_rng(11)
    cfg = _cfg(q_block=q_block, topk=topk, local_window=w, dilation=dil)
    T = sum(seqlens)
    qp = rng.standard_normal((T, cfg.heads_kv, cfg.proxy_dim))
    kp = rng.standard_normal((T, cfg.heads_kv, cfg.proxy_dim))
    cu = np.concatenate([[0], np.cumsum(seqlens)])
    S = om.proxy_block_scores(qp, kp, cu, cfg)
    idx, cnt = om.select_blocks(S, cu, cfg)
    _invariants(idx, cnt, cu, cfg)
    nqb, nkb, _ = om.totals(om.doc_grid(cu, cfg))
    ptr, inv = om.invert_index(idx, cnt, nkb)
    for g in range(cfg.heads_kv):
        assert ptr[g, -1] == cnt[g].sum()
        pairs_fwd = {(int(QB), int(KB)) for QB in range(nqb) for KB in idx[g, QB, :cnt[g, QB]]}
        pairs_inv = set()
        for KB in range(nkb):
            lst = list(inv[g, ptr[g, KB]:ptr[g, KB + 1]])
            assert lst == sorted(set(lst))
            pairs_inv |= {(int(QB), KB) for QB in lst}
        assert pairs_fwd == pairs_inv
        assert all(x == -1 for x in inv[g, ptr[g, -1]:])


def test_window_covers_everything_when_short():
    cfg = _cfg(q_block=128, topk=4, local_window=2)
    for I in range(6):
        sel = om.select_row(np.zeros(om.candidate_count(I, cfg)), I, cfg)
        assert sel == list(range(I + 1))
    # first row with candidates: diag 6, n = 7 > 6
    assert om.candidate_count(6, cfg) == 4
