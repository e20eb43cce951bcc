"""GPU parity for every configuration the ABI accepts, and for the forward's
re-accumulation branch, through the C ABI against the CPU oracle.

Coverage grid: for each built (head_dim, proxy_dim, dtype) -- (128, 64, bf16),
(64, 32, bf16), (64, 32, fp32) -- every group size G = Hq / Hkv in
{1, 2, 4, 8} and both query blocks (64, 128) reach a distinct set of kernel
instantiations (scoring, forward, proxy log-sum-exp, query-major and
KV-major backward, and the dqp reduction for G > 4 where the query-major
kernel is the generic one).  Each case runs on several documents with ragged
tails, with a top-k small enough that rows have real candidates.

Large logits: the forward takes a reference maximum per query from the first
32 keys of its block list and accumulates without rescaling; when a later key
scores more than 64 (base 2) above that reference the workgroup finds the
true row maxima and accumulates again.  The cases below plant keys that score
far above the first block's (a shared direction u: +k_amp u on the keys of
KV block 1 of every document, -k_amp u on every other key of group 0,
+q_amp u on group 0's queries), check on the host that the gap exceeds 64 (base 2) for
some query, and compare O, the LSEs and every gradient with the oracle.
"""
import math
from dataclasses import replace

import numpy as np
import pytest

from msa_inputs import WORKLOADS, round_bf16
from oracle import msa_oracle as om
from tests.gpu_common import cfgs, check_inverse, full_compare, log, run_gpu, small_case

pytestmark = pytest.mark.gpu

B128 = WORKLOADS["layer-32k"]          # bf16, d 128, dp 64, low-rank recipe
F32 = WORKLOADS["tiny-2k-fp32"]        # fp32, d 64, dp 32, i.i.d. recipe


def _grid():
    out = {}
    # bf16, d 64 / dp 32: every group size, both query blocks
    for G in (1, 2, 4, 8):
        for qb in (64, 128):
            out[f"bf16-d64-g{G}-qb{qb}"] = (B128, dict(head_dim=64, proxy_dim=32, heads_kv=2,
                                                       heads_q=2 * G, q_block=qb, topk=4),
                                            (1700, 333))
    # fp32, d 64 / dp 32: the group sizes and query blocks the tiny workload does not have
    for G, qb in ((1, 64), (1, 128), (2, 64), (2, 128), (4, 128), (8, 64), (8, 128)):
        out[f"f32-d64-g{G}-qb{qb}"] = (F32, dict(heads_kv=2, heads_q=2 * G, q_block=qb, topk=3),
                                       (1500, 421))
    # bf16, d 128 / dp 64: the (G, query block) pairs the main parity cases do not have
    for G, qb in ((1, 128), (2, 64), (8, 64)):
        out[f"bf16-d128-g{G}-qb{qb}"] = (B128, dict(heads_kv=2, heads_q=2 * G, q_block=qb, topk=4),
                                         (1700, 333))
    return out


GRID = _grid()


@pytest.mark.parametrize("name", list(GRID))
def test_config_grid_parity(name):
    w0, over, seqlens = GRID[name]
    w, cfg, ocfg = cfgs(w0, **over)
    case = small_case(w, seqlens, seed=21)
    log(f"[{name}] T={sum(seqlens)} d={w.head_dim} dp={w.proxy_dim} {w.dtype} G={w.group} "
        f"Bq={w.q_block} topk={w.topk}")
    res = run_gpu(case, cfg, backward=True)
    check_inverse(res, ocfg)
    full_compare(case, res, ocfg, tag=name)


# --------------------------------------------------------------------------
# large logits: the forward's second pass
# --------------------------------------------------------------------------

HOT = 1          # the KV block (per document) whose keys score high


def _plant_large_logits(case, ocfg, q_amp: float, k_amp: float, seed: int):
    """Add the shared direction u (unit norm) to group 0: +k_amp u on the keys
    of KV block HOT of every document, -k_amp u on the other keys, +q_amp u on
    every query of the group.  With softmax scale s the HOT keys then score
    about 2 s q_amp k_amp above the others (in nats)."""
    rng = np.random.default_rng(seed)
    d = ocfg.head_dim
    u = rng.standard_normal(d)
    u /= np.linalg.norm(u)
    q, k = case.q.astype(np.float64), case.k.astype(np.float64)
    sign = -np.ones(k.shape[0])
    for b in range(len(case.seqlens)):
        s0, L = int(case.cu_seqlens[b]), int(case.seqlens[b])
        lo, hi = s0 + HOT * 128, min(s0 + (HOT + 1) * 128, s0 + L)
        if lo < hi:
            sign[lo:hi] = 1.0
    k[:, 0, :] += k_amp * sign[:, None] * u[None, :]
    q[:, :ocfg.G, :] += q_amp * u[None, None, :]
    if case.workload.dtype == "bf16":
        case.q, case.k = round_bf16(q), round_bf16(k)
    else:
        case.q, case.k = q.astype(np.float32), k.astype(np.float32)
    return case


def _largest_gap(case, ocfg, q2k_idx, q2k_cnt):
    """max over group-0 queries of (row maximum - maximum over the first 32 keys
    of the row's list), base 2, after the softmax scale: what the forward's
    fixed reference misses by."""
    docs = om.doc_grid(case.cu_seqlens, ocfg)
    best = -np.inf
    l2e = math.log2(math.e)
    for doc in docs:
        for I in range(doc.nq):
            QB = doc.qb0 + I
            sel = [int(x) for x in q2k_idx[0, QB, :q2k_cnt[0, QB]]]
            rows = np.arange(doc.start + I * ocfg.q_block,
                             min(doc.start + (I + 1) * ocfg.q_block, doc.start + doc.length))
            first = doc.start + (sel[0] - doc.kb0) * 128 + np.arange(32)
            keys = np.concatenate([doc.start + (J - doc.kb0) * 128 + np.arange(128) for J in sel])
            keys = keys[keys < doc.start + doc.length]
            for h in range(ocfg.G):
                qh = case.q[rows, h, :].astype(np.float64)
                z = qh @ case.k[keys, 0, :].astype(np.float64).T * ocfg.scale * l2e
                z[keys[None, :] > rows[:, None]] = -np.inf
                zf = qh @ case.k[first, 0, :].astype(np.float64).T * ocfg.scale * l2e
                zf[first[None, :] > rows[:, None]] = -np.inf
                best = max(best, float((z.max(axis=1) - zf.max(axis=1)).max()))
    return best


LARGE = {
    # (workload, overrides, seqlens, planted gap in base 2)
    "bf16-d128-gap100": (B128, dict(heads_kv=2, heads_q=8, topk=3), (1100, 700), 100.0),
    # above 128 (base 2) the first pass's exponentials overflow to infinity
    "bf16-d128-gap150-qb128": (B128, dict(heads_kv=2, heads_q=16, q_block=128, topk=3), (900, 600), 150.0),
    "bf16-d64-gap100": (B128, dict(head_dim=64, proxy_dim=32, heads_kv=2, heads_q=8, topk=3), (1100, 700),
                        100.0),
    "f32-d64-gap100": (F32, dict(topk=3), (1100, 700), 100.0),
    "f32-d64-gap150-qb128": (F32, dict(q_block=128, topk=3), (900, 600), 150.0),
}


@pytest.mark.parametrize("name", list(LARGE))
def test_forward_large_logits_parity(name):
    """Amplitudes q_amp = 1.5 k_amp and softmax scale s = 1 / k_amp: the
    planted gap 2 s q_amp k_amp = 3 k_amp (nats).  dK scales with s q_amp =
    1.5 (its u component does not cancel); dQ's u component cancels (each row
    of dS sums to zero) up to the bf16 rounding of dS times s k_amp = 1, a
    small share of dQ; the spread of the logits off the planted direction
    stays about that of the ordinary inputs.  (These ratios were chosen by
    emulating the bf16 rounding of P and dS on the CPU: both the dQ cosine
    and the dK / dV max-abs errors keep a margin of about two.)"""
    w0, over, seqlens, gap = LARGE[name]
    k_amp = gap / math.log2(math.e) / 3.0
    scale = 1.0 / k_amp
    w, cfg, ocfg = cfgs(w0, **over)
    cfg, ocfg = replace(cfg, softmax_scale=scale), replace(ocfg, softmax_scale=scale)
    case = _plant_large_logits(small_case(w, seqlens, seed=31), ocfg, 1.5 * k_amp, k_amp, seed=32)
    log(f"[{name}] T={sum(seqlens)} planted gap {gap} (base 2), softmax scale {scale:.3e}")
    res = run_gpu(case, cfg, backward=True)
    got = _largest_gap(case, ocfg, res["q2k_idx"], res["q2k_cnt"])
    log(f"  largest gap over the first-32-key reference: {got:.1f} (base 2)")
    assert got > 64.0, "the inputs do not reach the forward's second pass"
    check_inverse(res, ocfg)
    full_compare(case, res, ocfg, tag=name)
