"""Shared helpers for the GPU parity tests: run the HIP path through the C ABI
and compare it with the CPU oracle on the same seeded inputs."""
from __future__ import annotations

import math
import sys
from dataclasses import replace

import numpy as np
import torch

import block_sparse_attention_proxy_amd as msa
from msa_inputs import Workload, make_case
from oracle import msa_oracle as om

ATOL = 2e-2          # max-abs bound on O and every gradient
COS_MIN = 0.9995     # cosine-similarity bound (fp64, flattened tensor)
LSE_ATOL = 1e-3      # sanity bound on LSE and LSE_p


def log(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def cfgs(w: Workload, **over):
    w = replace(w, **over) if over else w
    c = msa.Config(w.heads_q, w.heads_kv, w.head_dim, w.proxy_dim, w.q_block, w.topk,
                   w.local_window, 128, 0.0, 0.0, w.proxy_loss_weight, w.dtype, w.dilation,
                   w.proxy_heads)
    o = om.Config(w.heads_q, w.heads_kv, w.head_dim, w.proxy_dim, w.q_block, w.topk,
                  w.local_window, 128, None, None, w.proxy_loss_weight, w.dilation, w.proxy_heads)
    return w, c, o


def device_inputs(case, dtype):
    dt = torch.bfloat16 if dtype == "bf16" else torch.float32
    out = {}
    for name in ("q", "k", "v", "qp", "kp", "dO"):
        out[name] = torch.from_numpy(getattr(case, name)).to(dt).cuda()
    out["cu"] = torch.from_numpy(case.cu_seqlens).cuda()
    return out


def run_gpu(case, cfg: msa.Config, backward=True, scores=True):
    """Every stage through the C ABI; returns host numpy copies."""
    x = device_inputs(case, cfg.dtype)
    vl = msa.Varlen(x["cu"], case.cu_seqlens)
    buf = msa.Buffers(cfg, vl, device="cuda", need_bwd=backward)
    buf.scores.fill_(float("nan"))
    msa.run_forward(cfg, vl, x["q"], x["k"], x["v"], x["qp"], x["kp"], buf)
    if backward:
        msa.run_backward(cfg, vl, x["q"], x["k"], x["v"], x["qp"], x["kp"], x["dO"], buf)
    torch.cuda.synchronize()
    names = ["q2k_idx", "q2k_cnt", "k2q_ptr", "k2q_idx", "o", "lse", "lse_p"]
    if scores:
        names.append("scores")
    if backward:
        names += ["dq", "dk", "dv", "dqp", "dkp"]
    res = {n: getattr(buf, n).float().cpu().numpy() if getattr(buf, n).dtype in (torch.bfloat16, torch.float32)
           else getattr(buf, n).cpu().numpy() for n in names}
    res["layout"] = buf.layout
    return res


def stats(got, ref):
    g = np.asarray(got, dtype=np.float64).ravel()
    r = np.asarray(ref, dtype=np.float64).ravel()
    maxabs = float(np.abs(g - r).max()) if g.size else 0.0
    den = float(np.linalg.norm(g) * np.linalg.norm(r))
    cos = float(g @ r / den) if den > 0 else (1.0 if maxabs == 0 else 0.0)
    return maxabs, cos


def assert_close(name, got, ref, atol=ATOL, cos_min=COS_MIN):
    maxabs, cos = stats(got, ref)
    log(f"  {name:6s} max-abs {maxabs:.3e}  cos {cos:.7f}  |ref|max {np.abs(ref).max():.3e}")
    assert maxabs <= atol, f"{name}: max-abs {maxabs} > {atol}"
    assert cos >= cos_min, f"{name}: cosine {cos} < {cos_min}"


def candidate_mask(cu, ocfg):
    """Boolean [score_elems] of the entries the scoring must write."""
    docs = om.doc_grid(cu, ocfg)
    _, _, ns = om.totals(docs)
    m = np.zeros(ns, dtype=bool)
    for d in docs:
        for I in range(d.nq):
            nc = om.candidate_count(I, ocfg)
            m[d.s0 + I * d.nk: d.s0 + I * d.nk + nc] = True
    return m


def scores_as_oracle(gpu_scores, mask):
    S = np.full(gpu_scores.shape, -np.inf)
    S[:, mask] = gpu_scores[:, mask].astype(np.float64)
    return S


def check_inverse(res, ocfg):
    """k2q must be exactly the oracle's inverse of the GPU's own q2k."""
    nkb = res["layout"]["total_kvblocks"]
    ptr, idx = om.invert_index(res["q2k_idx"], res["q2k_cnt"], nkb)
    np.testing.assert_array_equal(res["k2q_ptr"], ptr)
    np.testing.assert_array_equal(res["k2q_idx"], idx)


def score_tolerance(case, ocfg):
    """Bound on |fp32 GPU score - fp64 score| per group: dp * 2^-23 * max|qp| * max|kp|
    (a dot-product rounding bound with the Cauchy-Schwarz estimate of sum |a_c b_c|)."""
    qn = np.linalg.norm(case.qp.astype(np.float64), axis=2).max(axis=0)
    kn = np.linalg.norm(case.kp.astype(np.float64), axis=2).max(axis=0)
    return ocfg.proxy_dim * 2.0 ** -23 * qn * kn


def oracle_attention(case, ocfg, q2k_idx, q2k_cnt, O_for_D=None):
    args = [getattr(case, n).astype(np.float64) for n in ("q", "k", "v", "qp", "kp", "dO")]
    O, LSE, LSEp = om.forward(*args[:5], case.cu_seqlens, q2k_idx, q2k_cnt, ocfg)
    grads = om.backward(*args, case.cu_seqlens, q2k_idx, q2k_cnt, ocfg, O_for_D=O_for_D)
    return O, LSE, LSEp, grads


def valid_lse(lse, T):
    return lse[:, :T]


def full_compare(case, res, ocfg, tag=""):
    log(f"[{tag}] T={case.q.shape[0]} oracle attention on the GPU's block lists")
    O, LSE, LSEp, (dq, dk, dv, dqp, dkp) = oracle_attention(case, ocfg, res["q2k_idx"], res["q2k_cnt"])
    assert_close("O", res["o"], O)
    assert_close("LSE", res["lse"], LSE, atol=LSE_ATOL, cos_min=0.0)
    assert_close("LSE_p", res["lse_p"], LSEp, atol=LSE_ATOL, cos_min=0.0)
    assert_close("dq", res["dq"], dq)
    assert_close("dk", res["dk"], dk)
    assert_close("dv", res["dv"], dv)
    assert_close("dqp", res["dqp"], dqp)
    assert_close("dkp", res["dkp"], dkp)


def small_case(w: Workload, seqlens, seed=0, exact_proxy=False):
    return make_case(w, seed=seed, seqlens=list(seqlens), exact_proxy=exact_proxy)


def tiny_tol_for(w):
    return (1e-4, 0.999999) if w.dtype == "f32" else (ATOL, COS_MIN)


__all__ = ["log", "cfgs", "run_gpu", "stats", "assert_close", "candidate_mask", "scores_as_oracle",
           "check_inverse", "score_tolerance", "oracle_attention", "full_compare", "small_case",
           "math"]
