"""GPU parity at the full workload sizes, in the launch configuration the
benchmark times (same workloads, seed, dtype, buffers and entry points).

The oracle cannot run a whole 32k-1M token layer, so it checks sampled outputs
one by one, with the inputs gathered row by row from the seeded device tensors:

* sampled query blocks (first, middle and ragged last blocks of the longest and
  shortest documents, plus random ones): the fp32 block scores of the row are
  within the dot-product rounding bound of the fp64 scores; selecting the GPU's
  own scores gives the GPU's block list bit for bit, and the list is a valid
  top-k of the fp64 scores up to that bound; O, LSE, LSE_p, dQ and dqp of the
  block equal the oracle's for the GPU's block list;
* sampled KV blocks (the last block of a document, and random blocks with
  short inverted lists so that the oracle finishes in seconds): dK, dV and dkp
  summed over every query block that selected them;
* the KV blocks with the longest inverted list and with the list at the 99th
  percentile: the same element-wise check, the oracle's sum taken in ranges of
  query blocks (one progress line per range);
* the 1M-token packing again with one proxy head shared by every group, and
  with a dilated forced window: the same sampled checks (with the shared
  head's lists, scores and gradients);
* whole-layer identities that hold at any size: per group, the sum over keys
  of dV equals the sum over queries and heads of dO (softmax rows sum to one),
  and the sums over keys of dK and dkp vanish (each row of dS and of dY sums to
  zero), within bounds set by bf16 rounding of the probabilities.
"""
import math
import os
import time
from dataclasses import replace

import numpy as np
import pytest
import torch

import block_sparse_attention_proxy_amd as msa
from msa_inputs import WORKLOADS, make_case_torch, seqlens_of
from oracle import msa_oracle as om
from tests.gpu_common import ATOL, COS_MIN, LSE_ATOL, cfgs, log, stats

pytestmark = pytest.mark.gpu

FULL = ["layer-32k", "layer-128k-gqa8", "layer-512k-window2", "varlen-1m-packed"]
SEED = 0                     # the benchmark's default seed
MAX_LIST = 24                # sampled KV blocks: at most this many query blocks in their list


class DeviceRows:
    """x[rows, h, cols] of a device tensor [T, H, X] as a host float32 array
    (the indexing the oracle uses)."""

    def __init__(self, t):
        self.t = t

    def __getitem__(self, idx):
        rows, h, cols = idx
        r = torch.as_tensor(np.asarray(rows, dtype=np.int64), device=self.t.device)
        return self.t.index_select(0, r)[:, h, cols].float().cpu().numpy()


def _run(name):
    w = WORKLOADS[name]
    w, cfg, ocfg = cfgs(w)
    seqlens = seqlens_of(w, SEED)
    log(f"[{name}] T={sum(seqlens)} docs={len(seqlens)}: inputs")
    x = make_case_torch(w, SEED, device="cuda", seqlens=seqlens)
    cu = x["cu_seqlens"].cpu().numpy()
    vl = msa.Varlen(x["cu_seqlens"], cu)
    buf = msa.Buffers(cfg, vl, device="cuda", need_bwd=True)
    log(f"[{name}] forward + backward through the C ABI")
    msa.run_forward(cfg, vl, x["q"], x["k"], x["v"], x["qp"], x["kp"], buf)
    msa.run_backward(cfg, vl, x["q"], x["k"], x["v"], x["qp"], x["kp"], x["dO"], buf)
    torch.cuda.synchronize()
    return w, ocfg, x, cu, buf


@pytest.fixture(scope="module", params=FULL)
def full_run(request):
    """One full-size run per workload, shared by the tests below."""
    run = _run(request.param)
    yield (request.param,) + run
    del run
    torch.cuda.empty_cache()


def _query_samples(docs, ocfg, rng, n_random=3):
    longest = max(docs, key=lambda d: d.length)
    shortest = min((d for d in docs if d.nq > 0), key=lambda d: d.length)
    picks = [(longest, 0), (longest, longest.nq // 2), (longest, longest.nq - 1),
             (shortest, shortest.nq - 1)]
    live = [d for d in docs if d.nq > 0]
    for _ in range(n_random):
        d = live[rng.integers(len(live))]
        picks.append((d, int(rng.integers(d.nq))))
    out, seen = [], set()
    for d, I in picks:
        g = int(rng.integers(ocfg.heads_kv))
        if (g, d.qb0 + I) not in seen:
            seen.add((g, d.qb0 + I))
            out.append((d, g, I))
    return out


def _key_samples(docs, ocfg, k2q_ptr, rng, n_random=2):
    """(group, KV block) samples; a group's inverted lists are its proxy
    head's (head 0 for every group when the head is shared)."""
    lens = np.diff(k2q_ptr, axis=1)                       # [Hp, NKB]
    out = []
    longest = max(docs, key=lambda d: d.length)
    g = int(rng.integers(ocfg.heads_kv))
    out.append((g, longest.kb0 + longest.nk - 1))          # last (possibly partial) block
    short = np.argwhere((lens >= 1) & (lens <= MAX_LIST))
    for j in rng.permutation(len(short))[:n_random]:
        p, KB = int(short[j][0]), int(short[j][1])
        out.append((int(rng.integers(ocfg.heads_kv)) if ocfg.proxy_heads == 1 else p, KB))
    return [(g, KB) for g, KB in out if 1 <= lens[ocfg.proxy_of(g), KB] <= 4 * MAX_LIST]


def _close(name, got, ref, atol=ATOL, cos_min=COS_MIN):
    maxabs, cos = stats(got, ref)
    log(f"  {name:6s} max-abs {maxabs:.3e}  cos {cos:.7f}  n={np.asarray(ref).size}")
    assert maxabs <= atol, f"{name}: max-abs {maxabs} > {atol}"
    assert cos >= cos_min, f"{name}: cosine {cos} < {cos_min}"


def test_fullsize_sampled_parity(full_run):
    _check_sampled(*full_run)


def _check_sampled(name, w, ocfg, x, cu, buf):
    """Selection, query side and key side on sampled blocks (see the module
    docstring); with a shared proxy head the block lists, scores and proxy
    gradients are those of head 0."""
    docs = om.doc_grid(cu, ocfg)
    rng = np.random.default_rng(20261202)
    L = {n: DeviceRows(x[n]) for n in ("q", "k", "v", "qp", "kp", "dO")}
    q2k_idx = buf.q2k_idx.cpu().numpy()
    q2k_cnt = buf.q2k_cnt.cpu().numpy()
    k2q_ptr = buf.k2q_ptr.cpu().numpy()
    G = ocfg.G

    # ---- selection on sampled rows
    qs = _query_samples(docs, ocfg, rng)
    for d, g, I in qs:
        QB = d.qb0 + I
        p = ocfg.proxy_of(g)
        got = [int(v) - d.kb0 for v in q2k_idx[p, QB, :q2k_cnt[p, QB]]]
        nc = om.candidate_count(I, ocfg)
        log(f"[{name}] selection p={p} doc@{d.start} len={d.length} I={I} candidates={nc}")
        if nc == 0:
            assert got == om.select_row(np.zeros(0), I, ocfg)
            continue
        s_gpu = buf.scores[p, d.s0 + I * d.nk: d.s0 + I * d.nk + nc].double().cpu().numpy()
        s_or = om.proxy_row_scores(L["qp"], L["kp"], d, p, I, ocfg)
        rows = np.arange(d.start + I * ocfg.q_block, min(d.start + (I + 1) * ocfg.q_block, d.start + d.length))
        keys = np.arange(d.start, d.start + nc * ocfg.kv_block)
        qn = np.linalg.norm(L["qp"][rows, p, :].astype(np.float64), axis=1).max()
        kn = np.linalg.norm(L["kp"][keys, p, :].astype(np.float64), axis=1).max()
        tau = ocfg.proxy_dim * 2.0 ** -23 * qn * kn
        err = np.abs(s_gpu - s_or).max()
        log(f"  scores max |gpu - fp64| {err:.3e} (bound {tau:.3e})")
        assert err <= tau
        assert got == om.select_row(s_gpu, I, ocfg), "selection of the GPU's own scores"
        picked = [J for J in got if J < nc]
        rest = np.setdiff1d(np.arange(nc), picked)
        if len(rest) and len(picked):
            assert s_or[picked].min() >= s_or[rest].max() - 2 * tau, "not a top-k of the fp64 scores"

    # ---- query side
    samples = [(g, d.qb0 + I) for d, g, I in qs]
    log(f"[{name}] oracle query side on {len(samples)} blocks")
    ref = om.sampled_query_side(L["q"], L["k"], L["v"], L["qp"], L["kp"], L["dO"], cu, q2k_idx, q2k_cnt,
                                ocfg, samples)
    acc = {k: ([], []) for k in ("O", "dQ", "dqp", "LSE", "LSE_p")}
    for r in ref:
        rows, g = r["rows"], r["g"]
        heads = list(range(g * G, (g + 1) * G))
        rt = torch.as_tensor(rows, device="cuda")
        o = buf.o.index_select(0, rt)[:, heads, :].float().cpu().numpy()
        dq = buf.dq.index_select(0, rt)[:, heads, :].cpu().numpy()
        dqp = buf.dqp.index_select(0, rt)[:, r["p"], :].cpu().numpy()
        lse = buf.lse[heads][:, rt].cpu().numpy()
        lsep = buf.lse_p[r["p"], rt].cpu().numpy()
        for k_, got in (("O", o), ("dQ", dq), ("dqp", dqp), ("LSE", lse), ("LSE_p", lsep)):
            acc[k_][0].append(np.ravel(got))
            acc[k_][1].append(np.ravel(r[k_]))
    for k_ in ("O", "dQ", "dqp"):
        _close(k_, np.concatenate(acc[k_][0]), np.concatenate(acc[k_][1]))
    for k_ in ("LSE", "LSE_p"):
        _close(k_, np.concatenate(acc[k_][0]), np.concatenate(acc[k_][1]), atol=LSE_ATOL, cos_min=0.0)

    # ---- key side
    ks = _key_samples(docs, ocfg, k2q_ptr, rng)
    lens = [int(k2q_ptr[ocfg.proxy_of(g), KB + 1] - k2q_ptr[ocfg.proxy_of(g), KB]) for g, KB in ks]
    log(f"[{name}] oracle key side on {len(ks)} blocks, list lengths {lens}")
    assert ks, "no KV block sampled"
    ref = om.sampled_key_side(L["q"], L["k"], L["v"], L["qp"], L["kp"], L["dO"], cu, q2k_idx, q2k_cnt,
                              ocfg, ks)
    acc = {k_: ([], []) for k_ in ("dK", "dV", "dkp")}
    for r in ref:
        kt = torch.as_tensor(r["keys"], device="cuda")
        for k_, t, hd in (("dK", buf.dk, r["g"]), ("dV", buf.dv, r["g"]), ("dkp", buf.dkp, r["p"])):
            acc[k_][0].append(np.ravel(t.index_select(0, kt)[:, hd, :].cpu().numpy()))
            acc[k_][1].append(np.ravel(r[k_]))
    for k_ in ("dK", "dV", "dkp"):
        _close(k_, np.concatenate(acc[k_][0]), np.concatenate(acc[k_][1]))


def test_fullsize_sum_identities(full_run):
    _check_identities(*full_run)


def _check_identities(name, w, ocfg, x, cu, buf):
    """Whole-layer identities (one proxy head per group): per group, sum over
    keys of dV = sum over queries and heads of dO, sums over keys of dK and
    dkp vanish, within bf16-rounding bounds."""
    G, Hkv, d, dp = ocfg.G, ocfg.heads_kv, ocfg.head_dim, ocfg.proxy_dim
    T = int(cu[-1])
    f64 = torch.float64
    z = lambda *shape: torch.zeros(shape, dtype=f64, device="cuda")
    sv, sk, sp = z(Hkv, d), z(Hkv, d), z(Hkv, dp)
    ref_v, ssq_do, ssq_q, ssq_qp = z(Hkv, d), z(Hkv, d), z(Hkv, d), z(Hkv, dp)
    step = 1 << 16
    for s0 in range(0, T, step):
        sl = slice(s0, min(T, s0 + step))
        sv += buf.dv[sl].to(f64).sum(0)
        sk += buf.dk[sl].to(f64).sum(0)
        sp += buf.dkp[sl].to(f64).sum(0)
        dO = x["dO"][sl].to(f64).view(-1, Hkv, G, d)
        ref_v += dO.sum(dim=(0, 2))
        ssq_do += dO.pow(2).sum(dim=(0, 2))
        del dO
        q = x["q"][sl].to(f64).view(-1, Hkv, G, d)
        ssq_q += q.pow(2).sum(dim=(0, 2))
        del q
        ssq_qp += x["qp"][sl].to(f64).pow(2).sum(0)
    # sum_t dV[t, g] = sum over queries and heads of g of dO; the rounding of
    # the probabilities to bf16 leaves ~2^-9 * sqrt(sum dO^2) per component
    err = (sv - ref_v).abs()
    bound = 2e-2 * ssq_do.sqrt()
    log(f"[{name}] sum dV: max err {err.max().item():.3e}, max ratio to bound {(err / bound).max().item():.3f}")
    assert bool((err <= bound).all())
    # sum_t dK[t, g] = 0 and sum_t dkp[t, g] = 0
    bk = 2e-2 * ocfg.scale * ssq_q.sqrt()
    log(f"[{name}] sum dK: max {sk.abs().max().item():.3e}, max ratio to bound {(sk.abs() / bk).max().item():.3f}")
    assert bool((sk.abs() <= bk).all())
    bp = 2e-2 * ocfg.proxy_loss_weight * ocfg.pscale * ssq_qp.sqrt()
    log(f"[{name}] sum dkp: max {sp.abs().max().item():.3e}, max ratio to bound {(sp.abs() / bp).max().item():.3f}")
    assert bool((sp.abs() <= bp).all())
    assert math.isfinite(buf.dq.abs().max().item())


def _doc_on_host(x, doc, g, G):
    """The document's rows of group g as host float32 arrays (heads of g for q
    and dO), in the oracle's [T, H, X] indexing with one KV group."""
    sl = slice(doc.start, doc.start + doc.length)
    return {n: x[n][sl, hs].float().cpu().numpy()
            for n, hs in (("q", slice(g * G, (g + 1) * G)), ("k", slice(g, g + 1)), ("v", slice(g, g + 1)),
                          ("qp", slice(g, g + 1)), ("kp", slice(g, g + 1)), ("dO", slice(g * G, (g + 1) * G)))}


@pytest.mark.timeout(1800)
def test_fullsize_hot_lists(full_run):
    """dK, dV and dkp element-wise on the KV block chosen by the most query
    blocks, and on one at the 99th percentile of list length.  The oracle runs
    on the block's document alone (packing invariance: a packed document's
    results are those of the document run by itself), over ranges of query
    blocks in parallel threads, and the parts are summed.  The list lengths
    (per group: max, 99th percentile, mean) are logged."""
    from concurrent.futures import ThreadPoolExecutor, as_completed
    from dataclasses import replace
    from threadpoolctl import threadpool_limits
    name, w, ocfg, x, cu, buf = full_run
    k2q_ptr = buf.k2q_ptr.cpu().numpy()
    lens = np.diff(k2q_ptr, axis=1)                       # [Hkv, NKB]
    for g in range(lens.shape[0]):
        nz = lens[g][lens[g] > 0]
        log(f"[{name}] group {g}: inverted lists max {nz.max()}, p99 {int(np.percentile(nz, 99))}, "
            f"mean {nz.mean():.1f} over {nz.size} KV blocks")
    g_hot, kb_hot = np.unravel_index(int(np.argmax(lens)), lens.shape)
    flat = lens.ravel()
    p99 = np.percentile(flat[flat > 0], 99)
    j99 = int(np.argmin(np.where(flat > 0, np.abs(flat - p99), np.inf)))
    g99, kb99 = np.unravel_index(j99, lens.shape)
    docs = om.doc_grid(cu, ocfg)
    q2k_idx = buf.q2k_idx.cpu().numpy()
    q2k_cnt = buf.q2k_cnt.cpu().numpy()
    G = ocfg.G
    one = replace(ocfg, heads_q=G, heads_kv=1)
    workers = max(1, min(16, len(os.sched_getaffinity(0))))
    for tag, g, KB in (("longest", int(g_hot), int(kb_hot)), ("p99", int(g99), int(kb99))):
        doc = next(d for d in docs if d.kb0 <= KB < d.kb0 + d.nk)
        n = int(lens[g, KB])
        log(f"[{name}] {tag} list: g={g} KB={KB} (block {KB - doc.kb0} of a {doc.length}-token document), "
            f"{n} query blocks")
        h = _doc_on_host(x, doc, g, G)
        rows = q2k_idx[g, doc.qb0:doc.qb0 + doc.nq]
        idx1 = np.where(rows >= 0, rows - doc.kb0, -1)[None].astype(np.int32)
        cnt1 = q2k_cnt[g, doc.qb0:doc.qb0 + doc.nq][None]
        cu1 = np.array([0, doc.length], dtype=np.int32)
        has = np.nonzero((rows == KB).any(axis=1))[0]
        step = max(1, -(-len(has) // (4 * workers)))
        ranges = [(int(has[i]), int(has[min(len(has), i + step) - 1]) + 1) for i in range(0, len(has), step)]

        def part(r):
            return om.sampled_key_side(h["q"], h["k"], h["v"], h["qp"], h["kp"], h["dO"], cu1, idx1, cnt1,
                                       one, [(0, KB - doc.kb0)], qblocks=r)[0]

        acc, t0, done = None, time.time(), 0
        with threadpool_limits(1), ThreadPoolExecutor(workers) as ex:
            futs = [ex.submit(part, r) for r in ranges]
            for fu in as_completed(futs):
                p = fu.result()
                if acc is None:
                    acc = p
                else:
                    for k_ in ("dK", "dV", "dkp"):
                        acc[k_] = acc[k_] + p[k_]
                done += 1
                if done % max(1, len(ranges) // 8) == 0 or done == len(ranges):
                    log(f"  {done}/{len(ranges)} ranges of query blocks done, {time.time() - t0:.0f} s")
        kt = torch.as_tensor(acc["keys"] + doc.start, device=buf.dk.device)
        for k_, t in (("dK", buf.dk), ("dV", buf.dv), ("dkp", buf.dkp)):
            _close(k_, t.index_select(0, kt)[:, g, :].cpu().numpy(), acc[k_])


@pytest.mark.parametrize("tag,over", [("shared head", dict(proxy_heads=1)),
                                      ("window 2 dilation 4", dict(local_window=2, dilation=4))])
def test_fullsize_block_pattern_variants(tag, over):
    """The 1M-token packing with a block-pattern variant at full size: one
    proxy head shared by every KV group (R1s), or a forced window of 2 blocks
    with dilation 4 (R3d).  The same sampled selection, query-side and
    key-side checks; with the shared head they use its lists, scores and
    gradients (T over every group's heads)."""
    name = "varlen-1m-packed"
    w, cfg, ocfg = cfgs(WORKLOADS[name], **over)
    seqlens = seqlens_of(w, SEED)
    log(f"[{name} {tag}] T={sum(seqlens)} docs={len(seqlens)}: inputs")
    x = make_case_torch(w, SEED, device="cuda", seqlens=seqlens)
    cu = x["cu_seqlens"].cpu().numpy()
    vl = msa.Varlen(x["cu_seqlens"], cu)
    buf = msa.Buffers(cfg, vl, device="cuda", need_bwd=True)
    assert tuple(buf.dqp.shape) == (sum(seqlens), ocfg.Hp, w.proxy_dim)
    log(f"[{name} {tag}] forward + backward through the C ABI")
    msa.run_forward(cfg, vl, x["q"], x["k"], x["v"], x["qp"], x["kp"], buf)
    msa.run_backward(cfg, vl, x["q"], x["k"], x["v"], x["qp"], x["kp"], x["dO"], buf)
    torch.cuda.synchronize()
    _check_sampled(f"{name} {tag}", w, ocfg, x, cu, buf)
    del buf, x
    torch.cuda.empty_cache()


def test_fullsize_single_1m_document():
    """The largest single document measured: 1,048,576 tokens in one sequence
    (the 1M-token geometry, k = 64, unpacked).  Candidate rows reach 8191
    blocks (the selection's re-read path), the proxy scores cover an 8192 x
    8192 block grid per group, and inverted lists are at their longest.  The
    same sampled selection, query-side and key-side checks, and the
    whole-layer identities."""
    w0 = WORKLOADS["varlen-1m-packed"]
    w = replace(w0, name="single-1m", seqlens=(1 << 20,), doc_mode="fixed", total_tokens=0)
    w, cfg, ocfg = cfgs(w)
    seqlens = seqlens_of(w, SEED)
    assert seqlens == [1 << 20]
    log(f"[single-1m] T={sum(seqlens)}: inputs")
    x = make_case_torch(w, SEED, device="cuda", seqlens=seqlens)
    cu = x["cu_seqlens"].cpu().numpy()
    vl = msa.Varlen(x["cu_seqlens"], cu)
    buf = msa.Buffers(cfg, vl, device="cuda", need_bwd=True)
    log("[single-1m] forward + backward through the C ABI")
    msa.run_forward(cfg, vl, x["q"], x["k"], x["v"], x["qp"], x["kp"], buf)
    msa.run_backward(cfg, vl, x["q"], x["k"], x["v"], x["qp"], x["kp"], x["dO"], buf)
    torch.cuda.synchronize()
    lens = np.diff(buf.k2q_ptr.cpu().numpy(), axis=1)
    log(f"[single-1m] inverted lists: longest {lens.max()}, mean {lens.mean():.1f}")
    _check_sampled("single-1m", w, ocfg, x, cu, buf)
    _check_identities("single-1m", w, ocfg, x, cu, buf)
    del buf, x
    torch.cuda.empty_cache()
