"""Pins for the oracle's sparse GQA forward and fused (main + proxy) backward.

Pins: the dense special case (top-k covering every block) against torch's CPU
float64 scaled-dot-product attention and autograd (the pages' own check was
against a standard PyTorch implementation [socker-news Flash-MSA summary,
要約]), explicit-loop brute force, closed forms, central finite differences,
invariants, and packing invariance for varlen inputs [same summary, 'varlen'].
"""
import math

import numpy as np
import pytest
import torch

from oracle import msa_oracle as om


def _cfg(**kw):
    base = dict(heads_q=4, heads_kv=2, head_dim=16, proxy_dim=8, q_block=64, topk=2,
                local_window=0, kv_block=128)
    base.update(kw)
    return om.Config(**base)


def _inputs(rng, T, cfg, scale=1.0):
    q = scale * rng.standard_normal((T, cfg.heads_q, cfg.head_dim))
    k = scale * rng.standard_normal((T, cfg.heads_kv, cfg.head_dim))
    v = rng.standard_normal((T, cfg.heads_kv, cfg.head_dim))
    qp = scale * rng.standard_normal((T, cfg.heads_kv, cfg.proxy_dim))
    kp = scale * rng.standard_normal((T, cfg.heads_kv, cfg.proxy_dim))
    dO = rng.standard_normal((T, cfg.heads_q, cfg.head_dim))
    return q, k, v, qp, kp, dO


def _select(qp, kp, cu, cfg):
    S = om.proxy_block_scores(qp, kp, cu, cfg)
    return om.select_blocks(S, cu, cfg)


def _torch_dense(q, k, v, cu, G):
    """Causal GQA via torch SDPA per document (float64 CPU)."""
    outs = []
    for b in range(len(cu) - 1):
        s, e = int(cu[b]), int(cu[b + 1])
        if e == s:
            continue
        Q = torch.from_numpy(q[s:e]).permute(1, 0, 2)
        K = torch.from_numpy(k[s:e]).permute(1, 0, 2).repeat_interleave(G, 0)
        V = torch.from_numpy(v[s:e]).permute(1, 0, 2).repeat_interleave(G, 0)
        outs.append(torch.nn.functional.scaled_dot_product_attention(
            Q, K, V, is_causal=True).permute(1, 0, 2))
    return torch.cat(outs).numpy()


@pytest.mark.parametrize("seqlens", [(600,), (130, 0, 777, 64)])
def test_dense_special_case(seqlens):
    rng = np.random.default_rng(0)
    cfg = _cfg(topk=64)          # covers every block of these documents
    T = sum(seqlens)
    q, k, v, qp, kp, dO = _inputs(rng, T, cfg)
    cu = np.concatenate([[0], np.cumsum(seqlens)])
    idx, cnt = _select(qp, kp, cu, cfg)
    O, LSE, _ = om.forward(q, k, v, qp, kp, cu, idx, cnt, cfg)
    O_t = _torch_dense(q, k, v, cu, cfg.G)
    np.testing.assert_allclose(O, O_t, atol=1e-12, rtol=0)
    O_d, LSE_d = om.dense_causal_gqa(q, k, v, cu, cfg.scale, cfg.G)
    np.testing.assert_allclose(O, O_d, atol=1e-12, rtol=0)
    np.testing.assert_allclose(LSE, LSE_d, atol=1e-12, rtol=0)


def test_dense_backward_vs_autograd():
    rng = np.random.default_rng(5)
    cfg = _cfg(topk=64)
    seqlens = (300, 200)
    T = sum(seqlens)
    q, k, v, qp, kp, dO = _inputs(rng, T, cfg)
    cu = np.concatenate([[0], np.cumsum(seqlens)])
    idx, cnt = _select(qp, kp, cu, cfg)
    dq, dk, dv, _, _ = om.backward(q, k, v, qp, kp, dO, cu, idx, cnt, cfg)
    tq, tk, tv = (torch.from_numpy(x).requires_grad_() for x in (q, k, v))
    outs = []
    for b in range(len(cu) - 1):
        s, e = int(cu[b]), int(cu[b + 1])
        Q = tq[s:e].permute(1, 0, 2)
        K = tk[s:e].permute(1, 0, 2).repeat_interleave(cfg.G, 0)
        V = tv[s:e].permute(1, 0, 2).repeat_interleave(cfg.G, 0)
        outs.append(torch.nn.functional.scaled_dot_product_attention(
            Q, K, V, is_causal=True).permute(1, 0, 2))
    torch.cat(outs).backward(torch.from_numpy(dO))
    np.testing.assert_allclose(dq, tq.grad.numpy(), atol=1e-11, rtol=0)
    np.testing.assert_allclose(dk, tk.grad.numpy(), atol=1e-11, rtol=0)
    np.testing.assert_allclose(dv, tv.grad.numpy(), atol=1e-11, rtol=0)


def test_bruteforce_loops_tiny():
    """Explicit per-token loops with math.exp over the selected keys."""
    rng = np.random.default_rng(2)
    cfg = _cfg(topk=2, q_block=64, head_dim=4, proxy_dim=4, heads_q=2, heads_kv=1)
    T = 3 * 128 + 50
    q, k, v, qp, kp, dO = _inputs(rng, T, cfg)
    cu = np.array([0, T])
    idx, cnt = _select(qp, kp, cu, cfg)
    O, LSE, LSEp = om.forward(q, k, v, qp, kp, cu, idx, cnt, cfg)
    for h in range(cfg.heads_q):
        for t in range(0, T, 7):
            blocks = set(idx[0, t // cfg.q_block, :cnt[0, t // cfg.q_block]].tolist())
            keys = [u for u in range(t + 1) if u // 128 in blocks]
            z = [cfg.scale * sum(q[t, h, c] * k[u, 0, c] for c in range(4)) for u in keys]
            m = max(z)
            ssum = sum(math.exp(x - m) for x in z)
            assert abs(LSE[h, t] - (m + math.log(ssum))) < 1e-12
            for c in range(4):
                o = sum(math.exp(x - m) / ssum * v[u, 0, c] for x, u in zip(z, keys))
                assert abs(O[t, h, c] - o) < 1e-12
            y = [cfg.pscale * sum(qp[t, 0, c] * kp[u, 0, c] for c in range(4)) for u in keys]
            my = max(y)
            assert abs(LSEp[0, t] - (my + math.log(sum(math.exp(x - my) for x in y)))) < 1e-12


def test_closed_form_zero_query():
    """q = 0: uniform attention over A_i, so O_i is the mean of v over A_i and
    LSE_i = ln |A_i|; kp = 0 likewise gives LSE_p = ln |A_i|."""
    rng = np.random.default_rng(9)
    cfg = _cfg(topk=2, q_block=128, local_window=0)
    T = 5 * 128 + 11
    q, k, v, qp, kp, dO = _inputs(rng, T, cfg)
    cu = np.array([0, T])
    idx, cnt = _select(qp, kp, cu, cfg)
    O, LSE, LSEp = om.forward(np.zeros_like(q), k, v, qp, np.zeros_like(kp), cu, idx, cnt, cfg)
    for t in range(T):
        I = t // 128
        blocks = idx[0, I, :cnt[0, I]]
        keys = np.array([u for u in range(t + 1) if u // 128 in blocks])
        for h in range(cfg.G):           # heads of group 0
            np.testing.assert_allclose(O[t, h], v[keys, 0].mean(0), atol=1e-12)
            assert abs(LSE[h, t] - math.log(len(keys))) < 1e-12
        assert abs(LSEp[0, t] - math.log(len(keys))) < 1e-12


def _fd_setup(seed=4):
    rng = np.random.default_rng(seed)
    cfg = _cfg(topk=2, q_block=64, local_window=1, head_dim=8, proxy_dim=4)
    seqlens = (450, 300)
    T = sum(seqlens)
    q, k, v, qp, kp, dO = _inputs(rng, T, cfg, scale=0.7)
    cu = np.concatenate([[0], np.cumsum(seqlens)])
    idx, cnt = _select(qp, kp, cu, cfg)
    return rng, cfg, cu, idx, cnt, [q, k, v, qp, kp, dO]


def test_main_backward_finite_differences():
    rng, cfg, cu, idx, cnt, X = _fd_setup()
    grads = om.backward(*X, cu, idx, cnt, cfg)
    h = 1e-5
    for which in range(3):                      # q, k, v
        G = grads[which]
        for _ in range(6):
            pos = tuple(int(rng.integers(0, s)) for s in X[which].shape)
            plus = [x.copy() for x in X]
            minus = [x.copy() for x in X]
            plus[which][pos] += h
            minus[which][pos] -= h
            lp, _ = om.losses(*plus, cu, idx, cnt, cfg)
            lm, _ = om.losses(*minus, cu, idx, cnt, cfg)
            fd = (lp - lm) / (2 * h)
            assert abs(fd - G[pos]) < 1e-6 * max(1.0, abs(fd)), (which, pos, fd, G[pos])
        # a random direction
        Dir = rng.standard_normal(X[which].shape)
        plus = [x.copy() for x in X]
        minus = [x.copy() for x in X]
        plus[which] += h * Dir
        minus[which] -= h * Dir
        fd = (om.losses(*plus, cu, idx, cnt, cfg)[0] - om.losses(*minus, cu, idx, cnt, cfg)[0]) / (2 * h)
        assert abs(fd - (G * Dir).sum()) < 1e-5 * max(1.0, abs(fd))


def test_proxy_backward_finite_differences():
    rng, cfg, cu, idx, cnt, X = _fd_setup(6)
    _, _, _, dqp, dkp = om.backward(*X, cu, idx, cnt, cfg)
    Tfix = om.group_mean_probs(*X[:5], cu, idx, cnt, cfg)
    h = 1e-5
    for which, G in ((3, dqp), (4, dkp)):
        for _ in range(6):
            pos = tuple(int(rng.integers(0, s)) for s in X[which].shape)
            plus = [x.copy() for x in X]
            minus = [x.copy() for x in X]
            plus[which][pos] += h
            minus[which][pos] -= h
            fd = (om.losses(*plus, cu, idx, cnt, cfg, T_fixed=Tfix)[1]
                  - om.losses(*minus, cu, idx, cnt, cfg, T_fixed=Tfix)[1]) / (2 * h)
            assert abs(fd - G[pos]) < 1e-6 * max(1.0, abs(fd)), (which, pos, fd, G[pos])
        Dir = rng.standard_normal(X[which].shape)
        plus = [x.copy() for x in X]
        minus = [x.copy() for x in X]
        plus[which] += h * Dir
        minus[which] -= h * Dir
        fd = (om.losses(*plus, cu, idx, cnt, cfg, T_fixed=Tfix)[1]
              - om.losses(*minus, cu, idx, cnt, cfg, T_fixed=Tfix)[1]) / (2 * h)
        assert abs(fd - (G * Dir).sum()) < 1e-5 * max(1.0, abs(fd))


def test_gradient_invariants():
    """Per (document, group): sum_u dK = 0 and sum_u dkp = 0 (softmax rows of
    dS and dY sum to zero); sum_u dV = sum over the group's heads of dO; T is a
    probability distribution over each row's selected keys."""
    _, cfg, cu, idx, cnt, X = _fd_setup(8)
    q, k, v, qp, kp, dO = X
    dq, dk, dv, dqp, dkp = om.backward(*X, cu, idx, cnt, cfg)
    for b in range(len(cu) - 1):
        s, e = int(cu[b]), int(cu[b + 1])
        for g in range(cfg.heads_kv):
            np.testing.assert_allclose(dk[s:e, g].sum(0), 0, atol=1e-10)
            np.testing.assert_allclose(dkp[s:e, g].sum(0), 0, atol=1e-10)
            np.testing.assert_allclose(dv[s:e, g].sum(0),
                                       dO[s:e, g * cfg.G:(g + 1) * cfg.G].sum((0, 1)), atol=1e-10)
    Tm = om.group_mean_probs(q, k, v, qp, kp, cu, idx, cnt, cfg)
    for T in Tm.values():
        np.testing.assert_allclose(T.sum(1), 1.0, atol=1e-12)


def test_proxy_equals_main_special_case():
    """G = 1, qp = q, kp = k, dp = d and s_p = s: Q = T, so L_aux = 0 and the
    proxy gradients vanish."""
    rng = np.random.default_rng(12)
    cfg = _cfg(heads_q=2, heads_kv=2, head_dim=8, proxy_dim=8, topk=2)
    T = 400
    q, k, v, _, _, dO = _inputs(rng, T, cfg)
    cu = np.array([0, T])
    idx, cnt = _select(q.copy(), k.copy(), cu, cfg)
    _, _, _, dqp, dkp = om.backward(q, k, v, q, k, dO, cu, idx, cnt, cfg)
    assert np.abs(dqp).max() < 1e-13 and np.abs(dkp).max() < 1e-13
    _, La = om.losses(q, k, v, q, k, dO, cu, idx, cnt, cfg)
    assert abs(La) < 1e-10


def test_uniform_proxy_special_case():
    """kp = 0: Q is uniform over A_i, so dY = lam (1/|A_i| - T)."""
    rng = np.random.default_rng(13)
    cfg = _cfg(topk=2, proxy_loss_weight=0.5)
    T = 300
    q, k, v, qp, kp, dO = _inputs(rng, T, cfg)
    cu = np.array([0, T])
    idx, cnt = _select(qp, kp, cu, cfg)
    docs = om.doc_grid(cu, cfg)
    fw = om.qblock_forward(q, k, v, qp, np.zeros_like(kp), docs[0], 1, 3,
                           list(idx[1, 3, :cnt[1, 3]]), cfg)
    bw = om.qblock_backward(fw, q, k, v, qp, np.zeros_like(kp), dO, 1, cfg)
    nvalid = fw["mask"].sum(1, keepdims=True)
    np.testing.assert_allclose(fw["Q"], np.where(fw["mask"], 1.0 / nvalid, 0.0), atol=1e-14)
    np.testing.assert_allclose(bw["dqp"], 0.0, atol=1e-14)     # kp = 0
    dY = 0.5 * (fw["Q"] - bw["T"])
    np.testing.assert_allclose(bw["dkp"], cfg.pscale * dY.T @ qp[fw["rows"], 1], atol=1e-13)


def test_packing_invariance():
    """A packed batch equals the concatenation of its documents run alone."""
    rng = np.random.default_rng(21)
    cfg = _cfg(topk=2, q_block=64, local_window=1)
    seqlens = (333, 512, 129)
    T = sum(seqlens)
    X = _inputs(rng, T, cfg)
    cu = np.concatenate([[0], np.cumsum(seqlens)])
    packed = om.run_all(*X, cu, cfg)
    s = 0
    for L in seqlens:
        part = om.run_all(*[x[s:s + L] for x in X], np.array([0, L]), cfg)
        for key in ("O", "dq", "dk", "dv", "dqp", "dkp"):
            np.testing.assert_allclose(packed[key][s:s + L], part[key], atol=1e-13)
        np.testing.assert_allclose(packed["LSE"][:, s:s + L], part["LSE"], atol=1e-13)
        s += L


def test_sampled_matches_full():
    rng = np.random.default_rng(30)
    cfg = _cfg(topk=3, q_block=64, local_window=1)
    seqlens = (700, 260)
    T = sum(seqlens)
    X = _inputs(rng, T, cfg)
    cu = np.concatenate([[0], np.cumsum(seqlens)])
    full = om.run_all(*X, cu, cfg)
    qs = om.sampled_query_side(*X, cu, full["q2k_idx"], full["q2k_cnt"], cfg, [(0, 3), (1, 11), (1, 15)])
    for r in qs:
        hs = slice(r["g"] * cfg.G, (r["g"] + 1) * cfg.G)
        np.testing.assert_allclose(r["O"], full["O"][r["rows"]][:, hs], atol=1e-13)
        np.testing.assert_allclose(r["LSE"], full["LSE"][hs][:, r["rows"]], atol=1e-13)
        np.testing.assert_allclose(r["dQ"], full["dq"][r["rows"]][:, hs], atol=1e-13)
        np.testing.assert_allclose(r["dqp"], full["dqp"][r["rows"], r["g"]], atol=1e-13)
    ks = om.sampled_key_side(*X, cu, full["q2k_idx"], full["q2k_cnt"], cfg, [(0, 0), (1, 4), (0, 7)])
    for r in ks:
        np.testing.assert_allclose(r["dK"], full["dk"][r["keys"], r["g"]], atol=1e-12)
        np.testing.assert_allclose(r["dV"], full["dv"][r["keys"], r["g"]], atol=1e-12)
        np.testing.assert_allclose(r["dkp"], full["dkp"][r["keys"], r["g"]], atol=1e-12)
    # restricted to ranges of query blocks, the parts sum to the whole
    parts = [om.sampled_key_side(*X, cu, full["q2k_idx"], full["q2k_cnt"], cfg, [(0, 0), (1, 4), (0, 7)],
                                 qblocks=(lo, lo + 4)) for lo in range(0, 12, 4)]
    for i, r in enumerate(ks):
        for key in ("dK", "dV", "dkp"):
            np.testing.assert_allclose(sum(p[i][key] for p in parts), r[key], atol=1e-12)


def test_sampled_matches_full_shared_head():
    """The sampled evaluators with one shared proxy head (R1s): dqp and dkp of
    the shared head (T over every group's heads) equal the layer backward's."""
    rng = np.random.default_rng(31)
    cfg = _cfg(topk=3, q_block=64, local_window=1, proxy_heads=1)
    seqlens = (700, 260)
    T = sum(seqlens)
    X = _inputs(rng, T, cfg)
    cu = np.concatenate([[0], np.cumsum(seqlens)])
    full = om.run_all(*X, cu, cfg)
    assert full["dqp"].shape[1] == 1 and full["dkp"].shape[1] == 1
    qs = om.sampled_query_side(*X, cu, full["q2k_idx"], full["q2k_cnt"], cfg, [(0, 3), (1, 11), (1, 15)])
    for r in qs:
        hs = slice(r["g"] * cfg.G, (r["g"] + 1) * cfg.G)
        assert r["p"] == 0
        np.testing.assert_allclose(r["O"], full["O"][r["rows"]][:, hs], atol=1e-13)
        np.testing.assert_allclose(r["LSE_p"], full["LSEp"][0, r["rows"]], atol=1e-13)
        np.testing.assert_allclose(r["dQ"], full["dq"][r["rows"]][:, hs], atol=1e-13)
        np.testing.assert_allclose(r["dqp"], full["dqp"][r["rows"], 0], atol=1e-13)
    ks = om.sampled_key_side(*X, cu, full["q2k_idx"], full["q2k_cnt"], cfg, [(0, 0), (1, 4), (0, 7)])
    for r in ks:
        np.testing.assert_allclose(r["dK"], full["dk"][r["keys"], r["g"]], atol=1e-12)
        np.testing.assert_allclose(r["dV"], full["dv"][r["keys"], r["g"]], atol=1e-12)
        np.testing.assert_allclose(r["dkp"], full["dkp"][r["keys"], 0], atol=1e-12)


# ---------------------------------------------------------------------------
# the shared proxy head (one proxy head for all KV groups)
# ---------------------------------------------------------------------------

def _shared_setup(seed, heads_q=4, heads_kv=2):
    rng = np.random.default_rng(seed)
    cfg = _cfg(heads_q=heads_q, heads_kv=heads_kv, topk=2, q_block=64, local_window=1, head_dim=8,
               proxy_dim=4, proxy_heads=1)
    seqlens = (450, 300)
    T = sum(seqlens)
    q, k, v, _, _, dO = _inputs(rng, T, cfg, scale=0.7)
    qp = 0.7 * rng.standard_normal((T, 1, cfg.proxy_dim))
    kp = 0.7 * rng.standard_normal((T, 1, cfg.proxy_dim))
    cu = np.concatenate([[0], np.cumsum(seqlens)])
    idx, cnt = _select(qp, kp, cu, cfg)
    return rng, cfg, cu, idx, cnt, [q, k, v, qp, kp, dO]


def test_shared_proxy_with_one_group_is_the_per_group_reading():
    """With one KV group the shared head and the per-group head are the same."""
    _, cfg, cu, idx, cnt, X = _shared_setup(31, heads_q=3, heads_kv=1)
    per = om.Config(**{**cfg.__dict__, "proxy_heads": 0})
    a = om.run_all(*X, cu, cfg)
    b = om.run_all(*X, cu, per)
    for key in a:
        assert np.array_equal(a[key], b[key]), key


def test_shared_proxy_is_the_mean_of_replicated_groups():
    """T over all Hq heads is the mean of the groups' means, and the proxy
    gradients are linear in T: the shared head's dqp, dkp equal the average
    over groups of the per-group reading run with qp, kp and the block lists
    copied to every group; LSE_p and every main output are unchanged."""
    _, cfg, cu, idx, cnt, X = _shared_setup(32)
    q, k, v, qp, kp, dO = X
    Hkv = cfg.heads_kv
    per = om.Config(**{**cfg.__dict__, "proxy_heads": 0})
    rep = [np.repeat(qp, Hkv, axis=1), np.repeat(kp, Hkv, axis=1)]
    idx_r, cnt_r = np.repeat(idx, Hkv, axis=0), np.repeat(cnt, Hkv, axis=0)
    O, LSE, LSEp = om.forward(q, k, v, qp, kp, cu, idx, cnt, cfg)
    O2, LSE2, LSEp2 = om.forward(q, k, v, *rep, cu, idx_r, cnt_r, per)
    assert np.array_equal(O, O2) and np.array_equal(LSE, LSE2)
    for g in range(Hkv):
        assert np.array_equal(LSEp[0], LSEp2[g])
    g1 = om.backward(q, k, v, qp, kp, dO, cu, idx, cnt, cfg)
    g2 = om.backward(q, k, v, *rep, dO, cu, idx_r, cnt_r, per)
    for a, b in zip(g1[:3], g2[:3]):
        assert np.array_equal(a, b)
    np.testing.assert_allclose(g1[3][:, 0], g2[3].mean(axis=1), rtol=0, atol=1e-13)
    np.testing.assert_allclose(g1[4][:, 0], g2[4].mean(axis=1), rtol=0, atol=1e-13)
    # and it is not any single group's reading
    assert np.abs(g1[3][:, 0] - g2[3][:, 0]).max() > 1e-3


def test_shared_proxy_finite_differences():
    rng, cfg, cu, idx, cnt, X = _shared_setup(33)
    _, _, _, dqp, dkp = om.backward(*X, cu, idx, cnt, cfg)
    assert dqp.shape[1] == 1 and dkp.shape[1] == 1
    Tfix = om.group_mean_probs(*X[:5], cu, idx, cnt, cfg)
    h = 1e-5
    for which, G in ((3, dqp), (4, dkp)):
        for _ in range(6):
            pos = tuple(int(rng.integers(0, s)) for s in X[which].shape)
            plus = [x.copy() for x in X]
            minus = [x.copy() for x in X]
            plus[which][pos] += h
            minus[which][pos] -= h
            fd = (om.losses(*plus, cu, idx, cnt, cfg, T_fixed=Tfix)[1]
                  - om.losses(*minus, cu, idx, cnt, cfg, T_fixed=Tfix)[1]) / (2 * h)
            assert abs(fd - G[pos]) < 1e-6 * max(1.0, abs(fd)), (which, pos, fd, G[pos])


def test_shared_proxy_invariants():
    """sum_u dkp = 0 per document (rows of dY sum to zero); T is a distribution."""
    _, cfg, cu, idx, cnt, X = _shared_setup(34)
    _, _, _, _, dkp = om.backward(*X, cu, idx, cnt, cfg)
    for b in range(len(cu) - 1):
        np.testing.assert_allclose(dkp[int(cu[b]):int(cu[b + 1]), 0].sum(0), 0, atol=1e-10)
    for T in om.group_mean_probs(*X[:5], cu, idx, cnt, cfg).values():
        np.testing.assert_allclose(T.sum(1), 1.0, atol=1e-12)
