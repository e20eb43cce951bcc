"""GPU checks of the PyTorch drop-in (``msa_attention`` with autograd): it
returns what the C-ABI calls return on the same inputs, its gradients agree
with the oracle on its own block lists, and ``dense=True`` reproduces plain
causal attention and its gradients (fp64 autograd on the CPU)."""
import numpy as np
import pytest
import torch

import block_sparse_attention_proxy_amd as msa
from msa_inputs import WORKLOADS
from oracle import msa_oracle as om
from tests.gpu_common import assert_close, cfgs, full_compare, log, run_gpu, small_case

pytestmark = pytest.mark.gpu


def _autograd_run(case, w, dense=False):
    # (the workload's dilation and proxy-head count are passed through)
    dt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    leaves = {n: torch.from_numpy(getattr(case, n)).to(dt).cuda().requires_grad_(True)
              for n in ("q", "k", "v", "qp", "kp")}
    cu = torch.from_numpy(case.cu_seqlens).cuda()
    o = msa.msa_attention(*(leaves[n] for n in ("q", "k", "v", "qp", "kp")), cu, topk=w.topk,
                          q_block=w.q_block, local_window=w.local_window,
                          proxy_loss_weight=w.proxy_loss_weight,
                          cu_seqlens_host=[int(c) for c in case.cu_seqlens], dense=dense,
                          dilation=w.dilation, proxy_heads=w.proxy_heads)
    o.backward(torch.from_numpy(case.dO).to(dt).cuda())
    torch.cuda.synchronize()
    out = {"o": o.detach().float().cpu().numpy()}
    for n, g in (("q", "dq"), ("k", "dk"), ("v", "dv"), ("qp", "dqp"), ("kp", "dkp")):
        out[g] = leaves[n].grad.float().cpu().numpy()
    return out


@pytest.mark.parametrize("name,seqlens,shared", [("tiny-2k-fp32", (2048,), 0), ("layer-32k", (1500, 0, 700), 0),
                                                 ("tiny-2k-fp32", (2048,), 1)])
def test_autograd_equals_c_abi_path(name, seqlens, shared):
    """Same kernels, same inputs: the autograd wrapper's O is the C-ABI path's
    O bit for bit, and its gradients are the fp32 gradients (bf16 inputs get
    them rounded to bf16)."""
    w, cfg, ocfg = cfgs(WORKLOADS[name], topk=4, proxy_heads=shared)
    case = small_case(w, seqlens, seed=7)
    ref = run_gpu(case, cfg, backward=True, scores=False)
    got = _autograd_run(case, w)
    assert np.array_equal(got["o"], ref["o"])
    for g in ("dq", "dk", "dv", "dqp", "dkp"):
        if w.dtype == "f32":
            assert np.array_equal(got[g], ref[g]), g
        else:
            r = torch.from_numpy(ref[g]).to(torch.bfloat16).float().numpy()
            assert np.array_equal(got[g], r), g
    log(f"[{name}] autograd path identical to the C-ABI path")
    if w.dtype == "f32":
        full_compare(case, ref, ocfg, tag=name)


def test_autograd_dense_is_causal_attention():
    """dense=True: O, dq, dk, dv equal plain causal GQA attention and its
    gradients, computed by fp64 autograd on the CPU with no block notion."""
    w, cfg, ocfg = cfgs(WORKLOADS["layer-32k"])
    case = small_case(w, (1300, 520), seed=8)
    got = _autograd_run(case, w, dense=True)
    G = w.heads_q // w.heads_kv
    scale = 1.0 / np.sqrt(w.head_dim)
    q = torch.from_numpy(case.q.astype(np.float64)).requires_grad_(True)
    k = torch.from_numpy(case.k.astype(np.float64)).requires_grad_(True)
    v = torch.from_numpy(case.v.astype(np.float64)).requires_grad_(True)
    outs = []
    cu = [int(c) for c in case.cu_seqlens]
    for b in range(len(cu) - 1):
        s, e = cu[b], cu[b + 1]
        L = e - s
        kk = k[s:e].repeat_interleave(G, dim=1)             # [L, Hq, d]
        vv = v[s:e].repeat_interleave(G, dim=1)
        z = torch.einsum("ihd,jhd->hij", q[s:e], kk) * scale
        z = z.masked_fill(~torch.tril(torch.ones(L, L, dtype=torch.bool)), float("-inf"))
        outs.append(torch.einsum("hij,jhd->ihd", torch.softmax(z, dim=-1), vv))
    O = torch.cat(outs, dim=0)
    O.backward(torch.from_numpy(case.dO.astype(np.float64)))
    assert_close("O", got["o"], O.detach().numpy())
    assert_close("dq", got["dq"], q.grad.numpy())
    assert_close("dk", got["dk"], k.grad.numpy())
    assert_close("dv", got["dv"], v.grad.numpy())
    # the proxy gradients over the full lists, from the oracle
    topk_d = -(-max(e - s for s, e in zip(cu[:-1], cu[1:])) // 128)
    ocfg_d = om.Config(w.heads_q, w.heads_kv, w.head_dim, w.proxy_dim, w.q_block, topk_d, w.local_window)
    _, _, ns = om.totals(om.doc_grid(case.cu_seqlens, ocfg_d))
    idx, cnt = om.select_blocks(np.zeros((w.heads_kv, ns)), case.cu_seqlens, ocfg_d)
    args = [getattr(case, n).astype(np.float64) for n in ("q", "k", "v", "qp", "kp", "dO")]
    _, _, _, dqp, dkp = om.backward(*args, case.cu_seqlens, idx, cnt, ocfg_d)
    assert_close("dqp", got["dqp"], dqp)
    assert_close("dkp", got["dkp"], dkp)


def test_autograd_inplace_output_edit_raises():
    """O is saved for the backward like the inputs: changing the returned
    output in place before the backward is an autograd error, not a silent
    change of D = rowsum(dO O)."""
    w, cfg, ocfg = cfgs(WORKLOADS["layer-32k"], topk=4)
    case = small_case(w, (900,), seed=8)
    leaves = [torch.from_numpy(getattr(case, n)).to(torch.bfloat16).cuda().requires_grad_(True)
              for n in ("q", "k", "v", "qp", "kp")]
    cu = torch.from_numpy(case.cu_seqlens).cuda()
    o = msa.msa_attention(*leaves, cu, topk=w.topk, q_block=w.q_block,
                          cu_seqlens_host=[int(c) for c in case.cu_seqlens])
    o.data.mul_(1.0)          # no version bump: allowed
    with torch.no_grad():
        o.mul_(2.0)           # a real in-place edit
    with pytest.raises(RuntimeError, match="modified by an inplace operation"):
        o.backward(torch.from_numpy(case.dO).to(torch.bfloat16).cuda())
