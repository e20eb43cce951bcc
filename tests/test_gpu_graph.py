"""The whole training step -- proxy scores, selection with the inverted index,
forward, fused backward -- captured in a HIP graph (torch.cuda.graph) and
replayed: every replay must give the eager results bit for bit.  The
persistent kernels clear their work-queue counters with a kernel of their
own (no memset node), so the graph can be replayed any number of times.
Outputs are overwritten with garbage between replays, with eager work and
synchronisations in between, so a replay that skipped or reused anything
would show."""
import numpy as np
import pytest
import torch

import block_sparse_attention_proxy_amd as msa
from msa_inputs import WORKLOADS
from tests.gpu_common import cfgs, device_inputs, log, small_case

pytestmark = pytest.mark.gpu

OUTS = ("scores", "q2k_idx", "q2k_cnt", "k2q_ptr", "k2q_idx", "o", "lse", "lse_p",
        "dq", "dk", "dv", "dqp", "dkp")


def _step(cfg, vl, x, buf):
    msa.run_forward(cfg, vl, x["q"], x["k"], x["v"], x["qp"], x["kp"], buf)
    msa.run_backward(cfg, vl, x["q"], x["k"], x["v"], x["qp"], x["kp"], x["dO"], buf)


def _garbage(buf):
    for n in OUTS:
        t = getattr(buf, n)
        if t.dtype.is_floating_point:
            t.fill_(float("nan"))
        else:
            t.fill_(-7)


@pytest.mark.parametrize("name,over,seqlens", [
    ("layer-32k", dict(topk=4), (3000, 1300, 129)),                # G = 4, q_block 64
    ("layer-128k-gqa8", dict(topk=3, proxy_heads=1), (2100, 900)),  # G = 8, shared proxy head
])
def test_step_graph_replay(name, over, seqlens):
    w, cfg, _ = cfgs(WORKLOADS[name], **over)
    case = small_case(w, seqlens, seed=5)
    log(f"[graph {name}] T={sum(seqlens)} docs={seqlens}")
    x = device_inputs(case, cfg.dtype)
    vl = msa.Varlen(x["cu"], case.cu_seqlens)
    buf = msa.Buffers(cfg, vl, device="cuda", need_bwd=True)
    _garbage(buf)                               # score entries the scoring never writes stay NaN
    _step(cfg, vl, x, buf)                      # eager (also raises the LDS limits once)
    torch.cuda.synchronize()
    ref = {n: getattr(buf, n).clone() for n in OUTS}

    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        with torch.cuda.graph(g, stream=side):
            _step(cfg, vl, x, buf)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()

    for rep in range(3):
        _garbage(buf)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for n in OUTS:
            got, want = getattr(buf, n), ref[n]
            same = torch.equal(got, want) if not got.dtype.is_floating_point else \
                bool(torch.equal(torch.nan_to_num(got, nan=1.5), torch.nan_to_num(want, nan=1.5)))
            assert same, f"replay {rep}: {n} differs from the eager step"
        log(f"  replay {rep}: all {len(OUTS)} outputs equal the eager step")
        # eager work between replays
        _step(cfg, vl, x, buf)
        torch.cuda.synchronize()
        for n in ("o", "dk"):
            assert torch.equal(getattr(buf, n), ref[n])
    del g
    np.testing.assert_equal(ref["q2k_cnt"].cpu().numpy().min() >= 1, True)
