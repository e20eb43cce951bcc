"""GPU check of the allocation-free selection entry point: through the C ABI,
msa_select_blocks_noalloc gives the same block lists and inverted index, bit
for bit, as msa_select_blocks with a workspace, on two calls in a row (the
second with a smaller packing, which must not see the first call's counters),
and on a shared proxy head."""
import numpy as np
import pytest
import torch

import block_sparse_attention_proxy_amd as msa
from msa_inputs import WORKLOADS
from tests.gpu_common import cfgs, log, small_case

pytestmark = pytest.mark.gpu


def _select_both(case, cfg):
    dt = torch.bfloat16 if cfg.dtype == "bf16" else torch.float32
    qp = torch.from_numpy(case.qp).to(dt).cuda()
    kp = torch.from_numpy(case.kp).to(dt).cuda()
    vl = msa.Varlen(torch.from_numpy(case.cu_seqlens).cuda(), case.cu_seqlens)
    ref = msa.Buffers(cfg, vl, device="cuda", need_bwd=False)
    msa.msa_proxy_scores(cfg, vl, qp, kp, ref.scores, ref.workspace)
    msa.msa_select_blocks(cfg, vl, ref.scores, ref.q2k_idx, ref.q2k_cnt, ref.k2q_ptr, ref.k2q_idx,
                          ref.workspace)
    # outputs of the allocation-free call, pre-filled with garbage
    got = {n: torch.full_like(getattr(ref, n), -7) for n in ("q2k_idx", "q2k_cnt", "k2q_ptr", "k2q_idx")}
    msa.msa_select_blocks_noalloc(cfg, vl, ref.scores, got["q2k_idx"], got["q2k_cnt"], got["k2q_ptr"],
                                  got["k2q_idx"])
    torch.cuda.synchronize()
    for n in got:
        a, b = getattr(ref, n).cpu().numpy(), got[n].cpu().numpy()
        assert np.array_equal(a, b), n
    return ref


@pytest.mark.parametrize("name,over", [("layer-32k", dict(topk=4)),
                                       ("layer-512k-window2", dict(topk=3)),
                                       ("layer-32k", dict(topk=4, proxy_heads=1))])
def test_select_noalloc_equals_workspace_path(name, over):
    w, cfg, _ = cfgs(WORKLOADS[name], **over)
    big = small_case(w, (5000, 77, 3100, 0, 900), seed=41)
    small = small_case(w, (1300, 200), seed=42)
    log(f"[{name} {over}] first call: T={sum(big.seqlens)}")
    r1 = _select_both(big, cfg)
    log(f"[{name} {over}] second call, smaller: T={sum(small.seqlens)}")
    r2 = _select_both(small, cfg)
    assert r1.k2q_ptr.shape[1] > r2.k2q_ptr.shape[1]
