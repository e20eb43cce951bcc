"""The FLOP model bench.py prices the path with: its selected-pair count
equals a brute-force count of the causal (query, key) pairs inside the
oracle's block lists."""
import numpy as np
import pytest

import bench
from oracle import msa_oracle as om


@pytest.mark.parametrize("seqlens,q_block,topk,w,dil", [((1000, 300, 2000), 64, 4, 0, 1),
                                                        ((3000, 129), 128, 3, 2, 1),
                                                        ((2600, 700), 64, 3, 2, 3),
                                                        ((1500,), 128, 40, 0, 1)])
def test_selected_pairs_counts_the_lists(seqlens, q_block, topk, w, dil):
    cfg = om.Config(2, 1, 8, 4, q_block, topk, w, dilation=dil)
    cu = np.concatenate([[0], np.cumsum(seqlens)])
    rng = np.random.default_rng(5)
    _, _, ns = om.totals(om.doc_grid(cu, cfg))
    idx, cnt = om.select_blocks(rng.standard_normal((1, ns)), cu, cfg)
    pairs = 0
    for d in om.doc_grid(cu, cfg):
        for I in range(d.nq):
            for t in range(I * q_block, min((I + 1) * q_block, d.length)):
                for KB in idx[0, d.qb0 + I, :cnt[0, d.qb0 + I]]:
                    J = int(KB) - d.kb0
                    pairs += max(0, min(t + 1, (J + 1) * 128, d.length) - J * 128)
    assert bench.selected_pairs(seqlens, q_block, topk, w, dil) == pairs
