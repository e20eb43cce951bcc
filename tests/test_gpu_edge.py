"""GPU parity on the method's degenerate cases, through the C ABI against the
oracle: top-k of 1 (only the forced blocks), documents of one token and
shorter than a query block, a window wider than most documents, a dilated
window whose stride skips whole documents' worth of blocks, the shared proxy
head in fp32, a batch whose every document but one is empty, KV-major
work-item counts that do not divide evenly over the per-XCD queues, and two
heads per group with long inverted lists."""
import pytest

from msa_inputs import WORKLOADS
from tests.gpu_common import cfgs, check_inverse, full_compare, log, run_gpu, small_case

pytestmark = pytest.mark.gpu

CASES = {
    "topk1": (WORKLOADS["layer-32k"], dict(topk=1), (1300, 700)),
    "topk1-window": (WORKLOADS["layer-512k-window2"], dict(topk=1), (1500, 90)),
    "tiny-docs": (WORKLOADS["layer-32k"], dict(topk=2), (1, 63, 64, 65, 127, 128, 129, 1)),
    "wide-window": (WORKLOADS["layer-512k-window2"], dict(topk=2, local_window=6), (2000, 300, 900)),
    "dilated-wide": (WORKLOADS["layer-32k"], dict(topk=3, local_window=3, dilation=5), (3000, 640)),
    "shared-fp32": (WORKLOADS["tiny-2k-fp32"], dict(topk=3, proxy_heads=1, local_window=1), (1500, 600)),
    "one-nonempty": (WORKLOADS["layer-32k"], dict(topk=3), (0, 0, 1900, 0)),
    # KV-major work queue with a (group, KV block) count that is not a multiple
    # of the eight queues (57 and 125 items: uneven queues, the later ones
    # drained by stealing), fewer items than compute units, G = 4 and 8
    "queue-uneven-g4": (WORKLOADS["layer-32k"], dict(heads_q=12, heads_kv=3, topk=3), (700, 1300, 129)),
    "queue-uneven-g8": (WORKLOADS["layer-128k-gqa8"], dict(heads_q=40, heads_kv=5, topk=3), (900, 2100)),
    "queue-uneven-g2": (WORKLOADS["layer-32k"], dict(heads_q=6, heads_kv=3, topk=3), (700, 1300, 129)),
    # G = 2 in the two-role KV-major kernel: a chunk's qp rows cycle through
    # three ring slots; long lists (up to 47 entries) wrap the ring many times
    "g2-long-lists": (WORKLOADS["layer-512k-window2"], dict(heads_q=16, topk=8), (6000,)),
}


@pytest.mark.parametrize("name", list(CASES))
def test_edge_parity(name):
    w0, over, seqlens = CASES[name]
    w, cfg, ocfg = cfgs(w0, **over)
    case = small_case(w, seqlens, seed=11)
    log(f"[{name}] T={sum(seqlens)} docs={seqlens}")
    res = run_gpu(case, cfg, backward=True)
    check_inverse(res, ocfg)
    full_compare(case, res, ocfg, tag=name)
