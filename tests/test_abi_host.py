"""Host-side checks of the C ABI (no GPU needed): the library loads, exports
every symbol include/msa.h declares, computes layouts that agree with the
oracle's block grid, and rejects bad arguments before any launch."""
import ctypes
import os
import re

import numpy as np
import pytest
import torch

import block_sparse_attention_proxy_amd as msa
from block_sparse_attention_proxy_amd import _lib
from oracle import msa_oracle as om

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_exports_match_header():
    lib = msa.load()
    header = open(os.path.join(ROOT, "include", "msa.h")).read()
    declared = set(re.findall(r"\b(msa_[a-z_]+)\s*\(", header))
    assert declared == set(_lib.EXPORTS)
    for name in declared:
        assert hasattr(lib, name), name
    assert lib.msa_abi_version() == 1
    assert lib.msa_status_string(0).decode() == "ok"


@pytest.mark.parametrize("seqlens,q_block,topk,w", [((2048,), 64, 4, 0), ((3000, 0, 129, 5000), 128, 3, 2),
                                                    ((32768,), 64, 16, 0), ((700, 64, 1), 64, 1, 0)])
def test_layout_matches_oracle_grid(seqlens, q_block, topk, w):
    cu = np.concatenate([[0], np.cumsum(seqlens)]).astype(np.int32)
    cfg = msa.Config(8, 2, 64, 32, q_block, topk, w, dtype="f32")
    lay = msa.msa_get_layout(cfg, msa.Varlen(torch.from_numpy(cu)))
    ocfg = om.Config(8, 2, 64, 32, q_block, topk, w)
    docs = om.doc_grid(cu, ocfg)
    nqb, nkb, ns = om.totals(docs)
    assert lay["total_qblocks"] == nqb and lay["total_kvblocks"] == nkb and lay["score_elems"] == ns
    assert lay["sel_stride"] == topk + w and lay["k2q_capacity"] == nqb * (topk + w)
    pairs = 0
    for d in docs:
        for I in range(d.nq):
            rows = min(q_block, d.length - I * q_block)
            pairs += rows * om.candidate_count(I, ocfg) * 128
    assert lay["scored_pairs"] == pairs
    assert lay["max_qblocks_doc"] == max(d.nq for d in docs)
    assert lay["workspace_bytes"] > 0


def _err(fn):
    with pytest.raises(msa.MsaError) as e:
        fn()
    return e.value


@pytest.mark.parametrize("kw,status", [
    (dict(heads_q=12, heads_kv=8), _lib.MSA_ERR_INVALID_ARG),
    (dict(head_dim=96), _lib.MSA_ERR_UNSUPPORTED),
    (dict(q_block=32), _lib.MSA_ERR_UNSUPPORTED),
    (dict(kv_block=64), _lib.MSA_ERR_UNSUPPORTED),
    (dict(topk=0), _lib.MSA_ERR_INVALID_ARG),
    (dict(local_window=-1), _lib.MSA_ERR_INVALID_ARG),
    (dict(heads_q=24, heads_kv=4), _lib.MSA_ERR_UNSUPPORTED),   # group of 6
    (dict(dtype="f32"), _lib.MSA_ERR_UNSUPPORTED),              # fp32 only at d = 64
])
def test_config_rejected(kw, status):
    base = dict(heads_q=32, heads_kv=8, head_dim=128, proxy_dim=64, q_block=128, topk=8)
    base.update(kw)
    cfg = msa.Config(**base)
    e = _err(lambda: msa.msa_get_layout(cfg, msa.Varlen(torch.tensor([0, 1000], dtype=torch.int32))))
    assert e.status == status


@pytest.mark.parametrize("cu,msg", [([1, 100], "cu_seqlens\\[0\\]"), ([0, 100, 50], "decreases"),
                                    ([0], "batch")])
def test_bad_cu_seqlens(cu, msg):
    cfg = msa.Config(8, 2, 64, 32, 64, 4, dtype="f32")
    e = _err(lambda: msa.msa_get_layout(cfg, msa.Varlen(torch.tensor(cu, dtype=torch.int32))))
    assert e.status == _lib.MSA_ERR_INVALID_ARG and re.search(msg, str(e))


def test_total_tokens_mismatch_and_nulls():
    lib = msa.load()
    cfg = msa.Config(8, 2, 64, 32, 64, 4, dtype="f32").to_c()
    host = np.array([0, 500], dtype=np.int32)
    vl = _lib.MsaVarlen(None, host.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)), 1, 499)
    lay = _lib.MsaLayout()
    assert lib.msa_get_layout(ctypes.byref(cfg), ctypes.byref(vl), ctypes.byref(lay)) == _lib.MSA_ERR_INVALID_ARG
    assert b"total_tokens" in lib.msa_last_error()
    vl.total_tokens = 500
    # null tensors are refused on the host, before any HIP call
    st = lib.msa_fwd(ctypes.byref(cfg), ctypes.byref(vl), *([None] * 10), None, 0, None)
    assert st == _lib.MSA_ERR_INVALID_ARG and b"must be non-null" in lib.msa_last_error()
    st = lib.msa_bwd(ctypes.byref(cfg), ctypes.byref(vl), *([None] * 18), None, 0, None)
    assert st == _lib.MSA_ERR_INVALID_ARG
    # a misaligned pointer
    bogus = 16 * 1024 + 4
    st = lib.msa_proxy_scores(ctypes.byref(cfg), ctypes.byref(vl), bogus, 16 * 1024, 16 * 1024,
                              16 * 1024, 1 << 20, None)
    assert st == _lib.MSA_ERR_INVALID_ARG and b"aligned" in lib.msa_last_error()
    # a workspace that is too small
    st = lib.msa_proxy_scores(ctypes.byref(cfg), ctypes.byref(vl), 16 * 1024, 16 * 1024, 16 * 1024,
                              16 * 1024, 16, None)
    assert st == _lib.MSA_ERR_WORKSPACE


def test_python_wrappers_check_tensors():
    cfg = msa.Config(8, 2, 64, 32, 64, 4, dtype="f32")
    vl = msa.Varlen(torch.tensor([0, 256], dtype=torch.int32))
    cpu = torch.zeros(256, 2, 32)
    with pytest.raises(ValueError, match="device tensor"):
        msa.msa_proxy_scores(cfg, vl, cpu, cpu, torch.zeros(2, 4), torch.zeros(16, dtype=torch.uint8))
