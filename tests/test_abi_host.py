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
    assert lib.msa_abi_version() == _lib.ABI_VERSION == 4
    assert ctypes.sizeof(_lib.MsaConfig) == 14 * 4
    assert ctypes.sizeof(_lib.MsaLayout) == 9 * 8
    assert lib.msa_status_string(0).decode() == "ok"


@pytest.mark.parametrize("seqlens,q_block,topk,w,dil", [((2048,), 64, 4, 0, 1), ((3000, 0, 129, 5000), 128, 3, 2, 1),
                                                        ((32768,), 64, 16, 0, 1), ((700, 64, 1), 64, 1, 0, 1),
                                                        ((3000, 0, 129, 5000), 128, 3, 2, 3),
                                                        ((32768,), 64, 16, 4, 2), ((4000,), 64, 2, 1, 0)])
def test_layout_matches_oracle_grid(seqlens, q_block, topk, w, dil):
    cu = np.concatenate([[0], np.cumsum(seqlens)]).astype(np.int32)
    cfg = msa.Config(8, 2, 64, 32, q_block, topk, w, dtype="f32", dilation=dil)
    lay = msa.msa_get_layout(cfg, msa.Varlen(torch.from_numpy(cu)))
    ocfg = om.Config(8, 2, 64, 32, q_block, topk, w, dilation=max(dil, 1))
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
    (dict(dilation=-1), _lib.MSA_ERR_INVALID_ARG),
    (dict(proxy_heads=2), _lib.MSA_ERR_INVALID_ARG),            # neither 1 nor heads_kv
    (dict(local_window=1 << 12, dilation=1 << 9), _lib.MSA_ERR_INVALID_ARG),
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


def test_buffer_lifetimes_and_saved_bytes():
    """The autograd path keeps only O, the LSEs and the block lists from the
    forward; scores and workspace are released, gradients come with the
    backward.  Sizes follow the layout (host-side; CPU tensors stand in)."""
    seqlens = (3000, 129, 5000)
    cu = np.concatenate([[0], np.cumsum(seqlens)]).astype(np.int32)
    T, Hq, Hkv, d, dp = int(cu[-1]), 8, 2, 64, 32
    cfg = msa.Config(Hq, Hkv, d, dp, 128, 3, 2, dtype="bf16")
    buf = msa.Buffers(cfg, msa.Varlen(torch.from_numpy(cu)), device="cpu", need_bwd=False)
    lay = buf.layout
    assert not hasattr(buf, "dq")
    buf.release_transients()
    assert buf.scores is None and buf.workspace is None
    sb = buf.saved_bytes()
    nqb, nkb, st = lay["total_qblocks"], lay["total_kvblocks"], lay["sel_stride"]
    assert sb == {"o": T * Hq * d * 2, "lse": 4 * Hq * T, "lse_p": 4 * Hkv * T,
                  "q2k_idx": 4 * Hkv * nqb * st, "q2k_cnt": 4 * Hkv * nqb,
                  "k2q_ptr": 4 * Hkv * (nkb + 1), "k2q_idx": 4 * Hkv * lay["k2q_capacity"]}
    buf.alloc_backward()
    assert buf.workspace.numel() >= lay["workspace_bytes"]
    assert tuple(buf.dq.shape) == (T, Hq, d) and tuple(buf.dkp.shape) == (T, Hkv, dp)
    assert buf.dq.dtype == torch.float32


@pytest.mark.parametrize("proxy_heads,Hp", [(0, 8), (8, 8), (1, 1)])
def test_layout_proxy_heads(proxy_heads, Hp):
    """Hp leads every per-proxy-head tensor; the shared head adds workspace for
    exactly the per-group proxy gradients (fp32 dqp and dkp per KV group) that
    are averaged into its own; its inputs are read in place, never copied."""
    cu = torch.tensor([0, 3000, 4100], dtype=torch.int32)
    base = msa.msa_get_layout(msa.Config(32, 8, 128, 64, 128, 8), msa.Varlen(cu))
    lay = msa.msa_get_layout(msa.Config(32, 8, 128, 64, 128, 8, proxy_heads=proxy_heads), msa.Varlen(cu))
    assert lay["proxy_heads"] == Hp
    assert {k: v for k, v in lay.items() if k not in ("workspace_bytes", "proxy_heads")} == \
           {k: v for k, v in base.items() if k not in ("workspace_bytes", "proxy_heads")}
    T = 4100
    grads = 2 * 4 * T * 8 * 64                                       # dqp, dkp per group
    if Hp == 1:
        assert base["workspace_bytes"] + grads <= lay["workspace_bytes"] <= base["workspace_bytes"] + grads + 512
    else:
        assert lay["workspace_bytes"] == base["workspace_bytes"]


def test_select_noalloc_rejects_packings_beyond_its_scratch():
    """The allocation-free selection entry point checks its scratch need on the
    host and refuses a packing that does not fit, before anything is launched
    (so this runs without a GPU: the device pointers are never used)."""
    lib = msa.load()
    cap = lib.msa_select_blocks_noalloc_max_bytes()
    assert cap == 16 << 20
    seqlens = [1 << 21] * 16                    # 32M tokens: 2^21 per document
    cu = np.concatenate([[0], np.cumsum(seqlens)]).astype(np.int32)
    cfg = msa.Config(32, 8, 128, 64, 128, 64, 0, dtype="bf16").to_c()
    fake = 1 << 20                              # aligned, never dereferenced
    vl = _lib.MsaVarlen(fake, cu.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)), len(seqlens), int(cu[-1]))
    st = lib.msa_select_blocks_noalloc(ctypes.byref(cfg), ctypes.byref(vl), fake, fake, fake, fake, fake, None)
    assert st == _lib.MSA_ERR_WORKSPACE
    msg = lib.msa_last_error().decode()
    assert "scratch" in msg and str(cap) in msg
    # a small packing passes the host checks up to the first device call
    small = np.array([0, 4096], dtype=np.int32)
    vl2 = _lib.MsaVarlen(fake, small.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)), 1, 4096)
    lay = _lib.MsaLayout()
    assert lib.msa_get_layout(ctypes.byref(cfg), ctypes.byref(vl2), ctypes.byref(lay)) == _lib.MSA_OK
