"""Python face of the C ABI: the same entry points, taking torch tensors.

Each function checks devices, dtypes, shapes and contiguity, then passes raw
pointers and the current HIP stream to libmsa.so.  No computation happens
here.
"""
from __future__ import annotations

import ctypes
from dataclasses import dataclass
from typing import Optional, Sequence

import numpy as np
import torch

from . import _lib
from ._lib import MsaConfig, MsaLayout, MsaVarlen, check, load


@dataclass(frozen=True)
class Config:
    """Mirror of ``msa_config``.  Scales of 0 mean 1/sqrt(d) and 1/sqrt(dp)."""
    heads_q: int
    heads_kv: int
    head_dim: int
    proxy_dim: int
    q_block: int
    topk: int
    local_window: int = 0
    kv_block: int = 128
    softmax_scale: float = 0.0
    proxy_scale: float = 0.0
    proxy_loss_weight: float = 1.0
    dtype: str = "bf16"
    dilation: int = 1
    proxy_heads: int = 0       # 0 = one proxy head per KV group; 1 = one shared proxy head

    def to_c(self) -> MsaConfig:
        return MsaConfig(self.heads_q, self.heads_kv, self.head_dim, self.proxy_dim, self.kv_block,
                         self.q_block, self.topk, self.local_window, self.softmax_scale,
                         self.proxy_scale, self.proxy_loss_weight,
                         _lib.MSA_BF16 if self.dtype == "bf16" else _lib.MSA_F32, self.dilation,
                         self.proxy_heads)

    @property
    def torch_dtype(self):
        return torch.bfloat16 if self.dtype == "bf16" else torch.float32


class Varlen:
    """cu_seqlens on the device plus the host copy the library reads for sizes."""

    def __init__(self, cu_seqlens: torch.Tensor, cu_seqlens_host: Optional[Sequence[int]] = None):
        if cu_seqlens.dtype != torch.int32:
            raise ValueError("cu_seqlens must be int32")
        self.cu = cu_seqlens.contiguous()
        host = cu_seqlens.cpu().numpy() if cu_seqlens_host is None else cu_seqlens_host
        self.host = np.ascontiguousarray(np.asarray(host, dtype=np.int32))
        self.batch = len(self.host) - 1
        self.total = int(self.host[-1]) if len(self.host) else 0

    def to_c(self) -> MsaVarlen:
        ptr = self.host.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))
        dev = self.cu.data_ptr() if self.cu.is_cuda else None
        return MsaVarlen(dev, ptr, self.batch, self.total)


def _stream(stream) -> Optional[int]:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def _ptr(t: Optional[torch.Tensor], name: str, dtype=None, shape=None):
    if t is None:
        raise ValueError(f"{name} is required")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    return t.data_ptr()


def msa_get_layout(cfg: Config, vl: Varlen) -> dict:
    lib = load()
    out = MsaLayout()
    c, v = cfg.to_c(), vl.to_c()
    check(lib.msa_get_layout(ctypes.byref(c), ctypes.byref(v), ctypes.byref(out)))
    return out.as_dict()


def msa_proxy_scores(cfg: Config, vl: Varlen, qp, kp, block_scores, workspace, stream=None):
    lib = load()
    lay = msa_get_layout(cfg, vl)
    T, Hp, dp = vl.total, lay["proxy_heads"], cfg.proxy_dim
    dt = cfg.torch_dtype
    a = [_ptr(qp, "qp", dt, (T, Hp, dp)), _ptr(kp, "kp", dt, (T, Hp, dp)),
         _ptr(block_scores, "block_scores", torch.float32, (Hp, lay["score_elems"])),
         _ptr(workspace, "workspace", torch.uint8)]
    c, v = cfg.to_c(), vl.to_c()
    check(lib.msa_proxy_scores(ctypes.byref(c), ctypes.byref(v), a[0], a[1], a[2], a[3],
                               workspace.numel(), _stream(stream)))


def msa_select_blocks(cfg: Config, vl: Varlen, block_scores, q2k_idx, q2k_cnt, k2q_ptr, k2q_idx,
                      workspace, stream=None):
    lib = load()
    lay = msa_get_layout(cfg, vl)
    Hp = lay["proxy_heads"]
    i32 = torch.int32
    a = [_ptr(block_scores, "block_scores", torch.float32, (Hp, lay["score_elems"])),
         _ptr(q2k_idx, "q2k_idx", i32, (Hp, lay["total_qblocks"], lay["sel_stride"])),
         _ptr(q2k_cnt, "q2k_cnt", i32, (Hp, lay["total_qblocks"])),
         _ptr(k2q_ptr, "k2q_ptr", i32, (Hp, lay["total_kvblocks"] + 1)),
         _ptr(k2q_idx, "k2q_idx", i32, (Hp, lay["k2q_capacity"])),
         _ptr(workspace, "workspace", torch.uint8)]
    c, v = cfg.to_c(), vl.to_c()
    check(lib.msa_select_blocks(ctypes.byref(c), ctypes.byref(v), *a, workspace.numel(),
                                _stream(stream)))


def msa_select_blocks_noalloc(cfg: Config, vl: Varlen, block_scores, q2k_idx, q2k_cnt, k2q_ptr, k2q_idx,
                              stream=None):
    """msa_select_blocks with the library's static scratch instead of a
    workspace (no device allocation); calls on one GPU must not overlap."""
    lib = load()
    lay = msa_get_layout(cfg, vl)
    Hp = lay["proxy_heads"]
    i32 = torch.int32
    a = [_ptr(block_scores, "block_scores", torch.float32, (Hp, lay["score_elems"])),
         _ptr(q2k_idx, "q2k_idx", i32, (Hp, lay["total_qblocks"], lay["sel_stride"])),
         _ptr(q2k_cnt, "q2k_cnt", i32, (Hp, lay["total_qblocks"])),
         _ptr(k2q_ptr, "k2q_ptr", i32, (Hp, lay["total_kvblocks"] + 1)),
         _ptr(k2q_idx, "k2q_idx", i32, (Hp, lay["k2q_capacity"]))]
    c, v = cfg.to_c(), vl.to_c()
    check(lib.msa_select_blocks_noalloc(ctypes.byref(c), ctypes.byref(v), *a, _stream(stream)))


def msa_fwd(cfg: Config, vl: Varlen, q, k, v, qp, kp, q2k_idx, q2k_cnt, o, lse, lse_p, workspace,
            stream=None):
    lib = load()
    lay = msa_get_layout(cfg, vl)
    T, Hq, Hkv, d, dp = vl.total, cfg.heads_q, cfg.heads_kv, cfg.head_dim, cfg.proxy_dim
    Hp = lay["proxy_heads"]
    dt, i32, f32 = cfg.torch_dtype, torch.int32, torch.float32
    a = [_ptr(q, "q", dt, (T, Hq, d)), _ptr(k, "k", dt, (T, Hkv, d)), _ptr(v, "v", dt, (T, Hkv, d)),
         _ptr(qp, "qp", dt, (T, Hp, dp)), _ptr(kp, "kp", dt, (T, Hp, dp)),
         _ptr(q2k_idx, "q2k_idx", i32, (Hp, lay["total_qblocks"], lay["sel_stride"])),
         _ptr(q2k_cnt, "q2k_cnt", i32, (Hp, lay["total_qblocks"])),
         _ptr(o, "o", dt, (T, Hq, d)), _ptr(lse, "lse", f32, (Hq, T)),
         _ptr(lse_p, "lse_p", f32, (Hp, T)), _ptr(workspace, "workspace", torch.uint8)]
    c, vv = cfg.to_c(), vl.to_c()
    check(lib.msa_fwd(ctypes.byref(c), ctypes.byref(vv), *a, workspace.numel(), _stream(stream)))


def msa_bwd(cfg: Config, vl: Varlen, q, k, v, qp, kp, o, lse, lse_p, dout, q2k_idx, q2k_cnt,
            k2q_ptr, k2q_idx, dq, dk, dv, dqp, dkp, workspace, stream=None):
    lib = load()
    lay = msa_get_layout(cfg, vl)
    T, Hq, Hkv, d, dp = vl.total, cfg.heads_q, cfg.heads_kv, cfg.head_dim, cfg.proxy_dim
    Hp = lay["proxy_heads"]
    dt, i32, f32 = cfg.torch_dtype, torch.int32, torch.float32
    a = [_ptr(q, "q", dt, (T, Hq, d)), _ptr(k, "k", dt, (T, Hkv, d)), _ptr(v, "v", dt, (T, Hkv, d)),
         _ptr(qp, "qp", dt, (T, Hp, dp)), _ptr(kp, "kp", dt, (T, Hp, dp)),
         _ptr(o, "o", dt, (T, Hq, d)), _ptr(lse, "lse", f32, (Hq, T)),
         _ptr(lse_p, "lse_p", f32, (Hp, T)), _ptr(dout, "dout", dt, (T, Hq, d)),
         _ptr(q2k_idx, "q2k_idx", i32, (Hp, lay["total_qblocks"], lay["sel_stride"])),
         _ptr(q2k_cnt, "q2k_cnt", i32, (Hp, lay["total_qblocks"])),
         _ptr(k2q_ptr, "k2q_ptr", i32, (Hp, lay["total_kvblocks"] + 1)),
         _ptr(k2q_idx, "k2q_idx", i32, (Hp, lay["k2q_capacity"])),
         _ptr(dq, "dq", f32, (T, Hq, d)), _ptr(dk, "dk", f32, (T, Hkv, d)),
         _ptr(dv, "dv", f32, (T, Hkv, d)), _ptr(dqp, "dqp", f32, (T, Hp, dp)),
         _ptr(dkp, "dkp", f32, (T, Hp, dp)), _ptr(workspace, "workspace", torch.uint8)]
    c, vv = cfg.to_c(), vl.to_c()
    check(lib.msa_bwd(ctypes.byref(c), ctypes.byref(vv), *a, workspace.numel(), _stream(stream)))


def kernel_resources() -> list:
    """Per-kernel VGPRs, LDS bytes, scratch bytes and resident workgroups per CU (needs a GPU)."""
    lib = load()
    out = []
    for i in range(lib.msa_kernel_count()):
        name = ctypes.create_string_buffer(96)
        regs, lds, scr, occ = (ctypes.c_int32() for _ in range(4))
        check(lib.msa_kernel_info(i, name, 96, ctypes.byref(regs), ctypes.byref(lds),
                                  ctypes.byref(scr), ctypes.byref(occ)))
        out.append(dict(name=name.value.decode(), vgprs=regs.value, lds_bytes=lds.value,
                        scratch_bytes=scr.value, workgroups_per_cu=occ.value))
    return out


def profile_enable(on: bool = True) -> None:
    """Start (or stop) per-kernel HIP-event timing on this thread."""
    check(load().msa_profile_enable(1 if on else 0))


def profile_collect() -> dict:
    """Wait for the recorded events; {kernel name: (total ms, launches)}; clears the record."""
    lib = load()
    n = lib.msa_profile_collect()
    out = {}
    for i in range(n):
        name = ctypes.create_string_buffer(64)
        ms, cnt = ctypes.c_double(), ctypes.c_int64()
        check(lib.msa_profile_entry(i, name, 64, ctypes.byref(ms), ctypes.byref(cnt)))
        out[name.value.decode()] = (ms.value, cnt.value)
    return out


class Buffers:
    """Every device buffer of one layer call, allocated once with torch."""

    def __init__(self, cfg: Config, vl: Varlen, device="cuda", need_bwd: bool = True):
        lay = msa_get_layout(cfg, vl)
        self.layout = lay
        T, Hq, Hkv, d, dp = vl.total, cfg.heads_q, cfg.heads_kv, cfg.head_dim, cfg.proxy_dim
        Hp = lay["proxy_heads"]
        i32, f32 = torch.int32, torch.float32
        z = dict(device=device)
        self.workspace = torch.empty(max(lay["workspace_bytes"], 16), dtype=torch.uint8, **z)
        self.scores = torch.empty((Hp, max(lay["score_elems"], 1)), dtype=f32, **z)[:, :lay["score_elems"]]
        if lay["score_elems"] == 0:
            self.scores = torch.empty((Hp, 0), dtype=f32, **z)
        self.q2k_idx = torch.empty((Hp, lay["total_qblocks"], lay["sel_stride"]), dtype=i32, **z)
        self.q2k_cnt = torch.empty((Hp, lay["total_qblocks"]), dtype=i32, **z)
        self.k2q_ptr = torch.empty((Hp, lay["total_kvblocks"] + 1), dtype=i32, **z)
        self.k2q_idx = torch.empty((Hp, lay["k2q_capacity"]), dtype=i32, **z)
        self.o = torch.empty((T, Hq, d), dtype=cfg.torch_dtype, **z)
        self.lse = torch.empty((Hq, T), dtype=f32, **z)
        self.lse_p = torch.empty((Hp, T), dtype=f32, **z)
        self._shape = (T, Hq, Hkv, Hp, d, dp, device)
        if need_bwd:
            self.alloc_backward()

    def alloc_backward(self):
        """The gradient outputs (fp32) and, if released, the workspace."""
        T, Hq, Hkv, Hp, d, dp, device = self._shape
        f32, z = torch.float32, dict(device=device)
        if getattr(self, "workspace", None) is None:
            self.workspace = torch.empty(max(self.layout["workspace_bytes"], 16), dtype=torch.uint8, **z)
        self.dq = torch.empty((T, Hq, d), dtype=f32, **z)
        self.dk = torch.empty((T, Hkv, d), dtype=f32, **z)
        self.dv = torch.empty((T, Hkv, d), dtype=f32, **z)
        self.dqp = torch.empty((T, Hp, dp), dtype=f32, **z)
        self.dkp = torch.empty((T, Hp, dp), dtype=f32, **z)

    def release_transients(self):
        """Drop what the backward does not read: the block scores and the
        workspace (every call rebuilds its tables; the backward's per-query
        vectors are written in the backward itself)."""
        self.scores = None
        self.workspace = None

    def saved_bytes(self) -> dict:
        """Bytes kept from the forward for the backward, besides the inputs."""
        out = {}
        for n in ("o", "lse", "lse_p", "q2k_idx", "q2k_cnt", "k2q_ptr", "k2q_idx"):
            t = getattr(self, n)
            out[n] = t.numel() * t.element_size()
        return out


def run_forward(cfg: Config, vl: Varlen, q, k, v, qp, kp, buf: Buffers, stream=None):
    """proxy scores -> selection (+ inverted index) -> sparse forward."""
    msa_proxy_scores(cfg, vl, qp, kp, buf.scores, buf.workspace, stream)
    msa_select_blocks(cfg, vl, buf.scores, buf.q2k_idx, buf.q2k_cnt, buf.k2q_ptr, buf.k2q_idx,
                      buf.workspace, stream)
    msa_fwd(cfg, vl, q, k, v, qp, kp, buf.q2k_idx, buf.q2k_cnt, buf.o, buf.lse, buf.lse_p,
            buf.workspace, stream)


def run_backward(cfg: Config, vl: Varlen, q, k, v, qp, kp, dout, buf: Buffers, stream=None):
    msa_bwd(cfg, vl, q, k, v, qp, kp, buf.o, buf.lse, buf.lse_p, dout, buf.q2k_idx, buf.q2k_cnt,
            buf.k2q_ptr, buf.k2q_idx, buf.dq, buf.dk, buf.dv, buf.dqp, buf.dkp, buf.workspace, stream)
