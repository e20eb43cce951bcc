"""PyTorch drop-in for MSA attention (the pages' user-facing form is a
PyTorch drop-in API: keelcrux "Flash-MSA: Ein Training mit einer Million
Tokens", Under the hood).

``msa_attention`` returns O and, through autograd, gradients for q, k, v and
for the proxy inputs qp, kp.  The proxy gradient is that of the distillation
KL between the group-mean main attention (held constant) and the proxy
softmax over the selected keys, weighted by ``proxy_loss_weight``; it is
delivered alongside the main gradients by the fused backward.
"""
from __future__ import annotations

from typing import Optional, Sequence

import torch

from .ops import Buffers, Config, Varlen, run_backward, run_forward


class _MSAFunction(torch.autograd.Function):
    @staticmethod
    def forward(ctx, q, k, v, qp, kp, cfg: Config, vl: Varlen):
        q, k, v, qp, kp = (t.contiguous() for t in (q, k, v, qp, kp))
        buf = Buffers(cfg, vl, device=q.device, need_bwd=False)
        run_forward(cfg, vl, q, k, v, qp, kp, buf)
        # keep O, the LSEs and the block lists; scores and workspace are
        # released once the stream has consumed them (the caching allocator
        # reuses them only for work ordered after this point on the stream)
        buf.release_transients()
        ctx.cfg, ctx.vl, ctx.buf = cfg, vl, buf
        # O is saved like the inputs, so that an in-place change of the
        # returned output is caught by autograd's version check
        ctx.save_for_backward(q, k, v, qp, kp, buf.o)
        return buf.o

    @staticmethod
    def backward(ctx, dout):
        q, k, v, qp, kp, o = ctx.saved_tensors
        buf = ctx.buf
        buf.o = o
        buf.alloc_backward()
        run_backward(ctx.cfg, ctx.vl, q, k, v, qp, kp, dout.contiguous().to(q.dtype), buf)
        dt = q.dtype
        grads = (buf.dq.to(dt), buf.dk.to(dt), buf.dv.to(dt), buf.dqp.to(dt), buf.dkp.to(dt))
        ctx.buf = None
        return grads + (None, None)


def msa_attention(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, qp: torch.Tensor,
                  kp: torch.Tensor, cu_seqlens: torch.Tensor, *, topk: int, q_block: int = 128,
                  local_window: int = 0, softmax_scale: Optional[float] = None,
                  proxy_scale: Optional[float] = None, proxy_loss_weight: float = 1.0,
                  cu_seqlens_host: Optional[Sequence[int]] = None, dense: bool = False,
                  dilation: int = 1, proxy_heads: int = 0):
    """Block-sparse GQA attention with proxy-head block selection.

    q [T, Hq, d]; k, v [T, Hkv, d]; qp, kp [T, Hp, dp]; cu_seqlens int32 [B+1].
    Hp = Hkv (one proxy head per KV group, ``proxy_heads=0``) or 1 (one proxy
    head shared by every group, ``proxy_heads=1``).
    ``dense=True`` selects every causal block (top-k = all blocks; window and
    dilation are then moot).  ``dilation`` spaces the forced window blocks (1 = contiguous window).
    """
    T, Hq, d = q.shape
    Hkv, dp = k.shape[1], qp.shape[2]
    vl = Varlen(cu_seqlens.to(torch.int32), cu_seqlens_host)
    if dense:
        longest = max(int(vl.host[i + 1] - vl.host[i]) for i in range(vl.batch)) if vl.batch else 0
        topk = max(1, -(-longest // 128))
        local_window, dilation = 0, 1           # every block up to the diagonal
    cfg = Config(Hq, Hkv, d, dp, q_block, topk, local_window, 128, softmax_scale or 0.0,
                 proxy_scale or 0.0, proxy_loss_weight,
                 "bf16" if q.dtype == torch.bfloat16 else "f32", dilation, proxy_heads)
    return _MSAFunction.apply(q, k, v, qp, kp, cfg, vl)
