"""MI355X-native MiniMax Sparse Attention (MSA) training hot path.

Proxy-head block scoring with max-pooling, top-k block selection, sparse GQA
forward and the fused main + proxy backward, as hand-written HIP kernels for
gfx950 behind the C ABI in include/msa.h (libmsa.so).  This package is the
thin Python binding: argument marshalling over that ABI, with torch used for
device memory and streams.
"""
from ._lib import EXPORTS, LIB_PATH, MsaError, load  # noqa: F401
from .ops import (Buffers, Config, Varlen, kernel_resources, msa_bwd, msa_fwd,  # noqa: F401
                  msa_get_layout, msa_proxy_scores, msa_select_blocks, msa_select_blocks_noalloc,
                  profile_collect,
                  profile_enable, run_backward, run_forward)
from .attention import msa_attention  # noqa: F401
