"""Build libmsa.so (the HIP kernels and the C ABI) for gfx950, in-tree.

    python -m block_sparse_attention_proxy_amd.build [--jobs N] [--resource-report FILE]

Each translation unit is compiled with hipcc in parallel, then linked into
``block_sparse_attention_proxy_amd/libmsa.so``.  With ``--resource-report``
the compiler's per-kernel resource usage (VGPR, AGPR, SGPR, LDS, scratch,
occupancy) is written to FILE.
"""
from __future__ import annotations

import argparse
import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libmsa.so")
SOURCES = ["select.hip", "attn_fwd.hip", "attn_bwd.hip", "attn_bwd_kv.hip", "attn_bwd_q.hip", "proxy_share.hip", "msa_api.cpp"]
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (set HIPCC or install ROCm)")


def common_flags():
    return [f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-function",
            "-Wno-unused-variable", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            f"-I{os.path.join(os.path.dirname(PKG), 'include')}"]


def _compile(src: str, report: bool):
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    cmd = [hipcc()] + common_flags() + ["-c", os.path.join(CSRC, src), "-o", obj]
    if report and src.endswith(".hip"):
        cmd += ["-Rpass-analysis=kernel-resource-usage"]
    p = subprocess.run(cmd, capture_output=True, text=True)
    if p.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{p.stderr[-8000:]}")
    return obj, p.stderr


def build(jobs: int = 4, resource_report: str | None = None, verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    with ThreadPoolExecutor(max_workers=max(1, jobs)) as ex:
        results = list(ex.map(lambda s: _compile(s, resource_report is not None), SOURCES))
    objs = [r[0] for r in results]
    tmp = LIB + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp] + objs
    p = subprocess.run(cmd, capture_output=True, text=True)
    if p.returncode != 0:
        raise RuntimeError(f"link failed:\n{p.stderr[-8000:]}")
    os.replace(tmp, LIB)
    if resource_report:
        lines = []
        for src, (_, err) in zip(SOURCES, results):
            for ln in err.splitlines():
                if "remark:" in ln and ("Function Name" in ln or "VGPRs" in ln or "AGPRs" in ln
                                        or "ScratchSize" in ln or "Occupancy" in ln or "LDS Size" in ln
                                        or "SGPRs:" in ln):
                    lines.append(ln.split("remark: ", 1)[-1])
        with open(resource_report, "w") as f:
            f.write("\n".join(lines) + "\n")
    if verbose:
        for src, (_, err) in zip(SOURCES, results):
            warn = [l for l in err.splitlines() if "warning" in l and "packed-fp32-ops" not in l]
            if warn:
                print(f"{src}: {len(warn)} warnings", file=sys.stderr)
                print("\n".join(warn[:20]), file=sys.stderr)
    return LIB


def main(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("--jobs", type=int, default=4)
    ap.add_argument("--resource-report", default=None)
    a = ap.parse_args(argv)
    print(build(a.jobs, a.resource_report, verbose=True))


if __name__ == "__main__":
    main()
