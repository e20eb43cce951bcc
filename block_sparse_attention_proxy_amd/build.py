"""Build libmsa.so (the HIP kernels and the C ABI) for gfx950, in-tree.

    python -m block_sparse_attention_proxy_amd.build [--jobs N] [--resource-report FILE]

Each translation unit is compiled with hipcc in parallel, then linked into
``block_sparse_attention_proxy_amd/libmsa.so``.  The compiler's per-kernel
resource usage (VGPR, AGPR, SGPR, LDS, scratch, occupancy) is collected on
every build, and the build fails if any kernel uses scratch memory: spill
loads and stores are vector-memory operations that count on the same
``vmcnt`` counter the LDS-copy rings wait on, so a spilling kernel would
serialise its copies (and the compiler, which does not see copies issued
from inline assembly, would wait for its own spill loads with vmcnt(0)).
With ``--resource-report FILE`` the usage is written to FILE as a table.
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
SOURCES = ["select.hip", "attn_fwd.hip", "attn_bwd.hip", "attn_bwd_kv.hip", "attn_bwd_q.hip", "proxy_share.hip", "work_queue.hip", "msa_api.cpp"]
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
    if src.endswith(".hip"):
        cmd += ["-Rpass-analysis=kernel-resource-usage"]
    p = subprocess.run(cmd, capture_output=True, text=True)
    if p.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{p.stderr[-8000:]}")
    return obj, p.stderr


def _drop_params(sig: str) -> str:
    """The name part of a demangled signature: everything before the
    parenthesis that opens its final parameter list."""
    if not sig.endswith(")"):
        return sig
    depth = 0
    for i in range(len(sig) - 1, -1, -1):
        depth += {")": 1, "(": -1}.get(sig[i], 0)
        if depth == 0:
            return sig[:i]
    return sig


def _demangle(names):
    """Kernel names without their parameter lists.  The host c++filt does not
    know the bf16 builtin's mangling (DF16b), so it is renamed to a vendor
    type first (which shifts later substitutions: only the part before the
    parameter list is kept)."""
    try:
        p = subprocess.run(["c++filt"], input="\n".join(n.replace("DF16b", "u6__bf16") for n in names),
                           capture_output=True, text=True)
        out = p.stdout.splitlines()
        if p.returncode == 0 and len(out) == len(names):
            return [_drop_params(o).replace("void ", "", 1) for o in out]
    except OSError:
        pass
    return list(names)


def resource_usage(results):
    """Per-kernel resource usage from the compilers' kernel-resource-usage
    remarks: a list of dicts (source, kernel, sgprs, vgprs, agprs, scratch,
    waves_per_simd, lds_bytes)."""
    keys = {"TotalSGPRs": "sgprs", "VGPRs": "vgprs", "AGPRs": "agprs",
            "ScratchSize [bytes/lane]": "scratch", "Occupancy [waves/SIMD]": "waves_per_simd",
            "LDS Size [bytes/block]": "lds_bytes"}
    rows = []
    for src, (_, err) in zip(SOURCES, results):
        cur = None
        for ln in err.splitlines():
            if "remark:" not in ln or "kernel-resource-usage" not in ln:
                continue
            body = ln.split("remark: ", 1)[-1].split(" [-Rpass-analysis", 1)[0].strip()
            if body.startswith("Function Name:"):
                cur = {"source": src, "kernel": body.split(":", 1)[1].strip()}
                rows.append(cur)
            elif cur is not None and ":" in body:
                k, v = body.rsplit(":", 1)
                if k.strip() in keys:
                    cur[keys[k.strip()]] = int(v.strip())
    for r, dm in zip(rows, _demangle([r["kernel"] for r in rows])):
        r["kernel"] = dm
    return rows


def format_report(rows) -> str:
    lines = ["| source | kernel | VGPRs | AGPRs | SGPRs | LDS bytes (static) | scratch B/lane | waves/SIMD |",
             "|---|---|---:|---:|---:|---:|---:|---:|"]
    for r in rows:
        lines.append(f"| {r['source']} | `{r['kernel']}` | {r.get('vgprs', '')} | {r.get('agprs', '')} | "
                     f"{r.get('sgprs', '')} | {r.get('lds_bytes', '')} | {r.get('scratch', '')} | "
                     f"{r.get('waves_per_simd', '')} |")
    return "\n".join(lines) + "\n"


def build(jobs: int = 4, resource_report: str | None = None, verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    with ThreadPoolExecutor(max_workers=max(1, jobs)) as ex:
        results = list(ex.map(lambda s: _compile(s, resource_report is not None), SOURCES))
    rows = resource_usage(results)
    if resource_report:
        with open(resource_report, "w") as f:
            f.write(format_report(rows))
    spills = [r for r in rows if r.get("scratch", 0) > 0]
    if spills:
        raise RuntimeError("kernels use scratch memory (register spills), which serialises the LDS-copy "
                           "rings: " + "; ".join(f"{r['kernel']} ({r['scratch']} B/lane)" for r in spills))
    if not rows:
        raise RuntimeError("no kernel resource usage was reported by the compiler")
    objs = [r[0] for r in results]
    tmp = LIB + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp] + objs
    p = subprocess.run(cmd, capture_output=True, text=True)
    if p.returncode != 0:
        raise RuntimeError(f"link failed:\n{p.stderr[-8000:]}")
    os.replace(tmp, LIB)
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
