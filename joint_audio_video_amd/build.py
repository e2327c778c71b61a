"""Build libdit.so in-tree with hipcc for gfx950.

Usage: python joint_audio_video_amd/build.py   (or __graft_entry__.build()); run
as a file, not with -m: the package's __init__ loads the built library and
refuses to import without it.

python joint_audio_video_amd/build.py --resources prints, instead of building,
a markdown table of every device kernel's registers, scratch, LDS and
occupancy as the compiler reports them for gfx950.

Every source under csrc/ is compiled to an object in _build/ and linked into
joint_audio_video_amd/libdit.so.  The build always recompiles (it is the
"does it build" check), in parallel.
"""
from __future__ import annotations

import concurrent.futures
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libdit.so")
ARCH = "gfx950"

HIPCC = os.environ.get("HIPCC", shutil.which("hipcc") or "/opt/rocm/bin/hipcc")

COMMON_FLAGS = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
    # never let the compiler form packed-fp32 (v_pk_*_f32) instructions
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
    f"-I{INCLUDE}", f"-I{CSRC}",
]

SOURCES = ["abi.cpp", "layout.cpp", "adaln.hip", "rope.hip", "gemm.hip", "attn.hip",
           "attn_fp8.hip", "attn_bwd.hip", "grad.hip", "denoise.hip", "nft.hip"]


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC, *COMMON_FLAGS, "-x", "hip", "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return obj


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp"
    # The library needs libamdhip64.so.7.  PyTorch ships its own copy under the
    # same soname; the binding imports torch first so that the dynamic linker
    # reuses that copy (two HIP/HSA runtimes in one process break both).
    cmd = [HIPCC, "-shared", "-fPIC", f"--offload-arch={ARCH}", *objs, "-o", tmp,
           "-Wl,--no-undefined"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


def _demangle(name: str) -> str:
    tool = shutil.which("c++filt") or shutil.which("llvm-cxxfilt")
    out = name
    if tool:
        r = subprocess.run([tool, name], capture_output=True, text=True)
        if r.returncode == 0 and r.stdout.strip():
            out = r.stdout.strip()
    return out.replace("(anonymous namespace)::", "").split("(")[0].replace("void ", "")


def resource_rows(sources=None) -> list:
    """The compiler's kernel-resource-usage remarks for the given .hip sources
    (default: all), one dict per device kernel."""
    import re
    keys = ("VGPRs", "AGPRs", "ScratchSize [bytes/lane]", "Occupancy [waves/SIMD]",
            "LDS Size [bytes/block]", "SGPRs Spill")
    srcs = [src for src in (SOURCES if sources is None else sources) if src.endswith(".hip")]

    def remarks(src):
        cmd = [HIPCC, *COMMON_FLAGS, "-x", "hip", "--cuda-device-only", "-c",
               os.path.join(CSRC, src), "-o", os.devnull, "-Rpass-analysis=kernel-resource-usage"]
        return subprocess.run(cmd, capture_output=True, text=True).stderr

    with concurrent.futures.ThreadPoolExecutor(max_workers=min(8, len(srcs) or 1)) as ex:
        outs = list(ex.map(remarks, srcs))
    rows = []
    for src, err in zip(srcs, outs):
        cur = None
        for line in err.splitlines():
            m = re.search(r"remark:\s+Function Name: (\S+)", line)
            if m:
                cur = {"name": _demangle(m.group(1)), "src": src}
                rows.append(cur)
                continue
            for k in keys:
                m = re.search(r"remark:\s+" + re.escape(k) + r": (\d+)", line)
                if m and cur is not None:
                    cur[k] = m.group(1)
    return rows


def resources() -> str:
    """Markdown table of the compiler's kernel-resource-usage remarks for every .hip source."""
    rows = resource_rows()
    out = ["| source | kernel | VGPRs | AGPRs | scratch B/lane | SGPR spills | LDS B/workgroup | "
           "waves/SIMD |",
           "|---|---|---|---|---|---|---|---|"]
    for r in rows:
        out.append(f"| {r['src']} | {r['name']} | {r.get('VGPRs', '')} | {r.get('AGPRs', '')} | "
                   f"{r.get('ScratchSize [bytes/lane]', '')} | {r.get('SGPRs Spill', '')} | "
                   f"{r.get('LDS Size [bytes/block]', '')} | "
                   f"{r.get('Occupancy [waves/SIMD]', '')} |")
    return "\n".join(out)


if __name__ == "__main__":
    if "--resources" in sys.argv[1:]:
        print(resources())
    else:
        build(verbose=True)
    sys.exit(0)
