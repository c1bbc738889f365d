"""Builds the HIP library ``libdsa_amd.so`` in-tree with hipcc for gfx950."""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libdsa_amd.so")
# measurement micro-kernels (the benchmark's achievable-peak figures), a library of their own
PEAKS_LIB = os.path.join(PKG, "libdsa_peaks.so")
# debug build of the same sources whose kernels fill their LDS with NaN first (tests only)
LDS_POISON_LIB = os.path.join(PKG, "libdsa_amd_lds_poison.so")
PEAKS_SOURCE = "peaks.hip"
SOURCES = ["dsa_api.cpp", "validate.cpp", "selftest.hip", "indexer.hip", "topk.hip", "fused.hip", "sparse_mla.hip"]
ARCH = "gfx950"
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

COMMON_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-fvisibility=hidden",
    # Keep the compiler from forming packed-fp32 VALU ops.
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"), "-I", CSRC,
]


# Per-source flags. The indexer's MFMA accumulators are read by VALU code
# right after every product: asking for the VGPR form of the MFMAs saves an
# accumulator-to-VGPR copy per element.
SOURCE_FLAGS = {"indexer.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"]}


def _compile(src: str, obj: str, extra) -> None:
    cmd = [HIPCC, *COMMON_FLAGS, *SOURCE_FLAGS.get(src, []), *extra, "-x", "hip", "-c", os.path.join(CSRC, src),
           "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stdout}\n{r.stderr}")
    # surface real warnings (the host pass does not know the packed-fp32 feature: harmless)
    noise = "is not a recognized feature for this target"
    msgs = [ln for ln in (r.stderr or "").splitlines() if ln.strip() and noise not in ln and "(ignoring feature)" not in ln]
    if msgs:
        print("\n".join(msgs), file=sys.stderr)


def build(extra_flags=None, out: str = LIB) -> str:
    """Compile every source and link the shared library. Returns its path."""
    extra = list(extra_flags or [])
    objdir = os.path.join(PKG, "_build", os.path.splitext(os.path.basename(out))[0])
    os.makedirs(objdir, exist_ok=True)
    objs = [os.path.join(objdir, os.path.splitext(s)[0] + ".o") for s in SOURCES]
    with ThreadPoolExecutor(max_workers=len(SOURCES)) as ex:
        list(ex.map(lambda so: _compile(so[0], so[1], extra), zip(SOURCES, objs)))
    tmp = out + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, out)
    if out == LIB:
        build_peaks()
        build(["-DDSA_LDS_POISON"], LDS_POISON_LIB)
    return out


def build_peaks(out: str = PEAKS_LIB) -> str:
    """Compile the measurement micro-kernels into their own shared library."""
    objdir = os.path.join(PKG, "_build")
    os.makedirs(objdir, exist_ok=True)
    obj = os.path.join(objdir, "peaks.o")
    _compile(PEAKS_SOURCE, obj, [])
    tmp = out + ".tmp"
    r = subprocess.run([HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", obj, "-o", tmp], capture_output=True,
                       text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build())
