"""Build libbsa.so in-tree with hipcc for gfx950.

    python -m long_context_block_amd.build        # or: from long_context_block_amd.build import build

Every HIP source under csrc/ is compiled to an object with -fPIC and the objects are linked
into long_context_block_amd/libbsa.so.  Packed-fp32 instruction selection is disabled
(-Xclang -target-feature -Xclang -packed-fp32-ops) for all device code.
"""

from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
OBJDIR = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libbsa.so")
ARCH = os.environ.get("BSA_OFFLOAD_ARCH", "gfx950")

HIPCC_FLAGS = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
    f"-I{INCLUDE}", f"-I{CSRC}",
]
# Per-source extras.  fwd_bf16.hip keeps MFMA results in VGPRs: two wavefronts per SIMD, and the
# rare rescale multiplies the accumulators in place instead of shuttling them through AGPRs.
# bwd_dkdv.hip likewise: its scores feed the vector unit directly, and its resident K, V operands
# go to AGPRs instead.
EXTRA_FLAGS = {
    "fwd_bf16.hip": ["-mllvm", "--amdgpu-mfma-vgpr-form"],
    "fwd_bf16_basic.hip": ["-mllvm", "--amdgpu-mfma-vgpr-form"],
    "bwd_bf16.hip": ["-mllvm", "--amdgpu-mfma-vgpr-form"],
    "bwd_dkdv.hip": ["-mllvm", "--amdgpu-mfma-vgpr-form"],
}


def _hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (set HIPCC or install ROCm)")


def sources() -> list[str]:
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".hip"))


def _compile(hipcc: str, src: str, verbose: bool) -> str:
    obj = os.path.join(OBJDIR, os.path.basename(src)[:-4] + ".o")
    cmd = [hipcc, *HIPCC_FLAGS, *EXTRA_FLAGS.get(os.path.basename(src), []), "-c", src, "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stdout}\n{r.stderr}")
    if verbose and r.stderr.strip():
        print(r.stderr, file=sys.stderr)
    return obj


def check_m0(hipcc: str, src: str) -> None:
    """The asynchronous LDS copy helpers set M0 in inline asm; M0 is reserved by the compiler and
    cannot be declared clobbered, so the generated code must contain no other M0 user.  Compile
    the device code to assembly and check that every M0 write is a helper's, immediately
    followed by its global_load_lds_dword(x4), and that nothing else references M0."""
    out = os.path.join(OBJDIR, os.path.basename(src)[:-4] + ".s")
    cmd = [hipcc, *HIPCC_FLAGS, *EXTRA_FLAGS.get(os.path.basename(src), []), "--cuda-device-only", "-S", src,
           "-o", out]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc -S failed for {src}:\n{r.stderr}")
    lines = [ln.strip() for ln in open(out)]
    for k, ln in enumerate(lines):
        if ln.startswith(";"):
            continue
        op = ln.split(" ", 1)[0]
        # indexed register moves address registers through M0 without naming it
        if op.startswith(("s_set_gpr_idx", "s_movrel", "v_movrel")):
            raise RuntimeError(f"{src}: indexed register move (implicit M0 user) in generated code: {ln!r}")
        if "m0" not in ln.replace(",", " ").split():
            continue
        nxt = lines[k + 1] if k + 1 < len(lines) else ""
        if not (ln.startswith("s_mov_b32 m0,") and nxt.startswith("global_load_lds_dword")):
            raise RuntimeError(f"{src}: unexpected M0 use in generated code: {ln!r}")


def build(verbose: bool = False) -> str:
    """Compile every csrc/*.hip and link libbsa.so; returns the library path."""
    hipcc = _hipcc()
    os.makedirs(OBJDIR, exist_ok=True)
    srcs = sources()
    with ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(lambda s: _compile(hipcc, s, verbose), srcs))
    # every source, before anything is installed: the copy helpers reach some of them through
    # headers, and a library whose code fails the check must never replace the previous one
    with ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        list(ex.map(lambda s: check_m0(hipcc, s), srcs))
    tmp = LIB + ".tmp"
    cmd = [hipcc, "-shared", "-fPIC", f"--offload-arch={ARCH}", *objs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    try:
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
        os.replace(tmp, LIB)
    finally:
        if os.path.exists(tmp):
            os.remove(tmp)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
