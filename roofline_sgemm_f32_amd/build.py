"""Build libsgemm.so (HIP, gfx950 only) in-tree with hipcc.

Every HIP source is compiled with packed-FP32 vector instructions disabled
(``-target-feature -packed-fp32-ops``), so the vector ALU kernels use plain
v_fma_f32; the matrix-core kernel is unaffected.  Usage:
``python -m roofline_sgemm_f32_amd.build``.
"""
from __future__ import annotations

import concurrent.futures as cf
import glob
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libsgemm.so")
ARCH = "gfx950"

HIPFLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-fPIC", "-std=c++17", "-Wall",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libsgemm.so)")


def sources() -> list[str]:
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")))


def _compile(src: str, obj_dir: str, extra: list[str]) -> str:
    obj = os.path.join(obj_dir, os.path.basename(src) + ".o")
    cmd = [hipcc(), *HIPFLAGS, *extra, "-c", src, "-o", obj]
    res = subprocess.run(cmd, capture_output=True, text=True)
    # The host pass does not know the packed-FP32 feature; that warning is
    # expected and harmless.  Anything else is shown.
    noise = "'-packed-fp32-ops' is not a recognized feature"
    msgs = [ln for ln in (res.stdout + res.stderr).splitlines() if noise not in ln and ln.strip()]
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n" + "\n".join(msgs))
    if msgs:
        print("\n".join(msgs), file=sys.stderr)
    return obj


def build(extra: list[str] | None = None, out: str | None = None) -> str:
    """Compile every csrc/*.hip for gfx950 and link libsgemm.so (always)."""
    extra = extra or []
    out = out or LIB
    obj_dir = os.path.join(HERE, "_build")
    os.makedirs(obj_dir, exist_ok=True)
    srcs = sources()
    with cf.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(lambda s: _compile(s, obj_dir, extra), srcs))
    tmp = out + ".tmp%d" % os.getpid()
    subprocess.check_call([hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp])
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build())
