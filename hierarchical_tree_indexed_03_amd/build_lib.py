"""Compiles the HIP sources under csrc/ into libzha.so (gfx950) next to this file.

    python -m hierarchical_tree_indexed_03_amd.build_lib [--variant=debug|asan]
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
OUT = os.path.join(HERE, "libzha.so")
PROBE_OUT = os.path.join(HERE, "libzha_probe.so")   # benchmark-only measurement kernels
OBJDIR = os.path.join(HERE, "_build")
# variants: the same sources with the device invariant checks compiled in (-DZHA_DEBUG), and
# the host side built with AddressSanitizer and UndefinedBehaviorSanitizer (device code as
# usual) for the host-validation tests
VARIANTS = {
    "release": dict(out=OUT, objdir=OBJDIR, flags=[], link=[]),
    "debug": dict(out=os.path.join(HERE, "libzha_debug.so"), objdir=os.path.join(HERE, "_build_debug"),
                  flags=["-DZHA_DEBUG"], link=[]),
    "asan": dict(out=os.path.join(HERE, "libzha_asan.so"), objdir=os.path.join(HERE, "_build_asan"),
                 flags=["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                        "-Xarch_host", "-fno-omit-frame-pointer", "-Xarch_host", "-fno-sanitize-recover=undefined"],
                 link=["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined"]),
}
ARCH = os.environ.get("ZHA_OFFLOAD_ARCH", "gfx950")

FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-fPIC", "-std=c++17",
    # packed fp32 VALU forms stay off: plain v_fma_f32 etc. only
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"), "-I", CSRC,
    "-Wno-unused-result",
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def sources() -> list[str]:
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".hip"))


def build(verbose: bool = False, variant: str = "release") -> str:
    """Compiles every source of csrc/ into the variant's library (and, for the release
    variant, the probe library); returns the library path."""
    var = VARIANTS[variant]
    objdir, out = var["objdir"], var["out"]
    os.makedirs(objdir, exist_ok=True)
    cc = hipcc()
    objs = []

    def compile_one(src):
        obj = os.path.join(objdir, os.path.basename(src)[:-4] + ".o")
        cmd = [cc, *FLAGS, *var["flags"], "-c", src, "-o", obj]
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
        if verbose and r.stderr.strip():
            print(r.stderr, file=sys.stderr)
        return obj

    with cf.ThreadPoolExecutor(max(1, min(8, os.cpu_count() or 1))) as ex:
        objs = list(ex.map(compile_one, sources()))
    tmp = out + ".tmp"
    cmd = [cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", *var["link"], "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, out)
    if variant != "release":
        return out
    probe_src = os.path.join(CSRC, "probe", "probe.hip")
    tmp = PROBE_OUT + ".tmp"
    cmd = [cc, *FLAGS, "-shared", "-fPIC", "-o", tmp, probe_src]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"probe build failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, PROBE_OUT)
    return OUT


if __name__ == "__main__":
    variant = next((a.split("=", 1)[1] for a in sys.argv[1:] if a.startswith("--variant=")), "release")
    print(build(verbose="-v" in sys.argv, variant=variant))
