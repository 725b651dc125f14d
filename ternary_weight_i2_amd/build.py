"""Build libbitnet_i2s.so in-tree with hipcc for gfx950 (MI355X).

    python -m ternary_weight_i2_amd.build
"""
from __future__ import annotations

import glob
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
OUT = os.path.join(HERE, "libbitnet_i2s.so")
OUT_STAMPS = os.path.join(HERE, "libbitnet_i2s_stamps.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    "-fvisibility=hidden",
    # keep the compiler from emitting packed fp32 VALU ops
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-result",
]


def sources() -> list[str]:
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")))


def _run(cmd: list[str], verbose: bool) -> None:
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    errs = [ln for ln in res.stderr.splitlines()
            if "packed-fp32-ops" not in ln and ln.strip()]
    if res.returncode != 0:
        sys.stderr.write("\n".join(errs) + "\n")
        raise RuntimeError(f"hipcc failed ({res.returncode}): {' '.join(cmd[-3:])}")
    if verbose and errs:
        sys.stderr.write("\n".join(errs) + "\n")


def build(verbose: bool = False) -> str:
    """Compile each translation unit in parallel, then link the shared
    library and its instrumented twin (-DBITNET_STAMPS: per-launch start/end
    stamps of the decode GEMV, include/bitnet_i2s_stamps.h)."""
    import tempfile
    from concurrent.futures import ThreadPoolExecutor
    inc = ["-I", os.path.join(ROOT, "include"), "-I", CSRC]
    srcs = sources()
    variants = ((OUT, []), (OUT_STAMPS, ["-DBITNET_STAMPS"]))
    with tempfile.TemporaryDirectory(prefix="bitnet_build_") as tmpdir:
        jobs, objs = [], []
        for vi, (_, defs) in enumerate(variants):
            vo = [os.path.join(tmpdir, f"{vi}_" + os.path.basename(s)[:-4] + ".o") for s in srcs]
            jobs += [[HIPCC, *FLAGS, *defs, *inc, "-c", s, "-o", o] for s, o in zip(srcs, vo)]
            objs.append(vo)
        workers = max(1, min(len(jobs), os.cpu_count() or 1, 16))
        with ThreadPoolExecutor(workers) as ex:
            list(ex.map(lambda c: _run(c, verbose), jobs))
        for (out, _), vo in zip(variants, objs):
            tmp = out + ".tmp"
            _run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *vo, "-o", tmp], verbose)
            os.replace(tmp, out)
    return OUT


if __name__ == "__main__":
    print(build(verbose=True))
