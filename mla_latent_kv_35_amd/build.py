"""Build libmla.so (the C-ABI library) in-tree for gfx950 with hipcc.

Usage: python -m mla_latent_kv_35_amd.build [--jobs N] [--save-temps DIR]
"""
from __future__ import annotations

import argparse
import concurrent.futures as cf
import os
import shutil
import subprocess
import sys
import tempfile

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")
ROOT = os.path.dirname(PKG)
LIB = os.path.join(PKG, "libmla.so")
ARCH = "gfx950"

SOURCES = ["mla_api.hip", "decode_pipe.hip", "decode_simple.hip", "combine.hip",
           "rope.hip", "absorb.hip", "out_proj.hip", "append.hip", "prefill.hip",
           "gemm_nt.hip", "probe.hip"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

COMMON_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    "-I", os.path.join(ROOT, "include"),
    # no packed-fp32 instructions (v_pk_{add,mul,fma}_f32) in device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
]


# Per-file code-generation options. The decode kernel keeps its MFMA
# accumulators in VGPRs: its rare accumulator rescale is plain VALU work there,
# and the query fragments (MFMA B operands) can live in AGPRs.
EXTRA_FLAGS = {
}


def _compile(src: str, obj: str, save_temps: str | None) -> None:
    cmd = [HIPCC, *COMMON_FLAGS, *EXTRA_FLAGS.get(src, []), "-c", os.path.join(CSRC, src),
           "-o", obj]
    if save_temps:
        cmd += ["-save-temps=obj"]
    r = subprocess.run(cmd, capture_output=True, text=True,
                       cwd=save_temps if save_temps else None)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stderr}")
    err = "\n".join(l for l in r.stderr.splitlines()
                    if "error" in l.lower() and "packed-fp32-ops" not in l)
    if err:
        print(err, file=sys.stderr)


def build(jobs: int = 8, save_temps: str | None = None, verbose: bool = True) -> str:
    tmp = tempfile.mkdtemp(prefix="mla_build_")
    try:
        objs = [os.path.join(save_temps or tmp, s.replace(".hip", ".o")) for s in SOURCES]
        with cf.ThreadPoolExecutor(max_workers=max(1, jobs)) as ex:
            futs = [ex.submit(_compile, s, o, save_temps) for s, o in zip(SOURCES, objs)]
            for f in futs:
                f.result()
        out_tmp = LIB + ".tmp"
        cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", out_tmp, *objs]
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"link failed:\n{r.stderr}")
        os.replace(out_tmp, LIB)
        if verbose:
            print(f"built {LIB}")
        return LIB
    finally:
        shutil.rmtree(tmp, ignore_errors=True)


def main() -> None:
    ap = argparse.ArgumentParser()
    ap.add_argument("--jobs", type=int, default=8)
    ap.add_argument("--save-temps", default=None)
    a = ap.parse_args()
    if a.save_temps:
        os.makedirs(a.save_temps, exist_ok=True)
    build(a.jobs, a.save_temps)


if __name__ == "__main__":
    main()
