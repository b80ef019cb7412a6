"""Builds libpagedattn.so (gfx950) in-tree with hipcc.

    python -m paged_attention_prefill_amd.build [--verbose]

Every HIP source under csrc/ is compiled for gfx950 with packed-fp32
instructions disabled, then linked into paged_attention_prefill_amd/libpagedattn.so.
"""

import argparse
import concurrent.futures as cf
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
ROOT = os.path.dirname(HERE)
BUILD_DIR = os.path.join(ROOT, "_build")
LIB = os.path.join(HERE, "libpagedattn.so")
SOURCES = ["attn_mixed.hip", "attn_mfma_dma.hip", "attn_prefill_w4.hip", "attn_decode.hip", "attn_mfma.hip",
           "attn_valu.hip", "merge.hip", "kv_write.hip", "mixed_route.hip", "pagedattn_api.hip", "ceilings.hip"]
ARCH = "gfx950"

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
CFLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    # never emit packed fp32 arithmetic (v_pk_fma_f32 and friends)
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"),
]


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    out = (r.stdout or "") + (r.stderr or "")
    # the host pass does not know the packed-fp32 feature; that warning is noise
    lines = [l for l in out.splitlines() if "packed-fp32-ops" not in l]
    if r.returncode != 0:
        raise RuntimeError(f"command failed ({r.returncode}): {' '.join(cmd)}\n" + "\n".join(lines))
    if verbose and lines:
        print("\n".join(lines), flush=True)


def build(verbose=False, jobs=4, extra_flags=()):
    os.makedirs(BUILD_DIR, exist_ok=True)
    objs = []
    cmds = []
    for src in SOURCES:
        obj = os.path.join(BUILD_DIR, src.replace(".hip", ".o"))
        objs.append(obj)
        cmds.append([HIPCC, *CFLAGS, *extra_flags, "-c", os.path.join(CSRC, src), "-o", obj])
    with cf.ThreadPoolExecutor(max_workers=jobs) as ex:
        for f in [ex.submit(_run, c, verbose) for c in cmds]:
            f.result()
    tmp = LIB + ".tmp"
    _run([HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs], verbose)
    os.replace(tmp, LIB)
    return LIB


def main(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("--verbose", action="store_true")
    ap.add_argument("--jobs", type=int, default=4)
    a = ap.parse_args(argv)
    print(build(verbose=a.verbose, jobs=a.jobs))


if __name__ == "__main__":
    sys.exit(main())
