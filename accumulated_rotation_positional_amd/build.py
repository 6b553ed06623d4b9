"""Build libarp.so (the gfx950 HIP kernels and their C ABI) in-tree with hipcc.

Every source is compiled for gfx950 only.  ``-packed-fp32-ops`` keeps the
compiler from emitting packed fp32 arithmetic; ``-ffp-contract=fast`` (the HIP
default) is kept, and nothing is built with fast-math, so the angle scan's
fixed-point conversions are compiled as written.
"""
from __future__ import annotations

import concurrent.futures
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(HERE, "_build")
TARGET = os.path.join(HERE, "libarp.so")
SCAN_TEST_TARGET = os.path.join(HERE, "libarp_scan_from_source.so")
SOURCES = ["api.hip", "angle_scan.hip", "rotate.hip", "attn_f32.hip", "attn_bf16.hip", "attn_bwd.hip", "decode.hip"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
FLAGS = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-Wall",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
# The attention kernel takes maxima only over finite logits and -inf (masked
# keys), so it needs no NaN quieting around v_max: without this flag every
# operand of a maximum is first canonicalised, doubling the softmax's
# max instructions.
FILE_FLAGS = {"attn_bf16.hip": ["-fno-honor-nans"]}


def _compile(src: str, verbose: bool, define: str | None = None) -> str:
    stem = src.replace(".hip", "") + ("_" + define.split("=")[0].lower() if define else "")
    obj = os.path.join(BUILD, stem + ".o")
    extra = [f"-D{define}"] if define else []
    cmd = [HIPCC, *FLAGS, *FILE_FLAGS.get(src, []), *extra, "-c", os.path.join(CSRC, src), "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    # hipcc's host pass does not know the packed-fp32 feature and says so; drop that line.
    noise = "'-packed-fp32-ops' is not a recognized feature"
    msgs = "\n".join(ln for ln in (r.stdout + r.stderr).splitlines() if noise not in ln)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{msgs}")
    if msgs.strip() and verbose:
        print(msgs, flush=True)
    return obj


def _link(objs, target: str, verbose: bool) -> None:
    tmp = target + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, target)


def build(verbose: bool = False) -> str:
    """Compile every source for gfx950 and link libarp.so; always rebuilds.
    Also links the scan test variant (SCAN_TEST_TARGET): the same objects but
    an angle scan built with ARP_SCAN_FALLBACK_POLLS=0, which reduces every
    predecessor chunk from its source instead of reading published prefixes
    (the tests check its angles bit for bit against libarp.so's)."""
    os.makedirs(BUILD, exist_ok=True)
    jobs = [(s, None) for s in SOURCES] + [("angle_scan.hip", "ARP_SCAN_FALLBACK_POLLS=0")]
    with concurrent.futures.ThreadPoolExecutor(max_workers=len(jobs)) as ex:
        objs = list(ex.map(lambda j: _compile(j[0], verbose, j[1]), jobs))
    _link(objs[:len(SOURCES)], TARGET, verbose)
    variant = [objs[-1] if s == "angle_scan.hip" else o for s, o in zip(SOURCES, objs)]
    _link(variant, SCAN_TEST_TARGET, verbose)
    return TARGET


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
