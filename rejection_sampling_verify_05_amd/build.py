"""Build libspecverify.so (HIP, gfx950) next to this file with hipcc."""
from __future__ import annotations

import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
SOURCES = [os.path.join(HERE, "csrc", n) for n in ("sv_api.hip", "sv_stats.hip", "sv_topk.hip", "sv_topp.hip",
                                                    "sv_epilogue.hip", "sv_draft.hip", "sv_lmhead.hip")]
OUTPUT = os.path.join(HERE, "libspecverify.so")

# -ffp-contract=off: every fp32 operation on logits rounds once (the penalty and
# the greedy/top-k comparisons must match IEEE arithmetic bit for bit).
# -packed-fp32-ops: no v_pk_*_f32 instructions.
# -fvisibility=hidden: only the C ABI (SV_API in include/specverify.h) is exported.
HIPCC_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared", "-ffp-contract=off",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function", "-fvisibility=hidden",
]


def hipcc() -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    return os.path.join(rocm, "bin", "hipcc")


def build_library(verbose: bool = False) -> str:
    tmp = OUTPUT + ".tmp"
    cmd = [hipcc(), *HIPCC_FLAGS, f"-I{os.path.join(ROOT, 'include')}", "-o", tmp, *SOURCES]
    r = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    msgs = "\n".join(l for l in (r.stdout + r.stderr).splitlines() if noise not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed ({r.returncode}):\n{msgs}")
    if verbose and msgs.strip():
        print(msgs)
    os.replace(tmp, OUTPUT)
    return OUTPUT


if __name__ == "__main__":
    print(build_library(verbose=True))
