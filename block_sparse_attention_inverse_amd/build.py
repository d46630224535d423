"""Build ``libbsa.so`` (the C-ABI library) from ``csrc/*.hip`` for gfx950.

Each translation unit is compiled separately with hipcc and linked into one
shared library that lives next to this file (in-tree, so that it travels
with the source tree).  Usage: ``python -m block_sparse_attention_inverse_amd.build``.

``--sanitize-host`` builds the host code (argument checks, launch set-up)
with AddressSanitizer and UndefinedBehaviorSanitizer; the device code is
unchanged.  Load it with clang's ASan runtime preloaded (see the README) and
run the host-only ABI tests; build again without the flag afterwards.
"""
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libbsa.so")
OBJ_DIR = os.path.join(HERE, "_build")
SOURCES = [
    "capi.hip", "permute.hip", "mask.hip", "fused.hip", "order.hip", "quant.hip", "attn.hip",
    "attn_bf16.hip", "calib.hip", "comp.hip",
]
ARCH = "gfx950"

HIPCC_FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++20",
    "-fPIC",
    "-Wall",
    # fp32 divide and sqrt correctly rounded (the block-scoring contract)
    "-fhip-fp32-correctly-rounded-divide-sqrt",
    # keep packed-fp32 VALU ops out of the generated code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


# per-source extra flags.  The bf16 attention kernel takes no NaN inputs into
# account (a NaN in Q, K or V gives unspecified output), which lets its row
# maxima fuse into v_max3 without quieting every operand first.
EXTRA_FLAGS = {
    "attn_bf16.hip": ["-fno-honor-nans"],
    # the INT8 kernel reads its MFMA results with VALU ops: keep them in VGPRs.
    # Its scales are finite for finite inputs (a NaN scale gives unspecified
    # output), so its maxima need no NaN quieting either.
    "attn.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form", "-fno-honor-nans"],
    # the dense block-statistics kernel reads every score with VALU ops too
    "calib.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
}


def _hipcc():
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", "hipcc"):
        if cand and (os.path.sep not in cand or os.path.exists(cand)):
            return cand
    return "hipcc"


# host-only sanitizers: each -fsanitize goes to the host pass alone
HOST_SANITIZE = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                 "-Xarch_host", "-fno-sanitize=function", "-Xarch_host", "-fno-omit-frame-pointer"]


def _compile(src, verbose, sanitize=False):
    obj = os.path.join(OBJ_DIR, os.path.splitext(src)[0] + ".o")
    cmd = [_hipcc(), *HIPCC_FLAGS, *EXTRA_FLAGS.get(src, []), *(HOST_SANITIZE if sanitize else []),
           "-c", os.path.join(CSRC, src), "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    noise = "'-packed-fp32-ops' is not a recognized feature"
    msg = "\n".join(l for l in (r.stdout + r.stderr).splitlines() if noise not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{msg}")
    if msg.strip() and verbose:
        print(msg)
    return obj


def build(verbose: bool = False, jobs: int = 6, sanitize_host: bool = False) -> str:
    os.makedirs(OBJ_DIR, exist_ok=True)
    with ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose, sanitize_host), SOURCES))
    san = ["-shared-libsan", "-Xarch_host", "-fsanitize=address,undefined"] if sanitize_host else []
    cmd = [_hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *san, "-o", LIB + ".tmp", *objs]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(LIB + ".tmp", LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv, sanitize_host="--sanitize-host" in sys.argv))
