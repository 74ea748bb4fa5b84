"""Build libqf.so (gfx950) in-tree from fp4_fake_quant_amd/csrc.

Usage: python -m fp4_fake_quant_amd.build   (or __graft_entry__.build())

Numerics flags that the bit-exact contract depends on:
  -ffp-contract=off                          no fused multiply-add unless written
  -fhip-fp32-correctly-rounded-divide-sqrt   IEEE division (no v_rcp shortcut)
  -fno-gpu-flush-denormals-to-zero           keep fp32 subnormals
  -Xclang -target-feature -Xclang -packed-fp32-ops   no packed fp32 VALU ops
"""

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libqf.so")
BUILD = os.path.join(HERE, "_build")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-fPIC", "-std=c++17",
    "-ffp-contract=off", "-fhip-fp32-correctly-rounded-divide-sqrt", "-fno-gpu-flush-denormals-to-zero",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-result", "-Wno-unused-command-line-argument",
]


def sources():
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith((".hip", ".cpp")))


def _compile(src):
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    cmd = [HIPCC] + FLAGS + ["-x", "hip", "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    # hipcc's host pass warns that it does not know the packed-fp32 feature: harmless
    err = "\n".join(l for l in r.stderr.splitlines() if "packed-fp32-ops" not in l and l.strip())
    return obj, r.returncode, err


def build(verbose=False):
    os.makedirs(BUILD, exist_ok=True)
    srcs = sources()
    with ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        results = list(ex.map(_compile, srcs))
    failed = [(o, e) for o, rc, e in results if rc != 0]
    for o, rc, e in results:
        if e and (verbose or rc != 0):
            print(e, file=sys.stderr)
    if failed:
        raise RuntimeError("hipcc failed for: " + ", ".join(os.path.basename(o) for o, _ in failed))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp] + [o for o, _, _ in results]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n" + r.stderr)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
