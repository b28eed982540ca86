"""Build libcbs.so (the HIP kernels and the C-ABI host library) in-tree with hipcc
for gfx950."""
from __future__ import annotations

import os
import subprocess
import sys

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG_DIR, "csrc")
BUILD_DIR = os.path.join(PKG_DIR, "_build")
LIB_PATH = os.path.join(PKG_DIR, "libcbs.so")
ARCH = "gfx950"

# No packed-fp32 instructions (v_pk_*_f32) are emitted for the device code.
DEVICE_FLAGS = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
COMMON = ["--offload-arch=" + ARCH, "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-function",
          "-Wno-unused-command-line-argument"]


def _hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", "hipcc"):
        if cand and (os.path.sep not in cand or os.path.exists(cand)):
            return cand
    return "hipcc"


def _run(cmd):
    print("+", " ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)


def check_mfma_guards(hipcc: str) -> None:
    """Fail the build if any MFMA of the conv kernels sits in an EXEC-masked
    region.  MFMA ignores EXEC, so an MFMA under a per-lane condition would
    still execute for the whole wave; every MFMA guard must be a scalar
    (wave-uniform) branch.  Scans the device assembly of this build."""
    import re
    asm = os.path.join(BUILD_DIR, "cbs_kernels.s")
    _run([hipcc, "--cuda-device-only", "-S", os.path.join(CSRC, "cbs_kernels.hip"), "-o", asm, "-O3"]
         + COMMON + DEVICE_FLAGS)
    text = open(asm).read()
    bad = []
    for name in re.findall(r"^(_ZN3cbs(?:10conv_igemm|8conv_lds)\w+):", text, re.M):
        body = text[text.index(name + ":"):text.index(".Lfunc_end", text.index(name + ":"))]
        masked = False
        for line in body.split("\n"):
            t = line.strip()
            if re.match(r"s_(and|andn2|xor|or)_saveexec", t):
                masked = True
            elif t.startswith("s_or_b64 exec") or t.startswith("s_mov_b64 exec"):
                masked = False
            elif t.startswith("v_mfma") and masked:
                bad.append(name)
                break
    if bad:
        raise RuntimeError("MFMA inside an EXEC-masked region in: %s" % ", ".join(bad))


def build(verbose: bool = True) -> str:
    """Compile every source and link libcbs.so.  Always recompiles."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    hipcc = _hipcc()
    check_mfma_guards(hipcc)
    k_obj = os.path.join(BUILD_DIR, "cbs_kernels.o")
    h_obj = os.path.join(BUILD_DIR, "cbs_host.o")
    # kernels: -O3, device code without packed fp32
    _run([hipcc, "-c", os.path.join(CSRC, "cbs_kernels.hip"), "-o", k_obj, "-O3"] + COMMON + DEVICE_FLAGS)
    # host library: every double product/sum rounded as written (no FMA contraction)
    _run([hipcc, "-c", os.path.join(CSRC, "cbs_host.cpp"), "-o", h_obj, "-O2", "-ffp-contract=off"]
         + COMMON + DEVICE_FLAGS)
    tmp = LIB_PATH + ".tmp%d" % os.getpid()
    _run([hipcc, "-shared", "-o", tmp, k_obj, h_obj, "--offload-arch=" + ARCH, "-fPIC"])
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    build()
    sys.exit(0)
