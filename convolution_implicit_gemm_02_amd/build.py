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


# Two tiny kernels that calibrate the check: an MFMA under a per-lane
# condition (must be flagged) and one under a wave-uniform condition (must not).
_GUARD_PROBE = r"""
#include <hip/hip_runtime.h>
typedef float f4 __attribute__((ext_vector_type(4)));
__global__ void probe_masked(const float *a, f4 *o, int n) {
  f4 acc = {0, 0, 0, 0};
  if ((int)threadIdx.x < n) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a[threadIdx.x], a[threadIdx.x + 64], acc, 0, 0, 0);
  o[threadIdx.x] = acc;
}
__global__ void probe_uniform(const float *a, f4 *o, int n) {
  f4 acc = {0, 0, 0, 0};
  if (n > 3) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a[threadIdx.x], a[threadIdx.x + 64], acc, 0, 0, 0);
  o[threadIdx.x] = acc;
}
"""


def masked_mfma_kernels(text: str, pattern: str):
    """Kernels of a device assembly whose MFMAs may run under a partial EXEC.

    An EXEC-masked region opens at s_*_saveexec and closes where EXEC is
    restored (s_or_b64/s_mov_b64 exec), at the label its s_cbranch_execz
    jumps to, or at an unconditional branch out of the masked body."""
    import re
    bad = []
    for name in re.findall(pattern, text, re.M):
        i = text.index(name + ":")
        body = text[i:text.index(".Lfunc_end", i)].split("\n")
        masked, target = False, None
        for k, line in enumerate(body):
            t = line.strip()
            if re.match(r"s_(and|andn2|xor|or)_saveexec", t):
                masked = True
                nxt = body[k + 1].strip() if k + 1 < len(body) else ""
                target = nxt.split()[1] if nxt.startswith("s_cbranch_execz") else None
            elif masked and (t.startswith("s_or_b64 exec") or t.startswith("s_mov_b64 exec")
                             or t.startswith("s_branch ") or t.startswith("s_endpgm")
                             or (target is not None and t == target + ":")):
                masked, target = False, None
            elif t.startswith("v_mfma") and masked:
                bad.append(name)
                break
    return bad


SCALAR_LINE = 64  # bytes per scalar data cache line


def _sload_lines(line: str):
    """Scalar-cache lines an s_load_dword[xN] sX, s[0:1], OFF of the argument block touches."""
    import re
    m = re.match(r"s_load_dword(?:x(\d+))?\s+\S+,\s*s\[0:1\],\s*(0x[0-9a-f]+|\d+)", line)
    if not m:
        return None
    n = int(m.group(1) or 1)
    off = int(m.group(2), 0)
    return set(range(off // SCALAR_LINE, (off + 4 * n - 1) // SCALAR_LINE + 1))


def late_argument_loads(text: str, pattern: str, max_rounds: int = 1):
    """Kernels of a device assembly whose kernel-argument reads (scalar loads:
    the conv kernels make no other) cost more than one memory round trip:
    loads issued after a wait for earlier ones that touch a cache line of the
    argument block no earlier round requested (a load of a line already on its
    way hits the scalar cache), or any load after the first MFMA (a dependent
    round trip after the main loop).  Returns (flagged names, number of
    kernels with at least one argument load before their first MFMA)."""
    import re
    bad, early = [], 0
    for name in re.findall(pattern, text, re.M):
        i = text.index(name + ":")
        body = [line.strip() for line in text[i:text.index(".Lfunc_end", i)].split("\n")]
        first = next((k for k, line in enumerate(body) if line.startswith("v_mfma")), len(body))
        rounds, pending, late = 0, False, False
        requested = set()
        for k, line in enumerate(body):
            if line.startswith("s_load_"):
                lines = _sload_lines(line)
                new_lines = lines is None or not lines <= requested
                if not pending and new_lines:
                    rounds += 1
                if new_lines:
                    pending = True
                if lines:
                    requested |= lines
                late |= k > first
            elif "lgkmcnt" in line:
                pending = False
        early += any(line.startswith("s_load_") for line in body[:first])
        if rounds > max_rounds or late:
            bad.append(name)
    return bad, early


def flat_memory_ops(text: str, pattern: str):
    """Kernels that access memory through FLAT instructions (a generic pointer
    whose global address space the compiler lost): slower than global/buffer
    ones, and they also wait on the LDS counter."""
    import re
    bad = []
    for name in re.findall(pattern, text, re.M):
        i = text.index(name + ":")
        body = text[i:text.index(".Lfunc_end", i)]
        if re.search(r"^\s+flat_(load|store|atomic)", body, re.M):
            bad.append(name)
    return bad


VARIANTS = 12  # kernel variants, one translation unit each (cbs_variant.hip with -DCBS_VAR=n)
CONV_KERNELS = r"^(_ZN3cbs(?:10conv_igemm|8conv_lds|9conv_halo|7conv_ws)\w+):"
# grouped launches read their member's arguments in a second round, at an
# offset that depends on the first (the group's workgroup ranges)
GROUP_KERNELS = r"^(_ZN3cbs(?:16conv_igemm_group|14conv_lds_group)\w+):"
GROUP_VARIANTS = (0, 1, 2, 5, 6, 7, 8, 9)  # variants with grouped kernels (not the raw-accumulator hooks)
# the raw-accumulator variants (cbs_run_layer_raw_acc, a test hook) may read
# their arguments in two rounds, still none after the first MFMA
RAW_VARIANTS = (3, 4, 10, 11)


def _jobs() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 4
    return max(1, min(8, n))


def _parallel(cmds):
    from concurrent.futures import ThreadPoolExecutor
    with ThreadPoolExecutor(max_workers=_jobs()) as ex:
        for f in [ex.submit(_run, c) for c in cmds]:
            f.result()


def check_mfma_guards(hipcc: str) -> None:
    """Fail the build if any MFMA of the conv kernels may run under a partial
    EXEC mask.  MFMA ignores EXEC, so an MFMA under a per-lane condition would
    still execute for the whole wave; every MFMA guard must be a scalar
    (wave-uniform) branch.  Scans the device assembly of every variant of this
    build, after checking that the scan flags a known-masked probe and passes a
    uniform one.  Also fails if a conv kernel reads a kernel argument after its
    first MFMA (a memory round trip at the end of every launch)."""
    import re
    probe_src = os.path.join(BUILD_DIR, "guard_probe.hip")
    probe_asm = os.path.join(BUILD_DIR, "guard_probe.s")
    with open(probe_src, "w") as f:
        f.write(_GUARD_PROBE)
    cmds = [[hipcc, "--cuda-device-only", "-S", probe_src, "-o", probe_asm, "-O3"] + COMMON + DEVICE_FLAGS]
    asms = []
    for v in range(VARIANTS):
        asm = os.path.join(BUILD_DIR, "cbs_variant_%d.s" % v)
        asms.append(asm)
        cmds.append([hipcc, "--cuda-device-only", "-S", os.path.join(CSRC, "cbs_variant.hip"), "-o", asm, "-O3",
                     "-DCBS_VAR=%d" % v] + COMMON + DEVICE_FLAGS)
    _parallel(cmds)
    flagged = masked_mfma_kernels(open(probe_asm).read(), r"^(_Z\d+probe_\w+):")
    if not any("probe_masked" in n for n in flagged) or any("probe_uniform" in n for n in flagged):
        raise RuntimeError("MFMA guard check failed its calibration (flagged: %s)" % flagged)
    bad, late = [], []
    for asm in asms:
        text = open(asm).read()
        n = len(re.findall(CONV_KERNELS, text, re.M))
        if n < 3:
            raise RuntimeError("MFMA guard check found no conv kernels in %s" % asm)
        bad += masked_mfma_kernels(text, CONV_KERNELS)
        flagged, early = late_argument_loads(text, CONV_KERNELS,
                                             max_rounds=2 if asms.index(asm) in RAW_VARIANTS else 1)
        if early < n:
            raise RuntimeError("argument-load check matched no early scalar loads in %s" % asm)
        late += flagged
        late += ["%s (FLAT access)" % k for k in flat_memory_ops(text, CONV_KERNELS)]
        ng = len(re.findall(GROUP_KERNELS, text, re.M))
        if (ng > 0) != (asms.index(asm) in GROUP_VARIANTS):
            raise RuntimeError("grouped kernels expected exactly in variants %s (%s has %d)" % (GROUP_VARIANTS, asm, ng))
        bad += masked_mfma_kernels(text, GROUP_KERNELS)
        late += late_argument_loads(text, GROUP_KERNELS, max_rounds=2)[0]
        late += ["%s (FLAT access)" % k for k in flat_memory_ops(text, GROUP_KERNELS)]
    if bad:
        raise RuntimeError("MFMA inside an EXEC-masked region in: %s" % ", ".join(bad))
    if late:
        raise RuntimeError("kernel argument read after the main loop, or FLAT access, in: %s" % ", ".join(late))


def build(verbose: bool = True) -> str:
    """Compile every source and link libcbs.so.  Always recompiles."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    hipcc = _hipcc()
    check_mfma_guards(hipcc)
    objs, cmds = [], []
    k_obj = os.path.join(BUILD_DIR, "cbs_kernels.o")
    cmds.append([hipcc, "-c", os.path.join(CSRC, "cbs_kernels.hip"), "-o", k_obj, "-O3"] + COMMON + DEVICE_FLAGS)
    objs.append(k_obj)
    n_obj = os.path.join(BUILD_DIR, "cbs_noalloc.o")
    cmds.append([hipcc, "-c", os.path.join(CSRC, "cbs_noalloc.hip"), "-o", n_obj, "-O3"] + COMMON + DEVICE_FLAGS)
    objs.append(n_obj)
    for v in range(VARIANTS):
        o = os.path.join(BUILD_DIR, "cbs_variant_%d.o" % v)
        cmds.append([hipcc, "-c", os.path.join(CSRC, "cbs_variant.hip"), "-o", o, "-O3", "-DCBS_VAR=%d" % v]
                    + COMMON + DEVICE_FLAGS)
        objs.append(o)
    # host library: every double product/sum rounded as written (no FMA contraction)
    h_obj = os.path.join(BUILD_DIR, "cbs_host.o")
    cmds.append([hipcc, "-c", os.path.join(CSRC, "cbs_host.cpp"), "-o", h_obj, "-O2", "-ffp-contract=off"]
                + COMMON + DEVICE_FLAGS)
    objs.append(h_obj)
    _parallel(cmds)
    tmp = LIB_PATH + ".tmp%d" % os.getpid()
    _run([hipcc, "-shared", "-o", tmp] + objs + ["--offload-arch=" + ARCH, "-fPIC"])
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    build()
    sys.exit(0)
