"""Build libpagedkv.so in-tree with hipcc for gfx950.

    python -m paged_kv_cache_413_amd.build        (or call build())

Every translation unit is compiled as HIP for gfx950 only.  Packed-FP32 VALU
instructions are disabled for device code (-packed-fp32-ops).
"""
from __future__ import annotations

import os
import re
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")
ROOT = os.path.dirname(PKG)
LIB = os.path.join(PKG, "libpagedkv.so")
BUILD_DIR = os.path.join(ROOT, "_build")

ARCH = "gfx950"
FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-function",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    f"-I{os.path.join(ROOT, 'include')}",
]
# Per-source device flags.  The decode kernels keep their MFMA operands and
# accumulators in ordinary vector registers: the compiler's default puts the output
# accumulator in AGPRs and then copies all of it to VGPRs and back around the
# (rarely taken) online-softmax rescale of every block -- ~60 moves per block, which
# the MXFP4 decode, bound by its vector work, cannot afford.  (The prefill source does
# not compile with this option, and does not need it.)
SOURCE_FLAGS = {
    "attn_mfma.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=1"],
    # The prefill kernels take row maxima of scores that are never NaN (keys past a
    # sequence are masked to -inf before any maximum): without NaN semantics a maximum
    # is one v_max3 per three inputs instead of a quieting v_max per input first.  The
    # vector ALU is the prefill kernel's busier unit (measured: 5 % off the call).
    "prefill_mfma.hip": ["-fno-honor-nans"],
}


# Every source is compiled with the compiler's per-kernel resource report; build() checks
# it (check_resources) and writes it next to the library (resource_usage.txt).
REMARKS = ["-Rpass-analysis=kernel-resource-usage"]
RESOURCE_REPORT = os.path.join(PKG, "resource_usage.txt")


def parse_resource_remarks(text: str) -> dict:
    """{kernel name: {field: value}} from the compiler's kernel-resource-usage remarks."""
    out, cur = {}, None
    for ln in text.splitlines():
        if "remark:" not in ln:
            continue
        m = re.search(r"Function Name: (\S+)", ln)
        if m:
            cur = out.setdefault(m.group(1), {})
            continue
        m = re.search(r":\s{2,}([A-Za-z][^:\[]*?)(?: \[[^\]]*\])?: (\S+) \[-Rpass-analysis", ln)
        if m and cur is not None:
            cur[m.group(1).strip()] = m.group(2)
    return out


# LDS-shared prefill: five stages of one 32-token block of K and V in bf16 (2 x D x 32
# x 2 bytes each); any more LDS than that is a register array the compiler moved to
# LDS (a run-time index into it), which costs a store and a load per use.
def _prefill_stage_lds(name: str):
    m = re.search(r"prefill_lds_kernelILi\d+ELi(\d+)ELi\d+E", name)
    return 5 * 2 * int(m.group(1)) * 32 * 2 if m else None


# Kernels that use no LDS by design (the decode kernels hold everything in registers):
# any LDS in them is a register array the compiler moved there (a run-time index).
NO_LDS = ("decode_auto_kernel", "decode_fixed_kernel")


def check_resources(usage: dict) -> list:
    """Problems in the per-kernel resource report: scratch memory anywhere (no kernel is
    meant to touch it: registers spilled to memory, or a stack), LDS beyond the prefill
    stages, LDS in the decode kernels.  Registers spilled into other registers (SGPRs
    into vector lanes, VGPRs into AGPRs) cost moves, not memory, and are only reported."""
    bad = []
    for name, f in usage.items():
        if name.startswith("__") or "kernel" not in name:
            continue
        if f.get("ScratchSize", "0") != "0":
            bad.append(f"{name}: scratch {f['ScratchSize']} bytes per lane")
        if f.get("Dynamic Stack", "False") != "False":
            bad.append(f"{name}: dynamic stack")
        lim = _prefill_stage_lds(name)
        if lim is not None and int(f.get("LDS Size", "0")) > lim:
            bad.append(f"{name}: LDS {f['LDS Size']} bytes > {lim} of its stages")
        if any(k in name for k in NO_LDS) and int(f.get("LDS Size", "0")) > 0:
            bad.append(f"{name}: LDS {f['LDS Size']} bytes in a kernel that uses none")
    return bad


def _hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def sources():
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC)
                  if f.endswith(".hip") or f.endswith(".cpp"))


def _compile(hipcc, src):
    obj = os.path.join(BUILD_DIR, os.path.basename(src) + ".o")
    cmd = [hipcc, *FLAGS, *SOURCE_FLAGS.get(os.path.basename(src), []), *REMARKS, "-x", "hip", "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    usage = parse_resource_remarks(r.stderr)
    # hipcc's host pass does not know the packed-fp32 feature; keep other warnings (the
    # resource remarks and their source excerpts go to the report instead)
    lines, skip = [], False
    for ln in r.stderr.splitlines():
        if "remark:" in ln:
            skip = True
            continue
        if skip and (ln.startswith(" ") or not ln.strip()):
            continue
        skip = False
        if "packed-fp32-ops" not in ln and "not a recognized feature" not in ln and ln.strip():
            lines.append(ln)
    if lines:
        sys.stderr.write("\n".join(lines) + "\n")
    return obj, usage


def build(verbose: bool = True) -> str:
    hipcc = _hipcc()
    os.makedirs(BUILD_DIR, exist_ok=True)
    srcs = sources()
    with ThreadPoolExecutor(min(8, len(srcs))) as ex:
        done = list(ex.map(lambda s: _compile(hipcc, s), srcs))
    objs = [o for o, _ in done]
    usage = {}
    for _, u in done:
        usage.update(u)
    with open(RESOURCE_REPORT, "w") as f:
        f.write("kernel\tVGPRs\tAGPRs\tSGPRs\tSGPR spills (to vector lanes)\tVGPR spills (to AGPRs)\t"
                "scratch B/lane\tLDS B\twaves/SIMD\n")
        for name in sorted(usage):
            u = usage[name]
            if "kernel" in name and not name.startswith("__"):
                f.write(f"{name}\t{u.get('VGPRs')}\t{u.get('AGPRs')}\t{u.get('TotalSGPRs')}\t{u.get('SGPRs Spill')}\t"
                        f"{u.get('VGPRs Spill')}\t"
                        f"{u.get('ScratchSize')}\t{u.get('LDS Size')}\t{u.get('Occupancy')}\n")
    bad = check_resources(usage)
    if bad:
        raise RuntimeError("kernel resource check failed:\n  " + "\n  ".join(bad))
    tmp = LIB + ".tmp"
    cmd = [hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB} from {len(srcs)} sources")
    return LIB


if __name__ == "__main__":
    build()
