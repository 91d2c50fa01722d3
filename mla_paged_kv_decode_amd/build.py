"""Build libmla_decode.so (gfx950 only) in-tree with hipcc.

The library holds the host runtime (csrc/mla_api.cpp) and the HIP kernels
(csrc/mla_kernels.hip).  The compiler's kernel-resource remarks are parsed
into a per-kernel report (VGPRs, AGPRs, scratch, LDS, spills) printed after
the build and kept next to the library as kernel_resources.txt.  The build
fails if a kernel of the default paths spills a VGPR (spill_gate), or if the
assembly shows an MFMA hazard or a spill inside a tile loop (asm_lint).
"""
from __future__ import annotations

import os
import re
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
LIB = os.path.join(HERE, "libmla_decode.so")
SOURCES = [os.path.join(HERE, "csrc", "mla_kernels.hip"), os.path.join(HERE, "csrc", "mla_api.cpp")]
# The HBM -> LDS streaming probe bench.py measures the achievable read rate with: a library of its
# own, outside the decode library's C ABI.
PROBE_LIB = os.path.join(HERE, "libmla_stream_probe.so")
PROBE_SOURCES = [os.path.join(HERE, "csrc", "stream_probe.hip")]
ARCH = "gfx950"

FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    "-I", os.path.join(ROOT, "include"),
    # keep hipcc from forming packed fp32 instructions (v_pk_*_f32)
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-inline-asm",
    "-Rpass-analysis=kernel-resource-usage",
]


def _hipcc() -> str:
    for cand in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build the library)")


def parse_resources(text: str) -> dict:
    kernels, cur = {}, None
    for line in text.splitlines():
        m = re.search(r"remark: Function Name: (\S+)", line)
        if m:
            cur = kernels.setdefault(m.group(1), {})
            continue
        m = re.search(r"remark:\s+([A-Za-z][A-Za-z /\[\]]*?):\s+(\d+)", line)
        if m and cur is not None:
            cur[m.group(1).strip()] = int(m.group(2))
    return kernels


# Kernels that must not spill a VGPR: the split-KV instantiations the default paths run over pages
# of at least a tile (E4M3 without a window; every 16-bit dtype and layout, with or without one),
# the merges and the pack kernel.  The others (E4M3 with a window or over short pages in the
# four-wave kernel, the twelve-wave kernel, 16-bit kernels over short pages) spill a few values
# outside their tile loop, which the assembly lint keeps out of the loop itself.
_SPLIT = re.compile(r"mla_split_kv_partialILi(\d)ELb([01])ELb([01])ELb([01])E")


def must_not_spill(name: str) -> bool:
    m = _SPLIT.search(name)
    if m:
        dt, fast, win = int(m.group(1)), m.group(2) == "1", m.group(3) == "1"
        return fast and (dt != 2 or not win)
    return "mla_combine" in name or "mla_kv_pack" in name


def spill_gate(resources: dict) -> list:
    """Names (with their VGPR spill counts) of the kernels that must not spill but do."""
    return [f"{k}: {r.get('VGPRs Spill')} VGPRs spilled" for k, r in sorted(resources.items())
            if must_not_spill(k) and r.get("VGPRs Spill", 0) != 0]


def lint_assembly() -> None:
    """Compile the kernels to gfx950 assembly and check the inline-asm MFMA hazards (asm_lint)."""
    import tempfile

    sys.path.insert(0, HERE)
    import asm_lint

    with tempfile.TemporaryDirectory() as d:
        out = os.path.join(d, "mla_kernels.s")
        # (-fPIC as in the library build: it changes the device code's register allocation)
        cmd = [_hipcc(), f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "--cuda-device-only", "-S",
               "-I", os.path.join(ROOT, "include"), "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
               "-Wno-inline-asm", SOURCES[0], "-o", out]
        proc = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
        if proc.returncode != 0:
            sys.stderr.write(proc.stdout)
            raise RuntimeError(f"hipcc -S failed ({proc.returncode})")
        with open(out) as f:
            report = asm_lint.lint(f.read())
    bad = {k: v for k, v in report.items() if v}
    if not report:
        raise RuntimeError("asm lint found no split-KV kernel in the assembly")
    if bad:
        for k, v in bad.items():
            sys.stderr.write(f"{k}:\n  " + "\n  ".join(v[:20]) + "\n")
        raise RuntimeError("MFMA hazards or loop spills in the generated assembly (see above)")


def build(verbose: bool = False) -> str:
    tmp = LIB + ".tmp"
    cmd = [_hipcc(), *FLAGS, *SOURCES, "-o", tmp]
    proc = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    if proc.returncode != 0:
        sys.stderr.write(proc.stdout)
        raise RuntimeError(f"hipcc failed ({proc.returncode})")
    res = parse_resources(proc.stdout)
    try:
        spills = spill_gate(res)
        if spills:
            raise RuntimeError("VGPR spills in kernels that must not spill:\n  " + "\n  ".join(spills))
        lint_assembly()
    except Exception:
        os.remove(tmp)
        raise
    os.replace(tmp, LIB)
    lines = []
    for name, r in sorted(res.items()):
        lines.append(
            f"{name}: VGPRs={r.get('VGPRs')} AGPRs={r.get('AGPRs')} scratch={r.get('ScratchSize [bytes/lane]')} "
            f"LDS={r.get('LDS Size [bytes/block]')} vgpr_spill={r.get('VGPRs Spill')} sgpr_spill={r.get('SGPRs Spill')} "
            f"occupancy={r.get('Occupancy [waves/SIMD]')}")
    with open(os.path.join(HERE, "kernel_resources.txt"), "w") as f:
        f.write("\n".join(lines) + "\n")
    if verbose:
        print("\n".join(lines))
    build_probe()
    return LIB


def build_probe() -> str:
    tmp = PROBE_LIB + ".tmp"
    flags = [f for f in FLAGS if not f.startswith("-Rpass")]
    proc = subprocess.run([_hipcc(), *flags, *PROBE_SOURCES, "-o", tmp], stdout=subprocess.PIPE,
                          stderr=subprocess.STDOUT, text=True)
    if proc.returncode != 0:
        sys.stderr.write(proc.stdout)
        raise RuntimeError(f"hipcc failed on the streaming probe ({proc.returncode})")
    os.replace(tmp, PROBE_LIB)
    return PROBE_LIB


if __name__ == "__main__":
    print(build(verbose=True))
