"""Builds libmlaverify.so (the gfx950 HIP kernels and the C ABI) in place with hipcc.

Usage: python -m mla_tree_verify_mlaverify_amd.build [--verbose]
"""

from __future__ import annotations

import os
import re
import shutil
import subprocess
import sys

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG_DIR)
CSRC = os.path.join(PKG_DIR, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB_NAME = "libmlaverify.so"
LIB_PATH = os.path.join(PKG_DIR, LIB_NAME)
SOURCES = ("api.hip", "kernels.hip", "relocate.hip", "accept.hip")
ARCH = "gfx950"

HIPCC_FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-Wall",
    # keep the compiler from forming packed fp32 VALU ops (v_pk_*_f32)
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # the partial kernel keeps its output accumulator in AGPRs that only its inline asm
    # touches; the compiler must never spill VGPRs into them (spills go to scratch instead)
    "-mllvm", "-amdgpu-spill-vgpr-to-agpr=0",
    # score MFMAs accumulate in VGPRs (the AGPRs are all taken by the output accumulator)
    "-mllvm", "-amdgpu-mfma-vgpr-form=1",
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: install ROCm or set HIPCC")


def audit_agprs(asm: str) -> list[str]:
    """AGPR uses outside inline asm in compiler output (each would clobber the accumulator)."""
    bad, in_asm, func = [], False, "?"
    agpr = re.compile(r"(?<![\w.])a(\d+|\[\d+:\d+\])")
    for line in asm.splitlines():
        st = line.strip()
        if st.startswith(";;#ASMSTART"):
            in_asm = True
        elif st.startswith(";;#ASMEND"):
            in_asm = False
        elif re.match(r"[A-Za-z_][\w$.]*:", line):  # a symbol (not a block comment or local label)
            func = line.split(":", 1)[0]
        elif not in_asm and line.startswith("\t") and st and st[0].isalpha():
            code = st.split(";", 1)[0]
            # gather_helper runs only on waves that hold no rows and end right after it, so
            # nothing there can meet the output accumulator
            if agpr.search(code) and "gather_helper" not in func:
                bad.append(f"{func}: {code}")
    return bad


def _vgprs(operand: str) -> set[int]:
    m = re.fullmatch(r"v\[(\d+):(\d+)\]", operand) or re.fullmatch(r"v(\d+)", operand)
    if not m:
        return set()
    lo = int(m.group(1))
    hi = int(m.group(2)) if m.lastindex == 2 else lo
    return set(range(lo, hi + 1))


def audit_mfma_operands(asm: str, wait_states: int = 2) -> list[str]:
    """Inline-asm MFMAs carry no wait states of their own, so check that no VALU instruction
    writes one of their A/B operands within `wait_states` wait states before them (the
    VALU-write -> MFMA-read hazard).  A label inside that window is reported too, since the
    instruction reaching it from elsewhere is not known here."""
    bad, in_asm, func, recent = [], False, "?", []
    for line in asm.splitlines():
        st = line.strip()
        if st.startswith(";;#ASMSTART"):
            in_asm = True
            continue
        if st.startswith(";;#ASMEND"):
            in_asm = False
            continue
        if line and not line[0].isspace() and st.endswith(":"):
            if st.startswith("."):
                recent.append(("<label>", ""))  # a branch target
            else:
                func, recent = st[:-1], []  # a new function: nothing precedes its entry
            continue
        if not (line.startswith("\t") and st and st[0].isalpha()):
            continue
        code = st.split(";", 1)[0].strip()
        op, _, args = code.partition(" ")
        ops = [a.strip() for a in args.split(",")] if args else []
        if in_asm and op.startswith("v_mfma") and len(ops) >= 3:
            srcs = _vgprs(ops[1]) | _vgprs(ops[2])
            ws = 0
            for pop, pargs in reversed(recent):
                if ws >= wait_states:
                    break
                if pop == "<label>":
                    bad.append(f"{func}: label within {wait_states} wait states before {code}")
                    break
                if pop.startswith("v_") and not pop.startswith("v_mfma") and pargs and _vgprs(pargs[0]) & srcs:
                    bad.append(f"{func}: {pop} {', '.join(pargs)} -> {code}")
                    break
                m = re.fullmatch(r"s_nop", pop)
                ws += (int(pargs[0], 0) + 1) if m and pargs else 1
        recent.append((op, ops))
        recent = recent[-8:]
    return bad


def check_device_code(src: str, verbose: bool = False) -> None:
    """Compile src to gfx950 assembly and refuse it if the compiler touched an AGPR or placed a
    VALU write of an asm MFMA operand inside the hazard window."""
    cmd = [hipcc(), *HIPCC_FLAGS, "-I", INCLUDE, "-I", CSRC, "--cuda-device-only", "-S", src, "-o", "-"]
    out = subprocess.run(cmd, capture_output=True, text=True)
    if out.returncode:
        raise RuntimeError("hipcc -S failed:\n" + out.stderr)
    bad = audit_agprs(out.stdout)
    if bad:
        raise RuntimeError("compiler-generated AGPR accesses in " + src + ":\n  " + "\n  ".join(bad[:20]))
    bad = audit_mfma_operands(out.stdout)
    if bad:
        raise RuntimeError("VALU write too close before an inline-asm MFMA in " + src + ":\n  " + "\n  ".join(bad[:20]))
    if verbose:
        for m in re.finditer(r"\.name:\s+(\S+)[\s\S]*?\.private_segment_fixed_size:\s+(\d+)[\s\S]*?\.vgpr_count:\s+(\d+)",
                             out.stdout):
            print(f"{m.group(1)}: scratch {m.group(2)} B, vgpr+agpr {m.group(3)}", flush=True)


def build(verbose: bool = False) -> str:
    """Compile every source for gfx950 and link the shared library; returns its path."""
    objs = []
    build_dir = os.path.join(PKG_DIR, "_build")
    os.makedirs(build_dir, exist_ok=True)
    procs = []
    for src in SOURCES:
        obj = os.path.join(build_dir, src.replace(".hip", ".o"))
        cmd = [hipcc(), *HIPCC_FLAGS, "-I", INCLUDE, "-I", CSRC, "-c", os.path.join(CSRC, src), "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append((cmd, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)))
        objs.append(obj)
    failed = False
    for cmd, p in procs:
        out, _ = p.communicate()
        out = "\n".join(line for line in out.splitlines() if "packed-fp32-ops" not in line)
        if out.strip() and (verbose or p.returncode):
            print(out, file=sys.stderr)
        if p.returncode:
            failed = True
    if failed:
        raise RuntimeError("hipcc failed")
    check_device_code(os.path.join(CSRC, "kernels.hip"), verbose)
    tmp = LIB_PATH + ".tmp"
    link = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    if verbose:
        print(" ".join(link), flush=True)
    subprocess.run(link, check=True)
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    print(build(verbose="--verbose" in sys.argv))
