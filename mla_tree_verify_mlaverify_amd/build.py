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
SOURCES = ("api.hip", "kernels.hip", "relocate.hip", "accept.hip", "probe.hip")
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


HELPER_MARK = "mlv-helper-waves"  # inline-asm comment at the entry of the helper waves' code


def _functions(asm: str):
    """(name, lines) of every function in the assembly."""
    name, body = None, []
    for line in asm.splitlines():
        if re.match(r"[A-Za-z_][\w$.]*:", line) and not line.startswith(".L"):
            if name:
                yield name, body
            name, body = line.split(":", 1)[0], []
        elif name:
            body.append(line)
    if name:
        yield name, body


def _blocks(lines):
    """Split a function body into basic blocks: [(label, [(line, in_asm)]), ...] and successor lists.
    A block starts at a label or a '; %bb.N:' comment, or after a terminator.  The helper-wave
    marker also starts a block (the code before it and after it are kept apart)."""
    blocks, cur, in_asm = [], None, False

    def new(label):
        nonlocal cur
        cur = [label, []]
        blocks.append(cur)

    new("<entry>")
    for line in lines:
        st = line.strip()
        if st.startswith(";;#ASMSTART"):
            in_asm = True
            continue
        if st.startswith(";;#ASMEND"):
            in_asm = False
            continue
        m = re.match(r"(\.LBB\w+):", line) or re.match(r"; (%bb\.\d+):", line)
        if m:
            new(m.group(1))
            continue
        if in_asm and HELPER_MARK in st:
            new("<helper>")
            continue
        if line.startswith("\t") and st and st[0].isalpha():
            cur[1].append((st.split(";", 1)[0].strip(), in_asm))
    labels = {b[0]: i for i, b in enumerate(blocks)}
    succ = []
    for i, (_, ins) in enumerate(blocks):
        out, fall = [], True
        for code, _asm in ins:
            op, _, arg = code.partition(" ")
            if op.startswith("s_cbranch") or op == "s_branch":
                tgt = arg.strip()
                if tgt in labels:
                    out.append(labels[tgt])
                if op == "s_branch":
                    fall = False
            elif op in ("s_endpgm", "s_setpc_b64"):
                fall = False
        if fall and i + 1 < len(blocks):
            out.append(i + 1)
        succ.append(out)
    return blocks, succ


def audit_agprs(asm: str) -> list[str]:
    """AGPR uses outside inline asm that the waves holding the output accumulator can execute.

    Only the inline-asm MFMAs and accumulator moves may name an AGPR on those waves.  The
    helper waves (which hold no rows) may: their code is entered at the HELPER_MARK marker,
    and everything reachable from the kernel entry without passing the marker is audited.
    Code the compiler shares between both paths is therefore audited too."""
    bad = []
    agpr = re.compile(r"(?<![\w.])a(\d+|\[\d+:\d+\])")
    for func, lines in _functions(asm):
        blocks, succ = _blocks(lines)
        helper = {i for i, b in enumerate(blocks) if b[0] == "<helper>"}
        seen, stack = {0}, [0]
        while stack:
            i = stack.pop()
            for j in succ[i]:
                if j not in seen and j not in helper:
                    seen.add(j)
                    stack.append(j)
        for i in sorted(seen):
            for code, in_asm in blocks[i][1]:
                if not in_asm and agpr.search(code):
                    bad.append(f"{func}: {code}")
    return bad


def audit_m0(asm: str) -> list[str]:
    """Instructions outside inline asm that name m0.  The LDS-DMA gathers set m0 inside their
    asm statements and declare it clobbered, which the compiler does not honour for reserved
    registers, so compiler-generated code must not keep anything live in m0."""
    bad, in_asm, func = [], False, "?"
    for line in asm.splitlines():
        st = line.strip()
        if st.startswith(";;#ASMSTART"):
            in_asm = True
        elif st.startswith(";;#ASMEND"):
            in_asm = False
        elif re.match(r"[A-Za-z_][\w$.]*:", line):
            func = line.split(":", 1)[0]
        elif not in_asm and line.startswith("\t") and st and st[0].isalpha():
            code = st.split(";", 1)[0]
            if re.search(r"\bm0\b", code):
                bad.append(f"{func}: {code}")
    return bad


def kernel_resources(asm: str) -> list[tuple[str, int, int]]:
    """(kernel, private segment bytes, VGPR+AGPR count) of every kernel in the assembly."""
    return [(m.group(1), int(m.group(2)), int(m.group(3))) for m in re.finditer(
        r"\.name:\s+(\S+)[\s\S]*?\.private_segment_fixed_size:\s+(\d+)[\s\S]*?\.vgpr_count:\s+(\d+)", asm)]


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
        if st.startswith(";"):
            continue  # a comment line (block comments such as "; %bb.3:" included)
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
    bad = audit_m0(out.stdout)
    if bad:
        raise RuntimeError("compiler-generated m0 accesses in " + src + ":\n  " + "\n  ".join(bad[:20]))
    res = kernel_resources(out.stdout)
    if not res:
        raise RuntimeError("no kernel metadata found in the assembly of " + src)
    # spills to scratch are slow and, in the partial kernel, a sign that the register plan broke
    spilled = [f"{n}: {b} B" for n, b, _ in res if b > 0]
    if spilled:
        raise RuntimeError("kernels with private (scratch) memory in " + src + ":\n  " + "\n  ".join(spilled))
    if verbose:
        for n, b, v in res:
            print(f"{n}: scratch {b} B, vgpr+agpr {v}", flush=True)


ASAN_LIB_PATH = os.path.join(PKG_DIR, "libmlaverify_asan.so")


def asan_runtime() -> str:
    """clang's shared AddressSanitizer runtime of the ROCm toolchain (preloaded by the ASan tests)."""
    import glob

    hits = sorted(glob.glob(os.path.join(os.path.dirname(os.path.dirname(hipcc())), "llvm", "lib", "clang", "*", "lib",
                                         "linux", "libclang_rt.asan-x86_64.so")))
    if not hits:
        raise RuntimeError("clang's libclang_rt.asan-x86_64.so not found next to hipcc")
    return hits[-1]


def build_asan(verbose: bool = False) -> str:
    """The same library with the host code built under AddressSanitizer (device code unchanged), for
    CPU tests of the C ABI's host paths.  Load it with asan_runtime() preloaded."""
    build_dir = os.path.join(PKG_DIR, "_build", "asan")
    os.makedirs(build_dir, exist_ok=True)
    flags = [f for f in HIPCC_FLAGS if f != "-O3"] + ["-O1", "-g", "-Xarch_host", "-fsanitize=address",
                                                        "-Xarch_host", "-fno-omit-frame-pointer"]
    objs, procs = [], []
    for src in SOURCES:
        obj = os.path.join(build_dir, src.replace(".hip", ".o"))
        cmd = [hipcc(), *flags, "-I", INCLUDE, "-I", CSRC, "-c", os.path.join(CSRC, src), "-o", obj]
        procs.append(subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True))
        objs.append(obj)
    for p in procs:
        out, _ = p.communicate()
        if p.returncode:
            raise RuntimeError("hipcc (ASan build) failed:\n" + out[-4000:])
    tmp = ASAN_LIB_PATH + ".tmp"
    subprocess.run([hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-Xarch_host", "-fsanitize=address",
                    "-shared-libasan", "-o", tmp, *objs], check=True)
    os.replace(tmp, ASAN_LIB_PATH)
    return ASAN_LIB_PATH


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
    if "--asan" in sys.argv:
        print(build_asan(verbose="--verbose" in sys.argv))
