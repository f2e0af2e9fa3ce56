"""Build libattn_bwd.so (HIP, gfx950) in-tree.

    python -m attention_backward_amd.build [--out PATH] [-D NAME=VALUE ...]

Compiles every csrc/*.hip for gfx950 with hipcc and links them into
attention_backward_amd/libattn_bwd.so (or PATH, with its objects beside it; -D passes a
preprocessor definition, e.g. a tile parameter, to every file).  Packed-fp32 instruction selection is disabled
(``-target-feature -packed-fp32-ops``); float atomics, where used, are the hardware ones.

Each source is also compiled to device assembly, and the build fails if compiler-generated code
anywhere in it uses the m0 register, which the inline-assembly global/buffer->LDS copies overwrite
(see ``m0_outside_inline_asm``).
"""
from __future__ import annotations

import concurrent.futures as cf
import glob
import os
import re
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libattn_bwd.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

CFLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-munsafe-fp-atomics",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # MFMA results and accumulators in VGPRs: the kernels are laid out to fit 256 VGPRs per
    # wave, and AGPR-form accumulators made the register allocator shuttle them every step.
    "-mllvm", "-amdgpu-mfma-vgpr-form=1",
    "-I", INCLUDE,
    "-I", CSRC,
]
# Kernels that run one wave per SIMD (up to 512 registers) keep their accumulators in AGPRs, where
# the MFMAs read and write them directly; the VGPR form would park them there anyway and copy
# them back and forth every step.
AGPR_FORM = {"sparse_dkdv.hip", "sparse_bwd.hip"}


def _flags(src: str):
    if os.path.basename(src) not in AGPR_FORM:
        return CFLAGS
    i = CFLAGS.index("-amdgpu-mfma-vgpr-form=1")
    return CFLAGS[: i - 1] + CFLAGS[i + 1:]


def _compile(src: str, build_dir: str = BUILD, defines=()) -> str:
    obj = os.path.join(build_dir, os.path.basename(src) + ".o")
    cmd = [HIPCC, *_flags(src), *[f"-D{d}" for d in defines], "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stdout}\n{r.stderr}")
    asm = os.path.join(build_dir, os.path.basename(src) + ".s")
    cmd = [HIPCC, *_flags(src), *[f"-D{d}" for d in defines], "--cuda-device-only", "-S", src, "-o", asm]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc -S failed for {src}:\n{r.stdout}\n{r.stderr}")
    bad = m0_outside_inline_asm(asm)
    if bad:
        raise RuntimeError(f"{src}: compiler-generated code uses m0, which the global/buffer->LDS copy "
                           f"statements overwrite without restoring it:\n" + "\n".join(bad[:20]))
    return obj


_M0 = re.compile(r"(?<![\w$])m0(?![\w])")


def m0_outside_inline_asm(asm_path: str):
    """Lines of the device assembly that name m0 outside inline-assembly statements.

    The direct global->LDS copies (common.h: g2lds16/g2lds4/b2lds16/b2lds4) set m0 to their LDS
    destination from inline assembly; the compiler is told m0 is clobbered, but it may not preserve
    a value of its own there across the statement.  A kernel whose compiler-generated code reads or
    writes m0 (indexed register moves, messages, ...) could then see the copies' value, so the build
    refuses it.  Inline-assembly statements sit between ;;#ASMSTART and ;;#ASMEND markers."""
    bad, inside, func = [], False, "?"
    with open(asm_path) as fh:
        for n, line in enumerate(fh, 1):
            t = line.strip()
            if t.startswith(";;#ASMSTART"):
                inside = True
                continue
            if t.startswith(";;#ASMEND"):
                inside = False
                continue
            if t.endswith(":") and not t.startswith((".", ";")):
                func = t[:-1]
            code = t.split(";", 1)[0]
            if not inside and code and not code.startswith(".") and _M0.search(code):
                bad.append(f"  {os.path.basename(asm_path)}:{n} in {func}: {code}")
    return bad


def build(verbose: bool = False, out: str = LIB, defines=()) -> str:
    build_dir = BUILD if out == LIB else out + ".objs"
    os.makedirs(build_dir, exist_ok=True)
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    with cf.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(lambda s_: _compile(s_, build_dir, defines), srcs))
    tmp = out + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, out)
    if verbose:
        print(f"built {out}")
    return out


if __name__ == "__main__":
    import argparse

    ap = argparse.ArgumentParser()
    ap.add_argument("--out", default=LIB)
    ap.add_argument("-D", dest="defines", action="append", default=[])
    a = ap.parse_args()
    build(verbose=True, out=os.path.abspath(a.out), defines=a.defines)
    sys.exit(0)
