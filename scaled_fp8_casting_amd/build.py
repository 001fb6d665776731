"""Build libnarrowcast.so (HIP, gfx950) in-tree.

    python -m scaled_fp8_casting_amd.build [--jobs N]

Each .hip source under csrc/ is compiled to an object in parallel, then the
objects are linked into scaled_fp8_casting_amd/libnarrowcast.so.  Always
rebuilds.  The device assembly of every source is scanned as well
(scan_device_asm); the build fails if a select or conditional branch takes
its condition from a carry flag.
"""

import argparse
import concurrent.futures as cf
import os
import re
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libnarrowcast.so")
ARCH = "gfx950"

HIPCC_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    "-I", os.path.join(ROOT, "include"), "-I", CSRC,
    # packed fp32 instructions stay off (plain float code only)
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
]


def hipcc():
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def sources():
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".hip"))


# Scalar instructions that write the condition code SCC.  Carry-producing
# arithmetic is listed separately: a select or conditional branch whose
# nearest SCC writer is one of these reads a carry, never a comparison.
_SCC_CARRY = re.compile(r"^s_(add|sub|addc|subb)_[iu]32$|^s_addk_i32$|^s_lshl[1-4]_add_u32$")
_SCC_OTHER = re.compile(
    r"^s_(cmp|cmpk|bitcmp[01])_|^s_(and|or|xor|andn[12]|orn[12]|nand|nor|xnor)_(b32|b64|saveexec_b64)$"
    r"|^s_(lshl|lshr|ashr)_[bi](32|64)$|^s_(min|max)_[iu]32$|^s_bfe_|^s_(not|wqm|bcnt[01]|quadmask)_"
    r"|^s_abs_i32$|^s_absdiff_i32$")
_SCC_READ = re.compile(r"^s_cselect_|^s_cbranch_scc[01]$|^s_cmovk?_")


def scan_device_asm(text):
    """Selects and branches on SCC whose nearest SCC writer in the same basic
    block is carry arithmetic: the signature of a vector compare whose copy
    into SCC was dropped by code generation.  Returns (line, reader, writer)."""
    found = []
    writer = None
    for no, raw in enumerate(text.splitlines(), 1):
        line = raw.split(";")[0].strip()
        if line.endswith(":"):              # a label starts a new block
            writer = None
            continue
        if not line or line.startswith("."):
            continue
        op = line.split()[0]
        # s_cselect_b64 m, -1, 0 right after carry arithmetic saves the carry
        # as a mask (wide integer arithmetic): intended, not reported
        carry_save = op == "s_cselect_b64" and line.replace(" ", "").endswith(",-1,0")
        if (_SCC_READ.match(op) and not carry_save and writer is not None
                and _SCC_CARRY.match(writer[1])):
            found.append((no, line, writer[0]))
        if _SCC_CARRY.match(op) or _SCC_OTHER.match(op):
            writer = (line, op)
        if op.startswith("s_cbranch") or op in ("s_branch", "s_endpgm", "s_setpc_b64"):
            writer = None
    return found


def _check_asm(src, extra):
    asm = os.path.join(BUILD, os.path.basename(src) + ".s")
    cmd = [hipcc(), *HIPCC_FLAGS, *extra, "--cuda-device-only", "-S", src, "-o", asm]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"device assembly failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    with open(asm) as f:
        bad = scan_device_asm(f.read())
    if bad:
        rows = "\n".join(f"  {asm}:{no}: {rd}   (SCC from: {wr})" for no, rd, wr in bad[:20])
        raise RuntimeError(f"device code selects on a carry flag ({len(bad)} sites):\n{rows}")
    return asm


def _compile(src, extra):
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    cmd = [hipcc(), *HIPCC_FLAGS, *extra, "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return obj


def build(jobs: int = 8, extra=()) -> str:
    os.makedirs(BUILD, exist_ok=True)
    srcs = sources()
    with cf.ThreadPoolExecutor(max_workers=max(1, min(jobs, 2 * len(srcs)))) as ex:
        checks = [ex.submit(_check_asm, s, list(extra)) for s in srcs]
        objs = list(ex.map(lambda s: _compile(s, list(extra)), srcs))
        for c in checks:
            c.result()
    tmp = LIB + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    return LIB


def main(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("--jobs", type=int, default=8)
    a = ap.parse_args(argv)
    print(build(a.jobs))


if __name__ == "__main__":
    sys.exit(main())
