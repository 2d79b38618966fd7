"""Builds libpsispec.so (hand-written HIP for gfx950) in-tree with hipcc.

Every .hip file under csrc/ is compiled for gfx950 only, in parallel, then
linked into lossless_speculative_verification_amd/libpsispec.so. Packed FP32
instruction selection is disabled for every source.

It also writes kernel_code.json beside the library: a hash of the gfx950
assembly of each k_stats32 instance, so that measurements taken on that
kernel (its HBM byte counters) can be matched to the code that runs. And it
checks the assembly of lmhead.hip: its direct global-to-LDS loads set M0 in
asm statements, which is only safe while the compiler itself leaves M0 alone
in that file (M0 cannot be declared clobbered).
"""
from __future__ import annotations

import glob
import hashlib
import json
import os
import re
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(ROOT, "_build", "psispec")
LIB = os.path.join(HERE, "libpsispec.so")
CODE_JSON = os.path.join(HERE, "kernel_code.json")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-Wall",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-I", os.path.join(ROOT, "include"), "-I", CSRC]


def sources():
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")))


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    procs = []
    objs = []
    for src in sources():
        obj = os.path.join(BUILD, os.path.basename(src) + ".o")
        objs.append(obj)
        cmd = [HIPCC, *FLAGS, "-c", src, "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append((src, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT)))
    failed = []
    for src, p in procs:
        out, _ = p.communicate()
        text = out.decode(errors="replace")
        # hipcc's host pass does not know the gfx950-only feature flag; that notice is harmless
        lines = [l for l in text.splitlines() if "packed-fp32-ops" not in l]
        if lines and (verbose or p.returncode != 0):
            print("\n".join(lines), file=sys.stderr)
        if p.returncode != 0:
            failed.append(src)
    if failed:
        raise RuntimeError("hipcc failed for: " + ", ".join(failed))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, *objs]
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    write_code_hashes()
    check_m0()
    return LIB


def function_hashes(asm: str, pattern: str) -> dict:
    """sha256 (16 hex digits) of the instructions of every function whose
    mangled name matches `pattern`, comments and blank lines dropped, and the
    function number in local branch labels (.LBB<function>_<block>) removed,
    so that adding a function to the file does not change the hash."""
    out = {}
    lines = asm.splitlines()
    for i, line in enumerate(lines):
        m = re.match(r"^(_Z\S+):", line)
        if not m or not re.search(pattern, m.group(1)):
            continue
        body = []
        for l in lines[i + 1:]:
            if l.startswith(".Lfunc_end"):
                break
            l = l.split(";", 1)[0].strip()
            if l:
                body.append(re.sub(r"\.LBB\d+_", ".LBB_", l))
        out[m.group(1)] = hashlib.sha256("\n".join(body).encode()).hexdigest()[:16]
    return out


def write_code_hashes() -> None:
    os.makedirs(BUILD, exist_ok=True)
    asm = os.path.join(BUILD, "stats.s")
    cmd = [HIPCC, *[f for f in FLAGS if f != "-fPIC"], "--cuda-device-only", "-S",
           os.path.join(CSRC, "stats.hip"), "-o", asm]
    subprocess.run(cmd, check=True, stdout=subprocess.DEVNULL, stderr=subprocess.DEVNULL)
    with open(asm) as f:
        hashes = function_hashes(f.read(), r"k_stats32")
    with open(CODE_JSON, "w") as f:
        json.dump(hashes, f, indent=1, sort_keys=True)


def m0_violations(asm: str) -> list:
    """Instructions that touch M0 other than the direct-load sequence
    `s_mov_b32 m0, sN` / `s_nop 0` / `global_load_lds_dwordx4`."""
    lines = [l.split(";", 1)[0].strip() for l in asm.splitlines()]
    lines = [l for l in lines if l and not l.startswith((".", "_")) and not l.endswith(":")]
    bad = []
    for i, l in enumerate(lines):
        if not re.search(r"\bm0\b", l):
            continue
        ok = (re.match(r"^s_mov_b32\s+m0,\s*s\d+$", l) and i + 2 < len(lines) and lines[i + 1] == "s_nop 0"
              and lines[i + 2].startswith("global_load_lds_dwordx4"))
        if not ok:
            bad.append(l)
    return bad


def check_m0() -> None:
    asm = os.path.join(BUILD, "lmhead.s")
    cmd = [HIPCC, *[f for f in FLAGS if f != "-fPIC"], "--cuda-device-only", "-S",
           os.path.join(CSRC, "lmhead.hip"), "-o", asm]
    subprocess.run(cmd, check=True, stdout=subprocess.DEVNULL, stderr=subprocess.DEVNULL)
    with open(asm) as f:
        bad = m0_violations(f.read())
    if bad:
        raise RuntimeError("lmhead.hip: M0 used outside the direct-load sequence: " + "; ".join(bad[:5]))


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
