"""Compile the gfx950 HIP library (libmla_hip.so) in-tree with hipcc.

    python -m decode_attention_03_amd.build

Every HIP source is compiled for gfx950 only, with packed-FP32 instruction
selection disabled, and linked into decode_attention_03_amd/libmla_hip.so.
"""

import hashlib
import json
import os
import re
import subprocess
import sys
import tempfile
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD_DIR = os.path.join(PKG, "_build")
LIB_NAME = "libmla_hip.so"
LIB_PATH = os.path.join(PKG, LIB_NAME)
# the same sources with MLA_DEBUG=1: device-side checks of the caller contract
DEBUG_BUILD_DIR = os.path.join(PKG, "_build_debug")
DEBUG_LIB_PATH = os.path.join(PKG, "libmla_hip_debug.so")
# sha256 of the gfx950 assembly of each kernel source, written by build()
DEVICE_CODE_PATH = os.path.join(BUILD_DIR, "device_code.json")
KERNEL_SOURCES = ["mla_split.hip", "mla_merge.hip", "mla_kv.hip", "mla_peaks.hip"]

SOURCES = ["mla_split.hip", "mla_merge.hip", "mla_kv.hip", "mla_peaks.hip", "mla_api.cpp"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-Wall",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    f"-I{INCLUDE}",
    f"-I{CSRC}",
]


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in res.stdout.splitlines() if "packed-fp32-ops" not in l)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{' '.join(cmd)}\n{out}")
    if verbose and out.strip():
        print(out)
    return out


def _demangle(names):
    """Demangled C++ names (c++filt), or the names unchanged without it."""
    try:
        res = subprocess.run(["c++filt"], input="\n".join(names), stdout=subprocess.PIPE, text=True,
                             check=True)
        out = res.stdout.splitlines()
        return out if len(out) == len(names) else list(names)
    except (OSError, subprocess.CalledProcessError):
        return list(names)


def device_code_sha256(src, verbose=False):
    """sha256 of the gfx950 assembly hipcc emits for one kernel source, with the
    per-compilation unit id symbol (the only part that changes from one
    compile of the same source to the next) and the function index in local
    labels and comments (which another kernel added to or removed from the
    source shifts) normalised, and the sha256 of
    each kernel function's own assembly (label to end of function) by
    demangled name.  Host-only edits of a source leave them unchanged; a
    change of a kernel's device code changes its hash and the file's, and
    leaves the hashes of the source's other kernels as they were."""
    with tempfile.TemporaryDirectory() as tmp:
        out = os.path.join(tmp, "dev.s")
        _run([HIPCC] + FLAGS + ["--cuda-device-only", "-S", os.path.join(CSRC, src), "-o", out], verbose)
        text = open(out).read()
    whole, bodies = assembly_sha256(text)
    names = sorted(bodies)
    return whole, dict(zip(_demangle(names), (bodies[n] for n in names)))


def assembly_sha256(text):
    """(sha256 of the whole normalised assembly, {mangled kernel name: sha256
    of that function's normalised assembly}) for hipcc's assembly `text`: the
    compile-unit id symbol, the function index in local labels and the
    compiler's comments are normalised away (see device_code_sha256)."""
    text = re.sub(r"__hip_cuid_[0-9a-f]+", "__hip_cuid", text)
    # local labels carry the function's index in the file (.LBB<f>_<n>,
    # .Lfunc_end<f>), as do the compiler's comments: adding or removing
    # another kernel renumbers them.  Comments and trailing blanks go.
    text = re.sub(r"\.L(BB|func_end|tmp)\d+", r".L\1", text)
    text = "\n".join(l for l in (re.sub(r"\s*;.*$", "", l).rstrip() for l in text.splitlines()) if l)
    bodies = {}
    cur, lines = None, []
    for line in text.splitlines():
        m = re.match(r"^(_Z\S+):", line)
        if m:
            cur, lines = m.group(1), []
        if cur is not None:
            lines.append(line)
            if re.match(r"^\.Lfunc_end\d*:", line):
                bodies[cur] = hashlib.sha256("\n".join(lines).encode()).hexdigest()
                cur = None
    return hashlib.sha256(text.encode()).hexdigest(), bodies


def build(verbose=False, debug=False):
    """Compile every source and link the shared library; returns its path.
    With debug=True the sources are compiled with MLA_DEBUG=1 into the debug
    library (libmla_hip_debug.so) instead."""
    bdir = DEBUG_BUILD_DIR if debug else BUILD_DIR
    lib = DEBUG_LIB_PATH if debug else LIB_PATH
    flags = FLAGS + (["-DMLA_DEBUG=1"] if debug else [])
    os.makedirs(bdir, exist_ok=True)
    objs = []
    cmds = []
    for src in SOURCES:
        obj = os.path.join(bdir, os.path.splitext(src)[0] + ".o")
        lang = ["-x", "hip"] if src.endswith(".cpp") else []
        cmds.append([HIPCC] + flags + lang + ["-c", os.path.join(CSRC, src), "-o", obj])
        objs.append(obj)
    with ThreadPoolExecutor(max_workers=min(len(cmds) + len(KERNEL_SOURCES), 8)) as ex:
        hashes = [] if debug else [ex.submit(device_code_sha256, k, verbose) for k in KERNEL_SOURCES]
        list(ex.map(lambda c: _run(c, verbose), cmds))
        if not debug:
            rec = {"kernels": {}}
            for k, h in zip(KERNEL_SOURCES, hashes):
                rec[k], rec["kernels"][k] = h.result()
            json.dump(rec, open(DEVICE_CODE_PATH, "w"), indent=1)
    tmp = lib + ".tmp"
    _run([HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp] + objs, verbose)
    os.replace(tmp, lib)
    return lib


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv, debug="--debug" in sys.argv))
