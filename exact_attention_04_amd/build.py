"""Build the HIP library libea_attn.so in-tree for gfx950 with hipcc.

    python -m exact_attention_04_amd.build          # or build() from Python

Compiles every source under csrc/ (the kernels and the C ABI) and links them
into exact_attention_04_amd/libea_attn.so next to this file.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
import tempfile

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG_DIR)
CSRC = os.path.join(PKG_DIR, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB_NAME = "libea_attn.so"
LIB_PATH = os.path.join(PKG_DIR, LIB_NAME)

ARCH = "gfx950"
# Packed fp32 VALU forms are kept out of the generated code: the kernels are
# written against scalar fp32 arithmetic.
DEVICE_FLAGS = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
COMMON = ["-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-function", f"-I{INCLUDE}", f"-I{CSRC}"]


def _hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: set HIPCC or install ROCm")


def _rocm_root(hipcc: str) -> str:
    return os.path.dirname(os.path.dirname(os.path.realpath(hipcc)))


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in res.stdout.splitlines()
                    if "packed-fp32-ops" not in l and "hip-link" not in l and l.strip())
    if res.returncode != 0:
        raise RuntimeError(f"build step failed ({res.returncode}): {' '.join(cmd)}\n{out}")
    if out and verbose:
        print(out, flush=True)


def elf_section_names(path: str) -> set:
    """Section names of a 64-bit little-endian ELF file."""
    import struct
    with open(path, "rb") as f:
        data = f.read()
    if data[:4] != b"\x7fELF" or data[4] != 2 or data[5] != 1:
        raise RuntimeError(f"{path}: not a 64-bit little-endian ELF file")
    shoff, = struct.unpack_from("<Q", data, 0x28)
    shentsize, shnum, shstrndx = struct.unpack_from("<HHH", data, 0x3A)
    def sh(i):
        return struct.unpack_from("<IIQQQQIIQQ", data, shoff + i * shentsize)
    stroff = sh(shstrndx)[4]
    names = set()
    for i in range(shnum):
        nm = sh(i)[0]
        end = data.index(b"\0", stroff + nm)
        names.add(data[stroff + nm:end].decode())
    return names


def build(verbose: bool = False, jobs: int = 4) -> str:
    """Compile the kernels and the ABI layer; returns the path of the library."""
    hipcc = _hipcc()
    srcs = sorted(f for f in os.listdir(CSRC) if f.endswith((".hip", ".cpp")))
    tmp = tempfile.mkdtemp(prefix="ea_build_")
    try:
        procs = []
        objs = []
        for s in srcs:
            obj = os.path.join(tmp, s + ".o")
            objs.append(obj)
            lang = ["-x", "hip", f"--offload-arch={ARCH}"] + DEVICE_FLAGS if s.endswith(".hip") else ["-x", "c++", "-D__HIP_PLATFORM_AMD__", f"-I{_rocm_root(hipcc)}/include"]
            cmd = [hipcc] + lang + COMMON + ["-c", os.path.join(CSRC, s), "-o", obj]
            procs.append((cmd, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)))
        for cmd, pr in procs:
            out, _ = pr.communicate()
            out = "\n".join(l for l in out.splitlines() if "packed-fp32-ops" not in l and l.strip())
            if pr.returncode != 0:
                raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{out}")
            if out and verbose:
                print(out, flush=True)
        tmp_lib = os.path.join(tmp, LIB_NAME)
        # --no-undefined: a kernel whose host stub was not emitted must fail
        # the build here, not the first call at run time
        _run([hipcc, "-shared", "-fPIC", f"--offload-arch={ARCH}", "-Wl,--no-undefined", "-o", tmp_lib] + objs, verbose)
        if ".hip_fatbin" not in elf_section_names(tmp_lib):
            raise RuntimeError(f"{LIB_NAME} has no .hip_fatbin section: no GPU code was embedded")
        os.replace(tmp_lib, LIB_PATH)
    finally:
        shutil.rmtree(tmp, ignore_errors=True)
    return LIB_PATH


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
