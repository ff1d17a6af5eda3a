"""Build libw4a8.so (HIP, gfx950) in-tree with hipcc.

    python -m moe_grouped_precision_amd.build          # build
    python -m moe_grouped_precision_amd.build --check  # build, then list exported symbols

The library is placed next to this file so that it travels with the source
tree.  Every HIP source is compiled with packed-fp32 instructions disabled.
"""

from __future__ import annotations

import os
import shutil
import subprocess
import sys
import tempfile

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
ROOT = os.path.dirname(HERE)
LIB = os.path.join(HERE, "libw4a8.so")
SOURCES = ["api.cpp", "prep.hip", "gemm.hip", "quant.hip", "combine.hip", "a16.hip"]
# roofline probes (sustained MFMA rate and HBM read bandwidth), a library of
# their own: the benchmark loads them, the GEMM path does not
PROBE_LIB = os.path.join(HERE, "libw4a8_probe.so")
PROBE_SOURCES = ["probe.hip"]
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libw4a8)")


def compile_flags(debug: bool = False):
    flags = [
        f"--offload-arch={ARCH}",
        "-std=c++17",
        "-fPIC",
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-I", os.path.join(ROOT, "include"),
        "-I", CSRC,
        "-Wall",
        # the K-loop asm names m0 (the LDS base of direct-to-LDS loads) as
        # clobbered; the compiler notes that it does not preserve m0, which is
        # what the kernels expect
        "-Wno-inline-asm",
    ]
    flags += ["-O0", "-g"] if debug else ["-O3"]
    return flags


# sources whose K loops issue inline-asm memory operations: their device
# assembly is checked after every build (see asmcheck.py)
ASM_CHECKED = ["gemm.hip"]


def check_device_asm(cc: str, tmp: str, verbose: bool = False) -> None:
    """Emit the gfx950 assembly of the inline-asm kernels and run the static
    check on it; raise if it reports anything."""
    from . import asmcheck

    for src in ASM_CHECKED:
        path = os.path.join(CSRC, src)
        asm = os.path.join(tmp, src.replace(".", "_") + ".s")
        cmd = [cc, "-x", "hip", *compile_flags(), "--cuda-device-only", "-S", path, "-o", asm]
        if verbose:
            print(" ".join(cmd), flush=True)
        res = subprocess.run(cmd, capture_output=True, text=True)
        if res.returncode != 0:
            raise RuntimeError(f"hipcc -S failed on {src}:\n{res.stderr}")
        findings = asmcheck.check(asm)
        if findings:
            raise RuntimeError(f"device assembly of {src} fails the load/wait check:\n" +
                               "\n".join(findings[:20]))


def _link(cc, tmp, sources, out, verbose, debug):
    objs = []
    for src in sources:
        path = os.path.join(CSRC, src)
        obj = os.path.join(tmp, src.replace(".", "_") + ".o")
        cmd = [cc, "-x", "hip", *compile_flags(debug), "-c", path, "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        res = subprocess.run(cmd, capture_output=True, text=True)
        if res.returncode != 0:
            raise RuntimeError(f"hipcc failed on {src}:\n{res.stderr}")
        objs.append(obj)
    tmp_lib = os.path.join(tmp, os.path.basename(out))
    cmd = [cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp_lib]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed:\n{res.stderr}")
    shutil.copyfile(tmp_lib, out + ".tmp")
    os.replace(out + ".tmp", out)


def build(verbose: bool = False, debug: bool = False) -> str:
    """Compile every source, check the device assembly of the inline-asm
    kernels, and link libw4a8.so and libw4a8_probe.so; returns the GEMM
    library's path."""
    cc = hipcc()
    with tempfile.TemporaryDirectory(prefix="w4a8_build_") as tmp:
        if not debug:
            check_device_asm(cc, tmp, verbose)
        _link(cc, tmp, SOURCES, LIB, verbose, debug)
        _link(cc, tmp, PROBE_SOURCES, PROBE_LIB, verbose, debug)
    return LIB


def main(argv=None):
    argv = sys.argv[1:] if argv is None else argv
    path = build(verbose="-v" in argv, debug="--debug" in argv)
    print(path)
    if "--check" in argv:
        out = subprocess.run(["nm", "-D", "--defined-only", path], capture_output=True, text=True).stdout
        print("\n".join(l for l in out.splitlines() if " w4a8_" in l))


if __name__ == "__main__":
    main()
