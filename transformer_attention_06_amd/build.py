"""Build libattn_fwd.so (gfx950) in-tree with hipcc.

    python -m transformer_attention_06_amd.build [--verbose]
"""

import os
import shutil
import subprocess
import sys
import tempfile

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libattn_fwd.so")
ARCH = "gfx950"

SOURCES = ["attn_api.cpp", "attn_fwd_kernels.hip"]

# Packed-fp32 VALU forms are kept out of the device code.
DEVICE_FLAGS = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def hipcc():
    path = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(path):
        raise RuntimeError("hipcc not found; ROCm is required to build libattn_fwd.so")
    return path


def build(verbose=False, extra_flags=()):
    """Compile every source into LIB; returns the library path.  The device
    assembly of the kernels is compiled alongside and checked for MFMA wait
    states (asm_check); the library is only installed if that check passes."""
    tmp = LIB + ".tmp"
    common = [f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", f"-I{INCLUDE}", f"-I{CSRC}",
              *DEVICE_FLAGS, *extra_flags]
    cmd = [hipcc(), *common, "-shared", "-Wall", "-Wno-unused-result", "-Wno-pass-failed", "-o", tmp]
    cmd += [os.path.join(CSRC, s) for s in SOURCES]
    with tempfile.TemporaryDirectory() as td:
        asm = os.path.join(td, "kernels.s")
        acmd = [hipcc(), *common, "--cuda-device-only", "-S", "-o", asm,
                os.path.join(CSRC, "attn_fwd_kernels.hip")]
        if verbose:
            print(" ".join(cmd), flush=True)
            print(" ".join(acmd), flush=True)
        lib_p = subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.PIPE, text=True)
        asm_p = subprocess.Popen(acmd, stdout=subprocess.PIPE, stderr=subprocess.PIPE, text=True)
        out, err = lib_p.communicate()
        aout, aerr = asm_p.communicate()
        if lib_p.returncode != 0:
            sys.stderr.write(out + err)
            raise RuntimeError(f"hipcc failed with exit code {lib_p.returncode}")
        if asm_p.returncode != 0:
            sys.stderr.write(aout + aerr)
            raise RuntimeError(f"hipcc (device assembly) failed with exit code {asm_p.returncode}")
        if verbose and (out or err):
            sys.stderr.write(out + err)
        sys.path.insert(0, PKG)
        try:
            import asm_check
        finally:
            sys.path.pop(0)
        with open(asm) as f:
            problems = asm_check.check_asm(f.read())
    if problems:
        os.remove(tmp)
        raise RuntimeError("MFMA wait-state check failed:\n" + "\n".join(problems[:20]))
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="--verbose" in sys.argv))
