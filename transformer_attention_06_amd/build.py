"""Build libattn_fwd.so (gfx950) in-tree with hipcc.

    python -m transformer_attention_06_amd.build [--verbose]
"""

import hashlib
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

# kernels whose MFMAs are inline assembly: their device assembly is checked
ASM_CHECKED = [f"attn_fwd_{t}_d{d}.hip" for t in ("bf16", "f16", "f32") for d in (64, 128)] + \
              [f"attn_fwd_{t}_d{d}.hip" for t in ("bf16", "f16") for d in (80, 96, 112, 144, 160, 192, 256)] + \
              [f"attn_fwd_mask_{t}_d{d}.hip" for t in ("bf16", "f16") for d in (64, 128)]
SOURCES = ["attn_api.cpp", "attn_fwd_kernels.hip", *ASM_CHECKED, "attn_decode_kernels.hip",
           "attn_masked_kernels.hip"]


def source_hash():
    """First 16 hex digits of the SHA-256 over every source the library is
    built from (csrc/ and the public header, in name order).  The build
    embeds it in attn_version(), so a loaded library names the sources it
    came from."""
    h = hashlib.sha256()
    files = sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC)
                   if f.endswith((".hip", ".cpp", ".h")))
    files.append(os.path.join(INCLUDE, "attn_fwd.h"))
    for path in files:
        h.update(os.path.basename(path).encode())
        with open(path, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


# Packed-fp32 VALU forms are kept out of the device code.
DEVICE_FLAGS = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def hipcc():
    path = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(path):
        raise RuntimeError("hipcc not found; ROCm is required to build libattn_fwd.so")
    return path


def build(verbose=False, extra_flags=()):
    """Compile every source into LIB; returns the library path.  The sources
    compile to objects in parallel; the device assembly of the attention
    kernels is compiled alongside and checked for MFMA wait states
    (asm_check); the library is only installed if that check passes."""
    tmp = LIB + ".tmp"
    common = [f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", f"-I{INCLUDE}", f"-I{CSRC}",
              f'-DATTN_SRC_HASH="{source_hash()}"', *DEVICE_FLAGS, *extra_flags]
    with tempfile.TemporaryDirectory() as td:
        objs, procs, asms = [], [], []
        for src in SOURCES:
            stem = os.path.splitext(src)[0]
            obj = os.path.join(td, stem + ".o")
            objs.append(obj)
            cmd = [hipcc(), *common, "-c", "-Wall", "-Wno-unused-result", "-Wno-pass-failed", "-o", obj,
                   os.path.join(CSRC, src)]
            cwd = None
            if src in ASM_CHECKED:
                # one compilation that also leaves the device assembly behind
                cwd = os.path.join(td, stem)
                os.mkdir(cwd)
                cmd.insert(-3, "-save-temps")
                asms.append(os.path.join(cwd, f"{stem}-hip-amdgcn-amd-amdhsa-{ARCH}.s"))
            procs.append((cmd, subprocess.Popen(cmd, cwd=cwd, stdout=subprocess.PIPE, stderr=subprocess.PIPE,
                                                text=True)))
        for cmd, pr in procs:
            out, err = pr.communicate()
            if verbose:
                print(" ".join(cmd), flush=True)
                if out or err:
                    sys.stderr.write(out + err)
            if pr.returncode != 0:
                sys.stderr.write(out + err)
                raise RuntimeError(f"hipcc failed with exit code {pr.returncode}: {' '.join(cmd[-1:])}")
        link = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
        lk = subprocess.run(link, capture_output=True, text=True)
        if lk.returncode != 0:
            sys.stderr.write(lk.stdout + lk.stderr)
            raise RuntimeError(f"link failed with exit code {lk.returncode}")
        # a shared library links with undefined symbols; a kernel whose host
        # stub was not emitted would only fail when the library is loaded
        nm = subprocess.run(["nm", "-D", "--undefined-only", tmp], capture_output=True, text=True)
        missing = [l.split()[-1] for l in nm.stdout.splitlines() if "_GLOBAL__N_" in l]
        if missing:
            os.remove(tmp)
            raise RuntimeError("kernel host stubs missing from the library: " + ", ".join(missing[:5]))
        sys.path.insert(0, PKG)
        try:
            import asm_check
        finally:
            sys.path.pop(0)
        problems = []
        for asm in asms:
            with open(asm) as f:
                problems += asm_check.check_asm(f.read())
    if problems:
        os.remove(tmp)
        raise RuntimeError("MFMA wait-state check failed:\n" + "\n".join(problems[:20]))
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="--verbose" in sys.argv))
