"""Compiles the HIP sources into block_sparse_backward_amd/liblazyflash.so (gfx950).

Run as ``python -m block_sparse_backward_amd.build``; ``__graft_entry__.build()``
calls :func:`build`.  Objects go to ``_build/`` at the repository root.
"""
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
OBJDIR = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "liblazyflash.so")

SOURCES = ["lf_api.hip", "lf_select.hip", "lf_fwd.hip", "lf_bwd.hip"]
# the select kernels decide the kept set: no fused multiply-add anywhere there
EXTRA = {
    "lf_select.hip": ["-ffp-contract=off"],
    # MFMA results stay in VGPRs (no copies between the two register files
    # around the score products)
    "lf_bwd.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
}

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
COMMON = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    "-munsafe-fp-atomics",
    # packed fp32 instructions are kept out of every kernel
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-result", "-Wno-unused-function",
    "-I", os.path.join(ROOT, "include"), "-I", CSRC,
]


def build(verbose=False, jobs=None, lib=LIB, objdir=OBJDIR, host_flags=()):
    """Compile every source (always) and link the shared library `lib`.

    `host_flags` are extra flags for the host half of every source only (each
    is passed after -Xarch_host, so the gfx950 code is built as usual); the
    sanitized build of the C-ABI layer's host code uses them."""
    os.makedirs(objdir, exist_ok=True)
    xhost = [f for flag in host_flags for f in ("-Xarch_host", flag)]
    procs = []
    objs = []
    for src in SOURCES:
        obj = os.path.join(objdir, src.replace(".hip", ".o"))
        objs.append(obj)
        cmd = [HIPCC, *COMMON, *EXTRA.get(src, []), *xhost, "-c", os.path.join(CSRC, src),
               "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append((src, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT)))
    failed = []
    for src, p in procs:
        out, _ = p.communicate()
        text = out.decode(errors="replace")
        if p.returncode != 0:
            failed.append(src)
            sys.stderr.write(text)
        elif verbose and text.strip():
            sys.stderr.write(text)
    if failed:
        raise RuntimeError("hipcc failed for: " + ", ".join(failed))
    tmp = lib + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *xhost, "-o", tmp, *objs]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    shutil.move(tmp, lib)
    return lib


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
