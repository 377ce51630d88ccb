"""Build libfa_varlen.so for gfx950 with hipcc (in-tree, no JIT cache).

Usage: python -m variable_length_flashattention_fa_amd.csrc.build  [--arch gfx950]
"""
from __future__ import annotations

import argparse
import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
PKG = os.path.dirname(HERE)
ROOT = os.path.dirname(PKG)
INCLUDE = os.path.join(ROOT, "include")
LIBDIR = os.path.join(PKG, "lib")
LIBNAME = "libfa_varlen.so"

# (source, object name, extra flags).  The 16-bit kernels feed MFMA results straight into VALU
# work (exp, dS): their MFMA destinations stay in VGPRs instead of accumulation registers that
# would need copying back.  fa_bwd16.hip and fa_fwd.hip compile in parts (one per kernel and
# dtype), in parallel.
_VGPR_FORM = ["-mllvm", "-amdgpu-mfma-vgpr-form"]
HIP_UNITS = [("fa_kernels.hip", "fa_kernels", []), ("fa_api.cpp", "fa_api", []),
             ("fa_workspace.cpp", "fa_workspace", []), ("fa_noalloc.hip", "fa_noalloc", [])]
HIP_UNITS += [("fa_bwd16.hip", f"fa_bwd16_p{i}", _VGPR_FORM + [f"-DFA_BWD16_PART={i}"]) for i in (1, 2, 3, 4)]
HIP_UNITS += [("fa_fwd.hip", f"fa_fwd_p{i}", _VGPR_FORM + [f"-DFA_FWD_PART={i}"]) for i in (1, 2)]
HIP_SOURCES = sorted({u[0] for u in HIP_UNITS})
CXX_SOURCES = ["fa_worklist.cpp"]


def _hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build the library)")


def _run(cmd):
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    # the host pass does not know the packed-fp32 feature and says so; that is harmless
    lines = [l for l in r.stdout.splitlines() if "packed-fp32-ops" not in l and "--hip-link" not in l]
    if r.returncode != 0:
        raise RuntimeError("build step failed:\n" + " ".join(cmd) + "\n" + "\n".join(lines))
    return "\n".join(lines)


def build(arch: str = "gfx950", verbose: bool = False) -> str:
    hipcc = _hipcc()
    objdir = os.path.join(PKG, "_build")
    os.makedirs(objdir, exist_ok=True)
    os.makedirs(LIBDIR, exist_ok=True)
    common = ["-O3", "-std=c++17", "-fPIC", f"-I{INCLUDE}", f"-I{HERE}", "-Wall"]
    hip_flags = [f"--offload-arch={arch}", "-munsafe-fp-atomics",
                 # keep the compiler from forming packed fp32 ops (v_pk_*_f32)
                 "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
    jobs = []
    objs = []
    for src, name, extra in HIP_UNITS:
        obj = os.path.join(objdir, name + ".o")
        lang = [] if src.endswith(".hip") else ["-x", "hip"]
        jobs.append([hipcc] + common + hip_flags + extra + lang + ["-c", os.path.join(HERE, src), "-o", obj])
        objs.append(obj)
    for src in CXX_SOURCES:
        obj = os.path.join(objdir, src + ".o")
        jobs.append(["g++"] + common + ["-c", os.path.join(HERE, src), "-o", obj])
        objs.append(obj)
    with cf.ThreadPoolExecutor(max_workers=len(jobs)) as ex:
        outs = list(ex.map(_run, jobs))
    if verbose:
        for o in outs:
            if o:
                print(o)
    out = os.path.join(LIBDIR, LIBNAME)
    tmp = out + ".tmp"
    _run([hipcc, "-shared", f"--offload-arch={arch}", "-o", tmp] + objs)
    os.replace(tmp, out)
    return out


# Host sources of the C ABI (validation, work lists, library memory): the ones the CPU sanitizer
# build instruments.
HOST_SANITIZED = ["fa_worklist.cpp", "fa_api.cpp", "fa_workspace.cpp"]
SANITIZED_LIBNAME = "libfa_varlen_host_asan.so"


def build_host_sanitized(arch: str = "gfx950") -> str:
    """libfa_varlen_host_asan.so: the host sources compiled by g++ with AddressSanitizer and
    UndefinedBehaviorSanitizer, linked with the (uninstrumented) kernel objects of build().

    For CPU tests of validation and work lists under the sanitizers (load it with libasan
    preloaded).  Builds the kernel objects first if they are missing."""
    objdir = os.path.join(PKG, "_build")
    kernel_objs = [os.path.join(objdir, name + ".o") for src, name, _ in HIP_UNITS
                   if src.endswith(".hip")]
    if not all(os.path.exists(o) for o in kernel_objs):
        build(arch)
    rocm = os.path.dirname(os.path.dirname(os.path.realpath(_hipcc())))
    san = ["-fsanitize=address,undefined", "-fno-sanitize-recover=undefined", "-fno-omit-frame-pointer", "-g"]
    flags = ["-O1", "-std=c++17", "-fPIC", f"-I{INCLUDE}", f"-I{HERE}", f"-I{os.path.join(rocm, 'include')}",
             "-D__HIP_PLATFORM_AMD__", "-Wall"] + san
    sobjdir = os.path.join(objdir, "host_asan")
    os.makedirs(sobjdir, exist_ok=True)
    objs = []
    jobs = []
    for src in HOST_SANITIZED:
        obj = os.path.join(sobjdir, src + ".o")
        jobs.append(["g++"] + flags + ["-x", "c++", "-c", os.path.join(HERE, src), "-o", obj])
        objs.append(obj)
    with cf.ThreadPoolExecutor(max_workers=len(jobs)) as ex:
        list(ex.map(_run, jobs))
    out = os.path.join(LIBDIR, SANITIZED_LIBNAME)
    tmp = out + ".tmp"
    _run(["g++", "-shared"] + san + ["-o", tmp] + objs + kernel_objs +
         [f"-L{os.path.join(rocm, 'lib')}", "-lamdhip64", f"-Wl,-rpath,{os.path.join(rocm, 'lib')}"])
    os.replace(tmp, out)
    return out


def main(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("--arch", default="gfx950")
    ap.add_argument("-v", "--verbose", action="store_true")
    ap.add_argument("--host-sanitized", action="store_true",
                    help="also build lib/libfa_varlen_host_asan.so (host sources under ASan / UBSan)")
    args = ap.parse_args(argv)
    print(build(args.arch, args.verbose))
    if args.host_sanitized:
        print(build_host_sanitized(args.arch))


if __name__ == "__main__":
    main(sys.argv[1:])
