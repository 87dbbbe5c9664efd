"""Build libefla.so (HIP kernels + C ABI) in-tree for gfx950 with hipcc.

    python -m delta_rule_sequence_amd.build              # libefla.so
    python -m delta_rule_sequence_amd.build --sanitize   # libefla_hostsan.so (host code only)
    python -m delta_rule_sequence_amd.build --lds-poison # libefla_ldspoison.so (debug)
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
OUT = os.path.join(PKG, "libefla.so")
BUILD_DIR = os.path.join(PKG, "_build")

SOURCES = ["efla_api.hip", "efla_prep.hip", "efla_ut.hip", "efla_scan_fwd.hip",
           "efla_scan_seg.hip", "efla_scan_bwd.hip", "efla_chunk_bwd.hip", "efla_decode.hip"]

# -packed-fp32-ops: keep hipcc from emitting packed fp32 vector instructions.
FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-Wall",
         "-Wno-unused-function", "-Wno-unused-command-line-argument",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-I" + os.path.join(ROOT, "include")]

# Per-file flags. The two state scans keep their MFMA accumulators in VGPRs rather than the
# compiler's default AGPR placement: their accumulators feed VALU work (bf16 conversion, the
# next product's operands) every chunk, and copying them out of AGPRs cost about a third of
# the forward scan's VALU instructions (measured: 2-4% faster scans, identical results).
FILE_FLAGS = {
    "efla_scan_fwd.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
    "efla_scan_bwd.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
}


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found; the EFLA library needs ROCm's hipcc to build")


def _run(cmd):
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    noise = "packed-fp32-ops"
    msg = "\n".join(l for l in r.stdout.splitlines() if noise not in l and l.strip())
    if r.returncode != 0:
        raise RuntimeError("command failed: %s\n%s" % (" ".join(cmd), msg))
    return msg


# The same sources with AddressSanitizer and UndefinedBehaviorSanitizer on the host code only
# (argument checks, sizing, workspace carving), for exercising the host paths of the C ABI on a
# machine without a GPU. Each -fsanitize= follows -Xarch_host, so device code is built as usual
# and not instrumented.
SAN_OUT = os.path.join(PKG, "libefla_hostsan.so")
SAN_FLAGS = ["--offload-arch=gfx950", "-O3", "-Xarch_host", "-O1", "-Xarch_host", "-g",
             "-fno-omit-frame-pointer", "-std=c++17", "-fPIC", "-Wall",
             "-Wno-unused-function", "-Wno-unused-command-line-argument",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
             "-Xarch_host", "-fno-sanitize-recover=all",
             "-I" + os.path.join(ROOT, "include")]


def sanitizer_runtime() -> str:
    """Path of the compiler's AddressSanitizer runtime (preloaded into the process that loads
    libefla_hostsan.so; it also carries the UndefinedBehaviorSanitizer handlers)."""
    r = subprocess.run([os.path.join(os.path.dirname(hipcc()), "..", "llvm", "bin", "clang"),
                        "-print-file-name=libclang_rt.asan-x86_64.so"],
                       stdout=subprocess.PIPE, stderr=subprocess.DEVNULL, text=True)
    path = r.stdout.strip()
    if r.returncode != 0 or not os.path.isabs(path) or not os.path.exists(path):
        raise RuntimeError("AddressSanitizer runtime not found next to hipcc")
    return path


# Debug build with -DEFLA_LDS_POISON: every kernel fills its dynamic LDS with NaN bytes before it
# starts, so a read of LDS that the kernel did not write first shows up as NaN in the results.
POISON_OUT = os.path.join(PKG, "libefla_ldspoison.so")


def build(verbose: bool = False, sanitize: bool = False, lds_poison: bool = False) -> str:
    """Compile every source and link libefla.so (sanitize: libefla_hostsan.so, host code
    instrumented; lds_poison: libefla_ldspoison.so); returns its path."""
    assert not (sanitize and lds_poison), "one variant at a time"
    cc = hipcc()
    bdir = BUILD_DIR + ("_hostsan" if sanitize else "_ldspoison" if lds_poison else "")
    out = SAN_OUT if sanitize else POISON_OUT if lds_poison else OUT
    os.makedirs(bdir, exist_ok=True)
    objs = [os.path.join(bdir, s.replace(".hip", ".o")) for s in SOURCES]

    def compile_one(i):
        src = os.path.join(CSRC, SOURCES[i])
        flags = SAN_FLAGS if sanitize else FLAGS + FILE_FLAGS.get(SOURCES[i], [])
        if lds_poison:
            flags = flags + ["-DEFLA_LDS_POISON"]
        return _run([cc] + flags + ["-c", src, "-o", objs[i]])

    with ThreadPoolExecutor(max_workers=min(len(SOURCES), os.cpu_count() or 4)) as ex:
        logs = list(ex.map(compile_one, range(len(SOURCES))))
    tmp = out + ".tmp%d" % os.getpid()
    link = [cc, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp] + objs
    if sanitize:
        link[2:2] = ["-Xarch_host", "-fsanitize=address",
                     "-Xarch_host", "-fsanitize=undefined", "-shared-libsan"]
    logs.append(_run(link))
    os.replace(tmp, out)
    if verbose:
        for l in logs:
            if l:
                print(l)
    return out


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv, sanitize="--sanitize" in sys.argv,
                lds_poison="--lds-poison" in sys.argv))
