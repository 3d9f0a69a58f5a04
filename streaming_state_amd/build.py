"""Build ``libssm_stream.so`` (gfx950) in-tree with hipcc.

Run ``python -m streaming_state_amd.build`` or call ``build()``.  The sources
are the host runtime (``csrc/ssm_host.cpp``) and the kernels
(``csrc/*.hip``); every file is compiled for gfx950 only, with packed fp32
instructions disabled.  ``ssm_abi_latency`` (``csrc/abi_latency.cpp``) is a
small program that times the C ABI's scan call with no binding in the loop.
"""
import os
import subprocess
import sys
import tempfile
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libssm_stream.so")
LATENCY = os.path.join(HERE, "ssm_abi_latency")
SOURCES = ["ssm_host.cpp", "ssm_decode.hip", "ssm_kernels.hip", "ssm_scan.hip", "ssm_ssd.hip", "ssm_ssd_pair.hip", "ssm_chunk.hip", "ssm_conv.hip", "ssm_static.hip", "ssm_gdn.hip"]
ARCH = "gfx950"

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-Wall",
         "-Wno-unused-function", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-I", os.path.join(ROOT, "include"), "-I", CSRC]


def sources():
    return [os.path.join(CSRC, s) for s in SOURCES if os.path.exists(os.path.join(CSRC, s))]


def build(verbose=False):
    """Compile every source and link the shared library (always rebuilds)."""
    srcs = sources()
    with tempfile.TemporaryDirectory(prefix="ssm_build_") as tmp:
        def compile_one(src):
            obj = os.path.join(tmp, os.path.basename(src) + ".o")
            lang = ["-x", "hip"] if src.endswith(".hip") else ["-x", "hip"]
            cmd = [HIPCC] + FLAGS + lang + ["-c", src, "-o", obj]
            r = subprocess.run(cmd, capture_output=True, text=True)
            if r.returncode != 0:
                raise RuntimeError(f"hipcc failed on {src}:\n{r.stderr}")
            if verbose:
                noise = [ln for ln in r.stderr.splitlines() if "packed-fp32-ops" not in ln]
                if noise:
                    print("\n".join(noise), file=sys.stderr)
            return obj
        with ThreadPoolExecutor(max_workers=min(4, len(srcs))) as ex:
            objs = list(ex.map(compile_one, srcs))
        tmp_lib = LIB + ".tmp%d" % os.getpid()
        cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp_lib] + objs
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"link failed:\n{r.stderr}")
        os.replace(tmp_lib, LIB)
        # the C-ABI latency probe, linked against the library just built
        tmp_exe = LATENCY + ".tmp%d" % os.getpid()
        cmd = [HIPCC] + FLAGS + ["-x", "hip", os.path.join(CSRC, "abi_latency.cpp"), "-o", tmp_exe,
               "-L", HERE, "-lssm_stream", "-Wl,-rpath,$ORIGIN"]
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"hipcc failed on abi_latency.cpp:\n{r.stderr}")
        os.replace(tmp_exe, LATENCY)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
