"""Build libringattn.so for gfx950 with hipcc (in-tree, no GPU needed).

Usage: ``python -m ring_attention_context_amd.build`` or ``build()``.
Every HIP source is compiled with packed-fp32 instructions disabled
(``-Xclang -target-feature -Xclang -packed-fp32-ops``); hipcc's host pass
warns that it does not know that feature, which is harmless.
"""

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD_DIR = os.path.join(PKG, "_build")
LIB_PATH = os.path.join(PKG, "libringattn.so")

SOURCES = ["status.cpp", "partition.cpp", "attn_api.cpp", "lse_merge.hip", "attn_f32.hip",
           "attn_bf16.hip", "attn_bwd.hip", "v_transpose.hip", "ring.hip", "allgather.hip",
           "noalloc.hip"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
COMMON = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", f"-I{INCLUDE}", f"-I{CSRC}",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-Wall", "-Wno-unused-function"]


def _compile_cmd(src):
    obj = os.path.join(BUILD_DIR, src + ".o")
    lang = ["-x", "hip"]  # .cpp sources use the HIP runtime too
    return obj, [HIPCC, *lang, *COMMON, "-c", os.path.join(CSRC, src), "-o", obj]


def build(verbose=False, extra_flags=()):
    """Compile every source and link libringattn.so. Always rebuilds."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    procs, objs = [], []
    for src in SOURCES:
        obj, cmd = _compile_cmd(src)
        cmd = cmd[:-4] + list(extra_flags) + cmd[-4:]
        objs.append(obj)
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append((src, subprocess.Popen(cmd, stdout=subprocess.PIPE,
                                            stderr=subprocess.STDOUT, text=True)))
    failed = []
    for src, p in procs:
        out, _ = p.communicate()
        noise = [ln for ln in out.splitlines() if "packed-fp32-ops" not in ln
                 and "not a recognized feature" not in ln and ln.strip()]
        if p.returncode != 0:
            failed.append(src)
            print(out, file=sys.stderr)
        elif noise and verbose:
            print("\n".join(noise))
    if failed:
        raise RuntimeError(f"hipcc failed for {failed}")
    tmp = LIB_PATH + ".tmp"
    link = [HIPCC, "-shared", "-fPIC", f"--offload-arch={ARCH}", *objs, "-o", tmp]
    if verbose:
        print(" ".join(link), flush=True)
    subprocess.run(link, check=True)
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
