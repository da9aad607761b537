"""Build libw4moe.so (HIP kernels for gfx950 + the C-ABI host code) in-tree."""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libw4moe.so")
SOURCES = ["w4_gemm.hip", "w4_attn.hip", "w4_glue.hip", "w4_noalloc.hip", "w4_host.cpp"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    # every multiply and add is rounded as written; fused ops only where fmaf() says so
    "-ffp-contract=off",
    # no packed-FP32 instructions
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"), "-I", CSRC,
    "-Wall", "-Wno-unused-result",
]


def build(force: bool = True, jobs: int = 4) -> str:
    srcs = [os.path.join(CSRC, s) for s in SOURCES]
    deps = srcs + [os.path.join(CSRC, h) for h in ("w4_internal.h", "w4_device.h", "w4_tile.h")] + \
        [os.path.join(ROOT, "include", "w4moe.h")]
    if not force and os.path.exists(LIB) and os.path.getmtime(LIB) >= max(os.path.getmtime(d) for d in deps):
        return LIB
    objdir = os.path.join(HERE, "_build")
    os.makedirs(objdir, exist_ok=True)
    objs, procs = [], []
    for s in srcs:
        o = os.path.join(objdir, os.path.basename(s) + ".o")
        objs.append(o)
        lang = ["-x", "hip"] if s.endswith(".cpp") else []
        cmd = [HIPCC] + [f for f in FLAGS if f != "-shared"] + lang + ["-c", s, "-o", o]
        procs.append((subprocess.Popen(cmd), s))
        if len(procs) >= jobs:
            p, src = procs.pop(0)
            if p.wait():
                raise RuntimeError(f"hipcc failed on {src}")
    for p, src in procs:
        if p.wait():
            raise RuntimeError(f"hipcc failed on {src}")
    tmp = LIB + ".tmp"
    subprocess.run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp] + objs, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build())
