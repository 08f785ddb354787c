"""Build step for libgdn.so (the gfx950 HIP kernels and their C ABI).

Compiles every ``csrc/*.hip`` with hipcc for gfx950 into ``libgdn.so`` beside
this file.  Flags are pinned for the whole library: -O3, no fast-math, no
floating-point contraction (every fused multiply-add is an explicit fmaf in
the source), and packed-fp32 instruction selection disabled.
"""
import glob
import os
import subprocess
import sys
import tempfile

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
LIB = os.path.join(HERE, "libgdn.so")
ARCH = os.environ.get("GDN_OFFLOAD_ARCH", "gfx950")

HIPFLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    "-ffp-contract=off", "-fno-fast-math",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
]


def sources():
    return sorted(glob.glob(os.path.join(HERE, "csrc", "*.hip")))


def build(out: str = LIB, verbose: bool = False, jobs: int = 8) -> str:
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    inc = ["-I", os.path.join(ROOT, "include"), "-I", os.path.join(HERE, "csrc")]
    with tempfile.TemporaryDirectory(prefix="gdn_build_") as tmp:
        objs, procs = [], []
        for src in sources():
            obj = os.path.join(tmp, os.path.basename(src) + ".o")
            cmd = [hipcc, *HIPFLAGS, *inc, "-c", src, "-o", obj]
            if verbose:
                print(" ".join(cmd), flush=True)
            procs.append((src, subprocess.Popen(cmd, stderr=subprocess.PIPE, text=True)))
            objs.append(obj)
            while len([p for _, p in procs if p.poll() is None]) >= jobs:
                procs[0][1].wait()
        for src, p in procs:
            _, err = p.communicate()
            errs = [ln for ln in err.splitlines() if "packed-fp32-ops" not in ln]
            if p.returncode != 0:
                raise RuntimeError(f"hipcc failed on {src}:\n" + "\n".join(errs))
            if verbose and errs:
                print("\n".join(errs))
        tmp_out = out + ".tmp"
        subprocess.run([hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp_out],
                       check=True)
        os.replace(tmp_out, out)
    return out


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
