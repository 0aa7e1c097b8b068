"""Build libk3g.so (the HIP kernels and their C ABI) for gfx950 with hipcc.

Every HIP source is compiled with packed fp32 instructions turned off
(-target-feature -packed-fp32-ops); the host pass warns that it does not know
the feature, which is harmless.
"""
import glob
import os
import subprocess
import sys
import tempfile

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
LIB = os.path.join(HERE, "libk3g.so")
ARCH = "gfx950"


def sources():
    return sorted(glob.glob(os.path.join(HERE, "csrc", "*.hip")))


def build(verbose: bool = False, jobs: int = 8, defines=(), out: str = LIB) -> str:
    """Compile every csrc/*.hip and link `out`. `defines` are extra -D flags
    (build-time kernel variants)."""
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    flags = [*[f"-D{d}" for d in defines], "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-I", os.path.join(ROOT, "include"),
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", "-Wall", "-Wno-unused-result"]
    objs = []
    with tempfile.TemporaryDirectory(prefix="k3g_build_") as tmp:
        procs = []
        for src in sources():
            obj = os.path.join(tmp, os.path.basename(src) + ".o")
            cmd = [hipcc, *flags, "-c", src, "-o", obj]
            if verbose:
                print(" ".join(cmd), flush=True)
            procs.append((src, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT)))
            objs.append(obj)
            while len([p for _, p in procs if p.poll() is None]) >= jobs:
                procs[0][1].wait()
        failed = False
        for src, p in procs:
            log = p.communicate()[0].decode(errors="replace")
            lines = [ln for ln in log.splitlines() if "packed-fp32-ops" not in ln]
            if lines and (verbose or p.returncode):
                print("\n".join(lines), flush=True)
            if p.returncode:
                print(f"build failed: {src}", file=sys.stderr, flush=True)
                failed = True
        if failed:
            raise RuntimeError("hipcc failed")
        out_tmp = out + f".tmp{os.getpid()}"
        cmd = [hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", out_tmp, *objs]
        if verbose:
            print(" ".join(cmd), flush=True)
        subprocess.run(cmd, check=True)
        os.replace(out_tmp, out)
    return out


if __name__ == "__main__":
    build(verbose="-v" in sys.argv)
