"""Build the HIP library libbissd.so for gfx950 with hipcc, in-tree.

Every .hip source under csrc/ is compiled into one shared library exporting
the C ABI declared in include/bissd.h.
"""
import glob
import os
import subprocess
import sys
import tempfile

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
LIB = os.path.join(HERE, "libbissd.so")
ARCH = os.environ.get("BISSD_OFFLOAD_ARCH", "gfx950")


def sources():
    return sorted(glob.glob(os.path.join(HERE, "csrc", "*.hip")))


def _run(cmd):
    return subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)


def _messages(text):
    # the host pass does not know the packed-fp32 feature flag; that warning is expected
    return [l for l in text.splitlines() if "packed-fp32-ops" not in l and l.strip()]


def build(verbose: bool = False) -> str:
    """Compile every source to an object in parallel, then link."""
    hipcc = os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "bin", "hipcc")
    flags = [f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             "-Wall", "-Wno-unused-function",
             "-I", os.path.join(ROOT, "include"), "-I", os.path.join(HERE, "csrc")]
    msgs = []
    with tempfile.TemporaryDirectory(prefix="bissd_build_") as tmpdir:
        objs, procs = [], []
        for src in sources():
            obj = os.path.join(tmpdir, os.path.basename(src) + ".o")
            cmd = [hipcc] + flags + ["-c", src, "-o", obj]
            if verbose:
                print(" ".join(cmd), flush=True)
            objs.append(obj)
            procs.append((src, _run(cmd)))
        failed = []
        for src, p in procs:
            out, _ = p.communicate()
            msgs += _messages(out)
            if p.returncode != 0:
                failed.append(os.path.basename(src))
        if failed:
            sys.stderr.write("\n".join(msgs) + "\n")
            raise RuntimeError(f"hipcc failed on {', '.join(failed)}")
        tmp = LIB + ".tmp"
        p = _run([hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp] + objs)
        out, _ = p.communicate()
        msgs += _messages(out)
        if p.returncode != 0:
            sys.stderr.write("\n".join(msgs) + "\n")
            raise RuntimeError("hipcc failed linking libbissd.so")
    if verbose and msgs:
        print("\n".join(msgs))
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
