"""Build libtis.so (the HIP kernels and the C ABI) for gfx950 with hipcc."""
import glob
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
LIB = os.path.join(HERE, "libtis.so")
ARCH = os.environ.get("TIS_OFFLOAD_ARCH", "gfx950")


def sources():
    return sorted(glob.glob(os.path.join(HERE, "csrc", "*.hip")))


def build(verbose: bool = False, jobs: int = 4) -> str:
    """Compile every .hip source to an object in parallel, then link."""
    objdir = os.path.join(HERE, "_build")
    os.makedirs(objdir, exist_ok=True)
    flags = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-Wall",
             "-Wno-unused-result", "-I", os.path.join(ROOT, "include"),
             # no packed fp32 instructions in device code
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
    procs, objs = [], []
    for src in sources():
        obj = os.path.join(objdir, os.path.basename(src) + ".o")
        objs.append(obj)
        cmd = ["hipcc", "-c", src, "-o", obj] + flags
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append((cmd, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT)))
        if len(procs) >= jobs:
            _wait(procs.pop(0))
    while procs:
        _wait(procs.pop(0))
    tmp = LIB + ".tmp"
    link = ["hipcc", "-shared", "-fPIC", f"--offload-arch={ARCH}", "-o", tmp] + objs
    if verbose:
        print(" ".join(link), flush=True)
    subprocess.run(link, check=True)
    os.replace(tmp, LIB)
    return LIB


def _wait(item):
    cmd, p = item
    out, _ = p.communicate()
    text = out.decode(errors="replace")
    # the host pass does not know the device-only target feature: harmless
    lines = [l for l in text.splitlines() if "packed-fp32-ops" not in l]
    if p.returncode != 0:
        raise RuntimeError("build failed: " + " ".join(cmd) + "\n" + "\n".join(lines))
    if lines:
        print("\n".join(lines), flush=True)


if __name__ == "__main__":
    print(build(verbose=True))
