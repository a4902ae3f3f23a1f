"""Build libgq.so in-tree with hipcc for gfx950."""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIBDIR = os.path.join(HERE, "_lib")
SO = os.path.join(LIBDIR, "libgq.so")
SOURCES = ["gq_abi.cpp", "gq_chunker.cpp", "gq_kernels.hip", "gq_check.hip", "gq_noalloc.hip"]
ARCH = "gfx950"

HIPCC_FLAGS = [
    "-O3", "-std=c++17", "-fPIC", "--offload-arch=" + ARCH,
    # numerics the parity contract relies on
    "-ffp-contract=off", "-fno-gpu-flush-denormals-to-zero",
    "-fhip-fp32-correctly-rounded-divide-sqrt",
    # keep the compiler from emitting packed fp32 instructions
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-command-line-argument",
]


def hipcc():
    root = os.environ.get("ROCM_PATH", "/opt/rocm")
    return os.path.join(root, "bin", "hipcc")


def build(verbose=False):
    """Compile every source to an object and link libgq.so (always
    rebuilds)."""
    os.makedirs(LIBDIR, exist_ok=True)
    objs, procs = [], []
    for src in SOURCES:   # the sources compile in parallel
        obj = os.path.join(LIBDIR, os.path.splitext(src)[0] + ".o")
        cmd = [hipcc(), *HIPCC_FLAGS, "-c", os.path.join(CSRC, src), "-o", obj]
        if src.endswith(".cpp"):
            cmd[1:1] = ["-x", "hip"]
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append((subprocess.Popen(cmd), cmd))
        objs.append(obj)
    failed = [cmd for p, cmd in procs if p.wait() != 0]
    if failed:
        raise subprocess.CalledProcessError(1, failed[0])
    tmp = SO + ".tmp%d" % os.getpid()
    cmd = [hipcc(), "--offload-arch=" + ARCH, "-shared", "-fPIC", "-o", tmp, *objs]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, SO)
    for o in objs:
        os.remove(o)
    return SO


def build_abi_check(verbose=False):
    """The tests' C++ driver of the C ABI (tests/c_abi), linked against
    libgq.so."""
    root = os.path.dirname(HERE)
    src = os.path.join(root, "tests", "c_abi", "abi_step.cpp")
    out = os.path.join(root, "tests", "c_abi", "libabi_step.so")
    if not os.path.exists(src):
        return None
    cmd = [hipcc(), "-O2", "-std=c++17", "-fPIC", "-shared", "-x", "hip",
           "--offload-arch=" + ARCH, src, "-o", out, "-L", LIBDIR, "-lgq",
           "-Wl,-rpath," + LIBDIR, "-Wl,-rpath,$ORIGIN/../../gradient_compression_allreduce_amd/_lib"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    return out


if __name__ == "__main__":
    print(build(verbose=True))
