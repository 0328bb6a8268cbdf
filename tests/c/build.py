"""Build tests/c/abi_parity, a C program that drives librma.so through
include/rma.h and checks it against the C oracle (test infrastructure).

    python tests/c/build.py

Needs bounded_memory_decode_amd/librma.so and oracle/librma_oracle.so built
first; links them and the HIP runtime with gcc.  No GPU is needed to build.
"""
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")
SRC = os.path.join(HERE, "abi_parity.c")
EXE = os.path.join(HERE, "abi_parity")


def build(verbose: bool = False) -> str:
    cc = shutil.which("gcc") or shutil.which("cc")
    if cc is None:
        raise RuntimeError("no C compiler found")
    pkg = os.path.join(ROOT, "bounded_memory_decode_amd")
    orc = os.path.join(ROOT, "oracle")
    for lib in (os.path.join(pkg, "librma.so"), os.path.join(orc, "librma_oracle.so")):
        if not os.path.exists(lib):
            raise RuntimeError(f"{lib} is missing: build the libraries first")
    rpath = "$ORIGIN/../../bounded_memory_decode_amd:$ORIGIN/../../oracle:" + \
        os.path.join(ROCM, "lib")
    cmd = [cc, "-O2", "-std=c11", "-Wall", "-D__HIP_PLATFORM_AMD__",
           "-I", os.path.join(ROCM, "include"), "-I", os.path.join(ROOT, "include"), "-I", orc,
           SRC, "-o", EXE + ".tmp", "-L", pkg, "-lrma", "-L", orc, "-lrma_oracle",
           "-L", os.path.join(ROCM, "lib"), "-lamdhip64", "-lm", f"-Wl,-rpath,{rpath}"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"building {EXE} failed:\n{r.stderr}")
    os.replace(EXE + ".tmp", EXE)
    if verbose:
        print(f"built {EXE}")
    return EXE


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
