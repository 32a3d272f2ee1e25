"""Build libnvfp4.so (gfx950) in-tree with hipcc.

All kernels and the C ABI layer go into one shared library next to this file.
FP contraction is off (the kernels ask for fused multiply-adds explicitly
where they want them) and packed fp32 instructions are disabled.
"""
import glob
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
OUT = os.path.join(HERE, "libnvfp4.so")
# Reference-rate probes the benchmark measures the chip with (not the NVFP4 path).
PROBES_SRC = os.path.join(HERE, "probes", "peaks.hip")
PROBES_OUT = os.path.join(HERE, "libnvfp4_probes.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared", "-ffp-contract=off",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", "-Wno-unused-command-line-argument"]


def sources():
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")))


def build(verbose: bool = False, extra=()) -> str:
    tmp = OUT + ".tmp"
    cmd = [HIPCC] + FLAGS + list(extra) + sources() + ["-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    err = "\n".join(l for l in (r.stderr or "").splitlines()
                    if "packed-fp32-ops" not in l and l.strip())
    if r.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + err)
    if verbose and err:
        print(err)
    # -shared links with unresolved symbols allowed; a kernel whose host stub
    # failed to instantiate would only show up at load time.  Refuse it here.
    nm = subprocess.run(["nm", "-D", "--undefined-only", tmp], capture_output=True, text=True)
    missing = [l.split()[-1] for l in nm.stdout.splitlines() if "nvfp4" in l]
    if nm.returncode != 0 or missing:
        os.remove(tmp)
        raise RuntimeError("libnvfp4.so has unresolved library symbols: " + ", ".join(missing or [nm.stderr]))
    os.replace(tmp, OUT)
    build_probes(verbose)
    return OUT


def build_probes(verbose: bool = False) -> str:
    tmp = PROBES_OUT + ".tmp"
    cmd = [HIPCC] + FLAGS + [PROBES_SRC, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed on the probes:\n" + (r.stderr or ""))
    os.replace(tmp, PROBES_OUT)
    return PROBES_OUT


if __name__ == "__main__":
    build(verbose=True, extra=sys.argv[1:])
