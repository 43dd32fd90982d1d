"""Build libepilora.so (the HIP kernels and the C ABI) for gfx950, in-tree.

    python -m fp4_gemm_amd.build [--jobs N] [--verbose]

Each .hip file under csrc/ is compiled to an object with hipcc, then they are
linked into fp4_gemm_amd/libepilora.so.  Flags:
  --offload-arch=gfx950                 MI355X only
  -fhip-fp32-correctly-rounded-divide-sqrt
                                        IEEE fp32 division (the activation and
                                        weight quantizers divide per element)
  -Xclang -target-feature -Xclang -packed-fp32-ops
                                        no packed fp32 instructions
No fast-math flag is used anywhere.
"""

import argparse
import concurrent.futures as cf
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
OUT = os.path.join(HERE, "libepilora.so")
# The streaming-read probe the benchmark uses as a bandwidth ceiling; a
# library of its own, outside the layer's ABI.
PROBE_SRC = os.path.join(HERE, "probe", "stream_read.hip")
PROBE_OUT = os.path.join(HERE, "libepilora_probe.so")
BUILD = os.path.join(HERE, "_build")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

CFLAGS = [
    "-O3", "-std=c++17", "-fPIC", "--offload-arch=gfx950",
    "-fhip-fp32-correctly-rounded-divide-sqrt",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function", "-Wno-unused-variable", "-Wno-unused-but-set-variable",
]


def sources():
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".hip"))


def _compile(src, verbose):
    obj = os.path.join(BUILD, os.path.basename(src)[:-4] + ".o")
    cmd = [HIPCC] + CFLAGS + ["-c", src, "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{res.stdout}\n{res.stderr}")
    if verbose and res.stderr.strip():
        print(res.stderr, file=sys.stderr)
    return obj


def _link(objs, out, verbose):
    tmp = out + ".tmp"
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp] + objs
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed:\n{res.stdout}\n{res.stderr}")
    os.replace(tmp, out)


def build(jobs=None, verbose=False):
    """Compile every kernel source and link libepilora.so (and the read
    probe's libepilora_probe.so); returns the library's path."""
    os.makedirs(BUILD, exist_ok=True)
    srcs = sources()
    jobs = jobs or min(len(srcs) + 1, os.cpu_count() or 4, 8)
    with cf.ThreadPoolExecutor(max_workers=jobs) as ex:
        futs = [ex.submit(_compile, s, verbose) for s in srcs + [PROBE_SRC]]
        objs = [f.result() for f in futs]
    _link(objs[-1:], PROBE_OUT, verbose)
    objs = objs[:-1]
    _link(objs, OUT, verbose)
    return OUT


if __name__ == "__main__":
    ap = argparse.ArgumentParser()
    ap.add_argument("--jobs", type=int, default=None)
    ap.add_argument("--verbose", action="store_true")
    a = ap.parse_args()
    print(build(a.jobs, a.verbose))
