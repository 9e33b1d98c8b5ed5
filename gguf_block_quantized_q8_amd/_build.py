"""Build libggq.so (the HIP library behind include/ggq.h) for gfx950, in-tree.

Every csrc/*.hip file is compiled with hipcc to an object (in parallel) and
linked into gguf_block_quantized_q8_amd/libggq.so.  No fast-math: the q8_1
quantizer relies on IEEE fp32 division.  Packed fp32 VALU instructions are
disabled.
"""
import concurrent.futures as cf
import glob
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libggq.so")
ARCH = "gfx950"
FLAGS = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-munsafe-fp-atomics", "-Wall", "-Wno-unused-function",
         "-I", os.path.join(HERE, "..", "include")]


def sources():
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")))


# Per-source flags: the MFMA kernels keep their accumulators in ordinary VGPRs
# (no AGPR round trip before the fp32 rescale that follows each MFMA).
SRC_FLAGS = {"mmq.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=1"],
             "ceiling.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=1"]}


def _compile(src, verbose):
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    cmd = ["hipcc", *FLAGS, *SRC_FLAGS.get(os.path.basename(src), []), "-c", src, "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    out = "\n".join(l for l in (r.stdout + r.stderr).splitlines() if "not a recognized feature" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{out}")
    if out.strip() and verbose:
        print(out, flush=True)
    return obj


def build(verbose: bool = False, jobs: int = 8) -> str:
    os.makedirs(BUILD, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose), sources()))
    cmd = ["hipcc", "-shared", f"--offload-arch={ARCH}", "-o", LIB + ".tmp", *objs]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(LIB + ".tmp", LIB)
    return LIB


def build_host_sanitized(out: str) -> str:
    """libggq with the C ABI's host code (api.hip: validation, workspace carving,
    dispatch) under clang's AddressSanitizer and UndefinedBehaviorSanitizer; the
    kernel sources are linked from the regular build's objects (build() first).
    Device code is never instrumented.  Load it into a process that preloads the
    clang ASan runtime."""
    objs = [os.path.join(BUILD, os.path.basename(s) + ".o") for s in sources() if not s.endswith("api.hip")]
    missing = [o for o in objs if not os.path.exists(o)]
    if missing:
        raise RuntimeError(f"build() first: missing {missing}")
    api_o = out + ".api.o"
    san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-omit-frame-pointer", "-Xarch_host", "-fno-sanitize-recover=undefined"]
    flags = [f for f in FLAGS if f != "-O3"] + ["-O1", "-g"]
    src = os.path.join(CSRC, "api.hip")
    r = subprocess.run(["hipcc", *flags, *san, "-c", src, "-o", api_o], capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stderr}")
    subprocess.run(["hipcc", "-shared", f"--offload-arch={ARCH}", "-o", out, api_o, *objs], check=True)
    os.remove(api_o)
    return out


if __name__ == "__main__":
    print(build(verbose=True))
