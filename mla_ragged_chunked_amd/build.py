"""Build libmla_ragged.so in-tree with hipcc for gfx950.

Every source in csrc/ is compiled to an object under _build/ (in parallel)
and linked into mla_ragged_chunked_amd/libmla_ragged.so. Always compiles:
the result is what the tests, the smoke check and the benchmark load.
"""
import os
import subprocess
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libmla_ragged.so")
ROOT = os.path.dirname(HERE)

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
COMMON = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
          "-I", os.path.join(ROOT, "include"),
          # packed fp32 VALU ops stay off (hipcc would otherwise form them)
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-Wno-unused-command-line-argument",
          # the LDS DMA asm in the prefill kernel declares M0 clobbered on purpose
          "-Wno-inline-asm"]
SOURCES = ["abi.cpp", "planner.cpp", "prefill_bf16.hip", "prefill_fp32.hip", "merge.hip",
           "decompress.hip", "device_plan.hip", "prefill_absorbed.hip", "decompress_prefill.hip"]
# Per-source flags. The fused decompression + prefill kernel holds 256
# registers of weights per lane; with MFMA results in VGPRs those weights
# fill the AGPRs as MFMA sources and nothing is copied between the two
# files or spilled (the default form keeps results in AGPRs and spills).
SOURCE_FLAGS = {"decompress_prefill.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=1"]}


def _compile(src: str, extra=()) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    lang = ["-x", "hip"] if src.endswith(".hip") else []
    cmd = [HIPCC, *COMMON, *SOURCE_FLAGS.get(src, []), *extra, *lang, "-c",
           os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    msgs = "\n".join(l for l in (r.stdout + r.stderr).splitlines() if noise not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{' '.join(cmd)}\n{msgs}")
    if msgs.strip():
        print(msgs)
    return obj


def build(verbose: bool = False, extra=()) -> str:
    os.makedirs(BUILD, exist_ok=True)
    with ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
        objs = list(ex.map(lambda s: _compile(s, extra), SOURCES))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, "-shared", "-fPIC", f"--offload-arch={ARCH}", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{' '.join(cmd)}\n{r.stdout}{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


if __name__ == "__main__":
    build(verbose=True)
