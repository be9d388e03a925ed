"""Build libfp4.so (the HIP/C ABI library) in-tree for gfx950.

Each .hip file under csrc/ is compiled by hipcc to an object in _build/ and
the objects are linked into bit_block_scaled_fp4_amd/libfp4.so. Flags:
  --offload-arch=gfx950           CDNA4 (MI355X) code only
  -Xclang -target-feature -Xclang -packed-fp32-ops
                                  no packed fp32 VALU instructions
  -fhip-fp32-correctly-rounded-divide-sqrt
                                  IEEE-exact fp32 division (quantiser bytes)
  -ffp-contract=off (quantize.hip only)
                                  no fused multiply-add in the quantiser
"""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libfp4.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

COMMON = ["--offload-arch=gfx950", "-O3", "-fPIC", "-std=c++17", "-Wall", "-fvisibility=hidden",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-fhip-fp32-correctly-rounded-divide-sqrt"]
# gemv_mfma.hip: MFMA results in VGPRs (the 8-row kernel adds every MFMA
# result into fp32 accumulators on the vector ALUs; AGPR results would cost a
# v_accvgpr_read per value).
PER_FILE = {"quantize.hip": ["-ffp-contract=off"],
            "gemv_mfma.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=1"]}
SOURCES = ["fp4_api.hip", "quantize.hip", "gemv.hip", "gemv_mfma.hip", "prefill.hip", "prefill_a4.hip", "argmax.hip", "device.hip",
           "read_probe.hip", "noalloc.hip", "neighbours.hip"]


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, src.replace(".hip", ".o"))
    cmd = [HIPCC, *COMMON, *PER_FILE.get(src, []), "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    msgs = [ln for ln in (r.stdout + r.stderr).splitlines() if "packed-fp32-ops" not in ln]
    if r.returncode != 0:
        raise RuntimeError("hipcc failed for %s:\n%s" % (src, "\n".join(msgs)))
    if msgs:
        sys.stderr.write("\n".join(msgs) + "\n")
    return obj


def build() -> str:
    os.makedirs(BUILD, exist_ok=True)
    with ThreadPoolExecutor(max_workers=min(4, os.cpu_count() or 1)) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp%d" % os.getpid()
    r = subprocess.run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp],
                       capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n" + r.stdout + r.stderr)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build())
