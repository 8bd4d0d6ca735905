"""Build libw12.so (the HIP C-ABI library) in-tree for gfx950.

    python -m lossless_bit_weight_amd.build

Each .hip source is compiled to an object in parallel, then linked with
hipcc into lossless_bit_weight_amd/libw12.so.  Packed-FP32 instruction
selection is disabled for device code.
"""
from __future__ import annotations

import os
import re
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
OUT = os.path.join(HERE, "libw12.so")
BUILD_DIR = os.path.join(ROOT, "_build")
# (source, object name, extra defines): the kernel instantiation unit is
# compiled once per x height so the build runs in parallel.
SOURCES = [("w12_api.hip", "w12_api", []), ("w12_pack.hip", "w12_pack", []),
           ("w12_exc.hip", "w12_exc", []), ("w12_gemm.hip", "w12_gemm", []),
           ("w12_probe.hip", "w12_probe", [])]
SOURCES += [("w12_gemm_inst.hip", "w12_gemv_m%d" % m, ["-DW12_INST_M=%d" % m]) for m in range(1, 9)]
SOURCES += [("w12_gemm_inst.hip", "w12_mfma", ["-DW12_INST_MFMA"]),
            ("w12_gemm_inst.hip", "w12_mfma8", ["-DW12_INST_MFMA8"]),
            ("w12_gemm_inst.hip", "w12_mfma16", ["-DW12_INST_MFMA16"]),
            ("w12_gemm_inst.hip", "w12_mfma8_big", ["-DW12_INST_MFMA8_BIG"])]
ARCH = os.environ.get("W12_OFFLOAD_ARCH", "gfx950")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC",
    "-Rpass-analysis=kernel-resource-usage",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function", "-I" + os.path.join(ROOT, "include"),
]


def _check_resources(src: str, remarks: list[str]) -> None:
    """Fail the build if any kernel spills to scratch memory: a variant that
    round-trips registers through memory is never worth shipping.  (A VGPR
    spilled into an accumulation register, with no scratch, costs two moves
    and is allowed.)"""
    kernel = None
    bad = []
    for line in remarks:
        m = re.search(r"remark: Function Name: (\S+)", line)
        if m:
            kernel = m.group(1)
            continue
        m = re.search(r"remark: +(ScratchSize \[bytes/lane\]): (\d+)", line)
        if m and int(m.group(2)) > 0:
            bad.append("%s: %s = %s" % (kernel, m.group(1), m.group(2)))
    if bad:
        raise RuntimeError("kernels in %s spill or use scratch:\n  %s" % (src, "\n  ".join(bad)))


def _compile(item) -> str:
    src, name, defines = item
    obj = os.path.join(BUILD_DIR, name + ".o")
    cmd = [HIPCC, *FLAGS, *defines, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    lines = r.stderr.splitlines()
    remarks = [l for l in lines if "remark:" in l]
    # the host pass does not know the device-only feature flag: drop that note
    err = "\n".join(l for l in lines
                    if "packed-fp32-ops" not in l and "remark:" not in l and l.strip()
                    and not l.lstrip().startswith(("|", "^")) and not re.match(r"^\s*\d+ \|", l))
    if r.returncode != 0:
        raise RuntimeError("hipcc failed for %s:\n%s" % (src, err))
    try:
        _check_resources(name, remarks)
    except RuntimeError:
        os.remove(obj)   # never link, or later reuse, an object that spills
        raise
    return obj


def build() -> str:
    os.makedirs(BUILD_DIR, exist_ok=True)
    workers = max(1, min(len(SOURCES), os.cpu_count() or 1))
    with ThreadPoolExecutor(max_workers=workers) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = OUT + ".tmp%d" % os.getpid()
    subprocess.check_call([HIPCC, "--offload-arch=" + ARCH, "-shared", "-fPIC", *objs, "-o", tmp])
    os.replace(tmp, OUT)
    return OUT


if __name__ == "__main__":
    print(build())
