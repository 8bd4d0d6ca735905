"""The weight ring's wait counts in the compiled main loops (host only: the
kernels are compiled to gfx950 assembly here, nothing runs).

Every kernel keeps D groups of weights in flight; the compiler's
`s_waitcnt vmcnt(N)` before each group must wait for that group only.  A
`vmcnt(0)` inside the main loop drains the ring and turns the stream into
one memory round trip per window -- this happened to the BF16 control's
LDS-staged kernels (the x chunk loaded after the ring was primed), which
made the control slower than its W12 counterpart for a reason that has
nothing to do with the weight format.  These tests pin exact waits for the
three fetches (W12, BF16, W12 with an exception list) in the kernels the
defaults use from M = 9 to 32."""
import os
import re
import shutil
import subprocess

import pytest

from lossless_bit_weight_amd import build

pytestmark = pytest.mark.skipif(shutil.which(build.HIPCC) is None and not os.path.exists(build.HIPCC),
                                reason="hipcc not available")


def _asm(define: str, tmp_path) -> str:
    out = tmp_path / (define + ".s")
    flags = [f for f in build.FLAGS if not f.startswith("-Rpass")]
    cmd = [build.HIPCC, *flags, "-D" + define, "--cuda-device-only", "-S",
           os.path.join(build.CSRC, "w12_gemm_inst.hip"), "-o", str(out)]
    subprocess.run(cmd, check=True, capture_output=True, text=True)
    return out.read_text()


def _main_loop(asm: str, fetch: str, targs: str) -> list[str]:
    """The loop with the most matrix-core instructions in the kernel
    gemm_kernel<fetch, targs...> (its main loop)."""
    name = "_ZN3w124kern11gemm_kernelINS0_%d%sE%sEEEvNS_8GemmArgsE" % (len(fetch), fetch, targs)
    i = asm.index(name + ":")
    lines = asm[i:asm.index(".Lfunc_end", i)].splitlines()
    labels = {m.group(1): k for k, l in enumerate(lines) if (m := re.match(r"(\.LBB\d+_\d+):", l))}
    best = None
    for k, l in enumerate(lines):
        m = re.search(r"s_cbranch\w* (\.LBB\d+_\d+)|s_branch (\.LBB\d+_\d+)", l)
        if not m:
            continue
        head = labels.get(m.group(1) or m.group(2))
        if head is None or head >= k:
            continue
        body = lines[head:k + 1]
        mfmas = sum(1 for b in body if "v_mfma" in b)
        if best is None or mfmas > best[0]:
            best = (mfmas, body)
    assert best is not None and best[0] > 0, name
    return best[1]


# gemm_kernel<F, MFMA, MR, R, KW, D, CHUNKED, XD, NW> as mangled template
# arguments: 512-thread workgroups with x staged in LDS in chunks (the
# defaults from M = 9), 16 and 32 rows, two and four K-waves
MFMA8_CHUNKED = ["Lb1ELi16ELi1ELi4ELi2ELb1ELb0ELi8", "Lb1ELi32ELi1ELi2ELi2ELb1ELb0ELi8",
                 "Lb1ELi32ELi1ELi4ELi2ELb1ELb0ELi8"]


@pytest.fixture(scope="module")
def mfma8_asm(tmp_path_factory):
    return _asm("W12_INST_MFMA8", tmp_path_factory.mktemp("isa"))


@pytest.mark.parametrize("fetch", ["FetchW12", "FetchBF16", "FetchW12X"])
@pytest.mark.parametrize("targs", MFMA8_CHUNKED)
def test_chunked_loop_waits_exactly(mfma8_asm, fetch, targs):
    body = _main_loop(mfma8_asm, fetch, targs)
    waits = [l for l in body if "s_waitcnt" in l and "vmcnt" in l]
    assert waits, "no weight waits in the loop at all"
    assert not any(re.search(r"vmcnt\(0\)", w) for w in waits), (fetch, targs, waits)


# 1024-thread workgroups (the down projection's default from M = 9)
MFMA16_CHUNKED = ["Lb1ELi16ELi1ELi4ELi2ELb1ELb0ELi16", "Lb1ELi32ELi1ELi4ELi2ELb1ELb0ELi16"]


@pytest.fixture(scope="module")
def mfma16_asm(tmp_path_factory):
    return _asm("W12_INST_MFMA16", tmp_path_factory.mktemp("isa16"))


@pytest.mark.parametrize("fetch", ["FetchW12", "FetchBF16"])
@pytest.mark.parametrize("targs", MFMA16_CHUNKED)
def test_chunked_loop_waits_exactly_16_waves(mfma16_asm, fetch, targs):
    body = _main_loop(mfma16_asm, fetch, targs)
    waits = [l for l in body if "s_waitcnt" in l and "vmcnt" in l]
    assert waits, "no weight waits in the loop at all"
    assert not any(re.search(r"vmcnt\(0\)", w) for w in waits), (fetch, targs, waits)


@pytest.mark.parametrize("targs", MFMA8_CHUNKED)
def test_in_loop_corrections_wait_for_nothing(mfma8_asm, targs):
    """With an exception list the LDS-staged kernels apply each group's
    entries inside the main loop, reading them with v_readlane from
    registers loaded in the prologue (the kernel's only lane reads).  They
    are waited for once, before the loop; a wait on memory in front of
    those reads would stall every pass."""
    name = "_ZN3w124kern11gemm_kernelINS0_9FetchW12XE%sEEEvNS_8GemmArgsE" % targs
    i = mfma8_asm.index(name + ":")
    body = mfma8_asm[i:mfma8_asm.index(".Lfunc_end", i)].splitlines()
    reads = [k for k, l in enumerate(body) if "v_readlane" in l]
    assert reads, "no in-loop corrections found"
    for k in reads:
        assert not any("vmcnt" in l for l in body[max(0, k - 4):k]), (targs, body[max(0, k - 4):k + 1])
