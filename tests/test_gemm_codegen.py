"""Properties of the compiled grouped GEMMs that their speed rests on, checked in the gfx950
assembly hipcc emits for csrc/ffn.hip and csrc/ffn_mx.hip (no GPU needed).

The slice copies are issued from inline asm, so the compiler's own vmcnt bookkeeping does not see
them: any `s_waitcnt vmcnt` the compiler adds waits for every copy in flight.  Such a wait inside
a K loop's MFMA blocks (for instance for a register a pending vector read would write, or the
reload of a spilled register) turns the copy ring into a serial load-then-compute loop.  The GEMM
kernels therefore must (a) spill no registers and (b) carry no compiler-inserted vmcnt wait in
any basic block that issues MFMAs."""
import os
import re
import subprocess

import pytest

from conftest import ROOT

CSRC = os.path.join(ROOT, "mixture_experts_routed_router_amd", "csrc")


def _asm(src):
    from mixture_experts_routed_router_amd import build
    cmd = [build.hipcc(), *build.COMPILE_FLAGS, "-I", os.path.join(ROOT, "include"), "--cuda-device-only",
           "-S", "-o", "-", os.path.join(CSRC, src)]
    return subprocess.run(cmd, check=True, capture_output=True, text=True).stdout


def _kernels(asm, pattern):
    """{name: list of asm lines} of the kernels whose symbol matches pattern."""
    lines = asm.split("\n")
    out = {}
    for i, l in enumerate(lines):
        m = re.match(r"^(_Z\S+):\s*(;.*)?$", l)
        if m and re.search(pattern, m.group(1)):
            j = next(k for k in range(i, len(lines)) if "s_endpgm" in lines[k])
            out[m.group(1)] = lines[i:j + 1]
    return out


def _mfma_block_waits(body):
    """Compiler-inserted (outside inline asm) vmcnt waits in basic blocks that issue MFMAs."""
    bad, block, in_asm = [], [], False
    def flush():
        if any("v_mfma" in x for x in block):
            bad.extend(x for x in block if x.startswith("!"))
    for l in body:
        if ";;#ASMSTART" in l:
            in_asm = True
        elif ";;#ASMEND" in l:
            in_asm = False
            continue
        if re.match(r"^\.LBB\d+_\d+:", l) or l.strip().startswith("s_branch") or "s_cbranch" in l:
            flush()
            block = []
            continue
        t = l.strip()
        if t.startswith("s_waitcnt") and "vmcnt" in t and not in_asm:
            block.append("!" + t)
        elif t.startswith("v_mfma"):
            block.append(t)
    flush()
    return bad


@pytest.fixture(scope="module")
def ffn_asm():
    return _asm("ffn.hip")


@pytest.fixture(scope="module")
def ffn_mx_asm():
    return _asm("ffn_mx.hip")


def _spills(asm, name):
    m = re.search(re.escape(name) + r"[\s\S]*?\.vgpr_spill_count:\s+(\d+)", asm.split(".amdgpu_metadata")[-1])
    return int(m.group(1))


@pytest.mark.parametrize("which", ["bf16", "mx"])
def test_gemm_kernels_spill_nothing(which, ffn_asm, ffn_mx_asm):
    asm = ffn_asm if which == "bf16" else ffn_mx_asm
    pat = r"ffn_bf16_kernel" if which == "bf16" else r"ffn_mx_kernel"
    ks = _kernels(asm, pat)
    assert len(ks) >= 2, list(ks)
    for name in ks:
        assert _spills(asm, name) == 0, name


@pytest.mark.parametrize("which", ["bf16", "mx"])
def test_gemm_mfma_blocks_have_no_compiler_vmcnt_waits(which, ffn_asm, ffn_mx_asm):
    asm = ffn_asm if which == "bf16" else ffn_mx_asm
    pat = r"ffn_bf16_kernel" if which == "bf16" else r"ffn_mx_kernel"
    ks = _kernels(asm, pat)
    assert len(ks) >= 2, list(ks)
    for name, body in ks.items():
        assert sum("v_mfma" in l for l in body) > 0, name
        assert _mfma_block_waits(body) == [], name
