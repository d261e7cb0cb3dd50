"""Properties of the compiled MFMA kernels that their speed rests on, checked in the gfx950
assembly hipcc emits for csrc/ffn.hip, csrc/ffn_mx.hip and csrc/router.hip (no GPU needed).

The slice copies are issued from inline asm, so the compiler's own vmcnt bookkeeping does not see
them: any `s_waitcnt vmcnt` the compiler adds waits for every copy in flight.  Such a wait inside
a K loop's MFMA blocks (for instance for a register a pending vector read would write, or the
reload of a spilled register) turns the copy ring into a serial load-then-compute loop.  The
kernels therefore must (a) spill no registers and (b) carry no compiler-inserted vmcnt wait in
any basic block that issues MFMAs.  (c) Where the accumulators live in the accumulation
registers, the innermost loop that issues MFMAs must not copy them: a branch around an MFMA once
made the compiler move every accumulator to the general registers and back around each MFMA,
which cost the router kernel more than half its time."""
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


def _inner_loop_acc_copies(body):
    """Accumulator copies (general-to-accumulation register writes other than zeroing, and
    accumulation-to-accumulation moves) in the MFMA blocks of the deepest loop level that issues
    MFMAs, by the loop depth the compiler notes at each block label."""
    blocks, cur, depth = [], [], 0
    for i, l in enumerate(body):
        m = re.match(r"^\.LBB\d+_\d+:(.*)$", l)
        if m or l.strip().startswith("s_branch") or "s_cbranch" in l:
            blocks.append((depth, cur))
            cur = []
            if m:
                notes = [m.group(1)]
                j = i + 1
                while j < len(body) and body[j].lstrip().startswith(";"):
                    notes.append(body[j])
                    j += 1
                ds = [int(x) for n in notes for x in re.findall(r"Depth=(\d+)", n)]
                depth = max(ds) if ds else 0
            continue
        cur.append(l.strip())
    blocks.append((depth, cur))
    mf = [(d, b) for d, b in blocks if any(x.startswith("v_mfma") for x in b)]
    if not mf:
        return []
    deepest = max(d for d, _ in mf)
    return [x for d, b in mf if d == deepest for x in b
            if (x.startswith("v_accvgpr_write") and not re.search(r",\s*0$", x))
            or x.startswith("v_accvgpr_mov")]


@pytest.fixture(scope="module")
def router_asm():
    return _asm("router.hip")


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


def test_router_kernels_spill_nothing_and_wait_for_no_copy(router_asm):
    ks = _kernels(router_asm, r"router_bf16_kernel")
    assert len(ks) >= 10, list(ks)
    for name, body in ks.items():
        assert _spills(router_asm, name) == 0, name
        assert _mfma_block_waits(body) == [], name


@pytest.mark.parametrize("which", ["bf16", "mx", "router"])
def test_mfma_loops_copy_no_accumulators(which, ffn_asm, ffn_mx_asm, router_asm):
    asm, pat = {"bf16": (ffn_asm, r"ffn_bf16_kernel"), "mx": (ffn_mx_asm, r"ffn_mx_kernel"),
                "router": (router_asm, r"router_bf16_kernel")}[which]
    ks = _kernels(asm, pat)
    assert len(ks) >= 2, list(ks)
    for name, body in ks.items():
        copies = _inner_loop_acc_copies(body)
        assert copies == [], (name, copies[:4])
