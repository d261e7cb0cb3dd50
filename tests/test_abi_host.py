"""The C-ABI library on the host (no GPU): it loads, exports every symbol include/moe.h
declares, reports the static bounds, and rejects bad arguments before launching anything."""
import ctypes
import os
import re

import pytest

from conftest import ROOT

HEADER = os.path.join(ROOT, "include", "moe.h")
LIB = os.path.join(ROOT, "mixture_experts_routed_router_amd", "libmoe.so")
INVALID, UNSUPPORTED = 1, 2


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(LIB):
        from mixture_experts_routed_router_amd import build
        build.build()
    from mixture_experts_routed_router_amd import binding
    return binding.lib()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z_0-9]+)\s*\(", text)))


def test_header_declares_the_five_calls():
    names = declared_functions()
    for call in ("moe_route", "moe_permute", "moe_plan", "moe_expert_ffn", "moe_combine"):
        assert call in names


def test_library_exports_every_declared_symbol(lib):
    for name in declared_functions():
        assert hasattr(lib, name), name


def test_static_bounds(lib):
    from mixture_experts_routed_router_amd import binding as b
    assert b.moe_max_rows(4096, 8, 64, 128) == 4096 * 8 + 64 * 127
    assert b.moe_max_rows(64, 8, 4, 128) == 64 * 4 + 4 * 127  # fewer local experts than K
    assert b.moe_max_blocks(4096, 8, 64, 8, 128) == 4096 * 8 // 128 + 64 * 8
    assert b.moe_max_blocks(100, 3, 5, 5, 16) == -(-300 // 16) + 25
    assert b.moe_max_moves(64, 8) == 72
    assert b.moe_ffn_workspace_elems(290) == 32 + 15 * 290
    assert b.moe_permute_workspace_elems(4096, 64) == 256 * 64
    assert b.moe_permute_workspace_elems(37, 3) == 3 * 3
    assert b.moe_max_rows(0, 8, 64, 128) == -1
    assert b.moe_max_rows(16, 8, 64, 100) == -1  # block_m must be a power of two in 16..256
    assert lib.moe_status_string(2) == b"unsupported shape or dtype"


# fake, 16-byte aligned device addresses: every call below must fail its host checks first
P = [ctypes.c_void_p(0x1000 * (i + 1)) for i in range(16)]
NULL = None


def test_route_rejects(lib):
    assert lib.moe_route(NULL, 8, 8, 2, 1, P[1], P[2], P[3], NULL) == INVALID
    assert lib.moe_route(P[0], 8, 8, 9, 1, P[1], P[2], P[3], NULL) == INVALID  # K > E
    assert lib.moe_route(P[0], 0, 8, 2, 1, P[1], P[2], P[3], NULL) == INVALID
    assert lib.moe_route(P[0], 8, 512, 2, 1, P[1], P[2], P[3], NULL) == UNSUPPORTED
    assert lib.moe_route(P[0], 8, 64, 17, 1, P[1], P[2], P[3], NULL) == UNSUPPORTED


def test_route_ref_and_router_reject(lib):
    assert lib.moe_route_ref(P[0], 8, 64, 4, 3, P[1], P[2], P[3], NULL) == INVALID   # k_ref < K
    assert lib.moe_route_ref(P[0], 8, 64, 4, 65, P[1], P[2], P[3], NULL) == INVALID  # k_ref > E
    assert lib.moe_route_ref(P[0], 8, 64, 4, 20, P[1], P[2], P[3], NULL) == UNSUPPORTED
    rt = lambda x=P[0], dt=1, T=64, H=128, E=64, K=4, k_ref=4: lib.moe_router_topk(
        x, dt, P[1], T, H, E, K, k_ref, NULL, P[2], P[3], P[4], NULL)
    assert rt(x=NULL) == INVALID
    assert rt(dt=3) == INVALID
    assert rt(k_ref=2) == INVALID
    assert rt(x=ctypes.c_void_p(0x1008)) == INVALID   # misaligned
    assert rt(H=100) == UNSUPPORTED                   # bf16 needs H % 64 == 0
    assert rt(E=300, K=4) == UNSUPPORTED


def _permute(lib, **kw):
    a = dict(x=P[0], dt=1, T=64, H=128, K=2, E=8, ids=P[1], counts=P[2], begin=0, stride=1,
             E_loc=8, bm=128, offsets=P[3], entry_pos=P[4], row_token=P[5], xp=P[6],
             max_rows=64 * 2 + 8 * 127, ws=P[7], ws_elems=4 * 8)
    a.update(kw)
    return lib.moe_permute(a["x"], a["dt"], a["T"], a["H"], a["K"], a["E"], a["ids"],
                           a["counts"], a["begin"], a["stride"], a["E_loc"], a["bm"],
                           a["offsets"], a["entry_pos"], a["row_token"], a["xp"], a["max_rows"],
                           a["ws"], a["ws_elems"], NULL)


def test_permute_rejects(lib):
    assert _permute(lib, x=NULL) == INVALID
    assert _permute(lib, dt=7) == INVALID
    assert _permute(lib, bm=100) == INVALID
    assert _permute(lib, max_rows=64 * 2 + 8 * 127 - 1) == INVALID  # below the static bound
    assert _permute(lib, ws_elems=31) == INVALID
    assert _permute(lib, H=100) == INVALID                          # 200-byte rows
    assert _permute(lib, x=ctypes.c_void_p(0x1008)) == INVALID      # misaligned
    assert _permute(lib, begin=3, stride=1, E_loc=6) == INVALID     # local set past E
    assert _permute(lib, K=9) == INVALID                            # K > E


def test_plan_rejects(lib):
    def plan(E=8, begin=0, stride=1, E_loc=8, Pn=4, bm=128, max_moves=12, max_blocks=16,
             counts=P[0], moves=P[2], blocks=P[4]):
        return lib.moe_plan(counts, E, begin, stride, E_loc, Pn, bm, P[1], moves, P[3], max_moves,
                            blocks, P[5], max_blocks, NULL, NULL)
    assert plan(counts=NULL) == INVALID
    # moves and blocks are written as 16-byte records
    assert plan(moves=ctypes.c_void_p(P[2].value + 4)) == INVALID
    assert plan(blocks=ctypes.c_void_p(P[4].value + 8)) == INVALID
    assert plan(Pn=3) == INVALID            # P must divide E_loc
    assert plan(bm=48) == INVALID
    assert plan(max_blocks=0) == INVALID
    assert plan(E=256, E_loc=256, Pn=128) == UNSUPPORTED
    assert plan(E=512, E_loc=512, Pn=8) == UNSUPPORTED


def test_plan_blocks_rejects(lib):
    def plan(E=8, begin=0, stride=1, E_loc=8, Pn=4, bm=128, s=1, max_moves=32, max_blocks=16,
             counts=P[0]):
        return lib.moe_plan_blocks(counts, E, begin, stride, E_loc, Pn, bm, s, P[1], P[2], P[3],
                                   max_moves, P[4], P[5], max_blocks, NULL, NULL)
    assert plan(counts=NULL) == INVALID
    assert plan(Pn=3) == INVALID            # P must divide E_loc
    assert plan(bm=48) == INVALID
    assert plan(s=-1) == INVALID
    assert plan(max_blocks=0) == INVALID
    assert plan(E=256, E_loc=256, Pn=128) == UNSUPPORTED
    assert plan(E=128, E_loc=128, Pn=1) == UNSUPPORTED    # 128 experts per rank
    assert plan(s=70000) == UNSUPPORTED


def test_mx_quantize_rejects(lib):
    q = lambda src=P[0], dt=1, rows=4, cols=64, fmt=0, codes=P[1], scales=P[2]: \
        lib.moe_mx_quantize(src, dt, rows, cols, fmt, codes, scales, NULL)
    assert q(src=NULL) == INVALID
    assert q(cols=48) == INVALID          # not a multiple of 32
    assert q(fmt=2) == INVALID
    assert q(dt=5) == INVALID
    assert q(codes=ctypes.c_void_p(0x1004)) == INVALID  # misaligned


def test_mx_scale_pitch(lib):
    assert lib.moe_mx_scale_pitch(2048) == 64
    assert lib.moe_mx_scale_pitch(2880) == 92   # 90 scales, padded to a multiple of 4
    assert lib.moe_mx_scale_pitch(64) == 4
    assert lib.moe_mx_scale_pitch(32) == 4


def test_mx_ffn_rejects(lib):
    def ffn(xq=P[0], xs=P[1], row_token=P[2], x_rows=64, H=128, I=256, blocks=P[3],
            ws_elems=272, max_rows=1024, w1s=P[5]):
        return lib.moe_expert_ffn_mx(xq, xs, row_token, x_rows, P[4], w1s, P[6], P[7], H, I, 8,
                                     blocks, P[8], 16, P[9], P[10], P[11], max_rows, P[12],
                                     ws_elems, NULL)
    assert ffn(xq=NULL) == INVALID
    assert ffn(blocks=NULL) == INVALID
    assert ffn(xq=ctypes.c_void_p(0x1008)) == INVALID        # codes 16-byte aligned
    assert ffn(w1s=ctypes.c_void_p(0x1002)) == INVALID       # scales 4-byte aligned
    assert ffn(H=96) == UNSUPPORTED                          # multiples of 64
    assert ffn(I=2880 + 32) == UNSUPPORTED
    assert ffn(H=32) == INVALID
    assert ffn(ws_elems=271) == INVALID
    assert ffn(x_rows=0) == INVALID
    assert ffn(row_token=NULL, x_rows=1000) == INVALID       # materialised rows < max_rows
    assert ffn(x_rows=1 << 23, H=1024) == UNSUPPORTED        # 8 GiB of codes: 32-bit offsets
    assert lib.moe_expert_ffn_mx_fc2(P[0], P[1], P[2], P[3], 128, 256, 8, P[4], P[5], 16,
                                     ctypes.c_void_p(0x1008), 1024, P[6], 272, NULL) == INVALID


def test_ffn_and_combine_reject(lib):
    ffn = lambda dt, H, I, blocks=P[3], ws_elems=272: lib.moe_expert_ffn(
        P[0], P[1], P[2], dt, H, I, 8, blocks, P[4], 16, P[5], P[6], 1024, P[7], ws_elems, NULL)
    assert ffn(1, 128, 256, blocks=NULL) == INVALID
    assert ffn(5, 128, 256) == INVALID
    assert ffn(1, 2880, 100) == UNSUPPORTED   # bf16 needs multiples of 64
    assert ffn(0, 126, 256) == UNSUPPORTED    # float32 needs multiples of 4
    assert ffn(1, 128, 256, ws_elems=271) == INVALID  # schedule scratch below 32 + 15*max_blocks
    gather = lambda row_token=P[8], T=64, H=128, ws_elems=272: lib.moe_expert_ffn_gather(
        P[0], row_token, T, P[1], P[2], 1, H, 256, 8, P[3], P[4], 16, P[5], P[6], 1024, P[7],
        ws_elems, NULL)
    sched = lib.moe_expert_ffn_tile_schedule
    assert sched(P[3], P[4], 16, 8, 1024, P[7], 271, NULL) == INVALID
    assert sched(NULL, P[4], 16, 8, 1024, P[7], 272, NULL) == INVALID
    assert sched(P[3], P[4], 16, 300, 1024, P[7], 272, NULL) == UNSUPPORTED
    assert sched(P[3], P[4], 16, 8, 0, P[7], 272, NULL) == INVALID              # no rows
    assert sched(ctypes.c_void_p(0x1008), P[4], 16, 8, 1024, P[7], 272, NULL) == INVALID  # 16-B records
    assert ffn(1, 128, 256, blocks=ctypes.c_void_p(0x1008)) == INVALID
    assert gather(row_token=NULL) == INVALID
    assert gather(T=0) == INVALID
    assert gather(ws_elems=271) == INVALID
    assert gather(T=1 << 22, H=1024) == UNSUPPORTED  # 8 GiB of x: past 32-bit row offsets
    assert lib.moe_combine(P[0], 1, P[1], P[2], 4, 100, 2, P[3], NULL) == INVALID  # 200-B rows
    assert lib.moe_combine(P[0], 1, P[1], NULL, 4, 128, 2, P[3], NULL) == INVALID
    assert lib.moe_combine(P[0], 1, P[1], P[2], 0, 128, 2, P[3], NULL) == INVALID
    assert lib.moe_combine(P[0], 1, P[1], P[2], 4, 128, 17, P[3], NULL) == UNSUPPORTED  # K > 16


def test_direct_rows_reject(lib):
    def fc2d(act=P[0], row_token=P[7], entry_pos=P[8], topk_w=P[9], out=P[10], row_direct=P[11],
             dt=1, H=128, I=256, T=64, K=8, max_rows=1024, ws_elems=272, E_loc=8):
        return lib.moe_expert_ffn_fc2_direct(act, P[1], dt, H, I, E_loc, P[2], P[3], 16, P[4],
                                             max_rows, row_token, entry_pos, topk_w, T, K, out,
                                             row_direct, P[5], ws_elems, NULL)
    for arg in ("act", "row_token", "entry_pos", "topk_w", "out", "row_direct"):
        assert fc2d(**{arg: NULL}) == INVALID, arg
    assert fc2d(out=ctypes.c_void_p(0x1008)) == INVALID    # 16-byte aligned rows
    assert fc2d(T=0) == INVALID
    assert fc2d(K=0) == INVALID
    assert fc2d(K=17) == UNSUPPORTED                        # the combine's top-k bound
    assert fc2d(ws_elems=271) == INVALID
    assert fc2d(H=2880, I=100) == UNSUPPORTED               # bf16 needs multiples of 64
    assert fc2d(E_loc=300) == UNSUPPORTED
    assert fc2d(max_rows=1 << 27) == UNSUPPORTED            # 32-bit offsets into row_direct
    mx = lambda actq=P[0], row_token=P[7], out=P[10], K=8, ws_elems=272: (
        lib.moe_expert_ffn_mx_fc2_direct(actq, P[1], P[2], P[3], 128, 256, 8, P[4], P[5], 16,
                                         P[6], 1024, row_token, P[8], P[9], 64, K, out, P[11],
                                         P[12], ws_elems, NULL))
    assert mx(actq=NULL) == INVALID
    assert mx(row_token=NULL) == INVALID
    assert mx(out=ctypes.c_void_p(0x1008)) == INVALID
    assert mx(ws_elems=271) == INVALID
    assert mx(K=17) == UNSUPPORTED
    multi = lib.moe_combine_multi
    assert multi(P[0], 1, P[1], P[2], 4, 100, 2, P[3], NULL) == INVALID  # 200-B rows
    assert multi(P[0], 1, P[1], NULL, 4, 128, 2, P[3], NULL) == INVALID
    assert multi(P[0], 3, P[1], P[2], 4, 128, 2, P[3], NULL) == INVALID
    assert multi(P[0], 1, P[1], P[2], 4, 128, 17, P[3], NULL) == UNSUPPORTED


def test_binding_fails_loudly_without_a_gpu_tensor(lib):
    import torch
    from mixture_experts_routed_router_amd import binding
    with pytest.raises(binding.MoeError):
        binding.moe_route(torch.zeros(4, 8), 2, torch.zeros(4, 2, dtype=torch.int32),
                          torch.zeros(4, 2), torch.zeros(8, dtype=torch.int32))
