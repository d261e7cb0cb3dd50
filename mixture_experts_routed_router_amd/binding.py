"""Python binding of libmoe: one function per C-ABI call, same names, argument marshalling only.

Every function takes torch CUDA tensors (device memory) and passes their data pointers and
the current HIP stream to the C call; all computation happens in the HIP kernels of
libmoe.so.  There is no fallback: if the library is missing, or a call returns an error,
a ``MoeError`` is raised.

``RoutedExperts`` holds every buffer of the path, allocated once at the static bounds the
library reports (no allocation per call), and runs the five calls in order on one stream.
"""
from __future__ import annotations

import ctypes
import os

import torch

_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libmoe.so")
_lib = None

MOE_F32, MOE_BF16 = 0, 1
_STATUS = {0: "ok", 1: "invalid argument", 2: "unsupported shape or dtype", 3: "kernel launch failed"}

_vp = ctypes.c_void_p
_i32 = ctypes.c_int
_i64 = ctypes.c_int64

# name -> (restype, argtypes); mirrors include/moe.h
_SIGNATURES = {
    "moe_status_string": (ctypes.c_char_p, [_i32]),
    "moe_max_rows": (_i64, [_i32, _i32, _i32, _i32]),
    "moe_max_blocks": (ctypes.c_int32, [_i32, _i32, _i32, _i32, _i32]),
    "moe_max_moves": (ctypes.c_int32, [_i32, _i32]),
    "moe_permute_workspace_elems": (_i64, [_i32, _i32]),
    "moe_ffn_workspace_elems": (_i64, [_i32]),
    "moe_route": (_i32, [_vp, _i32, _i32, _i32, _i32, _vp, _vp, _vp, _vp]),
    "moe_permute": (_i32, [_vp, _i32, _i32, _i32, _i32, _i32, _vp, _vp, _i32, _i32, _i32, _i32,
                           _vp, _vp, _vp, _vp, _i64, _vp, _i64, _vp]),
    "moe_plan": (_i32, [_vp, _i32, _i32, _i32, _i32, _i32, _i32, _vp, _vp, _vp, _i32, _vp, _vp,
                        _i32, _vp, _vp]),
    "moe_expert_ffn": (_i32, [_vp, _vp, _vp, _i32, _i32, _i32, _i32, _vp, _vp, _i32, _vp, _vp,
                              _i64, _vp, _i64, _vp]),
    "moe_expert_ffn_fc1": (_i32, [_vp, _vp, _i32, _i32, _i32, _i32, _vp, _vp, _i32, _vp, _i64,
                                  _vp, _i64, _vp]),
    "moe_expert_ffn_fc2": (_i32, [_vp, _vp, _i32, _i32, _i32, _i32, _vp, _vp, _i32, _vp, _i64,
                                  _vp, _i64, _vp]),
    "moe_expert_ffn_gather": (_i32, [_vp, _vp, _i32, _vp, _vp, _i32, _i32, _i32, _i32, _vp,
                                     _vp, _i32, _vp, _vp, _i64, _vp, _i64, _vp]),
    "moe_expert_ffn_gather_noalloc": (_i32, [_vp, _vp, _i32, _vp, _vp, _i32, _i32, _i32, _i32,
                                             _vp, _vp, _i32, _vp, _vp, _i64, _vp]),
    "moe_expert_ffn_fc1_gather": (_i32, [_vp, _vp, _i32, _vp, _i32, _i32, _i32, _i32, _vp, _vp,
                                         _i32, _vp, _i64, _vp, _i64, _vp]),
    "moe_expert_ffn_tile_schedule": (_i32, [_vp, _vp, _i32, _i32, _i64, _vp, _i64, _vp]),
    "moe_plan_blocks": (_i32, [_vp, _i32, _i32, _i32, _i32, _i32, _i32, _i32, _vp, _vp, _vp, _i32,
                               _vp, _vp, _i32, _vp, _vp]),
    "moe_mx_quantize": (_i32, [_vp, _i32, _i64, _i64, _i32, _vp, _vp, _vp]),
    "moe_mx_scale_pitch": (_i64, [_i64]),
    "moe_expert_ffn_mx": (_i32, [_vp, _vp, _vp, _i64, _vp, _vp, _vp, _vp, _i32, _i32, _i32, _vp,
                                 _vp, _i32, _vp, _vp, _vp, _i64, _vp, _i64, _vp]),
    "moe_expert_ffn_mx_fc1": (_i32, [_vp, _vp, _vp, _i64, _vp, _vp, _i32, _i32, _i32, _vp, _vp,
                                     _i32, _vp, _vp, _i64, _vp, _i64, _vp]),
    "moe_expert_ffn_mx_fc2": (_i32, [_vp, _vp, _vp, _vp, _i32, _i32, _i32, _vp, _vp, _i32, _vp,
                                     _i64, _vp, _i64, _vp]),
    "moe_route_ref": (_i32, [_vp, _i32, _i32, _i32, _i32, _vp, _vp, _vp, _vp]),
    "moe_router_topk": (_i32, [_vp, _i32, _vp, _i32, _i32, _i32, _i32, _i32, _vp, _vp, _vp, _vp,
                               _vp]),
    "moe_combine": (_i32, [_vp, _i32, _vp, _vp, _i32, _i32, _i32, _vp, _vp]),
    "moe_combine_multi": (_i32, [_vp, _i32, _vp, _vp, _i32, _i32, _i32, _vp, _vp]),
    "moe_expert_ffn_mx_fc2_direct": (_i32, [_vp, _vp, _vp, _vp, _i32, _i32, _i32, _vp, _vp, _i32,
                                            _vp, _i64, _vp, _vp, _vp, _i32, _i32, _vp, _vp, _vp,
                                            _i64, _vp]),
    "moe_expert_ffn_fc2_direct": (_i32, [_vp, _vp, _i32, _i32, _i32, _i32, _vp, _vp, _i32, _vp,
                                         _i64, _vp, _vp, _vp, _i32, _i32, _vp, _vp, _vp, _i64,
                                         _vp]),
}


class MoeError(RuntimeError):
    pass


def library_path() -> str:
    return _LIB_PATH


def lib():
    """The loaded libmoe (ctypes).  torch is imported first so that the library binds to the
    HIP runtime torch already loaded (one runtime per process, shared streams)."""
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            raise MoeError(f"{_LIB_PATH} is not built; run `python -m "
                           "mixture_experts_routed_router_amd.build` (hipcc, gfx950)")
        handle = ctypes.CDLL(_LIB_PATH)
        for name, (res, args) in _SIGNATURES.items():
            fn = getattr(handle, name)
            fn.restype = res
            fn.argtypes = args
        _lib = handle
    return _lib


def _check(status: int, call: str):
    if status != 0:
        raise MoeError(f"{call}: {_STATUS.get(status, status)}")


def _ptr(t, dtype=None, name="tensor"):
    if t is None:
        return None
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise MoeError(f"{name} must be a CUDA tensor")
    if not t.is_contiguous():
        raise MoeError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise MoeError(f"{name} must be {dtype}, got {t.dtype}")
    return t.data_ptr()


def _dt(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return MOE_BF16
    if t.dtype == torch.float32:
        return MOE_F32
    raise MoeError(f"unsupported dtype {t.dtype}")


def _stream(stream=None):
    s = stream if stream is not None else torch.cuda.current_stream()
    return s.cuda_stream


# ----------------------------------------------------------------------- bounds ---

def moe_max_rows(T: int, K: int, E_loc: int, block_m: int) -> int:
    return int(lib().moe_max_rows(T, K, E_loc, block_m))


def moe_max_blocks(T: int, K: int, E_loc: int, P: int, block_m: int) -> int:
    return int(lib().moe_max_blocks(T, K, E_loc, P, block_m))


def moe_max_moves(E_loc: int, P: int) -> int:
    return int(lib().moe_max_moves(E_loc, P))


def moe_permute_workspace_elems(T: int, E_loc: int) -> int:
    return int(lib().moe_permute_workspace_elems(T, E_loc))


def moe_ffn_workspace_elems(max_blocks: int) -> int:
    return int(lib().moe_ffn_workspace_elems(max_blocks))


# ------------------------------------------------------------------------ calls ---

def moe_route(logits, K, topk_ids, topk_w, expert_counts, renormalize=True, stream=None):
    T, E = logits.shape
    _check(lib().moe_route(_ptr(logits, torch.float32, "logits"), T, E, K, int(bool(renormalize)),
                           _ptr(topk_ids, torch.int32, "topk_ids"),
                           _ptr(topk_w, torch.float32, "topk_w"),
                           _ptr(expert_counts, torch.int32, "expert_counts"), _stream(stream)),
           "moe_route")


def moe_route_ref(logits, K, k_ref, topk_ids, topk_w, expert_counts, stream=None):
    T, E = logits.shape
    _check(lib().moe_route_ref(_ptr(logits, torch.float32, "logits"), T, E, K, k_ref,
                               _ptr(topk_ids, torch.int32, "topk_ids"),
                               _ptr(topk_w, torch.float32, "topk_w"),
                               _ptr(expert_counts, torch.int32, "expert_counts"),
                               _stream(stream)),
           "moe_route_ref")


def moe_router_topk(x, w_router, K, k_ref, topk_ids, topk_w, expert_counts, logits=None,
                    stream=None):
    """Router scores x . w_router^T (float32 accumulation) and the top-k on them; logits
    ([T, E] float32) receives the scores when given."""
    T, H = x.shape
    E = w_router.shape[0]
    if w_router.shape[1] != H:
        raise MoeError("moe_router_topk: w_router must be [E, H]")
    _check(lib().moe_router_topk(_ptr(x, None, "x"), _dt(x), _ptr(w_router, x.dtype, "w_router"),
                                 T, H, E, K, k_ref, _ptr(logits, torch.float32, "logits"),
                                 _ptr(topk_ids, torch.int32, "topk_ids"),
                                 _ptr(topk_w, torch.float32, "topk_w"),
                                 _ptr(expert_counts, torch.int32, "expert_counts"),
                                 _stream(stream)),
           "moe_router_topk")


def moe_permute(x, topk_ids, expert_counts, E, expert_begin, expert_stride, E_loc, block_m,
                expert_offsets, entry_pos, row_token, xp, workspace, stream=None):
    """xp may be None: indices only (for moe_expert_ffn_gather)."""
    T, H = x.shape
    K = topk_ids.shape[1]
    if xp is not None and xp.shape[0] != row_token.shape[0]:
        raise MoeError("moe_permute: xp and row_token must have max_rows rows")
    _check(lib().moe_permute(_ptr(x, None, "x"), _dt(x), T, H, K, E,
                             _ptr(topk_ids, torch.int32, "topk_ids"),
                             _ptr(expert_counts, torch.int32, "expert_counts"),
                             expert_begin, expert_stride, E_loc, block_m,
                             _ptr(expert_offsets, torch.int32, "expert_offsets"),
                             _ptr(entry_pos, torch.int32, "entry_pos"),
                             _ptr(row_token, torch.int32, "row_token"),
                             _ptr(xp, x.dtype, "xp"), row_token.shape[0],
                             _ptr(workspace, torch.int32, "workspace"), workspace.numel(),
                             _stream(stream)),
           "moe_permute")


def moe_plan(expert_counts, E, expert_begin, expert_stride, E_loc, P, block_m, q, moves,
             n_moves, blocks, n_blocks, err_word=None, stream=None):
    _check(lib().moe_plan(_ptr(expert_counts, torch.int32, "expert_counts"), E, expert_begin,
                          expert_stride, E_loc, P, block_m, _ptr(q, torch.int32, "q"),
                          _ptr(moves, torch.int32, "moves"), _ptr(n_moves, torch.int32, "n_moves"),
                          moves.shape[0], _ptr(blocks, torch.int32, "blocks"),
                          _ptr(n_blocks, torch.int32, "n_blocks"), blocks.shape[0],
                          _ptr(err_word, torch.int32, "err_word"), _stream(stream)),
           "moe_plan")


def moe_plan_blocks(expert_counts, E, expert_begin, expert_stride, E_loc, P, block_m,
                    replica_budget, q, moves, n_moves, blocks, n_blocks, err_word=None,
                    stream=None):
    _check(lib().moe_plan_blocks(_ptr(expert_counts, torch.int32, "expert_counts"), E,
                                 expert_begin, expert_stride, E_loc, P, block_m, replica_budget,
                                 _ptr(q, torch.int32, "q"), _ptr(moves, torch.int32, "moves"),
                                 _ptr(n_moves, torch.int32, "n_moves"), moves.shape[0],
                                 _ptr(blocks, torch.int32, "blocks"),
                                 _ptr(n_blocks, torch.int32, "n_blocks"), blocks.shape[0],
                                 _ptr(err_word, torch.int32, "err_word"), _stream(stream)),
           "moe_plan_blocks")


def moe_expert_ffn(xp, w1, w2, blocks, n_blocks, act, yp, workspace, stream=None):
    E_loc, two_I, H = w1.shape
    I = two_I // 2
    if xp.shape[1] != H or w2.shape != (E_loc, H, I) or act.shape[1] != I or yp.shape[1] != H:
        raise MoeError("moe_expert_ffn: inconsistent shapes")
    if act.shape[0] < xp.shape[0] or yp.shape[0] < xp.shape[0]:
        raise MoeError("moe_expert_ffn: act/yp have fewer rows than xp")
    dt = _dt(xp)
    _check(lib().moe_expert_ffn(_ptr(xp, xp.dtype, "xp"), _ptr(w1, xp.dtype, "w1"),
                                _ptr(w2, xp.dtype, "w2"), dt, H, I, E_loc,
                                _ptr(blocks, torch.int32, "blocks"),
                                _ptr(n_blocks, torch.int32, "n_blocks"), blocks.shape[0],
                                _ptr(act, xp.dtype, "act"), _ptr(yp, xp.dtype, "yp"),
                                xp.shape[0], _ptr(workspace, torch.int32, "workspace"),
                                workspace.numel(), _stream(stream)),
           "moe_expert_ffn")


def moe_expert_ffn_tile_schedule(blocks, n_blocks, E_loc, max_rows, workspace, stream=None):
    """The GEMM tile schedule (and the table check) that the FC1 calls compute first (for
    timing it alone)."""
    _check(lib().moe_expert_ffn_tile_schedule(_ptr(blocks, torch.int32, "blocks"),
                                              _ptr(n_blocks, torch.int32, "n_blocks"),
                                              blocks.shape[0], E_loc, int(max_rows),
                                              _ptr(workspace, torch.int32, "workspace"),
                                              workspace.numel(), _stream(stream)),
           "moe_expert_ffn_tile_schedule")


# workspace word holding the FFN's table error bits (MOE_FFN_WS_ERR and MOE_FFN_ERR_* in moe.h)
FFN_WS_ERR = 1
FFN_ERR_EXPERT, FFN_ERR_ROWS, FFN_ERR_RANGE, FFN_ERR_COUNT = 1, 2, 4, 8


# largest block table moe_expert_ffn_gather_noalloc takes (MOE_FFN_NOALLOC_MAX_BLOCKS in moe.h)
FFN_NOALLOC_MAX_BLOCKS = 16384


def moe_expert_ffn_gather_noalloc(x, row_token, w1, w2, blocks, n_blocks, act, yp, stream=None):
    """moe_expert_ffn_gather with the library's static per-GPU scratch instead of a workspace
    (allocates nothing; calls that overlap on one GPU race)."""
    T, H = x.shape
    E_loc, two_I, _ = w1.shape
    I = two_I // 2
    rows = row_token.shape[0]
    if w1.shape[2] != H or w2.shape != (E_loc, H, I) or act.shape[1] != I or yp.shape[1] != H:
        raise MoeError("moe_expert_ffn_gather_noalloc: inconsistent shapes")
    if act.shape[0] < rows or yp.shape[0] < rows:
        raise MoeError("moe_expert_ffn_gather_noalloc: act/yp have fewer rows than row_token")
    _check(lib().moe_expert_ffn_gather_noalloc(_ptr(x, x.dtype, "x"),
                                               _ptr(row_token, torch.int32, "row_token"), T,
                                               _ptr(w1, x.dtype, "w1"), _ptr(w2, x.dtype, "w2"),
                                               _dt(x), H, I, E_loc,
                                               _ptr(blocks, torch.int32, "blocks"),
                                               _ptr(n_blocks, torch.int32, "n_blocks"),
                                               blocks.shape[0], _ptr(act, x.dtype, "act"),
                                               _ptr(yp, x.dtype, "yp"), rows, _stream(stream)),
           "moe_expert_ffn_gather_noalloc")


def moe_expert_ffn_gather(x, row_token, w1, w2, blocks, n_blocks, act, yp, workspace,
                          stream=None):
    """moe_expert_ffn on rows gathered from x by row_token (no permuted copy of x)."""
    T, H = x.shape
    E_loc, two_I, _ = w1.shape
    I = two_I // 2
    rows = row_token.shape[0]
    if w1.shape[2] != H or w2.shape != (E_loc, H, I) or act.shape[1] != I or yp.shape[1] != H:
        raise MoeError("moe_expert_ffn_gather: inconsistent shapes")
    if act.shape[0] < rows or yp.shape[0] < rows:
        raise MoeError("moe_expert_ffn_gather: act/yp have fewer rows than row_token")
    _check(lib().moe_expert_ffn_gather(_ptr(x, x.dtype, "x"),
                                       _ptr(row_token, torch.int32, "row_token"), T,
                                       _ptr(w1, x.dtype, "w1"), _ptr(w2, x.dtype, "w2"), _dt(x),
                                       H, I, E_loc, _ptr(blocks, torch.int32, "blocks"),
                                       _ptr(n_blocks, torch.int32, "n_blocks"), blocks.shape[0],
                                       _ptr(act, x.dtype, "act"), _ptr(yp, x.dtype, "yp"), rows,
                                       _ptr(workspace, torch.int32, "workspace"),
                                       workspace.numel(), _stream(stream)),
           "moe_expert_ffn_gather")


def moe_expert_ffn_fc1_gather(x, row_token, w1, blocks, n_blocks, act, workspace, stream=None):
    T, H = x.shape
    E_loc, two_I, _ = w1.shape
    I = two_I // 2
    rows = row_token.shape[0]
    if w1.shape[2] != H or act.shape[1] != I or act.shape[0] < rows:
        raise MoeError("moe_expert_ffn_fc1_gather: inconsistent shapes")
    _check(lib().moe_expert_ffn_fc1_gather(_ptr(x, x.dtype, "x"),
                                           _ptr(row_token, torch.int32, "row_token"), T,
                                           _ptr(w1, x.dtype, "w1"), _dt(x), H, I, E_loc,
                                           _ptr(blocks, torch.int32, "blocks"),
                                           _ptr(n_blocks, torch.int32, "n_blocks"),
                                           blocks.shape[0], _ptr(act, x.dtype, "act"), rows,
                                           _ptr(workspace, torch.int32, "workspace"),
                                           workspace.numel(), _stream(stream)),
           "moe_expert_ffn_fc1_gather")


def moe_expert_ffn_fc1(xp, w1, blocks, n_blocks, act, workspace, stream=None):
    E_loc, two_I, H = w1.shape
    I = two_I // 2
    if xp.shape[1] != H or act.shape[1] != I or act.shape[0] < xp.shape[0]:
        raise MoeError("moe_expert_ffn_fc1: inconsistent shapes")
    _check(lib().moe_expert_ffn_fc1(_ptr(xp, xp.dtype, "xp"), _ptr(w1, xp.dtype, "w1"), _dt(xp),
                                    H, I, E_loc, _ptr(blocks, torch.int32, "blocks"),
                                    _ptr(n_blocks, torch.int32, "n_blocks"), blocks.shape[0],
                                    _ptr(act, xp.dtype, "act"), xp.shape[0],
                                    _ptr(workspace, torch.int32, "workspace"), workspace.numel(),
                                    _stream(stream)),
           "moe_expert_ffn_fc1")


def moe_expert_ffn_fc2(act, w2, blocks, n_blocks, yp, workspace, stream=None):
    E_loc, H, I = w2.shape
    if act.shape[1] != I or yp.shape[1] != H or yp.shape[0] < act.shape[0]:
        raise MoeError("moe_expert_ffn_fc2: inconsistent shapes")
    _check(lib().moe_expert_ffn_fc2(_ptr(act, act.dtype, "act"), _ptr(w2, act.dtype, "w2"),
                                    _dt(act), H, I, E_loc, _ptr(blocks, torch.int32, "blocks"),
                                    _ptr(n_blocks, torch.int32, "n_blocks"), blocks.shape[0],
                                    _ptr(yp, act.dtype, "yp"), act.shape[0],
                                    _ptr(workspace, torch.int32, "workspace"), workspace.numel(),
                                    _stream(stream)),
           "moe_expert_ffn_fc2")


def moe_expert_ffn_fc2_direct(act, w2, blocks, n_blocks, yp, row_token, entry_pos, topk_w, out,
                              row_direct, workspace, stream=None):
    E_loc, H, I = w2.shape
    T, K = topk_w.shape
    if act.shape[1] != I or yp.shape[1] != H or yp.shape[0] < act.shape[0]:
        raise MoeError("moe_expert_ffn_fc2_direct: inconsistent shapes")
    if out.shape != (T, H) or entry_pos.numel() != T * K or row_token.numel() < act.shape[0]:
        raise MoeError("moe_expert_ffn_fc2_direct: inconsistent shapes")
    if row_direct.numel() < 2 * act.shape[0]:
        raise MoeError("moe_expert_ffn_fc2_direct: row_direct needs 2 * max_rows entries")
    _check(lib().moe_expert_ffn_fc2_direct(
        _ptr(act, act.dtype, "act"), _ptr(w2, act.dtype, "w2"), _dt(act), H, I, E_loc,
        _ptr(blocks, torch.int32, "blocks"), _ptr(n_blocks, torch.int32, "n_blocks"),
        blocks.shape[0], _ptr(yp, act.dtype, "yp"), act.shape[0],
        _ptr(row_token, torch.int32, "row_token"), _ptr(entry_pos, torch.int32, "entry_pos"),
        _ptr(topk_w, torch.float32, "topk_w"), T, K, _ptr(out, act.dtype, "out"),
        _ptr(row_direct, torch.int32, "row_direct"), _ptr(workspace, torch.int32, "workspace"),
        workspace.numel(), _stream(stream)),
        "moe_expert_ffn_fc2_direct")


MOE_MX_FP8, MOE_MX_FP4 = 0, 1


def moe_mx_scale_pitch(cols: int) -> int:
    """Bytes per row of an MX scale array for rows of `cols` values (cols/32 rounded up to 4)."""
    return int(lib().moe_mx_scale_pitch(cols))


def moe_mx_quantize(src, fmt, codes, scales, stream=None):
    """src [..., rows, cols] float32/bf16 -> codes uint8 [..., cols] (FP8) or [..., cols/2] (FP4),
    scales uint8 [..., moe_mx_scale_pitch(cols)] (E8M0); leading dimensions are flattened."""
    cols = src.shape[-1]
    rows = src.numel() // cols if cols else 0
    want = cols if fmt == MOE_MX_FP8 else cols // 2
    pitch = moe_mx_scale_pitch(cols)
    if (codes.shape[:-1] != src.shape[:-1] or codes.shape[-1] != want
            or scales.shape[:-1] != src.shape[:-1] or scales.shape[-1] != pitch):
        raise MoeError("moe_mx_quantize: codes / scales shapes do not match src")
    _check(lib().moe_mx_quantize(_ptr(src, None, "src"), _dt(src), rows, cols, fmt,
                                 _ptr(codes, torch.uint8, "codes"),
                                 _ptr(scales, torch.uint8, "scales"), _stream(stream)),
           "moe_mx_quantize")


def _mx_ffn_shapes(call, w1q, w2q, actq, yp):
    E_loc, two_I, H2 = w1q.shape
    I, H = two_I // 2, 2 * H2
    if w2q.shape != (E_loc, H, I // 2):
        raise MoeError(f"{call}: w2q must be [E_loc, H, I/2] = {(E_loc, H, I // 2)}")
    if actq is not None and actq.shape[1] != I:
        raise MoeError(f"{call}: actq must have I = {I} columns")
    if yp is not None and (yp.shape[1] != H or yp.dtype != torch.bfloat16):
        raise MoeError(f"{call}: yp must be bf16 with H = {H} columns")
    return E_loc, H, I


def _mx_scales(call, s, lead, cols, name):
    want = tuple(lead) + (moe_mx_scale_pitch(cols),)
    if tuple(s.shape) != want:
        raise MoeError(f"{call}: {name} must be {want}, got {tuple(s.shape)}")
    return _ptr(s, torch.uint8, name)


def moe_expert_ffn_mx_fc1(xq, xs, row_token, w1q, w1s, blocks, n_blocks, actq, acts, workspace,
                          stream=None):
    """FC1 with MXFP8 input rows (xq/xs; gathered by row_token when given) and MXFP4 W1; the
    activation leaves in MXFP8 (actq/acts)."""
    call = "moe_expert_ffn_mx_fc1"
    E_loc, two_I, H2 = w1q.shape
    I, H = two_I // 2, 2 * H2
    rows = actq.shape[0]
    if xq.shape[1] != H or actq.shape[1] != I:
        raise MoeError(f"{call}: inconsistent shapes")
    if row_token is not None and row_token.shape[0] > rows:
        raise MoeError(f"{call}: actq has fewer rows than row_token")
    _check(lib().moe_expert_ffn_mx_fc1(
        _ptr(xq, torch.uint8, "xq"), _mx_scales(call, xs, xq.shape[:1], H, "xs"),
        _ptr(row_token, torch.int32, "row_token"), xq.shape[0], _ptr(w1q, torch.uint8, "w1q"),
        _mx_scales(call, w1s, w1q.shape[:2], H, "w1s"), H, I, E_loc,
        _ptr(blocks, torch.int32, "blocks"), _ptr(n_blocks, torch.int32, "n_blocks"),
        blocks.shape[0], _ptr(actq, torch.uint8, "actq"),
        _mx_scales(call, acts, actq.shape[:1], I, "acts"), rows,
        _ptr(workspace, torch.int32, "workspace"), workspace.numel(), _stream(stream)), call)


def moe_expert_ffn_mx_fc2(actq, acts, w2q, w2s, blocks, n_blocks, yp, workspace, stream=None):
    call = "moe_expert_ffn_mx_fc2"
    E_loc, H, I2 = w2q.shape
    I = 2 * I2
    rows = actq.shape[0]
    if actq.shape[1] != I or yp.shape != (rows, H) or yp.dtype != torch.bfloat16:
        raise MoeError(f"{call}: inconsistent shapes")
    _check(lib().moe_expert_ffn_mx_fc2(
        _ptr(actq, torch.uint8, "actq"), _mx_scales(call, acts, actq.shape[:1], I, "acts"),
        _ptr(w2q, torch.uint8, "w2q"), _mx_scales(call, w2s, w2q.shape[:2], I, "w2s"), H, I,
        E_loc, _ptr(blocks, torch.int32, "blocks"), _ptr(n_blocks, torch.int32, "n_blocks"),
        blocks.shape[0], _ptr(yp, torch.bfloat16, "yp"), rows,
        _ptr(workspace, torch.int32, "workspace"), workspace.numel(), _stream(stream)), call)


def moe_expert_ffn_mx_fc2_direct(actq, acts, w2q, w2s, blocks, n_blocks, yp, row_token, entry_pos,
                                 topk_w, out, row_direct, workspace, stream=None):
    call = "moe_expert_ffn_mx_fc2_direct"
    E_loc, H, I2 = w2q.shape
    I = 2 * I2
    rows = actq.shape[0]
    T, K = topk_w.shape
    if actq.shape[1] != I or yp.shape != (rows, H) or yp.dtype != torch.bfloat16:
        raise MoeError(f"{call}: inconsistent shapes")
    if out.shape != (T, H) or entry_pos.numel() != T * K or row_token.numel() < rows:
        raise MoeError(f"{call}: inconsistent shapes")
    if row_direct.numel() < 2 * rows:
        raise MoeError(f"{call}: row_direct needs 2 * max_rows entries")
    _check(lib().moe_expert_ffn_mx_fc2_direct(
        _ptr(actq, torch.uint8, "actq"), _mx_scales(call, acts, actq.shape[:1], I, "acts"),
        _ptr(w2q, torch.uint8, "w2q"), _mx_scales(call, w2s, w2q.shape[:2], I, "w2s"), H, I,
        E_loc, _ptr(blocks, torch.int32, "blocks"), _ptr(n_blocks, torch.int32, "n_blocks"),
        blocks.shape[0], _ptr(yp, torch.bfloat16, "yp"), rows,
        _ptr(row_token, torch.int32, "row_token"), _ptr(entry_pos, torch.int32, "entry_pos"),
        _ptr(topk_w, torch.float32, "topk_w"), T, K, _ptr(out, torch.bfloat16, "out"),
        _ptr(row_direct, torch.int32, "row_direct"), _ptr(workspace, torch.int32, "workspace"),
        workspace.numel(), _stream(stream)), call)


def moe_expert_ffn_mx(xq, xs, row_token, w1q, w1s, w2q, w2s, blocks, n_blocks, actq, acts, yp,
                      workspace, stream=None):
    """The SwiGLU expert FFN with MXFP4 weights and MXFP8 activations (FC1 then FC2)."""
    call = "moe_expert_ffn_mx"
    E_loc, H, I = _mx_ffn_shapes(call, w1q, w2q, actq, yp)
    rows = actq.shape[0]
    if xq.shape[1] != H or yp.shape[0] != rows:
        raise MoeError(f"{call}: inconsistent shapes")
    if row_token is not None and row_token.shape[0] > rows:
        raise MoeError(f"{call}: actq has fewer rows than row_token")
    _check(lib().moe_expert_ffn_mx(
        _ptr(xq, torch.uint8, "xq"), _mx_scales(call, xs, xq.shape[:1], H, "xs"),
        _ptr(row_token, torch.int32, "row_token"), xq.shape[0], _ptr(w1q, torch.uint8, "w1q"),
        _mx_scales(call, w1s, w1q.shape[:2], H, "w1s"), _ptr(w2q, torch.uint8, "w2q"),
        _mx_scales(call, w2s, w2q.shape[:2], I, "w2s"), H, I, E_loc,
        _ptr(blocks, torch.int32, "blocks"), _ptr(n_blocks, torch.int32, "n_blocks"),
        blocks.shape[0], _ptr(actq, torch.uint8, "actq"),
        _mx_scales(call, acts, actq.shape[:1], I, "acts"), _ptr(yp, torch.bfloat16, "yp"), rows,
        _ptr(workspace, torch.int32, "workspace"), workspace.numel(), _stream(stream)), call)


def mx_quantize_weights(W1, W2, stream=None):
    """Expert weights W1 [E_loc, 2I, H] and W2 [E_loc, H, I] (bf16 or float32, on the GPU) in
    MXFP4: ((w1q, w1s), (w2q, w2s)), the weight arguments of the MX path."""
    out = []
    for W in (W1, W2):
        cols = W.shape[-1]
        q = torch.empty(*W.shape[:-1], cols // 2, dtype=torch.uint8, device=W.device)
        sc = torch.empty(*W.shape[:-1], moe_mx_scale_pitch(cols), dtype=torch.uint8,
                         device=W.device)
        moe_mx_quantize(W, MOE_MX_FP4, q, sc, stream)
        out.append((q, sc))
    return tuple(out)


def moe_combine(yp, topk_w, entry_pos, out, stream=None):
    T, K = topk_w.shape
    H = yp.shape[1]
    if out.shape != (T, H) or entry_pos.numel() != T * K:
        raise MoeError("moe_combine: inconsistent shapes")
    _check(lib().moe_combine(_ptr(yp, None, "yp"), _dt(yp), _ptr(topk_w, torch.float32, "topk_w"),
                             _ptr(entry_pos, torch.int32, "entry_pos"), T, H, K,
                             _ptr(out, yp.dtype, "out"), _stream(stream)),
           "moe_combine")


def moe_combine_multi(yp, topk_w, entry_pos, out, stream=None):
    T, K = topk_w.shape
    H = yp.shape[1]
    if out.shape != (T, H) or entry_pos.numel() != T * K:
        raise MoeError("moe_combine_multi: inconsistent shapes")
    _check(lib().moe_combine_multi(_ptr(yp, None, "yp"), _dt(yp),
                                   _ptr(topk_w, torch.float32, "topk_w"),
                                   _ptr(entry_pos, torch.int32, "entry_pos"), T, H, K,
                                   _ptr(out, yp.dtype, "out"), _stream(stream)),
           "moe_combine_multi")


# ------------------------------------------------------------- whole layer path ---

class RoutedExperts:
    """Static buffers for one layer shape and the five calls in order.

    Buffers are sized once from the library's static bounds (T, K, E_loc, P, block_m), so a
    forward pass allocates nothing.  Weights are device tensors W1 [E_loc, 2I, H],
    W2 [E_loc, H, I] in the activation dtype; with precision="mx", the MXFP4 pairs that
    mx_quantize_weights returns (x is then quantized to MXFP8 inside the step).
    """

    def __init__(self, T, H, E, K, I, P, dtype=torch.bfloat16, E_loc=None, expert_begin=0,
                 expert_stride=1, block_m=128, renormalize=True, device="cuda", gather=False,
                 planner="moonep", replica_budget=None, precision="bf16", direct=False):
        self.T, self.H, self.E, self.K, self.I, self.P = T, H, E, K, I, P
        if precision not in ("bf16", "mx"):
            raise MoeError(f"unknown precision {precision!r} (bf16 or mx)")
        # mx: x is quantized to MXFP8 per token row, the expert GEMMs run on MXFP4 weights
        # (mx_quantize_weights) and gather their input rows; act is MXFP8, yp / out bf16
        self.precision = precision
        if precision == "mx":
            if dtype != torch.bfloat16:
                raise MoeError("the MX path takes bf16 activations")
            gather = True
        if planner not in ("moonep", "megaflux"):
            raise MoeError(f"unknown planner {planner!r} (moonep or megaflux)")
        # moonep: moe_plan (exact per-rank entry capacity); megaflux: moe_plan_blocks
        # (block-granular replicas under a per-rank budget, E_loc / (4 P) by default)
        self.planner = planner
        self.replica_budget = (replica_budget if replica_budget is not None
                               else (E_loc or E) // (4 * P))
        self.gather = gather  # FC1 reads x rows through row_token; xp is never written
        # direct: FC2 writes the weighted out rows of one-entry tokens and the combine skips
        # them (moe_expert_ffn_fc2_direct / moe_expert_ffn_mx_fc2_direct + moe_combine_multi)
        self.direct = direct
        self.E_loc = E_loc or E
        self.begin, self.stride, self.block_m = expert_begin, expert_stride, block_m
        self.renormalize = renormalize
        self.dtype = dtype
        i32 = dict(dtype=torch.int32, device=device)
        self.max_rows = moe_max_rows(T, K, self.E_loc, block_m)
        self.max_blocks = moe_max_blocks(T, K, self.E_loc, P, block_m)
        self.max_moves = moe_max_moves(self.E_loc, P)
        if min(self.max_rows, self.max_blocks, self.max_moves) < 0:
            raise MoeError("invalid layer shape")
        self.topk_ids = torch.empty((T, K), **i32)
        self.topk_w = torch.empty((T, K), dtype=torch.float32, device=device)
        self.counts = torch.empty((E,), **i32)
        self.offsets = torch.empty((self.E_loc + 1,), **i32)
        self.entry_pos = torch.empty((T * K,), **i32)
        self.row_token = torch.empty((self.max_rows,), **i32)
        self.workspace = torch.empty((moe_permute_workspace_elems(T, self.E_loc),), **i32)
        self.xp = None if gather else torch.empty((self.max_rows, H), dtype=dtype, device=device)
        self.q = torch.empty((self.E_loc, P), **i32)
        self.moves = torch.empty((self.max_moves, 4), **i32)
        self.n_moves = torch.empty((1,), **i32)
        self.blocks = torch.empty((self.max_blocks, 4), **i32)
        self.n_blocks = torch.empty((1,), **i32)
        self.err_word = torch.empty((1,), **i32)
        self.ffn_workspace = torch.empty((moe_ffn_workspace_elems(self.max_blocks),), **i32)
        u8 = dict(dtype=torch.uint8, device=device)
        if precision == "mx":
            self.act = None
            self.xq = torch.empty((T, H), **u8)
            self.xs = torch.empty((T, moe_mx_scale_pitch(H)), **u8)
            self.actq = torch.empty((self.max_rows, I), **u8)
            self.acts = torch.empty((self.max_rows, moe_mx_scale_pitch(I)), **u8)
        else:
            self.act = torch.empty((self.max_rows, I), dtype=dtype, device=device)
        self.yp = torch.empty((self.max_rows, H), dtype=dtype, device=device)
        self.out = torch.empty((T, H), dtype=dtype, device=device)
        self.row_direct = torch.empty((2 * self.max_rows,), **i32) if direct else None

    def route(self, logits, stream=None):
        moe_route(logits, self.K, self.topk_ids, self.topk_w, self.counts, self.renormalize, stream)

    def permute(self, x, stream=None):
        self._x = x
        moe_permute(x, self.topk_ids, self.counts, self.E, self.begin, self.stride, self.E_loc,
                    self.block_m, self.offsets, self.entry_pos, self.row_token, self.xp,
                    self.workspace, stream)

    def plan(self, stream=None):
        if self.planner == "megaflux":
            moe_plan_blocks(self.counts, self.E, self.begin, self.stride, self.E_loc, self.P,
                            self.block_m, self.replica_budget, self.q, self.moves, self.n_moves,
                            self.blocks, self.n_blocks, self.err_word, stream)
            return
        moe_plan(self.counts, self.E, self.begin, self.stride, self.E_loc, self.P, self.block_m,
                 self.q, self.moves, self.n_moves, self.blocks, self.n_blocks, self.err_word,
                 stream)

    def quantize_x(self, x, stream=None):
        """MX path: x [T, H] bf16 -> MXFP8 codes and scales (per token row)."""
        moe_mx_quantize(x, MOE_MX_FP8, self.xq, self.xs, stream)

    def expert_ffn(self, w1, w2, stream=None):
        if self.precision == "mx" and self.direct:
            self.expert_ffn_fc1(w1, stream)
            self.expert_ffn_fc2(w2, stream)
            return
        if self.precision == "mx":
            (w1q, w1s), (w2q, w2s) = w1, w2
            moe_expert_ffn_mx(self.xq, self.xs, self.row_token, w1q, w1s, w2q, w2s, self.blocks,
                              self.n_blocks, self.actq, self.acts, self.yp, self.ffn_workspace,
                              stream)
            return
        if self.direct:
            self.expert_ffn_fc1(w1, stream)
            self.expert_ffn_fc2(w2, stream)
            return
        if self.gather:
            moe_expert_ffn_gather(self._x, self.row_token, w1, w2, self.blocks, self.n_blocks,
                                  self.act, self.yp, self.ffn_workspace, stream)
        else:
            moe_expert_ffn(self.xp, w1, w2, self.blocks, self.n_blocks, self.act, self.yp,
                           self.ffn_workspace, stream)

    def expert_ffn_fc1(self, w1, stream=None):
        if self.precision == "mx":
            moe_expert_ffn_mx_fc1(self.xq, self.xs, self.row_token, w1[0], w1[1], self.blocks,
                                  self.n_blocks, self.actq, self.acts, self.ffn_workspace, stream)
            return
        if self.gather:
            moe_expert_ffn_fc1_gather(self._x, self.row_token, w1, self.blocks, self.n_blocks,
                                      self.act, self.ffn_workspace, stream)
        else:
            moe_expert_ffn_fc1(self.xp, w1, self.blocks, self.n_blocks, self.act,
                               self.ffn_workspace, stream)

    def expert_ffn_fc2(self, w2, stream=None):
        if self.precision == "mx" and self.direct:
            moe_expert_ffn_mx_fc2_direct(self.actq, self.acts, w2[0], w2[1], self.blocks,
                                         self.n_blocks, self.yp, self.row_token, self.entry_pos,
                                         self.topk_w, self.out, self.row_direct,
                                         self.ffn_workspace, stream)
            return
        if self.precision == "mx":
            moe_expert_ffn_mx_fc2(self.actq, self.acts, w2[0], w2[1], self.blocks, self.n_blocks,
                                  self.yp, self.ffn_workspace, stream)
            return
        if self.direct:
            moe_expert_ffn_fc2_direct(self.act, w2, self.blocks, self.n_blocks, self.yp,
                                      self.row_token, self.entry_pos, self.topk_w, self.out,
                                      self.row_direct, self.ffn_workspace, stream)
            return
        moe_expert_ffn_fc2(self.act, w2, self.blocks, self.n_blocks, self.yp, self.ffn_workspace,
                           stream)

    def tile_schedule(self, stream=None):
        moe_expert_ffn_tile_schedule(self.blocks, self.n_blocks, self.E_loc, self.max_rows,
                                     self.ffn_workspace, stream)

    def ffn_error(self) -> int:
        """The last FC1 call's table error bits (FFN_ERR_*; 0 for a plan's own table).
        Synchronises the current stream."""
        return int(self.ffn_workspace[FFN_WS_ERR].item())

    def combine(self, stream=None):
        if self.direct:
            moe_combine_multi(self.yp, self.topk_w, self.entry_pos, self.out, stream)
            return
        moe_combine(self.yp, self.topk_w, self.entry_pos, self.out, stream)

    def forward(self, logits, x, w1, w2, stream=None):
        """route -> permute -> plan -> expert FFN -> combine; returns the static `out`."""
        self.route(logits, stream)
        self.permute(x, stream)
        if self.precision == "mx":
            self.quantize_x(x, stream)
        self.plan(stream)
        self.expert_ffn(w1, w2, stream)
        self.combine(stream)
        return self.out

    def capture(self, logits, x, w1, w2):
        """Record forward() on these tensors into a HIP graph (torch.cuda.CUDAGraph).

        Each replay reruns the whole path on whatever logits / x / w1 / w2 hold at that time
        and leaves the results in the static buffers.  The path launches kernels only (its
        counters are cleared by kernels, not memsets), and every kernel reads its data-dependent
        sizes on the device, so one graph serves every batch of this shape.  One eager forward
        runs first, outside the capture."""
        self.forward(logits, x, w1, w2)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            self.forward(logits, x, w1, w2)
        return graph
