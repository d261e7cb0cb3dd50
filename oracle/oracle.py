"""Python wrapper over ``oracle.c``, the plain CPU reference of the routed-expert path.

TEST INFRASTRUCTURE ONLY: imported by ``tests/``, by ``__graft_entry__.smoke()`` and by the
CPU-baseline leg of ``bench.py``; never by the product package.  It shares no code with the
HIP library.  Arrays are numpy; bf16 data travels as ``np.uint16`` bit patterns.

Every function is the plain definition of its step (see the citations in ``oracle.c``):
route  -- top-k by (larger logit, smaller id), softmax weights renormalised over the picks
          (route_ref: normalised by the mass of the top k_ref experts);
router_logits -- linear router scores x . w_r^T in double, rounded to float32;
permute -- stable expert-major order by flat index, beta-aligned segments;
plan   -- the greedy donor->receiver balance to exact per-rank capacity, then <=beta blocks;
plan_blocks -- the block-granular replica planner: four greedy searches, the best, refined;
ffn    -- SwiGLU expert FFN in double with bf16 rounding at act and yp;
combine -- routing-weight sum in double, k ascending;
mx_*   -- OCP MX formats (MXFP8 E4M3 / MXFP4 E2M1, one E8M0 scale per 32 values) and the FFN in them.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None

_i32p = ctypes.POINTER(ctypes.c_int32)
_f32p = ctypes.POINTER(ctypes.c_float)


def build(force: bool = False) -> str:
    """Compile oracle.c into liboracle.so next to it (gcc, OpenMP, no fast-math)."""
    if force or not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
        tmp = _LIB_PATH + ".tmp"
        subprocess.check_call(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c11",
                               "-Wall", "-Wno-unused-function", _SRC, "-o", tmp, "-lm"])
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is None:
        build()
        lib = ctypes.CDLL(_LIB_PATH)
        lib.oracle_double_to_bf16.restype = ctypes.c_uint16
        lib.oracle_double_to_bf16.argtypes = [ctypes.c_double]
        lib.oracle_num_threads.restype = ctypes.c_int
        lib.oracle_set_num_threads.restype = ctypes.c_int
        lib.oracle_set_num_threads.argtypes = [ctypes.c_int]
        for name in ("oracle_route", "oracle_route_ref", "oracle_router_logits", "oracle_permute",
                     "oracle_plan", "oracle_plan_blocks", "oracle_ffn_rows", "oracle_ffn_blocks",
                     "oracle_combine", "oracle_mx_quantize", "oracle_mx_dequantize",
                     "oracle_ffn_mx_rows"):
            getattr(lib, name).restype = ctypes.c_int
        _lib = lib
    return _lib


def _p(a: np.ndarray):
    assert a.flags["C_CONTIGUOUS"], "oracle arrays must be C-contiguous"
    return ctypes.c_void_p(a.ctypes.data)


def _check(rc: int, what: str):
    if rc != 0:
        raise RuntimeError(f"oracle {what} failed with code {rc}")


def num_threads() -> int:
    return int(_load().oracle_num_threads())


def set_num_threads(n: int) -> int:
    """Threads of the oracle's OpenMP loops from now on; returns the count in effect."""
    return int(_load().oracle_set_num_threads(int(n)))


def double_to_bf16(v: float) -> int:
    return int(_load().oracle_double_to_bf16(float(v)))


def _dt_code(a: np.ndarray) -> int:
    if a.dtype == np.uint16:
        return 1
    if a.dtype == np.float32:
        return 0
    raise TypeError(f"oracle arrays are float32 or bf16 bits (uint16), got {a.dtype}")


def route(logits: np.ndarray, K: int, renormalize: bool = True):
    """-> ids [T,K] int32, w [T,K] float32, counts [E] int32."""
    logits = np.ascontiguousarray(logits, dtype=np.float32)
    T, E = logits.shape
    ids = np.empty((T, K), np.int32)
    w = np.empty((T, K), np.float32)
    counts = np.empty((E,), np.int32)
    _check(_load().oracle_route(_p(logits), T, E, K, int(bool(renormalize)), _p(ids), _p(w),
                                _p(counts)), "route")
    return ids, w, counts


def route_ref(logits: np.ndarray, K: int, k_ref: int):
    """Top-K ids with weights normalised by the mass of the top k_ref experts (K <= k_ref <=
    E).  -> ids [T,K] int32, w [T,K] float32, counts [E] int32."""
    logits = np.ascontiguousarray(logits, dtype=np.float32)
    T, E = logits.shape
    ids = np.empty((T, K), np.int32)
    w = np.empty((T, K), np.float32)
    counts = np.empty((E,), np.int32)
    _check(_load().oracle_route_ref(_p(logits), T, E, K, k_ref, _p(ids), _p(w), _p(counts)),
           "route_ref")
    return ids, w, counts


def router_logits(x: np.ndarray, w_r: np.ndarray) -> np.ndarray:
    """Linear router scores x . w_r^T -> [T, E] float32 (x, w_r: float32, or bf16 bits as
    uint16)."""
    x = np.ascontiguousarray(x)
    w_r = np.ascontiguousarray(w_r)
    dt = _dt_code(x)
    assert _dt_code(w_r) == dt and x.shape[1] == w_r.shape[1]
    T, H = x.shape
    E = w_r.shape[0]
    logits = np.empty((T, E), np.float32)
    _check(_load().oracle_router_logits(_p(x), dt, _p(w_r), T, H, E, _p(logits)), "router_logits")
    return logits


def max_rows(T: int, K: int, E_loc: int, beta: int) -> int:
    """Static bound on the padded row count: local entries plus one partial block each."""
    return min(T * K, T * E_loc) + E_loc * (beta - 1)


def permute(ids: np.ndarray, counts: np.ndarray, E: int, begin: int, stride: int, E_loc: int,
            beta: int, x: np.ndarray | None = None):
    """-> offsets [E_loc+1], entry_pos [T*K], row_token [rows_pad], xp [rows_pad, H] or None."""
    ids = np.ascontiguousarray(ids, dtype=np.int32)
    counts = np.ascontiguousarray(counts, dtype=np.int32)
    T, K = ids.shape
    mr = max_rows(T, K, E_loc, beta)
    offsets = np.empty((E_loc + 1,), np.int32)
    entry_pos = np.empty((T * K,), np.int32)
    row_token = np.empty((mr,), np.int32)
    if x is not None:
        x = np.ascontiguousarray(x)
        assert x.shape[0] == T
        xp = np.zeros((mr,) + x.shape[1:], x.dtype)
        row_bytes = x[0].nbytes
        xptr, xpptr = _p(x), _p(xp)
    else:
        xp, row_bytes, xptr, xpptr = None, 0, None, None
    _check(_load().oracle_permute(_p(ids), _p(counts), T, K, E, begin, stride, E_loc, beta,
                                  xptr, ctypes.c_int64(row_bytes), _p(offsets), _p(entry_pos),
                                  _p(row_token), xpptr, ctypes.c_int64(mr)), "permute")
    rows_pad = int(offsets[-1])
    return offsets, entry_pos, row_token[:rows_pad].copy(), (xp[:rows_pad] if xp is not None else None)


def plan(counts: np.ndarray, E: int, begin: int, stride: int, E_loc: int, P: int, beta: int,
         T: int | None = None, K: int | None = None):
    """-> q [E_loc, P], moves [n_moves, 4] (donor, receiver, expert, rows),
    blocks [n_blocks, 4] (rank, expert, first row, rows)."""
    counts = np.ascontiguousarray(counts, dtype=np.int32)
    N = int(sum(int(counts[begin + l * stride]) for l in range(E_loc)))
    max_moves = E_loc + P
    max_blocks = (N + beta - 1) // beta + E_loc * P
    q = np.empty((E_loc, P), np.int32)
    moves = np.empty((max_moves, 4), np.int32)
    blocks = np.empty((max(max_blocks, 1), 4), np.int32)
    nm = ctypes.c_int32(0)
    nb = ctypes.c_int32(0)
    _check(_load().oracle_plan(_p(counts), E, begin, stride, E_loc, P, beta, _p(q), _p(moves),
                               ctypes.byref(nm), max_moves, _p(blocks), ctypes.byref(nb),
                               max(max_blocks, 1)), "plan")
    return q, moves[: nm.value].copy(), blocks[: nb.value].copy()


def plan_blocks(counts: np.ndarray, E: int, begin: int, stride: int, E_loc: int, P: int,
                beta: int, s: int):
    """Block-granular replica plan with replica budget s per rank.  -> q [E_loc, P] rows,
    moves [n_replicas, 4] (owner, rank, expert, rows), blocks [n_blocks, 4]."""
    counts = np.ascontiguousarray(counts, dtype=np.int32)
    N = int(sum(int(counts[begin + l * stride]) for l in range(E_loc)))
    max_moves = E_loc * P
    max_blocks = (N + beta - 1) // beta + E_loc * P
    q = np.empty((E_loc, P), np.int32)
    moves = np.empty((max_moves, 4), np.int32)
    blocks = np.empty((max(max_blocks, 1), 4), np.int32)
    nm = ctypes.c_int32(0)
    nb = ctypes.c_int32(0)
    _check(_load().oracle_plan_blocks(_p(counts), E, begin, stride, E_loc, P, beta, s, _p(q),
                                      _p(moves), ctypes.byref(nm), max_moves, _p(blocks),
                                      ctypes.byref(nb), max(max_blocks, 1)), "plan_blocks")
    return q, moves[: nm.value].copy(), blocks[: nb.value].copy()


def ffn_rows(xp: np.ndarray, w1: np.ndarray, w2: np.ndarray, rows: np.ndarray,
             row_expert: np.ndarray):
    """SwiGLU FFN for selected rows of xp. -> act [n, I], yp [n, H] (dtype of xp)."""
    xp = np.ascontiguousarray(xp)
    w1 = np.ascontiguousarray(w1)
    w2 = np.ascontiguousarray(w2)
    dt = _dt_code(xp)
    assert _dt_code(w1) == dt and _dt_code(w2) == dt
    H = xp.shape[1]
    I = w1.shape[1] // 2
    assert w1.shape[2] == H and w2.shape[1] == H and w2.shape[2] == I
    rows = np.ascontiguousarray(rows, dtype=np.int32)
    row_expert = np.ascontiguousarray(row_expert, dtype=np.int32)
    n = rows.shape[0]
    act = np.empty((n, I), xp.dtype)
    yp = np.empty((n, H), xp.dtype)
    _check(_load().oracle_ffn_rows(_p(xp), dt, H, I, _p(w1), _p(w2), _p(rows), _p(row_expert), n,
                                   _p(act), _p(yp)), "ffn_rows")
    return act, yp


def ffn_blocks(xp: np.ndarray, w1: np.ndarray, w2: np.ndarray, blocks: np.ndarray):
    """SwiGLU FFN over a block table. -> act [rows, I], yp [rows, H], rows = xp.shape[0];
    rows no block covers are left zero."""
    xp = np.ascontiguousarray(xp)
    dt = _dt_code(xp)
    H = xp.shape[1]
    I = w1.shape[1] // 2
    blocks = np.ascontiguousarray(blocks, dtype=np.int32).reshape(-1, 4)
    act = np.zeros((xp.shape[0], I), xp.dtype)
    yp = np.zeros((xp.shape[0], H), xp.dtype)
    _check(_load().oracle_ffn_blocks(_p(xp), dt, H, I, _p(np.ascontiguousarray(w1)),
                                     _p(np.ascontiguousarray(w2)), _p(blocks), blocks.shape[0],
                                     _p(act), _p(yp)), "ffn_blocks")
    return act, yp


MX_FP8, MX_FP4 = 0, 1


def mx_quantize(a: np.ndarray, fmt: int):
    """[rows, cols] float32 or bf16 bits -> (codes uint8 [rows, cols] (FP8) or [rows, cols/2] (FP4,
    low nibble first), scales uint8 [rows, cols/32])."""
    a = np.ascontiguousarray(a)
    dt = _dt_code(a)
    rows, cols = a.shape
    codes = np.zeros((rows, cols if fmt == MX_FP8 else cols // 2), np.uint8)
    scales = np.zeros((rows, cols // 32), np.uint8)
    _check(_load().oracle_mx_quantize(_p(a), dt, ctypes.c_int64(rows), ctypes.c_int64(cols), fmt,
                                      _p(codes), _p(scales)), "mx_quantize")
    return codes, scales


def mx_dequantize(codes: np.ndarray, scales: np.ndarray, cols: int, fmt: int) -> np.ndarray:
    codes = np.ascontiguousarray(codes, np.uint8)
    scales = np.ascontiguousarray(scales, np.uint8)
    rows = codes.shape[0]
    out = np.empty((rows, cols), np.float64)
    _check(_load().oracle_mx_dequantize(_p(codes), _p(scales), ctypes.c_int64(rows),
                                        ctypes.c_int64(cols), fmt, _p(out)), "mx_dequantize")
    return out


def ffn_mx_rows(xq, xs, w1q, w1s, w2q, w2s, H, I, rows, row_expert):
    """MX SwiGLU FFN for selected rows. -> actq [n, I] uint8, acts [n, I/32] uint8, yp [n, H] bf16
    bits (uint16)."""
    rows = np.ascontiguousarray(rows, np.int32)
    row_expert = np.ascontiguousarray(row_expert, np.int32)
    n = rows.shape[0]
    actq = np.zeros((n, I), np.uint8)
    acts = np.zeros((n, I // 32), np.uint8)
    yp = np.zeros((n, H), np.uint16)
    args = [np.ascontiguousarray(v, np.uint8) for v in (xq, xs, w1q, w1s, w2q, w2s)]
    _check(_load().oracle_ffn_mx_rows(_p(args[0]), _p(args[1]), H, I, _p(args[2]), _p(args[3]),
                                      _p(args[4]), _p(args[5]), _p(rows), _p(row_expert), n,
                                      _p(actq), _p(acts), _p(yp)), "ffn_mx_rows")
    return actq, acts, yp


def combine(yp: np.ndarray, w: np.ndarray, entry_pos: np.ndarray, T: int, K: int):
    """-> out [T, H] (dtype of yp)."""
    yp = np.ascontiguousarray(yp)
    dt = _dt_code(yp)
    H = yp.shape[1]
    w = np.ascontiguousarray(w, dtype=np.float32).reshape(T, K)
    entry_pos = np.ascontiguousarray(entry_pos, dtype=np.int32).reshape(T * K)
    out = np.empty((T, H), yp.dtype)
    _check(_load().oracle_combine(_p(yp), dt, _p(w), _p(entry_pos), T, H, K, _p(out)), "combine")
    return out


def bf16_to_f64(a: np.ndarray) -> np.ndarray:
    """Widen bf16 bit patterns (uint16) to float64 exactly."""
    return (a.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
