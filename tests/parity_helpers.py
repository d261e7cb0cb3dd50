"""Helpers of the GPU parity tests: run the HIP path through the C ABI, run the oracle on the
same inputs, compare.  Test infrastructure only."""
from __future__ import annotations

import dataclasses

import numpy as np
import torch

import oracle
from mixture_experts_routed_router_amd import binding, inputs

BF16_TOL = 5e-3   # relative Frobenius error for bf16 outputs (float32 accumulation)
F32_TOL = 1e-5    # relative Frobenius error for the float32 layer
W_TOL = 1e-6      # absolute error of routing weights


def rel_frob(got: np.ndarray, ref: np.ndarray) -> float:
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    n = np.linalg.norm(ref)
    return float(np.linalg.norm(got - ref) / (n if n > 0 else 1.0))


def check_rows(got: np.ndarray, ref: np.ndarray, what: str, row_tol: float = 1e-2,
               ulp_rel: float = 2.0 ** -7, rms_frac: float = 2e-3, extra=None) -> dict:
    """Element-resolving comparison of bf16 output rows (float64 views) with the oracle's, next
    to the layer-wide relative Frobenius bar:
      * every row's own relative Frobenius error is at most row_tol, and
      * every element satisfies |got - ref| <= ulp_rel |ref| + rms_frac rms(ref row) + extra.
    Both sides round to bf16 once from float32 (HIP) or float64 (oracle) accumulation, so a
    correct element differs by at most one bf16 ulp (<= 2^-7 |ref|) plus the accumulation
    difference, which is orders of magnitude below rms_frac of the row.  `extra` carries what
    the step's own inputs already differ by, propagated exactly (the sum over the reduction of
    |input difference| x |weight|): an input that rounded to the neighbouring bf16 value moves
    the output by that much and no more.  A wrong element, a wrong column block or a wrong row
    moves by about the row's rms.  Returns the worst figures."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    assert got.shape == ref.shape, (what, got.shape, ref.shape)
    rms = np.sqrt(np.mean(ref * ref, axis=1, keepdims=True))
    diff = np.abs(got - ref)
    bound = ulp_rel * np.abs(ref) + rms_frac * rms + 1e-30
    if extra is not None:
        bound = bound + 1.01 * np.asarray(extra, np.float64)
    viol = diff > bound
    assert not viol.any(), (what, "elements out of bound", int(viol.sum()),
                            [tuple(int(v) for v in i) for i in np.argwhere(viol)[:8]])
    rnorm = np.linalg.norm(ref, axis=1)
    row_err = np.linalg.norm(got - ref, axis=1) / np.where(rnorm > 0, rnorm, 1.0)
    assert row_err.max(initial=0.0) <= row_tol, (what, "row", int(row_err.argmax()), float(row_err.max()))
    return {"max_row_err": float(row_err.max(initial=0.0)),
            "max_elem_ratio": float((diff / bound).max(initial=0.0))}


def to_f64(a: np.ndarray) -> np.ndarray:
    return oracle.bf16_to_f64(a) if a.dtype == np.uint16 else a.astype(np.float64)


def host(t: torch.Tensor) -> np.ndarray:
    """Device tensor -> numpy (bf16 as uint16 bits)."""
    return inputs.as_oracle_array(t.detach().cpu())


@dataclasses.dataclass
class Case:
    """One layer instance: shapes, host inputs (the shared seeded inputs) and device copies."""
    T: int
    H: int
    E: int
    K: int
    I: int
    P: int
    dtype: torch.dtype
    logits: np.ndarray
    x: torch.Tensor
    W1: torch.Tensor
    W2: torch.Tensor
    E_loc: int = 0
    begin: int = 0
    stride: int = 1
    block_m: int = 128
    renormalize: bool = True

    @property
    def n_local(self):
        return self.E_loc or self.E

    @property
    def tol(self):
        return F32_TOL if self.dtype == torch.float32 else BF16_TOL


def workload_case(name: str, skew, weights=None, T: int | None = None) -> Case:
    w = inputs.WORKLOADS[name]
    logits = inputs.make_logits(w, skew)
    x = inputs.make_x(w)
    if T is not None:
        logits, x = logits[:T].copy(), x[:T].contiguous()
    W1, W2 = weights if weights is not None else inputs.make_weights(w)
    return Case(T=logits.shape[0], H=w.H, E=w.E, K=w.K, I=w.I, P=w.P,
                dtype=torch.float32 if w.dtype == "f32" else torch.bfloat16, logits=logits, x=x,
                W1=W1, W2=W2, E_loc=w.E_loc, begin=w.expert_begin, stride=w.expert_stride,
                block_m=w.beta)


def random_case(seed, T, H, E, K, I, P, dtype=torch.bfloat16, E_loc=0, begin=0, stride=1,
                block_m=128, logit_bias=None, renormalize=True) -> Case:
    rng = np.random.default_rng(seed)
    logits = rng.standard_normal((T, E), dtype=np.float32)
    if logit_bias is not None:
        logits = logits + np.asarray(logit_bias, np.float32)[None, :]
    n_loc = E_loc or E
    x = torch.from_numpy(rng.standard_normal((T, H), dtype=np.float32)).to(dtype)
    W1 = torch.from_numpy((rng.standard_normal((n_loc, 2 * I, H), dtype=np.float32) * 0.05)).to(dtype)
    W2 = torch.from_numpy((rng.standard_normal((n_loc, H, I), dtype=np.float32) * 0.05)).to(dtype)
    return Case(T=T, H=H, E=E, K=K, I=I, P=P, dtype=dtype, logits=logits, x=x, W1=W1, W2=W2,
                E_loc=E_loc, begin=begin, stride=stride, block_m=block_m, renormalize=renormalize)


def run_gpu(c: Case, dev="cuda", gather=False, direct=False):
    """The whole path through the C ABI; returns the layer object (all buffers on device).
    gather: FC1 reads x rows through row_token and xp is not materialised.  direct: the down
    GEMM writes the out rows of one-entry tokens and the combine skips them."""
    layer = binding.RoutedExperts(c.T, c.H, c.E, c.K, c.I, c.P, dtype=c.dtype, E_loc=c.n_local,
                                  expert_begin=c.begin, expert_stride=c.stride,
                                  block_m=c.block_m, renormalize=c.renormalize, device=dev,
                                  gather=gather, direct=direct)
    logits = torch.from_numpy(c.logits).to(dev)
    x = c.x.to(dev)
    W1, W2 = c.W1.to(dev), c.W2.to(dev)
    layer.forward(logits, x, W1, W2)
    torch.cuda.synchronize()
    layer._inputs = (logits, x, W1, W2)
    return layer


@dataclasses.dataclass
class OracleIndex:
    ids: np.ndarray
    w: np.ndarray
    counts: np.ndarray
    offsets: np.ndarray
    entry_pos: np.ndarray
    row_token: np.ndarray
    q: np.ndarray
    moves: np.ndarray
    blocks: np.ndarray


def oracle_index(c: Case) -> OracleIndex:
    """Route, permutation indices and plan from the oracle (cheap at every size)."""
    ids, w, counts = oracle.route(c.logits, c.K, c.renormalize)
    offs, ep, rt, _ = oracle.permute(ids, counts, c.E, c.begin, c.stride, c.n_local, c.block_m)
    q, moves, blocks = oracle.plan(counts, c.E, c.begin, c.stride, c.n_local, c.P, c.block_m)
    return OracleIndex(ids, w, counts, offs, ep, rt, q, moves, blocks)


def check_index_parity(layer, ref: OracleIndex):
    """Bit-exact ids, counts, offsets, entry_pos, row_token, q, moves, blocks; weights 1e-6."""
    assert np.array_equal(host(layer.topk_ids), ref.ids), "topk_ids"
    assert np.array_equal(host(layer.counts), ref.counts), "expert_counts"
    dw = np.max(np.abs(host(layer.topk_w).astype(np.float64) - ref.w))
    assert dw <= W_TOL, f"topk_w max abs diff {dw}"
    assert np.array_equal(host(layer.offsets), ref.offsets), "expert_offsets"
    assert np.array_equal(host(layer.entry_pos), ref.entry_pos), "entry_pos"
    rows_pad = int(ref.offsets[-1])
    assert np.array_equal(host(layer.row_token)[:rows_pad], ref.row_token), "row_token"
    assert np.array_equal(host(layer.q), ref.q), "q"
    nm = int(host(layer.n_moves)[0])
    assert nm == ref.moves.shape[0], "n_moves"
    assert np.array_equal(host(layer.moves)[:nm], ref.moves), "moves"
    nb = int(host(layer.n_blocks)[0])
    assert nb == ref.blocks.shape[0], "n_blocks"
    assert np.array_equal(host(layer.blocks)[:nb], ref.blocks), "blocks"
    assert int(host(layer.err_word)[0]) == 0, "plan err_word"


def check_xp(layer, c: Case, ref: OracleIndex):
    """Valid rows of xp are exact copies of their token's row of x."""
    rows_pad = int(ref.offsets[-1])
    valid = torch.from_numpy(np.nonzero(ref.row_token >= 0)[0]).to(layer.xp.device)
    tok = torch.from_numpy(ref.row_token[ref.row_token >= 0].astype(np.int64)).to(layer.xp.device)
    x = layer._inputs[1]
    assert rows_pad <= layer.xp.shape[0]
    assert torch.equal(layer.xp[valid], x[tok]), "xp rows"


def row_experts(blocks: np.ndarray, rows: np.ndarray) -> np.ndarray:
    """Local expert of each permuted row, from the block table."""
    ex = np.full(int(blocks[:, 2].max() + blocks[:, 3].max() + 1) if len(blocks) else 1, -1)
    for _, l, b0, m in blocks.tolist():
        ex[b0:b0 + m] = l
    return ex[rows]


def tile_rows(ref: OracleIndex, seed: int = 0, piece: int = 128, sub: int = 32) -> np.ndarray:
    """One random row from every `sub`-row block of every `piece`-row cut of each expert's
    rows.  The FFN's tile schedule cuts each expert's row range into 128-row pieces (two per
    256-row GEMM tile) and each wave computes 32-row blocks of a piece, so this reaches every
    tile, both halves, and every 32-row block of the GEMMs, over all their column tiles."""
    rng = np.random.default_rng(seed)
    out = []
    for l in range(len(ref.offsets) - 1):
        first = int(ref.offsets[l])
        n = int(np.count_nonzero(ref.row_token[first:int(ref.offsets[l + 1])] >= 0))
        for p0 in range(0, n, piece):
            for s0 in range(p0, min(p0 + piece, n), sub):
                out.append(first + int(rng.integers(s0, min(s0 + sub, n))))
    return np.array(sorted(set(out)), np.int64)


def sample_rows(ref: OracleIndex, n: int, seed: int = 0) -> np.ndarray:
    """Valid rows to check one by one: first and last rows of blocks (tile edges, partial
    blocks) plus random rows."""
    rng = np.random.default_rng(seed)
    valid = np.nonzero(ref.row_token >= 0)[0]
    edges = []
    for _, _, b0, m in ref.blocks.tolist():
        edges += [b0, b0 + m - 1]
    edges = np.unique(np.array(edges, np.int64))
    pick = rng.choice(edges, size=min(len(edges), n // 2), replace=False) if len(edges) else []
    rest = rng.choice(valid, size=min(len(valid), n - len(pick)), replace=False)
    return np.unique(np.concatenate([np.asarray(pick, np.int64), rest.astype(np.int64)]))
