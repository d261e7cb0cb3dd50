"""Seeded synthetic inputs for the routed-expert path of one MoE layer.

This module only draws random numbers and lays them out; it holds none of the path's
arithmetic (no top-k, no softmax, no permutation, no GEMM).  It is the one module that both
the GPU path's tests/benchmark and the CPU oracle's tests take their inputs from.

Workloads (shapes and routing skew) follow the layer shapes the MoE pages discuss:
router logits are N(0, 1) plus log p_e with a Zipf popularity p_e proportional to
(e + 1)^(-s) over expert id (MegaFlux §4.1 uses Zipf expert popularity as its controlled
skew model); activations x ~ N(0, 1); expert weights ~ N(0, 0.02^2).  The bf16 workloads
round x and the weights to bf16 (nearest-even) once; those bits are the inputs.

Seeds: numpy PCG64 streams from SeedSequence([seed_id, stream, slot, ...]):
  logits  -> [seed_id, 0, logit_slot]
  x       -> [seed_id, 1, x_slot]
  W1[l]   -> [seed_id, 2, l],   W2[l] -> [seed_id, 3, l]   (l = local expert index)
  W_r     -> [seed_id, 4, 0]   (linear router rows, all E experts)
"""
from __future__ import annotations

import dataclasses
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import torch

WEIGHT_STD = 0.02
# Logit bias given to experts 0..3 in the "hot4" routing case, so that those four experts
# draw at least 40% of all routed entries of the Qwen3-shaped layer (checked by a CPU test).
HOT4_BIAS = 2.6


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    T: int          # tokens in the batch
    H: int          # hidden size
    E: int          # experts the router chooses among
    K: int          # experts per token (top-k)
    I: int          # SwiGLU intermediate size per expert
    P: int          # logical rank partitions the plan balances over
    dtype: str      # "f32" or "bf16"
    seed_id: int
    skews: tuple    # Zipf exponents (floats) or "hot4"
    E_loc: int = 0  # local experts (0 -> E)
    expert_begin: int = 0
    expert_stride: int = 1
    x_slot: int = 0
    logit_slot_base: int = 0
    beta: int = 128

    @property
    def n_local(self) -> int:
        return self.E_loc or self.E

    def skew_label(self, skew) -> str:
        return skew if isinstance(skew, str) else f"s{skew:g}"


WORKLOADS = {
    w.name: w
    for w in [
        Workload("tiny_f32", T=64, H=128, E=8, K=2, I=256, P=4, dtype="f32", seed_id=0,
                 skews=(1.0,)),
        Workload("olmoe_shaped", T=4096, H=2048, E=64, K=8, I=1024, P=8, dtype="bf16",
                 seed_id=1, skews=(0.0, 0.5, 1.2)),
        Workload("qwen3_30b_a3b_shaped", T=8192, H=2048, E=128, K=8, I=768, P=16, dtype="bf16",
                 seed_id=2, skews=(0.0, 0.8, 1.5, "hot4")),
        Workload("gpt_oss_120b_shaped", T=16384, H=2880, E=128, K=4, I=2880, P=8, dtype="bf16",
                 seed_id=3, skews=(0.0, 1.0, 2.0)),
        Workload("gpt_oss_120b_decode", T=64, H=2880, E=128, K=4, I=2880, P=8, dtype="bf16",
                 seed_id=3, skews=(0.0, 1.0, 2.0), x_slot=1, logit_slot_base=100),
        # One GPU's share of a DeepSeek-V3-sized layer: 256 experts routed globally (top-8),
        # the local experts are ids 3, 11, 19, ... (ids = 3 mod 8), 32 of them.
        Workload("deepseek_v3_share", T=32768, H=7168, E=256, K=8, I=2048, P=8, dtype="bf16",
                 seed_id=4, skews=(0.0, 1.0), E_loc=32, expert_begin=3, expert_stride=8),
    ]
}


def _rng(*key: int) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence(list(key)))


def zipf_log_popularity(E: int, s: float) -> np.ndarray:
    """log p_e for p_e proportional to (e+1)^(-s), normalised over the E experts."""
    logp = -s * np.log(np.arange(1, E + 1, dtype=np.float64))
    logp -= np.log(np.exp(logp).sum())
    return logp


def make_logits(w: Workload, skew) -> np.ndarray:
    """Router logits [T, E] float32: N(0,1) + log p_e (Zipf), or + HOT4_BIAS on experts 0..3."""
    slot = w.logit_slot_base + list(w.skews).index(skew)
    z = _rng(w.seed_id, 0, slot).standard_normal((w.T, w.E), dtype=np.float32)
    if skew == "hot4":
        bias = np.zeros((w.E,), np.float32)
        bias[:4] = HOT4_BIAS
    else:
        bias = zipf_log_popularity(w.E, float(skew)).astype(np.float32)
    return z + bias[None, :]


def _to_dtype(a: np.ndarray, dtype: str) -> torch.Tensor:
    t = torch.from_numpy(a)
    return t.to(torch.bfloat16) if dtype == "bf16" else t


def make_x(w: Workload) -> torch.Tensor:
    """Activations [T, H] on the CPU: float32 N(0,1), rounded to bf16 for bf16 workloads."""
    a = _rng(w.seed_id, 1, w.x_slot).standard_normal((w.T, w.H), dtype=np.float32)
    return _to_dtype(a, w.dtype)


def _one_expert(w: Workload, stream: int, l: int, shape) -> torch.Tensor:
    a = _rng(w.seed_id, stream, l).standard_normal(shape, dtype=np.float32)
    a *= np.float32(WEIGHT_STD)
    return _to_dtype(a, w.dtype)


def make_weights(w: Workload, experts=None, threads: int = 8):
    """Expert weights on the CPU for the listed local experts (all by default):
    W1 [n, 2I, H] (rows 0..I-1 gate, I..2I-1 up) and W2 [n, H, I]."""
    experts = list(range(w.n_local)) if experts is None else list(experts)
    dt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    W1 = torch.empty((len(experts), 2 * w.I, w.H), dtype=dt)
    W2 = torch.empty((len(experts), w.H, w.I), dtype=dt)

    def fill(j):
        l = experts[j]
        W1[j] = _one_expert(w, 2, l, (2 * w.I, w.H))
        W2[j] = _one_expert(w, 3, l, (w.H, w.I))

    with ThreadPoolExecutor(max(1, threads)) as ex:
        list(ex.map(fill, range(len(experts))))
    return W1, W2


def make_router_weights(w: Workload) -> torch.Tensor:
    """Linear router rows W_r [E, H] on the CPU: N(0, 0.02^2), rounded to bf16 for bf16
    workloads (router scores x . W_r^T then have a spread of about 0.02 sqrt(H))."""
    a = _rng(w.seed_id, 4, 0).standard_normal((w.E, w.H), dtype=np.float32)
    a *= np.float32(WEIGHT_STD)
    return _to_dtype(a, w.dtype)


def as_oracle_array(t: torch.Tensor) -> np.ndarray:
    """CPU tensor -> numpy array the oracle takes (bf16 as uint16 bit patterns)."""
    t = t.contiguous().cpu()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def from_bf16_bits(a: np.ndarray) -> torch.Tensor:
    """numpy uint16 bf16 bit patterns -> CPU bf16 tensor."""
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16)


def rows_of_config_text() -> dict:
    """Sizes of each workload, for reports."""
    out = {}
    for name, w in WORKLOADS.items():
        out[name] = dict(T=w.T, H=w.H, E=w.E, E_loc=w.n_local, K=w.K, I=w.I, P=w.P,
                         dtype=w.dtype, skews=[w.skew_label(s) for s in w.skews])
    return out


def ceil_div(a: int, b: int) -> int:
    return -(-a // b)

