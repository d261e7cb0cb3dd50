"""GPU parity of the router entry points (through the C ABI) against the CPU oracle.

moe_router_topk: the float32 scores against the oracle's (x . W_r^T in double, rounded to
float32) within the worst-case bound of float32 summation, 2 (H + 1) u sum_h |x_h w_eh| with
u = 2^-24 (any order, each addition rounded), and a relative Frobenius error of at most 1e-5;
then the top-k decided on the GPU's own float32 scores, so that both sides take the integer
decision in the same precision: ids and counts bit-exact, weights within 1e-6 of the oracle's
route_ref on those scores.  moe_route_ref: the same bar on precomputed logits."""
import zlib

import numpy as np
import pytest
import torch

import oracle
from mixture_experts_routed_router_amd import binding, inputs
from parity_helpers import host, rel_frob

pytestmark = pytest.mark.gpu

U = 2.0 ** -24


def _announce(msg):
    print(f"\n[router] {msg}", flush=True)


def _abs(a: np.ndarray) -> np.ndarray:
    return (a & np.uint16(0x7FFF)) if a.dtype == np.uint16 else np.abs(a)


def _outputs(T, E, K, dev="cuda"):
    return (torch.full((T, K), -1, dtype=torch.int32, device=dev),
            torch.full((T, K), -1.0, dtype=torch.float32, device=dev),
            torch.full((E,), -7, dtype=torch.int32, device=dev))


def _check_topk(g_logits, ids, w, counts, K, k_ref, T_all=None):
    r_ids, r_w, r_counts = oracle.route_ref(g_logits, K, k_ref)
    assert np.array_equal(host(ids), r_ids), "topk ids"
    assert np.array_equal(host(counts), r_counts), "expert counts"
    dw = np.abs(host(w).astype(np.float64) - r_w.astype(np.float64)).max()
    assert dw <= 1e-6, f"routing weights |dw| {dw}"


def _check_logits(g, x_o, w_o, rows=None):
    """GPU scores g [n, E] against the oracle's on token rows `rows` of x (all if None)."""
    xs = x_o if rows is None else x_o[rows]
    ref = oracle.router_logits(xs, w_o)
    mag = oracle.router_logits(_abs(xs), _abs(w_o)).astype(np.float64)
    H = x_o.shape[1]
    bound = 2.0 * (H + 1) * U * mag + 1e-30
    d = np.abs(g.astype(np.float64) - ref.astype(np.float64))
    worst = float((d / bound).max())
    assert worst <= 1.0, f"router score outside the float32 summation bound ({worst:.3f}x)"
    e = rel_frob(g.astype(np.float64), ref.astype(np.float64))
    assert e <= 1e-5, f"router score rel err {e}"
    return e


def _run_router(x_dev, wr_dev, K, k_ref, with_logits=True):
    T, E = x_dev.shape[0], wr_dev.shape[0]
    ids, w, counts = _outputs(T, E, K)
    logits = torch.full((T, E), float("nan"), dtype=torch.float32, device="cuda") if with_logits else None
    binding.moe_router_topk(x_dev, wr_dev, K, k_ref, ids, w, counts, logits=logits)
    torch.cuda.synchronize()
    return logits, ids, w, counts


def _random_inputs(seed, T, H, E, dtype):
    rng = np.random.default_rng(seed)
    x = torch.from_numpy(rng.standard_normal((T, H), dtype=np.float32)).to(dtype)
    wr = torch.from_numpy(rng.standard_normal((E, H), dtype=np.float32) * 0.05).to(dtype)
    return x, wr


SMALL = [
    # name, T, H, E, K, k_ref, dtype
    ("bf16_e64_k8", 300, 256, 64, 8, 8, torch.bfloat16),
    ("bf16_e64_kref9", 300, 256, 64, 8, 9, torch.bfloat16),
    ("bf16_e128_kref16", 300, 128, 128, 4, 16, torch.bfloat16),
    ("bf16_e256_softmax", 1000, 192, 256, 8, 256, torch.bfloat16),
    ("bf16_e20_ragged", 77, 64, 20, 6, 7, torch.bfloat16),
    ("bf16_t1", 1, 128, 64, 8, 64, torch.bfloat16),
    ("bf16_k1", 555, 64, 32, 1, 1, torch.bfloat16),
    ("bf16_k16", 300, 128, 96, 16, 16, torch.bfloat16),
    # 257 tiles of 64 tokens: the 64-token tile shape and the grid-stride loop
    ("bf16_tm64_stride", 16400, 64, 64, 8, 8, torch.bfloat16),
    # 128-token tiles for E > 128 (192 and 256 router rows), ragged E and T, grid-stride
    ("bf16_tm128_e160", 32768 + 77, 128, 160, 6, 7, torch.bfloat16),
    ("bf16_tm128_e200", 32768, 64, 200, 8, 8, torch.bfloat16),
    # 128-token tiles (8 waves) with top-k lists of 16 and of 4, and one token past a tile
    ("bf16_tm128_k16", 32768, 64, 256, 16, 16, torch.bfloat16),
    ("bf16_tm128_k4_e192", 32768 + 1, 64, 192, 4, 4, torch.bfloat16),
    ("f32_ragged_h", 200, 100, 40, 3, 40, torch.float32),
    ("f32_e256_k16", 130, 64, 256, 16, 16, torch.float32),
    ("f32_e8_kref3", 64, 128, 8, 2, 3, torch.float32),
]


@pytest.mark.parametrize("name,T,H,E,K,k_ref,dtype", SMALL)
def test_router_topk_small(name, T, H, E, K, k_ref, dtype):
    _announce(f"{name} T={T} H={H} E={E} K={K} k_ref={k_ref}")
    x, wr = _random_inputs(zlib.crc32(name.encode()), T, H, E, dtype)
    logits, ids, w, counts = _run_router(x.cuda(), wr.cuda(), K, k_ref)
    g = host(logits)
    _check_logits(g, inputs.as_oracle_array(x), inputs.as_oracle_array(wr))
    _check_topk(g, ids, w, counts, K, k_ref)
    # without the score output: the same picks and weights, bit for bit
    _, ids2, w2, counts2 = _run_router(x.cuda(), wr.cuda(), K, k_ref, with_logits=False)
    assert torch.equal(ids, ids2) and torch.equal(w, w2) and torch.equal(counts, counts2)


def test_router_topk_tiny_f32_workload():
    wl = inputs.WORKLOADS["tiny_f32"]
    x, wr = inputs.make_x(wl), inputs.make_router_weights(wl)
    for k_ref in (wl.K, wl.K + 1, wl.E):
        _announce(f"tiny_f32 k_ref={k_ref}")
        logits, ids, w, counts = _run_router(x.cuda(), wr.cuda(), wl.K, k_ref)
        g = host(logits)
        _check_logits(g, inputs.as_oracle_array(x), inputs.as_oracle_array(wr))
        _check_topk(g, ids, w, counts, wl.K, k_ref)


@pytest.mark.parametrize("name", ["olmoe_shaped", "qwen3_30b_a3b_shaped", "gpt_oss_120b_shaped",
                                  "gpt_oss_120b_decode", "deepseek_v3_share"])
def test_router_topk_full_size(name):
    """Full layer sizes: every score row for OLMoE's shape, 1024 sampled token rows for the
    larger ones; the top-k on every token."""
    wl = inputs.WORKLOADS[name]
    _announce(f"{name} T={wl.T} H={wl.H} E={wl.E} K={wl.K}")
    x, wr = inputs.make_x(wl), inputs.make_router_weights(wl)
    x_dev, wr_dev = x.cuda(), wr.cuda()
    logits, ids, w, counts = _run_router(x_dev, wr_dev, wl.K, wl.K)
    g = host(logits)
    x_o, w_o = inputs.as_oracle_array(x), inputs.as_oracle_array(wr)
    if wl.T * wl.H * wl.E <= 1 << 30:
        _check_logits(g, x_o, w_o)
    else:
        rows = np.sort(np.random.default_rng(7).choice(wl.T, 1024, replace=False))
        rows[-1] = wl.T - 1  # the ragged end of the last tile
        _check_logits(g[rows], x_o, w_o, rows=rows)
    _check_topk(g, ids, w, counts, wl.K, wl.K)
    assert int(host(counts).sum()) == wl.T * wl.K


SCAN_FORMS = [
    # T, E, K, k_ref, offset (floats the rows start past a 16-byte boundary)
    (16400, 256, 8, 8, 0),     # 4 lanes per token, staged slices
    (16400, 256, 8, 8, 1),     # rows not 16-byte aligned: float-by-float scan
    (16400, 130, 8, 130, 0),   # E not a power of two: float-by-float, plain softmax denominator
    (3000, 64, 6, 64, 0),      # 16 lanes per token, staged, plain softmax denominator
    (3000, 61, 5, 7, 0),       # E odd, k_ref = K + 2
    (2000, 128, 16, 16, 3),    # K = 16, rows 12 bytes off
    (1, 256, 8, 8, 0),         # one token
    # staged reads (4 lanes per token from T = 16369) across the slice counts of the scan:
    (16400, 256, 4, 4, 0),     # KM 4: groups of 4, four slices
    (16400, 256, 16, 16, 0),   # KM 16 over 64 experts per lane
    (16400, 256, 8, 256, 0),   # plain softmax denominator from the staged values
    (16400, 64, 8, 8, 0),      # 16 experts per lane: two slices
    (16401, 128, 4, 4, 0),     # a last wave with one token
]


@pytest.mark.parametrize("T,E,K,k_ref,offset", SCAN_FORMS)
def test_route_ref_scan_forms(T, E, K, k_ref, offset):
    """moe_route_ref reads a wave's rows as staged 16-byte column slices when the rows fill the
    lanes exactly (E a power of two) and the logits are 16-byte aligned, else each lane reads its
    row float by float: both forms against the oracle, over the scan's group and slice layouts,
    with exact ties, +0 / -0 pairs (equal logits) and subnormal logits planted in some rows."""
    _announce(f"scan T={T} E={E} K={K} k_ref={k_ref} offset={offset}")
    rng = np.random.default_rng(zlib.crc32(f"scan {T} {E} {offset}".encode()))
    logits = rng.standard_normal((T, E), dtype=np.float32)
    logits[::7, ::3] = 0.5                                    # ties at the top
    logits[1::11, :] = 0.0
    logits[1::11, 1::2] = -0.0                                # rows of +0 / -0 only
    logits[2::13, : E // 2] = np.float32(1e-40)               # subnormals either sign
    logits[2::13, E // 2:] = np.float32(-1e-40)
    logits[3::17, E - 1] = 3e38                               # the last expert wins
    buf = torch.full((T * E + offset,), float("nan"), dtype=torch.float32, device="cuda")
    d_logits = buf[offset:].view(T, E)
    d_logits.copy_(torch.from_numpy(logits))
    ids, w, counts = _outputs(T, E, K)
    binding.moe_route_ref(d_logits, K, k_ref, ids, w, counts)
    torch.cuda.synchronize()
    _check_topk(logits, ids, w, counts, K, k_ref)


@pytest.mark.parametrize("name,skew", [("olmoe_shaped", 1.2), ("qwen3_30b_a3b_shaped", "hot4")])
def test_route_ref_workload_logits(name, skew):
    """moe_route_ref on the workload's precomputed logits for k_ref = K, K + 1, 16 and E."""
    wl = inputs.WORKLOADS[name]
    logits = inputs.make_logits(wl, skew)
    d_logits = torch.from_numpy(logits).cuda()
    for k_ref in sorted({wl.K, wl.K + 1, 16, wl.E}):
        _announce(f"{name} {skew} k_ref={k_ref}")
        ids, w, counts = _outputs(wl.T, wl.E, wl.K)
        binding.moe_route_ref(d_logits, wl.K, k_ref, ids, w, counts)
        torch.cuda.synchronize()
        _check_topk(logits, ids, w, counts, wl.K, k_ref)


def test_route_ref_k_equals_route():
    """k_ref = K is moe_route with renormalisation and k_ref = E is moe_route without it: the
    same outputs bit for bit."""
    wl = inputs.WORKLOADS["olmoe_shaped"]
    d_logits = torch.from_numpy(inputs.make_logits(wl, 0.5)).cuda()
    for k_ref, renorm in ((wl.K, True), (wl.E, False)):
        a = _outputs(wl.T, wl.E, wl.K)
        b = _outputs(wl.T, wl.E, wl.K)
        binding.moe_route_ref(d_logits, wl.K, k_ref, *a)
        binding.moe_route(d_logits, wl.K, *b, renormalize=renorm)
        torch.cuda.synchronize()
        for u, v in zip(a, b):
            assert torch.equal(u, v)
