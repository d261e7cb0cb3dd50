"""GPU parity of the block-granular replica plan (moe_plan_blocks, through the C ABI) against
the CPU oracle: q, the replica list, the block table and their counts bit for bit, err_word 0;
and the whole path planned this way gives the same outputs, bit for bit, as with moe_plan
(each row is computed once either way, with the same accumulation order)."""
import json
import os

import numpy as np
import pytest
import torch

import oracle
from mixture_experts_routed_router_amd import binding, inputs
from parity_helpers import host, oracle_index, run_gpu, workload_case

pytestmark = pytest.mark.gpu

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _announce(msg):
    print(f"\n[plan_blocks] {msg}", flush=True)


def _gpu_plan(counts, E, begin, stride, E_loc, P, beta, s):
    i32 = dict(dtype=torch.int32, device="cuda")
    N = int(np.asarray(counts, np.int64).sum())
    max_blocks = -(-N // beta) + E_loc * P  # every expert may end in a partial block
    q = torch.full((E_loc, P), -5, **i32)
    moves = torch.full((E_loc * P, 4), -5, **i32)  # one per replica at most
    blocks = torch.full((max_blocks, 4), -5, **i32)
    n_moves, n_blocks, err = (torch.full((1,), -5, **i32) for _ in range(3))
    d_counts = torch.from_numpy(np.ascontiguousarray(counts, np.int32)).cuda()
    binding.moe_plan_blocks(d_counts, E, begin, stride, E_loc, P, beta, s, q, moves, n_moves,
                            blocks, n_blocks, err)
    torch.cuda.synchronize()
    nm, nb = int(n_moves.item()), int(n_blocks.item())
    return host(q), host(moves)[:nm], host(blocks)[:nb], int(err.item())


def _check(counts, E, begin, stride, E_loc, P, beta, s, label):
    q, moves, blocks, err = _gpu_plan(counts, E, begin, stride, E_loc, P, beta, s)
    rq, rmoves, rblocks = oracle.plan_blocks(np.asarray(counts, np.int32), E, begin, stride,
                                             E_loc, P, beta, s)
    assert err == 0, label
    assert np.array_equal(q, rq), (label, "q")
    assert np.array_equal(moves, rmoves), (label, "moves")
    assert np.array_equal(blocks, rblocks), (label, "blocks")
    return rq, rmoves, rblocks


def test_plan_blocks_golden_cases():
    """The hand-worked plans, scaled to block_m = 16 (the ABI's smallest; counts scaled by the
    same factor keep every block boundary, so the plans are the same in blocks)."""
    for c in json.load(open(os.path.join(GOLDEN, "megaflux_plan_cases.json")))["cases"]:
        _announce(c["name"])
        n = len(c["counts"])
        f = 16 // c["beta"]
        rq, _, _ = _check([v * f for v in c["counts"]], n, 0, 1, n, c["P"], 16, c["s"], c["name"])
        assert np.array_equal(rq, np.array(c["q"]) * f), c["name"]


@pytest.mark.parametrize("name", list(inputs.WORKLOADS))
def test_plan_blocks_workloads(name):
    """Every workload and skew at budgets 0, E_loc / (4P) (the pages' setting), 2 and E_loc."""
    w = inputs.WORKLOADS[name]
    for skew in w.skews:
        _, _, counts = oracle.route(inputs.make_logits(w, skew), w.K)
        for s in sorted({0, w.n_local // (4 * w.P), 2, w.n_local}):
            _announce(f"{name} {w.skew_label(skew)} s={s}")
            _check(counts, w.E, w.expert_begin, w.expert_stride, w.n_local, w.P, w.beta, s,
                   f"{name} {skew} s={s}")


def test_plan_blocks_random_shapes():
    """Random count vectors across the limits: up to 64 ranks, 64 experts per rank, 256 local
    experts, E_loc * P = 4096, block sizes 16..256, budgets 0..8, heavy skew and empty experts."""
    rng = np.random.default_rng(21)
    shapes = [(64, 64, 16), (256, 16, 32), (64, 1, 128), (256, 4, 128), (128, 32, 64),
              (16, 16, 256), (8, 2, 16), (4096 // 64, 64, 16)]
    for trial in range(40):
        E_loc, P, beta = shapes[trial % len(shapes)]
        scale = int(rng.integers(1, 4000))
        z = np.minimum(rng.zipf(1.3 + rng.random(), size=E_loc), 1 << 20).astype(np.int64)
        counts = z * scale // 7  # no int64 overflow; anything this large is capped below
        counts[rng.random(E_loc) < 0.2] = 0
        counts = np.minimum(counts, 20000).astype(np.int32)
        s = int(rng.integers(0, 9))
        _check(counts, E_loc, 0, 1, E_loc, P, beta, s, f"trial {trial}")


@pytest.mark.parametrize("name,skew", [("olmoe_shaped", 1.2), ("qwen3_30b_a3b_shaped", "hot4"),
                                       ("deepseek_v3_share", 1.0), ("gpt_oss_120b_decode", 2.0)])
def test_path_with_block_plan_matches_moonep_plan(name, skew):
    """The whole path with the block-granular plan: its block table matches the oracle's, and
    act / yp on every valid row and out on every token equal the moe_plan path bit for bit."""
    w = inputs.WORKLOADS[name]
    T = min(w.T, 2048)
    c = workload_case(name, skew, T=T)
    _announce(f"{name} {skew} T={T}")
    a = run_gpu(c, gather=True)
    logits, x, W1, W2 = a._inputs
    b = binding.RoutedExperts(c.T, c.H, c.E, c.K, c.I, c.P, dtype=c.dtype, E_loc=c.n_local,
                              expert_begin=c.begin, expert_stride=c.stride, block_m=c.block_m,
                              device="cuda", gather=True, planner="megaflux")
    b.forward(logits, x, W1, W2)
    torch.cuda.synchronize()
    ref = oracle_index(c)
    _, rmoves, rblocks = oracle.plan_blocks(ref.counts, c.E, c.begin, c.stride, c.n_local, c.P,
                                            c.block_m, b.replica_budget)
    nb = int(b.n_blocks.item())
    assert np.array_equal(host(b.blocks)[:nb], rblocks)
    assert int(b.err_word.item()) == 0
    rows = int(host(a.offsets)[-1])
    valid = torch.nonzero(a.row_token[:rows] >= 0).squeeze(1)
    assert torch.equal(a.act[valid], b.act[valid]), "act"
    assert torch.equal(a.yp[valid], b.yp[valid]), "yp"
    assert torch.equal(a.out, b.out), "out"
