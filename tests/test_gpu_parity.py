"""GPU parity: the HIP path (through the C ABI) against the CPU oracle on the same seeded
inputs.  Bit-exact for ids, counts, offsets, permutation, plan and block table; routing
weights within 1e-6; act / yp / out within a relative Frobenius error of 5e-3 (bf16, float32
accumulation) or 1e-5 (float32 layer)."""
import gc

import numpy as np
import pytest
import torch

import oracle
from mixture_experts_routed_router_amd import binding, inputs
from parity_helpers import (check_index_parity, check_rows, check_xp, host, oracle_index,
                            random_case, rel_frob, row_experts, run_gpu, sample_rows, tile_rows,
                            to_f64, workload_case)

pytestmark = pytest.mark.gpu


def _announce(msg):
    print(f"\n[parity] {msg}", flush=True)


def _full_check(c, layer, ref):
    """Every output against the oracle on every row (small layers)."""
    check_index_parity(layer, ref)
    x = inputs.as_oracle_array(c.x)
    _, _, _, xp = oracle.permute(ref.ids, ref.counts, c.E, c.begin, c.stride, c.n_local,
                                 c.block_m, x)
    valid = ref.row_token >= 0
    assert np.array_equal(host(layer.xp)[: len(valid)][valid], xp[valid]), "xp"
    W1, W2 = inputs.as_oracle_array(c.W1), inputs.as_oracle_array(c.W2)
    act, yp = oracle.ffn_blocks(xp, W1, W2, ref.blocks)
    g_act = host(layer.act)[: len(valid)][valid]
    g_yp = host(layer.yp)[: len(valid)][valid]
    e_act = rel_frob(to_f64(g_act), to_f64(act[valid]))
    e_yp = rel_frob(to_f64(g_yp), to_f64(yp[valid]))
    assert e_act <= c.tol, f"act rel err {e_act}"
    assert e_yp <= c.tol, f"yp rel err {e_yp}"
    # combine on the GPU's own yp, then the whole chain on the oracle's yp
    out_same_yp = oracle.combine(host(layer.yp)[: len(valid)], host(layer.topk_w), ref.entry_pos,
                                 c.T, c.K)
    out_chain = oracle.combine(yp, ref.w, ref.entry_pos, c.T, c.K)
    g_out = to_f64(host(layer.out))
    e_comb = rel_frob(g_out, to_f64(out_same_yp))
    e_chain = rel_frob(g_out, to_f64(out_chain))
    assert e_comb <= c.tol, f"combine rel err {e_comb}"
    assert e_chain <= c.tol, f"end-to-end rel err {e_chain}"
    return dict(act=e_act, yp=e_yp, combine=e_comb, chain=e_chain)


# --------------------------------------------------------------- small layers: full ---

def test_tiny_f32_full():
    c = workload_case("tiny_f32", 1.0)
    _announce("tiny_f32 s=1")
    errs = _full_check(c, run_gpu(c), oracle_index(c))
    print(errs)


@pytest.mark.parametrize("name,kw", [
    ("ragged", dict(seed=1, T=37, H=128, E=12, K=3, I=192, P=4, block_m=32)),
    ("single_token", dict(seed=2, T=1, H=64, E=8, K=2, I=64, P=2)),
    ("k1", dict(seed=3, T=200, H=128, E=8, K=1, I=128, P=4, block_m=16)),
    ("subset_local", dict(seed=4, T=300, H=128, E=16, K=3, I=128, P=2, E_loc=4, begin=1,
                          stride=3, block_m=64)),
    ("hot_experts", dict(seed=5, T=700, H=64, E=8, K=2, I=64, P=4,
                         logit_bias=[30, 29, 0, 0, 0, 0, 0, 0])),
    ("tall_blocks", dict(seed=6, T=600, H=128, E=4, K=2, I=128, P=2, block_m=256)),
    ("no_renorm", dict(seed=7, T=96, H=64, E=16, K=4, I=64, P=4, renormalize=False)),
    ("wide_k", dict(seed=8, T=80, H=64, E=256, K=16, I=64, P=16, block_m=16)),
    ("f32_ragged", dict(seed=9, T=50, H=32, E=6, K=2, I=48, P=3, dtype=torch.float32,
                        block_m=16)),
    # plan reductions: 64 ranks (cross-row rank groups), 32 and 128 experts per rank (cross-row
    # and several experts per lane), a single rank (no moves)
    ("many_ranks", dict(seed=11, T=300, H=64, E=64, K=4, I=64, P=64, block_m=16,
                        logit_bias=[1.5] * 8 + [0.0] * 56)),
    ("g32", dict(seed=13, T=500, H=64, E=128, K=4, I=64, P=4, block_m=64,
                 logit_bias=[1.0] * 32 + [0.0] * 96)),
    ("wide_groups", dict(seed=12, T=400, H=64, E=256, K=8, I=64, P=2, block_m=32,
                         logit_bias=[0.8] * 128 + [0.0] * 128)),
    ("one_rank", dict(seed=14, T=100, H=64, E=16, K=2, I=64, P=1)),
    # more than 3072 blocks: the FFN tile schedule walks the block table in global memory
    ("many_blocks", dict(seed=15, T=8192, H=64, E=64, K=8, I=64, P=8, block_m=16)),
    # the permutation's two index passes at their limit (64 blocks of 256 tokens x 256 local
    # experts = 16384 count values; the last block sums 63 x 256 of them), and one block past
    # it (the three-pass form)
    ("two_pass_limit", dict(seed=16, T=16384, H=64, E=256, K=4, I=64, P=8, block_m=16)),
    ("three_pass", dict(seed=17, T=16385, H=64, E=256, K=4, I=64, P=8, block_m=16)),
    # the two-pass form with the largest top-k (16 entries per token in one place pass)
    ("two_pass_k16", dict(seed=18, T=16384, H=64, E=64, K=16, I=64, P=8, block_m=16)),
    # decode-sized layers (a handful of rows per expert): experts of 1..32 rows, of 33..64
    # rows, exactly 64 rows (4 experts taking every token), 65 rows, and wider H and I
    ("decode_small", dict(seed=19, T=64, H=256, E=32, K=4, I=192, P=4, block_m=16)),
    ("decode_two_blocks", dict(seed=20, T=64, H=128, E=6, K=4, I=128, P=2, block_m=32)),
    ("decode_64_rows", dict(seed=21, T=64, H=128, E=4, K=4, I=64, P=2, block_m=64)),
    ("decode_65_rows", dict(seed=22, T=65, H=128, E=4, K=4, I=64, P=2, block_m=64)),
    ("decode_wide", dict(seed=23, T=16, H=320, E=16, K=4, I=448, P=4, block_m=16)),
])
def test_small_layers_full(name, kw):
    c = random_case(**kw)
    _announce(f"small {name} {kw}")
    print(_full_check(c, run_gpu(c), oracle_index(c)))


def test_equal_logits_ties():
    """All-equal logits: every token picks experts 0..K-1 (lowest ids), weights 1/K."""
    c = random_case(seed=10, T=64, H=64, E=8, K=3, I=64, P=4)
    c.logits[:] = 0.0
    layer = run_gpu(c)
    ref = oracle_index(c)
    assert np.all(ref.ids == np.arange(3)[None, :])
    _full_check(c, layer, ref)


def test_olmoe_first_tokens_full():
    c = workload_case("olmoe_shaped", 1.2, T=512)
    _announce("olmoe_shaped s=1.2, first 512 tokens, every row")
    print(_full_check(c, run_gpu(c), oracle_index(c)))


def test_repeat_runs_are_bit_identical():
    """Race check: the whole path twice on the same inputs gives the same bits everywhere."""
    c = workload_case("qwen3_30b_a3b_shaped", 1.5, T=2048)
    a = run_gpu(c)
    b = run_gpu(c)
    for name in ("topk_ids", "topk_w", "counts", "offsets", "entry_pos", "q", "n_moves",
                 "n_blocks", "out"):
        assert torch.equal(getattr(a, name), getattr(b, name)), name
    # only the first n_moves / n_blocks entries of these tables are written
    nm, nb = int(a.n_moves.item()), int(a.n_blocks.item())
    assert torch.equal(a.moves[:nm], b.moves[:nm]), "moves"
    assert torch.equal(a.blocks[:nb], b.blocks[:nb]), "blocks"
    rows = int(host(a.offsets)[-1])
    assert torch.equal(a.row_token[:rows], b.row_token[:rows]), "row_token"
    valid = torch.nonzero(a.row_token[:rows] >= 0).squeeze(1)  # padding rows are never written
    for name in ("xp", "act", "yp"):
        assert torch.equal(getattr(a, name)[valid], getattr(b, name)[valid]), name


def test_graph_replay_matches_eager():
    """The whole path captured as one HIP graph: replays on new logits written in place, with
    eager calls and synchronisations between them, reproduce the eager results bit for bit."""
    c = workload_case("olmoe_shaped", 1.2, T=1024)
    _announce("graph replay vs eager, olmoe_shaped first 1024 tokens")
    layer = run_gpu(c)
    logits, x, W1, W2 = layer._inputs
    graph = layer.capture(logits, x, W1, W2)
    names = ("topk_ids", "topk_w", "counts", "offsets", "entry_pos", "q", "n_moves", "n_blocks",
             "out")
    w = inputs.WORKLOADS["olmoe_shaped"]
    for skew in (0.0, 1.2, 0.5):
        logits.copy_(torch.from_numpy(inputs.make_logits(w, skew)[: c.T].copy()))
        layer.forward(logits, x, W1, W2)  # eager reference
        torch.cuda.synchronize()
        ref = {n: getattr(layer, n).clone() for n in names}
        nb = int(ref["n_blocks"].item())
        ref_blocks = layer.blocks[:nb].clone()
        rows = int(ref["offsets"][-1].item())
        valid = torch.nonzero(layer.row_token[:rows] >= 0).squeeze(1)
        ref_yp = layer.yp[valid].clone()
        for n in ("out", "yp", "act", "topk_ids", "topk_w", "entry_pos"):
            getattr(layer, n).zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for n in names:
            assert torch.equal(getattr(layer, n), ref[n]), (skew, n)
        assert torch.equal(layer.blocks[:nb], ref_blocks), (skew, "blocks")
        assert torch.equal(layer.yp[valid], ref_yp), (skew, "yp")
    del graph


@pytest.mark.parametrize("name,kw,drop", [
    # every other block: each expert's blocks no longer cover one row range (table in LDS)
    ("every_other", dict(seed=1, T=600, H=128, E=12, K=3, I=192, P=4, block_m=32), 2),
    # a decode-sized layer (experts of about 48 rows in 16-row blocks) with every third block
    # left out: experts of two row runs, paired into tiles of two halves
    ("decode_runs", dict(seed=24, T=64, H=128, E=4, K=3, I=128, P=2, block_m=16), 3),
    # a quarter of 4130 blocks dropped: 3098 blocks, walked in global memory
    ("many_blocks", dict(seed=15, T=8192, H=64, E=64, K=8, I=64, P=8, block_m=16), 4),
])
def test_ffn_arbitrary_block_table(name, kw, drop):
    """moe_expert_ffn on a block table that is not a moe_plan table (some blocks left out):
    covered rows against the oracle, the other rows untouched."""
    _announce(f"ffn on a partial block table: {name}")
    c = random_case(**kw)
    layer = run_gpu(c)
    ref = oracle_index(c)
    nb = int(layer.n_blocks.item())
    full = host(layer.blocks[:nb])
    keep = np.array([i % drop != drop - 1 for i in range(nb)])
    sub = np.ascontiguousarray(full[keep])
    dev = layer.blocks.device
    sub_buf = torch.zeros_like(layer.blocks)
    sub_buf[: len(sub)] = torch.from_numpy(sub).to(dev)
    n_sub = torch.tensor([len(sub)], dtype=torch.int32, device=dev)
    act = torch.zeros_like(layer.act)
    yp = torch.zeros_like(layer.yp)
    _, _, W1, W2 = layer._inputs
    binding.moe_expert_ffn(layer.xp, W1, W2, sub_buf, n_sub, act, yp, layer.ffn_workspace)
    torch.cuda.synchronize()
    x = inputs.as_oracle_array(c.x)
    _, _, _, xp = oracle.permute(ref.ids, ref.counts, c.E, c.begin, c.stride, c.n_local,
                                 c.block_m, x)
    act_o, yp_o = oracle.ffn_blocks(xp, inputs.as_oracle_array(c.W1),
                                    inputs.as_oracle_array(c.W2), sub)
    covered = np.zeros(xp.shape[0], bool)
    for _, _, first, rows in sub:
        covered[first:first + rows] = True
    g_act, g_yp = host(act)[: len(covered)], host(yp)[: len(covered)]
    e_act = rel_frob(to_f64(g_act[covered]), to_f64(act_o[covered]))
    e_yp = rel_frob(to_f64(g_yp[covered]), to_f64(yp_o[covered]))
    assert e_act <= c.tol and e_yp <= c.tol, (e_act, e_yp)
    assert not to_f64(g_act[~covered]).any() and not to_f64(g_yp[~covered]).any(), "untouched"


@pytest.mark.parametrize("name,kw", [
    ("lds_walk", dict(seed=1, T=600, H=128, E=12, K=3, I=192, P=4, block_m=32)),
    ("global_walk", dict(seed=15, T=8192, H=64, E=64, K=8, I=64, P=8, block_m=16)),
    ("float32", dict(seed=3, T=200, H=64, E=8, K=2, I=128, P=4, block_m=32,
                     dtype=torch.float32)),
])
def test_ffn_checks_the_block_table(name, kw):
    """A table with bad entries (expert outside [0, E_loc), rows outside [0, 256], a row range
    outside [0, max_rows), n_blocks past max_blocks): the FFN skips exactly those entries and
    reports their bits in the workspace's error word; every intact block is computed as the
    oracle computes it and no other row is written.  A negative n_blocks computes nothing."""
    _announce(f"ffn on a table with bad entries: {name}")
    c = random_case(**kw)
    layer = run_gpu(c)
    assert layer.ffn_error() == 0
    ref = oracle_index(c)
    nb = int(layer.n_blocks.item())
    tab = host(layer.blocks[:nb]).copy()
    max_rows, E_loc = layer.max_rows, c.n_local
    bad = {1: (1, E_loc + 3), 3: (1, -1), 5: (3, 300), 7: (3, -4), 9: (2, max_rows - 3),
           11: (2, -64)}
    assert nb > max(bad) + 2
    for i, (field, v) in bad.items():
        tab[i, field] = v
    keep = np.array([i not in bad for i in range(nb)])
    dev = layer.blocks.device
    buf = torch.zeros_like(layer.blocks)  # entries past nb: (0, 0, 0, 0), 0 rows: skipped
    buf[:nb] = torch.from_numpy(tab).to(dev)
    n_over = torch.tensor([layer.max_blocks + 5], dtype=torch.int32, device=dev)
    act = torch.zeros_like(layer.act)
    yp = torch.zeros_like(layer.yp)
    _, _, W1, W2 = layer._inputs
    binding.moe_expert_ffn(layer.xp, W1, W2, buf, n_over, act, yp, layer.ffn_workspace)
    torch.cuda.synchronize()
    err = int(layer.ffn_workspace[binding.FFN_WS_ERR].item())
    assert err == (binding.FFN_ERR_EXPERT | binding.FFN_ERR_ROWS | binding.FFN_ERR_RANGE |
                   binding.FFN_ERR_COUNT), err
    sub = np.ascontiguousarray(host(layer.blocks[:nb])[keep])
    x = inputs.as_oracle_array(c.x)
    _, _, _, xp = oracle.permute(ref.ids, ref.counts, c.E, c.begin, c.stride, c.n_local,
                                 c.block_m, x)
    act_o, yp_o = oracle.ffn_blocks(xp, inputs.as_oracle_array(c.W1),
                                    inputs.as_oracle_array(c.W2), sub)
    covered = np.zeros(xp.shape[0], bool)
    for _, _, first, rows in sub:
        covered[first:first + rows] = True
    g_act, g_yp = host(act), host(yp)
    n = len(covered)
    e_act = rel_frob(to_f64(g_act[:n][covered]), to_f64(act_o[covered]))
    e_yp = rel_frob(to_f64(g_yp[:n][covered]), to_f64(yp_o[covered]))
    assert e_act <= c.tol and e_yp <= c.tol, (e_act, e_yp)
    assert not to_f64(g_act[:n][~covered]).any() and not to_f64(g_yp[:n][~covered]).any()
    assert not to_f64(g_act[n:]).any() and not to_f64(g_yp[n:]).any(), "rows past the segments"
    # a negative block count: nothing computed, the count bit set
    act.zero_()
    n_neg = torch.tensor([-3], dtype=torch.int32, device=dev)
    binding.moe_expert_ffn(layer.xp, W1, W2, layer.blocks, n_neg, act, yp, layer.ffn_workspace)
    torch.cuda.synchronize()
    assert int(layer.ffn_workspace[binding.FFN_WS_ERR].item()) == binding.FFN_ERR_COUNT
    assert torch.count_nonzero(act) == 0
    # and the plan's own table again: error word back to 0
    binding.moe_expert_ffn(layer.xp, W1, W2, layer.blocks, layer.n_blocks, act, yp,
                           layer.ffn_workspace)
    assert layer.ffn_error() == 0


# ------------------------------------------------- gather-on-load expert FFN ---

GATHER_CASES = [
    ("ragged", dict(seed=1, T=37, H=128, E=12, K=3, I=192, P=4, block_m=32)),
    ("subset_local", dict(seed=4, T=300, H=128, E=16, K=3, I=128, P=2, E_loc=4, begin=1,
                          stride=3, block_m=64)),
    ("hot_experts", dict(seed=5, T=700, H=64, E=8, K=2, I=64, P=4,
                         logit_bias=[30, 29, 0, 0, 0, 0, 0, 0])),
    ("wide_k", dict(seed=8, T=80, H=64, E=256, K=16, I=64, P=16, block_m=16)),
    ("f32_ragged", dict(seed=9, T=50, H=32, E=6, K=2, I=48, P=3, dtype=torch.float32,
                        block_m=16)),
    ("many_blocks", dict(seed=15, T=8192, H=64, E=64, K=8, I=64, P=8, block_m=16)),
]


def _gather_vs_materialised(c):
    """The gather path against the materialising path (bit for bit) and the oracle."""
    mat = run_gpu(c)
    gat = run_gpu(c, gather=True)
    ref = oracle_index(c)
    check_index_parity(gat, ref)
    assert gat.xp is None
    rows = int(host(mat.offsets)[-1])
    valid = torch.nonzero(mat.row_token[:rows] >= 0).squeeze(1)
    for name in ("act", "yp"):
        assert torch.equal(getattr(gat, name)[valid], getattr(mat, name)[valid]), name
    assert torch.equal(gat.out, mat.out), "out"
    return mat, gat, ref


@pytest.mark.parametrize("name,kw", GATHER_CASES)
def test_gather_small_layers(name, kw):
    c = random_case(**kw)
    _announce(f"gather {name} {kw}")
    _, gat, ref = _gather_vs_materialised(c)
    # and against the oracle on every row
    x = inputs.as_oracle_array(c.x)
    _, _, _, xp = oracle.permute(ref.ids, ref.counts, c.E, c.begin, c.stride, c.n_local,
                                 c.block_m, x)
    valid = ref.row_token >= 0
    act, yp = oracle.ffn_blocks(xp, inputs.as_oracle_array(c.W1), inputs.as_oracle_array(c.W2),
                                ref.blocks)
    e_act = rel_frob(to_f64(host(gat.act)[: len(valid)][valid]), to_f64(act[valid]))
    e_out = rel_frob(to_f64(host(gat.out)), to_f64(oracle.combine(yp, ref.w, ref.entry_pos,
                                                                   c.T, c.K)))
    assert e_act <= c.tol and e_out <= c.tol, (e_act, e_out)


# ------------------------------------------------------ full-size layers: sampled ---

FULL = [(n, s) for n in ("olmoe_shaped", "qwen3_30b_a3b_shaped", "gpt_oss_120b_shaped",
                         "gpt_oss_120b_decode", "deepseek_v3_share")
        for s in inputs.WORKLOADS[n].skews]

_weights_cache = {}


def _weights(name):
    w = inputs.WORKLOADS[name]
    key = (w.seed_id, w.H, w.I, w.n_local)
    if key not in _weights_cache:
        _weights_cache.clear()
        gc.collect()
        _weights_cache[key] = inputs.make_weights(w, threads=16)
    return _weights_cache[key]


@pytest.mark.parametrize("name,skew", FULL)
def test_full_size_sampled(name, skew):
    """At the full layer size, on both FFN input paths: index outputs bit-exact on every
    entry; the benchmarked gather-on-load path bit-identical to the materialising path on
    every valid row of act and yp and on every token of out; and the gather path's act / yp on
    sampled rows (one per 32-row block of every 128-row piece of every expert, block edges,
    random rows, and every row behind the sampled tokens) and out on sampled tokens against
    the oracle, which computes those one by one, with per-row and per-element bounds beside
    the layer-wide relative Frobenius bar."""
    _announce(f"full {name} skew={skew}")
    c = workload_case(name, skew, weights=_weights(name))
    mat = run_gpu(c)
    ref = oracle_index(c)
    check_index_parity(mat, ref)
    check_xp(mat, c, ref)
    layer = run_gpu(c, gather=True)
    check_index_parity(layer, ref)
    rows_pad = int(ref.offsets[-1])
    valid = torch.nonzero(mat.row_token[:rows_pad] >= 0).squeeze(1)
    for nm in ("act", "yp"):
        assert torch.equal(getattr(layer, nm)[valid], getattr(mat, nm)[valid]), ("gather vs xp", nm)
    assert torch.equal(layer.out, mat.out), ("gather vs xp", "out")
    del mat
    torch.cuda.empty_cache()

    # sampled tokens (with at least one local entry) + sampled rows
    rng = np.random.default_rng(1)
    ep = ref.entry_pos.reshape(c.T, c.K)
    has_local = np.nonzero((ep >= 0).any(1))[0]
    toks = np.sort(rng.choice(has_local, size=min(16, len(has_local)), replace=False))
    tok_rows = ep[toks][ep[toks] >= 0]
    rows = np.unique(np.concatenate([tile_rows(ref), sample_rows(ref, 48), tok_rows]))
    ex = row_experts(ref.blocks, rows)
    x_rows = inputs.as_oracle_array(c.x)[ref.row_token[rows]]
    act, yp = oracle.ffn_rows(x_rows, inputs.as_oracle_array(c.W1), inputs.as_oracle_array(c.W2),
                              np.arange(len(rows), dtype=np.int32), ex.astype(np.int32))
    rows_t = torch.from_numpy(rows).to(layer.act.device)
    g_act, g_yp = to_f64(host(layer.act[rows_t])), to_f64(host(layer.yp[rows_t]))
    e_act = rel_frob(g_act, to_f64(act))
    e_yp = rel_frob(g_yp, to_f64(yp))
    s_act = check_rows(g_act, to_f64(act), "act")
    # yp: FC2's input rows (act) may already differ by a rounding flip; propagate that exactly
    d_act = np.abs(g_act - to_f64(act))
    prop_yp = np.zeros_like(g_yp)
    for l in np.unique(ex):
        m = ex == l
        if d_act[m].any():
            prop_yp[m] = d_act[m] @ np.abs(c.W2[int(l)].double().numpy()).T
    s_yp = check_rows(g_yp, to_f64(yp), "yp", extra=prop_yp)
    # end to end on the sampled tokens: oracle combine over the oracle's yp rows
    remap = {int(r): j for j, r in enumerate(rows)}
    ep_t = np.array([[remap[int(p)] if p >= 0 else -1 for p in ep[t]] for t in toks], np.int32)
    out_ref = oracle.combine(yp, ref.w[toks], ep_t, len(toks), c.K)
    toks_t = torch.from_numpy(toks).to(layer.out.device)
    g_out = to_f64(host(layer.out[toks_t]))
    e_out = rel_frob(g_out, to_f64(out_ref))
    # out: the combine's inputs (yp rows) may differ by what the check above allowed
    d_yp = np.abs(g_yp - to_f64(yp))
    prop_out = np.zeros_like(g_out)
    for j, t in enumerate(toks):
        for k in range(c.K):
            if ep_t[j, k] >= 0:
                prop_out[j] += abs(float(ref.w[t, k])) * d_yp[ep_t[j, k]]
    s_out = check_rows(g_out, to_f64(out_ref), "out (oracle chain)", extra=prop_out)
    # the combine alone, element by element: the oracle's combine over the GPU's own yp rows
    out_own = oracle.combine(host(layer.yp[rows_t]), ref.w[toks], ep_t, len(toks), c.K)
    check_rows(g_out, to_f64(out_own), "out (combine of the GPU's yp)", rms_frac=1e-4)
    # tokens with no local entry are exactly zero
    none_local = np.nonzero(~(ep >= 0).any(1))[0][:64]
    if len(none_local):
        assert torch.count_nonzero(layer.out[torch.from_numpy(none_local).to(layer.out.device)]) == 0
    print(f"rows={len(rows)} tokens={len(toks)} act={e_act:.2e} yp={e_yp:.2e} out={e_out:.2e} "
          f"row/elem act={s_act} yp={s_yp} out={s_out}")
    assert e_act <= c.tol and e_yp <= c.tol and e_out <= c.tol
    del layer
    torch.cuda.empty_cache()
