"""GPU parity of the direct rows (moe_expert_ffn_fc2_direct + moe_combine_multi): the down GEMM
stores the weighted output row of every token with exactly one local entry and the combine skips
those tokens.  `out` must be bit-identical to moe_expert_ffn_fc2 followed by moe_combine on the
same FC1 output (which the other parity tests hold to the oracle), and end to end within the
oracle's tolerance; the row table the call writes is index work and is compared bit for bit
with one computed on the host from entry_pos; rows of the other tokens are stored to yp as
before."""
import numpy as np
import pytest
import torch

import oracle
from mixture_experts_routed_router_amd import binding, inputs
from parity_helpers import (host, oracle_index, random_case, rel_frob, run_gpu, to_f64,
                            workload_case)

pytestmark = pytest.mark.gpu


def _announce(msg):
    print(f"\n[direct] {msg}", flush=True)


def _host_direct_table(entry_pos: np.ndarray, row_token: np.ndarray, T: int, K: int,
                       w: np.ndarray, max_rows: int):
    """Row p -> its token when that token's only local entry is row p, else -1; its weight."""
    ep = entry_pos.reshape(T, K)
    n_local = (ep >= 0).sum(axis=1)
    tok = np.full(max_rows, -1, np.int32)
    wbits = np.zeros(max_rows, np.int32)
    for t in np.nonzero(n_local == 1)[0]:
        k = int(np.nonzero(ep[t] >= 0)[0][0])
        p = int(ep[t, k])
        if row_token[p] == t:
            tok[p] = t
            wbits[p] = np.float32(w[t, k]).view(np.int32)
    return tok, wbits, n_local


def _check_direct(c, layer, oracle_chain=True):
    """out of the direct path against the plain path on the same act; the row table; yp of the
    other tokens' rows; optionally out against the oracle's whole chain."""
    _, _, W1, W2 = layer._inputs
    T, K, max_rows = c.T, c.K, layer.max_rows
    yp2 = torch.zeros_like(layer.yp)
    out2 = torch.zeros_like(layer.out)
    binding.moe_expert_ffn_fc2(layer.act, W2, layer.blocks, layer.n_blocks, yp2,
                               layer.ffn_workspace)
    binding.moe_combine(yp2, layer.topk_w, layer.entry_pos, out2)
    torch.cuda.synchronize()
    assert torch.equal(layer.out, out2), "out: direct rows + combine_multi vs fc2 + combine"
    ep, rt = host(layer.entry_pos), host(layer.row_token)
    tok, wbits, n_local = _host_direct_table(ep, rt, T, K, host(layer.topk_w), max_rows)
    rd = host(layer.row_direct)
    assert np.array_equal(rd[:max_rows], tok), "row table: tokens"
    assert np.array_equal(rd[max_rows:][tok >= 0], wbits[tok >= 0]), "row table: weights"
    assert not rd[max_rows:][tok < 0].any(), "row table: weight words of other rows"
    rows = int(host(layer.offsets)[-1])
    other = np.nonzero((rt[:rows] >= 0) & (tok[:rows] < 0))[0]
    idx = torch.from_numpy(other).to(layer.yp.device)
    assert torch.equal(layer.yp[idx], yp2[idx]), "yp rows of tokens with 0 or >= 2 entries"
    errs = dict(direct_tokens=int((n_local == 1).sum()), tokens=T)
    if oracle_chain:
        ref = oracle_index(c)
        x = inputs.as_oracle_array(c.x)
        _, _, _, xp = oracle.permute(ref.ids, ref.counts, c.E, c.begin, c.stride, c.n_local,
                                     c.block_m, x)
        _, yp_o = oracle.ffn_blocks(xp, inputs.as_oracle_array(c.W1),
                                    inputs.as_oracle_array(c.W2), ref.blocks)
        out_o = oracle.combine(yp_o, ref.w, ref.entry_pos, T, K)
        errs["chain"] = rel_frob(to_f64(host(layer.out)), to_f64(out_o))
        assert errs["chain"] <= c.tol, errs
    return errs


@pytest.mark.parametrize("name,kw", [
    # local experts a strided subset: tokens with 0, 1, 2 and 3 local entries
    ("subset_local", dict(seed=4, T=300, H=128, E=16, K=3, I=128, P=2, E_loc=4, begin=1,
                          stride=3, block_m=64)),
    # one GPU's share of a 64-expert top-8 layer (8 local experts, ids = 5 mod 8)
    ("share_of_64", dict(seed=31, T=1000, H=256, E=64, K=8, I=192, P=4, E_loc=8, begin=5,
                         stride=8, block_m=32)),
    # top-1 over a local subset: every token with a local entry is a one-entry token
    ("k1_subset", dict(seed=32, T=700, H=128, E=32, K=1, I=128, P=2, E_loc=8, begin=0,
                       stride=4, block_m=16)),
    # every expert local: no one-entry token (the combine computes every row)
    ("all_local", dict(seed=1, T=37, H=128, E=12, K=3, I=192, P=4, block_m=32)),
    # decode-sized experts (64-row GEMM items) on a subset
    ("decode_subset", dict(seed=33, T=64, H=256, E=32, K=4, I=192, P=2, E_loc=8, begin=2,
                           stride=4, block_m=16)),
    ("single_token", dict(seed=34, T=1, H=64, E=8, K=2, I=64, P=2, E_loc=2, begin=0,
                          stride=4)),
    # float32 layer: the direct rows of the float32 down GEMM
    ("f32_subset", dict(seed=35, T=120, H=64, E=12, K=3, I=96, P=3, E_loc=6, begin=0, stride=2,
                        block_m=16, dtype=torch.float32)),
])
@pytest.mark.parametrize("gather", [False, True])
def test_direct_rows_small(name, kw, gather):
    c = random_case(**kw)
    _announce(f"{name} gather={gather} {kw}")
    print(_check_direct(c, run_gpu(c, gather=gather, direct=True)))


def test_direct_rows_tiny_f32():
    c = workload_case("tiny_f32", 1.0)
    _announce("tiny_f32 s=1")
    print(_check_direct(c, run_gpu(c, direct=True)))


@pytest.mark.parametrize("skew", [1.0, 0.0])
def test_direct_rows_deepseek_v3_share(skew):
    """The full-size layer the bench times (gather-on-load FC1), both skews: out bit-identical
    to the plain down GEMM + combine on the same act (the plain path is held to the oracle at
    full size by the other parity tests)."""
    c = workload_case("deepseek_v3_share", skew)
    _announce(f"deepseek_v3_share s={skew}, full size, gather")
    print(_check_direct(c, run_gpu(c, gather=True, direct=True), oracle_chain=False))


def test_direct_rows_graph_replay():
    """The direct path captured as one HIP graph: replays on new logits reproduce the eager
    results bit for bit."""
    c = random_case(seed=31, T=1000, H=256, E=64, K=8, I=192, P=4, E_loc=8, begin=5, stride=8,
                    block_m=32)
    _announce("graph replay of the direct path")
    layer = run_gpu(c, gather=True, direct=True)
    logits, x, W1, W2 = layer._inputs
    graph = layer.capture(logits, x, W1, W2)
    rng = np.random.default_rng(36)
    for _ in range(3):
        logits.copy_(torch.from_numpy(rng.standard_normal((c.T, c.E), dtype=np.float32)))
        layer.forward(logits, x, W1, W2)
        torch.cuda.synchronize()
        ref_out = layer.out.clone()
        layer.out.zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(layer.out, ref_out)
    del graph


@pytest.mark.parametrize("name,kw", [
    ("share_of_64", dict(seed=31, T=1000, H=256, E=64, K=8, I=256, P=4, E_loc=8, begin=5,
                         stride=8, block_m=32)),
    ("k1_subset", dict(seed=32, T=700, H=128, E=32, K=1, I=128, P=2, E_loc=8, begin=0,
                       stride=4, block_m=16)),
    ("decode_subset", dict(seed=33, T=64, H=256, E=32, K=4, I=192, P=2, E_loc=8, begin=2,
                           stride=4, block_m=16)),
])
def test_direct_rows_mx(name, kw):
    """The MX down GEMM with direct rows (moe_expert_ffn_mx_fc2_direct) + moe_combine_multi:
    out bit-identical to moe_expert_ffn_mx_fc2 + moe_combine on the same MXFP8 activation, the
    row table as the host computes it, yp of the other tokens' rows unchanged."""
    c = random_case(**kw)
    _announce(f"mx {name} {kw}")
    dev = "cuda"
    layer = binding.RoutedExperts(c.T, c.H, c.E, c.K, c.I, c.P, dtype=c.dtype, E_loc=c.n_local,
                                  expert_begin=c.begin, expert_stride=c.stride,
                                  block_m=c.block_m, device=dev, precision="mx", direct=True)
    logits = torch.from_numpy(c.logits).to(dev)
    x = c.x.to(dev)
    (w1q, w1s), (w2q, w2s) = binding.mx_quantize_weights(c.W1.to(dev), c.W2.to(dev))
    layer.forward(logits, x, (w1q, w1s), (w2q, w2s))
    yp2 = torch.zeros_like(layer.yp)
    out2 = torch.zeros_like(layer.out)
    binding.moe_expert_ffn_mx_fc2(layer.actq, layer.acts, w2q, w2s, layer.blocks, layer.n_blocks,
                                  yp2, layer.ffn_workspace)
    binding.moe_combine(yp2, layer.topk_w, layer.entry_pos, out2)
    torch.cuda.synchronize()
    assert torch.equal(layer.out, out2), "out: MX direct rows + combine_multi vs MX fc2 + combine"
    T, K, max_rows = c.T, c.K, layer.max_rows
    ep, rt = host(layer.entry_pos), host(layer.row_token)
    tok, wbits, n_local = _host_direct_table(ep, rt, T, K, host(layer.topk_w), max_rows)
    rd = host(layer.row_direct)
    assert np.array_equal(rd[:max_rows], tok), "row table: tokens"
    assert np.array_equal(rd[max_rows:][tok >= 0], wbits[tok >= 0]), "row table: weights"
    rows = int(host(layer.offsets)[-1])
    other = torch.from_numpy(np.nonzero((rt[:rows] >= 0) & (tok[:rows] < 0))[0]).to(dev)
    assert torch.equal(layer.yp[other], yp2[other]), "yp rows of tokens with 0 or >= 2 entries"
    print(dict(direct_tokens=int((n_local == 1).sum()), tokens=T))


def test_direct_rows_mx_deepseek_v3_share():
    """The MX path of the full-size DeepSeek-V3 share (skew 1) with direct rows: out bit-identical
    to the plain MX down GEMM + combine on the same activation."""
    c = workload_case("deepseek_v3_share", 1.0)
    _announce("mx deepseek_v3_share s=1, full size")
    dev = "cuda"
    layer = binding.RoutedExperts(c.T, c.H, c.E, c.K, c.I, c.P, dtype=c.dtype, E_loc=c.n_local,
                                  expert_begin=c.begin, expert_stride=c.stride,
                                  block_m=c.block_m, device=dev, precision="mx", direct=True)
    logits = torch.from_numpy(c.logits).to(dev)
    x = c.x.to(dev)
    (w1q, w1s), (w2q, w2s) = binding.mx_quantize_weights(c.W1.to(dev), c.W2.to(dev))
    layer.forward(logits, x, (w1q, w1s), (w2q, w2s))
    yp2 = torch.zeros_like(layer.yp)
    out2 = torch.zeros_like(layer.out)
    binding.moe_expert_ffn_mx_fc2(layer.actq, layer.acts, w2q, w2s, layer.blocks, layer.n_blocks,
                                  yp2, layer.ffn_workspace)
    binding.moe_combine(yp2, layer.topk_w, layer.entry_pos, out2)
    torch.cuda.synchronize()
    assert torch.equal(layer.out, out2)


def test_direct_rows_partial_block_table():
    """moe_expert_ffn_fc2_direct on a block table with every third block left out: covered rows
    of one-entry tokens land in out (bit for bit the one-entry combine of the plain FC2's row),
    the other covered rows in yp as the plain FC2 stores them, and nothing else is written."""
    c = random_case(seed=31, T=1000, H=256, E=64, K=8, I=192, P=4, E_loc=8, begin=5, stride=8,
                    block_m=32)
    _announce("direct rows on a partial block table")
    layer = run_gpu(c, direct=True)
    _, _, W1, W2 = layer._inputs
    nb = int(layer.n_blocks.item())
    full = host(layer.blocks[:nb])
    sub = np.ascontiguousarray(full[np.array([i % 3 != 2 for i in range(nb)])])
    dev = layer.blocks.device
    sub_buf = torch.zeros_like(layer.blocks)
    sub_buf[: len(sub)] = torch.from_numpy(sub).to(dev)
    n_sub = torch.tensor([len(sub)], dtype=torch.int32, device=dev)
    act = torch.zeros_like(layer.act)
    binding.moe_expert_ffn_fc1(layer.xp, W1, sub_buf, n_sub, act, layer.ffn_workspace)
    yp_d, out_d = torch.zeros_like(layer.yp), torch.zeros_like(layer.out)
    binding.moe_expert_ffn_fc2_direct(act, W2, sub_buf, n_sub, yp_d, layer.row_token,
                                      layer.entry_pos, layer.topk_w, out_d, layer.row_direct,
                                      layer.ffn_workspace)
    yp_p = torch.zeros_like(layer.yp)
    binding.moe_expert_ffn_fc2(act, W2, sub_buf, n_sub, yp_p, layer.ffn_workspace)
    out_one = torch.zeros_like(layer.out)  # the one-entry combine of every plain row
    binding.moe_combine(yp_p, layer.topk_w, layer.entry_pos, out_one)
    torch.cuda.synchronize()
    covered = np.zeros(layer.max_rows, bool)
    for _, _, first, rows in sub:
        covered[first:first + rows] = True
    tok, _, _ = _host_direct_table(host(layer.entry_pos), host(layer.row_token), c.T, c.K,
                                   host(layer.topk_w), layer.max_rows)
    direct_rows = np.nonzero(covered & (tok >= 0))[0]
    other_rows = np.nonzero(covered & (tok < 0))[0]
    assert len(direct_rows) > 0 and len(other_rows) > 0
    toks = torch.from_numpy(tok[direct_rows].astype(np.int64)).to(dev)
    assert torch.equal(out_d[toks], out_one[toks]), "direct rows: out"
    written = torch.zeros(c.T, dtype=torch.bool, device=dev)
    written[toks] = True
    assert not out_d[~written].any(), "out rows of other tokens untouched"
    oth = torch.from_numpy(other_rows).to(dev)
    assert torch.equal(yp_d[oth], yp_p[oth]), "other covered rows: yp"
    mask = torch.from_numpy(covered & (tok < 0)).to(dev)
    assert not yp_d[~mask].any(), "yp rows not stored by the call untouched"
