"""GPU parity of the MX expert FFN (moe_expert_ffn_mx: MXFP4 weights, MXFP8 activations, through
the C ABI) against the CPU oracle (oracle.ffn_mx_rows, float64 over the MX values).

Inputs are quantized twice, independently: on the GPU (moe_mx_quantize) for the HIP path and by
the oracle (oracle.mx_quantize) for the oracle; the codes are compared bit for bit.  Then:
  act  (MXFP8 codes + E8M0 scales): the HIP path computes the activation in float32, the
       oracle in float64, and both quantize it with the same rule, so a code can differ where
       the value lies within float32 rounding of a rounding midpoint (or a block maximum within
       it of a power of two).  Bar: at most 1 code in 1000 differs, and the dequantized
       activations agree to a relative Frobenius error of 2e-3.
  yp   (bf16): against the oracle's yp, relative Frobenius error <= 5e-3 (the bf16 bar); and
       against FC2 recomputed in float64 from the HIP path's own activation codes (oracle
       dequantization, a matmul), <= 1e-3: float32 against float64 accumulation of the same
       MX products differs only by bf16 rounding flips.
"""
import gc

import numpy as np
import pytest
import torch

import oracle
from mixture_experts_routed_router_amd import binding, inputs
from parity_helpers import (BF16_TOL, host, oracle_index, random_case, rel_frob, row_experts,
                            run_gpu, sample_rows, workload_case)

pytestmark = pytest.mark.gpu

FP8, FP4 = binding.MOE_MX_FP8, binding.MOE_MX_FP4
ACT_TOL = 2e-3        # dequantized MXFP8 activation, relative Frobenius
ACT_CODE_DIFF = 1e-3  # largest fraction of activation codes that may differ
FC2_TOL = 1e-3        # yp against float64 FC2 over the HIP path's own activation codes


def _announce(msg):
    print(f"\n[mx-ffn] {msg}", flush=True)


def _quantize_gpu(t, fmt):
    cols = t.shape[-1]
    codes = torch.zeros(*t.shape[:-1], cols if fmt == FP8 else cols // 2, dtype=torch.uint8,
                        device=t.device)
    scales = torch.zeros(*t.shape[:-1], binding.moe_mx_scale_pitch(cols), dtype=torch.uint8,
                         device=t.device)
    binding.moe_mx_quantize(t, fmt, codes, scales)
    return codes, scales


class MxRun:
    """The MX FFN on a layer's block table (route / permute / plan from the bf16 run)."""

    def __init__(self, layer, c, gather, blocks=None, n_blocks=None):
        _, x, W1, W2 = layer._inputs
        self.H, self.I = c.H, c.I
        self.w1q, self.w1s = _quantize_gpu(W1, FP4)
        self.w2q, self.w2s = _quantize_gpu(W2, FP4)
        self.gather = gather
        src = x if gather else layer.xp
        self.xq, self.xs = _quantize_gpu(src, FP8)
        rows = layer.act.shape[0]
        dev = x.device
        self.actq = torch.zeros(rows, c.I, dtype=torch.uint8, device=dev)
        self.acts = torch.zeros(rows, binding.moe_mx_scale_pitch(c.I), dtype=torch.uint8, device=dev)
        self.yp = torch.zeros(rows, c.H, dtype=torch.bfloat16, device=dev)
        self.blocks = layer.blocks if blocks is None else blocks
        self.n_blocks = layer.n_blocks if n_blocks is None else n_blocks
        self.layer = layer
        self.run()

    def run(self):
        binding.moe_expert_ffn_mx(self.xq, self.xs, self.layer.row_token if self.gather else None,
                                  self.w1q, self.w1s, self.w2q, self.w2s, self.blocks,
                                  self.n_blocks, self.actq, self.acts, self.yp,
                                  self.layer.ffn_workspace)
        torch.cuda.synchronize()


def _check_rows(c, mx: MxRun, ref, rows, label):
    """Rows (permuted positions) of the MX run against the oracle."""
    H, I = c.H, c.I
    nbh, nbi = H // 32, I // 32
    x_o = inputs.as_oracle_array(c.x)
    tok = ref.row_token[rows]
    assert (tok >= 0).all()
    ex = row_experts(ref.blocks, rows)
    uniq, ex_local = np.unique(ex, return_inverse=True)
    # the oracle's own quantization of the inputs it needs
    xq_o, xs_o = oracle.mx_quantize(x_o[tok], FP8)
    W1o = inputs.as_oracle_array(c.W1[torch.from_numpy(uniq)])
    W2o = inputs.as_oracle_array(c.W2[torch.from_numpy(uniq)])
    w1q_o, w1s_o = oracle.mx_quantize(W1o.reshape(-1, H), FP4)
    w2q_o, w2s_o = oracle.mx_quantize(W2o.reshape(-1, I), FP4)
    # the HIP path's quantized inputs are the same codes
    u_t = torch.from_numpy(uniq).to(mx.w1q.device)
    assert np.array_equal(host(mx.w1q[u_t]).reshape(-1, H // 2), w1q_o), f"{label}: W1 codes"
    assert np.array_equal(host(mx.w1s[u_t]).reshape(-1, mx.w1s.shape[-1])[:, :nbh], w1s_o), f"{label}: W1 scales"
    assert np.array_equal(host(mx.w2q[u_t]).reshape(-1, I // 2), w2q_o), f"{label}: W2 codes"
    src_rows = torch.from_numpy(tok if mx.gather else rows).to(mx.xq.device)
    assert np.array_equal(host(mx.xq[src_rows]), xq_o), f"{label}: x codes"
    assert np.array_equal(host(mx.xs[src_rows])[:, :nbh], xs_o), f"{label}: x scales"

    actq_o, acts_o, yp_o = oracle.ffn_mx_rows(xq_o, xs_o, w1q_o, w1s_o, w2q_o, w2s_o, H, I,
                                              np.arange(len(rows), dtype=np.int32),
                                              ex_local.astype(np.int32))
    rows_t = torch.from_numpy(rows).to(mx.actq.device)
    g_actq = host(mx.actq[rows_t])
    g_acts = host(mx.acts[rows_t])[:, :nbi]
    g_yp = oracle.bf16_to_f64(host(mx.yp[rows_t]))
    code_diff = float(np.mean(g_actq != actq_o)) if g_actq.size else 0.0
    a_g = oracle.mx_dequantize(g_actq, g_acts, I, FP8)
    a_o = oracle.mx_dequantize(actq_o, acts_o, I, FP8)
    e_act = rel_frob(a_g, a_o)
    e_yp = rel_frob(g_yp, oracle.bf16_to_f64(yp_o))
    # FC2 alone, in float64 from the HIP path's activation codes (one expert at a time)
    fc2 = np.zeros((len(rows), H))
    for j in range(len(uniq)):
        sel = ex_local == j
        w2_deq = oracle.mx_dequantize(w2q_o[j * H:(j + 1) * H], w2s_o[j * H:(j + 1) * H], I, FP4)
        fc2[sel] = a_g[sel] @ w2_deq.T
    fc2_bf16 = torch.from_numpy(fc2).to(torch.bfloat16).to(torch.float64).numpy()
    e_fc2 = rel_frob(g_yp, fc2_bf16)
    print(f"{label}: rows={len(rows)} act codes differing={code_diff:.1e} act={e_act:.2e} "
          f"yp={e_yp:.2e} fc2(same act)={e_fc2:.2e}", flush=True)
    assert code_diff <= ACT_CODE_DIFF, f"{label}: act codes differ in {code_diff:.2e}"
    assert e_act <= ACT_TOL, f"{label}: act rel err {e_act}"
    assert e_yp <= BF16_TOL, f"{label}: yp rel err {e_yp}"
    assert e_fc2 <= FC2_TOL, f"{label}: fc2 rel err {e_fc2}"


SMALL = [
    # K % 128 == 64 in FC2 (I = 192) and half an FC1 column tile; ragged blocks at beta 32
    ("ragged", dict(seed=1, T=37, H=128, E=12, K=3, I=192, P=4, block_m=32)),
    # K % 128 == 64 in FC1 (H = 192)
    ("h_tail", dict(seed=2, T=200, H=192, E=8, K=2, I=128, P=2, block_m=64)),
    # one half slice of K in FC1 (H = 64), several tiles per expert
    ("many_blocks", dict(seed=15, T=4096, H=64, E=64, K=8, I=64, P=8, block_m=16)),
    ("subset_local", dict(seed=4, T=300, H=128, E=16, K=3, I=128, P=2, E_loc=4, begin=1,
                          stride=3, block_m=64)),
    ("hot_experts", dict(seed=5, T=700, H=256, E=8, K=2, I=320, P=4,
                         logit_bias=[30, 29, 0, 0, 0, 0, 0, 0])),
    ("wide_k", dict(seed=8, T=80, H=128, E=256, K=16, I=64, P=16, block_m=16)),
]


@pytest.mark.parametrize("name,kw", SMALL)
def test_mx_ffn_small_layers(name, kw):
    """Every valid row against the oracle, gather-on-load and materialised inputs; the two
    paths bit-identical."""
    _announce(f"small {name} {kw}")
    c = random_case(**kw)
    layer = run_gpu(c)
    ref = oracle_index(c)
    mat = MxRun(layer, c, gather=False)
    layer_g = run_gpu(c, gather=True)
    gat = MxRun(layer_g, c, gather=True)
    rows = np.nonzero(ref.row_token >= 0)[0]
    rows_t = torch.from_numpy(rows).to(mat.actq.device)
    for name_ in ("actq", "acts", "yp"):
        a, b = getattr(gat, name_)[rows_t], getattr(mat, name_)[rows_t]
        assert torch.equal(a, b), f"gather vs materialised: {name_}"
    _check_rows(c, gat, ref, rows, name)


def test_mx_ffn_repeat_and_untouched_rows():
    """Two runs bit-identical; rows outside a partial block table stay untouched."""
    _announce("repeat + partial table")
    c = random_case(seed=3, T=600, H=128, E=12, K=3, I=192, P=4, block_m=32)
    layer = run_gpu(c, gather=True)
    ref = oracle_index(c)
    mx = MxRun(layer, c, gather=True)
    first = [t.clone() for t in (mx.actq, mx.acts, mx.yp)]
    mx.run()
    for a, b, n in zip(first, (mx.actq, mx.acts, mx.yp), ("actq", "acts", "yp")):
        assert torch.equal(a, b), f"repeat: {n}"
    # every other block
    nb = int(layer.n_blocks.item())
    full = host(layer.blocks[:nb])
    sub = np.ascontiguousarray(full[::2])
    dev = layer.blocks.device
    sub_buf = torch.zeros_like(layer.blocks)
    sub_buf[: len(sub)] = torch.from_numpy(sub).to(dev)
    n_sub = torch.tensor([len(sub)], dtype=torch.int32, device=dev)
    part = MxRun(layer, c, gather=True, blocks=sub_buf, n_blocks=n_sub)
    covered = np.zeros(part.actq.shape[0], bool)
    for _, _, first_row, m in sub.tolist():
        covered[first_row:first_row + m] = True
    cov_t = torch.from_numpy(covered).to(dev)
    assert torch.equal(part.actq[cov_t], mx.actq[cov_t]) and torch.equal(part.yp[cov_t], mx.yp[cov_t])
    assert not part.actq[~cov_t].any() and not part.acts[~cov_t].any() and not part.yp[~cov_t].any()
    n = len(ref.row_token)
    rows = np.nonzero(covered[:n] & (ref.row_token >= 0))[0][:200]
    _check_rows(c, part, ref, rows, "partial table")


FULL = [("olmoe_shaped", 1.2), ("gpt_oss_120b_shaped", 1.2), ("deepseek_v3_share", 1.2),
        ("gpt_oss_120b_decode", 1.2)]


@pytest.mark.parametrize("name,skew", FULL)
def test_mx_ffn_full_size_sampled(name, skew):
    """At the full layer size (gather-on-load, the benchmarked configuration): sampled rows of
    a few experts against the oracle, which computes them one by one."""
    _announce(f"full {name} skew={skew}")
    w = inputs.WORKLOADS[name]
    if skew not in w.skews:
        skew = w.skews[0]
    c = workload_case(name, skew, weights=inputs.make_weights(w, threads=16))
    layer = run_gpu(c, gather=True)
    ref = oracle_index(c)
    mx = MxRun(layer, c, gather=True)
    rows = sample_rows(ref, 64, seed=2)
    ex = row_experts(ref.blocks, rows)
    keep = np.isin(ex, np.unique(ex)[:4])  # rows of at most 4 experts (oracle quantizes those)
    _check_rows(c, mx, ref, rows[keep], name)
    del layer, mx
    gc.collect()
    torch.cuda.empty_cache()


def _mx_layer(c):
    dev = "cuda"
    layer = binding.RoutedExperts(c.T, c.H, c.E, c.K, c.I, c.P, dtype=c.dtype, E_loc=c.n_local,
                                  expert_begin=c.begin, expert_stride=c.stride,
                                  block_m=c.block_m, renormalize=c.renormalize, device=dev,
                                  precision="mx")
    logits = torch.from_numpy(c.logits).to(dev)
    x = c.x.to(dev)
    w1, w2 = binding.mx_quantize_weights(c.W1.to(dev), c.W2.to(dev))
    return layer, logits, x, w1, w2


@pytest.mark.parametrize("name,kw", [SMALL[0], SMALL[3], SMALL[4]])
def test_mx_layer_end_to_end(name, kw):
    """RoutedExperts(precision="mx"): the whole step (route, permute, MXFP8 quantization of x,
    plan, MX FFN, combine) against the oracle: index outputs bit-exact, yp per row, out per
    token (oracle combine over the oracle's MX yp)."""
    from parity_helpers import check_index_parity
    _announce(f"mx layer {name}")
    c = random_case(**kw)
    layer, logits, x, w1, w2 = _mx_layer(c)
    layer.forward(logits, x, w1, w2)
    torch.cuda.synchronize()
    ref = oracle_index(c)
    check_index_parity(layer, ref)
    assert np.array_equal(host(layer.xq), oracle.mx_quantize(inputs.as_oracle_array(c.x), FP8)[0])
    rows = np.nonzero(ref.row_token >= 0)[0]
    mx = MxRun.__new__(MxRun)  # the layer's own buffers, checked like an MxRun
    mx.H, mx.I, mx.gather = c.H, c.I, True
    (mx.w1q, mx.w1s), (mx.w2q, mx.w2s) = w1, w2
    mx.xq, mx.xs, mx.actq, mx.acts, mx.yp = layer.xq, layer.xs, layer.actq, layer.acts, layer.yp
    _check_rows(c, mx, ref, rows, f"layer {name}")
    # out against the oracle's combine of the oracle's MX yp (all local rows)
    x_o = inputs.as_oracle_array(c.x)
    ex = row_experts(ref.blocks, rows)
    xq_o, xs_o = oracle.mx_quantize(x_o[ref.row_token[rows]], FP8)
    w1q_o, w1s_o = oracle.mx_quantize(inputs.as_oracle_array(c.W1).reshape(-1, c.H), FP4)
    w2q_o, w2s_o = oracle.mx_quantize(inputs.as_oracle_array(c.W2).reshape(-1, c.I), FP4)
    _, _, yp_o = oracle.ffn_mx_rows(xq_o, xs_o, w1q_o, w1s_o, w2q_o, w2s_o, c.H, c.I,
                                    np.arange(len(rows), dtype=np.int32), ex.astype(np.int32))
    yp_full = np.zeros((len(ref.row_token), c.H), np.uint16)
    yp_full[rows] = yp_o
    out_o = oracle.combine(yp_full, ref.w, ref.entry_pos, c.T, c.K)
    e_out = rel_frob(oracle.bf16_to_f64(host(layer.out)), oracle.bf16_to_f64(out_o))
    print(f"layer {name}: out={e_out:.2e}", flush=True)
    assert e_out <= BF16_TOL, e_out


def test_mx_layer_graph_replay():
    """The MX step captured in a HIP graph: every replay (with eager work between) equals the
    eager step bit for bit."""
    _announce("mx layer graph replay")
    c = random_case(seed=12, T=500, H=256, E=16, K=4, I=192, P=4, block_m=32)
    layer, logits, x, w1, w2 = _mx_layer(c)
    layer.forward(logits, x, w1, w2)
    torch.cuda.synchronize()
    eager = [t.clone() for t in (layer.out, layer.actq, layer.yp)]
    graph = layer.capture(logits, x, w1, w2)
    for _ in range(3):
        layer.out.zero_()  # every row of out is rewritten by the step
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(layer.out, eager[0]), "out"
        assert torch.equal(layer.actq, eager[1]), "actq"
        assert torch.equal(layer.yp, eager[2]), "yp"
    del graph
