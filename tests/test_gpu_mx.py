"""GPU parity of the MX quantization (moe_mx_quantize, through the C ABI) against the CPU
oracle: codes and E8M0 scales bit for bit, for bf16 and float32 inputs, both formats, across
dynamic ranges, all-zero blocks, ties and saturation."""
import numpy as np
import pytest
import torch

import oracle
from mixture_experts_routed_router_amd import binding, inputs
from parity_helpers import host

pytestmark = pytest.mark.gpu


def _gpu_quantize(t, fmt):
    rows, cols = t.shape
    codes = torch.full((rows, cols if fmt == binding.MOE_MX_FP8 else cols // 2), 0xAA,
                       dtype=torch.uint8, device="cuda")
    pitch = binding.moe_mx_scale_pitch(cols)
    scales = torch.full((rows, pitch), 0xAA, dtype=torch.uint8, device="cuda")
    binding.moe_mx_quantize(t.cuda(), fmt, codes, scales)
    torch.cuda.synchronize()
    s = host(scales)
    # the padding of a scale row (pitch > cols / 32) is not written
    assert (s[:, cols // 32:] == 0xAA).all()
    return host(codes), s[:, : cols // 32]


def _check(t, label):
    for fmt in (binding.MOE_MX_FP8, binding.MOE_MX_FP4):
        c, s = _gpu_quantize(t, fmt)
        rc, rs = oracle.mx_quantize(inputs.as_oracle_array(t), fmt)
        assert np.array_equal(s, rs), (label, fmt, "scales")
        assert np.array_equal(c, rc), (label, fmt, "codes")


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_mx_quantize_random(dtype):
    rng = np.random.default_rng(17)
    a = rng.standard_normal((300, 512)) * np.exp2(rng.integers(-40, 40, (300, 1)))
    a[7] = 0.0                                  # all-zero blocks
    a[8, :32] = 1e-38                           # tiny values
    a[9, ::2] *= -1
    a[10] = np.round(a[10] * 4) / 4             # many exact grid points
    _check(torch.from_numpy(a.astype(np.float32)).to(dtype), str(dtype))


def test_mx_quantize_ties_and_saturation():
    # values at every E2M1 / E4M3 midpoint and beyond the largest value, under unit scales
    fp4 = [0, 0.25, 0.5, 0.75, 1, 1.25, 1.5, 1.75, 2, 2.5, 3, 3.5, 4, 5, 6, 6.5]
    fp4 = fp4 + [-v for v in fp4]
    fp8 = [448.0] + [1 + k / 16 for k in range(16)] + [2.0 ** -10 * k for k in range(15)]
    _check(torch.tensor([fp4, fp8], dtype=torch.float32), "midpoints")
    _check(torch.tensor([fp4, fp8], dtype=torch.float32).to(torch.bfloat16), "midpoints bf16")


def test_mx_quantize_padded_scale_rows():
    """Rows of 2880 values (90 scales, padded to 92 per row) and of 64 values (2 -> 4)."""
    rng = np.random.default_rng(23)
    _check(torch.from_numpy(rng.standard_normal((33, 2880), dtype=np.float32)).to(torch.bfloat16),
           "2880 cols")
    _check(torch.from_numpy(rng.standard_normal((5, 64), dtype=np.float32)), "64 cols")


def test_mx_quantize_expert_weights():
    """One OLMoE-shaped expert's W1 and W2 (bf16, N(0, 0.02^2)) into MXFP4, as the layer's
    weights would be prepared."""
    w = inputs.WORKLOADS["olmoe_shaped"]
    W1, W2 = inputs.make_weights(w, experts=[5])
    _check(W1[0], "W1")
    _check(W2[0], "W2")
