"""moe_expert_ffn_gather_noalloc (the FFN with the library's static per-GPU scratch, for callers
that cannot allocate) against moe_expert_ffn_gather with a caller workspace: act and yp bit for
bit on every valid row, over calls in a row on one GPU, the later ones smaller."""
import pytest
import torch

from mixture_experts_routed_router_amd import binding
from parity_helpers import host, random_case, run_gpu

pytestmark = pytest.mark.gpu

CASES = [
    ("bf16_large", dict(seed=21, T=1200, H=256, E=16, K=4, I=320, P=4, block_m=64)),
    ("bf16_smaller", dict(seed=22, T=150, H=128, E=8, K=2, I=192, P=4, block_m=32)),
    ("f32_small", dict(seed=23, T=64, H=64, E=8, K=2, I=128, P=4, block_m=16,
                       dtype=torch.float32)),
]


def test_noalloc_matches_workspace_entry_point():
    for name, kw in CASES:
        print(f"\n[noalloc] {name} {kw}", flush=True)
        c = random_case(**kw)
        layer = run_gpu(c, gather=True)  # moe_expert_ffn_gather with the layer's workspace
        _, x, W1, W2 = layer._inputs
        act = torch.zeros_like(layer.act)
        yp = torch.zeros_like(layer.yp)
        binding.moe_expert_ffn_gather_noalloc(x, layer.row_token, W1, W2, layer.blocks,
                                              layer.n_blocks, act, yp)
        torch.cuda.synchronize()
        rows = int(host(layer.offsets)[-1])
        valid = torch.nonzero(layer.row_token[:rows] >= 0).squeeze(1)
        assert valid.numel() > 0
        assert torch.equal(act[valid], layer.act[valid]), (name, "act")
        assert torch.equal(yp[valid], layer.yp[valid]), (name, "yp")
        # rows no block covers stay untouched
        mask = torch.ones(act.shape[0], dtype=torch.bool, device=act.device)
        mask[valid] = False
        assert torch.count_nonzero(act[mask]) == 0 and torch.count_nonzero(yp[mask]) == 0, name
        del layer
        torch.cuda.empty_cache()


def test_noalloc_rejects_tables_beyond_its_scratch():
    dev = "cuda"
    x = torch.zeros((4, 64), dtype=torch.bfloat16, device=dev)
    w1 = torch.zeros((2, 128, 64), dtype=torch.bfloat16, device=dev)
    w2 = torch.zeros((2, 64, 64), dtype=torch.bfloat16, device=dev)
    rt = torch.zeros((64,), dtype=torch.int32, device=dev)
    blocks = torch.zeros((binding.FFN_NOALLOC_MAX_BLOCKS + 1, 4), dtype=torch.int32, device=dev)
    nb = torch.zeros((1,), dtype=torch.int32, device=dev)
    act = torch.zeros((64, 64), dtype=torch.bfloat16, device=dev)
    yp = torch.zeros((64, 64), dtype=torch.bfloat16, device=dev)
    with pytest.raises(binding.MoeError):
        binding.moe_expert_ffn_gather_noalloc(x, rt, w1, w2, blocks, nb, act, yp)
