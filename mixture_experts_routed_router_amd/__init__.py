"""Routed-expert path of one MoE layer on one AMD Instinct MI355X (gfx950).

Five calls, each a C-ABI entry point of ``libmoe.so`` (hand-written HIP for CDNA4):
``moe_route`` -> ``moe_permute`` -> ``moe_plan`` -> ``moe_expert_ffn`` -> ``moe_combine``.
The Python functions of the same names (in ``mixture_experts_routed_router_amd.binding``) only
marshal torch tensors (device memory) and the current stream into those calls.
"""

__all__ = ["binding", "inputs"]
