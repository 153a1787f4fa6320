"""MI355X-native forward pass of a ternary-expert (PQ2_0 / PTQ1_0) MoE block.

The compute path is the HIP library libmoe_ternary.so (C ABI in
include/moe_ternary.h); this package is its thin Python binding.
"""
from .binding import (EXPORTS, PQ2_0, PTQ1_0, QUANT_ABSMEAN, QUANT_LLOYD, STAGES, ExpertBanks, MoeError,
                      StageTimer, alloc_workspace, block_bytes, draft_head, forward, forward_factored, forward_noalloc, forward_q, lib, lowrank_apply, pack,
                      packed_bytes, ple_gather, quantize_device, route, route_factored, tile_container, unpack, unpack_device,
                      untile_container, workspace_bytes)
from .layers import build_banks, pack_expert

__all__ = ["EXPORTS", "PQ2_0", "PTQ1_0", "QUANT_ABSMEAN", "QUANT_LLOYD", "STAGES", "StageTimer", "ExpertBanks",
           "MoeError", "alloc_workspace", "block_bytes", "draft_head", "forward", "forward_factored", "forward_noalloc", "forward_q", "lib", "lowrank_apply", "pack",
           "packed_bytes", "ple_gather", "quantize_device", "route", "route_factored", "tile_container", "unpack", "unpack_device",
           "untile_container", "workspace_bytes", "build_banks", "pack_expert"]
