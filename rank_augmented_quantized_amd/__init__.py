"""Rank-augmented W4A4 linear layer for MI355X (gfx950).

The computation lives in the HIP library ``libtq.so`` (C ABI: include/tq.h);
``rank_augmented_quantized_amd.tq`` is its Python binding.
"""

from .tq import (  # noqa: F401
    TQError,
    linear_group_workspace,
    linear_workspace,
    load,
    tq_codes_bytes,
    tq_debug_accumulate,
    tq_linear,
    tq_linear_asym,
    tq_linear_asym_workspace_offsets,
    tq_linear_group,
    tq_linear_group_workspace_bytes,
    tq_linear_mp,
    tq_linear_mp_asym,
    tq_linear_mp_asym_workspace_bytes,
    tq_linear_mp_asym_workspace_offsets,
    tq_linear_mp_rht,
    tq_linear_mp_workspace_bytes,
    tq_linear_mp_workspace_offsets,
    tq_linear_qlr,
    tq_linear_qlr_workspace_bytes,
    tq_linear_qlr_workspace_offsets,
    tq_linear_workspace_bytes,
    tq_linear_workspace_offsets,
    tq_lowrank_group_bytes,
    tq_lowrank_q_bytes,
    tq_pack_lowrank,
    tq_pack_lowrank_group,
    tq_pack_lowrank_q,
    tq_pack_rht,
    tq_pack_weight,
    tq_profile_enable,
    tq_profile_read,
    tq_profile_reset,
    tq_quantize_act,
    tq_weight_colsum,
)
