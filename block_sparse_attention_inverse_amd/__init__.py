"""MI355X-native block-sparse self-attention over 3D video tokens.

Public surface (Python names mirror the C ABI in include/bsa.h):
``permute``, ``mask_capacity``, ``mask_workspace``, ``build_mask``,
``permute_pool``, ``build_mask_pooled``, ``build_mask_pooled_noalloc`` (no
device allocation: a fixed scratch inside the library), ``order_workspace``,
``order_scores``, ``select_orders``, ``quantize_int8``, ``forward``,
``forward_int8``, ``forward_natural``, ``forward_int8_natural``, ``debug_int8_qk``, ``debug_int8_pv``, the offline calibration
``attn_block_stats``, ``paro_metric``, ``paro_select`` (chained by
``paro_calibrate``), the static masks ``mask_from_block_sums`` and
``mask_from_bits``, the Top-K / Top-P / noise-perturbed selection
``block_scores`` + ``mask_from_scores``, the first-order compensation of skipped
keys ``fo_compensate`` (``fo_workspace``), plus ``LayerPlan`` / ``layer_forward`` which chain the
per-step calls.
The HIP library is loaded on first use and must be built; there is no
fallback path.  ``synth`` holds the seeded synthetic workload generators.
"""
from .api import (  # noqa: F401
    LayerPlan,
    abi_version,
    attn_block_stats,
    block_scores,
    build_mask,
    build_mask_pooled,
    build_mask_pooled_noalloc,
    debug_int8_pv,
    debug_int8_qk,
    fo_compensate,
    fo_workspace,
    forward,
    forward_int8,
    forward_int8_natural,
    forward_natural,
    last_error,
    layer_forward,
    mask_capacity,
    mask_from_bits,
    mask_from_block_sums,
    mask_from_scores,
    mask_params,
    mask_workspace,
    order_scores,
    order_workspace,
    paro_calibrate,
    paro_metric,
    paro_select,
    permute,
    permute_pool,
    quantize_int8,
    scores_select_workspace,
    select_orders,
)
from ._lib import BsaError, MaskParams  # noqa: F401
