"""MI355X-native Gated DeltaNet core: decode step, conv update, chunked prefill.

The computation lives in ``libgdn.so`` (hand-written HIP kernels for gfx950,
C ABI in ``include/gdn.h``); this package is its thin ctypes binding.
"""
from ._abi import (  # noqa: F401
    DEFAULT_DECODE_FLAGS, DEFAULT_PREFILL_FLAGS, EFLAG_SEQLENS, EFLAG_SLOT_RANGE,
    EFLAG_SLOT_REPEAT, EXPORTED, FLAG_QK_L2NORM, FLAG_SILU, FLAG_STEP_FUSED, FLAG_STEP_SPLIT,
    FLAG_PREFILL_NS3, FLAG_PREFILL_NS4, FLAG_PREFILL_SEQUENTIAL, FLAG_PREFILL_SINGLE_ROLE,
    FLAG_VALIDATE, GDN_BF16, GDN_F32, NORM_GATE_SIGMOID, NORM_ZERO_CENTRED, gdn_gated_rmsnorm,
    GateInputs, GDNError, gdn_conv_update, gdn_decode_recurrent, gdn_decode_step,
    gdn_decode_step_fused, gdn_decode_step_gated, gdn_decode_step_noalloc, gdn_decode_workspace_size,
    gdn_dims, gdn_gate_inputs, gdn_mixed_step,
    gdn_mixed_workspace_size,
    gdn_prefill_chunked, gdn_prefill_chunked_gated, gdn_prefill_segmented,
    gdn_prefill_segmented_workspace_size, gdn_prefill_workspace_size, gdn_strerror,
    load_library, make_dims, MixedStreams,
)
