"""PACE periodic / channel-aligned 4-bit recurrent-state decode and chunked prefill for
AMD Instinct MI355X (gfx950).

The compute path is the HIP library libpace.so (C ABI in include/pace.h); this package
is its thin Python binding plus configuration presets.  PyTorch supplies device memory
and streams only.
"""
from ._lib import (  # noqa: F401
    LIB, LIB_PATH, EXPORTS, LayerConfig, PaceError, layout, head_alloc, decode_step,
    flush_requant, prefill_chunk, prefill_workspace_bytes, bf16_decode_step, calibrate_heads,
    prepare_decode_step, prepare_bf16_decode_step, prepare_prefill_chunk,
    PACE_OK, PACE_EINVAL, PACE_EUNSUPPORTED, PACE_EHIP,
)
from .presets import bf16_periodic, pace4, pace48, tiny_ref  # noqa: F401
