"""MI355X (gfx950) LittleBit factorised-linear forward: Python binding of liblittlebit.

The HIP library (``liblittlebit.so``, built by ``binary_rank_gemm_amd.build``)
does all of the arithmetic; this package only marshals arguments.
"""
from ._binding import (  # noqa: F401
    BF16,
    BF16_FP32,
    EXPORTS,
    FP32,
    REGIME_AUTO,
    REGIME_DECODE,
    REGIME_EXACT,
    REGIME_PREFILL,
    LbPath,
    Linear,
    LittleBitError,
    BoundStack,
    Stack,
    auto_regime,
    lib,
    init_dual_svid,
    pack_signs,
    pack_signs_host,
    packed_words_per_row,
    rank_for_bpw,
    unpack_signs,
)
