"""CPU fp64 oracle (test infrastructure; see littlebit_oracle's header)."""
from .littlebit_oracle import (  # noqa: F401
    check_sign_factor,
    decode_bf16,
    decode_fp16,
    decode_path,
    forward,
    forward_factored,
    forward_rows,
    linear_storage_bytes,
    pack_signs,
    rank_for_bpw,
    reconstruct_w,
    scale_bits_per_weight,
    sign_bits_per_weight,
    unpack_signs,
    words_per_row,
)
from . import dual_svid  # noqa: F401
