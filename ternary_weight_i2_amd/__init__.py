"""MI355X-native BitNet b1.58 W2A8 (I2_S) matmul: Python binding.

The compute lives in ``libbitnet_i2s.so`` (hand-written HIP for gfx950,
C ABI declared in ``include/bitnet_i2s.h``).  This package only marshals
torch tensors into that ABI; it loads the library lazily and raises if it
is missing -- there is no fallback path.
"""
from ._binding import (  # noqa: F401
    BitnetError, I2SMatrix, abi_version, absmean_pack, ffn, ffn_act_quant, gemm, gemm_group,
    gemv, gemv_group, gemv_lut, lib_path, linear, load, pack, pack_f32, quant_act,
    stamps_read, stamps_reset, use_library,
)
