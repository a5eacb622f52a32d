"""GIFT FP8 gradient round trip on MI355X (gfx950).

The compute lives in libgift.so (HIP kernels behind the C ABI of
include/gift.h); this package is its Python binding.  Build the library with
``python -m fac_whitening_gift_amd.build``.
"""

from ._lib import (  # noqa: F401
    Factor, Layer, GroupCall, GiftError, load, status_name, build_hash,
    OP_WHITEN_QUANTIZE, OP_DEQUANT_UNWHITEN, OP_EUCLID_ROUNDTRIP, OP_ROUNDTRIP_ERROR,
    OP_UNWHITEN_F32, gift_dequant_accumulate, gift_unwhiten_f32,
    gift_refresh_factor, gift_refresh_workspace_bytes, gift_whiten_quantize,
    gift_dequant_unwhiten, gift_euclid_fp8_roundtrip, gift_roundtrip_error,
    gift_group_workspace_bytes, gift_draw_sketch, gift_factor_pack_bytes, gift_block_factor_pack_bytes,
    gift_prepare_factor, gift_refresh_factors, gift_refresh_group_workspace_bytes,
    gift_whiten_quantize_static, gift_static_scratch_bytes, factor_cols, MAX_RANK,
    RANK, MAX_SKETCH, SKETCH_WIDTH, sketch_width_for, BLOCK, DTYPE_F32, DTYPE_BF16, DAMP_FLOOR, DAMP_FLOOR_PLUS_TAIL,
    SCALE_TENSOR, SCALE_BLOCK128, SCALE_MXFP4, MX_BLOCK, FLAG_NONFINITE, FLAG_ZERO_AMAX, EXPORTS,
    COEF_ALPHA, COEF_BETA, COEF_LAMBDA_ISO, COEF_LAMBDA_FLOOR, COEF_TRACE, COEF_SIGMA2_TAIL,
    COEF_DW, COEF_DU, COEF_COUNT,
)
