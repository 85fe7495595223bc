"""Activation-sparse ReLU FFN layer in TwELL form for AMD Instinct MI355X (gfx950).

The compute lives in ``libsparse_ffn.so`` (hand-written HIP kernels behind a C ABI, see
``include/sparse_ffn.h``); ``sparse_ffn`` is a thin ctypes binding to it.
"""
from .sparse_ffn import (  # noqa: F401
    Config, SparseFFN, TwellBuffers, SffnError, twell_pack, twell_stats, check, buffer_sizes,
    count_histogram, choose_ell_width,
    buffer_bytes, BUFFER_FIELDS,
    profile_enable, profile_only, profile_reset, profile_read, probe_gather_fma, lib, LIB_PATH,
    SFFN_OK, SFFN_ERR_INVALID_ARGUMENT, SFFN_ERR_UNSUPPORTED, SFFN_ERR_BACKUP_OVERFLOW,
    SFFN_ERR_DEVICE, DOWN_AUTO, DOWN_GATHER, DOWN_MFMA, DOWN_TILES, DOWN_UNION, DOWN_SPARSE,
    DOWN_GATHER_DENSITY_DEFAULT, DOWN_MFMA_DENSITY_DEFAULT, DOWN_TILES_MIN_T, DOWN_MFMA_MIN_T,
    MAX_TILES,
)
