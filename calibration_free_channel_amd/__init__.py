"""Calibration-free MoE channel-selection reader for AMD Instinct MI355X (gfx950).

The decode path is hand-written HIP in ``libcfr.so`` (C ABI: include/cfr.h);
this package is its Python binding.  Build with
``python -m calibration_free_channel_amd.build``.
"""
from .reader import (Config, Reader, pack_host, read_bytes, read_bytes_batch, read_bytes_shared,
                     sizes, DEFAULT_ROT_SEED, RANK_SCORE,
                     RANK_EXPECTED_ERROR)

__all__ = ["Config", "Reader", "pack_host", "read_bytes", "read_bytes_batch", "read_bytes_shared", "sizes", "DEFAULT_ROT_SEED", "RANK_SCORE",
           "RANK_EXPECTED_ERROR"]
