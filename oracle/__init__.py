"""CPU oracle for the calibration-free MoE channel-selection reader.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or run anything in this
package.  The product path (the HIP library and its Python binding) never
imports it, and this package imports nothing from the product path; the two
share only the seeded input generators in ``synth``.

The oracle is slow and plain on purpose: numpy float64 throughout, library
primitives (matmul, eigh, sort) used as single steps, no blocking or fusion
beyond what the method's definition states.

Citation legend used in this package:
  [zh §S]  the Chinese summary page of "Channel Selection for
           Mixture-of-Experts Decoding Needs No Calibration Data"
           (Kim, Hwang; paper.rainbus.top/paper/2610.37386), section S.
  [ko §S]  the Korean summary page of the same paper, titled
           "MoE 채널 선택은 캘리브레이션 없이 top-k로 충분하다"
           (onedev.kr/papers/1435), section S.

Parity status per function (what pins it) is listed in each module header.
"""
from .numerics import bf16_to_f64, weights_f64, f64_to_f16_bits, f16_bits_to_f64
from .rotation import (splitmix64_stream, sign_vector, sylvester_hadamard,
                       rotate_rows, rotate_x_f64,
                       rotation_matrix, SQRT128)
from .sketch import ternarize_blocks, unit_geometry, pack_units, unpack_units
from .lowrank import recovery_basis
from .dense import dense_moe
from .route import route
from .topk import topk_desc
from .accounting import read_bytes, resident_bytes
from .expected_error import (silu_grad, block_norms2, sketch_variance, activation_variance,
                             expected_error_score)
from .reader import OracleReader
from .shared import decode_shared

__all__ = [
    "decode_shared",
    "bf16_to_f64", "weights_f64", "f64_to_f16_bits", "f16_bits_to_f64", "splitmix64_stream",
    "sign_vector", "sylvester_hadamard", "rotate_rows", "rotate_x_f64",
    "rotation_matrix", "SQRT128", "ternarize_blocks",
    "unit_geometry", "pack_units", "unpack_units", "recovery_basis", "dense_moe",
    "route", "topk_desc", "read_bytes", "resident_bytes", "OracleReader", "silu_grad",
    "block_norms2", "sketch_variance", "activation_variance", "expected_error_score",
]
