"""Number formats used by the reader's stored state.  (Oracle: test infrastructure.)

* BF16 checkpoint weights are decoded exactly (bf16 -> fp32 is a bit shift,
  fp32 -> fp64 is exact).
* The sketch scale is stored as FP16 ([zh §前置知识 / Hadamard旋转与三元Sketch]).
  Every fp64 -> fp16 conversion rounds once, to nearest, ties to even.  numpy's
  float64 -> float16 cast does exactly that (it does not pass through fp32);
  tests pin it against exact rational rounding on halfway and subnormal cases.

Pins: tests/test_oracle_numerics.py (exact rational rounding, double-rounding
trap, subnormals, overflow).
"""
import numpy as np


def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    b = np.asarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


def weights_f64(w: np.ndarray) -> np.ndarray:
    """Weights as float64: BF16 bit patterns (uint16) decoded exactly, or
    real-valued weights (a dequantized 4-bit checkpoint, oracle/int4.py)
    taken as they are."""
    w = np.asarray(w)
    return bf16_to_f64(w) if w.dtype == np.uint16 else w.astype(np.float64)


def f64_to_f16_bits(a) -> np.ndarray:
    """Round float64 to IEEE binary16, nearest-even, in a single rounding."""
    with np.errstate(over="ignore"):
        return np.asarray(a, dtype=np.float64).astype(np.float16).view(np.uint16)


def f16_bits_to_f64(bits) -> np.ndarray:
    return np.asarray(bits, dtype=np.uint16).view(np.float16).astype(np.float64)
