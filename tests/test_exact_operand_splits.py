"""The exact bf16 operand split the Q6_K grouped GEMM relies on (CPU).

Q6_K's weight is d * v with v = sc * (q - 32), sc the half block's int8 scale and q a 6-bit
code. The GEMM feeds v to the bf16 MFMA as two operands that must each be exactly
representable in bf16 and sum to v exactly, so that the product with an exact bf16
activation carries no rounding before the fp32 accumulation. With w = v - 128 taken as a
16-bit two's-complement integer:
  hi = w with its low 7 bits cleared (a multiple of 128), and
  lo = 128 + (w & 127), which is the bf16 of biased exponent 134 and mantissa w & 127.
This checks the identity and both exactness conditions for every (sc, q), and that lo's bit
pattern is 0x4300 | (w & 127), the form the kernel builds.
"""
import numpy as np
import pytest


def _bf16_exact(x: np.ndarray) -> np.ndarray:
    bits = x.astype(np.float32).view(np.uint32)
    return (bits & 0xFFFF) == 0


@pytest.mark.parametrize("sc_range", [(-128, 0), (0, 128)])
def test_q6k_two_part_split_is_exact(sc_range):
    sc = np.arange(*sc_range, dtype=np.int64)[:, None]
    q = np.arange(64, dtype=np.int64)[None, :]
    v = sc * (q - 32)
    assert np.abs(v).max() <= 4096
    w16 = (v - 128) & 0xFFFF                       # the packed 16-bit lane the kernel forms
    hi16 = w16 & 0xFF80
    hi = np.where(hi16 >= 0x8000, hi16 - 0x10000, hi16)
    rem = w16 & 0x7F
    lo = 128 + rem
    assert np.array_equal(hi + lo, v)
    assert _bf16_exact(hi.astype(np.float64)).all()
    assert _bf16_exact(lo.astype(np.float64)).all()
    # lo's bf16 bits are 0x4300 | rem: exponent field 134 (2^7), mantissa rem
    lo_bits = (lo.astype(np.float32).view(np.uint32) >> 16).astype(np.int64)
    assert np.array_equal(lo_bits, 0x4300 | rem)
    # hi spans multiples of 128 within [-4224, 3968]: at most 6 significant bits
    assert hi.min() >= -4224 and hi.max() <= 3968 and (hi % 128 == 0).all()
