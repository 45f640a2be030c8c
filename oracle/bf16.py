"""Exact bfloat16 <-> float64 conversions for the oracle (test infrastructure only).

bfloat16 keeps the float32 sign and 8-bit exponent and 7 stored fraction bits
(8 significant bits).  A bf16 bit pattern widens exactly to float32 by a
16-bit left shift, and float32 widens exactly to float64.

Rounding to bf16 here is textbook round-to-nearest, ties-to-even, applied to
the float64 value directly (no intermediate float32 step, so there is no
double rounding).  NaN inputs are outside the contract.
"""

import numpy as np

# bf16 normals have 8 significant bits; the smallest normal is 2**-126, and
# subnormals are multiples of 2**-133.
_BF16_SIG_BITS = 8
_BF16_MIN_NORMAL_EXP = -126
_BF16_SUBNORMAL_QUANTUM_EXP = -133
# float32 mirrors the same scheme with 24 significant bits.
_F32_SIG_BITS = 24
_F32_MIN_NORMAL_EXP = -126
_F32_SUBNORMAL_QUANTUM_EXP = -149


def bf16_bits_to_f64(bits):
    """Widen bf16 bit patterns (uint16) to float64 exactly."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    with np.errstate(invalid="ignore"):          # NaN patterns stay NaN
        return b.view(np.float32).astype(np.float64)


def _round_to_grid(x, sig_bits, min_normal_exp, sub_quantum_exp):
    """Round float64 ``x`` to the nearest value with ``sig_bits`` significant
    bits (ties to even), with a subnormal floor at ``2**sub_quantum_exp``.

    ``frexp`` writes x = m * 2**e with 0.5 <= |m| < 1, so a number with
    ``sig_bits`` significant bits is an integer multiple of 2**(e - sig_bits).
    Scaling by a power of two is exact, and ``np.rint`` rounds half to even.
    """
    x = np.asarray(x, dtype=np.float64)
    _, e = np.frexp(x)
    # |x| >= 2**min_normal_exp  <=>  e - 1 >= min_normal_exp
    q_exp = np.where(e - 1 >= min_normal_exp, e - sig_bits, sub_quantum_exp)
    r = np.rint(np.ldexp(x, -q_exp))
    return np.ldexp(r, q_exp)


def round_bf16(x):
    """Round float64 values to the nearest bf16 value (RNE); returns float64.

    Values that round beyond the largest finite bf16 become +-inf, as IEEE
    round-to-nearest requires.
    """
    y = _round_to_grid(x, _BF16_SIG_BITS, _BF16_MIN_NORMAL_EXP, _BF16_SUBNORMAL_QUANTUM_EXP)
    with np.errstate(over="ignore"):
        return y.astype(np.float32).astype(np.float64)


def round_f32(x):
    """Round float64 values to the nearest float32 value (RNE); returns float64."""
    y = _round_to_grid(x, _F32_SIG_BITS, _F32_MIN_NORMAL_EXP, _F32_SUBNORMAL_QUANTUM_EXP)
    with np.errstate(over="ignore"):
        return y.astype(np.float32).astype(np.float64)


def f64_to_bf16_bits(x):
    """Round float64 values to bf16 (RNE) and return the uint16 bit patterns."""
    y = round_bf16(x).astype(np.float32)
    return (y.view(np.uint32) >> np.uint32(16)).astype(np.uint16)
