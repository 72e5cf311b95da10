"""Reduced-precision attention inputs: MXFP6 queries and keys, FP8 values, in fp64.

What the step does ("The road to the fastest, cheapest H3", section "Accelerating the
denoiser", item 2, reducing precision in video attention: on MI355X the video attention
runs with MXFP6 queries and keys and FP8 values).  The attention itself is unchanged:
softmax attention over the dequantized queries, keys and values (the definition in
attention.py, over the same cache model and visible sets).

The pages name the formats and nothing more, so this module takes the plainest reading of
the OCP Microscaling (MX) formats specification v1.0 (listed with the design notes):

  FP6 E2M3   sign, 2 exponent bits (bias 1), 3 mantissa bits; no inf/NaN.  Normal values
             (1 + m/8) 2^(e-1), subnormal (e = 0) m/8.  Largest 7.5, smallest normal 1.0,
             smallest subnormal 0.125.
  FP8 E4M3   sign, 4 exponent bits (bias 7), 3 mantissa bits; S.1111.111 is NaN, no inf.
             Normal (1 + m/8) 2^(e-7), subnormal m/8 2^-6.  Largest 448, smallest normal
             2^-6, smallest subnormal 2^-9.
  MXFP6      blocks of 32 consecutive elements along head_dim share one E8M0 scale 2^X
             (X in [-127, 127]).  X = floor(log2(max |x| of the block)) - 2, where 2 is the
             exponent of E2M3's largest binade, clamped to [-127, 127] (an all-zero block
             gets -127); element = E2M3(x / 2^X).
  FP8 values E4M3 per element, no block scale (the pages say FP8, not MXFP8).

Conversion of a real value to an element format: round to the nearest representable value,
ties to the even mantissa, magnitudes beyond the largest value saturate to it, and the sign
bit is the input's (so -0.0 and negatives that round to zero keep a set sign bit).

Every function here is written from those definitions in fp64, element by element where
that is clearer; no blocking beyond the 32-element scale blocks.

TEST INFRASTRUCTURE ONLY (see the package docstring).
"""
import numpy as np

# (exponent bits, mantissa bits, exponent bias, largest finite magnitude)
E2M3 = (2, 3, 1, 7.5)
E4M3 = (4, 3, 7, 448.0)
MX_BLOCK = 32
E2M3_EMAX = 2         # exponent of E2M3's largest binade [4, 8)
SCALE_MIN, SCALE_MAX = -127, 127


def element_value(code, fmt):
    """Value of one element code (an int, sign bit on top) in format fmt; NaN for E4M3's NaN."""
    eb, mb, bias, _ = fmt
    width = 1 + eb + mb
    code = int(code)
    sign = -1.0 if (code >> (width - 1)) & 1 else 1.0
    e = (code >> mb) & ((1 << eb) - 1)
    m = code & ((1 << mb) - 1)
    if fmt == E4M3 and e == 15 and m == 7:
        return float("nan")
    if e == 0:
        return sign * (m / 2.0 ** mb) * 2.0 ** (1 - bias)
    return sign * (1.0 + m / 2.0 ** mb) * 2.0 ** (e - bias)


def decode(codes, fmt):
    """Element codes (any integer array) -> fp64 values of the same shape."""
    codes = np.asarray(codes)
    table = np.array([element_value(c, fmt) for c in range(1 << (1 + fmt[0] + fmt[1]))])
    return table[codes.astype(np.int64)]


def encode(x, fmt):
    """fp64 values -> element codes (uint8), round to nearest even with saturation.

    For |x| with binade E = floor(log2 |x|) (at least the smallest normal binade 1 - bias),
    the representable values near |x| are spaced 2^(E - mantissa bits); |x| is divided by
    that spacing, rounded half to even (numpy's rint), multiplied back and clipped to the
    largest value, and the result's bits are assembled."""
    eb, mb, bias, vmax = fmt
    x = np.asarray(x, dtype=np.float64)
    a = np.abs(x)
    if not np.isfinite(a).all():
        raise ValueError("inputs must be finite")
    emin = 1 - bias
    _, fe = np.frexp(a)                      # a = f 2^fe with f in [0.5, 1): binade fe - 1
    ex = np.where(a > 0, fe - 1, emin).astype(np.float64)
    ex = np.maximum(ex, emin)
    quantum = np.exp2(ex - mb)
    r = np.rint(a / quantum) * quantum
    r = np.minimum(r, vmax)
    # assemble bits of the rounded magnitude r (exactly representable now)
    sub = r < 2.0 ** emin
    m_sub = np.rint(r / 2.0 ** (emin - mb))
    _, re = np.frexp(np.where(sub, 1.0, r))
    e_norm = (re - 1) + bias
    m_norm = np.rint((np.where(sub, 1.0, r) / np.exp2(re - 1) - 1.0) * 2 ** mb)
    e_field = np.where(sub, 0, e_norm).astype(np.int64)
    m_field = np.where(sub, m_sub, m_norm).astype(np.int64)
    sign = np.signbit(x).astype(np.int64)
    return ((sign << (eb + mb)) | (e_field << mb) | m_field).astype(np.uint8)


def mx_scale_exponents(x):
    """x [..., D] (D a multiple of 32) -> E8M0 exponents X [..., D/32] (int64)."""
    x = np.asarray(x, dtype=np.float64)
    if x.shape[-1] % MX_BLOCK:
        raise ValueError("head_dim must be a multiple of the block size")
    blocks = x.reshape(x.shape[:-1] + (x.shape[-1] // MX_BLOCK, MX_BLOCK))
    amax = np.abs(blocks).max(axis=-1)
    _, fe = np.frexp(amax)
    X = np.where(amax > 0, (fe - 1) - E2M3_EMAX, SCALE_MIN)
    return np.clip(X, SCALE_MIN, SCALE_MAX).astype(np.int64)


def mx_quantize(x):
    """x [..., D] fp64 -> (E2M3 codes uint8 [..., D], scale exponents int64 [..., D/32])."""
    x = np.asarray(x, dtype=np.float64)
    X = mx_scale_exponents(x)
    per_elem = np.repeat(X, MX_BLOCK, axis=-1)
    return encode(x / np.exp2(per_elem), E2M3), X


def mx_dequantize(codes, X):
    """Inverse of the element mapping: value = E2M3(code) * 2^X of its block."""
    return decode(codes, E2M3) * np.exp2(np.repeat(np.asarray(X), MX_BLOCK, axis=-1))


def mxfp6_values(x):
    """x [..., D] -> the MXFP6-dequantized values (fp64) that the attention uses."""
    return mx_dequantize(*mx_quantize(x))


def fp8_values(x):
    """x [...] -> the FP8 E4M3-dequantized values (fp64)."""
    return decode(encode(x, E4M3), E4M3)

