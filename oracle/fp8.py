"""8-bit floating-point operands — TEST INFRASTRUCTURE ONLY.

The pages name 16-bit GEMM operands and a BF16 mode but no 8-bit format;
the 8-bit operand variant follows the two formats of the OCP 8-bit floating
point specification (OFP8) as gfx950's MFMA reads them:

* E4M3 ("e4m3fn"): 1 sign, 4 exponent bits (bias 7), 3 mantissa bits; no
  infinities, the all-ones pattern S.1111.111 is NaN, so the largest finite
  magnitude is 1.75 * 2^8 = 448; subnormals down to 2^-9.
* E5M2: 1 sign, 5 exponent bits (bias 15), 2 mantissa bits, IEEE-style
  infinities and NaNs; largest finite 1.75 * 2^15 = 57344; subnormals down
  to 2^-16.

Reading taken for the scaling (the pages fix none): one scale per tensor,
s = FMAX / max|x| computed in fp32 (1 when max|x| is 0), the value x * s
rounded once to fp32, clamped to [-FMAX, FMAX], then rounded to the format
to nearest, ties to even; the product of two such operands is
(sum over K of a8 b8) / (s_a s_b). The code decision is taken in fp32 on
both sides (the same precision the device uses).
"""
import numpy as np

FORMATS = {
    # name: (exponent bits, mantissa bits, bias, largest finite)
    "e4m3": (4, 3, 7, 448.0),
    "e5m2": (5, 2, 15, 57344.0),
}


def _params(fmt):
    e, m, bias, fmax = FORMATS[fmt]
    emin = 1 - bias  # exponent of the smallest normal
    return e, m, bias, fmax, emin


def round_to_format(v, fmt):
    """Nearest representable value of the format, ties to even mantissa, for
    finite |v| <= FMAX (the caller clamps). float64 in, float64 out."""
    _, m, _, fmax, emin = _params(fmt)
    v = np.asarray(v, np.float64)
    a = np.abs(v)
    # exponent of the binade holding |v| (subnormals share emin's quantum)
    with np.errstate(divide="ignore"):
        ex = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    ex = np.maximum(ex, emin)
    quantum = np.exp2(ex - m)
    q = a / quantum  # exact: division by a power of two
    r = np.floor(q)
    frac = q - r
    up = (frac > 0.5) | ((frac == 0.5) & (np.mod(r, 2) == 1))
    r = r + up
    out = np.sign(v) * r * quantum
    assert np.all(np.abs(out) <= fmax), "value above the format's range: clamp first"
    return out


def encode(v, fmt):
    """Bit patterns (uint8) of representable values v."""
    e, m, bias, _, emin = _params(fmt)
    v = np.asarray(v, np.float64)
    sign = (np.signbit(v)).astype(np.uint32)
    a = np.abs(v)
    with np.errstate(divide="ignore"):
        ex = np.floor(np.log2(np.where(a > 0, a, 1.0))).astype(np.int64)
    normal = (a > 0) & (ex >= emin)
    exp_field = np.where(normal, ex + bias, 0)
    quantum = np.exp2(np.where(normal, ex, emin) - m)
    mant = np.where(normal, a / quantum - (1 << m), a / quantum)
    mant = np.where(a > 0, mant, 0.0)
    assert np.all(mant == np.floor(mant)) and np.all(mant < (1 << m)), "not representable"
    bits = (sign << (e + m)) | (exp_field.astype(np.uint32) << m) | mant.astype(np.uint32)
    return bits.astype(np.uint8)


def decode(codes, fmt):
    """float64 values of bit patterns (NaN / inf patterns decode as such)."""
    e, m, bias, _, emin = _params(fmt)
    c = np.asarray(codes, np.uint8).astype(np.int64)
    sign = np.where((c >> (e + m)) & 1, -1.0, 1.0)
    ef = (c >> m) & ((1 << e) - 1)
    mf = c & ((1 << m) - 1)
    val = np.where(ef == 0, mf * np.exp2(emin - m), (1.0 + mf / (1 << m)) * np.exp2(ef - bias))
    if fmt == "e4m3":
        val = np.where((ef == (1 << e) - 1) & (mf == (1 << m) - 1), np.nan, val)
    else:
        top = ef == (1 << e) - 1
        val = np.where(top & (mf == 0), np.inf, np.where(top, np.nan, val))
    return sign * val


def quantize(x, fmt):
    """Per-tensor scaled quantization of an fp32 array: returns (codes
    uint8 of x's shape, inv_scale as float32 = 1 / s)."""
    _, _, _, fmax, _ = _params(fmt)
    x = np.asarray(x, np.float32)
    amax = np.float32(np.max(np.abs(x))) if x.size else np.float32(0)
    s = np.float32(1.0) if amax == 0 else np.float32(np.float32(fmax) / amax)
    v = (x * s).astype(np.float32)  # one fp32 rounding, as on the device
    v = np.clip(v, -fmax, fmax).astype(np.float64)
    q = round_to_format(v, fmt)
    return encode(q, fmt), np.float32(np.float32(1.0) / s)


def gemm_nt(a_codes, fmt_a, inv_a, b_codes, fmt_b, inv_b):
    """C[M, N] = (A8 B8^T) * inv_a * inv_b with A8 [M, K], B8 [N, K] the
    decoded operands; float64."""
    A = decode(a_codes, fmt_a)
    B = decode(b_codes, fmt_b)
    return (A @ B.T) * (float(inv_a) * float(inv_b))
