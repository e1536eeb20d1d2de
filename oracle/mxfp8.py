"""Plain fp64 CPU oracle of MXFP8 quantisation (the softmax branch's 8-bit mode).

TEST INFRASTRUCTURE.  Only tests/, __graft_entry__.smoke() and bench.py's
cpu_baseline leg may import or call this module.  It shares no code with the
HIP path and imports nothing from the product package.

Sources.  [P3] (10100.com article on Video DeltaNet, section 实验结果, the
paragraph on scaling with sequence length) reports the 8-step denoiser run in
MXFP8; the pages say no more about it.  The format is the Open Compute
Project's Microscaling (MX) specification v1.0: an MXFP8 block is 32 elements
in FP8 E4M3 (the OCP 8-bit float, "OFP8": sign, 4 exponent bits with bias 7,
3 mantissa bits, no infinities, S.1111.111 the only NaN, 448 the largest
finite value) sharing one E8M0 scale (an 8-bit biased exponent: 2^(code-127),
code 255 NaN).  Converting a block V: the shared exponent is
floor(log2(max_i |V_i|)) minus the largest exponent of the element format
(8 for E4M3), and each element is V_i / 2^shared, rounded to E4M3.

Readings where the specification leaves a choice (also listed in the
repository's design notes):
  * element rounding is to the nearest E4M3 value, ties to the even code
    (mantissa LSB 0), and magnitudes at or above 448 saturate to 448 (no NaN
    is produced from finite input);
  * the shared exponent is clamped to the E8M0 range [-127, 127]; an all-zero
    block gets scale code 0 and zero elements;
  * the sign bit of a code is set when the scaled input is negative, also
    when it rounds to zero (-0 in E4M3).

Layout used by the path: a [rows, d] tensor gives codes [rows, d] (uint8)
and scales [rows, d / 32] (uint8, block b covers columns 32 b .. 32 b + 31).
"""
import numpy as np

E4M3_MAX = 448.0
E4M3_EMAX = 8          # 448 = 1.75 * 2^8
BLOCK = 32


def e4m3_value(code: int) -> float:
    """Value of an E4M3 code from its fields (NaN for S.1111.111)."""
    code = int(code) & 0xFF
    s = -1.0 if code & 0x80 else 1.0
    e = (code >> 3) & 0xF
    m = code & 0x7
    if e == 0xF and m == 0x7:
        return float("nan")
    if e == 0:
        return s * (m / 8.0) * 2.0 ** -6           # subnormal: 0.mmm * 2^(1 - bias)
    return s * (1.0 + m / 8.0) * 2.0 ** (e - 7)    # normal: 1.mmm * 2^(e - bias)


# every finite non-negative E4M3 value, indexed by code 0 .. 126 (increasing)
_POS = np.array([e4m3_value(c) for c in range(0x7F)])


def e4m3_encode(y) -> np.ndarray:
    """Nearest E4M3 code of each element of y (float64), ties to the even code,
    saturating at 448."""
    y = np.asarray(y, dtype=np.float64)
    a = np.abs(y)
    hi = np.searchsorted(_POS, a, side="left")     # first value >= a
    hi = np.minimum(hi, len(_POS) - 1)
    lo = np.maximum(hi - 1, 0)
    d_lo = a - _POS[lo]
    d_hi = _POS[hi] - a
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0) & (hi != lo))
    code = np.where(pick_hi, hi, lo)
    code = np.where(a >= E4M3_MAX, 0x7E, code)
    code = code | np.where(y < 0, 0x80, 0)
    return code.astype(np.uint8)


def e4m3_decode(codes) -> np.ndarray:
    table = np.array([e4m3_value(c) for c in range(256)])
    return table[np.asarray(codes, dtype=np.int64)]


def shared_exponent(amax: np.ndarray) -> np.ndarray:
    """floor(log2(amax)) - 8, clamped to [-127, 127]; -127 where amax == 0."""
    amax = np.asarray(amax, dtype=np.float64)
    _, e = np.frexp(np.where(amax > 0, amax, 1.0))   # amax = m 2^e, m in [0.5, 1)
    se = (e - 1) - E4M3_EMAX
    se = np.where(amax > 0, se, -127)
    return np.clip(se, -127, 127).astype(np.int64)


def quantize(x: np.ndarray):
    """MXFP8 of x [..., d] (d a multiple of 32) along the last axis:
    (codes uint8 [..., d], scales uint8 [..., d / 32])."""
    x = np.asarray(x, dtype=np.float64)
    d = x.shape[-1]
    assert d % BLOCK == 0
    xb = x.reshape(x.shape[:-1] + (d // BLOCK, BLOCK))
    se = shared_exponent(np.max(np.abs(xb), axis=-1))
    y = xb / np.ldexp(1.0, se)[..., None]            # exact: division by a power of two
    codes = e4m3_encode(y).reshape(x.shape)
    scales = (se + 127).astype(np.uint8)
    return codes, scales


def dequantize(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """Values (float64) of MXFP8 codes and their block scales."""
    v = e4m3_decode(codes)
    d = v.shape[-1]
    vb = v.reshape(v.shape[:-1] + (d // BLOCK, BLOCK))
    x = vb * np.ldexp(1.0, np.asarray(scales, dtype=np.int64) - 127)[..., None]
    return x.reshape(v.shape)
