"""Number formats of the routed-MoE call, each written from its definition.

TEST INFRASTRUCTURE ONLY (see the package header).

The pages name the formats but do not define them: MXFP4 experts and
activations ("IQ2R: load GLM-5.3 packed MoE checkpoints with TP slicing",
status comments: the stock MXFP4 arm is A4W4), FP8 mid blocks with a scale
("glm53: FP8 mid hand-off ...", Modifications table, row "mid as FP8 once"),
BF16 outputs. The definitions used here are the public ones:

* E2M1 (OCP Microscaling Formats v1.0, FP4 element): sign bit 3, magnitudes
  0, 0.5, 1, 1.5, 2, 3, 4, 6 for codes 0..7.
* E8M0 (same spec, scale): value 2^(code - 127); code 255 is NaN.
* MX block quantization (same spec, section on conversion): shared scale
  X = 2^(floor(log2(amax)) - emax_elem), emax_elem = 2 for E2M1; elements
  v / X rounded to nearest, ties to even, saturating at 6.
* E4M3FN (OCP 8-bit floating point spec): bias 7, 3 mantissa bits, no
  infinities, max 448, codes 0x7F / 0xFF NaN; subnormals m * 2^-9.
* bfloat16: the top 16 bits of an IEEE binary32.

Parity pins (tests/test_oracle_formats.py): the E4M3 table and encoder against
torch.float8_e4m3fn (an independent implementation); bf16 rounding against
torch's binary32 -> bfloat16 cast; E2M1 midpoints and saturation against
hand-derived values; MX scale rule against closed-form cases.
"""

from __future__ import annotations

import numpy as np

# ---------------------------------------------------------------- E2M1 (FP4)
E2M1_MAG = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])


def e2m1_decode(codes: np.ndarray) -> np.ndarray:
    """4-bit codes (0..15, bit 3 = sign) -> float64."""
    c = np.asarray(codes).astype(np.int64)
    mag = E2M1_MAG[c & 7]
    return np.where(c & 8, -mag, mag)


def _nearest_even(mag: np.ndarray, table: np.ndarray) -> np.ndarray:
    """Index of the table value nearest to mag (table sorted ascending, from 0);
    a tie goes to the even index; above the table's end, the last index."""
    n = len(table)
    i = np.clip(np.searchsorted(table, mag, side="right") - 1, 0, n - 1)
    j = np.minimum(i + 1, n - 1)
    d_lo = mag - table[i]
    d_hi = table[j] - mag
    up = (j != i) & ((d_hi < d_lo) | ((d_hi == d_lo) & (j % 2 == 0)))
    return np.where(up, j, i)


def e2m1_encode(v: np.ndarray) -> np.ndarray:
    """float -> E2M1 code, round to nearest with ties to the even code,
    saturating to +-6; the sign bit is copied from v (so -0.0 -> code 8)."""
    v = np.asarray(v, dtype=np.float64)
    code = _nearest_even(np.abs(v), E2M1_MAG).astype(np.uint8)
    return np.where(np.signbit(v), code | np.uint8(8), code).astype(np.uint8)


def pack_fp4(codes: np.ndarray) -> np.ndarray:
    """[..., 2n] codes -> [..., n] bytes; element 2i in the low nibble."""
    c = np.asarray(codes, dtype=np.uint8)
    return (c[..., 0::2] | (c[..., 1::2] << 4)).astype(np.uint8)


def unpack_fp4(packed: np.ndarray) -> np.ndarray:
    """[..., n] bytes -> [..., 2n] codes (low nibble first)."""
    p = np.asarray(packed, dtype=np.uint8)
    out = np.empty(p.shape[:-1] + (2 * p.shape[-1],), dtype=np.uint8)
    out[..., 0::2] = p & 15
    out[..., 1::2] = p >> 4
    return out


# ---------------------------------------------------------------- E8M0
def e8m0_decode(codes: np.ndarray) -> np.ndarray:
    c = np.asarray(codes).astype(np.int64)
    if np.any(c == 255):
        raise ValueError("E8M0 code 255 is NaN")
    return np.ldexp(1.0, c - 127)


# ---------------------------------------------------------------- E4M3FN
def e4m3_decode(codes: np.ndarray) -> np.ndarray:
    """8-bit E4M3FN codes -> float64 (NaN for 0x7F / 0xFF)."""
    c = np.asarray(codes).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    exp = (c >> 3) & 15
    man = c & 7
    mag = np.where(exp == 0, np.ldexp(man.astype(np.float64), -9),
                   np.ldexp(1.0 + man / 8.0, exp - 7))
    mag = np.where((c & 0x7F) == 0x7F, np.nan, mag)
    return sign * mag


E4M3_POS = e4m3_decode(np.arange(127))  # codes 0..126: 0 .. 448 ascending
E4M3_MAX = 448.0


def e4m3_encode(v: np.ndarray) -> np.ndarray:
    """float -> E4M3FN code: nearest finite value, ties to the even code,
    saturating to +-448; the sign bit is copied from v."""
    v = np.asarray(v, dtype=np.float64)
    if np.any(np.isnan(v)):
        raise ValueError("NaN has no saturating E4M3 code")
    code = _nearest_even(np.abs(v), E4M3_POS).astype(np.uint8)
    return np.where(np.signbit(v), code | np.uint8(0x80), code).astype(np.uint8)


# ---------------------------------------------------------------- bfloat16
def bf16_decode(bits: np.ndarray) -> np.ndarray:
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return b.view(np.float32).astype(np.float64)


def bf16_encode(v: np.ndarray) -> np.ndarray:
    """float64 -> bf16 bits, one rounding to nearest even (no binary32 step).

    bf16 keeps 8 significant bits; normal exponents down to 2^-126, below
    that a fixed quantum of 2^-133; overflow past the largest finite -> inf.
    """
    v = np.asarray(v, dtype=np.float64)
    _, e = np.frexp(v)  # v = m 2^e, 0.5 <= |m| < 1
    q = np.maximum(e - 8, -133)
    r = np.ldexp(np.rint(np.ldexp(v, -q)), q)  # numpy rint: half to even
    with np.errstate(over="ignore"):
        f = r.astype(np.float32)
    return (f.view(np.uint32) >> 16).astype(np.uint16)


# ---------------------------------------------------------------- MX (FP4) blocks
def mx_fp4_quantize(x: np.ndarray, block: int = 32):
    """MX quantization along the last axis in blocks of 32.

    Returns (codes [..., n] uint8 E2M1, scale codes [..., n/32] uint8 E8M0).
    Scale exponent = floor(log2(amax)) - 2, taken exactly from the binary
    exponent; clamped to the E8M0 range [-127, 127]; an all-zero block gets
    code 0 and zero elements. Elements x * 2^-exp go to E2M1 (RNE, saturating).
    """
    x = np.asarray(x, dtype=np.float64)
    n = x.shape[-1]
    assert n % block == 0
    xb = x.reshape(x.shape[:-1] + (n // block, block))
    amax = np.abs(xb).max(-1)
    _, ex = np.frexp(amax)  # amax = m 2^ex, m in [0.5, 1): floor(log2 amax) = ex - 1
    sexp = np.where(amax > 0, ex - 1 - 2, -127)
    scode = np.clip(sexp + 127, 0, 254)
    v = np.ldexp(xb, -(scode - 127)[..., None])
    codes = e2m1_encode(v).reshape(x.shape)
    return codes, scode.astype(np.uint8)


def mx_fp4_decode(codes: np.ndarray, scodes: np.ndarray, block: int = 32) -> np.ndarray:
    """E2M1 codes [..., n] and E8M0 scale codes [..., n/32] -> float64 values."""
    v = e2m1_decode(codes)
    n = v.shape[-1]
    s = e8m0_decode(scodes)
    return (v.reshape(v.shape[:-1] + (n // block, block)) * s[..., None]).reshape(v.shape)


# ---------------------------------------------------------------- FP8 blocks
def fp8_block_quantize(h: np.ndarray, block: int = 128):
    """Per block of 128 along the last axis: s = fl32(amax / 448) (IEEE
    binary32 division), q = E4M3(fl32(h / s)) (RNE, saturating); an all-zero
    block gets s = 0 and zero codes.

    Returns (codes [..., n] uint8, scales [..., n/128] float32).
    """
    h = np.asarray(h, dtype=np.float32)
    n = h.shape[-1]
    assert n % block == 0
    hb = h.reshape(h.shape[:-1] + (n // block, block))
    amax = np.abs(hb).max(-1)
    s = (amax / np.float32(E4M3_MAX)).astype(np.float32)
    safe = np.where(s > 0, s, np.float32(1.0)).astype(np.float32)
    v = (hb / safe[..., None]).astype(np.float32)
    v = np.where(s[..., None] > 0, v, np.float32(0.0))
    codes = e4m3_encode(v.astype(np.float64)).reshape(h.shape)
    return codes, s


def fp8_block_decode(codes: np.ndarray, scales: np.ndarray, block: int = 128) -> np.ndarray:
    v = e4m3_decode(codes)
    n = v.shape[-1]
    return (v.reshape(v.shape[:-1] + (n // block, block)) *
            np.asarray(scales, np.float64)[..., None]).reshape(v.shape)
