"""fp8 e4m3fn block quantisation of Q and K, fp64/fp32 reference (test infrastructure only).

Source: FlashAttention-3 abstract (Daily Papers listing): block quantisation for
FP8 attention; the combined-sweep workload quantises Q and K to fp8 e4m3 with one
scale per 64-token block. The e4m3fn format (OCP 8-bit floating point): sign bit,
4 exponent bits with bias 7, 3 mantissa bits, subnormals m/8 * 2^-6, no infinities,
S.1111.111 is NaN, so the largest finite magnitude is 1.75 * 2^8 = 448.

Reading (the pages fix only "per-block scale"): scale = amax / 448 over the 64 x D
values of the block, computed in fp32 (an all-zero block gets scale 1); each value
is divided by the scale in fp32 (correctly rounded) and encoded round-to-nearest-even
(ties to the code with an even mantissa), saturating at +-448. Both the rounding of
the quotient and the choice of the code are taken in fp32, the precision the GPU
takes them in.

Incoherent processing (FlashAttention-3 abstract, Daily Papers listing, named beside block
quantisation with no formula; reading): Q and K are multiplied by the same orthogonal
matrix M = diag(s) H / sqrt(D) before quantisation, H the D x D Sylvester Hadamard matrix
and s a vector of random signs that the caller draws, so that Q M (K M)^T = Q K^T while
a few large channels are spread over all of them. Each row x becomes y = H (s . x),
formed by the fast Walsh-Hadamard transform in fp32 (stages of stride 1, 2, ..., D/2,
each pair (i, i + stride) -> (a + b, a - b)), the order and precision the GPU uses, so
that both sides take the same fp8 codes; the 1/D of M M^T is carried by the key side's
scales (a power of two, exact).
"""
import numpy as np

E4M3_MAX = 448.0


def e4m3fn_values() -> np.ndarray:
    """Value of every code 0..255 (NaN for the two NaN codes), from the format definition."""
    vals = np.empty(256)
    for c in range(256):
        s = -1.0 if c & 0x80 else 1.0
        e = (c >> 3) & 0xF
        m = c & 0x7
        if e == 0xF and m == 0x7:
            vals[c] = np.nan
        elif e == 0:
            vals[c] = s * (m / 8.0) * 2.0 ** -6
        else:
            vals[c] = s * (1.0 + m / 8.0) * 2.0 ** (e - 7)
    return vals


_VALS = e4m3fn_values()
_POS_CODES = np.arange(0, 0x7F)                 # +0 .. +448, ascending values
_POS_VALS = _VALS[_POS_CODES]


def encode_e4m3fn(x) -> np.ndarray:
    """Nearest e4m3fn code of each value (ties to the even code), saturating at +-448;
    NaN -> 0x7F. Signed zeros keep their sign."""
    x = np.asarray(x, dtype=np.float64)
    a = np.minimum(np.abs(x), E4M3_MAX)
    hi = np.clip(np.searchsorted(_POS_VALS, a, side="left"), 0, len(_POS_VALS) - 1)   # first value >= a
    lo = np.maximum(hi - 1, 0)
    d_lo = a - _POS_VALS[lo]
    d_hi = _POS_VALS[hi] - a
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (_POS_CODES[hi] % 2 == 0))
    code = np.where(pick_hi, _POS_CODES[hi], _POS_CODES[lo]).astype(np.uint8)
    code = np.where(np.signbit(x), code | 0x80, code).astype(np.uint8)
    return np.where(np.isnan(x), np.uint8(0x7F), code).astype(np.uint8)


def decode_e4m3fn(codes) -> np.ndarray:
    return _VALS[np.asarray(codes, dtype=np.uint8)]


def quantize_blocks(x, n: int = 64):
    """x [..., S, D] (any float) -> (codes uint8 [..., S, D], scales float32 [..., S/n])."""
    x32 = np.asarray(x, dtype=np.float32)
    *lead, S, D = x32.shape
    blk = x32.reshape(*lead, S // n, n, D)
    amax = np.abs(blk).max(axis=(-2, -1))
    scales = np.where(amax > 0, amax / np.float32(E4M3_MAX), np.float32(1.0)).astype(np.float32)
    q = (blk / scales[..., None, None]).astype(np.float32)
    codes = encode_e4m3fn(q).reshape(*lead, S, D)
    return codes, scales


def fwht_rows(x, signs) -> np.ndarray:
    """y = H (s . x) for every row of x [..., D] (D a power of two), in fp32 with the stage
    order stated above."""
    y = (np.asarray(x, dtype=np.float32) * np.asarray(signs, dtype=np.float32)).astype(np.float32)
    D = y.shape[-1]
    assert D & (D - 1) == 0, "D must be a power of two"
    h = 1
    while h < D:
        v = y.reshape(*y.shape[:-1], D // (2 * h), 2, h)
        a, b = v[..., 0, :], v[..., 1, :]
        y = np.stack([a + b, a - b], axis=-2).reshape(*y.shape[:-1], D).astype(np.float32)
        h *= 2
    return y


def quantize_blocks_rotated(x, signs, key_side: bool, n: int = 64):
    """Incoherent processing then block quantisation: codes and scales of fwht_rows(x, s);
    on the key side the scales also carry the 1/D of M M^T, so that dequantised q . k
    equals q . k of the unrotated rows."""
    y = fwht_rows(x, signs)
    codes, scales = quantize_blocks(y, n)
    if key_side:
        scales = (scales * np.float32(1.0 / y.shape[-1])).astype(np.float32)
    return codes, scales
