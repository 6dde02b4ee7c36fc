"""Pins for the fp8 e4m3fn block quantiser of the oracle (CPU only).

The encoder searches the table of code values built from the format definition;
it is checked against torch's own float8_e4m3fn cast (a library routine) on values
of every kind inside the format's range, and by round trips and closed-form
properties; the block quantiser against its defining properties.
"""
import numpy as np
import torch

from oracle.fp8 import (decode_e4m3fn, e4m3fn_values, encode_e4m3fn, fwht_rows, quantize_blocks,
                        quantize_blocks_rotated)


def _torch_codes(x32: np.ndarray) -> np.ndarray:
    return torch.from_numpy(x32).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def test_format_table():
    v = e4m3fn_values()
    assert np.isnan(v[0x7F]) and np.isnan(v[0xFF])
    assert v[0x7E] == 448.0 and v[0xFE] == -448.0
    assert v[0x01] == 2.0 ** -9 and v[0x08] == 2.0 ** -6 and v[0x38] == 1.0
    fin = v[np.isfinite(v)]
    assert len(fin) == 254 and len(set(np.abs(fin))) == 127     # +-0 .. 448


def test_round_trip_of_every_code():
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)
    assert np.array_equal(encode_e4m3fn(decode_e4m3fn(codes)), codes)


def test_matches_torch_cast_inside_the_range():
    rng = np.random.default_rng(0)
    v = e4m3fn_values()
    pos = np.sort(v[np.isfinite(v) & (v >= 0)])
    mids = (pos[1:] + pos[:-1]) / 2                              # exact ties (representable in fp32)
    x = np.concatenate([
        rng.uniform(-463.9, 463.9, 20000),
        rng.normal(0, 1, 20000),
        rng.uniform(-2.0 ** -6, 2.0 ** -6, 5000),                  # subnormal range
        mids, -mids, pos, -pos,
        np.nextafter(mids, 0), np.nextafter(mids, 1000),           # just below / above each tie
        [0.0, -0.0, 447.9, 448.0, 450.0, 463.99, -463.99],
    ]).astype(np.float32)
    ours = encode_e4m3fn(x)
    assert np.array_equal(ours, _torch_codes(x))


def test_saturation_and_nan():
    x = np.array([464.0, 500.0, 1e30, -1e30, np.inf, -np.inf, np.nan], dtype=np.float32)
    assert list(encode_e4m3fn(x)) == [0x7E, 0x7E, 0x7E, 0xFE, 0x7E, 0xFE, 0x7F]


def test_block_quantiser_properties():
    rng = np.random.default_rng(1)
    x = rng.standard_normal((2, 3, 256, 64)).astype(np.float32) * rng.uniform(0.01, 100, (2, 3, 1, 1))
    x[0, 1, 64:128] = 0.0                                          # an all-zero block
    codes, scales = quantize_blocks(x, 64)
    assert codes.dtype == np.uint8 and scales.dtype == np.float32 and scales.shape == (2, 3, 4)
    assert scales[0, 1, 1] == 1.0 and np.all(codes[0, 1, 64:128] == 0)
    blk = x.reshape(2, 3, 4, 64, 64)
    cb = codes.reshape(2, 3, 4, 64, 64)
    for idx in np.ndindex(2, 3, 4):
        if not np.any(blk[idx]):
            continue
        assert scales[idx] == np.float32(np.abs(blk[idx]).max()) / np.float32(448.0)
        amax_pos = np.unravel_index(np.abs(blk[idx]).argmax(), (64, 64))
        assert cb[idx][amax_pos] & 0x7F == 0x7E                    # the block maximum maps to 448
        dec = decode_e4m3fn(cb[idx]) * scales[idx]
        err = np.abs(dec - blk[idx])
        # half a mantissa step: 2^-4 relative in the normal range, 2^-10 * scale below it
        assert np.all(err <= np.maximum(np.abs(blk[idx]) * 2.0 ** -4, scales[idx] * 2.0 ** -10) * (1 + 1e-6))


def test_block_quantiser_equals_torch_reference_path():
    # scale and quotient in fp32, then torch's float8 cast: the same definition by library routines
    rng = np.random.default_rng(2)
    x = torch.from_numpy(rng.standard_normal((1, 2, 192, 128)).astype(np.float32)).to(torch.bfloat16)
    codes, scales = quantize_blocks(x.float().numpy(), 64)
    xf = x.float().reshape(1, 2, 3, 64, 128)
    amax = xf.abs().amax(dim=(3, 4))
    ts = torch.where(amax > 0, amax / 448.0, torch.ones_like(amax))
    tq = (xf / ts[..., None, None]).to(torch.float8_e4m3fn).view(torch.uint8).reshape(1, 2, 192, 128)
    assert np.array_equal(scales, ts.numpy())
    assert np.array_equal(codes, tq.numpy())


# --------------------------------------------------------------------------- incoherent processing
def test_fwht_equals_the_hadamard_matrix_product():
    """fwht_rows(x, s) = H (s . x) with H from scipy's Sylvester construction (computed in
    fp64 there): equal up to the fp32 rounding of the butterflies."""
    from scipy.linalg import hadamard
    rng = np.random.default_rng(0)
    for D in (2, 8, 64, 128):
        x = rng.normal(0.0, 1.0, (5, D)).astype(np.float32)
        s = rng.choice([-1.0, 1.0], D)
        ref = (x.astype(np.float64) * s) @ hadamard(D).T.astype(np.float64)
        got = fwht_rows(x, s).astype(np.float64)
        assert np.allclose(got, ref, rtol=0, atol=1e-5 * np.sqrt(D) * np.abs(x).max())


def test_fwht_special_rows_and_orthogonality():
    """A unit row e_j with all signs +1 maps to column j of H (entries +-1, exact); the
    transform with signs is orthogonal up to 1/D: <y_q, y_k> = D <q, k>, |y|^2 = D |x|^2."""
    from scipy.linalg import hadamard
    D = 64
    Hm = hadamard(D)
    for j in (0, 1, 17, 63):
        e = np.zeros((1, D), dtype=np.float32)
        e[0, j] = 1.0
        assert np.array_equal(fwht_rows(e, np.ones(D))[0], Hm[:, j].astype(np.float32))
    rng = np.random.default_rng(1)
    s = rng.choice([-1.0, 1.0], D)
    q = rng.normal(0.0, 1.0, (7, D)).astype(np.float32)
    k = rng.normal(0.0, 1.0, (7, D)).astype(np.float32)
    yq, yk = fwht_rows(q, s).astype(np.float64), fwht_rows(k, s).astype(np.float64)
    assert np.allclose(yq @ yk.T, D * (q.astype(np.float64) @ k.astype(np.float64).T), rtol=1e-5, atol=1e-4)
    assert np.allclose((yq ** 2).sum(1), D * (q.astype(np.float64) ** 2).sum(1), rtol=1e-5)


def test_rotated_quantisation_lowers_attention_error_with_outliers():
    """The point of the rotation (FlashAttention-3 abstract: lower fp8 error than a plain fp8
    attention): Gaussian Q, K, V with 1% of the entries of Q and K scaled by 10 (outliers at
    random places). Attention from the dequantised fp8 Q and K is compared with attention in
    fp64 on the exact inputs; the rotated quantisation (key scales carrying the 1/D) lowers the
    RMS error well below the plain block quantisation's, and changes nothing much on
    Gaussian inputs without outliers."""
    rng = np.random.default_rng(2)
    S, D = 256, 128

    def attn(q, k, v):
        L = q @ k.T / np.sqrt(D)
        P = np.exp(L - L.max(1, keepdims=True))
        return (P / P.sum(1, keepdims=True)) @ v

    def deq(c, sc):
        return (decode_e4m3fn(c).reshape(-1, 64, D) * sc[:, None, None]).reshape(c.shape)

    def errors(q, k, v, s):
        ref = attn(q, k, v)
        (cq, sq), (ck, sk) = quantize_blocks(q), quantize_blocks(k)
        (rq, rsq), (rk, rsk) = quantize_blocks_rotated(q, s, key_side=False), quantize_blocks_rotated(k, s, key_side=True)
        rms = lambda o: float(np.sqrt(((o - ref) ** 2).mean()))
        return rms(attn(deq(cq, sq), deq(ck, sk), v)), rms(attn(deq(rq, rsq), deq(rk, rsk), v))

    s = rng.choice([-1.0, 1.0], D)
    q, k, v = rng.normal(0.0, 1.0, (3, S, D))
    for x in (q, k):
        x[rng.random(x.shape) < 0.01] *= 10.0
    plain, rot = errors(q, k, v, s)
    assert rot < 0.75 * plain, (plain, rot)
    q, k, v = rng.normal(0.0, 1.0, (3, S, D))
    plain, rot = errors(q, k, v, s)
    assert 0.8 * plain < rot < 1.25 * plain, (plain, rot)
