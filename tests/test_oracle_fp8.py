"""Pins for the oracle's FP8 pieces: the E4M3 codec, the Hadamard rotation and block quantisation.

- codec: decoded values and encoder rounding are checked against torch's
  float8_e4m3fn (a library implementation of the same OCP format), against
  fixed values of the format (448 is the largest finite value, as the pages
  state), and by exhaustive round trips;
- Hadamard: against scipy.linalg.hadamard, orthonormality, and the score
  invariance (QM)(KM)^T = QK^T stated on the FlashAttention 2 & 3 page;
- block quantisation: the scale rule amax/448 (1 for an all-zero block), the
  rounding error bound of E4M3, ragged last blocks, and the page's claim that
  rotating before quantising lowers the error when a feature has outliers.
"""

import math

import numpy as np
import pytest
import torch

from oracle.e4m3 import E4M3_MAX, e4m3_decode, e4m3_encode
from oracle.fp8 import block_dequantize, block_quantize, fp8_reference
from oracle.hadamard import incoherent_rotate, sylvester_hadamard


def torch_decode(codes):
    return torch.from_numpy(np.asarray(codes, np.uint8)).view(torch.float8_e4m3fn).to(torch.float64).numpy()


def torch_encode(x32):
    return torch.from_numpy(np.asarray(x32, np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


# ---------------------------------------------------------------- codec

def test_decode_fixed_values():
    d = e4m3_decode(np.array([0x7E, 0xFE, 0x01, 0x08, 0x38, 0x00, 0x80, 0x7F, 0xFF], np.uint8))
    assert d[0] == E4M3_MAX == 448.0 and d[1] == -448.0
    assert d[2] == 2.0 ** -9 and d[3] == 2.0 ** -6 and d[4] == 1.0
    assert d[5] == 0.0 and d[6] == 0.0 and math.copysign(1, d[6]) < 0
    assert np.isnan(d[7]) and np.isnan(d[8])


def test_decode_all_codes_matches_torch():
    codes = np.arange(256, dtype=np.uint8)
    ours, ref = e4m3_decode(codes), torch_decode(codes)
    assert np.array_equal(np.isnan(ours), np.isnan(ref))
    ok = ~np.isnan(ref)
    assert np.array_equal(ours[ok], ref[ok])
    assert np.nanmax(ours) == 448.0


def test_encode_roundtrip_all_finite_codes():
    codes = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], np.uint8)
    assert len(codes) == 254
    assert np.array_equal(e4m3_encode(e4m3_decode(codes)), codes)


def test_encode_matches_torch_in_range():
    rng = np.random.default_rng(0)
    x = np.concatenate([
        rng.uniform(-448, 448, 20000), rng.standard_normal(20000) * 0.01,
        rng.standard_normal(20000) * 2.0 ** -8,
    ]).astype(np.float32)
    # every midpoint between neighbouring finite values, and points just beside them
    vals = np.unique(np.abs(e4m3_decode(np.arange(0x7F, dtype=np.uint8))))
    mids = ((vals[1:] + vals[:-1]) / 2).astype(np.float32)
    x = np.concatenate([x, mids, -mids, np.nextafter(mids, np.float32(0)), np.nextafter(mids, np.float32(1e9))])
    assert np.array_equal(e4m3_encode(x), torch_encode(x))


def test_encode_ties_to_even_and_saturation():
    assert e4m3_encode(np.float32(1.0625)) == 0x38     # between 1.0 (0x38) and 1.125 (0x39)
    assert e4m3_encode(np.float32(1.1875)) == 0x3A     # between 1.125 and 1.25 (0x3a)
    assert e4m3_encode(np.float32(2.0 ** -10)) == 0x00  # half the smallest subnormal: ties to 0
    assert e4m3_encode(np.float32(1.5 * 2.0 ** -10)) == 0x01
    for big in (448.0, 449.0, 464.0, 480.0, 1e9, np.inf):
        assert e4m3_encode(np.float32(big)) == 0x7E
        assert e4m3_encode(np.float32(-big)) == 0xFE
    assert e4m3_encode(np.float32(np.nan)) == 0x7F
    assert e4m3_encode(np.float32(-0.0)) == 0x80


# ---------------------------------------------------------------- Hadamard rotation

@pytest.mark.parametrize("n", [1, 2, 4, 8, 64, 128, 256])
def test_hadamard_matches_scipy(n):
    from scipy.linalg import hadamard

    assert np.array_equal(sylvester_hadamard(n, normalized=False), hadamard(n).astype(np.float64))
    h = sylvester_hadamard(n)
    np.testing.assert_allclose(h @ h.T, np.eye(n), atol=1e-14)


def test_rotation_preserves_scores_and_norms():
    rng = np.random.default_rng(1)
    q, k = rng.standard_normal((2, 50, 128))
    signs = np.where(rng.random(128) > 0.5, 1.0, -1.0)
    qr, kr = incoherent_rotate(q, signs), incoherent_rotate(k, signs)
    assert np.abs(qr @ kr.T - q @ k.T).max() < 1e-12
    np.testing.assert_allclose(np.linalg.norm(qr, axis=1), np.linalg.norm(q, axis=1), rtol=1e-13)
    # the signs matter for the rotated values (but not for the scores)
    assert np.abs(incoherent_rotate(q, -signs) - qr).max() > 0.1


def test_rotation_spreads_a_spike():
    d = 128
    x = np.zeros((1, d))
    x[0, 7] = 25.0
    r = incoherent_rotate(x, np.ones(d))
    np.testing.assert_allclose(np.abs(r), 25.0 / math.sqrt(d), rtol=1e-14)


def test_rotation_lowers_fp8_error_with_outlier_feature():
    # the first page's demonstration: an outlier feature x25 in Q and K
    rng = np.random.default_rng(2)
    d = 128
    q = rng.standard_normal((64, d)).astype(np.float32)
    k = rng.standard_normal((64, d)).astype(np.float32)
    q[:, 7] *= 25.0
    k[:, 7] *= 25.0
    ref = q.astype(np.float64) @ k.T.astype(np.float64)
    signs = np.where(rng.random(d) > 0.5, 1.0, -1.0)

    def deq(x):
        c, s = block_quantize(x[None])
        return block_dequantize(c, s)[0]

    err_plain = np.abs(deq(q) @ deq(k).T - ref).mean()
    qr = incoherent_rotate(q, signs).astype(np.float32)
    kr = incoherent_rotate(k, signs).astype(np.float32)
    err_rot = np.abs(deq(qr) @ deq(kr).T - ref).mean()
    assert err_rot < 0.7 * err_plain


# ---------------------------------------------------------------- block quantisation

def test_block_scale_rule():
    x = np.zeros((1, 130, 16), np.float32)
    x[0, 3, 5] = -7.0            # block 0 amax 7
    x[0, 70, 0] = 0.5            # block 1 amax 0.5
    codes, s = block_quantize(x)  # block 2 (rows 128, 129) is all zero
    assert s.shape == (1, 3)
    assert s[0, 0] == np.float32(7.0) / np.float32(448.0)
    assert s[0, 1] == np.float32(0.5) / np.float32(448.0)
    assert s[0, 2] == 1.0
    assert codes[0, 3, 5] == 0xFE and codes[0, 70, 0] == 0x7E
    assert (codes[0, 128:] == 0).all()


def test_block_quantize_error_bound():
    rng = np.random.default_rng(3)
    x = (rng.standard_normal((2, 3, 200, 32)) * rng.uniform(0.01, 100, (2, 3, 200, 1))).astype(np.float32)
    codes, s = block_quantize(x)
    deq = block_dequantize(codes, s)
    row_s = np.repeat(s.astype(np.float64), 64, axis=-1)[..., :200, None]
    y = np.abs(x / row_s)
    # E4M3: 3 mantissa bits -> relative half-step 2^-4 for normals, absolute 2^-10 for subnormals
    bound = np.maximum(y * 2.0 ** -4, 2.0 ** -10) * row_s * (1 + 1e-6)
    assert (np.abs(deq - x) <= bound).all()
    assert (np.abs(x / row_s) <= 448.0 * (1 + 1e-6)).all()


def test_fp8_reference_small_case():
    rng = np.random.default_rng(4)
    q, k, v = (rng.standard_normal((1, 2, 128, 64)).astype(np.float32) for _ in range(3))
    signs = np.where(rng.random(64) > 0.5, 1.0, -1.0)
    res = fp8_reference(q, k, v, signs, 1 / 8, False)
    # input quantisation alone moves the result; with only 128 keys it averages out less
    # than at the fp8 workload's 8192, so this is a sanity bound, not the contract tolerance
    err = np.abs(res["O_deq"] - res["O_true"])
    assert err.max() < 0.1 and err.mean() < 0.01
    assert res["q8"].dtype == np.uint8 and res["sq"].shape == (1, 2, 2)
