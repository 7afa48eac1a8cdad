"""Pins for the oracle's activation quantizers."""
import numpy as np
import pytest

from brute import E2M1, int8_bruteforce, nearest_e2m1_code, unpack_codes


def test_int8_properties_and_bruteforce(oracle):
    rng = np.random.default_rng(0)
    v = (rng.standard_normal((6, 96)) * rng.uniform(0.1, 100, (6, 1))).astype(np.float32)
    v[3, 7] = -np.abs(v[3]).max() * 1.0  # ties for amax with a negative sign
    q, s = oracle.quant_int8(v)
    for r in range(v.shape[0]):
        amax = np.abs(v[r]).max()
        assert s[r] == np.float32(amax) / np.float32(127)
        assert np.abs(q[r]).max() == 127
        assert np.array_equal(q[r].astype(np.int64), int8_bruteforce(v[r], s[r]))
        err = np.abs(v[r].astype(np.float64) - q[r] * np.float64(s[r]))
        assert np.all(err <= 0.5 * s[r] * (1 + 1e-6) + 1e-30)


def test_int8_zero_row(oracle):
    q, s = oracle.quant_int8(np.zeros((2, 64), np.float32))
    assert np.all(q == 0) and np.all(s == 0)


def test_mxfp4_against_bruteforce(oracle):
    rng = np.random.default_rng(1)
    v = (rng.standard_normal((5, 256)) * np.exp2(rng.integers(-10, 12, (5, 1)))).astype(np.float32)
    codes, scales = oracle.quant_mxfp4(v)
    c = unpack_codes(codes)
    for r in range(v.shape[0]):
        for b in range(v.shape[1] // 32):
            blk = v[r, 32 * b: 32 * b + 32].astype(np.float64)
            amax = np.abs(blk).max()
            e = int(scales[r, b])
            # shared exponent: amax * 2^(127-e) in [4, 8)
            assert 4.0 <= amax * 2.0 ** (127 - e) < 8.0
            for i in range(32):
                vs = blk[i] * 2.0 ** (127 - e)
                assert c[r, 32 * b + i] == nearest_e2m1_code(vs), (r, b, i, vs)


@pytest.mark.parametrize("vs,val", [(0.25, 0.0), (0.75, 1.0), (1.25, 1.0), (1.75, 2.0), (2.5, 2.0),
                                    (3.5, 4.0), (5.0, 4.0), (5.01, 6.0), (7.9, 6.0), (-0.25, -0.0),
                                    (-2.5, -2.0), (0.2499, 0.0), (0.2501, 0.5)])
def test_mxfp4_constructed_midpoints(oracle, vs, val):
    # a block whose amax is 4.0 has shared exponent 0 (scale byte 127): the
    # element is quantized unscaled
    blk = np.zeros((1, 32), np.float32)
    blk[0, 0] = 4.0
    blk[0, 5] = vs
    codes, scales = oracle.quant_mxfp4(blk)
    assert scales[0, 0] == 127
    got = E2M1[unpack_codes(codes)[0, 5]]
    assert got == val and np.signbit(got) == np.signbit(val)


def test_mxfp4_power_of_two_amax_and_zero_block(oracle):
    blk = np.zeros((2, 32), np.float32)
    blk[0, :] = 0.0
    blk[1, 3] = 2.0 ** -20
    codes, scales = oracle.quant_mxfp4(blk)
    assert scales[0, 0] == 0 and np.all(codes[0] == 0)
    assert scales[1, 0] == 127 - 20 - 2
    assert E2M1[unpack_codes(codes)[1, 3]] == 4.0
