"""Pins of the oracle's block-scaled FP8 dense projection (MXFP8: E4M3
elements, one E8M0 scale per 32 along K) against things other than itself:
torch's own float8_e4m3fn conversion (an independent implementation of the
OCP E4M3 format), brute-force searches, numpy float64 matmuls and closed
forms."""
import numpy as np
import pytest
import torch

import oracle


def torch_e4m3(codes: np.ndarray) -> np.ndarray:
    return torch.from_numpy(codes.astype(np.uint8)).view(torch.float8_e4m3fn).float().numpy()


def test_e4m3_decode_all_codes():
    codes = np.arange(256, dtype=np.uint8)
    ours, ref = oracle.e4m3_table(), torch_e4m3(codes)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan) and nan.sum() == 2  # 0x7f, 0xff
    assert np.array_equal(ours[~nan].view(np.uint32), ref[~nan].view(np.uint32))  # incl. the sign of -0
    assert ours[0x7e] == 448.0 and ours[0x01] == 2.0 ** -9


def test_mxfp8_rounding_matches_torch_in_range():
    """Elements whose scaled magnitude is below 464 (where rounding to
    nearest-even stays finite) round as torch rounds fp32 to E4M3."""
    rng = np.random.default_rng(3)
    v = (rng.standard_normal((64, 256)) * np.exp2(rng.integers(-20, 21, (64, 256)))).astype(np.float32)
    v[5, :32] = 0.0  # an all-zero block
    codes, scales = oracle.quant_mxfp8(v)
    deq = oracle.e4m3_table()[codes]
    scaled = v * np.exp2(127.0 - np.repeat(scales.astype(np.float64), 32, axis=1))
    ref = torch.from_numpy(scaled.astype(np.float32)).to(torch.float8_e4m3fn).float().numpy()
    inr = np.abs(scaled) < 464
    assert inr.mean() > 0.9
    assert np.array_equal(deq[inr], ref[inr])
    # above it: saturation at 448 with the sign kept (torch gives NaN there)
    assert np.all(np.abs(deq[~inr]) == 448.0)
    assert np.array_equal(np.signbit(deq[~inr]), np.signbit(v[~inr]))
    assert np.all(codes[5, :32] == 0) and scales[5, 0] == 0


def test_mxfp8_scale_rule_on_powers_of_two():
    """A block whose largest magnitude is 2^j gets the scale byte j - 8 + 127
    and that element encodes 256 = 2^8 (code 0x78) exactly."""
    for j in (-100, -20, -1, 0, 1, 7, 30, 100):
        blk = np.full((1, 32), 2.0 ** (j - 3), np.float32)
        blk[0, 7] = -(2.0 ** j)
        codes, scales = oracle.quant_mxfp8(blk)
        assert scales[0, 0] == j - 8 + 127
        assert codes[0, 7] == 0xF8  # -256
        assert oracle.e4m3_table()[codes[0, 0]] == 32.0


def test_mxfp8_ties_to_even_brute_force():
    """Midpoints between neighbouring E4M3 magnitudes round to the code with
    an even mantissa; a brute-force nearest search over the grid agrees on
    random values."""
    tab = oracle.e4m3_table()[:127].astype(np.float64)  # finite magnitudes, ascending
    mids = (tab[:-1] + tab[1:]) / 2
    # place each midpoint in a block whose amax is 256 (scale byte 127 - 0 = 127 -> scale 1 with amax 2^8)
    for i0 in range(0, len(mids), 31):
        chunk = mids[i0:i0 + 31]
        blk = np.zeros((1, 32), np.float32)
        blk[0, 0] = 256.0
        blk[0, 1:1 + len(chunk)] = chunk
        codes, scales = oracle.quant_mxfp8(blk)
        assert scales[0, 0] == 127
        for j, m in enumerate(chunk):
            lo = np.searchsorted(tab, m) - 1
            want = lo if lo % 2 == 0 else lo + 1
            assert codes[0, 1 + j] == want, (m, codes[0, 1 + j], want)
    rng = np.random.default_rng(4)
    v = rng.uniform(-447, 447, (1, 256)).astype(np.float32)
    v[0, ::32] = 300.0  # amax in [256, 512): scale byte 127, values unscaled
    codes, _ = oracle.quant_mxfp8(v)
    for k in range(256):
        a = abs(float(v[0, k]))
        d = np.abs(tab - a)
        best = np.flatnonzero(d == d.min())
        want = best[0] if len(best) == 1 else [b for b in best if b % 2 == 0][0]
        assert codes[0, k] & 0x7F == want


def dequant(codes, scales):
    vals = torch_e4m3(codes).astype(np.float64)
    return vals * np.exp2(np.repeat(scales.astype(np.float64), 32, axis=1) - 127.0)


@pytest.mark.parametrize("M,N,K", [(3, 8, 64), (17, 40, 256), (5, 64, 1024)])
def test_dense_equals_float64_matmul(M, N, K):
    rng = np.random.default_rng(M * N + K)
    x = (rng.standard_normal((M, K)) * np.exp2(rng.integers(-3, 4, (M, K)))).astype(np.float32)
    xq, xs = oracle.quant_mxfp8(x)
    wq = rng.integers(0, 256, (N, K)).astype(np.uint8)
    wq[(wq & 0x7F) == 0x7F] ^= 1  # no NaN codes
    ws = rng.integers(117, 126, (N, K // 32)).astype(np.uint8)
    y, bound = oracle.dense_mxfp8(xq, xs, wq, ws, bound=True)
    ref = dequant(xq, xs) @ dequant(wq, ws).T
    # one rounding of the (float64-exact) value: within half an fp32 ulp plus
    # float64 summation noise
    assert np.all(np.abs(y.astype(np.float64) - ref) <= np.abs(ref) * 2.0 ** -24 + bound * 1e-15)
    assert np.all(bound >= np.abs(ref) * (1 - 1e-12))


def test_dense_one_hot_and_scale_doubling():
    rng = np.random.default_rng(9)
    K, N = 128, 16
    wq = rng.integers(0, 256, (N, K)).astype(np.uint8)
    wq[(wq & 0x7F) == 0x7F] ^= 1
    ws = rng.integers(117, 126, (N, K // 32)).astype(np.uint8)
    wd = dequant(wq, ws)
    for k in (0, 31, 32, 77, 127):
        x = np.zeros((1, K), np.float32)
        x[0, k] = 1.0
        y = oracle.dense_fp8(x, wq, ws)
        assert np.array_equal(y[0], wd[:, k].astype(np.float32))  # exact: one product
    x = rng.standard_normal((4, K)).astype(np.float32)
    y1 = oracle.dense_fp8(x, wq, ws)
    y2 = oracle.dense_fp8(x, wq, ws + 1)
    assert np.array_equal(y2, y1 * 2)
