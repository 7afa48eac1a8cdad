"""Pins for the oracle's format decoding, exp and sigmoid."""
import math
import os

import numpy as np
import pytest

from brute import ulp32

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "e2m1_e8m0.txt")


def _golden():
    e2m1, e8m0 = {}, {}
    for line in open(GOLDEN):
        if line.startswith("#") or not line.strip():
            continue
        kind, k, v = line.split()
        (e2m1 if kind == "e2m1" else e8m0)[int(k)] = float(v)
    return e2m1, e8m0


def test_e2m1_table_exact(oracle):
    e2m1, _ = _golden()
    tab = oracle.e2m1_table()
    for c in range(16):
        assert tab[c] == e2m1[c], c
        assert math.copysign(1.0, tab[c]) == math.copysign(1.0, e2m1[c]), c


def test_e8m0_all_bytes(oracle):
    _, e8m0 = _golden()
    for b in range(255):
        assert oracle.e8m0(b) == 2.0 ** (b - 127), b
    for b, v in e8m0.items():
        if math.isnan(v):
            assert math.isnan(oracle.e8m0(b))
        else:
            assert oracle.e8m0(b) == np.float32(v)


def test_expf_within_2ulp_dense_sweep(oracle):
    z = np.linspace(-87.0, 88.72, 2_000_001, dtype=np.float32)
    z = np.concatenate([z, np.float32([0.0, -0.0, 1e-8, -1e-8, 0.5, -0.5, 88.72283172607421875])])
    got = oracle.expf(z).astype(np.float64)
    ref = np.exp(z.astype(np.float64))
    err = np.abs(got - ref) / ulp32(ref.astype(np.float32))
    assert err.max() <= 2.0, float(err.max())


def test_expf_special_values(oracle):
    assert oracle.expf(0.0)[0] == 1.0
    assert np.isinf(oracle.expf(89.0)[0])
    assert np.isinf(oracle.expf(88.7228394)[0])  # next fp32 above the largest finite input
    assert oracle.expf(-104.0)[0] == 0.0
    assert np.isnan(oracle.expf(np.nan)[0])
    # subnormal results: within one subnormal step of float64
    z = np.linspace(-103.9, -87.5, 10001, dtype=np.float32)
    got = oracle.expf(z).astype(np.float64)
    ref = np.exp(z.astype(np.float64))
    assert np.max(np.abs(got - ref)) <= 2.0 ** -149


def test_sigmoid_within_3ulp(oracle):
    z = np.linspace(-40.0, 40.0, 400_001, dtype=np.float32)
    got = oracle.sigmoidf(z).astype(np.float64)
    ref = 1.0 / (1.0 + np.exp(-z.astype(np.float64)))
    err = np.abs(got - ref) / ulp32(ref.astype(np.float32))
    assert err.max() <= 3.0, float(err.max())
    assert oracle.sigmoidf(0.0)[0] == 0.5
    assert oracle.sigmoidf(100.0)[0] == 1.0
    assert oracle.sigmoidf(-88.0)[0] > 0.0
    # 1/(1+exp(-z)) in fp32: exp(-z) overflows to inf below z = -88.72, so the
    # defined sigmoid returns 0 there (the true value is below 2^-127).
    assert oracle.sigmoidf(-100.0)[0] == 0.0
