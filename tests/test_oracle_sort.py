"""Pins for the oracle's expert sort."""
import numpy as np
import pytest


@pytest.mark.parametrize("P,E,block_m", [(0, 8, 16), (1, 8, 1), (8, 8, 1), (24, 256, 16),
                                          (384, 256, 32), (1000, 7, 128), (5000, 256, 64)])
def test_sort_against_python_sorted(oracle, P, E, block_m):
    rng = np.random.default_rng(P + E + block_m)
    ids = rng.integers(0, E, P).astype(np.int32)
    r = oracle.sort(ids, E, block_m)
    ref = sorted(range(P), key=lambda i: (int(ids[i]), i))
    counts = np.bincount(ids, minlength=E)
    assert np.array_equal(r["counts"], counts)
    assert r["offsets"][0] == 0
    seg = (counts + block_m - 1) // block_m * block_m
    assert np.array_equal(np.diff(r["offsets"]), seg)
    assert np.all(r["offsets"] % block_m == 0)
    real = r["sorted"][r["sorted"] < P]
    assert real.tolist() == ref  # stable, expert-major
    # a permutation of 0..P-1 plus sentinels; pos is its inverse
    assert sorted(real.tolist()) == list(range(P))
    assert np.all((r["sorted"] == P) | (r["sorted"] < P))
    if P:
        assert np.array_equal(r["sorted"][r["pos"]], np.arange(P))
    for e in range(E):
        lo, hi = r["offsets"][e], r["offsets"][e + 1]
        seg_ids = r["sorted"][lo:hi]
        assert np.all(seg_ids[: counts[e]] < P) and np.all(seg_ids[counts[e]:] == P)
        assert np.all(ids[seg_ids[: counts[e]]] == e)
    tiles = np.repeat(np.arange(E), seg // block_m)
    assert np.array_equal(r["tile_expert"], tiles)
    assert r["n_tiles"] == r["total"] // block_m


def test_sort_all_on_one_expert(oracle):
    ids = np.full(100, 3, np.int32)
    r = oracle.sort(ids, 8, 32)
    assert r["counts"][3] == 100 and r["total"] == 128
    assert r["sorted"][:100].tolist() == list(range(100))
    assert np.all(r["sorted"][100:] == 100)
    assert r["tile_expert"].tolist() == [3, 3, 3, 3]
