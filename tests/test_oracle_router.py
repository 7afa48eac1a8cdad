"""Pins for the oracle's router (logits, sigmoid top-k, renormalization)."""
import numpy as np
import pytest

from fp4_routed_mixture_amd import synth as S


def _gamma(n):
    u = 2.0 ** -24
    return n * u / (1 - n * u)


@pytest.mark.parametrize("T,H,E", [(3, 256, 8), (5, 4096, 37), (2, 128, 256)])
def test_logits_within_fp32_bound(oracle, T, H, E):
    rng = np.random.default_rng(7)
    x = rng.standard_normal((T, H)).astype(np.float32)
    wr = (0.02 * rng.standard_normal((E, H))).astype(np.float32)
    b = rng.standard_normal(E).astype(np.float32)
    got = oracle.router_logits(x, wr, b).astype(np.float64)
    x64, w64 = x.astype(np.float64), wr.astype(np.float64)
    ref = x64 @ w64.T
    # chain of H/64 fmas, six tree levels, one bias add
    bound = _gamma(H // 64 + 6) * (np.abs(x64) @ np.abs(w64).T) + 2.0 ** -24 * np.abs(ref + b)
    err = np.abs(got - (ref + b.astype(np.float64)))
    assert np.all(err <= bound + 1e-30), float((err / (bound + 1e-30)).max())


def test_logits_exact_on_integer_data(oracle):
    # small integers: every partial sum is exact in fp32, any order gives the
    # integer dot product
    rng = np.random.default_rng(1)
    x = rng.integers(-8, 9, (4, 512)).astype(np.float32)
    wr = rng.integers(-8, 9, (6, 512)).astype(np.float32)
    got = oracle.router_logits(x, wr)
    ref = x.astype(np.int64) @ wr.astype(np.int64).T
    assert np.array_equal(got, ref.astype(np.float32))


def test_bf16_input_is_upcast_exactly(oracle):
    x = np.random.default_rng(2).standard_normal((3, 256)).astype(np.float32)
    xb = S.f32_to_bf16_bits(x)
    xf = oracle.x_to_f32(xb)
    assert np.array_equal(xf.view(np.uint32), xb.astype(np.uint32) << 16)
    # rounding to bf16 is the nearest-even bf16 of x
    err = np.abs(xf.astype(np.float64) - x)
    assert np.all(err <= np.spacing(np.abs(xf)).astype(np.float64) * 2 ** 16 / 2 + 1e-45)


def _topk_bruteforce(scores, k):
    T, E = scores.shape
    out = np.empty((T, k), np.int64)
    for t in range(T):
        order = sorted(range(E), key=lambda e: (-float(scores[t, e]), e))
        out[t] = order[:k]
    return out


@pytest.mark.parametrize("E,k", [(8, 2), (256, 6), (16, 16), (5, 1)])
def test_topk_matches_full_sort(oracle, E, k):
    rng = np.random.default_rng(E * 10 + k)
    logits = (rng.standard_normal((40, E)) * 1.5).astype(np.float32)
    ids, w, sc = oracle.topk(logits, k, return_scores=True)
    # scores are the pinned sigmoid of the logits
    assert np.array_equal(sc, oracle.sigmoidf(logits))
    assert np.array_equal(ids, _topk_bruteforce(sc, k))
    # invariants: k distinct ids in range, positive weights, sum 1, non-increasing
    for t in range(ids.shape[0]):
        assert len(set(ids[t].tolist())) == k
    assert ids.min() >= 0 and ids.max() < E
    assert np.all(w > 0)
    assert np.all(np.abs(w.astype(np.float64).sum(1) - 1.0) <= k * 2.0 ** -23)
    assert np.all(np.diff(w, axis=1) <= 0)
    # weights = s_j / S with S the fp32 left-to-right sum, IEEE division
    s_sel = np.take_along_axis(sc, ids, axis=1)
    S_ = np.zeros(ids.shape[0], np.float32)
    for j in range(k):
        S_ = (S_ + s_sel[:, j]).astype(np.float32)
    assert np.array_equal(w, (s_sel / S_[:, None]).astype(np.float32))


def test_topk_ties_go_to_lower_index(oracle):
    logits = np.zeros((2, 8), np.float32)
    logits[0, [1, 3, 6]] = 2.0
    logits[1, :] = 30.0  # every score saturates to 1.0
    ids, w = oracle.topk(logits, 2)
    assert ids[0].tolist() == [1, 3]
    assert ids[1].tolist() == [0, 1]
    assert np.all(w[1] == 0.5)


def test_routing_with_bias_moves_selection(oracle):
    rng = np.random.default_rng(3)
    x = rng.standard_normal((16, 256)).astype(np.float32)
    wr = (0.02 * rng.standard_normal((8, 256))).astype(np.float32)
    b = np.full(8, -20.0, np.float32)
    b[5] = 20.0
    ids, _ = oracle.route(x, wr, b, 2)
    assert np.all(ids[:, 0] == 5)
