"""The W2 layout check: exact column matching recovers a row permutation of
W2 and rejects everything else; pinned on random matrices and on the
oracle's own layer (a permuted W2 permutes the output columns exactly)."""
import numpy as np
import pytest

from fp4_routed_mixture_amd import layout as L
from fp4_routed_mixture_amd import synth as S


def test_recover_random_permutation():
    rng = np.random.default_rng(1)
    ref = rng.standard_normal((6, 300)).astype(np.float32)
    pi = rng.permutation(300).astype(np.int32)
    got = L.recover_row_permutation(ref, ref[:, pi])
    assert np.array_equal(got, pi)
    inv = L.inverse_permutation(pi)
    assert np.array_equal(pi[inv], np.arange(300))
    assert np.array_equal(inv[pi], np.arange(300))


def test_recover_rejects_non_permutations():
    rng = np.random.default_rng(2)
    ref = rng.standard_normal((4, 64)).astype(np.float32)
    bad = ref[:, rng.permutation(64)].copy()
    bad[2, 17] = np.nextafter(bad[2, 17], np.float32(np.inf))  # one ulp off in one column
    with pytest.raises(L.LayoutError):
        L.recover_row_permutation(ref, bad)
    dup = ref.copy()
    dup[:, 5] = ref[:, 9]  # two outputs claim reference column 9
    with pytest.raises(L.LayoutError):
        L.recover_row_permutation(ref, dup)
    with pytest.raises(L.LayoutError):
        L.recover_row_permutation(dup, ref)  # repeated reference columns are ambiguous
    with pytest.raises(L.LayoutError):
        L.inverse_permutation([0, 0, 1])


def test_interleave_permutation_is_a_permutation():
    for n, g in [(256, 16), (4096, 32), (64, 64)]:
        pi = L.interleave_permutation(n, g)
        assert np.array_equal(np.sort(pi), np.arange(n))
    pi = L.interleave_permutation(8, 2)
    assert list(pi) == [0, 4, 1, 5, 2, 6, 3, 7]


def _layer(oracle, w, experts):
    x = S.activations(w)
    return oracle.moe_layer(x, S.router_weights(w), S.router_bias(w), experts, w.top_k, w.act_mode)["out"]


@pytest.mark.parametrize("group", [16, 32])
def test_oracle_w2_row_permutation_permutes_output_columns(oracle, group):
    """W2 rows permuted together with their scales: the layer's output columns
    are permuted exactly, parity with the canonical layout fails, and the
    matching recovers the permutation (int8 mode, every step exact)."""
    w = S.WORKLOADS["tiny"]
    canon = [S.expert_weights(w, 0, e) for e in range(w.E)]
    pi = L.interleave_permutation(w.H, group)
    bad = [(a, b, c[pi], d[pi]) for (a, b, c, d) in canon]
    out_ok = _layer(oracle, w, canon)
    out_bad = _layer(oracle, w, bad)
    assert not np.array_equal(out_ok, out_bad)
    assert np.array_equal(out_bad, out_ok[:, pi])
    assert np.array_equal(L.recover_row_permutation(out_ok, out_bad), pi)
    # repair: reading the stored rows through the inverse restores the layer
    inv = L.inverse_permutation(pi)
    fixed = [(a, b, c[inv], d[inv]) for (a, b, c, d) in bad]
    assert np.array_equal(_layer(oracle, w, fixed), out_ok)


def test_oracle_codes_moved_without_scales_is_not_a_permutation(oracle):
    w = S.WORKLOADS["tiny"]
    canon = [S.expert_weights(w, 0, e) for e in range(w.E)]
    pi = L.interleave_permutation(w.H, 16)
    bad = [(a, b, c[pi], d) for (a, b, c, d) in canon]  # scales left in place
    out_ok = _layer(oracle, w, canon)
    out_bad = _layer(oracle, w, bad)
    with pytest.raises(L.LayoutError):
        L.recover_row_permutation(out_ok, out_bad)
