"""Pins for the oracle's expert GEMMs, activation and whole layer."""
import numpy as np
import pytest

from brute import E2M1, dequant, silu64, unpack_codes
from fp4_routed_mixture_amd import synth as S

TINY = S.WORKLOADS["tiny"]


def _experts(w=TINY, layer=0):
    return [S.expert_weights(w, layer, e) for e in range(w.E)]


def _rand_weights(rng, N, K):
    return (rng.integers(0, 256, (N, K // 2)).astype(np.uint8),
            rng.integers(121, 126, (N, K // 32)).astype(np.uint8))


@pytest.mark.parametrize("K,N", [(256, 64), (128, 40)])
def test_gemm_int8_row_exact_vs_float64(oracle, K, N):
    rng = np.random.default_rng(K + N)
    wc, ws = _rand_weights(rng, N, K)
    q = rng.integers(-127, 128, K).astype(np.int8)
    s = np.float32(0.0371)
    got = oracle.gemm_row_int8(q, s, wc, ws)
    W = dequant(wc, ws)                      # [N, K] float64
    acc = W @ q.astype(np.float64)           # exact: dyadic values, < 2^24 range
    ref = (np.float64(s) * acc).astype(np.float32)
    assert np.array_equal(got, ref)


def test_gemm_mxfp4_row_exact_vs_float64(oracle):
    rng = np.random.default_rng(5)
    K, N = 256, 48
    wc, ws = _rand_weights(rng, N, K)
    xc = rng.integers(0, 256, K // 2).astype(np.uint8)
    xs = rng.integers(120, 131, K // 32).astype(np.uint8)
    got = oracle.gemm_row_mxfp4(xc, xs, wc, ws)
    ref = (dequant(wc, ws) @ dequant(xc[None], xs[None])[0]).astype(np.float32)
    assert np.array_equal(got, ref)


def test_gemm_nibble_order_and_one_hot(oracle):
    # one-hot int8 row with q=127, s=1/127 exactly representable? use s=1:
    # h_n = 127 * W[n, i]; pins the nibble order and the scale exponent
    rng = np.random.default_rng(9)
    K, N = 128, 16
    wc, ws = _rand_weights(rng, N, K)
    W = dequant(wc, ws)
    for i in (0, 1, 2, 63, 127):
        q = np.zeros(K, np.int8)
        q[i] = 127
        got = oracle.gemm_row_int8(q, np.float32(1.0), wc, ws)
        assert np.array_equal(got, (127.0 * W[:, i]).astype(np.float32)), i


def test_silu_mul_close_to_float64(oracle):
    rng = np.random.default_rng(4)
    h = (rng.standard_normal(512) * 30).astype(np.float32)
    a = oracle.silu_mul(h)
    g, u = h[:256].astype(np.float64), h[256:].astype(np.float64)
    ref = silu64(g) * u
    # exp(-g) overflows for g < -88.72 and the product becomes 0 (true value
    # below 1e-30): an absolute floor covers that end
    assert np.all(np.abs(a - ref) <= 6 * 2.0 ** -24 * np.abs(ref) + 1e-30)


def _dense_mlp64(xq, xs, W13, W2, act_mode, oracle):
    """Dense float64 MLP on dequantized weights with the same quantizers."""
    if act_mode == 0:
        h = xs * (xq.astype(np.float64) @ W13.T)
    else:
        h = dequant(xq[None], xs[None])[0] @ W13.T
    I = W13.shape[0] // 2
    a = (h[:I] * (1.0 / (1.0 + np.exp(-h[:I])))) * h[I:]
    return h, a


@pytest.mark.parametrize("act_mode", [0, 1])
def test_single_expert_k1_equals_dense_mlp(oracle, act_mode):
    w = S.Workload("one", 3, 256, 128, 1, 1, S.X_F32, act_mode, False, 11)
    ex = S.expert_weights(w, 0, 0)
    x = S.activations(w)
    wr = S.router_weights(w)
    r = oracle.moe_layer(x, wr, None, [ex], 1, act_mode, intermediates=True)
    W13, W2 = dequant(ex[0], ex[1]), dequant(ex[2], ex[3])
    for t in range(w.T):
        xs = r["xs"][t]
        h, a = _dense_mlp64(r["xq"][t], xs, W13, W2, act_mode, oracle)
        # G1 is exact in fp32 for these operands: bit-equal after rounding
        assert np.array_equal(r["h"][t], h.astype(np.float32))
        # activation within a few ulps of float64
        a32 = oracle.silu_mul(r["h"][t]).astype(np.float64)
        assert np.all(np.abs(a32 - a) <= 8 * 2.0 ** -24 * np.abs(a) + 1e-30)
        if act_mode == 0:
            y = np.float64(r["as"][t]) * (r["aq"][t].astype(np.float64) @ W2.T)
        else:
            y = dequant(r["aq"][t][None], r["as"][t][None])[0] @ W2.T
        assert np.all(np.abs(r["y"][t] - y) <= 2.0 ** -20 * np.abs(y).max())
        assert r["w"][t, 0] == 1.0
        assert np.array_equal(r["out"][t], r["y"][t])  # k = 1: out = y
    # and end to end close to an unquantized-activation float64 MLP
    # (quantization error only: int8 rows lose little, E2M1 activations with
    # the OCP shared exponent lose up to a quarter of a block's amax)
    xf = x.astype(np.float64)
    h = xf @ W13.T
    a = silu64(h[:, :128]) * h[:, 128:]
    y = a @ W2.T
    rms = np.sqrt(np.mean(y ** 2))
    assert np.sqrt(np.mean((r["out"] - y) ** 2)) < (0.02 if act_mode == 0 else 0.3) * rms


@pytest.mark.parametrize("act_mode", [0, 1])
def test_scale_exponent_plus_one_doubles_output(oracle, act_mode):
    w = TINY
    ex = _experts(w)
    x, wr = S.activations(w), S.router_weights(w)
    base = oracle.moe_layer(x, wr, None, ex, w.top_k, act_mode)["out"]
    ex2 = [(a, b, c, (d + 1).astype(np.uint8)) for a, b, c, d in ex]
    dbl = oracle.moe_layer(x, wr, None, ex2, w.top_k, act_mode)["out"]
    assert np.array_equal(dbl, 2 * base)


def test_zero_weights_give_zero(oracle):
    w = TINY
    ex = [(np.zeros_like(a), b, np.zeros_like(c), d) for a, b, c, d in _experts(w)]
    out = oracle.moe_layer(S.activations(w), S.router_weights(w), None, ex, 2, 0)["out"]
    assert np.all(out == 0)


@pytest.mark.parametrize("act_mode", [0, 1])
def test_token_permutation_equivariance(oracle, act_mode):
    w = TINY
    ex = _experts(w)
    x, wr = S.activations(w, T=9), S.router_weights(w)
    perm = np.random.default_rng(0).permutation(9)
    a = oracle.moe_layer(x, wr, None, ex, 2, act_mode)
    b = oracle.moe_layer(x[perm], wr, None, ex, 2, act_mode)
    assert np.array_equal(b["out"], a["out"][perm])
    assert np.array_equal(b["ids"], a["ids"][perm])


@pytest.mark.parametrize("act_mode", [0, 1])
def test_expert_relabel_equivariance(oracle, act_mode):
    w = TINY
    ex = _experts(w)
    x, wr = S.activations(w, T=7), S.router_weights(w)
    rng = np.random.default_rng(1)
    bias = rng.standard_normal(w.E).astype(np.float32)
    sigma = rng.permutation(w.E)  # new expert j = old expert sigma[j]
    a = oracle.moe_layer(x, wr, bias, ex, 2, act_mode)
    b = oracle.moe_layer(x, wr[sigma], bias[sigma], [ex[s] for s in sigma], 2, act_mode)
    assert np.array_equal(a["out"], b["out"])
    assert np.array_equal(sigma[b["ids"]], a["ids"])


def test_identical_experts_make_router_irrelevant(oracle):
    w = TINY
    e0 = S.expert_weights(w, 0, 0)
    x = S.activations(w, T=6)
    r = oracle.moe_layer(x, S.router_weights(w), None, [e0] * w.E, 2, 0)
    one = oracle.moe_layer(x, S.router_weights(w)[:1], None, [e0], 1, 0)
    # sum_j w_j * y = y * (sum_j w_j), with sum_j w_j = 1 up to rounding
    assert np.allclose(r["out"], one["out"], rtol=4 * 2.0 ** -23, atol=0)


def test_combine_within_fp32_bound(oracle):
    w = TINY
    r = oracle.moe_layer(S.activations(w, T=6), S.router_weights(w), None, _experts(w), 2, 0,
                         intermediates=True)
    y = r["y"].reshape(6, 2, -1).astype(np.float64)
    ref = np.einsum("tj,tjn->tn", r["w"].astype(np.float64), y)
    bound = 2 * 2.0 ** -24 * np.einsum("tj,tjn->tn", np.abs(r["w"]), np.abs(y))
    assert np.all(np.abs(r["out"] - ref) <= bound + 1e-30)


def test_rmsnorm_within_bound(oracle):
    x = (np.random.default_rng(2).standard_normal((4, 4096)) * 300).astype(np.float32)
    got = oracle.rmsnorm(x).astype(np.float64)
    x64 = x.astype(np.float64)
    ref = x64 / np.sqrt(np.mean(x64 ** 2, axis=1, keepdims=True) + 1e-6)
    assert np.all(np.abs(got - ref) <= 1e-5 * np.abs(ref) + 1e-7)


@pytest.mark.parametrize("act_mode", [0, 1])
def test_routed_layer_reproduces_the_routed_part(oracle, act_mode):
    """Given the router's own routing, the router-free layer is the layer."""
    w = TINY
    ex = _experts(w)
    x, wr = S.activations(w, T=9), S.router_weights(w)
    full = oracle.moe_layer(x, wr, None, ex, 2, act_mode, intermediates=True)
    r = oracle.moe_layer_routed(x, full["ids"], full["w"], ex, act_mode, intermediates=True)
    for n in ("out", "xq", "xs", "h", "aq", "as", "y"):
        assert np.array_equal(r[n], full[n]), n


@pytest.mark.parametrize("act_mode", [0, 1])
def test_routed_layer_one_row_per_pair(oracle, act_mode):
    """Each (token, slot) pair as its own row with k = 1, as an expert-parallel
    rank receives them: row p's output is fl32(w_p * y_p) with y_p the pair's
    down-projection in the whole layer."""
    w = TINY
    ex = _experts(w)
    x, wr = S.activations(w, T=5), S.router_weights(w)
    full = oracle.moe_layer(x, wr, None, ex, 2, act_mode, intermediates=True)
    rows = np.repeat(x, 2, axis=0)  # pair p = t*k + j reads token t
    r = oracle.moe_layer_routed(rows, full["ids"].reshape(-1, 1), full["w"].reshape(-1, 1), ex, act_mode)
    want = (full["w"].reshape(-1, 1).astype(np.float32) * full["y"]).astype(np.float32)
    assert np.array_equal(r["out"], want)


def test_routed_layer_rejects_bad_ids(oracle):
    w = TINY
    ex = _experts(w)
    x = S.activations(w, T=2)
    ids = np.array([[0, 1], [2, w.E]], np.int32)
    with pytest.raises(ValueError):
        oracle.moe_layer_routed(x, ids, np.full((2, 2), 0.5, np.float32), ex, 0)
