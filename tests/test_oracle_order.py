"""Pins of the oracle's summation and multiplication orders (the readings that
make routing and the decode path reproducible bit for bit). Each reading is
an order of fp32 operations, so an error bound cannot tell it from another
order; these tests can:

- constructed inputs whose products are powers of two, where a value of
  2^24 swallows a following +1 (the tie 2^24 + 1 rounds to the even 2^24) and
  the expected result is worked out by hand in each test's comment, with the
  result the nearest wrong orders would give beside it;
- where the values cannot be chosen (sigmoid scores, expert outputs), an
  emulation of the stated order in exact rational arithmetic rounded once per
  operation, checked bit for bit, together with a check that the plausible
  wrong order gives a different result on the same data (so the test has
  teeth)."""
from fractions import Fraction

import numpy as np
import pytest

from exact_fp import add32, fma32, fma32_vec, round_f32
from fp4_routed_mixture_amd import synth as S

P24 = 2.0 ** 24


def test_round_f32_helper():
    assert round_f32(Fraction(2 ** 24 + 1)) == P24          # tie to even
    assert round_f32(Fraction(2 ** 24 + 3)) == P24 + 4      # tie to even (upward)
    assert round_f32(Fraction(1, 3)) == np.float32(1 / 3)
    assert fma32(1 + 2.0 ** -12, 1 + 2.0 ** -12, -(1 + 2.0 ** -11)) == 2.0 ** -24
    # the vectorized fma against the rational one, including a case that
    # double rounding gets wrong: (4097 * 2^-30) * (16773121 * 2^-30) + 1 is
    # 1 + 2^-24 + 2^-60 (4097 * 16773121 = 2^36 + 1), which rounds to the
    # midpoint 1 + 2^-24 in float64 and then to 1 in fp32; the fma gives
    # 1 + 2^-23
    a, b = np.float32(4097 * 2.0 ** -30), np.float32(16773121 * 2.0 ** -30)
    assert fma32_vec(a, b, np.float32(1)) == np.float32(1 + 2.0 ** -23) == fma32(a, b, 1.0)
    assert fma32_vec(-a, b, np.float32(-1)) == np.float32(-(1 + 2.0 ** -23))
    rng = np.random.default_rng(3)
    x, y, z = ((rng.standard_normal(3000) * np.exp2(rng.integers(-30, 30, 3000))).astype(np.float32) for _ in range(3))
    z[:1000] = -(x[:1000].astype(np.float64) * y[:1000]).astype(np.float32)  # heavy cancellation
    v = fma32_vec(x, y, z)
    assert all(v[i] == fma32(x[i], y[i], z[i]) for i in range(3000))


# ------------------------------------------------------- router logits (R6)
def logit_of(oracle, H, products, bias=None):
    """Logit of token 0 / expert 0 whose k-th product x_k * w_k is
    products[k] (x_k = 1, w_k = the value; all other products 0)."""
    x = np.zeros((1, H), np.float32)
    wr = np.zeros((1, H), np.float32)
    for k, v in products.items():
        x[0, k] = 1.0
        wr[0, k] = v
    b = None if bias is None else np.array([bias], np.float32)
    return float(oracle.router_logits(x, wr, b)[0, 0])


@pytest.mark.parametrize("H", [256, 4096])
def test_router_chunk_is_an_ascending_fma_chain(oracle, H):
    # chunk 0 holds 2^24, 1, 1, 1 at k = 0..3. Ascending chain: 2^24, then
    # each + 1 is a tie that rounds back to 2^24 -> 2^24. Descending chain:
    # 3 + 2^24 = 2^24 + 3 -> 2^24 + 4; exact sum rounded once: 2^24 + 4;
    # pairwise inside the chunk: 2^24 + 2.
    assert logit_of(oracle, H, {0: P24, 1: 1.0, 2: 1.0, 3: 1.0}) == P24
    # fused: p = -(1 + 2^-11), then fma((1 + 2^-12), (1 + 2^-12), p) is
    # exactly 2^-24; with the product rounded first it would be 0
    a = 1 + 2.0 ** -12
    x = np.zeros((1, H), np.float32)
    wr = np.zeros((1, H), np.float32)
    x[0, 0], wr[0, 0] = 1.0, -(1 + 2.0 ** -11)
    x[0, 1], wr[0, 1] = a, a
    assert float(oracle.router_logits(x, wr)[0, 0]) == 2.0 ** -24


@pytest.mark.parametrize("H", [256, 4096])
def test_router_chunks_are_h_over_64_long(oracle, H):
    L = H // 64
    # 2^24 at k = 0 and ones at L-2, L-1: all in chunk 0, both ones lost ->
    # 2^24 (chunks of L/2 would put the ones in chunk 1: 2^24 + 2)
    assert logit_of(oracle, H, {0: P24, L - 2: 1.0, L - 1: 1.0}) == P24
    # 2^24 at L-2, ones at L-1, L, L+1: chunk 0 = 2^24 (its one lost), chunk
    # 1 = 2, tree 2^24 + 2 (one chain, or chunks of 2L: 2^24; chunks of L-1:
    # 2^24 + 3 -> 2^24 + 4)
    assert logit_of(oracle, H, {L - 2: P24, L - 1: 1.0, L: 1.0, L + 1: 1.0}) == P24 + 2


@pytest.mark.parametrize("H", [256, 4096])
def test_router_chunk_sums_form_a_pairwise_tree(oracle, H):
    L = H // 64
    # chunk sums c0 = 1, c1 = 1, c2 = 2^24, c3 = 1. Tree: (1 + 1) = 2,
    # (2^24 + 1) -> 2^24, 2 + 2^24 = 2^24 + 2 exact. Left to right:
    # 2 + 2^24 + 1 = 2^24 + 3 -> 2^24 + 4.
    assert logit_of(oracle, H, {0: 1.0, L: 1.0, 2 * L: P24, 3 * L: 1.0}) == P24 + 2
    # across the halves: c0 = 1, c31 = 1, c32 = 2^24, c63 = 1. Left half 2,
    # right half 2^24 + 1 -> 2^24, top 2^24 + 2. Left to right over chunks,
    # or over slices of 8 chunks: 2^24 + 3 -> 2^24 + 4.
    assert logit_of(oracle, H, {0: 1.0, 31 * L: 1.0, 32 * L: P24, 63 * L: 1.0}) == P24 + 2


def test_router_bias_is_added_last(oracle):
    # c0 = 1, c1 = 2^24: tree 2^24 + 1 -> 2^24; + b = 1 -> 2^24 + 1 -> 2^24.
    # The bias as the chain's start value: (1 + 1) + 2^24 = 2^24 + 2.
    L = 4096 // 64
    assert logit_of(oracle, 4096, {0: 1.0, L: P24}, bias=1.0) == P24
    # and it is one fp32 add: 2^24 + 2 from the tree, + 1 -> 2^24 + 3 -> 2^24 + 4
    assert logit_of(oracle, 4096, {0: 2.0, L: P24}, bias=1.0) == P24 + 4


def test_router_random_rows_equal_exact_emulation(oracle):
    """Random data: the oracle's logits equal the reading emulated in exact
    arithmetic (one rounding per fma and per add) for every output, and the
    reversed chain would differ on some of them."""
    rng = np.random.default_rng(11)
    H, E = 256, 6
    x = rng.standard_normal((2, H)).astype(np.float32)
    wr = (rng.standard_normal((E, H)) * np.exp2(rng.integers(-6, 7, (E, H)))).astype(np.float32)
    b = rng.standard_normal(E).astype(np.float32)
    got = oracle.router_logits(x, wr, b)
    L = H // 64
    differs = 0
    for t in range(2):
        for e in range(E):
            def chunks(rev):
                out = []
                for c in range(64):
                    p = np.float32(0)
                    ks = range(c * L, (c + 1) * L)
                    for k in (reversed(ks) if rev else ks):
                        p = fma32(x[t, k], wr[e, k], p)
                    out.append(p)
                return out
            def tree(part):
                while len(part) > 1:
                    part = [add32(part[2 * j], part[2 * j + 1]) for j in range(len(part) // 2)]
                return part[0]
            want = add32(tree(chunks(False)), b[e])
            assert got[t, e] == want, (t, e)
            differs += add32(tree(chunks(True)), b[e]) != want
    assert differs > 0


# ------------------------------------------------------- block sums (R16)
def e2m1_code(v):
    from brute import E2M1
    idx = np.flatnonzero(np.asarray(E2M1, np.float64) == v)
    return int(idx[0])


def pack_row(vals):
    codes = [e2m1_code(v) for v in vals]
    return np.array([codes[2 * i] | (codes[2 * i + 1] << 4) for i in range(len(codes) // 2)], np.uint8)


def test_int8_gemm_blocks_ascending_scale_last(oracle):
    # K = 128, four blocks. Block 0: q = 64 times w = 1 (isum of doubled
    # E2M1 values 128 = 2^7) at scale byte 145 -> 2^7 * 2^(145 - 128) = 2^24;
    # blocks 1, 2: q = 1 times w = 0.5 (isum 1) at byte 128 -> 1; block 3 zero.
    # Ascending: 2^24 (+1 lost twice), times s = 3 -> 3 * 2^24 = 50331648.
    # Descending: 3 * (2^24 + 2) -> 50331656; s applied per block: 50331656.
    K = 128
    q = np.zeros(K, np.int8)
    q[0], q[32], q[64] = 64, 1, 1
    w = np.zeros(K)
    w[0], w[32], w[64] = 1.0, 0.5, 0.5
    ws = np.array([[145, 128, 128, 127]], np.uint8)
    out = oracle.gemm_row_int8(q, 3.0, pack_row(w)[None, :], ws)
    assert out[0] == np.float32(50331648.0)


def test_mxfp4_gemm_blocks_ascending(oracle):
    # Block 0: x = 1, w = 1 (doubled values 2 * 2: isum 4) at scale bytes
    # 150 + 128 -> 4 * 2^(278 - 256) = 2^24; blocks 1, 2: isum 4 at 127 + 127
    # -> 4 * 2^-2 = 1. Ascending 2^24; descending 2^24 + 2.
    K = 128
    xv = np.zeros(K)
    xv[0] = xv[32] = xv[64] = 1.0
    xs = np.array([150, 127, 127, 127], np.uint8)
    ws = np.array([[128, 127, 127, 127]], np.uint8)
    out = oracle.gemm_row_mxfp4(pack_row(xv), xs, pack_row(xv)[None, :], ws)
    assert out[0] == np.float32(P24)


# ------------------------------------------------------ activation (R15)
def test_silu_mul_multiply_order(oracle):
    """a = (g * sigma(g)) * u as two correctly rounded fp32 multiplies, with
    sigma the oracle's own sigmoid (pinned to float64 separately); g * (sigma
    * u) differs on part of the same data."""
    rng = np.random.default_rng(5)
    I = 4096
    g = (rng.standard_normal(I) * 4).astype(np.float32)
    u = rng.standard_normal(I).astype(np.float32)
    a = oracle.silu_mul(np.concatenate([g, u]))
    s = oracle.sigmoidf(g).astype(np.float32)
    want = (g * s).astype(np.float32) * u
    assert np.array_equal(a.view(np.uint32), want.astype(np.float32).view(np.uint32))
    other = g * (s * u).astype(np.float32)
    assert np.any(other.astype(np.float32) != want)


# ------------------------------------------------------ renormalization (R5)
def test_renormalization_sums_in_slot_order(oracle):
    """w_j = s_j / S with S = ((s_0 + s_1) + s_2) + ... over the slots (each
    add and the division correctly rounded in fp32); summing the slots in
    reverse gives another S on part of the rows."""
    rng = np.random.default_rng(8)
    T, E, k = 512, 64, 6
    logits = (rng.standard_normal((T, E)) * 2).astype(np.float32)
    ids, w, sc = oracle.topk(logits, k, return_scores=True)
    s = np.take_along_axis(sc, ids.astype(np.int64), axis=1)
    S = np.zeros(T, np.float32)
    for j in range(k):
        S = (S + s[:, j]).astype(np.float32)
    want = (s / S[:, None]).astype(np.float32)
    assert np.array_equal(w.view(np.uint32), want.view(np.uint32))
    Sr = np.zeros(T, np.float32)
    for j in reversed(range(k)):
        Sr = (Sr + s[:, j]).astype(np.float32)
    assert np.any(Sr != S)


# ------------------------------------------------------------ combine (R17)
def test_combine_is_an_ascending_fma_chain(oracle):
    """out[t] = fma(w_{k-1}, y_{k-1}, ... fma(w_0, y_0, 0)) per element,
    emulated exactly on the layer's own y; the unfused chain and the
    reversed chain each differ on some elements."""
    w = S.WORKLOADS["tiny"]
    ex = [S.expert_weights(w, 0, e) for e in range(w.E)]
    T, k = 3, 4
    x = S.activations(w, T=T)
    rng = np.random.default_rng(12)
    ids = np.stack([rng.choice(w.E, k, replace=False) for _ in range(T)]).astype(np.int32)
    wts = (rng.random((T, k)) + 0.25).astype(np.float32)
    r = oracle.moe_layer_routed(x, ids, wts, ex, 0, intermediates=True)
    y = r["y"].reshape(T, k, -1)
    n_check = 64
    unfused = reversed_ = 0
    for t in range(T):
        for n in range(n_check):
            acc = np.float32(0)
            for j in range(k):
                acc = fma32(wts[t, j], y[t, j, n], acc)
            assert r["out"][t, n] == acc, (t, n)
            acc_u = np.float32(0)
            for j in range(k):
                acc_u = np.float32(acc_u + np.float32(wts[t, j] * y[t, j, n]))
            unfused += acc_u != acc
            acc_r = np.float32(0)
            for j in reversed(range(k)):
                acc_r = fma32(wts[t, j], y[t, j, n], acc_r)
            reversed_ += acc_r != acc
    assert unfused > 0 and reversed_ > 0


# ------------------------------------------------------------ RMSNorm (R21)
def test_rmsnorm_eps_and_order(oracle):
    # all ones, H = 4096: ss = 4096, ss / H = 1, + 1e-6f -> 1 + 8 * 2^-23
    # (1e-6 is 8.39 ulps of 1), sqrt -> 1 + 2^-21, out = 1 / (1 + 2^-21) ->
    # 1 - 2^-21. Eps added before the division by H, or left out: out = 1.
    H = 4096
    out = oracle.rmsnorm(np.ones((1, H), np.float32))
    assert np.all(out == np.float32(1 - 2.0 ** -21))
    # squares 2^24 then 63 ones over chunk 0 (x = 2^12, then 1 at k = 1..63):
    # the ascending chain loses every one, ss = 2^24, r = sqrt(4096 + 1e-6)
    # -> 64 exactly and out = x / 64. A reversed chain: 63 + 2^24 -> 2^24 + 64,
    # r -> 64 + 2^-13 and out[0] < 64.
    x = np.zeros((1, H), np.float32)
    x[0, 0] = 2.0 ** 12
    x[0, 1:64] = 1.0
    out = oracle.rmsnorm(x)
    assert out[0, 0] == 64.0 and np.all(out[0, 1:64] == 2.0 ** -6) and np.all(out[0, 64:] == 0)
