"""GPU parity of the whole layer (moe_forward through the C ABI) against the
oracle, at small sizes element by element and at the full workload sizes on
sampled tokens (every output depends only on its own token)."""
import numpy as np
import pytest
import torch

import oracle
from fp4_routed_mixture_amd import binding as B
from fp4_routed_mixture_amd import synth as S
from fp4_routed_mixture_amd import synth_device as SD
from gpu_util import assert_close_rms, oracle_layer, require_gpu, run_forward

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


_layers = {}


def dev_layer(name, layer=0):
    key = (name, layer)
    if key not in _layers:
        _layers.clear()
        torch.cuda.empty_cache()
        _layers[key] = SD.load_layer(S.WORKLOADS[name], layer)
    return _layers[key]


def _compare_full(w, g, o, exact_y: bool):
    assert np.array_equal(g["ids"], o["ids"])
    assert np.array_equal(g["w"].view(np.uint32), o["w"].view(np.uint32))
    if "xq" in o and "xq" in g:
        assert np.array_equal(g["xq"].view(np.uint8), o["xq"].view(np.uint8)), "quantized x differs"
        assert np.array_equal(np.ascontiguousarray(g["xs"]).view(np.uint8),
                              np.ascontiguousarray(o["xs"]).view(np.uint8))
    if "aq" in o and "aq" in g:
        diff = (g["aq"].view(np.uint8) != o["aq"].view(np.uint8))
        assert diff.sum() == 0, f"requantized activation differs in {diff.sum()} bytes"
    if exact_y and "y" in g:
        assert np.array_equal(g["y"], o["y"]), f"y differs: max {np.abs(g['y'] - o['y']).max()}"
    return assert_close_rms(g["out"], o["out"])


@pytest.mark.parametrize("name", ["tiny", "tiny_mxfp4"])
def test_forward_tiny_with_intermediates(name):
    w = S.WORKLOADS[name]
    print(f"[forward] {S.describe(w)}", flush=True)
    g = run_forward(w, dev_layer(name), SD.activations(w), taps=True)
    o = oracle_layer(w, S.activations(w), intermediates=True)
    # int8 mode: every step is exact, the output matches bit for bit
    _compare_full(w, g, o, exact_y=(w.act_mode == S.ACT_INT8))
    if w.act_mode == S.ACT_INT8:
        assert np.array_equal(g["out"], o["out"])


@pytest.mark.parametrize("name", ["decode_t4", "decode_t64_zipf", "decode_t4_tp4"])
def test_forward_decode_full(name):
    w = S.WORKLOADS[name]
    print(f"[forward] {S.describe(w)}", flush=True)
    g = run_forward(w, dev_layer(name), SD.activations(w), taps=True)
    o = oracle_layer(w, S.activations(w), intermediates=True)
    err, rms = _compare_full(w, g, o, exact_y=True)
    assert np.array_equal(g["out"], o["out"])
    print(f"max|err| {err:.3g} rms {rms:.3g}")


def _sample_tokens(w, ids, n, seed=0):
    """Tokens that include the heaviest expert's, the lightest experts', the
    last token (ragged tail) and random ones."""
    rng = np.random.default_rng(seed)
    T = ids.shape[0]
    load = np.bincount(ids.ravel(), minlength=w.E)
    heavy = np.argmax(load)
    light = [e for e in np.argsort(load) if load[e] > 0][:3]
    pick = {0, T - 1, int(np.nonzero((ids == heavy).any(1))[0][-1])}
    for e in light:
        pick.add(int(np.nonzero((ids == e).any(1))[0][0]))
    while len(pick) < n:
        pick.add(int(rng.integers(0, T)))
    return np.array(sorted(pick))


@pytest.mark.parametrize("name,n", [("prefill_t4604_zipf", 48), ("prefill_t16384_zipf", 24),
                                    ("prefill_t4604_zipf_tp4", 32)])
def test_forward_prefill_sampled(name, n):
    w = S.WORKLOADS[name]
    print(f"[forward] {S.describe(w)}", flush=True)
    g = run_forward(w, dev_layer(name), SD.activations(w), taps=True)
    x_h = S.activations(w)
    ids_o, w_o = oracle.route(x_h, S.router_weights(w), S.router_bias(w), w.top_k)
    assert np.array_equal(g["ids"], ids_o)
    assert np.array_equal(g["w"].view(np.uint32), w_o.view(np.uint32))
    toks = _sample_tokens(w, ids_o, n)
    o = oracle_layer(w, x_h[toks], intermediates=True)
    assert np.array_equal(g["xq"][toks], o["xq"])
    pairs = (toks[:, None] * w.top_k + np.arange(w.top_k)).ravel()
    flips = int((g["aq"][pairs] != o["aq"]).sum())
    print(f"requant byte differences: {flips} of {o['aq'].size}")
    assert flips == 0
    err, rms = assert_close_rms(g["out"][toks], o["out"])
    print(f"max|err| {err:.3g} rms {rms:.3g}")
    # full-output properties that hold at any size
    assert np.isfinite(g["out"]).all()


@pytest.mark.parametrize("T", [1, 15, 17, 63, 65])
@pytest.mark.parametrize("name", ["decode_t64_zipf", "prefill_t4604_zipf"])
def test_forward_ragged_token_counts(name, T):
    w = S.WORKLOADS[name]
    g = run_forward(w, dev_layer(name), SD.activations(w, T=T), T=T)
    o = oracle_layer(w, S.activations(w, T=T))
    assert np.array_equal(g["ids"], o["ids"])
    assert_close_rms(g["out"], o["out"])


def test_forward_deterministic():
    w = S.WORKLOADS["prefill_t4604_zipf"]
    x = SD.activations(w)
    a = run_forward(w, dev_layer(w.name), x)
    b = run_forward(w, dev_layer(w.name), x)
    assert np.array_equal(a["out"], b["out"])


@pytest.mark.parametrize("act_mode", [0, 1])
def test_all_tokens_one_expert(act_mode):
    """A bias that sends every token to the same experts: one expert holds all
    pairs (the degenerate load of a saturated Zipf head)."""
    w = S.Workload("one_hot", 300, 256, 128, 8, 2, S.X_F32, act_mode, False, 7)
    lay = SD.load_layer(w)
    bias = np.full(8, -30.0, np.float32)
    bias[[2, 5]] = 30.0
    lay["bias"] = torch.from_numpy(bias).cuda()
    g = run_forward(w, lay, SD.activations(w))
    o = oracle_layer(w, S.activations(w), bias=bias)
    assert set(np.unique(g["ids"]).tolist()) == {2, 5}
    assert_close_rms(g["out"], o["out"])


def test_single_expert_k1_is_dense_mlp_on_gpu():
    w = S.Workload("dense", 40, 256, 128, 1, 1, S.X_F32, S.ACT_INT8, False, 11)
    g = run_forward(w, SD.load_layer(w), SD.activations(w))
    o = oracle_layer(w, S.activations(w))
    assert np.all(g["ids"] == 0) and np.all(g["w"] == 1.0)
    assert np.array_equal(g["out"], o["out"])


@pytest.mark.parametrize("k", list(range(1, 17)))
def test_forward_every_top_k(k):
    """Each top-k from 1 to 16 (the combine has one kernel instance per k):
    a small int8 layer equals the oracle bit for bit, routing and output."""
    w = S.Workload(f"topk{k}", 5, 256, 128, 16, k, S.X_BF16, S.ACT_INT8, False, 100 + k)
    print(f"[every top-k] {S.describe(w)}", flush=True)
    g = run_forward(w, SD.load_layer(w), SD.activations(w))
    o = oracle_layer(w, S.activations(w))
    assert np.array_equal(g["ids"], o["ids"])
    assert np.array_equal(g["out"], o["out"])
