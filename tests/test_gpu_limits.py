"""GPU parity at the shape limits the C ABI accepts: the most experts and the
largest top-k (E = 1024, k = 16), the largest K of each GEMM (H = 16384 for
gate/up, I = 16384 for down), and a batch of one token, in both activation
modes. int8 mode must match the oracle bit for bit, MXFP4 within the
tolerance; routing always bit for bit."""
import numpy as np
import pytest
import torch

from fp4_routed_mixture_amd import binding as B
from fp4_routed_mixture_amd import synth as S
from fp4_routed_mixture_amd import synth_device as SD
from gpu_util import assert_close_rms, oracle_layer, require_gpu, run_forward

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()
    yield
    torch.cuda.empty_cache()


CASES = [
    # name, T, H, I, E, k
    ("max_experts_topk", 24, 256, 128, 1024, 16),
    ("max_h", 9, 16384, 256, 4, 2),
    ("max_i", 9, 256, 16384, 4, 2),
    ("one_token", 1, 4096, 2048, 256, 6),
]


@pytest.mark.parametrize("act_mode", [S.ACT_INT8, S.ACT_MXFP4])
@pytest.mark.parametrize("name,T,H,I,E,k", CASES)
def test_shape_limits(name, T, H, I, E, k, act_mode):
    w = S.Workload(name, T, H, I, E, k, S.X_BF16, act_mode, False, 31)
    print(f"[limits] {S.describe(w)}", flush=True)
    layer = SD.load_layer(w)
    g = run_forward(w, layer, SD.activations(w), taps=True)
    o = oracle_layer(w, S.activations(w), intermediates=True)
    assert np.array_equal(g["ids"], o["ids"])
    assert np.array_equal(g["w"].view(np.uint32), o["w"].view(np.uint32))
    # every id distinct per token, weights sum to 1 within k ulps
    assert all(len(set(r)) == k for r in g["ids"].tolist())
    assert np.all(np.abs(g["w"].astype(np.float64).sum(1) - 1.0) <= k * 2.0 ** -23)
    if act_mode == S.ACT_INT8:
        assert np.array_equal(g["out"], o["out"])
    else:
        assert int((g["aq"] != o["aq"]).sum()) == 0
        assert_close_rms(g["out"], o["out"])
    del layer


LARGE_EXPERT_CASES = [
    # experts holding hundreds of rows: many full sort tiles per expert, ragged
    # last tiles, one expert far heavier than the rest, and K = 4096 (the
    # pair-row scales of a tile fill the most LDS)
    ("two_experts", 300, 1024, 512, 2, 2),
    ("ragged_heavy", 777, 2048, 1024, 8, 3),
    ("k4096", 260, 4096, 2048, 2, 2),
]


@pytest.mark.parametrize("name,T,H,I,E,k", LARGE_EXPERT_CASES)
def test_large_experts(name, T, H, I, E, k):
    w = S.Workload(name, T, H, I, E, k, S.X_BF16, S.ACT_MXFP4, False, 41)
    print(f"[large-experts] {S.describe(w)}", flush=True)
    layer = SD.load_layer(w)
    g = run_forward(w, layer, SD.activations(w), taps=True)
    o = oracle_layer(w, S.activations(w), intermediates=True)
    assert np.array_equal(g["ids"], o["ids"])
    assert int((g["aq"] != o["aq"]).sum()) == 0
    assert_close_rms(g["out"], o["out"])
    del layer


def test_max_tokens_sampled():
    """The most tokens the 32-bit activation offsets of the prefill GEMMs
    allow: 2^20 tokens of H = 7936, whose MXFP4 codes fill 4.16e9 of the 2^32
    bytes, k = 1 over 4 experts (about 2^18 rows, thousands of sort tiles, per
    expert). x comes from torch's seeded device generator. Routing and the
    output are compared with the oracle on sampled tokens: the first ones,
    both sides of the 2^31-byte point of the quantized x, the last ones and
    random ones (a token's output depends on its own row only)."""
    T, H, I, E, k = 1 << 20, 7936, 256, 4, 1
    w = S.Workload("max_tokens", T, H, I, E, k, S.X_BF16, S.ACT_MXFP4, False, 45)
    print(f"[limits] {S.describe(w)}", flush=True)
    layer = SD.load_layer(w)
    gen = torch.Generator(device="cuda")
    gen.manual_seed(46)
    x = torch.empty((T, H), dtype=torch.bfloat16, device="cuda")
    step = 1 << 16
    for i in range(0, T, step):
        x[i:i + step] = torch.randn((step, H), generator=gen, device="cuda").to(torch.bfloat16)
    cfg = SD.config(w, T)
    ws = SD.workspace(cfg)
    out = torch.empty((T, H), dtype=torch.float32, device="cuda")
    ids = torch.empty((T, k), dtype=torch.int32, device="cuda")
    wts = torch.empty((T, k), dtype=torch.float32, device="cuda")
    B.moe_forward(cfg, x, layer["router_w"], layer["bias"], layer["w13"], layer["w13s"], layer["w2"], layer["w2s"],
                  out, ids, wts, ws)
    torch.cuda.synchronize()
    mid = (1 << 31) // (H // 2)
    rows = np.unique(np.concatenate([np.arange(0, 3), np.arange(mid - 2, mid + 3), np.arange(T - 3, T),
                                     np.random.default_rng(7).choice(T, 24, replace=False)]))
    idx = torch.from_numpy(rows).cuda()
    xr = x[idx].view(torch.int16).cpu().numpy().view(np.uint16)
    o = oracle_layer(w, xr)
    assert np.array_equal(ids[idx].cpu().numpy(), o["ids"])
    assert np.array_equal(wts[idx].cpu().numpy().view(np.uint32), o["w"].view(np.uint32))
    err, rms = assert_close_rms(out[idx].cpu().numpy(), o["out"])
    print(f"  {len(rows)} sampled tokens: max|err| {err:.3g} (rms {rms:.3g})", flush=True)
    del x, out, ws, layer
    torch.cuda.empty_cache()
