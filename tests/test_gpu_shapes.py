"""A seeded sweep over layer shapes inside the ABI's limits, both activation
modes and both weight layouts, against the oracle: token counts that straddle
the tiny-batch and sort-block switches, hidden and intermediate sizes of odd
multiples of the block sizes, expert counts that are not powers of two, top-k
up to the expert count, bf16 and fp32 x, uniform and biased routing.
Routing must match bit for bit; int8 outputs bit for bit; MXFP4 requantized
activations byte for byte and outputs within the tolerance."""
import numpy as np
import pytest
import torch

from fp4_routed_mixture_amd import binding as B
from fp4_routed_mixture_amd import synth as S
from fp4_routed_mixture_amd import synth_device as SD
from gpu_util import assert_close_rms, oracle_layer, require_gpu

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()
    yield
    torch.cuda.empty_cache()


def sweep(n=16, seed=2026):
    rng = np.random.default_rng(seed)
    cases = []
    for i in range(n):
        E = int(rng.choice([1, 3, 7, 12, 33, 64, 100]))
        k = int(rng.integers(1, min(E, 8) + 1))
        cases.append(dict(
            T=int(rng.choice([1, 2, 5, 16, 17, 31, 33, 64, 65, 130, 257])),
            H=256 * int(rng.integers(1, 9)),      # 256 .. 2048
            I=128 * int(rng.integers(1, 9)),      # 128 .. 1024
            E=E, k=k,
            x=int(rng.integers(0, 2)), act=int(rng.integers(0, 2)), zipf=bool(rng.integers(0, 2)) and E >= 8,
            layout=int(rng.integers(0, 2)), seed=100 + i))
    return cases


# plus the switch of the expert sort from one workgroup to the multi-block
# path (P = T k around 1024 pairs) in both modes
CASES = sweep(24) + [dict(T=T, H=1024, I=512, E=256, k=6, x=1, act=act, zipf=True, layout=1, seed=200 + T + act)
                     for T in (170, 171) for act in (0, 1)]


@pytest.mark.parametrize("c", CASES, ids=[f"T{c['T']}_H{c['H']}_I{c['I']}_E{c['E']}_k{c['k']}_x{c['x']}_a{c['act']}"
                                          f"_z{int(c['zipf'])}_l{c['layout']}" for c in CASES])
def test_shape_sweep(c):
    w = S.Workload("sweep", c["T"], c["H"], c["I"], c["E"], c["k"], c["x"], c["act"], c["zipf"], c["seed"])
    print(f"[sweep] {S.describe(w)} layout={c['layout']}", flush=True)
    lay = SD.load_layer(w, keep_canonical=c["layout"] == B.MOE_LAYOUT_CANONICAL)
    x = SD.activations(w)
    T = w.T
    cfg = SD.config(w, T, weight_layout=c["layout"])
    ws = SD.workspace(cfg)
    out = torch.empty((T, w.H), dtype=torch.float32, device="cuda")
    ids = torch.empty((T, w.top_k), dtype=torch.int32, device="cuda")
    wts = torch.empty((T, w.top_k), dtype=torch.float32, device="cuda")
    P = T * w.top_k
    mx = w.act_mode == S.ACT_MXFP4
    taps = {"aq": torch.empty((P, w.I // 2) if mx else (P, w.I), dtype=torch.uint8 if mx else torch.int8,
                              device="cuda"),
            "as": torch.empty((P, w.I // 32) if mx else (P,), dtype=torch.uint8 if mx else torch.float32,
                              device="cuda")}
    if c["layout"] == B.MOE_LAYOUT_CANONICAL:
        w13, w13s, w2, w2s = lay["canonical"]
    else:
        w13, w13s, w2, w2s = lay["w13"], lay["w13s"], lay["w2"], lay["w2s"]
    B.moe_forward_taps(cfg, x, lay["router_w"], lay["bias"], w13, w13s, w2, w2s, out, ids, wts, taps, ws)
    torch.cuda.synchronize()
    o = oracle_layer(w, S.activations(w), intermediates=True)
    assert np.array_equal(ids.cpu().numpy(), o["ids"])
    assert np.array_equal(wts.cpu().numpy().view(np.uint32), o["w"].view(np.uint32))
    g_out = out.cpu().numpy()
    if mx:
        assert np.array_equal(taps["aq"].cpu().numpy(), o["aq"]), "requantized activations differ"
        assert_close_rms(g_out, o["out"])
    else:
        assert np.array_equal(g_out.view(np.uint32), o["out"].view(np.uint32))
    del lay, ws
