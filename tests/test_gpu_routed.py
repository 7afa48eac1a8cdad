"""moe_forward_routed (the layer without its router) through the C ABI.

With the router's own ids and weights it must reproduce moe_forward bit for
bit. As an expert-parallel rank uses it -- the (token, expert) pairs routed to
one block of experts, one row per pair with top_k = 1, the rank's slice of
the experts -- it is checked against the oracle's router-free layer."""
import numpy as np
import pytest
import torch

import oracle
from fp4_routed_mixture_amd import binding as B
from fp4_routed_mixture_amd import synth as S
from fp4_routed_mixture_amd import synth_device as SD
from gpu_util import assert_close_rms, require_gpu, run_forward

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()
    yield
    torch.cuda.empty_cache()


def _routed(w, lay, x, ids, wts, E=None, taps=None):
    T, k = ids.shape
    cfg = B.make_config(T, w.H, w.I, w.E if E is None else E, k, w.x_dtype, w.act_mode, B.MOE_LAYOUT_PREPACKED)
    ws = SD.workspace(cfg)
    out = torch.empty((T, w.H), dtype=torch.float32, device="cuda")
    B.moe_forward_routed(cfg, x, ids, wts, lay["w13"], lay["w13s"], lay["w2"], lay["w2s"], out, ws, taps=taps)
    torch.cuda.synchronize()
    return out


CASES = [
    ("routed_int8", 37, 1024, 256, 16, 4, S.ACT_INT8, False),
    ("routed_mxfp4_zipf", 300, 1024, 512, 64, 4, S.ACT_MXFP4, True),
    ("routed_mxfp4_large", 2000, 2048, 1024, 32, 6, S.ACT_MXFP4, False),
]


@pytest.mark.parametrize("name,T,H,I,E,k,act,zipf", CASES)
def test_routed_with_router_routing_equals_forward(name, T, H, I, E, k, act, zipf):
    w = S.Workload(name, T, H, I, E, k, S.X_BF16, act, zipf, 21)
    print(f"[routed] {S.describe(w)}", flush=True)
    lay = SD.load_layer(w)
    x = SD.activations(w)
    g = run_forward(w, lay, x)
    ids = torch.from_numpy(g["ids"]).cuda()
    wts = torch.from_numpy(g["w"]).cuda()
    out = _routed(w, lay, x, ids, wts).cpu().numpy()
    assert np.array_equal(out, g["out"])
    del lay


@pytest.mark.parametrize("act", [S.ACT_INT8, S.ACT_MXFP4])
def test_routed_expert_parallel_rank(act):
    """Experts 16r .. 16r+15 on rank r of 4; the heaviest rank computes its
    pairs as rows (top_k = 1) with its slice of the prepacked weights."""
    w = S.Workload("ep_rank", 400, 1024, 512, 64, 4, S.X_BF16, act, True, 22)
    print(f"[routed] {S.describe(w)} expert-parallel rank", flush=True)
    lay = SD.load_layer(w)
    x = SD.activations(w)
    g = run_forward(w, lay, x)
    ids = g["ids"].ravel()
    ranks = ids // 16
    r = int(np.argmax(np.bincount(ranks, minlength=4)))
    pairs = np.nonzero(ranks == r)[0]
    tok = pairs // w.top_k
    ids_l = (ids[pairs] - 16 * r).astype(np.int32).reshape(-1, 1)
    w_l = g["w"].ravel()[pairs].astype(np.float32).reshape(-1, 1)
    local = {n: lay[n].view(w.E, -1)[16 * r:16 * r + 16].contiguous() for n in ("w13", "w13s", "w2", "w2s")}
    x_rows = x[torch.from_numpy(tok).cuda()].contiguous()
    out = _routed(w, local, x_rows, torch.from_numpy(ids_l).cuda(), torch.from_numpy(w_l).cuda(), E=16)
    out = out.cpu().numpy()
    ex = [S.expert_weights(w, 0, 16 * r + e) for e in range(16)]
    o = oracle.moe_layer_routed(S.activations(w)[tok], ids_l, w_l, ex, act)
    if act == S.ACT_INT8:
        assert np.array_equal(out, o["out"])
    else:
        assert_close_rms(out, o["out"])
    # a row is fl32(w * y) of its pair in the whole layer (int8: exact)
    if act == S.ACT_INT8:
        full = oracle.moe_layer(S.activations(w), S.router_weights(w), S.router_bias(w),
                                [S.expert_weights(w, 0, e) for e in range(w.E)], w.top_k, act, intermediates=True)
        want = (w_l * full["y"][pairs]).astype(np.float32)
        assert np.array_equal(out, want)
    del lay, local


def test_routed_out_of_range_ids_are_clamped():
    w = S.Workload("routed_clamp", 8, 256, 128, 8, 2, S.X_F32, S.ACT_INT8, False, 23)
    lay = SD.load_layer(w)
    x = SD.activations(w)
    ids = np.tile(np.array([[-5, 99]], np.int32), (8, 1))
    wts = np.full((8, 2), 0.5, np.float32)
    out = _routed(w, lay, x, torch.from_numpy(ids).cuda(), torch.from_numpy(wts).cuda()).cpu().numpy()
    clamped = np.tile(np.array([[0, 7]], np.int32), (8, 1))
    ref = _routed(w, lay, x, torch.from_numpy(clamped).cuda(), torch.from_numpy(wts).cuda()).cpu().numpy()
    assert np.array_equal(out, ref)
