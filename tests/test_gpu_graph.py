"""HIP-graph capture of the library's calls: a captured layer stack and a
captured single layer are replayed several times, with eager work and
synchronizations between the replays, and every replay must reproduce the
eager result bit for bit (the kernels are deterministic and a captured launch
is the same launch). One replay of each is also checked against the oracle."""
import numpy as np
import pytest
import torch

import oracle
from fp4_routed_mixture_amd import binding as B
from fp4_routed_mixture_amd import synth as S
from fp4_routed_mixture_amd import synth_device as SD
from gpu_util import TOL, oracle_layer, require_gpu

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()
    yield
    torch.cuda.empty_cache()


def _capture(fn):
    """fn() captured into a graph after one warm-up call on a side stream."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    return g


def test_stack_graph_replays():
    w = S.Workload("graph_stack3", 24, 1024, 256, 16, 4, S.X_F32, S.ACT_INT8, False, 12, 3)
    L = w.layers
    print(f"[graph] {S.describe(w)} layers={L}", flush=True)
    layers = [SD.load_layer(w, l) for l in range(L)]
    cfg = SD.config(w)
    ws = torch.empty(B.moe_stack_workspace_size(cfg), dtype=torch.uint8, device="cuda")
    x0_h = S.activations(w)
    x0 = torch.from_numpy(x0_h).cuda()

    # eager reference
    x_ref = x0.clone()
    y_ref = torch.empty((L, w.T, w.H), dtype=torch.float32, device="cuda")
    B.moe_forward_stack(cfg, x_ref, layers, ws, layer_out=y_ref)
    torch.cuda.synchronize()

    xg = x0.clone()
    yg = torch.empty_like(y_ref)
    g = _capture(lambda: B.moe_forward_stack(cfg, xg, layers, ws, layer_out=yg))
    x_other = torch.from_numpy(S.activations(w, layer=1)).cuda()
    for rep in range(4):
        xg.copy_(x0)
        yg.zero_()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(xg, x_ref), f"replay {rep}: final stream differs"
        assert torch.equal(yg, y_ref), f"replay {rep}: layer outputs differ"
        # eager work between replays, on the same workspace and stream
        xe = x_other.clone()
        B.moe_forward_stack(cfg, xe, layers, ws)
        torch.cuda.synchronize()

    # layer 0 of the replayed stack against the oracle (exact in int8 mode)
    o = oracle_layer(w, oracle.rmsnorm(x0_h), layer=0)
    assert np.array_equal(o["out"], yg[0].cpu().numpy())
    del layers, ws


@pytest.mark.parametrize("name,T,H,I,E,k,act", [
    ("graph_decode_int8", 4, 1024, 256, 16, 4, S.ACT_INT8),
    ("graph_prefill_mxfp4", 300, 1024, 512, 8, 2, S.ACT_MXFP4),
])
def test_layer_graph_replays(name, T, H, I, E, k, act):
    w = S.Workload(name, T, H, I, E, k, S.X_BF16, act, False, 13)
    print(f"[graph] {S.describe(w)}", flush=True)
    L = SD.load_layer(w)
    cfg = SD.config(w)
    ws = SD.workspace(cfg)
    xin = SD.activations(w).clone()
    out = torch.empty((T, H), dtype=torch.float32, device="cuda")
    ids = torch.empty((T, k), dtype=torch.int32, device="cuda")
    wts = torch.empty((T, k), dtype=torch.float32, device="cuda")

    def call():
        B.moe_forward(cfg, xin, L["router_w"], L["bias"], L["w13"], L["w13s"], L["w2"], L["w2s"], out, ids, wts, ws)

    inputs = [SD.activations(w, layer=i) for i in range(3)]
    refs = []
    for xi in inputs:
        xin.copy_(xi)
        call()
        torch.cuda.synchronize()
        refs.append((out.clone(), ids.clone(), wts.clone()))

    g = _capture(call)
    for rep in range(6):
        i = rep % 3
        xin.copy_(inputs[i])
        out.zero_()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(ids, refs[i][1]) and torch.equal(wts, refs[i][2]), f"replay {rep}: routing differs"
        assert torch.equal(out, refs[i][0]), f"replay {rep}: output differs"
        call()  # eager work between replays
        torch.cuda.synchronize()

    xin.copy_(inputs[0])
    g.replay()
    torch.cuda.synchronize()
    o = oracle_layer(w, S.activations(w, layer=0))
    assert np.array_equal(ids.cpu().numpy(), o["ids"])
    got = out.cpu().numpy()
    rms = float(np.sqrt(np.mean(o["out"].astype(np.float64) ** 2)))
    assert float(np.abs(got - o["out"]).max()) <= TOL * rms
    del L, ws


@pytest.mark.parametrize("M,N,K,layout", [
    (17, 1536, 4096, B.MOE_LAYOUT_PREPACKED),   # small-batch kernel, K split over workgroups + reduce
    (200, 2304, 2048, B.MOE_LAYOUT_CANONICAL),  # wide kernel, 128-row tiles
])
def test_dense_graph_replays(M, N, K, layout):
    """The FP8 dense projection (quantizer + GEMM, and the K-split reduction
    of small batches) captured and replayed with other inputs in place: every
    replay equals the eager call on the same input bit for bit."""
    w = S.DenseWorkload("graph_dense", M, K, N, S.X_BF16, 47)
    print(f"[graph] dense M={M} N={N} K={K} layout={layout}", flush=True)
    wq_h, ws_h = S.dense_weights(w)
    wq, wsc = torch.from_numpy(wq_h).cuda(), torch.from_numpy(ws_h).cuda()
    if layout == B.MOE_LAYOUT_PREPACKED:
        cb, sb = B.moe_dense_fp8_prepacked_size(N, K)
        pq = torch.empty(cb, dtype=torch.uint8, device="cuda")
        ps = torch.empty(sb, dtype=torch.uint8, device="cuda")
        B.moe_dense_fp8_prepack(N, K, wq, wsc, pq, ps)
        wq, wsc = pq, ps
    cfg = B.make_dense_config(M, N, K, S.X_BF16, layout)
    work = torch.empty(B.moe_dense_fp8_workspace_size(cfg), dtype=torch.uint8, device="cuda")
    inputs = [torch.from_numpy(S.dense_activations(S.DenseWorkload("graph_dense", M, K, N, S.X_BF16, 48 + i))
                               .view(np.int16)).cuda() for i in range(3)]
    x = torch.empty_like(inputs[0])
    y = torch.empty((M, N), dtype=torch.float32, device="cuda")

    def call():
        B.moe_dense_fp8_forward(cfg, x, wq, wsc, y, work)

    refs = []
    for xi in inputs:
        x.copy_(xi)
        call()
        torch.cuda.synchronize()
        refs.append(y.clone())
    g = _capture(call)
    for rep in range(6):
        i = rep % 3
        x.copy_(inputs[i])
        y.zero_()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(y.view(torch.int32), refs[i].view(torch.int32)), f"replay {rep} differs"
        call()  # eager work between replays, on the same workspace
        torch.cuda.synchronize()
