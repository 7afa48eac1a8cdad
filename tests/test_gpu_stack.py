"""The 43-layer decode stack (x <- x + moe_l(rmsnorm(x)), 43 layers with
distinct weights, 32 tokens, int8 activations) through moe_forward_stack,
checked teacher-forced: the input of a sampled layer is rebuilt on the host
from the starting stream and the per-layer outputs the call returns (the
residual update is one fp32 add, reproduced exactly), normalized by the
oracle's RMSNorm and run through the oracle's layer, which must match the
device's output for that layer bit for bit (every step is exact in int8
mode)."""
import numpy as np
import pytest
import torch

import oracle
from fp4_routed_mixture_amd import binding as B
from fp4_routed_mixture_amd import synth as S
from fp4_routed_mixture_amd import synth_device as SD
from gpu_util import oracle_layer, require_gpu

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()
    yield
    torch.cuda.empty_cache()


def _run_stack(w, L):
    layers = []
    for l in range(L):
        layers.append(SD.load_layer(w, l))
    torch.cuda.synchronize()
    cfg = SD.config(w)
    ws = torch.empty(B.moe_stack_workspace_size(cfg), dtype=torch.uint8, device="cuda")
    x0 = S.activations(w)  # fp32 [T][H]
    x = torch.from_numpy(x0).cuda()
    y = torch.empty((L, w.T, w.H), dtype=torch.float32, device="cuda")
    B.moe_forward_stack(cfg, x, layers, ws, layer_out=y)
    torch.cuda.synchronize()
    out = x.cpu().numpy(), y.cpu().numpy()
    del layers, ws, x, y
    torch.cuda.empty_cache()
    return x0, out[0], out[1]


SMALL = {"stack5_tiny": S.Workload("stack5_tiny", 8, 256, 128, 8, 2, S.X_F32, S.ACT_INT8, False, 9, 5),
         "stack3_h1024": S.Workload("stack3_h1024", 24, 1024, 256, 16, 4, S.X_F32, S.ACT_INT8, False, 10, 3)}


@pytest.mark.parametrize("name,L,check", [("stack5_tiny", 5, (0, 1, 2, 3, 4)), ("stack3_h1024", 3, (0, 1, 2)),
                                          ("stack43_decode_t32", 43, (0, 1, 21, 42))])
def test_stack_teacher_forced(name, L, check):
    w = SMALL[name] if name in SMALL else S.WORKLOADS[name]
    print(f"[stack] {S.describe(w)} layers={L}", flush=True)
    x0, xL, y = _run_stack(w, L)
    assert np.isfinite(y).all() and np.isfinite(xL).all()
    # the residual stream, rebuilt on the host
    xs = [x0]
    for l in range(L):
        xs.append((xs[-1] + y[l]).astype(np.float32))
    assert np.array_equal(xs[L], xL)
    for l in check:
        print(f"[stack] layer {l}", flush=True)
        xn = oracle.rmsnorm(xs[l])
        o = oracle_layer(w, xn, layer=l)
        assert np.array_equal(o["out"], y[l]), f"layer {l}: max |diff| {np.abs(o['out'] - y[l]).max()}"


def test_stack_taps_equal_stack():
    """moe_forward_stack_taps with per-layer taps (gate/up events on some
    layers, a layer's y and sort arrays on another) leaves the stream exactly
    as moe_forward_stack does, and its taps hold that layer's data."""
    w = S.Workload("stack_taps", 8, 256, 128, 8, 2, S.X_F32, S.ACT_INT8, False, 13, 4)
    L = w.layers
    layers = [SD.load_layer(w, l) for l in range(L)]
    cfg = SD.config(w)
    ws = torch.empty(B.moe_stack_workspace_size(cfg), dtype=torch.uint8, device="cuda")
    x0 = torch.from_numpy(S.activations(w)).cuda()
    x_ref = x0.clone()
    y_ref = torch.empty((L, w.T, w.H), dtype=torch.float32, device="cuda")
    B.moe_forward_stack(cfg, x_ref, layers, ws, layer_out=y_ref)
    import ctypes as C
    import bench
    he = bench.HipEvents()
    nst = len(B.STAGES)
    gu = B.STAGES.index("gate_up")
    evs = []
    taps = [None] * L
    for l in (0, 2):
        arr = (C.c_void_p * (2 * nst))()
        pair = he.create(2)
        arr[2 * gu], arr[2 * gu + 1] = pair[0], pair[1]
        evs.append(arr)
        taps[l] = {"events": arr}
    P = w.T * w.top_k
    y1 = torch.empty((P, w.H), dtype=torch.float32, device="cuda")
    pos1 = torch.empty(P, dtype=torch.int32, device="cuda")
    taps[1] = {"y": y1, "pair_pos": pos1}
    x = x0.clone()
    bm = B.moe_forward_stack_taps(cfg, x, layers, ws, taps)
    torch.cuda.synchronize()
    assert bm == B.MOE_BLOCK_M_INT8
    assert np.array_equal(x.cpu().numpy(), x_ref.cpu().numpy())
    for arr in evs:
        assert he.elapsed_ms(arr[2 * gu], arr[2 * gu + 1]) > 0
        he.destroy([arr[2 * gu], arr[2 * gu + 1]])
    # layer 1's y tap equals the oracle's per-pair down projections for that
    # layer's input (int8: every step exact)
    o = oracle_layer(w, oracle.rmsnorm((x0 + y_ref[0]).cpu().numpy()), layer=1, intermediates=True)
    assert np.array_equal(y1.cpu().numpy(), o["y"])
