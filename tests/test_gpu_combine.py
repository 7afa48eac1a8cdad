"""The prefill layer's combine against its definition, element by element:
every output must be the fma chain over the slots (j ascending, from 0) of
the layer's own routing weights and y rows, bit for bit (the layer tests
compare out with the oracle within a tolerance, since y itself rounds in
another order there; this pins the combine step exactly). The calls share
one workspace and their tokens differ (the batch rotated by one, then
reversed), so a y row left over from the previous call, read in place of the
new one, would show; the rotated and reversed batches must also give the
first call's rows moved along with their tokens."""
import numpy as np
import pytest
import torch

from exact_fp import fma32_vec
from fp4_routed_mixture_amd import binding as B
from fp4_routed_mixture_amd import synth as S
from fp4_routed_mixture_amd import synth_device as SD
from gpu_util import require_gpu

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


def fma_chain(wts, y, k):
    """out[t] = fma(w[t][k-1], y[t k + k - 1], ... fma(w[t][0], y[t k], 0))."""
    T = wts.shape[0]
    yr = y.reshape(T, k, -1)
    acc = np.zeros(yr[:, 0].shape, np.float32)
    for j in range(k):
        acc = fma32_vec(np.broadcast_to(wts[:, j:j + 1], acc.shape), yr[:, j], acc)
    return acc


@pytest.mark.parametrize("name", ["tiny_mxfp4", "prefill_t4604_zipf"])
def test_combine_is_the_fma_chain_across_calls(name):
    w = S.WORKLOADS[name]
    print(f"[combine] {S.describe(w)}", flush=True)
    L = SD.load_layer(w, 0)
    x = SD.activations(w)
    T, k, H = x.shape[0], w.top_k, w.H
    cfg = SD.config(w, T)
    ws = SD.workspace(cfg)
    batches = [x, torch.roll(x, shifts=1, dims=0), torch.flip(x, dims=[0])]
    moves = [np.arange(T), np.roll(np.arange(T), 1), np.arange(T)[::-1]]  # row i of the batch = token moves[i]
    first = None
    for call, xb in enumerate(batches):
        xb = xb.contiguous()
        out = torch.empty((T, H), dtype=torch.float32, device="cuda")
        ids = torch.empty((T, k), dtype=torch.int32, device="cuda")
        wts = torch.empty((T, k), dtype=torch.float32, device="cuda")
        taps = {"y": torch.empty((T * k, H), dtype=torch.float32, device="cuda")}
        B.moe_forward_taps(cfg, xb, L["router_w"], L["bias"], L["w13"], L["w13s"], L["w2"], L["w2s"], out, ids, wts,
                           taps, ws)
        torch.cuda.synchronize()
        o, wt, y = out.cpu().numpy(), wts.cpu().numpy(), taps["y"].cpu().numpy()
        want = fma_chain(wt, y, k)
        diff = o.view(np.uint32) != want.view(np.uint32)
        assert not diff.any(), f"call {call}: {diff.sum()} elements differ, first at {np.argwhere(diff)[:3].tolist()}"
        if first is None:
            first = o
        else:
            assert np.array_equal(o.view(np.uint32), first[moves[call]].view(np.uint32)), f"call {call}"
        print(f"  call {call}: {o.size} elements equal the fma chain", flush=True)
        del out, taps, y
    del ws
    torch.cuda.empty_cache()
