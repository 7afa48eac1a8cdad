"""moe_forward_noalloc (the layer on the library's fixed per-device scratch
array, for callers that cannot allocate) against moe_forward on a caller
workspace: the same kernels, so the same bits, on two calls in a row, the
second with a smaller batch (the array keeps the first call's contents).
Collected last: it must also pass in a fresh process run alone."""
import ctypes as C

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


def _call(w, lay, T, noalloc):
    x = SD.activations(w, T=T)
    cfg = SD.config(w, T)
    out = torch.full((T, w.H), float("nan"), dtype=torch.float32, device="cuda")
    ids = torch.full((T, w.top_k), -1, dtype=torch.int32, device="cuda")
    wts = torch.empty((T, w.top_k), dtype=torch.float32, device="cuda")
    args = (cfg, x, lay["router_w"], lay["bias"], lay["w13"], lay["w13s"], lay["w2"], lay["w2s"], out, ids, wts)
    if noalloc:
        B.moe_forward_noalloc(*args)
    else:
        B.moe_forward(*args, SD.workspace(cfg))
    torch.cuda.synchronize()
    return out.cpu().numpy(), ids.cpu().numpy(), wts.cpu().numpy()


# (workload, first T, second smaller T): int8 decode up to 64 tokens (60 MiB
# of scratch) and MXFP4 batches within the 64 MiB array
CASES = [("decode_t64_zipf", 64, 4), ("decode_t4", 4, 1), ("prefill_t4604_zipf", 300, 37), ("tiny_mxfp4", 4, 3)]


@pytest.mark.parametrize("name,t1,t2", CASES)
def test_noalloc_equals_workspace_call(name, t1, t2):
    w = S.WORKLOADS[name]
    print(f"[noalloc] {S.describe(w)} T={t1} then T={t2}", flush=True)
    lay = SD.load_layer(w)
    for T in (t1, t2):
        got = _call(w, lay, T, noalloc=True)
        ref = _call(w, lay, T, noalloc=False)
        for g, r in zip(got, ref):
            assert np.array_equal(g.view(np.uint32), r.view(np.uint32)), f"T={T}: noalloc differs from moe_forward"
        if T <= 64:
            o = oracle_layer(w, S.activations(w, T=T))
            assert np.array_equal(got[1], o["ids"])
            assert_close_rms(got[0], o["out"])
    del lay


def test_noalloc_rejects_configs_beyond_the_array():
    """A batch whose workspace exceeds the array is refused before any launch."""
    w = S.WORKLOADS["prefill_t4604_zipf"]
    cfg = SD.config(w)
    assert B.moe_workspace_size(cfg) > B.MOE_NOALLOC_SCRATCH_BYTES
    st = B.lib().moe_forward_noalloc(C.byref(cfg), 0x10000, 0x10000, None, 0x10000, 0x10000, 0x10000, 0x10000,
                                     0x10000 + (1 << 30), None, None, None)
    assert st == 5
