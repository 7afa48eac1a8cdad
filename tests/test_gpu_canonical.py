"""moe_forward on weights in the canonical interchange layout (weight_layout =
MOE_LAYOUT_CANONICAL) equals the call on the prepacked copy of the same
weights bit for bit: the kernels differ only in their weight address maps.
Both are checked against the oracle where the prepacked path is."""
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


def _forward(w, lay, x, layout, T=None):
    T = x.shape[0]
    cfg = SD.config(w, T, weight_layout=layout)
    ws = SD.workspace(cfg)
    out = torch.empty((T, w.H), dtype=torch.float32, device="cuda")
    ids = torch.empty((T, w.top_k), dtype=torch.int32, device="cuda")
    wts = torch.empty((T, w.top_k), dtype=torch.float32, device="cuda")
    if layout == B.MOE_LAYOUT_CANONICAL:
        w13, w13s, w2, w2s = lay["canonical"]
    else:
        w13, w13s, w2, w2s = lay["w13"], lay["w13s"], lay["w2"], lay["w2s"]
    B.moe_forward(cfg, x, lay["router_w"], lay["bias"], w13, w13s, w2, w2s, out, ids, wts, ws)
    torch.cuda.synchronize()
    return out.cpu().numpy(), ids.cpu().numpy()


# I = 384 gives the down GEMM K = 384: a last K-step group of two steps,
# whose canonical scale row ends four bytes into the group
SMALL = [S.Workload("canon_i384_int8", 9, 512, 384, 8, 3, S.X_BF16, S.ACT_INT8, False, 21),
         S.Workload("canon_i384_mx", 70, 512, 384, 8, 3, S.X_BF16, S.ACT_MXFP4, False, 22)]


@pytest.mark.parametrize("name", ["tiny", "tiny_mxfp4", "decode_t4", "decode_t64_zipf", "canon_i384_int8",
                                  "canon_i384_mx", "prefill_t4604_zipf"])
def test_canonical_equals_prepacked(name):
    w = {x.name: x for x in SMALL}.get(name) or S.WORKLOADS[name]
    print(f"[canonical] {S.describe(w)}", flush=True)
    lay = SD.load_layer(w, keep_canonical=True)
    x = SD.activations(w)
    out_c, ids_c = _forward(w, lay, x, B.MOE_LAYOUT_CANONICAL)
    out_p, ids_p = _forward(w, lay, x, B.MOE_LAYOUT_PREPACKED)
    del lay
    torch.cuda.empty_cache()
    assert np.array_equal(ids_c, ids_p)
    assert np.array_equal(out_c.view(np.uint32), out_p.view(np.uint32)), "canonical and prepacked outputs differ"
    if w.T <= 70:
        o = oracle_layer(w, S.activations(w))
        assert np.array_equal(ids_c, o["ids"])
        assert_close_rms(out_c, o["out"])


def test_canonical_routed_and_stack():
    """The router-free layer and a two-layer stack read canonical weights too."""
    w = S.Workload("canon_stack", 8, 256, 128, 8, 2, S.X_F32, S.ACT_INT8, False, 23, 2)
    lays = [SD.load_layer(w, l, keep_canonical=True) for l in range(2)]
    x0 = torch.from_numpy(S.activations(w)).cuda()
    outs = {}
    for layout in (B.MOE_LAYOUT_CANONICAL, B.MOE_LAYOUT_PREPACKED):
        cfg = SD.config(w, weight_layout=layout)
        if layout == B.MOE_LAYOUT_CANONICAL:
            dl = [dict(router_w=L["router_w"], bias=L["bias"], w13=L["canonical"][0], w13s=L["canonical"][1],
                       w2=L["canonical"][2], w2s=L["canonical"][3]) for L in lays]
        else:
            dl = lays
        ws = torch.empty(B.moe_stack_workspace_size(cfg), dtype=torch.uint8, device="cuda")
        x = x0.clone()
        B.moe_forward_stack(cfg, x, dl, ws)
        ids = torch.from_numpy(np.array([[1, 5], [0, 7], [3, 3 ^ 1], [6, 2], [4, 0], [2, 6], [7, 1], [5, 4]],
                                        np.int32)).cuda()
        wts = torch.full((w.T, 2), 0.5, dtype=torch.float32, device="cuda")
        out = torch.empty((w.T, w.H), dtype=torch.float32, device="cuda")
        B.moe_forward_routed(cfg, x0, ids, wts, dl[0]["w13"], dl[0]["w13s"], dl[0]["w2"], dl[0]["w2s"], out,
                             SD.workspace(cfg))
        torch.cuda.synchronize()
        outs[layout] = (x.cpu().numpy(), out.cpu().numpy())
    for a, b in zip(outs[B.MOE_LAYOUT_CANONICAL], outs[B.MOE_LAYOUT_PREPACKED]):
        assert np.array_equal(a.view(np.uint32), b.view(np.uint32))
