"""Invariants of the layer on the GPU (through the C ABI), in both activation
modes. A pair's result does not depend on where the sort puts it, so
permuting tokens or relabelling experts permutes the outputs bit for bit."""
import numpy as np
import pytest
import torch

from fp4_routed_mixture_amd import binding as B
from fp4_routed_mixture_amd import synth as S
from fp4_routed_mixture_amd import synth_device as SD
from gpu_util import require_gpu, run_forward

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()
    yield
    torch.cuda.empty_cache()


SHAPES = [
    ("inv_int8", 48, 1024, 256, 32, 4, S.ACT_INT8, False),
    ("inv_mxfp4_zipf", 320, 1024, 512, 32, 4, S.ACT_MXFP4, True),
]


@pytest.mark.parametrize("name,T,H,I,E,k,act,zipf", SHAPES)
def test_token_permutation_equivariance(name, T, H, I, E, k, act, zipf):
    w = S.Workload(name, T, H, I, E, k, S.X_BF16, act, zipf, 31)
    lay = SD.load_layer(w)
    x = SD.activations(w)
    perm = torch.from_numpy(np.random.default_rng(0).permutation(T)).cuda()
    a = run_forward(w, lay, x)
    b = run_forward(w, lay, x[perm].contiguous())
    p = perm.cpu().numpy()
    assert np.array_equal(b["ids"], a["ids"][p])
    assert np.array_equal(b["out"], a["out"][p])


@pytest.mark.parametrize("name,T,H,I,E,k,act,zipf", SHAPES)
def test_expert_relabel_equivariance(name, T, H, I, E, k, act, zipf):
    """New expert j = old expert sigma[j]: router rows, bias and the experts'
    prepacked weight blocks move together; ids map back, outputs are equal."""
    w = S.Workload(name, T, H, I, E, k, S.X_BF16, act, zipf, 32)
    lay = SD.load_layer(w)
    x = SD.activations(w)
    sigma = np.random.default_rng(1).permutation(E)
    sg = torch.from_numpy(sigma).cuda()
    rel = {n: lay[n].view(E, -1)[sg].contiguous().view(-1) for n in ("w13", "w13s", "w2", "w2s")}
    rel["router_w"] = lay["router_w"][sg].contiguous()
    rel["bias"] = None if lay["bias"] is None else lay["bias"][sg].contiguous()
    a = run_forward(w, lay, x)
    b = run_forward(w, rel, x)
    assert np.array_equal(sigma[b["ids"]], a["ids"])
    assert np.array_equal(b["out"], a["out"])


@pytest.mark.parametrize("act", [S.ACT_INT8, S.ACT_MXFP4])
def test_zero_weights_give_zero(act):
    w = S.Workload("inv_zero", 20, 512, 256, 8, 2, S.X_F32, act, False, 33)
    lay = SD.load_layer(w)
    for n in ("w13", "w2"):
        lay[n] = torch.zeros_like(lay[n])  # E2M1 code 0 is +0 under any scale
    g = run_forward(w, lay, SD.activations(w))
    assert np.all(g["out"] == 0)


@pytest.mark.parametrize("act", [S.ACT_INT8, S.ACT_MXFP4])
def test_identical_experts_make_router_irrelevant(act):
    """Every expert has expert 0's weights: the output is expert 0's output
    times sum_j w_j = 1 (up to the rounding of the renormalization)."""
    w = S.Workload("inv_same", 24, 512, 256, 8, 3, S.X_F32, act, False, 34)
    lay = SD.load_layer(w)
    same = {n: lay[n].view(w.E, -1)[:1].expand(w.E, -1).contiguous().view(-1) for n in ("w13", "w13s", "w2", "w2s")}
    same["router_w"], same["bias"] = lay["router_w"], None
    g = run_forward(w, same, SD.activations(w))
    w1 = S.Workload("inv_one", 24, 512, 256, 1, 1, S.X_F32, act, False, 34)
    one = {n: lay[n].view(w.E, -1)[:1].contiguous().view(-1) for n in ("w13", "w13s", "w2", "w2s")}
    one["router_w"], one["bias"] = lay["router_w"][:1].contiguous(), None
    o = run_forward(w1, one, SD.activations(w))
    assert np.all(o["w"] == 1.0)
    assert np.allclose(g["out"], o["out"], rtol=8 * 2.0 ** -23, atol=0)
