"""The W2 layout check through the C ABI: W2 rows stored in a permuted order
(codes and scales together) permute the layer's output columns, the host-side
matching identifies the permutation, and moe_prepack's row_perm repairs it at
load time; codes moved without their scales are refused. Checked against the
device's own canonical-layout output and against the oracle."""
import numpy as np
import pytest
import torch

from fp4_routed_mixture_amd import binding as B
from fp4_routed_mixture_amd import layout as L
from fp4_routed_mixture_amd import synth as S
from fp4_routed_mixture_amd import synth_device as SD
from gpu_util import assert_close_rms, oracle_layer, require_gpu, run_forward

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


def _dev(w, packed):
    b = S.router_bias(w)
    return {"w13": packed[0], "w13s": packed[1], "w2": packed[2], "w2s": packed[3],
            "router_w": torch.from_numpy(S.router_weights(w)).cuda(),
            "bias": None if b is None else torch.from_numpy(b).cuda()}


@pytest.mark.parametrize("act_mode,group", [(S.ACT_INT8, 16), (S.ACT_INT8, 32), (S.ACT_MXFP4, 16)])
def test_w2_layout_permutation_detected_and_repaired(act_mode, group):
    w = S.Workload("layout", 48, 1024, 256, 16, 4, S.X_BF16, act_mode, False, 21)
    print(f"[layout] {S.describe(w)} group={group}", flush=True)
    canon = SD.canonical_weights(w)
    x = SD.activations(w)
    ok = run_forward(w, _dev(w, SD.prepack(w, canon)), x)
    # the oracle agrees with the canonical layout (bit for bit in int8 mode)
    o = oracle_layer(w, S.activations(w))
    if act_mode == S.ACT_INT8:
        assert np.array_equal(ok["out"], o["out"])
    else:
        assert_close_rms(ok["out"], o["out"])

    pi = L.interleave_permutation(w.H, group)
    pit = torch.from_numpy(pi.astype(np.int64)).cuda()
    w13, w13s, w2, w2s = canon
    bad_canon = (w13, w13s, w2[:, pit].contiguous(), w2s[:, pit].contiguous())
    bad = run_forward(w, _dev(w, SD.prepack(w, bad_canon)), x)
    assert np.array_equal(bad["ids"], ok["ids"])
    assert not np.array_equal(bad["out"], ok["out"])
    if act_mode == S.ACT_INT8:
        # every step is exact: the columns are permuted bit for bit
        assert np.array_equal(bad["out"], ok["out"][:, pi])
        assert np.array_equal(L.recover_row_permutation(ok["out"], bad["out"]), pi)
    else:
        assert_close_rms(bad["out"], ok["out"][:, pi])

    # repair at load time: packed row r reads stored row inv[r]
    inv = torch.from_numpy(L.inverse_permutation(pi)).cuda()
    fixed = run_forward(w, _dev(w, SD.prepack(w, bad_canon, row_perm2=inv)), x)
    assert np.array_equal(fixed["out"], ok["out"])


def test_w2_codes_without_scales_is_not_a_permutation():
    w = S.Workload("layout", 48, 1024, 256, 16, 4, S.X_BF16, S.ACT_INT8, False, 22)
    canon = SD.canonical_weights(w)
    x = SD.activations(w)
    ok = run_forward(w, _dev(w, SD.prepack(w, canon)), x)
    pit = torch.from_numpy(L.interleave_permutation(w.H, 16).astype(np.int64)).cuda()
    w13, w13s, w2, w2s = canon
    bad = run_forward(w, _dev(w, SD.prepack(w, (w13, w13s, w2[:, pit].contiguous(), w2s))), x)
    with pytest.raises(L.LayoutError):
        L.recover_row_permutation(ok["out"], bad["out"])
