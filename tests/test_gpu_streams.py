"""Concurrent calls on different streams, each with its own workspace and
outputs (the header allows it): the results equal the same calls made one
after another, bit for bit. A decode layer, a prefill layer and an FP8 dense
projection run side by side on three streams of default priority, several
rounds with changing inputs."""
import numpy as np
import pytest
import torch

from fp4_routed_mixture_amd import binding as B
from fp4_routed_mixture_amd import synth as S
from fp4_routed_mixture_amd import synth_device as SD
from gpu_util import require_gpu

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()
    yield
    torch.cuda.empty_cache()


class LayerJob:
    def __init__(self, w):
        self.w = w
        self.L = SD.load_layer(w)
        self.cfg = SD.config(w)
        self.ws = SD.workspace(self.cfg)
        self.inputs = [SD.activations(w, layer=i) for i in range(3)]
        self.out = torch.empty((w.T, w.H), dtype=torch.float32, device="cuda")

    def run(self, i, stream=None):
        L = self.L
        B.moe_forward(self.cfg, self.inputs[i], L["router_w"], L["bias"], L["w13"], L["w13s"], L["w2"], L["w2s"],
                      self.out, None, None, self.ws, stream=stream)


class DenseJob:
    def __init__(self, M, N, K):
        w = S.DenseWorkload("streams_dense", M, K, N, S.X_BF16, 51)
        self.wq, self.wsc = (torch.from_numpy(a).cuda() for a in S.dense_weights(w))
        self.cfg = B.make_dense_config(M, N, K, S.X_BF16)
        self.work = torch.empty(B.moe_dense_fp8_workspace_size(self.cfg), dtype=torch.uint8, device="cuda")
        self.inputs = [torch.from_numpy(S.dense_activations(S.DenseWorkload("d", M, K, N, S.X_BF16, 52 + i))
                                        .view(np.int16)).cuda() for i in range(3)]
        self.out = torch.empty((M, N), dtype=torch.float32, device="cuda")

    def run(self, i, stream=None):
        B.moe_dense_fp8_forward(self.cfg, self.inputs[i], self.wq, self.wsc, self.out, self.work, stream=stream)


def test_concurrent_streams_equal_sequential():
    jobs = [LayerJob(S.Workload("streams_decode", 8, 2048, 1024, 64, 6, S.X_BF16, S.ACT_INT8, False, 53)),
            LayerJob(S.Workload("streams_prefill", 700, 2048, 1024, 32, 4, S.X_BF16, S.ACT_MXFP4, True, 54)),
            DenseJob(300, 2048, 2048)]
    print("[streams] decode T=8, prefill T=700, dense M=300, on three streams", flush=True)
    refs = []
    for i in range(3):
        row = []
        for j in jobs:
            j.run(i)
            torch.cuda.synchronize()
            row.append(j.out.clone())
        refs.append(row)
    streams = [torch.cuda.Stream() for _ in jobs]
    for rnd in range(6):
        i = rnd % 3
        start = torch.cuda.current_stream()
        for s in streams:
            s.wait_stream(start)
        for j, s in zip(jobs, streams):
            with torch.cuda.stream(s):
                for o in range(2):  # two back-to-back calls per stream overlap the other streams' calls
                    j.run((i + o) % 3, stream=s)
        torch.cuda.synchronize()
        last = (i + 1) % 3
        for k, j in enumerate(jobs):
            assert torch.equal(j.out.view(torch.int32), refs[last][k].view(torch.int32)), f"round {rnd} job {k}"
