"""GPU parity of the individual steps (through the C ABI) against the oracle:
routing, sort, quantization and the load-time prepack are bit-exact."""
import json
import os

import numpy as np
import pytest
import torch

import oracle
from fp4_routed_mixture_amd import binding as B
from fp4_routed_mixture_amd import synth as S
from fp4_routed_mixture_amd import synth_device as SD
from gpu_util import assert_close_rms, oracle_layer, require_gpu, run_forward, sha

pytestmark = pytest.mark.gpu

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "routing_hashes.json")))


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


def test_device_generator_matches_host():
    for (seed, layer, tensor, first, n, scale) in [(0, 0, 0, 0, 4096, False), (1, 3, 2, 8 * 12345, 8192, False),
                                                   (4, 42, 1, 8 * 999, 4096, True), (3, 0, 3, 0, 65536, True)]:
        out = torch.empty(n, dtype=torch.uint8, device="cuda")
        SD.fill(seed, layer, tensor, first, out, scale)
        host = (S.scale_bytes if scale else S.code_bytes)(seed, layer, tensor, first, n)
        assert np.array_equal(out.cpu().numpy(), host), (seed, layer, tensor)


@pytest.mark.parametrize("which", [0, 1])
@pytest.mark.parametrize("shape", [(8, 256, 128), (3, 4096, 2048)])
def test_prepack_roundtrip_and_permutation(which, shape):
    E, H, I = shape
    N, K = (2 * I, H) if which == 0 else (H, I)
    codes = torch.randint(0, 256, (E, N, K // 2), dtype=torch.uint8, device="cuda")
    scales = torch.randint(121, 126, (E, N, K // 32), dtype=torch.uint8, device="cuda")
    cb, sb = B.moe_prepacked_size(which, E, N, K)
    assert cb == codes.numel()
    pc = torch.empty(cb, dtype=torch.uint8, device="cuda")
    ps = torch.empty(sb, dtype=torch.uint8, device="cuda")
    B.moe_prepack(which, E, N, K, codes, scales, None, pc, ps)
    c2, s2 = torch.empty_like(codes), torch.empty_like(scales)
    B.moe_unpack(which, E, N, K, pc, ps, c2, s2)
    torch.cuda.synchronize()
    assert torch.equal(c2, codes) and torch.equal(s2, scales)
    # prepack is a bijection on the code bytes: same multiset
    assert torch.equal(torch.sort(pc).values, torch.sort(codes.flatten()).values)
    # a row permutation is applied to codes and scales together
    perm = torch.randperm(N, device="cuda").to(torch.int32)
    B.moe_prepack(which, E, N, K, codes, scales, perm, pc, ps)
    B.moe_unpack(which, E, N, K, pc, ps, c2, s2)
    torch.cuda.synchronize()
    pl = perm.long()
    assert torch.equal(c2, codes[:, pl]) and torch.equal(s2, scales[:, pl])


ROUTE_CASES = ["tiny", "decode_t4", "decode_t64_zipf", "stack43_decode_t32", "prefill_t4604_zipf",
               "prefill_t16384_zipf"]


@pytest.mark.parametrize("name", ROUTE_CASES)
def test_route_bitexact_and_hashes(name):
    w = S.WORKLOADS[name]
    print(f"[route] {S.describe(w)}", flush=True)
    x_h = S.activations(w)
    wr_h, b_h = S.router_weights(w), S.router_bias(w)
    cfg = SD.config(w)
    ws = SD.workspace(cfg)
    x = SD.activations(w)
    wr = torch.from_numpy(wr_h).cuda()
    b = None if b_h is None else torch.from_numpy(b_h).cuda()
    ids = torch.empty((w.T, w.top_k), dtype=torch.int32, device="cuda")
    wts = torch.empty((w.T, w.top_k), dtype=torch.float32, device="cuda")
    B.moe_route(cfg, x, wr, b, ids, wts, ws)
    torch.cuda.synchronize()
    ids_o, w_o = oracle.route(x_h, wr_h, b_h, w.top_k)
    ids_g, w_g = ids.cpu().numpy(), wts.cpu().numpy()
    assert np.array_equal(ids_g, ids_o), f"{(ids_g != ids_o).sum()} id mismatches"
    assert np.array_equal(w_g.view(np.uint32), w_o.view(np.uint32)), "routing weights differ in bits"
    assert sha(ids_g) == GOLD[name]["ids_sha256"]
    assert sha(w_g) == GOLD[name]["w_sha256"]


@pytest.mark.parametrize("T", [1, 5, 64, 65, 200])
def test_router_kernels_agree(T):
    """The wave-per-expert kernel (small T) and the tiled kernel (large T) give
    the same logits bit for bit; checked through routing on both sides of the
    switch against the oracle."""
    w = S.WORKLOADS["decode_t64_zipf"]
    x_h = S.activations(w, T=T)
    wr_h, b_h = S.router_weights(w), S.router_bias(w)
    cfg = SD.config(w, T)
    ws = SD.workspace(cfg)
    ids = torch.empty((T, w.top_k), dtype=torch.int32, device="cuda")
    wts = torch.empty((T, w.top_k), dtype=torch.float32, device="cuda")
    B.moe_route(cfg, SD.activations(w, T=T), torch.from_numpy(wr_h).cuda(), torch.from_numpy(b_h).cuda(), ids, wts, ws)
    torch.cuda.synchronize()
    ids_o, w_o = oracle.route(x_h, wr_h, b_h, w.top_k)
    assert np.array_equal(ids.cpu().numpy(), ids_o)
    assert np.array_equal(wts.cpu().numpy().view(np.uint32), w_o.view(np.uint32))


# (T, H, E, x dtype): tiny batches (16 four-chunk slices), small batches (64
# one-chunk slices), large batches on the matrix cores (H % 2048 == 0) and on
# the VALU (other H); E not a multiple of a tile included.
LOGIT_CASES = [(4, 4096, 256, S.X_BF16), (16, 4096, 256, S.X_F32), (17, 4096, 256, S.X_BF16),
               (64, 8192, 128, S.X_F32), (65, 4096, 256, S.X_BF16), (300, 4096, 64, S.X_F32),
               (1000, 2048, 100, S.X_BF16), (200, 1024, 256, S.X_BF16), (130, 256, 8, S.X_F32),
               (600, 2304, 96, S.X_BF16), (48, 1280, 40, S.X_F32)]


@pytest.mark.parametrize("T,H,E,xd", LOGIT_CASES)
@pytest.mark.parametrize("data", ["normal", "wide", "subnormal"])
def test_router_logits_bitexact(T, H, E, xd, data):
    """moe_router_logits equals the oracle's pinned reduction order bit for bit.
    'wide' scales every operand by 2^-12 .. 2^12, so the products of one
    logit span 48 binades and nearly every partial sum rounds: a reduction
    that differed from chained fmas in ascending k anywhere would show.
    'subnormal' puts nearly all products below 2^-126 (subnormal fp32) and
    most chunk sums too, with logits on both sides of 2^-126: a step that
    flushed subnormal inputs or results to zero would show."""
    rng = np.random.default_rng(T * 7 + H + E)
    if data == "normal":
        x32 = rng.standard_normal((T, H)).astype(np.float32)
        wr = (0.02 * rng.standard_normal((E, H))).astype(np.float32)
    elif data == "subnormal":
        x32 = (rng.standard_normal((T, H)) * np.exp2(rng.integers(-6, 7, (T, H)) - 62.0)).astype(np.float32)
        wr = (rng.standard_normal((E, H)) * np.exp2(rng.integers(-6, 7, (E, H)) - 74.0)).astype(np.float32)
    else:
        x32 = (rng.standard_normal((T, H)) * np.exp2(rng.integers(-12, 13, (T, H)))).astype(np.float32)
        wr = (rng.standard_normal((E, H)) * np.exp2(rng.integers(-12, 13, (E, H)) - 24.0)).astype(np.float32)
    bias = (0.5 * rng.standard_normal(E)).astype(np.float32)
    if data == "subnormal":
        bias = (rng.standard_normal(E) * 2.0 ** -130).astype(np.float32)  # subnormal too
        prod = x32[0][:, None] * wr.T
        assert ((np.abs(prod) < 2.0 ** -126) & (prod != 0)).mean() > 0.5, "the case must make subnormal products"
    if xd == S.X_F32:
        x_h, x_d = x32, torch.from_numpy(x32).cuda()
    else:
        x_h = S.f32_to_bf16_bits(x32)
        x_d = torch.from_numpy(x_h.view(np.int16)).cuda().view(torch.bfloat16)
    cfg = B.make_config(T, H, 256, E, min(6, E), xd)
    ws = torch.empty(B.moe_workspace_size(cfg), dtype=torch.uint8, device="cuda")
    out = torch.empty((T, E), dtype=torch.float32, device="cuda")
    B.moe_router_logits(cfg, x_d, torch.from_numpy(wr).cuda(), torch.from_numpy(bias).cuda(), out, ws)
    torch.cuda.synchronize()
    ref = oracle.router_logits(x_h, wr, bias)
    got = out.cpu().numpy()
    assert np.array_equal(got.view(np.uint32), ref.view(np.uint32)), f"{(got != ref).sum()} logits differ"


def _gpu_sort(ids_h, E, block_m):
    P = ids_h.size
    T = max(P, 1)
    cfg = B.make_config(T, 256, 128, E, 1)
    cap = P + min(E, P) * (block_m - 1)
    ids = torch.from_numpy(ids_h.astype(np.int32).reshape(-1)).cuda() if P else torch.zeros(1, dtype=torch.int32,
                                                                                            device="cuda")
    counts = torch.empty(E, dtype=torch.int32, device="cuda")
    offsets = torch.empty(E + 1, dtype=torch.int32, device="cuda")
    srt = torch.full((cap + 1,), -7, dtype=torch.int32, device="cuda")
    pos = torch.empty(max(P, 1), dtype=torch.int32, device="cuda")
    tiles = torch.full((cap // block_m + 2,), -7, dtype=torch.int32, device="cuda")
    nt = torch.empty(1, dtype=torch.int32, device="cuda")
    cfg.T = P  # top_k = 1: P = T
    ws = torch.empty(max(P * 4 + 256 + ((P + 1023) // 1024) * E * 4 + 256, 256), dtype=torch.uint8, device="cuda")
    B.moe_sort(cfg, block_m, ids, counts, offsets, srt, pos, tiles, nt, ws)
    torch.cuda.synchronize()
    return {"counts": counts.cpu().numpy(), "offsets": offsets.cpu().numpy(), "sorted": srt.cpu().numpy(),
            "pos": pos.cpu().numpy()[:P], "tiles": tiles.cpu().numpy(), "n_tiles": int(nt.item())}


@pytest.mark.parametrize("P,E,block_m,dist", [(1, 8, 1, "u"), (24, 256, 16, "u"), (384, 256, 16, "zipf"),
                                              (1024, 256, 128, "u"), (1025, 256, 128, "u"),
                                              (27624, 256, 128, "zipf"), (98304, 256, 128, "zipf"),
                                              (5000, 7, 64, "u"), (3000, 1024, 32, "u"), (2000, 8, 128, "one")])
def test_sort_bitexact(P, E, block_m, dist):
    rng = np.random.default_rng(P + E)
    if dist == "u":
        ids = rng.integers(0, E, P)
    elif dist == "one":
        ids = np.full(P, E - 1)
    else:
        p = np.arange(1, E + 1) ** -1.1
        ids = rng.choice(E, P, p=p / p.sum())
    ids = ids.astype(np.int32)
    g = _gpu_sort(ids, E, block_m)
    o = oracle.sort(ids, E, block_m)
    assert np.array_equal(g["counts"], o["counts"])
    assert np.array_equal(g["offsets"], o["offsets"])
    assert np.array_equal(g["sorted"][: o["total"]], o["sorted"])
    assert np.array_equal(g["pos"], o["pos"])
    assert g["n_tiles"] == o["n_tiles"]
    assert np.array_equal(g["tiles"][: o["n_tiles"]], o["tile_expert"])


# Tiny batches (T <= 16, T * E <= 4096) route and sort in one workgroup from
# 16 four-chunk slice sums; other small batches use 64 one-chunk slices and
# the separate top-k and sort kernels. The cases span that switch.
ROUTE_SORT_CASES = [
    ("rs_t1", 1, 4096, 256, 256, 6, S.X_BF16, S.ACT_INT8, False),
    ("rs_t4", 4, 4096, 256, 256, 6, S.X_BF16, S.ACT_INT8, False),
    ("rs_t4_f32", 4, 4096, 256, 256, 6, S.X_F32, S.ACT_INT8, False),
    ("rs_t16_zipf", 16, 4096, 256, 256, 6, S.X_BF16, S.ACT_INT8, True),
    ("rs_t4_e1024", 4, 4096, 256, 1024, 8, S.X_BF16, S.ACT_INT8, False),
    ("rs_t8_e512_k16_mx", 8, 8192, 256, 512, 16, S.X_BF16, S.ACT_MXFP4, True),
    ("rs_t3_f32_mx", 3, 4096, 256, 64, 4, S.X_F32, S.ACT_MXFP4, False),
    ("rs_t16_e512", 16, 4096, 256, 512, 6, S.X_BF16, S.ACT_INT8, False),
    ("rs_t17", 17, 4096, 256, 64, 4, S.X_BF16, S.ACT_INT8, False),
    ("rs_t32_zipf", 32, 4096, 256, 256, 6, S.X_BF16, S.ACT_INT8, True),
    ("rs_t64_zipf", 64, 4096, 256, 256, 6, S.X_BF16, S.ACT_INT8, True),
]


@pytest.mark.parametrize("name,T,H,I,E,k,xd,act,zipf", ROUTE_SORT_CASES)
def test_forward_routing_and_sort_bitexact(name, T, H, I, E, k, xd, act, zipf):
    """The routing and the sort arrays a whole-layer call produces (its taps)
    equal the oracle's route and sort bit for bit, and so does the output in
    int8 mode (MXFP4: within the tolerance)."""
    w = S.Workload(name, T, H, I, E, k, xd, act, zipf, 41)
    print(f"[route+sort] {S.describe(w)}", flush=True)
    g = run_forward(w, SD.load_layer(w), SD.activations(w), taps=True)
    ids_o, w_o = oracle.route(S.activations(w), S.router_weights(w), S.router_bias(w), k)
    assert np.array_equal(g["ids"], ids_o)
    assert np.array_equal(g["w"].view(np.uint32), w_o.view(np.uint32))
    o = oracle.sort(ids_o, E, g["block_m"])
    assert np.array_equal(g["counts"], o["counts"])
    assert np.array_equal(g["offsets"], o["offsets"])
    assert np.array_equal(g["sorted_pairs"][: o["total"]], o["sorted"])
    assert np.array_equal(g["pair_pos"][: T * k], o["pos"])
    ref = oracle_layer(w, S.activations(w))
    if act == S.ACT_INT8:
        assert np.array_equal(g["out"], ref["out"])
    else:
        assert_close_rms(g["out"], ref["out"])


@pytest.mark.parametrize("name", ["tiny", "decode_t4", "prefill_t4604_zipf"])
@pytest.mark.parametrize("mode", [0, 1])
def test_quantize_bitexact(name, mode):
    w = S.WORKLOADS[name]
    x_h = S.activations(w)
    xf = oracle.x_to_f32(x_h)
    cfg = B.make_config(w.T, w.H, w.I, w.E, w.top_k, w.x_dtype, mode)
    x = SD.activations(w)
    if mode == 0:
        q = torch.empty((w.T, w.H), dtype=torch.int8, device="cuda")
        s = torch.empty(w.T, dtype=torch.float32, device="cuda")
        qo, so = oracle.quant_int8(xf)
    else:
        q = torch.empty((w.T, w.H // 2), dtype=torch.uint8, device="cuda")
        s = torch.empty((w.T, w.H // 32), dtype=torch.uint8, device="cuda")
        qo, so = oracle.quant_mxfp4(xf)
    B.moe_quantize(cfg, w.T, w.H, w.x_dtype, x, q, s)
    torch.cuda.synchronize()
    assert np.array_equal(q.cpu().numpy(), qo)
    assert np.array_equal(s.cpu().numpy().view(np.uint8), np.ascontiguousarray(so).view(np.uint8))


def test_rmsnorm_and_residual_bitexact():
    rng = np.random.default_rng(5)
    xh = (rng.standard_normal((32, 4096)) * 1000).astype(np.float32)
    x = torch.from_numpy(xh).cuda()
    out = torch.empty_like(x)
    B.moe_rmsnorm(32, 4096, x, out)
    y = torch.from_numpy((rng.standard_normal((32, 4096))).astype(np.float32)).cuda()
    x2 = x.clone()
    B.moe_residual_add(x2.numel(), x2, y)
    torch.cuda.synchronize()
    assert np.array_equal(out.cpu().numpy().view(np.uint32), oracle.rmsnorm(xh).view(np.uint32))
    assert np.array_equal(x2.cpu().numpy(), (xh + y.cpu().numpy()).astype(np.float32))


@pytest.mark.parametrize("T,E,k", [(3, 256, 6), (200, 256, 6), (5, 1024, 16), (70, 8, 8)])
def test_topk_ties_go_to_lower_index(T, E, k):
    """Exact score ties (zero router weights, a bias with repeated values and
    scores that underflow to 0) are broken toward the lower expert index, and
    the slots follow (score desc, expert asc), as in the oracle."""
    H = 256
    rng = np.random.default_rng(E + T)
    x_h = rng.standard_normal((T, H)).astype(np.float32)
    wr_h = np.zeros((E, H), np.float32)
    levels = np.array([-200.0, -1.0, 0.0, 0.5, 0.5, 3.0], np.float32)
    b_h = levels[rng.integers(0, len(levels), E)]
    cfg = B.make_config(T, H, 128, E, k, S.X_F32, S.ACT_INT8)
    ws = SD.workspace(cfg)
    ids = torch.empty((T, k), dtype=torch.int32, device="cuda")
    wts = torch.empty((T, k), dtype=torch.float32, device="cuda")
    B.moe_route(cfg, torch.from_numpy(x_h).cuda(), torch.from_numpy(wr_h).cuda(), torch.from_numpy(b_h).cuda(), ids,
                wts, ws)
    torch.cuda.synchronize()
    ids_o, w_o = oracle.route(x_h, wr_h, b_h, k)
    assert np.array_equal(ids.cpu().numpy(), ids_o)
    assert np.array_equal(wts.cpu().numpy().view(np.uint32), w_o.view(np.uint32))
    # with every logit equal to its bias, the selection is the stable order
    order = sorted(range(E), key=lambda e: (-float(b_h[e]), e))[:k]
    assert all(list(r) == order for r in ids_o.tolist())


def test_device_exp_sigmoid_bitexact():
    """The kernels' fp32 exp and sigmoid (evaluated for every input, the
    out-of-range results selected afterwards) equal the oracle's bit for bit
    on 2^24 inputs spread over [-110, 95] plus the range edges, their
    neighbours, +-0, +-inf, NaN and subnormals."""
    rng = np.random.default_rng(77)
    z = np.concatenate([
        np.linspace(-110.0, 95.0, 1 << 23, dtype=np.float32),
        rng.uniform(-110.0, 95.0, 1 << 23).astype(np.float32),
        np.array([0.0, -0.0, np.inf, -np.inf, np.nan, 1e-45, -1e-45, 1e-38, -1e-38, 88.72283, -103.97208],
                 np.float32)])
    edges = np.array([float.fromhex("0x1.62e42ep+6"), -float.fromhex("0x1.9fe36ap+6")], np.float32)
    z = np.concatenate([z, np.nextafter(edges, np.float32(np.inf)), np.nextafter(edges, np.float32(-np.inf)), edges])
    e, s = SD.exp_sigmoid(torch.from_numpy(z).cuda())
    torch.cuda.synchronize()
    e, s = e.cpu().numpy(), s.cpu().numpy()
    ref_e, ref_s = oracle.expf(z), oracle.sigmoidf(z)
    assert np.array_equal(e.view(np.uint32), ref_e.view(np.uint32)), f"{(e.view(np.uint32) != ref_e.view(np.uint32)).sum()} exp differ"
    assert np.array_equal(s.view(np.uint32), ref_s.view(np.uint32)), f"{(s.view(np.uint32) != ref_s.view(np.uint32)).sum()} sigmoid differ"
