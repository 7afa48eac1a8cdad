"""Block-scaled FP8 (MXFP8) dense projection through the C ABI against the
oracle: the activation quantizer bit for bit, the GEMM within the fp32
accumulation bound of the exact block sums."""
import numpy as np
import pytest
import torch

import oracle
from fp4_routed_mixture_amd import binding as B
from fp4_routed_mixture_amd import synth as S
from gpu_util import require_gpu

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


def x_f32(x):
    return (x.astype(np.uint32) << 16).view(np.float32) if x.dtype == np.uint16 else x


def to_dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def e4m3_exponents(codes):
    """floor(log2 |v|) of each E4M3 code's value, -6 (the exponent field's
    value) for subnormals, -inf for zeros."""
    t = np.abs(oracle.e4m3_table().astype(np.float64))
    e = np.full(256, -np.inf)
    nz = (t > 0) & np.isfinite(t)
    e[nz] = np.maximum(np.floor(np.log2(t[nz])), -6.0)
    return e[codes]


def group_truncation_bound(xq, xs, wq, ws):
    """The matrix cores' FP8 summation (measured on gfx950, one 32x32x64
    scaled MFMA): products are added in groups of 8 consecutive k, each
    truncated toward zero at 2^(E_g - 13), E_g the largest exponent sum
    e(x_k) + e(w_k) + (sx_b - 127) + (sw_b - 127) in the group; so a
    group's sum is short of exact by less than 8 * 2^(E_g - 13). Returns
    sum_g 2^(E_g - 10) per output."""
    ex, ew = e4m3_exponents(xq), e4m3_exponents(wq)
    M, K = xq.shape
    N = wq.shape[0]
    sx = np.repeat(xs.astype(np.float64) - 127, 4, axis=1)  # per group of 8
    sw = np.repeat(ws.astype(np.float64) - 127, 4, axis=1)
    out = np.zeros((M, N))
    for g in range(K // 8):
        eg = np.full((M, N), -np.inf)
        for k in range(8 * g, 8 * g + 8):
            np.maximum(eg, ex[:, k][:, None] + ew[:, k][None, :], out=eg)
        out += np.exp2(eg + sx[:, g][:, None] + sw[:, g][None, :] - 10)
    return out


def check_bound(y, ref, ab, trunc, K, what):
    """|y - ref| <= (the group truncation bound) + K 2^-23 sum|terms| (fp32
    additions of the group sums, one rounding of unspecified mode each) +
    K 2^-126 (should terms in the fp32 subnormal range be flushed)."""
    err = np.abs(y.astype(np.float64) - ref.astype(np.float64))
    lim = trunc + K * 2.0 ** -23 * ab + K * 2.0 ** -126
    bad = err > lim
    assert not bad.any(), f"{what}: {bad.sum()} outside the bound, worst {(err / lim).max():.3g} of it"
    rms_ref = np.sqrt(np.mean(ref.astype(np.float64) ** 2))
    print(f"  {what}: max err {(err / lim).max():.3g} of the bound, rms err/rms {np.sqrt(np.mean(err**2))/rms_ref:.3g}")


def oracle_with_bound(xq, xs, wq, ws):
    ref, ab = oracle.dense_mxfp8(xq, xs, wq, ws, bound=True)
    return ref, ab, group_truncation_bound(xq, xs, wq, ws)


def special_rows(K=256):
    """Rows that exercise the quantizer's edges: zeros and -0, exact E4M3
    midpoints (ties), the saturation range, subnormal E4M3 results, fp32
    subnormal inputs, scales far from 127 and the clamps."""
    rng = np.random.default_rng(99)
    rows = []
    r = np.zeros(K, np.float32)
    r[1] = -0.0
    rows.append(r)                                        # all-zero blocks (one with -0)
    r = rng.standard_normal(K).astype(np.float32)
    r[0::32] = 256.0                                      # amax = 256: scale byte 127
    rows.append(r)
    t = oracle.e4m3_table().astype(np.float64)
    mags = np.unique(np.abs(t[np.isfinite(t)]))
    mids = ((mags[1:] + mags[:-1]) / 2).astype(np.float32)  # exact midpoints in fp32
    r = np.resize(mids, K).astype(np.float32)
    r[0::32] = 256.0                                      # keep the scale at 127
    r[1::2] *= -1
    rows.append(r)
    r = np.linspace(448.0, 511.0, K).astype(np.float32)   # scaled values in the saturation range
    r[0::32] = 511.0
    rows.append(r)
    r = (rng.standard_normal(K) * 2.0 ** -12).astype(np.float32)
    r[0::32] = 256.0                                      # subnormal E4M3 codes
    rows.append(r)
    rows.append((rng.standard_normal(K) * 2.0 ** -140).astype(np.float32))   # fp32 subnormal inputs
    rows.append((rng.standard_normal(K) * 2.0 ** 120).astype(np.float32))    # scale byte near 239
    rows.append((rng.standard_normal(K) * 2.0 ** -120).astype(np.float32))   # scale byte near 0
    r = np.full(K, 2.0 ** -149, np.float32)               # amax 2^-149: the scale clamps at 0
    r[3::7] = -(2.0 ** -149)
    rows.append(r)
    r = np.full(K, np.float32(3.3e38))
    r[::3] = -1.0e30                                      # amax near fp32 max
    rows.append(r)
    return np.stack(rows)


@pytest.mark.parametrize("case", ["dense_tiny", "dense_t32", "special_f32", "special_bf16", "dense_t4604", "kmax_bf16"])
def test_quantize_bitexact(case):
    if case == "kmax_bf16":
        # the quantizer's largest K (65536) on rows of mixed magnitude
        rng = np.random.default_rng(45)
        x = (rng.standard_normal((5, 65536)) * np.exp2(rng.integers(-30, 31, (5, 2048))).repeat(32, axis=1))
        x = S.f32_to_bf16_bits(x.astype(np.float32))
        in_dtype = B.MOE_X_BF16
    elif case.startswith("special"):
        x = special_rows()
        in_dtype = B.MOE_X_F32
        if case == "special_bf16":
            x = S.f32_to_bf16_bits(x)
            in_dtype = B.MOE_X_BF16
    else:
        w = S.DENSE_WORKLOADS[case]
        x = S.dense_activations(w)
        in_dtype = w.x_dtype
    R, K = x.shape
    print(f"[dense quantize] {case} rows={R} K={K}", flush=True)
    codes = torch.empty((R, K), dtype=torch.uint8, device="cuda")
    scales = torch.empty((R, K // 32), dtype=torch.uint8, device="cuda")
    B.moe_dense_fp8_quantize(R, K, in_dtype, to_dev(x), codes, scales)
    torch.cuda.synchronize()
    oc, os_ = oracle.quant_mxfp8(x_f32(x))
    assert np.array_equal(scales.cpu().numpy(), os_)
    got = codes.cpu().numpy()
    diff = got != oc
    assert not diff.any(), f"{diff.sum()} codes differ, first at {np.argwhere(diff)[:4].tolist()}"


def dense_case(name):
    """(M, N, K, x_dtype, seed) of the named parity case."""
    if name in S.DENSE_WORKLOADS:
        w = S.DENSE_WORKLOADS[name]
        return w
    extra = {
        # M above 32 with a ragged last 64-row tile and K % 256 == 128 (a
        # last half group); a single 32-row tile in the wide kernel (M = 33
        # .. 64 uses both token tiles, M <= 32 the small-batch kernel)
        "dense_m100_k384": S.DenseWorkload("dense_m100_k384", 100, 384, 512, S.X_F32, 31),
        "dense_m33_k128": S.DenseWorkload("dense_m33_k128", 33, 128, 256, S.X_BF16, 32),
        "dense_m64_k640": S.DenseWorkload("dense_m64_k640", 64, 640, 768, S.X_BF16, 33),
        "dense_m1_k4096": S.DenseWorkload("dense_m1_k4096", 1, 4096, 1536, S.X_BF16, 34),
        "dense_m17_k1152": S.DenseWorkload("dense_m17_k1152", 17, 1152, 8192, S.X_F32, 35),
        "dense_m200_k2048": S.DenseWorkload("dense_m200_k2048", 200, 2048, 2304, S.X_BF16, 36),
        # the largest K the ABI accepts, on both kernels: 128-row wide tiles
        # over 512 K-steps, and the small-batch kernel split 8 ways along K
        # (16 chunks of four K-steps per part)
        "dense_m40_kmax": S.DenseWorkload("dense_m40_kmax", 40, 32768, 256, S.X_BF16, 38),
        "dense_m3_kmax": S.DenseWorkload("dense_m3_kmax", 3, 32768, 512, S.X_F32, 39),
        # the largest N: 256 workgroups of 256 features, 2048 small-batch tiles
        "dense_m40_nmax": S.DenseWorkload("dense_m40_nmax", 40, 128, 65536, S.X_BF16, 41),
        "dense_m3_nmax": S.DenseWorkload("dense_m3_nmax", 3, 256, 65536, S.X_F32, 42),
    }
    return extra[name]


def run_gemm(w, xq, xs, wq, ws):
    cfg = B.make_dense_config(xq.shape[0], w.N, w.K, w.x_dtype)
    work = torch.empty(max(B.moe_dense_fp8_workspace_size(cfg), 1), dtype=torch.uint8, device="cuda")
    y = torch.empty((cfg.M, w.N), dtype=torch.float32, device="cuda")
    B.moe_dense_fp8_gemm(cfg, to_dev(xq), to_dev(xs), wq, ws, y, work)
    torch.cuda.synchronize()
    return y.cpu().numpy()


@pytest.mark.parametrize("name", ["dense_tiny", "dense_t32", "dense_m100_k384", "dense_m33_k128", "dense_m64_k640",
                                  "dense_m1_k4096", "dense_m17_k1152", "dense_m200_k2048", "dense_m40_kmax",
                                  "dense_m3_kmax", "dense_m40_nmax", "dense_m3_nmax"])
def test_gemm_parity(name):
    w = dense_case(name)
    print(f"[dense gemm] {name} M={w.M} N={w.N} K={w.K}", flush=True)
    wq_h, ws_h = S.dense_weights(w)
    xq, xs = oracle.quant_mxfp8(x_f32(S.dense_activations(w)))
    y = run_gemm(w, xq, xs, to_dev(wq_h), to_dev(ws_h))
    check_bound(y, *oracle_with_bound(xq, xs, wq_h, ws_h), w.K, name)


@pytest.mark.parametrize("M,N,K", [(32, 4096, 1024), (5, 512, 768), (200, 2304, 1024), (100, 512, 384),
                                   (64, 256, 128)])
def test_gemm_bitexact_narrow_range(M, N, K):
    """Codes with exponent fields 7 and 8 (|v| in [1, 3.75]) and scale bytes
    126..128: within a group of 8 every product keeps all its bits (the
    lowest, 2^(E_g - 8), lies above the truncation point 2^(E_g - 13)), and
    every partial sum is a multiple of 2^-7 below 2^17, exact in fp32. So
    the result must equal the exact value bit for bit, whatever the order of
    the additions: any misplaced element, scale byte or K-step shows."""
    print(f"[dense gemm exact] M={M} N={N} K={K}", flush=True)
    rng = np.random.default_rng([M, N, K])
    code = lambda shape: (rng.integers(0x38, 0x48, shape) | (rng.integers(0, 2, shape) << 7)).astype(np.uint8)
    xq, wq = code((M, K)), code((N, K))
    xs = rng.integers(127, 129, (M, K // 32)).astype(np.uint8)
    ws = rng.integers(126, 128, (N, K // 32)).astype(np.uint8)
    w = S.DenseWorkload("narrow", M, K, N, S.X_F32, 0)
    y = run_gemm(w, xq, xs, to_dev(wq), to_dev(ws))
    ref = oracle.dense_mxfp8(xq, xs, wq, ws)
    diff = y.view(np.uint32) != ref.view(np.uint32)
    assert not diff.any(), f"{diff.sum()} outputs differ, first at {np.argwhere(diff)[:4].tolist()}"


def test_gemm_special_scales():
    """Activation rows with scale bytes from 0 to 199 and subnormal E4M3
    codes, against weights with their generated scales: each lane's E8M0
    byte must reach the right 32-element block (bytes below 200 keep every
    sum finite)."""
    x = special_rows(512)
    w = S.DenseWorkload("dense_special", x.shape[0], 512, 256, S.X_F32, 37)
    wq_h, ws_h = S.dense_weights(w)
    xq, xs = oracle.quant_mxfp8(x)
    # per-block scale bytes that differ block by block in every row
    xs = ((xs.astype(np.int32) + np.arange(xs.shape[1])[None, :] % 5) % 200).astype(np.uint8)
    y = run_gemm(w, xq, xs, to_dev(wq_h), to_dev(ws_h))
    check_bound(y, *oracle_with_bound(xq, xs, wq_h, ws_h), w.K, "special scales")


@pytest.mark.parametrize("name", ["dense_t4604", "dense_t16384", "dense_t4604_n1536"])
def test_forward_full_size_sampled(name):
    """The full-size projection as timed (prepacked weights; quantize on the
    device, then the GEMM), checked on sampled token rows: the first rows,
    both sides of the 128-row wave tile and the 256-row workgroup tile
    boundaries, the last (ragged) rows and rows spread over the batch."""
    w = S.DENSE_WORKLOADS[name]
    print(f"[dense forward] {name} M={w.M} N={w.N} K={w.K}", flush=True)
    wq_h, ws_h = S.dense_weights(w)
    cb, sb = B.moe_dense_fp8_prepacked_size(w.N, w.K)
    pw = torch.empty(cb, dtype=torch.uint8, device="cuda")
    ps = torch.empty(sb, dtype=torch.uint8, device="cuda")
    B.moe_dense_fp8_prepack(w.N, w.K, to_dev(wq_h), to_dev(ws_h), pw, ps)
    x = S.dense_activations(w)
    cfg = B.make_dense_config(w.M, w.N, w.K, w.x_dtype, B.MOE_LAYOUT_PREPACKED)
    work = torch.empty(B.moe_dense_fp8_workspace_size(cfg), dtype=torch.uint8, device="cuda")
    y = torch.empty((w.M, w.N), dtype=torch.float32, device="cuda")
    B.moe_dense_fp8_forward(cfg, to_dev(x), pw, ps, y, work)
    torch.cuda.synchronize()
    rows = np.unique(np.concatenate([np.arange(0, 3), np.arange(126, 130), np.arange(254, 258),
                                     np.arange(w.M - 6, w.M),
                                     np.random.default_rng(5).choice(w.M, 20, replace=False)]))
    rows = rows[rows < w.M]
    xq, xs = oracle.quant_mxfp8(x_f32(x[rows]))
    check_bound(y[torch.from_numpy(rows).cuda()].cpu().numpy(), *oracle_with_bound(xq, xs, wq_h, ws_h), w.K, name)


def test_forward_max_rows_sampled():
    """2^20 token rows of K = 3968, so that the quantized rows fill 4.16e9 of
    the 2^32 bytes the token offsets may span: sampled rows at the start, on
    both sides of the 2^31-byte point and at the end must match the oracle.
    The activations come from torch's seeded device generator (a bf16 normal
    with a per-row power-of-two spread); only the sampled rows come to the
    host."""
    M, K, N = 1 << 20, 3968, 256
    print(f"[dense forward max rows] M={M} N={N} K={K}", flush=True)
    gen = torch.Generator(device="cuda")
    gen.manual_seed(43)
    x = torch.empty((M, K), dtype=torch.bfloat16, device="cuda")
    step = 1 << 16
    for i in range(0, M, step):
        spread = torch.exp2(torch.randint(-6, 7, (step, 1), generator=gen, device="cuda").float())
        x[i:i + step] = (torch.randn((step, K), generator=gen, device="cuda") * spread).to(torch.bfloat16)
    w = S.DenseWorkload("dense_max_rows", 1, K, N, S.X_BF16, 44)
    wq_h, ws_h = S.dense_weights(w)
    cfg = B.make_dense_config(M, N, K, B.MOE_X_BF16)
    work = torch.empty(B.moe_dense_fp8_workspace_size(cfg), dtype=torch.uint8, device="cuda")
    y = torch.empty((M, N), dtype=torch.float32, device="cuda")
    B.moe_dense_fp8_forward(cfg, x, to_dev(wq_h), to_dev(ws_h), y, work)
    torch.cuda.synchronize()
    mid = (1 << 31) // K
    rows = np.unique(np.concatenate([np.arange(0, 3), np.arange(mid - 2, mid + 3), np.arange(M - 4, M),
                                     np.random.default_rng(6).choice(M, 16, replace=False)]))
    idx = torch.from_numpy(rows).cuda()
    xr = x[idx].view(torch.int16).cpu().numpy().view(np.uint16)
    xq, xs = oracle.quant_mxfp8(x_f32(xr))
    check_bound(y[idx].cpu().numpy(), *oracle_with_bound(xq, xs, wq_h, ws_h), K, "max rows")
    del x, work, y
    torch.cuda.empty_cache()


def test_forward_equals_quantize_then_gemm_and_repeats():
    """moe_dense_fp8_forward is the quantizer followed by the GEMM, bit for
    bit, and two runs give the same bits (no atomics, fixed sum orders)."""
    for name in ("dense_t32", "dense_m200_k2048"):
        w = dense_case(name)
        wq, ws = (to_dev(a) for a in S.dense_weights(w))
        x = to_dev(S.dense_activations(w))
        cfg = B.make_dense_config(w.M, w.N, w.K, w.x_dtype)
        work = torch.empty(B.moe_dense_fp8_workspace_size(cfg), dtype=torch.uint8, device="cuda")
        y1 = torch.empty((w.M, w.N), dtype=torch.float32, device="cuda")
        y2 = torch.empty_like(y1)
        B.moe_dense_fp8_forward(cfg, x, wq, ws, y1, work)
        B.moe_dense_fp8_forward(cfg, x, wq, ws, y2, work)
        codes = torch.empty((w.M, w.K), dtype=torch.uint8, device="cuda")
        scales = torch.empty((w.M, w.K // 32), dtype=torch.uint8, device="cuda")
        B.moe_dense_fp8_quantize(w.M, w.K, w.x_dtype, x, codes, scales)
        y3 = torch.empty_like(y1)
        B.moe_dense_fp8_gemm(cfg, codes, scales, wq, ws, y3, work)
        torch.cuda.synchronize()
        assert torch.equal(y1.view(torch.int32), y2.view(torch.int32)), name
        assert torch.equal(y1.view(torch.int32), y3.view(torch.int32)), name


def test_zero_rows_and_errors():
    cfg = B.make_dense_config(0, 256, 256, B.MOE_X_F32)
    B.moe_dense_fp8_forward(cfg, None, None, None, None, torch.empty(1, dtype=torch.uint8, device="cuda"))
    cfg = B.make_dense_config(4, 256, 256, B.MOE_X_F32)
    x = torch.zeros((4, 256), dtype=torch.float32, device="cuda")
    w = torch.zeros((256, 256), dtype=torch.uint8, device="cuda")
    s = torch.full((256, 8), 127, dtype=torch.uint8, device="cuda")
    y = torch.empty((4, 256), dtype=torch.float32, device="cuda")
    with pytest.raises(B.MoEError):
        B.moe_dense_fp8_forward(cfg, x, w, s, y, torch.empty(1, dtype=torch.uint8, device="cuda"))
    work = torch.empty(B.moe_dense_fp8_workspace_size(cfg), dtype=torch.uint8, device="cuda")
    B.moe_dense_fp8_forward(cfg, x, w, s, y, work)
    torch.cuda.synchronize()
    assert torch.all(y == 0)


def host_pack(wq, ws):
    """The prepacked layout as the header defines it, built on the host."""
    N, K = wq.shape
    KT, G = K // 64, (K // 64 + 3) // 4
    pc = np.empty((N // 32, KT, 2, 64, 16), np.uint8)
    ps = np.full((N // 32, G, 64, 4), 127, np.uint8)
    for l in range(64):
        c, h = l % 32, l // 32
        for p in range(2):
            for kt in range(KT):
                k0 = 64 * kt + 32 * p + 16 * h
                pc[:, kt, p, l, :] = wq[c::32, k0:k0 + 16]
        for g in range(G):
            for j in range(4):
                if 4 * g + j < KT:
                    ps[:, g, l, j] = ws[c::32, 2 * (4 * g + j) + h]
    return pc.reshape(-1), ps.reshape(-1)


@pytest.mark.parametrize("N,K", [(64, 384), (512, 4096)])
def test_prepack_layout_and_roundtrip(N, K):
    w = S.DenseWorkload("pack", 1, K, N, S.X_F32, 40)
    wq, ws = S.dense_weights(w)
    cb, sb = B.moe_dense_fp8_prepacked_size(N, K)
    pw = torch.empty(cb, dtype=torch.uint8, device="cuda")
    ps = torch.empty(sb, dtype=torch.uint8, device="cuda")
    B.moe_dense_fp8_prepack(N, K, to_dev(wq), to_dev(ws), pw, ps)
    uq = torch.empty((N, K), dtype=torch.uint8, device="cuda")
    us = torch.empty((N, K // 32), dtype=torch.uint8, device="cuda")
    B.moe_dense_fp8_unpack(N, K, pw, ps, uq, us)
    torch.cuda.synchronize()
    hc, hs = host_pack(wq, ws)
    assert np.array_equal(pw.cpu().numpy(), hc)
    assert np.array_equal(ps.cpu().numpy(), hs)
    assert np.array_equal(uq.cpu().numpy(), wq) and np.array_equal(us.cpu().numpy(), ws)


@pytest.mark.parametrize("name", ["dense_tiny", "dense_t32", "dense_m1_k4096", "dense_m17_k1152", "dense_m100_k384",
                                  "dense_m64_k640", "dense_m200_k2048"])
def test_prepacked_equals_canonical(name):
    """The GEMMs on prepacked weights give the canonical-layout result bit for
    bit (the kernels differ only in their weight address maps), through both
    entry points."""
    w = dense_case(name)
    print(f"[dense prepacked] {name} M={w.M} N={w.N} K={w.K}", flush=True)
    wq_h, ws_h = S.dense_weights(w)
    wq, ws = to_dev(wq_h), to_dev(ws_h)
    cb, sb = B.moe_dense_fp8_prepacked_size(w.N, w.K)
    pw = torch.empty(cb, dtype=torch.uint8, device="cuda")
    ps = torch.empty(sb, dtype=torch.uint8, device="cuda")
    B.moe_dense_fp8_prepack(w.N, w.K, wq, ws, pw, ps)
    x = to_dev(S.dense_activations(w))
    xq_h, xs_h = oracle.quant_mxfp8(x_f32(S.dense_activations(w)))
    outs = []
    for layout, (a, b) in ((B.MOE_LAYOUT_CANONICAL, (wq, ws)), (B.MOE_LAYOUT_PREPACKED, (pw, ps))):
        cfg = B.make_dense_config(w.M, w.N, w.K, w.x_dtype, layout)
        work = torch.empty(max(B.moe_dense_fp8_workspace_size(cfg), 1), dtype=torch.uint8, device="cuda")
        y1 = torch.empty((w.M, w.N), dtype=torch.float32, device="cuda")
        y2 = torch.empty_like(y1)
        B.moe_dense_fp8_forward(cfg, x, a, b, y1, work)
        B.moe_dense_fp8_gemm(cfg, to_dev(xq_h), to_dev(xs_h), a, b, y2, work)
        torch.cuda.synchronize()
        outs.append((y1.cpu().numpy(), y2.cpu().numpy()))
    for i in range(2):
        assert np.array_equal(outs[0][i].view(np.uint32), outs[1][i].view(np.uint32)), name
    check_bound(outs[1][1], *oracle_with_bound(xq_h, xs_h, wq_h, ws_h), w.K, name)


def _sweep(n=12, seed=2027):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        out.append((int(rng.choice([1, 2, 7, 31, 32, 33, 64, 129, 200])), 256 * int(rng.integers(1, 9)),
                    128 * int(rng.integers(1, 17)), int(rng.integers(0, 2)), int(rng.integers(0, 2)), 60 + i))
    return out


@pytest.mark.parametrize("M,N,K,layout,xd,seed", _sweep())
def test_forward_shape_sweep(M, N, K, layout, xd, seed):
    """A seeded sweep of shapes through moe_dense_fp8_forward, either weight
    layout and either activation type: the quantized x must match the oracle
    (checked through the GEMM input it implies) and the output lie within the
    derived bound of the oracle's exact block sums."""
    w = S.DenseWorkload("dense_sweep", M, K, N, xd, seed)
    print(f"[dense sweep] M={M} N={N} K={K} layout={layout} x={xd}", flush=True)
    wq_h, ws_h = S.dense_weights(w)
    wq, wsc = to_dev(wq_h), to_dev(ws_h)
    if layout == B.MOE_LAYOUT_PREPACKED:
        cb, sb = B.moe_dense_fp8_prepacked_size(N, K)
        pq = torch.empty(cb, dtype=torch.uint8, device="cuda")
        ps = torch.empty(sb, dtype=torch.uint8, device="cuda")
        B.moe_dense_fp8_prepack(N, K, wq, wsc, pq, ps)
        wq, wsc = pq, ps
    x = S.dense_activations(w)
    cfg = B.make_dense_config(M, N, K, xd, layout)
    work = torch.empty(max(B.moe_dense_fp8_workspace_size(cfg), 1), dtype=torch.uint8, device="cuda")
    y = torch.empty((M, N), dtype=torch.float32, device="cuda")
    B.moe_dense_fp8_forward(cfg, to_dev(x), wq, wsc, y, work)
    torch.cuda.synchronize()
    xq, xs = oracle.quant_mxfp8(x_f32(x))
    check_bound(y.cpu().numpy(), *oracle_with_bound(xq, xs, wq_h, ws_h), K, f"sweep M{M} N{N} K{K}")
