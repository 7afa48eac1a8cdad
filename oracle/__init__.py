"""CPU oracle for the FP4 routed-MoE layer (ctypes wrapper over oracle.c).

TEST INFRASTRUCTURE ONLY: the test suite, the smoke check and the benchmark's
CPU-baseline leg may import this package; the library under
``fp4_routed_mixture_amd`` never does. It shares no code with the HIP path.

Pinned functions (each checked by ``tests/test_oracle_*.py`` against
something other than itself):
  e2m1_table, e8m0          exhaustive table from the OCP MX v1.0 format
  expf, sigmoidf            float64 math within 2 ulp; special values
  router_logits             float64 dot product within the fp32 error bound
  topk                      brute-force full sort of the scores
  sort                      Python sorted(); permutation invariants
  quant_int8, quant_mxfp4   brute-force nearest-grid search; constructed ties
  moe_layer                 E=1, k=1 equals a dense float64 MLP on the
                            dequantized weights; one-hot closed forms;
                            scale-exponent doubling; permutation
                            equivariance; identical experts; zero weights
  rmsnorm                   float64 RMS within its error bound
  e4m3_table, quant_mxfp8   torch's independent float8_e4m3fn conversion
                            (decode of all codes, nearest-even rounding in
                            range); brute-force grid search; saturation
  dense_mxfp8               numpy float64 matmul of the dequantized operands;
                            one-hot closed forms; scale-exponent doubling
"""
from __future__ import annotations

import ctypes as C
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

GCC_FLAGS = ["-O3", "-mavx2", "-fopenmp", "-ffp-contract=off", "-fno-fast-math", "-shared", "-fPIC"]


def build(force: bool = False) -> str:
    """Compile oracle.c with gcc (no GPU code involved)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", *GCC_FLAGS, _SRC, "-o", tmp, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


_lib = None


def lib():
    global _lib
    if _lib is None:
        _lib = C.CDLL(build())
        f32p = np.ctypeslib.ndpointer(np.float32, flags="C_CONTIGUOUS")
        i32p = np.ctypeslib.ndpointer(np.int32, flags="C_CONTIGUOUS")
        u8p = np.ctypeslib.ndpointer(np.uint8, flags="C_CONTIGUOUS")
        i8p = np.ctypeslib.ndpointer(np.int8, flags="C_CONTIGUOUS")
        L = _lib
        L.or_e2m1_value.restype = C.c_float
        L.or_e2m1_value.argtypes = [C.c_int]
        L.or_e8m0_value.restype = C.c_float
        L.or_e8m0_value.argtypes = [C.c_int]
        L.or_expf.restype = C.c_float
        L.or_expf.argtypes = [C.c_float]
        L.or_expf_n.argtypes = [C.c_int, f32p, f32p]
        L.or_sigmoidf_n.argtypes = [C.c_int, f32p, f32p]
        L.or_e2m1_table.argtypes = [f32p]
        L.or_x_to_f32.argtypes = [C.c_int, C.c_int, C.c_int, C.c_void_p, f32p]
        L.or_router_logits.argtypes = [C.c_int, C.c_int, C.c_int, f32p, f32p, C.c_void_p, f32p]
        L.or_topk.argtypes = [C.c_int, C.c_int, C.c_int, f32p, i32p, f32p, C.c_void_p]
        L.or_sort.restype = C.c_int
        L.or_sort.argtypes = [C.c_int, C.c_int, C.c_int, i32p, i32p, i32p, i32p, i32p, i32p, i32p]
        L.or_quant_int8.argtypes = [C.c_int, C.c_int, f32p, i8p, f32p]
        L.or_quant_mxfp4.argtypes = [C.c_int, C.c_int, f32p, u8p, u8p]
        L.or_gemm_row_int8.argtypes = [C.c_int, C.c_int, i8p, C.c_float, u8p, u8p, f32p]
        L.or_gemm_row_mxfp4.argtypes = [C.c_int, C.c_int, u8p, u8p, u8p, u8p, f32p]
        L.or_silu_mul.argtypes = [C.c_int, f32p, f32p]
        L.or_moe_layer.restype = C.c_int
        L.or_moe_layer.argtypes = [C.c_void_p, C.c_void_p, f32p, C.c_void_p,
                                   C.c_void_p, C.c_void_p, C.c_void_p, C.c_void_p,
                                   f32p, i32p, f32p,
                                   C.c_void_p, C.c_void_p, C.c_void_p, C.c_void_p, C.c_void_p, C.c_void_p]
        L.or_moe_layer_routed.restype = C.c_int
        L.or_moe_layer_routed.argtypes = [C.c_void_p, C.c_void_p, i32p, f32p,
                                          C.c_void_p, C.c_void_p, C.c_void_p, C.c_void_p, f32p,
                                          C.c_void_p, C.c_void_p, C.c_void_p, C.c_void_p, C.c_void_p, C.c_void_p]
        L.or_rmsnorm.argtypes = [C.c_int, C.c_int, f32p, f32p]
        L.or_e4m3_value.restype = C.c_float
        L.or_e4m3_value.argtypes = [C.c_int]
        L.or_quant_mxfp8.argtypes = [C.c_int, C.c_int, f32p, u8p, u8p]
        f64p = np.ctypeslib.ndpointer(np.float64, flags="C_CONTIGUOUS")
        L.or_dense_mxfp8.argtypes = [C.c_int, C.c_int, C.c_int, u8p, u8p, u8p, u8p, f32p, C.c_void_p]
        L.or_num_threads.restype = C.c_int
        L.or_set_num_threads.argtypes = [C.c_int]
    return _lib


class _Cfg(C.Structure):
    _fields_ = [(n, C.c_int32) for n in ("T", "H", "I", "E", "top_k", "x_dtype", "act_mode")]


def _f32(a):
    return np.ascontiguousarray(a, dtype=np.float32)


def _ptr(a):
    return None if a is None else a.ctypes.data_as(C.c_void_p)


# ---------------------------------------------------------------- formats --
def e2m1_table() -> np.ndarray:
    out = np.zeros(16, np.float32)
    lib().or_e2m1_table(out)
    return out


def e8m0(b: int) -> float:
    return lib().or_e8m0_value(int(b))


# ------------------------------------------------------------ exp/sigmoid --
def expf(z) -> np.ndarray:
    z = _f32(np.atleast_1d(z))
    out = np.empty_like(z)
    lib().or_expf_n(z.size, z.ravel(), out.ravel())
    return out


def sigmoidf(z) -> np.ndarray:
    z = _f32(np.atleast_1d(z))
    out = np.empty_like(z)
    lib().or_sigmoidf_n(z.size, z.ravel(), out.ravel())
    return out


# ----------------------------------------------------------------- router --
def x_to_f32(x: np.ndarray) -> np.ndarray:
    """fp32 array passes through; uint16 is read as bf16 bit patterns."""
    x = np.ascontiguousarray(x)
    T, H = x.shape
    out = np.empty((T, H), np.float32)
    lib().or_x_to_f32(T, H, 1 if x.dtype == np.uint16 else 0, x.ctypes.data_as(C.c_void_p), out)
    return out


def router_logits(x, wr, bias=None) -> np.ndarray:
    xf = x_to_f32(x)
    wr = _f32(wr)
    T, H = xf.shape
    E = wr.shape[0]
    assert H % 64 == 0
    b = None if bias is None else _f32(bias)
    out = np.empty((T, E), np.float32)
    lib().or_router_logits(T, H, E, xf, wr, _ptr(b), out)
    return out


def topk(logits, k: int, return_scores: bool = False):
    logits = _f32(logits)
    T, E = logits.shape
    ids = np.empty((T, k), np.int32)
    w = np.empty((T, k), np.float32)
    sc = np.empty((T, E), np.float32) if return_scores else None
    lib().or_topk(T, E, k, logits, ids, w, _ptr(sc))
    return (ids, w, sc) if return_scores else (ids, w)


def route(x, wr, bias, k: int):
    return topk(router_logits(x, wr, bias), k)


# ------------------------------------------------------------------- sort --
def sort(ids, E: int, block_m: int) -> dict:
    ids = np.ascontiguousarray(ids, dtype=np.int32).ravel()
    P = ids.size
    cap = P + min(E, max(P, 1)) * (block_m - 1) + 1
    counts = np.empty(E, np.int32)
    offsets = np.empty(E + 1, np.int32)
    sorted_ = np.empty(cap, np.int32)
    pos = np.empty(max(P, 1), np.int32)
    tiles = np.empty(cap // block_m + E + 1, np.int32)
    nt = np.zeros(1, np.int32)
    total = lib().or_sort(P, E, block_m, ids, counts, offsets, sorted_, pos, tiles, nt)
    return {"counts": counts, "offsets": offsets, "sorted": sorted_[:total], "pos": pos[:P],
            "tile_expert": tiles[:nt[0]], "n_tiles": int(nt[0]), "total": total}


# ---------------------------------------------------------------- quant ----
def quant_int8(v):
    v = _f32(v)
    R, K = v.shape
    q = np.empty((R, K), np.int8)
    s = np.empty(R, np.float32)
    lib().or_quant_int8(R, K, v, q, s)
    return q, s


def quant_mxfp4(v):
    v = _f32(v)
    R, K = v.shape
    assert K % 32 == 0
    codes = np.empty((R, K // 2), np.uint8)
    scales = np.empty((R, K // 32), np.uint8)
    lib().or_quant_mxfp4(R, K, v, codes, scales)
    return codes, scales


# ------------------------------------------------------------------ gemm ---
def gemm_row_int8(q_row, s: float, wc, ws):
    wc = np.ascontiguousarray(wc, np.uint8)
    ws = np.ascontiguousarray(ws, np.uint8)
    N, K2 = wc.shape
    out = np.empty(N, np.float32)
    lib().or_gemm_row_int8(2 * K2, N, np.ascontiguousarray(q_row, np.int8), float(s), wc, ws, out)
    return out


def gemm_row_mxfp4(xc_row, xs_row, wc, ws):
    wc = np.ascontiguousarray(wc, np.uint8)
    ws = np.ascontiguousarray(ws, np.uint8)
    N, K2 = wc.shape
    out = np.empty(N, np.float32)
    lib().or_gemm_row_mxfp4(2 * K2, N, np.ascontiguousarray(xc_row, np.uint8),
                            np.ascontiguousarray(xs_row, np.uint8), wc, ws, out)
    return out


def silu_mul(h):
    h = _f32(h)
    I = h.size // 2
    a = np.empty(I, np.float32)
    lib().or_silu_mul(I, h, a)
    return a


# ------------------------------------------------------------------ layer --
def _expert_pointers(experts, E):
    """(ptr arrays, kept arrays, I) for the per-expert canonical weights."""
    I = None
    arrs = [[], [], [], []]
    keep = []
    for e in range(E):
        ex = experts[e]
        if ex is None:
            for a in arrs:
                a.append(None)
            continue
        ex = [np.ascontiguousarray(a, np.uint8) for a in ex]
        keep.append(ex)
        I = ex[0].shape[0] // 2
        for a, v in zip(arrs, ex):
            a.append(v.ctypes.data_as(C.c_void_p).value)
    assert I is not None
    return [(C.c_void_p * E)(*a) for a in arrs], keep, I


def _intermediates(T, H, I, P, act_mode):
    mx = act_mode == 1
    return {
        "xq": np.empty((T, H // 2), np.uint8) if mx else np.empty((T, H), np.int8),
        "xs": np.empty((T, H // 32), np.uint8) if mx else np.empty(T, np.float32),
        "h": np.empty((P, 2 * I), np.float32),
        "aq": np.empty((P, I // 2), np.uint8) if mx else np.empty((P, I), np.int8),
        "as": np.empty((P, I // 32), np.uint8) if mx else np.empty(P, np.float32),
        "y": np.empty((P, H), np.float32),
    }


def _x_rows(x):
    x = np.ascontiguousarray(x)
    x_dtype = 1 if x.dtype == np.uint16 else 0
    return (x if x_dtype else _f32(x)), x_dtype


def moe_layer(x, wr, bias, experts, top_k: int, act_mode: int, intermediates: bool = False) -> dict:
    """The whole layer for the tokens in x.

    experts: a sequence of length E whose entry e is None or a tuple
    (w13 [2I,H/2], w13_scale [2I,H/32], w2 [H,I/2], w2_scale [H,I/32]) of
    canonical uint8 arrays. act_mode 0 = int8 rows, 1 = MXFP4.
    """
    x, x_dtype = _x_rows(x)
    T, H = x.shape
    wr = _f32(wr)
    E = wr.shape[0]
    ptr_arrays, keep, I = _expert_pointers(experts, E)
    cfg = _Cfg(T, H, I, E, top_k, x_dtype, act_mode)
    P = T * top_k
    out = np.empty((T, H), np.float32)
    ids = np.empty((T, top_k), np.int32)
    w = np.empty((T, top_k), np.float32)
    inter = _intermediates(T, H, I, P, act_mode) if intermediates else {}
    b = None if bias is None else _f32(bias)
    rc = lib().or_moe_layer(C.byref(cfg), x.ctypes.data_as(C.c_void_p), wr, _ptr(b),
                            *[C.cast(p, C.c_void_p) for p in ptr_arrays], out, ids, w,
                            *[_ptr(inter.get(n)) for n in ("xq", "xs", "h", "aq", "as", "y")])
    if rc != 0:
        raise ValueError("oracle: a routed expert has no weights")
    del keep
    res = {"out": out, "ids": ids, "w": w}
    res.update(inter)
    return res


def moe_layer_routed(x, ids, w, experts, act_mode: int, intermediates: bool = False) -> dict:
    """The layer's expert part for routing given by the caller: ids [T][k]
    (int32 in [0, E), E = len(experts)) and weights [T][k] (fp32); the same
    steps after the routing as moe_layer."""
    x, x_dtype = _x_rows(x)
    T, H = x.shape
    ids = np.ascontiguousarray(ids, np.int32)
    w = _f32(w)
    k = ids.shape[1]
    E = len(experts)
    ptr_arrays, keep, I = _expert_pointers(experts, E)
    cfg = _Cfg(T, H, I, E, k, x_dtype, act_mode)
    out = np.empty((T, H), np.float32)
    inter = _intermediates(T, H, I, T * k, act_mode) if intermediates else {}
    rc = lib().or_moe_layer_routed(C.byref(cfg), x.ctypes.data_as(C.c_void_p), ids, w,
                                   *[C.cast(p, C.c_void_p) for p in ptr_arrays], out,
                                   *[_ptr(inter.get(n)) for n in ("xq", "xs", "h", "aq", "as", "y")])
    if rc != 0:
        raise ValueError("oracle: an id is out of range or its expert has no weights")
    del keep
    res = {"out": out}
    res.update(inter)
    return res


# ------------------------------------------------------------ dense FP8 ---
def e4m3_table() -> np.ndarray:
    return np.array([lib().or_e4m3_value(c) for c in range(256)], np.float32)


def quant_mxfp8(v):
    """MXFP8 quantization per 32 along K: (codes [R][K] u8, E8M0 [R][K/32] u8)."""
    v = _f32(v)
    R, K = v.shape
    assert K % 32 == 0
    codes = np.empty((R, K), np.uint8)
    scales = np.empty((R, K // 32), np.uint8)
    lib().or_quant_mxfp8(R, K, v, codes, scales)
    return codes, scales


def dense_mxfp8(xq, xs, wq, ws, bound: bool = False):
    """Y = X W^T for MXFP8 X [M][K] and W [N][K] (exact block sums, float64
    accumulation, one rounding to fp32); with bound, also the float64
    sum of |products| times scales (the fp32 error budget's base)."""
    xq, xs = np.ascontiguousarray(xq, np.uint8), np.ascontiguousarray(xs, np.uint8)
    wq, ws = np.ascontiguousarray(wq, np.uint8), np.ascontiguousarray(ws, np.uint8)
    M, K = xq.shape
    N = wq.shape[0]
    out = np.empty((M, N), np.float32)
    ab = np.empty((M, N), np.float64) if bound else None
    lib().or_dense_mxfp8(M, N, K, xq, xs, wq, ws, out, _ptr(ab))
    return (out, ab) if bound else out


def dense_fp8(x, wq, ws, bound: bool = False):
    """The projection of x (fp32, or bf16 bit patterns): MXFP8 quantization of
    x per token, then dense_mxfp8."""
    xq, xs = quant_mxfp8(x_to_f32(x))
    return dense_mxfp8(xq, xs, wq, ws, bound)


def rmsnorm(x):
    x = _f32(x)
    T, H = x.shape
    out = np.empty_like(x)
    lib().or_rmsnorm(T, H, x, out)
    return out


def num_threads() -> int:
    return lib().or_num_threads()


def set_num_threads(n: int) -> None:
    lib().or_set_num_threads(int(n))
