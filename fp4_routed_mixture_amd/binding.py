"""Thin Python binding of the C ABI in include/fp4moe.h.

Argument marshalling only: every function forwards torch tensors' device
pointers, sizes and the current HIP stream to the function of the same name
in libfp4moe.so, and raises MoEError on a non-zero status. Nothing here
computes any part of the layer, and there is no fallback: if the HIP library
is missing, every call raises.
"""
from __future__ import annotations

import ctypes as C
import os

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libfp4moe.so")

MOE_OK = 0
MOE_X_F32, MOE_X_BF16 = 0, 1
MOE_ACT_INT8, MOE_ACT_MXFP4 = 0, 1
MOE_W13, MOE_W2 = 0, 1
MOE_LAYOUT_CANONICAL, MOE_LAYOUT_PREPACKED = 0, 1
MOE_BLOCK_M_INT8, MOE_BLOCK_M_MXFP4 = 16, 64
STAGES = ["router", "topk", "quant_x", "sort", "gate_up", "requant", "down", "combine"]

# every function that include/fp4moe.h declares
EXPORTS = ["moe_abi_version", "moe_status_string", "moe_last_hip_error", "moe_workspace_size",
           "moe_prepacked_size", "moe_prepack", "moe_unpack", "moe_route", "moe_router_logits", "moe_sort",
           "moe_quantize",
           "moe_forward", "moe_forward_taps", "moe_forward_routed", "moe_rmsnorm", "moe_residual_add",
           "moe_stack_workspace_size", "moe_forward_stack", "moe_forward_stack_taps", "moe_forward_noalloc",
           "moe_dense_fp8_workspace_size", "moe_dense_fp8_quantize", "moe_dense_fp8_gemm", "moe_dense_fp8_forward",
           "moe_dense_fp8_prepacked_size", "moe_dense_fp8_prepack", "moe_dense_fp8_unpack"]
MOE_NOALLOC_SCRATCH_BYTES = 64 << 20


class MoEError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        msg = f"{where}: {status_string(status)} (status {status})"
        if status == 6:
            msg += f", hip error {moe_last_hip_error()}"
        super().__init__(msg)


class moe_config(C.Structure):
    _fields_ = [(n, C.c_int32) for n in ("T", "H", "I", "E", "top_k", "x_dtype", "act_mode", "block_m",
                                         "weight_layout")]

    def __repr__(self):
        return "moe_config(" + ", ".join(f"{n}={getattr(self, n)}" for n, _ in self._fields_) + ")"


class moe_dense_config(C.Structure):
    _fields_ = [(n, C.c_int32) for n in ("M", "N", "K", "x_dtype", "weight_layout")]

    def __repr__(self):
        return "moe_dense_config(" + ", ".join(f"{n}={getattr(self, n)}" for n, _ in self._fields_) + ")"


class moe_taps(C.Structure):
    _fields_ = [("xq", C.c_void_p), ("xs", C.c_void_p), ("aq", C.c_void_p), ("as_", C.c_void_p),
                ("y", C.c_void_p), ("counts", C.c_void_p), ("offsets", C.c_void_p),
                ("sorted_pairs", C.c_void_p), ("pair_pos", C.c_void_p), ("block_m", C.c_void_p),
                ("events", C.c_void_p)]


_lib = None


def lib():
    """Load libfp4moe.so; raise if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -c 'import __graft_entry__ as g; g.build()'` (hipcc, gfx950)")
        L = C.CDLL(LIB_PATH)
        vp, i32, i64, sz = C.c_void_p, C.c_int32, C.c_int64, C.c_size_t
        cfgp = C.POINTER(moe_config)
        dcfgp = C.POINTER(moe_dense_config)
        sig = {
            "moe_abi_version": (C.c_int, []),
            "moe_status_string": (C.c_char_p, [C.c_int]),
            "moe_last_hip_error": (C.c_int, []),
            "moe_workspace_size": (C.c_int, [cfgp, C.POINTER(sz)]),
            "moe_prepacked_size": (C.c_int, [i32, i32, i32, i32, C.POINTER(sz), C.POINTER(sz)]),
            "moe_prepack": (C.c_int, [i32, i32, i32, i32, vp, vp, vp, vp, vp, vp]),
            "moe_unpack": (C.c_int, [i32, i32, i32, i32, vp, vp, vp, vp, vp]),
            "moe_route": (C.c_int, [cfgp, vp, vp, vp, vp, vp, vp, sz, vp]),
            "moe_router_logits": (C.c_int, [cfgp, vp, vp, vp, vp, vp, sz, vp]),
            "moe_sort": (C.c_int, [cfgp, i32, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]),
            "moe_quantize": (C.c_int, [cfgp, i32, i32, i32, vp, vp, vp, vp]),
            "moe_forward": (C.c_int, [cfgp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]),
            "moe_forward_taps": (C.c_int, [cfgp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp,
                                           C.POINTER(moe_taps), vp, sz, vp]),
            "moe_forward_routed": (C.c_int, [cfgp, vp, vp, vp, vp, vp, vp, vp, vp, C.POINTER(moe_taps), vp, sz,
                                             vp]),
            "moe_rmsnorm": (C.c_int, [i32, i32, vp, vp, vp]),
            "moe_residual_add": (C.c_int, [i64, vp, vp, vp]),
            "moe_stack_workspace_size": (C.c_int, [cfgp, C.POINTER(sz)]),
            "moe_forward_stack": (C.c_int, [cfgp, i32, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]),
            "moe_forward_stack_taps": (C.c_int, [cfgp, i32, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]),
            "moe_forward_noalloc": (C.c_int, [cfgp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp]),
            "moe_dense_fp8_workspace_size": (C.c_int, [dcfgp, C.POINTER(sz)]),
            "moe_dense_fp8_quantize": (C.c_int, [i32, i32, i32, vp, vp, vp, vp]),
            "moe_dense_fp8_gemm": (C.c_int, [dcfgp, vp, vp, vp, vp, vp, vp, sz, vp]),
            "moe_dense_fp8_forward": (C.c_int, [dcfgp, vp, vp, vp, vp, vp, sz, vp]),
            "moe_dense_fp8_prepacked_size": (C.c_int, [i32, i32, C.POINTER(sz), C.POINTER(sz)]),
            "moe_dense_fp8_prepack": (C.c_int, [i32, i32, vp, vp, vp, vp, vp]),
            "moe_dense_fp8_unpack": (C.c_int, [i32, i32, vp, vp, vp, vp, vp]),
        }
        for name, (res, args) in sig.items():
            f = getattr(L, name)
            f.restype = res
            f.argtypes = args
        _lib = L
    return _lib


def _p(t):
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _s(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream


def _check(status: int, where: str):
    if status != MOE_OK:
        raise MoEError(status, where)


def status_string(status: int) -> str:
    return lib().moe_status_string(status).decode()


def make_config(T, H, I, E, top_k, x_dtype=MOE_X_BF16, act_mode=MOE_ACT_INT8, weight_layout=MOE_LAYOUT_CANONICAL,
                block_m=0) -> moe_config:
    return moe_config(T, H, I, E, top_k, x_dtype, act_mode, block_m, weight_layout)


# ------------------------------------------------------------------ C ABI --
def moe_abi_version() -> int:
    return lib().moe_abi_version()


def moe_status_string(status: int) -> str:
    return status_string(status)


def moe_last_hip_error() -> int:
    return lib().moe_last_hip_error()


def moe_workspace_size(cfg: moe_config) -> int:
    n = C.c_size_t(0)
    _check(lib().moe_workspace_size(C.byref(cfg), C.byref(n)), "moe_workspace_size")
    return n.value


def moe_prepacked_size(which: int, E: int, N: int, K: int):
    cb, sb = C.c_size_t(0), C.c_size_t(0)
    _check(lib().moe_prepacked_size(which, E, N, K, C.byref(cb), C.byref(sb)), "moe_prepacked_size")
    return cb.value, sb.value


def moe_prepack(which, E, N, K, codes, scales, row_perm, packed_codes, packed_scales, stream=None):
    _check(lib().moe_prepack(which, E, N, K, _p(codes), _p(scales), _p(row_perm), _p(packed_codes),
                             _p(packed_scales), _s(stream)), "moe_prepack")


def moe_unpack(which, E, N, K, packed_codes, packed_scales, codes, scales, stream=None):
    _check(lib().moe_unpack(which, E, N, K, _p(packed_codes), _p(packed_scales), _p(codes), _p(scales),
                            _s(stream)), "moe_unpack")


def moe_route(cfg, x, router_w, router_bias, topk_ids, topk_w, workspace, stream=None):
    _check(lib().moe_route(C.byref(cfg), _p(x), _p(router_w), _p(router_bias), _p(topk_ids), _p(topk_w),
                           _p(workspace), workspace.numel() if workspace is not None else 0, _s(stream)),
           "moe_route")


def moe_router_logits(cfg, x, router_w, router_bias, logits, workspace, stream=None):
    """Router logits fp32 [T][E] (before the sigmoid) into the device tensor logits."""
    _check(lib().moe_router_logits(C.byref(cfg), _p(x), _p(router_w), _p(router_bias), _p(logits), _p(workspace),
                                   workspace.numel() if workspace is not None else 0, _s(stream)),
           "moe_router_logits")


def moe_sort(cfg, block_m, topk_ids, counts, offsets, sorted_pairs, pair_pos, tile_expert, n_tiles,
             workspace=None, stream=None):
    _check(lib().moe_sort(C.byref(cfg), block_m, _p(topk_ids), _p(counts), _p(offsets), _p(sorted_pairs),
                          _p(pair_pos), _p(tile_expert), _p(n_tiles), _p(workspace),
                          workspace.numel() if workspace is not None else 0, _s(stream)), "moe_sort")


def moe_quantize(cfg, rows, K, in_dtype, v, q, scales, stream=None):
    _check(lib().moe_quantize(C.byref(cfg), rows, K, in_dtype, _p(v), _p(q), _p(scales), _s(stream)),
           "moe_quantize")


def moe_forward(cfg, x, router_w, router_bias, w13, w13_scale, w2, w2_scale, out, topk_ids_out, topk_w_out,
                workspace, stream=None):
    _check(lib().moe_forward(C.byref(cfg), _p(x), _p(router_w), _p(router_bias), _p(w13), _p(w13_scale), _p(w2),
                             _p(w2_scale), _p(out), _p(topk_ids_out), _p(topk_w_out), _p(workspace),
                             workspace.numel(), _s(stream)), "moe_forward")


def moe_forward_noalloc(cfg, x, router_w, router_bias, w13, w13_scale, w2, w2_scale, out, topk_ids_out, topk_w_out,
                        stream=None):
    """moe_forward without a workspace: the library's fixed per-device
    scratch array (MOE_NOALLOC_SCRATCH_BYTES) is used instead."""
    _check(lib().moe_forward_noalloc(C.byref(cfg), _p(x), _p(router_w), _p(router_bias), _p(w13), _p(w13_scale),
                                     _p(w2), _p(w2_scale), _p(out), _p(topk_ids_out), _p(topk_w_out), _s(stream)),
           "moe_forward_noalloc")


def moe_forward_taps(cfg, x, router_w, router_bias, w13, w13_scale, w2, w2_scale, out, topk_ids_out, topk_w_out,
                     taps: dict, workspace, stream=None):
    """taps: dict with any of xq, xs, aq, as, y, counts, offsets, sorted_pairs,
    pair_pos (device tensors) and events (a ctypes array of 2*len(STAGES)
    hipEvent_t handles). Returns the block size the kernels used."""
    bm = C.c_int32(0)
    ev = taps.get("events")
    t = moe_taps(*(_p(taps.get(n)) for n in ("xq", "xs", "aq", "as", "y", "counts", "offsets",
                                              "sorted_pairs", "pair_pos")),
                 C.cast(C.pointer(bm), C.c_void_p), None if ev is None else C.cast(ev, C.c_void_p))
    _check(lib().moe_forward_taps(C.byref(cfg), _p(x), _p(router_w), _p(router_bias), _p(w13), _p(w13_scale),
                                  _p(w2), _p(w2_scale), _p(out), _p(topk_ids_out), _p(topk_w_out), C.byref(t),
                                  _p(workspace), workspace.numel(), _s(stream)), "moe_forward_taps")
    return bm.value


def moe_forward_routed(cfg, x, topk_ids, topk_w, w13, w13_scale, w2, w2_scale, out, workspace, taps=None,
                       stream=None):
    """The layer without its router: routing given as topk_ids [T][k] int32
    (in [0, E)) and topk_w [T][k] fp32 device tensors. taps as in
    moe_forward_taps (returns the block size the kernels used)."""
    bm = C.c_int32(0)
    tp = None
    if taps is not None:
        ev = taps.get("events")
        tp = moe_taps(*(_p(taps.get(n)) for n in ("xq", "xs", "aq", "as", "y", "counts", "offsets",
                                                   "sorted_pairs", "pair_pos")),
                      C.cast(C.pointer(bm), C.c_void_p), None if ev is None else C.cast(ev, C.c_void_p))
    _check(lib().moe_forward_routed(C.byref(cfg), _p(x), _p(topk_ids), _p(topk_w), _p(w13), _p(w13_scale), _p(w2),
                                    _p(w2_scale), _p(out), None if tp is None else C.byref(tp), _p(workspace),
                                    workspace.numel(), _s(stream)), "moe_forward_routed")
    return bm.value


def moe_rmsnorm(T, H, x, out, stream=None):
    _check(lib().moe_rmsnorm(T, H, _p(x), _p(out), _s(stream)), "moe_rmsnorm")


def moe_residual_add(n, x, y, stream=None):
    _check(lib().moe_residual_add(n, _p(x), _p(y), _s(stream)), "moe_residual_add")


def moe_stack_workspace_size(cfg) -> int:
    n = C.c_size_t(0)
    _check(lib().moe_stack_workspace_size(C.byref(cfg), C.byref(n)), "moe_stack_workspace_size")
    return n.value


def moe_forward_stack(cfg, x, layers, workspace, layer_out=None, stream=None):
    """layers: sequence of dicts with router_w, bias (or None), w13, w13s, w2,
    w2s device tensors (prepacked weights). x (fp32 [T][H]) is updated in
    place; layer_out (fp32 [L][T][H] or None) receives each layer's output."""
    L = len(layers)
    arr = lambda key: (C.c_void_p * max(L, 1))(*[_p(d[key]) for d in layers])
    keep = [arr(k) for k in ("router_w", "bias", "w13", "w13s", "w2", "w2s")]
    _check(lib().moe_forward_stack(C.byref(cfg), L, _p(x), *[C.cast(a, C.c_void_p) for a in keep], _p(layer_out),
                                   _p(workspace), workspace.numel(), _s(stream)), "moe_forward_stack")


def moe_forward_stack_taps(cfg, x, layers, workspace, layer_taps, layer_out=None, stream=None):
    """moe_forward_stack with per-layer taps: layer_taps is a sequence of L
    dicts (or None) as for moe_forward_taps; returns the block size used."""
    L = len(layers)
    arr = lambda key: (C.c_void_p * max(L, 1))(*[_p(d[key]) for d in layers])
    keep = [arr(k) for k in ("router_w", "bias", "w13", "w13s", "w2", "w2s")]
    bm = C.c_int32(0)
    tps = (moe_taps * max(L, 1))()
    for l, t in enumerate(layer_taps):
        if t is None:
            continue
        ev = t.get("events")
        tps[l] = moe_taps(*(_p(t.get(n)) for n in ("xq", "xs", "aq", "as", "y", "counts", "offsets",
                                                   "sorted_pairs", "pair_pos")),
                          C.cast(C.pointer(bm), C.c_void_p), None if ev is None else C.cast(ev, C.c_void_p))
    _check(lib().moe_forward_stack_taps(C.byref(cfg), L, _p(x), *[C.cast(a, C.c_void_p) for a in keep],
                                        _p(layer_out), C.cast(tps, C.c_void_p), _p(workspace), workspace.numel(),
                                        _s(stream)), "moe_forward_stack_taps")
    return bm.value


# ------------------------------------------------------------- dense FP8 --
def make_dense_config(M, N, K, x_dtype=MOE_X_BF16, weight_layout=MOE_LAYOUT_CANONICAL) -> moe_dense_config:
    return moe_dense_config(M, N, K, x_dtype, weight_layout)


def moe_dense_fp8_prepacked_size(N, K):
    cb, sb = C.c_size_t(0), C.c_size_t(0)
    _check(lib().moe_dense_fp8_prepacked_size(N, K, C.byref(cb), C.byref(sb)), "moe_dense_fp8_prepacked_size")
    return cb.value, sb.value


def moe_dense_fp8_prepack(N, K, w, w_scale, packed_w, packed_scale, stream=None):
    _check(lib().moe_dense_fp8_prepack(N, K, _p(w), _p(w_scale), _p(packed_w), _p(packed_scale), _s(stream)),
           "moe_dense_fp8_prepack")


def moe_dense_fp8_unpack(N, K, packed_w, packed_scale, w, w_scale, stream=None):
    _check(lib().moe_dense_fp8_unpack(N, K, _p(packed_w), _p(packed_scale), _p(w), _p(w_scale), _s(stream)),
           "moe_dense_fp8_unpack")


def moe_dense_fp8_workspace_size(cfg) -> int:
    n = C.c_size_t(0)
    _check(lib().moe_dense_fp8_workspace_size(C.byref(cfg), C.byref(n)), "moe_dense_fp8_workspace_size")
    return n.value


def moe_dense_fp8_quantize(rows, K, in_dtype, v, codes, scales, stream=None):
    _check(lib().moe_dense_fp8_quantize(rows, K, in_dtype, _p(v), _p(codes), _p(scales), _s(stream)),
           "moe_dense_fp8_quantize")


def moe_dense_fp8_gemm(cfg, xq, xs, w, w_scale, y, workspace=None, stream=None):
    nbytes = 0 if workspace is None else workspace.numel()
    _check(lib().moe_dense_fp8_gemm(C.byref(cfg), _p(xq), _p(xs), _p(w), _p(w_scale), _p(y), _p(workspace),
                                    nbytes, _s(stream)), "moe_dense_fp8_gemm")


def moe_dense_fp8_forward(cfg, x, w, w_scale, y, workspace, stream=None):
    _check(lib().moe_dense_fp8_forward(C.byref(cfg), _p(x), _p(w), _p(w_scale), _p(y), _p(workspace),
                                       workspace.numel(), _s(stream)), "moe_dense_fp8_forward")
