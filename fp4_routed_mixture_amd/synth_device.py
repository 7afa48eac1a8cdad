"""Seeded synthetic inputs placed in device memory.

The same numbers as ``synth`` (which the CPU oracle reads), generated where
they are needed: packed codes and scales by the SplitMix64 kernel of
libfp4moe_synth.so, Gaussians by numpy on the host and copied over. Holds none
of the layer's arithmetic. ``load_layer`` also runs the library's load-time
prepack (``moe_prepack``), which is how a user of the library would load
weights.
"""
from __future__ import annotations

import ctypes as C
import os

import numpy as np
import torch

from . import binding as B
from . import synth as S

SYNTH_LIB = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libfp4moe_synth.so")
_slib = None


def slib():
    global _slib
    if _slib is None:
        if not os.path.exists(SYNTH_LIB):
            raise RuntimeError(f"{SYNTH_LIB} is missing: build the HIP libraries first")
        L = C.CDLL(SYNTH_LIB)
        L.synth_fill.restype = C.c_int
        L.synth_fill.argtypes = [C.c_int, C.c_int, C.c_int, C.c_uint64, C.c_uint64, C.c_int, C.c_void_p, C.c_void_p]
        L.synth_stream_key.restype = C.c_uint64
        L.synth_stream_key.argtypes = [C.c_int, C.c_int, C.c_int]
        L.synth_exp_sigmoid.restype = C.c_int
        L.synth_exp_sigmoid.argtypes = [C.c_void_p, C.c_int, C.c_void_p, C.c_void_p, C.c_void_p]
        L.synth_mfma_probe.restype = C.c_int
        L.synth_mfma_probe.argtypes = [C.c_int, C.c_int, C.c_void_p, C.c_void_p, C.c_void_p]
        L.synth_mfma_probe_fmt.restype = C.c_int
        L.synth_mfma_probe_fmt.argtypes = [C.c_int, C.c_int, C.c_int, C.c_void_p, C.c_void_p, C.c_void_p]
        L.synth_stream_read.restype = C.c_int
        L.synth_stream_read.argtypes = [C.c_void_p, C.c_uint64, C.c_int, C.c_void_p, C.c_void_p]
        _slib = L
    return _slib


def fill(seed: int, layer: int, tensor: int, first_byte: int, out: torch.Tensor, scale_mode: bool) -> None:
    rc = slib().synth_fill(seed, layer, tensor, first_byte, out.numel() * out.element_size(), int(scale_mode),
                           out.data_ptr(), torch.cuda.current_stream().cuda_stream)
    if rc != 0:
        raise RuntimeError(f"synth_fill failed ({rc})")


def canonical_weights(w: S.Workload, layer: int = 0, device="cuda"):
    """All experts' canonical codes/scales on the device (uint8 tensors)."""
    H, I, E = w.H, w.I, w.E
    w13 = torch.empty((E, 2 * I, H // 2), dtype=torch.uint8, device=device)
    w13s = torch.empty((E, 2 * I, H // 32), dtype=torch.uint8, device=device)
    w2 = torch.empty((E, H, I // 2), dtype=torch.uint8, device=device)
    w2s = torch.empty((E, H, I // 32), dtype=torch.uint8, device=device)
    fill(w.seed, layer, S.TENSOR_W13_CODES, 0, w13, False)
    fill(w.seed, layer, S.TENSOR_W13_SCALES, 0, w13s, True)
    fill(w.seed, layer, S.TENSOR_W2_CODES, 0, w2, False)
    fill(w.seed, layer, S.TENSOR_W2_SCALES, 0, w2s, True)
    return w13, w13s, w2, w2s


def prepack(w: S.Workload, canon, row_perm13=None, row_perm2=None):
    """Prepacked copies of canonical (w13, w13s, w2, w2s)."""
    H, I, E = w.H, w.I, w.E
    w13, w13s, w2, w2s = canon
    dev = w13.device
    cb13, sb13 = B.moe_prepacked_size(B.MOE_W13, E, 2 * I, H)
    cb2, sb2 = B.moe_prepacked_size(B.MOE_W2, E, H, I)
    p13 = torch.empty(cb13, dtype=torch.uint8, device=dev)
    p13s = torch.empty(sb13, dtype=torch.uint8, device=dev)
    p2 = torch.empty(cb2, dtype=torch.uint8, device=dev)
    p2s = torch.empty(sb2, dtype=torch.uint8, device=dev)
    B.moe_prepack(B.MOE_W13, E, 2 * I, H, w13, w13s, row_perm13, p13, p13s)
    B.moe_prepack(B.MOE_W2, E, H, I, w2, w2s, row_perm2, p2, p2s)
    return p13, p13s, p2, p2s


def load_layer(w: S.Workload, layer: int = 0, device="cuda", keep_canonical: bool = False) -> dict:
    """Weights of one layer in the prepacked layout plus router weights/bias."""
    canon = canonical_weights(w, layer, device)
    packed = prepack(w, canon)
    out = {"w13": packed[0], "w13s": packed[1], "w2": packed[2], "w2s": packed[3],
           "router_w": torch.from_numpy(S.router_weights(w, layer)).to(device),
           "bias": None}
    b = S.router_bias(w, layer)
    if b is not None:
        out["bias"] = torch.from_numpy(b).to(device)
    if keep_canonical:
        out["canonical"] = canon
    else:
        del canon
    return out


def activations(w: S.Workload, layer: int = 0, device="cuda", T: int | None = None) -> torch.Tensor:
    x = S.activations(w, layer, T)
    if x.dtype == np.uint16:
        return torch.from_numpy(x.view(np.int16)).to(device).view(torch.bfloat16)
    return torch.from_numpy(x).to(device)


def config(w: S.Workload, T: int | None = None, weight_layout: int = B.MOE_LAYOUT_PREPACKED) -> B.moe_config:
    """The layer's configuration; weights as load_layer places them (prepacked)
    unless weight_layout says otherwise."""
    return B.make_config(w.T if T is None else T, w.H, w.I, w.E, w.top_k, w.x_dtype, w.act_mode, weight_layout)


def workspace(cfg: B.moe_config, device="cuda") -> torch.Tensor:
    n = B.moe_workspace_size(cfg)
    return torch.empty(max(n, 256), dtype=torch.uint8, device=device)


def stream_read(buf: torch.Tensor, blocks: int, sink: torch.Tensor) -> None:
    """Enqueue the streaming-read probe over buf (a benchmark ceiling, not
    part of the layer); sink holds blocks 16-byte words."""
    rc = slib().synth_stream_read(buf.data_ptr(), buf.numel() * buf.element_size(), blocks, sink.data_ptr(),
                                  torch.cuda.current_stream().cuda_stream)
    if rc != 0:
        raise RuntimeError(f"synth_stream_read failed ({rc})")


def mfma_probe(blocks: int, iters: int, out: torch.Tensor, clocks: torch.Tensor, fmt: str = "fp4") -> None:
    """Enqueue the MFMA rate probe (a benchmark ceiling, not part of the
    layer) on fmt "fp4" or "fp8" (scaled 32x32x64) or "fp32" (32x32x2)
    operands: out holds blocks * 256 floats, clocks blocks * 8 int64."""
    code = {"fp4": 0, "fp8": 1, "fp32": 2}[fmt]
    rc = slib().synth_mfma_probe_fmt(blocks, iters, code, out.data_ptr(), clocks.data_ptr(),
                                     torch.cuda.current_stream().cuda_stream)
    if rc != 0:
        raise RuntimeError(f"synth_mfma_probe failed ({rc})")


def exp_sigmoid(z: torch.Tensor):
    """The layer kernels' own fp32 exp and sigmoid of z (a test hook)."""
    e, s = torch.empty_like(z), torch.empty_like(z)
    rc = slib().synth_exp_sigmoid(z.data_ptr(), z.numel(), e.data_ptr(), s.data_ptr(),
                                  torch.cuda.current_stream().cuda_stream)
    if rc != 0:
        raise RuntimeError(f"synth_exp_sigmoid failed ({rc})")
    return e, s
