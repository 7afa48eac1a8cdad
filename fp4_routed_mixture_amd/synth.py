"""Seeded synthetic inputs for the routed-MoE layer.

This module only draws numbers. It holds none of the layer's arithmetic (no
routing, no quantization, no GEMM): both the HIP path and the CPU oracle take
their inputs from here, so it must stay free of either side's code.

Workloads (shapes from the DeepSeek-V4-Flash pages: 256 routed experts, 6 per
token and 43 layers on the gfx1201 deployment blog, section What we set out to
do; the 4,604-token prompt in the MI250 paper's abstract; hidden 4096 and
expert intermediate 2048, which with 43 x 256 x 3 matrices give the 277B
routed parameters of the blog's 284B-parameter model):

  tiny              T=4,     H=256,  I=128,  E=8,   k=2, fp32 x, uniform router
  decode_t4         T=4,     H=4096, I=2048, E=256, k=6, bf16 x, uniform, int8
  decode_t64_zipf   T=64,    same shapes, Zipf(1.1) expert load, int8
  prefill_t4604     T=4604,  same shapes, Zipf(1.1), MXFP4 activations
  stack43_decode    43 layers, T=32, uniform, int8, fp32 residual stream
  prefill_t16384    one layer, T=16384, Zipf(1.1), MXFP4

Generators:
  * Gaussians (x, router weights): numpy ``default_rng([seed, layer, tag])``,
    ``standard_normal(dtype=float32)``; tag 0 = x, 1 = router weights,
    2 = Zipf rank permutation. Router weights are 0.02 * N(0, 1) in fp32.
  * bf16 x: fp32 draws rounded to nearest-even bf16.
  * Packed E2M1 codes and E8M0 scales: SplitMix64 (Steele, Lea and Flood,
    "Fast splittable pseudorandom number generators", 2014) used as a counter
    generator: output i of a stream with key K is mix(K + (i + 1) * GAMMA),
    where mix is the SplitMix64 output finalizer. Each 64-bit output gives
    eight bytes, little-endian. A code byte is that byte (two E2M1 codes,
    uniform over all 16 values); a scale byte is 121 + (byte mod 5), i.e.
    2^-6 .. 2^-2. The stream key is mix((seed << 40) | (layer << 16) | tensor)
    with tensor 0 = W13 codes, 1 = W13 scales, 2 = W2 codes, 3 = W2 scales,
    4 = dense FP8 codes, 5 = dense FP8 scales.
  * Dense FP8 (E4M3) weight codes: the stream's bytes with the two NaN codes
    (0x7f, 0xff) replaced by their neighbours 0x7e, 0xfe (+-448); scales as
    above.
    A device kernel (csrc/synth.hip) implements the same definition so the
    43-layer stack (about 147 GB) can be generated in HBM; a GPU test checks
    that both produce the same bytes.
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np

GAMMA = np.uint64(0x9E3779B97F4A7C15)
_M1 = np.uint64(0xBF58476D1CE4E5B9)
_M2 = np.uint64(0x94D049BB133111EB)

TENSOR_W13_CODES = 0
TENSOR_W13_SCALES = 1
TENSOR_W2_CODES = 2
TENSOR_W2_SCALES = 3
TENSOR_DENSE_CODES = 4
TENSOR_DENSE_SCALES = 5

ACT_INT8 = 0
ACT_MXFP4 = 1
X_F32 = 0
X_BF16 = 1

# Zipf calibration: b_e = ZIPF_ALPHA * ln p_rank(e), p_r proportional to r^-1.1.
# ZIPF_ALPHA is chosen so that, at T=4604 with this router, the fitted slope of
# ln(load) against ln(rank) over ranks 11..200 is about -1.1 (checked by
# tests/test_synth.py::test_zipf_slope).
ZIPF_S = 1.1
ZIPF_ALPHA = 0.535


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    T: int
    H: int
    I: int
    E: int
    top_k: int
    x_dtype: int
    act_mode: int
    zipf: bool
    seed: int
    layers: int = 1

    @property
    def P(self) -> int:
        return self.T * self.top_k


WORKLOADS = {
    "tiny": Workload("tiny", 4, 256, 128, 8, 2, X_F32, ACT_INT8, False, 0),
    "tiny_mxfp4": Workload("tiny_mxfp4", 4, 256, 128, 8, 2, X_F32, ACT_MXFP4, False, 0),
    "decode_t4": Workload("decode_t4", 4, 4096, 2048, 256, 6, X_BF16, ACT_INT8, False, 1),
    "decode_t64_zipf": Workload("decode_t64_zipf", 64, 4096, 2048, 256, 6, X_BF16, ACT_INT8, True, 2),
    "prefill_t4604_zipf": Workload("prefill_t4604_zipf", 4604, 4096, 2048, 256, 6, X_BF16, ACT_MXFP4, True, 3),
    "stack43_decode_t32": Workload("stack43_decode_t32", 32, 4096, 2048, 256, 6, X_F32, ACT_INT8, False, 4, 43),
    "prefill_t16384_zipf": Workload("prefill_t16384_zipf", 16384, 4096, 2048, 256, 6, X_BF16, ACT_MXFP4, True, 4),
    # one GPU's share under tensor parallelism over I across 4 GPUs (I/4 of
    # every expert, the router replicated), at the decode and 4,604-token shapes
    "decode_t4_tp4": Workload("decode_t4_tp4", 4, 4096, 512, 256, 6, X_BF16, ACT_INT8, False, 1),
    "prefill_t4604_zipf_tp4": Workload("prefill_t4604_zipf_tp4", 4604, 4096, 512, 256, 6, X_BF16, ACT_MXFP4, True, 3),
}


# --------------------------------------------------------------------------
# SplitMix64 counter generator
# --------------------------------------------------------------------------
def _mix(z: np.ndarray) -> np.ndarray:
    z = (z ^ (z >> np.uint64(30))) * _M1
    z = (z ^ (z >> np.uint64(27))) * _M2
    return z ^ (z >> np.uint64(31))


def stream_key(seed: int, layer: int, tensor: int) -> int:
    raw = np.array([(seed << 40) | (layer << 16) | tensor], dtype=np.uint64)
    with np.errstate(over="ignore"):
        return int(_mix(raw)[0])


def splitmix_words(key: int, first: int, count: int) -> np.ndarray:
    """Outputs first .. first+count-1 of the stream with the given key."""
    with np.errstate(over="ignore"):
        i = np.arange(first + 1, first + count + 1, dtype=np.uint64)
        return _mix(np.uint64(key) + i * GAMMA)


def code_bytes(seed: int, layer: int, tensor: int, first_byte: int, nbytes: int) -> np.ndarray:
    """Packed E2M1 code bytes [first_byte, first_byte + nbytes) of a tensor."""
    assert first_byte % 8 == 0 and nbytes % 8 == 0
    w = splitmix_words(stream_key(seed, layer, tensor), first_byte // 8, nbytes // 8)
    return w.view(np.uint8).copy()


def scale_bytes(seed: int, layer: int, tensor: int, first_byte: int, nbytes: int) -> np.ndarray:
    """E8M0 scale bytes in 121..125 for [first_byte, first_byte + nbytes)."""
    raw = code_bytes(seed, layer, tensor, first_byte, nbytes)
    return (np.uint8(121) + raw % np.uint8(5)).astype(np.uint8)


def expert_weights(w: Workload, layer: int, e: int):
    """Canonical packed weights of one expert.

    Returns (w13 [2I, H/2] u8, w13_scale [2I, H/32] u8, w2 [H, I/2] u8,
    w2_scale [H, I/32] u8). Gate rows 0..I-1, up rows I..2I-1; the low nibble
    of each byte is the even element along K.
    """
    H, I = w.H, w.I
    n13, s13 = 2 * I * H // 2, 2 * I * H // 32
    n2, s2 = H * I // 2, H * I // 32
    w13 = code_bytes(w.seed, layer, TENSOR_W13_CODES, e * n13, n13).reshape(2 * I, H // 2)
    w13s = scale_bytes(w.seed, layer, TENSOR_W13_SCALES, e * s13, s13).reshape(2 * I, H // 32)
    w2 = code_bytes(w.seed, layer, TENSOR_W2_CODES, e * n2, n2).reshape(H, I // 2)
    w2s = scale_bytes(w.seed, layer, TENSOR_W2_SCALES, e * s2, s2).reshape(H, I // 32)
    return w13, w13s, w2, w2s


def all_expert_weights(w: Workload, layer: int = 0):
    """Canonical weights of every expert: [E, ...] arrays (small shapes only)."""
    H, I, E = w.H, w.I, w.E
    w13 = code_bytes(w.seed, layer, TENSOR_W13_CODES, 0, E * I * H).reshape(E, 2 * I, H // 2)
    w13s = scale_bytes(w.seed, layer, TENSOR_W13_SCALES, 0, E * 2 * I * H // 32).reshape(E, 2 * I, H // 32)
    w2 = code_bytes(w.seed, layer, TENSOR_W2_CODES, 0, E * H * I // 2).reshape(E, H, I // 2)
    w2s = scale_bytes(w.seed, layer, TENSOR_W2_SCALES, 0, E * H * I // 32).reshape(E, H, I // 32)
    return w13, w13s, w2, w2s


@dataclasses.dataclass(frozen=True)
class DenseWorkload:
    """A block-scaled FP8 dense projection: M tokens, K = input features (the
    hidden size), N = output features."""
    name: str
    M: int
    K: int
    N: int
    x_dtype: int
    seed: int


DENSE_WORKLOADS = {
    "dense_tiny": DenseWorkload("dense_tiny", 4, 256, 256, X_F32, 0),
    "dense_t32": DenseWorkload("dense_t32", 32, 4096, 4096, X_BF16, 5),
    "dense_t4604": DenseWorkload("dense_t4604", 4604, 4096, 4096, X_BF16, 6),
    "dense_t16384": DenseWorkload("dense_t16384", 16384, 4096, 4096, X_BF16, 7),
    "dense_t4604_n1536": DenseWorkload("dense_t4604_n1536", 4604, 4096, 1536, X_BF16, 8),
}


def dense_weights(w: DenseWorkload):
    """(codes [N][K] u8 E4M3 without NaN codes, E8M0 scales [N][K/32] u8)."""
    raw = code_bytes(w.seed, 0, TENSOR_DENSE_CODES, 0, w.N * w.K)
    nan = (raw & np.uint8(0x7F)) == np.uint8(0x7F)
    raw[nan] ^= np.uint8(1)
    sc = scale_bytes(w.seed, 0, TENSOR_DENSE_SCALES, 0, w.N * w.K // 32)
    return raw.reshape(w.N, w.K), sc.reshape(w.N, w.K // 32)


def dense_activations(w: DenseWorkload, M: int | None = None) -> np.ndarray:
    """x [M][K]: fp32 N(0, 1), or its nearest-even bf16 bit patterns."""
    M = w.M if M is None else M
    x = np.random.default_rng([w.seed, 0, 0]).standard_normal((M, w.K), dtype=np.float32)
    return f32_to_bf16_bits(x) if w.x_dtype == X_BF16 else x


# --------------------------------------------------------------------------
# Gaussians, bf16, Zipf bias
# --------------------------------------------------------------------------
def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round fp32 to nearest-even bf16; returns the uint16 bit patterns."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32).astype(np.uint64)
    lsb = (u >> np.uint64(16)) & np.uint64(1)
    r = (u + np.uint64(0x7FFF) + lsb) >> np.uint64(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


def activations_f32(w: Workload, layer: int = 0, T: int | None = None) -> np.ndarray:
    T = w.T if T is None else T
    rng = np.random.default_rng([w.seed, layer, 0])
    return rng.standard_normal((T, w.H), dtype=np.float32)


def activations(w: Workload, layer: int = 0, T: int | None = None) -> np.ndarray:
    """x as the layer receives it: fp32 array, or uint16 bf16 bit patterns."""
    x = activations_f32(w, layer, T)
    if w.x_dtype == X_BF16:
        return f32_to_bf16_bits(x)
    return x


def router_weights(w: Workload, layer: int = 0) -> np.ndarray:
    rng = np.random.default_rng([w.seed, layer, 1])
    return (np.float32(0.02) * rng.standard_normal((w.E, w.H), dtype=np.float32)).astype(np.float32)


def zipf_bias(E: int, seed: int, alpha: float = ZIPF_ALPHA, s: float = ZIPF_S) -> np.ndarray:
    """Per-expert logit bias making expert load roughly Zipf(s) over a random
    rank permutation: b_e = alpha * ln p_rank(e), p_r = r^-s / sum_r r^-s."""
    perm = np.random.default_rng([seed, 0, 2]).permutation(E)
    ranks = np.arange(1, E + 1, dtype=np.float64)
    p = ranks ** (-s)
    p /= p.sum()
    rank_of_e = perm + 1
    return (alpha * np.log(p[rank_of_e - 1])).astype(np.float32)


def zipf_rank_of_expert(E: int, seed: int) -> np.ndarray:
    return np.random.default_rng([seed, 0, 2]).permutation(E) + 1


def router_bias(w: Workload, layer: int = 0):
    return zipf_bias(w.E, w.seed) if w.zipf else None


def load_slope(counts_by_rank: np.ndarray, lo: int = 11, hi: int = 200) -> float:
    """Least-squares slope of ln(load) vs ln(rank) over ranks lo..hi (1-based)."""
    r = np.arange(lo, hi + 1, dtype=np.float64)
    c = counts_by_rank[lo - 1:hi].astype(np.float64)
    m = c > 0
    A = np.vstack([np.log(r[m]), np.ones(m.sum())]).T
    return float(np.linalg.lstsq(A, np.log(c[m]), rcond=None)[0][0])


def layer_bytes(w: Workload) -> dict:
    """Packed weight bytes (codes + scales) of one expert and of one layer."""
    H, I = w.H, w.I
    per_expert = (2 * I * H // 2 + 2 * I * H // 32) + (H * I // 2 + H * I // 32)
    return {"per_expert": per_expert, "per_layer": per_expert * w.E}


def describe(w: Workload) -> str:
    return (f"{w.name}: T={w.T} H={w.H} I={w.I} E={w.E} k={w.top_k} "
            f"x={'bf16' if w.x_dtype == X_BF16 else 'fp32'} "
            f"act={'mxfp4' if w.act_mode == ACT_MXFP4 else 'int8'} "
            f"{'zipf' if w.zipf else 'uniform'} seed={w.seed} layers={w.layers}")


def fmt_bytes(n: float) -> str:
    for u in ("B", "KB", "MB", "GB"):
        if abs(n) < 1000:
            return f"{n:.1f} {u}"
        n /= 1000
    return f"{n:.1f} TB"



