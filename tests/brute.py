"""Independent float64 / brute-force references used to pin the oracle.

Written from the format and method definitions, not from oracle.c: nothing
here calls the oracle, and nothing is ported from it.
"""
import numpy as np

# OCP Microscaling Formats (MX) v1.0, FP4 E2M1 element values for codes 0..7.
E2M1_POS = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])
E2M1 = np.concatenate([E2M1_POS, -E2M1_POS])


def unpack_codes(packed: np.ndarray) -> np.ndarray:
    """[..., K/2] bytes -> [..., K] codes; the low nibble is the even element."""
    lo = packed & 0x0F
    hi = packed >> 4
    return np.stack([lo, hi], axis=-1).reshape(*packed.shape[:-1], packed.shape[-1] * 2)


def dequant(codes_packed: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """Block-32 E2M1 x E8M0 -> float64, blocks along the last axis."""
    v = E2M1[unpack_codes(codes_packed)]
    s = np.exp2(scales.astype(np.float64) - 127.0)
    return v * np.repeat(s, 32, axis=-1)


def ulp32(x: np.ndarray) -> np.ndarray:
    x = np.abs(np.asarray(x, np.float32))
    return np.spacing(x).astype(np.float64)


def nearest_e2m1_code(v: float) -> int:
    """Brute force over all 16 codes: nearest value, ties to even mantissa,
    sign of zero from the sign of v."""
    best, bestd = None, None
    for c in range(16):
        if (c >= 8) != bool(np.signbit(v)):
            continue
        d = abs(abs(v) - abs(E2M1[c]))
        if best is None or d < bestd or (d == bestd and (c & 1) == 0 and (best & 1) == 1):
            best, bestd = c, d
    return best


def int8_bruteforce(v: np.ndarray, s: float) -> np.ndarray:
    """q in [-127,127] minimising |v/s - q| (computed from the fp32 quotient),
    ties to even, by scanning every candidate."""
    cand = np.arange(-127, 128, dtype=np.float64)
    out = np.empty(v.shape, np.int64)
    for i, x in enumerate(v.ravel()):
        r = float(np.float32(x) / np.float32(s))
        d = np.abs(r - cand)
        m = d.min()
        ties = cand[d == m]
        even = ties[np.mod(ties, 2) == 0]
        out.ravel()[i] = int(even[0] if len(even) else ties[0])
    return out


def silu64(g):
    return g / (1.0 + np.exp(-g))
