"""Write tests/golden/routing_hashes.json from the CPU oracle.

The MI250 paper (DeepSeek-V4-Flash on AMD gfx90a: Correctness Recovery and
Inference Performance Engineering, abstract) checks correctness on fixed
tokens and with hashes before optimizing. This script records, for each seeded workload, SHA-256 digests
of the oracle's routing ids (int32, little-endian, [T][k] row-major), routing
weights (fp32 bits) and expert-sort arrays. It calls only ``oracle`` and the
seeded input generators.

Run from the repository root: python tests/golden/make_golden.py
"""
import hashlib
import json
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402

import oracle  # noqa: E402
from fp4_routed_mixture_amd import synth as S  # noqa: E402

BLOCK_M = {"decode": 16, "prefill": 128}


def sha(a: np.ndarray) -> str:
    return hashlib.sha256(np.ascontiguousarray(a).astype(a.dtype.newbyteorder("<")).tobytes()).hexdigest()


def routing_record(w: S.Workload) -> dict:
    x = S.activations(w)
    ids, wts = oracle.route(x, S.router_weights(w), S.router_bias(w), w.top_k)
    rec = {"T": w.T, "E": w.E, "k": w.top_k, "ids_sha256": sha(ids), "w_sha256": sha(wts)}
    for name, bm in BLOCK_M.items():
        s = oracle.sort(ids, w.E, bm)
        rec[f"sort_bm{bm}"] = {k: sha(s[k]) for k in ("counts", "offsets", "sorted", "pos", "tile_expert")}
        rec[f"sort_bm{bm}"]["n_tiles"] = s["n_tiles"]
    rec["distinct_experts"] = int(len(np.unique(ids)))
    rec["max_load"] = int(np.bincount(ids.ravel(), minlength=w.E).max())
    return rec


def main():
    out = {}
    for name, w in S.WORKLOADS.items():
        out[name] = routing_record(w)
        print(name, out[name]["ids_sha256"][:16], "distinct", out[name]["distinct_experts"],
              "max_load", out[name]["max_load"], flush=True)
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "routing_hashes.json")
    with open(path, "w") as f:
        json.dump(out, f, indent=1, sort_keys=True)
        f.write("\n")


if __name__ == "__main__":
    main()
