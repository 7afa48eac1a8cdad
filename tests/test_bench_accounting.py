"""The benchmark's algorithmic accounting (the bytes and FLOPs its roofline
fractions divide by) against figures worked out by hand from the workload
shapes: an expert's packed W13 and W2 bytes, the layer's FP4 FLOPs
(2 P (H 2I + I H), 50,331,648 per pair at H 4096, I 2048), the 4-token
decode layer's bytes (about 23.2 distinct experts x 13.37 MB + the router
weights, about 314.5 MB), and the published peaks the fractions use."""
import bench
from fp4_routed_mixture_amd import synth as S


def test_per_expert_bytes():
    w = S.WORKLOADS["decode_t4"]  # H 4096, I 2048
    # W13: 4096 rows x 2048 code bytes + 4096 x 128 scale bytes; W2: 4096 x 1024 + 4096 x 64
    assert bench.per_expert_bytes(w) == (8_388_608 + 524_288, 4_194_304 + 262_144)


def test_prefill_chunk_accounting():
    w = S.WORKLOADS["prefill_t16384_zipf"]
    P = w.T * w.top_k  # 98,304 pairs
    acc = bench.layer_accounting(w, w.T, 256, 256, True, False)
    assert acc["layer_flops"] == 50_331_648 * P
    assert acc["gate_up_flops"] == 33_554_432 * P
    # every expert touched: 256 x 13,369,344 B, router weights 4 MiB, bf16 x 128 MiB, fp32 out 256 MiB
    assert acc["layer_bytes"] == 256 * 13_369_344 + 4 * 2 ** 20 + 128 * 2 ** 20 + 256 * 2 ** 20
    # gate/up: the W13 of 256 experts, MXFP4 x (codes 32 MiB + scales 2 MiB), MXFP4 a per pair (1,088 B)
    assert acc["gate_up_bytes"] == 256 * 8_912_896 + 32 * 2 ** 20 + 2 * 2 ** 20 + P * 1088


def test_decode_layer_bytes_match_the_worked_figure():
    w = S.WORKLOADS["decode_t4"]
    acc = bench.layer_accounting(w, w.T, 23.2, 23.2, True, True)
    assert abs(acc["layer_bytes"] / 1e6 - 314.5) < 0.05
    # int8 gate/up: x as FP8 hi/lo planes (2 bytes an element) in, fp32 a out
    assert acc["gate_up_bytes"] == 23.2 * 8_912_896 + 4 * 2 * 4096 + 24 * 2048 * 4


def test_published_peaks():
    assert bench.HBM_PEAK_GBS == 8000.0
    assert bench.FP4_PEAK_TFLOPS == 10100.0
    assert bench.FP8_PEAK_TFLOPS == 5000.0
