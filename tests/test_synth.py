"""The seeded input generators: known answers and the workload recipes."""
import numpy as np

from fp4_routed_mixture_amd import synth as S


def test_splitmix64_known_answer():
    # published SplitMix64 outputs for state 1234567 (Steele, Lea, Flood 2014;
    # the reference C implementation's sequence)
    assert S.splitmix_words(1234567, 0, 5).tolist() == [
        6457827717110365317, 3203168211198807973, 9817491932198370423,
        4593380528125082431, 16408922859458223821]


def test_counter_generator_is_random_access():
    key = S.stream_key(3, 7, 2)
    a = S.splitmix_words(key, 0, 1000)
    b = S.splitmix_words(key, 400, 100)
    assert np.array_equal(a[400:500], b)
    assert np.array_equal(S.code_bytes(1, 0, 0, 64, 64), S.code_bytes(1, 0, 0, 0, 256)[64:128])


def test_code_and_scale_distributions():
    c = S.code_bytes(1, 0, 0, 0, 1 << 20)
    nib = np.concatenate([c & 15, c >> 4])
    cnt = np.bincount(nib, minlength=16)
    assert cnt.min() > 0.97 * cnt.mean() and cnt.max() < 1.03 * cnt.mean()
    s = S.scale_bytes(1, 0, 1, 0, 1 << 16)
    assert s.min() == 121 and s.max() == 125


def test_expert_slices_match_whole_tensor():
    w = S.WORKLOADS["tiny"]
    allw = S.all_expert_weights(w)
    for e in (0, 3, 7):
        one = S.expert_weights(w, 0, e)
        for a, b in zip(allw, one):
            assert np.array_equal(a[e], b)


def test_bf16_round_to_nearest_even():
    x = np.array([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -9, -2.5, 3.0e38], np.float32)
    b = S.f32_to_bf16_bits(x)
    back = S.bf16_bits_to_f32(b)
    assert back[0] == 1.0
    assert back[1] == 1.0  # halfway, ties to even (1.0)
    assert back[2] == 1.0 + 2 ** -7  # above halfway
    assert back[3] == -2.5


def test_zipf_slope():
    """The calibrated bias gives a load slope of about -1.1 over ranks 11..200
    at the 4,604-token prefill shape (float64 logits; selection by logit is
    selection by sigmoid score)."""
    w = S.WORKLOADS["prefill_t4604_zipf"]
    x = S.bf16_bits_to_f32(S.activations(w)).astype(np.float64)
    wr = S.router_weights(w).astype(np.float64)
    l = x @ wr.T + S.router_bias(w).astype(np.float64)
    ids = np.argpartition(-l, w.top_k, axis=1)[:, : w.top_k]
    cnt = np.bincount(ids.ravel(), minlength=w.E)
    by_rank = np.zeros(w.E)
    by_rank[S.zipf_rank_of_expert(w.E, w.seed) - 1] = cnt
    assert abs(S.load_slope(by_rank) + 1.1) < 0.03
