"""Quality of the three schemes at equal budget, measured with the GPU codec
on synthetic caches (d = 128, 8 heads, 2048 tokens, 64 queries per head).

Claims checked (D'Alberto, "Statistical Inference and Quality Measures of KV
Cache Quantisations Inspired by TurboQuant", gist.science summary):
  Contribution 2 / Results: at n = 4, KQV has lower softmax KL and higher
    top-5 recall than QKQV on every key family;
  Contribution 1: QJL on keys inflates the score-error variance; with the
    scalar codec's distortion D_b measured here, the (n-1)-bit + sketch keys
    should show (pi/2) D_{n-1} / D_n times the n-bit scalar variance;
  Results: without rotation (KV) heavy-tailed keys break the key codec;
  Contribution 3: low-rank keys are the worst case for attention quality;
  Contribution 1 (unbiasedness): the sketched value side has projection
    ratio 1, the scalar side 1 - D_b.
The K-geometry crossover at n in {2, 3} that the summary reports is not
asserted: with direction error = 1 - cos of the reconstructed key it does not
appear in this setup (QKQV keys are worse at every budget).
"""
import math

import pytest
import torch

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def table():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from kv_cache_quantization_kqv_amd import quality
    print("case quality grid", flush=True)
    rows = quality.grid(device="cuda")
    return {(m.keys, m.scheme, m.n_bits): m for m in rows}


FAMILIES = ("gaussian", "heavytail", "lowrank", "focused")


@pytest.mark.parametrize("keys", FAMILIES)
def test_kqv_beats_qkqv_at_four_bits(table, keys):
    a, b = table[(keys, "KQV", 4)], table[(keys, "QKQV", 4)]
    assert a.kl * 2.0 < b.kl, (a.kl, b.kl)
    assert a.top5 > b.top5
    assert a.dir_o < b.dir_o


@pytest.mark.parametrize("keys", FAMILIES)
def test_qjl_on_keys_inflates_score_variance_as_predicted(table, keys):
    g3, g4 = table[(keys, "KQV", 3)], table[(keys, "KQV", 4)]
    d3 = 10 ** (-g3.snr_k / 10)            # scalar key codec distortion at 3 and 4 bits
    d4 = 10 ** (-g4.snr_k / 10)
    predicted = math.pi / 2 * d3 / d4
    ratio = table[(keys, "QKQV", 4)].score_var / g4.score_var
    assert ratio > math.pi / 2
    assert abs(ratio / predicted - 1) < 0.2, (ratio, predicted)


def test_heavy_tails_break_unrotated_keys(table):
    kv, kqv = table[("heavytail", "KV", 4)], table[("heavytail", "KQV", 4)]
    assert kv.dir_k > 5 * kqv.dir_k
    assert kv.kl > 10 * kqv.kl


def test_low_rank_keys_are_the_worst_case(table):
    lr = table[("lowrank", "KQV", 4)].kl
    for keys in ("gaussian", "heavytail", "focused"):
        assert lr > 3 * table[(keys, "KQV", 4)].kl


@pytest.mark.parametrize("keys", FAMILIES)
def test_kl_falls_with_budget(table, keys):
    for sc in ("KV", "KQV", "QKQV"):
        kl = [table[(keys, sc, n)].kl for n in (2, 3, 4)]
        assert kl[0] > kl[1] > kl[2], (sc, kl)


@pytest.mark.parametrize("n", [2, 3, 4])
def test_sketch_removes_the_scalar_shrinkage(table, n):
    """Lloyd-Max centroids give <x^, x> = (1 - D_b) ||x||^2 on average; the
    QJL residual estimate is unbiased, so the sketched side projects to 1."""
    kv, kqv = table[("gaussian", "KV", n)], table[("gaussian", "KQV", n)]
    d_b = 10 ** (-kv.snr_v / 10)
    assert abs(kv.proj_v - (1 - d_b)) < 0.01 * d_b + 2e-4
    assert abs(kqv.proj_v - 1.0) < 3e-3
    assert abs(kqv.proj_v - 1.0) < abs(kv.proj_v - 1.0)


@pytest.mark.parametrize("bits", [2, 3, 4])
def test_rotations_stay_under_the_rate_distortion_bound(bits):
    """KVQuant++ thread, 'Rate-distortion performance': whether the rotation
    is the (randomized) Hadamard or a Haar QR rotation, the per-element MSE of
    unit keys stays under sqrt(3 pi/2) 4^-b (the literal reading) and, on
    generic keys, under the whole-vector form (sqrt(3) pi/2) 4^-b / d.  On keys
    that the plain WHT maps to single spikes the plain WHT breaks the
    whole-vector form, while the randomized rotations do not."""
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from kv_cache_quantization_kqv_amd import quality
    print(f"case rotation mse bits={bits}", flush=True)
    lit = math.sqrt(3 * math.pi / 2) * 4.0 ** -bits
    tq = (math.sqrt(3) * math.pi / 2) * 4.0 ** -bits / 128
    for kind in ("gaussian", "heavytail", "lowrank"):
        for rot in ("wht", "rht", "qr"):
            e = quality.rotation_mse(kind, bits, rot)
            assert e <= lit and e <= tq, (kind, rot, e, tq)
    assert quality.rotation_mse("hadamard", bits, "wht") > tq
    assert quality.rotation_mse("hadamard", bits, "qr") <= tq
    # one sign draw maps every Hadamard row to the same magnitudes (a permuted
    # Walsh transform of the signs): average 32 draws
    e = sum(quality.rotation_mse("hadamard", bits, "rht", H=1, N=64, seed=3000 + 7 * k)
            for k in range(32)) / 32
    assert e <= tq, e
