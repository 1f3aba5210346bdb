"""Host checks of the quality harness's metric definitions (no GPU)."""
import math

import torch

from kv_cache_quantization_kqv_amd import quality as Q


def test_metric_definitions_on_known_inputs():
    x = torch.tensor([[3.0, 4.0], [1.0, 0.0]])
    assert Q._proj(x, x) == 1.0
    assert abs(Q._proj(x, 0.5 * x) - 0.5) < 1e-7
    assert abs(Q._dir_err(x, 2.0 * x)) < 1e-7
    xr = torch.tensor([[4.0, -3.0], [0.0, 1.0]])             # orthogonal rows
    assert abs(Q._dir_err(x, xr) - 1.0) < 1e-7
    assert abs(Q._snr_db(x, 0.9 * x) - 20.0) < 1e-4          # error 10% in amplitude


def test_attention_reference_and_kl_top5():
    g = torch.Generator().manual_seed(3)
    q = torch.randn(2, 5, 16, generator=g)
    K = torch.randn(2, 40, 16, generator=g)
    V = torch.randn(2, 40, 16, generator=g)
    p, o, s = Q.attention(q, K, V)
    assert torch.allclose(p.sum(-1), torch.ones(2, 5))
    ref = torch.softmax(torch.einsum("hqd,hnd->hqn", q, K) / 4.0, -1)
    assert torch.allclose(p, ref, atol=1e-6)
    assert torch.allclose(o, torch.einsum("hqn,hnd->hqd", ref, V), atol=1e-5)


def test_key_families_have_their_structure():
    lr = Q.make_keys("lowrank", 2, 512, 64, 5)
    sv = torch.linalg.svdvals(lr[0])
    assert sv[8] < 0.05 * sv[0]                              # rank 8 plus small noise
    ht = Q.make_keys("heavytail", 2, 4096, 64, 6)
    ch = ht[0].std(0)
    assert ch.max() / ch.median() > 3                        # outlier channels
    g = Q.make_keys("gaussian", 2, 4096, 64, 7)
    assert abs(float(g.std()) - 1) < 0.02
    f = Q.make_queries("focused", g, 8, 8)
    p, _, _ = Q.attention(f, g, g)
    assert float(p.max(-1).values.mean()) > 0.5              # peaked attention
    assert math.isfinite(float(Q.make_queries("heavytail", ht, 8, 9).std()))


def test_rank_statistics_match_scipy():
    """rank_biserial = 2 U / (n1 n2) - 1 with U the Mann-Whitney statistic of
    the first sample; ks_statistic = two-sample KS; energy_distance in 1-D is
    the square of scipy's (which returns the square root)."""
    import numpy as np
    from scipy import stats
    rng = np.random.default_rng(5)
    a = rng.standard_normal(300)
    b = rng.standard_normal(200) + 0.4
    b[:10] = a[:10]                                          # some ties
    u = stats.mannwhitneyu(a, b, alternative="two-sided").statistic
    assert abs(Q.rank_biserial(a, b) - (2 * u / (300 * 200) - 1)) < 1e-12
    assert abs(Q.ks_statistic(a, b) - stats.ks_2samp(a, b).statistic) < 1e-12
    assert abs(Q.energy_distance(a, b) - stats.energy_distance(a, b) ** 2) < 1e-9
    assert Q.rank_biserial(a, a) == 0.0 and Q.energy_distance(a, a) < 1e-12
    assert Q.rank_biserial(a + 100, b) == 1.0


def test_six_d_samples_on_known_errors():
    """Exact reconstructions give angle 0; a uniform 10% shrink gives -20 dB
    (oriented: larger is worse) and angle 0 at every site."""
    g = torch.Generator().manual_seed(4)
    K = torch.randn(2, 30, 8, generator=g, dtype=torch.float64)
    V = torch.randn(2, 30, 8, generator=g, dtype=torch.float64)
    q = torch.randn(2, 3, 8, generator=g, dtype=torch.float64)
    p, o, _ = Q.attention(q, K, V)
    x = Q.six_d_samples(p, K, 0.9 * K, V, 0.9 * V, o, 0.9 * o)
    assert x.shape == (6, 6)
    assert torch.allclose(x[:, [0, 2, 4]], torch.full((6, 3), -20.0, dtype=torch.float64), atol=1e-9)
    assert float(x[:, [1, 3, 5]].abs().max()) < 1e-6
    assert float(Q.kl_per_query(p, p).abs().max()) < 1e-12
