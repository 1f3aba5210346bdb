"""Quality harness: the KV / KQV / QKQV schemes at equal bit budget, measured
with this library's GPU codec on synthetic caches.

What is measured follows D'Alberto, "Statistical Inference and Quality
Measures of KV Cache Quantisations Inspired by TurboQuant" (gist.science
summary): section "Evaluation metrics" (scale and direction error of the key
cache, the value cache and the attention output; KL divergence between the
reference and the quantized softmax; top-5 routing recall), and the claims of
"Contribution 1" (QJL on keys inflates the score variance), "Contribution 2"
(KQV beats QKQV at n = 4), "Contribution 3" (low-rank keys are the worst case)
and "Results" (without rotation, heavy tails break the key codec).

Readings where the summary is silent (stated here, used throughout):
  scale error     SNR in dB, 10 log10(sum ||x||^2 / sum ||x - x^||^2)
  direction error 1 - cos(x, x^), mean over vectors
  KL              sum_j p_j log(p_j / p^_j), natural log, p = softmax(q K^T /
                  sqrt(d)) over all cached tokens; reported as the mean over
                  queries and as the worst case (maximum) and 99th percentile
                  ("Significance": the mean is too optimistic)
  top-5 recall    |top5(p) intersect top5(p^)| / 5, mean over queries
  score variance  variance of q . (k^ - k) / sqrt(d) over (query, token) pairs
  projection      mean of <x^, x> / ||x||^2: 1 - D_b for a scalar Lloyd-Max side
                  (centroid condition), 1 in expectation with the QJL sketch

Key distributions (synthetic, seeded): Gaussian; heavy-tailed (per-channel
scales |t_nu|, outliers in fixed channels); low-rank (rank 8 plus 0.1 noise);
focused (each query aimed at one cached key, so the softmax is peaked).
Values are Gaussian.  The reference attention uses the exact keys and values.

rotation_mse compares the rotations of the rotated schemes ("KVQuant++"
thread, "Rate-distortion performance": with the QR or the Hadamard rotation
the per-element MSE stays under sqrt(3 pi/2) 4^-b).

tail_sweep follows "Results" (as the tail weight grows, nu -> 1.05, the
rotated key codec keeps a stable direction error while the unrotated one
fails); amplification follows "Contribution 1" (QJL on keys inflates the
inner-product variance by pi/2 against the scalar residual, and by 2 pi when
an n-bit scalar scheme is compared with (n-1) bits + the 1-bit sketch: the
2 pi is the high-rate limit of (pi/2) D_{n-1} / D_n, since each bit quarters
the distortion); six_d follows "Evaluation metrics" (scale and direction at
the key cache, the value cache and the output, compared between schemes with
Mann-Whitney U / rank-biserial correlation, Kolmogorov-Smirnov and energy
distance).  Readings for the 6D samples: one 6-vector per query; the key and
value sites are weighted by that query's reference attention p (the tokens it
reads): SNR_site = 10 log10(sum_j p_j ||x_j||^2 / sum_j p_j ||x_j - x^_j||^2)
and phi_site = sum_j p_j angle(x_j, x^_j); the output site is the SNR and
angle of o^ against o.  Errors are oriented so that larger is worse: the
sample is (-SNR_K, phi_K, -SNR_V, phi_V, -SNR_T, phi_T).
"""
from __future__ import annotations

import json
import math
from dataclasses import asdict, dataclass

import torch

from . import synth
from .kvq import KVQCache

SCHEMES = ("KV", "KQV", "QKQV")


@dataclass
class Metrics:
    scheme: str
    n_bits: int
    keys: str
    snr_k: float
    dir_k: float
    snr_v: float
    dir_v: float
    snr_o: float
    dir_o: float
    kl: float
    kl_max: float
    kl_p99: float
    top5: float
    score_var: float
    proj_k: float
    proj_v: float


def _gen(seed, device):
    g = torch.Generator(device="cpu")
    g.manual_seed(int(seed))
    return g


def make_keys(kind: str, H: int, N: int, d: int, seed: int, nu: float = 3.0) -> torch.Tensor:
    """[H][N][d] fp32 keys of one synthetic family (CPU)."""
    g = _gen(seed, "cpu")
    if kind in ("gaussian", "focused"):
        return torch.randn(H, N, d, generator=g)
    if kind == "heavytail":
        # fixed outlier channels: per-channel scale |t_nu| (Student t drawn as
        # Z / sqrt(chi2_nu / nu), chi2_nu from a Gamma(nu/2, 2) variate)
        z = torch.randn(H, 1, d, generator=g)
        chi2 = torch._standard_gamma(torch.full((H, 1, d), nu / 2.0), generator=g) * 2.0
        s = (z / torch.sqrt(chi2 / nu)).abs()
        return torch.randn(H, N, d, generator=g) * s
    if kind == "lowrank":
        U = torch.randn(H, N, 8, generator=g)
        W = torch.randn(H, d, 8, generator=g)
        return U @ W.transpose(1, 2) + 0.1 * torch.randn(H, N, d, generator=g)
    raise ValueError(kind)


def make_queries(kind: str, keys: torch.Tensor, Q: int, seed: int) -> torch.Tensor:
    """[H][Q][d] fp32 queries.  'focused': each query is a random cached key
    scaled up plus noise, so its attention concentrates on that key; otherwise
    Gaussian with the keys' per-channel spread, normalised to unit mean
    variance."""
    g = _gen(seed, "cpu")
    H, N, d = keys.shape
    if kind == "focused":
        # 1.5 x a cached key: its logit is ~1.5 ||k||^2 / sqrt(d), far above
        # the others, so one token carries most of the weight
        idx = torch.randint(0, N, (H, Q), generator=g)
        base = torch.gather(keys, 1, idx[..., None].expand(H, Q, d))
        return 1.5 * base + 0.3 * torch.randn(H, Q, d, generator=g)
    # queries on the keys' scale: same marginal spread per channel
    sd = keys.std(dim=1, keepdim=True)
    return torch.randn(H, Q, d, generator=g) * sd / sd.pow(2).mean(-1, keepdim=True).sqrt()


def _snr_db(x, xh):
    return float(10.0 * torch.log10(x.pow(2).sum() / (x - xh).pow(2).sum().clamp_min(1e-30)))


def _proj(x, xh):
    x2, xh2 = x.reshape(-1, x.shape[-1]), xh.reshape(-1, x.shape[-1])
    return float(((x2 * xh2).sum(-1) / x2.pow(2).sum(-1).clamp_min(1e-30)).mean())


def _dir_err(x, xh):
    c = torch.nn.functional.cosine_similarity(x.reshape(-1, x.shape[-1]), xh.reshape(-1, x.shape[-1]),
                                              dim=-1, eps=1e-30)
    return float((1.0 - c).mean())


def roundtrip(scheme: str, n_bits: int, K: torch.Tensor, V: torch.Tensor, S_bf16, device,
              rotation: str = "wht", rot_param=None):
    """Quantize K and V ([H][N][d] fp32) with the GPU codec and reconstruct them."""
    H, N, d = K.shape
    cache = KVQCache(scheme, n_bits, d, 1, H, N, S_bf16=S_bf16, device=device, rotation=rotation,
                     rot_signs=rot_param if rotation == "rht" else None,
                     rot_Q=rot_param if rotation == "qr" else None)
    cache.quantize_k(K[None].to(device), 0)
    cache.quantize_v(V[None].to(device), 0)
    Kh = cache.dequantize(0, 0, N)[0]
    Vh = cache.dequantize(1, 0, N)[0]
    return Kh, Vh


def attention(q, K, V):
    """Reference softmax attention in fp32: q [H][Q][d], K, V [H][N][d]."""
    d = q.shape[-1]
    s = torch.matmul(q, K.transpose(1, 2).contiguous()) / math.sqrt(d)
    p = torch.softmax(s, dim=-1)
    return p, torch.matmul(p, V), s


def evaluate(scheme, n_bits, keys_kind, K, V, q, S_bf16, device) -> Metrics:
    Kd, Vd, qd = K.to(device), V.to(device), q.to(device)
    Kh, Vh = roundtrip(scheme, n_bits, K, V, S_bf16, device)
    p, o, s = attention(qd, Kd, Vd)
    ph, oh, sh = attention(qd, Kh, Vh)
    klq = kl_per_query(p, ph).flatten()
    t5 = torch.topk(p, 5, dim=-1).indices
    t5h = torch.topk(ph, 5, dim=-1).indices
    rec = (t5[..., :, None] == t5h[..., None, :]).any(-1).float().sum(-1).mean() / 5.0
    return Metrics(scheme, n_bits, keys_kind, _snr_db(Kd, Kh), _dir_err(Kd, Kh), _snr_db(Vd, Vh),
                   _dir_err(Vd, Vh), _snr_db(o, oh), _dir_err(o, oh), float(klq.mean()),
                   float(klq.max()), float(torch.quantile(klq.double(), 0.99)), float(rec),
                   float((sh - s).var()), _proj(Kd, Kh), _proj(Vd, Vh))


def kl_per_query(p, ph):
    """KL(p || p^) of every query row (natural log)."""
    return (p * (torch.log(p.clamp_min(1e-38)) - torch.log(ph.clamp_min(1e-38)))).sum(-1)


def rotation_mse(kind: str, bits: int, rotation: str, H=4, N=1024, d=128, seed=2025,
                 device="cuda"):
    """Per-element MSE of unit key directions through the K side of KQV at n =
    bits (n-bit scalar codec after the rotation), for a key family: the pages'
    families plus "hadamard" (rows of the normalised Hadamard matrix, each a
    single spike after the plain WHT).  Returns mean ||x - x^||^2 / d."""
    if kind == "hadamard":
        Hm = torch.tensor([[1.0]])
        while Hm.shape[0] < d:
            Hm = torch.cat([torch.cat([Hm, Hm], 1), torch.cat([Hm, -Hm], 1)], 0)
        Hm = Hm / math.sqrt(d)
        K = Hm[torch.arange(H * N) % d].reshape(H, N, d)
    else:
        K = make_keys(kind, H, N, d, seed)
    K = K / K.norm(dim=-1, keepdim=True)
    param = {"wht": None, "rht": synth.rotation_signs(d, seed + 1),
             "qr": synth.rotation_qr(d, seed + 2)}[rotation]
    S = synth.bits_u16(synth.sketch_bf16(d, d, 7))
    Kh, _ = roundtrip("KQV", bits, K, K, S, device, rotation, param)
    return float((Kh.float().cpu() - K).pow(2).sum(-1).mean() / d)


def _angle(x, xh):
    c = torch.nn.functional.cosine_similarity(x, xh, dim=-1, eps=1e-30)
    return torch.arccos(c.clamp(-1.0, 1.0))


def six_d_samples(p, K, Kh, V, Vh, o, oh):
    """[H Q][6] error samples (larger is worse): (-SNR_K, phi_K, -SNR_V, phi_V,
    -SNR_T, phi_T) per query, key and value sites weighted by the query's
    reference attention p [H][Q][N]."""
    def site(x, xh):
        e2 = (x - xh).pow(2).sum(-1)                      # [H][N]
        x2 = x.pow(2).sum(-1)
        ang = _angle(x, xh)                               # [H][N]
        num = torch.einsum("hqn,hn->hq", p, x2)
        den = torch.einsum("hqn,hn->hq", p, e2).clamp_min(1e-30)
        return -10.0 * torch.log10(num / den), torch.einsum("hqn,hn->hq", p, ang)
    snr_k, phi_k = site(K, Kh)
    snr_v, phi_v = site(V, Vh)
    snr_t = -10.0 * torch.log10(o.pow(2).sum(-1) / (o - oh).pow(2).sum(-1).clamp_min(1e-30))
    phi_t = _angle(o, oh)
    return torch.stack([snr_k, phi_k, snr_v, phi_v, snr_t, phi_t], -1).reshape(-1, 6).double()


def rank_biserial(a, b):
    """Rank-biserial correlation of the Mann-Whitney U test of samples a, b:
    P(a > b) - P(a < b) (ties count half), in [-1, 1]; positive when a tends
    to be larger."""
    a = torch.as_tensor(a, dtype=torch.float64).flatten()
    b = torch.as_tensor(b, dtype=torch.float64).flatten()
    allv = torch.cat([a, b])
    order = torch.argsort(allv, stable=True)
    ranks = torch.empty_like(allv)
    ranks[order] = torch.arange(1, allv.numel() + 1, dtype=torch.float64)
    # average ranks of ties
    sv = allv[order]
    i = 0
    n = sv.numel()
    while i < n:
        j = i
        while j + 1 < n and sv[j + 1] == sv[i]:
            j += 1
        if j > i:
            ranks[order[i:j + 1]] = (i + j + 2) / 2.0
        i = j + 1
    u_a = ranks[:a.numel()].sum() - a.numel() * (a.numel() + 1) / 2.0
    return float(2.0 * u_a / (a.numel() * b.numel()) - 1.0)


def ks_statistic(a, b):
    """Two-sample Kolmogorov-Smirnov statistic sup |F_a - F_b|."""
    a = torch.sort(torch.as_tensor(a, dtype=torch.float64).flatten()).values
    b = torch.sort(torch.as_tensor(b, dtype=torch.float64).flatten()).values
    x = torch.cat([a, b])
    fa = torch.searchsorted(a, x, right=True).double() / a.numel()
    fb = torch.searchsorted(b, x, right=True).double() / b.numel()
    return float((fa - fb).abs().max())


def energy_distance(X, Y):
    """Energy distance 2 E||X - Y|| - E||X - X'|| - E||Y - Y'|| of two samples of
    row vectors (V-statistics: every pair, the zero diagonal included)."""
    X = torch.as_tensor(X, dtype=torch.float64)
    Y = torch.as_tensor(Y, dtype=torch.float64)
    if X.dim() == 1:
        X, Y = X[:, None], Y[:, None]
    return float(2.0 * torch.cdist(X, Y).mean() - torch.cdist(X, X).mean() - torch.cdist(Y, Y).mean())


def six_d(keys_kind="gaussian", n_bits=4, H=8, N=2048, d=128, Q=64, seed=2024, device="cuda"):
    """6D error samples of the three schemes on one key family and their
    comparisons: for KQV against each other scheme, per dimension the
    rank-biserial correlation (positive: KQV's errors tend to be larger) and
    the KS statistic, and the energy distance between the two 6D samples after
    each dimension is standardised over the pooled sample."""
    S = synth.bits_u16(synth.sketch_bf16(d, d, 7))
    i = ("gaussian", "heavytail", "lowrank", "focused").index(keys_kind)
    K = make_keys(keys_kind, H, N, d, seed + 10 * i)
    V = torch.randn(H, N, d, generator=_gen(seed + 10 * i + 1, "cpu"))
    q = make_queries(keys_kind, K, Q, seed + 10 * i + 2)
    Kd, Vd, qd = K.to(device), V.to(device), q.to(device)
    p, o, _ = attention(qd, Kd, Vd)
    samples = {}
    for sc in SCHEMES:
        Kh, Vh = roundtrip(sc, n_bits, K, V, S, device)
        _, oh, _ = attention(qd, Kh, Vh)
        samples[sc] = six_d_samples(p, Kd, Kh, Vd, Vh, o, oh).cpu()
    comp = {}
    for other in ("QKQV", "KV"):
        a, b = samples["KQV"], samples[other]
        pooled = torch.cat([a, b])
        mu, sd = pooled.mean(0), pooled.std(0).clamp_min(1e-12)
        comp[other] = {"rank_biserial": [rank_biserial(a[:, k], b[:, k]) for k in range(6)],
                       "ks": [ks_statistic(a[:, k], b[:, k]) for k in range(6)],
                       "energy": energy_distance((a - mu) / sd, (b - mu) / sd)}
    return samples, comp


def tail_sweep(nus=(5.0, 3.0, 2.0, 1.5, 1.2, 1.05), n_bits=4, H=8, N=1024, d=128, seed=2030,
               device="cuda"):
    """Key direction error (1 - cos, mean over keys) of KV and KQV for
    heavy-tailed keys of growing tail weight: per-channel scales |t_nu|,
    divided by their maximum per head (the direction error does not depend on
    the overall scale, and the stored fp16 norms stay finite)."""
    S = synth.bits_u16(synth.sketch_bf16(d, d, 7))
    out = []
    for k, nu in enumerate(nus):
        g = _gen(seed + k, "cpu")
        z = torch.randn(H, 1, d, generator=g)
        chi2 = torch._standard_gamma(torch.full((H, 1, d), nu / 2.0), generator=g) * 2.0
        s = (z / torch.sqrt(chi2 / nu)).abs()
        s = s / s.amax(-1, keepdim=True)
        K = torch.randn(H, N, d, generator=g) * s
        row = {"nu": nu}
        for sc in ("KV", "KQV"):
            Kh, _ = roundtrip(sc, n_bits, K, K, S, device)
            row[sc] = _dir_err(K.to(device), Kh)
        out.append(row)
    return out


def amplification(H=8, N=2048, d=128, seed=2040, device="cuda"):
    """Scalar key codec distortion D_b (b = 1..4, Gaussian keys, from the
    n-bit key side of KQV) and the predicted variance amplification
    (pi/2) D_{b-1} / D_b of an (b-1)-bit + 1-bit-sketch key against a b-bit
    scalar key, whose high-rate limit is 2 pi; plus the measured score-error
    variance ratio of QKQV (n-1 bits + sketch on keys) to KQV (n bits) at n = 4."""
    S = synth.bits_u16(synth.sketch_bf16(d, d, 7))
    K = make_keys("gaussian", H, N, d, seed)
    V = torch.randn(H, N, d, generator=_gen(seed + 1, "cpu"))
    q = make_queries("gaussian", K, 64, seed + 2)
    Kd = K.to(device)
    D = {}
    for b in (1, 2, 3, 4):
        # b-bit scalar keys: the key side of KQV at n = b (KV at n = 1; on
        # isotropic Gaussian keys the rotation changes nothing in distribution)
        Kh, _ = roundtrip("KQV" if b >= 2 else "KV", b, K, V, S, device)
        D[b] = float(((Kd - Kh).pow(2).sum(-1) / Kd.pow(2).sum(-1)).mean())
    m4 = evaluate("KQV", 4, "gaussian", K, V, q, S, device)
    m4q = evaluate("QKQV", 4, "gaussian", K, V, q, S, device)
    pred = {b: math.pi / 2 * D[b - 1] / D[b] for b in (2, 3, 4)}
    return {"D": D, "ratio_D": {b: D[b - 1] / D[b] for b in (2, 3, 4)}, "predicted": pred,
            "measured_n4": m4q.score_var / m4.score_var, "limit": 2 * math.pi}


def grid(keys_kinds=("gaussian", "heavytail", "lowrank", "focused"), bits=(2, 3, 4), H=8, N=2048,
         d=128, Q=64, seed=2024, device="cuda", nu=3.0):
    """All (keys, scheme, n) cells on one set of inputs per key family."""
    S = synth.bits_u16(synth.sketch_bf16(d, d, 7))
    out = []
    for i, kind in enumerate(keys_kinds):
        K = make_keys(kind, H, N, d, seed + 10 * i, nu=nu)
        V = torch.randn(H, N, d, generator=_gen(seed + 10 * i + 1, "cpu"))
        q = make_queries(kind, K, Q, seed + 10 * i + 2)
        for n in bits:
            for sc in SCHEMES:
                out.append(evaluate(sc, n, kind, K, V, q, S, device))
    return out


def main():
    import argparse
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--N", type=int, default=2048)
    ap.add_argument("--H", type=int, default=8)
    ap.add_argument("--Q", type=int, default=64)
    ap.add_argument("--d", type=int, default=128)
    args = ap.parse_args()
    for m in grid(H=args.H, N=args.N, Q=args.Q, d=args.d):
        print(json.dumps(asdict(m)), flush=True)


if __name__ == "__main__":
    main()
