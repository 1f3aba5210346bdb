"""Seeded synthetic workloads (inputs only; none of the codec's arithmetic).

Both the GPU path and the CPU oracle consume the exact tensors made here.  The
distribution families follow the quality study the codec comes from (D'Alberto,
"Statistical Inference and Quality Measures of KV Cache Quantisations Inspired
by TurboQuant", gist.science summary, "Results": Gaussian, heavy-tailed and
low-rank keys), and the per-channel outlier structure of real key caches
("Your KV cache is not a bit problem but a geometry problem", "Keys: outliers
live in fixed channels").  No dataset or trained weight is involved.

The sketch matrix S (the random numbers the QJL sketch draws) is also an input:
iid N(0,1), rounded to bfloat16, row-major [m][d]; so are the random rotations
(the sign diagonal of a randomized Hadamard transform, a Haar rotation in SO(d)).
"""
from __future__ import annotations

from dataclasses import dataclass, field

import torch


def _gen(seed: int, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    return g


def gaussian(shape, seed: int, dtype=torch.bfloat16, device="cpu") -> torch.Tensor:
    """iid N(0,1) in fp32, then cast (round to nearest even) to ``dtype``."""
    x = torch.randn(*shape, generator=_gen(seed, device), device=device, dtype=torch.float32)
    return x.to(dtype)


def lowrank_heavytail_keys(B, H, N, d, seed: int, rank: int = 8, noise: float = 0.1,
                           df: int = 3, dtype=torch.bfloat16, device="cpu") -> torch.Tensor:
    """K[b,h] = (U W^T + noise*E) diag(s):  U [N,rank], W [d,rank], E [N,d] iid N(0,1);
    s_c = |t_df| per channel (Student t drawn as Z / sqrt(chi2_df / df)), fixed
    across tokens of one (b,h).  Generated one (b,h) at a time to bound memory."""
    g = _gen(seed, device)
    out = torch.empty(B, H, N, d, dtype=dtype, device=device)
    for b in range(B):
        for h in range(H):
            U = torch.randn(N, rank, generator=g, device=device)
            W = torch.randn(d, rank, generator=g, device=device)
            E = torch.randn(N, d, generator=g, device=device)
            z = torch.randn(d, generator=g, device=device)
            chi2 = torch.randn(df, d, generator=g, device=device).square().sum(0)
            s = (z / torch.sqrt(chi2 / df)).abs()
            out[b, h] = ((U @ W.T + noise * E) * s).to(dtype)
    return out


def sketch_bf16(m: int, d: int, seed: int = 7) -> torch.Tensor:
    """Gaussian sketch S [m][d], iid N(0,1) rounded to bf16 (CPU tensor)."""
    return gaussian((m, d), seed, torch.bfloat16, "cpu")


def rotation_signs(d: int, seed: int = 13):
    """Random diagonal of the randomized Hadamard rotation: d fair coin flips
    as 8 little-endian uint32 words (bit i set: coordinate i negated; bits at
    and beyond d zero)."""
    import numpy as np
    g = _gen(seed, "cpu")
    bits = torch.randint(0, 2, (d,), generator=g).numpy().astype(np.uint64)
    w = np.zeros(8, np.uint32)
    for i in range(d):
        w[i // 32] |= np.uint32(int(bits[i]) << (i % 32))
    return w


def rotation_qr(d: int, seed: int = 17):
    """A random rotation in SO(d) as fp32 [d][d]: QR of a Gaussian matrix
    (LAPACK via torch, fp64), columns scaled by sign(R_kk), first column
    negated when the determinant is -1, rounded to fp32."""
    g = _gen(seed, "cpu")
    A = torch.randn(d, d, generator=g, dtype=torch.float64)
    Q, R = torch.linalg.qr(A)
    Q = Q * torch.sign(torch.diagonal(R))[None, :]
    if torch.linalg.det(Q) < 0:
        Q[:, 0] = -Q[:, 0]
    return Q.to(torch.float32).numpy()


def bits_u16(t: torch.Tensor):
    """bf16 tensor -> numpy uint16 bit patterns (CPU copy)."""
    import numpy as np
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


@dataclass(frozen=True)
class Workload:
    name: str
    scheme: str
    n_bits: int
    B: int
    Hq: int
    Hkv: int
    d: int
    N: int
    dtype: torch.dtype
    keys: str            # "gaussian" | "lowrank_heavytail"
    chunk: int = 0       # prefill chunk (0 = whole context at once)
    decode_steps: int = 1
    seed: int = 0
    extra: dict = field(default_factory=dict)


# The five workloads (sizes as stated for the method's evaluation grid).
WORKLOADS = {
    "tiny_single_head": Workload("tiny_single_head", "KQV", 4, 1, 1, 1, 64, 256,
                                 torch.float32, "gaussian", seed=1001),
    "one_layer_decode": Workload("one_layer_decode", "KQV", 4, 1, 32, 32, 128, 4096,
                                 torch.bfloat16, "gaussian", seed=1002),
    "llama_gqa_decode": Workload("llama_gqa_decode", "KQV", 4, 16, 32, 8, 128, 32768,
                                 torch.bfloat16, "lowrank_heavytail", seed=1003),
    "bit_budget_sweep": Workload("bit_budget_sweep", "KQV", 4, 8, 8, 8, 128, 16384,
                                 torch.bfloat16, "gaussian", seed=1004),
    "long_context": Workload("long_context", "KQV", 4, 4, 32, 8, 128, 131072,
                             torch.bfloat16, "lowrank_heavytail", chunk=8192,
                             decode_steps=64, seed=1005),
}


def make_kvq(w: Workload, device="cpu", N: int | None = None, B: int | None = None):
    """(K, V, q) for a workload, optionally truncated to N tokens / B batch rows.
    K, V: [B][Hkv][N][d]; q: [B][Hq][d]."""
    N = w.N if N is None else N
    B = w.B if B is None else B
    if w.keys == "gaussian":
        K = gaussian((B, w.Hkv, N, w.d), w.seed * 10 + 1, w.dtype, device)
    else:
        K = lowrank_heavytail_keys(B, w.Hkv, N, w.d, w.seed * 10 + 1, dtype=w.dtype, device=device)
    V = gaussian((B, w.Hkv, N, w.d), w.seed * 10 + 2, w.dtype, device)
    q = gaussian((B, w.Hq, w.d), w.seed * 10 + 3, w.dtype, device)
    return K, V, q
