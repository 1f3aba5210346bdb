"""The per-token serving step (append one token's K and V, then decode over the
grown context) captured as a HIP graph and replayed: the library launches only
kernels on the caller's stream (no allocation, no memset, no synchronization),
so the step is capturable.  Every replay, with eager work and synchronizations
between replays, must reproduce the eager step bit for bit (the kernels are
deterministic and the replayed step rewrites the same slot)."""
import numpy as np
import pytest
import torch

from kv_cache_quantization_kqv_amd import synth
from kv_cache_quantization_kqv_amd.kvq import KVQCache

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


@pytest.mark.parametrize("scheme,n,d,window", [("KQV", 4, 128, False), ("QKQV", 3, 64, False),
                                               ("KQV", 4, 128, True)])
def test_append_decode_step_graph_replays(scheme, n, d, window):
    print(f"case graph {scheme}{n} d={d} window={window}", flush=True)
    dev = torch.device("cuda", 0)
    B, Hkv, G, N = 2, 2, 4, 300
    S = synth.bits_u16(synth.sketch_bf16(d, d, 7))
    cache = KVQCache(scheme, n, d, B, Hkv, 320, S_bf16=S, device=dev)
    K = synth.lowrank_heavytail_keys(B, Hkv, N, d, 41, dtype=torch.bfloat16).to(dev)
    V = synth.gaussian((B, Hkv, N, d), 42, torch.bfloat16).to(dev)
    q = synth.gaussian((B, Hkv * G, d), 43, torch.bfloat16).to(dev)
    p = N - 1
    cache.quantize_k(K[:, :, :p], 0)
    cache.quantize_v(V[:, :, :p], 0)
    kt, vt = K[:, :, p:p + 1].contiguous(), V[:, :, p:p + 1].contiguous()
    wk, wv = K[:, :, p - 8:].contiguous(), V[:, :, p - 8:].contiguous()
    ws = torch.zeros(cache.workspace_bytes(Hkv * G, N), dtype=torch.uint8, device=dev)
    out = torch.empty(B, Hkv * G, d, dtype=torch.float32, device=dev)

    def step():
        cache.quantize_k(kt, p)
        cache.quantize_v(vt, p)
        if window:      # slots [0, p - 8) compressed, the last 9 tokens full precision
            cache.decode_attention_window(q, 0, p - 8, wk, wv, out=out, workspace=ws)
        else:
            cache.decode_attention(q, N, out=out, workspace=ws)

    step()                                   # eager step (also warms per-kernel lookups)
    torch.cuda.synchronize(dev)
    want = out.clone()
    codes = [cache.view(nm).clone() for nm in ("k_codes", "v_codes", "k_norm", "v_norm")]

    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    other = torch.empty_like(out)
    for r in range(4):
        out.fill_(float("nan"))
        ws.fill_(0xA5)                       # the graph must not rely on stale workspace
        g.replay()
        torch.cuda.synchronize(dev)
        assert torch.equal(out, want), f"replay {r}"
        for c, nm in zip(codes, ("k_codes", "v_codes", "k_norm", "v_norm")):
            assert torch.equal(cache.view(nm), c), (r, nm)
        # eager work between replays: a decode over a shorter context
        cache.decode_attention(q, N - 37, out=other)
        torch.cuda.synchronize(dev)
        assert np.isfinite(other.cpu().numpy()).all()
