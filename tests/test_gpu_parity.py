"""GPU (HIP, through the C ABI) against the CPU oracle on the same seeded inputs.

Codes, norms, residual norms and sign bits: bit for bit.  Reconstructed vectors
and attention outputs: per vector / per (b, query head) relative error within
1e-5 for fp32 inputs and 2e-3 * ||o|| for bf16 inputs (the stated tolerances).
Sizes span several encoder tiles (32 or 64 tokens) with a ragged tail.
"""
import numpy as np
import pytest
import torch

from kv_cache_quantization_kqv_amd import synth
from oracle import ref
from parity_util import Pair, host_bits, rel_rows, v_sign_records

pytestmark = pytest.mark.gpu

SCHEME_BITS = [("KV", 1), ("KV", 2), ("KV", 3), ("KV", 4), ("KQV", 2), ("KQV", 3), ("KQV", 4),
               ("QKQV", 2), ("QKQV", 3), ("QKQV", 4)]
TOL = {torch.float32: 1e-5, torch.bfloat16: 2e-3}


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    torch.cuda.init()


def _inputs(B, H, T, d, dtype, seed, heavy=False):
    if heavy:
        K = synth.lowrank_heavytail_keys(B, H, T, d, seed, dtype=dtype)
    else:
        K = synth.gaussian((B, H, T, d), seed, dtype) * 3
    V = synth.gaussian((B, H, T, d), seed + 1, dtype)
    return K.to(dtype), V.to(dtype)


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16], ids=["f32", "bf16"])
@pytest.mark.parametrize("d", [8, 16, 32, 64, 128, 256])
@pytest.mark.parametrize("scheme,n", SCHEME_BITS, ids=[f"{s}{n}" for s, n in SCHEME_BITS])
def test_quantize_bit_exact(scheme, n, d, dtype):
    print(f"case quantize {scheme}{n} d={d} {dtype}", flush=True)
    B, H, T, t0, cap = 2, 3, 77, 5, 90
    P = Pair(scheme, n, d, B, H, cap)
    K, V = _inputs(B, H, T, d, dtype, 100 + d + n, heavy=(scheme != "KV"))
    P.write(K, V, t0)
    torch.cuda.synchronize()
    P.assert_bit_exact()


# Encoders walk tiles in a persistent-style grid (one or two rounds of resident
# blocks), so a wave takes a second tile only past 4 waves x 256 CUs x 3 blocks
# (the most any encoder keeps resident) = 3072 tiles.  These inputs have 6400
# tiles (32 or 64 tokens each) and so run the prefetch / stash loop over many
# tiles per wave, for each input type, rotation and bucketize kind.
MULTI_TILE = [("KQV", 4, 128, torch.bfloat16, "wht"), ("KQV", 4, 128, torch.float32, "wht"),
              ("KQV", 4, 128, torch.bfloat16, "rht"), ("KQV", 4, 128, torch.float32, "qr"),
              ("KV", 2, 128, torch.bfloat16, "wht"), ("KV", 4, 128, torch.float32, "wht"),
              ("QKQV", 3, 128, torch.float32, "wht"), ("KQV", 4, 64, torch.float32, "wht"),
              ("KQV", 2, 64, torch.bfloat16, "rht"), ("QKQV", 3, 64, torch.bfloat16, "qr"),
              ("KV", 2, 64, torch.float32, "wht"), ("QKQV", 3, 256, torch.float32, "qr")]


@pytest.mark.parametrize("scheme,n,d,dtype,rotation", MULTI_TILE,
                         ids=[f"{s}{n}-d{d}-{'bf16' if t == torch.bfloat16 else 'f32'}-{r}"
                              for s, n, d, t, r in MULTI_TILE])
def test_quantize_bit_exact_many_tiles_per_wave(scheme, n, d, dtype, rotation):
    # tokens per tile: 64 / lanes per vector (one lane per vector for the dense
    # rotation below d = 256, a lane pair at 256)
    vt = {128: 32 if rotation != "qr" else 64, 256: 32}.get(d, 64)
    B, H, t0 = 4, 8, 5
    T = 6400 // 32 * vt - t0                      # 200 tiles per (batch row, head)
    print(f"case quantize-many-tiles {scheme}{n} d={d} {dtype} {rotation} T={T}", flush=True)
    P = Pair(scheme, n, d, B, H, T + t0 + 11, rotation=rotation)
    K, V = _inputs(B, H, T, d, dtype, 2100 + d + n, heavy=(scheme != "KV"))
    P.write(K, V, t0)
    torch.cuda.synchronize()
    P.assert_bit_exact()


@pytest.mark.parametrize("d", [8, 64, 128, 256])
@pytest.mark.parametrize("scheme,n", [("KV", 4), ("KQV", 4), ("KQV", 2), ("QKQV", 3)])
def test_dequantize_matches_oracle(scheme, n, d):
    print(f"case dequantize {scheme}{n} d={d}", flush=True)
    B, H, T, cap = 2, 2, 70, 70
    P = Pair(scheme, n, d, B, H, cap)
    K, V = _inputs(B, H, T, d, torch.float32, 300 + d)
    P.write(K, V, 0)
    for which, oc in ((0, P.ok), (1, P.ov)):
        got = P.gpu.dequantize(which, 3, 60).cpu().numpy()
        want = oc.dequantize(3, 60, P.S, nthreads=8)
        err = rel_rows(got, want)
        assert err.max() < 1e-5, (which, err.max())


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16], ids=["f32", "bf16"])
@pytest.mark.parametrize("d", [8, 32, 64, 128, 256])
@pytest.mark.parametrize("scheme,n", [("KV", 2), ("KV", 4), ("KQV", 2), ("KQV", 3), ("KQV", 4),
                                      ("QKQV", 2), ("QKQV", 4)])
def test_decode_matches_oracle(scheme, n, d, dtype):
    print(f"case decode {scheme}{n} d={d} {dtype}", flush=True)
    B, Hkv, G, N = 2, 2, 2, 300
    P = Pair(scheme, n, d, B, Hkv, N + 3)
    K, V = _inputs(B, Hkv, N, d, dtype, 500 + d + n, heavy=True)
    P.write(K, V, 0)
    q = synth.gaussian((B, Hkv * G, d), 900 + d, dtype)
    want = P.attention(q, N)
    for splits in (0, 1, 7):
        got = P.gpu.decode_attention(q.cuda(), N, splits=splits).cpu().numpy()
        err = rel_rows(got, want)
        assert err.max() < TOL[dtype], (splits, err.max())


@pytest.mark.parametrize("G", [1, 2, 4, 8])
def test_decode_gqa_ratios(G):
    print(f"case gqa G={G}", flush=True)
    B, Hkv, d, N = 2, 2, 128, 517
    P = Pair("KQV", 4, d, B, Hkv, N)
    K, V = _inputs(B, Hkv, N, d, torch.bfloat16, 700 + G, heavy=True)
    P.write(K, V, 0)
    q = synth.gaussian((B, Hkv * G, d), 800 + G, torch.bfloat16)
    want = P.attention(q, N)
    got = P.gpu.decode_attention(q.cuda(), N).cpu().numpy()
    assert rel_rows(got, want).max() < 2e-3
    # same cache, fp32 query.  K and V are bf16 inputs (stated tolerance 2e-3);
    # the heavy-tailed keys give scores of magnitude ~1e2, where fp32 score
    # rounding alone moves softmax weights by ~1e-5 relative, so check 1e-4.
    qf = q.float()
    got = P.gpu.decode_attention(qf.cuda(), N).cpu().numpy()
    assert rel_rows(got, P.attention(qf, N)).max() < 1e-4


def test_tiny_single_head_workload():
    """d=64, N=256, one head, fp32 K, V, q ~ N(0,1); KQV n=4 (K 4-bit after WHT;
    V 3-bit + 1-bit sketch, S 64x64); quantize both, one decode step."""
    w = synth.WORKLOADS["tiny_single_head"]
    K, V, q = synth.make_kvq(w)
    P = Pair(w.scheme, w.n_bits, w.d, w.B, w.Hkv, w.N)
    P.write(K, V, 0)
    torch.cuda.synchronize()
    P.assert_bit_exact()
    got = P.gpu.decode_attention(q.cuda(), w.N).cpu().numpy()
    assert rel_rows(got, P.attention(q, w.N)).max() < 1e-5


def test_chunked_and_token_appends_equal_one_shot():
    """Per-token append ("Systems tax": quantise each arriving token, nothing else
    moves): chunked and single-token writes give the same bytes as one write."""
    B, H, d, T = 2, 2, 128, 150
    K, V = _inputs(B, H, T, d, torch.bfloat16, 41, heavy=True)
    one = Pair("KQV", 4, d, B, H, T)
    one.write(K, V, 0)
    many = Pair("KQV", 4, d, B, H, T)
    for t0, t1 in [(0, 64), (64, 100), (100, 147)]:
        many.gpu.quantize_k(K[:, :, t0:t1].cuda(), t0)
        many.gpu.quantize_v(V[:, :, t0:t1].cuda(), t0)
    for t in range(147, T):
        many.gpu.quantize_k(K[:, :, t:t + 1].cuda(), t)
        many.gpu.quantize_v(V[:, :, t:t + 1].cuda(), t)
    for name in one.gpu.bufs:
        assert torch.equal(one.gpu.bufs[name], many.gpu.bufs[name]), name
    one.assert_bit_exact()


def test_strided_and_offset_input():
    B, H, T, d = 2, 3, 70, 64
    base = synth.gaussian((B, T, H, d), 51, torch.bfloat16)
    Kv = base.permute(0, 2, 1, 3)                  # [B][H][T][d] view, token stride H*d
    V = synth.gaussian((B, H, T, d), 52, torch.bfloat16)
    P = Pair("QKQV", 4, d, B, H, T + 10)
    P.gpu.quantize_k(base.cuda().permute(0, 2, 1, 3), 10)
    P.gpu.quantize_v(V.cuda(), 10)
    P.ok.quantize(synth.bits_u16(Kv.contiguous()), 10, P.S)
    P.ov.quantize(synth.bits_u16(V), 10, P.S)
    torch.cuda.synchronize()
    P.assert_bit_exact()


def test_sign_fixup_rows():
    """Sketch rows that are zero give z = 0 exactly: the certified-sign test fails
    and the fp64 recomputation must set the bit (ties -> 1); negated duplicate
    rows must give complementary bits."""
    d = 128
    S = synth.sketch_bf16(d, d, 9).clone()
    S[0:8] = 0
    S[8:16] = -S[16:24]
    e = torch.zeros(8, d, dtype=torch.bfloat16)
    for i in range(8):
        e[i, i] = 1
    S[24:32] = e                                   # z_k = r~_k exactly
    B, H, T = 1, 2, 96
    K, V = _inputs(B, H, T, d, torch.float32, 61)
    V[0, 0, :5] = 0                                # zero vectors
    P = Pair("QKQV", 3, d, B, H, T, S=S)
    P.write(K, V, 0)
    torch.cuda.synchronize()
    P.assert_bit_exact()
    sg = v_sign_records(P)
    assert np.all(sg[..., 0] == 0xFF)              # rows 0..7 are zero -> bit 1
    assert np.all(P.gpu.view("k_signs").cpu().numpy()[..., 0] == 0xFF)


def test_sign_exact_cancellation():
    """Sketch rows e_2j - e_2j+1 against residuals whose coordinates 2j and
    2j+1 are equal: S r~ is exactly zero, neither the MFMA sum nor the lanes'
    fp32 sum can decide, and the ascending fp64 sum (+0, bit 1) must."""
    d, B, H, T = 128, 1, 2, 70
    Hm = torch.tensor([[1.0]])
    while Hm.shape[0] < d:
        Hm = torch.cat([torch.cat([Hm, Hm], 1), torch.cat([Hm, -Hm], 1)], 0)
    g = torch.Generator().manual_seed(91)
    y = torch.randint(-40, 41, (B, H, T, d // 2), generator=g).double().repeat_interleave(2, -1)
    x = (y @ Hm.double()) / d                       # WHT of x is y, exactly, in fp32
    V = x.float()
    assert torch.equal(V.double(), x)
    S = synth.sketch_bf16(d, d, 12).clone()
    for j in range(d // 2):
        S[j] = 0
        S[j, 2 * j], S[j, 2 * j + 1] = 1, -1
    K = synth.gaussian((B, H, T, d), 92, torch.float32)
    P = Pair("KQV", 4, d, B, H, T, S=S)
    P.write(K, V, 0)
    torch.cuda.synchronize()
    P.assert_bit_exact()
    sg = v_sign_records(P)[:, :, :T]
    assert np.all(sg[..., : d // 16] == 0xFF)      # rows 0..63: z = 0 exactly -> bit 1


def test_zero_and_large_vectors():
    B, H, T, d = 1, 1, 40, 128
    K = torch.zeros(B, H, T, d)
    K[0, 0, 10:20] = synth.gaussian((10, d), 71, torch.float32) * 1e4   # norms beyond fp16 range
    V = synth.gaussian((B, H, T, d), 72, torch.float32)
    V[0, 0, :8] = 0
    P = Pair("KQV", 4, d, B, H, T)
    P.write(K, V, 0)
    torch.cuda.synchronize()
    P.assert_bit_exact()
    kn = P.gpu.view("k_norm").cpu().numpy().view(np.uint16)
    assert np.all(kn[0, 0, :10] == 0) and np.all(kn[0, 0, 10:20] == 0x7C00)


def test_single_token_context():
    B, H, d = 2, 2, 64
    K, V = _inputs(B, H, 4, d, torch.float32, 81)
    P = Pair("KQV", 4, d, B, H, 4)
    P.write(K, V, 0)
    q = synth.gaussian((B, H, d), 82, torch.float32)
    got = P.gpu.decode_attention(q.cuda(), 1).cpu().numpy()
    want = P.attention(q, 1)
    assert rel_rows(got, want).max() < 1e-5
    vh = P.gpu.dequantize(1, 0, 1).cpu().numpy()[:, :, 0]
    assert np.allclose(got, vh, rtol=1e-5, atol=1e-6)   # o = v^_1


@pytest.mark.parametrize("d", [8, 16, 32, 64, 128, 256])
@pytest.mark.parametrize("splits", [0, 3])
def test_decode_full_capacity_ragged_tail(d, splits):
    """n_ctx equal to the capacity with value records that are not 16-byte
    multiples (3-bit codes at d <= 64): the last value piece of the last split
    ends inside a 16-byte piece at the very end of the buffers."""
    print(f"case full-capacity tail d={d} splits={splits}", flush=True)
    B, Hkv, G, N = 2, 2, 4, (301 if d < 128 else 304)    # d = 128: whole 16-slot blocks
    P = Pair("KQV", 4, d, B, Hkv, N)
    K, V = _inputs(B, Hkv, N, d, torch.float32, 910 + d, heavy=True)
    P.write(K, V, 0)
    q = synth.gaussian((B, Hkv * G, d), 920 + d, torch.float32)
    got = P.gpu.decode_attention(q.cuda(), N, splits=splits).cpu().numpy()
    assert rel_rows(got, P.attention(q, N)).max() < 1e-5


WINDOW_CASES = {
    # name: (t_begin, t_end, window = list of (first, count) slices of the inputs)
    "recent128": (0, 572, [(572, 128)]),
    "sinks4_recent64": (4, 636, [(0, 4), (636, 64)]),
    "window_only": (0, 0, [(0, 300)]),
    "no_window_offset": (7, 700, []),
}


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16], ids=["f32", "bf16"])
@pytest.mark.parametrize("case", list(WINDOW_CASES))
@pytest.mark.parametrize("d", [8, 64, 128, 256])
@pytest.mark.parametrize("scheme,n", [("KQV", 4), ("KV", 3), ("QKQV", 2)])
def test_decode_window_matches_oracle(scheme, n, d, case, dtype):
    """Compressed slots [t_begin, t_end) plus full-precision sink and recent
    tokens (the exact inputs of those positions) in one softmax."""
    print(f"case window {scheme}{n} d={d} {case} {dtype}", flush=True)
    B, Hkv, G, N = 2, 2, 4, 700
    t_begin, t_end, win = WINDOW_CASES[case]
    P = Pair(scheme, n, d, B, Hkv, N)
    K, V = _inputs(B, Hkv, N, d, dtype, 1100 + d + n, heavy=True)
    P.write(K, V, 0)
    q = synth.gaussian((B, Hkv * G, d), 1200 + d, dtype)
    wk = torch.cat([K[:, :, a:a + c] for a, c in win], 2).contiguous() if win else None
    wv = torch.cat([V[:, :, a:a + c] for a, c in win], 2).contiguous() if win else None
    want = P.attention_window(q, t_begin, t_end, wk, wv)
    for splits in (0, 5):
        got = P.gpu.decode_attention_window(
            q.cuda(), t_begin, t_end, None if wk is None else wk.cuda(),
            None if wv is None else wv.cuda(), splits=splits).cpu().numpy()
        err = rel_rows(got, want)
        assert err.max() < TOL[dtype], (splits, err.max())


@pytest.mark.parametrize("G", [1, 2, 8])
def test_decode_window_gqa_and_largest_window(G):
    """Largest window (4096 tokens) with a short compressed range, fp32 query
    over bf16 inputs, every supported head grouping."""
    print(f"case window-max G={G}", flush=True)
    B, Hkv, d, N, W = 1, 2, 128, 300, 4096
    P = Pair("KQV", 4, d, B, Hkv, N)
    K, V = _inputs(B, Hkv, N, d, torch.bfloat16, 1300 + G)
    P.write(K, V, 0)
    wk = synth.gaussian((B, Hkv, W, d), 1310 + G, torch.bfloat16)
    wv = synth.gaussian((B, Hkv, W, d), 1320 + G, torch.bfloat16)
    q = synth.gaussian((B, Hkv * G, d), 1330 + G, torch.float32)
    got = P.gpu.decode_attention_window(q.cuda(), 11, 290, wk.cuda(), wv.cuda()).cpu().numpy()
    assert rel_rows(got, P.attention_window(q, 11, 290, wk, wv)).max() < 1e-5


def test_decode_window_equals_plain_decode_when_empty():
    """n_win = 0 over slots [0, n) is the plain decode entry point, bit for bit
    (same kernels, no window partial)."""
    B, Hkv, G, d, N = 2, 2, 4, 128, 513
    P = Pair("KQV", 4, d, B, Hkv, N)
    K, V = _inputs(B, Hkv, N, d, torch.float32, 1400, heavy=True)
    P.write(K, V, 0)
    q = synth.gaussian((B, Hkv * G, d), 1401, torch.float32).cuda()
    a = P.gpu.decode_attention(q, N, splits=3)
    b = P.gpu.decode_attention_window(q, 0, N, splits=3)
    assert torch.equal(a, b)


ROT_SCHEMES = [("KQV", 4), ("KQV", 2), ("QKQV", 3), ("QKQV", 2)]


ROT_CASES = [(d, r) for d in (8, 16, 32, 64, 128, 256) for r in ("rht", "qr")]


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16], ids=["f32", "bf16"])
@pytest.mark.parametrize("d,rotation", ROT_CASES, ids=[f"{r}-d{d}" for d, r in ROT_CASES])
@pytest.mark.parametrize("scheme,n", ROT_SCHEMES, ids=[f"{s}{n}" for s, n in ROT_SCHEMES])
def test_quantize_bit_exact_rotations(scheme, n, d, dtype, rotation):
    """Randomized Hadamard and dense SO(d) rotations ("KVQuant++" thread,
    "Entropy coding", "Rotation invariance guarantee"): codes, norms and sign
    bits bit for bit, over several tiles with a ragged tail."""
    print(f"case quantize-rot {rotation} {scheme}{n} d={d} {dtype}", flush=True)
    B, H, T, t0, cap = 2, 3, 141, 5, 150
    P = Pair(scheme, n, d, B, H, cap, rotation=rotation)
    K, V = _inputs(B, H, T, d, dtype, 1500 + d + n, heavy=True)
    P.write(K, V, t0)
    torch.cuda.synchronize()
    P.assert_bit_exact()


@pytest.mark.parametrize("d,rotation", [(32, "rht"), (32, "qr"), (128, "rht"), (128, "qr"),
                                        (8, "rht"), (8, "qr"), (256, "rht"), (256, "qr")])
def test_dequantize_and_decode_rotations(rotation, d):
    print(f"case decode-rot {rotation} d={d}", flush=True)
    B, Hkv, G, N = 2, 2, 4, 333
    for scheme, n in (("KQV", 4), ("QKQV", 3)):
        P = Pair(scheme, n, d, B, Hkv, N, rotation=rotation)
        K, V = _inputs(B, Hkv, N, d, torch.float32, 1600 + d, heavy=True)
        P.write(K, V, 0)
        for which, oc in ((0, P.ok), (1, P.ov)):
            got = P.gpu.dequantize(which, 2, 300).cpu().numpy()
            assert rel_rows(got, oc.dequantize(2, 300, P.S, nthreads=8)).max() < 1e-5
        q = synth.gaussian((B, Hkv * G, d), 1700 + d, torch.float32)
        want = P.attention(q, N)
        for splits in (0, 3):
            got = P.gpu.decode_attention(q.cuda(), N, splits=splits).cpu().numpy()
            assert rel_rows(got, want).max() < 1e-5, (scheme, splits)
        qb = q.to(torch.bfloat16)
        got = P.gpu.decode_attention(qb.cuda(), N).cpu().numpy()
        assert rel_rows(got, P.attention(qb, N)).max() < 1e-5
        # with a full-precision window as well
        wk, wv = K[:, :, 300:].contiguous(), V[:, :, 300:].contiguous()
        got = P.gpu.decode_attention_window(q.cuda(), 0, 300, wk.cuda(), wv.cuda()).cpu().numpy()
        assert rel_rows(got, P.attention_window(q, 0, 300, wk, wv)).max() < 1e-5


PREFILL_SCHEMES = [("KV", 4), ("KV", 2), ("KQV", 4), ("KQV", 3), ("KQV", 2), ("QKQV", 3),
                   ("QKQV", 2)]


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16], ids=["f32", "bf16"])
@pytest.mark.parametrize("d,G", [(8, 2), (16, 2), (32, 4), (64, 1), (128, 4), (128, 8), (256, 4)])
@pytest.mark.parametrize("scheme,n", PREFILL_SCHEMES, ids=[f"{s}{n}" for s, n in PREFILL_SCHEMES])
def test_prefill_matches_oracle(scheme, n, d, G, dtype):
    """Chunked prefill: a chunk of 37 query tokens at positions 150..186 over a
    cache of 187 slots, causal; and the same queries non-causally over every
    slot.  Rows span several 64-row tiles and the token range several 64-token
    tiles with ragged ends."""
    print(f"case prefill {scheme}{n} d={d} G={G} {dtype}", flush=True)
    B, Hkv, nq, p0 = 2, 2, 37, 150
    N = p0 + nq
    P = Pair(scheme, n, d, B, Hkv, N + 5)
    K, V = _inputs(B, Hkv, N, d, dtype, 1800 + d + n, heavy=True)
    P.write(K, V, 0)
    q = synth.gaussian((B, nq, Hkv * G, d), 1900 + d + G, dtype)
    for causal in (True, False):
        got = P.gpu.prefill_attention(q.cuda(), p0, N, causal=causal).cpu().numpy()
        err = rel_rows(got, P.prefill(q, p0, causal, N))
        assert err.max() < TOL[dtype], (causal, err.max())


@pytest.mark.parametrize("d", [8, 32, 64, 256])
@pytest.mark.parametrize("rotation", ["rht", "qr"])
def test_prefill_rotations_other_dims(rotation, d):
    """The multi-query path under both rotation variants away from d = 128
    (query rotation, the tile or small kernels, the finish's rotation back; at
    d = 256 the lane-pair dense encoder)."""
    print(f"case prefill-rot d={d} {rotation}", flush=True)
    B, Hkv, G, nq, p0 = 1, 2, 2, 21, 110
    N = p0 + nq
    for scheme, n in (("KQV", 4), ("QKQV", 3)):
        P = Pair(scheme, n, d, B, Hkv, N, rotation=rotation)
        K, V = _inputs(B, Hkv, N, d, torch.float32, 2050, heavy=True)
        P.write(K, V, 0)
        q = synth.gaussian((B, nq, Hkv * G, d), 2051, torch.float32)
        for causal in (True, False):
            got = P.gpu.prefill_attention(q.cuda(), p0, N, causal=causal).cpu().numpy()
            assert rel_rows(got, P.prefill(q, p0, causal, N)).max() < 1e-5, (scheme, causal)


@pytest.mark.parametrize("rotation", ["rht", "qr"])
def test_prefill_rotations_and_short_chunks(rotation):
    """Rotation variants; a single-token chunk (equals decode over the same
    slots); a chunk at the start of the cache (first row sees one slot)."""
    print(f"case prefill-rot {rotation}", flush=True)
    B, Hkv, G, d, N = 1, 2, 4, 128, 200
    P = Pair("KQV", 4, d, B, Hkv, N, rotation=rotation)
    K, V = _inputs(B, Hkv, N, d, torch.float32, 2000, heavy=True)
    P.write(K, V, 0)
    q = synth.gaussian((B, 70, Hkv * G, d), 2001, torch.float32)
    got = P.gpu.prefill_attention(q.cuda(), 0, N, causal=True).cpu().numpy()
    assert rel_rows(got, P.prefill(q, 0, True, N)).max() < 1e-5
    q1 = q[:, :1].contiguous()
    one = P.gpu.prefill_attention(q1.cuda(), N - 1, N, causal=True)[:, 0]
    dec = P.gpu.decode_attention(q1[:, 0].contiguous().cuda(), N)
    assert rel_rows(one.cpu().numpy(), dec.cpu().numpy().astype(np.float64)).max() < 1e-5


# (t_begin, t_end, window token runs taken from the exact inputs), over a
# 187-slot cache: sinks and recent tokens exact next to a compressed middle, a
# window alone, a compressed range from an offset inside a 16-slot block
PREFILL_WINDOW_CASES = {"recent": (0, 123, [(123, 64)]),
                        "sinks": (4, 150, [(0, 4), (150, 37)]),
                        "window_only": (150, 150, [(0, 4), (102, 48)]),
                        "offset": (21, 187, [])}


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16], ids=["f32", "bf16"])
@pytest.mark.parametrize("case", list(PREFILL_WINDOW_CASES))
@pytest.mark.parametrize("d", [8, 64, 128, 256])
@pytest.mark.parametrize("scheme,n", [("KQV", 4), ("QKQV", 3), ("KV", 2)])
def test_prefill_window_matches_oracle(scheme, n, d, case, dtype):
    """Multi-query attention with a full-precision window: a chunk of 37 query
    tokens at positions 150..186 over compressed slots [t_begin, t_end) (only
    those up to each query's position when causal) plus window tokens that
    every query sees, in one softmax per row."""
    print(f"case prefill-window {scheme}{n} d={d} {case} {dtype}", flush=True)
    B, Hkv, G, nq, p0 = 2, 2, 4, 37, 150
    N = p0 + nq
    t_begin, t_end, win = PREFILL_WINDOW_CASES[case]
    P = Pair(scheme, n, d, B, Hkv, N + 5)
    K, V = _inputs(B, Hkv, N, d, dtype, 2300 + d + n, heavy=True)
    P.write(K, V, 0)
    q = synth.gaussian((B, nq, Hkv * G, d), 2400 + d, dtype)
    wk = torch.cat([K[:, :, a:a + c] for a, c in win], 2).contiguous() if win else None
    wv = torch.cat([V[:, :, a:a + c] for a, c in win], 2).contiguous() if win else None
    for causal in (True, False):
        want = ref.prefill_attention_window(P.ok, P.ov, host_bits(q), p0, causal, t_begin, t_end,
                                            None if wk is None else host_bits(wk),
                                            None if wv is None else host_bits(wv), P.S, 8)
        got = P.gpu.prefill_attention_window(
            q.cuda(), p0, t_begin, t_end, None if wk is None else wk.cuda(),
            None if wv is None else wv.cuda(), causal=causal).cpu().numpy()
        err = rel_rows(got, want)
        assert err.max() < TOL[dtype], (causal, err.max())


def test_prefill_window_empty_equals_plain_prefill():
    """No window over [0, n): bit for bit the plain multi-query call."""
    B, Hkv, G, nq, p0, d = 2, 2, 4, 37, 150, 128
    N = p0 + nq
    P = Pair("KQV", 4, d, B, Hkv, N + 5)
    K, V = _inputs(B, Hkv, N, d, torch.bfloat16, 2500, heavy=True)
    P.write(K, V, 0)
    q = synth.gaussian((B, nq, Hkv * G, d), 2501, torch.bfloat16).cuda()
    a = P.gpu.prefill_attention(q, p0, N, causal=True)
    b = P.gpu.prefill_attention_window(q, p0, 0, N, causal=True)
    assert torch.equal(a, b)


@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("scheme,n", [("KQV", 4), ("QKQV", 2), ("KV", 3)])
def test_prefill_token_splits(scheme, n, causal):
    """Few query rows over a long cache: the library splits the slots (here
    several splits of a multiple of 64 slots with a ragged last split), and
    the finish merges them; rows whose causal limit ends inside an early split
    leave later splits empty."""
    print(f"case prefill-splits {scheme}{n} causal={causal}", flush=True)
    B, Hkv, G, d, N, nq = 1, 2, 2, 64, 1900, 9
    P = Pair(scheme, n, d, B, Hkv, N)
    K, V = _inputs(B, Hkv, N, d, torch.float32, 2100 + n, heavy=True)
    P.write(K, V, 0)
    q = synth.gaussian((B, nq, Hkv * G, d), 2101, torch.float32)
    for p0 in (0, 700, N - nq):
        got = P.gpu.prefill_attention(q.cuda(), p0, N, causal=causal).cpu().numpy()
        assert rel_rows(got, P.prefill(q, p0, causal, N)).max() < 1e-5, p0


@pytest.mark.parametrize("d", [8, 64, 128, 256])
def test_decode_stages_equal_one_call(d):
    """Prep, scan and merge launched by three staged calls give the one-call
    result bit for bit (same kernels, same workspace)."""
    from kv_cache_quantization_kqv_amd import kvq as _kvq
    print(f"case decode-stages d={d}", flush=True)
    B, Hkv, G, N = 2, 2, 4, 500
    P = Pair("KQV", 4, d, B, Hkv, N)
    K, V = _inputs(B, Hkv, N, d, torch.bfloat16, 1500 + d, heavy=True)
    P.write(K, V, 0)
    q = synth.gaussian((B, Hkv * G, d), 1501 + d, torch.bfloat16).cuda()
    ws = torch.zeros(P.gpu.workspace_bytes(Hkv * G, N, 3), dtype=torch.uint8, device="cuda")
    a = P.gpu.decode_attention(q, N, splits=3, workspace=ws).clone()
    out = torch.full_like(a, float("nan"))
    for st in (_kvq.KVQ_STAGE_PREP, _kvq.KVQ_STAGE_SCAN, _kvq.KVQ_STAGE_MERGE):
        P.gpu.decode_attention(q, N, splits=3, out=out, workspace=ws, stages=st)
    assert torch.equal(a, out)


def test_stream_read_probe_runs():
    from kv_cache_quantization_kqv_amd import kvq as _kvq
    buf = torch.ones(1 << 22, dtype=torch.uint8, device="cuda")
    out = torch.zeros(4, dtype=torch.int32, device="cuda")
    _kvq.kvq_probe_stream_read(buf.data_ptr(), buf.numel(), out.data_ptr(),
                               torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()

