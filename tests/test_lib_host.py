"""Host-side checks of libkvq that need no GPU: exported symbols, codebook and
sketch tables, layout sizes and argument validation (every case here fails
validation before any HIP call, so nothing is launched)."""
import ctypes as C
import math
import os
import re

import numpy as np
import pytest
from scipy import stats

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def K():
    from kv_cache_quantization_kqv_amd import kvq
    if not os.path.exists(kvq.LIB_PATH):
        from kv_cache_quantization_kqv_amd import _build
        _build.build()
    return kvq


def header_functions():
    text = open(os.path.join(ROOT, "include", "kvq.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(kvq_[a-z_0-9]+)\s*\(", text)))


def test_every_declared_symbol_is_exported(K):
    names = header_functions()
    assert len(names) >= 12
    lib = C.CDLL(K.LIB_PATH)
    for n in names:
        assert hasattr(lib, n), n
    assert set(K.EXPORTS) == set(names)
    assert K.lib().kvq_version().decode().startswith("libkvq")


@pytest.mark.parametrize("d", [3, 8, 16, 32, 64, 128, 256])
@pytest.mark.parametrize("bits", [1, 2, 3, 4])
def test_codebook_tables_equal_oracle_bit_for_bit(K, orc, d, bits):
    """The library's Lloyd-Max (Wallis-recurrence integrals) and the oracle's
    (Gauss-Legendre quadrature) are independent; their fp32 tables must agree."""
    cb = K.kvq_codebook_init(d, bits)
    c, t, _ = orc.codebook(d, bits)
    n = 1 << bits
    got_c = np.array(cb.centroid[:n], np.float32)
    got_t = np.array(cb.threshold[: n - 1], np.float32)
    assert np.array_equal(got_c.view(np.uint32), c.view(np.uint32)), (got_c - c)
    assert np.array_equal(got_t.view(np.uint32), t.view(np.uint32)), (got_t - t)
    assert cb.d == d and cb.bits == bits
    assert all(v == 0.0 for v in cb.centroid[n:]) and all(v == 0.0 for v in cb.threshold[n - 1:])


def test_codebook_errors(K):
    lib = K.lib()
    cb = K.kvq_codebook()
    assert lib.kvq_codebook_init(2, 2, C.byref(cb)) == 3
    assert lib.kvq_codebook_init(64, 0, C.byref(cb)) == 4
    assert lib.kvq_codebook_init(64, 5, C.byref(cb)) == 4
    assert lib.kvq_codebook_init(64, 2, None) == 1


def test_sketch_generator(K):
    S = K.kvq_sketch_init(7, 128, 128)
    assert np.array_equal(S, K.kvq_sketch_init(7, 128, 128))          # deterministic
    assert not np.array_equal(S, K.kvq_sketch_init(8, 128, 128))
    import torch
    vals = torch.from_numpy(S.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy().ravel()
    assert abs(vals.mean()) < 4 / math.sqrt(vals.size)
    assert abs(vals.var() - 1) < 0.03
    assert stats.kstest(vals, "norm").pvalue > 1e-4
    # rows are nearly orthogonal: S S^T / d ~ I
    Sm = vals.reshape(128, 128)
    G = Sm @ Sm.T / 128
    assert np.max(np.abs(np.diag(G) - 1)) < 0.5 and np.max(np.abs(G - np.diag(np.diag(G)))) < 0.5
    assert K.lib().kvq_sketch_init(1, 0, 4, None) == 1
    buf = np.zeros(4, np.uint16)
    assert K.lib().kvq_sketch_init(1, 0, 4, buf.ctypes.data) == 10


@pytest.mark.parametrize("scheme,n,want", [
    ("KV", 4, (4, 4, 0, 0, 0)), ("KQV", 4, (4, 3, 0, 1, 1)), ("QKQV", 4, (3, 3, 1, 1, 1)),
    ("KV", 1, (1, 1, 0, 0, 0)), ("KQV", 2, (2, 1, 0, 1, 1)), ("QKQV", 2, (1, 1, 1, 1, 1))])
def test_cache_init_and_layout(K, scheme, n, want):
    c = K.kvq_cache_init(K.SCHEMES[scheme], n, 128, 2, 3, 48)
    assert (c.k_bits, c.v_bits, c.k_qjl, c.v_qjl, c.rotate) == want
    sizes = K.kvq_cache_layout(K.SCHEMES[scheme], n, 128, 2, 3, 48)
    rec = 2 * 3 * 48
    kb, vb, kq, vq, _ = want
    assert sizes == [rec * 128 * kb // 8, rec * 16 * kq, rec * 2, rec * 2 * kq,
                     rec * 128 * vb // 8, rec * 16 * vq, rec * 2, rec * 2 * vq]
    # KQV at n=4, d=128: 134 bytes per (token, KV head)
    if scheme == "KQV" and n == 4:
        assert sum(sizes) // rec == 134


def test_cache_init_errors(K):
    lib = K.lib()
    c = K.kvq_cache()
    assert lib.kvq_cache_init(C.byref(c), 9, 4, 128, 1, 1, 1) == 5
    assert lib.kvq_cache_init(C.byref(c), 1, 1, 128, 1, 1, 1) == 4   # KQV needs n >= 2
    assert lib.kvq_cache_init(C.byref(c), 0, 5, 128, 1, 1, 1) == 4
    assert lib.kvq_cache_init(C.byref(c), 1, 4, 96, 1, 1, 1) == 3
    assert lib.kvq_cache_init(C.byref(c), 1, 4, 512, 1, 1, 1) == 3
    assert lib.kvq_cache_init(C.byref(c), 1, 4, 4, 1, 1, 1) == 3
    assert lib.kvq_cache_init(C.byref(c), 1, 4, 256, 1, 1, 1) == 0
    assert lib.kvq_cache_init(C.byref(c), 1, 4, 8, 1, 1, 1) == 0
    assert lib.kvq_cache_init(C.byref(c), 1, 4, 128, 0, 1, 1) == 10
    # d = 128: the value side's token groups need whole 16-slot blocks
    assert lib.kvq_cache_init(C.byref(c), 1, 4, 128, 1, 1, 50) == 10
    assert lib.kvq_cache_init(C.byref(c), 1, 4, 128, 1, 1, 48) == 0
    assert lib.kvq_cache_init(C.byref(c), 1, 4, 64, 1, 1, 50) == 0


def _fake_cache(K, scheme="KQV", n=4, d=64, B=1, H=2, cap=32):
    """A cache struct with 16-B aligned (host) addresses; only used for calls that
    must fail validation, so the addresses are never dereferenced."""
    c = K.kvq_cache_init(K.SCHEMES[scheme], n, d, B, H, cap)
    addr = 0x10000
    for name in ["k_codes", "k_norm", "v_codes", "v_norm", "S"]:
        setattr(c, name, addr)
        addr += 0x10000
    if c.k_qjl:
        c.k_signs, c.k_rnorm = addr, addr + 0x10000
        addr += 0x20000
    if c.v_qjl:
        c.v_signs, c.v_rnorm = addr, addr + 0x10000
    return c


def test_validation_status_codes(K):
    lib = K.lib()
    c = _fake_cache(K)
    p = C.byref(c)
    src = 0x900000
    # quantize
    assert lib.kvq_quantize_k(None, src, 1, 0, 4, 0, 0, 64, None) == 1
    assert lib.kvq_quantize_k(p, None, 1, 0, 4, 0, 0, 64, None) == 1
    assert lib.kvq_quantize_k(p, src, 7, 0, 4, 0, 0, 64, None) == 8
    assert lib.kvq_quantize_k(p, src, 1, 30, 4, 0, 0, 64, None) == 6
    assert lib.kvq_quantize_k(p, src, 1, 0, 0, 0, 0, 64, None) == 10
    assert lib.kvq_quantize_k(p, src, 1, -1, 4, 0, 0, 64, None) == 10
    assert lib.kvq_quantize_v(p, src + 2, 1, 0, 4, 0, 0, 64, None) == 2
    assert lib.kvq_quantize_v(p, src, 1, 0, 4, 0, 0, 65, None) == 2     # 130-B rows
    # dequantize
    assert lib.kvq_dequantize(p, 0, 0, 4, None, None) == 1
    assert lib.kvq_dequantize(p, 2, 0, 4, 0x800000, None) == 10
    assert lib.kvq_dequantize(p, 0, 30, 4, 0x800000, None) == 6
    assert lib.kvq_dequantize(p, 0, 0, 4, 0x800004, None) == 2
    # decode
    ws = C.c_size_t()
    assert lib.kvq_decode_workspace(p, 3, 8, 0, C.byref(ws)) == 9
    assert lib.kvq_decode_workspace(p, 6, 8, 0, C.byref(ws)) == 9       # G = 3
    assert lib.kvq_decode_workspace(p, 2, -1, 0, C.byref(ws)) == 10
    assert lib.kvq_decode_workspace(p, 2, 0, 0, C.byref(ws)) == 0      # window-only sizing
    assert lib.kvq_decode_workspace(p, 2, 33, 0, C.byref(ws)) == 6
    assert lib.kvq_decode_workspace(p, 2, 8, 0, C.byref(ws)) == 0
    need = ws.value
    d, rows, splits = 64, 2, K.kvq_decode_auto_splits(c, 2, 8)
    assert splits >= 1
    # prepared queries, split partials, the window partial
    assert need == 4 * (rows * d * 2 + rows * splits * (2 + 2 * d) + rows * (2 + d))
    q, out, w = 0xA00000, 0xB00000, 0xC00000
    assert lib.kvq_decode_attention(p, q, 1, 2, 8, 0, out, w, need - 1, None) == 7
    assert lib.kvq_decode_attention(p, q, 1, 2, 8, 0, out, None, need, None) == 7
    assert lib.kvq_decode_attention(p, q, 3, 2, 8, 0, out, w, need, None) == 8
    assert lib.kvq_decode_attention(p, q + 4, 1, 2, 8, 0, out, w, need, None) == 2
    assert lib.kvq_decode_attention(p, None, 1, 2, 8, 0, out, w, need, None) == 1
    assert lib.kvq_decode_attention(p, q, 1, 2, 8, -1, out, w, need, None) == 10
    assert lib.kvq_decode_attention(p, q, 1, 2, 0, 0, out, w, need, None) == 10
    # decode with a full-precision window: cache slots [t_begin, t_end) + n_win tokens
    wk, wv = 0xD00000, 0xE00000
    win = lib.kvq_decode_attention_window
    assert win(p, q, 1, 2, 5, 4, wk, wv, 1, 4, 0, out, w, need, None) == 10   # t_end < t_begin
    assert win(p, q, 1, 2, -1, 4, wk, wv, 1, 4, 0, out, w, need, None) == 10
    assert win(p, q, 1, 2, 0, 33, wk, wv, 1, 4, 0, out, w, need, None) == 6   # beyond capacity
    assert win(p, q, 1, 2, 3, 3, wk, wv, 1, 0, 0, out, w, need, None) == 10   # no token at all
    assert win(p, q, 1, 2, 0, 8, wk, wv, 1, 4097, 0, out, w, need, None) == 10
    assert win(p, q, 1, 2, 0, 8, wk, wv, 1, -1, 0, out, w, need, None) == 10
    assert win(p, q, 1, 2, 0, 8, None, wv, 1, 4, 0, out, w, need, None) == 1
    assert win(p, q, 1, 2, 0, 8, wk, None, 1, 4, 0, out, w, need, None) == 1
    assert win(p, q, 1, 2, 0, 8, wk, wv, 5, 4, 0, out, w, need, None) == 8
    assert win(p, q, 1, 2, 0, 8, wk + 2, wv, 1, 4, 0, out, w, need, None) == 2
    assert win(p, q, 1, 2, 0, 8, wk, wv + 8, 1, 4, 0, out, w, need, None) == 2
    assert win(p, q, 1, 2, 0, 8, wk, wv, 1, 4, 0, out, w, need - 1, None) == 7
    assert win(p, q, 3, 2, 0, 8, wk, wv, 1, 4, 0, out, w, need, None) == 8
    assert win(None, q, 1, 2, 0, 8, wk, wv, 1, 4, 0, out, w, need, None) == 1
    assert win(p, q, 1, 3, 0, 8, wk, wv, 1, 4, 0, out, w, need, None) == 9
    # broken cache structs
    bad = _fake_cache(K)
    bad.v_signs = 0
    assert lib.kvq_quantize_v(C.byref(bad), src, 1, 0, 4, 0, 0, 64, None) == 1
    bad = _fake_cache(K)
    bad.k_codes = 0x10008
    assert lib.kvq_quantize_k(C.byref(bad), src, 1, 0, 4, 0, 0, 64, None) == 2
    bad = _fake_cache(K)
    bad.v_bits = 4
    assert lib.kvq_quantize_k(C.byref(bad), src, 1, 0, 4, 0, 0, 64, None) == 5
    for s in range(12):
        assert K.status_str(s)


def test_auto_splits_fill_the_gpu(K):
    """Head dimension 128 (matrix-core scan, interleaved 64-token chunks): one
    round of resident blocks (3 per CU, 2 with the key sketch; 256 CUs where no
    device answers, as here), never more than one chunk per worker (4 workers
    per split).  Smaller heads (vector-unit scan): about 4096 blocks, split
    lengths whole 256-token rounds (at least 256) within the LDS logit buffer."""
    c = _fake_cache(K, d=128, B=16, H=8, cap=32768)
    assert K.kvq_decode_auto_splits(c, 32, 32768) == 6         # 128 units x 6 = 768
    c = _fake_cache(K, d=128, B=4, H=8, cap=131136)
    assert K.kvq_decode_auto_splits(c, 32, 131136) == 24       # 32 units x 24
    c = _fake_cache(K, scheme="QKQV", n=3, d=128, B=8, H=8, cap=16384)
    assert K.kvq_decode_auto_splits(c, 8, 16384) == 8          # QKQV: 64 units x 8 = 512
    c = _fake_cache(K, d=128, B=1, H=32, cap=4096)
    assert K.kvq_decode_auto_splits(c, 32, 4096) == 17         # <= 65 chunks (15-slot lead) -> 17
    c = _fake_cache(K, d=128, B=1, H=1, cap=512)
    assert K.kvq_decode_auto_splits(c, 1, 512) == 3            # <= 9 chunks -> 3 splits
    c = _fake_cache(K, d=64, B=1, H=1, cap=256)
    assert K.kvq_decode_auto_splits(c, 1, 256) == 1
    c = _fake_cache(K, d=64, B=1, H=1, cap=100000)
    assert K.kvq_decode_auto_splits(c, 1, 100000) == 391       # 256-token splits


def test_explicit_splits_below_the_lds_budget_rejected(K):
    """The vector-unit scan (head dimension below 128) keeps a split's logits
    in LDS; the matrix-core scan (128) has no such cap."""
    lib = K.lib()
    c = _fake_cache(K, d=64, B=1, H=2, cap=6000)
    ws = C.c_size_t()
    p = C.byref(c)
    assert lib.kvq_decode_workspace(p, 8, 5120, 4, C.byref(ws)) == 0      # 1280 per split
    assert lib.kvq_decode_workspace(p, 8, 5121, 4, C.byref(ws)) == 10
    assert lib.kvq_decode_workspace(p, 2, 5121, 1, C.byref(ws)) == 10     # one head: 5120
    assert lib.kvq_decode_workspace(p, 2, 5120, 1, C.byref(ws)) == 0
    assert lib.kvq_decode_workspace(p, 4, 5120, 2, C.byref(ws)) == 0      # two heads: 2560
    assert lib.kvq_decode_workspace(p, 4, 5121, 2, C.byref(ws)) == 10
    assert lib.kvq_decode_workspace(p, 8, 4096, 8193, C.byref(ws)) == 10
    c = _fake_cache(K, d=128, B=1, H=2, cap=6000)
    p = C.byref(c)
    assert lib.kvq_decode_workspace(p, 8, 6000, 1, C.byref(ws)) == 0


def _cell_bits(bits):
    """Mantissa bits of the encoder's bucketize cells (sign, exponent and MB
    mantissa bits of u's fp32 pattern): 2 for 4-bit codes, 1 for 3-bit codes."""
    return 2 if bits >= 4 else 1


@pytest.mark.parametrize("d", [16, 32, 64, 128, 256])
@pytest.mark.parametrize("bits", [1, 2, 3, 4])
def test_table_bucketize_precondition(K, d, bits):
    """At most one threshold per prefix cell and the smallest positive one
    above the prefix-0 cell (the encoder's exact table bucketize relies on it;
    the library re-checks before launch)."""
    cb = K.kvq_codebook_init(d, bits)
    n = 1 << bits
    pos = np.array(cb.threshold[n // 2: n - 1], np.float32)
    cells = pos.view(np.uint32) >> (23 - _cell_bits(bits))
    assert len(set(cells.tolist())) == len(cells)
    if len(cells):
        assert cells[0] != 0
    if len(pos) > 1:
        assert np.min(pos[1:] / pos[:-1]) > 1 + 2.0 ** -_cell_bits(bits)


def _cell_table(thr, mb):
    """The encoder's cell table, built as the kernel builds it: for each
    prefix (sign, exponent, mb mantissa bits) the count of thresholds below the
    cell and the threshold inside it (+inf if none)."""
    n, shift = 1 << (9 + mb), 23 - mb
    i = np.arange(n, dtype=np.uint64)
    a = ((i & (n // 2 - 1)) << shift).astype(np.uint32)
    b = (a | np.uint32((1 << shift) - 1)).astype(np.uint32)
    m0, m1 = a.view(np.float32), b.view(np.float32)
    neg = i >= n // 2
    lo = np.where(neg, -m1, m0)
    hi = np.where(neg, -m0, m1)
    below = np.array([np.sum(thr < l) for l in lo])
    inside = np.full(n, np.inf, np.float32)
    for k, t in enumerate(thr):
        sel = (t >= lo) & (t <= hi)
        inside[sel] = t
    return below, inside, shift


@pytest.mark.parametrize("d", [16, 64, 128])
@pytest.mark.parametrize("bits", [3, 4])
def test_cell_table_bucketize_counts_thresholds(K, d, bits):
    """count + (threshold < u) from the cell of u's bit pattern equals the
    plain count #{thresholds < u} (ties lower, -0 and +0 as IEEE floats), on
    random coordinates, on every threshold and its two fp32 neighbours, on
    both zeros and on the ends of every cell."""
    cb = K.kvq_codebook_init(d, bits)
    thr = np.array(cb.threshold[: (1 << bits) - 1], np.float32)
    below, inside, shift = _cell_table(thr, _cell_bits(bits))
    rng = np.random.default_rng(3)
    u = [rng.standard_normal(20000).astype(np.float32) / np.float32(np.sqrt(d)),
         thr, np.nextafter(thr, np.float32(np.inf)), np.nextafter(thr, np.float32(-np.inf)),
         np.array([0.0, -0.0, 1e-30, -1e-30, 1.0, -1.0, 1.999, -1.999], np.float32)]
    n = 1 << (9 + _cell_bits(bits))
    ends = (np.arange(n, dtype=np.uint64) << shift).astype(np.uint32)
    u += [ends.view(np.float32), (ends | np.uint32((1 << shift) - 1)).view(np.float32)]
    u = np.concatenate(u)
    u = u[np.isfinite(u)]
    idx = u.view(np.uint32) >> shift
    got = below[idx] + (inside[idx] < u)
    want = np.sum(thr[None, :] < u[:, None], axis=1)
    assert np.array_equal(got, want)


def test_bad_codebook_rejected(K):
    lib = K.lib()
    c = _fake_cache(K, d=64)
    c.cb_k.threshold[8] = c.cb_k.threshold[9] * 0.99        # two thresholds in one cell
    assert lib.kvq_quantize_k(C.byref(c), 0x900000, 1, 0, 4, 0, 0, 64, None) == 4
    c = _fake_cache(K, d=64)
    c.cb_v.centroid[0] = 0.5                                 # asymmetric table
    assert lib.kvq_quantize_v(C.byref(c), 0x900000, 1, 0, 4, 0, 0, 64, None) == 4
    c = _fake_cache(K, d=64)
    c.cb_k.threshold[8], c.cb_k.threshold[6] = 1e-39, -1e-39  # in the zero threshold's cell
    assert lib.kvq_quantize_k(C.byref(c), 0x900000, 1, 0, 4, 0, 0, 64, None) == 4


# --------------------------------------------------------------------------- rotations
@pytest.mark.parametrize("d", [8, 16, 32, 64, 128, 256])
def test_rotation_signs_generator(K, d):
    """Randomized Hadamard diagonal: deterministic per seed, no bits at or
    beyond d, about half the coordinates flipped over many draws."""
    a, b = K.kvq_rotation_signs(5, d), K.kvq_rotation_signs(5, d)
    assert np.array_equal(a, b)
    assert not np.array_equal(a, K.kvq_rotation_signs(6, d))
    bits = np.array([[(int(K.kvq_rotation_signs(s, d)[i // 32]) >> (i % 32)) & 1
                      for i in range(256)] for s in range(64)])
    assert not bits[:, d:].any()
    p = bits[:, :d].mean()
    assert abs(p - 0.5) < 4 * math.sqrt(0.25 / (64 * d))


@pytest.mark.parametrize("d", [16, 64, 128])
def test_rotation_qr_generator_is_haar_on_SO_d(K, d):
    """Dense rotation ("KVQuant++" thread, "Rotation invariance guarantee"):
    orthogonal to fp32 rounding, determinant +1 for every seed (about half of
    the raw QR factors have determinant -1), entries with mean 0 and variance
    1/d, and the first column uniform on the sphere (its first coordinate has
    the sphere-marginal variance 1/d, checked by a chi-square on d * q^2)."""
    Qs = [K.kvq_rotation_qr(s, d).astype(np.float64) for s in range(40)]
    for Q in Qs:
        assert np.abs(Q @ Q.T - np.eye(d)).max() < 4e-6
        assert abs(np.linalg.det(Q) - 1.0) < 1e-4
    assert np.array_equal(K.kvq_rotation_qr(3, d), K.kvq_rotation_qr(3, d))
    E = np.stack(Qs)
    assert abs(E.mean()) < 4 / math.sqrt(E.size * d)
    assert abs((E ** 2).mean() * d - 1.0) < 1e-5
    q00 = E[:, :, 0].ravel() ** 2 * d                # many coordinates of first columns
    assert abs(q00.mean() - 1.0) < 0.15


def test_cache_set_rotation_validation(K):
    lib = K.lib()
    kv = _fake_cache(K, scheme="KV", n=4)
    assert lib.kvq_cache_set_rotation(C.byref(kv), 1, np.zeros(4, np.uint32).ctypes.data, None) == 5
    assert lib.kvq_cache_set_rotation(C.byref(kv), 0, None, None) == 0
    c = _fake_cache(K, d=64)
    w = np.zeros(4, np.uint32)
    assert lib.kvq_cache_set_rotation(C.byref(c), 3, None, None) == 5
    assert lib.kvq_cache_set_rotation(C.byref(c), 1, None, None) == 1
    assert lib.kvq_cache_set_rotation(C.byref(c), 2, None, None) == 1
    assert lib.kvq_cache_set_rotation(C.byref(c), 2, None, 0x10008) == 2
    w[2] = 1                                         # beyond the d/32 words read at d = 64
    assert lib.kvq_cache_set_rotation(C.byref(c), 1, w.ctypes.data, None) == 0
    assert list(c.rot_signs) == [0] * 8
    c16 = _fake_cache(K, d=16)
    w16 = np.array([1 << 16, 0, 0, 0], np.uint32)    # coordinate 16 of a d = 16 cache
    assert lib.kvq_cache_set_rotation(C.byref(c16), 1, w16.ctypes.data, None) == 10
    w[:] = [0xFFFFFFFF, 0x80000001, 0, 0]
    assert lib.kvq_cache_set_rotation(C.byref(c), 1, w.ctypes.data, None) == 0
    assert c.rot_kind == 1 and list(c.rot_signs) == [0xFFFFFFFF, 0x80000001] + [0] * 6
    assert lib.kvq_cache_set_rotation(C.byref(c), 2, None, 0x900000) == 0
    assert c.rot_kind == 2 and c.rot_Q == 0x900000 and list(c.rot_signs) == [0] * 8
    # d = 256: all eight sign words; the dense rotation as at every d
    c256 = _fake_cache(K, d=256)
    w8 = np.arange(1, 9, dtype=np.uint32)
    assert lib.kvq_cache_set_rotation(C.byref(c256), 1, w8.ctypes.data, None) == 0
    assert list(c256.rot_signs) == list(range(1, 9))
    assert lib.kvq_cache_set_rotation(C.byref(c256), 2, None, 0x900000) == 0
    assert c256.rot_kind == 2 and c256.rot_Q == 0x900000
    assert lib.kvq_cache_set_rotation(C.byref(c256), 2, None, 0x900008) == 2
    c8 = _fake_cache(K, d=8)
    assert lib.kvq_cache_set_rotation(C.byref(c8), 2, None, 0x900000) == 0
    assert lib.kvq_cache_set_rotation(C.byref(c8), 1, np.array([1 << 8], np.uint32).ctypes.data,
                                      None) == 10
    # the struct is validated again by every entry point
    bad = _fake_cache(K, d=64)
    bad.rot_kind = 2                                 # dense rotation without Q
    assert lib.kvq_dequantize(C.byref(bad), 0, 0, 4, 0x800000, None) == 1
    bad.rot_kind = 7
    assert lib.kvq_dequantize(C.byref(bad), 0, 0, 4, 0x800000, None) == 5
    bad = _fake_cache(K, d=32)
    bad.rot_kind, bad.rot_signs[1] = 1, 1            # coordinate 32 of a d = 32 cache
    assert lib.kvq_quantize_k(C.byref(bad), 0x900000, 1, 0, 4, 0, 0, 32, None) == 10
    kv.rot_kind = 1
    assert lib.kvq_quantize_k(C.byref(kv), 0x900000, 1, 0, 4, 0, 0, 64, None) == 5


def test_prefill_validation_status_codes(K):
    lib = K.lib()
    c = _fake_cache(K)                               # KQV-4, d = 64, B = 1, Hkv = 2, cap = 32
    p = C.byref(c)
    ws = C.c_size_t()
    assert lib.kvq_prefill_workspace(p, 3, 5, C.byref(ws)) == 9
    assert lib.kvq_prefill_workspace(p, 6, 0, C.byref(ws)) == 10
    assert lib.kvq_prefill_workspace(p, 6, 5, C.byref(ws)) == 0   # G = 3 is fine here
    # q' (no K sketch), then (M, L, o', a) per row and split: one split here
    # (a 32-slot cache caps the splits at ceil(32 / 256) = 1), then the
    # window partial (M, L, o) per row
    assert ws.value == 4 * 1 * 6 * 5 * (64 + 1 * (2 + 2 * 64) + 2 + 64)
    need = ws.value
    q, out, w = 0xA00000, 0xB00000, 0xC00000
    f = lib.kvq_prefill_attention
    assert f(p, q, 1, 6, 5, 0, 1, 8, out, w, need - 1, None) == 7
    assert f(p, q, 1, 6, 5, 0, 1, 8, out, None, need, None) == 7
    assert f(p, q, 3, 6, 5, 0, 1, 8, out, w, need, None) == 8
    assert f(p, q + 4, 1, 6, 5, 0, 1, 8, out, w, need, None) == 2
    assert f(p, None, 1, 6, 5, 0, 1, 8, out, w, need, None) == 1
    assert f(p, q, 1, 6, 5, -1, 1, 8, out, w, need, None) == 10
    assert f(p, q, 1, 6, 5, 0, 2, 8, out, w, need, None) == 10
    assert f(p, q, 1, 6, 5, 0, 1, 0, out, w, need, None) == 10
    assert f(p, q, 1, 6, 5, 0, 1, 33, out, w, need, None) == 6
    assert f(p, q, 1, 6, 0, 0, 1, 8, out, w, need, None) == 10
    assert f(p, q, 1, 5, 5, 0, 1, 8, out, w, need, None) == 9
    q3 = _fake_cache(K, scheme="QKQV", n=3)
    assert lib.kvq_prefill_workspace(C.byref(q3), 2, 7, C.byref(ws)) == 0
    assert ws.value == 4 * 1 * 2 * 7 * (2 * 64 + 1 * (2 + 2 * 64) + 2 + 64)  # + S q'


def test_prefill_window_validation_status_codes(K):
    """kvq_prefill_attention_window checks its range, window and pointers
    before any launch (no GPU needed for these paths)."""
    lib = K.lib()
    c = _fake_cache(K)                               # KQV-4, d = 64, B = 1, Hkv = 2, cap = 32
    p = C.byref(c)
    ws = C.c_size_t()
    assert lib.kvq_prefill_workspace(p, 6, 5, C.byref(ws)) == 0
    need = ws.value
    q, out, w, wk, wv = 0xA00000, 0xB00000, 0xC00000, 0xD00000, 0xE00000
    f = lib.kvq_prefill_attention_window
    # (c, q, q_dtype, q_heads, n_q, q_pos0, causal, t_begin, t_end, wk, wv, w_dtype, n_win, out, ...)
    assert f(p, q, 1, 6, 5, 0, 1, 4, 3, wk, wv, 1, 2, out, w, need, None) == 10     # t_end < t_begin
    assert f(p, q, 1, 6, 5, 0, 1, 3, 3, None, None, 1, 0, out, w, need, None) == 10  # empty union
    assert f(p, q, 1, 6, 5, 0, 1, 0, 8, wk, wv, 1, 4097, out, w, need, None) == 10  # window too long
    assert f(p, q, 1, 6, 5, 0, 1, 0, 8, wk, wv, 1, -1, out, w, need, None) == 10
    assert f(p, q, 1, 6, 5, 0, 1, 0, 33, wk, wv, 1, 2, out, w, need, None) == 6     # past capacity
    assert f(p, q, 1, 6, 5, 0, 1, 0, 8, None, wv, 1, 2, out, w, need, None) == 1    # window pointers
    assert f(p, q, 1, 6, 5, 0, 1, 0, 8, wk + 4, wv, 1, 2, out, w, need, None) == 2
    assert f(p, q, 1, 6, 5, 0, 1, 0, 8, wk, wv, 5, 2, out, w, need, None) == 8       # window dtype
    assert f(p, q, 1, 6, 5, 0, 1, 0, 8, wk, wv, 1, 2, out, w, need - 1, None) == 7  # workspace
    assert f(p, q, 1, 6, 5, 0, 2, 0, 8, wk, wv, 1, 2, out, w, need, None) == 10     # causal flag


def test_prefill_splits_fill_the_gpu(K):
    """Few query rows over a long cache are split along the tokens (at least
    256 slots per split, at most 64 splits); many rows are not."""
    ws = C.c_size_t()
    lib = K.lib()
    c = _fake_cache(K, d=128, B=1, H=32, cap=4096)   # 32 KV heads, G = 1
    assert lib.kvq_prefill_workspace(C.byref(c), 32, 256, C.byref(ws)) == 0
    rows = 32 * 256
    # 4 row tiles x 32 heads = 128 blocks -> 8 splits
    assert ws.value == 4 * rows * (128 + 8 * (2 + 256) + 2 + 128)
    c = _fake_cache(K, d=128, B=16, H=8, cap=32768)  # GQA chunk: 2048 blocks, 1 split
    assert lib.kvq_prefill_workspace(C.byref(c), 32, 256, C.byref(ws)) == 0
    assert ws.value == 4 * 16 * 32 * 256 * (128 + 1 * (2 + 256) + 2 + 128)


def test_decode_stages_and_probe_validation(K):
    """Bad stage masks and bad probe arguments fail before any launch."""
    lib = K.lib()
    c = _fake_cache(K, d=128, B=1, H=2, cap=64)
    p = C.byref(c)
    ws = C.c_size_t()
    assert lib.kvq_decode_workspace(p, 8, 64, 0, C.byref(ws)) == 0
    q, out, w = 0xA00000, 0xB00000, 0xC00000
    for mask in (0, 8, -1):
        assert lib.kvq_decode_attention_stages(p, q, 1, 8, 64, 0, mask, out, w, ws.value, None) == 10
    assert lib.kvq_decode_attention_stages(p, q, 1, 8, 0, 0, 7, out, w, ws.value, None) == 10
    assert lib.kvq_decode_attention_stages(None, q, 1, 8, 64, 0, 7, out, w, ws.value, None) == 1
    assert lib.kvq_probe_stream_read(None, 64, out, None) == 1
    assert lib.kvq_probe_stream_read(q, 64, None, None) == 1
    assert lib.kvq_probe_stream_read(q + 4, 64, out, None) == 2
    assert lib.kvq_probe_stream_read(q, 40, out, None) == 10
    assert lib.kvq_probe_stream_read(q, 0, out, None) == 10

