"""ctypes front-end of the CPU oracle.  TEST INFRASTRUCTURE ONLY.

Only the test suite, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this module.  It loads ``oracle/liboracle.so`` (plain
C, see ``kvq_oracle.c``) and shares nothing with the product library.

Scheme composition follows D'Alberto, "Statistical Inference and Quality
Measures of KV Cache Quantisations Inspired by TurboQuant" (gist.science
technical summary), section "Quantization schemes", at a budget of n bits per
coordinate:
  KV   : no rotation; K and V n-bit Lloyd-Max; no sketch
  KQV  : WHT on both; K n-bit; V (n-1)-bit + 1-bit QJL sketch
  QKQV : WHT on both; K and V (n-1)-bit + 1-bit QJL sketch
"""
from __future__ import annotations

import ctypes as C
import os
from dataclasses import dataclass, field

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
_LIB = None

SCHEMES = {"KV": 0, "KQV": 1, "QKQV": 2}


def lib():
    global _LIB
    if _LIB is None:
        # KVQ_ORACLE_LIB: a differently built copy of the same source (the
        # sanitizer test runs the pins against an ASan / UBSan build)
        path = os.environ.get("KVQ_ORACLE_LIB") or os.path.join(HERE, "liboracle.so")
        if not os.path.exists(path):
            from . import build as _b
            _b.build()
        L = C.CDLL(path)
        vp, i32, i64 = C.c_void_p, C.c_int, C.c_longlong
        L.orc_codebook.argtypes = [i32, i32, vp, vp, vp]
        L.orc_codebook.restype = i32
        L.orc_f32_to_f16.argtypes = [C.c_float]
        L.orc_f32_to_f16.restype = C.c_uint16
        L.orc_f32_to_bf16.argtypes = [C.c_float]
        L.orc_f32_to_bf16.restype = C.c_uint16
        L.orc_bf16_to_f32.argtypes = [C.c_uint16]
        L.orc_bf16_to_f32.restype = C.c_float
        L.orc_f16_to_f64.argtypes = [C.c_uint16]
        L.orc_f16_to_f64.restype = C.c_double
        L.orc_wht_f32.argtypes = [vp, i32]
        L.orc_sumsq_f32.argtypes = [vp, i32]
        L.orc_sumsq_f32.restype = C.c_float
        L.orc_bucketize.argtypes = [C.c_float, vp, i32]
        L.orc_bucketize.restype = i32
        L.orc_encode.argtypes = [vp, i32, i32, vp, i32, vp, vp, i32, vp, i32, vp, vp, vp, vp]
        L.orc_decode.argtypes = [vp, vp, C.c_uint16, C.c_uint16, i32, i32, vp, i32, vp, i32, vp,
                                 i32, vp]
        L.orc_quantize_cache.argtypes = [vp, i32, i32, i32, i32, i32, i64, i64, i64, i32, i32,
                                         i32, vp, i32, vp, vp, i32, vp, i32, vp, vp, vp, vp, i32,
                                         i32]
        L.orc_dequantize_cache.argtypes = [vp, vp, vp, vp, i32, i32, i32, i32, i32, i32,
                                           i32, vp, i32, vp, i32, vp, i32, i32, vp, i32]
        L.orc_vgroup_code_bit.argtypes = [i32, C.c_size_t, i32, i32, vp, vp]
        L.orc_vgroup_sign_bit.argtypes = [C.c_size_t, i32, vp, vp]
        L.orc_load_record.argtypes = [vp, vp, i32, C.c_size_t, i32, i32, i32, i32, vp, vp]
        L.orc_attention_dense.argtypes = [vp, vp, vp, i32, i32, vp]
        L.orc_attention.argtypes = [vp, vp, vp, i32, i32, i32, i32, i32, vp, i32, i32, i32,
                                    vp, vp, i32, i32]
        _LIB = L
    return _LIB


def _p(a):
    return None if a is None else C.c_void_p(a.ctypes.data)


# ---------------------------------------------------------------- codebook
_CB_CACHE: dict = {}


def codebook(d: int, bits: int):
    """(centroids fp32 [2^b], thresholds fp32 [2^b-1], positive fp64 centroids)."""
    key = (d, bits)
    if key not in _CB_CACHE:
        K = 1 << bits
        c64 = np.zeros(K // 2, np.float64)
        c = np.zeros(K, np.float32)
        t = np.zeros(K - 1, np.float32)
        it = lib().orc_codebook(d, bits, _p(c64), _p(c), _p(t))
        if it < 0:
            raise ValueError("bad codebook arguments")
        _CB_CACHE[key] = (c, t, c64, it)
    c, t, c64, _ = _CB_CACHE[key]
    return c.copy(), t.copy(), c64.copy()


# ---------------------------------------------------------------- formats
def f32_to_f16_bits(x: float) -> int:
    return int(lib().orc_f32_to_f16(float(x)))


def f32_to_bf16_bits(x: float) -> int:
    return int(lib().orc_f32_to_bf16(float(x)))


def f16_bits_to_f64(h: int) -> float:
    return float(lib().orc_f16_to_f64(int(h)))


def bf16_bits_to_f32(h: int) -> float:
    return float(lib().orc_bf16_to_f32(int(h)))


def wht_f32(x: np.ndarray) -> np.ndarray:
    y = np.ascontiguousarray(x, dtype=np.float32).copy()
    lib().orc_wht_f32(_p(y), y.shape[0])
    return y


def sumsq_f32(x: np.ndarray) -> np.float32:
    y = np.ascontiguousarray(x, dtype=np.float32)
    return np.float32(lib().orc_sumsq_f32(_p(y), y.shape[0]))


def bucketize(u: float, thresholds: np.ndarray) -> int:
    t = np.ascontiguousarray(thresholds, dtype=np.float32)
    return int(lib().orc_bucketize(float(np.float32(u)), _p(t), t.shape[0]))


# ---------------------------------------------------------------- schemes
@dataclass(frozen=True)
class Side:
    rotate: int
    bits: int
    qjl: int


@dataclass(frozen=True)
class Rot:
    """Rotation of the rotated sides ("KVQuant++" thread, "Entropy coding",
    "Rotation invariance guarantee"): "wht" (y = H x), "rht" (y = H D x,
    param = uint32 sign words, bit i of word i/32) or "qr" (y = Q x, param = fp32 [d][d])."""
    kind: str = "wht"
    param: object = field(default=None, compare=False)

    def code(self, side: "Side") -> int:
        if not side.rotate:
            return 0
        return {"wht": 1, "rht": 2, "qr": 3}[self.kind]

    def array(self):
        if self.kind == "rht":
            return np.ascontiguousarray(self.param, dtype=np.uint32)
        if self.kind == "qr":
            return np.ascontiguousarray(self.param, dtype=np.float32)
        return None


WHT = Rot()


def scheme_sides(scheme: str, n: int):
    """(K side, V side) of a scheme at n bits per coordinate."""
    if scheme == "KV":
        return Side(0, n, 0), Side(0, n, 0)
    if scheme == "KQV":
        return Side(1, n, 0), Side(1, n - 1, 1)
    if scheme == "QKQV":
        return Side(1, n - 1, 1), Side(1, n - 1, 1)
    raise ValueError(scheme)


# ---------------------------------------------------------------- single vectors
def encode(x: np.ndarray, side: Side, S: np.ndarray | None = None, rot: Rot = WHT):
    """Encode one vector -> (codes bytes, sign bytes or None, norm f16 bits, rnorm f16 bits)."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    d = x.shape[0]
    c, t, _ = codebook(d, side.bits)
    codes = np.zeros(d * side.bits // 8, np.uint8)
    m = 0 if S is None else S.shape[0]
    signs = np.zeros(max(m // 8, 1), np.uint8)
    norm = np.zeros(1, np.uint16)
    rnorm = np.zeros(1, np.uint16)
    Sc = None if S is None else np.ascontiguousarray(S, dtype=np.uint16)
    rp = rot.array()
    lib().orc_encode(_p(x), d, rot.code(side), _p(rp), side.bits, _p(c), _p(t), side.qjl, _p(Sc),
                     m, _p(codes), _p(signs), _p(norm), _p(rnorm))
    return codes, (signs[: m // 8] if side.qjl else None), int(norm[0]), int(rnorm[0])


def decode(codes, signs, norm, rnorm, d, side: Side, S=None, rot: Rot = WHT) -> np.ndarray:
    c, _, _ = codebook(d, side.bits)
    out = np.zeros(d, np.float64)
    m = 0 if S is None else S.shape[0]
    Sc = None if S is None else np.ascontiguousarray(S, dtype=np.uint16)
    sg = None if signs is None else np.ascontiguousarray(signs, dtype=np.uint8)
    rp = rot.array()
    lib().orc_decode(_p(np.ascontiguousarray(codes, dtype=np.uint8)), _p(sg), int(norm), int(rnorm),
                     d, rot.code(side), _p(rp), side.bits, _p(c), side.qjl, _p(Sc), m, _p(out))
    return out


# ---------------------------------------------------------------- caches
class OracleCache:
    """Host arrays of one side (K or V) of a cache, laid out [B][H][cap][...].
    values=True marks the value side: at d = 128 its codes and sign bits are
    stored in token groups (orc_vgroup_code_bit / orc_vgroup_sign_bit), which
    needs cap to be a multiple of 16."""

    def __init__(self, B, H, cap, d, side: Side, m: int, rot: Rot = WHT, values: bool = False):
        self.B, self.H, self.cap, self.d, self.side, self.m = B, H, cap, d, side, m
        self.grouped = 1 if (values and d == 128) else 0
        if self.grouped and cap % 16:
            raise ValueError("value side at d = 128 needs cap % 16 == 0")
        self.rot, self.rp = rot, rot.array()
        self.codes = np.zeros((B, H, cap, d * side.bits // 8), np.uint8)
        self.signs = np.zeros((B, H, cap, m // 8), np.uint8) if side.qjl else None
        self.norm = np.zeros((B, H, cap), np.uint16)
        self.rnorm = np.zeros((B, H, cap), np.uint16) if side.qjl else None
        self.centroid, self.threshold, _ = codebook(d, side.bits)

    def quantize(self, src: np.ndarray, t0: int, S: np.ndarray | None, nthreads: int = 1):
        """src: [B][H][T][d] float32 array or uint16 bf16 bit patterns (any strides)."""
        if src.dtype == np.float32:
            dtype = 0
        elif src.dtype == np.uint16:
            dtype = 1
        else:
            raise TypeError(src.dtype)
        B, H, T, d = src.shape
        item = src.itemsize
        sb, sh, st, si = (s // item for s in src.strides)
        assert si == 1
        Sc = None if S is None else np.ascontiguousarray(S, dtype=np.uint16)
        lib().orc_quantize_cache(C.c_void_p(src.ctypes.data), dtype, B, H, T, d, sb, sh, st, t0,
                                 self.cap, self.rot.code(self.side), _p(self.rp), self.side.bits,
                                 _p(self.centroid),
                                 _p(self.threshold), self.side.qjl, _p(Sc), self.m,
                                 _p(self.codes), _p(self.signs), _p(self.norm), _p(self.rnorm),
                                 self.grouped, nthreads)

    def dequantize(self, t0: int, T: int, S: np.ndarray | None, nthreads: int = 1) -> np.ndarray:
        out = np.zeros((self.B, self.H, T, self.d), np.float64)
        Sc = None if S is None else np.ascontiguousarray(S, dtype=np.uint16)
        lib().orc_dequantize_cache(_p(self.codes), _p(self.signs), _p(self.norm), _p(self.rnorm),
                                   self.B, self.H, self.cap, t0, T, self.d,
                                   self.rot.code(self.side), _p(self.rp), self.side.bits,
                                   _p(self.centroid), self.side.qjl, _p(Sc),
                                   self.m, self.grouped, _p(out), nthreads)
        return out

    def view(self, b0: int, b1: int, h0: int = 0, h1: int | None = None) -> "OracleCache":
        """The same arrays restricted to batch rows [b0, b1) and KV heads
        [h0, h1) (shared memory; a partial head range needs a single batch
        row, so the view stays contiguous)."""
        h1 = self.H if h1 is None else h1
        if (h0, h1) != (0, self.H) and b1 != b0 + 1:
            raise ValueError("a partial head range needs a single batch row")
        v = OracleCache.__new__(OracleCache)
        v.__dict__.update(self.__dict__)
        v.B, v.H = b1 - b0, h1 - h0
        sl = (slice(b0, b1), slice(h0, h1))
        v.codes = self.codes[sl]
        v.signs = None if self.signs is None else self.signs[sl]
        v.norm = self.norm[sl]
        v.rnorm = None if self.rnorm is None else self.rnorm[sl]
        return v

    def _side_struct(self):
        return _OrcSide(_p(self.codes), _p(self.signs), _p(self.norm), _p(self.rnorm),
                        self.rot.code(self.side), self.side.bits, self.side.qjl,
                        _p(self.centroid), _p(self.rp), self.grouped)


class _OrcSide(C.Structure):
    _fields_ = [("codes", C.c_void_p), ("signs", C.c_void_p), ("norm", C.c_void_p),
                ("rnorm", C.c_void_p), ("rotate", C.c_int), ("bits", C.c_int),
                ("qjl", C.c_int), ("centroid", C.c_void_p), ("rparam", C.c_void_p),
                ("grouped", C.c_int)]


def attention(kc: OracleCache, vc: OracleCache, q: np.ndarray, n_ctx: int,
              S: np.ndarray | None, rows=None, nthreads: int = 1) -> np.ndarray:
    """q: [B][Hq][d] float32 or bf16 bit patterns (uint16).  Returns fp64 [B][Hq][d]
    (only the listed rows b*Hq+hq are filled when rows is given)."""
    q = np.ascontiguousarray(q)
    qd = 0 if q.dtype == np.float32 else 1
    B, Hq, d = q.shape
    out = np.zeros((B, Hq, d), np.float64)
    ks, vs = kc._side_struct(), vc._side_struct()
    Sc = None if S is None else np.ascontiguousarray(S, dtype=np.uint16)
    m = 0 if S is None else S.shape[0]
    if rows is not None:
        ra = np.ascontiguousarray(np.asarray(rows, dtype=np.int32))
        rp, nr = _p(ra), ra.shape[0]
    else:
        rp, nr = None, 0
    lib().orc_attention(C.byref(ks), C.byref(vs), _p(Sc), m, kc.B, kc.H, kc.cap, d,
                        C.c_void_p(q.ctypes.data), qd, Hq, n_ctx, _p(out), rp, nr, nthreads)
    return out


def attention_dense(q: np.ndarray, K: np.ndarray, V: np.ndarray) -> np.ndarray:
    """Plain fp64 attention of one query over explicit keys/values [n][d]."""
    q = np.ascontiguousarray(q, dtype=np.float64)
    K = np.ascontiguousarray(K, dtype=np.float64)
    V = np.ascontiguousarray(V, dtype=np.float64)
    out = np.zeros(q.shape[0], np.float64)
    lib().orc_attention_dense(_p(q), _p(K), _p(V), K.shape[0], q.shape[0], _p(out))
    return out


def _host_f64(x: np.ndarray) -> np.ndarray:
    """float32 array or uint16 bf16 bit patterns -> float64 (exact)."""
    if x.dtype == np.uint16:
        return (x.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return np.asarray(x, dtype=np.float64)


def attention_window(kc: OracleCache, vc: OracleCache, q: np.ndarray, t_begin: int, t_end: int,
                     wk: np.ndarray | None, wv: np.ndarray | None, S: np.ndarray | None,
                     nthreads: int = 1) -> np.ndarray:
    """Decode over compressed slots [t_begin, t_end) plus full-precision window
    tokens wk, wv [B][Hkv][n_win][d] (float32 or bf16 bits; None for none).

    "Your KV cache is not a bit problem but a geometry problem", sections
    "Systems tax" and "What we should do" (recent tokens kept unquantized) and
    "Frontier" (attention-sink tokens likewise): one softmax over the union of
    the reconstructed cache tokens and the exact window tokens, i.e. plain
    attention over the concatenated key and value lists.  Returns fp64
    [B][Hq][d]."""
    qd = _host_f64(np.ascontiguousarray(q))
    B, Hq, d = qd.shape
    G = Hq // kc.H
    T = t_end - t_begin
    if T > 0:
        Kh = kc.dequantize(t_begin, T, S, nthreads)
        Vh = vc.dequantize(t_begin, T, S, nthreads)
    else:
        Kh = np.zeros((B, kc.H, 0, d))
        Vh = np.zeros((B, kc.H, 0, d))
    if wk is not None:
        Kh = np.concatenate([Kh, _host_f64(wk)], axis=2)
        Vh = np.concatenate([Vh, _host_f64(wv)], axis=2)
    out = np.zeros((B, Hq, d), np.float64)
    for b in range(B):
        for hq in range(Hq):
            out[b, hq] = attention_dense(qd[b, hq], Kh[b, hq // G], Vh[b, hq // G])
    return out


def prefill_attention_window(kc: OracleCache, vc: OracleCache, q: np.ndarray, q_pos0: int,
                             causal: bool, t_begin: int, t_end: int, wk: np.ndarray | None,
                             wv: np.ndarray | None, S: np.ndarray | None,
                             nthreads: int = 1) -> np.ndarray:
    """Multi-query attention with a full-precision window: query token i (at
    position q_pos0 + i) attends over the reconstructed slots t in [t_begin,
    t_end), only t <= q_pos0 + i when causal, together with every window token
    wk, wv [B][Hkv][n_win][d] (float32 or bf16 bits; None for none).  The
    window holds tokens that precede the chunk -- attention sinks and the most
    recent tokens before it ("Your KV cache is not a bit problem but a geometry
    problem", "Systems tax", "What we should do", "Frontier") -- so every query
    of the chunk sees all of them.  One plain fp64 softmax per row over the
    union.  Returns fp64 [B][n_q][Hq][d]."""
    qd = _host_f64(np.ascontiguousarray(q))
    B, nq, Hq, d = qd.shape
    G = Hq // kc.H
    T = t_end - t_begin
    if T > 0:
        Kh = kc.dequantize(t_begin, T, S, nthreads)
        Vh = vc.dequantize(t_begin, T, S, nthreads)
    else:
        Kh = np.zeros((B, kc.H, 0, d))
        Vh = np.zeros((B, kc.H, 0, d))
    Kw = _host_f64(wk) if wk is not None else np.zeros((B, kc.H, 0, d))
    Vw = _host_f64(wv) if wv is not None else np.zeros((B, kc.H, 0, d))
    out = np.zeros((B, nq, Hq, d), np.float64)
    for b in range(B):
        for i in range(nq):
            lim = min(t_end, q_pos0 + i + 1) if causal else t_end
            n = max(0, lim - t_begin)
            for hq in range(Hq):
                h = hq // G
                K = np.concatenate([Kh[b, h, :n], Kw[b, h]], axis=0)
                V = np.concatenate([Vh[b, h, :n], Vw[b, h]], axis=0)
                out[b, i, hq] = attention_dense(qd[b, i, hq], K, V)
    return out


def prefill_attention(kc: OracleCache, vc: OracleCache, q: np.ndarray, q_pos0: int, causal: bool,
                      n_ctx: int, S: np.ndarray | None, nthreads: int = 1) -> np.ndarray:
    """Multi-query attention of q [B][n_q][Hq][d] (float32 or bf16 bits) over
    the reconstructed cache slots [0, n_ctx); query token i sits at position
    q_pos0 + i and, when causal, sees slots t <= q_pos0 + i ("Your KV cache is
    not a bit problem but a geometry problem", "Systems tax": a prompt chunk
    is appended, then attends).  Plain fp64 attention per row.  Returns fp64
    [B][n_q][Hq][d]."""
    qd = _host_f64(np.ascontiguousarray(q))
    B, nq, Hq, d = qd.shape
    G = Hq // kc.H
    Kh = kc.dequantize(0, n_ctx, S, nthreads)
    Vh = vc.dequantize(0, n_ctx, S, nthreads)
    out = np.zeros((B, nq, Hq, d), np.float64)
    for b in range(B):
        for i in range(nq):
            T = min(n_ctx, q_pos0 + i + 1) if causal else n_ctx
            for hq in range(Hq):
                out[b, i, hq] = attention_dense(qd[b, i, hq], Kh[b, hq // G, :T], Vh[b, hq // G, :T])
    return out
