"""Python binding of libkvq (include/kvq.h): ctypes marshalling only.

Every step of the codec and of decode attention runs in the library's gfx950
kernels; torch is used only to own device memory and to supply the stream.
If the shared library is missing this module raises on first use -- there is
no CPU fallback.
"""
from __future__ import annotations

import ctypes as C
import os

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libkvq.so")

KVQ_OK = 0
STATUS_NAMES = {0: "KVQ_OK", 1: "KVQ_ERR_NULL", 2: "KVQ_ERR_ALIGN", 3: "KVQ_ERR_DIM",
                4: "KVQ_ERR_BITS", 5: "KVQ_ERR_SCHEME", 6: "KVQ_ERR_CAPACITY",
                7: "KVQ_ERR_WORKSPACE", 8: "KVQ_ERR_DTYPE", 9: "KVQ_ERR_HEADS",
                10: "KVQ_ERR_RANGE", 11: "KVQ_ERR_HIP"}
SCHEMES = {"KV": 0, "KQV": 1, "QKQV": 2}
ROTATIONS = {"wht": 0, "rht": 1, "qr": 2}
KVQ_F32, KVQ_BF16 = 0, 1

EXPORTS = ["kvq_codebook_init", "kvq_sketch_init", "kvq_cache_init", "kvq_cache_set_rotation",
           "kvq_rotation_signs", "kvq_rotation_qr", "kvq_cache_layout", "kvq_quantize_k",
           "kvq_quantize_v", "kvq_dequantize", "kvq_decode_attention",
           "kvq_decode_attention_window", "kvq_decode_attention_noalloc",
           "kvq_decode_attention_stages", "kvq_probe_stream_read",
           "kvq_decode_workspace", "kvq_decode_auto_splits",
           "kvq_prefill_attention", "kvq_prefill_attention_window", "kvq_prefill_workspace",
           "kvq_status_str", "kvq_version"]


class KVQError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {STATUS_NAMES.get(status, status)} ({status_str(status)})")


class kvq_codebook(C.Structure):
    _fields_ = [("d", C.c_int32), ("bits", C.c_int32), ("centroid", C.c_float * 16),
                ("threshold", C.c_float * 15)]


class kvq_cache(C.Structure):
    _fields_ = [("scheme", C.c_int32), ("n_bits", C.c_int32), ("d", C.c_int32), ("m", C.c_int32),
                ("batch", C.c_int32), ("kv_heads", C.c_int32), ("capacity", C.c_int32),
                ("k_bits", C.c_int32), ("v_bits", C.c_int32), ("k_qjl", C.c_int32),
                ("v_qjl", C.c_int32), ("rotate", C.c_int32),
                ("cb_k", kvq_codebook), ("cb_v", kvq_codebook),
                ("S", C.c_void_p),
                ("k_codes", C.c_void_p), ("k_signs", C.c_void_p),
                ("v_codes", C.c_void_p), ("v_signs", C.c_void_p),
                ("k_norm", C.c_void_p), ("k_rnorm", C.c_void_p),
                ("v_norm", C.c_void_p), ("v_rnorm", C.c_void_p),
                ("rot_kind", C.c_int32), ("rot_signs", C.c_uint32 * 8),
                ("rot_Q", C.c_void_p)]


_LIB = None


def lib():
    """Load libkvq.so (built in-tree by ``__graft_entry__.build()``)."""
    global _LIB
    if _LIB is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"libkvq.so not found at {LIB_PATH}; run __graft_entry__.build()")
        L = C.CDLL(LIB_PATH)
        i32, i64, vp, sz = C.c_int, C.c_int64, C.c_void_p, C.c_size_t
        cb_p, cache_p = C.POINTER(kvq_codebook), C.POINTER(kvq_cache)
        sig = {
            "kvq_codebook_init": ([i32, i32, cb_p], i32),
            "kvq_sketch_init": ([C.c_uint64, i32, i32, vp], i32),
            "kvq_cache_init": ([cache_p, i32, i32, i32, i32, i32, i32], i32),
            "kvq_cache_set_rotation": ([cache_p, i32, vp, vp], i32),
            "kvq_rotation_signs": ([C.c_uint64, i32, vp], i32),
            "kvq_rotation_qr": ([C.c_uint64, i32, vp], i32),
            "kvq_cache_layout": ([i32, i32, i32, i32, i32, i32, C.POINTER(sz)], i32),
            "kvq_quantize_k": ([cache_p, vp, i32, i32, i32, i64, i64, i64, vp], i32),
            "kvq_quantize_v": ([cache_p, vp, i32, i32, i32, i64, i64, i64, vp], i32),
            "kvq_dequantize": ([cache_p, i32, i32, i32, vp, vp], i32),
            "kvq_decode_attention": ([cache_p, vp, i32, i32, i32, i32, vp, vp, sz, vp], i32),
            "kvq_decode_attention_window": ([cache_p, vp, i32, i32, i32, i32, vp, vp, i32, i32,
                                             i32, vp, vp, sz, vp], i32),
            "kvq_decode_attention_noalloc": ([cache_p, vp, i32, i32, i32, i32, vp, vp], i32),
            "kvq_decode_attention_stages": ([cache_p, vp, i32, i32, i32, i32, i32, vp, vp, sz, vp],
                                            i32),
            "kvq_probe_stream_read": ([vp, sz, vp, vp], i32),
            "kvq_decode_workspace": ([cache_p, i32, i32, i32, C.POINTER(sz)], i32),
            "kvq_decode_auto_splits": ([cache_p, i32, i32], i32),
            "kvq_prefill_attention": ([cache_p, vp, i32, i32, i32, i32, i32, i32, vp, vp, sz, vp],
                                      i32),
            "kvq_prefill_attention_window": ([cache_p, vp, i32, i32, i32, i32, i32, i32, i32, vp, vp,
                                              i32, i32, vp, vp, sz, vp], i32),
            "kvq_prefill_workspace": ([cache_p, i32, i32, C.POINTER(sz)], i32),
            "kvq_status_str": ([i32], C.c_char_p),
            "kvq_version": ([], C.c_char_p),
        }
        for name, (args, res) in sig.items():
            f = getattr(L, name)
            f.argtypes = args
            f.restype = res
        _LIB = L
    return _LIB


def status_str(s: int) -> str:
    return lib().kvq_status_str(int(s)).decode()


def _check(s: int, where: str):
    if s != KVQ_OK:
        raise KVQError(s, where)


# ------------------------------------------------------------------ host entry points
def kvq_codebook_init(d: int, bits: int) -> kvq_codebook:
    cb = kvq_codebook()
    _check(lib().kvq_codebook_init(d, bits, C.byref(cb)), "kvq_codebook_init")
    return cb


def kvq_sketch_init(seed: int, m: int, d: int) -> np.ndarray:
    out = np.zeros((m, d), np.uint16)
    _check(lib().kvq_sketch_init(seed, m, d, out.ctypes.data), "kvq_sketch_init")
    return out


def kvq_cache_init(scheme: int, n_bits: int, d: int, batch: int, kv_heads: int,
                   capacity: int) -> kvq_cache:
    c = kvq_cache()
    _check(lib().kvq_cache_init(C.byref(c), scheme, n_bits, d, batch, kv_heads, capacity),
           "kvq_cache_init")
    return c


def kvq_rotation_signs(seed: int, d: int) -> np.ndarray:
    out = np.zeros(8, np.uint32)
    _check(lib().kvq_rotation_signs(seed, d, out.ctypes.data), "kvq_rotation_signs")
    return out


def kvq_rotation_qr(seed: int, d: int) -> np.ndarray:
    out = np.zeros((d, d), np.float32)
    _check(lib().kvq_rotation_qr(seed, d, out.ctypes.data), "kvq_rotation_qr")
    return out


def kvq_cache_set_rotation(c: kvq_cache, kind: int, signs=None, Q_device: int = 0):
    sp = None
    if signs is not None:
        signs = np.ascontiguousarray(signs, dtype=np.uint32)
        sp = signs.ctypes.data
    _check(lib().kvq_cache_set_rotation(C.byref(c), kind, sp, Q_device or None),
           "kvq_cache_set_rotation")


def kvq_cache_layout(scheme: int, n_bits: int, d: int, batch: int, kv_heads: int,
                     capacity: int):
    out = (C.c_size_t * 8)()
    _check(lib().kvq_cache_layout(scheme, n_bits, d, batch, kv_heads, capacity, out),
           "kvq_cache_layout")
    return list(out)


# ------------------------------------------------------------------ device entry points
def kvq_quantize_k(c: kvq_cache, src: int, dtype: int, t0: int, T: int, sb: int, sh: int,
                   st: int, stream: int = 0):
    _check(lib().kvq_quantize_k(C.byref(c), src, dtype, t0, T, sb, sh, st, stream), "kvq_quantize_k")


def kvq_quantize_v(c: kvq_cache, src: int, dtype: int, t0: int, T: int, sb: int, sh: int,
                   st: int, stream: int = 0):
    _check(lib().kvq_quantize_v(C.byref(c), src, dtype, t0, T, sb, sh, st, stream), "kvq_quantize_v")


def kvq_dequantize(c: kvq_cache, which: int, t0: int, T: int, out: int, stream: int = 0):
    _check(lib().kvq_dequantize(C.byref(c), which, t0, T, out, stream), "kvq_dequantize")


def kvq_decode_workspace(c: kvq_cache, q_heads: int, n_ctx: int, splits: int = 0) -> int:
    n = C.c_size_t()
    _check(lib().kvq_decode_workspace(C.byref(c), q_heads, n_ctx, splits, C.byref(n)),
           "kvq_decode_workspace")
    return n.value


def kvq_decode_auto_splits(c: kvq_cache, q_heads: int, n_ctx: int) -> int:
    return int(lib().kvq_decode_auto_splits(C.byref(c), q_heads, n_ctx))


def kvq_decode_attention(c: kvq_cache, q: int, q_dtype: int, q_heads: int, n_ctx: int,
                         splits: int, out: int, workspace: int, ws_bytes: int, stream: int = 0):
    _check(lib().kvq_decode_attention(C.byref(c), q, q_dtype, q_heads, n_ctx, splits, out,
                                      workspace, ws_bytes, stream), "kvq_decode_attention")


def kvq_decode_attention_window(c: kvq_cache, q: int, q_dtype: int, q_heads: int, t_begin: int,
                                t_end: int, wk: int, wv: int, w_dtype: int, n_win: int,
                                splits: int, out: int, workspace: int, ws_bytes: int,
                                stream: int = 0):
    _check(lib().kvq_decode_attention_window(C.byref(c), q, q_dtype, q_heads, t_begin, t_end, wk,
                                             wv, w_dtype, n_win, splits, out, workspace, ws_bytes,
                                             stream), "kvq_decode_attention_window")


def kvq_decode_attention_noalloc(c: kvq_cache, q: int, q_dtype: int, q_heads: int, n_ctx: int,
                                 splits: int, out: int, stream: int = 0):
    _check(lib().kvq_decode_attention_noalloc(C.byref(c), q, q_dtype, q_heads, n_ctx, splits,
                                              out, stream), "kvq_decode_attention_noalloc")


KVQ_STAGE_PREP, KVQ_STAGE_SCAN, KVQ_STAGE_MERGE, KVQ_STAGE_ALL = 1, 2, 4, 7


def kvq_decode_attention_stages(c: kvq_cache, q: int, q_dtype: int, q_heads: int, n_ctx: int,
                                splits: int, stages: int, out: int, workspace: int, ws_bytes: int,
                                stream: int = 0):
    _check(lib().kvq_decode_attention_stages(C.byref(c), q, q_dtype, q_heads, n_ctx, splits, stages,
                                             out, workspace, ws_bytes, stream),
           "kvq_decode_attention_stages")


def kvq_probe_stream_read(buf: int, nbytes: int, out: int, stream: int = 0):
    _check(lib().kvq_probe_stream_read(buf, nbytes, out, stream), "kvq_probe_stream_read")


def kvq_prefill_workspace(c: kvq_cache, q_heads: int, n_q: int) -> int:
    n = C.c_size_t()
    _check(lib().kvq_prefill_workspace(C.byref(c), q_heads, n_q, C.byref(n)),
           "kvq_prefill_workspace")
    return n.value


def kvq_prefill_attention(c: kvq_cache, q: int, q_dtype: int, q_heads: int, n_q: int,
                          q_pos0: int, causal: int, n_ctx: int, out: int, workspace: int,
                          ws_bytes: int, stream: int = 0):
    _check(lib().kvq_prefill_attention(C.byref(c), q, q_dtype, q_heads, n_q, q_pos0, causal,
                                       n_ctx, out, workspace, ws_bytes, stream),
           "kvq_prefill_attention")


def kvq_prefill_attention_window(c: kvq_cache, q: int, q_dtype: int, q_heads: int, n_q: int,
                                 q_pos0: int, causal: int, t_begin: int, t_end: int, wk: int,
                                 wv: int, w_dtype: int, n_win: int, out: int, workspace: int,
                                 ws_bytes: int, stream: int = 0):
    _check(lib().kvq_prefill_attention_window(C.byref(c), q, q_dtype, q_heads, n_q, q_pos0, causal,
                                              t_begin, t_end, wk, wv, w_dtype, n_win, out,
                                              workspace, ws_bytes, stream),
           "kvq_prefill_attention_window")


# ------------------------------------------------------------------ torch-owned cache
class KVQCache:
    """A compressed KV cache whose buffers are torch device tensors.

    Thin marshalling over the C ABI: allocation (torch), pointer/stride/stream
    plumbing, and status checks.  Mirrors the construct / compress / decompress
    interface of the "KVQuant++" thread ("Deployment and usage") with the
    per-token append and whole-cache decode read of the KV-cache problem.
    """

    BUFS = ["k_codes", "k_signs", "k_norm", "k_rnorm", "v_codes", "v_signs", "v_norm", "v_rnorm"]

    def __init__(self, scheme: str, n_bits: int, d: int, batch: int, kv_heads: int,
                 capacity: int, S_bf16=None, device="cuda", rotation: str = "wht",
                 rot_signs=None, rot_Q=None, rot_seed: int = 11):
        """rotation (rotated schemes): "wht", "rht" (rot_signs: uint32 words, d/32 used,
        default kvq_rotation_signs(rot_seed)) or "qr" (rot_Q: d x d fp32,
        default kvq_rotation_qr(rot_seed))."""
        import torch
        self.torch = torch
        self.scheme, self.n_bits, self.d = scheme, n_bits, d
        self.batch, self.kv_heads, self.capacity = batch, kv_heads, capacity
        dev = torch.device(device)
        if dev.type == "cuda" and dev.index is None:
            dev = torch.device("cuda", torch.cuda.current_device())
        self.device = dev
        self.c = kvq_cache_init(SCHEMES[scheme], n_bits, d, batch, kv_heads, capacity)
        sizes = kvq_cache_layout(SCHEMES[scheme], n_bits, d, batch, kv_heads, capacity)
        self.bufs = {}
        for name, nbytes in zip(self.BUFS, sizes):
            if nbytes == 0:
                continue
            dt = torch.uint8 if name.endswith(("codes", "signs")) else torch.int16
            n = nbytes if dt == torch.uint8 else nbytes // 2
            t = torch.zeros(n, dtype=dt, device=self.device)
            self.bufs[name] = t
            setattr(self.c, name, t.data_ptr())
        self.S = None
        if self.c.k_qjl or self.c.v_qjl:
            if S_bf16 is None:
                S_bf16 = kvq_sketch_init(7, d, d)
            S_np = np.ascontiguousarray(np.asarray(S_bf16).view(np.uint16))
            self.S = torch.from_numpy(S_np.view(np.int16)).to(self.device)
            self.c.S = self.S.data_ptr()
        self.rotation, self.rot_Q = rotation, None
        kind = ROTATIONS[rotation]
        if kind == 1:
            signs = kvq_rotation_signs(rot_seed, d) if rot_signs is None else rot_signs
            kvq_cache_set_rotation(self.c, kind, signs=signs)
        elif kind == 2:
            Q = kvq_rotation_qr(rot_seed, d) if rot_Q is None else np.asarray(rot_Q, np.float32)
            self.rot_Q = torch.from_numpy(np.ascontiguousarray(Q)).to(self.device)
            kvq_cache_set_rotation(self.c, kind, Q_device=self.rot_Q.data_ptr())

    # views of the raw buffers in their documented shapes
    def view(self, name: str):
        t = self.bufs[name]
        B, H, cap = self.batch, self.kv_heads, self.capacity
        if name.endswith("norm"):
            return t.view(B, H, cap)
        return t.view(B, H, cap, -1)

    def _stream(self):
        return self.torch.cuda.current_stream(self.device).cuda_stream

    def _quantize(self, fn, x, t0: int):
        torch = self.torch
        if x.device != self.device:
            raise ValueError("input must live on the cache's device")
        if x.dim() != 4 or x.shape[0] != self.batch or x.shape[1] != self.kv_heads or x.shape[3] != self.d:
            raise ValueError(f"expected [B={self.batch}][H={self.kv_heads}][T][d={self.d}], got {tuple(x.shape)}")
        if x.stride(3) != 1:
            raise ValueError("innermost dimension must be contiguous")
        dt = {torch.float32: KVQ_F32, torch.bfloat16: KVQ_BF16}.get(x.dtype)
        if dt is None:
            raise TypeError(f"unsupported dtype {x.dtype}")
        fn(self.c, x.data_ptr(), dt, t0, x.shape[2], x.stride(0), x.stride(1), x.stride(2),
           self._stream())

    def quantize_k(self, k, t0: int = 0):
        self._quantize(kvq_quantize_k, k, t0)

    def quantize_v(self, v, t0: int = 0):
        self._quantize(kvq_quantize_v, v, t0)

    def dequantize(self, which: int, t0: int, T: int):
        out = self.torch.empty(self.batch, self.kv_heads, T, self.d, dtype=self.torch.float32,
                               device=self.device)
        kvq_dequantize(self.c, which, t0, T, out.data_ptr(), self._stream())
        return out

    def workspace_bytes(self, q_heads: int, n_ctx: int, splits: int = 0) -> int:
        return kvq_decode_workspace(self.c, q_heads, n_ctx, splits)

    def decode_attention(self, q, n_ctx: int, splits: int = 0, out=None, workspace=None,
                         stages: int = KVQ_STAGE_ALL):
        """Decode over cache slots [0, n_ctx); stages (KVQ_STAGE_* mask) runs only
        those stages (the workspace carries the intermediate results)."""
        torch = self.torch
        if q.dim() != 3 or q.shape[0] != self.batch or q.shape[2] != self.d or not q.is_contiguous():
            raise ValueError("q must be a contiguous [B][q_heads][d] tensor")
        dt = {torch.float32: KVQ_F32, torch.bfloat16: KVQ_BF16}.get(q.dtype)
        if dt is None:
            raise TypeError(f"unsupported dtype {q.dtype}")
        Hq = q.shape[1]
        nbytes = self.workspace_bytes(Hq, n_ctx, splits)
        if workspace is None or workspace.numel() < nbytes:
            workspace = torch.empty(max(nbytes, 16), dtype=torch.uint8, device=self.device)
        if out is None:
            out = torch.empty(self.batch, Hq, self.d, dtype=torch.float32, device=self.device)
        if stages == KVQ_STAGE_ALL:
            kvq_decode_attention(self.c, q.data_ptr(), dt, Hq, n_ctx, splits, out.data_ptr(),
                                 workspace.data_ptr(), workspace.numel(), self._stream())
        else:
            kvq_decode_attention_stages(self.c, q.data_ptr(), dt, Hq, n_ctx, splits, stages,
                                        out.data_ptr(), workspace.data_ptr(), workspace.numel(),
                                        self._stream())
        return out

    def prefill_attention(self, q, q_pos0: int, n_ctx: int, causal: bool = True, out=None,
                          workspace=None):
        """Multi-query attention of q [B][n_q][q_heads][d] (query token i at
        position q_pos0 + i) over cache slots [0, n_ctx); out [B][n_q][q_heads][d]."""
        torch = self.torch
        if q.dim() != 4 or q.shape[0] != self.batch or q.shape[3] != self.d or not q.is_contiguous():
            raise ValueError("q must be a contiguous [B][n_q][q_heads][d] tensor")
        dt = {torch.float32: KVQ_F32, torch.bfloat16: KVQ_BF16}.get(q.dtype)
        if dt is None:
            raise TypeError(f"unsupported dtype {q.dtype}")
        n_q, Hq = q.shape[1], q.shape[2]
        nbytes = kvq_prefill_workspace(self.c, Hq, n_q)
        if workspace is None or workspace.numel() < nbytes:
            workspace = torch.empty(max(nbytes, 16), dtype=torch.uint8, device=self.device)
        if out is None:
            out = torch.empty(self.batch, n_q, Hq, self.d, dtype=torch.float32, device=self.device)
        kvq_prefill_attention(self.c, q.data_ptr(), dt, Hq, n_q, q_pos0, int(bool(causal)), n_ctx,
                              out.data_ptr(), workspace.data_ptr(), workspace.numel(),
                              self._stream())
        return out

    def prefill_attention_window(self, q, q_pos0: int, t_begin: int, t_end: int, wk=None, wv=None,
                                 causal: bool = True, out=None, workspace=None):
        """Multi-query attention of q [B][n_q][q_heads][d] over cache slots
        [t_begin, t_end) (causal: up to each query's position) plus the
        full-precision tokens wk, wv ([B][kv_heads][n_win][d], fp32 or bf16;
        None for none), which every query sees."""
        torch = self.torch
        if q.dim() != 4 or q.shape[0] != self.batch or q.shape[3] != self.d or not q.is_contiguous():
            raise ValueError("q must be a contiguous [B][n_q][q_heads][d] tensor")
        dts = {torch.float32: KVQ_F32, torch.bfloat16: KVQ_BF16}
        dt = dts.get(q.dtype)
        if dt is None:
            raise TypeError(f"unsupported dtype {q.dtype}")
        n_win, wdt, pk, pv = 0, KVQ_F32, 0, 0
        if wk is not None:
            shape = (self.batch, self.kv_heads, wk.shape[2] if wk.dim() == 4 else -1, self.d)
            if (wk.dim() != 4 or tuple(wk.shape) != shape or wv is None
                    or tuple(wv.shape) != shape or wk.dtype != wv.dtype
                    or not (wk.is_contiguous() and wv.is_contiguous())):
                raise ValueError("wk, wv must be contiguous [B][kv_heads][n_win][d] tensors")
            wdt = dts.get(wk.dtype)
            if wdt is None:
                raise TypeError(f"unsupported dtype {wk.dtype}")
            n_win, pk, pv = wk.shape[2], wk.data_ptr(), wv.data_ptr()
        n_q, Hq = q.shape[1], q.shape[2]
        nbytes = kvq_prefill_workspace(self.c, Hq, n_q)
        if workspace is None or workspace.numel() < nbytes:
            workspace = torch.empty(max(nbytes, 16), dtype=torch.uint8, device=self.device)
        if out is None:
            out = torch.empty(self.batch, n_q, Hq, self.d, dtype=torch.float32, device=self.device)
        kvq_prefill_attention_window(self.c, q.data_ptr(), dt, Hq, n_q, q_pos0, int(bool(causal)),
                                     t_begin, t_end, pk, pv, wdt, n_win, out.data_ptr(),
                                     workspace.data_ptr(), workspace.numel(), self._stream())
        return out

    def decode_attention_window(self, q, t_begin: int, t_end: int, wk=None, wv=None,
                                splits: int = 0, out=None, workspace=None):
        """Decode over cache slots [t_begin, t_end) plus the full-precision
        tokens wk, wv ([B][kv_heads][n_win][d], fp32 or bf16; None for none)."""
        torch = self.torch
        if q.dim() != 3 or q.shape[0] != self.batch or q.shape[2] != self.d or not q.is_contiguous():
            raise ValueError("q must be a contiguous [B][q_heads][d] tensor")
        dts = {torch.float32: KVQ_F32, torch.bfloat16: KVQ_BF16}
        dt = dts.get(q.dtype)
        if dt is None:
            raise TypeError(f"unsupported dtype {q.dtype}")
        n_win, wdt, pk, pv = 0, KVQ_F32, 0, 0
        if wk is not None:
            shape = (self.batch, self.kv_heads, wk.shape[2] if wk.dim() == 4 else -1, self.d)
            if (wk.dim() != 4 or tuple(wk.shape) != shape or wv is None
                    or tuple(wv.shape) != shape or wk.dtype != wv.dtype
                    or not (wk.is_contiguous() and wv.is_contiguous())):
                raise ValueError("wk, wv must be contiguous [B][kv_heads][n_win][d] tensors")
            wdt = dts.get(wk.dtype)
            if wdt is None:
                raise TypeError(f"unsupported dtype {wk.dtype}")
            n_win, pk, pv = wk.shape[2], wk.data_ptr(), wv.data_ptr()
        Hq = q.shape[1]
        nbytes = self.workspace_bytes(Hq, t_end - t_begin, splits)
        if workspace is None or workspace.numel() < nbytes:
            workspace = torch.empty(max(nbytes, 16), dtype=torch.uint8, device=self.device)
        if out is None:
            out = torch.empty(self.batch, Hq, self.d, dtype=torch.float32, device=self.device)
        kvq_decode_attention_window(self.c, q.data_ptr(), dt, Hq, t_begin, t_end, pk, pv, wdt,
                                    n_win, splits, out.data_ptr(), workspace.data_ptr(),
                                    workspace.numel(), self._stream())
        return out
