"""ctypes wrappers over the C oracle (test infrastructure only).

Every function takes and returns numpy arrays in the same host layouts the
library documents for device memory:
  kv     [n_seq, cap, 144]  uint8   FP4 K codes | V codes | 8 K scales | 8 V scales
  idxk   [n_seq, cap, 64]   uint8   E4M3 indexer keys
  wk, wv [n_layers, n_seq, w_cap, 128] uint8  E4M3 window rows, slot = pos % w_cap
"""
from __future__ import annotations

import ctypes as C
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libcsa2_oracle.so")
_lib = None

_u8p = np.ctypeslib.ndpointer(np.uint8, flags="C_CONTIGUOUS")
_f32p = np.ctypeslib.ndpointer(np.float32, flags="C_CONTIGUOUS")
_f64p = np.ctypeslib.ndpointer(np.float64, flags="C_CONTIGUOUS")
_i32p = np.ctypeslib.ndpointer(np.int32, flags="C_CONTIGUOUS")
_i64p = np.ctypeslib.ndpointer(np.int64, flags="C_CONTIGUOUS")

REC = 144
D, H, HI, DI, WINDOW = 128, 16, 4, 64, 128


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            from . import build as _b
            _b.build()
        L = C.CDLL(_LIB_PATH)
        L.oracle_e2m1_value.argtypes = [C.c_uint8]
        L.oracle_e2m1_value.restype = C.c_double
        L.oracle_e4m3_value.argtypes = [C.c_uint8]
        L.oracle_e4m3_value.restype = C.c_double
        L.oracle_e4m3_encode.argtypes = [C.c_float]
        L.oracle_e4m3_encode.restype = C.c_uint8
        L.oracle_fp4_group.argtypes = [_f32p, _u8p, _u8p]
        L.oracle_fp4_group.restype = None
        L.oracle_record_bytes.restype = C.c_int
        L.oracle_quantize_kv.argtypes = [
            _u8p, C.c_void_p, C.c_float, C.c_int64, C.c_int32, C.c_void_p, C.c_void_p,
            C.c_float, C.c_float, C.c_int32, C.c_int32, _f32p, _f32p, C.c_void_p,
            C.c_void_p, C.c_void_p, _i32p, _i64p, C.c_int64]
        L.oracle_quantize_kv.restype = None
        L.oracle_compress_kv.argtypes = (L.oracle_quantize_kv.argtypes[:11] +
                                         [C.c_void_p, C.c_void_p] +
                                         L.oracle_quantize_kv.argtypes[13:] + [C.c_int32])
        L.oracle_compress_kv.restype = None
        L.oracle_index_score.argtypes = [_u8p, C.c_float, _f32p, _f32p]
        L.oracle_index_score.restype = C.c_double
        L.oracle_score_range.argtypes = [_u8p, C.c_float, _f32p, _f32p, C.c_int64, _f64p]
        L.oracle_score_range.restype = None
        L.oracle_topk.argtypes = [_f64p, C.c_void_p, C.c_int64, C.c_int32, _i32p,
                                  C.POINTER(C.c_double)]
        L.oracle_topk.restype = C.c_int32
        L.oracle_index_full.argtypes = [
            _u8p, C.c_float, C.c_int64, _f32p, _f32p, _i32p, _i64p, C.c_int32, C.c_int32,
            C.c_int32, C.c_int32, _i32p, _i32p, _f64p, _f64p]
        L.oracle_index_full.restype = None
        L.oracle_index_reindex.argtypes = [
            _u8p, C.c_float, C.c_int64, _f32p, _f32p, _i32p, _i64p, C.c_int32, _i32p,
            C.c_int32, C.c_int32, C.c_int32, _i32p, _f64p]
        L.oracle_index_reindex.restype = None
        L.oracle_decode_attn.argtypes = [
            _u8p, C.c_int64, _u8p, _u8p, C.c_float, C.c_float, C.c_int32, C.c_int32,
            C.c_int32, _f32p, _i32p, _i32p, _i64p, C.c_int32, C.c_int32, C.c_float, _f32p]
        L.oracle_decode_attn.restype = None
        _lib = L
    return _lib


def _c(a, dt):
    return np.ascontiguousarray(a, dtype=dt)


def _ptr(a):
    return None if a is None else a.ctypes.data


# ----------------------------------------------------------------- codecs

def e2m1_value(nib: int) -> float:
    return lib().oracle_e2m1_value(nib)


def e4m3_value(code: int) -> float:
    return lib().oracle_e4m3_value(code)


def e4m3_encode(x: float) -> int:
    return lib().oracle_e4m3_encode(x)


def e4m3_encode_array(x: np.ndarray) -> np.ndarray:
    f = lib().oracle_e4m3_encode
    return np.array([f(float(v)) for v in np.asarray(x, np.float32).ravel()],
                    np.uint8).reshape(np.shape(x))


def fp4_group(x16: np.ndarray):
    """(nibbles[16], scale_code) of one 16-channel group."""
    x = _c(x16, np.float32)
    assert x.shape == (16,)
    nib = np.zeros(16, np.uint8)
    sc = np.zeros(1, np.uint8)
    lib().oracle_fp4_group(x, nib, sc)
    return nib, int(sc[0])


def record_bytes() -> int:
    return lib().oracle_record_bytes()


# ------------------------------------------------------------ cache store

class Cache:
    """Host-side compressed cache in the library's documented layouts."""

    def __init__(self, n_seq, cap, n_layers=1, w_cap=WINDOW, idxk_scale=1.0,
                 wk_scale=1.0, wv_scale=1.0):
        self.n_seq, self.cap, self.n_layers, self.w_cap = n_seq, cap, n_layers, w_cap
        self.idxk_scale, self.wk_scale, self.wv_scale = idxk_scale, wk_scale, wv_scale
        self.kv = np.zeros((n_seq, cap, REC), np.uint8)
        self.idxk = np.zeros((n_seq, cap, DI), np.uint8)
        self.wk = np.zeros((n_layers, n_seq, w_cap, D), np.uint8)
        self.wv = np.zeros((n_layers, n_seq, w_cap, D), np.uint8)

    def quantize(self, k, v, idx_k, win_k, win_v, seq, pos):
        """Write n rows; win_k / win_v are [n_layers, n, 128] or None."""
        k, v = _c(k, np.float32), _c(v, np.float32)
        n = k.shape[0]
        idx_k = None if idx_k is None else _c(idx_k, np.float32)
        win_k = None if win_k is None else _c(win_k, np.float32)
        win_v = None if win_v is None else _c(win_v, np.float32)
        seq, pos = _c(seq, np.int32), _c(pos, np.int64)
        assert pos.size == n and seq.size == n
        assert np.all((pos >= 0) & (pos < self.cap)) and np.all((seq >= 0) & (seq < self.n_seq))
        if win_k is not None:
            assert win_k.shape == (self.n_layers, n, D) and win_v.shape == win_k.shape
        lib().oracle_quantize_kv(
            self.kv, _ptr(self.idxk), self.idxk_scale, self.cap, self.n_seq,
            _ptr(self.wk), _ptr(self.wv), self.wk_scale, self.wv_scale, self.w_cap,
            self.n_layers, k, v, _ptr(idx_k), _ptr(win_k), _ptr(win_v), seq, pos, n)

    def compress(self, k, v, idx_k, win_k, win_v, seq, pos, m):
        """Write n tokens at compression m (1 or 2): rows i*m .. i*m+m-1 (token
        positions m*e .. m*e+m-1 of one sequence) become global entry e = pos[i*m] / m,
        their fp32 mean quantised like a token row; window rows for every token.
        k = v = None (idx_k None): window rows only."""
        n = win_k.shape[1] if k is None else k.shape[0]
        assert m in (1, 2) and (k is None or n % m == 0)
        assert (k is None) == (v is None) and (k is not None or idx_k is None)
        k = None if k is None else _c(k, np.float32)
        v = None if v is None else _c(v, np.float32)
        idx_k = None if idx_k is None else _c(idx_k, np.float32)
        win_k = None if win_k is None else _c(win_k, np.float32)
        win_v = None if win_v is None else _c(win_v, np.float32)
        seq, pos = _c(seq, np.int32), _c(pos, np.int64)
        assert pos.size == n and seq.size == n
        assert np.all((pos >= 0) & (pos < m * self.cap)) and np.all((seq >= 0) & (seq < self.n_seq))
        if win_k is not None:
            assert win_k.shape == (self.n_layers, n, D) and win_v.shape == win_k.shape
        lib().oracle_compress_kv(
            self.kv, _ptr(self.idxk), self.idxk_scale, self.cap, self.n_seq,
            _ptr(self.wk), _ptr(self.wv), self.wk_scale, self.wv_scale, self.w_cap,
            self.n_layers, _ptr(k), _ptr(v), _ptr(idx_k), _ptr(win_k), _ptr(win_v), seq, pos,
            n, m)

    # -- indexer
    def scores(self, seq: int, q_idx, w, N: int) -> np.ndarray:
        out = np.zeros(max(N, 1), np.float64)
        lib().oracle_score_range(np.ascontiguousarray(self.idxk[seq]), self.idxk_scale,
                                 _c(q_idx, np.float32).reshape(-1), _c(w, np.float32).reshape(-1),
                                 N, out)
        return out[:N]

    def index_full(self, q_idx, w, seq, ctx, n_blocks=2048, block=8, topk=512):
        q_idx, w = _c(q_idx, np.float32), _c(w, np.float32)
        seq, ctx = _c(seq, np.int32), _c(ctx, np.int64)
        B = seq.size
        assert np.all(ctx <= self.cap) and np.all(ctx >= 0)
        pool = np.zeros((B, n_blocks), np.int32)
        idx = np.zeros((B, topk), np.int32)
        kb = np.zeros(B, np.float64)
        kp = np.zeros(B, np.float64)
        lib().oracle_index_full(self.idxk, self.idxk_scale, self.cap, q_idx, w, seq, ctx, B,
                                n_blocks, block, topk, pool, idx, kb, kp)
        return pool, idx, kb, kp

    def index_reindex(self, q_idx, w, seq, ctx, pool, block=8, topk=512):
        q_idx, w = _c(q_idx, np.float32), _c(w, np.float32)
        seq, ctx, pool = _c(seq, np.int32), _c(ctx, np.int64), _c(pool, np.int32)
        B, n_blocks = pool.shape
        idx = np.zeros((B, topk), np.int32)
        kp = np.zeros(B, np.float64)
        lib().oracle_index_reindex(self.idxk, self.idxk_scale, self.cap, q_idx, w, seq, ctx,
                                   B, pool, n_blocks, block, topk, idx, kp)
        return idx, kp

    # -- attention
    def decode_attn(self, layer, q, idx, seq, ctx, sm_scale=None):
        q, idx = _c(q, np.float32), _c(idx, np.int32)
        seq, ctx = _c(seq, np.int32), _c(ctx, np.int64)
        B, topk = idx.shape
        assert q.shape == (B, H, D)
        if sm_scale is None:
            sm_scale = float(np.float32(1.0 / np.sqrt(D)))
        out = np.zeros((B, H, D), np.float32)
        lib().oracle_decode_attn(self.kv, self.cap, self.wk, self.wv, self.wk_scale,
                                 self.wv_scale, self.w_cap, self.n_seq, layer, q, idx, seq,
                                 ctx, B, topk, sm_scale, out)
        return out


def topk(values, k, ids=None):
    """(ascending indices padded with -1, count, k-th value) of the k largest."""
    v = _c(values, np.float64)
    n = v.size
    out = np.zeros(k, np.int32)
    kth = C.c_double()
    idp = None
    if ids is not None:
        idp = _c(ids, np.int64)
    m = lib().oracle_topk(v, _ptr(idp), n, k, out, C.byref(kth))
    return out, m, kth.value
