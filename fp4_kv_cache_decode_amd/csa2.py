"""Thin ctypes binding over libcsa2.so (the C ABI in include/csa2.h).

Argument marshalling only: every step of the decode path runs in the HIP
kernels of libcsa2.  torch supplies device memory and the stream.  If the
library is missing or fails to load, every call raises; there is no fallback.
"""
from __future__ import annotations

import ctypes as C
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libcsa2.so")

OK, ERR_INVALID_ARG, ERR_UNSUPPORTED, ERR_WORKSPACE, ERR_LAUNCH = range(5)
OP_INDEX_FULL, OP_INDEX_REINDEX, OP_DECODE_ATTN, OP_SELECT_POOL = 1, 2, 3, 4
OP_REINDEX_LAYER_FUSED = 5

D, HEADS, IDX_HEADS, IDX_DIM, WINDOW, RECORD, BLOCK = 128, 16, 4, 64, 128, 144, 8


class Csa2Error(RuntimeError):
    def __init__(self, status: int, where: str):
        super().__init__(f"{where}: {status_string(status)} (status {status})")
        self.status = status


class csa2_cache(C.Structure):
    _fields_ = [("kv", C.c_void_p), ("idxk", C.c_void_p), ("idxk_scale", C.c_float),
                ("n_seq", C.c_int32), ("cap", C.c_int64), ("page_table", C.c_void_p),
                ("page_tokens", C.c_int32), ("n_pages", C.c_int32)]


class csa2_window(C.Structure):
    _fields_ = [("k", C.c_void_p), ("v", C.c_void_p), ("k_scale", C.c_float),
                ("v_scale", C.c_float), ("n_layers", C.c_int32), ("n_seq", C.c_int32),
                ("w_cap", C.c_int32)]


_lib = None
_P = C.c_void_p


def lib():
    """Load libcsa2.so (raises OSError when it is not built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise OSError(f"libcsa2.so not built at {LIB_PATH}; run "
                          "`python -m fp4_kv_cache_decode_amd.build`")
        L = C.CDLL(LIB_PATH)
        L.csa2_quantize_kv.argtypes = [C.POINTER(csa2_cache), C.POINTER(csa2_window), _P, _P, _P,
                                       _P, _P, _P, _P, C.c_int64, _P]
        L.csa2_compress_kv.argtypes = [C.POINTER(csa2_cache), C.POINTER(csa2_window), _P, _P, _P,
                                       _P, _P, _P, _P, C.c_int64, C.c_int32, _P]
        L.csa2_index_full.argtypes = [C.POINTER(csa2_cache), _P, _P, _P, _P, C.c_int32, C.c_int64,
                                      C.c_int32, C.c_int32, C.c_int32, _P, _P, _P, C.c_size_t, _P]
        L.csa2_index_reindex.argtypes = [C.POINTER(csa2_cache), _P, _P, _P, _P, C.c_int32, _P,
                                         C.c_int32, C.c_int32, C.c_int32, _P, _P, C.c_size_t, _P]
        L.csa2_index_block_scores.argtypes = [C.POINTER(csa2_cache), _P, _P, _P, _P, C.c_int32,
                                              C.c_int64, _P, C.c_int64, _P]
        L.csa2_index_select_pool.argtypes = [_P, C.c_int64, _P, C.c_int32, C.c_int64, C.c_int32,
                                             _P, _P, C.c_size_t, _P]
        L.csa2_decode_attn.argtypes = [C.POINTER(csa2_cache), C.POINTER(csa2_window), C.c_int32,
                                       _P, _P, _P, _P, C.c_int32, C.c_int32, C.c_float, _P, _P,
                                       C.c_size_t, _P]
        L.csa2_decode_attn_ex.argtypes = [C.POINTER(csa2_cache), C.POINTER(csa2_window),
                                          C.c_int32, _P, _P, _P, _P, C.c_int32, C.c_int32,
                                          C.c_float, _P, _P, _P, _P, C.c_size_t, _P]
        L.csa2_decode_attn_noalloc.argtypes = [C.POINTER(csa2_cache), C.POINTER(csa2_window),
                                               C.c_int32, _P, _P, _P, _P, C.c_int32, C.c_int32,
                                               C.c_float, _P, _P, _P, _P]
        L.csa2_reindex_layer_fused.argtypes = [C.POINTER(csa2_cache), C.POINTER(csa2_window),
                                               C.c_int32, _P, _P, _P, _P, _P, C.c_int32, _P,
                                               C.c_int32, C.c_int32, C.c_int32, C.c_float, _P,
                                               _P, _P, C.c_int32, _P, _P, C.c_size_t, _P]
        L.csa2_workspace_bytes.argtypes = [C.c_int32, C.c_int32, C.c_int64, C.c_int32, C.c_int32,
                                           C.c_int32]
        L.csa2_workspace_bytes.restype = C.c_size_t
        L.csa2_status_string.argtypes = [C.c_int]
        L.csa2_status_string.restype = C.c_char_p
        for f in ("csa2_quantize_kv", "csa2_compress_kv", "csa2_index_full", "csa2_index_reindex",
                  "csa2_decode_attn", "csa2_decode_attn_ex", "csa2_index_block_scores",
                  "csa2_index_select_pool", "csa2_decode_attn_noalloc",
                  "csa2_reindex_layer_fused"):
            getattr(L, f).restype = C.c_int
        _lib = L
    return _lib


def status_string(s: int) -> str:
    return lib().csa2_status_string(s).decode()


def _check(status: int, where: str) -> None:
    if status != OK:
        raise Csa2Error(status, where)


def _ptr(t):
    if t is None:
        return None
    if not isinstance(t, torch.Tensor):
        raise TypeError("expected a torch.Tensor")
    if not t.is_cuda:
        raise ValueError("expected a device tensor")
    if not t.is_contiguous():
        raise ValueError("expected a contiguous tensor")
    return t.data_ptr()


def _need(t, dtype, shape, name):
    if t is None:
        raise ValueError(f"{name} is required")
    if t.dtype != dtype:
        raise TypeError(f"{name}: expected {dtype}, got {t.dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: expected shape {tuple(shape)}, got {tuple(t.shape)}")


def _stream(stream):
    s = torch.cuda.current_stream() if stream is None else stream
    return s.cuda_stream


def workspace_bytes(op: int, B: int, max_ctx: int = 0, n_blocks: int = 2048, block: int = 8,
                    topk: int = 512) -> int:
    return int(lib().csa2_workspace_bytes(op, B, max_ctx, n_blocks, block, topk))


class Cache:
    """Device storage for the compressed cache and the per-layer window stores.

    Allocation goes through torch; the library only receives the pointers.
    With page_tokens > 0 the global store is paged: kv and idxk hold n_pages
    physical pages of page_tokens rows, and page_table[s][j] (int32, on the
    device) names the page that holds positions j*page_tokens.. of sequence s.
    The default table gives sequence s the pages s*cap/page_tokens + j.
    """

    def __init__(self, n_seq: int, cap: int, n_layers: int = 1, w_cap: int = WINDOW,
                 idxk_scale: float = 1.0, wk_scale: float = 1.0, wv_scale: float = 1.0,
                 device="cuda", page_tokens: int = 0, n_pages: int | None = None,
                 page_table=None):
        self.n_seq, self.cap, self.n_layers, self.w_cap = n_seq, cap, n_layers, w_cap
        self.page_tokens = page_tokens
        if page_tokens:
            if cap % page_tokens:
                raise ValueError("cap must be a multiple of page_tokens")
            per_seq = cap // page_tokens
            self.n_pages = n_seq * per_seq if n_pages is None else n_pages
            rows = (self.n_pages, page_tokens)
            if page_table is None:
                page_table = torch.arange(n_seq * per_seq, dtype=torch.int32).view(n_seq, per_seq)
            page_table = torch.as_tensor(page_table, dtype=torch.int32)
            if tuple(page_table.shape) != (n_seq, per_seq):
                raise ValueError(f"page_table: expected shape {(n_seq, per_seq)}")
            self.page_table = page_table.to(device).contiguous()
        else:
            self.n_pages, rows, self.page_table = 0, (n_seq, cap), None
        self.kv = torch.zeros((*rows, RECORD), dtype=torch.uint8, device=device)
        self.idxk = torch.zeros((*rows, IDX_DIM), dtype=torch.uint8, device=device)
        self.wk = torch.zeros((n_layers, n_seq, w_cap, D), dtype=torch.uint8, device=device)
        self.wv = torch.zeros_like(self.wk)
        pt = self.page_table.data_ptr() if page_tokens else None
        self.c = csa2_cache(self.kv.data_ptr(), self.idxk.data_ptr(), idxk_scale, n_seq, cap,
                            pt, page_tokens, self.n_pages)
        self.w = csa2_window(self.wk.data_ptr(), self.wv.data_ptr(), wk_scale, wv_scale,
                             n_layers, n_seq, w_cap)


def quantize_kv(cache: Cache, k, v, seq, pos, idx_k=None, win_k=None, win_v=None,
                stream=None) -> None:
    n = k.shape[0]
    _need(k, torch.float32, (n, D), "k")
    _need(v, torch.float32, (n, D), "v")
    _need(seq, torch.int32, (n,), "seq")
    _need(pos, torch.int64, (n,), "pos")
    if idx_k is not None:
        _need(idx_k, torch.float32, (n, IDX_DIM), "idx_k")
    if win_k is not None:
        _need(win_k, torch.float32, (cache.n_layers, n, D), "win_k")
        _need(win_v, torch.float32, (cache.n_layers, n, D), "win_v")
    st = lib().csa2_quantize_kv(C.byref(cache.c), C.byref(cache.w), _ptr(k), _ptr(v),
                                _ptr(idx_k), _ptr(win_k), _ptr(win_v), _ptr(seq), _ptr(pos), n,
                                _stream(stream))
    _check(st, "csa2_quantize_kv")


def compress_kv(cache: Cache, k, v, seq, pos, m: int, idx_k=None, win_k=None, win_v=None,
                stream=None) -> None:
    """csa2_compress_kv: n tokens; rows i*m .. i*m+m-1 become global entry
    pos[i*m] / m (their fp32 mean, quantised); window rows for every token.
    k = v = None: window rows only."""
    n = win_k.shape[1] if k is None else k.shape[0]
    if k is not None or v is not None:
        _need(k, torch.float32, (n, D), "k")
        _need(v, torch.float32, (n, D), "v")
    _need(seq, torch.int32, (n,), "seq")
    _need(pos, torch.int64, (n,), "pos")
    if idx_k is not None:
        _need(idx_k, torch.float32, (n, IDX_DIM), "idx_k")
    if win_k is not None:
        _need(win_k, torch.float32, (cache.n_layers, n, D), "win_k")
        _need(win_v, torch.float32, (cache.n_layers, n, D), "win_v")
    st = lib().csa2_compress_kv(C.byref(cache.c), C.byref(cache.w), _ptr(k), _ptr(v),
                                _ptr(idx_k), _ptr(win_k), _ptr(win_v), _ptr(seq), _ptr(pos), n,
                                m, _stream(stream))
    _check(st, "csa2_compress_kv")


def index_full(cache: Cache, q_idx, w, seq, ctx, max_ctx: int, pool, idx, ws,
               n_blocks: int = 2048, block: int = 8, topk: int = 512, stream=None) -> None:
    B = q_idx.shape[0]
    _need(q_idx, torch.float32, (B, IDX_HEADS, IDX_DIM), "q_idx")
    _need(w, torch.float32, (B, IDX_HEADS), "w")
    _need(seq, torch.int32, (B,), "seq")
    _need(ctx, torch.int64, (B,), "ctx")
    _need(idx, torch.int32, (B, topk), "idx")
    if pool is not None:
        _need(pool, torch.int32, (B, n_blocks), "pool")
    _need(ws, torch.uint8, None, "ws")
    st = lib().csa2_index_full(C.byref(cache.c), _ptr(q_idx), _ptr(w), _ptr(seq), _ptr(ctx), B,
                               max_ctx, n_blocks, block, topk, _ptr(pool), _ptr(idx), _ptr(ws),
                               ws.numel(), _stream(stream))
    _check(st, "csa2_index_full")


def block_stride(max_ctx: int) -> int:
    """Row stride (floats) for block scores of contexts up to max_ctx."""
    nb = -(-max_ctx // BLOCK)
    return -(-nb // 64) * 64


def index_block_scores(cache: Cache, q_idx, w, seq, ctx, max_ctx: int, M, stream=None) -> None:
    B = q_idx.shape[0]
    _need(q_idx, torch.float32, (B, IDX_HEADS, IDX_DIM), "q_idx")
    _need(w, torch.float32, (B, IDX_HEADS), "w")
    _need(seq, torch.int32, (B,), "seq")
    _need(ctx, torch.int64, (B,), "ctx")
    _need(M, torch.float32, None, "M")
    if M.dim() != 2 or M.shape[0] != B:
        raise ValueError("M: expected [B, m_stride]")
    st = lib().csa2_index_block_scores(C.byref(cache.c), _ptr(q_idx), _ptr(w), _ptr(seq),
                                       _ptr(ctx), B, max_ctx, _ptr(M), M.shape[1],
                                       _stream(stream))
    _check(st, "csa2_index_block_scores")


def index_select_pool(M, ctx, max_ctx: int, pool, ws=None, stream=None) -> None:
    B, n_blocks = pool.shape
    _need(M, torch.float32, None, "M")
    _need(ctx, torch.int64, (B,), "ctx")
    _need(pool, torch.int32, (B, n_blocks), "pool")
    if ws is not None:
        _need(ws, torch.uint8, None, "ws")
    st = lib().csa2_index_select_pool(_ptr(M), M.shape[1], _ptr(ctx), B, max_ctx, n_blocks,
                                      _ptr(pool), _ptr(ws), 0 if ws is None else ws.numel(),
                                      _stream(stream))
    _check(st, "csa2_index_select_pool")


def index_reindex(cache: Cache, q_idx, w, seq, ctx, pool, idx, ws, block: int = 8,
                  topk: int = 512, stream=None) -> None:
    B = q_idx.shape[0]
    n_blocks = pool.shape[1]
    _need(q_idx, torch.float32, (B, IDX_HEADS, IDX_DIM), "q_idx")
    _need(w, torch.float32, (B, IDX_HEADS), "w")
    _need(seq, torch.int32, (B,), "seq")
    _need(ctx, torch.int64, (B,), "ctx")
    _need(pool, torch.int32, (B, n_blocks), "pool")
    _need(idx, torch.int32, (B, topk), "idx")
    _need(ws, torch.uint8, None, "ws")
    st = lib().csa2_index_reindex(C.byref(cache.c), _ptr(q_idx), _ptr(w), _ptr(seq), _ptr(ctx),
                                  B, _ptr(pool), n_blocks, block, topk, _ptr(idx), _ptr(ws),
                                  ws.numel(), _stream(stream))
    _check(st, "csa2_index_reindex")


def decode_attn(cache: Cache, layer: int, q, idx, seq, ctx, out, ws, sm_scale=None,
                stream=None, kvg_in=None, kvg_out=None) -> None:
    """csa2_decode_attn; with kvg_out / kvg_in ([B][topk][144] uint8) it is
    csa2_decode_attn_ex, storing / reading the group's gathered main records."""
    B, topk = idx.shape
    _need(q, torch.float32, (B, HEADS, D), "q")
    _need(idx, torch.int32, (B, topk), "idx")
    _need(seq, torch.int32, (B,), "seq")
    _need(ctx, torch.int64, (B,), "ctx")
    _need(out, torch.float32, (B, HEADS, D), "out")
    _need(ws, torch.uint8, None, "ws")
    for name, g in (("kvg_in", kvg_in), ("kvg_out", kvg_out)):
        if g is not None:
            _need(g, torch.uint8, (B, topk, RECORD), name)
    if sm_scale is None:
        sm_scale = float(torch.tensor(D ** -0.5, dtype=torch.float32))
    L = lib()
    if kvg_in is None and kvg_out is None:
        st = L.csa2_decode_attn(C.byref(cache.c), C.byref(cache.w), layer, _ptr(q), _ptr(idx),
                                _ptr(seq), _ptr(ctx), B, topk, sm_scale, _ptr(out), _ptr(ws),
                                ws.numel(), _stream(stream))
        _check(st, "csa2_decode_attn")
        return
    st = L.csa2_decode_attn_ex(C.byref(cache.c), C.byref(cache.w), layer, _ptr(q), _ptr(idx),
                               _ptr(seq), _ptr(ctx), B, topk, sm_scale,
                               _ptr(kvg_in), _ptr(kvg_out), _ptr(out),
                               _ptr(ws), ws.numel(), _stream(stream))
    _check(st, "csa2_decode_attn_ex")


def decode_attn_noalloc(cache: Cache, layer: int, q, idx, seq, ctx, out, sm_scale=None,
                        stream=None, kvg_in=None, kvg_out=None) -> None:
    """csa2_decode_attn_noalloc: decode_attn with no workspace (the library's
    fixed per-GPU scratch holds the partial records)."""
    B, topk = idx.shape
    _need(q, torch.float32, (B, HEADS, D), "q")
    _need(idx, torch.int32, (B, topk), "idx")
    _need(seq, torch.int32, (B,), "seq")
    _need(ctx, torch.int64, (B,), "ctx")
    _need(out, torch.float32, (B, HEADS, D), "out")
    for name, g in (("kvg_in", kvg_in), ("kvg_out", kvg_out)):
        if g is not None:
            _need(g, torch.uint8, (B, topk, RECORD), name)
    if sm_scale is None:
        sm_scale = float(torch.tensor(D ** -0.5, dtype=torch.float32))
    st = lib().csa2_decode_attn_noalloc(C.byref(cache.c), C.byref(cache.w), layer, _ptr(q),
                                        _ptr(idx), _ptr(seq), _ptr(ctx), B, topk, sm_scale,
                                        _ptr(kvg_in), _ptr(kvg_out), _ptr(out), _stream(stream))
    _check(st, "csa2_decode_attn_noalloc")


def reindex_layer_fused(cache: Cache, layer: int, q_idx, w, q, seq, ctx, pool, idx, out, ws,
                        status, kvg_out=None, sm_scale=None, max_polls: int = 0,
                        block: int = 8, stream=None) -> None:
    """csa2_reindex_layer_fused: index_reindex then decode_attn (with kvg_out)
    in one cooperative launch.  ws (uint8, OP_REINDEX_LAYER_FUSED bytes) must be
    zero-filled before its first use; status (int32 [1]) is ORed with 1 when a
    grid barrier gave up."""
    B, topk = idx.shape
    n_blocks = pool.shape[1]
    _need(q_idx, torch.float32, (B, IDX_HEADS, IDX_DIM), "q_idx")
    _need(w, torch.float32, (B, IDX_HEADS), "w")
    _need(q, torch.float32, (B, HEADS, D), "q")
    _need(seq, torch.int32, (B,), "seq")
    _need(ctx, torch.int64, (B,), "ctx")
    _need(pool, torch.int32, (B, n_blocks), "pool")
    _need(idx, torch.int32, (B, topk), "idx")
    _need(out, torch.float32, (B, HEADS, D), "out")
    _need(ws, torch.uint8, None, "ws")
    _need(status, torch.int32, (1,), "status")
    if kvg_out is not None:
        _need(kvg_out, torch.uint8, (B, topk, RECORD), "kvg_out")
    if sm_scale is None:
        sm_scale = float(torch.tensor(D ** -0.5, dtype=torch.float32))
    st = lib().csa2_reindex_layer_fused(C.byref(cache.c), C.byref(cache.w), layer, _ptr(q_idx),
                                        _ptr(w), _ptr(q), _ptr(seq), _ptr(ctx), B, _ptr(pool),
                                        n_blocks, block, topk, sm_scale, _ptr(idx),
                                        _ptr(kvg_out), _ptr(out), max_polls, _ptr(status),
                                        _ptr(ws), ws.numel(), _stream(stream))
    _check(st, "csa2_reindex_layer_fused")


def alloc_workspace(op: int, B: int, max_ctx: int = 0, n_blocks: int = 2048, topk: int = 512,
                    device="cuda") -> torch.Tensor:
    n = workspace_bytes(op, B, max_ctx, n_blocks, BLOCK, topk)
    if n == 0 and B > 0 and op not in (OP_SELECT_POOL, OP_DECODE_ATTN):   # these may need none
        raise Csa2Error(ERR_INVALID_ARG, "csa2_workspace_bytes")
    return torch.empty(max(n, 1), dtype=torch.uint8, device=device)
