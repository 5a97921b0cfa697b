"""Seeded synthetic inputs for CSA2 decode over a compressed global KV cache.

This module only draws random numbers and lays them out. It holds none of the
method's arithmetic (no quantisation, scoring, selection or attention), so the
CPU oracle and the HIP path can both consume its output without sharing code.

Workloads follow the shapes the pages give for the decoder (origotech.dev deep
dive "Inside DeepSeek V4.1-Flash: KV cache, 1017 update, Harness stack",
section "How the architecture shrinks the KV cache": top-k 512, a 128-token
sliding window, 2,048 blocks of 8 positions, the 20-layer decoder pattern
[Full + 3 Reuse] + 4 x [Reindex + 3 Reuse]).  Value distributions:
  * main K/V rows, indexer keys and window rows: N(0,1) with ceil(1% of the
    channels) fixed outlier channels scaled by 8;
  * RoPE (interleaved pairs, base 1e4) on the first 64 K channels, so the rows
    handed to the quantiser are post-RoPE as the pages require;
  * attention and indexer queries: N(0,1); indexer head weights: U(0,1).

Every tensor is drawn from its own PCG64 stream keyed by
(seed, tensor id, layer, sequence, chunk), with positions generated in fixed
chunks of ``CHUNK`` rows, so any position range can be regenerated alone.
"""
from __future__ import annotations

import math
import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field

import numpy as np

# Shapes fixed by the pages / the workloads.
D = 128          # K and V channels (one shared KV head)
H = 16           # attention heads
HI = 4           # indexer heads
DI = 64          # indexer dims
WINDOW = 128     # sliding-window tokens
TOPK = 512       # selected global positions
N_BLOCKS = 2048  # candidate-pool blocks
BLOCK = 8        # positions per block
ROPE_DIMS = 64   # K channels that carry RoPE
ROPE_BASE = 10000.0
OUTLIER_FRAC = 0.01
OUTLIER_GAIN = 8.0

CHUNK = 65536    # rows per generator chunk

# tensor ids for stream keys
_K, _V, _IDXK, _WINK, _WINV, _Q, _QIDX, _W, _OUTL, _PAGES = range(10)


def _rng(seed: int, *key: int) -> np.random.Generator:
    ss = np.random.SeedSequence(entropy=seed, spawn_key=tuple(int(k) for k in key))
    return np.random.Generator(np.random.PCG64(ss))


def outlier_channels(seed: int, kind: int, width: int, layer: int = 0) -> np.ndarray:
    """The ceil(1%) outlier channels of one tensor kind (fixed across positions)."""
    n = max(1, math.ceil(OUTLIER_FRAC * width))
    return np.sort(_rng(seed, _OUTL, kind, layer).choice(width, size=n, replace=False))


def _normal_rows(seed: int, kind: int, layer: int, seq: int, p0: int, p1: int,
                 width: int) -> np.ndarray:
    """N(0,1) rows for positions [p0, p1), drawn chunk by chunk."""
    out = np.empty((p1 - p0, width), np.float32)
    c0, c1 = p0 // CHUNK, (p1 - 1) // CHUNK if p1 > p0 else p0 // CHUNK - 1
    for c in range(c0, c1 + 1):
        lo = max(p0, c * CHUNK)
        hi = min(p1, (c + 1) * CHUNK)
        # the generator fills row-major, so drawing only the chunk's first
        # hi - c*CHUNK rows yields the same values as drawing the whole chunk
        blk = _rng(seed, kind, layer, seq, c).standard_normal((hi - c * CHUNK, width),
                                                              dtype=np.float32)
        out[lo - p0:hi - p0] = blk[lo - c * CHUNK:]
    cols = outlier_channels(seed, kind, width, layer)
    out[:, cols] *= np.float32(OUTLIER_GAIN)
    return out


def _rope_inplace(x: np.ndarray, pos: np.ndarray) -> None:
    """Rotate interleaved channel pairs (2i, 2i+1), i < ROPE_DIMS/2, by pos*theta_i."""
    half = ROPE_DIMS // 2
    inv = ROPE_BASE ** (-np.arange(half, dtype=np.float64) * 2.0 / ROPE_DIMS)
    ang = pos.astype(np.float64)[:, None] * inv[None, :]
    c, s = np.cos(ang), np.sin(ang)
    a = x[:, 0:ROPE_DIMS:2].astype(np.float64)
    b = x[:, 1:ROPE_DIMS:2].astype(np.float64)
    x[:, 0:ROPE_DIMS:2] = (a * c - b * s).astype(np.float32)
    x[:, 1:ROPE_DIMS:2] = (a * s + b * c).astype(np.float32)


def kv_rows(seed: int, seq: int, p0: int, p1: int, group: int = 0):
    """Post-RoPE main K, main V [n,128] and indexer keys [n,64] for positions [p0,p1).
    group: which layer group's main KV (each Full layer of the encoder has its own)."""
    k = _normal_rows(seed, _K, group, seq, p0, p1, D)
    _rope_inplace(k, np.arange(p0, p1))
    v = _normal_rows(seed, _V, group, seq, p0, p1, D)
    ik = _normal_rows(seed, _IDXK, group, seq, p0, p1, DI)
    return k, v, ik


def window_rows(seed: int, layer: int, seq: int, p0: int, p1: int):
    """One layer's sliding-window K (post-RoPE) and V rows [n,128] for [p0,p1)."""
    k = _normal_rows(seed, _WINK, layer, seq, p0, p1, D)
    _rope_inplace(k, np.arange(p0, p1))
    v = _normal_rows(seed, _WINV, layer, seq, p0, p1, D)
    return k, v


def attn_queries(seed: int, layer: int, n: int, stream: int = 0) -> np.ndarray:
    """Attention queries [n,16,128], N(0,1)."""
    return _rng(seed, _Q, layer, stream).standard_normal((n, H, D), dtype=np.float32)


def index_queries(seed: int, layer: int, n: int, stream: int = 0):
    """Indexer queries [n,4,64] ~ N(0,1) and head weights [n,4] ~ U(0,1)."""
    q = _rng(seed, _QIDX, layer, stream).standard_normal((n, HI, DI), dtype=np.float32)
    w = _rng(seed, _W, layer, stream).random((n, HI), dtype=np.float32)
    return q, w


def page_table(seed: int, n_seq: int, cap: int, page_tokens: int, n_used, spare: int = 3):
    """A fragmented page layout for a paged cache: sequence s owns its first
    ceil(n_used[s] / page_tokens) logical pages, scattered over a shuffled pool
    of physical pages that also holds `spare` pages nobody owns; its remaining
    logical pages are -1.  Returns (table [n_seq][cap // page_tokens] int32,
    n_pages)."""
    per = cap // page_tokens
    need = [-(-int(n) // page_tokens) for n in n_used]
    n_pages = sum(need) + spare
    perm = _rng(seed, _PAGES, n_seq, page_tokens).permutation(n_pages).astype(np.int32)
    table = np.full((n_seq, per), -1, np.int32)
    at = 0
    for s in range(n_seq):
        table[s, :need[s]] = perm[at:at + need[s]]
        at += need[s]
    return table, n_pages


# ---------------------------------------------------------------------------
# Workloads
# ---------------------------------------------------------------------------

DECODER_20 = ("F", "R", "R", "R") + ("I", "R", "R", "R") * 4
# the encoder (same section): layers 1-2 sliding-window attention only ('S'),
# then 18 CSA2 layers at compression m = 2 as 3 x [Full + 5 Reuse]
ENCODER_20 = ("S", "S") + ("F", "R", "R", "R", "R", "R") * 3


@dataclass(frozen=True)
class Workload:
    """One synthetic workload: B queries over caches of N positions.

    layers: per-layer CSA2 mode, 'F' (Full), 'I' (Reindex), 'R' (Reuse), or 'S'
    (sliding window only).
    prefill: if set, the B queries are consecutive causal positions of one
    sequence starting at N (the chunk is written before the queries run).
    m: global-KV compression (tokens per global entry); each Full layer then
    keeps its own global store of cap // m entries.
    """
    name: str
    B: int
    N: int
    layers: tuple
    prefill: bool = False
    w_cap: int = WINDOW
    m: int = 1
    extra: dict = field(default_factory=dict)

    @property
    def n_seq(self) -> int:
        return 1 if self.prefill else self.B

    @property
    def cap(self) -> int:
        return self.N + (self.B if self.prefill else 0)

    def ctx(self) -> np.ndarray:
        """Visible positions per query (the current token included)."""
        if self.prefill:
            return self.N + 1 + np.arange(self.B, dtype=np.int64)
        return np.full(self.B, self.N, np.int64)

    def seq(self) -> np.ndarray:
        if self.prefill:
            return np.zeros(self.B, np.int32)
        return np.arange(self.B, dtype=np.int32)

    def index_layers(self):
        return [i for i, m in enumerate(self.layers) if m in "FI"]


WORKLOADS = {
    "full_4k_b1": Workload("full_4k_b1", B=1, N=4096, layers=("F",)),
    "group_64k_b32": Workload("group_64k_b32", B=32, N=65536, layers=("F", "R", "R", "R")),
    "hier_256k_b8": Workload("hier_256k_b8", B=8, N=262144,
                             layers=("F", "I", "R", "R", "R")),
    "decoder20_1m_b4": Workload("decoder20_1m_b4", B=4, N=1048576, layers=DECODER_20),
    # one Full layer and nothing after it: no Reindex layer needs the 2,048-block
    # pool, so the layer keeps TOPK blocks (all its top-k positions lie in them)
    "prefill_8k_over_128k": Workload("prefill_8k_over_128k", B=8192, N=131072,
                                     layers=("F",), prefill=True, w_cap=16384,
                                     extra={"pool_blocks": TOPK}),
    # likewise the encoder's Full layers, which serve no Reindex layer
    "encoder20_m2_chunk8k_over_128k": Workload("encoder20_m2_chunk8k_over_128k", B=8192,
                                               N=131072, layers=ENCODER_20, prefill=True,
                                               w_cap=16384, m=2,
                                               extra={"pool_blocks": TOPK}),
}


def parallel_map(fn, items, workers: int | None = None):
    """Thread-parallel map for the chunked generators (numpy releases the GIL)."""
    workers = workers or min(16, os.cpu_count() or 1)
    with ThreadPoolExecutor(workers) as ex:
        return list(ex.map(fn, items))
