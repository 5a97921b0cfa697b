#!/usr/bin/env python3
"""CSA2 decode benchmark on one MI355X.

A step is one decode token for every sequence of the workload through the
whole hot path: quantise-on-write of the new token (main KV, indexer key and
the window rows of every layer), the Full layer's indexer (block scores, the
2,048-block pool, top-512), the Reindex layers, and the gather/dequant
attention of every layer (Reuse layers pass the group's index list unchanged).

Default workload: the 20-layer decoder pattern [Full + 3 Reuse] + 4 x
[Reindex + 3 Reuse] at 1,048,576 cached tokens, batch 4, seeded synthetic
data.  Inputs are resident in HBM before the timed region; steps rotate over
cache replicas so the 268 MB indexer-key set is re-read from HBM every step
rather than from the 256 MB Infinity Cache.

Prints one JSON line (rank 0) with queries/s and the HBM roofline of the whole
decode step (the step's algorithmic bytes over its measured time), with the
Full layer's indexer scan, the step's largest single kernel by bytes, timed on
its own with HIP events on the launch stream and reported beside it; and the
CPU oracle timed on a bounded sample on the host, at one thread and at the
host's thread count.
"""
from __future__ import annotations

import argparse
import math
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402

PEAK_HBM_GBS = 8000.0
PEAK_FP32_TFS = 157.3      # MI355X published fp32 vector peak (packed FMA)
METRIC = "CSA2 decode queries/s at 1M ctx + achieved HBM GB/s as % of MI355X peak"
# the scan kernel's sources: its file and the scoring core it shares
SCORE_SRC = ",".join(os.path.join("fp4_kv_cache_decode_amd", "csrc", f)
                     for f in ("index_score.hip", "score_dev.h"))
COUNTER_FILE = os.path.join(ROOT, "profiles", "scan_decoder20_1m_b4_counters.txt")
STEP_COUNTER_FILE = os.path.join(ROOT, "profiles", "decoder20_1m_b4_step_counters.txt")
CSRC = os.path.join(ROOT, "fp4_kv_cache_decode_amd", "csrc")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def code_hash(text: str) -> str:
    """First 16 hex digits of the SHA-256 of a C++ source's code: // comments,
    trailing blanks and empty lines removed, so that editing a comment does not
    retire counters taken on the same code."""
    lines = []
    for line in text.splitlines():
        line = re.sub(r"//.*$", "", line).rstrip()
        if line:
            lines.append(line)
    return hashlib.sha256("\n".join(lines).encode()).hexdigest()[:16]


def source_hash(paths=SCORE_SRC) -> str:
    """Code hash of one source, or of a comma-separated list of sources
    (relative to the repository root), in the order given."""
    parts = []
    for p in paths.split(","):
        with open(os.path.join(ROOT, p), encoding="utf-8") as f:
            parts.append(f.read())
    return code_hash("\n".join(parts))


def counter_traffic(workload: str):
    """HBM bytes per scoring launch from committed rocprofv3 counters, scaled by
    the copy-kernel calibration; None if absent or the kernel source changed."""
    if not os.path.exists(COUNTER_FILE):
        return None
    txt = open(COUNTER_FILE).read()
    kv = dict(re.findall(r"^(\w+)\s*=\s*(\S+)\s*$", txt, flags=re.M))
    if kv.get("workload") != workload or kv.get("source_sha256") != source_hash():
        return None
    try:
        fetch = float(kv["score_fetch_kib"]) * 1024 * float(kv["copy_fetch_factor"])
        write = float(kv["score_write_kib"]) * 1024 * float(kv["copy_write_factor"])
    except (KeyError, ValueError):
        return None
    return fetch + write


def step_alg_bytes(wl) -> int:
    """Algorithmic HBM bytes of one decode step: what the method itself must
    read or write once per step, whatever the kernels' intermediates.  Per
    query: the Full layer's scan over N indexer keys (64 B each), each Reindex
    layer's 2,048 pool blocks of 8 keys, one gather of topk 144-byte records per
    Full or Reindex layer (its Reuse layers take the same rows), every layer's
    128 window rows (K and V, 128 B each) and its query and output (16 x 128
    fp32 each)."""
    from fp4_kv_cache_decode_amd import datagen as G
    n_full = sum(m == "F" for m in wl.layers)
    n_reindex = sum(m == "I" for m in wl.layers)
    per_q = (n_full * wl.N * G.DI +
             n_reindex * G.N_BLOCKS * G.BLOCK * G.DI +
             (n_full + n_reindex) * G.TOPK * 144 +
             len(wl.layers) * (G.WINDOW * 2 * G.D + 2 * G.H * G.D * 4))
    return wl.B * per_q


# the sources of the decode step's kernels (the device code of every kernel the
# step launches, and the helpers it includes)
STEP_SOURCES = ",".join(os.path.join("fp4_kv_cache_decode_amd", "csrc", f) for f in (
    "csa2_device.h", "quantize.hip", "index_score.hip", "score_dev.h", "topk.hip", "topk_dev.h",
    "attn.hip", "attn_dev.h"))


def step_counter_traffic(workload: str):
    """HBM bytes of one whole decode step from committed per-kernel counters:
    the sum over the step's kernels of calls x (FETCH_SIZE x fetch factor +
    WRITE_SIZE x write factor), in KiB per dispatch; None if the file is
    absent, names another workload, or the step kernels' sources changed since."""
    if not os.path.exists(STEP_COUNTER_FILE):
        return None
    txt = open(STEP_COUNTER_FILE).read()
    kv = dict(re.findall(r"^(\w+)\s*=\s*(\S+)\s*$", txt, flags=re.M))
    if kv.get("workload") != workload or kv.get("sources") != STEP_SOURCES:
        return None
    if kv.get("source_sha256") != source_hash(STEP_SOURCES):
        return None
    try:
        ff, wf = float(kv["copy_fetch_factor"]), float(kv["copy_write_factor"])
    except (KeyError, ValueError):
        return None
    rows = re.findall(r"^kernel\s+(\S+)\s+calls_per_step=(\d+)\s+fetch_kib=(\S+)\s+"
                      r"write_kib=(\S+)\s*$", txt, flags=re.M)
    if not rows:
        return None
    return sum(int(c) * (float(f) * 1024 * ff + float(w) * 1024 * wf) for _, c, f, w in rows)


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def set_oracle_threads(n: int) -> None:
    """Thread count of the oracle's OpenMP regions (calling thread's setting)."""
    import ctypes
    import ctypes.util
    name = ctypes.util.find_library("gomp") or "libgomp.so.1"
    ctypes.CDLL(name).omp_set_num_threads(int(n))


def row_counter_traffic(profile: str, workload: str):
    """HBM bytes per launch of a row's timed kernel from the machine-readable
    block of its committed profile (FETCH_SIZE and WRITE_SIZE in KiB per
    dispatch, scaled by the copy-kernel calibration); None if the file is
    absent, names another workload, or the kernel's source changed since."""
    path = os.path.join(ROOT, "profiles", profile)
    if not os.path.exists(path):
        return None
    kv = dict(re.findall(r"^(\w+)\s*=\s*(\S+)\s*$", open(path).read(), flags=re.M))
    src = kv.get("source", "-")
    if kv.get("workload") != workload or not all(
            os.path.exists(os.path.join(ROOT, p)) for p in src.split(",")):
        return None
    if kv.get("source_sha256") != source_hash(src):
        return None
    try:
        return (float(kv["fetch_kib"]) * 1024 * float(kv["copy_fetch_factor"]) +
                float(kv["write_kib"]) * 1024 * float(kv["copy_write_factor"]))
    except (KeyError, ValueError):
        return None


class Setup:
    """Device caches (replicas), per-layer inputs and output buffers."""

    def __init__(self, wl, seed, replicas, want_oracle, page_tokens=0):
        import torch

        import fp4_kv_cache_decode_amd.csa2 as K
        from fp4_kv_cache_decode_amd import datagen as G
        self.K, self.G, self.wl = K, G, wl
        B, N, L = wl.B, wl.N, len(wl.layers)
        dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
        self.dev = dev
        paging = {}
        if page_tokens:
            # every replica: the same fragmented layout over its own physical pool
            table, n_pages = G.page_table(seed, wl.n_seq, wl.cap, page_tokens,
                                          [wl.cap] * wl.n_seq)
            paging = dict(page_tokens=page_tokens, n_pages=n_pages,
                          page_table=torch.from_numpy(table))
        self.caches = [K.Cache(wl.n_seq, wl.cap, L, wl.w_cap, **paging)
                       for _ in range(replicas)]
        self.oc = None
        if want_oracle:
            import oracle as O
            self.oc = O.Cache(wl.n_seq, wl.cap, L, wl.w_cap)
        c0 = self.caches[0]
        t0 = time.time()
        w0 = max(0, N - G.WINDOW)
        for s in range(wl.n_seq):
            chunks = [(p, min(N, p + G.CHUNK)) for p in range(0, N, G.CHUNK)]
            gen = G.parallel_map(lambda pr: G.kv_rows(seed, s, pr[0], pr[1]), chunks)
            for (p0, p1), (k, v, ik) in zip(chunks, gen):
                seq = np.full(p1 - p0, s, np.int32)
                pos = np.arange(p0, p1, dtype=np.int64)
                K.quantize_kv(c0, dev(k), dev(v), dev(seq), dev(pos), idx_k=dev(ik))
                if self.oc is not None:
                    self.oc.quantize(k, v, ik, None, None, seq, pos)
            wk = np.stack([G.window_rows(seed, l, s, w0, N)[0] for l in range(L)])
            wv = np.stack([G.window_rows(seed, l, s, w0, N)[1] for l in range(L)])
            k, v, ik = G.kv_rows(seed, s, w0, N)
            seq = np.full(N - w0, s, np.int32)
            pos = np.arange(w0, N, dtype=np.int64)
            K.quantize_kv(c0, dev(k), dev(v), dev(seq), dev(pos), win_k=dev(wk), win_v=dev(wv))
            if self.oc is not None:
                self.oc.quantize(k, v, None, wk, wv, seq, pos)
            torch.cuda.synchronize()
            log(f"[bench] cache seq {s + 1}/{wl.n_seq} built ({time.time() - t0:.1f}s)")
        for c in self.caches[1:]:
            c.kv.copy_(c0.kv)
            c.idxk.copy_(c0.idxk)
            c.wk.copy_(c0.wk)
            c.wv.copy_(c0.wv)
        torch.cuda.synchronize()

        # the new token of every sequence: rows of position N-1 (already in the
        # cache; re-writing them is the step's quantise-on-write work)
        nk, nv, nik, nwk, nwv = [], [], [], [], []
        for s in range(wl.n_seq):
            k, v, ik = G.kv_rows(seed, s, N - 1, N)
            nk.append(k), nv.append(v), nik.append(ik)
            nwk.append(np.stack([G.window_rows(seed, l, s, N - 1, N)[0][0] for l in range(L)]))
            nwv.append(np.stack([G.window_rows(seed, l, s, N - 1, N)[1][0] for l in range(L)]))
        self.new = dict(k=dev(np.concatenate(nk)), v=dev(np.concatenate(nv)),
                        ik=dev(np.concatenate(nik)),
                        wk=dev(np.stack(nwk, axis=1)), wv=dev(np.stack(nwv, axis=1)),
                        seq=dev(np.arange(wl.n_seq, dtype=np.int32)),
                        pos=dev(np.full(wl.n_seq, N - 1, np.int64)))
        self.np_new = dict(k=np.concatenate(nk), v=np.concatenate(nv), ik=np.concatenate(nik),
                           wk=np.stack(nwk, axis=1), wv=np.stack(nwv, axis=1))
        # per-layer queries
        self.q = [G.attn_queries(seed, l, B) for l in range(L)]
        self.qi = {l: G.index_queries(seed, l, B) for l in wl.index_layers()}
        self.dq = [dev(x) for x in self.q]
        self.dqi = {l: (dev(a), dev(b)) for l, (a, b) in self.qi.items()}
        self.seq = dev(wl.seq())
        self.ctx = dev(wl.ctx())
        self.M = torch.empty((B, K.block_stride(N)), dtype=torch.float32, device="cuda")
        self.pool = torch.empty((B, G.N_BLOCKS), dtype=torch.int32, device="cuda")
        self.idx = torch.empty((B, G.TOPK), dtype=torch.int32, device="cuda")
        self.out = torch.empty((L, B, G.H, G.D), dtype=torch.float32, device="cuda")
        self.ws_ri = K.alloc_workspace(K.OP_INDEX_REINDEX, B)
        self.ws_sel = K.alloc_workspace(K.OP_SELECT_POOL, B, N)
        self.ws_at = K.alloc_workspace(K.OP_DECODE_ATTN, B)
        # the group's gathered main records: stored by its Full / Reindex layer,
        # read by its Reuse layers
        self.kvg = torch.empty((B, G.TOPK, K.RECORD), dtype=torch.uint8, device="cuda")

    # A step is three parts: the quantise-on-write of the new token, the Full
    # layer's scan over the whole context (the step's largest kernel by bytes,
    # timed with HIP events), and everything after it (pool, top-k, Reindex layers, attention).
    def part_quant(self, c):
        n = self.new
        self.K.quantize_kv(c, n["k"], n["v"], n["seq"], n["pos"], idx_k=n["ik"],
                           win_k=n["wk"], win_v=n["wv"])

    def part_scan(self, c):
        qi, wi = self.dqi[self.wl.layers.index("F")]
        self.K.index_block_scores(c, qi, wi, self.seq, self.ctx, self.wl.N, self.M)

    def part_rest(self, c):
        K, wl = self.K, self.wl
        for l, mode in enumerate(wl.layers):
            if mode == "F":
                qi, wi = self.dqi[l]
                K.index_select_pool(self.M, self.ctx, wl.N, self.pool, self.ws_sel)
                K.index_reindex(c, qi, wi, self.seq, self.ctx, self.pool, self.idx, self.ws_ri)
            elif mode == "I":
                qi, wi = self.dqi[l]
                K.index_reindex(c, qi, wi, self.seq, self.ctx, self.pool, self.idx, self.ws_ri)
            gather = dict(kvg_in=self.kvg) if mode == "R" else dict(kvg_out=self.kvg)
            K.decode_attn(c, l, self.dq[l], self.idx, self.seq, self.ctx, self.out[l],
                          self.ws_at, **gather)

    def capture(self):
        """HIP graphs of part_quant and part_rest for every replica."""
        import torch
        self.graphs = []
        stream = torch.cuda.Stream()
        for c in self.caches:
            ga, gb = torch.cuda.CUDAGraph(), torch.cuda.CUDAGraph()
            with torch.cuda.graph(ga, stream=stream):
                self.part_quant(c)
            with torch.cuda.graph(gb, stream=stream):
                self.part_rest(c)
            self.graphs.append((ga, gb))
        torch.cuda.synchronize()

    def step(self, r, ev=None):
        c = self.caches[r % len(self.caches)]
        graphs = getattr(self, "graphs", None)
        if graphs:
            graphs[r % len(self.caches)][0].replay()
        else:
            self.part_quant(c)
        if ev is not None:
            ev[0].record()
        self.part_scan(c)
        if ev is not None:
            ev[1].record()
        if graphs:
            graphs[r % len(self.caches)][1].replay()
        else:
            self.part_rest(c)


def oracle_step(S) -> float:
    """One step of the same workload through the oracle; returns seconds."""
    wl, oc = S.wl, S.oc
    seq, ctx = wl.seq(), wl.ctx()
    nn = S.np_new
    t0 = time.perf_counter()
    oc.quantize(nn["k"], nn["v"], nn["ik"], nn["wk"], nn["wv"], seq,
                np.full(wl.n_seq, wl.N - 1, np.int64))
    pool = idx = None
    for l, mode in enumerate(wl.layers):
        if mode == "F":
            qi, wi = S.qi[l]
            pool, idx, _, _ = oc.index_full(qi, wi, seq, ctx)
        elif mode == "I":
            qi, wi = S.qi[l]
            idx, _ = oc.index_reindex(qi, wi, seq, ctx, pool)
        oc.decode_attn(l, S.q[l], idx, seq, ctx)
    return time.perf_counter() - t0


def copy_bandwidth(nbytes=1 << 30, reps=10):
    """Device-to-device copy rate (read + write bytes / time) as a measured peak."""
    import torch
    a = torch.empty(nbytes // 4, dtype=torch.float32, device="cuda").fill_(1.0)
    b = torch.empty_like(a)
    for _ in range(2):
        b.copy_(a)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        b.copy_(a)
    e1.record()
    torch.cuda.synchronize()
    return 2 * nbytes * reps / (e0.elapsed_time(e1) * 1e-3) / 1e9


# ---------------------------------------------------------------------------
# Per-row measurements (not the default line): each times one hot-path row at
# its own bandwidth- or ALU-bound shape and reports it against its roofline.

def _common(args, metric, value, unit, ms, cfg, roofline, cpu=None, hib=True):
    return {"metric": metric, "value": value, "unit": unit, "n_gpus": 1, "steps": args.steps,
            "warmup": args.warmup, "ms_per_step": ms, "higher_is_better": hib,
            "scaling": "weak", "vs_baseline": None, "dtype": cfg.pop("dtype"),
            "data": "synthetic", "config": cfg, "roofline": roofline, "cpu_baseline": cpu}


def _event_loop(fn, steps, warmup):
    """Average milliseconds of fn(i) between HIP events on the current stream."""
    import torch
    for i in range(warmup):
        fn(i)
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(steps)]
    for i in range(steps):
        evs[i][0].record()
        fn(warmup + i)
        evs[i][1].record()
    torch.cuda.synchronize()
    return sum(a.elapsed_time(b) for a, b in evs) / steps


def _graph_loop(fn, n_calls, steps, warmup):
    """Average milliseconds per call of fn(0..n_calls-1) captured in one HIP
    graph, replayed back to back between one pair of events (no host work
    between the calls).  Returns (ms per call, calls timed)."""
    import torch
    for i in range(n_calls):
        fn(i)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=torch.cuda.Stream()):
        for i in range(n_calls):
            fn(i)
    reps = max(1, -(-steps // n_calls))
    for _ in range(max(1, -(-warmup // n_calls))):
        g.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        g.replay()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / (reps * n_calls), reps * n_calls


def row_quantize(args):
    """Bulk quantise-on-write of decoder20_1m_b4's cache: 4 x 1,048,576 rows of
    post-RoPE K, V and indexer keys in one call."""
    import torch
    import fp4_kv_cache_decode_amd.csa2 as K
    from fp4_kv_cache_decode_amd import datagen as G
    wl = G.WORKLOADS["decoder20_1m_b4"]
    n = wl.n_seq * wl.N
    t0 = time.time()
    k = torch.empty((n, G.D), dtype=torch.float32, device="cuda")
    v = torch.empty_like(k)
    ik = torch.empty((n, G.DI), dtype=torch.float32, device="cuda")
    jobs = [(s, p) for s in range(wl.n_seq) for p in range(0, wl.N, G.CHUNK)]
    for j0 in range(0, len(jobs), 16):
        part = jobs[j0:j0 + 16]
        rows = G.parallel_map(lambda sp: G.kv_rows(args.seed, sp[0], sp[1], sp[1] + G.CHUNK), part)
        for (s_, p), (kk, vv, ii) in zip(part, rows):
            r0 = s_ * wl.N + p
            k[r0:r0 + G.CHUNK].copy_(torch.from_numpy(kk))
            v[r0:r0 + G.CHUNK].copy_(torch.from_numpy(vv))
            ik[r0:r0 + G.CHUNK].copy_(torch.from_numpy(ii))
    seq = torch.arange(wl.n_seq, dtype=torch.int32, device="cuda").repeat_interleave(wl.N)
    pos = torch.arange(wl.N, dtype=torch.int64, device="cuda").repeat(wl.n_seq)
    caches = [K.Cache(wl.n_seq, wl.cap, 1) for _ in range(2)]
    torch.cuda.synchronize()
    log(f"[bench] quantize inputs ready ({time.time() - t0:.1f}s): {n} rows")
    ms = _event_loop(lambda i: K.quantize_kv(caches[i % 2], k, v, seq, pos, idx_k=ik),
                     args.steps, args.warmup)
    per_row = 2 * G.D * 4 + G.DI * 4 + 4 + 8 + 144 + 64
    alg = n * per_row
    gbs = alg / (ms * 1e-3) / 1e9
    log(f"[bench] bulk quantize {ms * 1e3:.1f} us, {gbs:.0f} GB/s")
    cfg = {"workload": "bulk quantize of decoder20_1m_b4 (4 x 1,048,576 rows)", "rows": n,
           "bytes_per_row": per_row, "dtype": "fp32"}
    traffic = row_counter_traffic("quantize_bulk_decoder20_1m_b4.txt", "quantize_bulk_4x1m")
    roof = {"bound": "hbm", "achieved": gbs, "peak": PEAK_HBM_GBS, "unit": "GB/s",
            "frac": gbs / PEAK_HBM_GBS, "traffic": traffic,
            "kernel": "quantize_kernel (csa2_quantize_kv)", "avg_us": ms * 1e3, "alg_bytes": alg}
    return _common(args, "CSA2 quantise-on-write rows/s", n / (ms * 1e-3), "rows/s", ms, cfg,
                   roof)


def row_gather(args):
    """Gather/dequant/attention at a bandwidth-bound shape: B=1,024 sequences of
    65,536 positions, top-512 plus the 128-token window, one layer per call,
    rotating over 4 (index set, layer) pairs so the 108 MB each call touches is
    read from HBM, not from the 256 MB Infinity Cache."""
    import torch
    import fp4_kv_cache_decode_amd.csa2 as K
    from fp4_kv_cache_decode_amd import datagen as G
    B, N, L, R = 1024, 65536, 4, 4
    t0 = time.time()
    c = K.Cache(B, N, L)
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    # sequence 0 from the generator, then replicated to every sequence
    for p in range(0, N, G.CHUNK):
        kk, vv, _ = G.kv_rows(args.seed, 0, p, p + G.CHUNK)
        K.quantize_kv(c, dev(kk), dev(vv), dev(np.zeros(G.CHUNK, np.int32)),
                      dev(np.arange(p, p + G.CHUNK, dtype=np.int64)))
    w0 = N - G.WINDOW
    kk, vv, _ = G.kv_rows(args.seed, 0, w0, N)
    wk = np.stack([G.window_rows(args.seed, l, 0, w0, N)[0] for l in range(L)])
    wv = np.stack([G.window_rows(args.seed, l, 0, w0, N)[1] for l in range(L)])
    K.quantize_kv(c, dev(kk), dev(vv), dev(np.zeros(G.WINDOW, np.int32)),
                  dev(np.arange(w0, N, dtype=np.int64)), win_k=dev(wk), win_v=dev(wv))
    c.kv[1:].copy_(c.kv[0:1].expand(B - 1, -1, -1))
    c.wk[:, 1:].copy_(c.wk[:, 0:1].expand(-1, B - 1, -1, -1))
    c.wv[:, 1:].copy_(c.wv[:, 0:1].expand(-1, B - 1, -1, -1))
    rng = np.random.default_rng(args.seed)
    idxs = []
    for r in range(R):
        sel = np.sort(np.argpartition(rng.random((B, N), dtype=np.float32), G.TOPK, axis=1)
                      [:, :G.TOPK], axis=1).astype(np.int32)
        idxs.append(dev(sel))
    qs = [dev(G.attn_queries(args.seed, l, B)) for l in range(L)]
    seq = dev(np.arange(B, dtype=np.int32))
    ctx = dev(np.full(B, N, np.int64))
    out = torch.empty((B, G.H, G.D), dtype=torch.float32, device="cuda")
    ws = K.alloc_workspace(K.OP_DECODE_ATTN, B)
    torch.cuda.synchronize()
    log(f"[bench] gather inputs ready ({time.time() - t0:.1f}s)")
    # one HIP graph of the R x L rotation, replayed back to back
    n_rot = R * L // math.gcd(R, L)
    ms, args.steps = _graph_loop(
        lambda i: K.decode_attn(c, i % L, qs[i % L], idxs[i % R], seq, ctx, out, ws),
        n_rot, args.steps, args.warmup)
    per_q = G.TOPK * 144 + G.WINDOW * 2 * G.D + G.H * G.D * 4 + G.TOPK * 4 + 12 + G.H * G.D * 4
    alg = B * per_q
    gbs = alg / (ms * 1e-3) / 1e9
    log(f"[bench] gather-attention {ms * 1e3:.1f} us, {gbs:.0f} GB/s")
    cfg = {"workload": "gather_attention_b1024_n64k", "batch": B, "ctx": N, "topk": G.TOPK,
           "window": G.WINDOW, "rotations": R, "launch": "hip-graph", "dtype": "fp32"}
    traffic = row_counter_traffic("attn_gather_b1024_n64k.txt", "gather_attention_b1024_n64k")
    roof = {"bound": "hbm", "achieved": gbs, "peak": PEAK_HBM_GBS, "unit": "GB/s",
            "frac": gbs / PEAK_HBM_GBS, "traffic": traffic,
            "kernel": "attn_stream_kernel (csa2_decode_attn)", "avg_us": ms * 1e3,
            "alg_bytes": alg}
    return _common(args, "CSA2 gather/dequant/attention queries/s", B / (ms * 1e-3), "queries/s",
                   ms, cfg, roof)


def _eager_loop(fn, n_calls, steps, warmup):
    """Average milliseconds per call of fn(i) launched eagerly back to back
    between one pair of events (the host stays ahead of the GPU)."""
    import torch
    for i in range(warmup):
        fn(i % n_calls)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for i in range(steps):
        fn(i % n_calls)
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / steps


def row_reindex_layer(args):
    """One Reindex layer of decoder20_1m_b4 (B=4, 1,048,576 tokens: pool scores
    over the group's 2,048-block pool, top-512, attention over 512 + 128
    entries with the gathered records stored for the Reuse layers), two ways:
    the separate calls (four kernels, replayed as a HIP graph and launched
    eagerly) and csa2_reindex_layer_fused (one cooperative launch, eagerly; in
    a graph too where capture accepts it).  Rotates over the workload's four
    Reindex layers' queries."""
    import torch
    import fp4_kv_cache_decode_amd.csa2 as K
    from fp4_kv_cache_decode_amd import datagen as G
    wl = G.WORKLOADS["decoder20_1m_b4"]
    S = Setup(wl, args.seed, 1, False)
    c, B = S.caches[0], wl.B
    layers = [l for l, m in enumerate(wl.layers) if m == "I"]
    # the group's pool from its Full layer
    S.part_scan(c)
    K.index_select_pool(S.M, S.ctx, wl.N, S.pool, S.ws_sel)
    ws_f = torch.zeros(K.workspace_bytes(K.OP_REINDEX_LAYER_FUSED, B, 0, G.N_BLOCKS, G.BLOCK,
                                         G.TOPK), dtype=torch.uint8, device="cuda")
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    out = torch.empty((B, G.H, G.D), dtype=torch.float32, device="cuda")

    def separate(i):
        l = layers[i]
        qi, wi = S.dqi[l]
        K.index_reindex(c, qi, wi, S.seq, S.ctx, S.pool, S.idx, S.ws_ri)
        K.decode_attn(c, l, S.dq[l], S.idx, S.seq, S.ctx, out, S.ws_at, kvg_out=S.kvg)

    def fused(i):
        l = layers[i]
        qi, wi = S.dqi[l]
        K.reindex_layer_fused(c, l, qi, wi, S.dq[l], S.seq, S.ctx, S.pool, S.idx, out, ws_f,
                              status, kvg_out=S.kvg)

    n = len(layers)
    sep_graph, _ = _graph_loop(separate, n, args.steps, args.warmup)
    sep_eager = _eager_loop(separate, n, args.steps, args.warmup)
    fused_eager = _eager_loop(fused, n, args.steps, args.warmup)
    try:
        fused_graph, _ = _graph_loop(fused, n, args.steps, args.warmup)
    except RuntimeError as e:            # capture refused the cooperative launch
        log(f"[bench] fused layer not capturable: {e}")
        fused_graph = None
    torch.cuda.synchronize()
    gave_up = int(status.item())
    log(f"[bench] Reindex layer: separate {sep_graph * 1e3:.2f} us (graph), "
        f"{sep_eager * 1e3:.2f} us (eager); fused {fused_eager * 1e3:.2f} us (eager)"
        + (f", {fused_graph * 1e3:.2f} us (graph)" if fused_graph else "")
        + f"; status {gave_up}")
    # bytes of one layer: pool keys, pool list, records, window rows, q, outputs
    alg = B * (G.N_BLOCKS * G.BLOCK * 64 + G.N_BLOCKS * 4 + G.TOPK * 144 * 2 +
               G.WINDOW * 2 * G.D + (4 * 64 + 4) * 4 + G.H * G.D * 4 * 2 + G.TOPK * 4)
    best = fused_graph if fused_graph else fused_eager
    gbs = alg / (best * 1e-3) / 1e9
    cfg = {"workload": "reindex_layer_decoder20_1m_b4", "batch": B, "ctx": wl.N,
           "topk": G.TOPK, "pool_blocks": G.N_BLOCKS, "window": G.WINDOW,
           "separate_graph_us": sep_graph * 1e3, "separate_eager_us": sep_eager * 1e3,
           "fused_eager_us": fused_eager * 1e3,
           "fused_graph_us": fused_graph * 1e3 if fused_graph else None,
           "fused_status": gave_up, "launch": "cooperative", "dtype": "fp32"}
    roof = {"bound": "hbm", "achieved": gbs, "peak": PEAK_HBM_GBS, "unit": "GB/s",
            "frac": gbs / PEAK_HBM_GBS, "traffic": None,
            "kernel": "reindex_layer_kernel (csa2_reindex_layer_fused)", "avg_us": best * 1e3,
            "alg_bytes": alg}
    return _common(args, "CSA2 fused Reindex layers/s", 1e3 / best, "layers/s", best, cfg,
                   roof)


def row_prefill(args):
    """The 8,192-token prefill chunk over a 131,072-token prefix: quantise the
    chunk (main KV, indexer keys, window rows), then the Full-layer indexer and
    attention for all 8,192 causal queries (seq 0, ctx_i = 131,073 + i).  The
    layer keeps its 512 best blocks (no Reindex layer follows it; --pool-blocks
    2048 builds the decoder's pool instead): the top-512 lie in them either way."""
    import torch
    import fp4_kv_cache_decode_amd.csa2 as K
    from fp4_kv_cache_decode_amd import datagen as G
    wl = G.WORKLOADS["prefill_8k_over_128k"]
    B, N0, cap = wl.B, wl.N, wl.cap
    nbk = args.pool_blocks or wl.extra["pool_blocks"]   # blocks the Full layer keeps
    t0 = time.time()
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    c = K.Cache(1, cap, 1, wl.w_cap)
    w_lo = N0 - G.WINDOW
    oc = None
    if not args.no_cpu_baseline:
        import oracle as O
        oc = O.Cache(1, cap, 1, wl.w_cap)
    for p in range(0, N0, G.CHUNK):
        kk, vv, ii = G.kv_rows(args.seed, 0, p, p + G.CHUNK)
        sq, ps = np.zeros(G.CHUNK, np.int32), np.arange(p, p + G.CHUNK, dtype=np.int64)
        K.quantize_kv(c, dev(kk), dev(vv), dev(sq), dev(ps), idx_k=dev(ii))
        if oc is not None:
            oc.quantize(kk, vv, ii, None, None, sq, ps)
    kk, vv, _ = G.kv_rows(args.seed, 0, w_lo, N0)
    wk, wv = G.window_rows(args.seed, 0, 0, w_lo, N0)
    sq, ps = np.zeros(G.WINDOW, np.int32), np.arange(w_lo, N0, dtype=np.int64)
    K.quantize_kv(c, dev(kk), dev(vv), dev(sq), dev(ps), win_k=dev(wk[None]), win_v=dev(wv[None]))
    if oc is not None:
        oc.quantize(kk, vv, None, wk[None], wv[None], sq, ps)
    # the chunk: its rows are written inside every timed step
    ck, cv, ci = G.kv_rows(args.seed, 0, N0, cap)
    cwk, cwv = G.window_rows(args.seed, 0, 0, N0, cap)
    chunk = dict(k=dev(ck), v=dev(cv), ik=dev(ci), wk=dev(cwk[None]), wv=dev(cwv[None]),
                 seq=dev(np.zeros(B, np.int32)), pos=dev(np.arange(N0, cap, dtype=np.int64)))
    if oc is not None:
        oc.quantize(ck, cv, ci, cwk[None], cwv[None], np.zeros(B, np.int32),
                    np.arange(N0, cap, dtype=np.int64))
    seq_np, ctx_np = wl.seq(), wl.ctx()
    qi_np, wi_np = G.index_queries(args.seed, 0, B)
    q_np = G.attn_queries(args.seed, 0, B)
    seq, ctx, qi, wi, q = dev(seq_np), dev(ctx_np), dev(qi_np), dev(wi_np), dev(q_np)
    M = torch.empty((B, K.block_stride(cap)), dtype=torch.float32, device="cuda")
    pool = torch.empty((B, nbk), dtype=torch.int32, device="cuda")
    idx = torch.empty((B, G.TOPK), dtype=torch.int32, device="cuda")
    out = torch.empty((B, G.H, G.D), dtype=torch.float32, device="cuda")
    ws_sel = K.alloc_workspace(K.OP_SELECT_POOL, B, cap, n_blocks=nbk)
    ws_ri = K.alloc_workspace(K.OP_INDEX_REINDEX, B, n_blocks=nbk)
    ws_at = K.alloc_workspace(K.OP_DECODE_ATTN, B)
    torch.cuda.synchronize()
    log(f"[bench] prefill inputs ready ({time.time() - t0:.1f}s)")

    scan_ev = []

    def step(i, timed=False):
        K.quantize_kv(c, chunk["k"], chunk["v"], chunk["seq"], chunk["pos"], idx_k=chunk["ik"],
                      win_k=chunk["wk"], win_v=chunk["wv"])
        if timed:
            e = (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
            e[0].record()
        K.index_block_scores(c, qi, wi, seq, ctx, cap, M)
        if timed:
            e[1].record()
            scan_ev.append(e)
        K.index_select_pool(M, ctx, cap, pool, ws_sel)
        K.index_reindex(c, qi, wi, seq, ctx, pool, idx, ws_ri)
        K.decode_attn(c, 0, q, idx, seq, ctx, out, ws_at)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    for i in range(args.steps):
        step(i, timed=True)
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t1) * 1e3 / args.steps
    scan_ms = sum(a.elapsed_time(b) for a, b in scan_ev) / len(scan_ev)
    key_evals = int(ctx_np.sum())
    flops = 2 * G.HI * G.DI * key_evals
    tfs = flops / (scan_ms * 1e-3) / 1e12
    log(f"[bench] prefill chunk {ms:.2f} ms, scan {scan_ms:.2f} ms = {tfs:.1f} TFLOP/s")
    cpu = None
    if oc is not None:
        # a strided sample of the chunk's queries through the oracle (index + attention)
        sample = np.arange(0, B, 16)
        ts = time.perf_counter()
        _, oidx, _, _ = oc.index_full(qi_np[sample], wi_np[sample], seq_np[sample], ctx_np[sample],
                                      n_blocks=nbk)
        oc.decode_attn(0, q_np[sample], oidx, seq_np[sample], ctx_np[sample])
        secs = time.perf_counter() - ts
        threads = int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1))
        cpu = {"value": sample.size / secs, "unit": "queries/s", "cores": threads,
               "kind": "oracle",
               "sample": f"{sample.size} of the chunk's 8,192 queries (every 16th) through "
                         f"the fp64 C oracle's indexer and attention, {secs:.1f} s wall"}
    cfg = {"workload": wl.name, "queries": B, "prefix": N0, "topk": G.TOPK,
           "pool_blocks": nbk, "window": G.WINDOW, "key_evals": key_evals, "dtype": "fp32"}
    traffic = row_counter_traffic("prefill_8k_over_128k_kernel_stats.txt",
                                  "prefill_8k_over_128k")
    roof = {"bound": "alu", "achieved": tfs, "peak": PEAK_FP32_TFS, "unit": "TFLOP/s",
            "frac": tfs / PEAK_FP32_TFS, "traffic": traffic,
            "kernel": "scan_kernel (csa2_index_block_scores)", "avg_us": scan_ms * 1e3,
            "flops": flops}
    return _common(args, "CSA2 chunked-prefill queries/s", B / (ms * 1e-3), "queries/s", ms, cfg,
                   roof, cpu)


def row_encoder(args):
    """The encoder side of CSA2 on one prefill chunk: 8,192 causal tokens after a
    131,072-token prefix through the 20 encoder layers -- layers 1-2 sliding
    window only, then 3 x [Full + 5 Reuse] at global-KV compression m = 2, each
    Full layer with its own store of 2-token entries (65,536 + 4,096 of them).
    A step writes the chunk (csa2_compress_kv: each group's entries and every
    layer's window rows), then runs every layer's indexer and attention for all
    8,192 queries (query i: ctx_i = 131,073 + i tokens, ctx_i // 2 entries).  A
    Full layer keeps its 512 best blocks: no Reindex layer follows it, and its
    top-512 positions all lie in those blocks."""
    import torch
    import fp4_kv_cache_decode_amd.csa2 as K
    from fp4_kv_cache_decode_amd import datagen as G
    wl = G.WORKLOADS["encoder20_m2_chunk8k_over_128k"]
    B, N0, m = wl.B, wl.N, wl.m
    cap_c = wl.cap // m
    nbk = args.pool_blocks or wl.extra["pool_blocks"]   # blocks a Full layer keeps
    groups = [i for i, x in enumerate(wl.layers) if x == "F"]
    swa = [i for i, x in enumerate(wl.layers) if x == "S"]
    span = [list(range(f, f + 6)) for f in groups]          # a group's 6 layers
    # the window stores of a group's layers live with its global store; the
    # window-only layers' with the first group's
    wins = [swa + span[0]] + span[1:]
    t0 = time.time()
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    want_cpu = not args.no_cpu_baseline
    if want_cpu:
        import oracle as O
    zeros = lambda n: np.zeros(n, np.int32)
    w_lo = N0 - G.WINDOW

    def windows(layers, p0, p1):
        rows = [G.window_rows(args.seed, l, 0, p0, p1) for l in layers]
        return np.stack([r[0] for r in rows]), np.stack([r[1] for r in rows])

    # one global store per group, with its layers' window stores
    gcs, ocs = [], []
    for gi, ls in enumerate(wins):
        gc = K.Cache(1, cap_c, len(ls), wl.w_cap)
        oc = O.Cache(1, cap_c, len(ls), wl.w_cap) if want_cpu else None
        for p in range(0, N0, G.CHUNK):
            k, v, ik = G.kv_rows(args.seed, 0, p, p + G.CHUNK, gi)
            pos = np.arange(p, p + G.CHUNK, dtype=np.int64)
            K.compress_kv(gc, dev(k), dev(v), dev(zeros(G.CHUNK)), dev(pos), m, idx_k=dev(ik))
            if oc is not None:
                oc.compress(k, v, ik, None, None, zeros(G.CHUNK), pos, m)
        wk, wv = windows(ls, w_lo, N0)
        pos = np.arange(w_lo, N0, dtype=np.int64)
        K.compress_kv(gc, None, None, dev(zeros(G.WINDOW)), dev(pos), m, win_k=dev(wk),
                      win_v=dev(wv))
        if oc is not None:
            oc.compress(None, None, None, wk, wv, zeros(G.WINDOW), pos, m)
        gcs.append(gc)
        ocs.append(oc)
    log(f"[bench] encoder prefixes built ({time.time() - t0:.1f}s)")

    # the chunk's rows, written inside every timed step
    cpos = np.arange(N0, N0 + B, dtype=np.int64)
    chunk = []
    for gi, ls in enumerate(wins):
        k, v, ik = G.kv_rows(args.seed, 0, N0, N0 + B, gi)
        wk, wv = windows(ls, N0, N0 + B)
        chunk.append(dict(k=dev(k), v=dev(v), ik=dev(ik), wk=dev(wk), wv=dev(wv)))
        if ocs[gi] is not None:
            ocs[gi].compress(k, v, ik, wk, wv, zeros(B), cpos, m)
    seq_np, ctx_np = wl.seq(), wl.ctx()
    ctxc_np = ctx_np // m
    seq, ctx, ctxc, pos_t = dev(seq_np), dev(ctx_np), dev(ctxc_np), dev(cpos)
    iq = [G.index_queries(args.seed, f, B) for f in groups]
    qi = [(dev(a), dev(b)) for a, b in iq]
    q_np = [G.attn_queries(args.seed, l, B) for l in range(len(wl.layers))]
    q = [dev(x) for x in q_np]
    # window-only layers: one absent main entry per query (the window carries them)
    none = torch.full((B, 1), -1, dtype=torch.int32, device="cuda")
    M = torch.empty((B, K.block_stride(cap_c)), dtype=torch.float32, device="cuda")
    pool = torch.empty((B, nbk), dtype=torch.int32, device="cuda")
    idx = torch.empty((B, G.TOPK), dtype=torch.int32, device="cuda")
    out = torch.empty((len(wl.layers), B, G.H, G.D), dtype=torch.float32, device="cuda")
    ws_sel = K.alloc_workspace(K.OP_SELECT_POOL, B, cap_c, n_blocks=nbk)
    ws_ri = K.alloc_workspace(K.OP_INDEX_REINDEX, B, n_blocks=nbk)
    ws_at = K.alloc_workspace(K.OP_DECODE_ATTN, B)
    torch.cuda.synchronize()
    log(f"[bench] encoder inputs ready ({time.time() - t0:.1f}s)")

    scan_ev = []

    def step(i, timed=False):
        for gi in range(len(wins)):
            c = chunk[gi]
            K.compress_kv(gcs[gi], c["k"], c["v"], seq, pos_t, m, idx_k=c["ik"], win_k=c["wk"],
                          win_v=c["wv"])
        for l in swa:
            K.decode_attn(gcs[0], wins[0].index(l), q[l], none, seq, ctx, out[l], ws_at)
        for gi, ls in enumerate(span):
            if timed:
                e = (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                e[0].record()
            K.index_block_scores(gcs[gi], qi[gi][0], qi[gi][1], seq, ctxc, cap_c, M)
            if timed:
                e[1].record()
                scan_ev.append(e)
            K.index_select_pool(M, ctxc, cap_c, pool, ws_sel)
            K.index_reindex(gcs[gi], qi[gi][0], qi[gi][1], seq, ctxc, pool, idx, ws_ri)
            # Reuse layers pass the Full layer's idx again: the 10 MB store stays cache
            # resident, while gathered records (kvg) would be 604 MB at this batch
            for l in ls:
                K.decode_attn(gcs[gi], wins[gi].index(l), q[l], idx, seq, ctx, out[l], ws_at)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    for i in range(args.steps):
        step(i, timed=True)
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t1) * 1e3 / args.steps
    scan_ms = sum(a.elapsed_time(b) for a, b in scan_ev) / args.steps    # the 3 scans of a step
    key_evals = int(ctxc_np.sum()) * len(groups)
    flops = 2 * G.HI * G.DI * key_evals
    tfs = flops / (scan_ms * 1e-3) / 1e12
    log(f"[bench] encoder chunk {ms:.2f} ms, scans {scan_ms:.2f} ms = {tfs:.1f} TFLOP/s")
    cpu = None
    if want_cpu:
        # a strided sample of the chunk's queries through the oracle: every
        # layer's indexer and attention
        sample = np.arange(0, B, 16)
        ss, sx, sxc = seq_np[sample], ctx_np[sample], ctxc_np[sample]
        nn = np.full((sample.size, 1), -1, np.int32)
        ts = time.perf_counter()
        for l in swa:
            ocs[0].decode_attn(wins[0].index(l), q_np[l][sample], nn, ss, sx)
        for gi, ls in enumerate(span):
            _, oidx, _, _ = ocs[gi].index_full(iq[gi][0][sample], iq[gi][1][sample], ss, sxc,
                                               n_blocks=nbk)
            for l in ls:
                ocs[gi].decode_attn(wins[gi].index(l), q_np[l][sample], oidx, ss, sx)
        secs = time.perf_counter() - ts
        threads = int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1))
        cpu = {"value": sample.size / secs, "unit": "queries/s", "cores": threads,
               "kind": "oracle",
               "sample": f"{sample.size} of the chunk's 8,192 queries (every 16th) through "
                         f"the fp64 C oracle's indexers and all 20 layers' attention, "
                         f"{secs:.1f} s wall"}
    cfg = {"workload": wl.name, "queries": B, "prefix": N0, "compression": m,
           "layers": "".join(wl.layers), "topk": G.TOPK, "pool_blocks": nbk,
           "window": G.WINDOW, "key_evals": key_evals, "dtype": "fp32"}
    roof = {"bound": "alu", "achieved": tfs, "peak": PEAK_FP32_TFS, "unit": "TFLOP/s",
            "frac": tfs / PEAK_FP32_TFS,
            "traffic": row_counter_traffic("encoder_chunk8k_m2_kernel_stats.txt",
                                           "encoder20_m2_chunk8k_over_128k"),
            "kernel": "scan_kernel (csa2_index_block_scores), the three Full layers' scans",
            "avg_us": scan_ms * 1e3, "flops": flops}
    return _common(args, "CSA2 encoder-chunk queries/s (m = 2)", B / (ms * 1e-3), "queries/s",
                   ms, cfg, roof, cpu)


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="decoder20_1m_b4")
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--replicas", type=int, default=2)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--page-tokens", type=int, default=0,
                    help="decode row on a paged cache: tokens per page (power of two >= 64), "
                         "pages scattered over a shuffled physical pool; 0 = contiguous")
    ap.add_argument("--eager", action="store_true",
                    help="launch every kernel from Python instead of replaying HIP graphs")
    ap.add_argument("--pool-blocks", type=int, default=0,
                    help="prefill and encoder rows: blocks a Full layer keeps (default: the "
                         "workload's, 512; 2048 builds the decoder's Reindex pool)")
    ap.add_argument("--copy-probe", action="store_true",
                    help="only run a 1 GiB device copy (counter calibration)")
    ap.add_argument("--row", default="decode",
                    choices=["decode", "quantize", "gather", "prefill", "reindex_layer",
                             "encoder"],
                    help="decode: the whole decode step (default); quantize: bulk quantise-on-write "
                         "of the 1M-context cache; gather: gather/dequant/attention at B=1024; "
                         "prefill: the 8,192-query chunk over a 131,072-token prefix; "
                         "reindex_layer: one Reindex layer, separate calls against the fused "
                         "cooperative launch; encoder: the 20 encoder layers (CSA2 at "
                         "compression 2) on the same chunk")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py measures one GPU only (--gpus {args.gpus} requested); "
              "the decode path needs no collectives and shards by sequence, so run one "
              "process per GPU", file=sys.stderr)
        sys.exit(2)

    import torch
    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        sys.exit(1)
    if args.copy_probe:
        log(f"[bench] copy probe: {copy_bandwidth():.0f} GB/s")
        return
    if args.row != "decode":
        res = {"quantize": row_quantize, "gather": row_gather, "prefill": row_prefill,
               "reindex_layer": row_reindex_layer, "encoder": row_encoder}[args.row](args)
        print(json.dumps(res), flush=True)
        return

    from fp4_kv_cache_decode_amd import datagen as G
    wl = G.WORKLOADS[args.workload]
    if wl.prefill:
        print("bench.py: prefill workloads are parity cases, not bench lines", file=sys.stderr)
        sys.exit(2)
    B, N = wl.B, wl.N
    want_cpu = not args.no_cpu_baseline
    log(f"[bench] workload {wl.name}: B={B} N={N} layers={''.join(wl.layers)}")
    S = Setup(wl, args.seed, args.replicas, want_cpu, args.page_tokens)

    copy_gbs = copy_bandwidth()
    log(f"[bench] device copy {copy_gbs:.0f} GB/s")

    for i in range(max(args.warmup, 1)):
        S.step(i)
    torch.cuda.synchronize()
    if not args.eager:
        S.capture()
        for i in range(args.warmup):
            S.step(i)
        torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        S.step(args.warmup + i, evs[i])
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms = (t1 - t0) * 1e3 / args.steps
    score_ms = sum(a.elapsed_time(b) for a, b in evs) / args.steps
    log(f"[bench] {ms:.3f} ms/step, Full-layer scan {score_ms * 1e3:.1f} us")

    # the Full layer's indexer scan, timed on its own with events
    n_keys = B * N
    scan_bytes = n_keys * 64 + B * (-(-N // 8)) * 4 + B * (4 * 64 + 4) * 4
    if args.page_tokens:
        scan_bytes += B * (-(-N // args.page_tokens)) * 4      # page-table entries
    scan_gbs = scan_bytes / (score_ms * 1e-3) / 1e9
    # the committed counters were taken on the contiguous cache
    scan_traffic = None if args.page_tokens else counter_traffic(wl.name)
    # the whole step: its algorithmic bytes over the measured step time
    alg_bytes = step_alg_bytes(wl)
    achieved = alg_bytes / (ms * 1e-3) / 1e9
    step_traffic = None if args.page_tokens else step_counter_traffic(wl.name)

    cpu = None
    if want_cpu:
        threads = int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1))
        # whole decode steps through the oracle: at one thread (one step, the
        # bounded sample), then at the host's thread count until ~10 s
        set_oracle_threads(1)
        secs1 = oracle_step(S)
        set_oracle_threads(threads)
        reps, secs = 0, 0.0
        while reps < 2 or (secs < 10.0 and reps < 50):
            secs += oracle_step(S)
            reps += 1
        cpu = {"value": B * reps / secs, "unit": "queries/s", "cores": threads,
               "kind": "oracle", "cpu_model": cpu_model(),
               "value_1_thread": B / secs1,
               "sample": f"{reps} full decode steps of {wl.name} ({B} queries x "
                         f"{len(wl.layers)} layers at {N} tokens each) through the fp64 C "
                         f"oracle, OpenMP over positions/queries on {threads} threads, "
                         f"{secs:.1f} s wall; value_1_thread: one such step on one thread, "
                         f"{secs1:.1f} s wall"}
        log(f"[bench] oracle {reps} steps in {secs:.2f} s on {threads} threads; "
            f"1 step in {secs1:.2f} s on 1 thread")

    res = {
        "metric": METRIC,
        "value": B / (ms * 1e-3),
        "unit": "queries/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp32",
        "data": "synthetic",
        "config": {"workload": wl.name, "batch": B, "ctx": N, "layers": "".join(wl.layers),
                   "topk": G.TOPK, "window": G.WINDOW, "pool_blocks": G.N_BLOCKS,
                   "block": G.BLOCK, "replicas": args.replicas, "seed": args.seed,
                   "launch": "eager" if args.eager else "hip-graph",
                   "cache": (f"paged, {args.page_tokens}-token pages over a shuffled pool"
                             if args.page_tokens else "contiguous")},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": PEAK_HBM_GBS,
                     "unit": "GB/s", "frac": achieved / PEAK_HBM_GBS,
                     "traffic": step_traffic,
                     "scope": "whole decode step (every kernel of the step, graph replay)",
                     "alg_bytes": alg_bytes, "avg_us": ms * 1e3,
                     "kernels": {"scan_kernel": {
                         "entry": "csa2_index_block_scores", "bound": "hbm",
                         "achieved": scan_gbs, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                         "frac": scan_gbs / PEAK_HBM_GBS, "traffic": scan_traffic,
                         "avg_us": score_ms * 1e3, "alg_bytes": scan_bytes}}},
        "cpu_baseline": cpu,
        "hbm_copy_gbs": copy_gbs,
    }
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
