"""Shared helpers for the GPU parity tests (imported by tests/test_gpu_*.py).

Both sides receive the same seeded rows from the input generator; the oracle
quantises them itself (it never sees a byte the HIP path wrote).
"""
from __future__ import annotations

import numpy as np

from fp4_kv_cache_decode_amd import datagen as G

REL_EXEMPT = 1e-5      # index-set exemption: |score - kth| <= 1e-5 * |kth|
ATTN_TOL = 2e-3        # max-abs bound on attention outputs


def rows_for(seed, s, p0, p1, n_layers, N, wlo=None):
    """Main rows for [p0,p1) and window rows of every layer for the part of
    [p0,p1) inside the window range [wlo, N)."""
    k, v, ik = G.kv_rows(seed, s, p0, p1)
    wlo = max(0, N - G.WINDOW) if wlo is None else wlo
    w0, w1 = max(p0, wlo), p1
    wk = wv = None
    if w1 > w0:
        wk = np.zeros((n_layers, w1 - w0, G.D), np.float32)
        wv = np.zeros_like(wk)
        for l in range(n_layers):
            wk[l], wv[l] = G.window_rows(seed, l, s, w0, w1)
    return k, v, ik, (w0, w1, wk, wv)


def fill_both(seed, n_seq, N, n_layers, ocache, gcache=None, chunk=1 << 18, wlo=None,
              workers=1):
    """Write positions [0,N) of every sequence into the oracle cache and (if
    given) the device cache, or each of a tuple of device caches, through
    csa2_quantize_kv.  With workers > 1 the rows of up to `workers` chunks are
    generated in parallel threads."""
    import torch
    from fp4_kv_cache_decode_amd import csa2
    for s in range(n_seq):
        starts = list(range(0, N, chunk))
        for g0 in range(0, len(starts), workers):
            group = [(p0, min(N, p0 + chunk)) for p0 in starts[g0:g0 + workers]]
            made = G.parallel_map(lambda pr: rows_for(seed, s, pr[0], pr[1], n_layers, N, wlo),
                                  group, workers) if workers > 1 else \
                [rows_for(seed, s, p0, p1, n_layers, N, wlo) for p0, p1 in group]
            for (p0, p1), rows in zip(group, made):
                _write_rows(s, p0, p1, rows, ocache, gcache, torch, csa2)


def _write_rows(s, p0, p1, rows, ocache, gcache, torch, csa2):
    k, v, ik, (w0, w1, wk, wv) = rows
    seq = np.full(p1 - p0, s, np.int32)
    pos = np.arange(p0, p1, dtype=np.int64)
    if ocache is not None:
        ocache.quantize(k, v, ik, None, None, seq, pos)
        if wk is not None:
            ocache.quantize(k[w0 - p0:], v[w0 - p0:], None, wk, wv, seq[w0 - p0:],
                            pos[w0 - p0:])
    gcaches = () if gcache is None else (gcache if isinstance(gcache, tuple) else (gcache,))
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    for gc in gcaches:
        csa2.quantize_kv(gc, dev(k), dev(v), dev(seq), dev(pos), idx_k=dev(ik))
        if wk is not None:
            csa2.quantize_kv(gc, dev(k[w0 - p0:]), dev(v[w0 - p0:]), dev(seq[w0 - p0:]),
                             dev(pos[w0 - p0:]), win_k=dev(wk), win_v=dev(wv))


def check_index_set(got, want, scores, kth, rel=REL_EXEMPT, exact=False):
    """got/want: index rows (ascending, -1 padded).  scores: callable giving the
    oracle score of an index.  Positions in the symmetric difference must lie
    within rel * |kth| of the oracle's k-th value (none allowed if exact)."""
    got = np.asarray(got)
    want = np.asarray(want)
    g = got[got >= 0]
    w = want[want >= 0]
    assert np.all(np.diff(g) > 0), "GPU indices not strictly ascending"
    assert np.all(got[len(g):] == -1), "GPU padding is not -1"
    assert len(g) == len(w), (len(g), len(w))
    diff = np.setxor1d(g, w)
    if exact:
        assert diff.size == 0, f"index sets differ at {diff[:10]}"
        return 0
    for t in diff:
        sc = scores(int(t))
        assert abs(sc - kth) <= rel * abs(kth), f"index {t}: score {sc} vs kth {kth}"
    return diff.size


def block_scores(pos_scores, N, block=8):
    nb = -(-N // block)
    pad = np.full(nb * block, -np.inf)
    pad[:N] = pos_scores
    return pad.reshape(nb, block).max(1)


def shuffled_pages(seed, n_seq, cap, page_tokens, n_used, spare=3):
    """(table, n_pages) of a shuffled physical pool with `spare` unowned pages
    and -1 entries past each sequence's n_used positions."""
    return G.page_table(seed, n_seq, cap, page_tokens, n_used, spare)


def unpage(phys, table, page_tokens, n):
    """Logical rows [n_seq][n][...] of a paged store [n_pages][page_tokens][...]."""
    t = np.arange(n)
    return phys[table[:, t // page_tokens], t % page_tokens]
