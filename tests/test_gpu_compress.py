"""GPU parity of global-KV compression (csa2_compress_kv) and of CSA2 layers
over a compressed store: the encoder's layers at m = 2 (origotech.dev deep
dive "Inside DeepSeek V4.1-Flash", section "How the architecture shrinks the
KV cache": layers 1-2 sliding window only, then 3 x [Full + 5 Reuse] at
compression 2).

Reading checked (the same on both sides): entry e stands for tokens 2e, 2e+1
and holds their fp32 mean, quantised as a token row; the window keeps every
token; a query with N tokens of context sees entries [0, N // 2) (the indexer
gets ctx // 2) and window rows [N - 128, N) (the attention gets ctx).

Bars: codes, scales and window bytes bit-exact; index sets exact up to the
1e-5 near-tie exemption; attention within 2e-3 max-abs of the oracle.
"""
import sys

import numpy as np
import pytest

import oracle as O
from fp4_kv_cache_decode_amd import datagen as G
from parity import ATTN_TOL, block_scores, check_index_set, shuffled_pages, unpage

pytestmark = [pytest.mark.gpu, pytest.mark.timeout(900)]

torch = pytest.importorskip("torch")


def _say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def K():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from fp4_kv_cache_decode_amd import csa2
    csa2.lib()
    return csa2


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def _both(K, oc, gc, k, v, ik, wk, wv, seq, pos, m):
    """One csa2_compress_kv call on the device cache and the same on the oracle's."""
    oc.compress(k, v, ik, wk, wv, seq, pos, m)
    d = lambda a: None if a is None else dev(a)
    K.compress_kv(gc, d(k), d(v), dev(seq), dev(pos), m, idx_k=d(ik), win_k=d(wk), win_v=d(wv))


def _midpoint_pairs(rng, n_pairs):
    """Token pairs whose fp32 mean puts every channel of a 16-channel group on an
    E2M1 midpoint or grid value at scale 1 (group maximum 6): the sums are exact,
    so the mean lands exactly there and the ties to even decide every code."""
    grid = np.array([6, .25, .75, 1.25, 1.75, 2.5, 3.5, 5, -.25, -.75, -1.25, -1.75, -2.5,
                     -3.5, -5, 0], np.float32)
    k = np.empty((2 * n_pairs, 128), np.float32)
    for i in range(n_pairs):
        mean = np.concatenate([rng.permutation(grid) for _ in range(8)])
        mean[::16] = 6 * rng.choice([-1, 1])          # group max stays 6
        d = np.float32(0.125) * rng.choice([-1, 1], 128).astype(np.float32)
        k[2 * i], k[2 * i + 1] = mean - d, mean + d
    return k


@pytest.mark.parametrize("paged", [False, True], ids=["contiguous", "paged64"])
def test_compress_m2_bit_exact(K, paged):
    rng = np.random.default_rng(21 + paged)
    n_seq, cap, n_layers, w_cap = 3, 1024, 2, 200
    L = [1000, 517, 1]                         # entries per sequence (2 L tokens)
    _say(f"compress m=2 paged={paged}: entries {L}")
    kw = dict(idxk_scale=0.37, wk_scale=1.7, wv_scale=0.5)
    oc = O.Cache(n_seq, cap, n_layers, w_cap, **kw)
    table = None
    if paged:
        table, n_pages = shuffled_pages(5, n_seq, cap, 64, L)
        gc = K.Cache(n_seq, cap, n_layers, w_cap, page_tokens=64, n_pages=n_pages,
                     page_table=torch.from_numpy(table), **kw)
    else:
        gc = K.Cache(n_seq, cap, n_layers, w_cap, **kw)
    seq = np.concatenate([np.full(2 * n, s, np.int32) for s, n in enumerate(L)])
    pos = np.concatenate([np.arange(2 * n, dtype=np.int64) for n in L])
    n = seq.size
    k = (rng.standard_normal((n, 128)) * np.repeat(rng.uniform(0.01, 30, (n // 2, 1)), 2, 0)
         ).astype(np.float32)
    v = (rng.standard_normal((n, 128)) * 3).astype(np.float32)
    ik = (rng.standard_normal((n, 64)) * 40).astype(np.float32)
    k[:64] = _midpoint_pairs(rng, 32)          # sequence 0, entries 0..31
    v[65] = -v[64]                             # a pair whose V mean is exactly zero
    v[66] = v[67]                              # a pair of equal rows
    _both(K, oc, gc, k, v, ik, None, None, seq, pos, 2)
    # window rows: the last (up to) 100 tokens of each sequence, re-writing the
    # same entries, then one token whose pair is not complete (window only)
    for s, ne in enumerate(L):
        t0 = 2 * max(0, ne - 50)
        sel = np.flatnonzero((seq == s) & (pos >= t0))
        wk = (rng.standard_normal((n_layers, sel.size, 128)) * 4).astype(np.float32)
        wv = (rng.standard_normal((n_layers, sel.size, 128)) * 2).astype(np.float32)
        _both(K, oc, gc, k[sel], v[sel], ik[sel], wk, wv, seq[sel], pos[sel], 2)
        one = np.array([2 * ne], np.int64)
        wk1 = (rng.standard_normal((n_layers, 1, 128)) * 4).astype(np.float32)
        _both(K, oc, gc, None, None, None, wk1, -wk1, np.array([s], np.int32), one, 2)
    torch.cuda.synchronize()
    gkv, gik = gc.kv.cpu().numpy(), gc.idxk.cpu().numpy()
    if paged:
        gkv, gik = unpage(gkv, table, 64, cap), unpage(gik, table, 64, cap)
        for s, ne in enumerate(L):                 # only the entries written
            assert np.array_equal(gkv[s, :ne], oc.kv[s, :ne])
            assert np.array_equal(gik[s, :ne], oc.idxk[s, :ne])
    else:
        assert np.array_equal(gkv, oc.kv)
        assert np.array_equal(gik, oc.idxk)
    assert np.array_equal(gc.wk.cpu().numpy(), oc.wk)
    assert np.array_equal(gc.wv.cpu().numpy(), oc.wv)


def test_compress_m1_is_quantize(K):
    rng = np.random.default_rng(23)
    n, n_seq, cap, n_layers = 777, 2, 2048, 2
    k = (rng.standard_normal((n, 128)) * 5).astype(np.float32)
    v = (rng.standard_normal((n, 128)) * 0.1).astype(np.float32)
    ik = (rng.standard_normal((n, 64)) * 2).astype(np.float32)
    wk = rng.standard_normal((n_layers, n, 128)).astype(np.float32)
    wv = rng.standard_normal((n_layers, n, 128)).astype(np.float32)
    seq = np.repeat(np.arange(n_seq, dtype=np.int32), [400, n - 400])
    pos = np.concatenate([np.arange(400), 1000 + np.arange(n - 400)]).astype(np.int64)
    a = K.Cache(n_seq, cap, n_layers, 1024)
    b = K.Cache(n_seq, cap, n_layers, 1024)
    K.quantize_kv(a, dev(k), dev(v), dev(seq), dev(pos), idx_k=dev(ik), win_k=dev(wk),
                  win_v=dev(wv))
    K.compress_kv(b, dev(k), dev(v), dev(seq), dev(pos), 1, idx_k=dev(ik), win_k=dev(wk),
                  win_v=dev(wv))
    torch.cuda.synchronize()
    for x, y in ((a.kv, b.kv), (a.idxk, b.idxk), (a.wk, b.wk), (a.wv, b.wv)):
        assert torch.equal(x, y)


def _fill_group(K, oc, gc, seed, s, N, layers, group=0):
    """Tokens [0, N) of sequence s at m = 2 (complete pairs), then window rows of
    every layer for [N - 128, N), the unpaired last token included."""
    n2 = N - N % 2
    k, v, ik = G.kv_rows(seed, s, 0, n2, group)
    _both(K, oc, gc, k, v, ik, None, None, np.full(n2, s, np.int32),
          np.arange(n2, dtype=np.int64), 2)
    w0 = max(0, N - G.WINDOW)
    wk = np.stack([G.window_rows(seed, l, s, w0, N)[0] for l in layers])
    wv = np.stack([G.window_rows(seed, l, s, w0, N)[1] for l in layers])
    _both(K, oc, gc, None, None, None, wk, wv, np.full(N - w0, s, np.int32),
          np.arange(w0, N, dtype=np.int64), 2)


@pytest.mark.parametrize("paged", [False, True], ids=["contiguous", "paged64"])
def test_encoder_group_m2_against_oracle(K, paged):
    """One sliding-window layer and one [Full + 5 Reuse] group at m = 2 over
    three sequences of 3,001, 4,096 and 515 tokens (a paged store: 64-entry
    pages over a shuffled pool)."""
    seed = 3
    Ns = np.array([3001, 4096, 515], np.int64)
    B, n_layers = Ns.size, 7                    # layer 0: window only; 1: Full; 2-6: Reuse
    cap = int(Ns.max()) // 2 + 64               # 2,112 entries = 33 pages of 64
    oc = O.Cache(B, cap, n_layers, 256)
    if paged:
        table, n_pages = shuffled_pages(7, B, cap, 64, Ns // 2)
        gc = K.Cache(B, cap, n_layers, 256, page_tokens=64, n_pages=n_pages,
                     page_table=torch.from_numpy(table))
    else:
        gc = K.Cache(B, cap, n_layers, 256)
    for s in range(B):
        _fill_group(K, oc, gc, seed, s, int(Ns[s]), range(n_layers))
    torch.cuda.synchronize()
    if paged:
        gkv = unpage(gc.kv.cpu().numpy(), table, 64, cap)
        for s in range(B):
            assert np.array_equal(gkv[s, :Ns[s] // 2], oc.kv[s, :Ns[s] // 2])
    else:
        assert np.array_equal(gc.kv.cpu().numpy(), oc.kv)
    assert np.array_equal(gc.wk.cpu().numpy(), oc.wk)

    seq = np.arange(B, dtype=np.int32)
    ctx, ctx_c = Ns, Ns // 2
    qi, wi = G.index_queries(seed, 1, B)
    nbk = G.WORKLOADS["encoder20_m2_chunk8k_over_128k"].extra["pool_blocks"]
    pool = torch.empty((B, nbk), dtype=torch.int32, device="cuda")
    idx = torch.empty((B, G.TOPK), dtype=torch.int32, device="cuda")
    ws = K.alloc_workspace(K.OP_INDEX_FULL, B, int(ctx_c.max()), n_blocks=nbk)
    K.index_full(gc, dev(qi), dev(wi), dev(seq), dev(ctx_c), int(ctx_c.max()), pool, idx, ws,
                 n_blocks=nbk)
    torch.cuda.synchronize()
    opool, oidx, kb, kp = oc.index_full(qi, wi, seq, ctx_c, n_blocks=nbk)
    # the encoder's 512 blocks hold the flat top-512: the decoder's 2,048-block pool agrees
    assert np.array_equal(oc.index_full(qi, wi, seq, ctx_c)[1], oidx)
    gpool, gidx = pool.cpu().numpy(), idx.cpu().numpy()
    for b in range(B):
        sc = oc.scores(b, qi[b], wi[b], int(ctx_c[b]))
        check_index_set(gpool[b], opool[b], lambda t: block_scores(sc, int(ctx_c[b]))[t], kb[b])
        check_index_set(gidx[b], oidx[b], lambda t: sc[t], kp[b])
        assert gidx[b].max() < ctx_c[b]

    ws_at = K.alloc_workspace(K.OP_DECODE_ATTN, B)
    out = torch.empty((B, G.H, G.D), dtype=torch.float32, device="cuda")
    none = np.full((B, G.TOPK), -1, np.int32)
    q0 = G.attn_queries(seed, 0, B)
    K.decode_attn(gc, 0, dev(q0), dev(none), dev(seq), dev(ctx), out, ws_at)
    torch.cuda.synchronize()
    err = float(np.abs(out.cpu().numpy() - oc.decode_attn(0, q0, none, seq, ctx)).max())
    _say(f"  window-only layer: max-abs err {err:.3g}")
    assert err <= ATTN_TOL
    kvg = torch.empty((B, G.TOPK, 144), dtype=torch.uint8, device="cuda")
    for l in range(1, n_layers):
        q = G.attn_queries(seed, l, B)
        g_in, g_out = (None, kvg) if l == 1 else (kvg, None)
        K.decode_attn(gc, l, dev(q), dev(oidx), dev(seq), dev(ctx), out, ws_at,
                      kvg_in=g_in, kvg_out=g_out)
        torch.cuda.synchronize()
        err = float(np.abs(out.cpu().numpy() - oc.decode_attn(l, q, oidx, seq, ctx)).max())
        _say(f"  layer {l} ({'Full' if l == 1 else 'Reuse'}): max-abs err {err:.3g}")
        assert err <= ATTN_TOL


def test_encoder_chunk_8k_over_128k_sampled(K):
    """The encoder row's launch configuration: 8,192 causal queries of one
    sequence after a 131,072-token prefix, one group's store at m = 2 (65,536 +
    4,096 entries), all queries in one call per stage; the oracle checks a
    strided sample (index sets, and the window-only, Full and Reuse layers)."""
    wl = G.WORKLOADS["encoder20_m2_chunk8k_over_128k"]
    B, N0, m = wl.B, wl.N, wl.m
    cap_c = wl.cap // m
    seed = 0
    layers = (0, 2, 3)                          # a window-only, a Full and a Reuse layer
    _say(f"encoder chunk: {B} queries, prefix {N0}, entries {cap_c}")
    oc = O.Cache(1, cap_c, len(layers), wl.w_cap)
    gc = K.Cache(1, cap_c, len(layers), wl.w_cap)
    for p in range(0, N0, G.CHUNK):
        k, v, ik = G.kv_rows(seed, 0, p, p + G.CHUNK)
        _both(K, oc, gc, k, v, ik, None, None, np.zeros(G.CHUNK, np.int32),
              np.arange(p, p + G.CHUNK, dtype=np.int64), m)
    w0 = N0 - G.WINDOW
    wk = np.stack([G.window_rows(seed, l, 0, w0, N0)[0] for l in layers])
    wv = np.stack([G.window_rows(seed, l, 0, w0, N0)[1] for l in layers])
    _both(K, oc, gc, None, None, None, wk, wv, np.zeros(G.WINDOW, np.int32),
          np.arange(w0, N0, dtype=np.int64), m)
    k, v, ik = G.kv_rows(seed, 0, N0, N0 + B)
    wk = np.stack([G.window_rows(seed, l, 0, N0, N0 + B)[0] for l in layers])
    wv = np.stack([G.window_rows(seed, l, 0, N0, N0 + B)[1] for l in layers])
    _both(K, oc, gc, k, v, ik, wk, wv, np.zeros(B, np.int32),
          np.arange(N0, N0 + B, dtype=np.int64), m)
    torch.cuda.synchronize()
    assert np.array_equal(gc.kv.cpu().numpy(), oc.kv)
    assert np.array_equal(gc.idxk.cpu().numpy(), oc.idxk)
    assert np.array_equal(gc.wk.cpu().numpy(), oc.wk)

    seq, ctx = wl.seq(), wl.ctx()
    ctx_c = ctx // m
    qi, wi = G.index_queries(seed, 2, B)
    nbk = wl.extra["pool_blocks"]
    pool = torch.empty((B, nbk), dtype=torch.int32, device="cuda")
    idx = torch.empty((B, G.TOPK), dtype=torch.int32, device="cuda")
    ws = K.alloc_workspace(K.OP_INDEX_FULL, B, cap_c, n_blocks=nbk)
    K.index_full(gc, dev(qi), dev(wi), dev(seq), dev(ctx_c), cap_c, pool, idx, ws, n_blocks=nbk)
    torch.cuda.synchronize()
    gpool, gidx = pool.cpu().numpy(), idx.cpu().numpy()
    sample = np.unique(np.r_[0, 1, 2, 3, 255, 256, 4095, 8190, 8191, np.arange(97, B, 1013)])
    opool, oidx, kb, kp = oc.index_full(qi[sample], wi[sample], seq[sample], ctx_c[sample],
                                        n_blocks=nbk)
    assert np.array_equal(oc.index_full(qi[sample], wi[sample], seq[sample], ctx_c[sample])[1],
                          oidx)
    n_exempt = 0
    for j, b in enumerate(sample):
        sc = oc.scores(0, qi[b], wi[b], int(ctx_c[b]))
        Mb = block_scores(sc, int(ctx_c[b]))
        n_exempt += check_index_set(gpool[b], opool[j], lambda t: Mb[t], kb[j])
        n_exempt += check_index_set(gidx[b], oidx[j], lambda t: sc[t], kp[j])
    _say(f"  {sample.size} sampled queries: pool and top-512 match, exempt diffs {n_exempt}")

    idx_mixed = gidx.copy()
    idx_mixed[sample] = oidx
    none = np.full((B, G.TOPK), -1, np.int32)
    out = torch.empty((B, G.H, G.D), dtype=torch.float32, device="cuda")
    ws_at = K.alloc_workspace(K.OP_DECODE_ATTN, B)
    for li, l in enumerate(layers):
        q = G.attn_queries(seed, l, B)
        use = none if l == 0 else idx_mixed
        K.decode_attn(gc, li, dev(q), dev(use), dev(seq), dev(ctx), out, ws_at)
        torch.cuda.synchronize()
        want = oc.decode_attn(li, q[sample], use[sample], seq[sample], ctx[sample])
        err = float(np.max(np.abs(out.cpu().numpy()[sample] - want)))
        _say(f"  encoder layer {l}: max-abs err over the sample {err:.3g}")
        assert err <= ATTN_TOL
