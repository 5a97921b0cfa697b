"""GPU parity of paged caches: the global store (main-KV records and indexer
keys) scattered over a shuffled pool of physical pages behind a page table.

Every result is checked against the oracle, which works on the logical cache
and knows nothing of pages, under the same bars as the contiguous tests.  It is
also checked bit for bit against the contiguous HIP path on the same rows.  The
page tables leave unowned pages in the pool, and entries of -1 past each
sequence's written positions.
"""
import sys

import numpy as np
import pytest

import oracle as O
from fp4_kv_cache_decode_amd import datagen as G
from parity import check_index_set, block_scores, fill_both, shuffled_pages, unpage

pytestmark = pytest.mark.gpu

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


def _paged(K, seed, n_seq, cap, P, n_used, n_layers=1, w_cap=G.WINDOW, **kw):
    table, n_pages = shuffled_pages(seed, n_seq, cap, P, n_used)
    return K.Cache(n_seq, cap, n_layers, w_cap, page_tokens=P, n_pages=n_pages,
                   page_table=torch.from_numpy(table), **kw), table


@pytest.mark.parametrize("P", [64, 256])
def test_paged_quantize_bit_exact(K, P):
    """Rows at random (seq, pos) land in the page the table names; the logical
    view equals the oracle's cache and the unowned pages stay untouched."""
    _say(f"paged quantize P={P}")
    rng = np.random.default_rng(P)
    n, n_seq, cap = 3000, 3, 4096
    k = (rng.standard_normal((n, 128)) * rng.uniform(0.01, 30, (n, 1))).astype(np.float32)
    v = (rng.standard_normal((n, 128)) * 3).astype(np.float32)
    ik = (rng.standard_normal((n, 64)) * 40).astype(np.float32)
    seq = rng.integers(0, n_seq, n).astype(np.int32)
    pos = rng.integers(0, cap, n).astype(np.int64)
    keep = np.unique(seq.astype(np.int64) * cap + pos, return_index=True)[1]
    seq, pos, k, v, ik = seq[keep], pos[keep], k[keep], v[keep], ik[keep]
    oc = O.Cache(n_seq, cap)
    oc.quantize(k, v, ik, None, None, seq, pos)
    gp, table = _paged(K, 5, n_seq, cap, P, [cap] * n_seq)
    K.quantize_kv(gp, dev(k), dev(v), dev(seq), dev(pos), idx_k=dev(ik))
    torch.cuda.synchronize()
    kv, idxk = gp.kv.cpu().numpy(), gp.idxk.cpu().numpy()
    assert np.array_equal(unpage(kv, table, P, cap), oc.kv)
    assert np.array_equal(unpage(idxk, table, P, cap), oc.idxk)
    unowned = np.setdiff1d(np.arange(gp.n_pages), table[table >= 0])
    assert unowned.size == 3
    assert not kv[unowned].any() and not idxk[unowned].any()


def _index_case(K, P, seed=11, N=40001, B=3):
    cap = (-(-N // P) + 2) * P                 # two unused (-1) pages per sequence
    oc = O.Cache(B, cap)
    gc = K.Cache(B, cap)
    gp, table = _paged(K, seed, B, cap, P, [N] * B)
    fill_both(seed, B, N, 1, oc, (gc, gp))
    torch.cuda.synchronize()
    assert (table[:, -2:] == -1).all()
    return oc, gc, gp


def _full(K, c, q, w, seq, ctx, max_ctx):
    B = q.shape[0]
    pool = torch.empty((B, 2048), dtype=torch.int32, device="cuda")
    idx = torch.empty((B, 512), dtype=torch.int32, device="cuda")
    M = torch.empty((B, K.block_stride(max_ctx)), dtype=torch.float32, device="cuda")
    K.index_full(c, dev(q), dev(w), dev(seq), dev(ctx), max_ctx, pool, idx,
                 K.alloc_workspace(K.OP_INDEX_FULL, B, max_ctx))
    K.index_block_scores(c, dev(q), dev(w), dev(seq), dev(ctx), max_ctx, M)
    torch.cuda.synchronize()
    return pool.cpu().numpy(), idx.cpu().numpy(), M.cpu().numpy()


@pytest.mark.parametrize("P", [64, 256])
def test_paged_index_full_and_reindex(K, P):
    """Full scan, pool, top-512 and a Reindex layer over a paged cache with
    ragged contexts (a partial last page, sequences of different lengths)."""
    _say(f"paged index_full / reindex P={P}")
    N, B = 40001, 3
    oc, gc, gp = _index_case(K, P, N=N, B=B)
    seq = np.array([2, 0, 1], np.int32)        # queries read sequences out of order
    ctx = np.array([N, N - 5, 20000], np.int64)
    q, w = G.index_queries(11, 0, B)
    pool_p, idx_p, M_p = _full(K, gp, q, w, seq, ctx, N)
    pool_c, idx_c, M_c = _full(K, gc, q, w, seq, ctx, N)
    assert np.array_equal(pool_p, pool_c) and np.array_equal(idx_p, idx_c)
    for b in range(B):
        nb = -(-int(ctx[b]) // 8)
        assert np.array_equal(M_p[b, :nb], M_c[b, :nb])
    opool, oidx, kb, kp = oc.index_full(q, w, seq, ctx)
    n_exempt = 0
    for b in range(B):
        sc = oc.scores(int(seq[b]), q[b], w[b], int(ctx[b]))
        Mb = block_scores(sc, int(ctx[b]))
        np.testing.assert_allclose(M_p[b, :Mb.size], Mb, rtol=2e-6, atol=1e-6)
        n_exempt += check_index_set(pool_p[b], opool[b], lambda j: Mb[j], kb[b])
        n_exempt += check_index_set(idx_p[b], oidx[b], lambda t: sc[t], kp[b])
    # a Reindex layer on the oracle's pool
    q1, w1 = G.index_queries(11, 1, B)
    oidx1, kp1 = oc.index_reindex(q1, w1, seq, ctx, opool)
    outs = []
    for c in (gp, gc):
        idx = torch.empty((B, 512), dtype=torch.int32, device="cuda")
        K.index_reindex(c, dev(q1), dev(w1), dev(seq), dev(ctx), dev(opool), idx,
                        K.alloc_workspace(K.OP_INDEX_REINDEX, B))
        torch.cuda.synchronize()
        outs.append(idx.cpu().numpy())
    assert np.array_equal(outs[0], outs[1])
    for b in range(B):
        sc = oc.scores(int(seq[b]), q1[b], w1[b], int(ctx[b]))
        n_exempt += check_index_set(outs[0][b], oidx1[b], lambda t: sc[t], kp1[b])
    _say(f"  exempt differences: {n_exempt}")


@pytest.mark.parametrize("B", [3, 96])
def test_paged_decode_attn(K, B):
    """Attention over a paged cache on both kernels (tile kernel at B = 3, split
    stream kernel at B = 96): against the oracle, bit for bit against the
    contiguous cache, and through the gathered-record path of Reuse layers."""
    _say(f"paged decode_attn B={B}")
    N, L, P, n_seq = 700, 2, 64, 3
    cap = 768                                   # pages 11 (positions >= 704) unused: -1
    oc = O.Cache(n_seq, cap, L, w_cap=1024)
    gc = K.Cache(n_seq, cap, L, w_cap=1024)
    gp, table = _paged(K, 7, n_seq, cap, P, [N] * n_seq, n_layers=L, w_cap=1024)
    assert (table[:, 11] == -1).all()
    fill_both(71, n_seq, N, L, oc, (gc, gp), wlo=0)
    rng = np.random.default_rng(B)
    seq = (np.arange(B) % n_seq).astype(np.int32)
    ctx = rng.integers(1, N + 1, B).astype(np.int64)
    ctx[:3] = [N, 129, 1]
    idx = np.full((B, 512), -1, np.int32)
    for b in range(B):
        m = int(rng.integers(0, min(512, int(ctx[b])) + 1))
        idx[b, :m] = np.sort(rng.choice(int(ctx[b]), m, replace=False))
    idx[0, :512] = np.sort(rng.choice(N, 512, replace=False))
    didx, dseq, dctx = dev(idx), dev(seq), dev(ctx)
    ws = K.alloc_workspace(K.OP_DECODE_ATTN, B)
    kvg = torch.zeros((B, 512, 144), dtype=torch.uint8, device="cuda")
    for layer in range(L):
        q = G.attn_queries(71, layer, B)
        outs = []
        for c, gather in ((gp, {}), (gc, {}), (gp, dict(kvg_out=kvg) if layer == 0 else
                                              dict(kvg_in=kvg))):
            out = torch.empty((B, 16, 128), dtype=torch.float32, device="cuda")
            K.decode_attn(c, layer, dev(q), didx, dseq, dctx, out, ws, **gather)
            torch.cuda.synchronize()
            outs.append(out.cpu().numpy())
        assert np.array_equal(outs[0], outs[1]), layer
        assert np.array_equal(outs[2], outs[0]), layer
        want = oc.decode_attn(layer, q, idx, seq, ctx)
        err = float(np.max(np.abs(outs[0] - want)))
        _say(f"  layer {layer}: max-abs err {err:.3g}")
        assert err <= 1e-4
    # the gathered records are the logical cache's records of the valid entries
    gh = kvg.cpu().numpy()
    valid = (idx >= 0) & (idx < ctx[:, None])
    bb, jj = np.nonzero(valid)
    assert np.array_equal(gh[bb, jj], oc.kv[seq[bb], idx[bb, jj]])


def test_window_restored_from_last_128_tokens(K):
    """The storage side of replaying the sliding window: the per-layer FP8
    window stores are dropped (zeroed) while the paged global store is kept;
    re-writing only the last 128 tokens' window rows restores the exact bytes
    attention reads, and the attention output bit for bit."""
    _say("window restore from the last 128 tokens")
    N, L, P, B, w_cap = 5000, 3, 256, 2, 160
    cap = 5120
    oc = O.Cache(B, cap, L, w_cap)
    gp, _ = _paged(K, 13, B, cap, P, [N] * B, n_layers=L, w_cap=w_cap)
    fill_both(29, B, N, L, oc, gp)
    seq = np.arange(B, dtype=np.int32)
    ctx = np.full(B, N, np.int64)
    qi, wi = G.index_queries(29, 0, B)
    _, idx, _, _ = oc.index_full(qi, wi, seq, ctx)
    ws = K.alloc_workspace(K.OP_DECODE_ATTN, B)

    def attend(layer):
        out = torch.empty((B, 16, 128), dtype=torch.float32, device="cuda")
        K.decode_attn(gp, layer, dev(G.attn_queries(29, layer, B)), dev(idx), dev(seq),
                      dev(ctx), out, ws)
        torch.cuda.synchronize()
        return out.cpu().numpy()

    before = [attend(layer) for layer in range(L)]
    wk0, wv0 = gp.wk.clone(), gp.wv.clone()
    gp.wk.zero_()
    gp.wv.zero_()
    w0 = N - G.WINDOW
    for s in range(B):
        k, v, _ = G.kv_rows(29, s, w0, N)
        wk = np.stack([G.window_rows(29, layer, s, w0, N)[0] for layer in range(L)])
        wv = np.stack([G.window_rows(29, layer, s, w0, N)[1] for layer in range(L)])
        K.quantize_kv(gp, dev(k), dev(v), dev(np.full(G.WINDOW, s, np.int32)),
                      dev(np.arange(w0, N, dtype=np.int64)), win_k=dev(wk), win_v=dev(wv))
    torch.cuda.synchronize()
    slots = np.arange(w0, N) % w_cap
    assert torch.equal(gp.wk[:, :, slots], wk0[:, :, slots])
    assert torch.equal(gp.wv[:, :, slots], wv0[:, :, slots])
    for layer in range(L):
        after = attend(layer)
        assert np.array_equal(after, before[layer]), layer
        want = oc.decode_attn(layer, G.attn_queries(29, layer, B), idx, seq, ctx)
        assert float(np.max(np.abs(after - want))) <= 1e-4
