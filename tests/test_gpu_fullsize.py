"""GPU parity at the full workload sizes, in the launch configuration the
benchmark times.

* decoder20_1m_b4: 4 sequences x 1,048,576 positions, the 20-layer pattern
  [Full + 3 Reuse] + 4 x [Reindex + 3 Reuse]; group_64k_b32: 32 x 65,536,
  Full + 3 Reuse; hier_256k_b8: 8 x 262,144, Full + Reindex + 3 Reuse.  Every
  output of the step is checked: block maxima, pool, the Full and Reindex index
  sets, and every layer's attention output.  decoder20_1m_b4 also runs every
  call on a paged copy of the cache (256-token pages over a shuffled pool), which
  must give the contiguous cache's outputs bit for bit.
* prefill_8k_over_128k: 8,192 causal queries over a 131,072-position prefix
  plus the chunk itself (seq = 0 for all, ctx_i = 131,073 + i).  The GPU runs all
  8,192 queries in one call per stage; the oracle checks a strided sample.

Stages are isolated as in the smaller parity tests: Reindex receives the
oracle's pool and attention the oracle's index sets, so that an exempt near tie
cannot cascade; the GPU-only chain is compared end to end where its index sets
equal the oracle's.  Attention runs as the benchmark runs it: a group's Full or
Reindex layer stores the gathered main records, its Reuse layers read them.
"""
import sys
import time

import numpy as np
import pytest

import oracle as O
from fp4_kv_cache_decode_amd import datagen as G
from parity import ATTN_TOL, REL_EXEMPT, block_scores, check_index_set, fill_both, shuffled_pages

pytestmark = [pytest.mark.gpu, pytest.mark.timeout(1200)]

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


def _check_block_maxima(gM, sc, N):
    """GPU block maxima against the oracle's fp64 scores (fp32 rounding only)."""
    want = block_scores(sc, N)
    got = gM[:want.size].astype(np.float64)
    err = np.abs(got - want) / (np.abs(want) + 1.0)
    assert float(err.max()) <= REL_EXEMPT, float(err.max())
    return float(err.max())


@pytest.mark.parametrize("name", ["decoder20_1m_b4", "group_64k_b32", "hier_256k_b8"])
def test_decode_step_full_size(K, name):
    wl = G.WORKLOADS[name]
    B, N, L = wl.B, wl.N, len(wl.layers)
    seed = 0
    _say(f"{name}: building caches B={B} N={N} L={L}")
    t0 = time.time()
    oc = O.Cache(wl.n_seq, wl.cap, L, wl.w_cap)
    gc = K.Cache(wl.n_seq, wl.cap, L, wl.w_cap)
    gp = None
    if name == "decoder20_1m_b4":
        P = 256
        table, n_pages = shuffled_pages(seed, wl.n_seq, wl.cap, P, [N] * wl.n_seq)
        gp = K.Cache(wl.n_seq, wl.cap, L, wl.w_cap, page_tokens=P, n_pages=n_pages,
                     page_table=torch.from_numpy(table))
    fill_both(seed, wl.n_seq, N, L, oc, gc if gp is None else (gc, gp), chunk=G.CHUNK,
              workers=16)
    torch.cuda.synchronize()
    _say(f"  caches built in {time.time() - t0:.1f}s")
    # the stored bytes are identical (quantise-on-write parity at full size)
    assert torch.equal(gc.idxk.cpu(), torch.from_numpy(oc.idxk))
    assert torch.equal(gc.kv.cpu(), torch.from_numpy(oc.kv))
    assert np.array_equal(gc.wk.cpu().numpy()[:, :, :], oc.wk) and \
        np.array_equal(gc.wv.cpu().numpy(), oc.wv)

    seq, ctx = wl.seq(), wl.ctx()
    dseq, dctx = dev(seq), dev(ctx)
    M = torch.empty((B, K.block_stride(N)), dtype=torch.float32, device="cuda")
    gpool_t = torch.empty((B, G.N_BLOCKS), dtype=torch.int32, device="cuda")
    gidx_t = torch.empty((B, G.TOPK), dtype=torch.int32, device="cuda")
    out_t = torch.empty((B, G.H, G.D), dtype=torch.float32, device="cuda")
    ws_ri = K.alloc_workspace(K.OP_INDEX_REINDEX, B)
    ws_sel = K.alloc_workspace(K.OP_SELECT_POOL, B, N)
    ws_at = K.alloc_workspace(K.OP_DECODE_ATTN, B)
    kvg = torch.empty((B, G.TOPK, K.RECORD), dtype=torch.uint8, device="cuda")
    kvg_p = torch.empty_like(kvg)

    def paged_same(fn, *outs):
        """Run fn(cache) on the paged copy into fresh buffers shaped like outs,
        then require the contiguous results bit for bit."""
        if gp is None:
            return
        got = fn(gp)
        torch.cuda.synchronize()
        for g, o in zip(got, outs):
            assert torch.equal(g, o)

    opool = oidx = None
    gpu_chain_equal = True
    n_exempt = 0
    for l, mode in enumerate(wl.layers):
        if mode in "FI":
            qi, wi = G.index_queries(seed, l, B)
            scs = [oc.scores(int(seq[b]), qi[b], wi[b], int(ctx[b])) for b in range(B)]
        if mode == "F":
            # the benchmark's Full-layer chain: scan, pool select, pool top-k
            K.index_block_scores(gc, dev(qi), dev(wi), dseq, dctx, N, M)
            K.index_select_pool(M, dctx, N, gpool_t, ws_sel)
            K.index_reindex(gc, dev(qi), dev(wi), dseq, dctx, gpool_t, gidx_t, ws_ri)
            torch.cuda.synchronize()

            def full_chain(c):
                Mx, px, ix = M.clone(), torch.empty_like(gpool_t), torch.empty_like(gidx_t)
                for b in range(B):                    # every block the scan must write
                    Mx[b, :-(-int(ctx[b]) // 8)] = float("nan")
                K.index_block_scores(c, dev(qi), dev(wi), dseq, dctx, N, Mx)
                K.index_select_pool(Mx, dctx, N, px, ws_sel)
                K.index_reindex(c, dev(qi), dev(wi), dseq, dctx, px, ix, ws_ri)
                return Mx, px, ix
            paged_same(full_chain, M, gpool_t, gidx_t)
            opool, oidx, kb, kp = oc.index_full(qi, wi, seq, ctx)
            gM, gpool, gidx = M.cpu().numpy(), gpool_t.cpu().numpy(), gidx_t.cpu().numpy()
            for b in range(B):
                e = _check_block_maxima(gM[b], scs[b], N)
                Mb = block_scores(scs[b], N)
                n_exempt += check_index_set(gpool[b], opool[b], lambda j: Mb[j], kb[b])
                n_exempt += check_index_set(gidx[b], oidx[b], lambda t: scs[b][t], kp[b])
            _say(f"  layer {l} Full: block maxima rel err {e:.2g}, exempt diffs {n_exempt}")
            gpu_chain_equal &= np.array_equal(gidx, oidx)
        elif mode == "I":
            # Reindex on the oracle's pool (isolated) ...
            K.index_reindex(gc, dev(qi), dev(wi), dseq, dctx, dev(opool), gidx_t, ws_ri)
            torch.cuda.synchronize()

            def reindex(c):
                ix = torch.empty_like(gidx_t)
                K.index_reindex(c, dev(qi), dev(wi), dseq, dctx, dev(opool), ix, ws_ri)
                return (ix,)
            paged_same(reindex, gidx_t)
            oidx, kp = oc.index_reindex(qi, wi, seq, ctx, opool)
            gidx = gidx_t.cpu().numpy()
            for b in range(B):
                n_exempt += check_index_set(gidx[b], oidx[b], lambda t: scs[b][t], kp[b])
            gpu_chain_equal &= np.array_equal(gidx, oidx)
            _say(f"  layer {l} Reindex: exempt diffs so far {n_exempt}")
        # attention of every layer on the group's (oracle) index set, as the
        # benchmark runs it: the group's first layer stores the gathered
        # records, its Reuse layers read them with the same idx
        q = G.attn_queries(seed, l, B)
        gather = dict(kvg_in=kvg) if mode == "R" else dict(kvg_out=kvg)
        K.decode_attn(gc, l, dev(q), dev(oidx), dseq, dctx, out_t, ws_at, **gather)
        torch.cuda.synchronize()

        def attend(c):
            ox = torch.empty_like(out_t)
            g = dict(kvg_in=kvg_p) if mode == "R" else dict(kvg_out=kvg_p)
            K.decode_attn(c, l, dev(q), dev(oidx), dseq, dctx, ox, ws_at, **g)
            return (ox,)
        paged_same(attend, out_t)
        want = oc.decode_attn(l, q, oidx, seq, ctx)
        err = float(np.max(np.abs(out_t.cpu().numpy() - want)))
        assert err <= ATTN_TOL, (l, err)
        if mode != "R":
            _say(f"  layer {l} attention max-abs err {err:.3g}")
    _say(f"  GPU index sets equal the oracle's in every layer: {gpu_chain_equal}")
    if gp is not None:
        _say("  paged cache (256-token pages): every output bit-identical")


def test_prefill_chunk_8k_over_128k(K):
    wl = G.WORKLOADS["prefill_8k_over_128k"]
    B, N0 = wl.B, wl.N                 # 8,192 queries after a 131,072-position prefix
    cap = wl.cap                       # 139,264 positions written
    seed = 0
    _say(f"prefill_8k_over_128k: building cache cap={cap} w_cap={wl.w_cap}")
    oc = O.Cache(1, cap, 1, wl.w_cap)
    gc = K.Cache(1, cap, 1, wl.w_cap)
    # window rows for every position a query's window can reach
    fill_both(seed, 1, cap, 1, oc, gc, chunk=G.CHUNK, wlo=N0 - G.WINDOW, workers=16)
    torch.cuda.synchronize()
    assert torch.equal(gc.kv.cpu(), torch.from_numpy(oc.kv))
    assert torch.equal(gc.idxk.cpu(), torch.from_numpy(oc.idxk))
    assert np.array_equal(gc.wk.cpu().numpy(), oc.wk)

    seq, ctx = wl.seq(), wl.ctx()
    qi, wi = G.index_queries(seed, 0, B)
    q = G.attn_queries(seed, 0, B)
    sample = np.unique(np.r_[0, 1, 7, 127, 128, 1000, 4095, 4096, 6000, 8190, 8191,
                             np.arange(257, B, 1031)])
    # the benchmark keeps 512 blocks (no Reindex layer follows); the decoder's
    # 2,048-block pool is checked too, and both give the same top-512
    oidx_by = {}
    for nbk in (wl.extra["pool_blocks"], G.N_BLOCKS):
        pool_t = torch.empty((B, nbk), dtype=torch.int32, device="cuda")
        idx_t = torch.empty((B, G.TOPK), dtype=torch.int32, device="cuda")
        ws = K.alloc_workspace(K.OP_INDEX_FULL, B, cap, n_blocks=nbk)
        t0 = time.time()
        K.index_full(gc, dev(qi), dev(wi), dev(seq), dev(ctx), cap, pool_t, idx_t, ws,
                     n_blocks=nbk)
        torch.cuda.synchronize()
        _say(f"  GPU index_full over {B} queries, {nbk} blocks: {time.time() - t0:.2f}s")
        gpool, gidx = pool_t.cpu().numpy(), idx_t.cpu().numpy()
        opool, oidx, kb, kp = oc.index_full(qi[sample], wi[sample], seq[sample], ctx[sample],
                                            n_blocks=nbk)
        n_exempt = 0
        for j, b in enumerate(sample):
            sc = oc.scores(0, qi[b], wi[b], int(ctx[b]))
            Mb = block_scores(sc, int(ctx[b]))
            n_exempt += check_index_set(gpool[b], opool[j], lambda t: Mb[t], kb[j])
            n_exempt += check_index_set(gidx[b], oidx[j], lambda t: sc[t], kp[j])
        _say(f"  {sample.size} sampled queries: blocks and top-512 match, exempt diffs {n_exempt}")
        oidx_by[nbk] = (gidx, oidx)
    gidx, oidx = oidx_by[wl.extra["pool_blocks"]]
    assert np.array_equal(oidx, oidx_by[G.N_BLOCKS][1])

    # attention for all queries in one call; the sampled rows use the oracle's sets
    idx_mixed = gidx.copy()
    idx_mixed[sample] = oidx
    out_t = torch.empty((B, G.H, G.D), dtype=torch.float32, device="cuda")
    ws_at = K.alloc_workspace(K.OP_DECODE_ATTN, B)
    K.decode_attn(gc, 0, dev(q), dev(idx_mixed), dev(seq), dev(ctx), out_t, ws_at)
    torch.cuda.synchronize()
    got = out_t.cpu().numpy()[sample]
    want = oc.decode_attn(0, q[sample], oidx, seq[sample], ctx[sample])
    err = float(np.max(np.abs(got - want)))
    _say(f"  attention max-abs err over the sample {err:.3g}")
    assert err <= ATTN_TOL


def test_gather_row_full_size(K):
    """The gather row's launch configuration: 1,024 queries, each on its own
    65,536-position sequence (one workgroup per query, no split), a random
    top-512 set per query plus the window.  Every sequence holds the same rows
    (as in the benchmark), so the oracle needs one sequence; a strided sample of
    queries is checked, in all four layers."""
    B, N, L = 1024, 65536, 4
    seed = 0
    _say(f"gather row: B={B} N={N} L={L}")
    oc = O.Cache(1, N, L)
    gc = K.Cache(B, N, L)
    fill_both(seed, 1, N, L, oc, gc, chunk=G.CHUNK)
    gc.kv[1:].copy_(gc.kv[0:1].expand(B - 1, -1, -1))
    gc.wk[:, 1:].copy_(gc.wk[:, 0:1].expand(-1, B - 1, -1, -1))
    gc.wv[:, 1:].copy_(gc.wv[:, 0:1].expand(-1, B - 1, -1, -1))
    rng = np.random.default_rng(seed)
    idx = np.sort(np.argpartition(rng.random((B, N), dtype=np.float32), G.TOPK, axis=1)
                  [:, :G.TOPK], axis=1).astype(np.int32)
    seq, ctx = np.arange(B, dtype=np.int32), np.full(B, N, np.int64)
    sample = np.r_[0, 1, np.arange(37, B, 97), B - 1]
    ws = K.alloc_workspace(K.OP_DECODE_ATTN, B)
    assert ws.numel() == 1                     # one workgroup per query: no partials
    out = torch.empty((B, G.H, G.D), dtype=torch.float32, device="cuda")
    for l in range(L):
        q = G.attn_queries(seed, l, B)
        K.decode_attn(gc, l, dev(q), dev(idx), dev(seq), dev(ctx), out, ws)
        torch.cuda.synchronize()
        want = oc.decode_attn(l, q[sample], idx[sample], np.zeros(sample.size, np.int32),
                              ctx[sample])
        err = float(np.max(np.abs(out.cpu().numpy()[sample] - want)))
        _say(f"  layer {l}: {sample.size} sampled queries, max-abs err {err:.3g}")
        assert err <= ATTN_TOL
