"""HIP-graph capture of a decode step: replays match eager launches exactly,
and both match the oracle.

The step (quantise-on-write, Full indexer, Reindex, attention with the group's
gathered records) is captured once and replayed several times with eager work
and synchronisations in between; every replay must reproduce the eager results
bit for bit.  The same holds for a paged cache (shuffled 128-token pages).  The
replayed pool and index sets are also checked against the oracle under the
near-tie exemption, and every layer's attention output within 2e-3 max-abs of
the oracle given the same index sets.
"""
import numpy as np
import pytest

import oracle as O
from fp4_kv_cache_decode_amd import datagen as G
from parity import ATTN_TOL, block_scores, check_index_set, fill_both

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")


@pytest.mark.parametrize("page_tokens", [0, 128])
def test_graph_replay_matches_eager(page_tokens):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from fp4_kv_cache_decode_amd import csa2 as K
    B, N, L = 3, 40000, 3
    if page_tokens:
        cap = -(-N // page_tokens) * page_tokens
        table, n_pages = G.page_table(23, B, cap, page_tokens, [N] * B)
        gc = K.Cache(B, cap, L, page_tokens=page_tokens, n_pages=n_pages,
                     page_table=torch.from_numpy(table))
    else:
        gc = K.Cache(B, N, L)
    oc = O.Cache(B, N, L)
    fill_both(23, B, N, L, oc, gc)
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    seq, ctx = dev(np.arange(B, dtype=np.int32)), dev(np.array([N, N - 7, 20000], np.int64))
    k, v, ik = G.kv_rows(23, 0, N - 1, N)
    new = dict(k=dev(np.repeat(k, B, 0)), v=dev(np.repeat(v, B, 0)), ik=dev(np.repeat(ik, B, 0)),
               wk=dev(np.zeros((L, B, 128), np.float32)), wv=dev(np.ones((L, B, 128), np.float32)),
               pos=dev(np.array([N - 1, N - 8, 19999], np.int64)))
    q0, w0 = (dev(x) for x in G.index_queries(23, 0, B))
    q1, w1 = (dev(x) for x in G.index_queries(23, 1, B))
    qa = [dev(G.attn_queries(23, l, B)) for l in range(L)]
    M = torch.empty((B, K.block_stride(N)), dtype=torch.float32, device="cuda")
    pool = torch.empty((B, 2048), dtype=torch.int32, device="cuda")
    idx = torch.empty((B, 512), dtype=torch.int32, device="cuda")
    idx1 = torch.empty((B, 512), dtype=torch.int32, device="cuda")
    out = torch.empty((L, B, 16, 128), dtype=torch.float32, device="cuda")
    ws_sel = K.alloc_workspace(K.OP_SELECT_POOL, B, N)
    ws_ri = K.alloc_workspace(K.OP_INDEX_REINDEX, B)
    ws_at = K.alloc_workspace(K.OP_DECODE_ATTN, B)
    kvg = torch.zeros((B, 512, K.RECORD), dtype=torch.uint8, device="cuda")

    def step():
        K.quantize_kv(gc, new["k"], new["v"], seq, new["pos"], idx_k=new["ik"], win_k=new["wk"],
                      win_v=new["wv"])
        K.index_block_scores(gc, q0, w0, seq, ctx, N, M)
        K.index_select_pool(M, ctx, N, pool, ws_sel)
        K.index_reindex(gc, q0, w0, seq, ctx, pool, idx, ws_ri)
        K.decode_attn(gc, 0, qa[0], idx, seq, ctx, out[0], ws_at)
        K.index_reindex(gc, q1, w1, seq, ctx, pool, idx1, ws_ri)
        K.decode_attn(gc, 1, qa[1], idx1, seq, ctx, out[1], ws_at, kvg_out=kvg)
        K.decode_attn(gc, 2, qa[2], idx1, seq, ctx, out[2], ws_at, kvg_in=kvg)

    step()
    torch.cuda.synchronize()
    want = [t.clone() for t in (pool, idx, idx1, out, gc.kv, gc.wk, kvg)]
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=torch.cuda.Stream()):
        step()
    for rep in range(4):
        for t in (pool, idx, idx1, out, kvg):
            t.fill_(-7 if t.dtype != torch.uint8 else 7)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = (pool, idx, idx1, out, gc.kv, gc.wk, kvg)
        for a, b in zip(got, want):
            assert torch.equal(a, b), f"replay {rep} differs"
        if rep == 0:
            _check_oracle(oc, new, seq, ctx, (q0, w0), (q1, w1), qa, pool, idx, idx1, out)
        step()                                  # eager work between replays
        torch.cuda.synchronize()


def _check_oracle(oc, new, seq, ctx, iq0, iq1, qa, pool, idx, idx1, out):
    """The replayed step against the oracle: the oracle applies the same
    quantise-on-write, then its Full indexer and Reindex layer; the GPU's index
    sets must match under the exemption and each layer's output must lie within
    the attention bound of the oracle's attention over the GPU's index sets."""
    h = lambda t: t.cpu().numpy()
    seq, ctx = h(seq), h(ctx)
    L, B = len(qa), seq.size
    oc.quantize(h(new["k"]), h(new["v"]), h(new["ik"]), h(new["wk"]), h(new["wv"]), seq,
                h(new["pos"]))
    q0, w0 = h(iq0[0]), h(iq0[1])
    q1, w1 = h(iq1[0]), h(iq1[1])
    opool, oidx0, kb, kp0 = oc.index_full(q0, w0, seq, ctx)
    oidx1, kp1 = oc.index_reindex(q1, w1, seq, ctx, opool)
    gpool, gidx0, gidx1 = h(pool), h(idx), h(idx1)
    for b in range(B):
        sc0 = oc.scores(int(seq[b]), q0[b], w0[b], int(ctx[b]))
        sc1 = oc.scores(int(seq[b]), q1[b], w1[b], int(ctx[b]))
        Mb = block_scores(sc0, int(ctx[b]))
        check_index_set(gpool[b], opool[b], lambda j: Mb[j], kb[b])
        check_index_set(gidx0[b], oidx0[b], lambda t: sc0[t], kp0[b])
        check_index_set(gidx1[b], oidx1[b], lambda t: sc1[t], kp1[b])
    gout = h(out)
    for l, gi in ((0, gidx0), (1, gidx1), (2, gidx1)):
        want = oc.decode_attn(l, h(qa[l]), gi, seq, ctx)
        err = float(np.max(np.abs(gout[l] - want)))
        assert err <= ATTN_TOL, f"layer {l}: max-abs {err}"
