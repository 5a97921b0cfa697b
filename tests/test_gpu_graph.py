"""HIP-graph capture of a decode step: replays match eager launches exactly.

The step (quantise-on-write, Full indexer, Reindex, attention) is captured once
and replayed several times with eager work and synchronisations in between;
every replay must reproduce the eager results bit for bit.
"""
import numpy as np
import pytest

from fp4_kv_cache_decode_amd import datagen as G
from parity import fill_both

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")


def test_graph_replay_matches_eager():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from fp4_kv_cache_decode_amd import csa2 as K
    B, N, L = 3, 40000, 3
    gc = K.Cache(B, N, L)
    fill_both(23, B, N, L, None, gc)
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
    out = torch.empty((L, B, 16, 128), dtype=torch.float32, device="cuda")
    ws_sel = K.alloc_workspace(K.OP_SELECT_POOL, B, N)
    ws_ri = K.alloc_workspace(K.OP_INDEX_REINDEX, B)
    ws_at = K.alloc_workspace(K.OP_DECODE_ATTN, B)

    def step():
        K.quantize_kv(gc, new["k"], new["v"], seq, new["pos"], idx_k=new["ik"], win_k=new["wk"],
                      win_v=new["wv"])
        K.index_block_scores(gc, q0, w0, seq, ctx, N, M)
        K.index_select_pool(M, ctx, N, pool, ws_sel)
        K.index_reindex(gc, q0, w0, seq, ctx, pool, idx, ws_ri)
        K.decode_attn(gc, 0, qa[0], idx, seq, ctx, out[0], ws_at)
        K.index_reindex(gc, q1, w1, seq, ctx, pool, idx, ws_ri)
        for l in (1, 2):
            K.decode_attn(gc, l, qa[l], idx, seq, ctx, out[l], ws_at)

    step()
    torch.cuda.synchronize()
    want = [t.clone() for t in (pool, idx, out, gc.kv[:, N - 8:], gc.wk)]
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=torch.cuda.Stream()):
        step()
    for rep in range(4):
        for t in (pool, idx, out):
            t.fill_(-7)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = (pool, idx, out, gc.kv[:, N - 8:], gc.wk)
        for a, b in zip(got, want):
            assert torch.equal(a, b), f"replay {rep} differs"
        step()                                  # eager work between replays
        torch.cuda.synchronize()
