"""GPU parity of the fused Reindex layer (csa2_reindex_layer_fused: pool scores,
top-k, attention tiles and merge in one cooperative launch, separated by grid
barriers).

Bars: the index set against the oracle's Reindex selection under the 1e-5
exemption; the output within 2e-3 (observed <= 1e-4) of the oracle's attention
over the kernel's own index set; idx, out and the gathered records bit for bit
equal to the separate calls (csa2_index_reindex, then csa2_decode_attn_ex with
kvg_out) on the same pool; barrier words left at zero; a forced give-up
reported through the status word, with every kernel still ending normally.
"""
import sys

import numpy as np
import pytest

import oracle as O
from fp4_kv_cache_decode_amd import datagen as G
from parity import ATTN_TOL, check_index_set, fill_both, shuffled_pages

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


class Layer:
    """One Reindex layer's inputs, built from seeded rows on both sides."""

    def __init__(self, K, seed, B, N, ctx, n_blocks, topk, layer=1, page_tokens=0):
        self.B, self.n_blocks, self.topk, self.layer = B, n_blocks, topk, layer
        n_layers = layer + 1
        cap = N if not page_tokens else (-(-N // page_tokens) + 1) * page_tokens
        self.oc = O.Cache(B, cap, n_layers)
        if page_tokens:
            table, n_pages = shuffled_pages(seed, B, cap, page_tokens, [N] * B)
            self.gc = K.Cache(B, cap, n_layers, page_tokens=page_tokens, n_pages=n_pages,
                              page_table=torch.from_numpy(table))
        else:
            self.gc = K.Cache(B, cap, n_layers)
        fill_both(seed, B, N, n_layers, self.oc, self.gc)
        torch.cuda.synchronize()
        self.seq = np.arange(B, dtype=np.int32)[::-1].copy()
        self.ctx = np.asarray(ctx, np.int64)
        q0, w0 = G.index_queries(seed, 0, B)
        self.qi, self.wi = G.index_queries(seed, 1, B)
        self.q = G.attn_queries(seed, layer, B)
        # the group's pool from the oracle's Full layer
        self.pool, _, _, _ = self.oc.index_full(q0, w0, self.seq, self.ctx, n_blocks=n_blocks,
                                                topk=min(topk, n_blocks * 8))
        self.d = dict(qi=dev(self.qi), wi=dev(self.wi), q=dev(self.q), seq=dev(self.seq),
                      ctx=dev(self.ctx), pool=dev(self.pool))

    def outputs(self):
        idx = torch.full((self.B, self.topk), -7, dtype=torch.int32, device="cuda")
        out = torch.full((self.B, 16, 128), 7.0, dtype=torch.float32, device="cuda")
        kvg = torch.zeros((self.B, self.topk, 144), dtype=torch.uint8, device="cuda")
        return idx, out, kvg

    def separate(self, K):
        d = self.d
        idx, out, kvg = self.outputs()
        ws = K.alloc_workspace(K.OP_INDEX_REINDEX, self.B, 0, self.n_blocks, self.topk)
        K.index_reindex(self.gc, d["qi"], d["wi"], d["seq"], d["ctx"], d["pool"], idx, ws,
                        topk=self.topk)
        wa = K.alloc_workspace(K.OP_DECODE_ATTN, self.B, 0, 0, self.topk)
        K.decode_attn(self.gc, self.layer, d["q"], idx, d["seq"], d["ctx"], out, wa,
                      kvg_out=kvg)
        torch.cuda.synchronize()
        return idx, out, kvg

    def workspace(self, K):
        n = K.workspace_bytes(K.OP_REINDEX_LAYER_FUSED, self.B, 0, self.n_blocks, 8, self.topk)
        return torch.zeros(n, dtype=torch.uint8, device="cuda")

    def fused(self, K, ws, status, max_polls=0):
        d = self.d
        idx, out, kvg = self.outputs()
        K.reindex_layer_fused(self.gc, self.layer, d["qi"], d["wi"], d["q"], d["seq"],
                              d["ctx"], d["pool"], idx, out, ws, status, kvg_out=kvg,
                              max_polls=max_polls)
        torch.cuda.synchronize()
        return idx, out, kvg


def _barrier_words(ws):
    """(the arrival count, the generation word): one uint32 at the start of
    each 128-byte line of the workspace's first 256 bytes."""
    w = ws[:256].view(torch.int32).cpu().numpy()[::32]
    return w[:1], int(w[1])


def _check_oracle(L, idx, out, kvg):
    """Index set against the oracle's Reindex selection, output against the
    oracle's attention over the kernel's own index set, gathered records
    against the cache's bytes."""
    oidx, kp = L.oc.index_reindex(L.qi, L.wi, L.seq, L.ctx, L.pool, topk=L.topk)
    gidx = idx.cpu().numpy()
    n_diff = 0
    for b in range(L.B):
        N = int(L.ctx[b])
        if N == 0:
            assert np.all(gidx[b] == -1)
            continue
        sc = L.oc.scores(int(L.seq[b]), L.qi[b], L.wi[b], N)
        n_diff += check_index_set(gidx[b], oidx[b], lambda t: sc[t], kp[b])
    want = L.oc.decode_attn(L.layer, L.q, gidx, L.seq, L.ctx)
    err = float(np.max(np.abs(out.cpu().numpy() - want)))
    assert err <= ATTN_TOL, err
    gh = kvg.cpu().numpy()
    valid = (gidx >= 0) & (gidx < L.ctx[:, None])
    bb, jj = np.nonzero(valid)
    assert np.array_equal(gh[bb, jj], L.oc.kv[L.seq[bb], gidx[bb, jj]])
    assert not gh[~valid].any()
    return n_diff, err


CASES = {
    # name: (seed, B, N, ctx, n_blocks, topk, page_tokens)
    "b4_pool2048": (11, 4, 60000, [60000, 59999, 20000, 16384], 2048, 512, 0),
    "b4_paged256": (12, 4, 40000, [40000, 39000, 17000, 30001], 2048, 512, 256),
    "b3_small_pool": (13, 3, 3000, [3000, 2999, 700], 64, 100, 0),
    "b2_topk2048": (14, 2, 40000, [40000, 39999], 2048, 2048, 0),
    "b2_pool4096": (15, 2, 50000, [50000, 45000], 4096, 512, 0),
    "b4_empty_and_one": (16, 4, 5000, [0, 1, 5000, 9], 64, 32, 0),
    "b16_pool2048": (17, 16, 20000, [20000 - 37 * i for i in range(16)], 2048, 512, 0),
}


@pytest.mark.parametrize("name", list(CASES))
def test_fused_layer_matches_oracle_and_separate_calls(K, name):
    seed, B, N, ctx, nb, topk, pt = CASES[name]
    _say(f"fused reindex layer {name}: B={B} N={N} n_blocks={nb} topk={topk} paged={pt}")
    L = Layer(K, seed, B, N, ctx, nb, topk, page_tokens=pt)
    ws = L.workspace(K)
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    got = L.fused(K, ws, status)
    assert int(status.item()) == 0
    sep = L.separate(K)
    for g, s, what in zip(got, sep, ("idx", "out", "kvg")):
        assert torch.equal(g, s), what
    n_diff, err = _check_oracle(L, *got)
    _say(f"  exempt index differences {n_diff}, attention max-abs {err:.3g}")
    # the barrier counts are back at 0, the generation advanced by 3
    counts, gen = _barrier_words(ws)
    assert not counts.any() and gen == 3, (counts, gen)


def _sweep_case(seed):
    """A seeded random shape inside the fused entry point's envelope: B x tiles
    <= 768 and one round of 1,024-thread workgroups within 256 CUs."""
    rng = np.random.default_rng(1000 + seed)
    while True:
        B = int(rng.integers(1, 13))
        nb = int(rng.choice([1, 7, 64, 300, 2048, 4096]))
        topk = int(rng.integers(1, min(2048, nb * 8) + 1))
        runs = -(-nb * 8 // 256)
        tiles = -(-topk // 64) + 2
        if B * tiles <= 768 and -(-B * runs // 4) <= 256 and -(-B * tiles // 4) <= 256:
            break
    N = int(rng.integers(max(1, nb), 30001))
    ctx = [int(rng.integers(0, N + 1)) for _ in range(B)]
    ctx[0] = N
    pt = int(rng.choice([0, 64, 1024]))
    return B, N, ctx, nb, topk, pt


@pytest.mark.parametrize("seed", range(6))
def test_fused_layer_random_sweep(K, seed):
    """Seeded random batches, pool sizes, top-k sizes, contexts (empty ones
    included) and page sizes: bit for bit against the separate calls, and the
    oracle's bars."""
    B, N, ctx, nb, topk, pt = _sweep_case(seed)
    _say(f"fused reindex layer sweep {seed}: B={B} N={N} n_blocks={nb} topk={topk} "
         f"paged={pt} ctx={ctx}")
    L = Layer(K, 300 + seed, B, N, ctx, nb, topk, page_tokens=pt)
    ws = L.workspace(K)
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    got = L.fused(K, ws, status)
    assert int(status.item()) == 0
    for g, s_, what in zip(got, L.separate(K), ("idx", "out", "kvg")):
        assert torch.equal(g, s_), what
    n_diff, err = _check_oracle(L, *got)
    _say(f"  exempt index differences {n_diff}, attention max-abs {err:.3g}")


def test_fused_layer_repeated_calls(K):
    """One zero-filled workspace serves calls in a row: identical results,
    count back at 0 after each, generation +3 per call."""
    _say("fused reindex layer repeated calls")
    L = Layer(K, 21, 4, 30000, [30000, 29000, 17000, 25000], 2048, 512)
    ws = L.workspace(K)
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    first = L.fused(K, ws, status)
    for call in range(2, 5):
        again = L.fused(K, ws, status)
        for g, s in zip(again, first):
            assert torch.equal(g, s)
        counts, gen = _barrier_words(ws)
        assert not counts.any() and gen == 3 * call, (counts, gen)
    assert int(status.item()) == 0


def test_fused_layer_reports_give_up(K):
    """Barrier words that are not zero (the count never reaches the grid size,
    so no barrier completes) make every workgroup give up after max_polls
    polls at each barrier: the
    launch still completes and the status word reports it.  After a zero fill
    the same workspace gives the separate calls' results again."""
    _say("fused reindex layer give-up path")
    L = Layer(K, 22, 4, 20000, [20000, 19000, 17000, 18000], 2048, 512)
    ws = L.workspace(K)
    ws[:4].view(torch.int32).fill_(1 << 30)
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    L.fused(K, ws, status, max_polls=8)
    assert int(status.item()) == 1
    ws.zero_()
    status.zero_()
    got = L.fused(K, ws, status)
    assert int(status.item()) == 0
    for g, s in zip(got, L.separate(K)):
        assert torch.equal(g, s)


def test_fused_layer_refuses_what_does_not_fit(K):
    """Batches whose single-round grid cannot be resident are refused on the
    host (CSA2_ERR_UNSUPPORTED), before any launch."""
    _say("fused reindex layer size limits")
    L = Layer(K, 23, 2, 3000, [3000, 2000], 64, 32)
    B = 17                       # 17 x 64 scoring runs / 4 per workgroup > 256 CUs
    d = lambda a: dev(np.repeat(a[:1], B, axis=0))
    idx = torch.empty((B, 512), dtype=torch.int32, device="cuda")
    out = torch.empty((B, 16, 128), dtype=torch.float32, device="cuda")
    pool = torch.zeros((B, 2048), dtype=torch.int32, device="cuda")
    ws = torch.zeros(K.workspace_bytes(K.OP_REINDEX_LAYER_FUSED, B, 0, 2048, 8, 512),
                     dtype=torch.uint8, device="cuda")
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    with pytest.raises(K.Csa2Error) as e:
        K.reindex_layer_fused(L.gc, 1, d(L.qi), d(L.wi), d(L.q), d(L.seq), d(L.ctx), pool, idx,
                              out, ws, status)
    assert e.value.status == K.ERR_UNSUPPORTED


def test_fused_layer_in_hip_graph(K):
    """The cooperative launch captured in a HIP graph: four replays, with eager
    work and synchronisations between them, each bit-identical to the eager
    call; the barrier count is back at zero and the generation advanced by 3
    per launch."""
    _say("fused reindex layer in a HIP graph")
    L = Layer(K, 24, 4, 20000, [20000, 19000, 17000, 18000], 2048, 512)
    ws = L.workspace(K)
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    want = L.fused(K, ws, status)
    d = L.d
    idx, out, kvg = L.outputs()
    stream = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        K.reindex_layer_fused(L.gc, L.layer, d["qi"], d["wi"], d["q"], d["seq"], d["ctx"],
                              d["pool"], idx, out, ws, status, kvg_out=kvg)
    torch.cuda.synchronize()
    for rep in range(4):
        idx.fill_(-7)
        out.fill_(7.0)
        kvg.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for a, b, what in zip((idx, out, kvg), want, ("idx", "out", "kvg")):
            assert torch.equal(a, b), (rep, what)
        L.separate(K)                   # eager work between replays
    counts, gen = _barrier_words(ws)
    assert not counts.any() and gen == 3 * 5, (counts, gen)
    assert int(status.item()) == 0
