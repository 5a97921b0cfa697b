"""Sequences whose records span more than 4 GiB.

Below that size both attention kernels read a sequence's records with 32-bit
offsets from the sequence's base; above it they use 64-bit offsets.  The same
rows quantised at the top of a 30,000,128-token sequence (positions past
2^32 / 144) and at the bottom of a 4,096-token one must give bit-identical
results: the attention output through the tile kernel (few queries) and the
stream kernel (many), the gathered-record buffer, and the output over those
gathered records; and the fused Reindex layer's index set (up to the shift),
output and gathered records.  The two contexts differ by a multiple of the
128-slot window, so the window rows land in the same slots.
"""
import numpy as np
import pytest

from fp4_kv_cache_decode_amd import datagen as G

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")

BIG, SMALL = 30_000_128, 4096
OFFSET = BIG - SMALL


@pytest.fixture(scope="module")
def caches():
    """The same rows at positions OFFSET.. of a BIG-token sequence and 0.. of a
    SMALL-token one, window rows of both layers included."""
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from fp4_kv_cache_decode_amd import csa2 as K
    assert BIG * K.RECORD > 2 ** 32 and OFFSET % G.WINDOW == 0
    L = 2
    big, small = K.Cache(1, BIG, L), K.Cache(1, SMALL, L)
    k, v, ik = G.kv_rows(41, 0, 0, SMALL)
    w0 = SMALL - G.WINDOW
    wk = np.stack([G.window_rows(41, l, 0, w0, SMALL)[0] for l in range(L)])
    wv = np.stack([G.window_rows(41, l, 0, w0, SMALL)[1] for l in range(L)])
    for cache, base in ((small, 0), (big, OFFSET)):
        K.quantize_kv(cache, dev(k[:w0]), dev(v[:w0]), dev(np.zeros(w0, np.int32)),
                      dev(np.arange(base, base + w0, dtype=np.int64)), idx_k=dev(ik[:w0]))
        K.quantize_kv(cache, dev(k[w0:]), dev(v[w0:]), dev(np.zeros(G.WINDOW, np.int32)),
                      dev(np.arange(base + w0, base + SMALL, dtype=np.int64)),
                      idx_k=dev(ik[w0:]), win_k=dev(wk), win_v=dev(wv))
    torch.cuda.synchronize()
    # the records themselves landed at both places
    assert torch.equal(big.kv[0, OFFSET:], small.kv[0])
    return K, big, small


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


@pytest.mark.parametrize("B", [8, 96])
def test_records_past_4gib_match_low_positions(caches, B):
    K, big, small = caches
    rng = np.random.default_rng(41)
    idx = np.sort(rng.integers(0, SMALL, (B, G.TOPK)), axis=1).astype(np.int32)
    idx[::3, -29:] = -1                                   # ragged lists
    seq = dev(np.zeros(B, np.int32))
    ws = K.alloc_workspace(K.OP_DECODE_ATTN, B)
    q = dev(G.attn_queries(41, 0, B))
    res = {}
    for name, cache, base, n in (("small", small, 0, SMALL), ("big", big, OFFSET, BIG)):
        ib = dev(np.where(idx >= 0, idx + base, -1).astype(np.int32))
        ctx = dev(np.full(B, n, np.int64))
        out = torch.empty((B, G.H, G.D), dtype=torch.float32, device="cuda")
        out_r = torch.empty_like(out)
        kvg = torch.zeros((B, G.TOPK, K.RECORD), dtype=torch.uint8, device="cuda")
        K.decode_attn(cache, 0, q, ib, seq, ctx, out, ws, kvg_out=kvg)
        K.decode_attn(cache, 1, q, ib, seq, ctx, out_r, ws, kvg_in=kvg)
        torch.cuda.synchronize()
        res[name] = (out, out_r, kvg)
    for a, b in zip(res["small"], res["big"]):
        assert torch.equal(a, b)
    assert torch.isfinite(res["big"][0]).all()


def test_fused_layer_past_4gib_matches_low_positions(caches):
    """The fused Reindex layer on the same two caches: a pool over the written
    blocks, the same queries; index sets equal up to the shift, outputs and
    gathered records bit-identical (the fused kernel's 64-bit-offset form
    against its 32-bit one)."""
    K, big, small = caches
    B, n_blocks = 4, SMALL // G.BLOCK
    qi, wi = G.index_queries(41, 1, B)
    q = dev(G.attn_queries(41, 1, B))
    seq = dev(np.zeros(B, np.int32))
    res = {}
    for name, cache, base, n in (("small", small, 0, SMALL), ("big", big, OFFSET, BIG)):
        pool = dev(np.tile(np.arange(n_blocks, dtype=np.int32) + base // G.BLOCK, (B, 1)))
        ctx = dev(np.full(B, n, np.int64))
        idx = torch.empty((B, G.TOPK), dtype=torch.int32, device="cuda")
        out = torch.empty((B, G.H, G.D), dtype=torch.float32, device="cuda")
        kvg = torch.zeros((B, G.TOPK, K.RECORD), dtype=torch.uint8, device="cuda")
        ws = torch.zeros(K.workspace_bytes(K.OP_REINDEX_LAYER_FUSED, B, 0, n_blocks, G.BLOCK,
                                           G.TOPK), dtype=torch.uint8, device="cuda")
        status = torch.zeros(1, dtype=torch.int32, device="cuda")
        K.reindex_layer_fused(cache, 1, dev(qi), dev(wi), q, seq, ctx, pool, idx, out, ws,
                              status, kvg_out=kvg)
        torch.cuda.synchronize()
        assert int(status.item()) == 0
        res[name] = (idx - base * (idx >= 0), out, kvg)
    for a, b in zip(res["small"], res["big"]):
        assert torch.equal(a, b)
    assert (res["small"][0] >= 0).all()
