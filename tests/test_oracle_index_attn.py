"""Pins for the oracle's indexer, top-k, hierarchy and attention (CPU only).

Independent references used here:
  * numpy fp64 matrix products over keys decoded with torch's float8_e4m3fn;
  * Python's sorted() as a brute-force top-k with ties to the lower index;
  * dense softmax attention in numpy over the whole cache, decoded with the
    E2M1 value table and torch's E4M3 table (sparse attention with k >= N must
    equal it);
  * closed forms: integer-valued scores (exact), q = 0 gives the mean of V, a
    single entry gives that entry's V.
"""
import numpy as np
import pytest
import torch

import oracle as O
from fp4_kv_cache_decode_amd import datagen as G

E2M1 = np.array([0, .5, 1, 1.5, 2, 3, 4, 6, -0., -.5, -1, -1.5, -2, -3, -4, -6])
E4M3 = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()


def _fill_cache(n_seq, N, seed, n_layers=1, w_cap=128, cap=None):
    cap = cap or N
    c = O.Cache(n_seq, cap, n_layers=n_layers, w_cap=w_cap)
    for s in range(n_seq):
        k, v, ik = G.kv_rows(seed, s, 0, N)
        wk = np.zeros((n_layers, N, 128), np.float32)
        wv = np.zeros_like(wk)
        for l in range(n_layers):
            wk[l], wv[l] = G.window_rows(seed, l, s, 0, N)
        c.quantize(k, v, ik, wk, wv, np.full(N, s, np.int32), np.arange(N, dtype=np.int64))
    return c


def _brute_topk(vals, k, ids=None):
    ids = np.arange(len(vals)) if ids is None else np.asarray(ids)
    order = sorted(range(len(vals)), key=lambda i: (-vals[i], ids[i]))[:k]
    sel = sorted(int(ids[i]) for i in order)
    return np.array(sel + [-1] * (k - len(sel)), np.int32)


def _np_scores(idxk_rows, q, w, scale=1.0):
    kh = E4M3[idxk_rows] * scale                      # [N, 64]
    d = kh @ q.astype(np.float64).T                    # [N, 4]
    return np.maximum(d, 0) @ w.astype(np.float64)


# ----------------------------------------------------------------- scores

def test_scores_match_numpy_reference():
    c = _fill_cache(1, 3000, seed=11)
    q, w = G.index_queries(11, 0, 1)
    got = c.scores(0, q[0], w[0], 3000)
    want = _np_scores(c.idxk[0, :3000], q[0], w[0])
    np.testing.assert_allclose(got, want, rtol=1e-12, atol=1e-12)
    assert np.all(got >= 0)


def test_scores_integer_valued_are_exact():
    rng = np.random.default_rng(5)
    c = O.Cache(1, 500)
    ints = rng.integers(-8, 9, size=(500, 64)).astype(np.float32)   # exact in E4M3
    c.quantize(np.zeros((500, 128), np.float32), np.zeros((500, 128), np.float32), ints,
               None, None, np.zeros(500, np.int32), np.arange(500, dtype=np.int64))
    q = rng.integers(-3, 4, size=(4, 64)).astype(np.float32)
    w = np.array([1, 2, 0.5, 0.25], np.float32)
    got = c.scores(0, q, w, 500)
    d = ints.astype(np.int64) @ q.astype(np.int64).T
    want = np.maximum(d, 0) @ np.array([1, 2, 0.5, 0.25])
    assert np.array_equal(got, want)


def test_scores_one_hot_weight_is_relu_of_one_head():
    c = _fill_cache(1, 700, seed=2)
    q, _ = G.index_queries(2, 0, 1)
    for h in range(4):
        w = np.zeros(4, np.float32)
        w[h] = 1
        got = c.scores(0, q[0], w, 700)
        dot = E4M3[c.idxk[0, :700]] @ q[0, h].astype(np.float64)
        np.testing.assert_allclose(got, np.maximum(dot, 0), rtol=1e-12, atol=1e-13)


# ----------------------------------------------------------------- top-k

@pytest.mark.parametrize("n,k,distinct", [(1, 1, 1), (5, 8, 3), (100, 10, 1), (4096, 512, 7),
                                          (4096, 512, 4096), (3000, 2048, 50), (0, 4, 1)])
def test_topk_matches_sorted(n, k, distinct):
    rng = np.random.default_rng(n + k)
    vals = rng.integers(0, distinct, n).astype(np.float64) if n else np.zeros(0)
    got, m, kth = O.topk(vals, k)
    want = _brute_topk(list(vals), k)
    assert np.array_equal(got, want)
    assert m == min(n, k)


def test_topk_with_ids_and_negative_zero():
    vals = np.array([0.0, -0.0, 1.0, -1.0, 0.0])
    ids = np.array([40, 10, 30, 20, 5], np.int64)
    got, m, kth = O.topk(vals, 3, ids)
    # 1.0 (id 30) first; then the zeros tie (+0 == -0) and go to the lower ids 5, 10
    assert list(got) == [5, 10, 30] and kth == 0.0


# ----------------------------------------------------------------- hierarchy

def _tie_heavy_cache(N, seed):
    """Indexer keys whose scores take few distinct values (many exact ties)."""
    rng = np.random.default_rng(seed)
    c = O.Cache(1, N)
    ik = np.zeros((N, 64), np.float32)
    ik[:, 0] = rng.integers(0, 4, N)
    c.quantize(np.zeros((N, 128), np.float32), np.zeros((N, 128), np.float32), ik, None, None,
               np.zeros(N, np.int32), np.arange(N, dtype=np.int64))
    q = np.zeros((1, 4, 64), np.float32)
    q[0, :, 0] = 1
    return c, q, np.ones((1, 4), np.float32)


@pytest.mark.parametrize("seed", range(40))
def test_hierarchical_equals_flat_topk(seed):
    """Pool of the best blocks by max, then top-k inside the pool == flat top-k."""
    rng = np.random.default_rng(seed)
    N = int(rng.integers(30, 400))
    block, n_blocks, topk = int(rng.integers(2, 9)), int(rng.integers(4, 20)), None
    topk = int(rng.integers(1, n_blocks + 1))          # topk <= n_blocks keeps the identity
    if seed % 2:
        c, q, w = _tie_heavy_cache(N, seed)
    else:
        c = _fill_cache(1, N, seed)
        q, w = G.index_queries(seed, 0, 1)
    pool, idx, kb, kp = c.index_full(q, w, [0], [N], n_blocks=n_blocks, block=block, topk=topk)
    sc = c.scores(0, q[0], w[0], N)
    assert np.array_equal(idx[0], _brute_topk(list(sc), topk))
    # pool = the n_blocks best block maxima, ties to the lower block
    nb = -(-N // block)
    M = [max(sc[j * block:min(N, (j + 1) * block)]) for j in range(nb)]
    assert np.array_equal(pool[0], _brute_topk(M, n_blocks))
    sel = idx[0][idx[0] >= 0]
    assert set(sel // block) <= set(pool[0][pool[0] >= 0])


@pytest.mark.parametrize("seed", range(6))
def test_as_many_blocks_as_positions_still_hold_the_flat_topk(seed):
    """The boundary n_blocks == topk: every top-k position lies in the top-k
    blocks (ties included), so a Full layer that keeps only that many blocks
    (no Reindex pool to serve) selects the flat top-k."""
    N, topk = 3000 + 37 * seed, 64
    c, q, w = _tie_heavy_cache(N, seed) if seed % 2 else (
        _fill_cache(1, N, seed), *G.index_queries(seed, 0, 1))
    _, idx, _, _ = c.index_full(q, w, [0], [N], n_blocks=topk, topk=topk)
    sc = c.scores(0, q[0], w[0], N)
    assert np.array_equal(idx[0], _brute_topk(list(sc), topk))


def test_small_context_pool_is_every_block():
    c = _fill_cache(1, 1000, seed=4)
    q, w = G.index_queries(4, 0, 1)
    pool, idx, _, _ = c.index_full(q, w, [0], [1000])
    assert list(pool[0][:125]) == list(range(125)) and np.all(pool[0][125:] == -1)
    assert np.all(idx[0] >= 0) and np.all(np.diff(idx[0]) > 0)


def test_small_context_pads_indices():
    c = _fill_cache(1, 300, seed=4)
    q, w = G.index_queries(4, 0, 1)
    pool, idx, _, _ = c.index_full(q, w, [0], [300])
    assert list(idx[0][:300]) == list(range(300)) and np.all(idx[0][300:] == -1)


def test_reindex_with_full_query_reproduces_full():
    N = 40000
    c = _fill_cache(1, N, seed=9)
    q, w = G.index_queries(9, 0, 1)
    pool, idx, _, _ = c.index_full(q, w, [0], [N])
    assert np.count_nonzero(pool[0] >= 0) == 2048
    ridx, _ = c.index_reindex(q, w, [0], [N], pool)
    assert np.array_equal(ridx, idx)
    q2, w2 = G.index_queries(9, 1, 1)
    ridx2, _ = c.index_reindex(q2, w2, [0], [N], pool)
    assert set(ridx2[0] // 8) <= set(pool[0])
    sc2 = c.scores(0, q2[0], w2[0], N)
    pos = np.concatenate([np.arange(8 * b, 8 * b + 8) for b in pool[0]])
    assert np.array_equal(ridx2[0], _brute_topk(list(sc2[pos]), 512, pos))


# ----------------------------------------------------------------- attention

def _dequant_cache(c, s):
    """Dequantised K, V [cap,128] of one sequence via the value tables."""
    rec = c.kv[s].astype(np.int64)
    def fp4(codes, scales):
        lo, hi = codes & 15, codes >> 4
        nib = np.stack([lo, hi], -1).reshape(codes.shape[0], 128)
        return E2M1[nib] * np.repeat(E4M3[scales], 16, axis=1)
    return fp4(rec[:, 0:64], rec[:, 128:136]), fp4(rec[:, 64:128], rec[:, 136:144])


def _dense_attn(c, layer, q, s, N, sm):
    K, V = _dequant_cache(c, s)
    u = np.arange(max(0, N - 128), N)
    Kw = E4M3[c.wk[layer, s, u % c.w_cap]] * c.wk_scale
    Vw = E4M3[c.wv[layer, s, u % c.w_cap]] * c.wv_scale
    KK = np.concatenate([K[:N], Kw])
    VV = np.concatenate([V[:N], Vw])
    z = q.astype(np.float64) @ KK.T * sm
    p = np.exp(z - z.max(1, keepdims=True))
    return (p / p.sum(1, keepdims=True)) @ VV


@pytest.mark.parametrize("N", [1, 37, 128, 300, 512])
def test_sparse_with_all_positions_equals_dense(N):
    c = _fill_cache(2, N, seed=N, n_layers=2, w_cap=160)
    q = G.attn_queries(N, 1, 2)
    idx = np.full((2, 512), -1, np.int32)
    idx[:, :N] = np.arange(N)
    sm = float(np.float32(1 / np.sqrt(128)))
    out = c.decode_attn(1, q, idx, [0, 1], [N, N], sm)
    for s in range(2):
        want = _dense_attn(c, 1, q[s], s, N, sm)
        np.testing.assert_allclose(out[s], want, rtol=2e-6, atol=2e-6)


def test_zero_query_gives_mean_of_values():
    N = 200
    c = _fill_cache(1, N, seed=3)
    idx = np.sort(np.random.default_rng(0).choice(N, 64, replace=False)).astype(np.int32)[None]
    out = c.decode_attn(0, np.zeros((1, 16, 128), np.float32), idx, [0], [N])
    K, V = _dequant_cache(c, 0)
    u = np.arange(N - 128, N)
    Vw = E4M3[c.wv[0, 0, u % 128]]
    want = np.concatenate([V[idx[0]], Vw]).mean(0)
    for h in range(16):
        np.testing.assert_allclose(out[0, h], want, rtol=1e-6, atol=1e-6)


def test_single_entry_gives_its_value():
    c = _fill_cache(1, 1, seed=8)
    q = G.attn_queries(8, 0, 1) * 10
    out = c.decode_attn(0, q, np.full((1, 512), -1, np.int32), [0], [1])
    want = E4M3[c.wv[0, 0, 0]].astype(np.float32)
    for h in range(16):
        assert np.array_equal(out[0, h], want)


@pytest.mark.parametrize("idx_len", [1, 512])
def test_no_main_entries_is_window_attention(idx_len):
    """A window-only layer (every index -1): softmax attention over the 128
    window rows of positions [N - 128, N) alone, dense numpy in fp64."""
    N = 1000
    c = _fill_cache(1, N, seed=21, n_layers=2, w_cap=160)
    q = G.attn_queries(21, 1, 1)
    sm = float(np.float32(1 / np.sqrt(128)))
    out = c.decode_attn(1, q, np.full((1, idx_len), -1, np.int32), [0], [N], sm)
    u = np.arange(N - 128, N)
    Kw = E4M3[c.wk[1, 0, u % c.w_cap]] * c.wk_scale
    Vw = E4M3[c.wv[1, 0, u % c.w_cap]] * c.wv_scale
    z = q[0].astype(np.float64) @ Kw.T * sm
    p = np.exp(z - z.max(1, keepdims=True))
    np.testing.assert_allclose(out[0], (p / p.sum(1, keepdims=True)) @ Vw, rtol=2e-6, atol=2e-6)


def test_reuse_layers_share_indices():
    """Reuse: same index list, different queries -> outputs differ only through q."""
    N = 2000
    c = _fill_cache(1, N, seed=12, n_layers=2)
    qi, wi = G.index_queries(12, 0, 1)
    _, idx, _, _ = c.index_full(qi, wi, [0], [N])
    q0, q1 = G.attn_queries(12, 0, 1), G.attn_queries(12, 1, 1)
    a = c.decode_attn(0, q0, idx, [0], [N])
    b = c.decode_attn(0, q0, idx.copy(), [0], [N])
    assert np.array_equal(a, b)
    assert not np.allclose(a, c.decode_attn(0, q1, idx, [0], [N]))
