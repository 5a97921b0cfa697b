"""Seeded randomized sweeps on the GPU.

* Top-k selection against a brute-force stable sort: random row lengths from 1
  to 140,000 (every select path: a 256-thread workgroup for rows of up to 4,096,
  one 1,024-thread workgroup at 16 or 32 values per thread, segments + merge,
  and the exact fallback), k from 1 to 4,096, and value
  distributions including ReLU-like, skewed, tie-heavy, signed-zero and mostly
  absent rows.
* Block scores of large batches (four queries per key pass) against the same
  queries scored in batches small enough for one query per workgroup row: bit
  for bit, for one-sequence, mixed and half-and-half batches with random
  contexts (zero included).
"""
import numpy as np
import pytest

from fp4_kv_cache_decode_amd import datagen as G
import test_gpu_topk as T

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def K():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from fp4_kv_cache_decode_amd import csa2
    csa2.lib()
    return csa2


def _row(rng, n, kind):
    if kind == "relu":
        return np.maximum(rng.standard_normal(n), 0).astype(np.float32) * rng.uniform(0.1, 50)
    if kind == "skew":
        return (rng.random(n) ** 4 * 30).astype(np.float32)
    if kind == "zeros_then_big":
        r = np.zeros(n, np.float32)
        m = int(rng.integers(1, n + 1))
        r[-m:] = rng.random(m) * 10
        return r
    return T._rows(rng, n, kind)


@pytest.mark.parametrize("seed", [7, 8])
def test_topk_random_sweep(K, seed):
    rng = np.random.default_rng(seed)
    kinds = ["normal", "few", "equal", "signed_zero", "absent", "narrow", "relu", "skew",
             "zeros_then_big"]
    for _ in range(30):
        B = int(rng.integers(1, 5))
        k = int(rng.choice([1, 8, 100, 512, 1000, 2048, 4096]))
        sizes = [int(rng.choice([rng.integers(1, 70), rng.integers(1, 20000),
                                 rng.integers(16000, 33000), rng.integers(33000, 140000)]))
                 for _ in range(B)]
        T.run(K, [_row(rng, n, kinds[int(rng.integers(len(kinds)))]) for n in sizes], k)


@pytest.mark.parametrize("seed", [21, 22])
def test_topk_short_rows_random_sweep(K, seed):
    """Batches whose rows are all at most 4,096 entries (the quarter-size
    workgroup), k from 1 to 4,096, every value distribution."""
    rng = np.random.default_rng(seed)
    kinds = ["normal", "few", "equal", "signed_zero", "absent", "narrow", "relu", "skew",
             "zeros_then_big"]
    for _ in range(30):
        B = int(rng.integers(1, 9))
        k = int(rng.choice([1, 8, 100, 512, 1000, 2048, 4096]))
        sizes = [int(rng.choice([rng.integers(1, 70), rng.integers(1, 4097), 4096]))
                 for _ in range(B)]
        T.run(K, [_row(rng, n, kinds[int(rng.integers(len(kinds)))]) for n in sizes], k)


def test_grouped_block_scores_random_sweep(K):
    rng = np.random.default_rng(11)
    N, n_seq = 4000, 3
    gc = K.Cache(n_seq, N, 1)
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    for s in range(n_seq):
        k, v, ik = G.kv_rows(11, s, 0, N)
        K.quantize_kv(gc, dev(k), dev(v), dev(np.full(N, s, np.int32)),
                      dev(np.arange(N, dtype=np.int64)), idx_k=dev(ik))
    stride = K.block_stride(N)
    for it in range(6):
        B = int(rng.integers(1024, 2600))
        mode = it % 3
        seq = np.zeros(B, np.int32) if mode == 0 else rng.integers(0, n_seq, B).astype(np.int32)
        if mode == 2:
            seq[: B // 2] = 1
        ctx = rng.integers(0, N + 1, B).astype(np.int64)
        q, w = G.index_queries(100 + it, 0, B)
        M = torch.full((B, stride), float("nan"), device="cuda")
        K.index_block_scores(gc, dev(q), dev(w), dev(seq), dev(ctx), N, M)
        Ms = torch.full((B, stride), float("nan"), device="cuda")
        for b0 in range(0, B, 500):
            b1 = min(B, b0 + 500)
            K.index_block_scores(gc, dev(q[b0:b1]), dev(w[b0:b1]), dev(seq[b0:b1]),
                                 dev(ctx[b0:b1]), N, Ms[b0:b1])
        torch.cuda.synchronize()
        assert np.array_equal(M.cpu().numpy(), Ms.cpu().numpy(), equal_nan=True), (it, B, mode)


def test_attention_random_sweep(K):
    """Random attention calls against the oracle: batch sizes on both kernels
    (tile, split stream, unsplit stream), top-k lengths 1..2,048 with padding,
    random contexts and window scales, contiguous and paged caches (shuffled
    64- or 256-token pages)."""
    import oracle as O
    from parity import fill_both, shuffled_pages
    rng = np.random.default_rng(21)
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    for it in range(8):
        n_seq, L = 3, 2
        N = int(rng.integers(200, 3000))
        P = int(rng.choice([0, 64, 256]))
        cap = -(-N // 256) * 256 + 256
        wk_s, wv_s = float(rng.choice([1.0, 0.05])), float(rng.choice([1.0, 40.0, 200.0]))
        oc = O.Cache(n_seq, cap, L, 4096, 1.0, wk_s, wv_s)
        if P:
            table, n_pages = shuffled_pages(it, n_seq, cap, P, [N] * n_seq)
            gc = K.Cache(n_seq, cap, L, 4096, 1.0, wk_s, wv_s, page_tokens=P, n_pages=n_pages,
                         page_table=torch.from_numpy(table))
        else:
            gc = K.Cache(n_seq, cap, L, 4096, 1.0, wk_s, wv_s)
        fill_both(300 + it, n_seq, N, L, oc, gc, wlo=0)
        B = int(rng.choice([1, 3, 40, 96, 300, 1100]))
        topk = int(rng.choice([1, 37, 512, 700, 2048]))
        seq = rng.integers(0, n_seq, B).astype(np.int32)
        ctx = rng.integers(1, N + 1, B).astype(np.int64)
        idx = np.full((B, topk), -1, np.int32)
        for b in range(B):
            m = int(rng.integers(0, min(topk, int(ctx[b])) + 1))
            idx[b, :m] = np.sort(rng.choice(int(ctx[b]), m, replace=False))
        layer = int(rng.integers(0, L))
        q = G.attn_queries(400 + it, layer, B)
        out = torch.empty((B, 16, 128), dtype=torch.float32, device="cuda")
        K.decode_attn(gc, layer, dev(q), dev(idx), dev(seq), dev(ctx), out,
                      K.alloc_workspace(K.OP_DECODE_ATTN, B, topk=topk))
        torch.cuda.synchronize()
        sample = np.unique(np.r_[0, B - 1, rng.integers(0, B, 12)])
        want = oc.decode_attn(layer, q[sample], idx[sample], seq[sample], ctx[sample])
        got = out.cpu().numpy()[sample]
        err = float(np.max(np.abs(got - want)))
        assert err <= 1e-4 * max(1.0, float(np.max(np.abs(want)))), (it, B, topk, P, err)
