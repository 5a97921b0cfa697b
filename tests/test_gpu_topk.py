"""GPU top-k selection against a brute-force sort (exact index sets).

Drives the selection kernel through csa2_index_select_pool with crafted rows:
continuous values, heavy ties (few distinct values, all equal), +0/-0, absent
(-inf) entries, rows that overflow the fast path's candidate list, and rows
longer than its bitmap (the radix fallback).  Ties go to the lower index and
the output is ascending with -1 padding.
"""
import numpy as np
import pytest

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def K():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from fp4_kv_cache_decode_amd import csa2
    csa2.lib()
    return csa2


def brute(row, k):
    v = np.asarray(row, np.float64)
    valid = np.nonzero(v != -np.inf)[0]
    # stable sort by descending value keeps ascending index among equals
    order = valid[np.argsort(-v[valid], kind="stable")][:k]
    sel = np.sort(order)
    return np.concatenate([sel, -np.ones(k - sel.size, np.int64)]).astype(np.int32)


def run(K, rows, k):
    B = len(rows)
    n = max(len(r) for r in rows)
    stride = K.block_stride(8 * n)
    M = np.full((B, stride), np.nan, np.float32)
    ctx = np.zeros(B, np.int64)
    for b, r in enumerate(rows):
        M[b, :len(r)] = r
        ctx[b] = 8 * len(r)
    pool = torch.empty((B, k), dtype=torch.int32, device="cuda")
    ws = K.alloc_workspace(K.OP_SELECT_POOL, B, int(8 * n), n_blocks=k)
    K.index_select_pool(torch.from_numpy(M).cuda(), torch.from_numpy(ctx).cuda(), int(8 * n), pool,
                        ws)
    torch.cuda.synchronize()
    got = pool.cpu().numpy()
    for b, r in enumerate(rows):
        want = brute(np.asarray(r, np.float32), k)
        bad = np.nonzero(got[b] != want)[0]
        assert bad.size == 0, (b, len(r), k, bad[:5], got[b][bad[:5]], want[bad[:5]])


def _rows(rng, n, kind):
    if kind == "normal":
        return rng.standard_normal(n).astype(np.float32) * 30
    if kind == "few":
        return rng.integers(0, 5, n).astype(np.float32)
    if kind == "equal":
        return np.full(n, 2.5, np.float32)
    if kind == "signed_zero":
        r = rng.choice([0.0, -0.0, 1.0, -1.0], n).astype(np.float32)
        return r
    if kind == "absent":
        r = rng.standard_normal(n).astype(np.float32)
        r[rng.random(n) < 0.7] = -np.inf
        return r
    if kind == "narrow":      # many values inside one 12-bit bucket: candidate overflow
        return (1000.0 + rng.random(n) * 0.5).astype(np.float32)
    raise ValueError(kind)


@pytest.mark.parametrize("n,k", [(1, 1), (5, 8), (100, 64), (2047, 2048), (4096, 512),
                                 (16384, 512), (16384, 2048), (16385, 2048), (32768, 2048),
                                 (50001, 512), (131072, 2048), (131072, 4096), (140000, 2048),
                                 (200003, 1000)])
@pytest.mark.parametrize("kind", ["normal", "few", "equal", "signed_zero", "absent", "narrow"])
def test_select_pool_matches_sort(K, n, k, kind):
    print(f"topk n={n} k={k} kind={kind}", flush=True)
    rng = np.random.default_rng(n * 7 + k)
    rows = [_rows(rng, n, kind), _rows(rng, max(1, n - 3), kind), _rows(rng, max(1, n // 3), kind)]
    run(K, rows, k)


def test_select_clustered_rows_take_the_fallback(K):
    """All the winners in one segment: the two-stage check must catch it."""
    rng = np.random.default_rng(5)
    n, k = 131072, 2048
    r = rng.standard_normal(n).astype(np.float32)
    r[40000:44096] += 100.0          # one 4096-entry segment holds every winner
    r2 = rng.standard_normal(n).astype(np.float32)
    r2[::64] += 50.0                 # winners spread evenly
    run(K, [r, r2], k)
