"""The seeded generator: any position range regenerates alone, with the same
values it has inside a larger range (chunk boundaries included)."""
import numpy as np

from fp4_kv_cache_decode_amd import datagen as G


def test_sub_ranges_match_the_full_range():
    C = G.CHUNK
    k, v, ik = G.kv_rows(3, 2, C - 300, C + 200)
    for p0, p1 in [(C - 300, C - 299), (C - 10, C + 10), (C, C + 200), (C - 300, C + 200)]:
        kk, vv, ii = G.kv_rows(3, 2, p0, p1)
        a, b = p0 - (C - 300), p1 - (C - 300)
        assert np.array_equal(kk, k[a:b]) and np.array_equal(vv, v[a:b])
        assert np.array_equal(ii, ik[a:b])
    wk, wv = G.window_rows(3, 1, 2, 0, 1000)
    wk2, wv2 = G.window_rows(3, 1, 2, 500, 700)
    assert np.array_equal(wk2, wk[500:700]) and np.array_equal(wv2, wv[500:700])


def test_streams_are_distinct_and_shaped():
    k0, _, _ = G.kv_rows(0, 0, 0, 64)
    k1, _, _ = G.kv_rows(0, 1, 0, 64)
    assert k0.shape == (64, G.D) and k0.dtype == np.float32
    assert not np.array_equal(k0, k1)
    q, w = G.index_queries(0, 0, 5)
    assert q.shape == (5, G.HI, G.DI) and w.shape == (5, G.HI)
    assert np.all((w >= 0) & (w < 1))


def test_page_table_layout():
    """A fragmented page layout: each sequence owns exactly the pages its rows
    need, no physical page is owned twice, the spare pages are owned by nobody,
    the rest of each row is -1, and the draw is seeded."""
    table, n_pages = G.page_table(3, 3, 1024, 64, [1000, 64, 1], spare=5)
    assert table.shape == (3, 16) and table.dtype == np.int32
    assert n_pages == 16 + 1 + 1 + 5
    need = [16, 1, 1]
    for s in range(3):
        assert (table[s, :need[s]] >= 0).all() and (table[s, need[s]:] == -1).all()
    owned = table[table >= 0]
    assert owned.size == 18 and np.unique(owned).size == 18
    assert owned.max() < n_pages
    again, _ = G.page_table(3, 3, 1024, 64, [1000, 64, 1], spare=5)
    assert np.array_equal(table, again)
    other, _ = G.page_table(4, 3, 1024, 64, [1000, 64, 1], spare=5)
    assert not np.array_equal(table, other)
