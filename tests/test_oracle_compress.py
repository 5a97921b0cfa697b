"""Pins of the oracle's global-KV compression (CPU only).

The pages run the encoder's CSA2 layers at compression m = 2 and the
decoder's at m = 1 (origotech.dev deep dive "Inside DeepSeek V4.1-Flash",
section "How the architecture shrinks the KV cache") but give no operator.
The reading pinned here: entry e of a sequence stands for tokens m*e ..
m*e + m - 1, its rows are their fp32 mean (one rounding of the exact mean for
m = 2), quantised as a token row is; the window keeps every token; a query
with N tokens of context sees entries [0, N // m) and window rows
[N - 128, N).

The expected bytes are built without the oracle's codec or its mean: the
exact rational mean rounded to the nearest fp32 by hand, then the FP4
brute force and torch's E4M3 of tests/test_oracle_layout.py, packed by the
documented record layout.
"""
from fractions import Fraction

import numpy as np

import oracle as O
from test_oracle_layout import E4M3, _e4m3, _fp4_vector

E2M1 = np.array([0, .5, 1, 1.5, 2, 3, 4, 6, -0., -.5, -1, -1.5, -2, -3, -4, -6])


def _round_f32(fr: Fraction) -> np.float32:
    """Nearest fp32 to an exact rational, ties to the even significand."""
    x = np.float32(float(fr))
    best = None
    for y in (np.nextafter(x, np.float32(-np.inf)), x, np.nextafter(x, np.float32(np.inf))):
        d = abs(Fraction(float(y)) - fr)
        even = (int(np.array(y, np.float32).view(np.uint32)) & 1) == 0
        if best is None or d < best[0] or (d == best[0] and even):
            best = (d, y)
    return np.float32(best[1])


def _exact_mean(rows) -> np.ndarray:
    return np.array([_round_f32(sum(Fraction(float(r[c])) for r in rows) / len(rows))
                     for c in range(rows[0].size)], np.float32)


def _inputs(rng, n, n_layers):
    k = (rng.standard_normal((n, 128)) * rng.uniform(0.05, 20, (n, 1))).astype(np.float32)
    v = (rng.standard_normal((n, 128)) * rng.uniform(0.05, 20, (n, 1))).astype(np.float32)
    ik = (rng.standard_normal((n, 64)) * 3).astype(np.float32)
    wk = (rng.standard_normal((n_layers, n, 128)) * 4).astype(np.float32)
    wv = (rng.standard_normal((n_layers, n, 128)) * 2).astype(np.float32)
    for l in range(n_layers):
        wk[l] += np.float32(10 * l)
    return k, v, ik, wk, wv


def test_m1_writes_the_bytes_of_quantize():
    rng = np.random.default_rng(11)
    n_seq, cap, n_layers, w_cap = 2, 64, 2, 16
    k, v, ik, wk, wv = _inputs(rng, 12, n_layers)
    seq = np.array([0, 1] * 6, np.int32)
    pos = np.array([3, 9, 40, 2, 17, 63, 0, 30, 5, 11, 60, 48], np.int64)
    a = O.Cache(n_seq, cap, n_layers, w_cap, idxk_scale=0.37, wk_scale=1.7, wv_scale=0.5)
    b = O.Cache(n_seq, cap, n_layers, w_cap, idxk_scale=0.37, wk_scale=1.7, wv_scale=0.5)
    a.quantize(k, v, ik, wk, wv, seq, pos)
    b.compress(k, v, ik, wk, wv, seq, pos, 1)
    for x, y in ((a.kv, b.kv), (a.idxk, b.idxk), (a.wk, b.wk), (a.wv, b.wv)):
        assert np.array_equal(x, y)


def test_m2_entries_are_the_quantised_fp32_mean_at_pos_over_two():
    rng = np.random.default_rng(12)
    n_seq, cap, n_layers, w_cap = 3, 20, 2, 11
    isc, wks, wvs = 0.37, 1.7, 0.5
    # groups: (seq, first position); positions within a sequence are distinct
    groups = [(0, 0), (2, 38), (1, 6), (0, 14), (2, 2), (1, 30)]
    seq = np.repeat(np.array([s for s, _ in groups], np.int32), 2)
    pos = np.array([p + j for _, p in groups for j in range(2)], np.int64)
    n = seq.size
    slots = {(int(s), int(p) % w_cap) for s, p in zip(seq, pos)}
    assert len(slots) == n
    k, v, ik, wk, wv = _inputs(rng, n, n_layers)
    k[3] = -k[2]                 # a group whose K mean is all zeros
    v[5] = v[4] * np.float32(3)  # one where the mean is twice a row

    c = O.Cache(n_seq, cap, n_layers, w_cap, idxk_scale=isc, wk_scale=wks, wv_scale=wvs)
    c.compress(k, v, ik, wk, wv, seq, pos, 2)

    kv = np.zeros((n_seq, cap, 144), np.uint8)
    idxk = np.zeros((n_seq, cap, 64), np.uint8)
    wks_ = np.zeros((n_layers, n_seq, w_cap, 128), np.uint8)
    wvs_ = np.zeros_like(wks_)
    for g, (s, p) in enumerate(groups):
        i0 = 2 * g
        mk = _exact_mean([k[i0], k[i0 + 1]])
        mv = _exact_mean([v[i0], v[i0 + 1]])
        mi = _exact_mean([ik[i0], ik[i0 + 1]])
        kc, ksc = _fp4_vector(mk)
        vc, vsc = _fp4_vector(mv)
        kv[s, p // 2] = np.concatenate([kc, vc, ksc, vsc])
        idxk[s, p // 2] = _e4m3(mi, isc)
    for i in range(n):
        s, p = int(seq[i]), int(pos[i])
        for l in range(n_layers):
            wks_[l, s, p % w_cap] = _e4m3(wk[l, i], wks)
            wvs_[l, s, p % w_cap] = _e4m3(wv[l, i], wvs)
    assert np.array_equal(c.kv, kv)
    assert np.array_equal(c.idxk, idxk)
    assert np.array_equal(c.wk, wks_)
    assert np.array_equal(c.wv, wvs_)


def test_m2_of_a_repeated_row_is_that_row():
    """Closed form: the mean of a row with itself is the row, so m = 2 over
    (r, r) writes quantize(r) at position p / 2."""
    rng = np.random.default_rng(13)
    k, v, ik, _, _ = _inputs(rng, 5, 1)
    seq = np.zeros(10, np.int32)
    pos = np.arange(10, dtype=np.int64)
    a = O.Cache(1, 8, idxk_scale=0.5)
    b = O.Cache(1, 8, idxk_scale=0.5)
    a.compress(np.repeat(k, 2, 0), np.repeat(v, 2, 0), np.repeat(ik, 2, 0), None, None,
               seq, pos, 2)
    b.quantize(k, v, ik, None, None, np.zeros(5, np.int32), np.arange(5, dtype=np.int64))
    assert np.array_equal(a.kv, b.kv)
    assert np.array_equal(a.idxk, b.idxk)


def test_m2_skips_groups_at_odd_positions_but_keeps_their_window_rows():
    rng = np.random.default_rng(14)
    k, v, ik, wk, wv = _inputs(rng, 4, 1)
    seq = np.zeros(4, np.int32)
    pos = np.array([3, 4, 8, 9], np.int64)          # first group starts at an odd position
    c = O.Cache(1, 8, 1, 16)
    c.compress(k, v, ik, wk, wv, seq, pos, 2)
    assert not c.kv[0, 1].any() and not c.kv[0, 2].any() and not c.idxk[0, 1].any()
    assert c.kv[0, 4].any()
    ref = O.Cache(1, 16, 1, 16)
    ref.quantize(k, v, None, wk, wv, seq, pos)
    assert np.array_equal(c.wk, ref.wk) and np.array_equal(c.wv, ref.wv)


def _decode_record(rec):
    out = []
    for off, sc_off in ((0, 128), (64, 136)):
        nib = np.empty(128, np.int64)
        nib[0::2] = rec[off:off + 64] & 15
        nib[1::2] = rec[off:off + 64] >> 4
        out.append(E2M1[nib] * E4M3[rec[sc_off:sc_off + 8]].repeat(16))
    return out


def test_m2_layer_sees_n_over_two_entries_and_the_raw_window():
    """A Full layer at m = 2 with top-k covering every entry: the index set is
    [0, N // 2) and the attention equals dense softmax attention (numpy, fp64)
    over those entries decoded with the value tables plus the window rows of
    positions [N - 128, N) -- the visibility reading of compressed entries."""
    rng = np.random.default_rng(15)
    N_tok = 301                    # odd: the last token has no complete pair
    w_cap = 160
    n = N_tok - 1
    k, v, ik, _, _ = _inputs(rng, N_tok, 1)
    wk = (rng.standard_normal((1, N_tok, 128))).astype(np.float32)
    wv = (rng.standard_normal((1, N_tok, 128))).astype(np.float32)
    c = O.Cache(1, 256, 1, w_cap)
    seq = np.zeros(N_tok, np.int32)
    pos = np.arange(N_tok, dtype=np.int64)
    c.compress(k[:n], v[:n], ik[:n], wk[:, :n], wv[:, :n], seq[:n], pos[:n], 2)
    # the unpaired last token only reaches the window
    before = c.kv.copy(), c.idxk.copy()
    c.compress(None, None, None, wk[:, n:], wv[:, n:], seq[n:], pos[n:], 2)
    assert np.array_equal(c.kv, before[0]) and np.array_equal(c.idxk, before[1])
    n_c = N_tok // 2
    q_idx = rng.standard_normal((1, 4, 64)).astype(np.float32)
    w = rng.uniform(0, 1, (1, 4)).astype(np.float32)
    ctx_c = np.array([n_c], np.int64)
    _, idx, _, _ = c.index_full(q_idx, w, np.zeros(1, np.int32), ctx_c, n_blocks=64,
                                topk=256)
    got = np.sort(idx[0][idx[0] >= 0])
    assert np.array_equal(got, np.arange(n_c))

    q = rng.standard_normal((1, 16, 128)).astype(np.float32)
    out = c.decode_attn(0, q, idx, np.zeros(1, np.int32), np.array([N_tok], np.int64))
    K, V = [], []
    for e in range(n_c):
        ke, ve = _decode_record(c.kv[0, e])
        K.append(ke)
        V.append(ve)
    for u in range(N_tok - 128, N_tok):
        K.append(E4M3[c.wk[0, 0, u % w_cap]])
        V.append(E4M3[c.wv[0, 0, u % w_cap]])
    K, V = np.array(K), np.array(V)
    z = q[0].astype(np.float64) @ K.T * float(np.float32(1 / np.sqrt(128)))
    p = np.exp(z - z.max(1, keepdims=True))
    ref = (p / p.sum(1, keepdims=True)) @ V
    assert np.max(np.abs(out[0] - ref)) < 1e-5
