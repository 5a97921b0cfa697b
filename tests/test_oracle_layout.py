"""Pin of where the oracle's quantise-on-write puts its bytes (CPU only).

The expected cache bytes are built here without the oracle's codec:
  * FP4 nibbles and E4M3 group-scale codes come from the exact rational
    brute force of tests/test_oracle_codecs.py (nearest of s * E2M1 with
    ties to the even code, s = E4M3(fp32(amax) / 6));
  * indexer-key and window codes come from torch's float8_e4m3fn conversion
    of the fp32 quotient x / scale;
  * they are packed by the documented layout: one 144-byte record per token
    with K codes at [0,64), V codes at [64,128), 8 K scales at [128,136) and
    8 V scales at [136,144), channel 2j in the low nibble of byte j; the
    indexer key at row seq*cap + pos; window row (layer, seq, pos % w_cap).
The format (FP4 E2M1 main KV with one E4M3 scale per 16 channels, FP8
window) is the one of trawling.dev "CSA2 and FP4 KV caching" and origotech.dev
deep dive, sub-section "FP4 and SWA Bounded Replay"; the byte order within a
record is this library's reading.

A K/V swap, a scale-block swap, a nibble-order slip, a wrong row or a window
layer/slot slip in the oracle fails this test.
"""
from fractions import Fraction

import numpy as np
import torch

import oracle as O
from test_oracle_codecs import _brute_group

E4M3 = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()


def _scale_code(s: Fraction) -> int:
    """E4M3 code of a non-negative representable value."""
    hits = [c for c in range(0x7F) if Fraction(float(E4M3[c])) == s]
    assert len(hits) == 1, s
    return hits[0]


def _fp4_vector(x):
    """(64 code bytes, 8 scale codes) of a 128-channel row, packed by hand."""
    codes = np.zeros(64, np.uint8)
    scales = np.zeros(8, np.uint8)
    for g in range(8):
        nib, s = _brute_group(x[16 * g:16 * g + 16])
        scales[g] = _scale_code(s)
        for j in range(8):
            codes[8 * g + j] = int(nib[2 * j]) | (int(nib[2 * j + 1]) << 4)
    return codes, scales


def _e4m3(x, scale):
    q = (np.asarray(x, np.float32) / np.float32(scale)).astype(np.float32)
    assert np.all(np.abs(q) < 448.0)       # inside torch's saturation-free range
    return torch.from_numpy(q).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def test_quantize_places_bytes_by_the_documented_layout():
    rng = np.random.default_rng(2024)
    n_seq, cap, n_layers, w_cap = 3, 40, 3, 13
    isc, wks, wvs = 0.37, 1.7, 0.5
    n = 9
    # distinct (seq, pos) rows with distinct window slots per sequence
    seq = np.array([0, 2, 1, 0, 2, 1, 0, 2, 1], np.int32)
    pos = np.array([5, 39, 0, 17, 3, 24, 33, 12, 10], np.int64)
    slots = {(int(s), int(p) % w_cap) for s, p in zip(seq, pos)}
    assert len(slots) == n
    k = (rng.standard_normal((n, 128)) * rng.uniform(0.05, 20, (n, 1))).astype(np.float32)
    v = (rng.standard_normal((n, 128)) * rng.uniform(0.05, 20, (n, 1))).astype(np.float32)
    v[0] = -k[0]                         # K and V of one row differ in every sign
    ik = (rng.standard_normal((n, 64)) * 3).astype(np.float32)
    wk = (rng.standard_normal((n_layers, n, 128)) * 4).astype(np.float32)
    wv = (rng.standard_normal((n_layers, n, 128)) * 2).astype(np.float32)
    for l in range(n_layers):                 # layers differ by construction
        wk[l] += np.float32(10 * l)

    c = O.Cache(n_seq, cap, n_layers, w_cap, idxk_scale=isc, wk_scale=wks, wv_scale=wvs)
    c.quantize(k, v, ik, wk, wv, seq, pos)

    kv = np.zeros((n_seq, cap, 144), np.uint8)
    idxk = np.zeros((n_seq, cap, 64), np.uint8)
    wks_ = np.zeros((n_layers, n_seq, w_cap, 128), np.uint8)
    wvs_ = np.zeros_like(wks_)
    for i in range(n):
        s, p = int(seq[i]), int(pos[i])
        kc, ksc = _fp4_vector(k[i])
        vc, vsc = _fp4_vector(v[i])
        kv[s, p] = np.concatenate([kc, vc, ksc, vsc])
        idxk[s, p] = _e4m3(ik[i], isc)
        for l in range(n_layers):
            wks_[l, s, p % w_cap] = _e4m3(wk[l, i], wks)
            wvs_[l, s, p % w_cap] = _e4m3(wv[l, i], wvs)

    assert np.array_equal(c.kv, kv)
    assert np.array_equal(c.idxk, idxk)
    assert np.array_equal(c.wk, wks_)
    assert np.array_equal(c.wv, wvs_)


def test_record_decodes_back_to_its_row_within_the_fp4_bound():
    """Decoding a record with the value tables (E2M1 set, torch E4M3) at the
    documented offsets gives back K from [0,64)+[128,136) and V from
    [64,128)+[136,144), each channel within half a grid step of its input."""
    e2m1 = np.array([0, .5, 1, 1.5, 2, 3, 4, 6, -0., -.5, -1, -1.5, -2, -3, -4, -6])
    rng = np.random.default_rng(5)
    k = (rng.standard_normal((4, 128)) * 3).astype(np.float32)
    v = (rng.standard_normal((4, 128)) * 0.2).astype(np.float32)
    c = O.Cache(1, 4)
    c.quantize(k, v, None, None, None, np.zeros(4, np.int32), np.arange(4))
    for i in range(4):
        rec = c.kv[0, i]
        for off, sc_off, x in ((0, 128, k[i]), (64, 136, v[i])):
            nib = np.empty(128, np.int64)
            nib[0::2] = rec[off:off + 64] & 15
            nib[1::2] = rec[off:off + 64] >> 4
            s = E4M3[rec[sc_off:sc_off + 8]].repeat(16)
            dec = e2m1[nib] * s
            # largest E2M1 step is 2 (between 4 and 6): half of it times the scale
            assert np.all(np.abs(dec - x) <= s + 1e-12)
            assert np.max(np.abs(dec - x)) < np.max(np.abs(x)) / 4
