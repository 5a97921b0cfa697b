"""csa2_decode_attn_noalloc (the library's fixed per-GPU scratch, no workspace)
against csa2_decode_attn_ex with a caller workspace, through the C ABI.

Calls in a row on one GPU share the scratch, each with a smaller batch than the
one before: B = 300 (split streaming path whose partial records would exceed
the scratch, so fewer splits: within the attention tolerance), B = 96 (split
streaming path, same plan: bit-identical) and B = 3 (tile kernel and merge,
same plan: bit-identical).  Each is also within 2e-3 of the oracle, and the
gathered-record variants (kvg_out, then kvg_in) match too.
"""
import sys

import numpy as np
import pytest

import oracle as O
from fp4_kv_cache_decode_amd import datagen as G
from parity import ATTN_TOL, fill_both

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")


def _say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def test_noalloc_matches_workspace_entry_point():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from fp4_kv_cache_decode_amd import csa2 as K
    n_seq, N, L, seed = 3, 3000, 2, 71
    oc = O.Cache(n_seq, N, L)
    gc = K.Cache(n_seq, N, L)
    fill_both(seed, n_seq, N, L, oc, gc)
    qi, wi = G.index_queries(seed, 0, n_seq)
    ctx3 = np.array([N, N - 11, 1500], np.int64)
    _, idx3, _, _ = oc.index_full(qi, wi, np.arange(n_seq, dtype=np.int32), ctx3)
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    for B, same_plan in ((300, False), (96, True), (3, True)):
        _say(f"noalloc attention B={B}")
        seq = (np.arange(B) % n_seq).astype(np.int32)
        ctx = ctx3[seq]
        idx = idx3[seq]
        q = G.attn_queries(seed, 1, B)
        want_ws = torch.empty((B, 16, 128), dtype=torch.float32, device="cuda")
        got = torch.full((B, 16, 128), -7.0, dtype=torch.float32, device="cuda")
        ws = K.alloc_workspace(K.OP_DECODE_ATTN, B)
        args = (dev(q), dev(idx), dev(seq), dev(ctx))
        K.decode_attn(gc, 1, *args, want_ws, ws)
        K.decode_attn_noalloc(gc, 1, *args, got)
        torch.cuda.synchronize()
        g, w = got.cpu().numpy(), want_ws.cpu().numpy()
        if same_plan:
            assert np.array_equal(g, w), f"B={B}: differs from the workspace entry point"
        err = float(np.max(np.abs(g - w)))
        assert err <= ATTN_TOL, f"B={B}: {err}"
        ref = oc.decode_attn(1, q, idx, seq, ctx)
        err_o = float(np.max(np.abs(g - ref)))
        _say(f"  vs workspace entry point {err:.3g}, vs oracle {err_o:.3g}")
        assert err_o <= ATTN_TOL
        # gathered records: stored by one call, read by the next
        kvg = torch.zeros((B, idx.shape[1], K.RECORD), dtype=torch.uint8, device="cuda")
        got2 = torch.empty_like(got)
        K.decode_attn_noalloc(gc, 0, *args, got2, kvg_out=kvg)
        K.decode_attn_noalloc(gc, 1, *args, got, kvg_in=kvg)
        torch.cuda.synchronize()
        assert np.array_equal(got.cpu().numpy(), g)
        ref0 = oc.decode_attn(0, q, idx, seq, ctx)
        assert float(np.max(np.abs(got2.cpu().numpy() - ref0))) <= ATTN_TOL
