"""The C-ABI library loads, exports what include/csa2.h declares, sizes its
workspaces consistently and rejects bad arguments on the host (CPU only: none
of these calls reaches a kernel launch)."""
import ctypes as C
import os
import re

import pytest

from conftest import ROOT

HEADER = os.path.join(ROOT, "include", "csa2.h")


@pytest.fixture(scope="module")
def L():
    from fp4_kv_cache_decode_amd import csa2
    if not os.path.exists(csa2.LIB_PATH):
        from fp4_kv_cache_decode_amd import build
        build.build()
    return csa2.lib()


def _declared():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(csa2_[a-z_]+)\s*\(", src)))


def test_header_declares_the_four_calls():
    names = _declared()
    for n in ("csa2_quantize_kv", "csa2_index_full", "csa2_index_reindex", "csa2_decode_attn",
              "csa2_workspace_bytes", "csa2_status_string"):
        assert n in names


def test_library_exports_every_declared_symbol(L):
    for name in _declared():
        assert hasattr(L, name), name


def test_status_strings(L):
    from fp4_kv_cache_decode_amd import csa2
    assert csa2.status_string(0) == "ok"
    assert "workspace" in csa2.status_string(3)


def test_workspace_sizes(L):
    from fp4_kv_cache_decode_amd import csa2 as K
    full = K.workspace_bytes(K.OP_INDEX_FULL, 4, 1 << 20, 2048, 8, 512)
    # block maxima (4 x 131072 fp32) + pool (4 x 2048 int32) + pool scores (4 x 16384 fp32)
    assert full >= 4 * 131072 * 4 + 4 * 2048 * 4 + 4 * 16384 * 4
    assert full % 256 == 0
    assert K.workspace_bytes(K.OP_INDEX_REINDEX, 4, 0, 2048, 8, 512) == 4 * 16384 * 4
    # attention: one partial record (m, l, O: 32 + 2048 floats) per split of a query
    part = (32 + 2048) * 4
    assert K.workspace_bytes(K.OP_DECODE_ATTN, 4, 0, 0, 0, 512) == 4 * 10 * part     # 10 tiles
    assert K.workspace_bytes(K.OP_DECODE_ATTN, 96, 0, 0, 0, 512) == 96 * 10 * part   # stream
    assert K.workspace_bytes(K.OP_DECODE_ATTN, 1024, 0, 0, 0, 512) == 0             # unsplit
    assert K.workspace_bytes(K.OP_INDEX_FULL, 4, 1 << 20, 2048, 4, 512) == 0      # block != 8
    assert K.workspace_bytes(K.OP_INDEX_FULL, 4, 1 << 20, 8192, 8, 512) == 0      # pool too big
    assert K.workspace_bytes(K.OP_DECODE_ATTN, 4, 0, 0, 0, 4096) == 0             # topk too big
    assert K.workspace_bytes(99, 4, 0, 0, 0, 512) == 0
    # block selection: one workgroup per row up to 32,768 blocks, segments beyond
    assert K.workspace_bytes(K.OP_SELECT_POOL, 4, 8 * 32768, 2048, 8, 1) == 0
    assert K.workspace_bytes(K.OP_SELECT_POOL, 4, 8 * 32768 + 1, 2048, 8, 1) > 0
    assert K.workspace_bytes(K.OP_SELECT_POOL, 4, 8 * 131072, 2048, 8, 1) > 0


FAKE = C.c_void_p(0x10000)   # never dereferenced: validation fails first


def _cache(K, kv=FAKE, idxk=FAKE, n_seq=1, cap=1024, scale=1.0):
    return K.csa2_cache(kv.value if kv else None, idxk.value if idxk else None, scale, n_seq, cap)


def _win(K, n_layers=1, n_seq=1, w_cap=128):
    return K.csa2_window(FAKE.value, FAKE.value, 1.0, 1.0, n_layers, n_seq, w_cap)


def test_quantize_error_paths(L):
    from fp4_kv_cache_decode_amd import csa2 as K
    c, w = _cache(K), _win(K)
    f = L.csa2_quantize_kv
    assert f(None, C.byref(w), FAKE, FAKE, None, None, None, FAKE, FAKE, 4, None) == 1
    assert f(C.byref(_cache(K, kv=None)), None, FAKE, FAKE, None, None, None, FAKE, FAKE, 4,
             None) == 1
    assert f(C.byref(c), None, None, FAKE, None, None, None, FAKE, FAKE, 4, None) == 1
    assert f(C.byref(c), None, FAKE, FAKE, None, None, None, FAKE, FAKE, -1, None) == 1
    assert f(C.byref(c), C.byref(w), FAKE, FAKE, None, FAKE, None, FAKE, FAKE, 4, None) == 1
    assert f(C.byref(c), None, FAKE, FAKE, None, FAKE, FAKE, FAKE, FAKE, 4, None) == 1
    assert f(C.byref(c), C.byref(_win(K, w_cap=64)), FAKE, FAKE, None, FAKE, FAKE, FAKE, FAKE,
             4, None) == 2
    assert f(C.byref(c), C.byref(_win(K, n_seq=2)), FAKE, FAKE, None, FAKE, FAKE, FAKE, FAKE,
             4, None) == 1
    assert f(C.byref(_cache(K, scale=0.0)), None, FAKE, FAKE, FAKE, None, None, FAKE, FAKE, 4,
             None) == 1
    assert f(C.byref(c), None, FAKE, FAKE, None, None, None, FAKE, FAKE, 0, None) == 0


def test_compress_error_paths(L):
    from fp4_kv_cache_decode_amd import csa2 as K
    c = _cache(K)
    f = L.csa2_compress_kv
    assert f(C.byref(c), None, FAKE, FAKE, None, None, None, FAKE, FAKE, 4, 3, None) == 2
    assert f(C.byref(c), None, FAKE, FAKE, None, None, None, FAKE, FAKE, 4, 0, None) == 2
    assert f(C.byref(c), None, FAKE, FAKE, None, None, None, FAKE, FAKE, 5, 2, None) == 1
    assert f(C.byref(c), None, None, FAKE, None, None, None, FAKE, FAKE, 4, 2, None) == 1
    assert f(C.byref(c), None, FAKE, FAKE, None, None, None, FAKE, FAKE, 0, 2, None) == 0
    # window only: k and v both NULL, no indexer keys, window rows given
    w = _win(K)
    assert f(C.byref(c), C.byref(w), None, FAKE, None, FAKE, FAKE, FAKE, FAKE, 4, 2, None) == 1
    assert f(C.byref(c), None, None, None, None, None, None, FAKE, FAKE, 4, 2, None) == 1
    assert f(C.byref(c), C.byref(w), None, None, FAKE, FAKE, FAKE, FAKE, FAKE, 4, 2, None) == 1
    assert f(C.byref(c), C.byref(w), None, None, None, FAKE, FAKE, FAKE, FAKE, 0, 2, None) == 0


def test_index_error_paths(L):
    from fp4_kv_cache_decode_amd import csa2 as K
    c = _cache(K)
    f = L.csa2_index_full
    ws_ok = K.workspace_bytes(K.OP_INDEX_FULL, 2, 1024, 64, 8, 32)
    args = lambda **kw: dict(dict(cache=C.byref(c), q=FAKE, w=FAKE, seq=FAKE, ctx=FAKE, B=2,
                                  max_ctx=1024, nb=64, block=8, topk=32, pool=None, idx=FAKE,
                                  ws=FAKE, wsb=ws_ok), **kw)
    call = lambda a: f(a["cache"], a["q"], a["w"], a["seq"], a["ctx"], a["B"], a["max_ctx"],
                       a["nb"], a["block"], a["topk"], a["pool"], a["idx"], a["ws"], a["wsb"],
                       None)
    assert call(args(cache=None)) == 1
    assert call(args(q=None)) == 1
    assert call(args(idx=None)) == 1
    assert call(args(block=16)) == 2
    assert call(args(nb=5000)) == 2
    assert call(args(topk=4096)) == 2
    assert call(args(nb=2, topk=32)) == 1            # topk > n_blocks * 8
    assert call(args(max_ctx=2048)) == 1             # beyond cap
    assert call(args(B=-1)) == 1
    assert call(args(ws=None)) == 3
    assert call(args(wsb=ws_ok - 1)) == 3
    assert call(args(B=0)) == 0
    r = L.csa2_index_reindex
    assert r(C.byref(c), FAKE, FAKE, FAKE, FAKE, 2, None, 64, 8, 32, FAKE, FAKE, 1 << 20,
             None) == 1
    assert r(C.byref(c), FAKE, FAKE, FAKE, FAKE, 2, FAKE, 64, 8, 32, FAKE, FAKE, 16, None) == 3


def test_attn_error_paths(L):
    from fp4_kv_cache_decode_amd import csa2 as K
    c, w = _cache(K), _win(K, n_layers=2)
    f = L.csa2_decode_attn
    ws = K.workspace_bytes(K.OP_DECODE_ATTN, 2, 0, 0, 0, 512)
    call = lambda **kw: f(kw.get("c", C.byref(c)), kw.get("w", C.byref(w)), kw.get("layer", 1),
                          FAKE, kw.get("idx", FAKE), FAKE, FAKE, kw.get("B", 2),
                          kw.get("topk", 512), kw.get("sm", 0.088), FAKE, kw.get("ws", FAKE),
                          kw.get("wsb", ws), None)
    assert call(w=None) == 1
    assert call(layer=2) == 1
    assert call(layer=-1) == 1
    assert call(idx=None) == 1
    assert call(topk=0) == 2
    assert call(topk=4096) == 2
    assert call(sm=float("nan")) == 1
    assert call(wsb=ws - 4) == 3
    assert call(B=0) == 0
    # the gathered-KV variant: the same checks, and at most one gathered buffer
    fx = L.csa2_decode_attn_ex
    call_ex = lambda gin, gout, **kw: fx(C.byref(c), C.byref(w), kw.get("layer", 1), FAKE, FAKE,
                                         FAKE, FAKE, kw.get("B", 2), 512, 0.088, gin, gout, FAKE,
                                         FAKE, ws, None)
    assert call_ex(FAKE, FAKE) == 1
    assert call_ex(FAKE, None, layer=2) == 1
    assert call_ex(None, FAKE, B=0) == 0
    assert call_ex(FAKE, None, B=0) == 0


def test_fused_layer_sizes_and_error_paths(L):
    """csa2_reindex_layer_fused: workspace = barrier words (two 128-byte lines)
    + pool scores + the tiles' partial records; host-side argument checks."""
    from fp4_kv_cache_decode_amd import csa2 as K
    part = (32 + 2048) * 4
    ws = K.workspace_bytes(K.OP_REINDEX_LAYER_FUSED, 4, 0, 2048, 8, 512)
    assert ws == 256 + 4 * 16384 * 4 + 4 * 10 * part
    assert K.workspace_bytes(K.OP_REINDEX_LAYER_FUSED, 4, 0, 2048, 4, 512) == 0   # block != 8
    assert K.workspace_bytes(K.OP_REINDEX_LAYER_FUSED, 4, 0, 8192, 8, 512) == 0   # pool too big
    c, w = _cache(K), _win(K, n_layers=2)
    f = L.csa2_reindex_layer_fused
    ws2 = K.workspace_bytes(K.OP_REINDEX_LAYER_FUSED, 2, 0, 64, 8, 32)

    def call(**kw):
        a = dict(c=C.byref(c), w=C.byref(w), layer=1, qi=FAKE, wt=FAKE, q=FAKE, seq=FAKE,
                 ctx=FAKE, B=2, pool=FAKE, nb=64, block=8, topk=32, sm=0.088, idx=FAKE,
                 kvg=None, out=FAKE, polls=0, status=FAKE, ws=FAKE, wsb=ws2)
        a.update(kw)
        return f(a["c"], a["w"], a["layer"], a["qi"], a["wt"], a["q"], a["seq"], a["ctx"],
                 a["B"], a["pool"], a["nb"], a["block"], a["topk"], a["sm"], a["idx"],
                 a["kvg"], a["out"], a["polls"], a["status"], a["ws"], a["wsb"], None)

    assert call(c=None) == 1
    assert call(w=None) == 1
    assert call(c=C.byref(_cache(K, idxk=None))) == 1
    assert call(qi=None) == 1
    assert call(q=None) == 1
    assert call(pool=None) == 1
    assert call(status=None) == 1
    assert call(layer=2) == 1
    assert call(sm=float("inf")) == 1
    assert call(block=16) == 2
    assert call(nb=5000) == 2
    assert call(nb=2, topk=32) == 1                   # topk > n_blocks * 8
    assert call(B=77, topk=512) == 2                  # 77 x 10 tiles > 768
    assert call(ws=None) == 3
    assert call(wsb=ws2 - 1) == 3
    assert call(B=0) == 0


def test_paged_cache_validation(L):
    """A page table needs a power-of-two page of 64..65,536 tokens that divides
    cap and at least one physical page; every entry point checks it."""
    from fp4_kv_cache_decode_amd import csa2 as K

    def paged(P, n_pages=8, cap=1024):
        return K.csa2_cache(FAKE.value, FAKE.value, 1.0, 1, cap, FAKE.value, P, n_pages)

    q = L.csa2_quantize_kv
    quant = lambda c: q(C.byref(c), None, FAKE, FAKE, None, None, None, FAKE, FAKE, 0, None)
    assert quant(paged(64)) == 0
    assert quant(paged(1024)) == 0
    for bad in (0, 32, 96, 1 << 17):
        assert quant(paged(bad)) == 2, bad
    assert quant(paged(256, cap=1000)) == 1     # cap not a multiple of the page
    assert quant(paged(256, n_pages=0)) == 1
    # a null table means contiguous: the page fields are not looked at
    assert quant(K.csa2_cache(FAKE.value, FAKE.value, 1.0, 1, 1000, None, 96, 0)) == 0
    w = _win(K)
    ws = K.workspace_bytes(K.OP_DECODE_ATTN, 2, 0, 0, 0, 512)
    attn = lambda c: L.csa2_decode_attn(C.byref(c), C.byref(w), 0, FAKE, FAKE, FAKE, FAKE, 0,
                                        512, 0.088, FAKE, FAKE, ws, None)
    assert attn(paged(128)) == 0
    assert attn(paged(100)) == 2
    full = lambda c: L.csa2_index_full(C.byref(c), FAKE, FAKE, FAKE, FAKE, 0, 1024, 64, 8, 32,
                                       None, FAKE, FAKE, 1 << 20, None)
    assert full(paged(128)) == 0
    assert full(paged(256, n_pages=-1)) == 1
    ri = lambda c: L.csa2_index_reindex(C.byref(c), FAKE, FAKE, FAKE, FAKE, 0, FAKE, 64, 8, 32,
                                        FAKE, FAKE, 1 << 20, None)
    assert ri(paged(64)) == 0
    assert ri(paged(48)) == 2


C_PROGRAM = r"""
#include <stdio.h>
#include <string.h>
#include "csa2.h"
int main(void) {
    csa2_cache c;
    memset(&c, 0, sizeof c);              /* a zeroed tail: contiguous cache */
    /* no GPU work: sizes and status strings are host functions */
    size_t part = (size_t)(32 + 2048) * 4;
    if (csa2_workspace_bytes(CSA2_OP_DECODE_ATTN, 4, 0, 0, 0, 512) != 4 * 10 * part) return 1;
    if (csa2_workspace_bytes(CSA2_OP_INDEX_REINDEX, 4, 0, 2048, CSA2_BLOCK, 512) != 4 * 16384 * 4)
        return 2;
    if (strcmp(csa2_status_string(CSA2_OK), "ok") != 0) return 3;
    if (csa2_quantize_kv(NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, 0, NULL) !=
        CSA2_ERR_INVALID_ARG) return 4;
    printf("c-abi ok %zu\n", sizeof c);
    return 0;
}
"""


def _hip_include():
    return os.environ.get("ROCM_PATH", "/opt/rocm") + "/include"


def test_header_compiles_as_c_and_cxx(tmp_path):
    """include/csa2.h is a plain C header (usable from C11 and C++17)."""
    import shutil
    import subprocess
    src = tmp_path / "h.c"
    src.write_text('#include "csa2.h"\nint main(void) { return CSA2_OK; }\n')
    for cc, args in (("gcc", ["-std=c11", "-x", "c"]), ("g++", ["-std=c++17", "-x", "c++"])):
        if shutil.which(cc) is None:
            pytest.skip(f"{cc} not available")
        r = subprocess.run([cc, *args, "-Wall", "-Werror=implicit-function-declaration",
                            "-fsyntax-only", "-D__HIP_PLATFORM_AMD__", "-I", _hip_include(),
                            "-I", os.path.join(ROOT, "include"), str(src)],
                           capture_output=True, text=True)
        assert r.returncode == 0, r.stderr[-2000:]


def test_c_program_links_and_calls_host_functions(L, tmp_path):
    """A C program links against libcsa2.so through the header alone and gets
    the documented sizes, status strings and argument errors."""
    import shutil
    import subprocess
    from fp4_kv_cache_decode_amd import csa2
    if shutil.which("gcc") is None:
        pytest.skip("gcc not available")
    src, exe = tmp_path / "p.c", tmp_path / "p"
    src.write_text(C_PROGRAM)
    libdir = os.path.dirname(csa2.LIB_PATH)
    rocm_lib = os.environ.get("ROCM_PATH", "/opt/rocm") + "/lib"
    r = subprocess.run(["gcc", "-std=c11", "-Wall", "-D__HIP_PLATFORM_AMD__", "-I", _hip_include(),
                        "-I", os.path.join(ROOT, "include"), str(src), "-o", str(exe),
                        f"-L{libdir}", "-l:libcsa2.so", f"-Wl,-rpath,{libdir}",
                        f"-L{rocm_lib}", f"-Wl,-rpath,{rocm_lib}", "-lamdhip64"],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=60)
    assert r.returncode == 0, (r.returncode, r.stdout, r.stderr[-1000:])
    assert r.stdout.startswith("c-abi ok")
