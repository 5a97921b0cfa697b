"""Host-side behaviour of bench.py (no GPU): the one-GPU guard and the source
hash that ties committed counters to the scan code."""
import os
import subprocess
import sys

from conftest import ROOT

sys.path.insert(0, ROOT)


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_code_hash_ignores_comments_and_blank_lines():
    import bench
    code = "int f(int x) {\n    return x + 1;  // add one\n}\n"
    same = "// a header\n\nint f(int x) {\n    return x + 1;\n\n}   \n"
    other = "int f(int x) {\n    return x + 2;\n}\n"
    assert bench.code_hash(code) == bench.code_hash(same)
    assert bench.code_hash(code) != bench.code_hash(other)
    assert len(bench.code_hash(code)) == 16


def test_counter_traffic_needs_matching_workload():
    import bench
    assert bench.counter_traffic("no_such_workload") is None


def test_row_counters_match_their_sources():
    """Each committed row profile names its timed kernel's source and counters
    taken on that source's current code (else the bench reports null traffic)."""
    import bench
    for prof, wl in (("quantize_bulk_decoder20_1m_b4.txt", "quantize_bulk_4x1m"),
                     ("attn_gather_b1024_n64k.txt", "gather_attention_b1024_n64k"),
                     ("prefill_8k_over_128k_kernel_stats.txt", "prefill_8k_over_128k"),
                     ("encoder_chunk8k_m2_kernel_stats.txt", "encoder20_m2_chunk8k_over_128k")):
        t = bench.row_counter_traffic(prof, wl)
        assert t is None or t > 0
        assert bench.row_counter_traffic(prof, "another_workload") is None


def test_source_hash_covers_every_listed_file():
    """A counter record names its kernel's sources as a comma-separated list;
    the hash covers all of them in order, so a change to any shared device
    header retires the counters."""
    import bench
    one = "fp4_kv_cache_decode_amd/csrc/attn.hip"
    two = one + ",fp4_kv_cache_decode_amd/csrc/attn_dev.h"
    texts = [open(os.path.join(ROOT, p)).read() for p in two.split(",")]
    assert bench.source_hash(one) == bench.code_hash(texts[0])
    assert bench.source_hash(two) == bench.code_hash("\n".join(texts))
    assert bench.source_hash(two) != bench.source_hash(one)
    # the step counters list the step kernels' sources, none of the host-only files
    step = bench.STEP_SOURCES.split(",")
    assert all(os.path.exists(os.path.join(ROOT, p)) for p in step)
    assert not any(p.endswith(("capi.hip", "layer.hip", "csa2_internal.h")) for p in step)
