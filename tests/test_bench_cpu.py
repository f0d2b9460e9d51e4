"""Host logic of bench.py, on the CPU: the algorithmic bytes it prices a step
at, the comment-blind source hash that ties profiles/traffic.json to the kernel
code it was measured on, and the refusal of more than one GPU."""
import dataclasses
import json
import os
import subprocess
import sys

import numpy as np

import bench
from paged_kv_cache_434_amd import workloads as W

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_algorithmic_bytes_of_the_llama3_8b_step():
    """The 8B decode step: K and V of all 154,680 context tokens at 2 bytes,
    4 bytes per used table entry, q in and out, the lengths, and the new
    token's K/V read and written (its slot comes from the table entry and the
    length already counted).  635,181,196 bytes, the figure the profiles and
    the design notes quote."""
    wl = W.make(2)
    b = bench.algorithmic_bytes(wl)
    L = wl.lens.astype(np.int64)
    assert int(L.sum()) == 154_680
    assert b["kv"] == 154_680 * 8 * 128 * 2 * 2
    tables = int(((L + 15) // 16).sum()) * 4
    assert b["attention"] == b["kv"] + tables + 64 * 32 * 128 * 2 * 2 + 64 * 4
    assert b["write"] == 64 * 8 * 128 * 2 * (2 + 2)
    assert b["step"] == 635_181_196


def test_quantized_bytes_count_codes_and_scales():
    """An E4M3 pool halves the K/V bytes and adds two binary32 scales per
    (block, KV head) read; E2M1 quarters them; per-row uint8 adds a scale and
    a zero point per row."""
    wl = W.make(2)
    L = wl.lens.astype(np.int64)
    nblk = int(((L + 15) // 16).sum())
    for quant, e, extra in (("fp8", 1, nblk * 8 * 2 * 4), ("fp4", 0.5, nblk * 8 * 2 * 4),
                            ("u8z", 1, int(L.sum()) * 8 * 2 * 5)):
        q = dataclasses.replace(wl, quant=quant)   # as bench.py --quant does
        b = bench.algorithmic_bytes(q)
        assert b["kv"] == int(154_680 * 8 * 128 * 2 * e)
        assert b["attention"] == b["kv"] + nblk * 4 + extra + 64 * 32 * 128 * 2 * 2 + 64 * 4


def test_source_hash_ignores_comments_only():
    """Comments and blank lines do not change the hash; code does."""
    src = {"a": "int f() {\n  return 1;  // one\n}\n", "b": "/* x */\nint g;\n"}
    rels = bench.KERNEL_SOURCES
    base = bench.kernel_source_hash(lambda rel: src["a"] if rel == rels[0] else src["b"])
    commented = bench.kernel_source_hash(
        lambda rel: ("// header\n\n" + src["a"]) if rel == rels[0] else src["b"] + "\n\n")
    changed = bench.kernel_source_hash(
        lambda rel: src["a"].replace("1", "2") if rel == rels[0] else src["b"])
    assert base == commented
    assert base != changed


def test_recorded_traffic_matches_the_current_kernel_sources():
    """Every HBM-traffic record under profiles/ was taken on the kernel code
    as it stands (else bench.py would report traffic as null)."""
    with open(os.path.join(ROOT, "profiles", "traffic.json")) as f:
        records = json.load(f)
    assert records
    h = bench.kernel_source_hash()
    assert {r["source_hash"] for r in records.values()} == {h}


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=300)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
