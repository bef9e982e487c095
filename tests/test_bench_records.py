"""Host logic of bench.py: which source changes void a workload's recorded
HBM-traffic counters, and the command line of its rate measurements (CPU
only)."""
import os
import shutil
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


@pytest.fixture()
def tree(tmp_path, monkeypatch):
    src = os.path.join(ROOT, "block_sparse_attention_selection_amd", "csrc")
    dst = tmp_path / "block_sparse_attention_selection_amd" / "csrc"
    shutil.copytree(src, dst)
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    return dst


def _touch(path):
    with open(path, "a") as f:
        f.write("\n// edited\n")


def _hashes():
    return {w: bench.kernel_sources_sha256(w) for w in bench.DOMINANT}


def test_every_dominant_kernel_has_a_source_file():
    for w, kernels in bench.DOMINANT.items():
        for k in kernels:
            assert k in bench.KERNEL_SOURCES, (w, k)


def test_a_kernel_file_voids_only_the_workloads_it_serves(tree):
    before = _hashes()
    _touch(tree / "msa_store.hip")
    after = _hashes()
    changed = {w for w in before if before[w] != after[w]}
    assert changed == {"kv_store_fp8"}


def test_the_tile_file_voids_the_prefill_workloads(tree):
    before = _hashes()
    _touch(tree / "msa_tiles.hip")
    after = _hashes()
    changed = {w for w in before if before[w] != after[w]}
    assert changed == {w for w, ks in bench.DOMINANT.items() if {"units", "tiles"} & set(ks)}


def test_shared_headers_and_the_host_file_void_everything(tree):
    for name in ("msa_internal.hpp", "msa_api.hip"):
        before = _hashes()
        _touch(tree / name)
        after = _hashes()
        assert all(before[w] != after[w] for w in before), name


def test_the_rate_program_voids_nothing(tree):
    # msa_rates.hip is a measurement program, not a kernel of any workload
    before = _hashes()
    _touch(tree / "msa_rates.hip")
    assert _hashes() == before


def test_micro_rejects_an_unknown_measurement_before_touching_the_gpu():
    import subprocess

    from block_sparse_attention_selection_amd.build import RATES

    if not os.path.exists(RATES):
        pytest.skip("lib/msa_rates is not built")
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--micro", "nonesuch"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "unknown measurement nonesuch" in r.stderr


def test_unique_kv_bytes_count_mxfp4_rows_at_68_bytes():
    # the bench's algorithmic bytes against a direct count: every distinct
    # (sequence, KV head, block) a valid pick reads, its keys below the used
    # length, times 2 (K and V) x the bytes of a row
    import numpy as np

    import workloads as W

    wl = W.make_custom(5, [1] * 6, [900, 2000, 700, 1500, 64, 129], 16, 2, 64, 6, causal=True)
    seen = set()
    for t in range(wl.Tq):
        s = int(np.searchsorted(wl.cu_seqlens_q, t, side="right") - 1)
        L = int(wl.used_kv_lens[s])
        pos = L - 1  # one token per sequence: the last position
        for g in range(wl.Hkv):
            for b in wl.selected[t, g]:
                b = int(b)
                if 0 <= b < (L + 127) // 128 and 128 * b <= pos:
                    seen.add((s, g, b, min(128, L - 128 * b)))
    keys = sum(n for (_, _, _, n) in seen)
    assert bench.accounting(wl)["unique_kv_bytes"] == keys * 2 * 128 * 2          # bf16 rows
    assert bench.accounting(W.to_mxfp4(wl))["unique_kv_bytes"] == keys * 2 * 68   # 64 code + 4 scale bytes
