"""Host-side checks of bench.py (no GPU): the algorithmic byte counts that
the effective bandwidth is computed from, and the one-GPU guard.

The byte counts follow the row sizes of "aclnnKvCompressEpilog" (约束说明:
kvCacheCol = (d - 64) + 128 + scale bytes, padded to 32 in mode 0) and of
indexer_quant_cache (MX-FP4 rows of d/2 bytes plus d/32 scale bytes): per
hit row the x row (and cos / sin rows when RoPE is on) is read and the
cache row written; every token reads its 4-byte slot; gamma is read once.
The expected totals below are that sum written out by hand for each
workload, not a call of the function under test."""
import os
import subprocess
import sys
from pathlib import Path

import pytest

ROOT = Path(__file__).resolve().parents[1]
sys.path.insert(0, str(ROOT))

import bench  # noqa: E402
import kvgen  # noqa: E402


def _hand_count(T, hits, read_row, write_row, gamma_bytes=0):
    return 4 * T + hits * (read_row + write_row) + gamma_bytes


@pytest.mark.parametrize("cfg, expected", [
    # mode-1 prefill d = 576: x row 1152 B, cache row (576-64)+128+8 = 648 B
    (2, _hand_count(16384, 16056, 1152, 648)),
    # MX-FP4 indexer d = 128: x row 256 B, 64 code bytes + 4 e8m0 scale bytes
    (3, _hand_count(131072, 129761, 256, 64 + 4)),
    # fused d = 576: x 1152 B + cos 128 B + sin 128 B, 672-byte cache row,
    # gamma of 512 bf16 values
    (4, _hand_count(262144, 254280, 1152 + 256, 672, 2 * 512)),
])
def test_algorithmic_bytes(cfg, expected):
    w = kvgen.config(cfg)
    assert bench.algorithmic_bytes(w) == expected


def test_published_totals():
    # the same totals as plain numbers (bytes per launch)
    assert _hand_count(16384, 16056, 1152, 648) == 28_966_336
    assert _hand_count(131072, 129761, 256, 68) == 42_566_852
    assert _hand_count(262144, 254280, 1408, 672, 1024) == 529_952_000


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, str(ROOT / "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, cwd=ROOT, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr or "1 GPU" in r.stderr or "--gpus 1" in r.stderr


def test_traffic_needs_matching_source():
    # measured traffic is reported only for the kernel source it was taken on
    assert bench.measured_traffic("no_such_workload") is None


def test_dense_count_adds_skipped_rows():
    w = kvgen.config(3)
    skipped = w.T - w.hits
    assert bench.algorithmic_bytes(w, dense=True) - bench.algorithmic_bytes(w) == skipped * 256


def test_pinned_restores_affinity():
    before = os.sched_getaffinity(0)
    with bench._pinned() as p:
        assert os.sched_getaffinity(0) == {p.core}
    assert os.sched_getaffinity(0) == before


def test_host_info():
    n, model = bench.host_info()
    assert n >= 1 and isinstance(model, str) and model


def test_code_hash_ignores_comments_only():
    a = "int f(int x) {\n  return x + 1;  // one more\n}\n"
    b = "/* a function */\nint f(int x) {\n  // the next value\n  return x   +   1;\n}\n"
    c = "int f(int x) {\n  return x + 2;  // one more\n}\n"
    assert bench.code_text(a) == bench.code_text(b)
    assert bench.code_text(a) != bench.code_text(c)


def test_algorithmic_split_by_hand():
    # fused d = 576: reads are the slots, x + cos + sin of every hit row and
    # gamma; writes are the 672-byte rows
    w = kvgen.config(4)
    r, wr = bench.algorithmic_split(w)
    assert r == 4 * 262144 + 254280 * 1408 + 1024
    assert wr == 254280 * 672
    assert r + wr == bench.algorithmic_bytes(w)
    # MX-FP4 indexer: 64 code bytes and a 4-byte scale row written per hit
    w = kvgen.config(3)
    assert bench.algorithmic_split(w) == (4 * 131072 + 129761 * 256, 129761 * 68)


def test_fp4_nope_bytes_by_hand():
    # quantMode 2's nope segment: the 512 nope values of x are read (the rope
    # columns are neither read nor written), gamma once, and 352 - 64 = 288
    # bytes (256 code bytes, 16 bf16 scales) written per hit row
    w = kvgen.config(7)
    hits = int(((w.slots >= 0) & (w.slots < w.cache.num_slots)).sum())
    assert bench.algorithmic_split(w) == (4 * 262144 + hits * 1024 + 1024, hits * 288)


def test_ceiling_mix_follows_the_workload():
    # the streaming mix closest (in log ratio) to the workload's read:write
    assert bench.mix_of(1408, 672) == (2, 1)
    assert bench.mix_of(1152, 648) == (2, 1)
    assert bench.mix_of(256, 68) == (4, 1)
    assert bench.mix_of(100, 100) == (1, 1)


def test_metric_is_named_for_the_workload():
    assert bench.metric_name(kvgen.config(4)) == bench.METRIC
    assert bench.metric_name(kvgen.config(3)).endswith("mxfp4_indexer_d128")
