"""The C ABI without Python or torch: tests/c_client (plain C11, built by
__graft_entry__.build()) uploads a case with hipMalloc / hipMemcpy, runs it
through kvepi_run_ex and through a prepared call, and writes the caches
back; both must equal the oracle's bytes."""
import os
import struct
import subprocess

import numpy as np
import pytest

import kvgen
from kvgen import CacheSpec

from parity import run_oracle

pytestmark = pytest.mark.gpu

BIN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "c_client")


def _cases():
    fused = kvgen.make("c_fused", 0, 300, 576, seed=500, norm=True, rope=True, skip_frac=0.1,
                       cache=CacheSpec(5, 64, 672, 64 * 672 + 96))
    mxfp4 = kvgen.make("c_mxfp4", 3, 400, 128, seed=501, row_sigma=1.0, skip_frac=0.05,
                       cache=CacheSpec(4, 128, 64, 128 * 64), aux=CacheSpec(4, 128, 4, 128 * 4))
    split = kvgen.make("c_split", 4, 100, 576, seed=502, norm=True, rope=True,
                       cache=CacheSpec(30, 4, 512, 4 * 512 + 8, 2),
                       aux=CacheSpec(30, 4, 64, 4 * 64, 2))
    x16 = kvgen.fp16_rows(np.random.default_rng(503), 200, 256, row_sigma=1.0)
    fp8row = kvgen.make("c_fp8row", 6, 200, 256, seed=503, x=x16, skip_frac=0.05,
                        cache=CacheSpec(25, 9, 256, 9 * 256), aux=CacheSpec(25, 9, 1, 9, 4))
    fp8row.x_fp16 = True
    batch = kvgen.make("c_batch", 1, 6 * 30, 256, seed=504, cache=CacheSpec(7, 40, 336, 40 * 336))
    batch.slots = kvgen.index_array(np.random.default_rng(505), 1, 6, 30, 7, 40, 0.1)
    batch.index_mode, batch.seq_len = 1, 30
    return {w.name: w for w in (fused, mxfp4, split, fp8row, batch)}


CASES = _cases()


def _write_case(w, path):
    def put(name, a):
        if a is not None:
            np.ascontiguousarray(a).tofile(os.path.join(path, name))
    put("x.bin", w.x.astype(np.uint16))
    put("slots.bin", w.slots.astype(np.int32))
    put("gamma.bin", w.gamma)
    put("cos.bin", w.cos)
    put("sin.bin", w.sin)
    put("cache.bin", w.cache_init)
    put("aux.bin", w.aux_init)
    eps_bits = struct.unpack("<I", struct.pack("<f", w.eps))[0]
    keys = dict(T=w.T, d=w.d, x_stride=w.d, mode=w.mode, group=w.group_size, eps_bits=eps_bits,
                x_fp16=int(w.x_fp16), index_mode=w.index_mode, seq_len=w.seq_len,
                rope_dim=w.rope_dim if w.mode == kvgen.MODE_BF16_SPLIT else 0,
                c_num=w.cache.block_num, c_size=w.cache.block_size, c_head=w.cache.head_dim,
                c_stride=w.cache.block_stride)
    if w.aux is not None:
        keys.update(a_num=w.aux.block_num, a_size=w.aux.block_size, a_head=w.aux.head_dim,
                    a_stride=w.aux.block_stride)
    with open(os.path.join(path, "case.txt"), "w") as f:
        for k, v in keys.items():
            f.write(f"{k} {int(v)}\n")


@pytest.mark.parametrize("name", list(CASES))
def test_c_client_matches_oracle(name, tmp_path):
    assert os.path.exists(BIN), "tests/c_client is not built (run __graft_entry__.build())"
    w = CASES[name]
    _write_case(w, str(tmp_path))
    print(f"c_client case {name}: T={w.T} d={w.d} mode={w.mode}", flush=True)
    r = subprocess.run([BIN, str(tmp_path)], capture_output=True, text=True, timeout=60)
    print(r.stdout)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "c_client ok" in r.stdout
    want, awant = run_oracle(w)
    for tag in ("run", "prep"):
        got = np.fromfile(os.path.join(str(tmp_path), f"{tag}.bin"), np.uint8)
        assert np.array_equal(got, want), (name, tag)
        if awant is not None:
            agot = np.fromfile(os.path.join(str(tmp_path), f"{tag}_aux.bin"), np.uint8)
            assert np.array_equal(agot, awant), (name, tag, "aux")
