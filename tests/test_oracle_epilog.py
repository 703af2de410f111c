"""Pins of the oracle's routing and row assembly.

- Every hit token's row lands at the paged address restated independently in
  kvgen.CacheSpec.row_offset: block slot // blockSize at the block stride,
  row slot % blockSize at headDim ("aclnnKvCompressEpilog" 约束说明).
- Exactly kvCacheCol bytes are written per row; the bytes of skipped (-1)
  tokens' rows, of rows no token hits, of the gaps between loosely laid-out
  blocks and past kvCacheCol keep their prefill ("indexer_quant_cache" 语义说明:
  rows not hit keep their values).
- The fused row equals the separate steps composed through their bf16
  outputs, and repeated runs are bit-identical (the pages state the operators
  are deterministic).
"""
import numpy as np
import pytest

import kvgen
import oracle
from kvgen import CacheSpec


def run_oracle(w):
    cache = w.cache_init.copy()
    aux = None if w.aux_init is None else w.aux_init.copy()
    oracle.epilog(w.mode, w.x, w.slots, cache, w.cache.geom, group_size=w.group_size,
                  gamma=w.gamma, cos=w.cos, sin=w.sin, eps=w.eps, aux_bytes=aux,
                  aux_geom=None if w.aux is None else w.aux.geom)
    return cache, aux


def expected_rows(w, t):
    """Row bytes for token t from the per-row steps."""
    x = w.x[t]
    if w.mode in (kvgen.MODE_MXFP4, kvgen.MODE_MXFP8):
        return oracle.quant_row(w.mode, x, w.group_size)
    if w.mode == kvgen.MODE_FP8_ROW:
        out, s = oracle.quant_row(w.mode, x, w.group_size)
        return out, s.view(np.uint8)
    nope = w.d - 64
    v = x.copy()
    if w.gamma is not None:
        v[:nope] = oracle.rmsnorm_row(x[:nope], w.gamma, w.eps)
    if w.cos is not None:
        v[nope:] = oracle.rope_row(x[nope:], w.cos[t], w.sin[t])
    if w.mode == kvgen.MODE_BF16_SPLIT:
        return v[:nope].view(np.uint8), v[nope:].view(np.uint8)
    return oracle.quant_row(w.mode, v, w.group_size)


def check_workload(w):
    cache, aux = run_oracle(w)
    touched = np.zeros(cache.size, bool)
    touched_aux = None if aux is None else np.zeros(aux.size, bool)
    for t in range(w.T):
        s = int(w.slots[t])
        if s < 0 or s >= w.cache.num_slots:
            continue
        row, arow = expected_rows(w, t)
        off = w.cache.row_offset(s)
        assert np.array_equal(cache[off:off + row.size], row), t
        touched[off:off + row.size] = True
        if arow is not None:
            aoff = w.aux.row_offset(s)
            assert np.array_equal(aux[aoff:aoff + arow.size], arow), t
            touched_aux[aoff:aoff + arow.size] = True
    assert np.all(cache[~touched] == kvgen.PREFILL)
    if aux is not None:
        assert np.all(aux[~touched_aux] == kvgen.PREFILL)
    return cache, aux


def small(mode, T, d, *, seed, cache, aux=None, **kw):
    return kvgen.make(f"small_{mode}_{d}", mode, T, d, seed=seed, cache=cache, aux=aux, **kw)


def test_config0_routing():
    check_workload(kvgen.config(0))


def test_config1_routing():
    check_workload(kvgen.config(1))


def test_mode1_odd_head_dim_323():
    # the page example d=256, quantMode=1: 323-byte rows packed at headDim 323
    w = small(1, 100, 256, seed=5, cache=CacheSpec(4, 32, 323, 32 * 323), skip_frac=0.1)
    check_workload(w)


def test_mode0_loose_blocks_and_wide_rows():
    # block stride larger than blockSize*headDim, headDim > kvCacheCol
    w = small(0, 200, 576, seed=6, cache=CacheSpec(8, 32, 700, 32 * 700 + 96),
              norm=True, rope=True, skip_frac=0.2)
    check_workload(w)


def test_mxfp4_routing():
    w = small(3, 300, 128, seed=7, cache=CacheSpec(16, 32, 64, 32 * 64 + 64),
              aux=CacheSpec(16, 32, 4, 32 * 4), skip_frac=0.05)
    check_workload(w)


def test_out_of_range_and_all_skipped():
    w = small(1, 64, 256, seed=8, cache=CacheSpec(4, 16, 336, 16 * 336))
    w.slots[:] = -1
    cache, _ = run_oracle(w)
    assert np.all(cache == kvgen.PREFILL)
    w.slots[:] = np.arange(64) + 64  # every slot >= num_slots (64): skipped
    cache, _ = run_oracle(w)
    assert np.all(cache == kvgen.PREFILL)
    w.slots[:] = np.where(np.arange(64) % 2 == 0, np.arange(64), -5 - np.arange(64))
    check_workload(w)


def test_fused_equals_composed_steps_bytes():
    # fused norm+rope+quant == quantise(bf16 RMSNorm output ++ bf16 RoPE output)
    w = small(0, 50, 576, seed=9, cache=CacheSpec(4, 16, 672, 16 * 672), norm=True,
              rope=True)
    cache, _ = run_oracle(w)
    w2 = small(0, 50, 576, seed=9, cache=CacheSpec(4, 16, 672, 16 * 672), norm=True,
               rope=True)
    nope = 512
    x2 = w2.x.copy()
    for t in range(w2.T):
        x2[t, :nope] = oracle.rmsnorm_row(w2.x[t, :nope], w2.gamma, w2.eps)
        x2[t, nope:] = oracle.rope_row(w2.x[t, nope:], w2.cos[t], w2.sin[t])
    w2.x, w2.gamma, w2.cos, w2.sin = x2, None, None, None
    cache2, _ = run_oracle(w2)
    assert np.array_equal(cache, cache2)


def test_deterministic():
    w = kvgen.config(0)
    a, _ = run_oracle(w)
    b, _ = run_oracle(w)
    assert np.array_equal(a, b)


def test_strided_x_rows():
    w = small(1, 40, 256, seed=10, cache=CacheSpec(4, 16, 336, 16 * 336))
    big = np.zeros((40, 320), np.uint16)
    big[:, :256] = w.x
    c1, _ = run_oracle(w)
    w.x = big[:, :256]
    c2, _ = run_oracle(w)
    assert np.array_equal(c1, c2)


@pytest.mark.parametrize("mode", [1, 3])
def test_rejects_bad_args(mode):
    w = small(mode, 8, 128, seed=1, cache=CacheSpec(1, 16, 64, 16 * 64),
              aux=CacheSpec(1, 16, 4, 64) if mode == 3 else None)
    with pytest.raises(ValueError):
        oracle.epilog(mode, w.x, w.slots, w.cache_init.copy(), w.cache.geom,
                      group_size=16, aux_bytes=None if w.aux is None else w.aux_init.copy(),
                      aux_geom=None if w.aux is None else w.aux.geom)


@pytest.mark.parametrize("mode,d,group,head,aux_head,ok", [
    (7, 576, 16, 384, None, True), (7, 576, 16, 383, None, False),  # kvCacheCol 384
    (0, 576, 64, 672, None, True), (0, 576, 64, 656, None, False),  # 656 -> 672 with padding
    (3, 128, 32, 64, 4, True), (3, 128, 32, 63, 4, False), (3, 128, 32, 64, 3, False),
])
def test_rejects_rows_wider_than_the_cache(mode, d, group, head, aux_head, ok):
    # headDim >= kvCacheCol ("aclnnKvCompressEpilog", 约束说明; "indexer_quant_cache",
    # 约束): a narrower cache is refused, never written past its rows
    aux = None if aux_head is None else CacheSpec(4, 16, aux_head, 16 * aux_head)
    w = small(mode, 20, d, seed=2, cache=CacheSpec(4, 16, head, 16 * head), aux=aux,
              group_size=group)
    args = (mode, w.x, w.slots, w.cache_init.copy(), w.cache.geom)
    kw = dict(group_size=group, aux_bytes=None if aux is None else w.aux_init.copy(),
              aux_geom=None if aux is None else aux.geom)
    if ok:
        oracle.epilog(*args, **kw)
    else:
        with pytest.raises(ValueError):
            oracle.epilog(*args, **kw)
