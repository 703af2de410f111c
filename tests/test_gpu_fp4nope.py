"""GPU parity of the FP4 nope mode (quantMode 2's nope segment of
"aclnnKvCompressEpilog", 计算公式 scene 3 and 约束说明) against the CPU oracle:
the whole cache allocation is compared byte for byte, so the 64 rope bytes of
every written row, which this mode leaves alone, are checked to keep their
prefill, as are unhit rows, block gaps and the bytes past kvCacheCol."""
import numpy as np
import pytest

import kvgen
from kvgen import CacheSpec, to_bf16

from parity import check, run_gpu

pytestmark = pytest.mark.gpu

MODE = kvgen.MODE_FP4_NOPE


def _w(T, d, g, *, seed, bs=16, head=None, stride_extra=0, norm=False, skip=0.1,
       row_sigma=1.5, x=None):
    import oracle
    _, kc, _ = oracle.row_bytes(MODE, d, g)
    head = head or kc
    nblk = (T + bs - 1) // bs + 2
    cache = CacheSpec(nblk, bs, head, bs * head + stride_extra)
    return kvgen.make(f"fp4nope_d{d}_g{g}", MODE, T, d, seed=seed, cache=cache, norm=norm,
                      skip_frac=skip, row_sigma=row_sigma, group_size=g, x=x)


def test_full_size_workload():
    w = kvgen.config(7)
    assert check(w, label="config 7 fp4_nope_d576") == 0


@pytest.mark.parametrize("g", [16, 32, 64])
@pytest.mark.parametrize("d", [128, 192, 320, 576, 1088, 4160, 8192])
@pytest.mark.parametrize("norm", [False, True])
def test_sweep(d, g, norm):
    T = 300 if d <= 1088 else 60
    w = _w(T, d, g, seed=d + g + norm, bs=7, stride_extra=32, norm=norm)
    assert check(w) == 0


@pytest.mark.parametrize("offset", [0, 1, 2, 4, 8])
@pytest.mark.parametrize("head_extra", [0, 3, 16])
def test_unaligned_rows(offset, head_extra):
    # cache bases and row pitches that are not 16-byte aligned take the
    # narrow-store path; padded pitches leave bytes past kvCacheCol alone
    import oracle
    kc = oracle.row_bytes(MODE, 576, 32)[1]
    w = _w(250, 576, 32, seed=31 + offset, bs=9, head=kc + head_extra, stride_extra=5,
           norm=True)
    assert check(w, offset=offset) == 0


def _special_rows(T, d, rng):
    """Rows built to reach every branch of the quantiser: all-zero groups
    (scale 0), tiny and huge magnitudes (outside the fast range), exact ties
    of v / s at E2M1 midpoints under a power-of-two scale, scales that round
    down so that v / s passes 6, and signed zeros."""
    x = np.zeros((T, d))
    n = d - 64
    for t in range(T):
        kind = t % 6
        if kind == 0:
            x[t, :n] = 0.0
            x[t, 1:n:7] = -0.0
        elif kind == 1:
            x[t, :n] = rng.standard_normal(n) * 2.0 ** -118  # below 2^-90
        elif kind == 2:
            x[t, :n] = rng.standard_normal(n) * 2.0 ** 110   # above 2^100
        elif kind == 3:
            # amax 3 in every group: s = 0.5, quotients on midpoints
            mids = np.array([0.125, 0.375, 0.625, 0.875, 1.25, 1.75, 2.5, 3.0])
            x[t, :n] = np.resize(mids, n) * np.where(rng.random(n) < 0.5, -1, 1)
            x[t, 0:n:16] = 3.0
        elif kind == 4:
            x[t, :n] = rng.uniform(-1.25, 1.25, n)
            x[t, 0:n:16] = 1.25      # 1.25 / 6 rounds down in bf16
        else:
            x[t, :n] = rng.standard_normal(n) * np.exp(rng.normal(0, 6, n))
        x[t, n:] = rng.standard_normal(64)
    return to_bf16(x)


@pytest.mark.parametrize("g", [16, 32, 64])
@pytest.mark.parametrize("norm", [False, True])
def test_special_values(g, norm):
    rng = np.random.default_rng(g)
    x = _special_rows(240, 576, rng)
    w = _w(240, 576, g, seed=40 + g, bs=8, norm=norm, skip=0.0, x=x)
    if norm:
        w.eps = 0.0 if g == 16 else 1e-6
    assert check(w) == 0


def test_many_iterations_per_wave(monkeypatch):
    monkeypatch.setenv("KVEPI_MAX_WAVES", "8")
    for norm in (False, True):
        w = _w(2000, 576, 32, seed=50 + norm, bs=13, stride_extra=16, norm=norm)
        assert check(w) == 0


def test_rope_and_fp16_are_rejected():
    import torch
    from kv_cache_epilog_amd import KvepiError, kvepi_run
    w = _w(8, 256, 16, seed=1)
    x = torch.zeros((8, 256), dtype=torch.bfloat16, device="cuda:0")
    slots = torch.arange(8, dtype=torch.int32, device="cuda:0")
    cache = torch.zeros((w.cache.block_num, w.cache.block_size, 1, w.cache.head_dim),
                        dtype=torch.uint8, device="cuda:0")
    cs = torch.zeros((8, 64), dtype=torch.bfloat16, device="cuda:0")
    with pytest.raises(KvepiError) as e:
        kvepi_run(x, slots, cache, MODE, 16, cos=cs, sin=cs)
    assert e.value.status == 4
    with pytest.raises(KvepiError) as e:
        kvepi_run(x.view(torch.float16), slots, cache, MODE, 16)
    assert e.value.status == 5
    torch.cuda.synchronize()
    assert int(cache.sum()) == 0
