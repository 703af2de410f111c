"""GPU parity (through the C ABI's _ex entry points) of the options: fp16
rows in the indexer modes and the index modes that place batch-major tokens
(per-batch rows, one block per chunk of tokens, per-batch start).  Every
test compares whole cache allocations byte for byte with the oracle."""
import numpy as np
import pytest

import kvgen
import oracle
from kvgen import CacheSpec

from parity import check, token_slots

pytestmark = pytest.mark.gpu


def _caches(mode, d, bn, bs, stride_extra=0, head=None):
    group = {3: 32, 5: 32, 6: 0}.get(mode, 64)
    _, kc, sc = oracle.row_bytes(mode, d, group) if mode != 4 else (0, d - 64, 64)
    head = head or kc
    cache = CacheSpec(bn, bs, head, bs * head + stride_extra, 2 if mode == 4 else 1)
    aux = None
    if mode in (3, 5):
        aux = CacheSpec(bn, bs, sc, bs * sc + stride_extra)
    elif mode == 6:
        aux = CacheSpec(bn, bs, 1, bs + stride_extra, 4)
    elif mode == 4:
        aux = CacheSpec(bn, bs, 64, bs * 64 + stride_extra, 2)
    return cache, aux


def _fp16_workload(mode, T, d, seed, x16, bs=3, stride_extra=5, skip=0.05):
    cache, aux = _caches(mode, d, (T + bs - 1) // bs + 2, bs, stride_extra)
    w = kvgen.make(f"f16_m{mode}_d{d}", mode, T, d, seed=seed, cache=cache, aux=aux,
                   skip_frac=skip, x=x16)
    w.x_fp16 = True
    return w


# ---- fp16 rows --------------------------------------------------------------------

@pytest.mark.parametrize("mode", [3, 5, 6])
@pytest.mark.parametrize("d", [32, 96, 128, 512, 2048, 8192])
def test_fp16_indexer_sweep(mode, d):
    T = 300 if d <= 512 else 60
    rng = np.random.default_rng(d + mode)
    w = _fp16_workload(mode, T, d, d + mode, kvgen.fp16_rows(rng, T, d, row_sigma=3.0))
    assert check(w) == 0


@pytest.mark.parametrize("mode", [3, 5, 6])
def test_fp16_special_values(mode):
    rng = np.random.default_rng(40 + mode)
    d, T = 128, 64
    x = rng.standard_normal((T, d))
    x[0] = 0.0
    x[1] = -0.0
    x[2] = rng.standard_normal(d) * 2.0 ** -20          # fp16 subnormals
    x[3] = rng.integers(-3, 4, d) * 2.0 ** -24           # the smallest subnormals
    x[4] = np.clip(rng.standard_normal(d) * 3e4, -65504, 65504)
    x[5, ::3] = 65504.0
    x[6] = np.where(rng.random(d) < 0.5, -0.0, 0.0)
    x[7] = np.round(rng.standard_normal(d) * 16) / 32     # exact ties
    x[8, 7] = 2.0 ** -24                                  # one subnormal in a zero row
    x[9] = 1 + rng.integers(0, 1024, d) * 2.0 ** -10      # 11-bit significands
    w = _fp16_workload(mode, T, d, 41, kvgen.to_fp16(x), skip=0.0)
    assert check(w) == 0


@pytest.mark.parametrize("mode", [3, 5])
def test_fp16_scale_exponent_sweep(mode):
    # groups of 32 whose amax walks every fp16 exponent, with code midpoints
    rng = np.random.default_rng(50 + mode)
    d, T = 128, 400
    vmax = 6.0 if mode == 3 else 448.0
    mids = ([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0] if mode == 3 else
            [2.0 ** -10, 3 * 2.0 ** -10, 1.0625, 1.1875, 9.5, 13.5, 17.0, 240.0, 416.0])
    x = np.zeros((T, d))
    gi = 0
    for r in range(T):
        for g in range(d // 32):
            k = -24 - int(np.log2(vmax)) + gi % 40  # amax from 2^-24 up to fp16 max
            gi += 1
            v = np.clip(rng.standard_normal(32) * vmax / 3, -vmax, vmax)
            v[0] = vmax
            v[1:9] = rng.choice(mids, 8) * np.where(rng.random(8) < 0.5, -1.0, 1.0)
            rng.shuffle(v)
            x[r, 32 * g:32 * g + 32] = np.clip(v * 2.0 ** k, -65504, 65504)
    w = _fp16_workload(mode, T, d, 51, kvgen.to_fp16(x), skip=0.0)
    assert check(w) == 0


# ---- index modes ------------------------------------------------------------------

def _indexed(mode, d, index_mode, B, S, bs, bn, seed, norm=False, rope=False, skip=0.1,
             stride_extra=16, x16=False):
    cache, aux = _caches(mode, d, bn, bs, stride_extra)
    T = B * S
    x = None
    if x16:
        x = kvgen.fp16_rows(np.random.default_rng(seed), T, d, row_sigma=1.0)
    w = kvgen.make(f"ix{index_mode}_m{mode}", mode, T, d, seed=seed, cache=cache, aux=aux,
                   norm=norm, rope=rope, row_sigma=1.0, x=x)
    rng = np.random.default_rng(seed + 1000)
    idx = kvgen.index_array(rng, index_mode, B, S, bn, bs, skip)
    if idx.size > 3:
        # values that would leave the cache (or the batch's rows) skip the token
        idx[2] = bs if index_mode != 2 else bn * bs
    w.slots = idx
    w.index_mode = index_mode
    w.seq_len = S
    w.x_fp16 = x16
    return w


CASES = [
    # (quant mode, d, norm, rope)
    (0, 576, True, True), (1, 256, False, False), (3, 128, False, False),
    (4, 576, True, True), (6, 128, False, False),
]


@pytest.mark.parametrize("case", CASES, ids=[f"m{c[0]}_d{c[1]}" for c in CASES])
@pytest.mark.parametrize("index_mode,B,S,bs", [
    (1, 9, 50, 64), (1, 3, 7, 7), (2, 5, 100, 16), (2, 4, 37, 10), (3, 6, 40, 48),
    (3, 2, 13, 13)])
def test_index_modes(case, index_mode, B, S, bs):
    mode, d, norm, rope = case
    nc = -(-S // bs)
    bn = B * nc + 3 if index_mode == 2 else B + 2
    w = _indexed(mode, d, index_mode, B, S, bs, bn, seed=B * 100 + S + mode, norm=norm,
                 rope=rope)
    assert (token_slots(w) >= 0).sum() > 0
    check(w)


@pytest.mark.parametrize("index_mode", [1, 2, 3])
@pytest.mark.parametrize("waves", [4, 64])
def test_index_modes_many_iterations_per_wave(index_mode, waves, monkeypatch):
    monkeypatch.setenv("KVEPI_MAX_WAVES", str(waves))
    B, S, bs = 16, 120, 128 if index_mode != 2 else 32
    bn = B * (-(-S // bs)) + 5 if index_mode == 2 else B + 1
    w = _indexed(0, 576, index_mode, B, S, bs, bn, seed=60 + index_mode, norm=True, rope=True)
    check(w)


def test_fp16_with_block_index():
    w = _indexed(5, 256, 2, 6, 45, 8, 6 * 6 + 2, seed=70, x16=True)
    assert check(w) == 0


# ---- rope segments of other lengths in the bf16 split mode ------------------------------

@pytest.mark.parametrize("dk,dv", [(2, 64), (6, 64), (32, 544), (128, 512), (96, 512),
                                   (10, 1024), (64, 512), (40, 8), (126, 200)])
def test_split_rope_lengths(dk, dv):
    d = dv + dk
    T, bs = 300, 7
    nblk = (T + bs - 1) // bs + 2
    cache = CacheSpec(nblk, bs, dv, bs * dv + 8, 2)
    aux = CacheSpec(nblk, bs, dk, bs * dk + 2, 2)
    w = kvgen.make(f"split_dk{dk}", 4, T, d, seed=dk + dv, cache=cache, aux=aux, norm=True,
                   rope=True, row_sigma=1.0, skip_frac=0.1, rope_dim=dk)
    # rows of x start 16-byte aligned: a d that is not a multiple of 8 takes
    # padded rows (a row stride above d)
    check(w, x_pad=(-d) % 8)


@pytest.mark.parametrize("waves", [4, 64])
def test_split_rope_length_many_iterations(waves, monkeypatch):
    monkeypatch.setenv("KVEPI_MAX_WAVES", str(waves))
    dk, dv, T, bs = 32, 512, 2001, 16
    nblk = (T + bs - 1) // bs + 2
    w = kvgen.make("split_dk32_it", 4, T, dv + dk, seed=77, cache=CacheSpec(nblk, bs, dv, bs * dv, 2),
                   aux=CacheSpec(nblk, bs, dk, bs * dk, 2), norm=True, rope=True, rope_dim=dk)
    check(w)


def test_split_rope_length_with_block_index():
    dk, dv = 48, 256
    B, S, bs = 4, 37, 8
    nc = -(-S // bs)
    bn = B * nc + 2
    w = kvgen.make("split_dk48_blk", 4, B * S, dv + dk, seed=78,
                   cache=CacheSpec(bn, bs, dv, bs * dv, 2), aux=CacheSpec(bn, bs, dk, bs * dk, 2),
                   norm=True, rope=True, rope_dim=dk)
    w.slots = kvgen.index_array(np.random.default_rng(79), 2, B, S, bn, bs, 0.1)
    w.index_mode = 2
    w.seq_len = S
    check(w)


@pytest.mark.parametrize("dk", [32, 10])
def test_split_rope_length_underflowing_products(dk):
    # the general rope length with every pair a case where rounding each
    # product on its own (the definition) and a fused multiply-add give
    # different bf16 outputs (tiny values times small cos / sin)
    from parity import plant_rope_cases
    dv, T, bs = 512, 32, 8
    d = dv + dk
    nblk = (T + bs - 1) // bs + 2
    w = kvgen.make(f"split_dk{dk}_uf", 4, T, d, seed=91 + dk,
                   cache=CacheSpec(nblk, bs, dv, bs * dv, 2),
                   aux=CacheSpec(nblk, bs, dk, bs * dk, 2), norm=True, rope=True, rope_dim=dk)
    assert plant_rope_cases(w, np.random.default_rng(dk), dk) == T * dk // 2
    check(w, x_pad=(-d) % 8)


def _index_fuzz_case(k):
    """A seeded random workload in one of the batch-major index modes: mode,
    row width, RMSNorm / RoPE, index mode, batches, sequence length, block
    size and count, skip density, fp16 rows (indexer modes)."""
    rng = np.random.default_rng(11000 + k)
    mode = int(rng.choice([0, 1, 3, 4, 5, 6]))
    d = 64 * int(rng.integers(2, 41)) if mode in (0, 1, 4) else 32 * int(rng.integers(1, 81))
    norm = mode == 4 or (mode in (0, 1) and bool(rng.random() < 0.5))
    rope = mode == 4 or (mode in (0, 1) and bool(rng.random() < 0.5))
    index_mode = int(rng.integers(1, 4))
    B, S = int(rng.integers(1, 13)), int(rng.integers(1, 160))
    if index_mode == 2:
        bs = int(rng.integers(1, 64))
        bn = B * (-(-S // bs)) + int(rng.integers(0, 4))
    else:
        bs = S + int(rng.integers(0, 40))
        bn = B + int(rng.integers(0, 4))
    x16 = mode in (3, 5, 6) and bool(rng.random() < 0.3)
    return _indexed(mode, d, index_mode, B, S, bs, bn, seed=11000 + k, norm=norm, rope=rope,
                    skip=float(rng.choice([0.0, 0.1, 0.5])),
                    stride_extra=int(rng.choice([0, 16, 40])), x16=x16)


@pytest.mark.parametrize("k", range(60))
def test_index_fuzz(k):
    check(_index_fuzz_case(k), f"index fuzz {k}")


def _rope_length_fuzz_case(k):
    """A seeded random bf16-split workload with a rope segment of random even
    length Dk (2..128) and a nope width Dv (a multiple of 8), random block
    layout, skips and RMSNorm spread."""
    rng = np.random.default_rng(13000 + k)
    dk = 2 * int(rng.integers(1, 65))
    dv = 8 * int(rng.integers(1, 200))
    if dk == 64:  # the 64-column segment takes the standard layout: d % 64 == 0
        dv = 64 * int(rng.integers(1, 25))
    d = dv + dk
    T, bs = int(rng.choice([1, 7, 64, int(rng.integers(1, 600))])), int(rng.integers(1, 40))
    nblk = (T + bs - 1) // bs + 2
    w = kvgen.make(f"rl{k}_dk{dk}_dv{dv}", 4, T, d, seed=13000 + k,
                   cache=CacheSpec(nblk, bs, dv, bs * dv + 8 * int(rng.integers(0, 3)), 2),
                   aux=CacheSpec(nblk, bs, dk, bs * dk + 2 * int(rng.integers(0, 5)), 2),
                   norm=True, rope=True, row_sigma=float(rng.choice([0.0, 2.0])),
                   skip_frac=float(rng.choice([0.0, 0.1])), rope_dim=dk)
    return w, (-d) % 8 + 8 * int(rng.integers(0, 3))


@pytest.mark.parametrize("k", range(30))
def test_rope_length_fuzz(k):
    w, x_pad = _rope_length_fuzz_case(k)
    check(w, f"rope length fuzz {k}", x_pad=x_pad)
