"""Pins of the oracle's fp16 rows ("indexer_quant_cache" 接口功能: float16 or
bfloat16 activations) and of its index modes ("aclnnKvRmsNormRopeCache",
index constraints: Norm, PA_BNSD, PA_BLK_BNSD; the blog on
aclnnDequantRopeQuantKvcache, cache modes: contiguous)."""
import numpy as np
import pytest

import kvgen
import oracle
from kvgen import CacheSpec, to_bf16


# ---- fp16 rows ----------------------------------------------------------------

def test_fp16_decode_matches_numpy_for_every_pattern():
    h = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    want = h.view(np.float16).astype(np.float32)
    got = np.array([oracle.fp16_to_f32(int(v)) for v in h], np.float32)
    nan = np.isnan(want)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan].view(np.uint32), want[~nan].view(np.uint32))


def _f16(values, d):
    v = np.zeros(d, np.float16)
    v[:len(values)] = values
    return v.view(np.uint16)


def test_fp16_mxfp8_hand_worked():
    # 1 + 2^-10 (not a bf16 value): amax <= 448 * 2^-8 = 1.75, > 448 * 2^-9;
    # v * 2^8 = 256.25 -> 256 = 0x78
    out, sc = oracle.quant_row(5, _f16([1 + 2.0 ** -10], 32), 32, x_fp16=True)
    assert sc[0] == 127 - 8 and out[0] == 0x78 and not out[1:].any()
    # the fp16 maximum 65504: E = 8 (146.2 <= 256), 65504 / 256 = 255.875 -> 256
    out, sc = oracle.quant_row(5, _f16([65504.0, -65504.0], 32), 32, x_fp16=True)
    assert sc[0] == 127 + 8 and list(out[:2]) == [0x78, 0xF8]
    # the smallest fp16 subnormal 2^-24: E = -32 (1.75 * 2^-24 >= 2^-24), code of 2^8
    out, sc = oracle.quant_row(5, _f16([2.0 ** -24], 32), 32, x_fp16=True)
    assert sc[0] == 127 - 32 and out[0] == 0x78


def test_fp16_mxfp4_hand_worked():
    # amax 3 + 3 * 2^-10: E = 0 would need amax <= 6: E = 0; v / 1 -> 3 (code 5)
    # 0.25 + 2^-12 is just above the 0 / 0.5 midpoint -> 0.5 (code 1)
    out, sc = oracle.quant_row(3, _f16([3 + 3 * 2.0 ** -10, 0.25 + 2.0 ** -12], 32), 32,
                               x_fp16=True)
    assert sc[0] == 127 and out[0] == (0x5 | (0x1 << 4))


def test_fp16_rows_equal_bf16_rows_when_values_fit_both():
    # values with at most 8 significant bits inside the fp16 range are the
    # same number in both formats: the codes and scales must not change
    rng = np.random.default_rng(5)
    for mode, g in ((3, 32), (5, 32), (6, 0)):
        for _ in range(50):
            m = rng.integers(-255, 256, 128).astype(np.float64)
            v = m * 2.0 ** rng.integers(-20, 7)
            b = to_bf16(v)
            h = v.astype(np.float16).view(np.uint16)
            assert np.array_equal(h.view(np.float16).astype(np.float64), v)
            ob, sb = oracle.quant_row(mode, b, g)
            oh, sh = oracle.quant_row(mode, h, g, x_fp16=True)
            assert np.array_equal(ob, oh) and np.array_equal(sb, sh)


def test_fp16_fp8_row_scale_is_amax_over_448():
    rng = np.random.default_rng(6)
    for _ in range(100):
        h = (rng.standard_normal(256) * 2.0 ** rng.integers(-10, 10)).astype(np.float16)
        out, s = oracle.quant_row(6, h.view(np.uint16), 0, x_fp16=True)
        amax = np.float32(np.abs(h.astype(np.float32)).max())
        assert s[0] == amax / np.float32(448.0)


def test_fp16_rejected_outside_indexer_modes():
    with pytest.raises(ValueError):
        oracle.quant_row(0, np.zeros(256, np.uint16), 64, x_fp16=True)


# ---- index modes ------------------------------------------------------------------

def _slots(mode, index, T, S, bn, bs):
    return [oracle.token_slot(mode, np.asarray(index, np.int32), t, S, bn, bs) for t in range(T)]


def test_batch_index_hand_worked():
    # B = 2, S = 3, cache [2, 4]: row index[b, s] of batch b; -1 and 4 skip
    idx = [0, 2, -1, 3, 0, 4]
    assert _slots(1, idx, 6, 3, 2, 4) == [0, 2, -1, 7, 4, -1]


def test_block_index_hand_worked():
    # B = 2, S = 5, block_size 2 -> 3 chunks per batch; cache of 5 blocks
    idx = [4, 0, -1, 7, 2, 9]
    assert _slots(2, idx, 10, 5, 5, 2) == [4, 5, 0, 1, -1, 6, 7, 2, 3, 8]


def test_batch_start_hand_worked():
    # B = 2, S = 3, cache [2, 5]: rows start .. start + 2; past the batch's rows skip
    assert _slots(3, [1, 3], 6, 3, 2, 5) == [1, 2, 3, 8, 9, -1]
    assert _slots(3, [-1, 0], 6, 3, 2, 5) == [-1, -1, -1, 5, 6, 7]


def _run(w, index, index_mode, seq_len):
    cache = w.cache_init.copy()
    aux = None if w.aux_init is None else w.aux_init.copy()
    oracle.epilog(w.mode, w.x, index, cache, w.cache.geom, group_size=w.group_size,
                  gamma=w.gamma, cos=w.cos, sin=w.sin, eps=w.eps, aux_bytes=aux,
                  aux_geom=None if w.aux is None else w.aux.geom, index_mode=index_mode,
                  seq_len=seq_len)
    return cache, aux


@pytest.mark.parametrize("mode", [0, 3, 4])
def test_block_index_equals_expanded_slots(mode):
    # the per-block index equals the per-token slot mode on the slots it
    # implies (the expansion written out here, independently of kvo_token_slot)
    B, S, bs, bn = 3, 37, 8, 20
    T = B * S
    d = 128 if mode == 3 else 576
    _, kc, sc = oracle.row_bytes(mode, d, 32 if mode == 3 else 64) if mode != 4 else (0, d - 64, 64)
    cache = CacheSpec(bn, bs, kc, bs * kc + 16, 2 if mode == 4 else 1)
    aux = None
    if mode == 3:
        aux = CacheSpec(bn, bs, sc, bs * sc + 3)
    elif mode == 4:
        aux = CacheSpec(bn, bs, 64, bs * 64, 2)
    w = kvgen.make("idx", mode, T, d, seed=mode, cache=cache, aux=aux, norm=mode in (0, 4),
                   rope=mode in (0, 4))
    rng = np.random.default_rng(mode)
    # BLOCK: one entry per chunk of bs tokens, naming distinct blocks (not
    # always at their first row), one chunk skipped
    nb_chunk = -(-S // bs)
    blk = rng.permutation(bn)[:B * nb_chunk]
    bidx = (blk * bs + rng.integers(0, bs, blk.size)).astype(np.int32)
    bidx[1] = -1
    expanded = np.full(T, -1, np.int32)
    for b in range(B):
        for s in range(S):
            v = bidx[b * nb_chunk + s // bs]
            if v >= 0:
                expanded[b * S + s] = (v // bs) * bs + s % bs
    a = _run(w, bidx, 2, S)
    e = _run(w, expanded, 0, 0)
    assert np.array_equal(a[0], e[0]) and (a[1] is None or np.array_equal(a[1], e[1]))


@pytest.mark.parametrize("mode", [1, 5, 6])
def test_batch_modes_equal_expanded_slots(mode):
    # the per-batch index and the per-batch start, expanded by hand
    B, S, Sc = 4, 10, 16
    T = B * S
    d = 128 if mode in (5, 6) else 256
    g = {5: 32, 6: 0}.get(mode, 64)
    _, kc, sc = oracle.row_bytes(mode, d, g)
    cache = CacheSpec(B + 1, Sc, kc, Sc * kc + 8)
    aux = None
    if mode == 5:
        aux = CacheSpec(B + 1, Sc, sc, Sc * sc)
    elif mode == 6:
        aux = CacheSpec(B + 1, Sc, 1, Sc, 4)
    w = kvgen.make("bidx", mode, T, d, seed=10 + mode, cache=cache, aux=aux, row_sigma=1.0)
    rng = np.random.default_rng(mode)
    # BATCH: a permutation of a batch's rows per batch, some -1 and one past Sc
    idx = np.concatenate([rng.permutation(Sc)[:S] for _ in range(B)]).astype(np.int32)
    idx[3] = -1
    idx[12] = Sc
    exp = np.array([b * Sc + idx[b * S + s] if 0 <= idx[b * S + s] < Sc else -1
                    for b in range(B) for s in range(S)], np.int32)
    a = _run(w, idx, 1, S)
    e = _run(w, exp, 0, 0)
    assert np.array_equal(a[0], e[0]) and (a[1] is None or np.array_equal(a[1], e[1]))
    # BATCH_START equals BATCH with index[b, s] = start_b + s
    start = np.array([0, 6, -1, 3], np.int32)
    per_tok = np.array([start[b] + s if start[b] >= 0 else -1 for b in range(B) for s in range(S)],
                       np.int32)
    a = _run(w, start, 3, S)
    e = _run(w, per_tok, 1, S)
    assert np.array_equal(a[0], e[0]) and (a[1] is None or np.array_equal(a[1], e[1]))
