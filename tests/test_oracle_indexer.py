"""Pins of the oracle's indexer modes ("indexer_quant_cache", 接口功能 and 约束):
mxfp8 -- E4M3 codes of the whole row in groups of 32, one e8m0 scale per
group in cache_scale; fp8 -- E4M3 codes of the whole row as one group, one
FLOAT scale per row in cache_scale.

The codes are worked out by hand from the E4M3 definition (bias 7, three
mantissa bits, 448 the largest finite value) and the e8m0 rule (the smallest
power of two 2^E with amax <= 448 * 2^E)."""
import struct

import numpy as np

import kvgen
import oracle
from kvgen import CacheSpec, to_bf16

from test_oracle_epilog import check_workload, run_oracle


def _row(values, d):
    v = np.zeros(d)
    v[:len(values)] = values
    return to_bf16(v)


def test_mxfp8_hand_worked_groups():
    d = 96
    v = np.zeros(d)
    v[0:4] = [1.0, 3.0, -0.5, 0.0]        # group 0: amax 3 -> E = -7 (3 <= 3.5)
    v[64:67] = [448.0, 2.0 ** -9, 2.0 ** -10]  # group 2: amax 448 -> E = 0
    out, sc = oracle.quant_row(5, to_bf16(v), 32)
    assert list(sc) == [120, 0, 127]        # E + 127; an all-zero group gives 0
    # group 0 codes of v * 2^7: 128 -> 0x70, 384 -> 0x7C, -64 -> 0xE8, 0 -> 0x00
    assert list(out[0:4]) == [0x70, 0x7C, 0xE8, 0x00]
    assert not out[4:64].any()
    # group 2: 448 -> 0x7E, 2^-9 (smallest subnormal) -> 0x01, 2^-10 ties to 0
    assert list(out[64:67]) == [0x7E, 0x01, 0x00]


def test_mxfp8_scale_rounds_up_to_cover_amax():
    rng = np.random.default_rng(1)
    for _ in range(200):
        v = to_bf16(rng.standard_normal(32) * 2.0 ** rng.integers(-60, 60))
        out, sc = oracle.quant_row(5, v, 32)
        E = int(sc[0]) - 127
        amax = np.abs(kvgen.bf16_to_f32(v)).max()
        assert amax <= 448.0 * 2.0 ** E and amax > 448.0 * 2.0 ** (E - 1)


def test_fp8_row_power_of_two_scale():
    # amax 7 -> scale 7/448 = 2^-6 exactly; codes of v * 64
    v = _row([7.0, 1.0, -0.125, 0.0], 64)
    out, s = oracle.quant_row(6, v, 0)
    assert s[0] == np.float32(2.0 ** -6)
    assert list(out[0:4]) == [0x7E, 0x68, 0xD0, 0x00]
    assert not out[4:].any()


def test_fp8_row_unit_scale_is_plain_e4m3():
    rng = np.random.default_rng(2)
    x = rng.standard_normal(128) * 40
    x[0] = 448.0
    v = to_bf16(x)
    out, s = oracle.quant_row(6, v, 0)
    assert s[0] == np.float32(1.0)
    assert np.array_equal(out, oracle.enc_e4m3(kvgen.bf16_to_f32(v)))


def test_fp8_row_zero_row():
    out, s = oracle.quant_row(6, np.zeros(64, np.uint16), 0)
    assert s[0] == 0.0 and not out.any()


def test_fp8_row_scale_bytes_and_dequant_bound():
    rng = np.random.default_rng(3)
    for _ in range(100):
        x = to_bf16(rng.standard_normal(128) * 2.0 ** rng.integers(-30, 30))
        out, s = oracle.quant_row(6, x, 0)
        v = kvgen.bf16_to_f32(x).astype(np.float64)
        assert s[0] == np.float32(np.float32(np.abs(v).max()) / np.float32(448.0))
        # decode E4M3: |v - dec(q) * s| <= half a code step at |v / s| (2^-4 relative
        # above 2^-6, 2^-10 absolute below)
        code = out.astype(np.int64)
        e = (code >> 3) & 0xF
        m = code & 7
        mag = np.where(e == 0, m * 2.0 ** -9, (1 + m / 8.0) * 2.0 ** (e - 7))
        dec = np.where(code & 0x80, -mag, mag) * float(s[0])
        q = np.abs(v / float(s[0]))
        half = np.where(q >= 2.0 ** -6, 2.0 ** (np.floor(np.log2(np.maximum(q, 2.0 ** -6))) - 4),
                        2.0 ** -10) * float(s[0])
        assert np.all(np.abs(v - dec) <= half * (1 + 1e-6))


def test_indexer_routing():
    for mode, aux_head, elem in ((5, 4, 1), (6, 1, 4)):
        w = kvgen.make(f"ix{mode}", mode, 300, 128, seed=11 + mode,
                       cache=CacheSpec(16, 32, 128, 32 * 128 + 64),
                       aux=CacheSpec(16, 32, aux_head, 32 * aux_head + 3, elem),
                       row_sigma=1.5, skip_frac=0.05)
        check_workload(w)


def test_fp8_row_scale_written_as_float():
    w = kvgen.make("ix6", 6, 8, 64, seed=4, cache=CacheSpec(1, 8, 64, 8 * 64),
                   aux=CacheSpec(1, 8, 1, 8, 4))
    w.slots[:] = np.arange(8)
    cache, aux = run_oracle(w)
    for t in range(8):
        amax = np.abs(kvgen.bf16_to_f32(w.x[t])).max()
        assert aux[4 * t:4 * t + 4].tobytes() == struct.pack("<f", np.float32(amax) / np.float32(448))
