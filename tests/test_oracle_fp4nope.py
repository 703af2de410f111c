"""Pins of the oracle's FP4 nope mode: the nope half of quantMode 2 of
"aclnnKvCompressEpilog" (计算公式 scene 3; 约束说明: quantGroupSize 16, 32 or
64 dividing d - 64, x bf16, concatCol = 64 + (d-64)/2 + ((d-64)/G)*2 padded
to 32 bytes).  The rope bytes of that mode are HiFloat8 codes, a format the
pages do not define, so this mode leaves the row's first 64 bytes untouched.

Readings checked here (the pages fix the formula, not these details): the
2-byte scale is bf16 (the page's other group mode stores "bf16 scale" and x
is bf16); the codes divide by the scale as stored; the fields follow the
formula's term order (rope | codes | scales | zero pad); element 2j sits in
the low nibble.  The codes below are worked out by hand from the E2M1
definition (magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6 as codes 0-7, sign in bit
3, nearest with ties to the even code, saturating at 6)."""
import numpy as np
import pytest

import kvgen
import oracle
from kvgen import CacheSpec, bf16_to_f32, to_bf16

from test_oracle_epilog import check_workload, run_oracle, small
from test_oracle_formats import e2m1_table

MODE = kvgen.MODE_FP4_NOPE


def test_hand_worked_row():
    # d = 128: 64 nope values in four groups of 16
    v = np.zeros(128)
    # group 0: amax 1 -> 1/6 = 0x3E2AAAAB in fp32 -> bf16 0x3E2B (rounds up)
    #   = 0.1669921875; 1/s = 5.988 -> 6 (code 7), 0.5/s = 2.994 -> 3 (5),
    #   0.25/s = 1.497 -> 1.5 (3), -1 -> 0xF
    v[0:4] = [1.0, 0.5, 0.25, -1.0]
    # group 1: amax 3 -> s = 0.5 exactly; the quotients 6, 0.25, 0.75, 2.5,
    #   5, -0.75, -0.25 give 7, ties 0 / 2 / 4 / 6 (even codes), 0xA, 0x8
    v[16:23] = [3.0, 0.125, 0.375, 1.25, 2.5, -0.375, -0.125]
    # group 2: amax 1.25 -> 1.25/6 = 0x3E555555 -> bf16 0x3E55 (rounds down)
    #   = 0.2080078125; 1.25/s = 6.009 saturates to 6 (7); 0.6 is bf16
    #   0.6015625, / s = 2.892 -> 3 (5)
    v[32:35] = [1.25, -1.25, 0.6]
    # group 3: all zero -> scale 0, codes 0
    out, none = oracle.quant_row(MODE, to_bf16(v), 16)
    assert none is None
    assert out.size == 128 - 64  # the bytes written: codes, scales, pad
    codes = list(out[:32])
    assert codes[0:2] == [0x57, 0xF3] and not any(codes[2:8])
    assert codes[8:12] == [0x07, 0x42, 0xA6, 0x08] and not any(codes[12:16])
    assert codes[16:18] == [0xF7, 0x05] and not any(codes[18:32])
    assert list(out[32:40]) == [0x2B, 0x3E, 0x00, 0x3F, 0x55, 0x3E, 0x00, 0x00]
    assert not out[40:].any()  # 104 -> 128: zero pad


def test_rope_columns_do_not_enter():
    rng = np.random.default_rng(3)
    v = to_bf16(rng.standard_normal(576))
    w = v.copy()
    w[512:] = to_bf16(rng.standard_normal(64) * 1e4)
    assert np.array_equal(oracle.quant_row(MODE, v, 32)[0], oracle.quant_row(MODE, w, 32)[0])


@pytest.mark.parametrize("g", [16, 32, 64])
def test_codes_are_nearest_under_the_stored_scale(g):
    # every code decodes to the E2M1 value nearest to v / s (ties to the even
    # code), s the stored bf16 scale of the group, and |v| / s never passes
    # 6 * (1 + 2^-7): a bf16 scale is within half a bf16 ulp of amax / 6
    mags = e2m1_table()  # code 0-7 -> magnitude
    rng = np.random.default_rng(g)
    for trial in range(20):
        v = to_bf16(rng.standard_normal(576) * np.exp(rng.normal(0, 3)))
        out, _ = oracle.quant_row(MODE, v, g)
        vf = bf16_to_f32(v[:512]).astype(np.float64)
        nib = np.empty(512, np.uint8)
        nib[0::2] = out[:256] & 0xF
        nib[1::2] = out[:256] >> 4
        sb = out[256:256 + 2 * (512 // g)].view(np.uint16)
        s = bf16_to_f32(sb).astype(np.float64)
        for k in range(512 // g):
            grp = vf[k * g:(k + 1) * g]
            assert s[k] == bf16_to_f32(to_bf16(np.float32(np.max(np.abs(grp))) / np.float32(6)))
            if s[k] == 0:
                assert not nib[k * g:(k + 1) * g].any()
                continue
            q = grp / s[k]  # exact in binary64 for bf16 / bf16
            assert np.max(np.abs(q)) <= 6 * (1 + 2.0 ** -7)
            for qi, ci in zip(q, nib[k * g:(k + 1) * g]):
                err = np.abs(mags - min(abs(qi), 6.0))
                best = np.flatnonzero(err == err.min())
                assert (ci & 7) in best, (qi, ci)
                if len(best) == 2:  # a tie: the even code
                    assert ci & 1 == 0
                if qi != 0:
                    assert (ci >> 3) == (qi < 0)


def test_routing_and_untouched_rope_bytes():
    # rows land at the paged address; bytes 0-63 of each hit row, unhit rows,
    # skipped tokens' rows and block gaps keep the prefill
    for norm in (False, True):
        w = small(MODE, 96, 256, seed=31 + norm, cache=CacheSpec(5, 24, 200, 24 * 200 + 48),
                  norm=norm, skip_frac=0.1, group_size=16, row_sigma=1.0)
        cache, _ = run_oracle(w)
        touched = np.zeros(cache.size, bool)
        for t in range(w.T):
            s = int(w.slots[t])
            if s < 0:
                continue
            v = w.x[t].copy()
            if norm:
                v[:192] = oracle.rmsnorm_row(w.x[t][:192], w.gamma, w.eps)
            row, _ = oracle.quant_row(MODE, v, 16)
            off = w.cache.row_offset(s)
            assert np.array_equal(cache[off + 64:off + 192], row), t
            touched[off + 64:off + 192] = True
        assert np.all(cache[~touched] == kvgen.PREFILL)


def test_rejections():
    w = small(MODE, 8, 256, seed=1, cache=CacheSpec(2, 8, 192, 8 * 192), group_size=16,
              rope=True)
    with pytest.raises(ValueError):  # the rope segment is not written: no RoPE
        run_oracle(w)
    for g in (8, 128, 0):
        with pytest.raises(ValueError):
            oracle.row_bytes(MODE, 256, g)
    with pytest.raises(ValueError):  # x must be bf16
        oracle.quant_row(MODE, np.zeros(256, np.uint16), 32, x_fp16=True)
    with pytest.raises(ValueError):  # quantMode 2 itself: HiFloat8 is not defined
        oracle.row_bytes(2, 576, 32)


def test_full_size_config_routing_sample():
    # the bench workload's first tokens through the whole-epilog routing
    w = kvgen.config(7)
    assert w.group_size == 32 and oracle.row_bytes(MODE, 576, 32) == (352, 352, 16)
    assert w.cache.head_dim == 352 and w.cache.block_stride == 128 * 352 * 5 // 4
