"""Pins of the oracle's rope segment of any even length Dk in the bf16 split
mode ("aclnnKvRmsNormRopeCache", 计算公式 (1) with x = kv[..., Dv:], and the
shape notes: Dk + Dv = D, Dk even)."""
import numpy as np
import pytest

import kvgen
import oracle
from kvgen import CacheSpec, to_bf16


def test_rope_dk4_hand_worked():
    # x = [a0, b0, a1, b1] = [1, 2, 3, 4]: y[j] = a_j c_j - b_j s_j,
    # y[j + 2] = b_j c_{j+2} + a_j s_{j+2}
    x = to_bf16([1, 2, 3, 4])
    c = to_bf16([1, 0.5, 2, 0.25])
    s = to_bf16([0.5, 1, 0.125, 4])
    y = kvgen.bf16_to_f32(oracle.rope_row_n(x, c, s))
    assert y.tolist() == [0.0, -2.5, 4.125, 13.0]


def test_rope_dk64_is_the_fixed_segment():
    rng = np.random.default_rng(0)
    for _ in range(20):
        x, c, s = (to_bf16(rng.standard_normal(64)) for _ in range(3))
        assert np.array_equal(oracle.rope_row_n(x, c, s), oracle.rope_row(x, c, s))


@pytest.mark.parametrize("dk", [2, 6, 32, 128])
def test_split_mode_closed_forms(dk):
    # gamma = 1 on a constant nope row gives 1 (rms of a constant row is the
    # constant, up to eps); cos = 1, sin = 0 de-interleaves the rope segment
    d = 64 + dk
    T = 5
    rng = np.random.default_rng(dk)
    x = np.empty((T, d))
    x[:, :64] = 3.0
    x[:, 64:] = rng.standard_normal((T, dk))
    w = kvgen.make("gdk", kvgen.MODE_BF16_SPLIT, T, d, seed=dk,
                   cache=CacheSpec(2, 8, 64, 8 * 64, 2), aux=CacheSpec(2, 8, dk, 8 * dk, 2),
                   norm=True, rope=True, x=to_bf16(x), rope_dim=dk, eps=0.0)
    w.gamma = to_bf16(np.ones(64))
    w.cos = to_bf16(np.ones((T, dk)))
    w.sin = to_bf16(np.zeros((T, dk)))
    w.slots[:] = np.arange(T)
    cache = w.cache_init.copy()
    aux = w.aux_init.copy()
    oracle.epilog(w.mode, w.x, w.slots, cache, w.cache.geom, group_size=0, gamma=w.gamma,
                  cos=w.cos, sin=w.sin, eps=0.0, aux_bytes=aux, aux_geom=w.aux.geom,
                  rope_dim=dk)
    ckv = cache.view(np.uint16)[:T * 64].reshape(T, 64)
    k = aux.view(np.uint16)[:T * dk].reshape(T, dk)
    assert np.all(ckv == to_bf16(1.0))
    seg = w.x[:, 64:]
    assert np.array_equal(k, np.concatenate([seg[:, 0::2], seg[:, 1::2]], axis=1))


def test_rope_dim_rejections():
    x = np.zeros((1, 96), np.uint16)
    c = np.zeros(8 * 64 * 2, np.uint8)  # 8 rows of 64 bf16
    a = np.zeros(8 * 64, np.uint8)
    g = np.zeros(64, np.uint16)
    cs = np.zeros((1, 32), np.uint16)
    for mode, d, dk in ((kvgen.MODE_BF16_SPLIT, 96, 31), (kvgen.MODE_BF16_SPLIT, 96, 34),
                        (kvgen.MODE_FP8_E8M0, 128, 32)):
        with pytest.raises(ValueError):
            oracle.epilog(mode, np.zeros((1, d), np.uint16), np.zeros(1, np.int32), c,
                          (1, 8, 64, 512), group_size=64, gamma=g, cos=cs, sin=cs,
                          aux_bytes=a, aux_geom=(1, 8, 32, 256), rope_dim=dk)
