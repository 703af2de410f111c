"""Pins of the oracle's dequant -> RoPE -> static int8 quantisation -> KV
cache operator (the blog on aclnnDequantRopeQuantKvcache: 计算步骤公式 steps
1-5, 两种 KV Cache 更新模式, 约束说明, and its call example)."""
import numpy as np
import pytest

import oracle
from oracle import DT_BF16, DT_FP16, DT_FP32, DT_INT32, INDEX_BATCH_START, INDEX_SLOT

import kvgen


# ---- fp16 rounding ---------------------------------------------------------------

def test_fp16_rounding_matches_numpy():
    rng = np.random.default_rng(0)
    # random binary32 patterns over the fp16 range, and the neighbours of every
    # fp16 midpoint (exact ties included)
    u = rng.integers(0, 0x47800000, 200000, dtype=np.uint32)
    v = u.view(np.float32)
    h = np.arange(0, 0x7C00, dtype=np.uint32).astype(np.uint16).view(np.float16).astype(np.float64)
    mids = ((h[:-1] + h[1:]) / 2).astype(np.float32)
    near = np.concatenate([mids, np.nextafter(mids, np.float32(0)), np.nextafter(mids, np.float32(1e9))])
    edge = np.array([65504, 65519.996, 65520, 65536, 1e9, 2.0 ** -24, 2.0 ** -25, 3 * 2.0 ** -26,
                     2.0 ** -14, 0.0], np.float32)
    vals = np.concatenate([v, near, edge])
    vals = np.concatenate([vals, -vals])
    with np.errstate(over="ignore"):
        want = vals.astype(np.float16).view(np.uint16)
    got = np.array([oracle.f32_to_fp16(float(f)) for f in vals], np.uint16)
    assert np.array_equal(got, want)


# ---- int8 quantisation ---------------------------------------------------------------

@pytest.mark.parametrize("v,scale,offset,want", [
    (2.5, 1.0, None, 2), (3.5, 1.0, None, 4), (-2.5, 1.0, None, -2), (-3.5, 1.0, None, -4),
    (127.5, 1.0, None, 127), (126.5, 1.0, None, 126), (-128.5, 1.0, None, -128),
    (-129.0, 1.0, None, -128), (1e6, 1.0, None, 127), (5.0, 2.0, 2.0, 4), (7.0, 2.0, 2.0, 6),
    (1.0, 3.0, None, 0), (2.0, 3.0, None, 1), (0.0, 1.0, -0.5, 0), (0.0, 1.0, 0.5, 0),
    (-0.0, 1.0, None, 0), (100.0, 0.5, -100.0, 100)])
def test_quant_int8_hand_worked(v, scale, offset, want):
    assert oracle.quant_int8(v, scale, offset) == want


# ---- whole operator -----------------------------------------------------------------

def _run(x, x_dtype, nq, nkv, D, cos, sin, out_dtype, *, T, Sc, Bc, index, index_mode, seq_len,
         prefill=0xAB, **kw):
    H = nkv * D
    geom = (Bc, Sc, H, Sc * H)
    k = np.full(Bc * Sc * H, prefill, np.uint8)
    v = np.full(Bc * Sc * H, prefill, np.uint8)
    q, ko, vo = oracle.drq(x, x_dtype, nq, nkv, D, cos, sin, out_dtype, scale_k=kw.pop("scale_k"),
                           scale_v=kw.pop("scale_v"), k_cache_bytes=k, v_cache_bytes=v,
                           cache_geom=geom, index=index, index_mode=index_mode, seq_len=seq_len,
                           **kw)
    return q, ko, vo, k.view(np.int8).reshape(Bc, Sc, H), v.view(np.int8).reshape(Bc, Sc, H)


def test_page_call_example():
    # the call example's inputs: B = S = 1, Nq = 2, Nkv = 1, D = 32 (H = 128),
    # int32 x all 1, fp16 cos / sin with bits 1 (2^-24), weight / activation /
    # bias / scales / offsets all 2.0, contiguous mode, indices [0], caches
    # [1, 128, 1, 32] prefilled with 6.
    nq, nkv, D = 2, 1, 32
    x = np.ones((1, 128), np.int32)
    cos = np.ones((1, D), np.uint16)
    two = lambda n: np.full(n, 2.0, np.float32)  # noqa: E731
    q, ko, vo, kc, vc = _run(x, DT_INT32, nq, nkv, D, cos, cos, DT_FP16, T=1, Sc=128, Bc=1,
                             index=np.array([0], np.int32), index_mode=INDEX_BATCH_START,
                             seq_len=1, prefill=6, weight_scale=two(128), act_scale=two(1),
                             bias=two(128), bias_dtype=DT_FP32, scale_k=two(32), scale_v=two(32),
                             offset_k=two(32), offset_v=two(32))
    # dequant: 1 * 2 * 2 + 2 = 6; RoPE: 6 c - 6 s = 0, 6 c + 6 s = 12 * 2^-24
    half = [0x0000] * 16 + [0x000C] * 16
    assert q.tolist() == [half * 2] and ko.tolist() == [half]
    assert vo.tolist() == [[0x4600] * 32]  # 6.0
    # k: 0 / 2 + 2 = 2 and 6 * 2^-24 + 2 -> 2; v: 6 / 2 + 2 = 5
    assert (kc[0, 0] == 2).all() and (vc[0, 0] == 5).all()
    assert (kc[0, 1:] == 6).all() and (vc[0, 1:] == 6).all()


@pytest.mark.parametrize("dt", [DT_BF16, DT_FP16])
def test_rope_closed_forms(dt):
    rng = np.random.default_rng(dt)
    nq, nkv, D, T = 2, 1, 64, 5
    H = (nq + 2 * nkv) * D
    to16 = kvgen.to_bf16 if dt == DT_BF16 else kvgen.to_fp16
    x = to16(rng.standard_normal((T, H)))
    ones, zeros = to16(np.ones((T, D))), to16(np.zeros((T, D)))
    kw = dict(T=T, Sc=8, Bc=1, index=np.arange(T, dtype=np.int32), index_mode=INDEX_SLOT,
              seq_len=0, scale_k=np.ones(nkv * D, np.float32), scale_v=np.ones(nkv * D, np.float32))
    # cos = 1, sin = 0: identity
    q, ko, vo, _, _ = _run(x, dt, nq, nkv, D, ones, zeros, dt, **kw)
    assert np.array_equal(q, x[:, :nq * D]) and np.array_equal(ko, x[:, nq * D:(nq + nkv) * D])
    assert np.array_equal(vo, x[:, (nq + nkv) * D:])
    # cos = 0, sin = 1: (a, b) -> (-b, a) per head half
    q, ko, _, _, _ = _run(x, dt, nq, nkv, D, zeros, ones, dt, **kw)
    for h in range(nq):
        a = x[:, h * D:h * D + D // 2]
        b = x[:, h * D + D // 2:(h + 1) * D]
        assert np.array_equal(q[:, h * D:h * D + D // 2], b ^ 0x8000)
        assert np.array_equal(q[:, h * D + D // 2:(h + 1) * D], a)


def test_dequant_exact_and_bias_dtypes_agree():
    # small int32 values with power-of-two weights are exact; a bias of small
    # integers is the same number in every bias dtype
    rng = np.random.default_rng(3)
    nq, nkv, D, T = 1, 1, 32, 4
    H = 3 * D
    x = rng.integers(-100, 100, (T, H)).astype(np.int32)
    w = (2.0 ** rng.integers(-3, 3, H)).astype(np.float32)
    act = (2.0 ** rng.integers(-2, 2, T)).astype(np.float32)
    bias = rng.integers(-4, 4, H)
    ones = kvgen.to_bf16(np.ones((T, D)))
    zeros = kvgen.to_bf16(np.zeros((T, D)))
    base = dict(T=T, Sc=4, Bc=1, index=np.arange(T, dtype=np.int32), index_mode=INDEX_SLOT,
                seq_len=0, scale_k=np.ones(D, np.float32), scale_v=np.ones(D, np.float32),
                weight_scale=w, act_scale=act)
    outs = []
    for bdt, b in ((DT_FP32, bias.astype(np.float32)), (DT_INT32, bias.astype(np.int32)),
                   (DT_BF16, kvgen.to_bf16(bias)), (DT_FP16, kvgen.to_fp16(bias))):
        outs.append(_run(x, DT_INT32, nq, nkv, D, ones, zeros, DT_BF16, bias=b, bias_dtype=bdt,
                         **base))
    for o in outs[1:]:
        for a, b in zip(outs[0], o):
            assert np.array_equal(a, b)
    want = x.astype(np.float64) * w[None, :] * act[:, None] + bias[None, :]
    got = np.concatenate([outs[0][0], outs[0][1], outs[0][2]], axis=1)
    # the binary32 dequantisation is exact here, so the output is its bf16 rounding
    assert np.array_equal(got, kvgen.to_bf16(want))
    # the v cache (scale 1): the bf16 values rounded half to even, saturated
    vb = kvgen.bf16_to_f32(kvgen.to_bf16(want[:, 2 * D:])).astype(np.float64)
    assert np.array_equal(outs[0][4][0, :T].astype(np.int64), np.clip(np.rint(vb), -128, 127))


def test_quant_dequant_bound():
    rng = np.random.default_rng(4)
    nq, nkv, D, T = 1, 2, 64, 16
    H = (nq + 2 * nkv) * D
    x = kvgen.to_fp16(rng.standard_normal((T, H)) * 4)
    sk = (rng.random(nkv * D) * 0.1 + 0.01).astype(np.float32)
    sv = (rng.random(nkv * D) * 0.1 + 0.01).astype(np.float32)
    ov = rng.integers(-5, 5, nkv * D).astype(np.float32)
    cos = kvgen.to_fp16(np.cos(rng.random((T, D))))
    sin = kvgen.to_fp16(np.sin(rng.random((T, D))))
    q, ko, vo, kc, vc = _run(x, DT_FP16, nq, nkv, D, cos, sin, DT_FP16, T=T, Sc=T, Bc=1,
                             index=np.arange(T, dtype=np.int32), index_mode=INDEX_SLOT, seq_len=0,
                             scale_k=sk, scale_v=sv, offset_v=ov)
    kf = ko.view(np.float16).astype(np.float64)
    vf = vo.view(np.float16).astype(np.float64)
    kq = kc[0].astype(np.float64)
    vq = vc[0].astype(np.float64)
    inr = np.abs(kf / sk) < 127
    assert np.all(np.abs(kq * sk - kf)[inr] <= 0.5 * np.broadcast_to(sk, kf.shape)[inr] * (1 + 1e-6))
    inr = np.abs(vf / sv + ov) < 127
    assert np.all(np.abs((vq - ov) * sv - vf)[inr] <= 0.5 * np.broadcast_to(sv, vf.shape)[inr] * (1 + 1e-6))


def test_contiguous_mode_equals_page_mode_on_expanded_rows():
    rng = np.random.default_rng(5)
    nq, nkv, D = 2, 1, 32
    B, S, Sc = 3, 5, 12
    T = B * S
    H = (nq + 2 * nkv) * D
    x = kvgen.to_bf16(rng.standard_normal((T, H)))
    cos = kvgen.to_bf16(rng.standard_normal((T, D)))
    sin = kvgen.to_bf16(rng.standard_normal((T, D)))
    kw = dict(T=T, Sc=Sc, Bc=B + 1, scale_k=np.full(D, 0.05, np.float32),
              scale_v=np.full(D, 0.07, np.float32))
    start = np.array([0, 7, -1], np.int32)  # the last batch skipped
    a = _run(x, DT_BF16, nq, nkv, D, cos, sin, DT_BF16, index=start,
             index_mode=INDEX_BATCH_START, seq_len=S, **kw)
    slots = np.array([b * Sc + start[b] + s if start[b] >= 0 else -1
                      for b in range(B) for s in range(S)], np.int32)
    e = _run(x, DT_BF16, nq, nkv, D, cos, sin, DT_BF16, index=slots, index_mode=INDEX_SLOT,
             seq_len=0, **kw)
    for u, w in zip(a, e):
        assert np.array_equal(u, w)


def test_rejects_mismatched_dtypes():
    x = np.zeros((1, 96), np.uint16)
    c = np.zeros((1, 32), np.uint16)
    kw = dict(T=1, Sc=1, Bc=1, index=np.zeros(1, np.int32), index_mode=INDEX_SLOT, seq_len=0,
              scale_k=np.ones(32, np.float32), scale_v=np.ones(32, np.float32))
    with pytest.raises(ValueError):  # 16-bit x must match the output dtype
        _run(x, DT_FP16, 1, 1, 32, c, c, DT_BF16, **kw)
    with pytest.raises(ValueError):  # int32 x needs weight_scale
        _run(x.astype(np.int32), DT_INT32, 1, 1, 32, c, c, DT_BF16, **kw)
