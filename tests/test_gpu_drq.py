"""GPU parity of the dequant -> RoPE -> static int8 quantisation -> KV cache
operator (through its C ABI) against the oracle: every output value and
every cache byte (untouched rows and gaps included) must be equal."""
import numpy as np
import pytest

import oracle
from drq_case import compare, make_case

pytestmark = pytest.mark.gpu

I32, BF, FP, F32 = oracle.DT_INT32, oracle.DT_BF16, oracle.DT_FP16, oracle.DT_FP32


@pytest.mark.parametrize("out", [BF, FP])
@pytest.mark.parametrize("bias", [None, F32, I32, BF, FP])
def test_int32_dequant(out, bias):
    c = make_case(100 + out * 10 + (bias or 0), T=300, nq=4, nkv=2, D=64, x_dtype=I32,
                  out_dtype=out, bias_dtype=bias)
    compare(c, "int32 dequant")


@pytest.mark.parametrize("out", [BF, FP])
@pytest.mark.parametrize("act,offsets,kv_output", [(False, False, True), (True, False, False),
                                                    (False, True, False)])
def test_int32_options(out, act, offsets, kv_output):
    c = make_case(200 + out, T=257, nq=2, nkv=1, D=128, x_dtype=I32, out_dtype=out,
                  bias_dtype=F32, act=act, offsets=offsets, kv_output=kv_output)
    compare(c, "int32 options")


@pytest.mark.parametrize("out", [BF, FP])
@pytest.mark.parametrize("nq,nkv,D", [(8, 8, 16), (2, 1, 32), (30, 1, 128), (2, 1, 16)])
def test_int32_head_shapes(out, nq, nkv, D):
    # int32 rows at the smallest head (D = 16: a unit is the whole head, and
    # heads of 16 make H = 64 with three or 24 heads), a small one, and the
    # largest row (H = 4096)
    c = make_case(250 + D + nq, T=150, nq=nq, nkv=nkv, D=D, x_dtype=I32, out_dtype=out,
                  bias_dtype=BF, act=True, offsets=True)
    compare(c, "int32 head shapes")


@pytest.mark.parametrize("dt", [BF, FP])
@pytest.mark.parametrize("nq,nkv,D", [(12, 3, 128), (2, 1, 32), (1, 1, 64), (8, 8, 16),
                                      (30, 1, 128)])
def test_16bit_activations(dt, nq, nkv, D):
    c = make_case(300 + D + nq, T=200, nq=nq, nkv=nkv, D=D, x_dtype=dt, out_dtype=dt)
    compare(c, "16-bit x")


def test_atk_shapes():
    # the operator's two end-to-end cases: fp16 x [1, 2304] (Nq*D 1536, Nkv*D
    # 384) and int32 x [1, 3584] (splits 1792 / 896 / 896, bf16 bias), page mode
    compare(make_case(1, T=1, nq=12, nkv=3, D=128, x_dtype=FP, out_dtype=FP, skip=0.0), "atk0")
    compare(make_case(2, T=1, nq=14, nkv=7, D=128, x_dtype=I32, out_dtype=BF, bias_dtype=BF,
                      skip=0.0), "atk1")


@pytest.mark.parametrize("bs,stride_extra,head", [(16, 0, None), (7, 24, None), (128, 8, 264),
                                                  (1, 0, None)])
def test_page_layouts(bs, stride_extra, head):
    c = make_case(400 + bs, T=500, nq=2, nkv=2, D=64, x_dtype=BF, out_dtype=BF, bs=bs,
                  stride_extra=stride_extra, head=head, skip=0.1)
    compare(c, "page layout")


@pytest.mark.parametrize("B,S,bs", [(4, 50, 64), (7, 13, 13), (1, 128, 200), (16, 1, 4)])
def test_contiguous_mode(B, S, bs):
    c = make_case(500 + B * S, T=B * S, nq=2, nkv=1, D=128, x_dtype=I32, out_dtype=FP,
                  bias_dtype=FP, cache_mode=1, seq_len=S, bs=bs)
    compare(c, "contiguous")


def test_padded_x_rows():
    c = make_case(600, T=100, nq=4, nkv=2, D=64, x_dtype=I32, out_dtype=BF, bias_dtype=I32,
                  x_pad=40)
    compare(c, "padded x")


def test_large_token_count():
    c = make_case(700, T=20000, nq=4, nkv=1, D=128, x_dtype=FP, out_dtype=FP, bs=128)
    compare(c, "T=20000")


def test_saturation_and_ties():
    # k / v values far beyond the int8 range and exact .5 quotients
    c = make_case(800, T=64, nq=1, nkv=1, D=64, x_dtype=BF, out_dtype=BF, skip=0.0)
    c.scale_k[:] = 0.01
    c.scale_v[:] = 0.5
    x = c.x.copy()
    # v heads: multiples of 0.25 -> quotients at .5 ties for scale 0.5
    v = np.round(np.random.default_rng(9).standard_normal((64, 64)) * 40) / 4
    x[:, 2 * 64:] = oracle_bits(v)
    c.x = x
    compare(c, "saturation")


def oracle_bits(v):
    import kvgen
    return kvgen.to_bf16(v)


@pytest.mark.parametrize("case", ["tiny_values", "tiny_scales", "huge_values", "huge_scales"])
def test_division_paths(case):
    # waves whose values or scales leave the range of the fast division take
    # IEEE division; both must give the oracle's codes
    c = make_case(900, T=256, nq=1, nkv=1, D=64, x_dtype=BF, out_dtype=BF, skip=0.0)
    rng = np.random.default_rng(10)
    x = c.x.copy()
    if case == "tiny_values":
        x[::3, 64:] = oracle_bits(rng.standard_normal((len(x[::3]), 128)) * 1e-12)
        c.scale_k[:] = 1e-13
        c.scale_v[:] = 1e-13
    elif case == "tiny_scales":
        c.scale_k[::5] = 1e-32
        c.scale_v[::7] = 3e-33
    elif case == "huge_values":
        x[::4, 64:] = oracle_bits(rng.standard_normal((len(x[::4]), 128)) * 1e25)
    else:
        c.scale_k[::3] = 1e31
        c.scale_v[::2] = 5e30
    c.x = x
    compare(c, case)


def test_duplicate_slot_check(monkeypatch):
    # KVEPI_CHECK_SLOTS in page mode: distinct slots pass the check and match
    # the oracle; a repeated slot is rejected with KVEPI_ERR_PARAM
    from kv_cache_epilog_amd.binding import KvepiError
    from drq_case import run_gpu
    monkeypatch.setenv("KVEPI_CHECK_SLOTS", "1")
    c = make_case(1000, T=64, nq=2, nkv=1, D=64, x_dtype=BF, out_dtype=BF, skip=0.1)
    compare(c, "distinct slots under the check")
    hit = np.nonzero(c.index >= 0)[0]
    c.index[hit[-1]] = c.index[hit[0]]
    with pytest.raises(KvepiError) as e:
        run_gpu(c)
    assert e.value.status == 4  # KVEPI_ERR_PARAM


def _drq_fuzz_case(k):
    """A seeded random case: x / output dtypes, head dim and head counts
    (H <= 4096, H % 64 == 0), bias dtype, activation scales, offsets, k / v
    outputs, page or contiguous mode, block size, head padding, block stride,
    skipped tokens and padded x rows."""
    rng = np.random.default_rng(9000 + k)
    xt = int(rng.choice([I32, BF, FP]))
    out = int(rng.choice([BF, FP])) if xt == I32 else xt
    while True:
        D = 16 * int(rng.integers(1, 17))
        nkv, nq = int(rng.integers(1, 9)), int(rng.integers(1, 33))
        H = (nq + 2 * nkv) * D
        if H % 64 == 0 and H <= 4096:
            break
    kw = dict(kv_output=bool(rng.random() < 0.5), x_pad=int(rng.choice([0, 0, 8, 32])),
              offsets=bool(rng.random() < 0.7), head=nkv * D + int(rng.choice([0, 0, 16, 32])),
              stride_extra=int(rng.choice([0, 0, 8, 64])))
    if xt == I32:
        kw["bias_dtype"] = [None, F32, I32, BF, FP][int(rng.integers(0, 5))]
        kw["act"] = bool(rng.random() < 0.7)
    if rng.random() < 0.3:
        S, B = int(rng.integers(1, 65)), int(rng.integers(1, 9))
        kw.update(cache_mode=1, seq_len=S, bs=S + int(rng.integers(0, 20)))
        T = B * S
    else:
        T = int(rng.choice([1, 2, 17, 64, int(rng.integers(1, 800))]))
        kw.update(bs=int(rng.choice([1, 3, 16, 128, int(rng.integers(1, 100))])),
                  skip=float(rng.choice([0.0, 0.05, 0.5])))
    return make_case(9000 + k, T=T, nq=nq, nkv=nkv, D=D, x_dtype=xt, out_dtype=out, **kw)


@pytest.mark.parametrize("k", range(80))
def test_fuzz(k):
    compare(_drq_fuzz_case(k), f"fuzz {k}")


# int32 x runs in persistent blocks that keep the per-channel parameters in
# LDS and load each thread's next unit before storing the current one; a grid
# capped at 1 or 3 blocks makes every thread run many units, through the
# pipeline's whole cycle (first unit, steady state, a last unit with nothing
# after it), on rows of every shape class
_MANY = [
    dict(T=300, nq=4, nkv=2, D=64, bias_dtype=F32, act=True, offsets=True),
    dict(T=257, nq=2, nkv=1, D=128, bias_dtype=BF, offsets=False, skip=0.3),
    dict(T=150, nq=30, nkv=1, D=128, bias_dtype=I32, offsets=True),
    dict(T=1000, nq=8, nkv=8, D=16, bias_dtype=None, act=False, kv_output=False),
    dict(T=7 * 13, nq=2, nkv=1, D=128, bias_dtype=FP, cache_mode=1, seq_len=13, bs=13),
    dict(T=64, nq=1, nkv=1, D=64, bias_dtype=FP, x_pad=40, skip=0.0),
]


@pytest.mark.parametrize("blocks", [1, 3])
@pytest.mark.parametrize("k", range(len(_MANY)))
@pytest.mark.parametrize("out", [BF, FP])
def test_int32_many_units_per_thread(monkeypatch, blocks, k, out):
    monkeypatch.setenv("KVEPI_DRQ_MAX_BLOCKS", str(blocks))
    c = make_case(1100 + 10 * k + out, x_dtype=I32, out_dtype=out, **_MANY[k])
    compare(c, f"int32, {blocks} blocks, case {k}")


def test_params_keep_their_tensors():
    # run_gpu passes temporaries (cos, sin, indices, scales, ...) straight
    # into drq_params; the params hold them, so freeing torch's cached blocks
    # back to the device before the launch (as a graph capture does) leaves
    # the launch's inputs allocated
    import torch
    from drq_case import run_gpu, run_oracle
    c = make_case(1200, T=200, nq=4, nkv=2, D=64, x_dtype=I32, out_dtype=BF, bias_dtype=F32)
    got = run_gpu(c, before_run=lambda: (__import__("gc").collect(), torch.cuda.empty_cache()))
    want = run_oracle(c)
    for g, w in zip(got, want):
        assert (g is None and w is None) or np.array_equal(g, w)
