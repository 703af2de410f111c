"""Pins of the oracle's per-row steps.

RMSNorm and RoPE ("aclnnKvRmsNormRopeCache" 计算公式 (1), (2)) are checked
against binary64 evaluations of the printed formulas on random rows (within
half a bf16 ulp plus the binary32 rounding the oracle performs), against their
closed-form special cases, and against the exact power-of-two scaling
invariance of RMSNorm.  The quantiser ("aclnnKvCompressEpilog" 计算公式 and
约束说明, "indexer_quant_cache" mxfp4) is checked on hand-worked rows, on the
page's row-size example, and on the dequantisation error bound.
"""
import os

import numpy as np
import pytest

import oracle
from kvgen import bf16_to_f32, to_bf16

from test_oracle_formats import e2m1_table, e4m3_table

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
EPS32 = float(np.float32(1e-6))


def bf16_ulp(y64):
    """Spacing of bf16 values at |y| (normal range)."""
    a = np.abs(y64)
    e = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    return 2.0 ** (e - 7)


def assert_close_bf16(got_bf16, y64, slack=2.0 ** -12):
    got = bf16_to_f32(got_bf16).astype(np.float64)
    err = np.abs(got - y64) / bf16_ulp(y64)
    assert np.all(err <= 0.5 + slack), float(err.max())


# ---- row geometry -----------------------------------------------------------

def _row_bytes_fixture():
    rows = []
    with open(os.path.join(GOLDEN, "row_bytes.txt")) as f:
        for line in f:
            line = line.split("#")[0].strip()
            if line:
                p = line.split()
                rows.append(tuple(int(v) for v in p[:6]) + (p[6],))
    return rows


@pytest.mark.parametrize("row", _row_bytes_fixture())
def test_row_bytes_golden(row):
    mode, d, g, cc, kc, sc, _kind = row
    assert oracle.row_bytes(mode, d, g) == (cc, kc, sc)


def test_quant_row_length_matches_page_example():
    # d=256, quantMode=1: the row written is exactly 323 bytes long.
    v = to_bf16(np.random.default_rng(0).standard_normal(256))
    out, _ = oracle.quant_row(1, v, 64)
    assert out.size == 323


@pytest.mark.parametrize("mode,d,g", [(0, 320, 64), (1, 100, 64), (1, 8256, 64),
                                      (1, 64, 64), (0, 256, 32), (3, 48, 32), (3, 128, 64),
                                      (2, 256, 64)])
def test_row_bytes_rejects(mode, d, g):
    if (mode, d, g) == (0, 320, 64):
        oracle.row_bytes(mode, d, g)  # valid: d % 64 == 0, 64 < d <= 8192
        return
    with pytest.raises(ValueError):
        oracle.row_bytes(mode, d, g)


# ---- RMSNorm ----------------------------------------------------------------

@pytest.mark.parametrize("n", [64, 192, 448, 512, 1000, 2048, 8128])
def test_rmsnorm_vs_binary64(n):
    rng = np.random.default_rng(n)
    for trial in range(8):
        scale = 10.0 ** rng.uniform(-3, 3)
        x = to_bf16(rng.standard_normal(n) * scale)
        g = to_bf16(rng.uniform(0.5, 1.5, n))
        y = oracle.rmsnorm_row(x, g, 1e-6)
        xf = bf16_to_f32(x).astype(np.float64)
        gf = bf16_to_f32(g).astype(np.float64)
        y64 = xf / np.sqrt(np.mean(xf * xf) + EPS32) * gf
        assert_close_bf16(y, y64)


def test_rmsnorm_constant_row_is_sign():
    for c in (0.75, -3.0, 1.0e-2, 200.0):
        x = to_bf16(np.full(512, c))
        y = oracle.rmsnorm_row(x, to_bf16(np.ones(512)), 0.0)
        assert np.all(bf16_to_f32(y) == np.sign(c))


def test_rmsnorm_power_of_two_invariance():
    rng = np.random.default_rng(7)
    x = to_bf16(rng.standard_normal(512))
    g = to_bf16(rng.uniform(0.5, 1.5, 512))
    y0 = oracle.rmsnorm_row(x, g, 0.0)
    for k in (-20, -3, 1, 5, 30):
        xk = to_bf16(bf16_to_f32(x).astype(np.float64) * 2.0 ** k)
        assert np.array_equal(oracle.rmsnorm_row(xk, g, 0.0), y0)


def test_rmsnorm_eps_matters():
    x = to_bf16(np.full(64, 1e-3))
    y = oracle.rmsnorm_row(x, to_bf16(np.ones(64)), 1e-6)
    y64 = 1e-3 / np.sqrt(bf16_to_f32(x)[0].astype(np.float64) ** 2 + EPS32)
    y64 = bf16_to_f32(x).astype(np.float64) / np.sqrt(
        bf16_to_f32(x).astype(np.float64)[0] ** 2 + EPS32)
    assert_close_bf16(y, y64)
    assert bf16_to_f32(y)[0] < 0.8  # eps (1e-6) dominates x^2 (1e-6 too)


def test_sumsq_tree_error_bound():
    rng = np.random.default_rng(11)
    for n in (64, 192, 512, 1000, 8128):
        x = to_bf16(rng.standard_normal(n) * 3)
        xf = bf16_to_f32(x).astype(np.float64)
        exact = float(np.sum(xf * xf))
        got = oracle.sumsq_tree(x)
        depth = int(np.ceil(np.log2(n)))
        assert abs(got - exact) <= depth * 2.0 ** -24 * exact * 1.01


# The summation order of the sum of squares.  The reading is a balanced
# pairwise tree over the index order, zero-padded at the end to the next power
# of two.  The sums below are written here from that description, independently
# of the oracle's code, together with the orders a plausible slip would give:
# a running sum, first-level pairs taken a half apart (i with i + p/2), and the
# zero padding placed in front.  The rows are chosen so that each of those
# orders gives a different fp32 sum from the reading's tree, so the oracle
# matches the tree and none of the others.

def _squares32(x_bf16):
    v = bf16_to_f32(x_bf16)
    return (v * v).astype(np.float32)  # one fp32 rounding (exact for normal bf16)


def _pad(sq, front=False):
    p = 1
    while p < sq.size:
        p *= 2
    z = np.zeros(p - sq.size, np.float32)
    return np.concatenate([z, sq] if front else [sq, z]).astype(np.float32)


def _tree_recursive(a):
    """Sum of a (a power-of-two length) as left half + right half, recursively,
    every addition in fp32."""
    if a.size == 1:
        return np.float32(a[0])
    h = a.size // 2
    return np.float32(_tree_recursive(a[:h]) + _tree_recursive(a[h:]))


def _tree_adjacent(a):
    while a.size > 1:
        a = (a[0::2] + a[1::2]).astype(np.float32)
    return np.float32(a[0])


def _tree_strided(a):
    while a.size > 1:
        h = a.size // 2
        a = (a[:h] + a[h:]).astype(np.float32)
    return np.float32(a[0])


def _running(sq):
    s = np.float32(0.0)
    for v in sq:
        s = np.float32(s + v)
    return s


def _order_rows(n, seed):
    """Seeded bf16 rows of length n with squares spread over many binades (so
    that the order of the additions shows), each of which separates the tree
    from every wrong order that differs from it at this length."""
    rng = np.random.default_rng(seed)
    found = []
    for _ in range(400):
        mag = np.exp(rng.normal(0.0, 2.5, n))
        x = to_bf16(rng.choice([-1.0, 1.0], n) * mag)
        sq = _squares32(x)
        tree = _tree_adjacent(_pad(sq))
        wrong = [_running(sq), _tree_strided(_pad(sq))]
        if n & (n - 1):
            wrong.append(_tree_adjacent(_pad(sq, front=True)))
        if all(w != tree for w in wrong):
            found.append((x, tree))
            if len(found) == 3:
                return found
    raise AssertionError(f"no separating row found for n = {n}")


def test_sumsq_tree_written_two_ways_agree():
    rng = np.random.default_rng(5)
    for n in (8, 448, 512, 576):
        a = _pad(_squares32(to_bf16(np.exp(rng.normal(0, 2.5, n)))))
        assert _tree_recursive(a) == _tree_adjacent(a)


@pytest.mark.parametrize("n,seed", [(448, 21), (512, 22)])
def test_sumsq_tree_order_is_pinned(n, seed):
    # 448 and 512 are nope lengths of the epilog's rows (d = 512 and 576)
    for x, tree in _order_rows(n, seed):
        got = np.float32(oracle.sumsq_tree(x))
        assert got == tree
        assert got == _tree_recursive(_pad(_squares32(x)))
        sq = _squares32(x)
        assert got != _running(sq)
        assert got != _tree_strided(_pad(sq))
        if n & (n - 1):
            assert got != _tree_adjacent(_pad(sq, front=True))


# ---- RoPE -------------------------------------------------------------------

def test_rope_identity_deinterleaves():
    rng = np.random.default_rng(3)
    x = to_bf16(rng.standard_normal(64))
    y = oracle.rope_row(x, to_bf16(np.ones(64)), to_bf16(np.zeros(64)))
    assert np.array_equal(y[:32], x[0::2]) and np.array_equal(y[32:], x[1::2])


def test_rope_quarter_turn():
    rng = np.random.default_rng(4)
    x = to_bf16(rng.standard_normal(64))
    y = oracle.rope_row(x, to_bf16(np.zeros(64)), to_bf16(np.ones(64)))
    assert np.array_equal(y[:32], x[1::2] ^ np.uint16(0x8000))
    assert np.array_equal(y[32:], x[0::2])


def test_rope_vs_binary64():
    rng = np.random.default_rng(5)
    for trial in range(200):
        x = to_bf16(rng.standard_normal(64) * 10.0 ** rng.uniform(-2, 2))
        c = to_bf16(rng.uniform(-1, 1, 64))  # halves differ on purpose
        s = to_bf16(rng.uniform(-1, 1, 64))
        y = oracle.rope_row(x, c, s)
        xf, cf, sf = (bf16_to_f32(a).astype(np.float64) for a in (x, c, s))
        x1, x2 = xf[0::2], xf[1::2]
        y64 = np.concatenate([x1, x2]) * cf + np.concatenate([-x2, x1]) * sf
        nz = np.abs(y64) > 1e-30
        assert_close_bf16(y[nz], y64[nz])


# ---- quantiser: hand-worked rows ---------------------------------------------

def _row(nope_vals, d=128, rope=None):
    v = np.zeros(d, np.float64)
    v[:len(nope_vals)] = nope_vals
    if rope is not None:
        v[d - 64:] = rope
    return to_bf16(v)


def test_mode0_handworked_unit_scale():
    # amax 448 -> scale 448/448 = 1.0 (bf16 0x3F80); codes are E4M3(x).
    rope = np.linspace(-2, 2, 64)
    v = _row([448.0, 1.0, -2.0, 3.0, 0.5, -0.0], rope=rope)
    out, _ = oracle.quant_row(0, v, 64)
    assert out.size == 224  # align32(64 + 128 + 2)
    # -0.0 keeps its sign: 0x80
    assert list(out[:6]) == [0x7E, 0x38, 0xC0, 0x44, 0x30, 0x80]
    assert np.all(out[6:64] == 0)
    assert np.array_equal(out[64:192].view(np.uint16), v[64:])  # rope kept, LE
    assert list(out[192:194]) == [0x80, 0x3F]
    assert np.all(out[194:] == 0)


def test_mode0_handworked_rounded_scale():
    # amax 100: 100/448 = 0.22321428..., bf16 RNE -> (1 + 101/128) * 2^-3
    # = 0.2236328125 (bits 0x3E65).  100/0.2236328125 = 447.16 -> 448 (0x7E);
    # 50/0.2236328125 = 223.58 -> 224 (0x76); -1/0.2236... = -4.4716 -> -4.5
    # (1.125*2^2, code 0xC9).
    v = _row([100.0, 50.0, -1.0])
    out, _ = oracle.quant_row(0, v, 64)
    assert list(out[:3]) == [0x7E, 0x76, 0xC9]
    assert list(out[192:194]) == [0x65, 0x3E]


def test_mode1_handworked():
    # amax 450 (a bf16 value) -> E = 1 (448 < 450 <= 896), byte 128;
    # 450/2 = 225 -> 224 (0x76); -3/2 = -1.5 -> 0xBC.  Second group: amax 448 -> E = 0, byte 127.
    # Third group: all zero -> E = -127, byte 0, codes 0.
    v = np.zeros(256, np.float64)
    v[0], v[1] = 450.0, -3.0
    v[64], v[65] = 448.0, 0.5
    v = to_bf16(v)
    out, _ = oracle.quant_row(1, v, 64)
    assert out.size == 323
    assert list(out[:2]) == [0x76, 0xBC]
    assert list(out[64:66]) == [0x7E, 0x30]
    assert np.all(out[128:192] == 0)
    assert list(out[320:323]) == [128, 127, 0]


def test_mxfp4_handworked():
    # amax 6 -> E = 0 (byte 127): 6 -> 7, -6 -> 0xF, 5 -> tie 4/6 -> 4 (code
    # 6), 0.25 -> 0; packed low nibble first: 0xF7, 0x06.
    # Second group amax 7 -> E = 1 (byte 128): 7/2 = 3.5 -> tie 3/4 -> 4
    # (code 6); 1/2 -> 0.5 (code 1): 0x16.
    v = np.zeros(64, np.float64)
    v[0:4] = [6.0, -6.0, 5.0, 0.25]
    v[32:34] = [7.0, 1.0]
    out, sc = oracle.quant_row(3, to_bf16(v), 32)
    assert out.size == 32 and sc.size == 2
    assert list(out[:2]) == [0xF7, 0x06]
    assert out[16] == 0x16
    assert list(sc) == [127, 128]


# ---- quantiser: dequantisation error bound ------------------------------------

def _decode_e4m3(codes):
    t = np.concatenate([e4m3_table(), [np.nan]])
    mag = t[codes & 0x7F]
    return np.where(codes & 0x80, -mag, mag)


def _decode_e2m1(codes):
    t = e2m1_table()
    mag = t[codes & 0x7]
    return np.where(codes & 0x8, -mag, mag)


def _grid_gap(table, mag):
    """Largest gap between adjacent representable magnitudes around mag."""
    idx = np.searchsorted(table, mag)
    lo = table[np.clip(idx - 1, 0, len(table) - 1)]
    hi = table[np.clip(idx + 1, 0, len(table) - 1)]
    return np.maximum(mag - lo, hi - mag)


@pytest.mark.parametrize("mode", [0, 1])
def test_fp8_dequant_error_bound(mode):
    rng = np.random.default_rng(20 + mode)
    d = 576
    for trial in range(50):
        x = rng.standard_normal(d) * np.exp(rng.normal(0, 3))
        x[rng.integers(0, d, 3)] *= 100
        v = to_bf16(x)
        out, _ = oracle.quant_row(mode, v, 64)
        vf = bf16_to_f32(v).astype(np.float64)
        codes = out[:512]
        if mode == 0:
            s = bf16_to_f32(out[640:656].view(np.uint16)).astype(np.float64)
        else:
            s = 2.0 ** (out[640:648].astype(np.float64) - 127)
        s_el = np.repeat(s, 64)
        deq = _decode_e4m3(codes) * s_el
        gap = _grid_gap(e4m3_table(), np.abs(_decode_e4m3(codes)))
        sat = np.abs(vf[:512]) / s_el > 448
        err = np.abs(vf[:512] - deq)
        assert np.all(err[~sat] <= 0.5 * gap[~sat] * s_el[~sat] * (1 + 2 ** -20))
        # saturation only comes from the bf16 rounding of the mode-0 scale
        assert np.all(np.abs(vf[:512][sat]) / s_el[sat] <= 448 * (1 + 2 ** -8))
        if mode == 1:
            assert not sat.any()
        # each group's scale brackets its amax
        amax = np.abs(vf[:512]).reshape(8, 64).max(axis=1)
        assert np.all(amax / s <= 448 * (1 + 2 ** -8))
        if mode == 1:
            assert np.all((amax / s > 224) | (amax == 0))
        # rope bytes are the input's rope columns
        assert np.array_equal(out[512:640].view(np.uint16), v[512:])


def test_mxfp4_dequant_error_bound():
    rng = np.random.default_rng(30)
    for trial in range(100):
        d = 128
        v = to_bf16(rng.standard_normal(d) * np.exp(rng.normal(0, 3)))
        out, sc = oracle.quant_row(3, v, 32)
        vf = bf16_to_f32(v).astype(np.float64)
        codes = np.empty(d, np.uint8)
        codes[0::2] = out & 0xF
        codes[1::2] = out >> 4
        s_el = np.repeat(2.0 ** (sc.astype(np.float64) - 127), 32)
        q = _decode_e2m1(codes)
        gap = _grid_gap(e2m1_table(), np.abs(q))
        assert np.all(np.abs(vf - q * s_el) <= 0.5 * gap * s_el * (1 + 2 ** -20))
        amax = np.abs(vf).reshape(4, 32).max(axis=1)
        assert np.all(amax / 2.0 ** (sc.astype(np.float64) - 127) <= 6)
