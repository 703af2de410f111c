"""GPU parity at exact rounding ties under every bf16 scale significand.

The staged quantisers (mode 0 and the FP4 nope mode, rows of d = 576 on 32
lanes) divide each value by the group's stored bf16 scale s = m * 2^e through
a table of double-length reciprocals of the 128 significands m, and the
codes then depend on that quotient being exact where it matters most: at a
value v = M * s whose quotient is exactly a rounding midpoint M of the code
format, where round-to-nearest-even decides.  Here every group's amax is a
bf16 value chosen so that the scale's significand is one of the 128 (all of
those that a bf16 amax can produce), and the other values of the group are
every such exact tie that is itself a bf16 value, with random signs.  The
whole cache is compared byte for byte with the oracle ("aclnnKvCompressEpilog",
计算公式 scenes 1 and 3: scale = amax / FP_MAX, codes of x / scale)."""
import numpy as np
import pytest

import kvgen
from kvgen import CacheSpec, bf16_to_f32, to_bf16

from parity import check

pytestmark = pytest.mark.gpu

# rounding midpoints of the code formats: E4M3FN between adjacent values
# (subnormals k * 2^-9 below 2^-6), up to the 432 between 416 and 448; E2M1
E4M3_VALUES = sorted({c * 2.0 ** -9 for c in range(8)} |
                     {(1 + f / 8) * 2.0 ** e for e in range(-6, 9) for f in range(8)
                      if (1 + f / 8) * 2.0 ** e <= 448})
E4M3_MIDS = [(a + b) / 2 for a, b in zip(E4M3_VALUES, E4M3_VALUES[1:])]
E2M1_VALUES = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]
E2M1_MIDS = [(a + b) / 2 for a, b in zip(E2M1_VALUES, E2M1_VALUES[1:])]


def _bf16(v):
    return bf16_to_f32(to_bf16(np.asarray(v, np.float64))).astype(np.float64)


def _amax_by_significand(fmax, e):
    """For each scale significand index k (m = 1 + k/128) that a bf16 amax
    can produce, one such amax: scale = bf16(fp32(amax) / fmax) = m * 2^e."""
    lo, hi = fmax * 2.0 ** e * 0.99, fmax * 2.0 ** (e + 1) * 1.01
    cands = np.arange(0, 0x7F80, dtype=np.uint32)  # positive finite bf16 patterns
    a = bf16_to_f32(cands.astype(np.uint16)).astype(np.float64)
    a = a[(a >= lo) & (a <= hi)]
    s = _bf16((a.astype(np.float32) / np.float32(fmax)).astype(np.float64))
    out = {}
    for ai, si in zip(a, s):
        m, ex = np.frexp(si)  # si = m * 2^ex, m in [0.5, 1)
        if ex - 1 != e:
            continue
        k = int(round((2 * m - 1) * 128))
        out.setdefault(k, (ai, si))
    return out


def _tie_rows(fmax, mids, values, G, nseg, d, rng, e=-3):
    """Rows of d values: groups of G in the first nseg columns, one group per
    reachable scale significand (cycled), each holding its amax and every
    exact tie M * s (and every exact code value times s) that is a bf16
    value below the amax; random values fill the rest of the row."""
    table = _amax_by_significand(fmax, e)
    groups = []
    for k in sorted(table):
        amax, s = table[k]
        cand = np.array([m * s for m in mids] + [v * s for v in values if v > 0])
        cand = cand[(cand <= amax) & (_bf16(cand) == cand)]
        g = np.resize(cand if cand.size else np.array([amax / 3]), G)
        g = g * np.where(rng.random(G) < 0.5, -1.0, 1.0)
        g[rng.integers(G)] = amax * (1 if rng.random() < 0.5 else -1)
        groups.append(g)
    per_row = nseg // G
    T = (len(groups) + per_row - 1) // per_row
    x = rng.standard_normal((T, d))
    for i, g in enumerate(groups):
        r, j = divmod(i, per_row)
        x[r, j * G:(j + 1) * G] = g
    for i in range(len(groups), T * per_row):  # fill the last row with more groups
        r, j = divmod(i, per_row)
        x[r, j * G:(j + 1) * G] = groups[i % len(groups)]
    return to_bf16(x), len(table)


def _reachable(fmax, e=-3):
    return len(_amax_by_significand(fmax, e))


def test_reachable_significands_cover_most_of_the_table():
    # a bf16 amax reaches most of the 128 significands of amax / FP_MAX as a
    # bf16 scale (every one it can reach is tested below)
    assert _reachable(448.0) >= 100
    assert _reachable(6.0) >= 100


# pad: extra bytes per cache row; a pitch that is not a multiple of 16 bytes
# takes the unstaged quantiser (a reciprocal per group instead of the table)
@pytest.mark.parametrize("pad", [0, 1])
@pytest.mark.parametrize("rope", [False, True])
def test_mode0_ties_at_every_scale_significand(rope, pad):
    import oracle
    rng = np.random.default_rng(61 + rope)
    d = 576
    x, nk = _tie_rows(448.0, E4M3_MIDS, E4M3_VALUES, 64, d - 64, d, rng)
    T = x.shape[0]
    _, kc, _ = oracle.row_bytes(0, d, 64)
    bs = 4
    nblk = (T + bs - 1) // bs + 2
    w = kvgen.make(f"ties_m0_rope{rope}", 0, T, d, seed=62, x=x, rope=rope,
                   cache=CacheSpec(nblk, bs, kc + pad, bs * (kc + pad)), skip_frac=0.0)
    assert nk >= 100
    assert check(w) == 0


@pytest.mark.parametrize("pad", [0, 1])
@pytest.mark.parametrize("g", [16, 32, 64])
def test_fp4_nope_ties_at_every_scale_significand(g, pad):
    import oracle
    rng = np.random.default_rng(70 + g)
    d = 576
    x, nk = _tie_rows(6.0, E2M1_MIDS, E2M1_VALUES, g, d - 64, d, rng)
    T = x.shape[0]
    mode = kvgen.MODE_FP4_NOPE
    _, kc, _ = oracle.row_bytes(mode, d, g)
    bs = 4
    nblk = (T + bs - 1) // bs + 2
    w = kvgen.make(f"ties_fp4nope_g{g}", mode, T, d, seed=71, x=x, group_size=g,
                   cache=CacheSpec(nblk, bs, kc + pad, bs * (kc + pad)), skip_frac=0.0)
    assert nk >= 100
    assert check(w) == 0
