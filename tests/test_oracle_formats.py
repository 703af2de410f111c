"""Pins of the oracle's number formats against things other than itself.

- E4M3FN / E2M1 encoders: hand-worked codes (tests/golden) and a brute-force
  nearest search over a code table decoded from the OCP format definitions,
  over every bf16 bit pattern (with near-tie low bits) and over whole fp32
  binades at the subnormal/normal/saturation boundaries.
- bf16 rounding: torch's conversion (round to nearest even) as the library
  routine.
- e8m0 exponent: a direct search over E for every positive finite bf16 amax.
"""
import os

import numpy as np
import pytest

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _read_pairs(name):
    rows = []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.split("#")[0].strip()
            if line:
                v, c = line.split()
                rows.append((float(v), int(c, 16)))
    return rows


# ---- decoded code tables from the format definitions ----------------------

def e4m3_table():
    """Magnitudes of E4M3FN codes 0x00..0x7E (0x7F is NaN)."""
    vals = []
    for code in range(0x7F):
        e, m = code >> 3, code & 7
        vals.append(m * 2.0 ** -9 if e == 0 else (1 + m / 8) * 2.0 ** (e - 7))
    return np.array(vals)


def e2m1_table():
    vals = []
    for code in range(8):
        e, m = code >> 1, code & 1
        vals.append(m * 0.5 if e == 0 else (1 + m / 2) * 2.0 ** (e - 1))
    return np.array(vals)


def brute_force_codes(v, table, sign_bit):
    """Nearest table entry to |v| (ties to the even code), saturating at the
    largest entry, with the sign of v in sign_bit."""
    v = np.asarray(v, np.float32)
    a = np.abs(v.astype(np.float64))
    assert np.all(np.diff(table) > 0)
    hi = np.clip(np.searchsorted(table, a, side="left"), 1, len(table) - 1)
    lo = hi - 1
    dlo = a - table[lo]
    dhi = table[hi] - a
    pick = np.where(dlo < dhi, lo, np.where(dhi < dlo, hi, np.where(lo % 2 == 0, lo, hi)))
    pick = np.where(a >= table[-1], len(table) - 1, pick)
    pick = np.where(a <= table[0], 0, pick)
    return (pick | np.where(np.signbit(v), sign_bit, 0)).astype(np.uint8)


def fp32_patterns():
    """Every bf16 pattern (finite) combined with low-bit patterns that sit
    exactly on, just above and just below bf16-representable ties."""
    hi = np.arange(1 << 16, dtype=np.uint32) << 16
    lows = np.array([0x0000, 0x0001, 0x7FFF, 0x8000, 0x8001, 0xFFFF, 0x1234, 0xC001],
                    np.uint32)
    bits = (hi[:, None] | lows[None, :]).reshape(-1)
    v = bits.view(np.float32)
    return v[np.isfinite(v)]


def binade(e):
    """All 2^23 fp32 values in [2^e, 2^(e+1)), both signs."""
    base = np.uint32((e + 127) << 23)
    m = np.arange(1 << 23, dtype=np.uint32)
    pos = (base | m).view(np.float32)
    return np.concatenate([pos, -pos])


# ---- E4M3 -----------------------------------------------------------------

def test_e4m3_handworked_codes():
    for v, c in _read_pairs("e4m3_codes.txt"):
        assert oracle.enc_e4m3(np.float32(v))[()] == c, (v, hex(c))


def test_e4m3_vs_brute_force_bf16_grid():
    v = fp32_patterns()
    got = oracle.enc_e4m3(v)
    want = brute_force_codes(v, e4m3_table(), 0x80)
    bad = np.nonzero(got != want)[0]
    assert bad.size == 0, [(float(v[i]), hex(got[i]), hex(want[i])) for i in bad[:10]]


@pytest.mark.parametrize("e", [-11, -10, -7, -6, -1, 0, 7, 8, 9])
def test_e4m3_vs_brute_force_full_binade(e):
    v = binade(e)
    got = oracle.enc_e4m3(v)
    want = brute_force_codes(v, e4m3_table(), 0x80)
    bad = np.nonzero(got != want)[0]
    assert bad.size == 0, [(float(v[i]), hex(got[i]), hex(want[i])) for i in bad[:10]]


def test_e4m3_never_nan_for_finite():
    v = fp32_patterns()
    assert not np.any((oracle.enc_e4m3(v) & 0x7F) == 0x7F)


# ---- E2M1 -----------------------------------------------------------------

def test_e2m1_handworked_codes():
    for v, c in _read_pairs("e2m1_codes.txt"):
        assert oracle.enc_e2m1(np.float32(v))[()] == c, (v, hex(c))


def test_e2m1_vs_brute_force_bf16_grid():
    v = fp32_patterns()
    got = oracle.enc_e2m1(v)
    want = brute_force_codes(v, e2m1_table(), 0x8)
    bad = np.nonzero(got != want)[0]
    assert bad.size == 0, [(float(v[i]), hex(got[i]), hex(want[i])) for i in bad[:10]]


@pytest.mark.parametrize("e", [-3, -2, -1, 0, 1, 2])
def test_e2m1_vs_brute_force_full_binade(e):
    v = binade(e)
    got = oracle.enc_e2m1(v)
    want = brute_force_codes(v, e2m1_table(), 0x8)
    bad = np.nonzero(got != want)[0]
    assert bad.size == 0, [(float(v[i]), hex(got[i]), hex(want[i])) for i in bad[:10]]


# ---- bf16 -----------------------------------------------------------------

def test_bf16_rounding_matches_torch():
    import torch
    rng = np.random.default_rng(123)
    rand = rng.integers(0, 1 << 32, size=1 << 22, dtype=np.uint64).astype(np.uint32)
    v = np.concatenate([fp32_patterns(), rand.view(np.float32)])
    v = v[np.isfinite(v)]
    got = oracle.f32_to_bf16(v)
    want = torch.from_numpy(v).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    bad = np.nonzero(got != want)[0]
    assert bad.size == 0, [(float(v[i]), hex(got[i]), hex(want[i])) for i in bad[:10]]


def test_bf16_overflow_rounds_to_inf():
    big = np.float32(np.finfo(np.float32).max)
    assert oracle.f32_to_bf16(np.array([big], np.float32))[0] == 0x7F80


# ---- e8m0 -----------------------------------------------------------------

@pytest.mark.parametrize("fmax", [448.0, 6.0])
def test_e8m0_exponent_direct_search(fmax):
    h = np.arange(1, 0x7F80, dtype=np.uint32)  # every positive finite bf16
    amax = (h << 16).view(np.float32)
    got = oracle.e8m0_exponent(amax, fmax)
    a64 = amax.astype(np.float64)
    want = np.full(a64.shape, 127, np.int32)
    for E in range(126, -128, -1):           # smallest E with amax <= fmax*2^E
        want = np.where(a64 <= fmax * 2.0 ** E, E, want)
    assert np.array_equal(got, want)
    # the power-of-two scale brackets amax: amax/2^E in (fmax/2, fmax] when
    # the clamp at -127 is not active
    mid = want > -127
    ratio = a64[mid] / 2.0 ** want[mid]
    assert np.all(ratio <= fmax) and np.all(ratio > fmax / 2)


def test_e8m0_zero_amax():
    assert oracle.e8m0_exponent(np.zeros(1, np.float32), 448.0)[0] == -127
