"""CPU check of the tie data of tests/test_gpu_ties.py: it must reach the
scale significands where the rounding of the code quotient is delicate, i.e.
hold values on which one multiply by the rounded reciprocal of the scale's
significand (instead of the double-length reciprocal the kernels use) gives
another code than the exact quotient.  A kernel making that mistake would
then fail the GPU test."""
import numpy as np

from kvgen import bf16_to_f32
import test_gpu_ties as T


def _code(q, values):
    a, best, bd = abs(q), 0, np.inf
    for c, v in enumerate(values):
        d = abs(a - v)
        if d < bd or (d == bd and c % 2 == 0):
            bd, best = d, c
    return best


def _one_multiply_misses(fmax, mids, values, G):
    x, _ = T._tie_rows(fmax, mids, values, G, 512, 576, np.random.default_rng(61))
    xf = bf16_to_f32(x).astype(np.float64)
    miss = set()
    for r in range(x.shape[0]):
        for g in range(512 // G):
            v = xf[r, g * G:(g + 1) * G]
            s = float(T._bf16(np.array([np.float32(np.max(np.abs(v))) / np.float32(fmax)]))[0])
            m, ex = np.frexp(s)
            r1 = np.float32(1.0) / np.float32(2 * m)
            for vi in v:
                q1 = float(np.float32(vi * np.float64(r1))) * 2.0 ** -(ex - 1)
                if _code(q1, values) != _code(vi / s, values):
                    miss.add(int(round((2 * m - 1) * 128)))
    return miss


def test_tie_data_catches_a_single_multiply_quotient():
    assert _one_multiply_misses(448.0, T.E4M3_MIDS, T.E4M3_VALUES, 64)
    assert _one_multiply_misses(6.0, T.E2M1_MIDS, T.E2M1_VALUES, 32)
