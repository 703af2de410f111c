"""CPU oracle of the fused KV-cache write epilog -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The product library never loads it, and
it shares no code with the HIP path.

The arithmetic lives in ``kvepi_oracle.c`` (plain single-threaded C, binary32
in source order, no contraction); this module only builds it with gcc and
marshals numpy arrays into it through ctypes.  bf16 arrays are ``np.uint16``
bit patterns.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "kvepi_oracle.c")
LIB_PATH = os.path.join(_HERE, "libkvepi_oracle.so")

MODE_FP8_BF16SCALE = 0
MODE_FP8_E8M0 = 1
MODE_MXFP4 = 3
MODE_BF16_SPLIT = 4
MODE_MXFP8 = 5
MODE_FP8_ROW = 6
MODE_FP4_NOPE = 7

_lib = None


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (no GPU needed)."""
    if force or not os.path.exists(LIB_PATH):
        tmp = LIB_PATH + ".tmp"
        subprocess.check_call([
            "gcc", "-O2", "-std=c99", "-ffp-contract=off", "-fno-fast-math",
            "-fno-finite-math-only", "-fPIC", "-shared", "-Wall", "-Wextra",
            "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, LIB_PATH)
    return LIB_PATH


class _Cache(ctypes.Structure):
    _fields_ = [("data", ctypes.c_void_p), ("block_num", ctypes.c_int64),
                ("block_size", ctypes.c_int64), ("head_dim", ctypes.c_int64),
                ("block_stride", ctypes.c_int64)]


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            build(force=True)
        L = ctypes.CDLL(LIB_PATH)
        P, I64, I32, F = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_float
        L.kvo_bf16_to_f32.argtypes = [ctypes.c_uint16]
        L.kvo_bf16_to_f32.restype = F
        L.kvo_f32_to_bf16.argtypes = [F]
        L.kvo_f32_to_bf16.restype = ctypes.c_uint16
        L.kvo_enc_e4m3.argtypes = [F]
        L.kvo_enc_e4m3.restype = ctypes.c_uint8
        L.kvo_enc_e2m1.argtypes = [F]
        L.kvo_enc_e2m1.restype = ctypes.c_uint8
        L.kvo_e8m0_exponent.argtypes = [F, F]
        L.kvo_e8m0_exponent.restype = ctypes.c_int
        for n in ("kvo_enc_e4m3_batch", "kvo_enc_e2m1_batch", "kvo_f32_to_bf16_batch"):
            getattr(L, n).argtypes = [P, P, I64]
            getattr(L, n).restype = None
        L.kvo_e8m0_exponent_batch.argtypes = [P, F, P, I64]
        L.kvo_e8m0_exponent_batch.restype = None
        L.kvo_rmsnorm_row.argtypes = [P, P, I64, F, P]
        L.kvo_rmsnorm_row.restype = None
        L.kvo_sumsq_tree.argtypes = [P, I64]
        L.kvo_sumsq_tree.restype = F
        L.kvo_rope_row.argtypes = [P, P, P, P]
        L.kvo_rope_row.restype = None
        L.kvo_row_bytes.argtypes = [ctypes.c_int, I64, I32, P, P, P]
        L.kvo_row_bytes.restype = ctypes.c_int
        L.kvo_quant_row.argtypes = [ctypes.c_int, P, I64, I32, P, P]
        L.kvo_quant_row.restype = ctypes.c_int
        L.kvo_epilog.argtypes = [ctypes.c_int, I64, I64, P, I64, P, P, P, F, P, I32,
                                 ctypes.POINTER(_Cache), ctypes.POINTER(_Cache)]
        L.kvo_epilog.restype = ctypes.c_int
        L.kvo_fp16_to_f32.argtypes = [ctypes.c_uint16]
        L.kvo_fp16_to_f32.restype = F
        L.kvo_quant_row_x.argtypes = [ctypes.c_int, P, I64, I32, ctypes.c_int, P, P]
        L.kvo_quant_row_x.restype = ctypes.c_int
        L.kvo_token_slot.argtypes = [ctypes.c_int, P, I64, I64, I64, I64]
        L.kvo_token_slot.restype = I64
        L.kvo_epilog_ex.argtypes = [ctypes.c_int, I64, I64, P, I64, ctypes.c_int, P, P, P, F,
                                    P, ctypes.c_int, I64, ctypes.c_int, I32,
                                    ctypes.POINTER(_Cache), ctypes.POINTER(_Cache)]
        L.kvo_rope_row_n.argtypes = [P, P, P, I64, P]
        L.kvo_rope_row_n.restype = None
        L.kvo_epilog_ex.restype = ctypes.c_int
        L.kvo_f32_to_fp16.argtypes = [F]
        L.kvo_f32_to_fp16.restype = ctypes.c_uint16
        L.kvo_quant_int8.argtypes = [F, F, P]
        L.kvo_quant_int8.restype = ctypes.c_int8
        L.kvo_drq.argtypes = [I64, ctypes.c_int, ctypes.c_int, ctypes.c_int, P, ctypes.c_int, I64,
                              P, P, ctypes.c_int, P, P, P, ctypes.c_int, P, P, P, P, P,
                              ctypes.c_int, I64, ctypes.POINTER(_Cache), ctypes.POINTER(_Cache),
                              P, P, P]
        L.kvo_drq.restype = ctypes.c_int
        _lib = L
    return _lib


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


# ---- number formats -------------------------------------------------------

def enc_e4m3(v) -> np.ndarray:
    v = _c(v, np.float32)
    out = np.empty(v.shape, np.uint8)
    lib().kvo_enc_e4m3_batch(_ptr(v), _ptr(out), v.size)
    return out


def enc_e2m1(v) -> np.ndarray:
    v = _c(v, np.float32)
    out = np.empty(v.shape, np.uint8)
    lib().kvo_enc_e2m1_batch(_ptr(v), _ptr(out), v.size)
    return out


def f32_to_bf16(v) -> np.ndarray:
    v = _c(v, np.float32)
    out = np.empty(v.shape, np.uint16)
    lib().kvo_f32_to_bf16_batch(_ptr(v), _ptr(out), v.size)
    return out


def e8m0_exponent(amax, fmax: float) -> np.ndarray:
    a = _c(amax, np.float32)
    out = np.empty(a.shape, np.int32)
    lib().kvo_e8m0_exponent_batch(_ptr(a), ctypes.c_float(fmax), _ptr(out), a.size)
    return out


# ---- per-row steps --------------------------------------------------------

def rmsnorm_row(x_bf16, gamma_bf16, eps: float) -> np.ndarray:
    x = _c(x_bf16, np.uint16)
    g = _c(gamma_bf16, np.uint16)
    y = np.empty(x.shape, np.uint16)
    lib().kvo_rmsnorm_row(_ptr(x), _ptr(g), x.size, ctypes.c_float(eps), _ptr(y))
    return y


def sumsq_tree(x_bf16) -> float:
    x = _c(x_bf16, np.uint16)
    return float(lib().kvo_sumsq_tree(_ptr(x), x.size))


def rope_row_n(x_bf16, cos_bf16, sin_bf16) -> np.ndarray:
    """RoPE of a rope segment of any even length n (cos / sin of length n)."""
    x = _c(x_bf16, np.uint16)
    c = _c(cos_bf16, np.uint16)
    s = _c(sin_bf16, np.uint16)
    assert x.size % 2 == 0 and c.size == s.size == x.size
    y = np.empty(x.size, np.uint16)
    lib().kvo_rope_row_n(_ptr(x), _ptr(c), _ptr(s), x.size, _ptr(y))
    return y


def rope_row(x_bf16, cos_bf16, sin_bf16) -> np.ndarray:
    x, c, s = _c(x_bf16, np.uint16), _c(cos_bf16, np.uint16), _c(sin_bf16, np.uint16)
    assert x.size == 64 and c.size == 64 and s.size == 64
    y = np.empty(64, np.uint16)
    lib().kvo_rope_row(_ptr(x), _ptr(c), _ptr(s), _ptr(y))
    return y


def row_bytes(mode: int, d: int, group_size: int):
    cc, kc, sc = ctypes.c_int64(), ctypes.c_int64(), ctypes.c_int64()
    rc = lib().kvo_row_bytes(mode, d, group_size, ctypes.byref(cc), ctypes.byref(kc),
                             ctypes.byref(sc))
    if rc != 0:
        raise ValueError(f"unsupported mode={mode} d={d} group={group_size}")
    return cc.value, kc.value, sc.value


def fp16_to_f32(h: int) -> float:
    return float(lib().kvo_fp16_to_f32(int(h)))


def quant_row(mode: int, v_bf16, group_size: int, *, x_fp16: bool = False):
    """Quantise one row of 16-bit values (bf16 bits, or fp16 bits with
    x_fp16 in the indexer modes)."""
    v = _c(v_bf16, np.uint16)
    _, kc, sc = row_bytes(mode, v.size, group_size)
    out = np.empty(kc, np.uint8)
    sout = np.empty(4 * sc, np.uint8)
    rc = lib().kvo_quant_row_x(mode, _ptr(v), v.size, group_size, int(x_fp16), _ptr(out),
                               _ptr(sout))
    if rc != 0:
        raise ValueError("quant_row rejected its arguments")
    if mode in (MODE_MXFP4, MODE_MXFP8):
        return out, sout[:sc]
    if mode == MODE_FP8_ROW:
        return out, sout[:4].view(np.float32)  # the fp32 scale
    if mode == MODE_FP4_NOPE:
        return out[64:].copy(), None  # the bytes written: the row from byte 64 on
    return out, None


# ---- whole epilog ---------------------------------------------------------

INDEX_SLOT, INDEX_BATCH, INDEX_BLOCK, INDEX_BATCH_START = 0, 1, 2, 3


def token_slot(index_mode: int, index, t: int, seq_len: int, block_num: int,
               block_size: int) -> int:
    idx = _c(index, np.int32)
    return int(lib().kvo_token_slot(index_mode, _ptr(idx), t, seq_len, block_num, block_size))


def epilog(mode: int, x, slot_mapping, cache_bytes, cache_geom, *, group_size: int,
           gamma=None, cos=None, sin=None, eps: float = 1e-6, aux_bytes=None,
           aux_geom=None, x_fp16: bool = False, index_mode: int = INDEX_SLOT,
           seq_len: int = 0, rope_dim: int = 64):
    """Run the oracle in place on host byte buffers.

    cache_geom / aux_geom: (block_num, block_size, head_dim, block_stride) in
    elements of the cache dtype.  x is uint16 [T, d] (row stride = its
    row stride in elements; fp16 bits with x_fp16).  slot_mapping is the
    index array of index_mode (T entries for INDEX_SLOT and INDEX_BATCH,
    B * ceil(seq_len / block_size) for INDEX_BLOCK, B for
    INDEX_BATCH_START, with B = T / seq_len)."""
    x = np.asarray(x, np.uint16)
    assert x.ndim == 2 and x.strides[1] == 2
    T, d = x.shape
    slots = _c(slot_mapping, np.int32)
    if index_mode in (INDEX_SLOT, INDEX_BATCH):
        assert slots.size == T
    else:
        B = T // seq_len
        n = B * (-(-seq_len // int(cache_geom[1]))) if index_mode == INDEX_BLOCK else B
        assert slots.size == n
    assert cache_bytes.dtype == np.uint8 and cache_bytes.flags.c_contiguous
    gamma = None if gamma is None else _c(gamma, np.uint16)
    cos = None if cos is None else _c(cos, np.uint16)
    sin = None if sin is None else _c(sin, np.uint16)
    # the buffers must hold every row of their geometry (elements of 2
    # bytes for the split mode's caches, 4 for the per-row FP8 scales)
    def span(g):
        bn, bs, hd, stride = (int(v) for v in g)
        return (bn - 1) * stride + bs * hd if bn > 0 else 0

    esz = 2 if mode == MODE_BF16_SPLIT else 1
    assert cache_bytes.size >= span(cache_geom) * esz
    c = _Cache(cache_bytes.ctypes.data, *[int(v) for v in cache_geom])
    a = None
    if aux_bytes is not None:
        assert aux_bytes.dtype == np.uint8 and aux_bytes.flags.c_contiguous
        aesz = {MODE_BF16_SPLIT: 2, MODE_FP8_ROW: 4}.get(mode, 1)
        assert aux_bytes.size >= span(aux_geom) * aesz
        a = _Cache(aux_bytes.ctypes.data, *[int(v) for v in aux_geom])
    rc = lib().kvo_epilog_ex(mode, T, d, x.ctypes.data_as(ctypes.c_void_p),
                             x.strides[0] // 2, int(x_fp16), _ptr(gamma), _ptr(cos),
                             _ptr(sin), ctypes.c_float(eps), _ptr(slots), index_mode,
                             seq_len, rope_dim, group_size, ctypes.byref(c),
                             ctypes.byref(a) if a is not None else None)
    if rc != 0:
        raise ValueError("oracle epilog rejected its arguments")


# ---- dequant -> RoPE -> int8 KV cache ---------------------------------------------

DT_BF16, DT_FP16, DT_INT32, DT_FP32 = 0, 1, 2, 3


def f32_to_fp16(f: float) -> int:
    return int(lib().kvo_f32_to_fp16(ctypes.c_float(f)))


def quant_int8(v: float, scale: float, offset=None) -> int:
    off = None if offset is None else ctypes.byref(ctypes.c_float(offset))
    return int(lib().kvo_quant_int8(ctypes.c_float(v), ctypes.c_float(scale), off))


def drq(x, x_dtype: int, nq: int, nkv: int, D: int, cos, sin, out_dtype: int, *, scale_k,
        scale_v, k_cache_bytes, v_cache_bytes, cache_geom, index, index_mode: int = INDEX_SLOT,
        seq_len: int = 0, weight_scale=None, act_scale=None, bias=None, bias_dtype: int = DT_FP32,
        offset_k=None, offset_v=None, kv_output: bool = True):
    """Runs the oracle in place on the two int8 caches (uint8 byte buffers of
    geometry cache_geom = (block_num, block_size, head_dim, block_stride));
    returns (q_out, k_out, v_out) as uint16 arrays (k_out / v_out None
    without kv_output).  x is int32 or uint16 [T, H] (16-bit bit patterns)."""
    x = np.ascontiguousarray(x)
    T = x.shape[0]
    H = (nq + 2 * nkv) * D
    assert x.shape[1] == H
    q_out = np.zeros((T, nq * D), np.uint16)
    k_out = np.zeros((T, nkv * D), np.uint16) if kv_output else None
    v_out = np.zeros((T, nkv * D), np.uint16) if kv_output else None
    kc = _Cache(k_cache_bytes.ctypes.data, *[int(v) for v in cache_geom])
    vc = _Cache(v_cache_bytes.ctypes.data, *[int(v) for v in cache_geom])
    f32 = lambda a: None if a is None else _c(a, np.float32)  # noqa: E731
    cos = _c(cos, np.uint16)
    sin = _c(sin, np.uint16)
    idx = _c(index, np.int32)
    ws, act, sk, sv, ok, ov = (f32(a) for a in (weight_scale, act_scale, scale_k, scale_v,
                                                 offset_k, offset_v))
    b = None
    if bias is not None:
        b = np.ascontiguousarray(bias)
    rc = lib().kvo_drq(T, nq, nkv, D, _ptr(x), x_dtype, H, _ptr(cos), _ptr(sin), out_dtype,
                       _ptr(ws), _ptr(act), _ptr(b), bias_dtype, _ptr(sk), _ptr(sv), _ptr(ok),
                       _ptr(ov), _ptr(idx), index_mode, seq_len, ctypes.byref(kc),
                       ctypes.byref(vc), _ptr(q_out), _ptr(k_out), _ptr(v_out))
    if rc != 0:
        raise ValueError("oracle drq rejected its arguments")
    return q_out, k_out, v_out

