"""Thin ctypes binding of libkvepi.so (argument marshalling only).

The functions carry the C ABI's names.  They take torch tensors for device
memory and torch's current HIP stream, turn them into the plain pointers and
sizes of ``include/kvepi.h``, and raise ``KvepiError`` on a non-OK status.
Every step of the epilog runs in the library's HIP kernels; there is no
fallback of any kind: if the library is missing this module raises on import
of the library.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libkvepi.so")

KVEPI_OK = 0
STATUS_NAMES = {0: "KVEPI_OK", 1: "KVEPI_ERR_NULLPTR", 2: "KVEPI_ERR_SHAPE",
                3: "KVEPI_ERR_LAYOUT", 4: "KVEPI_ERR_PARAM", 5: "KVEPI_ERR_UNSUPPORTED",
                6: "KVEPI_ERR_WORKSPACE", 7: "KVEPI_ERR_RUNTIME"}

KVEPI_MODE_FP8_BF16SCALE = 0
KVEPI_MODE_FP8_E8M0 = 1
KVEPI_MODE_HIF8_FP4 = 2
KVEPI_MODE_MXFP4 = 3
KVEPI_MODE_BF16_SPLIT = 4
KVEPI_MODE_MXFP8 = 5
KVEPI_MODE_FP8_ROW = 6
KVEPI_MODE_FP4_NOPE = 7

KVEPI_X_BF16 = 0
KVEPI_X_FP16 = 1
KVEPI_INDEX_SLOT = 0
KVEPI_INDEX_BATCH = 1
KVEPI_INDEX_BLOCK = 2
KVEPI_INDEX_BATCH_START = 3


class KvepiError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {kvepi_status_str(status)}")


class kvepi_cache(ctypes.Structure):
    _fields_ = [("data", ctypes.c_void_p), ("block_num", ctypes.c_int64),
                ("block_size", ctypes.c_int64), ("head_dim", ctypes.c_int64),
                ("block_stride", ctypes.c_int64)]


class kvepi_options(ctypes.Structure):
    _fields_ = [("x_dtype", ctypes.c_int32), ("index_mode", ctypes.c_int32),
                ("seq_len", ctypes.c_int64), ("rope_dim", ctypes.c_int32),
                ("reserved", ctypes.c_int32)]


class kvepi_prepared(ctypes.Structure):
    _fields_ = [("opaque", ctypes.c_uint64 * 128)]  # KVEPI_PREPARED_BYTES


_lib: Optional[ctypes.CDLL] = None


def lib() -> ctypes.CDLL:
    """Loads the in-tree HIP library; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is missing: build it with `python -m kv_cache_epilog_amd.build` "
                "(the epilog has no non-HIP implementation)")
        L = ctypes.CDLL(LIB_PATH)
        P, I64, I32, F = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_float
        CP = ctypes.POINTER(kvepi_cache)
        L.kvepi_row_bytes.argtypes = [I32, I64, I32, P, P, P]
        L.kvepi_row_bytes.restype = ctypes.c_int
        L.kvepi_get_workspace.argtypes = [P, I64, I64, I64, P, P, P, P, CP, CP, I32, I32, F, P]
        L.kvepi_get_workspace.restype = ctypes.c_int
        L.kvepi_run.argtypes = [P, I64, I64, I64, P, P, P, P, CP, CP, I32, I32, F, P,
                                ctypes.c_uint64, P]
        L.kvepi_run.restype = ctypes.c_int
        OP = ctypes.POINTER(kvepi_options)
        L.kvepi_get_workspace_ex.argtypes = [P, I64, I64, I64, P, P, P, P, CP, CP, I32, I32, F,
                                             OP, P]
        L.kvepi_get_workspace_ex.restype = ctypes.c_int
        L.kvepi_run_ex.argtypes = [P, I64, I64, I64, P, P, P, P, CP, CP, I32, I32, F, OP, P,
                                   ctypes.c_uint64, P]
        L.kvepi_run_ex.restype = ctypes.c_int
        PP = ctypes.POINTER(kvepi_prepared)
        L.kvepi_prepare_ex.argtypes = [P, I64, I64, I64, P, P, P, P, CP, CP, I32, I32, F, OP,
                                       PP]
        L.kvepi_prepare_ex.restype = ctypes.c_int
        L.kvepi_run_prepared.argtypes = [PP, P]
        L.kvepi_run_prepared.restype = ctypes.c_int
        L.kvepi_status_str.argtypes = [ctypes.c_int]
        L.kvepi_status_str.restype = ctypes.c_char_p
        L.kvepi_version.argtypes = []
        L.kvepi_version.restype = I32
        _lib = L
    return _lib


def kvepi_status_str(status: int) -> str:
    return lib().kvepi_status_str(int(status)).decode()


def kvepi_version() -> int:
    return int(lib().kvepi_version())


def kvepi_row_bytes(quant_mode: int, d: int, group_size: int):
    """(concat_col, kv_cache_col, scale_col) of a mode."""
    cc, kc, sc = ctypes.c_int64(), ctypes.c_int64(), ctypes.c_int64()
    st = lib().kvepi_row_bytes(quant_mode, d, group_size, ctypes.byref(cc), ctypes.byref(kc),
                               ctypes.byref(sc))
    if st != KVEPI_OK:
        raise KvepiError(st, "kvepi_row_bytes")
    return cc.value, kc.value, sc.value


# ---- marshalling -----------------------------------------------------------

def _ptr(t) -> Optional[int]:
    return None if t is None else int(t.data_ptr())


def _x_view(x):
    """x [..., d] -> (ptr, T, d, row_stride) without copying."""
    if x.dim() < 1 or x.element_size() != 2:
        raise ValueError("x must be a 16-bit (bf16 or fp16) tensor")
    d = x.shape[-1]
    if x.stride(-1) != 1:
        raise ValueError("x rows must be contiguous")
    if x.dim() == 1:
        return _ptr(x), 1, d, d
    if x.dim() == 2:
        return _ptr(x), x.shape[0], d, x.stride(0)
    if not x.is_contiguous():
        raise ValueError("x with more than 2 dims must be contiguous")
    return _ptr(x), x.numel() // d if d else 0, d, d


def cache_desc(cache) -> kvepi_cache:
    """A 4-D cache tensor [block_num, block_size, 1, head_dim] (any block
    stride; contiguous inside a block) -> kvepi_cache."""
    if cache.dim() != 4 or cache.shape[2] != 1:
        raise ValueError("cache must be [block_num, block_size, 1, head_dim]")
    if cache.stride(3) != 1 or cache.stride(1) != cache.shape[3]:
        raise ValueError("cache blocks must be contiguous inside")
    return kvepi_cache(_ptr(cache), cache.shape[0], cache.shape[1], cache.shape[3],
                       cache.stride(0))


# element size of the main cache and of cache_aux per mode: uint8 everywhere
# except the bf16 split mode (bf16 ckv and k caches) and the per-row FP8
# mode's fp32 cache_scale
_CACHE_ELEM = {KVEPI_MODE_BF16_SPLIT: 2}
_AUX_ELEM = {KVEPI_MODE_BF16_SPLIT: 2, KVEPI_MODE_FP8_ROW: 4}


def _same_device(x, **tensors):
    """Every given tensor is on x's device, and that is not host memory (the
    library dereferences them on the GPU only)."""
    if x.device.type == "cpu":
        raise ValueError("x must be a device (cuda) tensor, not a host tensor")
    for name, t in tensors.items():
        if t is not None and t.device != x.device:
            raise ValueError(f"{name} must be on {x.device} (got {t.device})")


def _index_entries(index_mode: int, T: int, seq_len: int, block_size: int) -> int:
    """Length of the int32 index array of an index mode (see kvepi_options)."""
    if index_mode in (KVEPI_INDEX_SLOT, KVEPI_INDEX_BATCH):
        return T
    if seq_len < 1 or T % seq_len:
        raise ValueError("seq_len must be >= 1 and divide the token count")
    B = T // seq_len
    if index_mode == KVEPI_INDEX_BLOCK:
        return B * -(-seq_len // block_size)
    return B  # KVEPI_INDEX_BATCH_START


def _args(x, slot_mapping, cache, quant_mode, group_size, gamma, cos, sin, cache_aux, eps,
          index_mode=KVEPI_INDEX_SLOT, seq_len=0, rope_dim=0):
    import torch
    _same_device(x, slot_mapping=slot_mapping, cache=cache, gamma=gamma, cos=cos, sin=sin,
                 cache_aux=cache_aux)
    xp, T, d, xs = _x_view(x)
    if slot_mapping.dtype != torch.int32 or not slot_mapping.is_contiguous():
        raise ValueError("slot_mapping must be a contiguous int32 tensor")
    c = cache_desc(cache)
    need = _index_entries(index_mode, T, seq_len, c.block_size)
    if slot_mapping.numel() != need:
        raise ValueError(f"the index array must have {need} entries for index mode "
                         f"{index_mode} (got {slot_mapping.numel()})")
    dk = rope_dim or 64
    dv = d if quant_mode in (KVEPI_MODE_MXFP4, KVEPI_MODE_MXFP8, KVEPI_MODE_FP8_ROW) else d - dk
    for name, t, n in (("gamma", gamma, dv), ("cos", cos, T * dk), ("sin", sin, T * dk)):
        if t is None:
            continue
        if not t.is_contiguous() or t.element_size() != 2:
            raise ValueError(f"{name} must be a contiguous bf16 tensor")
        if t.numel() < n:
            raise ValueError(f"{name} must hold at least {n} values (got {t.numel()})")
    if cache.element_size() != _CACHE_ELEM.get(quant_mode, 1):
        raise ValueError(f"the cache of mode {quant_mode} has {_CACHE_ELEM.get(quant_mode, 1)}-byte "
                         f"elements (got {cache.dtype})")
    a = None
    if cache_aux is not None:
        if cache_aux.element_size() != _AUX_ELEM.get(quant_mode, 1):
            raise ValueError(f"cache_aux of mode {quant_mode} has "
                             f"{_AUX_ELEM.get(quant_mode, 1)}-byte elements "
                             f"(got {cache_aux.dtype})")
        a = cache_desc(cache_aux)
    return (xp, T, d, xs, _ptr(gamma), _ptr(cos), _ptr(sin), _ptr(slot_mapping),
            ctypes.byref(c), None if a is None else ctypes.byref(a),
            int(quant_mode), int(group_size), ctypes.c_float(eps)), (c, a)


def _options(x, index_mode: int, seq_len: int, rope_dim: int = 0) -> kvepi_options:
    """x's dtype (fp16 or the bf16 default), the index mode and the rope
    segment length (0: 64)."""
    import torch
    return kvepi_options(KVEPI_X_FP16 if x.dtype == torch.float16 else KVEPI_X_BF16,
                         int(index_mode), int(seq_len), int(rope_dim), 0)


def kvepi_get_workspace(x, slot_mapping, cache, quant_mode: int, group_size: int = 64, *,
                        gamma=None, cos=None, sin=None, cache_aux=None,
                        eps: float = 1e-6, index_mode: int = KVEPI_INDEX_SLOT,
                        seq_len: int = 0, rope_dim: int = 0) -> int:
    """Stage one.  x may be bf16 or (indexer modes) fp16; index_mode and
    seq_len select how slot_mapping places the tokens (see kvepi_options)."""
    args, _keep = _args(x, slot_mapping, cache, quant_mode, group_size, gamma, cos, sin,
                        cache_aux, eps, index_mode, seq_len, rope_dim)
    opt = _options(x, index_mode, seq_len, rope_dim)
    ws = ctypes.c_uint64()
    st = lib().kvepi_get_workspace_ex(*args, ctypes.byref(opt), ctypes.byref(ws))
    if st != KVEPI_OK:
        raise KvepiError(st, "kvepi_get_workspace")
    return ws.value


def kvepi_run(x, slot_mapping, cache, quant_mode: int, group_size: int = 64, *,
              gamma=None, cos=None, sin=None, cache_aux=None, eps: float = 1e-6,
              index_mode: int = KVEPI_INDEX_SLOT, seq_len: int = 0, rope_dim: int = 0,
              workspace=None, stream=None) -> None:
    """Enqueue the epilog on `stream` (a torch.cuda.Stream; default: torch's
    current stream).  Updates cache / cache_aux in place, asynchronously.
    x may be bf16 or (indexer modes) fp16; index_mode and seq_len select how
    slot_mapping places the tokens (see kvepi_options).  Raises KvepiError
    with the library's status on a rejected call (nothing is written then);
    with KVEPI_CHECK_SLOTS=1 in the environment, repeated slots are such an
    error (the check synchronises the stream)."""
    import torch
    args, _keep = _args(x, slot_mapping, cache, quant_mode, group_size, gamma, cos, sin,
                        cache_aux, eps, index_mode, seq_len, rope_dim)
    opt = _options(x, index_mode, seq_len, rope_dim)
    if stream is None:
        stream = torch.cuda.current_stream(x.device)
    ws_ptr = None if workspace is None else _ptr(workspace)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = lib().kvepi_run_ex(*args, ctypes.byref(opt), ws_ptr, ws_bytes,
                            ctypes.c_void_p(stream.cuda_stream))
    if st != KVEPI_OK:
        raise KvepiError(st, "kvepi_run")


class KvepiPrepared:
    """A prepared epilog call (kvepi_prepare_ex): the C struct, the torch
    device and references to the tensors it was prepared with, which keeps
    their memory allocated (at the same addresses) while it is alive."""

    __slots__ = ("struct", "ref", "device", "tensors")

    def __init__(self, struct, device, tensors):
        self.struct = struct
        self.ref = ctypes.byref(struct)
        self.device = device
        self.tensors = tensors


def kvepi_prepare(x, slot_mapping, cache, quant_mode: int, group_size: int = 64, *,
                  gamma=None, cos=None, sin=None, cache_aux=None, eps: float = 1e-6,
                  index_mode: int = KVEPI_INDEX_SLOT, seq_len: int = 0,
                  rope_dim: int = 0) -> KvepiPrepared:
    """Validates a kvepi_run call once and works out its launch on the
    current device (kvepi_prepare_ex); kvepi_run_prepared then enqueues it.
    The same checks as kvepi_run, ValueError or KvepiError otherwise.  The
    tensors' contents may change between runs; the tensors themselves are
    fixed (a run reads and writes the memory they had at preparation)."""
    import torch
    args, _keep = _args(x, slot_mapping, cache, quant_mode, group_size, gamma, cos, sin,
                        cache_aux, eps, index_mode, seq_len, rope_dim)
    opt = _options(x, index_mode, seq_len, rope_dim)
    prep = kvepi_prepared()
    with torch.cuda.device(x.device):
        st = lib().kvepi_prepare_ex(*args, ctypes.byref(opt), ctypes.byref(prep))
    if st != KVEPI_OK:
        raise KvepiError(st, "kvepi_prepare_ex")
    return KvepiPrepared(prep, x.device, (x, slot_mapping, cache, gamma, cos, sin, cache_aux))


def kvepi_run_prepared(prepared: KvepiPrepared, stream=None) -> None:
    """Enqueue a prepared call on `stream` (a torch.cuda.Stream; default:
    torch's current stream on the prepared call's device).  The host's work
    per call is this one C call: no argument is validated or converted
    again.  Raises KvepiError on a rejected call (another current device
    than at preparation, or a refused launch)."""
    if stream is None:
        import torch
        stream = torch.cuda.current_stream(prepared.device)
    st = (_lib or lib()).kvepi_run_prepared(prepared.ref, stream.cuda_stream)
    if st != KVEPI_OK:
        raise KvepiError(st, "kvepi_run_prepared")


# ---- dequant -> RoPE -> int8 KV cache (include/kvepi_drq.h) -------------------------

KVEPI_DT_BF16 = 0
KVEPI_DT_FP16 = 1
KVEPI_DT_INT32 = 2
KVEPI_DT_FP32 = 3
KVEPI_DRQ_PAGE = 0
KVEPI_DRQ_CONTIGUOUS = 1


class kvepi_drq_params(ctypes.Structure):
    _fields_ = [("x", ctypes.c_void_p), ("x_dtype", ctypes.c_int32),
                ("out_dtype", ctypes.c_int32), ("num_tokens", ctypes.c_int64),
                ("x_row_stride", ctypes.c_int64), ("nq", ctypes.c_int32),
                ("nkv", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("cos", ctypes.c_void_p), ("sin", ctypes.c_void_p),
                ("weight_scale", ctypes.c_void_p), ("act_scale", ctypes.c_void_p),
                ("bias", ctypes.c_void_p), ("bias_dtype", ctypes.c_int32),
                ("scale_k", ctypes.c_void_p), ("scale_v", ctypes.c_void_p),
                ("offset_k", ctypes.c_void_p), ("offset_v", ctypes.c_void_p),
                ("indices", ctypes.c_void_p), ("cache_mode", ctypes.c_int32),
                ("seq_len", ctypes.c_int64), ("k_cache", kvepi_cache),
                ("v_cache", kvepi_cache), ("q_out", ctypes.c_void_p),
                ("k_out", ctypes.c_void_p), ("v_out", ctypes.c_void_p)]


def _drq_lib():
    L = lib()
    if not getattr(L, "_drq_typed", False):
        PP = ctypes.POINTER(kvepi_drq_params)
        L.kvepi_drq_get_workspace.argtypes = [PP, ctypes.c_void_p]
        L.kvepi_drq_get_workspace.restype = ctypes.c_int
        L.kvepi_drq_run.argtypes = [PP, ctypes.c_void_p, ctypes.c_uint64, ctypes.c_void_p]
        L.kvepi_drq_run.restype = ctypes.c_int
        L._drq_typed = True
    return L


def _dtype_code(t) -> int:
    import torch
    return {torch.bfloat16: KVEPI_DT_BF16, torch.float16: KVEPI_DT_FP16,
            torch.int32: KVEPI_DT_INT32, torch.float32: KVEPI_DT_FP32}[t.dtype]


def drq_params(x, cos, sin, k_cache, v_cache, indices, *, nq: int, nkv: int, head_dim: int,
               scale_k, scale_v, q_out, k_out=None, v_out=None, weight_scale=None,
               act_scale=None, bias=None, offset_k=None, offset_v=None,
               cache_mode: int = KVEPI_DRQ_PAGE, seq_len: int = 0) -> kvepi_drq_params:
    """torch tensors -> kvepi_drq_params (pointers, sizes and dtype codes).
    Checks what the pointers alone cannot carry: every tensor on x's device,
    their dtypes and element counts (ValueError otherwise).  The returned
    params hold references to the tensors: a launch made with them reads
    device memory that stays allocated while the params are alive (the
    pointers alone would not keep a temporary tensor's memory, which torch
    may free and even return to the device, as a graph capture does)."""
    import torch
    _same_device(x, cos=cos, sin=sin, k_cache=k_cache, v_cache=v_cache, indices=indices,
                 scale_k=scale_k, scale_v=scale_v, q_out=q_out, k_out=k_out, v_out=v_out,
                 weight_scale=weight_scale, act_scale=act_scale, bias=bias, offset_k=offset_k,
                 offset_v=offset_v)
    if x.dim() != 2 or x.stride(1) != 1:
        raise ValueError("x must be [T, H] with contiguous rows")
    T, D = x.shape[0], head_dim
    H, HK = (nq + 2 * nkv) * D, nkv * D
    if x.shape[1] != H:
        raise ValueError(f"x must have (nq + 2 nkv) * head_dim = {H} columns")
    out16 = (torch.bfloat16, torch.float16)
    f32 = torch.float32
    if cos.dtype not in out16 or sin.dtype != cos.dtype:
        raise ValueError("cos and sin must be bf16 or fp16 tensors of one dtype")
    if indices.dtype != torch.int32:
        raise ValueError("indices must be int32")
    if k_cache.element_size() != 1 or v_cache.element_size() != 1:
        raise ValueError("k_cache and v_cache are int8 caches (1-byte elements)")
    need_idx = T if cache_mode == KVEPI_DRQ_PAGE else (T // seq_len if seq_len else -1)
    checks = [("cos", cos, T * D, None), ("sin", sin, T * D, None),
              ("indices", indices, need_idx, None), ("scale_k", scale_k, HK, f32),
              ("scale_v", scale_v, HK, f32), ("q_out", q_out, T * nq * D, cos.dtype),
              ("k_out", k_out, T * HK, cos.dtype), ("v_out", v_out, T * HK, cos.dtype),
              ("weight_scale", weight_scale, H, f32), ("act_scale", act_scale, T, f32),
              ("bias", bias, H, None), ("offset_k", offset_k, HK, f32),
              ("offset_v", offset_v, HK, f32)]
    for name, t, n, dt in checks:
        if t is None:
            continue
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
        if dt is not None and t.dtype != dt:
            raise ValueError(f"{name} must be {dt} (got {t.dtype})")
        if t.numel() < n:
            raise ValueError(f"{name} must hold at least {n} values (got {t.numel()})")
    params = kvepi_drq_params(
        _ptr(x), _dtype_code(x), _dtype_code(cos), x.shape[0], x.stride(0), nq, nkv, head_dim,
        _ptr(cos), _ptr(sin), _ptr(weight_scale), _ptr(act_scale), _ptr(bias),
        KVEPI_DT_FP32 if bias is None else _dtype_code(bias), _ptr(scale_k), _ptr(scale_v),
        _ptr(offset_k), _ptr(offset_v), _ptr(indices), cache_mode, seq_len,
        cache_desc(k_cache), cache_desc(v_cache), _ptr(q_out), _ptr(k_out), _ptr(v_out))
    params._tensors = (x, cos, sin, k_cache, v_cache, indices, scale_k, scale_v, q_out, k_out,
                       v_out, weight_scale, act_scale, bias, offset_k, offset_v)
    return params


def kvepi_drq_get_workspace(params: kvepi_drq_params) -> int:
    ws = ctypes.c_uint64()
    st = _drq_lib().kvepi_drq_get_workspace(ctypes.byref(params), ctypes.byref(ws))
    if st != KVEPI_OK:
        raise KvepiError(st, "kvepi_drq_get_workspace")
    return ws.value


def kvepi_drq_run(params: kvepi_drq_params, *, stream=None, device=None) -> None:
    """Enqueue the dequant -> RoPE -> int8 KV cache operator on `stream`
    (default: torch's current stream).  Raises KvepiError on a rejected call
    (nothing is written then); with KVEPI_CHECK_SLOTS=1 in the environment,
    repeated page-mode slots are such an error."""
    import torch
    if stream is None:
        stream = torch.cuda.current_stream(device)
    st = _drq_lib().kvepi_drq_run(ctypes.byref(params), None, 0,
                                  ctypes.c_void_p(stream.cuda_stream))
    if st != KVEPI_OK:
        raise KvepiError(st, "kvepi_drq_run")
