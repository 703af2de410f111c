"""Seeded inputs for the dequant -> RoPE -> int8 KV cache operator and the
two runs compared by its parity tests: the HIP path through the C ABI and
the oracle.  Inputs follow the operator's own examples: int32 matmul
outputs with per-column weight scales, per-token activation scales and a
bias, or fp16/bf16 activations; cos/sin of random positions; per-channel
static scales sized to the k / v ranges."""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Optional

import numpy as np

import kvgen
import oracle

PREFILL = 0xAB


@dataclass
class DrqCase:
    T: int
    nq: int
    nkv: int
    D: int
    x: np.ndarray            # int32 or uint16 bits [T, H]
    x_dtype: int
    out_dtype: int
    cos: np.ndarray
    sin: np.ndarray
    scale_k: np.ndarray
    scale_v: np.ndarray
    index: np.ndarray
    cache_mode: int          # 0 page, 1 contiguous
    seq_len: int
    geom: tuple              # (block_num, block_size, head_dim, block_stride) bytes
    weight_scale: Optional[np.ndarray] = None
    act_scale: Optional[np.ndarray] = None
    bias: Optional[np.ndarray] = None
    bias_dtype: int = oracle.DT_FP32
    offset_k: Optional[np.ndarray] = None
    offset_v: Optional[np.ndarray] = None
    kv_output: bool = True
    x_pad: int = 0
    notes: dict = field(default_factory=dict)


def to16(a, dt):
    return kvgen.to_bf16(a) if dt == oracle.DT_BF16 else kvgen.to_fp16(a)


def make_case(seed, *, T, nq, nkv, D, x_dtype, out_dtype, cache_mode=0, bias_dtype=None,
              act=True, offsets=True, kv_output=True, bn=None, bs=16, head=None, stride_extra=0,
              skip=0.05, seq_len=0, x_pad=0) -> DrqCase:
    rng = np.random.default_rng(seed)
    H = (nq + 2 * nkv) * D
    ws = act_s = bias = None
    if x_dtype == oracle.DT_INT32:
        x = rng.integers(-(1 << 20), 1 << 20, (T, H)).astype(np.int32)
        ws = (rng.random(H) * 2e-4 + 1e-5).astype(np.float32)
        if act:
            act_s = rng.uniform(0.5, 2.0, T).astype(np.float32)
        if bias_dtype is not None:
            b = rng.standard_normal(H) * 4
            if bias_dtype == oracle.DT_FP32:
                bias = b.astype(np.float32)
            elif bias_dtype == oracle.DT_INT32:
                bias = np.round(b).astype(np.int32)
            else:
                bias = to16(b, bias_dtype)
        mag = 200.0
    else:
        x = to16(rng.standard_normal((T, H)) * 3, x_dtype)
        mag = 12.0
    pos = rng.integers(0, 32768, T).astype(np.float64)
    inv = 10000.0 ** (-2.0 * np.arange(D // 2) / D)
    ang = np.concatenate([pos[:, None] * inv[None, :]] * 2, axis=1)
    cos, sin = to16(np.cos(ang), out_dtype), to16(np.sin(ang), out_dtype)
    sk = (mag / 127 * rng.uniform(0.5, 1.5, nkv * D)).astype(np.float32)
    sv = (mag / 127 * rng.uniform(0.5, 1.5, nkv * D)).astype(np.float32)
    ok = ov = None
    if offsets:
        ok = rng.integers(-8, 8, nkv * D).astype(np.float32)
        ov = (rng.integers(-16, 16, nkv * D) / 2).astype(np.float32)  # .5 ties
    row = nkv * D
    head = head or row
    if cache_mode == 0:
        bn = bn or (T + bs - 1) // bs + 2
        index = rng.permutation(bn * bs)[:T].astype(np.int32)
        k = int(round(skip * T))
        if k:
            index[rng.choice(T, k, replace=False)] = -1
        if T > 3:
            index[3] = bn * bs  # outside the cache: skipped
    else:
        B = T // seq_len
        bn = bn or B + 1
        index = rng.integers(0, bs - seq_len + 1, B).astype(np.int32)
        if B > 1:
            index[1] = -1
    geom = (bn, bs, head, bs * head + stride_extra)
    return DrqCase(T, nq, nkv, D, x, x_dtype, out_dtype, cos, sin, sk, sv, index, cache_mode,
                   seq_len, geom, ws, act_s, bias, bias_dtype if bias is not None else
                   oracle.DT_FP32, ok, ov, kv_output, x_pad)


def run_oracle(c: DrqCase):
    n = c.geom[0] * c.geom[3]
    kc = np.full(n, PREFILL, np.uint8)
    vc = np.full(n, PREFILL, np.uint8)
    q, ko, vo = oracle.drq(c.x, c.x_dtype, c.nq, c.nkv, c.D, c.cos, c.sin, c.out_dtype,
                           scale_k=c.scale_k, scale_v=c.scale_v, k_cache_bytes=kc,
                           v_cache_bytes=vc, cache_geom=c.geom, index=c.index,
                           index_mode=oracle.INDEX_BATCH_START if c.cache_mode else
                           oracle.INDEX_SLOT, seq_len=c.seq_len, weight_scale=c.weight_scale,
                           act_scale=c.act_scale, bias=c.bias, bias_dtype=c.bias_dtype,
                           offset_k=c.offset_k, offset_v=c.offset_v, kv_output=c.kv_output)
    return q, ko, vo, kc, vc


def run_gpu(c: DrqCase, device="cuda:0"):
    import torch
    from kv_cache_epilog_amd import binding as B

    def dev(a, dtype=None):
        if a is None:
            return None
        t = torch.from_numpy(np.ascontiguousarray(a)).to(device)
        return t.view(dtype) if dtype is not None else t

    t16 = torch.bfloat16 if c.out_dtype == oracle.DT_BF16 else torch.float16
    H = c.x.shape[1]
    if c.x_dtype == oracle.DT_INT32:
        xb = np.zeros((c.T, H + c.x_pad), np.int32)
        xb[:, :H] = c.x
        x = dev(xb)[:, :H]
    else:
        xb = np.zeros((c.T, H + c.x_pad), np.uint16)
        xb[:, :H] = c.x
        x = dev(xb.view(np.int16), t16)[:, :H]
    bias = None
    if c.bias is not None:
        bias = dev(c.bias) if c.bias_dtype in (oracle.DT_FP32, oracle.DT_INT32) else \
            dev(c.bias.view(np.int16), torch.bfloat16 if c.bias_dtype == oracle.DT_BF16
                else torch.float16)
    bn, bs, head, stride = c.geom
    kflat = torch.full((bn * stride,), PREFILL, dtype=torch.uint8, device=device)
    vflat = torch.full((bn * stride,), PREFILL, dtype=torch.uint8, device=device)
    kview = kflat.as_strided((bn, bs, 1, head), (stride, head, head, 1))
    vview = vflat.as_strided((bn, bs, 1, head), (stride, head, head, 1))
    q = torch.zeros((c.T, c.nq * c.D), dtype=t16, device=device)
    ko = vo = None
    if c.kv_output:
        ko = torch.zeros((c.T, c.nkv * c.D), dtype=t16, device=device)
        vo = torch.zeros((c.T, c.nkv * c.D), dtype=t16, device=device)
    p = B.drq_params(x, dev(c.cos.view(np.int16), t16), dev(c.sin.view(np.int16), t16), kview,
                     vview, dev(c.index), nq=c.nq, nkv=c.nkv, head_dim=c.D,
                     scale_k=dev(c.scale_k), scale_v=dev(c.scale_v), q_out=q, k_out=ko,
                     v_out=vo, weight_scale=dev(c.weight_scale), act_scale=dev(c.act_scale),
                     bias=bias, offset_k=dev(c.offset_k), offset_v=dev(c.offset_v),
                     cache_mode=c.cache_mode, seq_len=c.seq_len)
    assert B.kvepi_drq_get_workspace(p) == 0
    B.kvepi_drq_run(p, device=device)
    torch.cuda.synchronize()
    as16 = lambda t: None if t is None else t.view(torch.int16).cpu().numpy().view(np.uint16)  # noqa
    return as16(q), as16(ko), as16(vo), kflat.cpu().numpy(), vflat.cpu().numpy()


def compare(c: DrqCase, label=""):
    got = run_gpu(c)
    want = run_oracle(c)
    names = ("q_out", "k_out", "v_out", "k_cache", "v_cache")
    for n, g, w in zip(names, got, want):
        if w is None:
            assert g is None
            continue
        d = np.nonzero(g.reshape(-1) != w.reshape(-1))[0]
        assert d.size == 0, (f"{label} {n}: {d.size} differ, first at {d[:6].tolist()}: got "
                             f"{g.reshape(-1)[d[:6]].tolist()} want {w.reshape(-1)[d[:6]].tolist()}")
