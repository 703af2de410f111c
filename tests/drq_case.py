"""The two runs compared by the parity tests of the dequant -> RoPE -> int8
KV cache operator: the HIP path through the C ABI and the oracle, on inputs
from kvgen.drq_make."""
from __future__ import annotations

import numpy as np

import oracle
from kvgen import DrqWorkload as DrqCase  # noqa: F401
from kvgen import drq_make as make_case  # noqa: F401

PREFILL = 0xAB


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


def run_gpu(c: DrqCase, device="cuda:0", before_run=None):
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
    if before_run is not None:
        before_run()
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
