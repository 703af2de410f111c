"""Launches captured in a HIP graph (torch.cuda.CUDAGraph) give the eager
results on every replay ("indexer_quant_cache": graph-mode calls agree with
eager ones).  Each replay follows eager work of the program's own (a refill
of the caches) and a synchronisation, and every replay is checked."""
import numpy as np
import pytest

import kvgen
from kvgen import CacheSpec

from parity import cache_tensor, run_gpu, run_oracle, to_dev_bf16

pytestmark = pytest.mark.gpu


def _workload(mode):
    if mode == 0:
        return kvgen.make("graph_fused", 0, 700, 576, seed=90,
                          cache=CacheSpec(8, 128, 672, 128 * 672 + 64), norm=True, rope=True,
                          skip_frac=0.05)
    return kvgen.make("graph_mxfp4", 3, 1000, 128, seed=91, cache=CacheSpec(10, 128, 64, 8192),
                      aux=CacheSpec(10, 128, 4, 512), row_sigma=1.0, skip_frac=0.05)


@pytest.mark.parametrize("mode", [0, 3])
def test_epilog_graph_replays_match_eager(mode):
    import torch
    from kv_cache_epilog_amd import kvepi_run
    w = _workload(mode)
    want, awant = run_oracle(w)
    eager, aeager = run_gpu(w)
    assert np.array_equal(eager, want)
    dev = "cuda:0"
    x = to_dev_bf16(w.x, dev)
    slots = torch.from_numpy(w.slots).to(dev)
    gamma = None if w.gamma is None else to_dev_bf16(w.gamma, dev)
    cos = None if w.cos is None else to_dev_bf16(w.cos, dev)
    sin = None if w.sin is None else to_dev_bf16(w.sin, dev)
    cache, flat = cache_tensor(w.cache, w.cache_init, dev)
    aux = aflat = None
    if w.aux is not None:
        aux, aflat = cache_tensor(w.aux, w.aux_init, dev)

    def launch():
        kvepi_run(x, slots, cache, w.mode, w.group_size, gamma=gamma, cos=cos, sin=sin,
                  cache_aux=aux, eps=w.eps)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        launch()  # warm-up outside the capture
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        launch()
    init = torch.from_numpy(w.cache_init).to(dev)
    ainit = None if w.aux_init is None else torch.from_numpy(w.aux_init).to(dev)
    for _ in range(3):
        flat[:w.cache.alloc_bytes].copy_(init)  # eager work between replays
        if aflat is not None:
            aflat[:w.aux.alloc_bytes].copy_(ainit)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(flat[:w.cache.alloc_bytes].cpu().numpy(), want)
        if awant is not None:
            assert np.array_equal(aflat[:w.aux.alloc_bytes].cpu().numpy(), awant)


def test_drq_graph_replays_match_eager():
    import torch
    from drq_case import PREFILL, make_case, run_oracle as drq_oracle
    from kv_cache_epilog_amd import binding as B
    c = make_case(92, T=300, nq=2, nkv=1, D=64, x_dtype=kvgen.DT_INT32,
                  out_dtype=kvgen.DT_BF16, bias_dtype=kvgen.DT_FP32)
    want = drq_oracle(c)
    dev = "cuda:0"
    up = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)  # noqa: E731
    t16 = torch.bfloat16
    bn, bs, head, stride = c.geom
    kflat = torch.full((bn * stride,), PREFILL, dtype=torch.uint8, device=dev)
    vflat = torch.full((bn * stride,), PREFILL, dtype=torch.uint8, device=dev)
    kview = kflat.as_strided((bn, bs, 1, head), (stride, head, head, 1))
    vview = vflat.as_strided((bn, bs, 1, head), (stride, head, head, 1))
    q = torch.zeros((c.T, c.nq * c.D), dtype=t16, device=dev)
    ko = torch.zeros((c.T, c.nkv * c.D), dtype=t16, device=dev)
    vo = torch.zeros((c.T, c.nkv * c.D), dtype=t16, device=dev)
    p = B.drq_params(up(c.x), up(c.cos.view(np.int16)).view(t16), up(c.sin.view(np.int16)).view(t16),
                     kview, vview, up(c.index), nq=c.nq, nkv=c.nkv, head_dim=c.D,
                     scale_k=up(c.scale_k), scale_v=up(c.scale_v), q_out=q, k_out=ko, v_out=vo,
                     weight_scale=up(c.weight_scale), act_scale=up(c.act_scale),
                     bias=up(c.bias), offset_k=up(c.offset_k), offset_v=up(c.offset_v))
    B.kvepi_drq_run(p)  # eager warm-up
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        B.kvepi_drq_run(p)
    for _ in range(3):
        kflat.fill_(PREFILL)
        vflat.fill_(PREFILL)
        q.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        as16 = lambda t: t.view(torch.int16).cpu().numpy().view(np.uint16)  # noqa: E731
        assert np.array_equal(as16(q), want[0])
        assert np.array_equal(as16(ko), want[1]) and np.array_equal(as16(vo), want[2])
        assert np.array_equal(kflat.cpu().numpy(), want[3])
        assert np.array_equal(vflat.cpu().numpy(), want[4])
