"""Prepared calls (kvepi_prepare / kvepi_run_prepared) write exactly what
kvepi_run writes: the named workloads at full size and a set of modes,
layouts and index modes byte for byte against the oracle; runs after the
buffers' contents have changed in place; replays from a HIP graph; the
empty call; and a grid fixed at preparation."""
import numpy as np
import pytest

import kvgen
from kvgen import CacheSpec

from parity import cache_tensor, check, run_oracle, to_dev_bf16

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("i", range(7))
def test_prepared_config_parity(i):
    w = kvgen.config(i)
    check(w, label=f"prepared config {i} {w.name}", prepared=True, repeat=2)


def _case(kind, seed):
    if kind == "fused":
        return kvgen.make("p_fused", 0, 700, 576, seed=seed,
                          cache=CacheSpec(8, 128, 672, 128 * 672 + 64), norm=True, rope=True,
                          skip_frac=0.05)
    if kind == "mode1":
        return kvgen.make("p_mode1", 1, 513, 576, seed=seed,
                          cache=CacheSpec(9, 64, 648, 64 * 648 + 40), row_sigma=1.5)
    if kind == "mxfp4":
        return kvgen.make("p_mxfp4", 3, 1000, 128, seed=seed, cache=CacheSpec(10, 128, 64, 8192),
                          aux=CacheSpec(10, 128, 4, 512), row_sigma=1.0, skip_frac=0.05)
    if kind == "split":
        return kvgen.make("p_split", 4, 200, 576, seed=seed,
                          cache=CacheSpec(42, 5, 512, 5 * 512 + 8, 2),
                          aux=CacheSpec(42, 5, 64, 5 * 64 + 8, 2), norm=True, rope=True)
    if kind == "fp8row_fp16":
        x16 = kvgen.fp16_rows(np.random.default_rng(seed), 300, 128, row_sigma=1.0)
        w = kvgen.make("p_fp8row", 6, 300, 128, seed=seed, cache=CacheSpec(40, 8, 128, 1024),
                       aux=CacheSpec(40, 8, 1, 8, 4), x=x16, skip_frac=0.05)
        w.x_fp16 = True
        return w
    if kind == "fp4nope":
        return kvgen.make("p_fp4nope", 7, 333, 576, seed=seed,
                          cache=CacheSpec(40, 9, 384, 9 * 384), norm=True, group_size=16,
                          row_sigma=1.0)
    if kind == "batch_index":
        # 8 batches of 40 tokens, each batch's rows one block of 48
        w = kvgen.make("p_batch", 0, 8 * 40, 256, seed=seed, cache=CacheSpec(9, 48, 352, 48 * 352))
        w.slots = kvgen.index_array(np.random.default_rng(seed + 1000), 1, 8, 40, 9, 48, 0.05)
        w.index_mode, w.seq_len = 1, 40
        return w
    raise ValueError(kind)


KINDS = ["fused", "mode1", "mxfp4", "split", "fp8row_fp16", "fp4nope", "batch_index"]


@pytest.mark.parametrize("kind", KINDS)
def test_prepared_modes(kind):
    w = _case(kind, 100 + KINDS.index(kind))
    check(w, label=f"prepared {kind}", prepared=True)


def _upload(w, dev):
    import torch
    x = to_dev_bf16(w.x, dev)
    if w.x_fp16:
        x = x.view(torch.float16)
    t = dict(x=x, slots=torch.from_numpy(w.slots).to(dev),
             gamma=None if w.gamma is None else to_dev_bf16(w.gamma, dev),
             cos=None if w.cos is None else to_dev_bf16(w.cos, dev),
             sin=None if w.sin is None else to_dev_bf16(w.sin, dev))
    t["cache"], t["flat"] = cache_tensor(w.cache, w.cache_init, dev)
    t["aux"] = t["aflat"] = None
    if w.aux is not None:
        t["aux"], t["aflat"] = cache_tensor(w.aux, w.aux_init, dev)
    return t


def _prepare(w, t):
    from kv_cache_epilog_amd import kvepi_prepare
    ix = dict(index_mode=w.index_mode, seq_len=w.seq_len)
    return kvepi_prepare(t["x"], t["slots"], t["cache"], w.mode, w.group_size, gamma=t["gamma"],
                         cos=t["cos"], sin=t["sin"], cache_aux=t["aux"], eps=w.eps, **ix)


def _refill(t, w):
    """Writes w's inputs (x, slots, gamma, cos, sin) into the tensors of t,
    in place."""
    import torch
    t["x"].view(torch.int16).copy_(torch.from_numpy(w.x.view(np.int16)))
    t["slots"].copy_(torch.from_numpy(w.slots))
    for k in ("gamma", "cos", "sin"):
        if t[k] is not None:
            t[k].view(torch.int16).copy_(torch.from_numpy(getattr(w, k).view(np.int16)))


def _got(w, t):
    got = t["flat"][:w.cache.alloc_bytes].cpu().numpy()
    agot = None if w.aux is None else t["aflat"][:w.aux.alloc_bytes].cpu().numpy()
    return got, agot


@pytest.mark.parametrize("kind", ["fused", "mxfp4", "batch_index"])
def test_prepared_runs_read_the_current_contents(kind):
    """One preparation, three runs: each with new x, slot and cos / sin
    values written into the same tensors; the cache keeps the earlier runs'
    rows wherever the new slots do not reach."""
    import torch
    from kv_cache_epilog_amd import kvepi_run_prepared
    seed = 200 + 10 * ["fused", "mxfp4", "batch_index"].index(kind)
    w = _case(kind, seed)
    t = _upload(w, "cuda:0")
    prep = _prepare(w, t)
    for r in range(3):
        wr = _case(kind, seed + r)
        wr.cache_init = w.cache_init  # the cache as the previous run left it
        wr.aux_init = w.aux_init
        want, awant = run_oracle(wr)
        _refill(t, wr)
        kvepi_run_prepared(prep)
        torch.cuda.synchronize()
        got, agot = _got(w, t)
        assert np.array_equal(got, want), f"run {r}"
        if awant is not None:
            assert np.array_equal(agot, awant), f"run {r}"
        w.cache_init, w.aux_init = want, awant


@pytest.mark.parametrize("kind", ["fused", "mxfp4"])
def test_prepared_graph_replays(kind):
    """A prepared call captured in a HIP graph: every replay, after eager
    work of the program's own (a refill of the inputs and of the cache) and
    a synchronisation, writes what the oracle writes for the inputs of that
    replay."""
    import torch
    from kv_cache_epilog_amd import kvepi_run_prepared
    seed = 300 + 10 * ["fused", "mxfp4"].index(kind)
    w = _case(kind, seed)
    t = _upload(w, "cuda:0")
    prep = _prepare(w, t)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        kvepi_run_prepared(prep)  # warm-up outside the capture
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        kvepi_run_prepared(prep)
    init = torch.from_numpy(w.cache_init).to("cuda:0")
    ainit = None if w.aux_init is None else torch.from_numpy(w.aux_init).to("cuda:0")
    for r in range(3):
        wr = _case(kind, seed + r)
        want, awant = run_oracle(wr)
        _refill(t, wr)
        t["flat"][:w.cache.alloc_bytes].copy_(init)
        if ainit is not None:
            t["aflat"][:w.aux.alloc_bytes].copy_(ainit)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got, agot = _got(w, t)
        assert np.array_equal(got, want), f"replay {r}"
        if awant is not None:
            assert np.array_equal(agot, awant), f"replay {r}"


def test_prepared_empty_call_is_a_no_op():
    import torch
    from kv_cache_epilog_amd import kvepi_prepare, kvepi_run_prepared
    dev = "cuda:0"
    x = torch.empty(0, 576, dtype=torch.bfloat16, device=dev)
    slots = torch.empty(0, dtype=torch.int32, device=dev)
    cache = torch.full((2, 16, 1, 672), 0xAB, dtype=torch.uint8, device=dev)
    prep = kvepi_prepare(x, slots, cache, 0, 64)
    kvepi_run_prepared(prep)
    torch.cuda.synchronize()
    assert bool((cache == 0xAB).all())


def test_prepared_grid_is_fixed_at_preparation(monkeypatch):
    """KVEPI_MAX_WAVES is read when the call is prepared: a call prepared
    with a cap of 8 waves keeps that grid (many iterations per wave) after
    the cap is gone, and still writes the oracle's bytes."""
    monkeypatch.setenv("KVEPI_MAX_WAVES", "8")
    w = _case("fused", 400)
    t = _upload(w, "cuda:0")
    prep = _prepare(w, t)
    monkeypatch.delenv("KVEPI_MAX_WAVES")
    import torch
    from kv_cache_epilog_amd import kvepi_run_prepared
    kvepi_run_prepared(prep)
    torch.cuda.synchronize()
    want, _ = run_oracle(w)
    got, _ = _got(w, t)
    assert np.array_equal(got, want)


# ---- the seeded random workloads of the other parity files, prepared ------------

@pytest.mark.parametrize("k", range(0, 160, 4))
def test_prepared_fuzz(k):
    from test_gpu_parity import _fuzz_case
    w, kw = _fuzz_case(k)
    assert check(w, f"prepared fuzz {k}: {w.name}", prepared=True, repeat=2, **kw) == 0


@pytest.mark.parametrize("k", range(0, 60, 3))
def test_prepared_index_fuzz(k):
    from test_gpu_options import _index_fuzz_case
    check(_index_fuzz_case(k), f"prepared index fuzz {k}", prepared=True)


@pytest.mark.parametrize("k", range(0, 30, 3))
def test_prepared_rope_length_fuzz(k):
    from test_gpu_options import _rope_length_fuzz_case
    w, x_pad = _rope_length_fuzz_case(k)
    check(w, f"prepared rope length fuzz {k}", prepared=True, x_pad=x_pad)
