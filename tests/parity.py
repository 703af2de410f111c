"""Helpers for the GPU parity tests: run a kvgen.Workload through the C ABI on
the GPU and through the oracle on the CPU, and compare every cache byte.

The bar: every byte bit-exact, except that a quantised code may differ from
the oracle's by one code step on at most 1e-5 of the codes (a fp32 division
tie decided differently); differences are counted and reported."""
from __future__ import annotations

import numpy as np

import kvgen
import oracle

CODE_STEP_FRACTION = 1e-5


def _torch():
    import torch
    return torch


def to_dev_bf16(a, device):
    torch = _torch()
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(device)


def cache_tensor(spec: kvgen.CacheSpec, init: np.ndarray, device, offset: int = 0):
    """Device cache [block_num, block_size, 1, head_dim] over a flat buffer,
    starting `offset` bytes into it; returns (view, flat_buffer)."""
    torch = _torch()
    flat = torch.empty(spec.alloc_bytes + offset + 16, dtype=torch.uint8, device=device)
    flat.fill_(kvgen.PREFILL)
    flat[offset:offset + spec.alloc_bytes].copy_(torch.from_numpy(init))
    if spec.elem_bytes == 1:
        view = flat.as_strided((spec.block_num, spec.block_size, 1, spec.head_dim),
                               (spec.block_stride, spec.head_dim, spec.head_dim, 1), offset)
    else:
        # bf16 (2-byte) or fp32 (4-byte) elements
        e = spec.elem_bytes
        assert offset % e == 0
        n = flat.numel() // e * e
        b = flat[:n].view(torch.bfloat16 if e == 2 else torch.float32)
        view = b.as_strided((spec.block_num, spec.block_size, 1, spec.head_dim),
                            (spec.block_stride, spec.head_dim, spec.head_dim, 1), offset // e)
    return view, flat


def run_gpu(w: kvgen.Workload, device="cuda:0", offset: int = 0, aux_offset: int = 0,
            x_pad: int = 0, stream=None, repeat: int = 1, prepared: bool = False):
    """Runs the HIP path; returns (cache_bytes, aux_bytes) as numpy arrays.
    prepared: through kvepi_prepare / kvepi_run_prepared instead of
    kvepi_run."""
    torch = _torch()
    from kv_cache_epilog_amd import (kvepi_get_workspace, kvepi_prepare, kvepi_run,
                                     kvepi_run_prepared)
    if x_pad:
        xb = np.zeros((w.T, w.d + x_pad), np.uint16)
        xb[:, :w.d] = w.x
        x = to_dev_bf16(xb, device)[:, :w.d]
    else:
        x = to_dev_bf16(w.x, device)
    if w.x_fp16:
        x = x.view(torch.float16)
    slots = torch.from_numpy(w.slots).to(device)
    gamma = None if w.gamma is None else to_dev_bf16(w.gamma, device)
    cos = None if w.cos is None else to_dev_bf16(w.cos, device)
    sin = None if w.sin is None else to_dev_bf16(w.sin, device)
    cache, flat = cache_tensor(w.cache, w.cache_init, device, offset)
    aux = aflat = None
    if w.aux is not None:
        aux, aflat = cache_tensor(w.aux, w.aux_init, device, aux_offset)
    ix = dict(index_mode=w.index_mode, seq_len=w.seq_len)
    if w.rope_dim != 64:
        ix["rope_dim"] = w.rope_dim
    ws = kvepi_get_workspace(x, slots, cache, w.mode, w.group_size, gamma=gamma, cos=cos,
                             sin=sin, cache_aux=aux, eps=w.eps, **ix)
    assert ws == 0
    if prepared:
        prep = kvepi_prepare(x, slots, cache, w.mode, w.group_size, gamma=gamma, cos=cos,
                             sin=sin, cache_aux=aux, eps=w.eps, **ix)
    for _ in range(repeat):
        if prepared:
            kvepi_run_prepared(prep, stream=stream)
        else:
            kvepi_run(x, slots, cache, w.mode, w.group_size, gamma=gamma, cos=cos, sin=sin,
                      cache_aux=aux, eps=w.eps, stream=stream, **ix)
    torch.cuda.synchronize()
    got = flat[offset:offset + w.cache.alloc_bytes].cpu().numpy()
    # bytes outside the cache view must be untouched as well
    rest = torch.cat([flat[:offset], flat[offset + w.cache.alloc_bytes:]]).cpu().numpy()
    assert np.all(rest == kvgen.PREFILL), "bytes outside the cache were written"
    agot = None
    if aux is not None:
        agot = aflat[aux_offset:aux_offset + w.aux.alloc_bytes].cpu().numpy()
        arest = torch.cat([aflat[:aux_offset], aflat[aux_offset + w.aux.alloc_bytes:]])
        assert np.all(arest.cpu().numpy() == kvgen.PREFILL)
    return got, agot


def run_oracle(w: kvgen.Workload):
    cache = w.cache_init.copy()
    aux = None if w.aux_init is None else w.aux_init.copy()
    oracle.epilog(w.mode, w.x, w.slots, cache, w.cache.geom, group_size=w.group_size,
                  gamma=w.gamma, cos=w.cos, sin=w.sin, eps=w.eps, aux_bytes=aux,
                  aux_geom=None if w.aux is None else w.aux.geom, x_fp16=w.x_fp16,
                  index_mode=w.index_mode, seq_len=w.seq_len, rope_dim=w.rope_dim)
    return cache, aux


def token_slots(w: kvgen.Workload) -> np.ndarray:
    """The slot of every token (-1: skipped) under the workload's index mode."""
    if w.index_mode == 0:
        return np.where((w.slots >= 0) & (w.slots < w.cache.num_slots), w.slots, -1)
    return np.array([oracle.token_slot(w.index_mode, w.slots, t, w.seq_len, w.cache.block_num,
                                       w.cache.block_size) for t in range(w.T)], np.int64)


def _code_positions(w: kvgen.Workload):
    """Byte offsets of quantised codes in the main cache, and their count."""
    ts = token_slots(w)
    hit = ts[ts >= 0].astype(np.int64)
    start = 0
    if w.mode in (kvgen.MODE_FP8_BF16SCALE, kvgen.MODE_FP8_E8M0):
        ncode = w.d - 64
    elif w.mode == kvgen.MODE_FP4_NOPE:
        start, ncode = 64, (w.d - 64) // 2  # code bytes after the 64 rope bytes
    elif w.mode == kvgen.MODE_MXFP4:
        ncode = w.d // 2
    elif w.mode in (kvgen.MODE_MXFP8, kvgen.MODE_FP8_ROW):
        ncode = w.d
    else:
        return np.zeros(0, np.int64), 0
    blk, pos = np.divmod(hit, w.cache.block_size)
    base = blk * w.cache.block_stride + pos * w.cache.head_dim + start
    return (base[:, None] + np.arange(ncode)[None, :]).reshape(-1), hit.size * ncode


def _one_step(a, b, nib: bool):
    if nib:
        ok = True
        for sh in (0, 4):
            x, y = (a >> sh) & 0xF, (b >> sh) & 0xF
            if x != y and not ((x & 8) == (y & 8) and abs((x & 7) - (y & 7)) == 1):
                ok = False
        return ok
    return (a & 0x80) == (b & 0x80) and abs(int(a & 0x7F) - int(b & 0x7F)) == 1


def compare(w: kvgen.Workload, got, want, agot=None, awant=None, label=""):
    """Asserts the parity bar; returns the number of one-step code differences."""
    assert got.shape == want.shape
    diff = np.nonzero(got != want)[0]
    n_step = 0
    if diff.size:
        code_pos, n_codes = _code_positions(w)
        is_code = np.isin(diff, code_pos)
        bad = diff[~is_code]
        assert bad.size == 0, (
            f"{label}: {bad.size} non-code bytes differ, first at {bad[:8].tolist()}: "
            f"got {got[bad[:8]].tolist()} want {want[bad[:8]].tolist()}")
        nib = w.mode in (kvgen.MODE_MXFP4, kvgen.MODE_FP4_NOPE)
        steps = [_one_step(int(got[i]), int(want[i]), nib) for i in diff]
        assert all(steps), f"{label}: a code differs by more than one step"
        n_step = diff.size
        assert n_step <= CODE_STEP_FRACTION * n_codes, (
            f"{label}: {n_step} one-step code differences among {n_codes} codes")
    if awant is not None:
        adiff = np.nonzero(agot != awant)[0]
        assert adiff.size == 0, (f"{label}: {adiff.size} aux bytes differ, first at "
                                 f"{adiff[:8].tolist()}: got {agot[adiff[:8]].tolist()} "
                                 f"want {awant[adiff[:8]].tolist()}")
    return n_step


def check(w: kvgen.Workload, label="", **kw):
    got, agot = run_gpu(w, **kw)
    want, awant = run_oracle(w)
    return compare(w, got, want, agot, awant, label or w.name)


def _bf16_values(rng, n, emin, emax):
    e = rng.integers(emin, emax + 1, n).astype(np.float64)
    m = rng.integers(128, 256, n) / 128.0
    sg = np.where(rng.random(n) < 0.5, -1.0, 1.0)
    return kvgen.to_bf16(sg * m * 2.0 ** e)


def rope_product_cases(rng, n):
    """n quadruples (p, q, c, s) of bf16 bit patterns for which p*c + q*s
    rounded to bf16 differs between rounding each product on its own (the
    definition) and rounding p*c + RN(q*s) once (a fused multiply-add):
    tiny p, q and small c, s, so that the products underflow and round."""
    out = []
    while sum(len(o[0]) for o in out) < n:
        N = 1 << 20
        p, q = _bf16_values(rng, N, -126, -112), _bf16_values(rng, N, -126, -112)
        c, s = _bf16_values(rng, N, -30, -8), _bf16_values(rng, N, -30, -8)
        pf, qf, cf, sf = (kvgen.bf16_to_f32(v).astype(np.float32) for v in (p, q, c, s))
        sep = kvgen.to_bf16((pf * cf).astype(np.float32) + (qf * sf).astype(np.float32))
        qs = (qf * sf).astype(np.float32).astype(np.float64)
        fused = kvgen.to_bf16((pf.astype(np.float64) * cf.astype(np.float64) + qs)
                              .astype(np.float32))
        k = np.nonzero(sep != fused)[0]
        out.append((p[k], q[k], c[k], s[k]))
    return tuple(np.concatenate([o[i] for o in out])[:n] for i in range(4))


def plant_rope_cases(w, rng, dk):
    """Fills every rope pair of w with such cases: even tokens exercise the
    first half (y[j] = a c[j] - b s[j]), odd tokens the second half
    (y[j + dk/2] = b c[j + dk/2] + a s[j + dk/2])."""
    h = dk // 2
    p, q, c, s = rope_product_cases(rng, w.T * h)
    neg = lambda v: v ^ np.uint16(0x8000)  # noqa: E731  (bf16 negation)
    base = w.d - dk
    i = 0
    for t in range(w.T):
        for j in range(h):
            if t % 2 == 0:   # a = p, -b = q, c[j], s[j]
                w.x[t, base + 2 * j], w.x[t, base + 2 * j + 1] = p[i], neg(q[i])
                w.cos[t, j], w.sin[t, j] = c[i], s[i]
            else:            # b = p, a = q, c[j + h], s[j + h]
                w.x[t, base + 2 * j + 1], w.x[t, base + 2 * j] = p[i], q[i]
                w.cos[t, j + h], w.sin[t, j + h] = c[i], s[i]
            i += 1
    return i
