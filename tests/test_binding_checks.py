"""The binding's own checks (no device needed): what the C ABI's plain
pointers cannot carry -- the device a tensor lives on, the element types of
the caches and the lengths of gamma, cos, sin and the index array -- raises
ValueError before any call.  Tensors on the 'meta' device stand in for GPU
tensors (nothing is dereferenced)."""
import pytest
import torch

from kv_cache_epilog_amd import binding as B

META = "meta"


def t(*shape, dtype=torch.bfloat16, device=META):
    return torch.empty(*shape, dtype=dtype, device=device)


def cache(bn=4, bs=16, hd=352, dtype=torch.uint8, device=META):
    return torch.empty(bn, bs, 1, hd, dtype=dtype, device=device)


def args(**kw):
    a = dict(x=t(64, 576), slot_mapping=t(64, dtype=torch.int32), cache=cache(hd=672),
             quant_mode=0, group_size=64, gamma=t(512), cos=t(64, 64), sin=t(64, 64),
             cache_aux=None, eps=1e-6)
    a.update(kw)
    return a


def call(**kw):
    a = args(**kw)
    extra = {k: a.pop(k) for k in ("index_mode", "seq_len", "rope_dim") if k in a}
    return B._args(a["x"], a["slot_mapping"], a["cache"], a["quant_mode"], a["group_size"],
                   a["gamma"], a["cos"], a["sin"], a["cache_aux"], a["eps"], **extra)


def test_valid_arguments_pass():
    call()
    call(quant_mode=7, group_size=32, cache=cache(hd=352), cos=None, sin=None)
    call(quant_mode=6, group_size=0, x=t(64, 128), gamma=None, cos=None, sin=None,
         cache=cache(hd=128), cache_aux=cache(hd=1, dtype=torch.float32))
    call(quant_mode=4, cache=cache(hd=512, dtype=torch.bfloat16),
         cache_aux=cache(hd=64, dtype=torch.bfloat16))
    # index modes: [B, ceil(S / block_size)] and [B]
    call(slot_mapping=t(2 * 2, dtype=torch.int32), index_mode=B.KVEPI_INDEX_BLOCK, seq_len=32)
    call(slot_mapping=t(4, dtype=torch.int32), index_mode=B.KVEPI_INDEX_BATCH_START,
         seq_len=16)


@pytest.mark.parametrize("kw", [
    dict(x=t(64, 576, device="cpu")),                                   # host x
    dict(slot_mapping=t(64, dtype=torch.int32, device="cpu")),          # host slots
    dict(gamma=t(512, device="cpu")),                                   # host gamma
    dict(cache=cache(hd=672, device="cpu")),                            # host cache
    dict(slot_mapping=t(64, dtype=torch.int64)),                        # not int32
    dict(slot_mapping=t(63, dtype=torch.int32)),                        # one per token
    dict(gamma=t(511)),                                                 # short gamma
    dict(cos=t(63, 64)),                                                # short cos
    dict(sin=t(64, 32)),                                                # short sin
    dict(cos=t(64, 64, dtype=torch.float32)),                           # not 16-bit
    dict(cache=cache(hd=672, dtype=torch.bfloat16)),                    # mode 0 is uint8
    dict(quant_mode=4, cache=cache(hd=512), cache_aux=cache(hd=64, dtype=torch.bfloat16)),
    dict(quant_mode=6, group_size=0, x=t(64, 128), gamma=None, cos=None, sin=None,
         cache=cache(hd=128), cache_aux=cache(hd=4)),                   # fp32 cache_scale
    dict(quant_mode=3, group_size=32, x=t(64, 128), gamma=None, cos=None, sin=None,
         cache=cache(hd=64), cache_aux=cache(hd=4, dtype=torch.float32)),
    dict(slot_mapping=t(7, dtype=torch.int32), index_mode=B.KVEPI_INDEX_BLOCK, seq_len=16),
    dict(slot_mapping=t(64, dtype=torch.int32), index_mode=B.KVEPI_INDEX_BATCH_START,
         seq_len=16),
    dict(slot_mapping=t(64, dtype=torch.int32), index_mode=B.KVEPI_INDEX_BATCH_START,
         seq_len=5),                                                    # 5 does not divide 64
])
def test_misuse_raises(kw):
    with pytest.raises(ValueError):
        call(**kw)


def drq(**kw):
    T, nq, nkv, D = 32, 2, 1, 64
    H = (nq + 2 * nkv) * D
    a = dict(x=t(T, H, dtype=torch.int32), cos=t(T, D, dtype=torch.float16),
             sin=t(T, D, dtype=torch.float16), k_cache=cache(hd=64), v_cache=cache(hd=64),
             indices=t(T, dtype=torch.int32), nq=nq, nkv=nkv, head_dim=D,
             scale_k=t(nkv * D, dtype=torch.float32), scale_v=t(nkv * D, dtype=torch.float32),
             q_out=t(T, nq * D, dtype=torch.float16), weight_scale=t(H, dtype=torch.float32))
    a.update(kw)
    pos = [a.pop(k) for k in ("x", "cos", "sin", "k_cache", "v_cache", "indices")]
    return B.drq_params(*pos, **a)


def test_drq_valid_arguments_pass():
    drq()
    drq(k_out=t(32, 64, dtype=torch.float16), v_out=t(32, 64, dtype=torch.float16),
        act_scale=t(32, dtype=torch.float32), bias=t(256, dtype=torch.bfloat16))


def test_drq_params_hold_their_tensors():
    # the params keep every tensor they point into alive, temporaries included
    import gc
    import weakref
    sk = t(64, dtype=torch.float32)
    ref = weakref.ref(sk)
    p = drq(scale_k=sk)
    del sk
    gc.collect()
    assert ref() is not None and any(x is ref() for x in p._tensors)
    del p
    gc.collect()
    assert ref() is None


@pytest.mark.parametrize("kw", [
    dict(x=t(32, 256, dtype=torch.int32, device="cpu")),
    dict(scale_k=t(64, dtype=torch.float32, device="cpu")),
    dict(scale_k=t(64, dtype=torch.float16)),
    dict(scale_v=t(63, dtype=torch.float32)),
    dict(q_out=t(32, 100, dtype=torch.float16)),
    dict(q_out=t(32, 128, dtype=torch.bfloat16)),       # outputs take cos's dtype
    dict(indices=t(32, dtype=torch.int64)),
    dict(indices=t(31, dtype=torch.int32)),
    dict(k_cache=cache(hd=64, dtype=torch.bfloat16)),
    dict(cos=t(32, 32, dtype=torch.float16)),
    dict(weight_scale=t(255, dtype=torch.float32)),
    dict(x=t(32, 255, dtype=torch.int32)),               # H = (nq + 2 nkv) * D
])
def test_drq_misuse_raises(kw):
    with pytest.raises(ValueError):
        drq(**kw)


@pytest.mark.parametrize("kw", [dict(x=t(64, 576, device="cpu")),
                                dict(slot_mapping=t(63, dtype=torch.int32))])
def test_prepare_checks_as_run(kw):
    # kvepi_prepare shares kvepi_run's checks: they raise before any call
    a = args(**kw)
    with pytest.raises(ValueError):
        B.kvepi_prepare(a.pop("x"), a.pop("slot_mapping"), a.pop("cache"), a.pop("quant_mode"),
                        a.pop("group_size"), **a)
