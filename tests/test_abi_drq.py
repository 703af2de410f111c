"""The dequant -> RoPE -> int8 KV cache operator's C ABI without a GPU:
validation of kvepi_drq_params in both stages (fake device pointers, never
dereferenced)."""
import ctypes

import pytest

from kv_cache_epilog_amd import binding as B

A = 0x100000  # 16-byte-aligned stand-in device addresses


def cache(data=0x900000, bn=4, bs=16, hd=128, stride=None):
    return B.kvepi_cache(data, bn, bs, hd, bs * hd if stride is None else stride)


def params(**kw):
    # int32 x [8, 512] (nq 2, nkv 1, D 128), bf16 outputs, page mode
    p = dict(x=A, x_dtype=B.KVEPI_DT_INT32, out_dtype=B.KVEPI_DT_BF16, num_tokens=8,
             x_row_stride=512, nq=2, nkv=1, head_dim=128, cos=A + 0x10000, sin=A + 0x20000,
             weight_scale=A + 0x30000, act_scale=None, bias=None, bias_dtype=B.KVEPI_DT_FP32,
             scale_k=A + 0x40000, scale_v=A + 0x50000, offset_k=None, offset_v=None,
             indices=A + 0x60000, cache_mode=B.KVEPI_DRQ_PAGE, seq_len=0, k_cache=cache(),
             v_cache=cache(data=0xA00000), q_out=A + 0x70000, k_out=None, v_out=None)
    p.update(kw)
    return B.kvepi_drq_params(**p)


def call(stage, p):
    L = B._drq_lib()
    if stage == 1:
        ws = ctypes.c_uint64(5)
        return L.kvepi_drq_get_workspace(ctypes.byref(p), ctypes.byref(ws)), ws.value
    return L.kvepi_drq_run(ctypes.byref(p), None, 0, None), None


def test_valid_calls_report_zero_workspace():
    assert call(1, params()) == (0, 0)
    assert call(1, params(x_dtype=B.KVEPI_DT_FP16, out_dtype=B.KVEPI_DT_FP16,
                          weight_scale=None)) == (0, 0)
    assert call(1, params(bias=A + 0x80000, bias_dtype=B.KVEPI_DT_BF16, act_scale=A + 4,
                          offset_k=A + 0x90000, offset_v=A + 0xA0000, k_out=A + 0xB0000,
                          v_out=A + 0xC0000)) == (0, 0)
    assert call(1, params(cache_mode=B.KVEPI_DRQ_CONTIGUOUS, seq_len=4)) == (0, 0)
    assert call(1, params(num_tokens=0, x=None, indices=None, cos=None, sin=None,
                          q_out=None)) == (0, 0)


BAD = [
    ("out dtype fp32", dict(out_dtype=B.KVEPI_DT_FP32), 4),
    ("16-bit x unlike the outputs", dict(x_dtype=B.KVEPI_DT_FP16, weight_scale=None), 4),
    ("int32 x without weight_scale", dict(weight_scale=None), 1),
    ("weight_scale with 16-bit x", dict(x_dtype=B.KVEPI_DT_BF16), 4),
    ("bias with 16-bit x", dict(x_dtype=B.KVEPI_DT_BF16, weight_scale=None, bias=A), 4),
    ("unknown bias dtype", dict(bias=A, bias_dtype=7), 4),
    ("head_dim not a multiple of 16", dict(head_dim=120, x_row_stride=480,
                                           k_cache=cache(hd=120), v_cache=cache(hd=120)), 2),
    ("H above 4096", dict(nq=31, x_row_stride=4224), 2),
    ("H not a multiple of 64", dict(head_dim=16, nq=1, nkv=1, x_row_stride=48), 2),
    ("no q heads", dict(nq=0), 2),
    ("x row stride below H", dict(x_row_stride=504), 3),
    ("x misaligned", dict(x=A + 4), 3),
    ("cos misaligned", dict(cos=A + 0x10008), 3),
    ("null cos", dict(cos=None), 1),
    ("null indices", dict(indices=None), 1),
    ("null q_out", dict(q_out=None), 1),
    ("null scale_v", dict(scale_v=None), 1),
    ("k_out without v_out", dict(k_out=A + 0xB0000), 4),
    ("cache rows too short", dict(k_cache=cache(hd=120)), 2),
    ("cache not 8-byte aligned", dict(v_cache=cache(data=0xA00004)), 3),
    ("cache blocks differ", dict(v_cache=cache(data=0xA00000, bn=5)), 2),
    ("unknown cache mode", dict(cache_mode=2), 4),
    ("contiguous without seq_len", dict(cache_mode=B.KVEPI_DRQ_CONTIGUOUS), 2),
    ("contiguous seq_len not dividing T", dict(cache_mode=B.KVEPI_DRQ_CONTIGUOUS, seq_len=3), 2),
    ("contiguous more batches than blocks", dict(cache_mode=B.KVEPI_DRQ_CONTIGUOUS, seq_len=1), 2),
    ("contiguous seq_len above block size", dict(cache_mode=B.KVEPI_DRQ_CONTIGUOUS, seq_len=8,
                                                 k_cache=cache(bs=4, stride=1024),
                                                 v_cache=cache(data=0xA00000, bs=4,
                                                               stride=1024)), 2),
]


@pytest.mark.parametrize("desc,kw,status", BAD, ids=[b[0] for b in BAD])
@pytest.mark.parametrize("stage", [1, 2])
def test_rejects(desc, kw, status, stage):
    st, _ = call(stage, params(**kw))
    assert st == status, (desc, B.kvepi_status_str(st))


def test_null_params_and_workspace_pointer():
    L = B._drq_lib()
    ws = ctypes.c_uint64()
    assert L.kvepi_drq_get_workspace(None, ctypes.byref(ws)) == 1
    assert L.kvepi_drq_get_workspace(ctypes.byref(params()), None) == 1


def test_valid_run_without_a_device_reports_runtime_error():
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is present")
    assert call(2, params()) == (7, None)


def test_slot_check_without_a_device_reports_runtime_error(monkeypatch):
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is present")
    monkeypatch.setenv("KVEPI_CHECK_SLOTS", "1")
    assert call(2, params()) == (7, None)
