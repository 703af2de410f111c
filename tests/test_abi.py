"""The C ABI without a GPU: the library loads, exports every function that
include/kvepi.h declares, reports the page's row geometry, and rejects bad
arguments before any launch (validation is pure host code; device pointers
are only checked for NULL and alignment, never dereferenced)."""
import ctypes
import os
import re

import pytest

from kv_cache_epilog_amd import binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADERS = [os.path.join(ROOT, "include", n) for n in sorted(os.listdir(os.path.join(ROOT, "include")))
           if n.endswith(".h")]
GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def declared_functions():
    text = "".join(open(h).read() for h in HEADERS)
    return sorted(set(re.findall(r"KVEPI_API\s+[\w\s\*]*?\b(kvepi_\w+)\s*\(", text)))


def test_exports_every_declared_symbol():
    names = declared_functions()
    assert set(names) == {"kvepi_row_bytes", "kvepi_get_workspace", "kvepi_run",
                          "kvepi_get_workspace_ex", "kvepi_run_ex", "kvepi_status_str",
                          "kvepi_version", "kvepi_drq_get_workspace", "kvepi_drq_run",
                          "kvepi_prepare_ex", "kvepi_run_prepared"}
    L = B.lib()
    for n in names:
        assert hasattr(L, n), n


def test_only_the_c_abi_is_exported():
    import subprocess
    out = subprocess.run(["nm", "-D", "--defined-only", B.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    funcs = {line.split()[-1] for line in out.splitlines() if " T " in line}
    assert funcs == set(declared_functions()), funcs


def test_version_and_status_strings():
    assert B.kvepi_version() == 140
    for code, name in B.STATUS_NAMES.items():
        assert B.kvepi_status_str(code).startswith(name)
    assert "UNKNOWN" in B.kvepi_status_str(99)


def _golden_rows():
    rows = []
    with open(os.path.join(GOLDEN, "row_bytes.txt")) as f:
        for line in f:
            line = line.split("#")[0].strip()
            if line:
                rows.append(tuple(int(v) for v in line.split()[:6]))
    return rows


@pytest.mark.parametrize("row", _golden_rows())
def test_row_bytes_page_values(row):
    mode, d, g, cc, kc, sc = row
    assert B.kvepi_row_bytes(mode, d, g) == (cc, kc, sc)


@pytest.mark.parametrize("mode,d,g,status", [
    (2, 256, 64, 5), (8, 256, 64, 5), (7, 256, 8, 4), (7, 256, 128, 4), (7, 100, 32, 2),
    (7, 8256, 64, 2), (0, 100, 64, 2), (0, 64, 64, 2), (1, 8256, 64, 2),
    (0, 256, 32, 4), (3, 48, 32, 2), (3, 128, 64, 4), (3, 8224, 32, 2),
    (5, 48, 32, 2), (5, 128, 64, 4), (5, 8224, 32, 2), (6, 96, 32, 4), (6, 48, 0, 2),
    (6, 128, 64, 4)])
def test_row_bytes_rejects(mode, d, g, status):
    with pytest.raises(B.KvepiError) as e:
        B.kvepi_row_bytes(mode, d, g)
    assert e.value.status == status


# ---- validation through both stages, with fake (never dereferenced) pointers --

P16 = 0x10000  # 16-byte-aligned stand-in device addresses
P16B = 0x20000
P16C = 0x30000
P16D = 0x40000


def _cache(data=0x50000, bn=8, bs=16, hd=352, stride=None):
    return B.kvepi_cache(data, bn, bs, hd, bs * hd if stride is None else stride)


def call(stage, *, x=P16, T=64, d=256, xs=None, gamma=None, cos=None, sin=None, slots=P16B,
         cache=None, aux=None, mode=0, group=64, eps=1e-6, ws_bytes=0):
    L = B.lib()
    cache = _cache() if cache is None else cache
    xs = d if xs is None else xs
    cp = ctypes.byref(cache) if cache is not False else None
    ap = ctypes.byref(aux) if aux is not None else None
    if stage == 1:
        ws = ctypes.c_uint64(123)
        st = L.kvepi_get_workspace(x, T, d, xs, gamma, cos, sin, slots, cp, ap, mode, group,
                                   ctypes.c_float(eps), ctypes.byref(ws))
        return st, ws.value
    if stage == 3:
        # kvepi_prepare_ex: the checks of stage one, then the device query
        prep = B.kvepi_prepared()
        prep.opaque[0] = 0xFFFF  # overwritten: invalid unless KVEPI_OK
        st = L.kvepi_prepare_ex(x, T, d, xs, gamma, cos, sin, slots, cp, ap, mode, group,
                                ctypes.c_float(eps), None, ctypes.byref(prep))
        return st, prep
    # stage 2: a valid call would launch -- only invalid calls are made here
    st = L.kvepi_run(x, T, d, xs, gamma, cos, sin, slots, cp, ap, mode, group,
                     ctypes.c_float(eps), None, ws_bytes, None)
    return st, None


def test_valid_call_reports_zero_workspace():
    assert call(1) == (0, 0)
    assert call(1, T=0, x=None, slots=None) == (0, 0)
    assert call(1, d=576, cache=_cache(hd=672), gamma=P16C, cos=P16D, sin=P16D + 0x1000) == (0, 0)
    aux = _cache(data=0x60000, hd=4)
    assert call(1, d=128, mode=3, group=32, cache=_cache(hd=64), aux=aux) == (0, 0)
    assert call(1, d=576, mode=1, cache=_cache(hd=648)) == (0, 0)
    assert call(1, d=128, mode=5, group=32, cache=_cache(hd=128), aux=aux) == (0, 0)
    assert call(1, d=128, mode=6, group=0, cache=_cache(hd=128),
                aux=_cache(data=0x60000, hd=1)) == (0, 0)
    assert call(1, d=128, mode=6, group=128, cache=_cache(hd=128),
                aux=_cache(data=0x60004, hd=3)) == (0, 0)
    ckv = _cache(hd=512)
    k = _cache(data=0x70000, hd=64)
    assert call(1, d=576, mode=4, cache=ckv, aux=k, gamma=P16C, cos=P16D,
                sin=P16D + 0x1000) == (0, 0)
    # the FP4 nope mode, with and without RMSNorm, any of its group sizes
    for g, hd in ((16, 384), (32, 352), (64, 352)):
        assert call(1, d=576, mode=7, group=g, cache=_cache(hd=hd)) == (0, 0)
    assert call(1, d=576, mode=7, group=32, cache=_cache(hd=352), gamma=P16C) == (0, 0)


BAD = [
    # (description, kwargs, expected status)
    ("mode 2 (HiFloat8)", dict(mode=2), 5),
    ("fp4 nope with RoPE", dict(mode=7, d=576, group=32, cache=_cache(hd=352), cos=P16C,
                                sin=P16D), 4),
    ("fp4 nope with an aux cache", dict(mode=7, d=576, group=32, cache=_cache(hd=352),
                                        aux=_cache(hd=4)), 4),
    ("fp4 nope group 8", dict(mode=7, d=576, group=8, cache=_cache(hd=352)), 4),
    ("fp4 nope headDim below kvCacheCol", dict(mode=7, d=576, group=16, cache=_cache(hd=383)),
     2),
    ("unknown mode", dict(mode=9), 5),
    ("d not a multiple of 64", dict(d=200), 2),
    ("d too large", dict(d=8256), 2),
    ("group size", dict(group=32), 4),
    ("negative T", dict(T=-1), 2),
    ("null x", dict(x=None), 1),
    ("null slots", dict(slots=None), 1),
    ("null cache", dict(cache=False), 1),
    ("null cache data", dict(cache=B.kvepi_cache(None, 8, 16, 352, 16 * 352)), 1),
    ("x misaligned", dict(x=P16 + 2), 3),
    ("x row stride < d", dict(xs=128), 3),
    ("x row stride not 16 B", dict(xs=260), 3),
    ("x row stride over 2^27", dict(xs=(1 << 27) + 8), 3),
    ("slots misaligned", dict(slots=P16B + 2), 3),
    ("cos without sin", dict(cos=P16C), 4),
    ("negative eps", dict(gamma=P16C, eps=-1.0), 4),
    ("nan eps", dict(gamma=P16C, eps=float("nan")), 4),
    ("gamma misaligned", dict(gamma=P16C + 8), 3),
    ("headDim below kvCacheCol", dict(cache=_cache(hd=351)), 2),
    ("block stride too small", dict(cache=_cache(stride=16 * 352 - 1)), 3),
    ("zero blocks", dict(cache=_cache(bn=0)), 2),
    ("num_slots over int32", dict(cache=_cache(bn=1 << 20, bs=1 << 12)), 2),
    ("aux given to mode 0", dict(aux=_cache(hd=4)), 4),
    ("mxfp4 without cache_scale", dict(mode=3, d=128, group=32, cache=_cache(hd=64)), 1),
    ("mxfp4 with gamma", dict(mode=3, d=128, group=32, cache=_cache(hd=64), gamma=P16C,
                              aux=_cache(hd=4)), 5),
    ("mxfp4 cache_scale too narrow", dict(mode=3, d=128, group=32, cache=_cache(hd=64),
                                          aux=_cache(hd=3)), 2),
    ("mxfp4 cache_scale other block count", dict(mode=3, d=128, group=32,
                                                 cache=_cache(hd=64), aux=_cache(bn=4, hd=4)), 2),
    ("mxfp8 without cache_scale", dict(mode=5, d=128, group=32, cache=_cache(hd=128)), 1),
    ("mxfp8 with rope", dict(mode=5, d=128, group=32, cache=_cache(hd=128), cos=P16C,
                             sin=P16D, aux=_cache(hd=4)), 5),
    ("mxfp8 cache too narrow", dict(mode=5, d=128, group=32, cache=_cache(hd=127),
                                    aux=_cache(hd=4)), 2),
    ("mxfp8 cache_scale too narrow", dict(mode=5, d=128, group=32, cache=_cache(hd=128),
                                          aux=_cache(hd=3)), 2),
    ("fp8 row with gamma", dict(mode=6, d=128, group=0, cache=_cache(hd=128), gamma=P16C,
                                aux=_cache(hd=1)), 5),
    ("fp8 row without cache_scale", dict(mode=6, d=128, group=0, cache=_cache(hd=128)), 1),
    ("fp8 row scale cache misaligned", dict(mode=6, d=128, group=0, cache=_cache(hd=128),
                                            aux=_cache(data=0x60002, hd=1)), 3),
    ("fp8 row group size", dict(mode=6, d=128, group=32, cache=_cache(hd=128),
                                aux=_cache(hd=1)), 4),
    ("split without rope", dict(mode=4, d=576, gamma=P16C, cache=_cache(hd=512),
                                aux=_cache(hd=64)), 4),
    ("split k cache too narrow", dict(mode=4, d=576, gamma=P16C, cos=P16D, sin=P16D,
                                      cache=_cache(hd=512), aux=_cache(hd=63)), 2),
    ("split ckv misaligned", dict(mode=4, d=576, gamma=P16C, cos=P16D, sin=P16D,
                                  cache=_cache(data=0x50001, hd=512), aux=_cache(hd=64)), 3),
]


@pytest.mark.parametrize("desc,kw,status", BAD, ids=[b[0] for b in BAD])
@pytest.mark.parametrize("stage", [1, 2, 3])
def test_rejects(desc, kw, status, stage):
    st, prep = call(stage, **kw)
    assert st == status, (desc, B.kvepi_status_str(st))
    if stage == 3:
        # a rejected preparation leaves a struct that kvepi_run_prepared refuses
        assert not any(prep.opaque)
        assert B.lib().kvepi_run_prepared(ctypes.byref(prep), None) == 4


def test_workspace_out_pointer_required():
    L = B.lib()
    c = _cache()
    st = L.kvepi_get_workspace(P16, 64, 256, 256, None, None, None, P16B, ctypes.byref(c), None,
                               0, 64, ctypes.c_float(1e-6), None)
    assert st == 1


def test_binding_refuses_to_run_without_library(monkeypatch, tmp_path):
    monkeypatch.setattr(B, "_lib", None)
    monkeypatch.setattr(B, "LIB_PATH", str(tmp_path / "missing.so"))
    with pytest.raises(RuntimeError, match="missing"):
        B.lib()


# ---- options: fp16 rows and index modes ----------------------------------------

def call_ex(stage, opt, **kw):
    """call() through the _ex entry points with a kvepi_options (or None)."""
    L = B.lib()
    x = kw.pop("x", P16)
    T = kw.pop("T", 64)
    d = kw.pop("d", 256)
    cache = kw.pop("cache", _cache())
    aux = kw.pop("aux", None)
    mode = kw.pop("mode", 0)
    group = kw.pop("group", 64)
    slots = kw.pop("slots", P16B)
    gamma, cos, sin = kw.pop("gamma", None), kw.pop("cos", None), kw.pop("sin", None)
    assert not kw
    ap = ctypes.byref(aux) if aux is not None else None
    op = ctypes.byref(opt) if opt is not None else None
    if stage == 1:
        ws = ctypes.c_uint64(7)
        st = L.kvepi_get_workspace_ex(x, T, d, d, gamma, cos, sin, slots, ctypes.byref(cache),
                                      ap, mode, group, ctypes.c_float(1e-6), op,
                                      ctypes.byref(ws))
        return st, ws.value
    if stage == 3:
        prep = B.kvepi_prepared()
        st = L.kvepi_prepare_ex(x, T, d, d, gamma, cos, sin, slots, ctypes.byref(cache), ap,
                                mode, group, ctypes.c_float(1e-6), op, ctypes.byref(prep))
        return st, prep
    st = L.kvepi_run_ex(x, T, d, d, gamma, cos, sin, slots, ctypes.byref(cache), ap, mode,
                        group, ctypes.c_float(1e-6), op, None, 0, None)
    return st, None


def O(x_dtype=0, index_mode=0, seq_len=0, rope_dim=0, reserved=0):
    return B.kvepi_options(x_dtype, index_mode, seq_len, rope_dim, reserved)


def test_ex_valid_calls():
    assert call_ex(1, None) == (0, 0)
    assert call_ex(1, O()) == (0, 0)
    ix = dict(d=128, group=32, cache=_cache(hd=128), aux=_cache(data=0x60000, hd=4))
    for mode, g in ((3, 32), (5, 32)):
        kw = dict(ix, mode=mode, group=g)
        if mode == 3:
            kw["cache"] = _cache(hd=64)
        assert call_ex(1, O(x_dtype=1), **kw) == (0, 0)
    assert call_ex(1, O(x_dtype=1), d=128, mode=6, group=0, cache=_cache(hd=128),
                   aux=_cache(data=0x60000, hd=1)) == (0, 0)
    # 64 tokens as 8 batches of 8 (cache of 8 blocks of 16 rows)
    for im in (1, 2, 3):
        assert call_ex(1, O(index_mode=im, seq_len=8)) == (0, 0)
    assert call_ex(1, O(index_mode=2, seq_len=64)) == (0, 0)
    assert call_ex(1, O(index_mode=1, seq_len=1), T=0, x=None, slots=None) == (0, 0)
    # the split mode with a 32-column rope segment: ckv rows 544, k rows 32
    assert call_ex(1, O(rope_dim=32), d=576, mode=4, gamma=P16C, cos=P16D,
                   sin=P16D + 0x1000, cache=_cache(hd=544),
                   aux=_cache(data=0x70000, hd=32)) == (0, 0)
    assert call_ex(1, O(rope_dim=64), d=576, mode=4, gamma=P16C, cos=P16D,
                   sin=P16D + 0x1000, cache=_cache(hd=512),
                   aux=_cache(data=0x70000, hd=64)) == (0, 0)


BAD_EX = [
    ("unknown x dtype", O(x_dtype=2), {}, 4),
    ("fp16 in mode 0", O(x_dtype=1), {}, 5),
    ("unknown index mode", O(index_mode=4), {}, 4),
    ("negative index mode", O(index_mode=-1), {}, 4),
    ("batch mode without seq_len", O(index_mode=1), {}, 2),
    ("seq_len not dividing T", O(index_mode=2, seq_len=7), {}, 2),
    ("more batches than blocks", O(index_mode=1, seq_len=4), {}, 2),
    ("batch start longer than a block", O(index_mode=3, seq_len=32), dict(T=64), 2),
    ("more start batches than blocks", O(index_mode=3, seq_len=2), {}, 2),
    ("reserved field set", O(reserved=1), {}, 4),
    ("rope length in mode 0", O(rope_dim=32), {}, 4),
    ("odd rope length in the split mode", O(rope_dim=33), dict(d=576, mode=4), 4),
    ("rope length above 128", O(rope_dim=130), dict(d=578, mode=4), 4),
    ("Dv not a multiple of 8", O(rope_dim=36), dict(d=576, mode=4), 2),
]


@pytest.mark.parametrize("desc,opt,kw,status", BAD_EX, ids=[b[0] for b in BAD_EX])
@pytest.mark.parametrize("stage", [1, 2, 3])
def test_ex_rejects(desc, opt, kw, status, stage):
    st, _ = call_ex(stage, opt, **kw)
    assert st == status, (desc, B.kvepi_status_str(st))



def test_valid_run_without_a_device_reports_runtime_error():
    # on a host without a GPU a valid call reaches the launch, which the HIP
    # runtime refuses: KVEPI_ERR_RUNTIME, not a crash
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is present")
    assert call(2) == (7, None)
    assert call_ex(2, O(index_mode=2, seq_len=8)) == (7, None)


def test_slot_check_without_a_device_reports_runtime_error(monkeypatch):
    # the debug check copies the slots to the host before the launch: on a
    # host without a GPU that copy fails, KVEPI_ERR_RUNTIME, not a crash
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is present")
    monkeypatch.setenv("KVEPI_CHECK_SLOTS", "1")
    assert call(2) == (7, None)


# ---- prepared calls ----------------------------------------------------------

def test_prepare_needs_its_out_pointer():
    L = B.lib()
    c = _cache()
    assert L.kvepi_prepare_ex(P16, 64, 256, 256, None, None, None, P16B, ctypes.byref(c), None,
                              0, 64, ctypes.c_float(1e-6), None, None) == 1


def test_run_prepared_refuses_null_and_unprepared_structs():
    L = B.lib()
    assert L.kvepi_run_prepared(None, None) == 1
    prep = B.kvepi_prepared()
    assert L.kvepi_run_prepared(ctypes.byref(prep), None) == 4
    for i in range(len(prep.opaque)):
        prep.opaque[i] = 0x0123456789ABCDEF
    assert L.kvepi_run_prepared(ctypes.byref(prep), None) == 4


def test_prepared_empty_call_runs_as_a_no_op():
    # num_tokens == 0 needs no device: prepared and run without one
    st, prep = call(3, T=0, x=None, slots=None)
    assert st == 0 and any(prep.opaque)
    assert B.lib().kvepi_run_prepared(ctypes.byref(prep), None) == 0
    st, prep = call_ex(3, O(index_mode=1, seq_len=1), T=0, x=None, slots=None)
    assert st == 0
    assert B.lib().kvepi_run_prepared(ctypes.byref(prep), None) == 0
    # a bytewise copy is as good as the original
    copy = B.kvepi_prepared.from_buffer_copy(prep)
    assert B.lib().kvepi_run_prepared(ctypes.byref(copy), None) == 0


def test_valid_prepare_without_a_device_reports_runtime_error():
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is present")
    st, prep = call(3)
    assert st == 7 and not any(prep.opaque)
    st, prep = call_ex(3, O(index_mode=2, seq_len=8))
    assert st == 7


@pytest.mark.parametrize("header", ["kvepi.h", "kvepi_drq.h"])
@pytest.mark.parametrize("lang,std", [("c", "-std=c99"), ("c", "-std=c11"), ("c++", "-std=c++11")])
def test_headers_compile_as_strict_c_and_cxx(header, lang, std, tmp_path):
    # the ABI headers are plain C: no HIP or torch types, no compiler extensions
    import subprocess
    src = tmp_path / ("t.c" if lang == "c" else "t.cpp")
    src.write_text(f'#include "{header}"\n#include "{header}"\nint main(void) {{ return 0; }}\n')
    cc = "gcc" if lang == "c" else "g++"
    r = subprocess.run([cc, std, "-Wall", "-Wextra", "-pedantic", "-Werror", "-fsyntax-only",
                        "-I", os.path.join(ROOT, "include"), str(src)],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr


def test_prepared_struct_size_matches_the_header():
    import re as _re
    text = open(os.path.join(ROOT, "include", "kvepi.h")).read()
    n = int(_re.search(r"#define KVEPI_PREPARED_BYTES (\d+)", text).group(1))
    assert ctypes.sizeof(B.kvepi_prepared) == n == 1024
    assert ctypes.alignment(B.kvepi_prepared) == 8
