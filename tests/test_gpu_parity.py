"""GPU parity of the HIP path (through the C ABI) against the CPU oracle.

Every test compares the whole cache allocation byte for byte (plus guard
bytes around it), so routing, skipped tokens, untouched rows, block gaps and
bytes past kvCacheCol are all checked, not only the written rows."""
import numpy as np
import pytest

import kvgen
from kvgen import CacheSpec

from parity import check, compare, run_gpu, run_oracle

pytestmark = pytest.mark.gpu


def _small(mode, T, d, *, seed, bs=16, head=None, stride_extra=0, aux_head=None,
           norm=False, rope=False, skip=0.1, row_sigma=0.0, **kw):
    import oracle
    group = {3: 32, 5: 32, 6: 0}.get(mode, 64)
    _, kc, sc = oracle.row_bytes(mode, d, group) if mode != 4 else (0, d - 64, 64)
    head = head or kc
    nblk = (T + bs - 1) // bs + 2
    cache = CacheSpec(nblk, bs, head, bs * head + stride_extra, 2 if mode == 4 else 1)
    aux = None
    if mode in (3, 5):
        ah = aux_head or sc
        aux = CacheSpec(nblk, bs, ah, bs * ah + stride_extra)
    elif mode == 6:
        ah = aux_head or 1
        aux = CacheSpec(nblk, bs, ah, bs * ah + stride_extra, 4)
    elif mode == 4:
        ah = aux_head or 64
        aux = CacheSpec(nblk, bs, ah, bs * ah + stride_extra, 2)
    return kvgen.make(f"m{mode}_d{d}_T{T}", mode, T, d, seed=seed, cache=cache, aux=aux,
                      norm=norm, rope=rope, skip_frac=skip, row_sigma=row_sigma, **kw)


# ---- the named workloads at full size ----------------------------------

@pytest.mark.parametrize("i", range(7))
def test_config_parity(i):
    w = kvgen.config(i)
    n = check(w, label=f"config {i} {w.name}")
    print(f"config {i} {w.name}: T={w.T} hits={w.hits} one-step code diffs={n}", flush=True)


def test_config_repeat_is_deterministic():
    w = kvgen.config(2)
    a, _ = run_gpu(w)
    b, _ = run_gpu(w, repeat=3)
    assert np.array_equal(a, b)


# ---- shape sweeps ---------------------------------------------------------------

@pytest.mark.parametrize("mode", [0, 1])
@pytest.mark.parametrize("d", [128, 192, 256, 384, 576, 640, 1088, 2112, 4160, 8192])
@pytest.mark.parametrize("norm,rope", [(False, False), (True, True), (True, False),
                                       (False, True)])
def test_fp8_modes_sweep(mode, d, norm, rope):
    T = 300 if d <= 1088 else 80
    w = _small(mode, T, d, seed=d + 7 * mode + 3 * norm + rope, bs=7, stride_extra=40,
               norm=norm, rope=rope, row_sigma=1.5)
    check(w)


@pytest.mark.parametrize("d", [128, 192, 256, 576, 1088, 4160, 8192])
def test_bf16_split_sweep(d):
    w = _small(4, 200, d, seed=d, bs=5, stride_extra=8, norm=True, rope=True, row_sigma=1.0)
    check(w)


@pytest.mark.parametrize("d", [32, 64, 96, 128, 160, 256, 512, 1024, 4096, 8192])
def test_mxfp4_sweep(d):
    w = _small(3, 400 if d <= 1024 else 60, d, seed=d, bs=3, stride_extra=5, row_sigma=2.0)
    check(w)


@pytest.mark.parametrize("mode", [5, 6])
@pytest.mark.parametrize("d", [32, 64, 96, 128, 160, 256, 512, 1024, 4096, 8192])
def test_indexer_fp8_sweep(mode, d):
    w = _small(mode, 400 if d <= 1024 else 60, d, seed=d + mode, bs=3, stride_extra=5,
               row_sigma=2.0)
    assert check(w) == 0


# ---- layouts and alignment ----------------------------------------------------------

@pytest.mark.parametrize("offset", [0, 1, 2, 4, 8])
def test_mode1_head_dim_323_any_alignment(offset):
    # the page's example row (d=256, mode 1 -> 323 bytes) packed at headDim 323
    w = _small(1, 250, 256, seed=11, bs=32, head=323)
    check(w, offset=offset)


@pytest.mark.parametrize("offset", [0, 1, 2, 6])
def test_mode0_odd_head_dim(offset):
    w = _small(0, 250, 576, seed=12, bs=9, head=681, stride_extra=3, norm=True, rope=True)
    check(w, offset=offset)


@pytest.mark.parametrize("offset,aux_offset", [(0, 0), (1, 3), (4, 1)])
def test_mxfp4_odd_layout(offset, aux_offset):
    w = _small(3, 300, 128, seed=13, bs=11, head=67, aux_head=5, stride_extra=1)
    check(w, offset=offset, aux_offset=aux_offset)


@pytest.mark.parametrize("offset,aux_offset", [(0, 0), (1, 3), (4, 1)])
def test_mxfp8_odd_layout(offset, aux_offset):
    w = _small(5, 300, 128, seed=23, bs=11, head=131, aux_head=5, stride_extra=1)
    check(w, offset=offset, aux_offset=aux_offset)


@pytest.mark.parametrize("offset,aux_offset", [(0, 0), (1, 4), (6, 12)])
def test_fp8_row_odd_layout(offset, aux_offset):
    w = _small(6, 300, 256, seed=24, bs=7, head=259, aux_head=3, stride_extra=1)
    check(w, offset=offset, aux_offset=aux_offset)


@pytest.mark.parametrize("bs", [1, 2, 3, 100, 128, 1000])
def test_block_sizes(bs):
    w = _small(0, 500, 576, seed=bs, bs=bs, stride_extra=32, norm=True, rope=True)
    check(w)


def test_strided_x_rows():
    w = _small(0, 200, 576, seed=14, norm=True, rope=True)
    check(w, x_pad=64)


def test_non_default_stream():
    import torch
    w = _small(1, 200, 576, seed=15)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        got, agot = run_gpu(w, stream=s)
    want, awant = run_oracle(w)
    compare(w, got, want, agot, awant)


# ---- degenerate inputs ------------------------------------------------------------------

def test_zero_tokens_is_noop():
    import torch
    from kv_cache_epilog_amd import kvepi_run
    w = _small(0, 16, 256, seed=16)
    x = torch.empty((0, 256), dtype=torch.bfloat16, device="cuda")
    slots = torch.empty((0,), dtype=torch.int32, device="cuda")
    from parity import cache_tensor
    cache, flat = cache_tensor(w.cache, w.cache_init, "cuda")
    kvepi_run(x, slots, cache, 0, 64)
    torch.cuda.synchronize()
    assert np.all(flat.cpu().numpy() == kvgen.PREFILL)


@pytest.mark.parametrize("mode", [0, 1, 3, 4, 5, 6])
def test_all_skipped_and_out_of_range(mode):
    d = 128 if mode in (3, 5, 6) else 576
    w = _small(mode, 200, d, seed=17, norm=mode == 4, rope=mode == 4)
    w.slots[:100] = -1
    w.slots[100:] = w.cache.num_slots + np.arange(100)
    w.slots[150] = -7
    w.slots[151] = np.iinfo(np.int32).max
    got, agot = run_gpu(w)
    assert np.all(got == kvgen.PREFILL)
    if agot is not None:
        assert np.all(agot == kvgen.PREFILL)


@pytest.mark.parametrize("mode", [0, 1, 3, 4, 5, 6])
def test_special_values(mode):
    # zero rows and groups, negative zeros, bf16 subnormals, huge values and
    # exact ties: exercises the exact-division fallbacks and code rounding.
    rng = np.random.default_rng(18)
    d = 128 if mode in (3, 5, 6) else 576
    T = 64
    x = rng.standard_normal((T, d))
    x[0] = 0.0
    x[1] = -0.0
    x[2, :64] = 0.0
    x[3] = rng.standard_normal(d) * 1e-39                 # bf16 subnormals
    x[4] = rng.standard_normal(d) * 1e30
    x[5] = np.clip(rng.standard_normal(d) * 3e38, -3.3e38, 3.3e38)  # near the bf16 max
    x[6] = np.where(rng.random(d) < 0.5, -0.0, 0.0)
    x[7, ::2] = 448.0
    x[8] = np.round(rng.standard_normal(d) * 8) / 16      # many exact ties
    x[9] = rng.standard_normal(d) * 2.0 ** -120
    x[10, 5] = 1e-40                                      # one subnormal in a normal row
    x[11] = 1.0
    xb = kvgen.to_bf16(x)
    w = _small(mode, T, d, seed=19, skip=0.0, norm=mode in (0, 4), rope=mode in (0, 4), x=xb)
    check(w)
    if mode in (0, 1):
        w0 = _small(mode, T, d, seed=19, skip=0.0, norm=True, rope=False, x=xb, eps=0.0)
        # with eps = 0 a row whose squares all underflow has rms = 0: nonzero
        # values become +-inf, zeros 0/0 = NaN.  NaN values are left out of a
        # group's maximum, so the all-zero rows (0, 1, 6) get scale 0 and
        # codes 0, and the subnormal row (3) an infinite scale with NaN codes
        check(w0)


def _exponent_sweep_rows(mode, T, d, seed):
    """Rows whose quantisation groups cycle through every power-of-two scale
    2^k a bf16 input can produce (k from -141 to the largest that keeps
    MAX * 2^k finite).  Each group holds its amax MAX * 2^k exactly (so the
    scale is 2^k in every mode), code midpoints (exact ties) times 2^k, and
    random values below the amax."""
    rng = np.random.default_rng(seed)
    if mode == 3:
        G, nseg, vmax = 32, d, 6.0
        mids = [0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0]
        kmax = 125
    elif mode == 5:
        G, nseg, vmax = 32, d, 448.0
        mids = [2.0 ** -10, 3 * 2.0 ** -10, 1.0625, 1.1875, 9.5, 13.5, 17.0, 240.0, 416.0]
        kmax = 119
    else:
        G, nseg, vmax = 64, d - 64, 448.0
        mids = [2.0 ** -10, 3 * 2.0 ** -10, 1.0625, 1.1875, 9.5, 13.5, 17.0, 240.0, 416.0]
        kmax = 119
    ks = np.arange(-141, kmax + 1)
    x = np.zeros((T, d))
    x[:, nseg:] = rng.standard_normal((T, d - nseg))
    gi = 0
    for r in range(T):
        for g in range(nseg // G):
            k = float(ks[gi % ks.size])
            gi += 1
            v = np.clip(rng.standard_normal(G) * vmax / 3, -vmax, vmax)
            v[0] = vmax if rng.random() < 0.5 else -vmax
            nm = G // 4
            v[1:1 + nm] = rng.choice(mids, nm) * np.where(rng.random(nm) < 0.5, -1.0, 1.0)
            rng.shuffle(v)
            x[r, g * G:(g + 1) * G] = v * 2.0 ** k
    return kvgen.to_bf16(x)


@pytest.mark.parametrize("mode", [0, 1, 3, 5])
def test_scale_exponent_sweep(mode):
    # every e8m0 / bf16 power-of-two scale, both sides of the range where the
    # kernel uses the hardware converts and fast division, with exact ties
    d = 128 if mode in (3, 5) else 576
    T = 400 if mode in (3, 5) else 200
    xb = _exponent_sweep_rows(mode, T, d, seed=20 + mode)
    w = _small(mode, T, d, seed=21, skip=0.0, x=xb)
    n = check(w)
    assert n == 0


def test_fp8_row_amax_sweep():
    # per-row FP8: row maxima over the whole bf16 range (the fast path covers
    # [2^-71, 2^100]), rows whose scale is a power of two (exact code ties),
    # and random rows whose scale is not
    rng = np.random.default_rng(25)
    d, T = 128, 600
    x = rng.standard_normal((T, d))
    for r in range(T):
        k = -141 + (r * 7) % 268  # 2^k spans subnormal to near the bf16 max
        amax = 448.0 * 2.0 ** min(k, 118)
        if r % 3 == 0:
            # the scale is exactly 2^k: code midpoints are exact ties
            mids = np.array([2.0 ** -10, 3 * 2.0 ** -10, 1.0625, 1.1875, 9.5, 13.5, 240.0])
            v = rng.choice(mids, d) * np.where(rng.random(d) < 0.5, -1.0, 1.0)
        else:
            v = np.clip(rng.standard_normal(d) * 100, -447, 447) * (1 + rng.random() / 7)
        v[r % d] = 448.0 if r % 2 else -448.0
        x[r] = v * 2.0 ** min(k, 118) if r % 3 == 0 else v / 448.0 * amax
    w = _small(6, T, d, seed=26, skip=0.0, x=kvgen.to_bf16(x))
    assert check(w) == 0


@pytest.mark.parametrize("waves", [4, 8, 64])
@pytest.mark.parametrize("case", ["fused576", "mode1_576", "mxfp4_128", "split576", "mode0_2112",
                                  "mode0_256", "mxfp8_128", "fp8row_128", "fp8row_1024"])
def test_many_iterations_per_wave(case, waves, monkeypatch):
    # a capped grid makes each wave run hundreds of iterations: slot windows
    # are reloaded many times and the pipeline runs through its steady state
    monkeypatch.setenv("KVEPI_MAX_WAVES", str(waves))
    T = 3001
    if case == "fused576":
        w = _small(0, T, 576, seed=31, bs=64, stride_extra=96, norm=True, rope=True)
    elif case == "mode1_576":
        w = _small(1, T, 576, seed=32, bs=17, row_sigma=2.0)
    elif case == "mxfp4_128":
        w = _small(3, T, 128, seed=33, bs=128, row_sigma=1.0)
    elif case == "split576":
        w = _small(4, T, 576, seed=34, bs=5, norm=True, rope=True)
    elif case == "mxfp8_128":
        w = _small(5, T, 128, seed=37, bs=128, row_sigma=1.0)
    elif case == "fp8row_128":
        w = _small(6, T, 128, seed=38, bs=64, row_sigma=1.0)
    elif case == "fp8row_1024":
        w = _small(6, 700, 1024, seed=39, bs=16, row_sigma=1.0)
    elif case == "mode0_2112":
        w = _small(0, 600, 2112, seed=35, bs=9, norm=True, rope=True)
    else:
        w = _small(0, T, 256, seed=36, bs=16)
    check(w)


def _tree_f32(a):
    s = np.asarray(a, np.float32)
    while s.size > 1:
        s = (s[0::2] + s[1::2]).astype(np.float32)
    return s[0]


def _rmsnorm_out(v, g, fused_pairs):
    """bf16 RMSNorm outputs of one row with eps = 0 (numpy fp32): the squares
    rounded one by one, or (fused_pairs) each pair summed with one rounding
    as an fma of the second square onto the first rounded square would."""
    if fused_pairs:
        p = (v[0::2] * v[0::2]).astype(np.float32)
        pairs = (v[1::2].astype(np.float64) ** 2 + p.astype(np.float64)).astype(np.float32)
        ss = _tree_f32(pairs)
    else:
        ss = _tree_f32((v * v).astype(np.float32))
    rms = np.sqrt(np.float32(ss / np.float32(v.size)))
    return kvgen.to_bf16(((v / rms).astype(np.float32) * g).astype(np.float32))


@pytest.mark.parametrize("mode", [4, 0])
def test_underflowing_squares(mode):
    # Rows of pairs (a, b) with a = M0 2^-70 (a^2 exact, in [2^-125, 2^-124))
    # and b = M1 2^-82 (b^2 between 0.5 and 0.75 of that binade's last
    # place, below the normal range): the definition rounds b^2 first (to a
    # half place, a tie when added to a^2), a fused pair sum rounds once, and
    # with eps = 0 the last place of the sum can reach rms.  Rows are kept
    # only where the two readings give different bf16 outputs with this
    # workload's gamma, so the comparison with the oracle exercises the case.
    rng = np.random.default_rng(23)
    T, d = 32, 576
    x = kvgen.to_bf16(rng.standard_normal((T, d)))
    # (the bf16 split writes the RoPE output to its second cache, so it
    # takes cos and sin; the rope columns do not enter the RMSNorm)
    w = _small(mode, T, d, seed=29, skip=0.0, norm=True, rope=mode == 4, x=x, eps=0.0)
    g = kvgen.bf16_to_f32(w.gamma).astype(np.float32)
    # (a one-place change of rms reaches a bf16 output only when an output
    # lies that close to a bf16 rounding boundary: about 1 row in 260 here)
    rows = []
    for _ in range(20000):
        sgn = np.where(rng.random(512) < 0.5, -1.0, 1.0)
        row = np.empty(512)
        row[0::2] = sgn[0::2] * rng.integers(182, 256, 256) * 2.0 ** -70
        row[1::2] = sgn[1::2] * rng.integers(182, 222, 256) * 2.0 ** -82
        bits = kvgen.to_bf16(row)
        v = kvgen.bf16_to_f32(bits).astype(np.float32)
        if not np.array_equal(_rmsnorm_out(v, g, True), _rmsnorm_out(v, g, False)):
            rows.append(bits)
            if len(rows) == T // 2:
                break
    assert len(rows) == T // 2
    for r, bits in enumerate(rows):
        w.x[r, :512] = bits
    check(w)


@pytest.mark.parametrize("mode", [0, 4])
def test_rope_underflowing_products(mode):
    # tiny rope values times small cos / sin: a product of two bf16 values
    # that underflows rounds, and a fused multiply-add would round the pair
    # once; every rope pair here is a case where that changes the bf16
    # output (found and checked on the CPU by plant_rope_cases)
    from parity import plant_rope_cases
    rng = np.random.default_rng(31)
    w = _small(mode, 32, 576, seed=37, skip=0.0, norm=True, rope=True)
    assert plant_rope_cases(w, rng, 64) == 32 * 32
    check(w)


def test_offsets_beyond_4gib():
    # A cache of about 4.7 GB written at slots whose byte offsets all lie
    # past 2^32, and x rows 128 MB apart (an 8 GB row stride span), so that
    # both the row addresses and the x addresses need 64-bit arithmetic.
    # The expected rows come from the oracle on a small cache of the same
    # row layout; only the touched rows and their neighbours are read back.
    import torch
    from kv_cache_epilog_amd import kvepi_run
    from parity import to_dev_bf16
    T, d, bs, kc = 64, 576, 128, 672
    small = _small(0, T, d, seed=41, skip=0.1, norm=True, rope=True)
    ocache, _ = run_oracle(small)
    dev = torch.device("cuda:0")
    bn, stride = 54000, bs * kc + 256          # a gap after every block
    flat = torch.full((bn * stride,), kvgen.PREFILL, dtype=torch.uint8, device=dev)
    view = flat.as_strided((bn, bs, 1, kc), (stride, kc, kc, 1))
    first = (2 ** 32 // stride + 1) * bs      # first slot of a block past 2^32
    rng = np.random.default_rng(41)
    big = rng.choice(np.arange(first, bn * bs - 1, 2), T, replace=False).astype(np.int32)
    big[small.slots < 0] = -1
    xs = 1 << 26                               # elements between rows of x
    xbuf = torch.empty((T, xs), dtype=torch.bfloat16, device=dev)
    x = xbuf[:, :d]
    x.copy_(to_dev_bf16(small.x, dev))
    kvepi_run(x, torch.from_numpy(big).to(dev), view, 0, 64,
              gamma=to_dev_bf16(small.gamma, dev), cos=to_dev_bf16(small.cos, dev),
              sin=to_dev_bf16(small.sin, dev), eps=small.eps)
    torch.cuda.synchronize()
    hit = np.nonzero(big >= 0)[0]
    off = np.array([(int(s) // bs) * stride + (int(s) % bs) * kc for s in big[hit]], np.int64)
    assert off.min() >= 2 ** 32
    idx = torch.from_numpy(off[:, None] + np.arange(kc)[None, :]).to(dev)
    got = flat[idx].cpu().numpy()
    want = np.stack([ocache[small.cache.row_offset(int(s)):][:kc] for s in small.slots[hit]])
    assert np.array_equal(got, want)
    # the next row (the slots are even, so never written) and the block gaps
    nxt = flat[idx + kc].cpu().numpy()
    assert np.all(nxt == kvgen.PREFILL)
    gaps = torch.from_numpy(((big[hit] // bs) * stride + bs * kc).astype(np.int64)[:, None]
                            + np.arange(256)[None, :]).to(dev)
    assert np.all(flat[gaps].cpu().numpy() == kvgen.PREFILL)
    del flat, view, xbuf
    torch.cuda.empty_cache()


def test_duplicate_slot_check(monkeypatch):
    # KVEPI_CHECK_SLOTS: two tokens naming one row are rejected with
    # KVEPI_ERR_PARAM before any launch (the cache keeps every byte); distinct
    # slots pass the check and give the oracle's bytes
    import torch
    from kv_cache_epilog_amd import kvepi_run
    from kv_cache_epilog_amd.binding import KvepiError
    from parity import cache_tensor, to_dev_bf16
    monkeypatch.setenv("KVEPI_CHECK_SLOTS", "1")
    w = _small(0, 64, 576, seed=43, skip=0.1, norm=True, rope=True)
    check(w)
    dev = torch.device("cuda:0")
    slots = w.slots.copy()
    hit = np.nonzero(slots >= 0)[0]
    slots[hit[-1]] = slots[hit[0]]
    cache, flat = cache_tensor(w.cache, w.cache_init, dev)
    with pytest.raises(KvepiError) as e:
        kvepi_run(to_dev_bf16(w.x, dev), torch.from_numpy(slots).to(dev), cache, 0, 64,
                  gamma=to_dev_bf16(w.gamma, dev), cos=to_dev_bf16(w.cos, dev),
                  sin=to_dev_bf16(w.sin, dev), eps=w.eps)
    assert e.value.status == 4  # KVEPI_ERR_PARAM
    torch.cuda.synchronize()
    assert np.all(flat.cpu().numpy() == kvgen.PREFILL)


def _fuzz_case(k):
    """A seeded random workload: mode, row width, RMSNorm / RoPE, token
    count, block size, head padding, block stride, skip density, row sigma,
    fp16 rows (indexer modes), buffer offsets and padded x rows."""
    rng = np.random.default_rng(7000 + k)
    mode = int(rng.choice([0, 1, 3, 4, 5, 6]))
    if mode in (0, 1, 4):
        d = 64 * int(rng.integers(2, 129))          # 128 .. 8192
    else:
        d = 32 * int(rng.integers(1, 257))          # 32 .. 8192
    norm = mode == 4 or (mode in (0, 1) and bool(rng.random() < 0.5))
    rope = mode == 4 or (mode in (0, 1) and bool(rng.random() < 0.5))
    T = int(rng.choice([1, 2, 63, 64, 65, 129, int(rng.integers(1, 1500))]))
    if d >= 4096:
        T = min(T, 300)
    bs = int(rng.choice([1, 3, 16, 128, int(rng.integers(1, 200))]))
    skip = float(rng.choice([0.0, 0.05, 0.3, 1.0]))
    sigma = float(rng.choice([0.0, 1.0, 3.0]))
    group = {3: 32, 5: 32, 6: 0}.get(mode, 64)
    import oracle
    kc = d - 64 if mode == 4 else oracle.row_bytes(mode, d, group)[1]
    head = kc + int(rng.choice([0, 0, 1, 3, 16]))
    stride_extra = int(rng.choice([0, 0, 5, 64]))
    x = None
    fp16 = mode in (3, 5, 6) and bool(rng.random() < 0.3)
    if fp16:
        x = kvgen.fp16_rows(rng, T, d, row_sigma=sigma)
    w = _small(mode, T, d, seed=7000 + k, bs=bs, head=head, stride_extra=stride_extra,
               norm=norm, rope=rope, skip=skip, row_sigma=sigma,
               **({} if x is None else {"x": x}))
    if fp16:
        w.x_fp16 = True
    kw = dict(offset=int(rng.choice([0, 0, 1, 7, 32])) * w.cache.elem_bytes,
              x_pad=int(rng.choice([0, 0, 8, 24])))
    if mode in (3, 5, 6):
        kw["aux_offset"] = int(rng.choice([0, 4]))
    return w, kw


@pytest.mark.parametrize("k", range(160))
def test_fuzz(k):
    w, kw = _fuzz_case(k)
    assert check(w, f"fuzz {k}: {w.name}", **kw) == 0


@pytest.mark.parametrize("k", range(40))
def test_fuzz_few_waves(k, monkeypatch):
    # the same random workloads on a grid capped at 8 waves, so that every
    # wave runs many iterations (slot windows, the two-deep pipeline's
    # hand-offs, the last partial window)
    monkeypatch.setenv("KVEPI_MAX_WAVES", "8")
    w, kw = _fuzz_case(k)
    assert check(w, f"fuzz few waves {k}: {w.name}", **kw) == 0
