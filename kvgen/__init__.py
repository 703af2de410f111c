"""Seeded synthetic workloads for the fused KV-cache write epilog.

This module only draws inputs: token rows, gamma, cos/sin tables, slot
mappings and prefilled caches.  It holds none of the epilog's arithmetic and
is shared by the oracle tests, the GPU parity tests, the smoke check and the
benchmark, so that both sides consume identical bytes.

bf16 tensors are numpy ``uint16`` bit patterns; fp32 draws are rounded to
bf16 by torch's CPU conversion (round to nearest even).

Shapes follow the workloads the pages describe: DeepSeek-style rows of
d = 576 (512 latent + 64 rope, "aclnnKvRmsNormRopeCache" 约束说明, N = 1) and
indexer rows of d = 128 ("indexer_quant_cache" 约束, d = 128 example).  No
public dataset is involved; every value is drawn from a seeded generator.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Optional

import numpy as np

MODE_FP8_BF16SCALE = 0
MODE_FP8_E8M0 = 1
MODE_MXFP4 = 3
MODE_BF16_SPLIT = 4
MODE_MXFP8 = 5
MODE_FP8_ROW = 6
MODE_FP4_NOPE = 7

PREFILL = 0xAB


def to_bf16(a: np.ndarray) -> np.ndarray:
    """Round fp32 (or fp64) values to bf16 bit patterns (torch, RNE)."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def bf16_to_f32(h: np.ndarray) -> np.ndarray:
    return (np.asarray(h, np.uint16).astype(np.uint32) << 16).view(np.float32)


@dataclass
class CacheSpec:
    """[block_num, block_size, 1, head_dim]; head_dim and block_stride in
    elements of ``elem_bytes`` bytes."""
    block_num: int
    block_size: int
    head_dim: int
    block_stride: int
    elem_bytes: int = 1

    @property
    def num_slots(self) -> int:
        return self.block_num * self.block_size

    @property
    def alloc_bytes(self) -> int:
        return ((self.block_num - 1) * self.block_stride
                + self.block_size * self.head_dim) * self.elem_bytes

    @property
    def geom(self):
        return (self.block_num, self.block_size, self.head_dim, self.block_stride)

    def row_offset(self, slot: int) -> int:
        """Byte offset of a slot's row (independent restatement of the paged
        layout, used by the tests' address checks)."""
        blk, pos = divmod(int(slot), self.block_size)
        return (blk * self.block_stride + pos * self.head_dim) * self.elem_bytes


@dataclass
class Workload:
    name: str
    mode: int
    T: int
    d: int
    group_size: int
    x: np.ndarray                      # uint16 [T, d]
    slots: np.ndarray                  # int32 [T]
    cache: CacheSpec
    cache_init: np.ndarray             # uint8 [cache.alloc_bytes]
    gamma: Optional[np.ndarray] = None  # uint16 [d-64]
    cos: Optional[np.ndarray] = None    # uint16 [T, 64]
    sin: Optional[np.ndarray] = None    # uint16 [T, 64]
    eps: float = 1e-6
    aux: Optional[CacheSpec] = None
    aux_init: Optional[np.ndarray] = None
    notes: dict = field(default_factory=dict)
    x_fp16: bool = False   # x holds fp16 bits (indexer modes)
    index_mode: int = 0    # 0: slots holds one slot per token; 1-3: see below
    seq_len: int = 0       # tokens per batch for index modes 1-3
    rope_dim: int = 64     # rope segment length (any even value in the bf16 split mode)

    @property
    def hits(self) -> int:
        return int(np.count_nonzero((self.slots >= 0)
                                    & (self.slots < self.cache.num_slots)))


def slot_mapping(rng, T: int, num_slots: int, skip_frac: float = 0.0,
                 n_skip: Optional[int] = None) -> np.ndarray:
    """Distinct slots drawn as the first T entries of a permutation of
    [0, num_slots), then exactly round(skip_frac * T) of them (or n_skip) set
    to -1 at random positions."""
    assert T <= num_slots
    s = rng.permutation(num_slots)[:T].astype(np.int32)
    k = int(round(skip_frac * T)) if n_skip is None else int(n_skip)
    if k:
        s[rng.choice(T, size=k, replace=False)] = -1
    return s


def to_fp16(a) -> np.ndarray:
    """fp16 bit patterns of float values (numpy's round to nearest even)."""
    return np.asarray(a, np.float64).astype(np.float16).view(np.uint16)


def fp16_rows(rng, T: int, d: int, row_sigma: float = 0.0) -> np.ndarray:
    """fp16 x ~ N(0,1) * per-row lognormal(0, row_sigma), clipped to the
    finite fp16 range."""
    x = rng.standard_normal((T, d))
    if row_sigma > 0:
        x *= rng.lognormal(0.0, row_sigma, size=(T, 1))
    return to_fp16(np.clip(x, -65504.0, 65504.0))


def index_array(rng, index_mode: int, B: int, S: int, block_num: int, block_size: int,
                skip_frac: float = 0.0) -> np.ndarray:
    """A valid index array for the batch-major index modes (tokens b*S + s):
    1 (per-batch rows): index[b, s] a random choice of distinct rows < block_size;
    2 (per-chunk blocks): one distinct block per chunk of block_size tokens,
      at a random row of it; 3 (per-batch start): index[b] in [0, block_size - S].
    round(skip_frac * len) entries are set to -1."""
    if index_mode == 1:
        assert S <= block_size and B <= block_num
        idx = np.concatenate([rng.permutation(block_size)[:S] for _ in range(B)])
    elif index_mode == 2:
        nc = -(-S // block_size)
        assert B * nc <= block_num
        blk = rng.permutation(block_num)[:B * nc]
        idx = blk * block_size + rng.integers(0, block_size, blk.size)
    else:
        assert S <= block_size and B <= block_num
        idx = rng.integers(0, block_size - S + 1, B)
    idx = idx.astype(np.int32)
    k = int(round(skip_frac * idx.size))
    if k:
        idx[rng.choice(idx.size, size=k, replace=False)] = -1
    return idx


def rope_tables(rng, T: int, max_pos: int, theta: float = 10000.0, dk: int = 64):
    """cos/sin [T, dk] for random integer positions < max_pos:
    cos[t, k] = cos(pos_t * theta^(-2 (k mod dk/2) / dk)), in fp64, rounded
    to bf16."""
    pos = rng.integers(0, max_pos, size=T).astype(np.float64)
    half = dk // 2
    inv = theta ** (-2.0 * np.arange(half, dtype=np.float64) / dk)
    ang = pos[:, None] * inv[None, :]
    ang = np.concatenate([ang, ang], axis=1)
    return to_bf16(np.cos(ang)), to_bf16(np.sin(ang)), pos


def normal_rows(rng, T: int, d: int, row_sigma: float = 0.0,
                outlier_frac: float = 0.0, outlier_mult: float = 100.0) -> np.ndarray:
    """x ~ N(0,1) * per-row lognormal(0, row_sigma), with exactly
    round(outlier_frac * T * d) random elements multiplied by outlier_mult."""
    x = rng.standard_normal((T, d), dtype=np.float32)
    if row_sigma > 0:
        x *= rng.lognormal(0.0, row_sigma, size=(T, 1)).astype(np.float32)
    n_out = int(round(outlier_frac * T * d))
    if n_out:
        idx = rng.choice(T * d, size=n_out, replace=False)
        x.reshape(-1)[idx] *= np.float32(outlier_mult)
    return to_bf16(x)


def make(name: str, mode: int, T: int, d: int, *, seed: int, cache: CacheSpec,
         aux: Optional[CacheSpec] = None, norm: bool = False, rope: bool = False,
         row_sigma: float = 0.0, outlier_frac: float = 0.0, skip_frac: float = 0.0,
         n_skip: Optional[int] = None, max_pos: int = 32768, eps: float = 1e-6,
         group_size: Optional[int] = None, x: Optional[np.ndarray] = None,
         rope_dim: int = 64) -> Workload:
    rng = np.random.default_rng(seed)
    if group_size is None:
        group_size = {MODE_MXFP4: 32, MODE_MXFP8: 32, MODE_FP8_ROW: 0,
                      MODE_FP4_NOPE: 32}.get(mode, 64)
    if x is None:
        x = normal_rows(rng, T, d, row_sigma, outlier_frac)
    gamma = cos = sin = None
    if norm:
        gamma = to_bf16(rng.uniform(0.5, 1.5, size=d - rope_dim))
    if rope:
        cos, sin, _ = rope_tables(rng, T, max_pos, dk=rope_dim)
    slots = slot_mapping(rng, T, cache.num_slots, skip_frac, n_skip)
    cache_init = np.full(cache.alloc_bytes, PREFILL, np.uint8)
    aux_init = None if aux is None else np.full(aux.alloc_bytes, PREFILL, np.uint8)
    w = Workload(name, mode, T, d, group_size, x, slots, cache, cache_init,
                 gamma, cos, sin, eps, aux, aux_init)
    w.rope_dim = rope_dim
    return w


# ---- the five named workloads ---------------------------------------------

CONFIG_NAMES = ("mode0_tiny_d256", "rmsnorm_rope_bf16_d576", "mode1_prefill_d576",
                "mxfp4_indexer_d128", "fused_epilog_d576",
                # the other indexer modes at the MX-FP4 indexer's shape
                "mxfp8_indexer_d128", "fp8row_indexer_d128",
                # quantMode 2's FP4 nope segment at the fused workload's shape
                "fp4_nope_d576")


def config(i: int) -> Workload:
    if i == 0:
        # quantMode 0, x [64,256] ~ N(0,1), group 64, cache [8,16,1,416] u8
        # prefilled 0xAB, 64 distinct slots in [0,128) with 8 set to -1.
        return make(CONFIG_NAMES[0], MODE_FP8_BF16SCALE, 64, 256, seed=0,
                    cache=CacheSpec(8, 16, 416, 16 * 416), n_skip=8)
    if i == 1:
        # RMSNorm(512) + RoPE(64) to bf16 ckv [1024,128,1,512] and
        # k [1024,128,1,64] caches; 64 tokens, 5% skipped.
        return make(CONFIG_NAMES[1], MODE_BF16_SPLIT, 64, 576, seed=1,
                    cache=CacheSpec(1024, 128, 512, 128 * 512, 2),
                    aux=CacheSpec(1024, 128, 64, 128 * 64, 2),
                    norm=True, rope=True, skip_frac=0.05, max_pos=32768)
    if i == 2:
        # quantMode 1 prefill: [16384,576], lognormal(0,2) row magnitudes and
        # 0.1% outliers x100; cache [512,128,1,656]; 2% skipped.
        return make(CONFIG_NAMES[2], MODE_FP8_E8M0, 16384, 576, seed=2,
                    cache=CacheSpec(512, 128, 656, 128 * 656),
                    row_sigma=2.0, outlier_frac=0.001, skip_frac=0.02)
    if i == 3:
        # MX-FP4 indexer: [131072,128], lognormal(0,1) rows; cache
        # [1024,128,1,64] u8 + cache_scale [1024,128,1,4]; 1% skipped.
        return make(CONFIG_NAMES[3], MODE_MXFP4, 131072, 128, seed=3,
                    cache=CacheSpec(1024, 128, 64, 128 * 64),
                    aux=CacheSpec(1024, 128, 4, 128 * 4),
                    row_sigma=1.0, skip_frac=0.01)
    if i == 4:
        # Full fused epilog: [262144,576], RMSNorm(512) + RoPE(64,
        # positions < 131072) then quantMode 0; 672-byte rows in a cache
        # [2048,128,1,672] whose block stride is 1.25x the dense one; 3% skipped.
        return make(CONFIG_NAMES[4], MODE_FP8_BF16SCALE, 262144, 576, seed=4,
                    cache=CacheSpec(2048, 128, 672, 128 * 672 * 5 // 4),
                    norm=True, rope=True, max_pos=131072, skip_frac=0.03)
    if i == 5:
        # MX-FP8 indexer at the shape of 3: codes [1024,128,1,128] u8 +
        # e8m0 cache_scale [1024,128,1,4]
        return make(CONFIG_NAMES[5], MODE_MXFP8, 131072, 128, seed=5,
                    cache=CacheSpec(1024, 128, 128, 128 * 128),
                    aux=CacheSpec(1024, 128, 4, 128 * 4),
                    row_sigma=1.0, skip_frac=0.01)
    if i == 6:
        # per-row FP8 indexer at the shape of 3: codes [1024,128,1,128] u8 +
        # fp32 cache_scale [1024,128,1,1]
        return make(CONFIG_NAMES[6], MODE_FP8_ROW, 131072, 128, seed=6,
                    cache=CacheSpec(1024, 128, 128, 128 * 128),
                    aux=CacheSpec(1024, 128, 1, 128 * 1, 4),
                    row_sigma=1.0, skip_frac=0.01)
    if i == 7:
        # quantMode 2's nope segment after RMSNorm at the shape of 4:
        # [262144,576], RMSNorm(512), group-32 E2M1 codes with bf16 scales;
        # 352-byte rows (64 rope bytes left untouched) in a cache
        # [2048,128,1,352] whose block stride is 1.25x the dense one; 3% skipped.
        return make(CONFIG_NAMES[7], MODE_FP4_NOPE, 262144, 576, seed=7,
                    cache=CacheSpec(2048, 128, 352, 128 * 352 * 5 // 4),
                    norm=True, skip_frac=0.03, group_size=32)
    raise IndexError(i)


# ---- the dequant -> RoPE -> int8 KV cache operator's inputs ----------------------
# Inputs follow the operator's own examples: int32 matmul outputs with
# per-column weight scales, per-token activation scales and a bias, or
# fp16/bf16 activations; cos/sin of random positions; per-channel static
# scales sized to the k / v ranges.

DT_BF16, DT_FP16, DT_INT32, DT_FP32 = 0, 1, 2, 3


@dataclass
class DrqWorkload:
    """Inputs of one dequant -> RoPE -> int8 KV cache call (cache given by its
    byte geometry; cache_mode 0 = page, 1 = contiguous)."""
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
    bias_dtype: int = DT_FP32
    offset_k: Optional[np.ndarray] = None
    offset_v: Optional[np.ndarray] = None
    kv_output: bool = True
    x_pad: int = 0
    notes: dict = field(default_factory=dict)


def to16(a, dt):
    """bf16 or fp16 bit patterns of float values (round to nearest even)."""
    return to_bf16(a) if dt == DT_BF16 else to_fp16(a)


def drq_make(seed, *, T, nq, nkv, D, x_dtype, out_dtype, cache_mode=0, bias_dtype=None,
              act=True, offsets=True, kv_output=True, bn=None, bs=16, head=None, stride_extra=0,
              skip=0.05, seq_len=0, x_pad=0) -> DrqWorkload:
    rng = np.random.default_rng(seed)
    H = (nq + 2 * nkv) * D
    ws = act_s = bias = None
    if x_dtype == DT_INT32:
        x = rng.integers(-(1 << 20), 1 << 20, (T, H)).astype(np.int32)
        ws = (rng.random(H) * 2e-4 + 1e-5).astype(np.float32)
        if act:
            act_s = rng.uniform(0.5, 2.0, T).astype(np.float32)
        if bias_dtype is not None:
            b = rng.standard_normal(H) * 4
            if bias_dtype == DT_FP32:
                bias = b.astype(np.float32)
            elif bias_dtype == DT_INT32:
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
    return DrqWorkload(T, nq, nkv, D, x, x_dtype, out_dtype, cos, sin, sk, sv, index, cache_mode,
                   seq_len, geom, ws, act_s, bias, bias_dtype if bias is not None else
                   DT_FP32, ok, ov, kv_output, x_pad)


DRQ_NAMES = ("drq_fp16_h2304", "drq_int32_h3584")


def drq_config(name: str) -> DrqWorkload:
    """Throughput workloads at the operator's two test shapes, with many
    tokens: fp16 x [65536, 2304] (12 q heads, 3 k / v heads of 128) and
    int32 x [32768, 3584] (14 / 7 / 7 heads of 128, bf16 bias, activation
    scales, offsets), page mode with 1 % skipped tokens, k / v outputs on."""
    if name == DRQ_NAMES[0]:
        return drq_make(10, T=65536, nq=12, nkv=3, D=128, x_dtype=DT_FP16, out_dtype=DT_FP16,
                        bs=128, skip=0.01)
    if name == DRQ_NAMES[1]:
        return drq_make(11, T=32768, nq=14, nkv=7, D=128, x_dtype=DT_INT32, out_dtype=DT_BF16,
                        bias_dtype=DT_BF16, bs=128, skip=0.01)
    raise KeyError(name)

