"""Seeded synthetic inputs for paged decode attention and the KV-cache write.

This module only draws and lays out input data: context lengths, a shuffled
block pool, block tables, K/V pools, queries, new tokens and their slots.  It
holds none of the attention arithmetic, so both the fp64 oracle and the HIP
path can consume the same arrays without sharing any of the method's code.

The workloads follow the problem statement of the PhotonInfer README
(Korean translation), section "Technical details > Paged attention": the KV
cache is kept in fixed-size blocks, each sequence reaches its tokens through
its own list of blocks, and one kernel writes the new K/V of many sequences.
The shapes are those of Llama-3.2-1B and Qwen3 attention layers, the two
model families the same README's performance section names.

Draw order for a given seed (fixed, so every consumer sees identical data):
  1. context lengths;
  2. the pool permutation (blocks drawn without replacement, handed to the
     sequences in batch order);
  3. the K pool;  4. the V pool;  5. q;  6. the new k and v for the write.
Values are float32 standard normals rounded to nearest-even into the stored
dtype.  Half-precision arrays are returned as their uint16 bit patterns.

Pool layout (the one the library documents): K and V pools are each
[num_blocks, num_kv_heads, block_size, head_dim], row-major.  Token t of
sequence b lives in physical block block_tables[b, t // block_size] at
offset t % block_size; the slot number of that position is
block * block_size + offset.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import Optional, Sequence

import numpy as np

DTYPES = ("f32", "f16", "bf16")

# quiet-NaN bit patterns used to poison memory that must never be read
NAN_BITS = {"f16": 0x7E00, "bf16": 0x7FC0}


def _round_to_dtype(x: np.ndarray, dtype: str) -> np.ndarray:
    """float32 samples -> stored representation (float32, or uint16 bits)."""
    if dtype == "f32":
        return np.ascontiguousarray(x, dtype=np.float32)
    if dtype == "f16":
        return np.ascontiguousarray(x.astype(np.float16).view(np.uint16))
    if dtype == "bf16":
        import torch  # CPU-only use: numpy has no bfloat16

        t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
        return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16).copy()
    raise ValueError(f"unknown dtype {dtype!r}")


def _poison(arr: np.ndarray, dtype: str):
    """Return the value that marks unreadable memory for this stored dtype."""
    if dtype == "f32":
        return np.float32(np.nan)
    return np.uint16(NAN_BITS[dtype])


@dataclass
class Workload:
    """One batch of decode inputs in host memory (stored dtype bits)."""

    name: str
    dtype: str
    num_seqs: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    block_size: int
    num_blocks: int
    scale: np.float32
    context_lens: np.ndarray  # int32 [B]
    block_tables: np.ndarray  # int32 [B, MB], padding -1
    k_cache: np.ndarray  # [NB, Hkv, bs, D] float32 or uint16 bits
    v_cache: np.ndarray
    q: np.ndarray  # [B, Hq, D]
    partition_size: int = 0  # 0: let the library choose
    # new tokens for the KV-cache write (one per sequence unless stated)
    new_k: Optional[np.ndarray] = None  # [T, Hkv, D]
    new_v: Optional[np.ndarray] = None
    slot_mapping: Optional[np.ndarray] = None  # int64 [T]
    meta: dict = field(default_factory=dict)

    @property
    def max_blocks_per_seq(self) -> int:
        return int(self.block_tables.shape[1])

    @property
    def elt_bytes(self) -> int:
        return 4 if self.dtype == "f32" else 2

    @property
    def max_context_len(self) -> int:
        return int(self.context_lens.max()) if self.num_seqs else 0

    def kv_bytes(self) -> int:
        """K+V bytes a decode must stream: sum_b L_b * 2 * Hkv * D * elt."""
        total_tokens = int(self.context_lens.astype(np.int64).clip(min=0).sum())
        return total_tokens * 2 * self.num_kv_heads * self.head_dim * self.elt_bytes


def make_case(
    seed: int,
    *,
    dtype: str,
    context_lens: Sequence[int],
    num_q_heads: int,
    num_kv_heads: int,
    head_dim: int,
    block_size: int,
    pool_blocks: Optional[int] = None,
    pool_factor: float = 1.25,
    scale: Optional[float] = None,
    partition_size: int = 0,
    write: bool = True,
    poison: bool = True,
    max_blocks_per_seq: Optional[int] = None,
    name: str = "case",
    rng: Optional[np.random.Generator] = None,
    pools: bool = True,
) -> Workload:
    """Build a workload with the given context lengths.

    ``write=True`` draws one new token per sequence (at position L_b - 1) and
    its slot; with ``poison=True`` that slot is NaN in the pool beforehand, so
    a decode that runs before the write, or a write that lands elsewhere,
    shows up as NaN.  Unused pool blocks and the tail slots >= L_b of every
    sequence's last block are NaN-poisoned as well.
    """
    if dtype not in DTYPES:
        raise ValueError(f"dtype must be one of {DTYPES}")
    rng = rng if rng is not None else np.random.default_rng(seed)
    lens = np.asarray(context_lens, dtype=np.int64)
    B = int(lens.shape[0])
    bs = int(block_size)
    # 2. pool permutation
    nblk = np.where(lens > 0, (lens + bs - 1) // bs, 0)
    used = int(nblk.sum())
    if pool_blocks is None:
        pool_blocks = max(used, int(math.ceil(pool_factor * used)), 1)
    if pool_blocks < used:
        raise ValueError(f"pool of {pool_blocks} blocks cannot hold {used}")
    mb = int(nblk.max()) if B else 0
    if max_blocks_per_seq is not None:
        if max_blocks_per_seq < mb:
            raise ValueError("max_blocks_per_seq smaller than the longest sequence")
        mb = int(max_blocks_per_seq)
    mb = max(mb, 1)
    perm = rng.permutation(pool_blocks).astype(np.int32)
    block_tables = np.full((B, mb), -1, dtype=np.int32)
    cursor = 0
    for b in range(B):
        n = int(nblk[b])
        block_tables[b, :n] = perm[cursor : cursor + n]
        cursor += n
    # 3./4. pools
    shape = (pool_blocks, num_kv_heads, bs, head_dim)
    k_cache = v_cache = None
    if pools:
        k_cache = _round_to_dtype(rng.standard_normal(shape, dtype=np.float32), dtype)
        v_cache = _round_to_dtype(rng.standard_normal(shape, dtype=np.float32), dtype)
    # 5. q
    q = _round_to_dtype(
        rng.standard_normal((B, num_q_heads, head_dim), dtype=np.float32), dtype
    )
    # 6. new tokens
    new_k = new_v = slots = None
    if write:
        new_k = _round_to_dtype(
            rng.standard_normal((B, num_kv_heads, head_dim), dtype=np.float32), dtype
        )
        new_v = _round_to_dtype(
            rng.standard_normal((B, num_kv_heads, head_dim), dtype=np.float32), dtype
        )
        slots = np.full(B, -1, dtype=np.int64)
        for b in range(B):
            if lens[b] > 0:
                pos = int(lens[b]) - 1
                slots[b] = int(block_tables[b, pos // bs]) * bs + pos % bs
    if poison and pools:
        bad = _poison(k_cache, dtype)
        in_use = np.zeros(pool_blocks, dtype=bool)
        in_use[perm[:used]] = True
        k_cache[~in_use] = bad
        v_cache[~in_use] = bad
        for b in range(B):
            n = int(nblk[b])
            if n == 0:
                continue
            last = int(block_tables[b, n - 1])
            tail = int(lens[b]) - (n - 1) * bs
            k_cache[last, :, tail:, :] = bad
            v_cache[last, :, tail:, :] = bad
        if write:
            for b in range(B):
                if slots[b] >= 0:
                    blk, off = divmod(int(slots[b]), bs)
                    k_cache[blk, :, off, :] = bad
                    v_cache[blk, :, off, :] = bad
    if scale is None:
        scale = 1.0 / math.sqrt(head_dim)
    return Workload(
        name=name,
        dtype=dtype,
        num_seqs=B,
        num_q_heads=num_q_heads,
        num_kv_heads=num_kv_heads,
        head_dim=head_dim,
        block_size=bs,
        num_blocks=pool_blocks,
        scale=np.float32(scale),
        context_lens=lens.astype(np.int32),
        block_tables=block_tables,
        k_cache=k_cache,
        v_cache=v_cache,
        q=q,
        partition_size=partition_size,
        new_k=new_k,
        new_v=new_v,
        slot_mapping=slots,
    )


# ---------------------------------------------------------------------------
# The five named workloads.  Seed = workload number.
# ---------------------------------------------------------------------------

CONFIG_NAMES = {
    1: "tiny paged decode: 2 seqs, L={5,37}, 4q/2kv heads, D=64, bs=16, fp32",
    2: "Llama-3.2-1B layer decode: batch 16, 32q/8kv, D=64, bs=16, L~U[100,1024], fp16",
    3: "continuous-batching mix: batch 64, 32q/8kv, D=64, bs=16, L log-uniform [16,4096], bf16, write+decode",
    4: "Qwen3-style layer decode: batch 128, 16q/8kv, D=128, bs=16, L~U[2048,8192], bf16",
    5: "skewed long context: batch 256, one seq at 32768 + 255 ~U[128,2048], 32q/8kv, D=64, bs=32, fp16, P=512",
}


def config_lens(cfg: int, rng: np.random.Generator) -> np.ndarray:
    """Step 1 of the draw order for each named workload."""
    if cfg == 1:
        return np.array([5, 37], dtype=np.int64)
    if cfg == 2:
        return rng.integers(100, 1024 + 1, size=16)
    if cfg == 3:
        u = rng.uniform(math.log(16), math.log(4097), size=64)
        return np.floor(np.exp(u)).astype(np.int64)
    if cfg == 4:
        return rng.integers(2048, 8192 + 1, size=128)
    if cfg == 5:
        rest = rng.integers(128, 2048 + 1, size=255)
        return np.concatenate([[32768], rest]).astype(np.int64)
    raise ValueError(f"no workload {cfg}")


CONFIG_SHAPES = {
    1: dict(dtype="f32", num_q_heads=4, num_kv_heads=2, head_dim=64, block_size=16,
            pool_blocks=8, scale=1.0 / 8),
    2: dict(dtype="f16", num_q_heads=32, num_kv_heads=8, head_dim=64, block_size=16,
            scale=1.0 / 8),
    3: dict(dtype="bf16", num_q_heads=32, num_kv_heads=8, head_dim=64, block_size=16,
            scale=1.0 / 8),
    4: dict(dtype="bf16", num_q_heads=16, num_kv_heads=8, head_dim=128, block_size=16,
            scale=1.0 / math.sqrt(128)),
    5: dict(dtype="f16", num_q_heads=32, num_kv_heads=8, head_dim=64, block_size=32,
            scale=1.0 / 8, partition_size=512),
}


def make_config(cfg: int, *, seed: Optional[int] = None, poison: bool = True,
                write: bool = True, pools: bool = True) -> Workload:
    """Named workload ``cfg`` (1..5); ``seed`` defaults to the workload number."""
    seed = cfg if seed is None else seed
    rng = np.random.default_rng(seed)
    lens = config_lens(cfg, rng)
    shape = dict(CONFIG_SHAPES[cfg])
    wl = make_case(seed, context_lens=lens, poison=poison, write=write, rng=rng,
                   name=f"cfg{cfg}", pools=pools, **shape)
    wl.meta["config"] = cfg
    wl.meta["description"] = CONFIG_NAMES[cfg]
    return wl


# ---------------------------------------------------------------------------
# Multi-token (causal) inputs: chunked prefill and the check of drafted tokens
# ---------------------------------------------------------------------------

@dataclass
class PrefillWorkload(Workload):
    """Inputs of a multi-token call: sequence b brings T_b new query tokens
    (rows query_start[b] .. query_start[b+1] - 1 of q, [N, Hq, D]) whose K/V
    are already in the pools; context_lens[b] counts the cached tokens, the
    new ones included, so row i of sequence b sits at position
    context_lens[b] - T_b + i."""

    query_start: Optional[np.ndarray] = None  # int32 [B + 1]

    @property
    def num_query_tokens(self) -> int:
        return int(self.query_start[-1])

    @property
    def max_query_len(self) -> int:
        return int(np.diff(self.query_start).max()) if self.num_seqs else 0


def make_prefill_case(seed: int, *, dtype: str, prefix_lens: Sequence[int],
                      query_lens: Sequence[int], num_q_heads: int, num_kv_heads: int,
                      head_dim: int, block_size: int, poison: bool = True,
                      rng: Optional[np.random.Generator] = None, name: str = "prefill",
                      **kw) -> PrefillWorkload:
    """Sequences with prefix_lens[b] cached tokens and query_lens[b] new ones
    (L_b = prefix + new).  Draw order: the pool permutation, the K pool, the
    V pool and the decode q as make_case, then the query rows."""
    rng = rng if rng is not None else np.random.default_rng(seed)
    pre = np.asarray(prefix_lens, dtype=np.int64)
    new = np.asarray(query_lens, dtype=np.int64)
    if pre.shape != new.shape or (pre < 0).any() or (new < 0).any():
        raise ValueError("prefix_lens and query_lens: equal length, non-negative")
    base = make_case(seed, dtype=dtype, context_lens=pre + new, num_q_heads=num_q_heads,
                     num_kv_heads=num_kv_heads, head_dim=head_dim, block_size=block_size,
                     write=False, poison=poison, rng=rng, name=name, **kw)
    qs = np.zeros(len(new) + 1, dtype=np.int32)
    qs[1:] = np.cumsum(new)
    q = _round_to_dtype(
        rng.standard_normal((int(qs[-1]), num_q_heads, head_dim), dtype=np.float32), dtype)
    fields = {k: getattr(base, k) for k in base.__dataclass_fields__}
    fields["q"] = q
    return PrefillWorkload(**fields, query_start=qs)


PREFILL_NAMES = {
    1: "tiny multi-token: 3 seqs, cached {0,5,40} + new {7,1,20}, 8q/2kv, D=64, bs=16, fp16",
    2: "chunked prefill, Llama-3.2-1B layer: 8 seqs x 256 new tokens after U[0,3072] cached, "
       "32q/8kv, D=64, bs=16, fp16",
    3: "drafted-token check, Qwen3-style layer: 64 seqs x 5 new tokens after U[2048,8192] "
       "cached, 16q/8kv, D=128, bs=16, bf16",
}


def make_prefill_config(n: int, *, seed: Optional[int] = None, poison: bool = True,
                        pools: bool = True) -> PrefillWorkload:
    """Named multi-token workload n (1..3); seed defaults to 100 + n.  Step 1
    of the draw order is the cached lengths (the new-token counts are fixed)."""
    seed = 100 + n if seed is None else seed
    rng = np.random.default_rng(seed)
    if n == 1:
        pre, new = [0, 5, 40], [7, 1, 20]
        shape = dict(dtype="f16", num_q_heads=8, num_kv_heads=2, head_dim=64, block_size=16)
    elif n == 2:
        pre, new = rng.integers(0, 3072 + 1, size=8), [256] * 8
        shape = dict(dtype="f16", num_q_heads=32, num_kv_heads=8, head_dim=64, block_size=16)
    elif n == 3:
        pre, new = rng.integers(2048, 8192 + 1, size=64), [5] * 64
        shape = dict(dtype="bf16", num_q_heads=16, num_kv_heads=8, head_dim=128,
                     block_size=16)
    else:
        raise ValueError(f"no multi-token workload {n}")
    wl = make_prefill_case(seed, prefix_lens=pre, query_lens=new, poison=poison, rng=rng,
                           name=f"prefill{n}", pools=pools, **shape)
    wl.meta["description"] = PREFILL_NAMES[n]
    return wl


# ---------------------------------------------------------------------------
# Device transfer (data movement only)
# ---------------------------------------------------------------------------
# Group-quantised INT8 pools (codes and per-group float32 scales)
# ---------------------------------------------------------------------------

INT8_POISON_CODE = -128  # never produced by the quantiser (codes lie in [-127, 127])


def int8_code_positions(block_size: int, head_dim: int, is_value: bool) -> np.ndarray:
    """[block_size, head_dim] positions of each (token offset, dim) code
    inside one block's run of block_size * head_dim codes, in the order the
    library documents: tiles of 16 tokens (offset = 16 * tile + row), then
    for K  ((tile * 64 + 16 * ((d % 32) // 8) + row) * (D / 32) + d // 32) * 8 + d % 8
    and V  ((tile * 64 + 16 * (row // 4) + d % 16) * (D / 16) + d // 16) * 4 + row % 4."""
    off = np.arange(block_size)[:, None]
    d = np.arange(head_dim)[None, :]
    tile, row = off // 16, off % 16
    if not is_value:
        pos = ((tile * 64 + 16 * ((d % 32) // 8) + row) * (head_dim // 32) + d // 32) * 8 + d % 8
    else:
        pos = ((tile * 64 + 16 * (row // 4) + d % 16) * (head_dim // 16) + d // 16) * 4 + row % 4
    return pos.astype(np.int64)


def int8_pack(codes: np.ndarray, is_value: bool) -> np.ndarray:
    """Logical codes [NB, Hkv, bs, D] -> the pool array [NB, Hkv, bs * D]."""
    NB, H, bs, D = codes.shape
    out = np.empty((NB, H, bs * D), dtype=np.int8)
    out[:, :, int8_code_positions(bs, D, is_value).reshape(-1)] = codes.reshape(NB, H, bs * D)
    return out


def int8_unpack(pool: np.ndarray, block_size: int, head_dim: int, is_value: bool) -> np.ndarray:
    """The pool array [NB, Hkv, bs * D] -> logical codes [NB, Hkv, bs, D]."""
    pos = int8_code_positions(block_size, head_dim, is_value)
    return pool[:, :, pos]


@dataclass
class Int8Workload(Workload):
    """Decode inputs over INT8 pools.  ``dtype`` is the dtype of q (and of
    the new tokens); k_cache / v_cache are unused (None).  k_codes and
    v_codes are int8 [NB, Hkv, bs * D] in the library's order (see
    int8_code_positions); k_scales, v_scales float32 [NB, Hkv, bs, D /
    group_size]."""

    group_size: int = 0
    k_codes: Optional[np.ndarray] = None
    v_codes: Optional[np.ndarray] = None
    k_scales: Optional[np.ndarray] = None
    v_scales: Optional[np.ndarray] = None

    def kv_bytes(self) -> int:
        """Codes and scales a decode must stream: per token and kv head,
        2 * D one-byte codes and 2 * D / group_size four-byte scales."""
        total_tokens = int(self.context_lens.astype(np.int64).clip(min=0).sum())
        per = 2 * self.head_dim + 2 * (self.head_dim // self.group_size) * 4
        return total_tokens * self.num_kv_heads * per


def make_int8_case(seed: int, *, q_dtype: str, context_lens: Sequence[int], num_q_heads: int,
                   num_kv_heads: int, head_dim: int, block_size: int, group_size: int,
                   pool_blocks: Optional[int] = None, pool_factor: float = 1.25,
                   scale: Optional[float] = None, write: bool = True, poison: bool = True,
                   max_blocks_per_seq: Optional[int] = None, name: str = "int8-case",
                   rng: Optional[np.random.Generator] = None,
                   scale_range=(0.005, 0.03)) -> Int8Workload:
    """Like make_case, with INT8 pools in place of the half/fp32 ones.

    Draw order: steps 1, 2, 5, 6 of make_case (lengths, pool permutation, q
    and the new tokens, all in q_dtype), then 7. the K codes, 8. the V codes
    (uniform integers in [-127, 127], drawn as [NB, Hkv, bs, D] and laid
    out in the pool order), 9. the K scales, 10. the V scales (float32
    uniform in ``scale_range``).  With ``poison`` every scale of an
    unused block, of the tail slots >= L_b and of the slot the write will
    fill is NaN, and the codes there are INT8_POISON_CODE."""
    if head_dim % group_size:
        raise ValueError("group_size must divide head_dim")
    rng = rng if rng is not None else np.random.default_rng(seed)
    base = make_case(seed, dtype=q_dtype, context_lens=context_lens, num_q_heads=num_q_heads,
                     num_kv_heads=num_kv_heads, head_dim=head_dim, block_size=block_size,
                     pool_blocks=pool_blocks, pool_factor=pool_factor, scale=scale, write=write,
                     poison=False, max_blocks_per_seq=max_blocks_per_seq, name=name, rng=rng,
                     pools=False)
    NB, Hkv, bs, D = base.num_blocks, num_kv_heads, block_size, head_dim
    ng = D // group_size
    k_codes = rng.integers(-127, 128, size=(NB, Hkv, bs, D), dtype=np.int8)
    v_codes = rng.integers(-127, 128, size=(NB, Hkv, bs, D), dtype=np.int8)
    lo, hi = scale_range
    k_scales = rng.uniform(lo, hi, size=(NB, Hkv, bs, ng)).astype(np.float32)
    v_scales = rng.uniform(lo, hi, size=(NB, Hkv, bs, ng)).astype(np.float32)
    if poison:
        lens = base.context_lens.astype(np.int64)
        nblk = np.where(lens > 0, (lens + bs - 1) // bs, 0)
        in_use = np.zeros(NB, dtype=bool)
        for b in range(base.num_seqs):
            in_use[base.block_tables[b, : nblk[b]]] = True
        dead = np.zeros((NB, bs), dtype=bool)
        dead[~in_use] = True
        for b in range(base.num_seqs):
            n = int(nblk[b])
            if n:
                dead[int(base.block_tables[b, n - 1]), int(lens[b]) - (n - 1) * bs:] = True
        if write:
            for s in base.slot_mapping:
                if s >= 0:
                    dead[int(s) // bs, int(s) % bs] = True
        blk, off = np.nonzero(dead)
        k_scales[blk, :, off, :] = np.nan
        v_scales[blk, :, off, :] = np.nan
        k_codes[blk, :, off, :] = INT8_POISON_CODE
        v_codes[blk, :, off, :] = INT8_POISON_CODE
    k_codes = int8_pack(k_codes, False)
    v_codes = int8_pack(v_codes, True)
    fields = {f: getattr(base, f) for f in Workload.__dataclass_fields__}
    return Int8Workload(**fields, group_size=group_size, k_codes=k_codes, v_codes=v_codes,
                        k_scales=k_scales, v_scales=v_scales)


def make_int8_config(cfg: int, *, group_size: int = 32, seed: Optional[int] = None,
                     poison: bool = True, write: bool = True) -> Int8Workload:
    """Named workload ``cfg`` (1..5) over INT8 pools: its lengths, shapes and
    pool permutation, with q in the workload's dtype (fp32 for workload 1)."""
    seed = cfg if seed is None else seed
    rng = np.random.default_rng(seed)
    lens = config_lens(cfg, rng)
    shape = dict(CONFIG_SHAPES[cfg])
    q_dtype = shape.pop("dtype")
    shape.pop("partition_size", None)
    wl = make_int8_case(seed, q_dtype=q_dtype, context_lens=lens, group_size=group_size,
                        poison=poison, write=write, rng=rng, name=f"cfg{cfg}-int8", **shape)
    wl.meta["config"] = cfg
    wl.meta["description"] = CONFIG_NAMES[cfg] + f", INT8 KV (groups of {group_size})"
    return wl


def int8_device_inputs(wl: Int8Workload, device="cuda"):
    """The INT8 workload's arrays as device tensors."""
    import torch

    d = dict(
        q=as_torch(wl.q, wl.dtype, device),
        k_codes=torch.from_numpy(wl.k_codes).to(device),
        v_codes=torch.from_numpy(wl.v_codes).to(device),
        k_scales=torch.from_numpy(wl.k_scales).to(device),
        v_scales=torch.from_numpy(wl.v_scales).to(device),
        block_tables=torch.from_numpy(wl.block_tables).to(device),
        context_lens=torch.from_numpy(wl.context_lens).to(device),
    )
    if wl.new_k is not None:
        d["new_k"] = as_torch(wl.new_k, wl.dtype, device)
        d["new_v"] = as_torch(wl.new_v, wl.dtype, device)
        d["slot_mapping"] = torch.from_numpy(wl.slot_mapping).to(device)
    return d


# ---------------------------------------------------------------------------

def torch_dtype(dtype: str):
    import torch

    return {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}[dtype]


def as_torch(arr: np.ndarray, dtype: str, device="cpu"):
    """Stored bits -> torch tensor of the stored dtype (a reinterpretation)."""
    import torch

    t = torch.from_numpy(np.ascontiguousarray(arr))
    if dtype != "f32":
        t = t.view(torch.int16).view(torch_dtype(dtype))
    return t.to(device)


def to_numpy_bits(t, dtype: str) -> np.ndarray:
    """torch tensor of a stored dtype -> numpy (float32, or uint16 bits)."""
    import torch

    t = t.detach().to("cpu").contiguous()
    if dtype == "f32":
        return t.numpy().copy()
    return t.view(torch.int16).numpy().view(np.uint16).copy()


def device_inputs(wl: Workload, device="cuda"):
    """The workload's arrays as device tensors, keyed like the call arguments."""
    import torch

    d = dict(
        q=as_torch(wl.q, wl.dtype, device),
        k_cache=as_torch(wl.k_cache, wl.dtype, device),
        v_cache=as_torch(wl.v_cache, wl.dtype, device),
        block_tables=torch.from_numpy(wl.block_tables).to(device),
        context_lens=torch.from_numpy(wl.context_lens).to(device),
    )
    if wl.new_k is not None:
        d["new_k"] = as_torch(wl.new_k, wl.dtype, device)
        d["new_v"] = as_torch(wl.new_v, wl.dtype, device)
        d["slot_mapping"] = torch.from_numpy(wl.slot_mapping).to(device)
    return d
