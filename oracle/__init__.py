"""fp64 CPU oracle for paged decode attention, its multi-token causal form,
and the KV-cache write.

TEST INFRASTRUCTURE.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
benchmark's ``cpu_baseline`` leg may import this package.  The product path
(``paged_kv_attention_24_amd``) never imports it and shares no code with it.

The arithmetic lives in ``oracle.c`` (plain C99, double precision, built by
gcc with OpenMP); this module only marshals numpy arrays into it.  What it
computes, for every sequence b and query head hq with L = context_lens[b]
(PhotonInfer README, Korean translation, "Technical details > Paged
attention"; the stable softmax of "Key features > GPU-optimised kernels"):

    out[b, hq] = sum_{t<L} softmax_t(scale * q[b, hq] . K_t) V_t,
    K_t = k_cache[block_tables[b, t // bs], hq // G, t % bs, :]

with G = num_q_heads // num_kv_heads.  Every function here is pinned by the
``-m "not gpu"`` tests in ``tests/test_oracle.py`` (closed forms, invariants,
torch's fp64 scaled-dot-product attention on a contiguous copy, exhaustive
decoder checks).
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")

DTYPE_CODE = {"f32": 0, "f16": 1, "bf16": 2}
STATUS = {0: "ok", 1: "bad argument", 2: "block id out of range",
          3: "context length exceeds the block table", 4: "out of memory"}


class OracleError(RuntimeError):
    pass


# gcc flags of the sanitizer build: AddressSanitizer and UndefinedBehavior-
# Sanitizer, every finding fatal (the process must load libasan first).
SANITIZE_FLAGS = ["-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
                  "-fno-sanitize-recover=all"]


def build(force: bool = True, path: Optional[str] = None, sanitize: bool = False) -> str:
    """Compile oracle.c into liboracle.so next to it (gcc, -O2, OpenMP), or
    into ``path``; ``sanitize`` builds with SANITIZE_FLAGS instead of -O2."""
    out = path or _LIB_PATH
    if not force and os.path.exists(out):
        return out
    tmp = out + ".tmp"
    opt = SANITIZE_FLAGS if sanitize else ["-O2"]
    cmd = ["gcc", *opt, "-std=c99", "-fopenmp", "-fPIC", "-shared", "-Wall",
           "-o", tmp, _SRC, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


_lib = None


def lib(path: Optional[str] = None):
    """Load (building first if absent) and return the ctypes handle."""
    global _lib
    if path is not None:
        return _declare(ctypes.CDLL(path))
    if _lib is None and os.environ.get("ORACLE_LIBRARY"):
        # another build of oracle.c (the sanitizer build of the tests)
        _lib = _declare(ctypes.CDLL(os.environ["ORACLE_LIBRARY"]))
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            build()
        _lib = _declare(ctypes.CDLL(_LIB_PATH))
    return _lib


def _declare(h):
    P = ctypes.c_void_p
    i32, i64, f64 = ctypes.c_int32, ctypes.c_int64, ctypes.c_double
    h.oracle_f16_to_f64.argtypes = [ctypes.c_uint16]
    h.oracle_f16_to_f64.restype = f64
    h.oracle_bf16_to_f64.argtypes = [ctypes.c_uint16]
    h.oracle_bf16_to_f64.restype = f64
    h.oracle_decode_array.argtypes = [P, ctypes.c_int, i64, P]
    h.oracle_decode_array.restype = None
    h.oracle_paged_attention_decode.argtypes = [
        P, P, P, P, ctypes.c_int, P, i32, P, i32, i32, i32, i32, i32, i32, f64, i32,
        P, i32, i32]
    h.oracle_paged_attention_decode.restype = ctypes.c_int
    h.oracle_paged_attention_decode_append.argtypes = [
        P, P, P, P, P, P, i64, i64, ctypes.c_int, P, i32, P, i32, i32, i32, i32, i32, i32, f64,
        P, i32, i32]
    h.oracle_paged_attention_decode_append.restype = ctypes.c_int
    h.oracle_paged_attention_prefill.argtypes = [
        P, P, P, P, ctypes.c_int, P, i32, P, P, i32, i32, i32, i32, i32, i32, f64, P, i32, i32]
    h.oracle_paged_attention_prefill.restype = ctypes.c_int
    h.oracle_kv_cache_write.argtypes = [P, P, i64, i64, P, i32, P, P, i32, i32, i32, i32, i32]
    h.oracle_kv_cache_write_rope.argtypes = [P, P, i64, i64, P, P, i32, P, i32, i32, P, P, i32,
                                             i32, i32, i32, ctypes.c_int]
    h.oracle_kv_cache_write_rope.restype = ctypes.c_int
    h.oracle_round_array.argtypes = [P, ctypes.c_int, i64, P]
    h.oracle_round_array.restype = None
    h.oracle_copy_blocks.argtypes = [P, P, P, i32, i32, i64]
    h.oracle_copy_blocks.restype = ctypes.c_int
    h.oracle_gather_blocks.argtypes = [P, P, P, P, i32, i32, i64]
    h.oracle_gather_blocks.restype = ctypes.c_int
    h.oracle_scatter_blocks.argtypes = [P, P, P, P, i32, i32, i64]
    h.oracle_scatter_blocks.restype = ctypes.c_int
    h.oracle_kv_cache_write.restype = ctypes.c_int
    h.oracle_quantize_group.argtypes = [P, i32, P]
    h.oracle_quantize_group.restype = ctypes.c_float
    h.oracle_kv_cache_write_int8.argtypes = [P, P, i64, i64, ctypes.c_int, P, i32, P, P, P, P,
                                             i32, i32, i32, i32, i32]
    h.oracle_kv_cache_write_int8.restype = ctypes.c_int
    h.oracle_paged_attention_decode_int8.argtypes = [
        P, P, ctypes.c_int, P, P, P, P, P, i32, P, i32, i32, i32, i32, i32, i32, i32, f64, i32,
        P, i32, i32]
    h.oracle_paged_attention_decode_int8.restype = ctypes.c_int
    return h


def _ptr(a: np.ndarray):
    return ctypes.c_void_p(a.ctypes.data)


def _check_stored(a: np.ndarray, dtype: str, what: str):
    want = np.float32 if dtype == "f32" else np.uint16
    if a.dtype != want:
        raise TypeError(f"{what}: expected {np.dtype(want)} storage for {dtype}, got {a.dtype}")
    if not a.flags["C_CONTIGUOUS"]:
        raise ValueError(f"{what} must be C-contiguous")


def decode_values(bits: np.ndarray, dtype: str, handle=None) -> np.ndarray:
    """Stored elements -> float64 through the oracle's own decoders."""
    h = handle or lib()
    a = np.ascontiguousarray(bits)
    _check_stored(a, dtype, "bits")
    out = np.empty(a.size, dtype=np.float64)
    h.oracle_decode_array(_ptr(a), DTYPE_CODE[dtype], a.size, _ptr(out))
    return out.reshape(a.shape)


def paged_attention_decode(q, k_cache, v_cache, block_tables, context_lens, scale,
                           num_kv_heads, block_size, dtype, *, rows=None,
                           partition_size: int = 0, threads: int = 0,
                           handle=None) -> np.ndarray:
    """fp64 decode.  Arrays hold stored bits (float32 or uint16).

    q [B, Hq, D]; k_cache, v_cache [NB, Hkv, bs, D]; block_tables int32
    [B, MB]; context_lens int32 [B].  ``rows`` (optional, int array [n, 2] of
    (b, hq) pairs) restricts the computation to those rows; the result is then
    [n, D], else [B, Hq, D].  ``partition_size`` > 0 assembles each row from
    partitions (the split identity), 0 evaluates the definition directly.
    ``scale`` is widened to double as given (pass the float32 value the
    device receives).
    """
    h = handle or lib()
    _check_stored(q, dtype, "q")
    _check_stored(k_cache, dtype, "k_cache")
    _check_stored(v_cache, dtype, "v_cache")
    bt = np.ascontiguousarray(block_tables, dtype=np.int32)
    cl = np.ascontiguousarray(context_lens, dtype=np.int32)
    B, Hq, D = q.shape
    NB, Hkv, bs, D2 = k_cache.shape
    if v_cache.shape != k_cache.shape or D2 != D or Hkv != num_kv_heads or bs != block_size:
        raise ValueError("cache shape does not match the arguments")
    if bt.ndim != 2 or bt.shape[0] != B or cl.shape != (B,):
        raise ValueError("block_tables / context_lens do not match q")
    if rows is not None:
        r = np.ascontiguousarray(rows, dtype=np.int32).reshape(-1, 2)
        out = np.empty((r.shape[0], D), dtype=np.float64)
        rp, nr = _ptr(r), r.shape[0]
    else:
        r = None
        out = np.empty((B, Hq, D), dtype=np.float64)
        rp, nr = None, 0
    rc = h.oracle_paged_attention_decode(
        _ptr(out), _ptr(q), _ptr(k_cache), _ptr(v_cache), DTYPE_CODE[dtype], _ptr(bt),
        bt.shape[1], _ptr(cl), B, Hq, Hkv, D, NB, bs, float(scale), int(partition_size),
        rp, nr, int(threads))
    if rc != 0:
        raise OracleError(f"oracle decode failed: {STATUS.get(rc, rc)}")
    return out


def paged_attention_decode_append(q, k_cache, v_cache, k_new, v_new, block_tables,
                                  context_lens, scale, num_kv_heads, block_size, dtype, *,
                                  rows=None, threads: int = 0, handle=None) -> np.ndarray:
    """fp64 decode in which each sequence's last position L_b - 1 takes its
    key/value from k_new[b], v_new[b] ([B, Hkv, D], any token stride) rather
    than from the pool.  Same array conventions as paged_attention_decode."""
    h = handle or lib()
    for a, w in ((q, "q"), (k_cache, "k_cache"), (v_cache, "v_cache")):
        _check_stored(a, dtype, w)
    bt = np.ascontiguousarray(block_tables, dtype=np.int32)
    cl = np.ascontiguousarray(context_lens, dtype=np.int32)
    B, Hq, D = q.shape
    NB, Hkv, bs, _ = k_cache.shape
    item = k_new.itemsize
    for a in (k_new, v_new):
        want = np.float32 if dtype == "f32" else np.uint16
        if a.dtype != want or a.shape != (B, Hkv, D) or a.strides[2] != item or \
                a.strides[1] != D * item:
            raise ValueError("k_new/v_new must be [B, Hkv, D] with contiguous heads")
    if rows is not None:
        r = np.ascontiguousarray(rows, dtype=np.int32).reshape(-1, 2)
        out = np.empty((r.shape[0], D), dtype=np.float64)
        rp, nr = _ptr(r), r.shape[0]
    else:
        out = np.empty((B, Hq, D), dtype=np.float64)
        rp, nr = None, 0
    rc = h.oracle_paged_attention_decode_append(
        _ptr(out), _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(k_new), _ptr(v_new),
        k_new.strides[0] // item, v_new.strides[0] // item, DTYPE_CODE[dtype], _ptr(bt),
        bt.shape[1], _ptr(cl), B, Hq, Hkv, D, NB, bs, float(scale), rp, nr, int(threads))
    if rc != 0:
        raise OracleError(f"oracle decode failed: {STATUS.get(rc, rc)}")
    return out


def paged_attention_prefill(q, k_cache, v_cache, block_tables, context_lens, query_start,
                            scale, num_kv_heads, block_size, dtype, *, rows=None,
                            threads: int = 0, handle=None) -> np.ndarray:
    """fp64 multi-token causal paged attention.

    q [N, Hq, D] holds the query rows of all sequences, sequence b owning
    rows [query_start[b], query_start[b+1]); with T_b rows and L_b =
    context_lens[b], its row i sits at position L_b - T_b + i and attends to
    the tokens at positions 0 .. L_b - T_b + i.  ``rows`` (optional [n, 2]
    pairs (r, hq)) restricts the computation; the result is then [n, D],
    else [N, Hq, D].
    """
    h = handle or lib()
    for a, w in ((q, "q"), (k_cache, "k_cache"), (v_cache, "v_cache")):
        _check_stored(a, dtype, w)
    bt = np.ascontiguousarray(block_tables, dtype=np.int32)
    cl = np.ascontiguousarray(context_lens, dtype=np.int32)
    qs = np.ascontiguousarray(query_start, dtype=np.int32)
    N, Hq, D = q.shape
    NB, Hkv, bs, D2 = k_cache.shape
    B = cl.shape[0]
    if v_cache.shape != k_cache.shape or D2 != D or Hkv != num_kv_heads or bs != block_size:
        raise ValueError("cache shape does not match the arguments")
    if bt.ndim != 2 or bt.shape[0] != B or qs.shape != (B + 1,) or int(qs[-1]) != N:
        raise ValueError("block_tables / query_start do not match q and context_lens")
    if rows is not None:
        r = np.ascontiguousarray(rows, dtype=np.int32).reshape(-1, 2)
        out = np.empty((r.shape[0], D), dtype=np.float64)
        rp, nr = _ptr(r), r.shape[0]
    else:
        out = np.empty((N, Hq, D), dtype=np.float64)
        rp, nr = None, 0
    rc = h.oracle_paged_attention_prefill(
        _ptr(out), _ptr(q), _ptr(k_cache), _ptr(v_cache), DTYPE_CODE[dtype], _ptr(bt),
        bt.shape[1], _ptr(cl), _ptr(qs), B, Hq, Hkv, D, NB, bs, float(scale), rp, nr,
        int(threads))
    if rc != 0:
        raise OracleError(f"oracle prefill failed: {STATUS.get(rc, rc)}")
    return out


def prefill_workload(wl, *, rows=None, threads=0, handle=None):
    """Oracle multi-token attention of a workloads.PrefillWorkload."""
    return paged_attention_prefill(
        wl.q, wl.k_cache, wl.v_cache, wl.block_tables, wl.context_lens, wl.query_start,
        wl.scale, wl.num_kv_heads, wl.block_size, wl.dtype, rows=rows, threads=threads,
        handle=handle)


def kv_cache_write(k, v, slot_mapping, k_cache, v_cache, dtype, handle=None) -> None:
    """In-place bitwise write of k, v [T, Hkv, D] (token stride = row length of
    the given arrays' first axis) into the pools at ``slot_mapping``."""
    h = handle or lib()
    for a, w in ((k, "k"), (v, "v"), (k_cache, "k_cache"), (v_cache, "v_cache")):
        want = np.float32 if dtype == "f32" else np.uint16
        if a.dtype != want:
            raise TypeError(f"{w}: expected {np.dtype(want)} storage")
    if not (k_cache.flags["C_CONTIGUOUS"] and v_cache.flags["C_CONTIGUOUS"]):
        raise ValueError("caches must be C-contiguous")
    NB, Hkv, bs, D = k_cache.shape
    T = k.shape[0]
    item = k.itemsize
    for a in (k, v):
        if a.shape[1:] != (Hkv, D) or a.strides[2] != item or a.strides[1] != D * item:
            raise ValueError("k/v must be [T, Hkv, D] with contiguous heads")
    sm = np.ascontiguousarray(slot_mapping, dtype=np.int64)
    rc = h.oracle_kv_cache_write(
        _ptr(k), _ptr(v), k.strides[0] // item if T else Hkv * D,
        v.strides[0] // item if T else Hkv * D, _ptr(sm), T, _ptr(k_cache), _ptr(v_cache),
        NB, bs, Hkv, D, item)
    if rc != 0:
        raise OracleError(f"oracle write failed: {STATUS.get(rc, rc)}")


def decode_workload(wl, *, rows=None, partition_size=0, threads=0, after_write=True,
                    handle=None):
    """Oracle decode of a workloads.Workload; applies its write first (on
    copies of the pools) when it carries new tokens and after_write is set."""
    kc, vc = wl.k_cache, wl.v_cache
    if after_write and wl.new_k is not None:
        kc, vc = kc.copy(), vc.copy()
        kv_cache_write(wl.new_k, wl.new_v, wl.slot_mapping, kc, vc, wl.dtype, handle=handle)
    return paged_attention_decode(
        wl.q, kc, vc, wl.block_tables, wl.context_lens, wl.scale, wl.num_kv_heads,
        wl.block_size, wl.dtype, rows=rows, partition_size=partition_size,
        threads=threads, handle=handle)


# ---------------------------------------------------------------------------
# block movement (preemption, GPU <-> CPU paging): bit copies of whole blocks
# ---------------------------------------------------------------------------

def _pools(k_cache, v_cache):
    if k_cache.shape != v_cache.shape or k_cache.dtype != v_cache.dtype:
        raise ValueError("K and V pools must match")
    if not (k_cache.flags["C_CONTIGUOUS"] and v_cache.flags["C_CONTIGUOUS"]):
        raise ValueError("pools must be C-contiguous")
    nb = k_cache.shape[0]
    return nb, k_cache.nbytes // nb


def copy_blocks(k_cache, v_cache, pairs, handle=None) -> None:
    """In place: for each (src, dst) row of pairs (int64 [n, 2]) block dst of
    both pools becomes a copy of block src, all sources read first."""
    h = handle or lib()
    nb, bb = _pools(k_cache, v_cache)
    pr = np.ascontiguousarray(pairs, dtype=np.int64).reshape(-1, 2)
    rc = h.oracle_copy_blocks(_ptr(k_cache), _ptr(v_cache), _ptr(pr), pr.shape[0], nb, bb)
    if rc != 0:
        raise OracleError(f"oracle copy_blocks failed: {STATUS.get(rc, rc)}")


def gather_blocks(k_cache, v_cache, ids, handle=None) -> np.ndarray:
    """[n, 2, block_bytes] uint8: K then V bytes of blocks ids (int64 [n]);
    rows of invalid ids are zero."""
    h = handle or lib()
    nb, bb = _pools(k_cache, v_cache)
    ix = np.ascontiguousarray(ids, dtype=np.int64)
    out = np.zeros((ix.shape[0], 2, bb), dtype=np.uint8)
    rc = h.oracle_gather_blocks(_ptr(out), _ptr(k_cache), _ptr(v_cache), _ptr(ix), ix.shape[0],
                                nb, bb)
    if rc != 0:
        raise OracleError(f"oracle gather_blocks failed: {STATUS.get(rc, rc)}")
    return out


def scatter_blocks(k_cache, v_cache, packed, ids, handle=None) -> None:
    """In place: blocks ids (int64 [n]) of the pools take packed [n, 2,
    block_bytes] (K then V)."""
    h = handle or lib()
    nb, bb = _pools(k_cache, v_cache)
    ix = np.ascontiguousarray(ids, dtype=np.int64)
    pk = np.ascontiguousarray(packed, dtype=np.uint8)
    if pk.shape != (ix.shape[0], 2, bb):
        raise ValueError("packed must be [n, 2, block_bytes]")
    rc = h.oracle_scatter_blocks(_ptr(k_cache), _ptr(v_cache), _ptr(pk), _ptr(ix), ix.shape[0],
                                 nb, bb)
    if rc != 0:
        raise OracleError(f"oracle scatter_blocks failed: {STATUS.get(rc, rc)}")


# ---------------------------------------------------------------------------
# KV-cache write with the rotary position embedding on the new keys
# ---------------------------------------------------------------------------

def round_floats(x, dtype, handle=None) -> np.ndarray:
    """float32 -> uint16 bit patterns of dtype ("f16"/"bf16"), nearest even."""
    h = handle or lib()
    src = np.ascontiguousarray(x, dtype=np.float32)
    out = np.empty(src.shape, dtype=np.uint16)
    h.oracle_round_array(_ptr(src), DTYPE_CODE[dtype], src.size, _ptr(out))
    return out


def kv_cache_write_rope(k, v, slot_mapping, positions, cos_sin, k_cache, v_cache, dtype,
                        handle=None) -> None:
    """In place: the write of k, v [T, Hkv, D] at slot_mapping with K rotated
    at positions (int32 [T]) by the table cos_sin (float32 [max_position,
    rotary_dim]: cos then sin of each position's rotary_dim / 2 angles)."""
    h = handle or lib()
    want = np.float32 if dtype == "f32" else np.uint16
    for a, w in ((k, "k"), (v, "v"), (k_cache, "k_cache"), (v_cache, "v_cache")):
        if a.dtype != want:
            raise TypeError(f"{w}: expected {np.dtype(want)} storage")
    NB, Hkv, bs, D = k_cache.shape
    T = k.shape[0]
    item = k.itemsize
    for a in (k, v):
        if a.shape[1:] != (Hkv, D) or a.strides[2] != item or a.strides[1] != D * item:
            raise ValueError("k/v must be [T, Hkv, D] with contiguous heads")
    sm = np.ascontiguousarray(slot_mapping, dtype=np.int64)
    pos = np.ascontiguousarray(positions, dtype=np.int32)
    cs = np.ascontiguousarray(cos_sin, dtype=np.float32)
    rc = h.oracle_kv_cache_write_rope(
        _ptr(k), _ptr(v), k.strides[0] // item if T else Hkv * D,
        v.strides[0] // item if T else Hkv * D, _ptr(sm), _ptr(pos), T, _ptr(cs), cs.shape[0],
        cs.shape[1], _ptr(k_cache), _ptr(v_cache), NB, bs, Hkv, D, DTYPE_CODE[dtype])
    if rc != 0:
        raise OracleError(f"oracle rope write failed: {STATUS.get(rc, rc)}")


# ---------------------------------------------------------------------------
# group-quantised INT8 KV cache (PhotonInfer README, "Technical details >
# INT8 quantisation": groups of 32, 64 or 128; applied here to the KV rows)
# ---------------------------------------------------------------------------

def quantize_group(x, handle=None):
    """One group of float32 values -> (int8 codes, float32 scale):
    s = amax / 127 and c = rint(x / s) in float32 (ties to even)."""
    h = handle or lib()
    a = np.ascontiguousarray(x, dtype=np.float32)
    codes = np.empty(a.size, dtype=np.int8)
    s = h.oracle_quantize_group(_ptr(a), a.size, _ptr(codes))
    return codes, np.float32(s)


def int8_pools(num_blocks, num_kv_heads, block_size, head_dim, group_size, fill_code=0,
               fill_scale=np.nan):
    """Empty INT8 pools: (k_codes, v_codes [NB, Hkv, bs * D] int8 in the
    documented operand order, k_scales, v_scales [NB, Hkv, bs, D /
    group_size] float32) filled with the given values."""
    G = head_dim // group_size
    kc = np.full((num_blocks, num_kv_heads, block_size * head_dim), fill_code, dtype=np.int8)
    vc = np.full((num_blocks, num_kv_heads, block_size * head_dim), fill_code, dtype=np.int8)
    ks = np.full((num_blocks, num_kv_heads, block_size, G), fill_scale, dtype=np.float32)
    vs = np.full((num_blocks, num_kv_heads, block_size, G), fill_scale, dtype=np.float32)
    return kc, vc, ks, vs


def _check_int8_pools(k_codes, v_codes, k_scales, v_scales):
    if k_scales.dtype != np.float32 or k_scales.ndim != 4 or v_scales.shape != k_scales.shape:
        raise ValueError("k_scales / v_scales float32 [NB,Hkv,bs,D/group] expected")
    NB, Hkv, bs, G = k_scales.shape
    if k_codes.dtype != np.int8 or v_codes.dtype != np.int8 or k_codes.ndim != 3 or \
            v_codes.shape != k_codes.shape or k_codes.shape[:2] != (NB, Hkv) or \
            k_codes.shape[2] % bs:
        raise ValueError("k_codes / v_codes int8 [NB,Hkv,bs*D] expected")
    D = k_codes.shape[2] // bs
    if D % G:
        raise ValueError("group count must divide head_dim")
    for a in (k_codes, v_codes, k_scales, v_scales):
        if not a.flags["C_CONTIGUOUS"]:
            raise ValueError("INT8 pools must be C-contiguous")
    return NB, Hkv, bs, D, D // G


def kv_cache_write_int8(k, v, slot_mapping, k_codes, v_codes, k_scales, v_scales, dtype,
                        handle=None) -> None:
    """In-place quantised write of k, v [T, Hkv, D] (stored bits of ``dtype``)
    into the INT8 pools at ``slot_mapping``."""
    h = handle or lib()
    NB, Hkv, bs, D, gs = _check_int8_pools(k_codes, v_codes, k_scales, v_scales)
    want = np.float32 if dtype == "f32" else np.uint16
    T = k.shape[0]
    item = k.itemsize
    for a in (k, v):
        if a.dtype != want or a.shape[1:] != (Hkv, D) or a.strides[2] != item or \
                a.strides[1] != D * item:
            raise ValueError("k/v must be [T, Hkv, D] stored bits with contiguous heads")
    sm = np.ascontiguousarray(slot_mapping, dtype=np.int64)
    rc = h.oracle_kv_cache_write_int8(
        _ptr(k), _ptr(v), k.strides[0] // item if T else Hkv * D,
        v.strides[0] // item if T else Hkv * D, DTYPE_CODE[dtype], _ptr(sm), T, _ptr(k_codes),
        _ptr(v_codes), _ptr(k_scales), _ptr(v_scales), NB, bs, Hkv, D, gs)
    if rc != 0:
        raise OracleError(f"oracle INT8 write failed: {STATUS.get(rc, rc)}")


def paged_attention_decode_int8(q, q_dtype, k_codes, v_codes, k_scales, v_scales, block_tables,
                                context_lens, scale, num_kv_heads, block_size, *, rows=None,
                                partition_size: int = 0, threads: int = 0,
                                handle=None) -> np.ndarray:
    """fp64 decode over INT8 pools (values code * scale); q [B, Hq, D] holds
    stored bits of ``q_dtype``.  ``rows``, ``partition_size`` and ``threads``
    as for paged_attention_decode."""
    h = handle or lib()
    _check_stored(q, q_dtype, "q")
    NB, Hkv, bs, D, gs = _check_int8_pools(k_codes, v_codes, k_scales, v_scales)
    bt = np.ascontiguousarray(block_tables, dtype=np.int32)
    cl = np.ascontiguousarray(context_lens, dtype=np.int32)
    B, Hq, D2 = q.shape
    if D2 != D or Hkv != num_kv_heads or bs != block_size:
        raise ValueError("pool shape does not match the arguments")
    if bt.ndim != 2 or bt.shape[0] != B or cl.shape != (B,):
        raise ValueError("block_tables / context_lens do not match q")
    if rows is not None:
        r = np.ascontiguousarray(rows, dtype=np.int32).reshape(-1, 2)
        out = np.empty((r.shape[0], D), dtype=np.float64)
        rp, nr = _ptr(r), r.shape[0]
    else:
        out = np.empty((B, Hq, D), dtype=np.float64)
        rp, nr = None, 0
    rc = h.oracle_paged_attention_decode_int8(
        _ptr(out), _ptr(q), DTYPE_CODE[q_dtype], _ptr(k_codes), _ptr(v_codes), _ptr(k_scales),
        _ptr(v_scales), _ptr(bt), bt.shape[1], _ptr(cl), B, Hq, Hkv, D, NB, bs, gs,
        float(scale), int(partition_size), rp, nr, int(threads))
    if rc != 0:
        raise OracleError(f"oracle INT8 decode failed: {STATUS.get(rc, rc)}")
    return out
