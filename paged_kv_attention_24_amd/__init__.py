"""Paged KV attention for AMD Instinct MI355X (gfx950).

Thin Python binding over the C ABI in ``include/pka.h`` (``libpka.so``,
built in this directory).  PyTorch supplies device memory and the current
stream; every step of the computation runs in the library's HIP kernels.
There is no CPU or PyTorch fallback: if the library is missing, or a tensor
is not on a GPU, the calls raise.

Operations (PhotonInfer README, Korean translation, "Technical details >
Paged attention" and "Key features > GPU-optimised kernels"):

  kv_cache_write(k, v, slot_mapping, k_cache, v_cache)
      one launch stores the new K/V rows of many sequences into the pools.
  paged_attention_decode(q, k_cache, v_cache, block_tables, context_lens,
                         scale, num_kv_heads, block_size)
      batched one-token attention over the block-wise cache.
  paged_attention_prefill(q, k_cache, v_cache, block_tables, context_lens,
                          query_start, scale, num_kv_heads, block_size)
      its multi-token causal form (chunked prefill, drafted-token check;
      "Continuous batching scheduler" and "Roadmap" of the same README).
  kv_cache_write_rope(k, v, slot_mapping, positions, cos_sin, k_cache, v_cache)
      the write with the rotary embedding applied to the new keys ("batched
      RoPE" among the README's fused operations).
  copy_blocks / gather_blocks / scatter_blocks / swap_out / swap_in
      whole-block moves for preempted requests and GPU <-> CPU paging.
  kv_cache_write_int8 / paged_attention_decode_int8
      the write and the decode over group-quantised INT8 pools ("Technical
      details > INT8 quantisation": groups of 32, 64 or 128).

Pools are [num_blocks, num_kv_heads, block_size, head_dim].

PKA_LIBRARY, if set, names another library file of this directory to load
instead of libpka.so (a build of the same sources with other flags).
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

__all__ = [
    "PkaError", "kv_cache_write", "paged_attention_decode", "paged_attention_decode_append",
    "paged_attention_decode_noalloc",
    "paged_attention_prefill", "kv_cache_write_rope", "copy_blocks", "gather_blocks", "scatter_blocks", "swap_out",
    "swap_in",
    "decode_partition_size",
    "decode_workspace_bytes", "PagedKVCache", "library_path", "load_library",
    "kv_cache_write_int8", "paged_attention_decode_int8", "decode_int8_partition_size",
    "decode_int8_workspace_bytes", "int8_pools", "paged_attention_decode_append_int8",
]

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_NAME = os.environ.get("PKA_LIBRARY", "libpka.so")
if os.path.basename(_LIB_NAME) != _LIB_NAME or not _LIB_NAME.startswith("libpka"):
    raise ImportError(f"PKA_LIBRARY={_LIB_NAME!r}: expected a libpka*.so file name of the package")
_LIB_PATH = os.path.join(_HERE, _LIB_NAME)

PKA_OK = 0
_DTYPE_CODES = None  # filled lazily (needs torch)


class PkaError(RuntimeError):
    """A non-OK pka_status; ``status`` holds the code."""

    def __init__(self, status: int, message: str):
        super().__init__(message)
        self.status = status


_lib = None


def library_path() -> str:
    return _LIB_PATH


def load_library():
    """Load libpka.so (built by ``paged_kv_attention_24_amd._build``)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        raise RuntimeError(
            f"{_LIB_PATH} is missing: build it with `python -m paged_kv_attention_24_amd._build` "
            "(or __graft_entry__.build()); there is no fallback path")
    lib = ctypes.CDLL(_LIB_PATH)
    P, i32, i64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64
    lib.pka_kv_cache_write.argtypes = [P, P, i64, i64, P, i32, P, P, i32, i32, i32, i32,
                                       ctypes.c_int, P]
    lib.pka_kv_cache_write.restype = ctypes.c_int
    lib.pka_decode_partition_size.argtypes = [i32, i32, i32, i32]
    lib.pka_decode_partition_size.restype = i32
    lib.pka_decode_workspace_bytes.argtypes = [i32, i32, i32, i32]
    lib.pka_decode_workspace_bytes.restype = ctypes.c_size_t
    lib.pka_paged_attention_decode.argtypes = [
        P, ctypes.c_int, P, P, P, P, i32, P, i32, i32, i32, i32, i32, i32, ctypes.c_float,
        ctypes.c_int, i32, i32, P, ctypes.c_size_t, P]
    lib.pka_paged_attention_decode.restype = ctypes.c_int
    lib.pka_paged_attention_decode_noalloc.argtypes = [
        P, ctypes.c_int, P, P, P, P, i32, P, i32, i32, i32, i32, i32, i32, ctypes.c_float,
        ctypes.c_int, i32, i32, P]
    lib.pka_paged_attention_decode_noalloc.restype = ctypes.c_int
    lib.pka_paged_attention_decode_append.argtypes = [
        P, ctypes.c_int, P, P, P, i64, i64, P, P, P, P, i32, P, i32, i32, i32, i32, i32, i32,
        ctypes.c_float, ctypes.c_int, i32, i32, P, ctypes.c_size_t, P]
    lib.pka_paged_attention_decode_append.restype = ctypes.c_int
    lib.pka_paged_attention_prefill.argtypes = [
        P, ctypes.c_int, P, P, P, P, i32, P, P, i32, i32, i32, i32, i32, i32, i32, i32,
        ctypes.c_float, ctypes.c_int, P]
    lib.pka_paged_attention_prefill.restype = ctypes.c_int
    lib.pka_kv_cache_write_rope.argtypes = [P, P, i64, i64, P, P, i32, P, i32, i32, P, P, i32,
                                            i32, i32, i32, ctypes.c_int, P]
    lib.pka_kv_cache_write_rope.restype = ctypes.c_int
    lib.pka_copy_blocks.argtypes = [P, P, P, i32, i32, i64, P]
    lib.pka_copy_blocks.restype = ctypes.c_int
    lib.pka_gather_blocks.argtypes = [P, P, P, P, i32, i32, i64, P]
    lib.pka_gather_blocks.restype = ctypes.c_int
    lib.pka_scatter_blocks.argtypes = [P, P, P, P, i32, i32, i64, P]
    lib.pka_scatter_blocks.restype = ctypes.c_int
    lib.pka_kv_cache_write_int8.argtypes = [P, P, i64, i64, ctypes.c_int, P, i32, P, P, P, P,
                                            i32, i32, i32, i32, i32, P]
    lib.pka_kv_cache_write_int8.restype = ctypes.c_int
    lib.pka_decode_int8_partition_size.argtypes = [i32, i32, i32, i32]
    lib.pka_decode_int8_partition_size.restype = i32
    lib.pka_decode_int8_workspace_bytes.argtypes = [i32, i32, i32, i32, i32]
    lib.pka_decode_int8_workspace_bytes.restype = ctypes.c_size_t
    lib.pka_paged_attention_decode_int8.argtypes = [
        P, ctypes.c_int, P, ctypes.c_int, P, P, P, P, P, i32, P, i32, i32, i32, i32, i32, i32,
        i32, ctypes.c_float, i32, i32, P, ctypes.c_size_t, P]
    lib.pka_paged_attention_decode_int8.restype = ctypes.c_int
    lib.pka_paged_attention_decode_append_int8.argtypes = [
        P, ctypes.c_int, P, ctypes.c_int, P, P, i64, i64, P, P, P, P, P, P, i32, P, i32, i32, i32,
        i32, i32, i32, i32, ctypes.c_float, i32, i32, P, ctypes.c_size_t, P]
    lib.pka_paged_attention_decode_append_int8.restype = ctypes.c_int
    lib.pka_status_string.argtypes = [ctypes.c_int]
    lib.pka_status_string.restype = ctypes.c_char_p
    lib.pka_last_error.argtypes = []
    lib.pka_last_error.restype = ctypes.c_char_p
    lib.pka_abi_version.argtypes = []
    lib.pka_abi_version.restype = i32
    _lib = lib
    return lib


def _check(status: int):
    if status != PKA_OK:
        lib = load_library()
        name = lib.pka_status_string(status).decode()
        detail = lib.pka_last_error().decode()
        raise PkaError(status, f"pka: {name}: {detail}")


PKA_ERR_INVALID_ARGUMENT = 1


def _invalid(msg: str):
    raise PkaError(PKA_ERR_INVALID_ARGUMENT, f"pka: invalid argument (validate=True): {msg}")


def _first(mask) -> tuple:
    import torch

    return tuple(int(x) for x in torch.nonzero(mask)[0])


def _validate_tables(block_tables, context_lens, num_blocks: int, block_size: int, hint: int = 0):
    """The device-data checks behind ``validate=True`` (they synchronise the
    stream): every length within the block table (and within the host hint
    when one is given), and every block-table entry a length uses inside
    [0, num_blocks).  The kernels clamp such inputs instead of failing."""
    import torch

    L = context_lens.to(torch.int64)
    if L.numel() == 0:
        return
    MB = block_tables.shape[1]
    cap = MB * block_size
    if bool((L > cap).any()):
        (b,) = _first(L > cap)
        _invalid(f"context_lens[{b}] = {int(L[b])} exceeds the table ({MB} blocks of {block_size})")
    if hint > 0 and bool((L > hint).any()):
        (b,) = _first(L > hint)
        _invalid(f"context_lens[{b}] = {int(L[b])} exceeds max_context_len = {hint}")
    used = (L.clamp(min=0) + block_size - 1) // block_size
    col = torch.arange(MB, device=L.device)
    bad = (col[None, :] < used[:, None]) & ((block_tables < 0) | (block_tables >= num_blocks))
    if bool(bad.any()):
        b, j = _first(bad)
        _invalid(f"block_tables[{b}, {j}] = {int(block_tables[b, j])} is outside [0, {num_blocks})")


def _validate_slots(slot_mapping, num_slots: int, block_tables=None, context_lens=None,
                    block_size: int = 0):
    """Stored slots (those inside the pool) must be distinct; with a block
    table, a slot stored for the last position of a sequence must not be
    one the same call reads for another position of any sequence."""
    import torch

    s = slot_mapping.to(torch.int64)
    store = (s >= 0) & (s < num_slots)
    if context_lens is not None:
        store &= context_lens.to(torch.int64) > 0
    st = s[store]
    if st.numel() != torch.unique(st).numel():
        _invalid("slot_mapping stores two tokens in one slot")
    if block_tables is None or st.numel() == 0:
        return
    L = context_lens.to(torch.int64).clamp(min=0)
    n_read = (L - 1).clamp(min=0)
    total = int(n_read.sum())
    if total == 0:
        return
    dev = L.device
    bi = torch.repeat_interleave(torch.arange(L.numel(), device=dev), n_read)
    start = torch.cumsum(n_read, 0) - n_read
    t = torch.arange(total, device=dev) - start[bi]
    read = block_tables[bi, t // block_size].to(torch.int64) * block_size + t % block_size
    if bool(torch.isin(st, read).any()):
        _invalid("a slot in slot_mapping is also read for another position")


def _dtype_code(dt) -> int:
    import torch

    codes = {torch.float32: 0, torch.float16: 1, torch.bfloat16: 2}
    if dt not in codes:
        raise TypeError(f"unsupported dtype {dt}; expected float32, float16 or bfloat16")
    return codes[dt]


def _stream_ptr(device) -> int:
    import torch

    return torch.cuda.current_stream(device).cuda_stream


def _require_gpu(*tensors):
    for t in tensors:
        if not t.is_cuda:
            raise ValueError("all tensors must be on a GPU; the library has no CPU path")
    dev = tensors[0].device
    for t in tensors[1:]:
        if t.device != dev:
            raise ValueError("all tensors must be on the same device")


def kv_cache_write(k, v, slot_mapping, k_cache, v_cache, *, validate: bool = False) -> None:
    """Store k, v [T, Hkv, D] into the pools at slot_mapping (int64 [T]).

    Slot s addresses block s // block_size, offset s % block_size; negative
    slots are skipped.  Bit-exact copy; mutates k_cache and v_cache.
    ``validate=True`` first checks on the device (synchronising) that the
    stored slots are distinct, and raises PkaError otherwise.
    """
    import torch

    _require_gpu(k, v, slot_mapping, k_cache, v_cache)
    if k_cache.dim() != 4 or v_cache.shape != k_cache.shape:
        raise ValueError("caches must be [num_blocks, num_kv_heads, block_size, head_dim]")
    NB, Hkv, bs, D = k_cache.shape
    if not (k_cache.is_contiguous() and v_cache.is_contiguous()):
        raise ValueError("caches must be contiguous")
    for name, t in (("k", k), ("v", v)):
        if t.dim() != 3 or tuple(t.shape[1:]) != (Hkv, D):
            raise ValueError(f"{name} must be [T, {Hkv}, {D}], got {tuple(t.shape)}")
        if t.stride(2) != 1 or t.stride(1) != D:
            raise ValueError(f"{name} must have contiguous heads (strides [*, {D}, 1])")
        if t.dtype != k_cache.dtype or v_cache.dtype != k_cache.dtype:
            raise TypeError("k, v and the caches must share one dtype")
    if slot_mapping.dtype != torch.int64 or slot_mapping.shape != (k.shape[0],) or \
            v.shape[0] != k.shape[0]:
        raise ValueError("slot_mapping must be int64 [T] with T = k.shape[0] = v.shape[0]")
    slot_mapping = slot_mapping.contiguous()
    T = k.shape[0]
    if validate:
        _validate_slots(slot_mapping, NB * bs)
    lib = load_library()
    _check(lib.pka_kv_cache_write(
        k.data_ptr(), v.data_ptr(), k.stride(0) if T else Hkv * D, v.stride(0) if T else Hkv * D,
        slot_mapping.data_ptr(), T, k_cache.data_ptr(), v_cache.data_ptr(), NB, bs, Hkv, D,
        _dtype_code(k_cache.dtype), _stream_ptr(k_cache.device)))


def decode_partition_size(num_seqs: int, num_kv_heads: int, block_size: int,
                          max_context_len: int) -> int:
    return int(load_library().pka_decode_partition_size(num_seqs, num_kv_heads, block_size,
                                                        max_context_len))


def decode_workspace_bytes(num_seqs: int, num_q_heads: int, num_kv_heads: int,
                           head_dim: int) -> int:
    """Bytes of scratch the decode needs on the current device (report
    counters plus two partial-result slots per wave of the decode grid); it
    does not depend on the context lengths."""
    return int(load_library().pka_decode_workspace_bytes(num_seqs, num_q_heads, num_kv_heads,
                                                         head_dim))


def _decode_setup(q, k_cache, v_cache, block_tables, context_lens, num_kv_heads, block_size,
                  out, out_dtype, partition_size, max_context_len, workspace,
                  use_workspace: bool = True):
    import torch

    _require_gpu(q, k_cache, v_cache, block_tables, context_lens)
    if k_cache.dim() != 4 or v_cache.shape != k_cache.shape:
        raise ValueError("caches must be [num_blocks, num_kv_heads, block_size, head_dim]")
    NB, Hkv, bs, D = k_cache.shape
    if Hkv != num_kv_heads or bs != block_size:
        raise ValueError(f"cache shape {tuple(k_cache.shape)} does not match num_kv_heads="
                         f"{num_kv_heads}, block_size={block_size}")
    if not (k_cache.is_contiguous() and v_cache.is_contiguous()):
        raise ValueError("caches must be contiguous")
    if q.dim() != 3 or q.shape[2] != D:
        raise ValueError(f"q must be [B, Hq, {D}]")
    if q.dtype != k_cache.dtype or v_cache.dtype != k_cache.dtype:
        raise TypeError("q and the caches must share one dtype")
    q = q.contiguous()
    B, Hq, _ = q.shape
    if block_tables.dtype != torch.int32 or block_tables.dim() != 2 or block_tables.shape[0] != B:
        raise ValueError("block_tables must be int32 [B, max_blocks_per_seq]")
    if context_lens.dtype != torch.int32 or context_lens.shape != (B,):
        raise ValueError("context_lens must be int32 [B]")
    block_tables = block_tables.contiguous()
    context_lens = context_lens.contiguous()
    MB = block_tables.shape[1]
    if out is None:
        odt = torch.float32 if out_dtype is None else out_dtype
        out = torch.empty((B, Hq, D), dtype=odt, device=q.device)
    else:
        if tuple(out.shape) != (B, Hq, D) or not out.is_contiguous() or out.device != q.device:
            raise ValueError("out must be a contiguous [B, Hq, D] tensor on q's device")
    hint = max_context_len if max_context_len > 0 else MB * bs
    hint = min(hint, MB * bs)
    P = int(partition_size)  # 0: the library default; the C ABI rejects bad values
    ws_ptr, ws_bytes = None, 0
    if B > 0 and use_workspace:
        need = decode_workspace_bytes(B, Hq, Hkv, D)
        if workspace is None:
            workspace = _cached_workspace(q.device, need)
        elif workspace.numel() * workspace.element_size() < need:
            raise ValueError(f"workspace holds {workspace.numel() * workspace.element_size()} "
                             f"bytes, {need} needed")
        ws_ptr, ws_bytes = workspace.data_ptr(), workspace.numel() * workspace.element_size()
    return dict(q=q, block_tables=block_tables, context_lens=context_lens, out=out, B=B, Hq=Hq,
                Hkv=Hkv, D=D, NB=NB, bs=bs, MB=MB, hint=hint, P=P, ws_ptr=ws_ptr,
                ws_bytes=ws_bytes)


def paged_attention_decode(q, k_cache, v_cache, block_tables, context_lens, scale: float,
                           num_kv_heads: int, block_size: int, *, out=None, out_dtype=None,
                           partition_size: int = 0, max_context_len: int = 0,
                           workspace=None, validate: bool = False):
    """out[b, hq] = softmax(scale * q[b, hq] . K^T) V over sequence b's cache.

    q [B, Hq, D] (the KV dtype); pools [NB, Hkv, bs, D]; block_tables int32
    [B, MB]; context_lens int32 [B] (device).  Returns out [B, Hq, D], fp32
    unless ``out_dtype`` (or ``out``) says the KV dtype.  ``max_context_len``
    is an optional host hint (no device sync); ``partition_size`` 0 lets the
    library choose.  ``workspace`` (uint8 device tensor, zero-filled before
    its first use; each call leaves it reusable) defaults to a cached one per
    device.  ``validate=True`` first checks the device data (synchronising):
    every length within the block table and within ``max_context_len`` when
    given, every block id a length uses inside the pool; PkaError otherwise.
    """
    a = _decode_setup(q, k_cache, v_cache, block_tables, context_lens, num_kv_heads,
                      block_size, out, out_dtype, partition_size, max_context_len, workspace)
    if a["B"] == 0:
        return a["out"]
    if validate:
        _validate_tables(a["block_tables"], a["context_lens"], a["NB"], a["bs"], max_context_len)
    lib = load_library()
    _check(lib.pka_paged_attention_decode(
        a["out"].data_ptr(), _dtype_code(a["out"].dtype), a["q"].data_ptr(), k_cache.data_ptr(),
        v_cache.data_ptr(), a["block_tables"].data_ptr(), a["MB"], a["context_lens"].data_ptr(),
        a["B"], a["Hq"], a["Hkv"], a["D"], a["NB"], a["bs"], float(scale),
        _dtype_code(k_cache.dtype), a["hint"], a["P"], a["ws_ptr"], a["ws_bytes"],
        _stream_ptr(q.device)))
    return a["out"]


def paged_attention_decode_noalloc(q, k_cache, v_cache, block_tables, context_lens,
                                   scale: float, num_kv_heads: int, block_size: int, *, out,
                                   partition_size: int = 0, max_context_len: int = 0):
    """paged_attention_decode into ``out`` with the library's static device
    scratch instead of a workspace: the call allocates no device memory when
    its inputs are already contiguous.  Calls that overlap on one GPU race
    (they share that scratch)."""
    if out is None:
        raise ValueError("out is required (the call allocates nothing)")
    a = _decode_setup(q, k_cache, v_cache, block_tables, context_lens, num_kv_heads,
                      block_size, out, None, partition_size, max_context_len, None,
                      use_workspace=False)
    if a["B"] == 0:
        return a["out"]
    lib = load_library()
    _check(lib.pka_paged_attention_decode_noalloc(
        a["out"].data_ptr(), _dtype_code(a["out"].dtype), a["q"].data_ptr(), k_cache.data_ptr(),
        v_cache.data_ptr(), a["block_tables"].data_ptr(), a["MB"], a["context_lens"].data_ptr(),
        a["B"], a["Hq"], a["Hkv"], a["D"], a["NB"], a["bs"], float(scale),
        _dtype_code(k_cache.dtype), a["hint"], a["P"], _stream_ptr(q.device)))
    return a["out"]


def paged_attention_decode_append(q, k_new, v_new, slot_mapping, k_cache, v_cache, block_tables,
                                  context_lens, scale: float, num_kv_heads: int,
                                  block_size: int, *, out=None, out_dtype=None,
                                  partition_size: int = 0, max_context_len: int = 0,
                                  workspace=None, validate: bool = False):
    """One fused decode step: store each sequence's new token (k_new[b],
    v_new[b], [B, Hkv, D]) at slot_mapping[b] (int64 [B]) and attend over
    its L_b tokens, the last of which is that new token.  Equal, bit for bit,
    to kv_cache_write followed by paged_attention_decode when slot_mapping[b]
    is the slot of position L_b - 1.  Mutates the pools; returns out.
    ``validate=True``: the checks of paged_attention_decode, plus distinct
    stored slots, none of them read for another position by this call."""
    import torch

    a = _decode_setup(q, k_cache, v_cache, block_tables, context_lens, num_kv_heads,
                      block_size, out, out_dtype, partition_size, max_context_len, workspace)
    B, Hkv, D = a["B"], a["Hkv"], a["D"]
    _require_gpu(k_new, v_new, slot_mapping)
    for name, t in (("k_new", k_new), ("v_new", v_new)):
        if t.dim() != 3 or tuple(t.shape) != (B, Hkv, D):
            raise ValueError(f"{name} must be [{B}, {Hkv}, {D}], got {tuple(t.shape)}")
        if t.stride(2) != 1 or t.stride(1) != D:
            raise ValueError(f"{name} must have contiguous heads (strides [*, {D}, 1])")
        if t.dtype != k_cache.dtype:
            raise TypeError(f"{name} must have the pools' dtype")
    if slot_mapping.dtype != torch.int64 or slot_mapping.shape != (B,):
        raise ValueError("slot_mapping must be int64 [B]")
    slot_mapping = slot_mapping.contiguous()
    if B == 0:
        return a["out"]
    if validate:
        _validate_tables(a["block_tables"], a["context_lens"], a["NB"], a["bs"], max_context_len)
        _validate_slots(slot_mapping, a["NB"] * a["bs"], a["block_tables"], a["context_lens"],
                        a["bs"])
    lib = load_library()
    _check(lib.pka_paged_attention_decode_append(
        a["out"].data_ptr(), _dtype_code(a["out"].dtype), a["q"].data_ptr(), k_new.data_ptr(),
        v_new.data_ptr(), k_new.stride(0), v_new.stride(0), slot_mapping.data_ptr(),
        k_cache.data_ptr(), v_cache.data_ptr(), a["block_tables"].data_ptr(), a["MB"],
        a["context_lens"].data_ptr(), B, a["Hq"], Hkv, D, a["NB"], a["bs"], float(scale),
        _dtype_code(k_cache.dtype), a["hint"], a["P"], a["ws_ptr"], a["ws_bytes"],
        _stream_ptr(q.device)))
    return a["out"]


def paged_attention_prefill(q, k_cache, v_cache, block_tables, context_lens, query_start,
                            scale: float, num_kv_heads: int, block_size: int, *, out=None,
                            out_dtype=None, max_query_len: int = 0, validate: bool = False):
    """Multi-token causal attention: q [N, Hq, D] holds the new tokens of all
    sequences, sequence b owning rows query_start[b] .. query_start[b+1] - 1
    (int32 [B + 1]); their K/V are already in the pools and context_lens[b]
    counts them, so new token i of sequence b sits at position
    context_lens[b] - T_b + i and attends to positions 0 .. that one.
    max_query_len, an upper bound of T_b, sizes the grid (0: N).  Returns
    out [N, Hq, D].  ``validate=True`` first checks the device data
    (synchronising): query_start non-decreasing from 0 to N, T_b <= L_b,
    T_b <= max_query_len when given, and the decode's table checks;
    PkaError otherwise."""
    import torch

    _require_gpu(q, k_cache, v_cache, block_tables, context_lens, query_start)
    if k_cache.dim() != 4 or v_cache.shape != k_cache.shape:
        raise ValueError("caches must be [num_blocks, num_kv_heads, block_size, head_dim]")
    NB, Hkv, bs, D = k_cache.shape
    if Hkv != num_kv_heads or bs != block_size:
        raise ValueError(f"cache shape {tuple(k_cache.shape)} does not match num_kv_heads="
                         f"{num_kv_heads}, block_size={block_size}")
    if not (k_cache.is_contiguous() and v_cache.is_contiguous()):
        raise ValueError("caches must be contiguous")
    if q.dim() != 3 or q.shape[2] != D:
        raise ValueError(f"q must be [N, Hq, {D}]")
    if q.dtype != k_cache.dtype or v_cache.dtype != k_cache.dtype:
        raise TypeError("q and the caches must share one dtype")
    q = q.contiguous()
    N, Hq, _ = q.shape
    B = context_lens.shape[0] if context_lens.dim() == 1 else -1
    if context_lens.dtype != torch.int32 or B < 0:
        raise ValueError("context_lens must be int32 [B]")
    if block_tables.dtype != torch.int32 or block_tables.dim() != 2 or block_tables.shape[0] != B:
        raise ValueError("block_tables must be int32 [B, max_blocks_per_seq]")
    if query_start.dtype != torch.int32 or tuple(query_start.shape) != (B + 1,):
        raise ValueError("query_start must be int32 [B + 1]")
    block_tables = block_tables.contiguous()
    context_lens = context_lens.contiguous()
    query_start = query_start.contiguous()
    if out is None:
        odt = torch.float32 if out_dtype is None else out_dtype
        out = torch.empty((N, Hq, D), dtype=odt, device=q.device)
    elif tuple(out.shape) != (N, Hq, D) or not out.is_contiguous() or out.device != q.device:
        raise ValueError("out must be a contiguous [N, Hq, D] tensor on q's device")
    if B == 0 or N == 0:
        return out
    if validate:
        qs = query_start.to(torch.int64)
        if int(qs[0]) != 0 or int(qs[-1]) != N or bool((qs[1:] < qs[:-1]).any()):
            _invalid(f"query_start must run non-decreasing from 0 to {N}")
        T = qs[1:] - qs[:-1]
        L = context_lens.to(torch.int64)
        if bool((T > L).any()):
            (b,) = _first(T > L)
            _invalid(f"sequence {b} has {int(T[b])} new tokens but context_lens {int(L[b])}")
        if max_query_len > 0 and bool((T > max_query_len).any()):
            (b,) = _first(T > max_query_len)
            _invalid(f"sequence {b} has {int(T[b])} new tokens, max_query_len = {max_query_len}")
        _validate_tables(block_tables, context_lens, NB, bs)
    lib = load_library()
    _check(lib.pka_paged_attention_prefill(
        out.data_ptr(), _dtype_code(out.dtype), q.data_ptr(), k_cache.data_ptr(),
        v_cache.data_ptr(), block_tables.data_ptr(), block_tables.shape[1],
        context_lens.data_ptr(), query_start.data_ptr(), B, N, int(max_query_len), Hq, Hkv, D,
        NB, bs, float(scale), _dtype_code(k_cache.dtype), _stream_ptr(q.device)))
    return out


def kv_cache_write_rope(k, v, slot_mapping, positions, cos_sin, k_cache, v_cache):
    """kv_cache_write with the rotary embedding applied to the new keys:
    token i at position positions[i] (int32 [T]; outside the table: skipped)
    has each K row rotated by the angles of cos_sin (float32 [max_position,
    rotary_dim]: per position the rotary_dim / 2 cosines, then the sines),
    pairing dims j and j + rotary_dim / 2, in fp32 rounded to the pool
    dtype.  V rows are stored unchanged."""
    import torch

    _require_gpu(k, v, slot_mapping, positions, cos_sin, k_cache, v_cache)
    if k_cache.dim() != 4 or v_cache.shape != k_cache.shape:
        raise ValueError("caches must be [num_blocks, num_kv_heads, block_size, head_dim]")
    NB, Hkv, bs, D = k_cache.shape
    T = k.shape[0]
    for name, t in (("k", k), ("v", v)):
        if t.dim() != 3 or tuple(t.shape[1:]) != (Hkv, D) or t.stride(2) != 1 or t.stride(1) != D:
            raise ValueError(f"{name} must be [T, {Hkv}, {D}] with contiguous heads")
        if t.dtype != k_cache.dtype:
            raise TypeError(f"{name} must have the pools' dtype")
    if slot_mapping.dtype != torch.int64 or slot_mapping.shape != (T,):
        raise ValueError("slot_mapping must be int64 [T]")
    if positions.dtype != torch.int32 or positions.shape != (T,):
        raise ValueError("positions must be int32 [T]")
    if cos_sin.dtype != torch.float32 or cos_sin.dim() != 2:
        raise ValueError("cos_sin must be float32 [max_position, rotary_dim]")
    cos_sin = cos_sin.contiguous()
    _check(load_library().pka_kv_cache_write_rope(
        k.data_ptr(), v.data_ptr(), k.stride(0), v.stride(0), slot_mapping.contiguous().data_ptr(),
        positions.contiguous().data_ptr(), T, cos_sin.data_ptr(), cos_sin.shape[0],
        cos_sin.shape[1], k_cache.data_ptr(), v_cache.data_ptr(), NB, bs, Hkv, D,
        _dtype_code(k_cache.dtype), _stream_ptr(k.device)))


def _block_pools(k_cache, v_cache):
    _require_gpu(k_cache, v_cache)
    if k_cache.shape != v_cache.shape or k_cache.dtype != v_cache.dtype or k_cache.dim() != 4:
        raise ValueError("K and V pools must be matching [num_blocks, Hkv, block_size, D] tensors")
    if not (k_cache.is_contiguous() and v_cache.is_contiguous()):
        raise ValueError("pools must be contiguous")
    nb = k_cache.shape[0]
    return nb, k_cache[0].numel() * k_cache.element_size()


def _ids(t, width):
    import torch

    _require_gpu(t)
    if t.dtype != torch.int64 or (t.dim() != (1 if width == 1 else 2)) or \
            (width == 2 and t.shape[1] != 2):
        raise ValueError("block ids must be int64 [n]" if width == 1 else
                         "block pairs must be int64 [n, 2] (src, dst)")
    return t.contiguous()


def copy_blocks(k_cache, v_cache, block_pairs):
    """Block dst of both pools becomes a copy of block src, for each (src,
    dst) row of block_pairs (device int64 [n, 2]); destinations distinct and
    never also sources."""
    nb, bb = _block_pools(k_cache, v_cache)
    pairs = _ids(block_pairs, 2)
    if pairs.shape[0] == 0:
        return
    _check(load_library().pka_copy_blocks(k_cache.data_ptr(), v_cache.data_ptr(),
                                          pairs.data_ptr(), pairs.shape[0], nb, bb,
                                          _stream_ptr(k_cache.device)))


def gather_blocks(k_cache, v_cache, block_ids, out=None):
    """Blocks block_ids (device int64 [n]) of both pools packed into a device
    uint8 tensor [n, 2, block_bytes] (K, then V)."""
    import torch

    nb, bb = _block_pools(k_cache, v_cache)
    ids = _ids(block_ids, 1)
    n = ids.shape[0]
    if out is None:
        out = torch.empty((n, 2, bb), dtype=torch.uint8, device=k_cache.device)
    elif tuple(out.shape) != (n, 2, bb) or out.dtype != torch.uint8 or not out.is_contiguous():
        raise ValueError(f"out must be a contiguous uint8 [{n}, 2, {bb}] tensor")
    if n:
        _check(load_library().pka_gather_blocks(out.data_ptr(), k_cache.data_ptr(),
                                                v_cache.data_ptr(), ids.data_ptr(), n, nb, bb,
                                                _stream_ptr(k_cache.device)))
    return out


def scatter_blocks(k_cache, v_cache, packed, block_ids):
    """The inverse of gather_blocks: blocks block_ids (distinct) of both pools
    take packed [n, 2, block_bytes] (a device tensor)."""
    import torch

    nb, bb = _block_pools(k_cache, v_cache)
    ids = _ids(block_ids, 1)
    n = ids.shape[0]
    _require_gpu(packed)
    if tuple(packed.shape) != (n, 2, bb) or packed.dtype != torch.uint8:
        raise ValueError(f"packed must be uint8 [{n}, 2, {bb}]")
    packed = packed.contiguous()
    if n:
        _check(load_library().pka_scatter_blocks(k_cache.data_ptr(), v_cache.data_ptr(),
                                                 packed.data_ptr(), ids.data_ptr(), n, nb, bb,
                                                 _stream_ptr(k_cache.device)))


def swap_out(k_cache, v_cache, block_ids, host=None):
    """Copy blocks block_ids of both pools to pinned host memory (one gather
    launch, then one device-to-host copy); returns the host uint8 tensor
    [n, 2, block_bytes].  Asynchronous: synchronise before reading it."""
    import torch

    staging = gather_blocks(k_cache, v_cache, block_ids)
    if host is None:
        host = torch.empty(staging.shape, dtype=torch.uint8, pin_memory=True)
    host.copy_(staging, non_blocking=True)
    return host


def swap_in(k_cache, v_cache, host, block_ids):
    """Copy host rows [n, 2, block_bytes] (from swap_out) into blocks
    block_ids of both pools: one host-to-device copy, then one scatter."""
    staging = host.to(k_cache.device, non_blocking=True)
    scatter_blocks(k_cache, v_cache, staging, block_ids)


_WORKSPACES = {}


def _cached_workspace(device, nbytes: int):
    """A zero-filled workspace per (device, current stream), grown on demand.

    Its leading report counters start at zero and every decode leaves them
    zero, so the buffer is reusable by later calls on the same stream.  Each
    stream gets its own buffer, so decodes issued on different streams never
    share counters or partial results.
    """
    import torch

    key = (str(device), torch.cuda.current_stream(device).cuda_stream)
    ws = _WORKSPACES.get(key)
    if ws is None or ws.numel() < nbytes:
        ws = torch.zeros(max(nbytes, 2 << 20), dtype=torch.uint8, device=device)
        _WORKSPACES[key] = ws
    return ws


class PagedKVCache:
    """A pair of K/V block pools on one device.

    ``write(k, v, slot_mapping)`` is the three-argument cache write;
    ``decode(q, block_tables, context_lens, scale)`` attends over it.
    """

    def __init__(self, num_blocks: int, block_size: int, num_kv_heads: int, head_dim: int,
                 dtype=None, device="cuda"):
        import torch

        dtype = dtype or torch.float16
        shape = (num_blocks, num_kv_heads, block_size, head_dim)
        self.k_cache = torch.empty(shape, dtype=dtype, device=device)
        self.v_cache = torch.empty(shape, dtype=dtype, device=device)
        self.block_size = block_size
        self.num_kv_heads = num_kv_heads

    def write(self, k, v, slot_mapping) -> None:
        kv_cache_write(k, v, slot_mapping, self.k_cache, self.v_cache)

    def decode(self, q, block_tables, context_lens, scale: float, **kw):
        return paged_attention_decode(q, self.k_cache, self.v_cache, block_tables, context_lens,
                                      scale, self.num_kv_heads, self.block_size, **kw)

    def decode_append(self, q, k_new, v_new, slot_mapping, block_tables, context_lens,
                      scale: float, **kw):
        return paged_attention_decode_append(q, k_new, v_new, slot_mapping, self.k_cache,
                                             self.v_cache, block_tables, context_lens, scale,
                                             self.num_kv_heads, self.block_size, **kw)


# ---------------------------------------------------------------------------
# group-quantised INT8 pools
# ---------------------------------------------------------------------------

_INT8_WORKSPACES = {}


def int8_pools(num_blocks: int, num_kv_heads: int, block_size: int, head_dim: int,
               group_size: int, device="cuda"):
    """Empty INT8 pools (k_codes, v_codes, k_scales, v_scales): int8
    [NB, Hkv, bs * D] twice (codes of one block and head in the library's
    operand order, see include/pka.h), float32 [NB, Hkv, bs, D / group_size]
    twice."""
    import torch

    if head_dim % group_size:
        raise ValueError("group_size must divide head_dim")
    ng = head_dim // group_size
    codes = (num_blocks, num_kv_heads, block_size * head_dim)
    scales = (num_blocks, num_kv_heads, block_size, ng)
    return (torch.empty(codes, dtype=torch.int8, device=device),
            torch.empty(codes, dtype=torch.int8, device=device),
            torch.empty(scales, dtype=torch.float32, device=device),
            torch.empty(scales, dtype=torch.float32, device=device))


def _int8_pool_shapes(k_codes, v_codes, k_scales, v_scales):
    import torch

    _require_gpu(k_codes, v_codes, k_scales, v_scales)
    if k_scales.dtype != torch.float32 or k_scales.dim() != 4 or v_scales.shape != k_scales.shape:
        raise ValueError("k_scales / v_scales must be float32 [NB, Hkv, bs, D / group_size]")
    NB, Hkv, bs, ng = k_scales.shape
    if k_codes.dtype != torch.int8 or v_codes.dtype != torch.int8 or k_codes.dim() != 3 or \
            v_codes.shape != k_codes.shape or tuple(k_codes.shape[:2]) != (NB, Hkv) or \
            k_codes.shape[2] % bs:
        raise ValueError("k_codes / v_codes must be int8 [NB, Hkv, bs * D]")
    D = k_codes.shape[2] // bs
    if ng <= 0 or D % ng:
        raise ValueError("the scale arrays' last dim must divide head_dim")
    for t in (k_codes, v_codes, k_scales, v_scales):
        if not t.is_contiguous():
            raise ValueError("INT8 pools must be contiguous")
    return NB, Hkv, bs, D, D // ng


def kv_cache_write_int8(k, v, slot_mapping, k_codes, v_codes, k_scales, v_scales) -> None:
    """Quantise k, v [T, Hkv, D] (float32, float16 or bfloat16) group by
    group and store them at slot_mapping (int64 [T]) in the INT8 pools;
    negative slots are skipped.  Mutates the four arrays."""
    import torch

    NB, Hkv, bs, D, gs = _int8_pool_shapes(k_codes, v_codes, k_scales, v_scales)
    _require_gpu(k, v, slot_mapping, k_codes)
    for name, t in (("k", k), ("v", v)):
        if t.dim() != 3 or tuple(t.shape[1:]) != (Hkv, D):
            raise ValueError(f"{name} must be [T, {Hkv}, {D}], got {tuple(t.shape)}")
        if t.stride(2) != 1 or t.stride(1) != D:
            raise ValueError(f"{name} must have contiguous heads (strides [*, {D}, 1])")
        if t.dtype != k.dtype:
            raise TypeError("k and v must share one dtype")
    if slot_mapping.dtype != torch.int64 or slot_mapping.shape != (k.shape[0],) or \
            v.shape[0] != k.shape[0]:
        raise ValueError("slot_mapping must be int64 [T] with T = k.shape[0] = v.shape[0]")
    slot_mapping = slot_mapping.contiguous()
    T = k.shape[0]
    lib = load_library()
    _check(lib.pka_kv_cache_write_int8(
        k.data_ptr(), v.data_ptr(), k.stride(0) if T else Hkv * D, v.stride(0) if T else Hkv * D,
        _dtype_code(k.dtype), slot_mapping.data_ptr(), T, k_codes.data_ptr(), v_codes.data_ptr(),
        k_scales.data_ptr(), v_scales.data_ptr(), NB, bs, Hkv, D, gs,
        _stream_ptr(k_codes.device)))


def decode_int8_partition_size(num_seqs: int, num_kv_heads: int, block_size: int,
                               max_context_len: int) -> int:
    return int(load_library().pka_decode_int8_partition_size(num_seqs, num_kv_heads, block_size,
                                                             max_context_len))


def decode_int8_workspace_bytes(num_seqs: int, num_q_heads: int, head_dim: int,
                                max_context_len: int, partition_size: int) -> int:
    return int(load_library().pka_decode_int8_workspace_bytes(num_seqs, num_q_heads, head_dim,
                                                              max_context_len, partition_size))


def paged_attention_decode_append_int8(q, k_new, v_new, slot_mapping, k_codes, v_codes, k_scales,
                                       v_scales, block_tables, context_lens, scale: float,
                                       num_kv_heads: int, block_size: int, *, out=None,
                                       out_dtype=None, partition_size: int = 0,
                                       max_context_len: int = 0, workspace=None,
                                       validate: bool = False):
    """One fused INT8 decode step: quantise and store each sequence's new
    token (k_new[b], v_new[b], [B, Hkv, D] in q's dtype) at slot_mapping[b]
    (int64 [B], the slot of position L_b - 1) and attend over its L_b tokens;
    bit-identical to kv_cache_write_int8 followed by
    paged_attention_decode_int8.  Mutates the pools; returns out."""
    import torch

    _, Hkv, _, D, _ = _int8_pool_shapes(k_codes, v_codes, k_scales, v_scales)
    _require_gpu(k_new, v_new, slot_mapping)
    B = q.shape[0]
    for name, t in (("k_new", k_new), ("v_new", v_new)):
        if t.dim() != 3 or tuple(t.shape) != (B, Hkv, D):
            raise ValueError(f"{name} must be [{B}, {Hkv}, {D}], got {tuple(t.shape)}")
        if t.stride(2) != 1 or t.stride(1) != D:
            raise ValueError(f"{name} must have contiguous heads (strides [*, {D}, 1])")
        if t.dtype != q.dtype:
            raise TypeError(f"{name} must have q's dtype")
    if slot_mapping.dtype != torch.int64 or slot_mapping.shape != (B,):
        raise ValueError("slot_mapping must be int64 [B]")
    return paged_attention_decode_int8(
        q, k_codes, v_codes, k_scales, v_scales, block_tables, context_lens, scale, num_kv_heads,
        block_size, out=out, out_dtype=out_dtype, partition_size=partition_size,
        max_context_len=max_context_len, workspace=workspace, validate=validate,
        _append=(k_new, v_new, slot_mapping.contiguous()))


def paged_attention_decode_int8(q, k_codes, v_codes, k_scales, v_scales, block_tables,
                                context_lens, scale: float, num_kv_heads: int, block_size: int,
                                *, out=None, out_dtype=None, partition_size: int = 0,
                                max_context_len: int = 0, workspace=None, validate: bool = False,
                                _append=None):
    """out[b, hq] = softmax(scale * q[b, hq] . K^T) V over sequence b's cache,
    K and V being code * scale of the INT8 pools.  q [B, Hq, D] float16 or
    bfloat16; returns out [B, Hq, D] (float32 unless ``out_dtype`` or ``out``
    says q's dtype).  Other arguments, ``validate`` included, as for
    paged_attention_decode (lengths beyond ``max_context_len`` are cut short
    by this kernel, so there validation catches an undersized hint); the
    workspace needs no initialisation."""
    import torch

    NB, Hkv, bs, D, gs = _int8_pool_shapes(k_codes, v_codes, k_scales, v_scales)
    _require_gpu(q, block_tables, context_lens, k_codes)
    if Hkv != num_kv_heads or bs != block_size:
        raise ValueError(f"pool shape does not match num_kv_heads={num_kv_heads}, "
                         f"block_size={block_size}")
    if q.dim() != 3 or q.shape[2] != D:
        raise ValueError(f"q must be [B, Hq, {D}]")
    q = q.contiguous()
    B, Hq, _ = q.shape
    if block_tables.dtype != torch.int32 or block_tables.dim() != 2 or block_tables.shape[0] != B:
        raise ValueError("block_tables must be int32 [B, max_blocks_per_seq]")
    if context_lens.dtype != torch.int32 or context_lens.shape != (B,):
        raise ValueError("context_lens must be int32 [B]")
    block_tables = block_tables.contiguous()
    context_lens = context_lens.contiguous()
    MB = block_tables.shape[1]
    if out is None:
        out = torch.empty((B, Hq, D), dtype=torch.float32 if out_dtype is None else out_dtype,
                          device=q.device)
    elif tuple(out.shape) != (B, Hq, D) or not out.is_contiguous() or out.device != q.device:
        raise ValueError("out must be a contiguous [B, Hq, D] tensor on q's device")
    if B == 0:
        return out
    if validate:
        _validate_tables(block_tables, context_lens, NB, bs, max_context_len)
        if _append is not None:
            _validate_slots(_append[2], NB * bs, block_tables, context_lens, bs)
    hint = max_context_len if max_context_len > 0 else MB * bs
    hint = min(hint, MB * bs)
    P = partition_size if partition_size > 0 else decode_int8_partition_size(B, Hkv, bs, hint)
    need = decode_int8_workspace_bytes(B, Hq, D, hint, P)
    ws_ptr, ws_bytes = None, 0
    if need > 0:
        if workspace is None:
            # one per (device, current stream): calls on different streams
            # never share partial rows
            key = (str(q.device), torch.cuda.current_stream(q.device).cuda_stream)
            workspace = _INT8_WORKSPACES.get(key)
            if workspace is None or workspace.numel() < need:
                workspace = torch.empty(max(need, 1 << 20), dtype=torch.uint8, device=q.device)
                _INT8_WORKSPACES[key] = workspace
        elif workspace.numel() * workspace.element_size() < need:
            raise ValueError(f"workspace holds {workspace.numel() * workspace.element_size()} "
                             f"bytes, {need} needed")
        ws_ptr, ws_bytes = workspace.data_ptr(), workspace.numel() * workspace.element_size()
    lib = load_library()
    if _append is not None:
        kn, vn, sm = _append
        _check(lib.pka_paged_attention_decode_append_int8(
            out.data_ptr(), _dtype_code(out.dtype), q.data_ptr(), _dtype_code(q.dtype),
            kn.data_ptr(), vn.data_ptr(), kn.stride(0), vn.stride(0), sm.data_ptr(),
            k_codes.data_ptr(), v_codes.data_ptr(), k_scales.data_ptr(), v_scales.data_ptr(),
            block_tables.data_ptr(), MB, context_lens.data_ptr(), B, Hq, Hkv, D, NB, bs, gs,
            float(scale), hint, P, ws_ptr, ws_bytes, _stream_ptr(q.device)))
        return out
    _check(lib.pka_paged_attention_decode_int8(
        out.data_ptr(), _dtype_code(out.dtype), q.data_ptr(), _dtype_code(q.dtype),
        k_codes.data_ptr(), v_codes.data_ptr(), k_scales.data_ptr(), v_scales.data_ptr(),
        block_tables.data_ptr(), MB, context_lens.data_ptr(), B, Hq, Hkv, D, NB, bs, gs,
        float(scale), hint, P, ws_ptr, ws_bytes, _stream_ptr(q.device)))
    return out
