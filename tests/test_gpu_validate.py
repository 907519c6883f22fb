"""GPU: the device-data checks behind ``validate=True``.

Each bad input must raise PkaError before any kernel runs (the kernels
themselves clamp such inputs instead of failing); good inputs must pass the
checks and give the same result as an unchecked call.
"""
import numpy as np
import pytest

from paged_kv_attention_24_amd import workloads as W

pytestmark = pytest.mark.gpu


def _decode_case(seed=3, lens=(5, 37, 100, 1)):
    # no NaN poison: the decodes here run without the write first
    return W.make_case(seed, dtype="f16", context_lens=list(lens), num_q_heads=8,
                       num_kv_heads=2, head_dim=64, block_size=16, name="validate",
                       poison=False)


def _decode(d, wl, **kw):
    import paged_kv_attention_24_amd as pka

    return pka.paged_attention_decode(d["q"], d["k_cache"], d["v_cache"], d["block_tables"],
                                      d["context_lens"], float(wl.scale), wl.num_kv_heads,
                                      wl.block_size, **kw)


def test_decode_good_inputs_pass_and_match():
    import torch

    wl = _decode_case()
    d = W.device_inputs(wl)
    print("[validate] decode, good inputs", flush=True)
    a = _decode(d, wl, validate=True, max_context_len=int(wl.context_lens.max()))
    b = _decode(d, wl)
    torch.cuda.synchronize()
    assert torch.equal(a, b)


@pytest.mark.parametrize("what", ["id_past_pool", "id_negative", "len_past_table", "hint_short"])
def test_decode_bad_inputs_raise(what):
    import torch

    import paged_kv_attention_24_amd as pka

    wl = _decode_case()
    d = W.device_inputs(wl)
    bt = d["block_tables"].clone()
    cl = d["context_lens"].clone()
    hint = 0
    if what == "id_past_pool":
        bt[2, 3] = wl.num_blocks  # entry 3 of a 100-token sequence is used
    elif what == "id_negative":
        bt[1, 2] = -1  # 37 tokens use entries 0..2
    elif what == "len_past_table":
        cl[0] = bt.shape[1] * wl.block_size + 1
    else:
        hint = int(wl.context_lens.max()) - 1
    print(f"[validate] decode, {what}", flush=True)
    with pytest.raises(pka.PkaError) as e:
        pka.paged_attention_decode(d["q"], d["k_cache"], d["v_cache"], bt, cl, float(wl.scale),
                                   wl.num_kv_heads, wl.block_size, max_context_len=hint,
                                   validate=True)
    assert e.value.status == 1
    torch.cuda.synchronize()


def test_decode_unused_entries_are_not_checked():
    import torch

    wl = _decode_case()
    d = W.device_inputs(wl)
    d["block_tables"][3, 1:] = -7  # a 1-token sequence uses entry 0 only
    print("[validate] decode, unused table entries", flush=True)
    _decode(d, wl, validate=True)
    torch.cuda.synchronize()


def _append(d, wl, slots, **kw):
    import paged_kv_attention_24_amd as pka

    return pka.paged_attention_decode_append(
        d["q"], d["new_k"], d["new_v"], slots, d["k_cache"], d["v_cache"], d["block_tables"],
        d["context_lens"], float(wl.scale), wl.num_kv_heads, wl.block_size, **kw)


def test_append_good_and_bad_slots():
    import torch

    import paged_kv_attention_24_amd as pka

    wl = _decode_case(seed=4)
    d = W.device_inputs(wl)
    good = d["slot_mapping"]
    print("[validate] append, good slots", flush=True)
    _append(d, wl, good, validate=True)
    torch.cuda.synchronize()
    # a slot stored twice
    dup = good.clone()
    dup[1] = dup[0]
    print("[validate] append, duplicate slot", flush=True)
    with pytest.raises(pka.PkaError):
        _append(d, wl, dup, validate=True)
    # a slot this call reads for another position (position 0 of sequence 2)
    bt = wl.block_tables
    clash = good.clone()
    clash[0] = int(bt[2, 0]) * wl.block_size
    print("[validate] append, slot read elsewhere", flush=True)
    with pytest.raises(pka.PkaError):
        _append(d, wl, clash, validate=True)
    # skipped slots (negative) are not stores: no error
    skip = good.clone()
    skip[0] = -1
    skip[1] = -1
    _append(d, wl, skip, validate=True)
    torch.cuda.synchronize()


def test_write_duplicate_slots_raise():
    import torch

    import paged_kv_attention_24_amd as pka

    wl = _decode_case(seed=5)
    d = W.device_inputs(wl)
    slots = d["slot_mapping"].clone()
    print("[validate] write, good then duplicate slots", flush=True)
    pka.kv_cache_write(d["new_k"], d["new_v"], slots, d["k_cache"], d["v_cache"], validate=True)
    slots[2] = slots[3]
    with pytest.raises(pka.PkaError):
        pka.kv_cache_write(d["new_k"], d["new_v"], slots, d["k_cache"], d["v_cache"],
                           validate=True)
    torch.cuda.synchronize()


@pytest.mark.parametrize("what", ["good", "start_not_zero", "decreasing", "more_new_than_cached",
                                  "max_query_len_short", "id_past_pool"])
def test_prefill_checks(what):
    import torch

    import paged_kv_attention_24_amd as pka

    wl = W.make_prefill_case(6, dtype="bf16", prefix_lens=[10, 0, 40], query_lens=[3, 5, 2],
                             num_q_heads=4, num_kv_heads=2, head_dim=64, block_size=16,
                             poison=False)
    dev = "cuda"
    q = W.as_torch(wl.q, wl.dtype, dev)
    kc = W.as_torch(wl.k_cache, wl.dtype, dev)
    vc = W.as_torch(wl.v_cache, wl.dtype, dev)
    bt = torch.from_numpy(wl.block_tables).to(dev)
    cl = torch.from_numpy(wl.context_lens).to(dev)
    qs = torch.from_numpy(wl.query_start).to(dev)
    mql = 0
    if what == "start_not_zero":
        qs = qs.clone()
        qs[0] = 1
    elif what == "decreasing":
        qs = qs.clone()
        qs[2] = int(qs[1]) - 1
    elif what == "more_new_than_cached":
        cl = cl.clone()
        cl[1] = 4  # 5 new tokens
    elif what == "max_query_len_short":
        mql = 4
    elif what == "id_past_pool":
        bt = bt.clone()
        bt[2, 0] = wl.num_blocks
    print(f"[validate] prefill, {what}", flush=True)
    call = lambda: pka.paged_attention_prefill(q, kc, vc, bt, cl, qs, float(wl.scale),
                                               wl.num_kv_heads, wl.block_size,
                                               max_query_len=mql, validate=True)
    if what == "good":
        a = call()
        b = pka.paged_attention_prefill(q, kc, vc, bt, cl, qs, float(wl.scale), wl.num_kv_heads,
                                        wl.block_size)
        torch.cuda.synchronize()
        assert torch.equal(a, b)
    else:
        with pytest.raises(pka.PkaError):
            call()
    torch.cuda.synchronize()


def test_int8_decode_undersized_hint_raises():
    import torch

    import paged_kv_attention_24_amd as pka

    wl = W.make_int8_case(7, q_dtype="f16", context_lens=[40, 300, 7], num_q_heads=8,
                          num_kv_heads=2, head_dim=64, block_size=16, group_size=32, write=True)
    d = W.int8_device_inputs(wl)
    args = (d["q"], d["k_codes"], d["v_codes"], d["k_scales"], d["v_scales"], d["block_tables"],
            d["context_lens"], float(wl.scale), wl.num_kv_heads, wl.block_size)
    print("[validate] int8 decode, hint", flush=True)
    pka.paged_attention_decode_int8(*args, max_context_len=300, validate=True)
    with pytest.raises(pka.PkaError):
        pka.paged_attention_decode_int8(*args, max_context_len=299, validate=True)
    # the fused step checks its slots too
    dup = d["slot_mapping"].clone()
    dup[0] = dup[1]
    with pytest.raises(pka.PkaError):
        pka.paged_attention_decode_append_int8(
            d["q"], d["new_k"], d["new_v"], dup, d["k_codes"], d["v_codes"], d["k_scales"],
            d["v_scales"], d["block_tables"], d["context_lens"], float(wl.scale),
            wl.num_kv_heads, wl.block_size, validate=True)
    torch.cuda.synchronize()
    assert np.isfinite(wl.scale)
