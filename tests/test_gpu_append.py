"""GPU: the fused decode step (store each sequence's new token + decode over
it, one launch) against the oracle: output within tolerance of the appended
decode, pools bit-exact against the oracle's write, and bit-identical to the
two-launch path (write, then decode) when the slot is position L-1's."""
import numpy as np
import pytest

import oracle
from gpu_util import check_close
from paged_kv_attention_24_amd import workloads as W

pytestmark = pytest.mark.gpu


def case(seed, dtype, lens, Hq, Hkv, D, bs, **kw):
    return W.make_case(seed, dtype=dtype, context_lens=lens, num_q_heads=Hq,
                       num_kv_heads=Hkv, head_dim=D, block_size=bs, **kw)


def fused(wl, partition_size=0, slot_mapping=None, stride_pad=0):
    import torch

    import paged_kv_attention_24_amd as pka

    d = W.device_inputs(wl, "cuda")
    k_new, v_new = d["new_k"], d["new_v"]
    if stride_pad:
        B, H, D = k_new.shape
        wide = torch.zeros((B, H + stride_pad, D), dtype=k_new.dtype, device="cuda")
        wide[:, :H] = k_new
        k_new = wide[:, :H]
    slots = d["slot_mapping"] if slot_mapping is None else torch.from_numpy(slot_mapping).cuda()
    out = pka.paged_attention_decode_append(
        d["q"], k_new, v_new, slots, d["k_cache"], d["v_cache"], d["block_tables"],
        d["context_lens"], float(wl.scale), wl.num_kv_heads, wl.block_size,
        partition_size=partition_size, max_context_len=wl.max_context_len)
    torch.cuda.synchronize()
    return (out.double().cpu().numpy(), W.to_numpy_bits(d["k_cache"], wl.dtype),
            W.to_numpy_bits(d["v_cache"], wl.dtype))


def two_launch(wl, partition_size=0):
    from gpu_util import gpu_decode

    return gpu_decode(wl, partition_size=partition_size)


def oracle_append(wl, rows=None):
    return oracle.paged_attention_decode_append(
        wl.q, wl.k_cache, wl.v_cache, wl.new_k, wl.new_v, wl.block_tables, wl.context_lens,
        wl.scale, wl.num_kv_heads, wl.block_size, wl.dtype, rows=rows)


def oracle_pools(wl, slots=None):
    kc, vc = wl.k_cache.copy(), wl.v_cache.copy()
    s = wl.slot_mapping if slots is None else slots
    keep = np.array([wl.context_lens[b] > 0 for b in range(wl.num_seqs)])
    s = np.where(keep, s, -1)
    oracle.kv_cache_write(wl.new_k, wl.new_v, s, kc, vc, wl.dtype)
    return kc, vc


@pytest.mark.parametrize("cfg", [1, 2, 3])
def test_named_workload(cfg):
    wl = W.make_config(cfg)
    print(f"[append] cfg{cfg}", flush=True)
    out, kc, vc = fused(wl)
    check_close(out, oracle_append(wl), wl.dtype, f"cfg{cfg}")
    ek, ev = oracle_pools(wl)
    assert kc.tobytes() == ek.tobytes() and vc.tobytes() == ev.tobytes()
    assert np.array_equal(out, two_launch(wl))


@pytest.mark.slow
def test_skewed_workload_sampled():
    wl = W.make_config(5)
    print("[append] cfg5", flush=True)
    out, kc, vc = fused(wl)
    rows = np.array([[0, h] for h in range(wl.num_q_heads)] +
                    [[b, (7 * b) % wl.num_q_heads] for b in range(1, wl.num_seqs, 9)],
                    dtype=np.int32)
    check_close(out[rows[:, 0], rows[:, 1]], oracle_append(wl, rows=rows), wl.dtype, "cfg5")
    ek, ev = oracle_pools(wl)
    assert kc.tobytes() == ek.tobytes() and vc.tobytes() == ev.tobytes()


SWEEP = [(dt, D, bs, G) for dt in ("f32", "f16", "bf16") for D in (64, 128) for bs in (16, 32)
         for G in (1, 4)]


@pytest.mark.parametrize("dtype,D,bs,G", SWEEP)
def test_sweep(dtype, D, bs, G):
    """Last positions at chunk, block and partition boundaries and just past
    them, several partition sizes (dense grid and device work list)."""
    Hkv = 2
    lens = [1, 2, bs, bs + 1, 32, 33, 64, 65, 96, 128, 129, 513, 1024, 1025]
    wl = case(3000 + D + bs + G, dtype, lens, Hkv * G, Hkv, D, bs)
    ref = oracle_append(wl)
    ek, ev = oracle_pools(wl)
    print(f"[append] sweep {dtype} D={D} bs={bs} G={G}", flush=True)
    for P in (0, bs, 128, 1024):
        out, kc, vc = fused(wl, partition_size=P)
        check_close(out, ref, dtype, f"P={P}")
        assert kc.tobytes() == ek.tobytes() and vc.tobytes() == ev.tobytes()


def test_negative_and_empty():
    """A negative slot stores nothing but the new token still takes part;
    an empty sequence stores nothing and yields zeros."""
    wl = case(31, "f16", [40, 0, 77, 1, 300], 8, 2, 64, 16)
    slots = wl.slot_mapping.copy()
    slots[0] = -1
    slots[1] = 5  # L = 0: must not be written
    out, kc, vc = fused(wl, slot_mapping=slots)
    check_close(out, oracle_append(wl), "f16")
    assert np.all(out[1] == 0)
    ek, ev = oracle_pools(wl, slots)
    assert kc.tobytes() == ek.tobytes() and vc.tobytes() == ev.tobytes()


def test_strided_new_rows():
    wl = case(32, "bf16", [17, 300, 64], 16, 4, 128, 16)
    out, kc, vc = fused(wl, stride_pad=3)
    check_close(out, oracle_append(wl), "bf16")
    ek, ev = oracle_pools(wl)
    assert kc.tobytes() == ek.tobytes()
