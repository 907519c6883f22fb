"""GPU: the KV-cache write with the rotary embedding on the new keys,
bit-exact against the oracle (both round the fp32 rotation to nearest even
in the pool dtype), and its use by the attention kernels."""
import numpy as np
import pytest

import oracle
from gpu_util import check_close
from paged_kv_attention_24_amd import workloads as W

pytestmark = pytest.mark.gpu


def rope_table(max_pos, R, base=500000.0):
    theta = base ** (-np.arange(0, R, 2, dtype=np.float64) / R)
    ang = np.arange(max_pos)[:, None] * theta[None, :]
    return np.concatenate([np.cos(ang), np.sin(ang)], 1).astype(np.float32)


def run_rope(seed, dtype, T, Hkv, D, bs, R, NB=64, max_pos=8192, bad=()):
    import torch

    import paged_kv_attention_24_amd as pka

    rng = np.random.default_rng(seed)
    k = W._round_to_dtype(rng.standard_normal((T, Hkv, D)).astype(np.float32), dtype)
    v = W._round_to_dtype(rng.standard_normal((T, Hkv, D)).astype(np.float32), dtype)
    slots = rng.permutation(NB * bs)[:T].astype(np.int64)
    pos = rng.integers(0, max_pos, T).astype(np.int32)
    for i, p in bad:
        pos[i] = p
    table = rope_table(max_pos, R)
    kc = W._round_to_dtype(rng.standard_normal((NB, Hkv, bs, D)).astype(np.float32), dtype)
    vc = W._round_to_dtype(rng.standard_normal((NB, Hkv, bs, D)).astype(np.float32), dtype)
    kd, vd = W.as_torch(kc, dtype, "cuda"), W.as_torch(vc, dtype, "cuda")
    pka.kv_cache_write_rope(W.as_torch(k, dtype, "cuda"), W.as_torch(v, dtype, "cuda"),
                            torch.from_numpy(slots).cuda(), torch.from_numpy(pos).cuda(),
                            torch.from_numpy(table).cuda(), kd, vd)
    torch.cuda.synchronize()
    oracle.kv_cache_write_rope(k, v, slots, pos, table, kc, vc, dtype)
    return W.to_numpy_bits(kd, dtype), W.to_numpy_bits(vd, dtype), kc, vc


@pytest.mark.parametrize("dtype,D,bs,R", [("f16", 64, 16, 64), ("bf16", 128, 32, 128),
                                          ("bf16", 64, 16, 32), ("f32", 64, 16, 64),
                                          ("f32", 128, 16, 48), ("f16", 128, 16, 16)])
def test_rope_write_bit_exact(dtype, D, bs, R):
    print(f"[rope] {dtype} D={D} bs={bs} R={R}", flush=True)
    gk, gv, ok, ov = run_rope(60 + D + R, dtype, 300, 4, D, bs, R, NB=128)
    assert gk.tobytes() == ok.tobytes()
    assert gv.tobytes() == ov.tobytes()


def test_rope_positions_outside_the_table_are_skipped():
    gk, gv, ok, ov = run_rope(70, "bf16", 40, 8, 64, 16, 64, bad=[(0, -1), (5, 8192), (9, 1 << 30)])
    assert gk.tobytes() == ok.tobytes() and gv.tobytes() == ov.tobytes()


def test_rotated_keys_give_the_rotated_attention():
    """Attention over keys written with the rotation equals the oracle on
    keys rotated by the oracle: the write composes with the decode."""
    import torch

    import paged_kv_attention_24_amd as pka

    wl = W.make_case(71, dtype="f16", context_lens=[30, 200, 7], num_q_heads=8, num_kv_heads=2,
                     head_dim=64, block_size=16)
    table = rope_table(4096, 64)
    pos = (wl.context_lens - 1).astype(np.int32)
    d = W.device_inputs(wl, "cuda")
    pka.kv_cache_write_rope(d["new_k"], d["new_v"], d["slot_mapping"],
                            torch.from_numpy(pos).cuda(), torch.from_numpy(table).cuda(),
                            d["k_cache"], d["v_cache"])
    out = pka.paged_attention_decode(d["q"], d["k_cache"], d["v_cache"], d["block_tables"],
                                     d["context_lens"], float(wl.scale), 2, 16)
    torch.cuda.synchronize()
    kc, vc = wl.k_cache.copy(), wl.v_cache.copy()
    oracle.kv_cache_write_rope(wl.new_k, wl.new_v, wl.slot_mapping, pos, table, kc, vc, "f16")
    ref = oracle.paged_attention_decode(wl.q, kc, vc, wl.block_tables, wl.context_lens,
                                        wl.scale, 2, 16, "f16")
    check_close(out.double().cpu().numpy(), ref, "f16")
