"""GPU: the multi-token attention, the RoPE write, the block moves and the INT8 write and decode
captured in a HIP graph and replayed several times, with eager calls in
between, give the eager results bit for bit."""
import numpy as np
import pytest

from paged_kv_attention_24_amd import workloads as W

pytestmark = pytest.mark.gpu


def replay_matches(call, outputs, reset=None, rounds=3):
    """Run call eagerly, then capture it and replay it `rounds` times (each
    replay after an eager call), comparing every output tensor."""
    import torch

    if reset:
        reset()
    call()
    torch.cuda.synchronize()
    ref = [o.clone() for o in outputs]
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        if reset:
            reset()
        call()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call()
    for _ in range(rounds):
        for o in outputs:
            o.fill_(0)
        if reset:
            reset()
        g.replay()
        torch.cuda.synchronize()
        for o, r in zip(outputs, ref):
            assert torch.equal(o, r)
        if reset:
            reset()
        call()
        torch.cuda.synchronize()
        for o, r in zip(outputs, ref):
            assert torch.equal(o, r)


def test_prefill_graph_replay():
    import torch

    import paged_kv_attention_24_amd as pka

    wl = W.make_prefill_case(80, dtype="bf16", prefix_lens=(100, 0, 37), query_lens=(40, 9, 64),
                             num_q_heads=16, num_kv_heads=4, head_dim=64, block_size=16)
    q = W.as_torch(wl.q, "bf16", "cuda")
    kc, vc = W.as_torch(wl.k_cache, "bf16", "cuda"), W.as_torch(wl.v_cache, "bf16", "cuda")
    bt = torch.from_numpy(wl.block_tables).cuda()
    cl = torch.from_numpy(wl.context_lens).cuda()
    qs = torch.from_numpy(wl.query_start).cuda()
    out = torch.empty((wl.num_query_tokens, 16, 64), device="cuda")
    replay_matches(lambda: pka.paged_attention_prefill(q, kc, vc, bt, cl, qs, float(wl.scale), 4,
                                                       16, out=out, max_query_len=64), [out])


def test_rope_write_graph_replay():
    import torch

    import paged_kv_attention_24_amd as pka

    rng = np.random.default_rng(81)
    T, H, D, NB, bs = 200, 8, 64, 64, 16
    k = torch.randn(T, H, D, device="cuda").half()
    v = torch.randn(T, H, D, device="cuda").half()
    slots = torch.from_numpy(rng.permutation(NB * bs)[:T].astype(np.int64)).cuda()
    pos = torch.from_numpy(rng.integers(0, 4096, T).astype(np.int32)).cuda()
    ang = np.arange(4096)[:, None] * (10000.0 ** (-np.arange(0, D, 2) / D))[None, :]
    table = torch.from_numpy(np.concatenate([np.cos(ang), np.sin(ang)], 1).astype(np.float32)).cuda()
    kc = torch.zeros(NB, H, bs, D, device="cuda").half()
    vc = torch.zeros_like(kc)
    replay_matches(lambda: pka.kv_cache_write_rope(k, v, slots, pos, table, kc, vc), [kc, vc])


def test_block_moves_graph_replay():
    import torch

    import paged_kv_attention_24_amd as pka

    NB = 256
    k0 = torch.randn(NB, 8, 16, 64, device="cuda").half()
    v0 = torch.randn(NB, 8, 16, 64, device="cuda").half()
    kc, vc = k0.clone(), v0.clone()
    perm = torch.randperm(NB, device="cuda")
    pairs = torch.stack([perm[:64], perm[64:128]], 1).to(torch.int64)
    ids = perm[128:160].to(torch.int64)
    packed = torch.empty((32, 2, 8 * 16 * 64 * 2), dtype=torch.uint8, device="cuda")

    def reset():
        kc.copy_(k0)
        vc.copy_(v0)

    def call():
        pka.copy_blocks(kc, vc, pairs)
        pka.gather_blocks(kc, vc, ids, out=packed)
        pka.scatter_blocks(kc, vc, packed, perm[160:192].to(torch.int64))

    replay_matches(call, [kc, vc, packed], reset=reset)


@pytest.mark.parametrize("P", [0, 32, 16])
def test_int8_write_and_decode_graph_replay(P):
    """The INT8 quantising write followed by the INT8 decode, captured
    together: one partition (a single launch), one wave per unit plus the
    merge launch (32-token partitions), and the persistent grid that plans
    in LDS (16-token partitions)."""
    import torch

    import paged_kv_attention_24_amd as pka

    # no NaN poison here: the replayed pools are compared with torch.equal
    wl = W.make_int8_case(82, q_dtype="f16", context_lens=(5, 37, 200, 1, 64), num_q_heads=8,
                          num_kv_heads=2, head_dim=64, block_size=16, group_size=32,
                          poison=False)
    d = W.int8_device_inputs(wl)
    pools = [d["k_codes"], d["v_codes"], d["k_scales"], d["v_scales"]]
    start = [t.clone() for t in pools]
    out = torch.empty((wl.num_seqs, 8, 64), device="cuda")

    def reset():
        for t, s0 in zip(pools, start):
            t.copy_(s0)

    def call():
        pka.kv_cache_write_int8(d["new_k"], d["new_v"], d["slot_mapping"], *pools)
        pka.paged_attention_decode_int8(d["q"], *pools, d["block_tables"], d["context_lens"],
                                        float(wl.scale), 2, 16, out=out, partition_size=P,
                                        max_context_len=wl.max_context_len)

    replay_matches(call, [out] + pools, reset=reset)
