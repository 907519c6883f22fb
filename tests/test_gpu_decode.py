"""GPU: paged decode attention against the fp64 oracle.

Tolerance (max-abs on the fp32 output): 1e-5 with fp32 KV, 2e-3 with
fp16/bf16 KV.  Every workload NaN-poisons the pool memory a correct kernel
must not read (unused blocks, the tail of each last block, and the slot the
write fills), so an over-read shows up as a non-finite output.
"""
import os

import numpy as np
import pytest

import oracle
from gpu_util import TOL, check_close, gpu_decode, oracle_full, sample_rows
from paged_kv_attention_24_amd import workloads as W

pytestmark = pytest.mark.gpu


def case(seed, dtype, lens, Hq, Hkv, D, bs, **kw):
    return W.make_case(seed, dtype=dtype, context_lens=lens, num_q_heads=Hq,
                       num_kv_heads=Hkv, head_dim=D, block_size=bs, **kw)


# ---------------------------------------------------------------------------
# the named workloads
# ---------------------------------------------------------------------------

def test_tiny_workload_full():
    wl = W.make_config(1)
    print("[decode] cfg1 tiny", flush=True)
    got = gpu_decode(wl)
    check_close(got, oracle_full(wl), "f32", "cfg1")
    golden = np.loadtxt(os.path.join(os.path.dirname(__file__), "golden",
                                     "tiny_decode_oracle.txt"), comments="#").reshape(2, 4, 64)
    assert np.max(np.abs(got - golden)) <= 1e-5


@pytest.mark.parametrize("cfg", [2, 3])
def test_named_workload_full(cfg):
    wl = W.make_config(cfg)
    print(f"[decode] cfg{cfg} full", flush=True)
    got = gpu_decode(wl)
    err = check_close(got, oracle_full(wl), wl.dtype, f"cfg{cfg}")
    print(f"[decode] cfg{cfg} max-abs err {err:.3g}", flush=True)


@pytest.mark.slow
@pytest.mark.parametrize("cfg", [4, 5])
def test_named_workload_sampled(cfg):
    """Full-size workloads in the benchmark's launch configuration; the
    oracle computes a sample of rows (all query heads of the longest
    sequence included), the rest is checked for finiteness."""
    wl = W.make_config(cfg)
    print(f"[decode] cfg{cfg} full size, sampled rows", flush=True)
    got = gpu_decode(wl)
    assert np.all(np.isfinite(got))
    longest = int(np.argmax(wl.context_lens))
    must = [(longest, h) for h in range(wl.num_q_heads)]
    rows = sample_rows(wl, 96, seed=cfg, must=must)
    ref = oracle.decode_workload(wl, rows=rows)
    err = check_close(got[rows[:, 0], rows[:, 1]], ref, wl.dtype, f"cfg{cfg}")
    print(f"[decode] cfg{cfg} sampled max-abs err {err:.3g}", flush=True)


# ---------------------------------------------------------------------------
# shape / dtype / length sweep (full comparison, several tiles, ragged tails)
# ---------------------------------------------------------------------------

SWEEP = []
for dtype in ("f32", "f16", "bf16"):
    for D in (64, 128):
        for bs in (16, 32):
            for G in (1, 2, 4, 8):
                SWEEP.append((dtype, D, bs, G))


@pytest.mark.parametrize("dtype,D,bs,G", SWEEP)
def test_sweep(dtype, D, bs, G):
    Hkv = 2 if G == 8 else 3
    lens = [1, bs - 1, bs, bs + 1, 63, 64, 65, 127, 129, 300, 513, 1100]
    wl = case(1000 + D + bs + G, dtype, lens, Hkv * G, Hkv, D, bs)
    ref = oracle_full(wl)
    print(f"[decode] sweep {dtype} D={D} bs={bs} G={G}", flush=True)
    for P in (0, bs, 64 if bs <= 64 else bs, 256, 1024):
        got = gpu_decode(wl, partition_size=P)
        check_close(got, ref, dtype, f"{dtype} D{D} bs{bs} G{G} P{P}")


# pair mode (the library's choice on small batches: one workgroup per
# (sequence, kv head) pair whose waves share its chunks) over batch shapes
# around the compute-unit count, with waves left without a chunk
PAIR_SHAPES = [
    # dtype, D, B, Hkv, lengths (cycled over the batch)
    ("f16", 64, 20, 8, [1024, 100, 517, 33]),        # 160 pairs
    ("bf16", 64, 16, 8, [1024, 700, 129, 1]),        # 128 pairs
    ("f16", 128, 10, 8, [1024, 31, 640, 257]),       # 80 pairs
    ("bf16", 128, 4, 2, [1, 33, 300, 2000]),         # 8 pairs, up to 2000 tokens
    ("f16", 64, 4, 2, [100, 7, 64, 65]),             # short
]


@pytest.mark.parametrize("dtype,D,B,Hkv,lens", PAIR_SHAPES)
def test_pair_mode_shapes(dtype, D, B, Hkv, lens):
    lens = [lens[i % len(lens)] for i in range(B)]
    wl = case(4000 + B + D, dtype, lens, 4 * Hkv, Hkv, D, 16)
    print(f"[decode] pair mode {dtype} D={D} B={B} Hkv={Hkv}", flush=True)
    a = gpu_decode(wl, partition_size=0)
    check_close(a, oracle_full(wl), dtype, "pair mode")
    assert np.array_equal(a, gpu_decode(wl, partition_size=0))


# ---------------------------------------------------------------------------
# edge cases and invariants on the GPU
# ---------------------------------------------------------------------------

def test_single_token_returns_v_exactly():
    wl = case(5, "bf16", [1, 1, 1, 1], 8, 2, 64, 16, write=False)
    got = gpu_decode(wl, partition_size=16)
    ref = oracle_full(wl)  # exactly V_0 (pinned)
    assert np.array_equal(got, ref)


def test_zero_length_rows_are_zero():
    wl = case(6, "f16", [0, 17, 0, 300], 8, 4, 64, 16, write=False)
    got = gpu_decode(wl)
    assert np.all(got[0] == 0) and np.all(got[2] == 0)
    check_close(got, oracle_full(wl), "f16")


def test_block_relabel_is_bit_exact():
    wl = case(7, "f16", [40, 513, 1000, 7], 32, 8, 64, 16, write=False)
    base = gpu_decode(wl, partition_size=128)
    perm = np.random.default_rng(1).permutation(wl.num_blocks).astype(np.int32)
    k2, v2 = np.empty_like(wl.k_cache), np.empty_like(wl.v_cache)
    k2[perm], v2[perm] = wl.k_cache, wl.v_cache
    wl.k_cache, wl.v_cache = k2, v2
    wl.block_tables = np.where(wl.block_tables >= 0, perm[np.maximum(wl.block_tables, 0)],
                               -1).astype(np.int32)
    again = gpu_decode(wl, partition_size=128)
    assert np.array_equal(base, again)


def test_batch_permutation():
    """Permuting the batch permutes the outputs.  The work is split evenly
    over the waves in batch order, so a sequence's parts (and the fp32
    rounding of their merge) depend on its place in the batch: the outputs
    agree to rounding, and each matches the oracle."""
    wl = case(8, "bf16", [40, 513, 1000, 7, 64], 16, 8, 128, 16, write=False)
    base = gpu_decode(wl, partition_size=256)
    ref = oracle_full(wl)
    p = np.array([4, 2, 0, 3, 1])
    wl.q = np.ascontiguousarray(wl.q[p])
    wl.block_tables = np.ascontiguousarray(wl.block_tables[p])
    wl.context_lens = np.ascontiguousarray(wl.context_lens[p])
    again = gpu_decode(wl, partition_size=256)
    assert np.max(np.abs(again - base[p])) <= 1e-5
    check_close(again, ref[p], "bf16")


def test_run_to_run_determinism():
    wl = W.make_config(3)
    a = gpu_decode(wl)
    b = gpu_decode(wl)
    assert np.array_equal(a, b)


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_half_output(dtype):
    """Output in the KV dtype: the fp32 result rounded to nearest even, so it
    sits within one half-ulp (plus the fp32 tolerance) of the oracle."""
    import torch

    wl = case(9, dtype, [5, 100, 700], 8, 2, 64, 16)
    got = gpu_decode(wl, out_dtype=W.torch_dtype(dtype))
    ref = oracle_full(wl)
    ulp = 2.0 ** (-10 if dtype == "f16" else -7)
    bound = 0.5 * ulp * np.maximum(np.abs(ref), 2.0 ** -14) * 2 + TOL[dtype]
    assert np.all(np.abs(got - ref) <= bound)
    del torch


def test_max_context_hint_smaller_grid():
    """A tight host hint gives the same result as the table-sized default."""
    wl = case(10, "f16", [100, 700, 1500], 32, 8, 64, 16, max_blocks_per_seq=200)
    a = gpu_decode(wl, max_context_len=1500)
    b = gpu_decode(wl, max_context_len=0)
    ref = oracle_full(wl)
    check_close(a, ref, "f16")
    check_close(b, ref, "f16")


def test_long_single_sequence_many_partitions():
    wl = case(11, "f16", [32768], 32, 8, 64, 32)
    got = gpu_decode(wl, partition_size=512)
    rows = np.array([[0, h] for h in range(32)], dtype=np.int32)
    ref = oracle.decode_workload(wl, rows=rows)
    check_close(got[0], ref, "f16", "32k")


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_skewed_work_list(dtype):
    """One long sequence among short and empty ones, with the smallest
    shares: the long one is split over many waves."""
    lens = [0, 5000, 1, 33, 0, 700, 16, 17] + [100] * 40
    wl = case(13, dtype, lens, 16, 4, 64, 16)
    got = gpu_decode(wl, partition_size=64)  # 79 partitions for the longest
    check_close(got, oracle_full(wl), dtype, "work list")
    assert np.all(got[0] == 0) and np.all(got[4] == 0)


def test_workspace_reuse_across_shapes():
    """One explicit workspace, zero-filled once, serves calls of different
    shapes back to back (its report counters stay at a fixed place and
    every call leaves them zero)."""
    import torch

    import paged_kv_attention_24_amd as pka

    ws = torch.zeros(64 << 20, dtype=torch.uint8, device="cuda")
    cases = [case(20, "f16", [900, 33, 2000], 32, 8, 64, 16),
             case(21, "bf16", [5000, 100], 16, 8, 128, 16),
             case(22, "f16", [300] * 20, 8, 2, 64, 32)]
    for rnd in range(2):
        for i, wl in enumerate(cases):
            d = W.device_inputs(wl, "cuda")
            pka.kv_cache_write(d["new_k"], d["new_v"], d["slot_mapping"], d["k_cache"],
                               d["v_cache"])
            out = pka.paged_attention_decode(d["q"], d["k_cache"], d["v_cache"],
                                             d["block_tables"], d["context_lens"],
                                             float(wl.scale), wl.num_kv_heads, wl.block_size,
                                             partition_size=64 if i != 1 else 256,
                                             workspace=ws)
            torch.cuda.synchronize()
            check_close(out.double().cpu().numpy(), oracle_full(wl), wl.dtype,
                        f"round {rnd} case {i}")
    assert int(ws[: 4 << 20].count_nonzero()) == 0  # report counters left at zero


def test_graph_replay_matches_eager():
    """Captured in a HIP graph, the multi-partition decode replays several
    times (eager calls in between) and matches the eager result bit for bit."""
    import torch

    import paged_kv_attention_24_amd as pka

    wl = case(23, "bf16", [3000, 40, 1500, 777], 32, 8, 64, 16)
    d = W.device_inputs(wl, "cuda")
    pka.kv_cache_write(d["new_k"], d["new_v"], d["slot_mapping"], d["k_cache"], d["v_cache"])
    ws = torch.zeros(16 << 20, dtype=torch.uint8, device="cuda")
    out = torch.empty((wl.num_seqs, wl.num_q_heads, wl.head_dim), device="cuda")

    def call(o):
        pka.paged_attention_decode(d["q"], d["k_cache"], d["v_cache"], d["block_tables"],
                                   d["context_lens"], float(wl.scale), wl.num_kv_heads,
                                   wl.block_size, partition_size=128, out=o, workspace=ws,
                                   max_context_len=wl.max_context_len)

    eager = torch.empty_like(out)
    call(eager)
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        call(out)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call(out)
    ref = eager.clone()
    for _ in range(3):
        out.zero_()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref)
        call(eager)
        torch.cuda.synchronize()
        assert torch.equal(eager, ref)
    check_close(ref.double().cpu().numpy(), oracle_full(wl), "bf16")


def test_bad_partition_size_is_rejected():
    import paged_kv_attention_24_amd as pka

    wl = case(12, "f16", [50], 8, 2, 64, 16, write=False)
    with pytest.raises(pka.PkaError):
        gpu_decode(wl, partition_size=24)
    with pytest.raises(pka.PkaError):
        gpu_decode(wl, partition_size=-16)
    # any positive multiple of the block size is a valid smallest share
    check_close(gpu_decode(wl, partition_size=4096), oracle_full(wl), "f16")


@pytest.mark.parametrize("scale", [0.0, -1e-40, -0.125, "large"])
@pytest.mark.parametrize("dtype,mode", [("f16", "pair"), ("bf16", "flat"), ("f32", "flat")])
def test_zero_negative_and_large_scales(scale, dtype, mode):
    """scale 0 is the plain mean of V over the tokens (the library hands the
    kernels 1e-30 for it, so that every part of a split pair keeps its
    weight); a negative scale flips every logit; a large one sharpens the
    softmax so that its reference moves often.  Pair mode combines in LDS,
    the flat split (64-token shares) through the workspace.  The large scale
    is 3 for 16-bit KV and 1 for fp32 KV: at 3 the largest logits reach ~140
    in log2 units, where float32 rounding of the logits alone moves the
    weights by ~1e-5, the fp32 bound."""
    if scale == "large":
        scale = 1.0 if dtype == "f32" else 3.0
    lens = [700, 33, 1, 250] if mode == "pair" else [3000, 700, 33, 1, 0, 1600] * 4
    wl = case(60, dtype, lens, 8, 2, 64, 16, scale=scale)
    print(f"[decode] scale {scale} {dtype} {mode}", flush=True)
    got = gpu_decode(wl, partition_size=0 if mode == "pair" else 64)
    check_close(got, oracle_full(wl), dtype, f"scale {scale} {mode}")


@pytest.mark.parametrize("B", [257, 300, 513, 1000])
def test_batches_with_several_lengths_per_thread(B):
    """Batches of 257-1000 sequences: each thread of the in-kernel plan reads
    and scans two to four lengths (the first one kept in a register, the
    rest read again), with empty sequences at those threads' first and
    later slots.  Every output row is compared."""
    rng = np.random.default_rng(B)
    lens = rng.integers(1, 160, size=B)
    lens[::7] = 0
    lens[1::256] = 0
    wl = case(40 + B, "bf16", [int(x) for x in lens], 4, 2, 64, 16)
    print(f"[decode] B={B} several lengths per thread", flush=True)
    got = gpu_decode(wl)
    assert np.all(got[lens == 0] == 0)
    check_close(got, oracle_full(wl), "bf16", f"B={B}")


@pytest.mark.parametrize("dtype,B", [("f16", 2048), ("bf16", 2049), ("f32", 2049)])
def test_large_batch_work_list(dtype, B):
    """Batches past the 2040 sequences one launch plans in its LDS run as
    several launches that share the workspace.  Sequences split over several
    waves, empty sequences mixed in; rows of the longest sequence and of the
    last sequences are always compared."""
    rng = np.random.default_rng(31)
    lens = rng.integers(1, 700, size=B)
    lens[::97] = 0
    lens[B - 1] = 1300
    wl = case(31, dtype, [int(x) for x in lens], 8, 2, 64, 16)
    got = gpu_decode(wl, partition_size=128)
    assert np.all(np.isfinite(got))
    assert np.all(got[lens == 0] == 0)
    must = [(B - 1, h) for h in range(8)] + [(B - 2, h) for h in range(8)] + [(0, 3), (2047, 5)]
    rows = sample_rows(wl, 160, seed=B, must=must)
    ref = oracle.decode_workload(wl, rows=rows)
    check_close(got[rows[:, 0], rows[:, 1]], ref, dtype, f"B={B}")
