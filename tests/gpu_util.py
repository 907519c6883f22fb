"""Helpers shared by the GPU parity tests: run the HIP path on a workload
and compare with the fp64 oracle.  The HIP path is reached only through the
package's ctypes binding, i.e. through the C ABI."""
from __future__ import annotations

import numpy as np

import oracle
from paged_kv_attention_24_amd import workloads as W

# tolerances on the decode output (fp32 out), max-abs vs the fp64 oracle
TOL = {"f32": 1e-5, "f16": 2e-3, "bf16": 2e-3}


def gpu_decode(wl, *, partition_size=None, out_dtype=None, device="cuda", write=True,
               max_context_len=None, return_caches=False):
    """kv_cache_write (if the workload carries new tokens) then decode on
    the GPU; returns the output as float64 numpy (and the caches' bits)."""
    import torch

    import paged_kv_attention_24_amd as pka

    d = W.device_inputs(wl, device)
    if write and wl.new_k is not None:
        pka.kv_cache_write(d["new_k"], d["new_v"], d["slot_mapping"], d["k_cache"], d["v_cache"])
    P = wl.partition_size if partition_size is None else partition_size
    out = pka.paged_attention_decode(
        d["q"], d["k_cache"], d["v_cache"], d["block_tables"], d["context_lens"],
        float(wl.scale), wl.num_kv_heads, wl.block_size, partition_size=P,
        max_context_len=wl.max_context_len if max_context_len is None else max_context_len,
        out_dtype=out_dtype)
    torch.cuda.synchronize()
    res = out.float().double().cpu().numpy()
    if return_caches:
        return res, (W.to_numpy_bits(d["k_cache"], wl.dtype), W.to_numpy_bits(d["v_cache"], wl.dtype))
    return res


def check_close(got, ref, dtype, what=""):
    assert got.shape == ref.shape, (got.shape, ref.shape)
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    err = float(np.max(np.abs(got - ref))) if got.size else 0.0
    assert err <= TOL[dtype], f"{what}: max-abs error {err:.3g} > {TOL[dtype]:g}"
    return err


def oracle_full(wl, **kw):
    return oracle.decode_workload(wl, **kw)


def sample_rows(wl, n, seed=0, must=()):
    rng = np.random.default_rng(seed)
    rows = {(int(b), int(h)) for b, h in must}
    while len(rows) < n:
        rows.add((int(rng.integers(0, wl.num_seqs)), int(rng.integers(0, wl.num_q_heads))))
    return np.array(sorted(rows), dtype=np.int32)
