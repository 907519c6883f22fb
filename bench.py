#!/usr/bin/env python3
"""Benchmark: batched paged decode attention + KV-cache write on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--config 2]

One step is one pass of the whole hot path over one batch: the batched
KV-cache write of one new token per sequence and the paged decode over it,
issued as one fused launch per layer (pka_paged_attention_decode_append;
bit-identical to the write followed by the decode).  The default workload
is the Llama-3.2-1B decode step at batch 16 (32 query / 8 kv heads,
head_dim 64, block_size 16, fp16 KV, context lengths U[100, 1024]), run
over 16 layer pools back to back, so one step is one decode step of the
16-layer model's attention; the 16 pools (~370 MB) exceed the 256 MB
Infinity Cache.  Inputs are resident in HBM before the timed region; the
timed region replays a HIP graph of the step (launch overhead of Python and
the runtime excluded, kernel-to-kernel gaps included).  The same step as two
launches per layer (write, then decode) is timed as well and reported.

Prints ONE JSON line: effective KV GB/s (sum_b L_b * 2 * Hkv * D * elt per
second), microseconds per layer, the roofline of the decode call, and the
fp64 CPU oracle timed on a bounded sample of the same workload.
"""
from __future__ import annotations

import argparse
import json
import os
import platform
import sys
import time

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, HERE)

HBM_PEAK_GBPS = 8000.0  # MI355X HBM3E, vendor specification
METRIC = "paged decode attention effective KV GB/s + % HBM peak; µs/layer at batch 16"


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--path", default="decode",
                    choices=["decode", "prefill", "blocks", "rope", "int8", "stream"],
                    help="decode step (the headline), multi-token causal attention, or "
                         "whole-block moves (preemption, paging), the RoPE write, or the "
                         "decode over group-quantised INT8 pools")
    ap.add_argument("--group-size", type=int, default=64,
                    help="INT8 path: quantisation group (32, 64 or 128 dims)")
    ap.add_argument("--no-compare", action="store_true",
                    help="INT8 path: skip timing the fp16/bf16 decode of the same shape "
                         "and the fused write + decode step")
    ap.add_argument("--config", type=int, default=2, choices=[2, 3, 4, 5],
                    help="workload (decode: 2 = Llama-3.2-1B batch 16, the headline; "
                         "prefill: 2 = chunked prefill, 3 = drafted-token check)")
    ap.add_argument("--layers", type=int, default=0,
                    help="pools per step (default: 16 for workload 2, else enough to exceed 1 GB)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="approximate CPU time budget of the oracle sample")
    ap.add_argument("--eager", action="store_true", help="time eager launches, not a HIP graph")
    ap.add_argument("--partition-size", type=int, default=0,
                    help="override the library's partition length (tokens)")
    ap.add_argument("--extra-configs", default="3,4,5",
                    help="decode workloads timed after the headline one (config 2 only), "
                         "each reported under configs.<n>; 'none' to skip")
    ap.add_argument("--no-extras", action="store_true",
                    help="decode: time only the fused step (no two-launch or hot timing), "
                         "so that a profiler sees that step's launches alone")
    ap.add_argument("--no-ceilings", action="store_true",
                    help="skip measuring the HBM read ceilings (csrc/calibrate.hip)")
    ap.add_argument("--calibration-copy-mib", type=int, default=0,
                    help="run one torch copy of this many MiB first (a known-size kernel for "
                         "scaling rocprofv3 FETCH_SIZE / WRITE_SIZE counters)")
    return ap.parse_args()


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


# the sources that define each kernel (hashed to tell whether a committed
# counter summary still describes it)
KERNEL_SOURCES = {"decode": ("paged_decode.hip", "cdna4.h", "pka_internal.h"),
                  "prefill": ("paged_prefill.hip", "cdna4.h", "pka_internal.h"),
                  "blocks": ("block_ops.hip", "pka_internal.h"),
                  "rope": ("kv_cache_write.hip", "cdna4.h", "pka_internal.h"),
                  "int8": ("paged_int8.hip", "cdna4.h", "pka_internal.h")}


def kernel_source_sha(path_kind):
    import hashlib

    h = hashlib.sha256()
    for name in KERNEL_SOURCES[path_kind]:
        h.update(open(os.path.join(HERE, "paged_kv_attention_24_amd", "csrc", name), "rb").read())
    return h.hexdigest()


def profile_fields(tag, path_kind="decode"):
    """The machine-read fields of the committed rocprofv3 counter summary
    profiles/<tag>.md, or {} when the kernel's sources have changed since the
    counters were taken (or no summary exists)."""
    path = os.path.join(HERE, "profiles", f"{tag}.md")
    if not os.path.exists(path):
        return {}
    fields = {}
    for line in open(path):
        if ":" in line:
            k, _, v = line.partition(":")
            fields[k.strip()] = v.strip()
    if fields.get("kernel_source_sha256") != kernel_source_sha(path_kind):
        return {}
    return fields


def measured_traffic(tag, path_kind="decode"):
    """HBM bytes per launch from the counter summary (None when stale)."""
    f = profile_fields(tag, path_kind)
    return int(f["traffic_bytes_per_launch"]) if "traffic_bytes_per_launch" in f else None


def measured_occupancy(tag, path_kind="decode"):
    """Mean resident waves per CU and the share of wave time spent waiting,
    from the same summary's SQ counter pass (None when stale or absent)."""
    f = profile_fields(tag, path_kind)
    if "resident_waves_per_cu" not in f:
        return None
    return {"resident_waves_per_cu": float(f["resident_waves_per_cu"]),
            "waiting_share": float(f["waiting_share"]),
            "source": f"profiles/{tag}.md (SQ_WAVE_CYCLES, SQ_WAIT_ANY, GRBM_GUI_ACTIVE)"}


PROFILE_TAGS = {2: "paged_decode_llama3_1b_b16", 3: "paged_decode_mix_b64",
                4: "paged_decode_qwen3_b128", 5: "paged_decode_skewed_b256"}


def fill_pool(shape, dtype, seed, device):
    import torch

    g = torch.Generator(device=device)
    g.manual_seed(seed)
    x = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
    return x.to(dtype)


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "this build measures one GPU only; run with --gpus 1 "
                                   "(multi-GPU sharding is described, not built)"}))
        return 2

    import torch

    import paged_kv_attention_24_amd as pka

    if not torch.cuda.is_available():
        raise SystemExit("bench.py needs a GPU")
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    pka.load_library()
    if args.path == "prefill":
        return run_prefill(args, dev)
    if args.path == "blocks":
        return run_blocks(args, dev)
    if args.path == "rope":
        return run_rope(args, dev)
    if args.path == "int8":
        return run_int8(args, dev)
    if args.path == "stream":
        return run_stream(args, dev)

    line = decode_line(args, dev)
    print(json.dumps(line), flush=True)
    return 0


def cpu_model() -> str:
    """The host CPU's model name (from /proc/cpuinfo where there is one)."""
    try:
        with open("/proc/cpuinfo") as f:
            for ln in f:
                if ln.startswith("model name"):
                    return ln.split(":", 1)[1].strip()
    except OSError:
        pass
    return platform.processor() or platform.machine()


def host_threads() -> int:
    return int(os.environ.get("OMP_NUM_THREADS", "0") or 0) or os.cpu_count()


def load_calibration():
    import ctypes

    path = os.path.join(HERE, "paged_kv_attention_24_amd", "libpka_calib.so")
    if not os.path.exists(path):
        raise SystemExit(f"{path} is missing: build with python -m paged_kv_attention_24_amd._build")
    lib = ctypes.CDLL(path)
    P, i64, i32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
    lib.pka_calib_stream_read.argtypes = [P, i64, P, i32, P]
    lib.pka_calib_stream_read.restype = i32
    lib.pka_calib_gather_read.argtypes = [P, P, i64, i32, P, i32, P]
    lib.pka_calib_gather_read.restype = i32
    return lib


def measure_ceilings(dev, reps=8, gib=4):
    """HBM read ceilings of this GPU (csrc/calibrate.hip): one contiguous read
    of a buffer far larger than the 256 MB MALL, and a gather of its 4 KiB
    tiles in random order (the access pattern of a block-table walk over a
    shuffled pool).  GB/s of bytes read."""
    import torch

    lib = load_calibration()
    nbytes = gib << 30
    buf = torch.ones(nbytes // 4, dtype=torch.int32, device=dev)
    sink = torch.zeros(256, dtype=torch.int32, device=dev)
    grid = torch.cuda.get_device_properties(dev).multi_processor_count * 8
    stream = torch.cuda.current_stream(dev).cuda_stream
    tile = 4096
    n_tiles = nbytes // tile
    gen = torch.Generator(device=dev)
    gen.manual_seed(11)
    order = torch.randperm(n_tiles, generator=gen, device=dev).to(torch.int32)

    def run_stream():
        if lib.pka_calib_stream_read(buf.data_ptr(), nbytes, sink.data_ptr(), grid, stream):
            raise RuntimeError("stream-read launch failed")

    def run_gather():
        if lib.pka_calib_gather_read(buf.data_ptr(), order.data_ptr(), n_tiles, tile,
                                     sink.data_ptr(), grid, stream):
            raise RuntimeError("gather-read launch failed")

    res = {}
    for name, fn in (("stream_read", run_stream), ("gather_4KiB", run_gather)):
        fn()
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / reps
        res[f"{name}_GBps"] = round(nbytes / (ms * 1e-3) / 1e9, 1)
        res[f"{name}_us"] = round(ms * 1e3, 1)
    res["buffer_GiB"] = gib
    res["source"] = "bench.py measure_ceilings(): libpka_calib.so (csrc/calibrate.hip), HIP events"
    del buf, order
    torch.cuda.empty_cache()
    return res


def run_stream(args, dev):
    """--path stream: the read ceilings alone, as one JSON line."""
    c = measure_ceilings(dev, reps=max(args.steps, 2))
    line = {
        "metric": "HBM read ceiling of a plain read-only kernel (calibration)",
        "value": c["stream_read_GBps"], "unit": "GB/s", "n_gpus": 1, "steps": max(args.steps, 2),
        "warmup": 1, "ms_per_step": round(c["stream_read_us"] / 1e3, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "u8",
        "data": "synthetic (4 GiB of ones)",
        "config": {"workload": f"contiguous read and random 4 KiB-tile gather of "
                               f"{c['buffer_GiB']} GiB", "parallelism": "single GPU"},
        "pct_hbm_peak": round(100.0 * c["stream_read_GBps"] / HBM_PEAK_GBPS, 2),
        "gather_4KiB_GBps": c["gather_4KiB_GBps"],
        "roofline": {"bound": "hbm", "kernel": "stream_read (csrc/calibrate.hip)",
                     "achieved": c["stream_read_GBps"], "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": round(c["stream_read_GBps"] / HBM_PEAK_GBPS, 4), "traffic": None},
        "cpu_baseline": None,
    }
    print(json.dumps(line), flush=True)
    return 0


def oracle_times(wl, kc_h, vc_h, *, full: bool, seconds: float, seed: int):
    """The fp64 oracle on the host, with all threads and with one: a full
    decode of one layer pool (full=True, repeated for about `seconds`), or a
    sample of rows scaled to the whole batch by context length (the oracle's
    work per row is proportional to it).  Returns (us all threads, us one
    thread, threads, sample text)."""
    import oracle

    B, Hq = wl.num_seqs, wl.num_q_heads
    L = wl.context_lens.astype(np.int64)
    rows = None
    scale_up = 1.0
    if not full:
        rng = np.random.default_rng(seed)
        n = min(64, B * Hq)
        pick = rng.choice(B * Hq, size=n, replace=False)
        rows = np.stack([pick // Hq, pick % Hq], axis=1).astype(np.int32)
        work = max(int(L[rows[:, 0]].sum()), 1)
        scale_up = float(L.sum() * Hq) / work

    def timed(threads, budget):
        n_done, t0 = 0, time.perf_counter()
        while True:
            oracle.paged_attention_decode(wl.q, kc_h, vc_h, wl.block_tables, wl.context_lens,
                                          wl.scale, wl.num_kv_heads, wl.block_size, wl.dtype,
                                          rows=rows, threads=threads)
            n_done += 1
            el = time.perf_counter() - t0
            if el >= budget or n_done >= 256:
                return el / n_done * 1e6 * scale_up, n_done, el

    threads = host_threads()
    us_all, n_all, el_all = timed(threads, seconds)
    us_one, n_one, el_one = timed(1, seconds / 2)
    what = (f"full decode of one layer pool ({B} seqs x {Hq} q-heads, {int(L.sum())} tokens)"
            if full else f"{len(rows)} random (seq, q-head) rows, scaled to the batch by "
                         f"context length (x{scale_up:.1f})")
    sample = (f"{what}: {n_all} runs in {el_all:.1f} s on {threads} threads, {n_one} runs in "
              f"{el_one:.1f} s on 1 thread; fp64 C oracle, OpenMP; host {cpu_model()}")
    return us_all, us_one, threads, sample


def measure_decode(args, dev, cfg, *, steps, warmup, headline, host_copy):
    """One workload's decode step (the fused new-token store + decode, one
    launch per layer pool), timed cold over R layer pools that together
    exceed the 256 MB MALL, and hot over pool 0 alone when it fits the MALL;
    plus the same step as two launches per layer.  Returns a dict of
    figures (and the workload)."""
    import torch

    import paged_kv_attention_24_amd as pka
    from paged_kv_attention_24_amd import workloads as W

    host_pools = cfg in (2, 3)
    wl = W.make_config(cfg, pools=host_pools, poison=False)
    tdt = W.torch_dtype(wl.dtype)
    B, Hq, Hkv, D, bs = wl.num_seqs, wl.num_q_heads, wl.num_kv_heads, wl.head_dim, wl.block_size
    pool_bytes = 2 * wl.num_blocks * Hkv * bs * D * wl.elt_bytes
    if headline and args.layers > 0:
        R = args.layers
    elif cfg == 2:
        R = 16
    else:
        R = max(1, int(np.ceil(1.0e9 / pool_bytes)))
    log(f"workload {cfg}: {wl.meta['description']}; pools per step {R} "
        f"({R * pool_bytes / 1e6:.0f} MB)")

    d0 = W.device_inputs(wl, dev) if host_pools else None
    q = W.as_torch(wl.q, wl.dtype, dev)
    bt = torch.from_numpy(wl.block_tables).to(dev)
    cl = torch.from_numpy(wl.context_lens).to(dev)
    new_k = W.as_torch(wl.new_k, wl.dtype, dev)
    new_v = W.as_torch(wl.new_v, wl.dtype, dev)
    slots = torch.from_numpy(wl.slot_mapping).to(dev)
    shape = (wl.num_blocks, Hkv, bs, D)
    kcs, vcs = [], []
    for r in range(R):
        if r == 0 and host_pools:
            kcs.append(d0["k_cache"])
            vcs.append(d0["v_cache"])
        else:
            kcs.append(fill_pool(shape, tdt, 1000 + 2 * r, dev))
            vcs.append(fill_pool(shape, tdt, 1001 + 2 * r, dev))
    P = (args.partition_size if headline else 0) or wl.partition_size  # 0: the library's choice
    ws_bytes = pka.decode_workspace_bytes(B, Hq, Hkv, D)
    ws = torch.zeros(max(ws_bytes, 256), dtype=torch.uint8, device=dev)  # counters start at 0
    outs = [torch.empty((B, Hq, D), dtype=torch.float32, device=dev) for _ in range(R)]
    torch.cuda.synchronize()

    def fused(r):
        pka.paged_attention_decode_append(q, new_k, new_v, slots, kcs[r], vcs[r], bt, cl,
                                          float(wl.scale), Hkv, bs, out=outs[r],
                                          partition_size=P, max_context_len=wl.max_context_len,
                                          workspace=ws)

    def step():  # one fused launch per layer: store the new tokens + decode
        for r in range(R):
            fused(r)

    def step_two_launch():
        for r in range(R):
            pka.kv_cache_write(new_k, new_v, slots, kcs[r], vcs[r])
            pka.paged_attention_decode(q, kcs[r], vcs[r], bt, cl, float(wl.scale), Hkv, bs,
                                       out=outs[r], partition_size=P,
                                       max_context_len=wl.max_context_len, workspace=ws)

    if headline and args.calibration_copy_mib > 0:
        n = args.calibration_copy_mib << 20
        src_c = torch.ones(n, dtype=torch.uint8, device=dev)
        dst_c = torch.empty_like(src_c)
        torch.cuda.synchronize()
        dst_c.copy_(src_c)
        torch.cuda.synchronize()
        del src_c, dst_c

    for _ in range(max(1, warmup)):
        step()
    torch.cuda.synchronize()
    use_graph = not args.eager
    t_wall0 = time.perf_counter()
    ms_step = timed_calls(step, steps, warmup, use_graph)
    t_wall = time.perf_counter() - t_wall0
    ms_two = None if args.no_extras else timed_calls(step_two_launch, steps, warmup, use_graph)
    # hot: the same R launches, all on pool 0, so its K/V stay in the 256 MB MALL
    hot_fits = pool_bytes <= 192e6 and not args.no_extras

    def step_hot():
        for _ in range(R):
            fused(0)

    ms_hot = timed_calls(step_hot, steps, warmup, use_graph) / R if hot_fits else None
    # fully cold (workload 2): 48 layer pools, over 1 GB, so that no launch can
    # find its K/V still in the MALL
    R_COLD = 48
    ms_cold = None
    if headline and cfg == 2 and R < R_COLD and not args.no_extras:
        for r in range(R, R_COLD):
            kcs.append(fill_pool(shape, tdt, 1000 + 2 * r, dev))
            vcs.append(fill_pool(shape, tdt, 1001 + 2 * r, dev))
            outs.append(torch.empty((B, Hq, D), dtype=torch.float32, device=dev))
        torch.cuda.synchronize()

        def step_cold():
            for r in range(R_COLD):
                fused(r)

        ms_cold = timed_calls(step_cold, steps, warmup, use_graph) / R_COLD
    log(f"workload {cfg}: step {ms_step * 1e3:.1f} us ({R} fused launches), two-launch "
        f"{ms_two * 1e3 if ms_two else float('nan'):.1f} us, hot "
        f"{ms_hot * 1e3 if ms_hot else float('nan'):.1f} us, 48 pools "
        f"{ms_cold * 1e3 if ms_cold else float('nan'):.1f} us; timed wall {t_wall:.2f} s")

    kv_bytes = wl.kv_bytes()
    us_per_layer = ms_step * 1e3 / R
    # one fused launch: algorithmic bytes = KV + q + out + block ids + lengths
    # + the new rows read and stored + the slots
    nblk = int(np.sum((wl.context_lens.astype(np.int64) + bs - 1) // bs))
    new_rows = B * Hkv * D * wl.elt_bytes * 2
    alg_bytes = kv_bytes + B * Hq * D * (wl.elt_bytes + 4) + nblk * 4 + B * 4 + 2 * new_rows + 8 * B
    res = dict(wl=wl, R=R, P=int(P), use_graph=use_graph, kv_bytes=kv_bytes, alg_bytes=alg_bytes,
               us_per_layer=us_per_layer, us_two=ms_two * 1e3 / R if ms_two else None,
               us_hot=ms_hot * 1e3 if ms_hot else None,
               us_cold48=ms_cold * 1e3 if ms_cold else None,
               value=kv_bytes * R / (ms_step * 1e-3) / 1e9,
               achieved=alg_bytes / (us_per_layer * 1e-6) / 1e9)
    if ms_hot:
        res["value_hot"] = kv_bytes / (ms_hot * 1e-3) / 1e9
    if host_copy:  # for the oracle, timed after every GPU measurement
        res["kc_h"] = W.to_numpy_bits(kcs[0], wl.dtype)
        res["vc_h"] = W.to_numpy_bits(vcs[0], wl.dtype)
    del kcs, vcs, outs, ws, d0
    torch.cuda.empty_cache()
    return res


def config_entry(m, cfg, ceilings, oracle_us=None):
    """The per-workload figures of the bench line."""
    wl = m["wl"]
    e = {
        "workload": wl.meta["description"],
        "layers_per_step": m["R"],
        "partition_size": m["P"],
        "sum_context_tokens": int(wl.context_lens.sum()),
        "us_per_layer": round(m["us_per_layer"], 3),
        "us_per_layer_hot": round(m["us_hot"], 3) if m["us_hot"] else None,
        "hot_note": ("the step's launches all on pool 0: its K/V stay resident in the 256 MB MALL"
                     if m["us_hot"] else "one layer pool exceeds the 256 MB MALL: no hot figure"),
        "us_per_layer_two_launch": round(m["us_two"], 3) if m["us_two"] else None,
        "effective_GBps": round(m["value"], 2),
        "pct_hbm_peak": round(100.0 * m["value"] / HBM_PEAK_GBPS, 2),
        "launches_per_layer": 1,
        "roofline": {
            "bound": "hbm", "kernel": "decode_kernel",
            "achieved": round(m["achieved"], 2), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
            "frac": round(m["achieved"] / HBM_PEAK_GBPS, 4),
            "frac_of_stream_read": (round(m["achieved"] / ceilings["stream_read_GBps"], 4)
                                    if ceilings else None),
            "traffic": measured_traffic(PROFILE_TAGS[cfg], "decode"),
            "occupancy": measured_occupancy(PROFILE_TAGS[cfg], "decode"),
            "traffic_source": f"profiles/{PROFILE_TAGS[cfg]}.md (rocprofv3 FETCH_SIZE + "
                              "WRITE_SIZE, copy-calibrated; null when the kernel changed since)",
            "algorithmic_bytes_per_launch": int(m["alg_bytes"]),
        },
    }
    if m.get("value_hot"):
        e["effective_GBps_hot"] = round(m["value_hot"], 2)
    if m.get("us_cold48"):
        e["us_per_layer_cold48"] = round(m["us_cold48"], 3)
        e["cold48_note"] = "the same fused launch cycled over 48 layer pools (1.1 GB, over 4x the MALL)"
    if oracle_us is not None:
        e["oracle"] = oracle_us
    return e


def decode_line(args, dev):
    cfg = args.config
    ceilings = None
    if not args.no_ceilings:
        ceilings = measure_ceilings(dev)
        log(f"read ceilings: {ceilings}")
    want_cpu = not args.no_cpu_baseline
    m = measure_decode(args, dev, cfg, steps=args.steps, warmup=args.warmup, headline=True,
                       host_copy=want_cpu)
    wl = m["wl"]
    B, Hq, Hkv, D, bs = wl.num_seqs, wl.num_q_heads, wl.num_kv_heads, wl.head_dim, wl.block_size

    extra_cfgs = [int(x) for x in args.extra_configs.split(",") if x.strip()] \
        if args.extra_configs not in ("", "none") and cfg == 2 else []
    measured = {}
    for c in extra_cfgs:
        measured[c] = measure_decode(args, dev, c,
                                     steps=max(5, min(args.steps, 20 if c != 4 else 10)),
                                     warmup=max(1, min(args.warmup, 3)), headline=False,
                                     host_copy=want_cpu)
    # every GPU measurement is done: the oracle's timings follow
    extra = {}
    for c, mc in measured.items():
        o = None
        if want_cpu:
            us_all, us_one, threads, sample = oracle_times(mc["wl"], mc["kc_h"], mc["vc_h"],
                                                           full=c == 3, seconds=3.0, seed=c)
            o = {"us_all_cores": round(us_all, 1), "us_1core": round(us_one, 1),
                 "cores": threads, "sample": sample}
        extra[str(c)] = config_entry(mc, c, ceilings, o)
    measured.clear()

    cpu = None
    if want_cpu:
        us_all, us_one, threads, sample = oracle_times(wl, m["kc_h"], m["vc_h"], full=True,
                                                       seconds=args.cpu_seconds, seed=cfg)
        cpu = {
            "value": round(m["kv_bytes"] / (us_all * 1e-6) / 1e9, 4),
            "unit": "GB/s",
            "cores": threads,
            "kind": "oracle",
            "sample": sample,
            "us_per_layer": round(us_all, 1),
            "value_1core": round(m["kv_bytes"] / (us_one * 1e-6) / 1e9, 4),
            "us_per_layer_1core": round(us_one, 1),
            "cpu_model": cpu_model(),
        }

    line = {
        "metric": METRIC,
        "value": round(m["value"], 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(m["us_per_layer"] * m["R"] / 1e3, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": wl.dtype,
        "data": "synthetic (seeded N(0,1) KV/q, shuffled block pool)",
        "config": {
            "workload": wl.meta["description"],
            "global_batch": B,
            "layers_per_step": m["R"],
            "num_q_heads": Hq, "num_kv_heads": Hkv, "head_dim": D, "block_size": bs,
            "kv_dtype": wl.dtype, "accumulate": "f32", "out_dtype": "f32",
            "sum_context_tokens": int(wl.context_lens.sum()),
            "partition_size": m["P"],
            "timing": "hip-graph replay" if m["use_graph"] else "eager",
            "parallelism": "single GPU",
        },
        "us_per_layer": round(m["us_per_layer"], 3),
        "us_per_layer_hot": round(m["us_hot"], 3) if m["us_hot"] else None,
        "hot_note": "the step's 16 launches all on pool 0: its K/V stay resident in the 256 MB "
                    "MALL; us_per_layer cycles 16 layer pools (370 MB) through it",
        "us_per_layer_two_launch": round(m["us_two"], 3) if m["us_two"] else None,
        "us_per_layer_cold48": round(m["us_cold48"], 3) if m.get("us_cold48") else None,
        "cold48_note": "the same fused launch cycled over 48 layer pools (1.1 GB, over 4x the MALL)",
        "pct_hbm_peak": round(100.0 * m["value"] / HBM_PEAK_GBPS, 2),
        "roofline": {
            "bound": "hbm",
            "kernel": "decode_kernel (one launch per layer: new-token store + decode + merge)",
            "launches_per_layer": 1,
            "achieved": round(m["achieved"], 2),
            "peak": HBM_PEAK_GBPS,
            "unit": "GB/s",
            "frac": round(m["achieved"] / HBM_PEAK_GBPS, 4),
            "frac_of_stream_read": (round(m["achieved"] / ceilings["stream_read_GBps"], 4)
                                    if ceilings else None),
            "traffic": measured_traffic(PROFILE_TAGS[cfg], "decode"),
            "occupancy": measured_occupancy(PROFILE_TAGS[cfg], "decode"),
            "traffic_source": f"profiles/{PROFILE_TAGS[cfg]}.md (rocprofv3 FETCH_SIZE + WRITE_SIZE, "
                              "copy-calibrated; null when the kernel changed since)",
            "us_per_launch": round(m["us_per_layer"], 3),
            "algorithmic_bytes_per_launch": int(m["alg_bytes"]),
        },
        "hbm_ceilings": ceilings,
        "configs": extra or None,
        "cpu_baseline": cpu,
    }
    return line


PREFILL_TAGS = {2: "paged_prefill_chunked_b8", 3: "paged_prefill_drafted_b64"}
MFMA_PEAK_TFLOPS = 2500.0  # MI355X dense fp16/bf16 matrix throughput, vendor specification


def timed_calls(fn, n, warmup, use_graph):
    """ms per call of fn: HIP-graph replay (or eager calls) bracketed by
    events on the current stream, after warmup calls."""
    import torch

    if use_graph:
        g = torch.cuda.CUDAGraph()
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            fn()
        torch.cuda.current_stream().wait_stream(s)
        torch.cuda.synchronize()
        with torch.cuda.graph(g):
            fn()
        run = g.replay
    else:
        run = fn
    for _ in range(max(1, warmup)):
        run()
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(n):
        run()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / n


def run_prefill(args, dev):
    """Multi-token causal attention: workload 2 (chunked prefill, matrix-core
    bound) or 3 (drafted-token check, HBM bound), over enough layer pools to
    exceed 1 GB, one launch per layer."""
    import torch

    import paged_kv_attention_24_amd as pka
    from paged_kv_attention_24_amd import workloads as W

    n = args.config if args.config in (2, 3) else 2
    wl = W.make_prefill_config(n, poison=False, pools=False)
    tdt = W.torch_dtype(wl.dtype)
    B, Hq, Hkv, D, bs = wl.num_seqs, wl.num_q_heads, wl.num_kv_heads, wl.head_dim, wl.block_size
    pool_bytes = 2 * wl.num_blocks * Hkv * bs * D * wl.elt_bytes
    R = args.layers if args.layers > 0 else max(1, int(np.ceil(1.0e9 / pool_bytes)))
    log(f"multi-token workload {n}: {wl.meta['description']}; pools per step {R} "
        f"({R * pool_bytes / 1e6:.0f} MB)")
    shape = (wl.num_blocks, Hkv, bs, D)
    kcs = [fill_pool(shape, tdt, 2000 + 2 * r, dev) for r in range(R)]
    vcs = [fill_pool(shape, tdt, 2001 + 2 * r, dev) for r in range(R)]
    q = W.as_torch(wl.q, wl.dtype, dev)
    bt = torch.from_numpy(wl.block_tables).to(dev)
    cl = torch.from_numpy(wl.context_lens).to(dev)
    qs = torch.from_numpy(wl.query_start).to(dev)
    N = wl.num_query_tokens
    outs = [torch.empty((N, Hq, D), dtype=torch.float32, device=dev) for _ in range(R)]

    def step():
        for r in range(R):
            pka.paged_attention_prefill(q, kcs[r], vcs[r], bt, cl, qs, float(wl.scale), Hkv, bs,
                                        out=outs[r], max_query_len=wl.max_query_len)

    if args.calibration_copy_mib > 0:
        src_c = torch.ones(args.calibration_copy_mib << 20, dtype=torch.uint8, device=dev)
        dst_c = torch.empty_like(src_c)
        dst_c.copy_(src_c)
        torch.cuda.synchronize()
        del src_c, dst_c
    step()
    torch.cuda.synchronize()
    ms = timed_calls(step, args.steps, args.warmup, not args.eager)
    us_layer = ms * 1e3 / R

    # per (new token, query head): 2 D flops for each score and 2 D for each
    # weighted value, over the pos + 1 visible tokens
    T = np.diff(wl.query_start).astype(np.int64)
    L = wl.context_lens.astype(np.int64)
    visible = sum(int(np.sum(L[b] - T[b] + np.arange(T[b]) + 1)) for b in range(B))
    flops = 4.0 * D * Hq * visible
    kv_bytes = int(L.sum()) * 2 * Hkv * D * wl.elt_bytes
    nblk = int(np.sum((L + bs - 1) // bs))
    alg_bytes = kv_bytes + N * Hq * D * (wl.elt_bytes + 4) + nblk * 4 + B * 4 + (B + 1) * 4
    tflops = flops / (us_layer * 1e-6) / 1e12
    gbps = alg_bytes / (us_layer * 1e-6) / 1e9
    mfma_bound = flops / alg_bytes > MFMA_PEAK_TFLOPS * 1e12 / (HBM_PEAK_GBPS * 1e9)
    if mfma_bound:
        metric = "multi-token paged attention TFLOP/s (chunked prefill)"
        value, unit = tflops, "TFLOP/s"
        roof = {"bound": "mfma", "achieved": round(tflops, 2), "peak": MFMA_PEAK_TFLOPS,
                "unit": "TFLOP/s", "frac": round(tflops / MFMA_PEAK_TFLOPS, 4)}
    else:
        metric = "multi-token paged attention effective GB/s (drafted-token check)"
        value, unit = gbps, "GB/s"
        roof = {"bound": "hbm", "achieved": round(gbps, 2), "peak": HBM_PEAK_GBPS,
                "unit": "GB/s", "frac": round(gbps / HBM_PEAK_GBPS, 4)}
    roof.update({
        "traffic": measured_traffic(PREFILL_TAGS[n], "prefill"),
        "occupancy": measured_occupancy(PREFILL_TAGS[n], "prefill"),
        "traffic_source": f"profiles/{PREFILL_TAGS[n]}.md (rocprofv3 FETCH_SIZE + WRITE_SIZE, "
                          "copy-calibrated; null when the kernel changed since)",
        "kernel": "prefill_kernel (one launch per layer)",
        "us_per_launch": round(us_layer, 3),
        "algorithmic_bytes_per_launch": int(alg_bytes),
        "flops_per_launch": int(flops),
    })

    cpu = None
    if not args.no_cpu_baseline:
        import oracle

        threads = int(os.environ.get("OMP_NUM_THREADS", "0") or 0) or os.cpu_count()
        kc_h = W.to_numpy_bits(kcs[0], wl.dtype)  # the first layer pool, on the host
        vc_h = W.to_numpy_bits(vcs[0], wl.dtype)
        rng = np.random.default_rng(0)
        rows = np.stack([rng.integers(0, N, 256), rng.integers(0, Hq, 256)], 1).astype(np.int32)
        row_b = np.searchsorted(wl.query_start, rows[:, 0], side="right") - 1
        pos = L[row_b] - T[row_b] + (rows[:, 0] - wl.query_start[row_b])
        s_flops = 4.0 * D * float(np.sum(pos + 1))
        s_bytes = float(np.sum(pos + 1)) * 2 * D * wl.elt_bytes
        n_done, t0 = 0, time.perf_counter()
        while True:
            oracle.paged_attention_prefill(wl.q, kc_h, vc_h, wl.block_tables, wl.context_lens,
                                           wl.query_start, wl.scale, Hkv, bs, wl.dtype,
                                           rows=rows, threads=threads)
            n_done += 1
            el = time.perf_counter() - t0
            if el >= args.cpu_seconds or n_done >= 512:
                break
        cpu_value = (s_flops * n_done / el / 1e12) if mfma_bound else (s_bytes * n_done / el / 1e9)
        cpu = {"value": round(cpu_value, 6), "unit": unit, "cores": threads, "kind": "oracle",
               "sample": f"256 random (new token, query head) rows of the workload, repeated "
                         f"{n_done}x in {el:.1f} s; fp64 C oracle, OpenMP"}

    line = {
        "metric": metric,
        "value": round(value, 3),
        "unit": unit,
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": wl.dtype,
        "data": "synthetic (seeded N(0,1) KV/q, shuffled block pool)",
        "config": {
            "workload": wl.meta["description"],
            "global_batch": B,
            "new_tokens": N,
            "layers_per_step": R,
            "num_q_heads": Hq, "num_kv_heads": Hkv, "head_dim": D, "block_size": bs,
            "kv_dtype": wl.dtype, "accumulate": "f32", "out_dtype": "f32",
            "sum_context_tokens": int(L.sum()),
            "timing": "hip-graph replay" if not args.eager else "eager",
            "parallelism": "single GPU",
        },
        "us_per_layer": round(us_layer, 3),
        "tflops": round(tflops, 3),
        "effective_gbps": round(gbps, 2),
        "roofline": roof,
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)
    return 0


BLOCKS_TAG = "block_moves_llama3_1b"


def run_blocks(args, dev):
    """Whole-block moves on the Llama-3.2-1B layer shape (8 kv heads, block
    16, head_dim 64, fp16: 16 KiB per block per pool) in pools of 16384
    blocks: copy 4096 random disjoint (src, dst) pairs per launch (HBM
    roofline: read + write of both pools' blocks); gather, scatter and the
    swaps through pinned host memory are timed beside it."""
    import torch

    import paged_kv_attention_24_amd as pka

    NB, H, BS, D, n = 16384, 8, 16, 64, 4096
    shape = (NB, H, BS, D)
    kc = fill_pool(shape, torch.float16, 3000, dev)
    vc = fill_pool(shape, torch.float16, 3001, dev)
    rng = np.random.default_rng(0)
    perm = rng.permutation(NB)
    pairs_h = np.stack([perm[:n], perm[n:2 * n]], 1).astype(np.int64)
    pairs = torch.from_numpy(pairs_h).to(dev)
    ids = torch.from_numpy(perm[:n].astype(np.int64)).to(dev)
    dst_ids = torch.from_numpy(perm[2 * n:3 * n].astype(np.int64)).to(dev)
    bb = H * BS * D * 2
    packed = torch.empty((n, 2, bb), dtype=torch.uint8, device=dev)
    host = torch.empty((n, 2, bb), dtype=torch.uint8, pin_memory=True)
    moved = 2 * n * bb  # bytes of blocks moved per launch (K and V)
    if args.calibration_copy_mib > 0:
        src_c = torch.ones(args.calibration_copy_mib << 20, dtype=torch.uint8, device=dev)
        dst_c = torch.empty_like(src_c)
        dst_c.copy_(src_c)
        torch.cuda.synchronize()
        del src_c, dst_c
    use_graph = not args.eager
    rep = 8  # launches per timed call (repeating a move rewrites the same bytes)

    def repeated(fn):
        def calls():
            for _ in range(rep):
                fn()
        return calls

    ms_copy = timed_calls(repeated(lambda: pka.copy_blocks(kc, vc, pairs)), args.steps,
                          args.warmup, use_graph) / rep
    ms_gather = timed_calls(repeated(lambda: pka.gather_blocks(kc, vc, ids, out=packed)),
                            args.steps, args.warmup, use_graph) / rep
    ms_scatter = timed_calls(repeated(lambda: pka.scatter_blocks(kc, vc, packed, dst_ids)),
                             args.steps, args.warmup, use_graph) / rep
    ms_out = timed_calls(lambda: pka.swap_out(kc, vc, ids, host=host), max(3, args.steps // 5),
                         2, False)
    ms_in = timed_calls(lambda: pka.swap_in(kc, vc, host, dst_ids), max(3, args.steps // 5), 2,
                        False)
    gbps = lambda ms, factor: factor * moved / (ms * 1e-3) / 1e9  # noqa: E731
    copy_gbps = gbps(ms_copy, 2)  # read + write
    alg = 2 * moved + n * 16      # blocks read and written, plus the (src, dst) pairs
    achieved = alg / (ms_copy * 1e-3) / 1e9

    cpu = None
    if not args.no_cpu_baseline:
        import oracle

        kh = W_to_bits(kc)
        vh = W_to_bits(vc)
        m = 512  # a sample of the pairs
        n_done, t0 = 0, time.perf_counter()
        while True:
            oracle.copy_blocks(kh, vh, pairs_h[:m])
            n_done += 1
            el = time.perf_counter() - t0
            if el >= args.cpu_seconds or n_done >= 64:
                break
        cpu = {"value": round(2 * 2 * m * bb * n_done / el / 1e9, 3), "unit": "GB/s", "cores": 1,
               "kind": "oracle",
               "sample": f"copy of {m} of the {n} pairs (the oracle snapshots both 512 MiB pools "
                         f"first), repeated {n_done}x in {el:.1f} s; single-threaded C"}

    line = {
        "metric": "paged KV block copy GB/s (read + write)",
        "value": round(copy_gbps, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_copy * rep, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16",
        "data": "synthetic (device-random pools, random disjoint block pairs)",
        "config": {
            "workload": f"block moves, Llama-3.2-1B layer pools: {NB} blocks of 8 kv heads x 16 "
                        f"x 64 fp16 (16 KiB per pool), {n} blocks per launch",
            "global_batch": n, "block_bytes_per_pool": bb,
            "timing": "hip-graph replay" if use_graph else "eager",
            "parallelism": "single GPU",
        },
        "us_copy": round(ms_copy * 1e3, 2),
        "gather_gbps": round(gbps(ms_gather, 2), 2),
        "scatter_gbps": round(gbps(ms_scatter, 2), 2),
        "swap_out_gbps_pcie_inclusive": round(gbps(ms_out, 1), 2),
        "swap_in_gbps_pcie_inclusive": round(gbps(ms_in, 1), 2),
        "roofline": {
            "bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBPS, 4),
            "traffic": measured_traffic(BLOCKS_TAG, "blocks"),
            "occupancy": measured_occupancy(BLOCKS_TAG, "blocks"),
            "traffic_source": f"profiles/{BLOCKS_TAG}.md (rocprofv3 FETCH_SIZE + WRITE_SIZE, "
                              "copy-calibrated; null when the kernel changed since)",
            "kernel": "move_blocks_kernel (copy mode, one launch)",
            "us_per_launch": round(ms_copy * 1e3, 3),
            "algorithmic_bytes_per_launch": int(alg),
        },
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)
    return 0


ROPE_TAG = "kv_write_rope_llama3_1b"


def run_rope(args, dev):
    """The KV-cache write with the rotary embedding on the new keys, for one
    prompt chunk of 16384 tokens on the Llama-3.2-1B layer shape (8 kv
    heads, head_dim 64, rotary over all 64 dims, fp16, block 16, pool of
    16384 blocks), beside the plain write of the same tokens."""
    import torch

    import paged_kv_attention_24_amd as pka

    NB, H, BS, D, T, R, MAXP = 16384, 8, 16, 64, 16384, 64, 131072
    kc = fill_pool((NB, H, BS, D), torch.float16, 4000, dev)
    vc = fill_pool((NB, H, BS, D), torch.float16, 4001, dev)
    k = fill_pool((T, H, D), torch.float16, 4002, dev)
    v = fill_pool((T, H, D), torch.float16, 4003, dev)
    rng = np.random.default_rng(0)
    slots = torch.from_numpy(rng.permutation(NB * BS)[:T].astype(np.int64)).to(dev)
    pos = torch.from_numpy(rng.integers(0, MAXP, T).astype(np.int32)).to(dev)
    theta = 500000.0 ** (-np.arange(0, R, 2, dtype=np.float64) / R)
    ang = np.arange(MAXP)[:, None] * theta[None, :]
    table = torch.from_numpy(np.concatenate([np.cos(ang), np.sin(ang)], 1).astype(np.float32)).to(dev)
    if args.calibration_copy_mib > 0:
        src_c = torch.ones(args.calibration_copy_mib << 20, dtype=torch.uint8, device=dev)
        dst_c = torch.empty_like(src_c)
        dst_c.copy_(src_c)
        torch.cuda.synchronize()
        del src_c, dst_c
    use_graph = not args.eager
    rep = 16  # launches per timed call: one short launch per graph would time the graph launch

    def rope_calls():
        for _ in range(rep):
            pka.kv_cache_write_rope(k, v, slots, pos, table, kc, vc)

    def plain_calls():
        for _ in range(rep):
            pka.kv_cache_write(k, v, slots, kc, vc)

    ms_rope = timed_calls(rope_calls, args.steps, args.warmup, use_graph) / rep
    ms_plain = timed_calls(plain_calls, args.steps, args.warmup, use_graph) / rep
    row = T * H * D * 2
    alg = 2 * row * 2 + T * (8 + 4) + T * R * 4  # K, V in and out; slots, positions; table rows
    gbps = alg / (ms_rope * 1e-3) / 1e9

    cpu = None
    if not args.no_cpu_baseline:
        import oracle

        from paged_kv_attention_24_amd import workloads as W

        m = 2048  # a sample of the tokens, into a host copy of a pool slice
        kh = W.to_numpy_bits(k[:m], "f16")
        vh = W.to_numpy_bits(v[:m], "f16")
        th = table.cpu().numpy()
        ph = pos[:m].cpu().numpy()
        sh = np.arange(m, dtype=np.int64)
        kp = np.zeros((m // BS, H, BS, D), dtype=np.uint16)
        vp = kp.copy()
        n_done, t0 = 0, time.perf_counter()
        while True:
            oracle.kv_cache_write_rope(kh, vh, sh, ph, th, kp, vp, "f16")
            n_done += 1
            el = time.perf_counter() - t0
            if el >= args.cpu_seconds or n_done >= 256:
                break
        cpu = {"value": round((2 * m * H * D * 2 * 2 + m * R * 4) * n_done / el / 1e9, 3),
               "unit": "GB/s", "cores": 1, "kind": "oracle",
               "sample": f"{m} of the {T} tokens, repeated {n_done}x in {el:.1f} s; "
                         "single-threaded C"}

    line = {
        "metric": "KV-cache write with rotary embedding, GB/s",
        "value": round(gbps, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_rope * rep, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16",
        "data": "synthetic (device-random rows and pools, random slots and positions)",
        "config": {
            "workload": f"RoPE KV write, Llama-3.2-1B layer: {T} tokens x 8 kv heads x 64 fp16, "
                        f"rotary over 64 dims, base 500000 table of {MAXP} positions",
            "global_batch": T, "timing": "hip-graph replay" if use_graph else "eager",
            "parallelism": "single GPU",
        },
        "us_rope_write": round(ms_rope * 1e3, 3),
        "us_plain_write": round(ms_plain * 1e3, 3),
        "roofline": {
            "bound": "hbm", "achieved": round(gbps, 2), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
            "frac": round(gbps / HBM_PEAK_GBPS, 4),
            "traffic": measured_traffic(ROPE_TAG, "rope"),
            "occupancy": measured_occupancy(ROPE_TAG, "rope"),
            "traffic_source": f"profiles/{ROPE_TAG}.md (rocprofv3 FETCH_SIZE + WRITE_SIZE, "
                              "copy-calibrated; null when the kernel changed since)",
            "kernel": "kv_cache_write_rope_kernel (one launch)",
            "us_per_launch": round(ms_rope * 1e3, 3),
            "algorithmic_bytes_per_launch": int(alg),
        },
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)
    return 0


INT8_TAGS = {2: "paged_decode_int8_llama3_1b_b16", 3: "paged_decode_int8_mix_b64",
             4: "paged_decode_int8_qwen3_b128", 5: "paged_decode_int8_skewed_b256"}


def run_int8(args, dev):
    """Decode over group-quantised INT8 pools (codes + float32 group scales)
    for workload 2-5's shapes and lengths, over enough layer pools to exceed
    1 GB (16 for workload 2), one call per layer (the decode launch, plus the
    merge launch when a sequence spans several partitions); beside it, the
    quantising write and the plain fp16/bf16 decode of the same shape."""
    import torch

    import paged_kv_attention_24_amd as pka
    from paged_kv_attention_24_amd import workloads as W

    cfg, gs = args.config, args.group_size
    wl = W.make_config(cfg, pools=False, poison=False, write=True)
    B, Hq, Hkv, D, bs = wl.num_seqs, wl.num_q_heads, wl.num_kv_heads, wl.head_dim, wl.block_size
    NB, ng = wl.num_blocks, D // gs
    q = W.as_torch(wl.q, wl.dtype, dev)
    bt = torch.from_numpy(wl.block_tables).to(dev)
    cl = torch.from_numpy(wl.context_lens).to(dev)
    pool_bytes = 2 * NB * Hkv * bs * (D + 4 * ng)
    R = args.layers if args.layers > 0 else (16 if cfg == 2 else max(1, int(np.ceil(1.0e9 / pool_bytes))))
    log(f"INT8 workload {cfg} (groups of {gs}): {wl.meta['description']}; pools per step {R} "
        f"({R * pool_bytes / 1e6:.0f} MB)")
    g = torch.Generator(device=dev)
    g.manual_seed(7000 + cfg)
    pools = []
    for r in range(R):
        kc = torch.randint(-127, 128, (NB, Hkv, bs * D), generator=g, device=dev, dtype=torch.int8)
        vc = torch.randint(-127, 128, (NB, Hkv, bs * D), generator=g, device=dev, dtype=torch.int8)
        ks = torch.empty((NB, Hkv, bs, ng), device=dev).uniform_(0.005, 0.03, generator=g)
        vs = torch.empty((NB, Hkv, bs, ng), device=dev).uniform_(0.005, 0.03, generator=g)
        pools.append((kc, vc, ks, vs))
    L = wl.max_context_len
    P = args.partition_size or pka.decode_int8_partition_size(B, Hkv, bs, L)
    ws = torch.empty(max(pka.decode_int8_workspace_bytes(B, Hq, D, L, P), 256), dtype=torch.uint8,
                     device=dev)
    outs = [torch.empty((B, Hq, D), dtype=torch.float32, device=dev) for _ in range(R)]
    if args.calibration_copy_mib > 0:
        src_c = torch.ones(args.calibration_copy_mib << 20, dtype=torch.uint8, device=dev)
        dst_c = torch.empty_like(src_c)
        dst_c.copy_(src_c)
        torch.cuda.synchronize()
        del src_c, dst_c
    torch.cuda.synchronize()

    def step():
        for r in range(R):
            kc, vc, ks, vs = pools[r]
            pka.paged_attention_decode_int8(q, kc, vc, ks, vs, bt, cl, float(wl.scale), Hkv, bs,
                                            out=outs[r], partition_size=P, max_context_len=L,
                                            workspace=ws)

    use_graph = not args.eager
    ms_step = timed_calls(step, args.steps, args.warmup, use_graph)
    us_layer = ms_step * 1e3 / R

    # the whole decode step in one call per layer: the new token of every
    # sequence quantised and stored at the slot of its position L - 1, then
    # the attention (pka_paged_attention_decode_append_int8)
    # (skipped with --no-compare, so that a profile's decode-kernel average
    # covers the plain decode launches alone)
    us_fused = None
    if not args.no_compare:
        new_k = W.as_torch(wl.new_k, wl.dtype, dev)
        new_v = W.as_torch(wl.new_v, wl.dtype, dev)
        slots = torch.from_numpy(wl.slot_mapping).to(dev)

        def fused_step():
            for r in range(R):
                kc, vc, ks, vs = pools[r]
                pka.paged_attention_decode_append_int8(q, new_k, new_v, slots, kc, vc, ks, vs, bt,
                                                       cl, float(wl.scale), Hkv, bs, out=outs[r],
                                                       partition_size=P, max_context_len=L,
                                                       workspace=ws)

        us_fused = timed_calls(fused_step, args.steps, args.warmup, use_graph) * 1e3 / R
        log(f"INT8 fused write + decode step {us_fused:.2f} us per layer")
    wl8 = W.Int8Workload(**{f: getattr(wl, f) for f in W.Workload.__dataclass_fields__},
                         group_size=gs)
    kv_bytes = wl8.kv_bytes()
    value = kv_bytes * R / (ms_step * 1e-3) / 1e9
    nblk = int(np.sum((wl.context_lens.astype(np.int64) + bs - 1) // bs))
    alg = kv_bytes + B * Hq * D * (2 + 4) + nblk * 4 + B * 4
    achieved = alg / (us_layer * 1e-6) / 1e9
    nparts = -(-L // P)
    log(f"INT8 decode {us_layer:.2f} us per layer, {value:.0f} GB/s effective, P={P} "
        f"({nparts} partitions)")

    # the quantising write: one new token per sequence (a decode step), and a
    # prompt chunk of 16384 tokens (at most the pool's slots) into random
    # slots of the first pool
    # (16 launches per timed graph: one short launch per graph would time
    # the graph launch)
    kc0, vc0, ks0, vs0 = pools[0]
    rep = 16
    tdt = W.torch_dtype(wl.dtype)
    wr = {}
    for name, T in (("decode_step", B), ("prompt_chunk", min(16384, NB * bs))):
        kn = fill_pool((T, Hkv, D), tdt, 7100 + T, dev)
        vn = fill_pool((T, Hkv, D), tdt, 7200 + T, dev)
        sl = torch.from_numpy(np.random.default_rng(T).permutation(NB * bs)[:T].astype(np.int64)).to(dev)

        def writes():
            for _ in range(rep):
                pka.kv_cache_write_int8(kn, vn, sl, kc0, vc0, ks0, vs0)

        ms_w = timed_calls(writes, args.steps, args.warmup, use_graph) / rep
        moved = T * Hkv * (2 * D * wl.elt_bytes + 2 * D + 8 * ng) + 8 * T
        wr[name] = {"tokens": T, "us_per_launch": round(ms_w * 1e3, 3),
                    "gbps": round(moved / (ms_w * 1e-3) / 1e9, 2)}
    log(f"INT8 write: {wr}")
    del pools
    torch.cuda.empty_cache()

    half = None
    if not args.no_compare:  # the fp16/bf16 decode of the same shape, over >= 1 GB of pools
        tdt = W.torch_dtype(wl.dtype)
        hbytes = 2 * NB * Hkv * bs * D * wl.elt_bytes
        Rh = 16 if cfg == 2 else max(1, int(np.ceil(1.0e9 / hbytes)))
        hp = [(fill_pool((NB, Hkv, bs, D), tdt, 8000 + 2 * r, dev),
               fill_pool((NB, Hkv, bs, D), tdt, 8001 + 2 * r, dev)) for r in range(Rh)]
        Ph = 512 if cfg == 5 else 0  # as the decode bench: workload 5's P, else the library's choice
        wsh = torch.zeros(max(pka.decode_workspace_bytes(B, Hq, Hkv, D), 256),
                          dtype=torch.uint8, device=dev)
        oh = torch.empty((B, Hq, D), dtype=torch.float32, device=dev)

        def half_step():
            for kc, vc in hp:
                pka.paged_attention_decode(q, kc, vc, bt, cl, float(wl.scale), Hkv, bs, out=oh,
                                           partition_size=Ph, max_context_len=L, workspace=wsh)

        ms_h = timed_calls(half_step, args.steps, args.warmup, use_graph)
        half = {"us_per_layer": round(ms_h * 1e3 / Rh, 3), "kv_dtype": wl.dtype,
                "layers_per_step": Rh, "partition_size": int(Ph),
                "effective_kv_gbps": round(wl.kv_bytes() * Rh / (ms_h * 1e-3) / 1e9, 2)}
        log(f"{wl.dtype} decode of the same shape: {half['us_per_layer']:.2f} us per layer")
        del hp

    cpu = None
    if not args.no_cpu_baseline and cfg in (2, 3):
        import oracle

        threads = int(os.environ.get("OMP_NUM_THREADS", "0") or 0) or os.cpu_count()
        rng = np.random.default_rng(cfg)
        hk = rng.integers(-127, 128, (NB, Hkv, bs * D), dtype=np.int8)
        hv = rng.integers(-127, 128, (NB, Hkv, bs * D), dtype=np.int8)
        hks = rng.uniform(0.005, 0.03, (NB, Hkv, bs, ng)).astype(np.float32)
        hvs = rng.uniform(0.005, 0.03, (NB, Hkv, bs, ng)).astype(np.float32)
        n_done, t0 = 0, time.perf_counter()
        while True:
            oracle.paged_attention_decode_int8(wl.q, wl.dtype, hk, hv, hks, hvs, wl.block_tables,
                                               wl.context_lens, wl.scale, Hkv, bs,
                                               threads=threads)
            n_done += 1
            el = time.perf_counter() - t0
            if el >= args.cpu_seconds or n_done >= 512:
                break
        cpu = {"value": round(kv_bytes * n_done / el / 1e9, 4), "unit": "GB/s", "cores": threads,
               "kind": "oracle",
               "sample": f"full INT8 decode of one layer pool ({B} seqs x {Hq} q-heads) repeated "
                         f"{n_done}x in {el:.1f} s; fp64 C oracle, OpenMP",
               "us_per_layer": round(el / n_done * 1e6, 1)}

    tag = INT8_TAGS[cfg] if gs == 64 else None
    line = {
        "metric": "paged decode attention over INT8 KV: effective KV GB/s (codes + scales)",
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": f"i8 KV, {wl.dtype} q, fp16 products, f32 accumulate",
        "data": "synthetic (uniform int8 codes, uniform [0.005, 0.03] scales, shuffled block pool)",
        "config": {
            "workload": wl.meta["description"] + f"; INT8 KV in groups of {gs}",
            "global_batch": B, "layers_per_step": R, "num_q_heads": Hq, "num_kv_heads": Hkv,
            "head_dim": D, "block_size": bs, "group_size": gs,
            "sum_context_tokens": int(wl.context_lens.sum()), "partition_size": int(P),
            "timing": "hip-graph replay" if use_graph else "eager",
            "parallelism": "single GPU",
        },
        "us_per_layer": round(us_layer, 3),
        "us_per_layer_fused_step": None if us_fused is None else round(us_fused, 3),
        "quantising_write": wr,
        "half_kv_decode_same_shape": half,
        "pct_hbm_peak": round(100.0 * value / HBM_PEAK_GBPS, 2),
        "roofline": {
            "bound": "hbm",
            "kernel": ("int8_decode_kernel (one launch per layer)" if nparts == 1 else
                       "int8_decode_kernel, partitions merged in the workgroup (one launch per layer)"
                       if nparts <= 8 else
                       "int8_decode_kernel + int8_merge_kernel (per layer)" if B <= 4096
                       else "int8_plan_kernel + int8_decode_kernel + int8_merge_kernel (per layer)"),
            "launches_per_layer": 1 if nparts <= 8 else (2 if B <= 4096 else 3),
            "achieved": round(achieved, 2),
            "peak": HBM_PEAK_GBPS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBPS, 4),
            "traffic": measured_traffic(tag, "int8") if tag else None,
            "occupancy": measured_occupancy(tag, "int8") if tag else None,
            "traffic_source": (f"profiles/{tag}.md (rocprofv3 FETCH_SIZE + WRITE_SIZE, "
                               "copy-calibrated; null when the kernel changed since)" if tag
                               else "not measured for this group size"),
            "us_per_launch": round(us_layer, 3),
            "algorithmic_bytes_per_launch": int(alg),
        },
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)
    return 0


def W_to_bits(t):
    from paged_kv_attention_24_amd import workloads as W

    return W.to_numpy_bits(t, "f16")


if __name__ == "__main__":
    sys.exit(main())
