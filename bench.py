"""Benchmark: one decode step of the paged KV-cache hot path on one MI355X.

A step is the whole path over one batch: the write of each sequence's new token
into the paged pool, the planner, and the decode (one pass, or the 512-token split
plus its log-sum-exp reduce): pc_reshape_and_cache, then pc_paged_attention_decode;
``--step fused`` runs the write and the decode as one launch
(pc_reshape_and_cache_decode, 16-bit pools).  The default workload is
64 sequences of 512..2048 tokens, 32 query / 8 KV heads, head size 128, bf16, one
pass (the GQA decode the throughput target is quoted on).  ``--kv fp8`` runs the
same step over an 8-bit (OCP E4M3) cache with per-kv-head scales: the write
quantises, the decode reads one byte per K/V element.

Inputs are resident in HBM before timing starts.  To keep the K/V stream honest
with respect to the 256 MB last-level cache, the step rotates over ``--copies``
independent copies of the pool (default: enough that more than 1 GiB of other K/V
is read between two visits of one copy); ``warm_cache`` reports the same step on
one copy back to back.

Prints ONE JSON line.  ``value`` is effective GB/s over the whole step: K/V bytes
of exactly seq_len tokens per sequence plus q and out, divided by the step time
(wall clock over the timed steps, bracketed by device synchronisations, with
nothing else enqueued).
``roofline`` is the decode launch alone (with the fused write when the step fuses
it, whose rows' bytes it then adds): its algorithmic bytes per launch over its
average launch time.  That time is measured with HIP events on the launch
stream over a run of back-to-back decode launches (rotating over the pool copies,
one event pair around the run, so the events' own dispatch cost is spread over the
run); the per-launch event pairs inside the timed steps are reported beside it
(``decode_kernel_us``, with median and p10/p90), and include one dispatch each.
Two yardsticks sit beside it: ``read_peak`` (pc_stream_read, one plain read of a 4 GiB
buffer; ``roofline.measured_read_peak``) and ``gather_read`` (pc_gather_read, a
loads-only gather of exactly the decode's K/V tiles from the same pools;
``roofline.measured_gather``, and ``frac_of_measured_gather`` = the gather's launch time
over the decode's).

Beside the headline step the same line carries ``other_configs`` (the other decode
workloads on their planned paths) and ``other_paths`` (decode over an 8-bit cache on
the headline and long-context workloads, a speculative-decode step and a
chunked-prefill step), each with its launches timed by HIP events around back-to-back
runs; the long-context workload's records are taken first.
"""

from __future__ import annotations

import argparse
import json
import os
import sys
import time

REPO = os.path.dirname(os.path.abspath(__file__))
for p in (REPO, os.path.join(REPO, "tests")):
    if p not in sys.path:
        sys.path.insert(0, p)

METRIC = "paged decode attention effective GB/s and % of MI355X HBM peak; tokens/s"
HBM_PEAK_GBS = 8000.0
PROFILE_TRAFFIC = os.path.join(REPO, "profiles", "hbm_traffic.json")


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--config", type=int, default=1, help="workload index 0..4 (1 = the headline workload)")
    ap.add_argument("--copies", type=int, default=0, help="pool copies to rotate over (0 = auto, >1 GiB apart)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=10.0, help="target CPU time of the oracle sample")
    ap.add_argument("--path", choices=["plan", "single", "split"], default="plan")
    ap.add_argument("--step", choices=["separate", "fused"], default="separate",
                    help="the step's write and decode as two launches, or as one (pc_reshape_and_cache_decode)")
    ap.add_argument("--kv", choices=["native", "fp8"], default="native",
                    help="cache element type: the query's type, or OCP E4M3 codes with per-kv-head scales")
    ap.add_argument("--alibi", action="store_true", help="add the ALiBi bias (geometric slopes, one per query head)")
    ap.add_argument("--block-size", type=int, default=16, choices=[8, 16, 32],
                    help="tokens per pool block (workloads 1 and 3)")
    ap.add_argument("--varlen", choices=["prefill", "spec"], default=None,
                    help="time multi-token queries instead: a chunked-prefill step (512-token chunks) or a "
                         "speculative-decode step (4 query tokens per request)")
    ap.add_argument("--other-configs", default="2,3,4",
                    help="workloads also timed on their planned path and reported under other_configs "
                         "(comma list; '' for none)")
    ap.add_argument("--other-paths", default="fp8:1,fp8:3,spec,prefill",
                    help="other paths also timed and reported under other_paths (comma list; '' for none): "
                         "fp8:N = workload N over an E4M3 cache, spec = speculative decode (4 query tokens per "
                         "request), prefill = chunked prefill (512-token chunks)")
    ap.add_argument("--read-peak-gib", type=int, default=4,
                    help="GiB read by the streaming-read yardstick (0: skip it)")
    ap.add_argument("--plan-grid", action="store_true",
                    help="time the one-pass path against split + reduce over a grid of batch shapes and length "
                         "mixes (the data the planner is fitted on); one JSON line per shape, then exit")
    ap.add_argument("--grid-max-gib", type=float, default=6.0, help="--plan-grid: skip shapes above this K/V size")
    ap.add_argument("--grid-heads", default="32/8,32/32",
                    help="--plan-grid: num_q_heads/num_kv_heads pairs (comma list)")
    ap.add_argument("--grid-units", default="", help="--plan-grid: unit counts (comma list; default the grid's)")
    ap.add_argument("--grid-max-len", default="", help="--plan-grid: longest lengths (comma list)")
    ap.add_argument("--grid-mixes", default="", help="--plan-grid: length mixes (comma list)")
    ap.add_argument("--grid-prefix", type=int, default=0,
                    help="--plan-grid: a shared prefix of this many tokens (a multiple of 16): every sequence's "
                         "first blocks, all but its last, point to the same physical blocks")
    ap.add_argument("--no-prefix-path", action="store_true",
                    help="a workload with a shared prefix on the split path: the plain split decode instead of "
                         "pc_paged_attention_decode_prefix")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB",
                    help="only run a plain device-to-device copy of MIB MiB five times (the reference kernel "
                         "that scales the FETCH_SIZE / WRITE_SIZE counters), then exit")
    return ap.parse_args()


# the sources each family of kernels is built from: a change to any of them voids the
# counters recorded for that family
KERNEL_SOURCES = {
    "decode": ("api.hip", "decode.hip", "decode_mfma.hip", "reduce.hip", "device_common.h", "launch.h",
               "mfma_common.h"),
    # multi-token steps of at most 16 (token, head) columns per request run on the decode's unit
    "varlen": ("api.hip", "varlen.hip", "decode_mfma.hip", "device_common.h", "launch.h", "mfma_common.h"),
}


def kernel_source_hash(family: str = "decode") -> str:
    import hashlib
    h = hashlib.sha256()
    csrc = os.path.join(REPO, "paged_kv_cache_reshape_amd", "csrc")
    for f in sorted(KERNEL_SOURCES[family]):
        with open(os.path.join(csrc, f), "rb") as fh:
            h.update(f.encode() + fh.read())
    return h.hexdigest()[:16]


def stored_traffic(workload: str, family: str = "decode"):
    """HBM bytes per launch of a workload's dominant kernel from committed rocprofv3
    counter runs, if they were taken on the current sources of that kernel; else None."""
    try:
        with open(PROFILE_TRAFFIC) as f:
            rec = json.load(f).get(workload)
    except (OSError, ValueError):
        return None
    if not rec or rec.get("source_hash") != kernel_source_hash(family):
        return None
    return rec.get("bytes_per_launch")


def cpu_baseline(wl, seconds: float):
    """The fp64 oracle on the host: the step's write plus the decode of the whole batch,
    repeated until about ``seconds`` of wall time have passed."""
    import oracle
    threads = min(host_cpus()[1], 16)
    pool = oracle.filled_pool(wl, step_write=False)

    def run(nthreads, budget):
        reps, t0 = 0, time.perf_counter()
        while True:
            oracle.write(wl, pool, wl.key, wl.value, wl.slot_mapping)
            oracle.decode(wl, pool, nthreads=nthreads)
            reps += 1
            el = time.perf_counter() - t0
            if el >= budget or reps >= 1000:
                return reps, el

    reps, el = run(threads, seconds)
    reps1, el1 = run(1, seconds / 3)
    what = f"full steps (write + fp64 decode of all {wl.num_seqs} sequences) of the same workload"
    reported, usable = host_cpus()
    return {"value": round(wl.effective_bytes() * reps / el / 1e9, 4), "unit": "GB/s", "cores": threads,
            "host_cpus": reported, "host_cpus_usable": usable,
            "threads_note": "threads = the CPUs this process may use, at most 16 (one GPU's share of the box)",
            "kind": "oracle", "sample": f"{reps} {what} in {el:.1f} s on {threads} host threads",
            "tokens_per_s": round(wl.num_seqs * reps / el, 3),
            "single_thread": {"value": round(wl.effective_bytes() * reps1 / el1 / 1e9, 4), "unit": "GB/s",
                              "cores": 1, "sample": f"{reps1} {what} in {el1:.1f} s on 1 host thread"}}


def host_cpus():
    """(CPUs the host reports, CPUs this process may run on)."""
    try:
        usable = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        usable = os.cpu_count() or 1
    return os.cpu_count() or usable, usable


def measure_read_peak(torch, pc, gib: int, reps: int = 10):
    """The streaming-read yardstick (pc_stream_read): every byte of a ``gib`` GiB buffer
    read once per launch, for both cache policies the decode uses; GB/s of the faster,
    from HIP events around ``reps`` back-to-back launches on the launch stream."""
    n = gib << 30
    buf = torch.empty(n, dtype=torch.uint8, device="cuda")
    buf.fill_(1)
    wgs = 256 * 16
    sink = torch.zeros(wgs, dtype=torch.int32, device="cuda")
    stream = torch.cuda.current_stream()
    rates = {}
    for pol in (0, 2):
        for _ in range(3):
            pc.stream_read(buf, sink, cache_policy=pol)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record(stream)
        for _ in range(reps):
            pc.stream_read(buf, sink, cache_policy=pol)
        e1.record(stream)
        torch.cuda.synchronize()
        rates["nt" if pol else "default"] = round(n / (e0.elapsed_time(e1) / reps * 1e-3) / 1e9, 1)
    del buf
    return {"gbs": max(rates.values()), "by_cache_policy": rates, "bytes_per_launch": n,
            "kernel": "stream_read_kernel (pc_stream_read)"}


def measure_gather(torch, pc, wl, pools, inp, steps: int):
    """The gather yardstick (pc_gather_read) over the workload's own pools and tables:
    every K/V tile its decode reads, loads only, for both cache policies of the V loads;
    microseconds per launch from HIP events around ``steps`` back-to-back launches
    (pool copies rotating as for the decode)."""
    if wl.block_size != 16:
        return None
    sink = torch.zeros(pc.GATHER_SINK_WORDS, dtype=torch.int32, device="cuda")
    stream = torch.cuda.current_stream()
    copies = len(pools)

    def one(i, pol):
        pool = pools[i % copies]
        kw = pool.layout_kwargs()
        pc.gather_read(pool.k, pool.v, inp.block_tables, inp.seq_lens, inp.max_seq_len, sink,
                       num_kv_heads=wl.num_kv_heads, head_size=wl.head_size, num_blocks=kw["num_blocks"],
                       block_stride=kw["block_stride"], token_stride=kw["token_stride"],
                       head_stride=kw["head_stride"], v_offset=kw.get("v_offset", 0), v_cache_policy=pol)

    us = {}
    for pol in (0, 2):
        for i in range(3):
            one(i, pol)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record(stream)
        for i in range(steps):
            one(i, pol)
        e1.record(stream)
        torch.cuda.synchronize()
        us["nt" if pol else "default"] = round(e0.elapsed_time(e1) / steps * 1e3, 2)
    return {"us_by_v_cache_policy": us, "us": min(us.values()), "kernel": "gather_read_kernel (pc_gather_read)",
            "timing": "HIP events around back-to-back launches on the launch stream, pool copies rotating"}


def measure_config(idx: int, steps: int, warmup: int, no_prefix_path: bool = False, kv: str = "native"):
    """One workload on the path the planner picks: the whole step (write, plan, decode
    and, on the split path, the reduce) by wall clock, and the decode alone and the call
    (decode and reduce) by HIP events around back-to-back launches (pool copies rotating,
    three alternating rounds of each).
    ``kv="fp8"``: the same workload over an E4M3 cache with per-kv-head scales."""
    import torch
    import gpu_harness as gh
    import paged_kv_cache_reshape_amd as pc
    from workloads import fp8_variant, make_config

    print(f"[bench] other workload {idx} ({kv} cache): generating", file=sys.stderr, flush=True)
    wl = make_config(idx)
    fp8 = kv == "fp8"
    if fp8:
        wl = fp8_variant(wl)
    S, Hq, D = wl.q.shape
    per_copy = (2 if wl.layout != "combined" else 1) * wl.pool_elems * wl.kv_esize
    copies = max(1, min(8, -(-(1 << 30) // max(1, wl.kv_bytes())) + 1))
    copies = max(1, min(copies, int(64e9 // per_copy)))
    pools = [gh.filled_pool(wl, step_write=False) for _ in range(copies)]
    inp = gh.DecodeInputs(wl)
    key, value = gh.to_dev(wl.key, wl.dtype), gh.to_dev(wl.value, wl.dtype)
    slots = torch.from_numpy(wl.slot_mapping).cuda()
    out = torch.empty_like(inp.q)
    msl = inp.max_seq_len
    dt = gh.TORCH_DT[wl.dtype]
    ps, P, _ = pc.paged_attention_plan_lens(wl.seq_lens, Hq, wl.num_kv_heads, D, wl.head_stride, dt,
                                            kv_fp8=fp8, shared_lens=wl.shared_lens())
    kw = {}
    if ps:
        kw = dict(partition_size=ps, exp_sums=torch.empty((S, Hq, P), device="cuda"),
                  max_logits=torch.empty((S, Hq, P), device="cuda"), tmp_out=torch.empty((S, Hq, P, D), device="cuda"))
    stream = torch.cuda.current_stream()
    use_prefix = bool(ps and wl.prefix_blocks and not fp8 and not no_prefix_path)
    if use_prefix:
        pkw = dict(exp_sums=kw["exp_sums"], max_logits=kw["max_logits"], tmp_out=kw["tmp_out"],
                   prefix_table=torch.from_numpy(wl.prefix_table()).cuda(),
                   shared_lens=torch.from_numpy(wl.shared_lens()).cuda())

    def decode(i):
        pool = pools[i % copies]
        if fp8:
            pc.paged_attention_decode_fp8(None if ps else out, inp.q, pool.k, pool.v, inp.block_tables, inp.seq_lens,
                                          msl, pool.k_scale, pool.v_scale, num_kv_heads=wl.num_kv_heads,
                                          scale=float(wl.scale), **pool.layout_kwargs(), **pool.scale_kwargs(), **kw)
            return
        if use_prefix:
            pc.paged_attention_decode_prefix(inp.q, pool.k, pool.v, inp.block_tables, inp.seq_lens, msl,
                                             num_kv_heads=wl.num_kv_heads, scale=float(wl.scale), **pkw,
                                             **pool.layout_kwargs())
            return
        pc.paged_attention_decode(None if ps else out, inp.q, pool.k, pool.v, inp.block_tables, inp.seq_lens, msl,
                                  num_kv_heads=wl.num_kv_heads, scale=float(wl.scale), **pool.layout_kwargs(), **kw)

    def reduce(i):
        pc.paged_attention_reduce(out, kw["exp_sums"], kw["max_logits"], kw["tmp_out"], inp.seq_lens)

    def call(i):
        decode(i)
        if ps:
            reduce(i)

    def step(i):
        pool = pools[i % copies]
        if fp8:
            pc.reshape_and_cache_fp8(key, value, pool.k, pool.v, slots, pool.k_scale, pool.v_scale,
                                     **pool.layout_kwargs(), **pool.scale_kwargs())
        else:
            pc.reshape_and_cache(key, value, pool.k, pool.v, slots, **pool.layout_kwargs())
        pc.paged_attention_plan_lens(wl.seq_lens, Hq, wl.num_kv_heads, D, wl.head_stride, dt,
                                     kv_fp8=fp8, shared_lens=wl.shared_lens())
        call(i)

    def batched(fn, n):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record(stream)
        for i in range(n):
            fn(i)
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / n * 1e3  # us

    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        step(i)
    torch.cuda.synchronize()
    step_us = (time.perf_counter() - t0) / steps * 1e6
    # decode alone and the call, in alternating rounds (one short run of either can catch
    # a slow stretch of the device); the means over the rounds are reported
    dec_r, call_r = [], []
    for _ in range(3):
        dec_r.append(batched(decode, steps))
        call_r.append(batched(call, steps))
    dec_us, call_us = sum(dec_r) / len(dec_r), sum(call_r) / len(call_r)
    # the reduce's share of the call (reduces alone back to back would wait on the host)
    red_us = call_us - dec_us
    eff = wl.effective_bytes()
    rec = {"workload": wl.name, "path": ("split (shared prefix)" if use_prefix else "split") if ps else "single",
           "num_seqs": S, "num_q_heads": Hq,
           "num_kv_heads": wl.num_kv_heads, "head_size": D, "dtype": wl.dtype, "layout": wl.layout,
           "kv_cache": "fp8_e4m3 (per-kv-head scales)" if fp8 else wl.dtype,
           "effective_bytes_per_step": eff, "us_per_step": round(step_us, 2),
           "tokens_per_s": round(S / (step_us * 1e-6), 1),
           "decode_us": round(dec_us, 2), "reduce_us": round(red_us, 2) if ps else None,
           "call_us": round(call_us, 2),
           "decode_us_rounds": [round(x, 2) for x in dec_r], "call_us_rounds": [round(x, 2) for x in call_r],
           "call_gbs": round(eff / (call_us * 1e-6) / 1e9, 1),
           "call_frac": round(eff / (call_us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
           "decode_frac": round(eff / (dec_us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
           "timing": "call = decode (+ reduce) back to back, HIP events on the launch stream, mean of three "
                     "rounds alternating with the decode alone; reduce_us = call minus decode; step = wall clock "
                     "of write + plan + call", "pool_copies": copies}
    if wl.prefix_blocks:
        uniq = wl.unique_kv_bytes() + wl.qo_bytes()
        rec.update(unique_bytes_per_step=uniq, unique_call_gbs=round(uniq / (call_us * 1e-6) / 1e9, 1),
                   unique_call_frac=round(uniq / (call_us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4))
    g = measure_gather(torch, pc, wl, pools, inp, steps)
    if g is not None:
        # a plain gather of the tiles the decode reads (a shared block once per sequence
        # that addresses it, where the shared-prefix path reads it once per group)
        g["decode_us_over_gather_us"] = round(dec_us / g["us"], 3)
        rec["gather"] = g
    del pools
    torch.cuda.empty_cache()
    return rec


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}); the path runs per GPU with no "
              "exchange between GPUs, so run it with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import torch

    if args.calibrate_copy:
        n = args.calibrate_copy << 20
        src = torch.ones(n, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes_per_launch": n, "launches": 5}), flush=True)
        return

    if args.varlen:
        return bench_varlen(args)
    if args.plan_grid:
        return bench_plan_grid(args)

    import gpu_harness as gh
    import paged_kv_cache_reshape_amd as pc
    from workloads import alibi_variant, fp8_variant, make_config

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    print(f"[bench] generating workload {args.config}", file=sys.stderr, flush=True)
    wl = make_config(args.config, block_size=args.block_size)
    if args.kv == "fp8":
        wl = fp8_variant(wl)
    if args.alibi:
        wl = alibi_variant(wl)
    S, Hq, D = wl.q.shape
    per_copy = (2 if wl.layout != "combined" else 1) * wl.pool_elems * wl.kv_esize
    copies = args.copies or max(1, min(8, -(-(1 << 30) // max(1, wl.kv_bytes())) + 1))
    copies = max(1, min(copies, int(64e9 // per_copy)))
    print(f"[bench] {wl.name}: {wl.kv_bytes() / 1e6:.1f} MB K/V per step, {copies} pool copies", file=sys.stderr,
          flush=True)
    pools = []
    for _ in range(copies):
        pools.append(gh.filled_pool(wl, step_write=False))
    inp = gh.DecodeInputs(wl)
    key = gh.to_dev(wl.key, wl.dtype)
    value = gh.to_dev(wl.value, wl.dtype)
    slots = torch.from_numpy(wl.slot_mapping).to(dev)
    out = torch.empty_like(inp.q)
    msl = inp.max_seq_len
    if args.path == "plan":
        ps, P, _ = pc.paged_attention_plan_lens(wl.seq_lens, Hq, wl.num_kv_heads, D, wl.head_stride,
                                                gh.TORCH_DT[wl.dtype], kv_fp8=wl.fp8, shared_lens=wl.shared_lens())
    elif args.path == "split":
        ps, P = pc.PARTITION_SIZE, -(-msl // pc.PARTITION_SIZE)
    else:
        ps, P = 0, 1
    path = "split" if ps else "single"
    es = ml = tmp = None
    if ps:
        es = torch.empty((S, Hq, P), device=dev)
        ml = torch.empty((S, Hq, P), device=dev)
        tmp = torch.empty((S, Hq, P, D), device=dev)
    stream = torch.cuda.current_stream(dev)
    fp8 = wl.fp8
    split_kw = dict(partition_size=ps, exp_sums=es, max_logits=ml, tmp_out=tmp) if ps else {}
    # sequences sharing a prefix, on the split path: each shared tile read once for many
    use_prefix = bool(ps and wl.prefix_blocks and not fp8 and args.step == "separate" and not args.no_prefix_path)
    if use_prefix:
        prefix_kw = dict(prefix_table=torch.from_numpy(wl.prefix_table()).to(dev),
                         shared_lens=torch.from_numpy(wl.shared_lens()).to(dev))

    def write(pool):
        if fp8:
            pc.reshape_and_cache_fp8(key, value, pool.k, pool.v, slots, pool.k_scale, pool.v_scale,
                                     **pool.layout_kwargs(), **pool.scale_kwargs())
        else:
            pc.reshape_and_cache(key, value, pool.k, pool.v, slots, **pool.layout_kwargs())

    def decode(pool):
        o = None if ps else out
        if fp8:
            pc.paged_attention_decode_fp8(o, inp.q, pool.k, pool.v, inp.block_tables, inp.seq_lens, msl,
                                          pool.k_scale, pool.v_scale, num_kv_heads=wl.num_kv_heads,
                                          scale=float(wl.scale), alibi_slopes=inp.alibi, **pool.layout_kwargs(),
                                          **pool.scale_kwargs(), **split_kw)
        elif use_prefix:
            pc.paged_attention_decode_prefix(inp.q, pool.k, pool.v, inp.block_tables, inp.seq_lens, msl,
                                             num_kv_heads=wl.num_kv_heads, scale=float(wl.scale),
                                             alibi_slopes=inp.alibi, exp_sums=es, max_logits=ml, tmp_out=tmp,
                                             **prefix_kw, **pool.layout_kwargs())
        else:
            pc.paged_attention_decode(o, inp.q, pool.k, pool.v, inp.block_tables, inp.seq_lens, msl,
                                      num_kv_heads=wl.num_kv_heads, scale=float(wl.scale), alibi_slopes=inp.alibi,
                                      **pool.layout_kwargs(), **split_kw)

    # the fused step: 16-bit pools, one new token per sequence (token s = sequence s's
    # newest), and not 8-token blocks with 8 query heads per kv head at head size 128
    can_fuse = (not fp8 and wl.dtype in ("bf16", "f16") and len(wl.slot_mapping) == S and
                not (wl.block_size == 8 and Hq == 8 * wl.num_kv_heads and D == 128))
    fused = args.step == "fused"
    if fused and not can_fuse:
        raise SystemExit("--step fused: 16-bit pools and one new token per sequence only")

    def fused_step(pool):
        o = None if ps else out
        pc.reshape_and_cache_decode(o, inp.q, key, value, pool.k, pool.v, slots, inp.block_tables, inp.seq_lens, msl,
                                    num_kv_heads=wl.num_kv_heads, scale=float(wl.scale), alibi_slopes=inp.alibi,
                                    **pool.layout_kwargs(), **split_kw)

    def step(i, ev=None):
        pool = pools[i % copies]
        if not fused:
            write(pool)
        pc.paged_attention_plan_lens(wl.seq_lens, Hq, wl.num_kv_heads, D, wl.head_stride, gh.TORCH_DT[wl.dtype],
                                     kv_fp8=wl.fp8, shared_lens=wl.shared_lens())
        if ev is not None:
            ev[0].record(stream)
        if fused:
            fused_step(pool)
        else:
            decode(pool)
        if ev is not None:
            ev[1].record(stream)
        if ps:
            pc.paged_attention_reduce(out, es, ml, tmp, inp.seq_lens)
            if ev is not None:
                ev[2].record(stream)

    def timed(n, rotate=True):
        """Wall time of n whole steps (barrier-free: nothing but the steps is enqueued)."""
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(n):
            step(i if rotate else 0)
        torch.cuda.synchronize()
        return time.perf_counter() - t0

    def per_launch(n):
        """The same steps with an event pair around each decode (and reduce) launch."""
        evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(n)]
        torch.cuda.synchronize()
        for i in range(n):
            step(i, evs[i])
        torch.cuda.synchronize()
        dec = [e[0].elapsed_time(e[1]) for e in evs]
        red = [e[1].elapsed_time(e[2]) for e in evs] if ps else [0.0] * n
        return dec, red

    def decode_only(i):
        """The step's decode launch alone (with the step's write when that is fused)."""
        (fused_step if fused else decode)(pools[i % copies])

    def batched(fn, n):
        """Average launch time of n back-to-back launches, one event pair on the stream."""
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record(stream)
        for i in range(n):
            fn(i)
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / n

    for i in range(args.warmup):
        step(i)
    print(f"[bench] warmup done, timing {args.steps} steps ({path} path)", file=sys.stderr, flush=True)
    el = timed(args.steps)
    dec_b = batched(decode_only, args.steps)
    dec, red = per_launch(args.steps)
    for i in range(3):
        step(0)
    wel = timed(args.steps, rotate=False)
    wdec_b = batched(lambda i: decode_only(0), args.steps)
    # for reference: the decode launch without the fused write, back to back
    plain_b = batched(lambda i: decode(pools[i % copies]), args.steps) if fused else None

    eff = wl.effective_bytes()
    # the fused launch also reads and writes the step's K/V rows
    launch_bytes = eff + (4 * S * wl.num_kv_heads * D * wl.esize if fused else 0)
    ms = el / args.steps * 1e3
    dec_ms = sum(dec) / len(dec)
    red_ms = sum(red) / len(red)
    achieved = launch_bytes / (dec_b * 1e-3) / 1e9
    q = lambda xs, f: round(float(sorted(xs)[min(len(xs) - 1, int(f * len(xs)))]) * 1e3, 2)
    traffic = stored_traffic(wl.name + (" (fused step)" if fused else ""))
    res = {
        "metric": METRIC,
        "value": round(eff / (ms * 1e-3) / 1e9, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": wl.dtype,
        "data": "synthetic",
        "config": {"workload": wl.name, "num_seqs": S, "num_q_heads": Hq, "num_kv_heads": wl.num_kv_heads,
                   "head_size": D, "block_size": wl.block_size, "layout": wl.layout,
                   "path": path + (" (shared prefix)" if use_prefix else ""),
                   "step": "fused" if fused else "separate",
                   "kv_cache": "fp8_e4m3 (per-kv-head scales)" if fp8 else wl.dtype,
                   "alibi": bool(args.alibi),
                   "max_seq_len": msl, "kv_bytes_per_step": wl.kv_bytes(), "effective_bytes_per_step": eff,
                   "pool_copies": copies},
        "tokens_per_s": round(S / (ms * 1e-3), 1),
        "us_per_call": round(ms * 1e3, 2),
        "hbm_frac_step": round(eff / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
        "decode_kernel_us": round(dec_ms * 1e3, 2),
        "decode_kernel_us_p10_p50_p90": [q(dec, 0.1), q(dec, 0.5), q(dec, 0.9)],
        "decode_kernel_us_batched": round(dec_b * 1e3, 2),
        "reduce_kernel_us": round(red_ms * 1e3, 2) if ps else None,
        "unfused_decode_kernel_us_batched": round(plain_b * 1e3, 2) if fused else None,
        "roofline": {"bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic,
                     "kernel": ("decode_split_kernel + decode_prefix_kernel" if use_prefix else
                                "decode_split_kernel" if ps else "decode_onepass_kernel") +
                               (" (with the step's K/V write)" if fused else ""),
                     "bytes_per_launch": launch_bytes, "launch_us": round(dec_b * 1e3, 2),
                     "timing": "HIP events around back-to-back launches on the launch stream"},
        "warm_cache": {"ms_per_step": round(wel / args.steps * 1e3, 5),
                       "decode_kernel_us_batched": round(wdec_b * 1e3, 2),
                       "value": round(eff / (wel / args.steps) / 1e9, 2)},
    }
    if ps:
        res["decode_plus_reduce_us_batched"] = round(batched(lambda i: (decode(pools[i % copies]), pc.paged_attention_reduce(
            out, es, ml, tmp, inp.seq_lens)), args.steps) * 1e3, 2)
        # the reduce's share of the pair (launched alone back to back, reduces of a few
        # microseconds wait on the host's launch rate instead)
        res["reduce_added_us_batched"] = round(res["decode_plus_reduce_us_batched"] - dec_b * 1e3, 2)
    if wl.prefix_blocks:
        uniq = wl.unique_kv_bytes() + wl.qo_bytes()
        res["config"]["unique_bytes_per_step"] = uniq
        res["unique_bytes"] = {"gbs_step": round(uniq / (ms * 1e-3) / 1e9, 2),
                               "gbs_decode_launch": round(uniq / (dec_b * 1e-3) / 1e9, 2),
                               "frac_decode_launch": round(uniq / (dec_b * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                               "note": "distinct physical K/V rows read (the shared prefix once) plus q and out"}
    print("[bench] gather yardstick", file=sys.stderr, flush=True)
    g = measure_gather(torch, pc, wl, pools, inp, args.steps)
    if g is not None:
        # the same algorithmic bytes over a plain gather's launch time: above 1 in
        # frac_of_measured_gather, the decode reads its tiles faster than a loads-only gather
        res["gather_read"] = g
        res["roofline"]["measured_gather"] = round(launch_bytes / (g["us"] * 1e-6) / 1e9, 1)
        res["roofline"]["frac_of_measured_gather"] = round(g["us"] / (dec_b * 1e3), 4)
    del pools
    torch.cuda.empty_cache()
    if args.read_peak_gib > 0:
        print("[bench] streaming-read yardstick", file=sys.stderr, flush=True)
        rp = measure_read_peak(torch, pc, args.read_peak_gib)
        res["roofline"]["measured_read_peak"] = rp["gbs"]
        res["roofline"]["frac_of_measured_read_peak"] = round(achieved / rp["gbs"], 4)
        res["read_peak"] = rp
    others = [int(x) for x in args.other_configs.split(",") if x.strip() != "" and int(x) != args.config]
    paths = [x.strip() for x in args.other_paths.split(",") if x.strip()]
    for p in paths:
        if not (p in ("spec", "prefill") or (p.startswith("fp8:") and p[4:].isdigit())):
            raise SystemExit(f"--other-paths: unknown path {p!r}")
    jobs = [("other_configs", str(i)) for i in others] + [("other_paths", p) for p in paths]
    # Long-context workload 3 first: its random 4 KiB tiles over a 1 GiB pool read 2-3%
    # slower once the process has allocated and freed workload 2's 10 GiB of pools; measured
    # first, it runs as in a process of its own.
    jobs.sort(key=lambda j: 0 if j[1] in ("3", "fp8:3") else 1)
    for group, key in jobs:
        if group == "other_configs":
            rec = measure_config(int(key), args.steps, args.warmup, args.no_prefix_path)
        elif key.startswith("fp8:"):
            rec = measure_config(int(key[4:]), args.steps, args.warmup, kv="fp8")
        else:
            rec = varlen_record(key, args.steps, args.warmup)
        res.setdefault(group, {})[key] = rec
    for group, keys in (("other_configs", [str(i) for i in others]), ("other_paths", paths)):
        if group in res:  # reported in the order asked for
            res[group] = {k: res[group][k] for k in keys}
    if not args.no_cpu_baseline:
        print("[bench] timing the CPU oracle", file=sys.stderr, flush=True)
        res["cpu_baseline"] = cpu_baseline(wl, args.cpu_seconds)
    print(json.dumps(res), flush=True)


def varlen_flops(wl, vq) -> int:
    """Algorithmic FLOPs of the multi-token attention: per (query row, head, visible
    token) one D-long multiply-add for q.k and one for P.V."""
    total = 0
    qs = vq.query_start_loc
    for r in range(wl.num_seqs):
        L, n = int(wl.seq_lens[r]), int(qs[r + 1] - qs[r])
        vis = sum(L - n + i + 1 for i in range(n)) if vq.causal else n * L
        total += vis
    return total * wl.num_q_heads * wl.head_size * 4


def measure_varlen(kind: str, steps: int, warmup: int, copies: int = 0):
    """A multi-token step (``kind`` 'prefill' or 'spec'): the write of every request's new
    rows, then the causal attention of those rows over the whole paged history; the
    step by wall clock, the attention alone by HIP events around back-to-back launches
    (pool copies rotating).  Returns (workload, step, seconds per step, ms per launch,
    pool copies)."""
    import torch
    import gpu_harness as gh
    import paged_kv_cache_reshape_amd as pc
    from workloads import varlen_config

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    print(f"[bench] generating varlen workload {kind}", file=sys.stderr, flush=True)
    wl, vq = varlen_config(kind)
    per_copy = 2 * wl.pool_elems * wl.esize
    copies = copies or max(1, min(8, -(-(1 << 30) // max(1, wl.kv_bytes())) + 1))
    copies = max(1, min(copies, int(64e9 // per_copy)))
    pools = [gh.filled_pool(wl) for _ in range(copies)]
    q = gh.to_dev(vq.q, wl.dtype)
    out = torch.empty_like(q)
    key, value = gh.to_dev(vq.key, wl.dtype), gh.to_dev(vq.value, wl.dtype)
    slots = torch.from_numpy(vq.slot_mapping).to(dev)
    qs = torch.from_numpy(vq.query_start_loc).to(dev)
    sl = torch.from_numpy(wl.seq_lens).to(dev)
    bt = torch.from_numpy(wl.block_tables).to(dev)
    stream = torch.cuda.current_stream(dev)

    def attend(i):
        pool = pools[i % copies]
        pc.paged_attention_varlen(out, q, pool.k, pool.v, bt, qs, sl, vq.max_query_len,
                                  num_kv_heads=wl.num_kv_heads, scale=float(wl.scale), causal=vq.causal,
                                  **pool.layout_kwargs())

    def step(i):
        pool = pools[i % copies]
        pc.reshape_and_cache(key, value, pool.k, pool.v, slots, **pool.layout_kwargs())
        attend(i)

    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        step(i)
    torch.cuda.synchronize()
    el = time.perf_counter() - t0
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(stream)
    for i in range(steps):
        attend(i)
    e1.record(stream)
    torch.cuda.synchronize()
    kern_ms = e0.elapsed_time(e1) / steps
    del pools
    torch.cuda.empty_cache()
    return wl, vq, el / steps, kern_ms, copies


def varlen_record(kind: str, steps: int, warmup: int):
    """The compact record of a multi-token step reported beside the headline line."""
    wl, vq, step_s, kern_ms, copies = measure_varlen(kind, steps, warmup)
    kv = wl.kv_bytes()
    qo = vq.total_q * wl.num_q_heads * wl.head_size * 2 * wl.esize
    rec = {"workload": wl.name, "kernel": "varlen_lds_kernel" if kind == "prefill" else
           "decode_onepass_kernel (16 query columns)", "query_tokens": vq.total_q,
           "us_per_step": round(step_s * 1e6, 2), "tokens_per_s": round(vq.total_q / step_s, 1),
           "attention_us": round(kern_ms * 1e3, 2), "pool_copies": copies,
           "timing": "attention_us: HIP events around back-to-back launches on the launch stream; "
                     "step = wall clock of write + attention"}
    if kind == "prefill":
        tf = varlen_flops(wl, vq) / (kern_ms * 1e-3) / 1e12
        rec.update(bound="mfma", tflops=round(tf, 2), frac=round(tf / 2500.0, 4))
    else:
        gbs = (kv + qo) / (kern_ms * 1e-3) / 1e9
        rec.update(bound="hbm", gbs=round(gbs, 1), frac=round(gbs / HBM_PEAK_GBS, 4))
    return rec


def bench_varlen(args):
    """Multi-token step: the write of every request's new rows, then the causal
    attention of those rows over the whole paged history."""
    wl, vq, step_s, kern_ms, copies = measure_varlen(args.varlen, args.steps, args.warmup, args.copies)
    flops = varlen_flops(wl, vq)
    kv = wl.kv_bytes()
    qo = vq.total_q * wl.num_q_heads * wl.head_size * 2 * wl.esize
    ms = step_s * 1e3
    toks = vq.total_q / (ms * 1e-3)
    if args.varlen == "prefill":
        metric, unit, value = "varlen chunked-prefill attention query tokens/s", "tokens/s", toks
        achieved = flops / (kern_ms * 1e-3) / 1e12
        roof = {"bound": "mfma", "achieved": round(achieved, 2), "peak": 2500.0, "unit": "TFLOP/s",
                "frac": round(achieved / 2500.0, 4), "traffic": stored_traffic(wl.name, "varlen"),
                "kernel": "varlen_lds_kernel",
                "flops_per_launch": flops, "launch_us": round(kern_ms * 1e3, 2)}
    else:
        metric, unit, value = "varlen speculative-decode attention effective GB/s", "GB/s", (kv + qo) / (ms * 1e-3) / 1e9
        achieved = (kv + qo) / (kern_ms * 1e-3) / 1e9
        roof = {"bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": stored_traffic(wl.name, "varlen"),
                "kernel": "decode_onepass_kernel (16 query columns)",
                "bytes_per_launch": kv + qo, "launch_us": round(kern_ms * 1e3, 2)}
    roof["timing"] = "HIP events around back-to-back launches on the launch stream"
    res = {"metric": metric, "value": round(value, 2), "unit": unit, "n_gpus": 1, "steps": args.steps,
           "warmup": args.warmup, "ms_per_step": round(ms, 5), "higher_is_better": True, "scaling": "weak",
           "vs_baseline": None, "dtype": wl.dtype, "data": "synthetic",
           "config": {"workload": wl.name, "num_reqs": wl.num_seqs, "query_tokens": vq.total_q,
                      "query_len": vq.max_query_len, "num_q_heads": wl.num_q_heads,
                      "num_kv_heads": wl.num_kv_heads, "head_size": wl.head_size, "causal": vq.causal,
                      "kv_bytes_per_step": kv, "attention_flops_per_step": flops, "pool_copies": copies},
           "tokens_per_s": round(toks, 1), "varlen_kernel_us_batched": round(kern_ms * 1e3, 2),
           "roofline": roof}
    if not args.no_cpu_baseline:
        import oracle
        print("[bench] timing the CPU oracle", file=sys.stderr, flush=True)
        threads = min(host_cpus()[1], 16)
        pool = oracle.filled_pool(wl)
        # a bounded sample: the first requests' query rows (the others get empty ranges)
        k = 1 if args.varlen == "prefill" else wl.num_seqs
        qs_h = vq.query_start_loc.copy()
        qs_h[k + 1:] = qs_h[k]
        rows = int(qs_h[k])
        reps, t0 = 0, time.perf_counter()
        while True:
            oracle.varlen(wl, pool, vq, q=vq.q[:rows], query_start_loc=qs_h, nthreads=threads)
            reps += 1
            el_c = time.perf_counter() - t0
            if el_c >= args.cpu_seconds or reps >= 1000:
                break
        res["cpu_baseline"] = {"value": round(reps * rows / el_c, 3), "unit": "tokens/s", "cores": threads,
                               "kind": "oracle",
                               "sample": f"{reps} x fp64 attention of the query rows of the first {k} request(s) "
                                         f"({rows} rows each) in {el_c:.1f} s on {threads} host threads"}
    print(json.dumps(res), flush=True)


# --plan-grid: units (= num_seqs * num_kv_heads), longest lengths and length mixes of the grid
GRID_UNITS = (32, 64, 128, 256, 512, 1024, 2048, 4096, 8192)
GRID_MAX_LEN = (512, 2048, 8192, 32768)
GRID_MIXES = ("fixed", "uniform", "loguniform")


def grid_lengths(S: int, max_len: int, mix: str, num_kv_heads: int = 0):
    """Sequence lengths of one grid shape: all max_len; uniform on [1, max_len]; or
    floor(exp(U[ln 16, ln(max_len + 1)))) -- each mix with its longest at max_len.  Each
    shape draws from its own seed, so a shape's lengths do not depend on the others."""
    import numpy as np
    key = f"{S}/{num_kv_heads}/{max_len}/{mix}".encode()
    rng = np.random.Generator(np.random.PCG64(int.from_bytes(key, "little") % (1 << 63)))
    if mix == "fixed":
        L = np.full(S, max_len)
    elif mix == "uniform":
        L = rng.integers(1, max_len + 1, S)
    else:
        L = np.floor(np.exp(rng.uniform(np.log(16), np.log(max_len + 1), S))).astype(np.int64)
    L[0] = max_len
    return np.clip(L, 1, max_len).astype(np.int32)


def grid_shared_lens(lens, prefix_tokens, block_size=16):
    """Per sequence of a --plan-grid batch: the leading tokens read from the shared prefix's
    blocks (every sequence's last block is its own)."""
    import numpy as np
    nb = -(-np.asarray(lens, np.int64) // block_size)
    return (np.minimum(prefix_tokens // block_size, np.maximum(nb - 1, 0)) * block_size).astype(np.int32)


def bench_plan_grid(args):
    """Both decode paths on synthetic batches: the pool is random bf16, each sequence's blocks
    a random draw from it; several table sets over disjoint blocks rotate so that no launch
    finds the previous one's K/V in cache.  Times are HIP events around back-to-back
    launches: the one-pass decode, and the split decode with its reduce."""
    import numpy as np
    import torch
    import paged_kv_cache_reshape_amd as pc

    torch.cuda.set_device(0)
    D, B, dt = 128, 16, torch.bfloat16
    stream = torch.cuda.current_stream()
    units_list = [int(x) for x in args.grid_units.split(",")] if args.grid_units else GRID_UNITS
    len_list = [int(x) for x in args.grid_max_len.split(",")] if args.grid_max_len else GRID_MAX_LEN
    mix_list = args.grid_mixes.split(",") if args.grid_mixes else GRID_MIXES

    def batched(fn, n):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record(stream)
        for i in range(n):
            fn(i)
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / n * 1e3

    heads = [tuple(int(x) for x in hh.split("/")) for hh in args.grid_heads.split(",") if hh]
    for Hq, Hkv in heads:
        for units in units_list:
            S = units // Hkv
            if S < 1:
                continue
            for max_len in len_list:
                for mix in mix_list:
                    L = grid_lengths(S, max_len, mix, Hkv)
                    nb = -(-L // B)
                    kv = int(L.astype(np.int64).sum()) * Hkv * D * 2 * 2
                    if kv > args.grid_max_gib * (1 << 30):
                        continue
                    sets = max(1, min(8, -(-(2 << 30) // kv)))
                    need = int(nb.sum())
                    blocks = need * sets
                    elems = blocks * Hkv * B * D
                    k_pool = torch.randn(elems, dtype=dt, device="cuda")
                    v_pool = torch.randn(elems, dtype=dt, device="cuda")
                    perm = torch.randperm(blocks, dtype=torch.int32)
                    W = int(nb.max())
                    tables = []
                    shb = grid_shared_lens(L, args.grid_prefix, B) // B  # shared prefix blocks per sequence
                    for c in range(sets):
                        t = torch.full((S, W), -1, dtype=torch.int32)
                        off = c * need
                        for si in range(S):
                            t[si, :nb[si]] = perm[off:off + nb[si]]
                            sh = int(shb[si])
                            if sh > 0:  # the blocks of set c's first sequence serve as the prefix
                                t[si, :sh] = perm[c * need:c * need + sh]
                            off += int(nb[si])
                        tables.append(t.cuda())
                    sl = torch.from_numpy(L).cuda()
                    q = torch.randn(S, Hq, D, dtype=dt, device="cuda")
                    out = torch.empty_like(q)
                    P = -(-max_len // pc.PARTITION_SIZE)
                    es = torch.empty((S, Hq, P), device="cuda")
                    ml = torch.empty_like(es)
                    tmp = torch.empty((S, Hq, P, D), device="cuda")
                    lay = dict(num_kv_heads=Hkv, scale=D ** -0.5, num_blocks=blocks, block_stride=Hkv * B * D,
                               token_stride=D, head_stride=B * D, block_size=B)

                    def single(i):
                        pc.paged_attention_decode(out, q, k_pool, v_pool, tables[i % sets], sl, max_len, **lay)

                    if args.grid_prefix:  # the split path given the sharing: each shared tile read once
                        shl = torch.from_numpy(grid_shared_lens(L, args.grid_prefix, B)).cuda()
                        pts = [t[int(np.argmax(shb)), :int(shb.max())].contiguous() for t in tables]

                    def split(i):
                        if args.grid_prefix:
                            pc.paged_attention_decode_prefix(q, k_pool, v_pool, tables[i % sets], sl, max_len,
                                                             exp_sums=es, max_logits=ml, tmp_out=tmp,
                                                             prefix_table=pts[i % sets], shared_lens=shl, **lay)
                        else:
                            pc.paged_attention_decode(None, q, k_pool, v_pool, tables[i % sets], sl, max_len,
                                                      partition_size=pc.PARTITION_SIZE, exp_sums=es, max_logits=ml,
                                                      tmp_out=tmp, **lay)
                        pc.paged_attention_reduce(out, es, ml, tmp, sl)

                    n = max(3, min(30, int(5000 // max(1, kv >> 20))))  # about 5 GB read per path
                    for fn in (single, split):
                        fn(0)
                    t1 = batched(single, n)
                    t2 = batched(split, n)
                    ps, _, _ = pc.paged_attention_plan_lens(L, Hq, Hkv, D, B * D, dt,
                                                            shared_lens=grid_shared_lens(L, args.grid_prefix, B))
                    print(json.dumps({"num_q_heads": Hq, "num_kv_heads": Hkv, "head_size": D, "num_seqs": S,
                                      "units": units, "max_len": max_len, "mix": mix,
                                      "mean_len": round(float(L.mean()), 1), "kv_bytes": kv,
                                      "prefix": args.grid_prefix,
                                      "single_us": round(t1, 2), "split_us": round(t2, 2),
                                      "faster": "single" if t1 <= t2 else "split",
                                      "plan": "split" if ps else "single", "launches": n}), flush=True)
                    del k_pool, v_pool, tables, es, ml, tmp
                    torch.cuda.empty_cache()


if __name__ == "__main__":
    main()
