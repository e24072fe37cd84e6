#!/usr/bin/env python3
"""Benchmark: paged-KV decode step (store + decode attention) on one GPU.

Workload (default): the Mistral-7B-style GQA batch -- 32 sequences x 4096
cached tokens, 32 query / 8 KV heads, head_dim 128, bf16, 16-token blocks,
32 independent layer pools (16 GiB of KV).  One step = for each of the 32
layers: store the new token of every sequence (slot mapping), then decode
attention over the whole cache including it -- one pkv_store_decode_attn
launch per layer (``--separate``: pkv_store then pkv_decode_attn).  Inputs are
synthetic N(0,1) values rounded to bf16 and a seeded random physical-block
permutation, resident in HBM before the timed region.

Prints ONE JSON line.  ``value`` is the step's algorithmic KV-cache traffic
(decode reads plus the store's reads and writes, all layers) / step time, in
GB/s.  ``roofline`` is the per-layer launch: its algorithmic bytes over its
average duration in the timed region (HIP events on the stream the launches
run on; the region holds nothing else), with an event-bracketed pass beside
it.  The chunked-prefill leg and the fp64 oracle on the host
cores are reported beside it.
"""
from __future__ import annotations

import argparse
import json
import os
import subprocess
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, vendor figure
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--layers", type=int, default=32)
    ap.add_argument("--partition-tokens", type=int, default=0)
    ap.add_argument("--separate", action="store_true",
                    help="time pkv_store + pkv_decode_attn as two launches per layer instead of "
                         "the fused pkv_store_decode_attn")
    ap.add_argument("--seed", type=int, default=3)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="target CPU time of the oracle baseline sample")
    ap.add_argument("--no-prefill", action="store_true")
    ap.add_argument("--no-fp8", action="store_true",
                    help="skip the FP8-cache leg of the decode workload")
    ap.add_argument("--no-other", action="store_true",
                    help="skip the Qwen-style MHA and continuous-batch decode workloads")
    ap.add_argument("--no-mixed", action="store_true",
                    help="skip the mixed decode + prefill iteration")
    ap.add_argument("--no-pool", action="store_true",
                    help="skip the block-pool bookkeeping and block-copy leg")
    ap.add_argument("--no-rope", action="store_true",
                    help="skip the step with the rotary embedding fused in")
    ap.add_argument("--prefill-iters", type=int, default=5)
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 1 GiB device copy (for scaling HBM byte counters)")
    return ap.parse_args()


def copy_calibration():
    """A plain device-to-device copy of exactly 1 GiB, three times: the
    reference reading for the FETCH_SIZE / WRITE_SIZE counters."""
    import torch

    n = 1 << 30
    src = torch.empty(n, dtype=torch.uint8, device="cuda")
    src.fill_(1)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes": n, "copies": 3}), flush=True)


def decode_bytes(wl) -> int:
    """Algorithmic bytes one decode launch must move: every cached K and V
    element once, q in, out back, the live block-table entries and lengths."""
    ctx = wl.context_lens.astype(np.int64)
    kv = int(ctx.sum()) * 2 * wl.num_kv_heads * wl.head_dim * 2
    qo = 2 * wl.num_seqs * wl.num_q_heads * wl.head_dim * 2
    table = 4 * int(((ctx + wl.block_size - 1) // wl.block_size).sum()) + 4 * wl.num_seqs
    return kv + qo + table


def store_bytes(wl) -> int:
    """Store: read and write each new token's K and V, plus its slot."""
    live = int((wl.slot_mapping >= 0).sum())
    return live * (2 * 2 * wl.num_kv_heads * wl.head_dim * 2) + 4 * wl.num_tokens


def prefill_flops(wl) -> float:
    """Causal pairs only: query i of prompt p sees c_p + i + 1 keys; 4 d flops
    per (query head, key) pair (Q K^T and P V)."""
    tot = 0
    for p in range(wl.num_seqs):
        n = int(wl.new_lens[p])
        c = int(wl.context_lens[p]) - n
        tot += n * c + n * (n + 1) // 2
    return 4.0 * wl.head_dim * wl.num_q_heads * tot


def launch_stats(durations_ms):
    """Per-launch HIP-event durations -> (average, stats dict).  The average
    is the mean of the central 90% of launches, so one launch stalled by
    something outside the kernel cannot move it; the plain mean and the
    median are reported beside it."""
    x = np.sort(np.asarray(durations_ms, dtype=np.float64))
    k = int(len(x) * 0.05)
    core = x[k:len(x) - k] if len(x) > 2 * k else x
    avg = float(core.mean())
    return avg, {"launches": int(len(x)), "trimmed_mean_us": round(avg * 1e3, 2),
                 "mean_us": round(float(x.mean()) * 1e3, 2),
                 "median_us": round(float(np.median(x)) * 1e3, 2)}


def recorded_traffic(kernel: str):
    """HBM bytes per launch of ``kernel`` as measured by rocprofv3 FETCH_SIZE /
    WRITE_SIZE passes (scaled by a plain-copy calibration) and recorded in a
    ``traffic_record:`` line of a summary under profiles/.  The record lists
    the sha256 of the kernel's source files when the counters were taken; if
    any of them has changed since, the figure no longer describes this kernel
    and None is returned."""
    import glob
    import hashlib

    for path in sorted(glob.glob(os.path.join(ROOT, "profiles", "*.md"))):
        for line in open(path, encoding="utf-8"):
            if not line.startswith("traffic_record:"):
                continue
            rec = json.loads(line.split(":", 1)[1])
            if rec.get("kernel") != kernel:
                continue
            same = all(
                os.path.exists(os.path.join(ROOT, f)) and hashlib.sha256(
                    open(os.path.join(ROOT, f), "rb").read()).hexdigest() == h
                for f, h in rec["sources"].items())
            return int(rec["bytes_per_launch"]) if same else None
    return None


def cpu_baseline(wl, t, seconds):
    """Time the fp64 oracle (as it stands) on whole layers of the same workload.

    Host copies of two layers' pools are taken once (outside the timing); each
    timed unit is one layer's store + decode over all sequences, alternating
    between the two copies.  The store rewrites the same slots with the same
    bits, so every repetition does identical work.  Repeats until about
    ``seconds`` of wall time inside the oracle; tokens/s per layer =
    sequences / time per layer."""
    import oracle
    from paged_kv_cache_pools_amd import workloads as W

    orc = oracle.get()
    threads = orc.default_threads()
    q = W.bf16_bits(t["q"][0])
    kn = W.bf16_bits(t["k_new"][0])
    vn = W.bf16_bits(t["v_new"][0])
    pools = [(W.bf16_bits(k).copy(), W.bf16_bits(v).copy())
             for k, v in zip(t["k_caches"], t["v_caches"])]
    layers_done, spent = 0, 0.0
    while spent < seconds and layers_done < 4096:
        kc, vc = pools[layers_done % len(pools)]
        t0 = time.perf_counter()
        orc.store(kn, vn, wl.slot_mapping, kc, vc)
        orc.decode(q, kc, vc, wl.block_tables, wl.context_lens, wl.scale, nthreads=threads)
        spent += time.perf_counter() - t0
        layers_done += 1
    per_layer = spent / layers_done
    # the same layer's decode on one thread
    kc, vc = pools[0]
    t0 = time.perf_counter()
    orc.decode(q, kc, vc, wl.block_tables, wl.context_lens, wl.scale, nthreads=1)
    one_thread = time.perf_counter() - t0
    return {
        "value": wl.num_seqs / per_layer, "unit": "tokens/s per layer", "cores": threads,
        "kind": "oracle",
        "sample": f"{layers_done} layer(s) of the same batch (store + decode of all "
                  f"{wl.num_seqs} seqs x {wl.max_context_len} tokens, alternating two layer "
                  f"pools), fp64 C oracle on {threads} threads, {per_layer * 1e3:.1f} ms per "
                  f"layer, {spent:.1f} s in total",
        "kv_gbs": decode_bytes(wl) / per_layer / 1e9,
        "one_thread": {"tokens_per_s_per_layer": round(wl.num_seqs / one_thread, 1),
                       "ms_per_layer": round(one_thread * 1e3, 1)},
        "host": {"cpu_model": cpu_model(), "nproc": os.cpu_count()},
        "prefill": cpu_prefill_sample(orc, threads),
    }


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def cpu_prefill_sample(orc, threads, cached=2048, new=128):
    """The oracle's chunked prefill on a bounded sample shaped like one prompt
    of the 8 x 2048 workload: 2048 cached + 128 new tokens, 32 query / 8 KV
    heads, d 128 (seeded N(0,1) bf16 on the host), on all threads; the rate
    in fp64 GFLOP/s of causal pairs and the time it implies for the whole
    8 x 2048 launch (859.53 GFLOP)."""
    import torch

    g = torch.Generator().manual_seed(5)
    hq, hkv, d = 32, 8, 128
    nb = (cached + new + 15) // 16

    def bits(*shape):
        x = torch.randn(*shape, generator=g).to(torch.bfloat16)
        return x.view(torch.int16).numpy().view(np.uint16)

    kc, vc, q = bits(nb, hkv, 16, d), bits(nb, hkv, 16, d), bits(new, hq, d)
    bt = np.arange(nb, dtype=np.int32)[None]
    cu = np.array([0, new], np.int32)
    ctx = np.array([cached + new], np.int32)
    t0 = time.perf_counter()
    orc.prefill(q, kc, vc, bt, cu, ctx, 1.0 / np.sqrt(d), nthreads=threads)
    dt = time.perf_counter() - t0
    flops = 4.0 * d * hq * (new * cached + new * (new + 1) / 2)
    rate = flops / dt
    return {"sample": f"1 prompt: {cached} cached + {new} new tokens, 32q/8kv, d 128, "
                      f"{threads} threads", "seconds": round(dt, 3),
            "gflops": round(rate / 1e9, 2), "implied_ms_8x2048": round(859.53e9 / rate * 1e3, 1)}


def main():
    args = parse()
    if args.copy_calibration:
        copy_calibration()
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the path has no multi-GPU component)", file=sys.stderr)
        sys.exit(2)
    import torch

    from paged_kv_cache_pools_amd import binding as B
    from paged_kv_cache_pools_amd import workloads as W

    B.load()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    L = args.layers
    wl = W.mistral_gqa(seed=args.seed, num_layers=L)
    gen = torch.Generator(device=dev)
    gen.manual_seed(wl.seed)

    def randn_bf16(shape):
        return W._randn_bf16(torch, shape, gen, dev)

    S, Hq, Hkv, D = wl.num_seqs, wl.num_q_heads, wl.num_kv_heads, wl.head_dim
    # Each layer's cache is one allocation [2][blocks][Hkv][16][d], K then V,
    # as serving engines lay out a layer's KV cache.  Where the V pool sits
    # relative to the K pool changes the step time by the HBM channels their
    # blocks map to: V right after K 85.2 us per launch, V 2 MiB further on
    # 87.7 us, all K pools allocated before all V pools 87.4 us (steady state,
    # one box, these 32 x 4096 pools).
    layer_kv = [randn_bf16((2, wl.num_blocks, Hkv, 16, D)) for _ in range(L)]
    t = {
        "q": [randn_bf16((S, Hq, D)) for _ in range(L)],
        "k_new": [randn_bf16((S, Hkv, D)) for _ in range(L)],
        "v_new": [randn_bf16((S, Hkv, D)) for _ in range(L)],
        "k_caches": [kv[0] for kv in layer_kv],
        "v_caches": [kv[1] for kv in layer_kv],
    }
    bt = torch.from_numpy(wl.block_tables).to(dev)
    ctx = torch.from_numpy(wl.context_lens).to(dev)
    slots = torch.from_numpy(wl.slot_mapping).to(dev)
    outs = [torch.empty((S, Hq, D), dtype=torch.bfloat16, device=dev) for _ in range(L)]
    P = args.partition_tokens or B.pkv_decode_partition_tokens(S, Hkv, wl.max_context_len)
    ws = torch.empty(max(16, B.pkv_decode_workspace_bytes(S, Hq, D, wl.max_context_len, P)),
                     dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream(dev)

    def launch(l):
        if args.separate:
            B.pkv_store(t["k_new"][l], t["v_new"][l], slots, t["k_caches"][l], t["v_caches"][l])
            B.pkv_decode_attn(t["q"][l], t["k_caches"][l], t["v_caches"][l], bt, ctx, wl.scale,
                              outs[l], max_context_len=wl.max_context_len, workspace=ws,
                              partition_tokens=P)
        else:
            B.pkv_store_decode_attn(t["k_new"][l], t["v_new"][l], slots, t["q"][l],
                                    t["k_caches"][l], t["v_caches"][l], bt, ctx, wl.scale,
                                    outs[l], max_context_len=wl.max_context_len, workspace=ws,
                                    partition_tokens=P)

    def step():
        for l in range(L):
            launch(l)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    # (1) the timed region: K steps, nothing but the launches between the two
    # events (a HIP event pair around every launch costs several us of GPU
    # time per layer, so per-launch timing has a pass of its own below)
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    wall0 = time.perf_counter()
    start.record(stream)
    for _ in range(args.steps):
        step()
    end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    total_ms = start.elapsed_time(end)
    ms_per_step = total_ms / args.steps

    # (2) per-launch durations for the roofline: the same K steps again, each
    # layer's launch(es) bracketed by HIP events on the stream they run on
    pairs = []
    for _ in range(args.steps):
        for l in range(L):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            if args.separate:  # time the decode launch only
                B.pkv_store(t["k_new"][l], t["v_new"][l], slots, t["k_caches"][l],
                            t["v_caches"][l])
                a.record(stream)
                B.pkv_decode_attn(t["q"][l], t["k_caches"][l], t["v_caches"][l], bt, ctx,
                                  wl.scale, outs[l], max_context_len=wl.max_context_len,
                                  workspace=ws, partition_tokens=P)
            else:
                a.record(stream)
                launch(l)
            b.record(stream)
            pairs.append((a, b))
    torch.cuda.synchronize()
    per_launch = [a.elapsed_time(b) for a, b in pairs]
    dec_avg_ms, dec_stats = launch_stats(per_launch)

    # (3) the same step with the rotary embedding fused in (q and the new k
    # rotated at position ctx - 1 by an fp32 cos/sin table of 4096 x 128)
    rope = None
    if not args.no_rope and not args.separate:
        table = torch.from_numpy(W.rope_table(wl.max_context_len, D)).to(dev)

        def rope_step():
            for l in range(L):
                B.pkv_store_decode_attn_rope(t["k_new"][l], t["v_new"][l], slots, t["q"][l],
                                             table, t["k_caches"][l], t["v_caches"][l], bt, ctx,
                                             wl.scale, outs[l], max_context_len=wl.max_context_len,
                                             workspace=ws, partition_tokens=P)

        for _ in range(args.warmup):
            rope_step()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for _ in range(args.steps):
            rope_step()
        b.record(stream)
        torch.cuda.synchronize()
        rope_ms = a.elapsed_time(b) / args.steps
        rope = {"launch": "pkv_store_decode_attn_rope", "ms_per_step": round(rope_ms, 4),
                "tokens_per_s_per_layer": round(S * L / (rope_ms * 1e-3), 1),
                "GB_s": round(L * (decode_bytes(wl) + store_bytes(wl)) / (rope_ms * 1e-3) / 1e9,
                              2),
                "step_time_vs_plain": round(rope_ms / ms_per_step, 4)}

    dbytes = decode_bytes(wl)
    sbytes = store_bytes(wl)
    kv_bytes_step = L * (dbytes + sbytes)
    value = kv_bytes_step / (ms_per_step * 1e-3) / 1e9
    # the timed launch per layer: decode alone, or the fused store + decode
    launch_bytes = dbytes if args.separate else dbytes + sbytes
    # The roofline's launch duration: the timed region holds nothing but the
    # K x L fused launches, so its length over K x L is their average duration
    # (dispatch gaps between launches included).  With --separate the region
    # also holds the store launches, and the event-bracketed decode launches
    # of pass (2) give the duration instead.
    launch_ms = dec_avg_ms if args.separate else ms_per_step / L
    achieved = launch_bytes / (launch_ms * 1e-3) / 1e9
    launch_timing = {"source": ("events around each decode launch (pass 2)" if args.separate
                                else "timed region / launches"),
                     "timed_region_us_per_launch": round(ms_per_step / L * 1e3, 2),
                     "event_bracketed": dec_stats}
    kernel = (f"decode_fused_kernel<{D},{Hq // Hkv}>" if P < 0
              else f"decode_split_kernel<{D},{Hq // Hkv}>+decode_reduce_kernel<{D}>")
    if not args.separate:
        kernel += " (fused store)"
    result = {
        "metric": "decode attention KV GB/s and % of MI355X HBM peak; tokens/s per layer",
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic N(0,1) bf16, seeded random physical-block permutation",
        "config": {"workload": "Mistral-7B-style GQA decode: 32 seqs x 4096 tokens, 32q/8kv "
                               "heads, d 128, 16-token blocks, 32 layer pools, store + decode",
                   "num_seqs": S, "context_len": int(wl.max_context_len), "num_q_heads": Hq,
                   "num_kv_heads": Hkv, "head_dim": D, "block_size": 16, "layers": L,
                   "work_split": (f"single pass, {-P} waves per (seq, kv head)" if P < 0
                                  else f"split-KV, {P}-token partitions + merge"),
                   "launches_per_layer": ("pkv_store + pkv_decode_attn" if args.separate
                                          else "pkv_store_decode_attn (store fused)")},
        "hbm_peak_frac": round(value / HBM_PEAK_GBS, 4),
        "tokens_per_s_per_layer": round(S * L / (ms_per_step * 1e-3), 1),
        "decode_us_per_layer": round(launch_ms * 1e3, 2),  # the timed launch (see kernel)
        "roofline": {"bound": "hbm", "kernel": kernel,
                     "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": recorded_traffic(kernel),
                     "algorithmic_bytes_per_launch": launch_bytes,
                     "launch_us": round(launch_ms * 1e3, 2), "launch_timing": launch_timing},
        "wall_s_timed": round(wall, 3),
    }
    if rope is not None:
        result["rope"] = rope

    # the oracle's host copies of two layers are taken before the 16 GiB of
    # pools are released for the other legs
    host = None
    if not args.no_cpu_baseline:
        host = {"q": [t["q"][0].cpu()], "k_new": [t["k_new"][0].cpu()],
                "v_new": [t["v_new"][0].cpu()],
                "k_caches": [x.cpu() for x in t["k_caches"][:2]],
                "v_caches": [x.cpu() for x in t["v_caches"][:2]]}
    del t
    torch.cuda.empty_cache()
    probe = bench_read_probe(torch, B, dev)
    result["read_probe"] = probe
    result["roofline"]["measured_read_gbs"] = probe["gbs"]
    result["roofline"]["frac_of_measured_read"] = round(achieved / probe["gbs"], 4)
    if not args.no_fp8:
        result["fp8"] = bench_fp8(args, torch, B, W, dev)
    if not args.no_prefill:
        result["prefill"] = bench_prefill(args, torch, B, W, dev)
    if not args.no_other:
        result["other_decode_workloads"] = [bench_other(torch, B, W, dev, name)
                                            for name in ("qwen_mha", "cont_batch")]
    if not args.no_mixed:
        result["mixed_step"] = [bench_mixed(torch, B, W, dev, name)
                                for name in ("mixed_step", "mixed_tail")]
    if not args.no_pool:
        result["block_pool"] = bench_pool(torch, B, W, dev)
    if host is not None:
        result["cpu_baseline"] = cpu_baseline(wl, host, args.cpu_seconds)
    print(json.dumps(result), flush=True)


def bench_read_probe(torch, B, dev, gib=4, iters=10):
    """The second denominator beside the nominal 8 TB/s: one streaming read
    kernel (pkv_read_probe: whole 4 KiB tiles per wave, as decode reads them,
    16-byte nontemporal loads) over a 4 GiB buffer, far past the L2 and the
    256 MB last-level cache, timed in this run (median of 10 launches, HIP
    events)."""
    nbytes = gib << 30
    buf = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    sink = torch.zeros(4, dtype=torch.int32, device=dev)
    stream = torch.cuda.current_stream(dev)
    for _ in range(2):
        B.pkv_read_probe(buf, sink)
    torch.cuda.synchronize()
    ms = []
    for _ in range(iters):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        B.pkv_read_probe(buf, sink)
        b.record(stream)
        torch.cuda.synchronize()
        ms.append(a.elapsed_time(b))
    med = float(np.median(ms))
    del buf
    torch.cuda.empty_cache()
    gbs = nbytes / (med * 1e-3) / 1e9
    return {"kernel": "pkv_read_probe (whole 4 KiB tiles per wave, 16-byte nontemporal loads)", "bytes": nbytes,
            "ms": round(med, 4), "gbs": round(gbs, 1),
            "frac_of_nominal": round(gbs / HBM_PEAK_GBS, 4)}


def mfma_peak_rocminfo():
    """Dense bf16 MFMA peak recomputed from rocminfo: compute units x maximum
    clock x 4096 flops per compute unit per cycle (4 SIMDs, each retiring a
    16x16x32 bf16 MFMA, 16384 flops, every 16 cycles).  None when rocminfo is
    unavailable."""
    import re
    try:
        text = subprocess.run(["rocminfo"], capture_output=True, text=True, timeout=60).stdout
    except (OSError, subprocess.SubprocessError):
        return None
    for agent in text.split("*******"):
        if not re.search(r"Name:\s+gfx950", agent):
            continue
        cu = re.search(r"Compute Unit:\s+(\d+)", agent)
        mhz = re.search(r"Max Clock Freq\. \(MHz\):\s+(\d+)", agent)
        if cu and mhz:
            return {"compute_units": int(cu.group(1)), "max_clock_mhz": int(mhz.group(1)),
                    "tflops": round(int(cu.group(1)) * int(mhz.group(1)) * 1e6 * 4096 / 1e12, 1)}
    return None


def bench_fp8(args, torch, B, W, dev):
    """The same decode step over FP8 caches (OCP E4M3 codes + one fp32 scale per
    token and KV head): per layer, one pkv_store_decode_attn_fp8 launch that
    quantizes and stores the 32 new tokens and attends over the cache
    including them (``--separate``: pkv_store_fp8 then pkv_decode_attn_fp8;
    the other form is timed beside it either way).  The pools hold random
    codes and scales (32 layers, 8.3 GB); timing as for the bf16 step (a timed
    region without per-launch events, then a pass with events around each
    timed launch)."""
    L = args.layers
    wl = W.mistral_gqa(seed=args.seed, num_layers=L)
    S, Hq, Hkv, D = wl.num_seqs, wl.num_q_heads, wl.num_kv_heads, wl.head_dim
    gen = torch.Generator(device=dev)
    gen.manual_seed(wl.seed + 1)
    rb = lambda shape: W._randn_bf16(torch, shape, gen, dev)
    q = [rb((S, Hq, D)) for _ in range(L)]
    kn = [rb((S, Hkv, D)) for _ in range(L)]
    vn = [rb((S, Hkv, D)) for _ in range(L)]
    pools = [W.make_fp8_pools(wl, device=dev, seed=wl.seed + l, nan_fill=False) for l in range(L)]
    bt = torch.from_numpy(wl.block_tables).to(dev)
    ctx = torch.from_numpy(wl.context_lens).to(dev)
    slots = torch.from_numpy(wl.slot_mapping).to(dev)
    outs = [torch.empty((S, Hq, D), dtype=torch.bfloat16, device=dev) for _ in range(L)]
    P = B.pkv_decode_partition_tokens_fp8(S, Hkv, wl.max_context_len)
    ws = torch.empty(max(16, B.pkv_decode_workspace_bytes(S, Hq, D, wl.max_context_len, P)),
                     dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream(dev)

    def store(l):
        B.pkv_store_fp8(kn[l], vn[l], slots, *pools[l])

    def decode(l):
        B.pkv_decode_attn_fp8(q[l], *pools[l], bt, ctx, wl.scale, outs[l],
                              max_context_len=wl.max_context_len, workspace=ws,
                              partition_tokens=P)

    def fused(l):
        B.pkv_store_decode_attn_fp8(kn[l], vn[l], slots, q[l], *pools[l], bt, ctx, wl.scale,
                                    outs[l], max_context_len=wl.max_context_len, workspace=ws,
                                    partition_tokens=P)

    def separate(l):
        store(l)
        decode(l)

    def timed_step(fn):
        for _ in range(args.warmup):
            for l in range(L):
                fn(l)
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for _ in range(args.steps):
            for l in range(L):
                fn(l)
        b.record(stream)
        torch.cuda.synchronize()
        return a.elapsed_time(b) / args.steps

    main, other = (separate, fused) if args.separate else (fused, separate)
    ms_per_step = timed_step(main)
    other_ms = timed_step(other)
    pairs = []
    for _ in range(args.steps):
        for l in range(L):
            if args.separate:  # time the decode launch only
                store(l)
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            decode(l) if args.separate else fused(l)
            e1.record(stream)
            pairs.append((e0, e1))
    torch.cuda.synchronize()
    dec_ms, dec_stats = launch_stats([x.elapsed_time(y) for x, y in pairs])
    ctx64 = wl.context_lens.astype(np.int64)
    # decode: codes + scales of every cached token, q in, out back, table, lengths
    dec_bytes = (int(ctx64.sum()) * 2 * Hkv * (D + 4) + 2 * S * Hq * D * 2
                 + 4 * int(((ctx64 + 15) // 16).sum()) + 4 * S)
    # store: bf16 k/v in, codes + scales out, slots
    st_bytes = S * 2 * Hkv * D * 2 + S * 2 * Hkv * (D + 4) + 4 * S
    step_gbs = L * (dec_bytes + st_bytes) / (ms_per_step * 1e-3) / 1e9
    launch_bytes = dec_bytes if args.separate else dec_bytes + st_bytes
    # as for the bf16 step: the timed region's average launch duration, or the
    # event-bracketed decode launches with --separate
    launch_ms = dec_ms if args.separate else ms_per_step / L
    achieved = launch_bytes / (launch_ms * 1e-3) / 1e9
    launch_timing = {"source": ("events around each decode launch" if args.separate
                                else "timed region / launches"),
                     "timed_region_us_per_launch": round(ms_per_step / L * 1e3, 2),
                     "event_bracketed": dec_stats}
    kernel = f"decode_fused_kernel<{D},{Hq // Hkv},fp8>" if P < 0 else \
        f"decode_split_kernel<{D},{Hq // Hkv},fp8>+decode_reduce_kernel<{D}>"
    del pools, q, kn, vn, outs
    torch.cuda.empty_cache()
    return {
        "workload": "the same 32 seqs x 4096 tokens, 32q/8kv, d 128, 32 layers, over FP8 (E4M3 + "
                    "fp32 scale per token and KV head) caches: "
                    + ("pkv_store_fp8 + pkv_decode_attn_fp8" if args.separate
                       else "pkv_store_decode_attn_fp8 (store fused)"),
        "work_split": (f"single pass, {-P} waves per (seq, kv head)" if P < 0
                       else f"split-KV, {P}-token partitions + merge"),
        "ms_per_step": round(ms_per_step, 4),
        ("fused_ms_per_step" if args.separate else "separate_ms_per_step"): round(other_ms, 4),
        "tokens_per_s_per_layer": round(S * L / (ms_per_step * 1e-3), 1),
        "kv_gbs": round(step_gbs, 2), "hbm_peak_frac": round(step_gbs / HBM_PEAK_GBS, 4),
        "decode_us_per_layer": round(launch_ms * 1e3, 2),  # the timed launch (see kernel)
        "roofline": {"bound": "hbm",
                     "kernel": kernel + ("" if args.separate else " (fused store)"),
                     "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": recorded_traffic(kernel + ("" if args.separate else " (fused store)")),
                     "algorithmic_bytes_per_launch": launch_bytes,
                     "launch_us": round(launch_ms * 1e3, 2), "launch_timing": launch_timing},
    }


def bench_other(torch, B, W, dev, name, iters=20):
    """Store + decode (fused launch) on one of the other decode workloads: the
    Qwen-style MHA batch (16 seqs, ctx U{128..2048}, 32 x 128 heads) or the
    continuous batch (256 seqs in 8 groups of 32 sharing a 2048-token prefix
    through identical block ids, lognormal tails).  Two pool copies alternate
    so consecutive launches do not find each other's K/V in cache.  Reports
    logical KV GB/s (every sequence's context) and, where blocks are shared,
    the unique-block rate too."""
    wl = W.CONFIGS[name]()
    t = W.make_tensors(wl, device=dev, layers=2, nan_fill=False)
    out = torch.empty_like(t["q"])
    P = B.pkv_decode_partition_tokens(wl.num_seqs, wl.num_kv_heads, wl.max_context_len)
    ws = torch.empty(max(16, B.pkv_decode_workspace_bytes(wl.num_seqs, wl.num_q_heads,
                                                          wl.head_dim, wl.max_context_len, P)),
                     dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream(dev)

    def run(l):
        B.pkv_store_decode_attn(t["k_new"], t["v_new"], t["slot_mapping"], t["q"],
                                t["k_caches"][l], t["v_caches"][l], t["block_tables"],
                                t["context_lens"], wl.scale, out,
                                max_context_len=wl.max_context_len, workspace=ws,
                                partition_tokens=P)

    for l in (0, 1, 0, 1):
        run(l)
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record(stream)
    for i in range(iters):
        run(i & 1)
    b.record(stream)
    torch.cuda.synchronize()
    us = a.elapsed_time(b) * 1e3 / iters
    logical = decode_bytes(wl) + store_bytes(wl)
    unique_tok = int(wl.used_blocks().shape[0]) * wl.block_size
    res = {"workload": name, "num_seqs": wl.num_seqs, "max_context_len": wl.max_context_len,
           "sum_context": int(wl.context_lens.sum()),
           "work_split": (f"single pass, {-P} waves" if P < 0 else f"split-KV, P = {P} + merge"),
           "us_per_launch": round(us, 2), "logical_kv_gbs": round(logical / us / 1e3, 1),
           "tokens_per_s": round(wl.num_seqs / (us * 1e-6), 1)}
    if wl.shared_blocks:
        uniq = unique_tok * 2 * wl.num_kv_heads * wl.head_dim * 2
        res["unique_kv_gbs"] = round(uniq / us / 1e3, 1)
        res["shared_prefix"] = bench_prefix(torch, B, wl, t, out, stream, iters, logical, uniq)
    del t
    return res


def bench_prefix(torch, B, wl, t, out, stream, iters, logical, uniq):
    """The same step as store + pkv_decode_attn_prefix: groups found by
    pkv_prefix_groups on the host tables, each group's prefix read once."""
    from paged_kv_cache_pools_amd import workloads as W

    dev = t["q"].device
    starts, plens, mg = B.pkv_prefix_groups(wl.block_tables, wl.context_lens)
    gs, pl = torch.from_numpy(starts).to(dev), torch.from_numpy(plens).to(dev)
    ptoks = (0, 128, 256, 512)
    ws = torch.empty(max(B.pkv_decode_prefix_workspace_bytes(
        wl.num_seqs, wl.num_q_heads, wl.num_kv_heads, wl.head_dim, wl.max_context_len, p)
        for p in ptoks), dtype=torch.uint8, device=dev)

    def run(l, p):
        B.pkv_store(t["k_new"], t["v_new"], t["slot_mapping"], t["k_caches"][l], t["v_caches"][l])
        B.pkv_decode_attn_prefix(t["q"], t["k_caches"][l], t["v_caches"][l], t["block_tables"],
                                 t["context_lens"], wl.scale, out, gs, pl, mg,
                                 max_context_len=wl.max_context_len, workspace=ws,
                                 partition_tokens=p)

    for p in ptoks:
        for l in (0, 1):
            run(l, p)
    torch.cuda.synchronize()
    sweep = {}
    for p in ptoks:
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for i in range(iters):
            run(i & 1, p)
        b.record(stream)
        torch.cuda.synchronize()
        sweep["auto" if p == 0 else str(p)] = round(a.elapsed_time(b) * 1e3 / iters, 2)
    us = sweep["auto"]

    # the same step over FP8 caches (random codes and scales; the new tokens
    # quantized by pkv_store_fp8), against the FP8 fused store + split decode
    pools8 = [W.make_fp8_pools(wl, device=dev, seed=wl.seed + l, nan_fill=False) for l in range(2)]
    P8 = B.pkv_decode_partition_tokens_fp8(wl.num_seqs, wl.num_kv_heads, wl.max_context_len)
    ws8 = torch.empty(max(16, B.pkv_decode_workspace_bytes(wl.num_seqs, wl.num_q_heads,
                                                           wl.head_dim, wl.max_context_len, P8)),
                      dtype=torch.uint8, device=dev)

    def run8(l):
        B.pkv_store_fp8(t["k_new"], t["v_new"], t["slot_mapping"], *pools8[l])
        B.pkv_decode_attn_prefix_fp8(t["q"], *pools8[l], t["block_tables"], t["context_lens"],
                                     wl.scale, out, gs, pl, mg, max_context_len=wl.max_context_len,
                                     workspace=ws)

    def plain8(l):
        B.pkv_store_decode_attn_fp8(t["k_new"], t["v_new"], t["slot_mapping"], t["q"], *pools8[l],
                                    t["block_tables"], t["context_lens"], wl.scale, out,
                                    max_context_len=wl.max_context_len, workspace=ws8,
                                    partition_tokens=P8)

    fp8 = {}
    for key, fn in (("us_per_step", run8), ("plain_decode_us", plain8)):
        for l in (0, 1, 0, 1):
            fn(l)
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for i in range(iters):
            fn(i & 1)
        b.record(stream)
        torch.cuda.synchronize()
        fp8[key] = round(a.elapsed_time(b) * 1e3 / iters, 2)
    del pools8
    fp8 = {"launch": "pkv_store_fp8 + pkv_decode_attn_prefix_fp8", **fp8,
           "plain_decode": "pkv_store_decode_attn_fp8, its own work split",
           "speedup_vs_plain": round(fp8["plain_decode_us"] / fp8["us_per_step"], 4)}
    return {"groups": len(plens), "prefix_lens": sorted(set(int(x) for x in plens)),
            "max_group_size": int(mg), "us_per_step": us,
            "us_by_partition_tokens": sweep, "logical_kv_gbs": round(logical / us / 1e3, 1),
            "unique_kv_gbs": round(uniq / us / 1e3, 1),
            "tokens_per_s": round(wl.num_seqs / (us * 1e-6), 1), "fp8": fp8}


def bench_pool(torch, B, W, dev, steps=64):
    """The block pool and the copy-on-write kernel.

    Host: the continuous batch (256 sequences in 8 groups sharing a 2048-token
    prompt, lognormal tails) admitted into a prefix-caching pool, then decode
    steps of 256 appends plus the 256 x 2048 block-table build.  Device:
    pkv_copy_blocks of 256 blocks across 64 pools (32 layers x K, V, 32 KiB
    per block and pool), 512 MiB read and 512 MiB written per launch, and one
    block (one fork's copy-on-write) for its latency."""
    wl = W.CONFIGS["cont_batch"]()
    rng = np.random.default_rng(wl.seed + 77)
    S = wl.num_seqs
    groups = 8
    shared = [rng.integers(0, 32000, 2048).tolist() for _ in range(groups)]
    prompts = [shared[i % groups] + rng.integers(0, 32000, int(wl.context_lens[i]) - 2048).tolist()
               for i in range(S)]
    nb = 20000
    pool = B.BlockPool(nb, 16, prefix_caching=True)
    t0 = time.perf_counter()
    cached = sum(pool.add_seq(i, prompts[i])[1] for i in range(S))
    admit_s = time.perf_counter() - t0
    used = nb - pool.num_free()
    ids = np.arange(S, dtype=np.int64)
    maxb = 2048
    toks = np.zeros(S, np.int32)
    t0 = time.perf_counter()
    for _ in range(steps):
        pool.append(ids, toks)
        pool.block_tables(ids, maxb)
    step_us = (time.perf_counter() - t0) / steps * 1e6
    total_tokens = int(sum(len(p) for p in prompts))
    host = {"workload": "continuous batch: 256 seqs, 8 groups sharing a 2048-token prompt, "
                        "lognormal tails, prefix caching on",
            "admit_ms": round(admit_s * 1e3, 2), "prompt_tokens": total_tokens,
            "tokens_from_cache": int(cached),
            "blocks_in_use": int(used), "blocks_without_sharing": int(-(-wl.context_lens // 16).sum()),
            "decode_step_us": round(step_us, 1),
            "decode_step": "256 appends + block tables [256][2048]"}
    del pool

    # device: the copy kernel
    npools, pool_blocks, bb = 64, 1024, 8 * 16 * 128 * 2
    pools = [torch.empty((pool_blocks, 8, 16, 128), dtype=torch.bfloat16, device=dev)
             for _ in range(npools)]
    for p in pools:
        p.normal_()
    pairs = [torch.from_numpy(np.stack([np.arange(256) + off, np.arange(256) + 512 + off],
                                       axis=1).astype(np.int32)).to(dev) for off in (0, 256)]
    one = torch.tensor([[3, 1000]], dtype=torch.int32, device=dev)
    stream = torch.cuda.current_stream(dev)
    for i in range(4):
        B.pkv_copy_blocks(pools, pairs[i & 1])
    torch.cuda.synchronize()
    iters = 10
    evs = []
    for i in range(iters):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        B.pkv_copy_blocks(pools, pairs[i & 1])
        b.record(stream)
        evs.append((a, b))
    torch.cuda.synchronize()
    ms, copy_stats = launch_stats([a.elapsed_time(b) for a, b in evs])
    nbytes = 2 * 256 * npools * bb + 256 * 8
    achieved = nbytes / (ms * 1e-3) / 1e9
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record(stream)
    for _ in range(20):
        B.pkv_copy_blocks(pools, one)
    b.record(stream)
    torch.cuda.synchronize()
    one_us = a.elapsed_time(b) * 1e3 / 20
    device = {"kernel": "copy_blocks_kernel<4,nt>", "pairs": 256, "pools": npools, "block_bytes": bb,
              "ms_per_launch": round(ms, 4),
              "roofline": {"bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS,
                           "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                           "traffic": recorded_traffic("copy_blocks_kernel<4,nt>"),
                           "algorithmic_bytes_per_launch": nbytes, "launch_timing": copy_stats},
              "one_block_all_pools_us": round(one_us, 2)}
    del pools
    torch.cuda.empty_cache()
    return {"host": host, "copy": device}


def bench_mixed(torch, B, W, dev, name="mixed_step", iters=20):
    """One continuous-batching iteration in one launch (pkv_mixed_attn), on
    the 32 x 4096 GQA decode batch plus prompt chunks: "mixed_step", 4 chunks
    of 496 new tokens after 0 / 512 / 1536 / 3072 cached ones (2016 new
    tokens), or "mixed_tail", one 64-token chunk after 4032 cached ones.
    Timed against the same work as two launches (pkv_decode_attn on the
    decode sequences, then pkv_prefill_attn on the chunks), and without the
    key-range split of prefill units.  Two layer pools alternate.  Each form
    is timed over a region of back-to-back calls, as the decode step is (an
    event pair around every call is reported beside it).  The bound for one
    launch that overlaps both kinds of work perfectly is
    max(decode bytes / HBM peak, prefill flops / bf16 MFMA peak)."""
    wl = W.CONFIGS[name]()
    nd = 32
    t = W.make_tensors(wl, device=dev, layers=2, nan_fill=False)
    for l in range(2):
        B.pkv_store(t["k_new"], t["v_new"], t["slot_mapping"], t["k_caches"][l], t["v_caches"][l])
    out = torch.empty_like(t["q"])
    mnl = int(wl.new_lens[nd:].max())
    mcl = int(wl.context_lens.max())
    q_dec, out_dec = t["q"][:nd], out[:nd]
    bt_dec, ctx_dec = t["block_tables"][:nd].contiguous(), t["context_lens"][:nd].contiguous()
    q_pf, out_pf = t["q"][nd:], out[nd:]
    bt_pf, ctx_pf = t["block_tables"][nd:].contiguous(), t["context_lens"][nd:].contiguous()
    cu_pf = (t["cu_new_lens"][nd:] - nd).contiguous()
    P = B.pkv_decode_partition_tokens(nd, wl.num_kv_heads, 4096)
    ws = torch.empty(max(16, B.pkv_decode_workspace_bytes(nd, wl.num_q_heads, wl.head_dim, 4096, P)),
                     dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream(dev)

    ws_bytes = B.pkv_mixed_workspace_bytes(wl.num_seqs, nd, mnl, mcl, wl.num_q_heads,
                                           wl.num_kv_heads, wl.head_dim)
    ws_mixed = torch.empty(max(ws_bytes, 16), dtype=torch.uint8, device=dev)

    def mixed(l):
        B.pkv_mixed_attn(t["q"], t["k_caches"][l], t["v_caches"][l], t["block_tables"],
                         t["cu_new_lens"], t["context_lens"], nd, wl.scale, out,
                         max_new_len=mnl, max_context_len=mcl, workspace=ws_mixed)

    def mixed_whole(l):
        B.pkv_mixed_attn(t["q"], t["k_caches"][l], t["v_caches"][l], t["block_tables"],
                         t["cu_new_lens"], t["context_lens"], nd, wl.scale, out,
                         max_new_len=mnl, max_context_len=mcl, split=False)

    def separate(l):
        B.pkv_decode_attn(q_dec, t["k_caches"][l], t["v_caches"][l], bt_dec, ctx_dec, wl.scale,
                          out_dec, max_context_len=4096, workspace=ws, partition_tokens=P)
        B.pkv_prefill_attn(q_pf, t["k_caches"][l], t["v_caches"][l], bt_pf, cu_pf, ctx_pf,
                           wl.scale, out_pf, max_new_len=mnl, max_context_len=mcl)

    def timed(fn):
        """(ms per call over one region of back-to-back calls, the stats of a
        second pass with an event pair around every call): the region is the
        figure, as for the decode step; the bracketed pass adds idle GPU time
        per call and is reported beside it."""
        for l in (0, 1, 0, 1):
            fn(l)
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for i in range(iters):
            fn(i & 1)
        b.record(stream)
        torch.cuda.synchronize()
        region_ms = a.elapsed_time(b) / iters
        evs = []
        for i in range(iters):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            fn(i & 1)
            b.record(stream)
            evs.append((a, b))
        torch.cuda.synchronize()
        _, stats = launch_stats([a.elapsed_time(b) for a, b in evs])
        return region_ms, {"source": "timed region / calls",
                           "timed_region_us_per_call": round(region_ms * 1e3, 2),
                           "event_bracketed": stats}

    for fn in (mixed, mixed_whole, separate):  # every variant warm before any is timed
        timed(fn)
    mixed_ms, mixed_stats = timed(mixed)
    whole_ms, _ = timed(mixed_whole)
    sep_ms, sep_stats = timed(separate)

    # the same iteration over FP8 caches (random codes and scales, the new
    # tokens quantized into them by pkv_store_fp8)
    pools8 = [W.make_fp8_pools(wl, device=dev, seed=wl.seed + l, nan_fill=False) for l in range(2)]
    for l in range(2):
        B.pkv_store_fp8(t["k_new"], t["v_new"], t["slot_mapping"], *pools8[l])
    P8 = B.pkv_decode_partition_tokens_fp8(nd, wl.num_kv_heads, 4096)

    def mixed8(l):
        B.pkv_mixed_attn_fp8(t["q"], *pools8[l], t["block_tables"], t["cu_new_lens"],
                             t["context_lens"], nd, wl.scale, out, max_new_len=mnl,
                             max_context_len=mcl, workspace=ws_mixed)

    def separate8(l):
        B.pkv_decode_attn_fp8(q_dec, *pools8[l], bt_dec, ctx_dec, wl.scale, out_dec,
                              max_context_len=4096, workspace=ws, partition_tokens=P8)
        B.pkv_prefill_attn_fp8(q_pf, *pools8[l], bt_pf, cu_pf, ctx_pf, wl.scale, out_pf,
                               max_new_len=mnl, max_context_len=mcl)

    for fn in (mixed8, separate8):
        timed(fn)
    mixed8_ms, _ = timed(mixed8)
    sep8_ms, _ = timed(separate8)
    del pools8
    S, Hq, Hkv, D = wl.num_seqs, wl.num_q_heads, wl.num_kv_heads, wl.head_dim
    dec_bytes = (int(wl.context_lens[:nd].sum()) * 2 * Hkv * D * 2 + 2 * nd * Hq * D * 2
                 + 4 * int((-(-wl.context_lens[:nd] // 16)).sum()) + 4 * nd)
    pf_flops = 0.0
    for p in range(nd, S):
        c, n = int(wl.context_lens[p] - wl.new_lens[p]), int(wl.new_lens[p])
        pf_flops += 4.0 * D * Hq * (n * c + n * (n + 1) / 2)
    t_hbm = dec_bytes / (HBM_PEAK_GBS * 1e9)
    t_mfma = pf_flops / (MFMA_BF16_PEAK_TFLOPS * 1e12)
    bound_ms = max(t_hbm, t_mfma) * 1e3
    del t
    torch.cuda.empty_cache()
    what = ("4 prefill chunks x 496 new (cached 0/512/1536/3072)" if name == "mixed_step"
            else "1 prefill chunk of 64 new after 4032 cached")
    return {"workload": f"{name}: 32 decode seqs x 4096 + {what}, 32q/8kv, d 128",
            "mixed_us": round(mixed_ms * 1e3, 2), "separate_us": round(sep_ms * 1e3, 2),
            "mixed_unsplit_us": round(whole_ms * 1e3, 2), "split_workspace_bytes": ws_bytes,
            "speedup_vs_separate": round(sep_ms / mixed_ms, 4),
            "fp8": {"launch": "pkv_mixed_attn_fp8", "mixed_us": round(mixed8_ms * 1e3, 2),
                    "separate_us": round(sep8_ms * 1e3, 2),
                    "speedup_vs_separate": round(sep8_ms / mixed8_ms, 4)},
            "decode_bytes": dec_bytes, "prefill_gflop": round(pf_flops / 1e9, 3),
            "roofline": {"bound": "hbm+mfma overlap", "kernel": "mixed_kernel<128,4>",
                         "bound_us": round(bound_ms * 1e3, 2),
                         "hbm_us": round(t_hbm * 1e6, 2), "mfma_us": round(t_mfma * 1e6, 2),
                         "frac": round(bound_ms / mixed_ms, 4),
                         "launch_timing": mixed_stats},
            "separate_timing": sep_stats}


def bench_prefill(args, torch, B, W, dev):
    """Chunked causal prefill, 8 prompts x 2048 new tokens after U{0..4096}
    cached, GQA 32/8, d 128: store of the new tokens, then MFMA attention."""
    wl = W.chunked_prefill()
    t = W.make_tensors(wl, device=dev, nan_fill=False)
    out = torch.empty_like(t["q"])
    stream = torch.cuda.current_stream(dev)

    def run():
        B.pkv_prefill_attn(t["q"], t["k_caches"][0], t["v_caches"][0], t["block_tables"],
                           t["cu_new_lens"], t["context_lens"], wl.scale, out,
                           max_new_len=wl.max_new_len, max_context_len=wl.max_context_len)

    def store():
        B.pkv_store(t["k_new"], t["v_new"], t["slot_mapping"], t["k_caches"][0], t["v_caches"][0])

    store()
    for _ in range(2):
        run()
    torch.cuda.synchronize()
    evs = []
    for _ in range(args.prefill_iters):
        a, b, c = (torch.cuda.Event(enable_timing=True) for _ in range(3))
        a.record(stream)
        store()
        b.record(stream)
        run()
        c.record(stream)
        evs.append((a, b, c))
    torch.cuda.synchronize()
    st_ms = float(np.median([a.elapsed_time(b) for a, b, _ in evs]))
    at_ms = float(np.median([b.elapsed_time(c) for _, b, c in evs]))
    fl = prefill_flops(wl)
    tf = fl / (at_ms * 1e-3) / 1e12
    peak = mfma_peak_rocminfo()

    # the same prefill over an FP8 cache (random codes and scales in every
    # slot; the new tokens quantized into it by pkv_store_fp8)
    pools = W.make_fp8_pools(wl, device=dev, nan_fill=False)

    def run8():
        B.pkv_prefill_attn_fp8(t["q"], *pools, t["block_tables"], t["cu_new_lens"],
                               t["context_lens"], wl.scale, out, max_new_len=wl.max_new_len,
                               max_context_len=wl.max_context_len)

    def store8():
        B.pkv_store_fp8(t["k_new"], t["v_new"], t["slot_mapping"], *pools)

    store8()
    for _ in range(2):
        run8()
    torch.cuda.synchronize()
    evs8 = []
    for _ in range(args.prefill_iters):
        a, b, c = (torch.cuda.Event(enable_timing=True) for _ in range(3))
        a.record(stream)
        store8()
        b.record(stream)
        run8()
        c.record(stream)
        evs8.append((a, b, c))
    torch.cuda.synchronize()
    st8 = float(np.median([a.elapsed_time(b) for a, b, _ in evs8]))
    at8 = float(np.median([b.elapsed_time(c) for _, b, c in evs8]))
    tf8 = fl / (at8 * 1e-3) / 1e12
    return {
        "workload": "chunked causal prefill: 8 prompts x 2048 new tokens, cached U{0..4096}, "
                    "32q/8kv, d 128",
        "attn_ms": round(at_ms, 4), "attn_tflops": round(tf, 2),
        "mfma_peak_frac": round(tf / MFMA_BF16_PEAK_TFLOPS, 4),
        "mfma_peak_rocminfo": peak,
        "mfma_frac_rocminfo": round(tf / peak["tflops"], 4) if peak else None,
        "causal_gflop": round(fl / 1e9, 2),
        "store_ms": round(st_ms, 4),
        "store_gbs": round(store_bytes(wl) / (st_ms * 1e-3) / 1e9, 2),
        "fp8": {"launch": "pkv_prefill_attn_fp8 (E4M3 cache, bf16 matrix products on the codes)",
                "attn_ms": round(at8, 4), "attn_tflops": round(tf8, 2),
                "mfma_peak_frac": round(tf8 / MFMA_BF16_PEAK_TFLOPS, 4),
                "time_vs_bf16": round(at8 / at_ms, 4),
                "store_fp8_ms": round(st8, 4)},
    }


if __name__ == "__main__":
    main()
