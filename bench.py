#!/usr/bin/env python3
"""Decode-step benchmark of the quantized-KV decode attention path on one MI355X.

A step is one pass of the whole hot path on one batch, one call of
kvq_append_decode_attn: append one token per sequence (entry conversion, the
fp16 window write -- done by the decode kernel when the token goes to the
window -- and a group flush whenever the window fills) and decode attention
of one query per head over the whole cache (split kernel and cross-split
merge, inside the kernel's workgroups or by a merge kernel).  Inputs are
seeded synthetic tensors already resident in HBM; the cache is prefilled
before timing.

Prints one JSON line.  `value` is achieved HBM throughput of the whole step
(algorithmic bytes: packed codes + fp16 scales/zeros + fp16 window + q + out
+ the append's own bytes, divided by the measured step time).  `roofline`
covers the dominant kernel (the split decode kernel), timed with HIP events
on the stream it runs on; its `traffic` is the HBM bytes per launch measured
with rocprofv3 counters (profiles/), reported only while the kernel sources
are unchanged since.  `cpu_baseline` is the CPU oracle timed on a bounded
sample of the same workload on this host's cores.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "quantized-KV decode attention: µs/step + achieved HBM GB/s (8B-shape, 32k ctx)"
HBM_PEAK_GBS = 8000.0


def in_bytes(w) -> int:
    return 4 if w.dtype == "f32" else 2


def quant_token_bytes(w, kb: int, vb: int) -> int:
    """Bytes per quantized token: codes, key scale/zero per channel shared by G
    tokens, value scale/zero per channel group, the key norm if any."""
    return w.D * (kb + vb) // 8 + 4 * w.D // w.G + 4 * (w.D // w.G) + 2 * int(w.token_norm)


def decode_bytes(w, n: int, gbits=None) -> int:
    """Algorithmic bytes of one decode over n cached tokens per sequence;
    gbits = (key bits, value bits) per group for position-adaptive caches."""
    nq = (max(0, n - w.sink - w.R) // w.G) * w.G
    nr = n - nq  # fp16 tokens: the attention sink and the recent window
    if gbits is None:
        quant = nq * quant_token_bytes(w, w.kbits, w.vbits)
    else:
        ng = nq // w.G
        quant = sum(w.G * quant_token_bytes(w, int(kb), int(vb)) for kb, vb in zip(gbits[0][:ng], gbits[1][:ng]))
    per_window_token = 4 * w.D  # fp16 K and V
    cache = w.B * w.Hkv * (quant + nr * per_window_token)
    return cache + w.B * w.Hq * w.D * (in_bytes(w) + 4)


def append_bytes(w, n_before: int, gbits=None) -> int:
    """Algorithmic bytes of appending one token to sequences holding n_before."""
    slices = w.B * w.Hkv
    b = slices * w.D * (2 * in_bytes(w) + 4)  # read k, v; write both as fp16
    nq0 = (max(0, n_before - w.sink - w.R) // w.G) * w.G
    nq1 = (max(0, n_before + 1 - w.sink - w.R) // w.G) * w.G
    if nq1 > nq0:  # one group flushed: read its fp16 tokens, write the page
        kb, vb = (w.kbits, w.vbits) if gbits is None else (int(gbits[0][nq0 // w.G]), int(gbits[1][nq0 // w.G]))
        page = w.G * quant_token_bytes(w, kb, vb)
        b += slices * (w.G * w.D * 4 + page)
    return b


def cpu_baseline(w, K_host, V_host, q_host, batches, threads: int) -> dict:
    """Time the oracle's decode step (fp64 dequant + attention) on the sampled
    batch rows (all kv heads), then scale to the full step."""
    import oracle
    from synth import to_oracle_input

    pairs = [(b, h) for b in batches for h in range(w.Hkv)]
    from concurrent.futures import ThreadPoolExecutor

    gb = None
    if w.adapt_delta:  # the prefill's group bits
        gb = oracle.adaptive_group_bits(w.G, w.R, w.sink, w.adapt_delta, [w.N], w.bits_low, (w.kbits, w.vbits),
                                        w.bits_high)

    def enc(bh):
        b, h = bh
        return oracle.encode_slice(to_oracle_input(K_host[b][h], w.dtype), to_oracle_input(V_host[b][h], w.dtype),
                                   w.dtype, w.D, w.kbits, w.vbits, w.G, w.R, w.rotate, sink=w.sink, hybrid=w.hybrid,
                                   token_norm=w.token_norm, group_bits=gb)

    t_enc = time.perf_counter()
    with ThreadPoolExecutor(threads) as ex:
        encs = list(ex.map(enc, pairs))
    t_enc = time.perf_counter() - t_enc
    jobs = []
    for (b, h), e in zip(pairs, encs):
        q = oracle.input_to_f64(to_oracle_input(q_host[b], w.dtype), w.dtype).reshape(w.Hq, w.D)
        if w.rotate:
            import numpy as np

            q = np.stack([oracle.rotate_f64(x) for x in q])
        jobs.append((q[h * w.gqa:(h + 1) * w.gqa], e, w.D, w.G, w.R))
    t0 = time.perf_counter()
    oracle.attend_slices_parallel(jobs, threads)
    dt = time.perf_counter() - t0
    full = dt * (w.B * w.Hkv) / len(pairs)
    # the same on one thread, over a few slices
    n1 = min(8, len(jobs))
    t1 = time.perf_counter()
    oracle.attend_slices_parallel(jobs[:n1], 1)
    dt1 = time.perf_counter() - t1
    full1 = dt1 * (w.B * w.Hkv) / n1
    step_bytes = decode_bytes(w, w.N, gb)
    return {
        "value": round(step_bytes / full / 1e9, 3),
        "unit": "GB/s",
        "us_per_step": round(full * 1e6, 1),
        "cores": threads,
        "kind": "oracle",
        "sample": f"decode step (fp64 dequant + attention) over {len(pairs)} of {w.B * w.Hkv} (batch, kv-head) "
                  f"slices at {w.N} tokens, {dt:.2f} s wall on {threads} threads, scaled by slice count",
        "one_core": {"value": round(step_bytes / full1 / 1e9, 4), "unit": "GB/s", "us_per_step": round(full1 * 1e6, 1),
                     "sample": f"the same over {n1} slices on 1 thread ({dt1:.2f} s), scaled by slice count"},
        "quantize": {"s_per_prefill": round(t_enc * (w.B * w.Hkv) / len(pairs), 2), "cores": threads,
                     "sample": f"the oracle's encoder (O1-O6) over the {len(pairs)} sampled slices' {w.N} tokens "
                               f"({t_enc:.2f} s), scaled by slice count"},
    }


def source_fingerprint(paths) -> str:
    """sha256 of the given sources with comments and whitespace removed."""
    import hashlib
    import re

    parts = []
    for rel in paths:
        with open(os.path.join(ROOT, rel)) as f:
            t = f.read()
        t = re.sub(r"/\*.*?\*/", "", t, flags=re.S)
        t = re.sub(r"//[^\n]*", "", t)
        parts.append(re.sub(r"\s+", "", t))
    return hashlib.sha256("".join(parts).encode()).hexdigest()


def measured_traffic(workload: str):
    """HBM bytes per decode launch from the rocprofv3 counter summary for this
    workload (profiles/decode_kernel_traffic_<workload>.md), or None when there
    is none or the decode kernel sources changed since the counters were taken."""
    import glob
    import re

    for path in glob.glob(os.path.join(ROOT, "profiles", "decode_kernel_traffic_*.md")):
        with open(path) as f:
            m = re.search(r"```json\s*(\{.*?\})\s*```", f.read(), flags=re.S)
        if not m:
            continue
        rec = json.loads(m.group(1))
        if rec.get("workload") != workload:
            continue
        if source_fingerprint(rec["fingerprint_of"]) != rec["source_fingerprint"]:
            return None
        return int(rec["traffic_bytes_per_launch"])
    return None


def copy_calibration(gib: float) -> int:
    """Device-to-device copies of exactly `gib` GiB (reads and writes that many
    bytes each time): the reference for scaling FETCH_SIZE / WRITE_SIZE."""
    import torch

    n = int(gib * (1 << 30)) // 4
    x = torch.ones(n, dtype=torch.float32, device="cuda")
    y = torch.empty_like(x)
    for _ in range(3):
        y.copy_(x)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes": n * 4, "copies": 3}), flush=True)
    return 0


def cpu_info() -> dict:
    """The CPU model and the cores this process may use: its affinity set,
    bounded by a cgroup CPU quota if one is set."""
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    usable = len(os.sched_getaffinity(0))
    quota = None
    try:
        with open("/sys/fs/cgroup/cpu.max") as f:
            q, per = f.read().split()[:2]
            if q != "max":
                quota = max(1, int(int(q) / int(per)))
    except (OSError, ValueError):
        pass
    return {"model": model, "affinity": usable, "cgroup_quota": quota,
            "usable": min(usable, quota) if quota else usable}


def percentiles(xs) -> dict:
    import numpy as np

    a = np.asarray(xs, dtype=np.float64)
    return {"p10": round(float(np.percentile(a, 10)), 2), "median": round(float(np.median(a)), 2),
            "p90": round(float(np.percentile(a, 90)), 2), "mean": round(float(a.mean()), 2), "n": int(a.size)}


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=64, help="timed steps (64 spans one group flush at G=64)")
    ap.add_argument("--warmup", type=int, default=96, help="untimed steps before the timed ones")
    ap.add_argument("--prefill-reps", type=int, default=8,
                    help="timed prefills (reset + append of the whole context) right before the warmup steps; "
                         "prefill_ms is their median.  They also keep the GPU busy up to the first step: after "
                         "an idle stretch the step time takes ~60 steps to settle")
    ap.add_argument("--dist-steps", type=int, default=64,
                    help="steps after the timed ones, each between two events, for the step-time percentiles")
    ap.add_argument("--evict-mall", type=float, default=0.0, metavar="GIB",
                    help="write GIB GiB of scratch between the percentile steps (outside their events), so "
                         "caches that fit the 256 MB MALL are read from HBM every step")
    ap.add_argument("--workload", type=int, default=2, help="index into synth.WORKLOADS (default: the 32k K4/V2 layer)")
    ap.add_argument("--splits", type=int, default=0, help="split count (0: the library's default)")
    ap.add_argument("--sink", type=int, default=0, help="attention-sink tokens kept in fp16 (a multiple of the group size)")
    ap.add_argument("--hybrid", action="store_true", help="per-group symmetric/asymmetric quantizer choice")
    ap.add_argument("--token-norm", action="store_true", help="key tokens divided by their norm before quantization")
    ap.add_argument("--adapt-delta", type=int, default=0,
                    help="position-adaptive bit widths: region size Delta in tokens (0: off)")
    ap.add_argument("--bits-low", default="2,2", help="key,value bits of the first Delta tokens")
    ap.add_argument("--bits-high", default="4,4", help="key,value bits of the last Delta tokens")
    ap.add_argument("--kernel-steps", type=int, default=32,
                    help="steps after the timed ones that time the decode launch (with and without it)")
    ap.add_argument("--drift", action="store_true",
                    help="also time the drift check (code histograms + KL per group) over every quantized group")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-sample-batches", type=int, default=16)
    ap.add_argument("--copy-calibration", type=float, default=0.0, metavar="GIB",
                    help="instead of the benchmark, copy GIB GiB device-to-device 3 times (a plain copy of known "
                         "size, used to scale HBM byte counters)")
    args = ap.parse_args()
    if args.copy_calibration > 0:
        return copy_calibration(args.copy_calibration)

    if args.gpus != 1:
        print(f"bench.py runs on one GPU only; --gpus {args.gpus} is not supported (this path has no multi-GPU "
              f"mode: every (batch, kv-head) slice is independent, so batches or kv heads would be split over "
              f"GPUs with no exchange, and a long context over GPUs with one merge of the split partials).",
              file=sys.stderr)
        return 2

    import torch

    import decode_attention_asym_amd as kvq
    from decode_attention_asym_amd.kvq import merge_partials
    from synth import WORKLOADS, Synth

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 1
    w = WORKLOADS[args.workload]
    if args.sink or args.hybrid or args.token_norm or args.adapt_delta:
        lo = tuple(int(x) for x in args.bits_low.split(","))
        hi = tuple(int(x) for x in args.bits_high.split(","))
        adapt = f"-adapt{args.adapt_delta}-lo{lo[0]}{lo[1]}-hi{hi[0]}{hi[1]}" if args.adapt_delta else ""
        w = w.replace(name=w.name + (f"-sink{args.sink}" if args.sink else "") + ("-hybrid" if args.hybrid else "")
                      + ("-tokennorm" if args.token_norm else "") + adapt,
                      sink=args.sink, hybrid=args.hybrid, token_norm=args.token_norm, adapt_delta=args.adapt_delta,
                      bits_low=lo if args.adapt_delta else (0, 0), bits_high=hi if args.adapt_delta else (0, 0))
    total = args.warmup + args.steps + 2 * args.kernel_steps + args.dist_steps
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    syn = Synth(w, dev, positions=w.N + total + 1)
    cache = kvq.KVQCache(kvq.config_for(w, max_tokens=w.N + total), device=dev)

    # every input and buffer exists before the prefill, so nothing but the
    # prefills runs between the first prefill and the first step
    print(f"[bench] {w.name}: generating inputs", file=sys.stderr, flush=True)
    K, V = syn.kv_all()
    batches = list(range(min(args.cpu_sample_batches, w.B)))
    K_host = [K[b].cpu() for b in batches] if not args.no_cpu_baseline else None
    V_host = [V[b].cpu() for b in batches] if not args.no_cpu_baseline else None
    step_kv = [syn.step_kv(i) for i in range(total)]
    qs = [syn.q(i) for i in range(total)]
    rows = w.B * w.Hq
    cfg_full = kvq.config_for(w, max_tokens=w.N + total)
    # a position-adaptive cache may use a few more splits than asked (at least one per run of equal bits)
    cap = max(args.splits, kvq.workspace_bytes(cfg_full) // (rows * (w.D + 4) * 4))
    partials = torch.empty(rows * cap * (w.D + 4), dtype=torch.float32, device=dev)
    out = torch.empty((w.B, w.Hq, w.D), dtype=torch.float32, device=dev)
    scratch = torch.empty(int(args.evict_mall * (1 << 30)) // 4, dtype=torch.float32, device=dev) \
        if args.evict_mall > 0 else None
    torch.cuda.synchronize()

    # the prefill: the first call on the fresh cache buffer (first touch of its
    # pages), then prefill_reps calls after a reset, each between two events;
    # the last one leaves the cache prefilled for the steps
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    cache.append(K, V)
    e1.record()
    torch.cuda.synchronize()
    prefill_first_ms = e0.elapsed_time(e1)
    pev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(max(1, args.prefill_reps))]
    for a, b in pev:
        cache.reset()
        a.record()
        cache.append(K, V)
        b.record()
    S = args.splits or cache.default_splits()  # host-side: the token count is known without the device
    # (split count, splits merged inside the decode kernel, partial records
    # per row the merge kernel combines): with the merge in the kernel a step
    # is one launch (the decode also writes the token's window slots), else
    # two (decode, merge kernel)
    S_used, merged, records = cache.decode_plan(S)

    def step(i):
        # one decode step: kvq_append_decode_attn (append one token, whose
        # window write the decode kernel does, then decode); with an explicit
        # --splits, kvq_append then kvq_decode_attn_splits
        k, v = step_kv[i]
        if args.splits:
            cache.append(k, v)
            cache.decode(qs[i], out, splits=S)
        else:
            cache.append_decode(k, v, qs[i], out)

    def step_separate(i):
        k, v = step_kv[i]
        cache.append(k, v)
        cache.decode(qs[i], out, splits=S)

    for i in range(args.warmup):
        step(i)
    # timed region: the K steps alone (no event inside it: an event recorded
    # between two kernels slows the kernel after it, measured +35 us on the
    # decode in a rocprofv3 trace, with or without the event's system fence)
    nk = args.kernel_steps
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(5)]
    n0 = cache.num_tokens
    torch.cuda.synchronize()
    ev[0].record()
    for i in range(args.steps):
        step(args.warmup + i)
    ev[1].record()
    # the decode kernel's average launch duration, by difference, right after
    # and with no host synchronization in between, so the GPU never idles
    # (an idle GPU restarts slower: the first ~60 steps after a pause of a few
    # ms run up to 3x the settled step time; with a synchronization here the
    # 175B-shaped MHA layer's first decode launches after it ran ~15% slower
    # in the trace): nk more steps as kvq_append + kvq_decode_attn_splits,
    # then nk steps without the decode launch (the append, and the merge
    # kernel when the decode does not merge its splits itself), each span
    # between two events
    if not merged:
        # valid records (o = 0, m = 0, l = 1) for the merge-only steps
        pv = partials[: rows * records * (w.D + 4)].view(rows * records, w.D + 4)
        pv.zero_()
        pv[:, w.D + 1] = 1.0
    ev[2].record()
    for i in range(nk):
        step_separate(args.warmup + args.steps + i)
    ev[3].record()
    for i in range(nk):
        k, v = step_kv[args.warmup + args.steps + nk + i]
        cache.append(k, v)
        if not merged:
            merge_partials(partials, out, rows, records, w.D)
    ev[4].record()
    torch.cuda.synchronize()
    # per-step percentiles: each step between two events of its own (an event
    # between kernels costs the next kernel a little, so these run slightly
    # above the back-to-back steps), optionally with a MALL-evicting write
    # between steps, outside the events
    base = args.warmup + args.steps + 2 * nk
    sev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(args.dist_steps)]
    for i, (a, b) in enumerate(sev):
        if scratch is not None:
            scratch.fill_(float(i))
        a.record()
        step(base + i)
        b.record()
    torch.cuda.synchronize()
    dist = percentiles([a.elapsed_time(b) * 1e3 for a, b in sev]) if sev else None
    if dist is not None:
        dist["evict_mall_gib"] = args.evict_mall
    prefill_list = sorted(a.elapsed_time(b) for a, b in pev)
    prefill_ms = prefill_list[len(prefill_list) // 2]
    print(f"[bench] prefill {w.N} tokens: {prefill_ms:.2f} ms median of {len(pev)} (first call "
          f"{prefill_first_ms:.2f} ms)", file=sys.stderr, flush=True)
    del K, V

    ms_total = ev[0].elapsed_time(ev[1])
    ms_step = ms_total / args.steps
    gbits = cache.group_bits() if w.adapt_delta else None  # a group's bits never change once quantized
    step_bytes = [decode_bytes(w, n0 + i + 1, gbits) + append_bytes(w, n0 + i, gbits) for i in range(args.steps)]
    value = sum(step_bytes) / (ms_total * 1e-3) / 1e9
    assert torch.isfinite(out).all()
    dec_avg_ms = (ev[2].elapsed_time(ev[3]) - ev[3].elapsed_time(ev[4])) / nk
    n1 = n0 + args.steps
    dec_bytes = [decode_bytes(w, n1 + i + 1, gbits) for i in range(nk)]
    achieved = (sum(dec_bytes) / len(dec_bytes)) / (dec_avg_ms * 1e-3) / 1e9

    drift = None
    if args.drift and not w.adapt_delta:
        ng = cache.num_groups()
        kh, vh = cache.code_histograms(0, max(1, ng // 3))
        for _ in range(2):
            cache.drift_check(kh, vh)
        torch.cuda.synchronize()
        d0, d1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        reps = 10
        d0.record()
        for _ in range(reps):
            _, _, fl = cache.drift_check(kh, vh)
        d1.record()
        torch.cuda.synchronize()
        us = d0.elapsed_time(d1) / reps * 1e3
        slices = w.B * w.Hkv
        nbytes = slices * ng * (w.G * w.D * (w.kbits + w.vbits) // 8 + 17)  # codes read, KL pair + flag written
        drift = {"kernel": "drift_kernel (code histograms + KL per group)", "groups": slices * ng,
                 "avg_us": round(us, 2), "bytes": nbytes, "achieved_gbs": round(nbytes / (us * 1e-6) / 1e9, 1),
                 "frac": round(nbytes / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
                 "flagged": int((fl != 0).sum().item())}

    cpu = None
    if not args.no_cpu_baseline:
        from synth import to_oracle_input  # noqa: F401

        ci = cpu_info()
        # every usable core, up to the 16-core CPU share a GPU gets on the
        # measurement hosts (they show more cores than one GPU's share)
        threads = min(16, ci["usable"])
        print(f"[bench] cpu baseline on {threads} threads ({ci['model']})", file=sys.stderr, flush=True)
        q0 = syn.q(0).cpu()
        cpu = cpu_baseline(w, K_host, V_host, q0, batches, threads)
        cpu["cpu_model"] = ci["model"]
        cpu["host_cpus"] = {"affinity": ci["affinity"], "cgroup_quota": ci["cgroup_quota"]}

    res = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "us_per_step": round(ms_step * 1e3, 2),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16",
        "dtype_detail": f"u{w.kbits}/u{w.vbits} codes and fp16 scale/zero/window; fp16 MFMA operands, fp32 accumulate and softmax; {w.dtype} inputs",
        "data": "synthetic",
        "config": {
            "workload": w.name, "batch": w.B, "q_heads": w.Hq, "kv_heads": w.Hkv, "head_dim": w.D,
            "context": w.N, "k_bits": w.kbits, "v_bits": w.vbits, "group": w.G, "residual": w.R,
            "rotate": w.rotate, "sink": w.sink, "hybrid": w.hybrid, "token_norm": w.token_norm, "splits": S_used,
            "splits_merged_in_kernel": merged, "merge_records": records,
            "adapt_delta": w.adapt_delta, "bits_low": list(w.bits_low), "bits_high": list(w.bits_high),
            "parallelism": "single-gpu",
        },
        "roofline": {
            "kernel": ("decode_fused_kernel (split dequant-attention, splits merged in the workgroup)"
                       if merged and S_used > 1 else
                       "decode_fused_kernel (split dequant-attention, each four splits merged in the workgroup)"
                       if 0 < records < S_used else "decode_kernel (split dequant-attention)"),
            "bound": "hbm",
            "achieved": round(achieved, 1),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": measured_traffic(w.name),
            "avg_us": round(dec_avg_ms * 1e3, 2),
            "launches_timed": nk,
            "timing": "per launch: (span of nk steps of append + decode) - (span of nk steps without the decode "
                      "launch), after the timed steps",
            "bytes_per_launch": int(sum(dec_bytes) / len(dec_bytes)),
        },
        "step_us_percentiles": dist,
        "prefill_ms": round(prefill_ms, 2),
        "prefill_reps": len(pev),
        "prefill_first_ms": round(prefill_first_ms, 2),
        **({"drift_check": drift} if drift else {}),
        "cpu_baseline": cpu,
    }
    print(json.dumps(res), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
