#!/usr/bin/env python
"""Benchmark of the routed int4 MoE layer on one MI355X.

Workload: the GLM-5.2-shaped layer (hidden 6144, expert intermediate 2048,
256 routed experts in 8 groups, top-8 of 4 groups, one shared expert, int4
codes with fp16 group-32 scales, fp32 router), batch-1 decode of 1,000
independent tokens (bf16 N(0,1) activations, uniform routing from a N(0,0.01)
correction bias).  One step = the 1,000 tokens, each its own
moe_layer_forward call with T = 1 (router + top-k, 8 routed experts + shared
expert, combine), enqueued back to back on one stream, all inputs resident in
HBM before timing starts.

Prints one JSON line on stdout; progress goes to stderr.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0  # MI355X HBM3E, published
METRIC = "routed-expert HBM GB/s (% of peak) + MoE-layer tokens/s, batch-1 int4 decode"


def log(msg: str) -> None:
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


# HBM counter record (rocprofv3 FETCH_SIZE / WRITE_SIZE) of the dominant
# decode kernel, the routed gate/up launch
TRAFFIC_RECORD = os.path.join(ROOT, "profiles", "gateup_kernel_glm_decode_traffic.md")
KERNEL_SOURCES = [os.path.join(ROOT, "routed_expert_int4_amd", "csrc", f)
                  for f in ("moe_decode.hip", "moe_device.h", "moe_kernels.h", "moe_layout.h")]
# Counter records of the grouped gate/up kernel per batched workload: HBM
# traffic (FETCH_SIZE / WRITE_SIZE) and matrix-core work (MFMA ops and busy
# cycles)
BATCH_TRAFFIC_RECORD = os.path.join(ROOT, "profiles", "batched_kernels_glm_hbm_counters.md")
BATCH_MFMA_RECORD = os.path.join(ROOT, "profiles", "batched_kernels_glm_mfma_counters.md")
BATCH_KERNEL_SOURCES = [os.path.join(ROOT, "routed_expert_int4_amd", "csrc", f)
                        for f in ("moe_batch.hip", "moe_decode.hip", "moe_device.h", "moe_kernels.h", "moe_layout.h")]


DTYPES = {
    "int4": "int4 weights x int16 fixed-point activations (two int8 parts), int32 dot, fp32 accumulate",
    "mxfp4": "MXFP4 weights (E2M1, E8M0 scales) x fp16 activation pairs, fp32 dot2 accumulate",
    "int8": "int8 weights (two nibble planes) x int16 fixed-point activations (two int8 parts), int32 dot, "
            "fp32 accumulate",
    "int2": "int2 weights (two rows per nibble) x int16 fixed-point activations (two int8 parts), int32 dot, "
            "fp32 accumulate",
}


def algorithmic_bytes(cfg):
    """Bytes each stage must move at least once per token (batch 1).

    Weights dominate: the fp32 router matrix and the shared expert's gate +
    up codes and scales for the router launch, gate + up of the 8 routed
    experts for the gate/up launch, the down codes and scales of all 9 for
    the down launch.  The
    activations (bf16 x, fp32 h and y) are counted where a launch reads or
    writes them.
    """
    eb = cfg.expert_bytes()
    n = cfg.top_k + cfg.n_shared
    sb = cfg.scale_bytes  # 2 (int4, int8: fp16 scales) or 1 (MXFP4, E8M0 scales)
    cb = cfg.hidden * cfg.inter // cfg.codes_per_byte  # code bytes of one matrix
    gu = 2 * (cb + cfg.inter * (cfg.hidden // 32) * sb)  # gate + up, codes + scales
    dn = cb + cfg.hidden * (cfg.inter // 32) * sb
    router = cfg.n_experts * cfg.hidden * 4 + cfg.n_experts * 4
    io = cfg.hidden * 2 + cfg.hidden * 4
    return {
        "expert": eb,
        "routed_per_token": cfg.top_k * eb,
        "layer_per_token": router + n * eb + io,
        # router launch: router weight + the shared expert's gate/up
        "router_launch": router + cfg.hidden * 2 + cfg.n_shared * gu,
        "gateup_launch": cfg.top_k * gu,
        "down_launch": n * dn + n * cfg.inter * 4 + cfg.hidden * 4,
        # gate/up + down launch: both of the above (h is written and read
        # inside the launch)
        "gateup_down_launch": cfg.top_k * gu + n * dn + n * cfg.inter * 4 + cfg.hidden * 4,
    }


def source_digest(sources=None) -> str:
    import hashlib
    h = hashlib.sha256()
    for path in sources or KERNEL_SOURCES:
        with open(path, "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def read_record(path, tag, sources, **match):
    """The last `tag:` JSON line of a committed counter record whose fields
    equal match, or None when there is none or the kernel sources' digest
    differs from the one the counters were taken on."""
    if not os.path.exists(path):
        return None
    rec = None
    with open(path) as f:
        for line in f:
            if line.startswith(tag + ":"):
                r = json.loads(line.split(":", 1)[1])
                if all(r.get(k) == v for k, v in match.items()):
                    rec = r
    if not rec or rec.get("source_sha256") != source_digest(sources):
        return None
    return rec


def measured_traffic(kernel):
    """HBM bytes per launch of a decode kernel (its name as rocprofv3 prints
    it, up to the argument list) from the committed rocprofv3 counter record.

    The record holds FETCH_SIZE and WRITE_SIZE per dispatch of the kernel,
    each scaled by what the counter reads for a device copy of known size,
    and the digest of the kernel sources they were taken on.  Returns None
    when there is no record or the kernel source has changed since.
    """
    rec = read_record(TRAFFIC_RECORD, "traffic-record", KERNEL_SOURCES, kernel_name=kernel)
    return int(rec["hbm_bytes_per_launch"]) if rec else None


def time_oracle(weights, sample):
    """Tokens/s of the fp64 oracle's full layer over sample (bf16 bits) on
    every host thread, and on one thread over a short prefix."""
    from oracle import oracle
    threads = int(os.environ.get("OMP_NUM_THREADS", "0")) or len(os.sched_getaffinity(0))
    oracle.layer_forward(weights, sample[:1], n_threads=threads)  # load + warm
    t0 = time.perf_counter()
    oracle.layer_forward(weights, sample, n_threads=threads)
    dt = time.perf_counter() - t0
    n1 = max(1, min(16, sample.shape[0]))
    t1 = time.perf_counter()
    oracle.layer_forward(weights, sample[:n1], n_threads=1)
    dt1 = time.perf_counter() - t1
    cpu_model = ""
    try:
        with open("/proc/cpuinfo") as f:
            cpu_model = next((l.split(":", 1)[1].strip() for l in f if l.startswith("model name")), "")
    except OSError:
        pass
    return {"tokens_per_s": sample.shape[0] / dt, "seconds": dt, "cores": threads,
            "tokens_per_s_1_thread": n1 / dt1, "cpu_model": cpu_model}


def cpu_baseline(weights, x_bits, n_tokens: int, bytes_per_token: int):
    r = time_oracle(weights, x_bits[:n_tokens])
    return {
        "value": round(r["tokens_per_s"] * bytes_per_token / 1e9, 4),
        "unit": "GB/s",
        "tokens_per_s": round(r["tokens_per_s"], 3),
        "cores": r["cores"],
        "kind": "oracle",
        "sample": f"first {n_tokens} of the 1000 tokens, full layer in fp64 (router, top-k, 8 routed + shared "
                  f"experts, combine), {r['seconds']:.1f} s",
        "tokens_per_s_1_thread": round(r["tokens_per_s_1_thread"], 3),
        "cpu_model": r["cpu_model"],
    }


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=5)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--tokens", type=int, default=1000, help="independent batch-1 tokens per step")
    ap.add_argument("--cpu-sample", type=int, default=640, help="tokens timed on the CPU oracle (0: skip)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="first run one device copy of 256 MiB (a known-size kernel for HBM counter scaling)")
    ap.add_argument("--workload", default="decode",
                    choices=["decode", "batch32", "prefill512", "cache-stack", "probes"],
                    help="decode: the headline batch-1 line (default); batch32 / prefill512: the batched "
                         "workloads; cache-stack: 12 layers behind the HBM expert cache; probes: the device "
                         "ceilings (HBM copy, host copies, bf16 GEMM); each prints its own line")
    ap.add_argument("--stack-tokens", type=int, default=256, help="sequential tokens of the cache-stack workload")
    ap.add_argument("--pin", type=int, default=-1,
                    help="cache-stack: experts pinned per layer by learned usage (-1: slots - top_k, 0: plain LRU)")
    ap.add_argument("--learn-tokens", type=int, default=128, help="cache-stack: tokens of the learning pass")
    ap.add_argument("--max-prefetch", type=int, default=0,
                    help="cache-stack: experts copied per call by the next-layer prefetch (0: top_k)")
    ap.add_argument("--chain", default="noise", choices=["noise", "residual"],
                    help="cache-stack: next layer input = bf16(y / rms(y) + N(0, 0.1)) (noise, the workload's "
                         "chaining) or the RMS-normalised running sum of those terms and the first input "
                         "(residual: a residual stream, which makes consecutive layers' inputs correlated)")
    ap.add_argument("--codec", default="int4", choices=["int4", "mxfp4", "int8", "int2"],
                    help="decode and cache-stack: expert weight codec (mxfp4: E2M1 codes, E8M0 scales; int8, "
                         "int2: one byte or 2 bits per weight, fp16 scales)")
    ap.add_argument("--top-p", type=float, default=1.0,
                    help="decode and cache-stack: adaptive expert top-p (1: plain top-k); decode prices its bytes "
                         "by the experts kept")
    ap.add_argument("--decode-launches", type=int, default=3, choices=[1, 2, 3],
                    help="decode: launches per token of the timed path (3: router, gate/up, down, the library's "
                         "default; 2: router launch + one gate/up + down launch; 1: one fused launch); the other "
                         "two are timed beside it for comparison")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only: --gpus {args.gpus} is not supported (this layer's path is "
              "single-GPU; sharding over more GPUs is not built)", file=sys.stderr)
        return 2
    if args.workload == "decode":
        return bench_decode(args)
    if args.workload == "cache-stack":
        return bench_cache_stack(args)
    if args.workload == "probes":
        return bench_probes(args)
    return bench_batched(args)


def bench_cache_stack(args) -> int:
    """12 stacked GLM-shaped layers behind the HBM expert cache (one JSON line).

    Layer l: weights seed 100 + l, the committed Zipf(1.1) bias of layer l
    (tests/golden/zipf_bias_stack.json); all 12 x 256 routed experts packed in
    pinned host memory (65.2 GB), 64 HBM slots per layer.  Sequential decode:
    token t enters layer 0 as x0[t]; each next layer's input is
    bf16(y / rms(y) + N(0, 0.1) noise).  Every layer call is one
    moe_layer_forward with T = 1, which reads the routing back to the host
    and copies missing experts on the cache's copy stream.

    Learning cache (the default, as colibri's auto-pin): a learning pass of
    --learn-tokens tokens (x0 seed 310, noise seed 410, not timed) records
    each layer's expert usage; then every layer pins its --pin most used
    experts (default slots - top_k, loaded before the timed region, as at
    start-up) and keeps the other slots as an LRU.  The timed run decodes
    --stack-tokens tokens (x0 seed 300, noise seed 400) with the LRU part
    empty.  The same tokens are then run again with plain LRU over all slots
    from a cold start.  Each configuration also runs with the speculative
    next-layer prefetch (layer l + 1's router on layer l's input, at most
    --max-prefetch copies per call), and each run records a copy/compute
    timeline over its second half (fraction of the copy engine's busy time
    during which a kernel ran).  --pin 0 times plain LRU only."""
    import numpy as np
    import torch

    from routed_expert_int4_amd import binding as B
    from routed_expert_int4_amd import synth
    from routed_expert_int4_amd.layer import DeviceLayer, ExpertCache, HostExpertStore

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    import dataclasses
    cfg = dataclasses.replace(synth.GLM, top_p=args.top_p, codec=args.codec)
    n_layers, slots, n_tok = 12, 64, args.stack_tokens
    n_pin = slots - cfg.top_k if args.pin < 0 else args.pin
    with open(os.path.join(ROOT, "tests", "golden", "zipf_bias_stack.json")) as f:
        biases = [np.asarray(l["bias"], dtype=np.float32) for l in json.load(f)["layers"]]
    cache = ExpertCache(cfg, n_layers, slots)
    layers = []
    w0 = None
    t0 = time.perf_counter()
    for l in range(n_layers):
        w = synth.gen_layer(cfg, seed=100 + l)
        w.bias = biases[l]
        cache.register(l, HostExpertStore(w))
        lay = DeviceLayer(w, max_T=1, resident=False)
        lay.attach_cache(cache, l)
        layers.append(lay)
        if l == 0:
            w0 = w  # kept for the CPU oracle's sample
        del w
        log(f"layer {l} ready ({time.perf_counter() - t0:.0f} s)")
    H = cfg.hidden
    y = torch.empty((1, H), dtype=torch.float32, device="cuda:0")
    ids = torch.empty((1, cfg.top_k), dtype=torch.int32, device="cuda:0")
    w = torch.empty((1, cfg.top_k), dtype=torch.float32, device="cuda:0")
    stream = torch.cuda.current_stream()

    def decode(x_seed, noise_seed, n, timeline_from=None):
        """n sequential tokens through the stack; returns (ms, stats at n/2,
        copy/compute timeline from token timeline_from on, or None)."""
        x0 = DeviceLayer.to_device_bf16(synth.gen_tokens(cfg, n, seed=x_seed))
        noise = torch.from_numpy(synth.gen_noise(cfg, n * n_layers, seed=noise_seed, std=0.1)).to("cuda:0")
        half = None
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for t in range(n):
            if t == n // 2:
                half = [cache.stats(l) for l in range(n_layers)]
            if t == timeline_from:
                cache.timeline(True)
            x = x0[t:t + 1]
            r = x.float() if args.chain == "residual" else None
            for l in range(n_layers):
                B.moe_layer_forward(layers[l].handle, x, 1, y, ids, w, stream)
                rms = torch.sqrt(torch.mean(y * y, dim=1, keepdim=True))
                z = y / rms + noise[t * n_layers + l:t * n_layers + l + 1]
                if args.chain == "residual":
                    # a residual stream: the layer's normalised output is added
                    # to the running sum, whose RMS-normalised value is the next input
                    r = r + z
                    z = r / torch.sqrt(torch.mean(r * r, dim=1, keepdim=True))
                x = z.to(torch.bfloat16)
        e1.record(stream)
        torch.cuda.synchronize()
        tl = None
        if timeline_from is not None:
            tl = cache.timeline_read()
            cache.timeline(False)
        return e0.elapsed_time(e1), half, tl

    keys = ("hits", "misses", "h2d_bytes", "prefetches", "prefetch_hits", "predicted_uses", "predicted_hits")

    def totals(stats):
        return {k: sum(st[k] for st in stats) for k in keys}

    def link(on):
        """Speculative next-layer prefetch: layer l predicts layer l + 1."""
        for l in range(n_layers - 1):
            layers[l].set_next(layers[l + 1] if on else None, args.max_prefetch)

    def empty_cache():
        for l in range(n_layers):
            cache.unpin(l, list(range(cfg.n_experts)))
            for e in range(cfg.n_experts):
                cache.evict(l, e)

    def reset(pins):
        """Empty slots, then the pinned experts loaded (as at start-up)."""
        empty_cache()
        p0 = time.perf_counter()
        if pins is not None:
            for l in range(n_layers):
                cache.pin(l, pins[l])
        torch.cuda.synchronize()
        return time.perf_counter() - p0

    def measured(label, prefetch, pins):
        """One timed run from the reset state, then a replica of it (same
        state, seeds and therefore the same cache decisions) with the
        copy/compute timeline recorded over its second half (its event
        stamps are kept out of the timed run)."""
        reset(pins)
        before = totals([cache.stats(l) for l in range(n_layers)])
        link(prefetch)
        log(f"{label}: decoding {n_tok} tokens through {n_layers} cached layers")
        ms, half, _ = decode(300, 400, n_tok)
        after = totals([cache.stats(l) for l in range(n_layers)])
        reset(pins)
        _, _, tl = decode(300, 400, n_tok, timeline_from=n_tok // 2)
        link(False)
        mid = totals(half)
        d = {k: after[k] - before[k] for k in after}
        d2 = {k: after[k] - mid[k] for k in after}
        r = {"tokens_per_s": n_tok / (ms / 1e3), "ms": ms, "routed_uses_per_token_layer":
             (d["hits"] + d["misses"]) / (n_tok * n_layers),
             "hit_rate": d["hits"] / max(d["hits"] + d["misses"], 1),
             "hit_rate_second_half": d2["hits"] / max(d2["hits"] + d2["misses"], 1),
             "h2d_bytes": d["h2d_bytes"], "h2d_gbs": d["h2d_bytes"] / (ms / 1e3) / 1e9,
             "misses": d["misses"], "prefetches": d["prefetches"], "prefetch_hits": d["prefetch_hits"],
             "prediction_accuracy": d["predicted_hits"] / d["predicted_uses"] if d["predicted_uses"] else None,
             "timeline_second_half": {
                 "copy_ms": tl["copy_ms"], "kernel_ms": tl["kernel_ms"], "overlap_ms": tl["overlap_ms"],
                 "span_ms": tl["span_ms"], "copies": tl["copies"], "kernels": tl["kernels"],
                 "truncated": tl["truncated"],
                 "copy_busy_frac": tl["copy_ms"] / tl["span_ms"] if tl["span_ms"] else None,
                 "copy_overlapped_frac": tl["overlap_ms"] / tl["copy_ms"] if tl["copy_ms"] else None}}
        acc = r["prediction_accuracy"]
        log(f"{label}: {r['tokens_per_s']:.1f} tokens/s, hit rate {r['hit_rate']:.4f}, "
            f"H2D {r['h2d_bytes'] / 1e9:.1f} GB at {r['h2d_gbs']:.1f} GB/s, prefetches {d['prefetches']} "
            f"(used {d['prefetch_hits']}), prediction accuracy {acc if acc is None else round(acc, 4)}, "
            f"copy busy {r['timeline_second_half']['copy_busy_frac']}, "
            f"overlapped {r['timeline_second_half']['copy_overlapped_frac']}")
        return r

    runs = {}
    pin_load_s = 0.0
    if n_pin > 0:
        log(f"learning pass: {args.learn_tokens} tokens")
        decode(310, 410, args.learn_tokens)
        # the n most used experts of each layer, ties to the lower index,
        # fixed now so that every run pins the same ones
        hot = [list(np.argsort(-cache.usage(l).astype(np.int64), kind="stable")[:n_pin]) for l in range(n_layers)]
        pin_load_s = reset(hot)
        for prefetch in (False, True):
            runs[("pinned", prefetch)] = measured(f"pinned {n_pin}" + (" + prefetch" if prefetch else ""),
                                                  prefetch, hot)
    for prefetch in (False, True):
        runs[("lru", prefetch)] = measured("plain LRU" + (" + prefetch" if prefetch else ""), prefetch, None)
    main_key = ("pinned", False) if n_pin > 0 else ("lru", False)
    main_run = runs[main_key]
    cpu = None
    if args.cpu_sample > 0:
        n = min(args.cpu_sample, 128)
        log(f"timing the CPU oracle on layer 0 for {n} tokens")
        r = time_oracle(w0, synth.gen_tokens(cfg, n, seed=300))
        cpu = {"value": round(r["tokens_per_s"] / n_layers, 4), "unit": "tokens/s",
               "tokens_per_s_one_layer": round(r["tokens_per_s"], 3), "cores": r["cores"], "kind": "oracle",
               "sample": f"layer 0 of the stack on the first {n} stack inputs (x0 seed 300), full layer in fp64 "
                         f"with every expert in host memory (no cache, no copies), {r['seconds']:.1f} s; "
                         f"through the stack = one layer's rate / {n_layers}",
               "tokens_per_s_1_thread": round(r["tokens_per_s_1_thread"] / n_layers, 4), "cpu_model": r["cpu_model"]}
        log(f"oracle: {cpu['value']} stack tokens/s on {cpu['cores']} threads")

    def rounded(r):
        return {k: (round(v, 4) if isinstance(v, float) else
                    ({kk: (round(vv, 4) if isinstance(vv, float) else vv) for kk, vv in v.items()}
                     if isinstance(v, dict) else v)) for k, v in r.items()}

    out = {
        "metric": "MoE-layer tokens/s through a 12-layer stack behind the HBM expert cache",
        "value": round(main_run["tokens_per_s"], 3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": 1,
        "warmup": 0,
        "ms_per_step": round(main_run["ms"], 3),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": DTYPES[cfg.codec],
        "data": "synthetic (seeded: layer weights 100 + l, Zipf bias per layer, x0 seed 300, noise seed 400; "
                "learning pass x0 seed 310, noise seed 410)",
        "config": {"workload": f"12 GLM-5.2-shaped MoE layers, {n_tok} sequential decode tokens, 64 HBM slots "
                               f"per layer ({n_pin} pinned by learned usage, the rest LRU), pinned host expert "
                               "store" + (f", adaptive expert top-p {cfg.top_p}" if cfg.top_p < 1.0 else "")
                               + (f", {cfg.codec} experts" if cfg.codec != "int4" else "")
                               + (", residual-stream chaining" if args.chain == "residual" else ""),
                   "chain": args.chain, "max_prefetch": args.max_prefetch or cfg.top_k,
                   "layers": n_layers, "slots_per_layer": slots, "pinned_per_layer": n_pin,
                   "learning_tokens": args.learn_tokens if n_pin > 0 else 0, "tokens": n_tok},
        "hit_rate": round(main_run["hit_rate"], 4),
        "hit_rate_second_half": round(main_run["hit_rate_second_half"], 4),
        "h2d_gbytes": round(main_run["h2d_bytes"] / 1e9, 3),
        "h2d_gbs": round(main_run["h2d_gbs"], 2),
        "pin_load_s": round(pin_load_s, 3),
        "timeline_second_half": rounded(main_run["timeline_second_half"]),
        "runs": {f"{kind}{'_prefetch' if pf else ''}": rounded(r) for (kind, pf), r in runs.items()},
        "roofline": {"kernel": "host-to-device expert copies (hipMemcpyAsync, pinned host)", "bound": "pcie",
                     "achieved": round(main_run["h2d_gbs"], 2), "peak": 64.0, "unit": "GB/s",
                     "frac": round(main_run["h2d_gbs"] / 64.0, 4), "traffic": None},
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)
    for lay in layers:
        lay.close()
    cache.close()
    return 0


def bench_probes(args) -> int:
    """Device ceilings the layer's numbers are read against (one JSON line):
    HBM GB/s of the library's read-only streaming kernel (moe_hbm_read_probe)
    and of a device-to-device copy (bytes read + bytes written) over buffers
    the size of the decode launches (56 MB, 113 MB, 197 MB) and of 1 GiB;
    pinned host-to-device and device-to-host copy GB/s (256 MiB); bf16 GEMM
    TFLOP/s (8192^3 through torch.matmul).  Each figure is the best of 10
    timed repeats after 3 warmups."""
    import torch

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = "cuda:0"

    def best_ms(fn, reps=10):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        for _ in range(3):
            fn()
        torch.cuda.synchronize()
        best = float("inf")
        for _ in range(reps):
            e0.record()
            fn()
            e1.record()
            torch.cuda.synchronize()
            best = min(best, e0.elapsed_time(e1))
        return best

    from routed_expert_int4_amd import binding as B
    read = {}
    for label, nbytes in (("56MB", 56_623_104), ("113MB", 113_246_208), ("1GiB", 1 << 30)):
        src = torch.ones(nbytes // 4, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        ms = best_ms(lambda: dst.copy_(src))
        read[label] = round(2 * nbytes / (ms / 1e3) / 1e9, 1)
        del src, dst
    # read-only streaming (the library's probe kernel) at the decode launches'
    # sizes (56.6 MB down, 113 MB routed gate/up, 197 MB one layer-token) and
    # 1 GiB; best over workgroup counts of 1 to 16 per CU and one workgroup
    # per 32 KiB tile (one pass)
    n_cu = torch.cuda.get_device_properties(0).multi_processor_count
    read_only = {}
    for label, nbytes in (("56MB", 56_623_104), ("113MB", 113_246_208), ("197MB", 197_432_320), ("1GiB", 1 << 30)):
        buf = torch.ones(nbytes // 4, dtype=torch.float32, device=dev)
        one_pass = (nbytes + 32767) // 32768  # one workgroup per 32 KiB tile
        sink = torch.empty(max(16 * n_cu, one_pass), dtype=torch.int32, device=dev)
        best = None
        for per_cu in (1, 2, 4, 8, 16, "one pass"):
            blocks = one_pass if per_cu == "one pass" else per_cu * n_cu
            ms = best_ms(lambda: B.moe_hbm_read_probe(buf, nbytes, sink, blocks))
            if best is None or ms < best[0]:
                best = (ms, per_cu)
        read_only[label] = {"gbs": round(nbytes / (best[0] / 1e3) / 1e9, 1), "workgroups_per_cu": best[1],
                            "us": round(best[0] * 1e3, 2)}
        del buf, sink
    host = torch.empty(256 << 20, dtype=torch.uint8, pin_memory=True)
    devb = torch.empty(256 << 20, dtype=torch.uint8, device=dev)
    h2d = (256 << 20) / (best_ms(lambda: devb.copy_(host, non_blocking=True)) / 1e3) / 1e9
    d2h = (256 << 20) / (best_ms(lambda: host.copy_(devb, non_blocking=True)) / 1e3) / 1e9
    n = 8192
    a = torch.randn(n, n, dtype=torch.bfloat16, device=dev)
    b = torch.randn(n, n, dtype=torch.bfloat16, device=dev)
    gemm = 2 * n ** 3 / (best_ms(lambda: torch.matmul(a, b)) / 1e3) / 1e12
    out = {
        "metric": "device ceilings: HBM read-only and copy GB/s, pinned host copy GB/s, bf16 GEMM TFLOP/s",
        "value": read_only["1GiB"]["gbs"], "unit": "GB/s", "n_gpus": 1, "steps": 10, "warmup": 3,
        "higher_is_better": True, "data": "synthetic",
        "config": {"workload": "probes: read-only streaming kernel (moe_hbm_read_probe), device-to-device copies, "
                               "pinned 256 MiB copies, 8192^3 bf16 matmul"},
        "hbm_read_only_gbs": read_only, "hbm_copy_gbs": read, "h2d_gbs": round(h2d, 1), "d2h_gbs": round(d2h, 1),
        "bf16_gemm_tflops": round(gemm, 1),
        "vs_peak": {"hbm_read_only_1GiB": round(read_only["1GiB"]["gbs"] / HBM_PEAK_GBS, 4),
                    "hbm_copy_1GiB": round(read["1GiB"] / HBM_PEAK_GBS, 4), "bf16_gemm": round(gemm / 2500.0, 4)},
    }
    print(json.dumps(out), flush=True)
    return 0


def bench_batched(args) -> int:
    """Batched workloads on the GLM-shaped layer (one JSON line).

    batch32: 32 calls of 32 tokens (x seed 4) with the committed Zipf(1.1)
    correction bias (speculative-verify-sized batches); one step = the 32
    calls.  prefill512: 8 chunks of 512 tokens (x seed 5, uniform routing);
    one step = the 8 chunks.  Algorithmic bytes per call: router weight +
    (distinct routed experts + shared) x expert bytes + x and y; flops per
    call: 2 x 3 x hidden x inter per (token, expert) over the routed and
    shared entries (matrix-core work of the grouped kernels)."""
    import numpy as np
    import torch

    from routed_expert_int4_amd import binding as B
    from routed_expert_int4_amd import synth
    from routed_expert_int4_amd.layer import DeviceLayer

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    import dataclasses
    cfg = dataclasses.replace(synth.GLM, codec=args.codec, top_p=args.top_p)
    if args.workload == "batch32":
        n_calls, T, seed = 32, 32, 4
        log("generating the GLM-shaped layer (seed 0) with the Zipf(1.1) bias")
        weights = synth.gen_layer(cfg, seed=0)
        with open(os.path.join(ROOT, "tests", "golden", "zipf_bias_glm.json")) as f:
            weights.bias = np.asarray(json.load(f)["bias"], dtype=np.float32)
        workload = "GLM-5.2-shaped MoE layer, 32 calls x 32 tokens, Zipf(1.1)-skewed routing"
    else:
        n_calls, T, seed = 8, 512, 5
        log("generating the GLM-shaped layer (seed 0)")
        weights = synth.gen_layer(cfg, seed=0)
        workload = "GLM-5.2-shaped MoE layer, prefill chunks of 512 tokens, 8 chunks per step"
    x_bits = synth.gen_tokens(cfg, n_calls * T, seed=seed)
    layer = DeviceLayer(weights, max_T=T)
    x = DeviceLayer.to_device_bf16(x_bits)
    y = torch.empty((n_calls * T, cfg.hidden), dtype=torch.float32, device="cuda:0")
    ids = torch.empty((n_calls * T, cfg.top_k), dtype=torch.int32, device="cuda:0")
    w = torch.empty((n_calls * T, cfg.top_k), dtype=torch.float32, device="cuda:0")
    stream = torch.cuda.current_stream()
    H, k = cfg.hidden, cfg.top_k

    def step():
        for c in range(n_calls):
            B.moe_layer_forward(layer.handle, x.data_ptr() + 2 * H * T * c, T, y.data_ptr() + 4 * H * T * c,
                                ids.data_ptr() + 4 * k * T * c, w.data_ptr() + 4 * k * T * c, stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(args.steps):
        step()
    e1.record(stream)
    torch.cuda.synchronize()
    ms_per_step = e0.elapsed_time(e1) / args.steps
    ids_h = ids.cpu().numpy().reshape(n_calls, T, k)
    # (id -1: a choice the top-p cut dropped; it is neither read nor computed)
    distinct = [len(np.unique(ids_h[c][ids_h[c] >= 0])) for c in range(n_calls)]
    single_max = 1 if T * k < 8 * cfg.n_experts or cfg.codec in ("int8", "int2") else 0
    singles = [int((np.unique(ids_h[c][ids_h[c] >= 0], return_counts=True)[1] <= single_max).sum())
               for c in range(n_calls)]
    eb = cfg.expert_bytes()
    router = cfg.n_experts * cfg.hidden * 4 + cfg.n_experts * 4
    bytes_step = sum(router + (d + cfg.n_shared) * eb + T * H * 6 for d in distinct)
    kept_entries = int((ids_h >= 0).sum())
    flops_step = (kept_entries + n_calls * T * cfg.n_shared) * 2 * 3 * H * cfg.inter
    tokens_per_s = n_calls * T * args.steps / (ms_per_step * args.steps / 1e3)
    gbs = bytes_step / (ms_per_step / 1e3) / 1e9
    tflops = flops_step / (ms_per_step / 1e3) / 1e12
    # per-stage spans, and the two grouped kernels stamped with their own
    # begin and end (HIP events on the launch stream), over one more step
    B.moe_layer_profile(layer.handle, True)
    step()
    torch.cuda.synchronize()
    kms, kn = B.moe_layer_profile_read(layer.handle)
    B.moe_layer_profile(layer.handle, False)
    stage_ms = [kms[i] for i in range(3)]
    # per call: the grouped MFMA kernel plus, in calls with 16-entry tiles,
    # the GEMV kernel of the experts with a single entry
    gu_ms, dn_ms = kms[4] + kms[6], kms[5] + kms[7]
    # algorithmic bytes of the two grouped kernels per step: the distinct
    # routed experts' and the shared expert's weights once per call, plus the
    # activations they read and the results they write
    sb = cfg.scale_bytes
    cb = H * cfg.inter // cfg.codes_per_byte
    gu_w = 2 * (cb + cfg.inter * (H // 32) * sb)
    dn_w = cb + H * (cfg.inter // 32) * sb
    pairs_step = kept_entries + n_calls * T * cfg.n_shared
    gu_bytes = sum((d + cfg.n_shared) * gu_w for d in distinct) + n_calls * T * H * 2 + pairs_step * cfg.inter * 4
    dn_bytes = sum((d + cfg.n_shared) * dn_w for d in distinct) + pairs_step * cfg.inter * 4 + pairs_step * H * 4
    gu_gbs = gu_bytes / (gu_ms / 1e3) / 1e9
    dn_gbs = dn_bytes / (dn_ms / 1e3) / 1e9
    gu_tf = pairs_step * 2 * 2 * H * cfg.inter / (gu_ms / 1e3) / 1e12
    dn_tf = pairs_step * 2 * H * cfg.inter / (dn_ms / 1e3) / 1e12
    log(f"{ms_per_step:.3f} ms/step, {tokens_per_s:.0f} tokens/s, {gbs:.0f} GB/s, {tflops:.1f} TFLOP/s; "
        f"stages ms {stage_ms}; grouped gate/up {1e3 * gu_ms / kn[4]:.1f} us x {kn[4]} ({gu_gbs:.0f} GB/s), "
        f"down {1e3 * dn_ms / kn[5]:.1f} us x {kn[5]} ({dn_gbs:.0f} GB/s); distinct experts per call "
        f"{min(distinct)}..{max(distinct)}")
    # counter records of this workload's grouped gate/up kernel (int4, plain
    # top-k), taken on the current kernel sources
    traffic, mfma = None, None
    if cfg.codec == "int4" and cfg.top_p >= 1.0:
        rec = read_record(BATCH_TRAFFIC_RECORD, "traffic-record", BATCH_KERNEL_SOURCES, workload=args.workload)
        if rec:
            traffic = int(rec["hbm_bytes_per_launch"])
        rec = read_record(BATCH_MFMA_RECORD, "mfma-record", BATCH_KERNEL_SOURCES, workload=args.workload)
        if rec:
            # matrix-core work the counters saw (zero-padded tile rows
            # included) over the bench's own launch time, and the MFMA
            # units' busy fraction over the launch
            mfma = {"flops_per_launch": rec["mfma_flops_per_dispatch"],
                    "tflops": round(rec["mfma_flops_per_dispatch"] / (gu_ms / kn[4] / 1e3) / 1e12, 2),
                    "busy_frac": rec["mfma_busy_frac"]}
    cpu = None
    if args.cpu_sample > 0:
        n = min(args.cpu_sample, 256)
        log(f"timing the CPU oracle on {n} tokens")
        r = time_oracle(weights, x_bits[:n])
        cpu = {"value": round(r["tokens_per_s"] * bytes_step / (n_calls * T) / 1e9, 4), "unit": "GB/s",
               "tokens_per_s": round(r["tokens_per_s"], 3), "cores": r["cores"], "kind": "oracle",
               "sample": f"first {n} tokens of the step, full layer in fp64 token by token (the oracle reads each "
                         f"token's experts itself), {r['seconds']:.1f} s; GB/s = tokens/s x the step's "
                         "algorithmic bytes per token",
               "tokens_per_s_1_thread": round(r["tokens_per_s_1_thread"], 3), "cpu_model": r["cpu_model"]}
        log(f"oracle: {cpu['tokens_per_s']} tokens/s on {cpu['cores']} threads")
    out = {
        "metric": f"MoE-layer tokens/s and HBM GB/s, batched {cfg.codec} calls",
        "value": round(gbs, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": f"{cfg.codec} weights x fp16 activations (MFMA), fp32 accumulate",
        "data": f"synthetic (seeded: weights seed 0, tokens seed {seed})",
        "config": {"workload": workload + (f", {cfg.codec} experts" if cfg.codec != "int4" else "")
                   + (f", adaptive expert top-p {cfg.top_p}" if cfg.top_p < 1.0 else ""), "tokens_per_call": T,
                   "calls_per_step": n_calls, "hidden": H, "expert_intermediate": cfg.inter,
                   "routed_experts": cfg.n_experts, "top_k": k},
        "tokens_per_s": round(tokens_per_s, 1),
        "pct_of_hbm_peak": round(100 * gbs / HBM_PEAK_GBS, 2),
        "distinct_experts_per_call": {"min": min(distinct), "max": max(distinct),
                                      "mean": round(float(np.mean(distinct)), 2)},
        "tflops": round(tflops, 2),
        "stage_ms_per_step": {"routing_dispatch": round(stage_ms[0], 4), "gateup_hprep": round(stage_ms[1], 4),
                              "down_combine": round(stage_ms[2], 4)},
        "grouped_kernels": {
            "gateup": {"avg_launch_us": round(1e3 * gu_ms / kn[4], 3), "launches_per_step": kn[4],
                       "bytes_per_step": gu_bytes, "gbs": round(gu_gbs, 1), "tflops": round(gu_tf, 2),
                       "mfma_kernel_us": round(1e3 * kms[4] / kn[4], 3),
                       "single_entry_gemv_us": round(1e3 * kms[6] / kn[6], 3) if kn[6] else None},
            "down": {"avg_launch_us": round(1e3 * dn_ms / kn[5], 3), "launches_per_step": kn[5],
                     "bytes_per_step": dn_bytes, "gbs": round(dn_gbs, 1), "tflops": round(dn_tf, 2),
                     "mfma_kernel_us": round(1e3 * kms[5] / kn[5], 3),
                     "single_entry_gemv_us": round(1e3 * kms[7] / kn[7], 3) if kn[7] else None},
            "single_entry_experts_per_call": round(float(np.mean(singles)), 2),
        },
        "roofline": {
            "kernel": "grouped gate/up + SwiGLU per call (batch_gateup_kernel, plus pair_gateup_kernel for the "
                      "experts with a single entry in calls with 16-entry tiles)",
            "bound": "hbm",
            "achieved": round(gu_gbs, 1),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(gu_gbs / HBM_PEAK_GBS, 4),
            "traffic": traffic,
            "bytes_per_launch": int(round(gu_bytes / kn[4])),
            "avg_launch_us": round(1e3 * gu_ms / kn[4], 3),
            "mfma_tflops": round(gu_tf, 2),
            "mfma_frac_of_fp16_dense_peak": round(gu_tf / 2500.0, 4),
            "mfma_counters": mfma,
        },
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)
    layer.close()
    return 0


def bench_decode(args) -> int:
    import numpy as np
    import torch

    from routed_expert_int4_amd import binding as B
    from routed_expert_int4_amd import synth
    from routed_expert_int4_amd.layer import DeviceLayer

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    import dataclasses
    cfg = dataclasses.replace(synth.GLM, top_p=args.top_p, codec=args.codec)
    nbytes = algorithmic_bytes(cfg)
    log("generating the GLM-shaped layer (seed 0) and 1000 tokens (seed 1)")
    weights = synth.gen_layer(cfg, seed=0)
    x_bits = synth.gen_tokens(cfg, args.tokens, seed=1)
    layer = DeviceLayer(weights, max_T=1)
    x = DeviceLayer.to_device_bf16(x_bits)
    y = torch.empty((args.tokens, cfg.hidden), dtype=torch.float32, device="cuda:0")
    ids = torch.empty((args.tokens, cfg.top_k), dtype=torch.int32, device="cuda:0")
    w = torch.empty((args.tokens, cfg.top_k), dtype=torch.float32, device="cuda:0")
    stream = torch.cuda.current_stream()
    if args.copy_calibration:
        src = torch.empty(256 << 20, dtype=torch.uint8, device="cuda:0")
        dst = torch.empty_like(src)
        src.fill_(1)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    # one call per token (batch-1 decode): pointers of token t's rows
    H, k = cfg.hidden, cfg.top_k
    px, py, pi, pw = x.data_ptr(), y.data_ptr(), ids.data_ptr(), w.data_ptr()
    st = stream.cuda_stream
    fwd = B.lib().moe_layer_forward

    def step():
        for t in range(args.tokens):
            rc = fwd(layer.handle, px + 2 * H * t, 1, py + 4 * H * t, pi + 4 * k * t, pw + 4 * k * t, st)
            if rc != 0:
                raise B.MoeError(rc, B.last_error())

    def kernel_avg_us():
        """Per-kind average launch duration (us) over one step, from HIP
        events stamped with each kernel's own begin and end on the launch
        stream (None for a kind that did not run)."""
        B.moe_layer_profile(layer.handle, True)
        step()
        torch.cuda.synchronize()
        kms, kn = B.moe_layer_profile_read(layer.handle)
        B.moe_layer_profile(layer.handle, False)
        return [1e3 * kms[k] / kn[k] if kn[k] else None for k in range(len(kn))]

    def time_mode(launches, warmup):
        """Steps of one decode mode: ms per step, tokens/s and the launches'
        average durations."""
        B.moe_layer_set_decode(layer.handle, launches)
        for _ in range(warmup):
            step()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        t0 = time.perf_counter()
        e0.record(stream)
        for _ in range(args.steps):
            step()
        e1.record(stream)
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        ms_total = e0.elapsed_time(e1)
        return {"ms_per_step": ms_total / args.steps, "tokens_per_s": args.tokens * args.steps / (ms_total / 1e3),
                "wall": wall, "avg_us": kernel_avg_us()}

    # what each mode's launches are and the bytes each must move
    KINDS = {1: [(3, "fused_one_token", "layer_per_token")],
             2: [(0, "router_shared_gateup", "router_launch"), (8, "gateup_down_combine", "gateup_down_launch")],
             3: [(0, "router_shared_gateup", "router_launch"), (1, "gateup_swiglu", "gateup_launch"),
                 (2, "down_combine", "down_launch")]}
    ROOFLINE_KERNEL = {
        1: (3, "the whole layer in one fused launch (fused_decode_kernel<192, 64, 24, 4, 0, 8>)",
            "void moe::(anonymous namespace)::fused_decode_kernel<192, 64, 24, 4, 0, 8>", "layer_per_token"),
        2: (8, "routed gate/up + SwiGLU, down projections of the 8 routed and the shared expert and the combine "
               "(gateup_down_kernel<192, 64, 24, 0>)",
            "void moe::(anonymous namespace)::gateup_down_kernel<192, 64, 24, 0>", "gateup_down_launch"),
        3: (1, "gate/up + SwiGLU of the 8 routed experts (gateup_kernel<192>)",
            "void moe::(anonymous namespace)::gateup_kernel<192, 0>", "gateup_launch")}

    def ran_mode(avg):
        """The mode the launches show (a mode without an instance for the
        shape or codec falls back to three launches)."""
        return 1 if avg[3] else (2 if avg[8] else 3)

    def mode_summary(r):
        m = ran_mode(r["avg_us"])
        kern = {name: round(r["avg_us"][k], 3) for k, name, _ in KINDS[m]}
        gbs = {name: round(nbytes[b] / (r["avg_us"][k] * 1e-6) / 1e9, 1) for k, name, b in KINDS[m]}
        return {"launches_per_token": m, "ms_per_step": round(r["ms_per_step"], 4),
                "tokens_per_s": round(r["tokens_per_s"], 1),
                "layer_gbs": round(r["tokens_per_s"] * nbytes["layer_per_token"] / 1e9, 2),
                "kernels_avg_us": kern, "kernels_gbs": gbs}

    log(f"warmup {args.warmup} step(s), decode mode {args.decode_launches}")
    log(f"timing {args.steps} step(s) of {args.tokens} tokens")
    main_run = time_mode(args.decode_launches, args.warmup)
    ids_main = ids.clone()
    ms_per_step = main_run["ms_per_step"]
    tokens_per_s = main_run["tokens_per_s"]
    mode = ran_mode(main_run["avg_us"])
    # with the top-p cut only the kept routed experts are read: price the
    # routed bytes by the mean kept count (every step routes the same tokens)
    kept = float((ids_main >= 0).sum().item()) / args.tokens
    if kept != cfg.top_k:
        scale_down = (kept + cfg.n_shared) / (cfg.top_k + cfg.n_shared)
        gu_kept = int(round(nbytes["gateup_launch"] * kept / cfg.top_k))
        dn_kept = int(round(nbytes["down_launch"] * scale_down))
        nbytes["routed_per_token"] = int(round(nbytes["routed_per_token"] * kept / cfg.top_k))
        nbytes["layer_per_token"] -= int(round((cfg.top_k - kept) * nbytes["expert"]))
        nbytes["gateup_launch"], nbytes["down_launch"] = gu_kept, dn_kept
        nbytes["gateup_down_launch"] = gu_kept + dn_kept
    routed_gbs = tokens_per_s * nbytes["routed_per_token"] / 1e9
    layer_gbs = tokens_per_s * nbytes["layer_per_token"] / 1e9
    log(f"{ms_per_step:.3f} ms/step, {tokens_per_s:.0f} tokens/s, routed {routed_gbs:.0f} GB/s "
        f"(wall {main_run['wall']:.2f} s), launches {mode}: {main_run['avg_us']}")
    main_summary = mode_summary(main_run)
    # the other decode modes on the same tokens, for comparison (bit-identical
    # results)
    others = {}
    for m in (3, 2, 1):
        if m != args.decode_launches:
            r = time_mode(m, max(1, args.warmup))
            others[str(m)] = mode_summary(r)
            log(f"decode mode {m}: {r['ms_per_step']:.3f} ms/step, kernels {others[str(m)]['kernels_avg_us']}")
    B.moe_layer_set_decode(layer.handle, args.decode_launches)
    rk, rdesc, rname, rbytes = ROOFLINE_KERNEL[mode]
    roof_us = main_run["avg_us"][rk]
    roof_gbs = nbytes[rbytes] / (roof_us * 1e-6) / 1e9

    cpu = None
    if args.cpu_sample > 0:
        n = min(args.cpu_sample, args.tokens)
        log(f"timing the CPU oracle on {n} tokens")
        cpu = cpu_baseline(weights, x_bits, n, nbytes["routed_per_token"])
        log(f"oracle: {cpu['tokens_per_s']} tokens/s on {cpu['cores']} threads")

    out = {
        "metric": METRIC,
        "value": round(routed_gbs, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": DTYPES[cfg.codec],
        "data": "synthetic (seeded: weights seed 0, tokens seed 1)",
        "config": {
            "workload": f"GLM-5.2-shaped MoE layer, batch-1 {cfg.codec} decode, 1000 independent tokens per step"
                        + (f", adaptive expert top-p {cfg.top_p}" if cfg.top_p < 1.0 else ""),
            "hidden": cfg.hidden, "expert_intermediate": cfg.inter, "routed_experts": cfg.n_experts,
            "groups": cfg.n_groups, "topk_group": cfg.topk_group, "top_k": cfg.top_k, "shared_experts": cfg.n_shared,
            "tokens_per_step": args.tokens, "parallelism": "single GPU",
        },
        "routed_experts_kept_per_token": round(kept, 3),
        "tokens_per_s": round(tokens_per_s, 1),
        "pct_of_hbm_peak": round(100 * routed_gbs / HBM_PEAK_GBS, 2),
        "layer_gbs": round(layer_gbs, 2),
        "layer_frac_of_hbm_peak": round(layer_gbs / HBM_PEAK_GBS, 4),
        "bytes_per_token": {"routed": nbytes["routed_per_token"], "layer": nbytes["layer_per_token"]},
        "decode_launches_per_token": mode,
        "kernels_avg_us": main_summary["kernels_avg_us"],
        "kernels_gbs": main_summary["kernels_gbs"],
        "other_decode_modes": others,
        "roofline": {
            "kernel": rdesc,
            "bound": "hbm",
            "achieved": round(roof_gbs, 1),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(roof_gbs / HBM_PEAK_GBS, 4),
            "traffic": measured_traffic(rname) if cfg.top_p >= 1.0 and cfg.codec == "int4" else None,
            "bytes_per_launch": nbytes[rbytes],
            "avg_launch_us": round(roof_us, 3),
        },
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)
    layer.close()
    return 0


if __name__ == "__main__":
    sys.exit(main())
