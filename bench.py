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


TRAFFIC_RECORD = os.path.join(ROOT, "profiles", "gateup_kernel_glm_decode_traffic.md")
KERNEL_SOURCES = [os.path.join(ROOT, "routed_expert_int4_amd", "csrc", f)
                  for f in ("moe_decode.hip", "moe_device.h", "moe_kernels.h", "moe_layout.h")]


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
    }


def source_digest() -> str:
    import hashlib
    h = hashlib.sha256()
    for path in KERNEL_SOURCES:
        with open(path, "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def measured_traffic():
    """HBM bytes per gate/up launch from the committed rocprofv3 counter record.

    The record holds FETCH_SIZE and WRITE_SIZE per dispatch of the gate/up
    kernel, each scaled by what the counter reads for a device copy of known
    size, and the digest of the kernel sources they were taken on.  Returns
    None when there is no record or the kernel source has changed since.
    """
    if not os.path.exists(TRAFFIC_RECORD):
        return None
    rec = None
    with open(TRAFFIC_RECORD) as f:
        for line in f:
            if line.startswith("traffic-record:"):
                rec = json.loads(line.split(":", 1)[1])
    if not rec or rec.get("source_sha256") != source_digest():
        return None
    return int(rec["hbm_bytes_per_launch"])


def cpu_baseline(weights, x_bits, n_tokens: int, bytes_per_token: int):
    from oracle import oracle
    threads = int(os.environ.get("OMP_NUM_THREADS", "0")) or len(os.sched_getaffinity(0))
    sample = x_bits[:n_tokens]
    oracle.layer_forward(weights, sample[:1], n_threads=threads)  # load + warm
    t0 = time.perf_counter()
    oracle.layer_forward(weights, sample, n_threads=threads)
    dt = time.perf_counter() - t0
    tps = n_tokens / dt
    # one thread on a short prefix, for the per-core figure
    n1 = max(1, min(16, n_tokens))
    t1 = time.perf_counter()
    oracle.layer_forward(weights, sample[:n1], n_threads=1)
    dt1 = time.perf_counter() - t1
    cpu_model = ""
    try:
        with open("/proc/cpuinfo") as f:
            cpu_model = next((l.split(":", 1)[1].strip() for l in f if l.startswith("model name")), "")
    except OSError:
        pass
    return {
        "value": round(tps * bytes_per_token / 1e9, 4),
        "unit": "GB/s",
        "tokens_per_s": round(tps, 3),
        "cores": threads,
        "kind": "oracle",
        "sample": f"first {n_tokens} of the 1000 tokens, full layer in fp64 (router, top-k, 8 routed + shared "
                  f"experts, combine), {dt:.1f} s",
        "tokens_per_s_1_thread": round(n1 / dt1, 3),
        "cpu_model": cpu_model,
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
    ap.add_argument("--codec", default="int4", choices=["int4", "mxfp4", "int8", "int2"],
                    help="decode and cache-stack: expert weight codec (mxfp4: E2M1 codes, E8M0 scales; int8, "
                         "int2: one byte or 2 bits per weight, fp16 scales)")
    ap.add_argument("--top-p", type=float, default=1.0,
                    help="decode and cache-stack: adaptive expert top-p (1: plain top-k); decode prices its bytes "
                         "by the experts kept")
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
    from a cold start (reported as lru_only).  --pin 0 times plain LRU only."""
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
    t0 = time.perf_counter()
    for l in range(n_layers):
        w = synth.gen_layer(cfg, seed=100 + l)
        w.bias = biases[l]
        cache.register(l, HostExpertStore(w))
        lay = DeviceLayer(w, max_T=1, resident=False)
        lay.attach_cache(cache, l)
        layers.append(lay)
        del w
        log(f"layer {l} ready ({time.perf_counter() - t0:.0f} s)")
    H = cfg.hidden
    y = torch.empty((1, H), dtype=torch.float32, device="cuda:0")
    ids = torch.empty((1, cfg.top_k), dtype=torch.int32, device="cuda:0")
    w = torch.empty((1, cfg.top_k), dtype=torch.float32, device="cuda:0")
    stream = torch.cuda.current_stream()

    def decode(x_seed, noise_seed, n):
        """n sequential tokens through the stack; returns (ms, stats at n/2)."""
        x0 = DeviceLayer.to_device_bf16(synth.gen_tokens(cfg, n, seed=x_seed))
        noise = torch.from_numpy(synth.gen_noise(cfg, n * n_layers, seed=noise_seed, std=0.1)).to("cuda:0")
        half = None
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for t in range(n):
            if t == n // 2:
                half = [cache.stats(l) for l in range(n_layers)]
            x = x0[t:t + 1]
            for l in range(n_layers):
                B.moe_layer_forward(layers[l].handle, x, 1, y, ids, w, stream)
                rms = torch.sqrt(torch.mean(y * y, dim=1, keepdim=True))
                x = (y / rms + noise[t * n_layers + l:t * n_layers + l + 1]).to(torch.bfloat16)
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1), half

    def totals(stats):
        return {k: sum(st[k] for st in stats) for k in ("hits", "misses", "h2d_bytes")}

    def measured(label):
        before = totals([cache.stats(l) for l in range(n_layers)])
        log(f"{label}: decoding {n_tok} tokens through {n_layers} cached layers")
        ms, half = decode(300, 400, n_tok)
        after = totals([cache.stats(l) for l in range(n_layers)])
        mid = totals(half)
        d = {k: after[k] - before[k] for k in after}
        d2 = {k: after[k] - mid[k] for k in after}
        r = {"tokens_per_s": n_tok / (ms / 1e3), "ms": ms, "routed_uses_per_token_layer":
             (d["hits"] + d["misses"]) / (n_tok * n_layers),
             "hit_rate": d["hits"] / max(d["hits"] + d["misses"], 1),
             "hit_rate_second_half": d2["hits"] / max(d2["hits"] + d2["misses"], 1),
             "h2d_bytes": d["h2d_bytes"], "h2d_gbs": d["h2d_bytes"] / (ms / 1e3) / 1e9}
        log(f"{label}: {r['tokens_per_s']:.1f} tokens/s, hit rate {r['hit_rate']:.4f}, "
            f"H2D {r['h2d_bytes'] / 1e9:.1f} GB at {r['h2d_gbs']:.1f} GB/s")
        return r

    def empty_cache():
        for l in range(n_layers):
            cache.unpin(l, list(range(cfg.n_experts)))
            for e in range(cfg.n_experts):
                cache.evict(l, e)

    pinned = None
    pin_load_s = 0.0
    if n_pin > 0:
        log(f"learning pass: {args.learn_tokens} tokens")
        decode(310, 410, args.learn_tokens)
        empty_cache()
        p0 = time.perf_counter()
        for l in range(n_layers):
            cache.autopin(l, n_pin)
        torch.cuda.synchronize()
        pin_load_s = time.perf_counter() - p0
        pinned = measured(f"autopin {n_pin}")
        empty_cache()
    lru_only = measured("plain LRU")
    main_run = pinned if pinned else lru_only
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
                               + (f", {cfg.codec} experts" if cfg.codec != "int4" else ""),
                   "layers": n_layers, "slots_per_layer": slots, "pinned_per_layer": n_pin,
                   "learning_tokens": args.learn_tokens if n_pin > 0 else 0, "tokens": n_tok},
        "hit_rate": round(main_run["hit_rate"], 4),
        "hit_rate_second_half": round(main_run["hit_rate_second_half"], 4),
        "h2d_gbytes": round(main_run["h2d_bytes"] / 1e9, 3),
        "h2d_gbs": round(main_run["h2d_gbs"], 2),
        "pin_load_s": round(pin_load_s, 3),
        "lru_only": {k: round(v, 4) for k, v in lru_only.items()},
        "roofline": {"kernel": "host-to-device expert copies (hipMemcpyAsync, pinned host)", "bound": "pcie",
                     "achieved": round(main_run["h2d_gbs"], 2), "peak": 64.0, "unit": "GB/s",
                     "frac": round(main_run["h2d_gbs"] / 64.0, 4), "traffic": None},
        "cpu_baseline": None,
    }
    print(json.dumps(out), flush=True)
    for lay in layers:
        lay.close()
    cache.close()
    return 0


def bench_probes(args) -> int:
    """Device ceilings the layer's numbers are read against (one JSON line):
    HBM GB/s of a device-to-device copy (bytes read + bytes written) over
    buffers the size of the decode launches (56 MB, 113 MB) and of 1 GiB;
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

    read = {}
    for label, nbytes in (("56MB", 56_623_104), ("113MB", 113_246_208), ("1GiB", 1 << 30)):
        src = torch.ones(nbytes // 4, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        ms = best_ms(lambda: dst.copy_(src))
        read[label] = round(2 * nbytes / (ms / 1e3) / 1e9, 1)
        del src, dst
    host = torch.empty(256 << 20, dtype=torch.uint8, pin_memory=True)
    devb = torch.empty(256 << 20, dtype=torch.uint8, device=dev)
    h2d = (256 << 20) / (best_ms(lambda: devb.copy_(host, non_blocking=True)) / 1e3) / 1e9
    d2h = (256 << 20) / (best_ms(lambda: host.copy_(devb, non_blocking=True)) / 1e3) / 1e9
    n = 8192
    a = torch.randn(n, n, dtype=torch.bfloat16, device=dev)
    b = torch.randn(n, n, dtype=torch.bfloat16, device=dev)
    gemm = 2 * n ** 3 / (best_ms(lambda: torch.matmul(a, b)) / 1e3) / 1e12
    out = {
        "metric": "device ceilings: HBM copy GB/s (read + write), pinned host copy GB/s, bf16 GEMM TFLOP/s",
        "value": read["1GiB"], "unit": "GB/s", "n_gpus": 1, "steps": 10, "warmup": 3,
        "higher_is_better": True, "data": "synthetic",
        "config": {"workload": "probes: device-to-device copies, pinned 256 MiB copies, 8192^3 bf16 matmul"},
        "hbm_copy_gbs": read, "h2d_gbs": round(h2d, 1), "d2h_gbs": round(d2h, 1), "bf16_gemm_tflops": round(gemm, 1),
        "vs_peak": {"hbm_copy_1GiB": round(read["1GiB"] / HBM_PEAK_GBS, 4), "bf16_gemm": round(gemm / 2500.0, 4)},
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
    eb = cfg.expert_bytes()
    router = cfg.n_experts * cfg.hidden * 4 + cfg.n_experts * 4
    bytes_step = sum(router + (d + cfg.n_shared) * eb + T * H * 6 for d in distinct)
    kept_entries = int((ids_h >= 0).sum())
    flops_step = (kept_entries + n_calls * T * cfg.n_shared) * 2 * 3 * H * cfg.inter
    tokens_per_s = n_calls * T * args.steps / (ms_per_step * args.steps / 1e3)
    gbs = bytes_step / (ms_per_step / 1e3) / 1e9
    tflops = flops_step / (ms_per_step / 1e3) / 1e12
    # per-stage durations (events around each stage of each call)
    B.moe_layer_profile(layer.handle, True)
    step()
    torch.cuda.synchronize()
    kms, kn = B.moe_layer_profile_read(layer.handle)
    B.moe_layer_profile(layer.handle, False)
    stage_ms = [kms[i] for i in range(3)]
    grouped_ms = stage_ms[1] + stage_ms[2]
    log(f"{ms_per_step:.3f} ms/step, {tokens_per_s:.0f} tokens/s, {gbs:.0f} GB/s, {tflops:.1f} TFLOP/s; "
        f"stages ms {stage_ms}; distinct experts per call {min(distinct)}..{max(distinct)}")
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
                   + (f", adaptive expert top-p {cfg.top_p}" if cfg.top_p < 1.0 else ""), "tokens_per_call": T, "calls_per_step": n_calls, "hidden": H,
                   "expert_intermediate": cfg.inter, "routed_experts": cfg.n_experts, "top_k": k},
        "tokens_per_s": round(tokens_per_s, 1),
        "pct_of_hbm_peak": round(100 * gbs / HBM_PEAK_GBS, 2),
        "distinct_experts_per_call": {"min": min(distinct), "max": max(distinct),
                                      "mean": round(float(np.mean(distinct)), 2)},
        "tflops": round(tflops, 2),
        "stage_ms_per_step": {"routing_dispatch": round(stage_ms[0], 4), "gateup_hprep": round(stage_ms[1], 4),
                              "down_combine": round(stage_ms[2], 4)},
        "roofline": {
            "kernel": "grouped gate/up + down (batch_gateup_kernel, batch_down_kernel)",
            "bound": "hbm",
            "achieved": round(bytes_step / (grouped_ms / 1e3) / 1e9, 1),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(bytes_step / (grouped_ms / 1e3) / 1e9 / HBM_PEAK_GBS, 4),
            "traffic": None,
            "mfma_tflops": round(flops_step / (grouped_ms / 1e3) / 1e12, 2),
            "mfma_frac_of_fp16_dense_peak": round(flops_step / (grouped_ms / 1e3) / 1e12 / 2500.0, 4),
        },
        "cpu_baseline": None,
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

    log(f"warmup {args.warmup} step(s)")
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    log(f"timing {args.steps} step(s) of {args.tokens} tokens")
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record(stream)
    for _ in range(args.steps):
        step()
    e1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_total = e0.elapsed_time(e1)
    ms_per_step = ms_total / args.steps
    tokens_per_s = args.tokens * args.steps / (ms_total / 1e3)
    # with the top-p cut only the kept routed experts are read: price the
    # routed bytes by the mean kept count (every step routes the same tokens)
    kept = float((ids >= 0).sum().item()) / args.tokens
    if kept != cfg.top_k:
        for key in ("routed_per_token", "gateup_launch"):
            nbytes[key] = int(round(nbytes[key] * kept / cfg.top_k))
        nbytes["layer_per_token"] -= int(round((cfg.top_k - kept) * nbytes["expert"]))
        nbytes["down_launch"] = int(round(nbytes["down_launch"] * (kept + cfg.n_shared) / (cfg.top_k + cfg.n_shared)))
    routed_gbs = tokens_per_s * nbytes["routed_per_token"] / 1e9
    layer_gbs = tokens_per_s * nbytes["layer_per_token"] / 1e9
    log(f"{ms_per_step:.3f} ms/step, {tokens_per_s:.0f} tokens/s, routed {routed_gbs:.0f} GB/s (wall {wall:.2f} s)")

    # per-kernel durations with HIP events on the launch stream (one step)
    B.moe_layer_profile(layer.handle, True)
    step()
    torch.cuda.synchronize()
    kms, kn = B.moe_layer_profile_read(layer.handle)
    B.moe_layer_profile(layer.handle, False)
    avg_us = [1e3 * kms[k] / max(kn[k], 1) for k in range(3)]
    gateup_gbs = nbytes["gateup_launch"] / (avg_us[1] * 1e-6) / 1e9
    down_gbs = nbytes["down_launch"] / (avg_us[2] * 1e-6) / 1e9
    router_gbs = nbytes["router_launch"] / (avg_us[0] * 1e-6) / 1e9
    log(f"kernel avg us: router {avg_us[0]:.2f} ({router_gbs:.0f} GB/s), gate/up {avg_us[1]:.2f} "
        f"({gateup_gbs:.0f} GB/s), down+combine {avg_us[2]:.2f} ({down_gbs:.0f} GB/s)")

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
        "bytes_per_token": {"routed": nbytes["routed_per_token"], "layer": nbytes["layer_per_token"]},
        "kernels_avg_us": {"router_shared_gateup": round(avg_us[0], 3), "gateup_swiglu": round(avg_us[1], 3),
                           "down_combine": round(avg_us[2], 3)},
        "kernels_gbs": {"router_shared_gateup": round(router_gbs, 1), "gateup_swiglu": round(gateup_gbs, 1),
                        "down_combine": round(down_gbs, 1)},
        "roofline": {
            "kernel": "gate/up + SwiGLU of the 8 routed experts (gateup_kernel<192>)",
            "bound": "hbm",
            "achieved": round(gateup_gbs, 1),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(gateup_gbs / HBM_PEAK_GBS, 4),
            "traffic": measured_traffic() if cfg.top_p >= 1.0 and cfg.codec == "int4" else None,
            "bytes_per_launch": nbytes["gateup_launch"],
            "avg_launch_us": round(avg_us[1], 3),
        },
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)
    layer.close()
    return 0


if __name__ == "__main__":
    sys.exit(main())
