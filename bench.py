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
                  for f in ("moe_decode.hip", "moe_kernels.h", "moe_layout.h")]


def algorithmic_bytes(cfg):
    """Bytes each stage must move at least once per token (batch 1).

    Weights dominate: gate + up codes and scales of the 8 routed experts and
    the shared expert for the gate/up launch, their down codes and scales
    for the down launch, the fp32 router matrix for the router launch.  The
    activations (bf16 x, fp32 h and y) are counted where a launch reads or
    writes them.
    """
    eb = cfg.expert_bytes()
    n = cfg.top_k + cfg.n_shared
    gu = 2 * (cfg.hidden * cfg.inter // 2 + cfg.inter * (cfg.hidden // 32) * 2)  # gate + up, codes + scales
    dn = cfg.hidden * cfg.inter // 2 + cfg.hidden * (cfg.inter // 32) * 2
    router = cfg.n_experts * cfg.hidden * 4 + cfg.n_experts * 4
    io = cfg.hidden * 2 + cfg.hidden * 4
    return {
        "expert": eb,
        "routed_per_token": cfg.top_k * eb,
        "layer_per_token": router + n * eb + io,
        "router_launch": router + cfg.hidden * 2,
        "gateup_launch": n * gu,
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
    size, and the digest of the kernel source they were taken on.  Returns
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
    return {
        "value": round(tps * bytes_per_token / 1e9, 4),
        "unit": "GB/s",
        "tokens_per_s": round(tps, 3),
        "cores": threads,
        "kind": "oracle",
        "sample": f"first {n_tokens} of the 1000 tokens, full layer in fp64 (router, top-k, 8 routed + shared "
                  f"experts, combine), {dt:.1f} s",
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
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only: --gpus {args.gpus} is not supported (this layer's path is "
              "single-GPU; sharding over more GPUs is not built)", file=sys.stderr)
        return 2

    import numpy as np
    import torch

    from routed_expert_int4_amd import binding as B
    from routed_expert_int4_amd import synth
    from routed_expert_int4_amd.layer import DeviceLayer

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    cfg = synth.GLM
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

    # parity spot check of this very run against the oracle (2 tokens)
    from oracle import oracle
    ref = oracle.layer_forward(weights, x_bits[:2])
    yh = y[:2].cpu().numpy().astype(np.float64)
    rel = float(max(np.abs(yh[t] - ref["y"][t]).max() / np.abs(ref["y"][t]).max() for t in range(2)))
    ids_ok = bool(np.array_equal(ids[:2].cpu().numpy(), ref["ids"]))

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
        "dtype": "int4 weights x fp16 activations, fp32 accumulate",
        "data": "synthetic (seeded: weights seed 0, tokens seed 1)",
        "config": {
            "workload": "GLM-5.2-shaped MoE layer, batch-1 int4 decode, 1000 independent tokens per step",
            "hidden": cfg.hidden, "expert_intermediate": cfg.inter, "routed_experts": cfg.n_experts,
            "groups": cfg.n_groups, "topk_group": cfg.topk_group, "top_k": cfg.top_k, "shared_experts": cfg.n_shared,
            "tokens_per_step": args.tokens, "parallelism": "single GPU",
        },
        "tokens_per_s": round(tokens_per_s, 1),
        "pct_of_hbm_peak": round(100 * routed_gbs / HBM_PEAK_GBS, 2),
        "layer_gbs": round(layer_gbs, 2),
        "bytes_per_token": {"routed": nbytes["routed_per_token"], "layer": nbytes["layer_per_token"]},
        "kernels_avg_us": {"router": round(avg_us[0], 3), "gateup_swiglu": round(avg_us[1], 3),
                           "down_combine": round(avg_us[2], 3)},
        "kernels_gbs": {"router": round(router_gbs, 1), "gateup_swiglu": round(gateup_gbs, 1),
                        "down_combine": round(down_gbs, 1)},
        "roofline": {
            "kernel": "gate/up + SwiGLU of the 8 routed experts and the shared expert (gateup_kernel<192,4,true>)",
            "bound": "hbm",
            "achieved": round(gateup_gbs, 1),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(gateup_gbs / HBM_PEAK_GBS, 4),
            "traffic": measured_traffic(),
            "bytes_per_launch": nbytes["gateup_launch"],
            "avg_launch_us": round(avg_us[1], 3),
        },
        "parity_spot": {"tokens": 2, "ids_equal": ids_ok, "max_rel_err": rel},
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)
    layer.close()
    return 0


if __name__ == "__main__":
    sys.exit(main())
