#!/usr/bin/env python3
"""Benchmark of the routed ternary-expert FFN on one MI355X.

Default workload (the headline metric): decode of the 24-layer MoE stack at
batch 1 (hidden 2048, 256 experts, top-8, intermediate 512), one captured HIP
graph step per token, 256 staged tokens with independent seeded bf16 inputs.
A step is one token through all 24 layers: router, softmax/top-8, grouping,
gate/up + SwiGLU, down projection and weighted combine with the residual.

Prints one JSON line (rank 0).  ``--workload prefill_4096`` times one
4096-token layer instead.  Inputs are synthetic and seeded; weights are
generated in host memory, packed on the device and stay resident in HBM
before the timed region starts.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "decode tok/s, 24-layer ternary MoE stack bs=1; % HBM peak; prefill tok/s"
HBM_PEAK_GBS = 8000.0
INT8_PEAK_TOPS = 5000.0


def log(msg):
    print(f"[bench {time.strftime('%H:%M:%S')}] {msg}", file=sys.stderr, flush=True)


def decode_bytes_per_token_layer(H, E, k, I, T=1):
    """Algorithmic HBM bytes of one layer for T tokens when every token's
    experts are distinct: k experts' packed weights and alphas, the fp32
    router, x read and the output written (fp32)."""
    expert = 3 * H * I // 4 + 4 * (2 * I + H)
    return k * T * expert + 4 * E * H + 2 * 4 * T * H


def build_layers(w, torch, N, S):
    layers = []
    for l in range(w.n_layers):
        W = S.gen_layer_weights(w, l)
        wt = torch.from_numpy(W.reshape(-1)).cuda()
        packed = torch.empty(W.size // 4, dtype=torch.uint8, device="cuda")
        N.maple_ternary_pack_device(wt, packed)
        del wt, W
        bias = S.gen_router_bias(w, l)
        layers.append(dict(
            Wr=torch.from_numpy(S.gen_router(w, l)).cuda(),
            bias=None if bias is None else torch.from_numpy(bias).cuda(),
            packed=packed, alpha=torch.from_numpy(S.gen_alpha(w, l)).cuda()))
        if l % 6 == 5 or l == w.n_layers - 1:
            log(f"layer {l + 1}/{w.n_layers} generated and packed on the device")
    torch.cuda.synchronize()
    return layers


def cpu_baseline_decode(w, budget_s):
    """The oracle (fp64 C, OpenMP) on a bounded sample: a few tokens through
    the full 24-layer stack, tok/s on this host."""
    import oracle
    from ternary_weight_moe_amd import synth as S
    log("cpu baseline: packing the stack for the oracle")
    Wr, bias, packed, alpha = [], [], [], []
    for l in range(w.n_layers):
        W = S.gen_layer_weights(w, l)
        packed.append(oracle.pack_layer(W, w.hidden, w.inter))
        del W
        Wr.append(S.gen_router(w, l))
        bias.append(S.gen_router_bias(w, l))
        alpha.append(S.gen_alpha(w, l))
    n, t_used = 0, 0.0
    while t_used < budget_s and n < 256:
        x = S.x_as_f32(w, S.gen_x(w, 1, token0=n)).astype(np.float64)
        t0 = time.perf_counter()
        oracle.moe_stack(x, Wr, bias, packed, alpha, k=w.top_k, inter=w.inter,
                         keep_logits=False, keep_delta=False)
        t_used += time.perf_counter() - t0
        n += 1
    return dict(value=n / t_used, unit="tok/s", cores=oracle.num_threads(), kind="oracle",
                sample=f"{n} tokens x {w.n_layers} layers, one token per call ({t_used:.1f} s)")


def bench_decode(args, torch, N, S):
    w = S.WORKLOADS["decode_stack"]
    H, E, k, I, L = w.hidden, w.n_experts, w.top_k, w.inter, w.n_layers
    layers = build_layers(w, torch, N, S)
    n_staged = w.n_tokens
    xs = S.gen_x(w, n_staged)
    staged = torch.from_numpy(xs.view(np.int16)).cuda().view(torch.bfloat16).reshape(n_staged, 1, H)
    d = N.make_dims(H, E, k, I, N.MAPLE_X_BF16)
    ws = torch.empty(N.maple_moe_workspace_bytes(d, 1), dtype=torch.uint8, device="cuda")
    x_work = torch.empty(1, H, dtype=torch.float32, device="cuda")
    out_all = torch.empty(n_staged, 1, H, dtype=torch.float32, device="cuda")
    g = N.MapleGraph(d, 1, staged, n_staged, x_work, out_all, [l["Wr"] for l in layers],
                     None, [l["packed"] for l in layers], [l["alpha"] for l in layers], ws)
    stream = torch.cuda.current_stream()
    for _ in range(args.warmup):
        g.launch(stream)
    torch.cuda.synchronize()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record(stream)
    for _ in range(args.steps):
        g.launch(stream)
    end.record(stream)
    torch.cuda.synchronize()
    ms = start.elapsed_time(end)
    ms_per_step = ms / args.steps
    tok_s = 1000.0 / ms_per_step
    assert torch.isfinite(out_all).all().item()
    bytes_tok = L * decode_bytes_per_token_layer(H, E, k, I)
    achieved = bytes_tok / (ms_per_step * 1e-3) / 1e9
    g.destroy()
    res = dict(
        metric=METRIC, value=tok_s, unit="tok/s", n_gpus=1, steps=args.steps,
        warmup=args.warmup, ms_per_step=ms_per_step, higher_is_better=True, scaling="weak",
        vs_baseline=None, dtype="f32", data="synthetic",
        config=dict(workload="decode_stack", hidden=H, experts=E, top_k=k, inter=I, layers=L,
                    batch=1, tokens_staged=n_staged, graph_steps=True),
        roofline=dict(bound="hbm", achieved=achieved, peak=HBM_PEAK_GBS, unit="GB/s",
                      frac=achieved / HBM_PEAK_GBS, traffic=None,
                      kernel="whole captured decode step",
                      algorithmic_bytes_per_launch=bytes_tok),
    )
    return res, w


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=256)
    ap.add_argument("--warmup", type=int, default=16)
    ap.add_argument("--workload", default="decode_stack", choices=["decode_stack"])
    ap.add_argument("--cpu-baseline-seconds", type=float, default=15.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    args = ap.parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU: this build has no multi-GPU path "
              "(every token is independent; see DESIGN.md for how it would shard). "
              "Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)
    import torch
    from ternary_weight_moe_amd import _native as N
    from ternary_weight_moe_amd import synth as S
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    N.load()  # fails loudly if the HIP library is missing
    res, w = bench_decode(args, torch, N, S)
    log(f"{res['value']:.1f} tok/s, {res['ms_per_step'] * 1000:.1f} us/step")
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline_decode(w, args.cpu_baseline_seconds)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
