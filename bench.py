#!/usr/bin/env python3
"""Benchmark of the routed ternary-expert FFN on one MI355X.

Default workload (the headline metric): decode of the 24-layer MoE stack at
batch 1 (hidden 2048, 256 experts, top-8, intermediate 512), one captured HIP
graph step per token, 256 staged tokens with independent seeded bf16 inputs.
A step is one token through all 24 pre-norm blocks: router, softmax/top-8,
grouping, gate/up + SwiGLU, down projection and weighted combine with the
residual.  ``--workload prefill_4096`` (or ``prefill_16384``) times one
layer over that many tokens instead; a step is then one layer call, replayed
from a captured HIP graph (the eager call's time is reported beside it).
``--workload batched_stack_zipf`` runs 64 tokens per step through the stack
with Zipf-skewed routing; ``--workload flashhead_decode`` times the clustered
output head alone, one token per call; ``--workload hybrid_attn_decode`` times
the attention of one decode step through the 24-layer sliding-window/global
pattern at 131,072 positions; ``--workload prefill_4096_a8`` is the 4096-token
layer with int8 activations; ``--workload ternary_convert`` converts one whole
layer of BF16 latent weights into ternary codes and alphas.

Prints one JSON line.  Inputs are synthetic and seeded; weights are generated
in host memory, packed on the device and resident in HBM before the timed
region starts.  After the timed region, a profiled pass of the same work
gives the dominant kernel's average duration for the roofline entry: for the
decode stack, replays of a second graph of the same step whose one-token
kernels stamp the GPU's real-time counter at every block's entry and exit
(graph mode, no eager launches); elsewhere HIP events around each kernel,
recorded by the library on the stream the kernel runs on.  The default
decode_stack line also carries a ``prefill_4096`` object (the 4096-token
layer, timed the same way as ``--workload prefill_4096``) unless
``--no-prefill`` is given, and a ``batched_stack_zipf`` object (64 tokens
per step through the stack, timed as ``--workload batched_stack_zipf``)
unless ``--no-batched`` is given.
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
HBM_PEAK_GBS = 8000.0      # MI355X HBM3E
INT8_PEAK_TOPS = 5000.0    # MI355X dense int8 MFMA
FP6_PEAK_TFLOPS = 10100.0  # MI355X dense fp6 / fp4 MFMA (the fast form's fp4 x fp6 products)


def log(msg):
    print(f"[bench {time.strftime('%H:%M:%S')}] {msg}", file=sys.stderr, flush=True)


# ---- algorithmic work per kernel launch ----------------------------------------------

def expert_bytes(H, I):
    """Packed ternary weights + fp32 alphas of one expert."""
    return 3 * H * I // 4 + 4 * (2 * I + H)


def decode_bytes(kernel, H, E, k, I, T=1):
    """Algorithmic HBM bytes of one launch of a decode-path kernel for T tokens
    whose k experts are all distinct (T * k experts read once)."""
    ne = T * k
    router = 4 * E * H + 4 * T * H + 4 * T * E
    gateup = ne * (2 * I * H // 4 + 4 * 2 * I) + 4 * T * H + 4 * ne * I
    down = ne * (H * I // 4 + 4 * H) + 4 * ne * I + 2 * 4 * T * H
    return {
        "d1_router": router, "d1_gateup": gateup + 4 * E, "d1_down": down,
        # two-kernel one-token path: the down kernel also reads the next
        # layer's router (its partial dots); the first layer's come from dec_router
        "dec_router": router, "dec_gateup": gateup + 4 * E, "dec_down": down + 4 * E * H,
        "router_gemv": 4 * E * H + 4 * T * H + 4 * T * E,
        "route_small": 4 * T * E + 4 * (3 * ne + 2 * E + 1),
        "gateup_gemv": ne * (2 * I * H // 4 + 4 * 2 * I) + 4 * T * H + 4 * ne * I,
        "down_combine_gemv": ne * (H * I // 4 + 4 * H) + 4 * ne * I + 2 * 4 * T * H,
    }.get(kernel)


def grouped_fine_bytes(kernel, H, E, k, I, T, D):
    """Algorithmic HBM bytes of one launch of a fine-form grouped kernel for T
    tokens whose slots fall on D distinct experts (each expert's weights read
    once): int8 limbs of x (3 planes), fp32 h and fp32 per-slot outputs."""
    Tk = T * k
    return {
        "quant_x": 4 * T * H + 3 * T * H + 20 * T,
        "gateup_mfma": D * (2 * I * H // 4 + 4 * 2 * I) + 3 * T * H + 20 * T + 4 * Tk * I,
        "down_mfma": D * (H * I // 4 + 4 * H) + 4 * Tk * I + 4 * Tk * H,
        "combine": 4 * Tk * H + 2 * 4 * T * H + 8 * Tk,
        "router_gemv": 4 * E * H + 4 * T * H + 4 * T * E,
    }.get(kernel)


def attn_bytes(Hq, Hkv, D, n):
    """Algorithmic HBM bytes of one decode-attention launch for one sequence
    attending to n positions: their keys and values (bf16, the new token's
    read from its input), the new key and value stored to the cache, the
    bf16 queries and the fp32 outputs.  Split partials are overhead, not
    counted."""
    return 2 * Hkv * n * D * 2 + 2 * Hkv * D * 2 + Hq * D * 2 + Hq * D * 4


def decode_bytes_per_token_layer(H, E, k, I):
    return k * expert_bytes(H, I) + 4 * E * H + 2 * 4 * H


def prefill_ops(kernel, H, k, I, T):
    """Algorithmic ops of one launch: 2 per multiply-add of a ternary weight with
    an activation, counted once (not once per digit plane or limb)."""
    return {"gateup_mfma": 2 * T * k * 2 * H * I, "down_mfma": 2 * T * k * H * I}.get(kernel)


# ---- measured HBM traffic --------------------------------------------------------------

# HBM bytes per launch of a kernel, from rocprofv3 --pmc runs of this script
# (summaries in profiles/*_traffic.md).  Reads: the L2's memory read requests
# counted by size (TCC_EA0_RDREQ_32B/_64B/_128B, weighted by their sizes),
# which a plain device copy of known size reproduces exactly; FETCH_SIZE's
# formula books this chip's 128-byte requests as 64 bytes (TCC_BUBBLE reads
# zero), so older entries scaled it by 2.0.  Writes: WRITE_SIZE, which the
# same copy reproduces unscaled.  An entry holds only while the kernel's
# sources hash as recorded; otherwise the kernel has changed since the
# counters were taken and the traffic is unknown.
TRAFFIC = {
    "decode_stack": {
        "dec_down": {"bytes": 4509757, "sources": ["decode1.hip", "digits.h", "internal.h", "limbs.h", "quant.h", "wave.h"], "digest": "c6fb03326e0be294"},
        "dec_gateup": {"bytes": 4742470, "sources": ["decode1.hip", "digits.h", "internal.h", "limbs.h", "quant.h", "wave.h"], "digest": "c6fb03326e0be294"},
        "dec_router": {"bytes": 2168254, "sources": ["decode1.hip", "digits.h", "internal.h", "limbs.h", "quant.h", "wave.h"], "digest": "c6fb03326e0be294"},
        "load_token": {"bytes": 13842, "sources": ["digits.h", "internal.h", "limbs.h", "misc.hip", "quant.h", "wave.h"], "digest": "bcde7b468f9449a2"},
        "store_token": {"bytes": 29588, "sources": ["digits.h", "internal.h", "limbs.h", "misc.hip", "quant.h", "wave.h"], "digest": "bcde7b468f9449a2"},
    },
    "prefill_4096": {
        "combine": {"bytes": 170791980, "sources": ["digits.h", "grouped.hip", "internal.h", "limbs.h", "quant.h", "wave.h"], "digest": "5543a65d10b19445"},
        "down_mfma": {"bytes": 244620696, "sources": ["digits.h", "grouped.hip", "internal.h", "limbs.h", "quant.h", "wave.h"], "digest": "5543a65d10b19445"},
        "gateup_mfma": {"bytes": 325966770, "sources": ["digits.h", "grouped.hip", "internal.h", "limbs.h", "quant.h", "wave.h"], "digest": "5543a65d10b19445"},
        "quant_x": {"bytes": 35893564, "sources": ["digits.h", "grouped.hip", "internal.h", "limbs.h", "quant.h", "wave.h"], "digest": "5543a65d10b19445"},
        "route_block": {"bytes": 343959, "sources": ["digits.h", "internal.h", "limbs.h", "quant.h", "route.hip", "wave.h"], "digest": "72b93e69c0213f7a"},
        "route_scan": {"bytes": 146366, "sources": ["digits.h", "internal.h", "limbs.h", "quant.h", "route.hip", "wave.h"], "digest": "72b93e69c0213f7a"},
        "route_scatter": {"bytes": 1209225, "sources": ["digits.h", "internal.h", "limbs.h", "quant.h", "route.hip", "wave.h"], "digest": "72b93e69c0213f7a"},
        "route_topk": {"bytes": 4488568, "sources": ["digits.h", "internal.h", "limbs.h", "quant.h", "route.hip", "wave.h"], "digest": "72b93e69c0213f7a"},
        "router_mfma": {"bytes": 37792632, "sources": ["digits.h", "internal.h", "limbs.h", "quant.h", "route.hip", "wave.h"], "digest": "72b93e69c0213f7a"},
        "split_router": {"bytes": 4206513, "sources": ["digits.h", "internal.h", "limbs.h", "quant.h", "route.hip", "wave.h"], "digest": "72b93e69c0213f7a"},
    },
    "prefill_4096_a8": {
        "combine": {"bytes": 170773632, "sources": ["digits.h", "grouped.hip", "internal.h", "limbs.h", "quant.h", "wave.h"], "digest": "5543a65d10b19445"},
        "down_mfma": {"bytes": 274868142, "sources": ["digits.h", "grouped.hip", "internal.h", "limbs.h", "quant.h", "wave.h"], "digest": "5543a65d10b19445"},
        "gateup_mfma": {"bytes": 268965192, "sources": ["digits.h", "grouped.hip", "internal.h", "limbs.h", "quant.h", "wave.h"], "digest": "5543a65d10b19445"},
        "quant_x": {"bytes": 25316412, "sources": ["digits.h", "grouped.hip", "internal.h", "limbs.h", "quant.h", "wave.h"], "digest": "5543a65d10b19445"},
        "route_block": {"bytes": 344000, "sources": ["digits.h", "internal.h", "limbs.h", "quant.h", "route.hip", "wave.h"], "digest": "72b93e69c0213f7a"},
        "route_scan": {"bytes": 146208, "sources": ["digits.h", "internal.h", "limbs.h", "quant.h", "route.hip", "wave.h"], "digest": "72b93e69c0213f7a"},
        "route_scatter": {"bytes": 1209440, "sources": ["digits.h", "internal.h", "limbs.h", "quant.h", "route.hip", "wave.h"], "digest": "72b93e69c0213f7a"},
        "route_topk": {"bytes": 4488576, "sources": ["digits.h", "internal.h", "limbs.h", "quant.h", "route.hip", "wave.h"], "digest": "72b93e69c0213f7a"},
        "router_mfma": {"bytes": 37792760, "sources": ["digits.h", "internal.h", "limbs.h", "quant.h", "route.hip", "wave.h"], "digest": "72b93e69c0213f7a"},
        "split_router": {"bytes": 4206784, "sources": ["digits.h", "internal.h", "limbs.h", "quant.h", "route.hip", "wave.h"], "digest": "72b93e69c0213f7a"},
    },
    "batched_stack_zipf": {
        "combine": {"bytes": 5270368, "sources": ["digits.h", "grouped.hip", "internal.h", "limbs.h", "quant.h", "wave.h"], "digest": "5543a65d10b19445"},
        "down_mfma": {"bytes": 39195102, "sources": ["digits.h", "grouped.hip", "internal.h", "limbs.h", "quant.h", "wave.h"], "digest": "5543a65d10b19445"},
        "gateup_mfma": {"bytes": 69929131, "sources": ["digits.h", "grouped.hip", "internal.h", "limbs.h", "quant.h", "wave.h"], "digest": "5543a65d10b19445"},
        "route_small": {"bytes": 2148644, "sources": ["digits.h", "internal.h", "limbs.h", "quant.h", "route.hip", "wave.h"], "digest": "72b93e69c0213f7a"},
        "router_split": {"bytes": 3694967, "sources": ["digits.h", "internal.h", "limbs.h", "quant.h", "route.hip", "wave.h"], "digest": "72b93e69c0213f7a"},
    },
    "hybrid_attn_decode": {
        "attn_combine": {"bytes": 1098556, "sources": ["attn.hip", "internal.h", "wave.h"], "digest": "a964e9de4f88bd05"},
        "attn_global": {"bytes": 269687732, "sources": ["attn.hip", "internal.h", "wave.h"], "digest": "a964e9de4f88bd05"},
        "attn_window": {"bytes": 1122883, "sources": ["attn.hip", "internal.h", "wave.h"], "digest": "a964e9de4f88bd05"},
    },
    "prefill_16384": {
        "combine": {"bytes": 694633812, "sources": ["digits.h", "grouped.hip", "internal.h", "limbs.h", "quant.h", "wave.h"], "digest": "5543a65d10b19445"},
        "down_mfma": {"bytes": 765244036, "sources": ["digits.h", "grouped.hip", "internal.h", "limbs.h", "quant.h", "wave.h"], "digest": "5543a65d10b19445"},
        "gateup_mfma": {"bytes": 912822520, "sources": ["digits.h", "grouped.hip", "internal.h", "limbs.h", "quant.h", "wave.h"], "digest": "5543a65d10b19445"},
        "quant_x": {"bytes": 143332496, "sources": ["digits.h", "grouped.hip", "internal.h", "limbs.h", "quant.h", "wave.h"], "digest": "5543a65d10b19445"},
        "route_block": {"bytes": 1327104, "sources": ["digits.h", "internal.h", "limbs.h", "quant.h", "route.hip", "wave.h"], "digest": "72b93e69c0213f7a"},
        "route_scan": {"bytes": 564576, "sources": ["digits.h", "internal.h", "limbs.h", "quant.h", "route.hip", "wave.h"], "digest": "72b93e69c0213f7a"},
        "route_scatter": {"bytes": 4767776, "sources": ["digits.h", "internal.h", "limbs.h", "quant.h", "route.hip", "wave.h"], "digest": "72b93e69c0213f7a"},
        "route_topk": {"bytes": 17858240, "sources": ["digits.h", "internal.h", "limbs.h", "quant.h", "route.hip", "wave.h"], "digest": "72b93e69c0213f7a"},
        "router_mfma": {"bytes": 253037740, "sources": ["digits.h", "internal.h", "limbs.h", "quant.h", "route.hip", "wave.h"], "digest": "72b93e69c0213f7a"},
        "split_router": {"bytes": 4207272, "sources": ["digits.h", "internal.h", "limbs.h", "quant.h", "route.hip", "wave.h"], "digest": "72b93e69c0213f7a"},
    },
    "flashhead_decode": {
        "head_final": {"bytes": 10688, "sources": ["head.hip", "internal.h", "wave.h"], "digest": "67332216d341ad8c"},
        "head_scores": {"bytes": 19559239, "sources": ["head.hip", "internal.h", "wave.h"], "digest": "67332216d341ad8c"},
        "head_search": {"bytes": 58789133, "sources": ["head.hip", "internal.h", "wave.h"], "digest": "67332216d341ad8c"},
        "head_select": {"bytes": 52057, "sources": ["head.hip", "internal.h", "wave.h"], "digest": "67332216d341ad8c"},
    },
    "ternary_convert": {
        "ternarize_g32": {"bytes": 606126446, "sources": ["convert.hip", "internal.h"], "digest": "030a18b7bb2f229e"},
        "ternarize_w2": {"bytes": 1209147332, "sources": ["convert.hip", "internal.h"], "digest": "030a18b7bb2f229e"},
    },
}


def source_digest(files):
    import hashlib
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(ROOT, "ternary_weight_moe_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def traffic_for(workload, kernel):
    ent = TRAFFIC.get(workload, {}).get(kernel)
    if ent is None or source_digest(ent["sources"]) != ent["digest"]:
        return None
    return ent["bytes"]


# ---- set-up ---------------------------------------------------------------------------

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


def oracle_layers(w):
    import oracle
    from ternary_weight_moe_amd import synth as S
    out = []
    for l in range(w.n_layers):
        W = S.gen_layer_weights(w, l)
        out.append(dict(Wr=S.gen_router(w, l), bias=S.gen_router_bias(w, l),
                        packed=oracle.pack_layer(W, w.hidden, w.inter), alpha=S.gen_alpha(w, l)))
        del W
    return out


GAP_RULE = 1e-4  # a token whose top-k logit gap falls below this in any layer is redrawn


def gap_rule_count(gaps):
    """gaps [L, T] of the sampled tokens (the oracle's l_(k) - l_(k+1)): how many
    token-layers fall below the gap rule, and how many tokens a parity test
    would redraw.  The bench's inputs are not redrawn (timing needs no unique
    routing); this says how often the rule would act on them."""
    g = np.asarray(gaps)
    return dict(gap=GAP_RULE, tokens=int(g.shape[1]), token_layers=int(g.size),
                token_layers_below=int((g < GAP_RULE).sum()),
                tokens_to_redraw=int((g < GAP_RULE).any(axis=0).sum()))


def cpu_baseline_decode(w, budget_s):
    """The oracle (fp64 C, OpenMP) on a bounded sample: tokens one at a time
    through the full 24-layer stack; tok/s on this host.  Also counts the
    sampled tokens' gap-rule hits."""
    import oracle
    from ternary_weight_moe_amd import synth as S
    log("cpu baseline: packing the stack for the oracle")
    L = oracle_layers(w)
    n, t_used, gaps = 0, 0.0, []
    while t_used < budget_s and n < 256:
        x = S.x_as_f32(w, S.gen_x(w, 1, token0=n)).astype(np.float64)
        t0 = time.perf_counter()
        r = oracle.moe_stack(x, [l["Wr"] for l in L], [l["bias"] for l in L],
                             [l["packed"] for l in L], [l["alpha"] for l in L], k=w.top_k,
                             inter=w.inter, keep_logits=True, keep_delta=False)
        t_used += time.perf_counter() - t0
        gaps.append(oracle.topk_gap(r["logits"], w.top_k))
        n += 1
    return dict(value=n / t_used, unit="tok/s", cores=oracle.num_threads(), kind="oracle",
                sample=f"{n} tokens x {w.n_layers} layers, one token per call "
                       f"({t_used:.1f} s of oracle time)",
                gap_rule=gap_rule_count(np.concatenate(gaps, axis=1)))


def cpu_baseline_batched(w, budget_s):
    """The oracle on a bounded sample of the batched workload: groups of 8 of the
    step's tokens through the whole stack until the budget is spent; tok/s."""
    import oracle
    from ternary_weight_moe_amd import synth as S
    L = oracle_layers(w)
    x_all = S.x_as_f32(w, S.gen_x(w, w.n_tokens)).astype(np.float64)
    n, t_used, gaps = 0, 0.0, []
    while t_used < budget_s and n < w.n_tokens:
        t0 = time.perf_counter()
        r = oracle.moe_stack(x_all[n:n + 8], [l["Wr"] for l in L], [l["bias"] for l in L],
                             [l["packed"] for l in L], [l["alpha"] for l in L], k=w.top_k,
                             inter=w.inter, keep_logits=True, keep_delta=False)
        t_used += time.perf_counter() - t0
        gaps.append(oracle.topk_gap(r["logits"], w.top_k))
        n += 8
    return dict(value=n / t_used, unit="tok/s", cores=oracle.num_threads(), kind="oracle",
                sample=f"{n} of the {w.n_tokens} tokens of one step, 8 per call, "
                       f"{w.n_layers} layers ({t_used:.1f} s of oracle time)",
                gap_rule=gap_rule_count(np.concatenate(gaps, axis=1)))


def cpu_baseline_prefill(w, budget_s, a8=False):
    """The oracle on a bounded sample of the prefill workload: token batches of
    the same layer until the time budget is spent; tok/s on this host.  With
    a8 the oracle runs its integer-activation mode."""
    import oracle
    from ternary_weight_moe_amd import synth as S
    L = oracle_layers(w)[0]
    n, t_used, chunk = 0, 0.0, 2 * oracle.num_threads()
    while t_used < budget_s and n < w.n_tokens:
        x = S.x_as_f32(w, S.gen_x(w, chunk, token0=n)).astype(np.float64)
        t0 = time.perf_counter()
        oracle.moe_layer(x, L["Wr"], L["bias"], L["packed"], L["alpha"], k=w.top_k,
                         inter=w.inter, a8=a8)
        t_used += time.perf_counter() - t0
        n += chunk
    return dict(value=n / t_used, unit="tok/s", cores=oracle.num_threads(), kind="oracle",
                sample=f"{n} of {w.n_tokens} tokens of one layer{' (A8 mode)' if a8 else ''}, "
                       f"{chunk} per call "
                       f"({t_used:.1f} s of oracle time)")


def profile_kernels(N, fn, steps):
    """Run fn() `steps` times with the library's event timing on; returns
    {kernel: (launches, avg ms)}."""
    import torch
    torch.cuda.synchronize()
    N.maple_profile_enable(True)
    for _ in range(steps):
        fn()
    torch.cuda.synchronize()
    summ = N.maple_profile_summary()
    N.maple_profile_enable(False)
    return {k: (n, ms / n) for k, (n, ms) in summ.items()}


def graph_stamp_profile(N, torch, make_graph, replays, burst=4):
    """Per-kernel spans inside graph replays: a graph captured while the
    library's device-stamp mode is on; after every burst of back-to-back
    replays the stamps of the last one are read.  Returns ({kernel:
    (launches per replay, avg us per launch)}, ms per stamped replay)."""
    stream = torch.cuda.current_stream()
    torch.cuda.synchronize()
    N.maple_profile_enable(2)
    g = make_graph()
    try:
        ms_stamped = timed(torch, lambda: g.launch(stream), 64, 8)
        acc = {}
        for _ in range(replays):
            for _ in range(burst):
                g.launch(stream)
            for kn, (n, ms) in N.maple_profile_summary().items():
                a = acc.setdefault(kn, [0, 0.0])
                a[0] = n
                a[1] += 1000.0 * ms / n
    finally:
        N.maple_profile_enable(0)
        g.destroy()
    return {kn: (n, us / replays) for kn, (n, us) in acc.items()}, ms_stamped


def dependent_launch_floor(torch, n_kernels=49, replays=64):
    """The time per kernel of a captured graph of n_kernels dependent
    one-element kernels (torch's in-place add), replayed back to back: the
    cost of a kernel boundary with no work, the floor under a decode step
    that has n_kernels dependent launches."""
    a = torch.zeros(1, device="cuda")
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        for _ in range(3):
            a.add_(1.0)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        for _ in range(n_kernels):
            a.add_(1.0)
    for _ in range(8):
        g.replay()
    torch.cuda.synchronize()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record()
    for _ in range(replays):
        g.replay()
    end.record()
    torch.cuda.synchronize()
    return 1000.0 * start.elapsed_time(end) / (replays * n_kernels)


def copy_probe(torch, mib):
    """A plain device-to-device copy of known size, launched a few times, so that
    hardware counter runs over this script can scale FETCH_SIZE / WRITE_SIZE."""
    n = mib * (1 << 20) // 4
    src = torch.ones(n, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    log(f"copy probe: 3 x {mib} MiB device-to-device copies")
    del src, dst


def timed(torch, fn, steps, warmup):
    stream = torch.cuda.current_stream()
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record(stream)
    for _ in range(steps):
        fn()
    end.record(stream)
    torch.cuda.synchronize()
    return start.elapsed_time(end) / steps


# ---- workloads ------------------------------------------------------------------------

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
    out_all = torch.zeros(n_staged, 1, H, dtype=torch.float32, device="cuda")
    lists = ([l["Wr"] for l in layers], None, [l["packed"] for l in layers],
             [l["alpha"] for l in layers])
    def make_graph():
        return N.MapleGraph(d, 1, staged, n_staged, x_work, out_all, *lists, ws)
    g = make_graph()
    stream = torch.cuda.current_stream()
    ms_per_step = timed(torch, lambda: g.launch(stream), args.steps, args.warmup)
    assert torch.isfinite(out_all).all().item(), "non-finite decode output"
    g.destroy()
    log(f"decode: {1000.0 / ms_per_step:.1f} tok/s, {ms_per_step * 1000:.1f} us/step")

    # graph-mode spans of the one-token kernels (a stamped graph of the same step)
    prof, ms_stamped = graph_stamp_profile(N, torch, make_graph, min(args.steps, 64))
    per_kernel = {}
    for kn, (n, avg_us) in prof.items():
        b = decode_bytes(kn, H, E, k, I)
        per_kernel[kn] = dict(launches_per_step=n, avg_us=avg_us, total_us_per_step=n * avg_us,
                              bytes=b, achieved_gbs=b / (avg_us * 1e-6) / 1e9 if b else None)
    span_sum_us = sum(v["total_us_per_step"] for v in per_kernel.values())
    log(f"graph-mode spans: {', '.join(f'{kn} {v[1]:.2f} us' for kn, v in prof.items())}; "
        f"sum {span_sum_us:.1f} of {ms_per_step * 1000:.1f} us per step")
    dom = max(per_kernel, key=lambda kn: per_kernel[kn]["total_us_per_step"])
    dom_bytes = decode_bytes(dom, H, E, k, I)
    dom_avg_s = prof[dom][1] * 1e-6
    achieved = dom_bytes / dom_avg_s / 1e9
    bytes_tok = L * decode_bytes_per_token_layer(H, E, k, I)
    step_gbs = bytes_tok / (ms_per_step * 1e-3) / 1e9
    # the graph also holds the two staging kernels (load the token, store the output)
    n_kernels = sum(v["launches_per_step"] for v in per_kernel.values()) + 2
    floor_us = dependent_launch_floor(torch, n_kernels)
    log(f"dependent empty-kernel floor: {floor_us:.2f} us per kernel, "
        f"{floor_us * n_kernels:.1f} us for the step's {n_kernels} kernels")
    return dict(
        metric=METRIC, value=1000.0 / ms_per_step, unit="tok/s", n_gpus=1, steps=args.steps,
        warmup=args.warmup, ms_per_step=ms_per_step, higher_is_better=True, scaling="weak",
        vs_baseline=None, dtype="f32", data="synthetic",
        config=dict(workload="decode_stack", hidden=H, experts=E, top_k=k, inter=I, layers=L,
                    batch=1, tokens_staged=n_staged, step="one captured HIP graph per token"),
        roofline=dict(bound="hbm", achieved=achieved, peak=HBM_PEAK_GBS, unit="GB/s",
                      frac=achieved / HBM_PEAK_GBS, traffic=traffic_for("decode_stack", dom),
                      kernel=dom,
                      algorithmic_bytes_per_launch=dom_bytes, avg_launch_us=dom_avg_s * 1e6,
                      timing="graph replays: first block entry to last block exit, "
                             "device real-time counter"),
        step_roofline=dict(algorithmic_bytes_per_step=bytes_tok, achieved_gbs=step_gbs,
                           frac_of_hbm_peak=step_gbs / HBM_PEAK_GBS),
        kernels_per_token=n_kernels,
        launch_floor=dict(us_per_dependent_kernel=floor_us,
                          us_per_step=floor_us * n_kernels,
                          what="graph of one-element dependent kernels, replayed back to back"),
        graph_kernel_span_sum_us=span_sum_us,
        stamped_graph_ms_per_step=ms_stamped,
        kernels=per_kernel,
    ), w


def bench_batched(args, torch, N, S):
    """Batched decode: 64 tokens per step through the 24-layer stack, router logits
    biased so that expert popularity is Zipf-skewed (skewed groups, empty
    experts).  A step is one call of maple_moe_stack_forward on 64 tokens."""
    w = S.WORKLOADS["batched_stack_zipf"]
    H, E, k, I, L, T = w.hidden, w.n_experts, w.top_k, w.inter, w.n_layers, w.n_tokens
    layers = build_layers(w, torch, N, S)
    xs = S.gen_x(w, T)
    x0 = torch.from_numpy(xs.view(np.int16)).cuda().view(torch.bfloat16).float()
    d = N.make_dims(H, E, k, I, 0)
    ws = torch.empty(N.maple_moe_workspace_bytes(d, T), dtype=torch.uint8, device="cuda")
    x = torch.empty_like(x0)
    lists = ([l["Wr"] for l in layers], [l["bias"] for l in layers], [l["packed"] for l in layers],
             [l["alpha"] for l in layers])

    def step(st=None):
        x.copy_(x0)
        N.maple_moe_stack_forward(d, T, x, *lists, ws, stream=st)
    ms_eager = timed(torch, step, args.steps, args.warmup)
    # the same step (restore x, one stack call) captured into a HIP graph and
    # replayed, as a serving loop at a fixed batch would run it
    st = torch.cuda.Stream()
    with torch.cuda.stream(st):
        step(st)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=st):
        step(st)
    ms_per_step = timed(torch, graph.replay, args.steps, args.warmup)
    assert torch.isfinite(x).all().item(), "non-finite batched output"
    del graph
    log(f"batched_stack_zipf: {T / ms_per_step * 1000:.0f} tok/s, {ms_per_step * 1000:.1f} us/step "
        f"(graph replays; eager calls {ms_eager * 1000:.1f} us)")
    prof = profile_kernels(N, step, min(args.steps, 8))
    per_kernel = {kn: dict(launches=n, avg_us=1000 * avg) for kn, (n, avg) in prof.items()}
    dom = max(prof, key=lambda kn: prof[kn][0] * prof[kn][1])
    # the realised routing of the step (the same call, with its routing copied out)
    idx = torch.empty(L, T, k, dtype=torch.int32, device="cuda")
    x.copy_(x0)
    N.maple_moe_stack_forward(d, T, x, *lists, ws, N.make_debug(idx=idx))
    idx = idx.cpu().numpy()
    counts = np.stack([np.bincount(idx[l].reshape(-1), minlength=E) for l in range(L)])
    distinct = (counts > 0).sum(1)
    D = float(distinct.mean())
    step_bytes = int(sum(int(dl) * expert_bytes(H, I) + 4 * E * H + T * H * 8 for dl in distinct))
    dom_bytes = grouped_fine_bytes(dom, H, E, k, I, T, D)
    dom_avg_s = prof[dom][1] * 1e-3
    achieved = dom_bytes / dom_avg_s / 1e9 if dom_bytes else None
    routing = dict(distinct_experts_per_layer=dict(min=int(distinct.min()), mean=D,
                                                   max=int(distinct.max())),
                   empty_experts_mean=float((counts == 0).sum(1).mean()),
                   largest_group=int(counts.max()),
                   layer0_group_sizes_desc=sorted(counts[0][counts[0] > 0].tolist(), reverse=True))
    log(f"routing: {routing['distinct_experts_per_layer']} distinct experts per layer, "
        f"largest group {routing['largest_group']}")
    step_gbs = step_bytes / (ms_per_step * 1e-3) / 1e9
    return dict(
        metric=METRIC, value=T / ms_per_step * 1000.0, unit="tok/s", n_gpus=1, steps=args.steps,
        warmup=args.warmup, ms_per_step=ms_per_step, higher_is_better=True, scaling="weak",
        vs_baseline=None, dtype="f32", data="synthetic",
        config=dict(workload="batched_stack_zipf", hidden=H, experts=E, top_k=k, inter=I,
                    layers=L, tokens_per_step=T,
                    step="one stack call on 64 tokens, replayed from a captured HIP graph",
                    eager_ms_per_step=ms_eager),
        roofline=dict(bound="hbm", achieved=achieved, peak=HBM_PEAK_GBS, unit="GB/s",
                      frac=achieved / HBM_PEAK_GBS if achieved else None,
                      traffic=traffic_for("batched_stack_zipf", dom), kernel=dom,
                      algorithmic_bytes_per_launch=dom_bytes,
                      avg_launch_us=dom_avg_s * 1e6,
                      timing="eager calls: each kernel's own dispatch begin to end (HIP events "
                             "on its launch)"),
        step_roofline=dict(algorithmic_bytes_per_step=step_bytes, achieved_gbs=step_gbs,
                           frac_of_hbm_peak=step_gbs / HBM_PEAK_GBS),
        routing=routing,
        kernels=per_kernel,
    ), w


def head_bytes(kernel, H, C, P, n_cand):
    """Algorithmic HBM bytes of one launch of an output-head kernel for one
    token with n_cand candidate rows (bf16 rows, fp32 h)."""
    return {
        "head_scores": C * 2 * H + 4 * H + 4 * C,
        "head_select": 4 * C + 8 * P + 4 * (P + 1),
        "head_search": n_cand * (2 * H + 4) + 4 * H + 8 * P + 8 * P,
    }.get(kernel)


def bench_head(args, torch, N, S):
    """Output head (FlashHead) for one token per call: centroid scores, the
    n_probe best clusters, exact search of their rows.  256 staged hidden
    states; calls are replayed from captured HIP graphs of 16 calls."""
    w = S.HEAD_WORKLOADS["flashhead_decode"]
    H, C, P = w.hidden, w.n_clusters, w.n_probe
    cen, rows, off, rt = S.gen_head_index(w)
    V = rows.shape[0]
    log(f"head index: V={V} rows, C={C} clusters, P={P} probed")
    dev = "cuda"
    d_cen = torch.from_numpy(cen.view(np.int16)).to(dev)
    d_rows = torch.from_numpy(rows.view(np.int16)).to(dev)
    d_off = torch.from_numpy(off).to(dev)
    d_rt = torch.from_numpy(rt).to(dev)
    NS = 256
    hs = torch.from_numpy(S.gen_head_h(w, NS)).to(dev)
    tok = torch.empty(NS, dtype=torch.int32, device=dev)
    lg = torch.empty(NS, device=dev)
    d = N.make_head_dims(H, V, C, P)
    ws = torch.empty(N.maple_head_workspace_bytes(d, 1), dtype=torch.uint8, device=dev)
    stream = torch.cuda.Stream()

    def call(i, s=None):
        N.maple_flashhead_forward(d, 1, hs[i], d_cen, d_rows, d_off, d_rt, tok[i:i + 1],
                                  lg[i:i + 1], ws, stream=s)
    G = 16
    graphs = []
    with torch.cuda.stream(stream):
        for i in range(G):  # warm the caches of every path once, eagerly
            call(i, stream)
    torch.cuda.synchronize()
    for g0 in range(0, NS, G):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=stream):
            for i in range(g0, g0 + G):
                call(i, stream)
        graphs.append(g)
    replays = max(1, args.steps // G)
    for r in range(max(1, args.warmup // G)):
        graphs[r % len(graphs)].replay()
    torch.cuda.synchronize()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record()
    for r in range(replays):
        graphs[r % len(graphs)].replay()
    end.record()
    torch.cuda.synchronize()
    n_tok = replays * G
    ms_per_step = start.elapsed_time(end) / n_tok
    assert bool((tok >= 0).all().item()), "head returned no token"
    log(f"flashhead: {1000 / ms_per_step:.0f} tok/s, {ms_per_step * 1000:.2f} us per token")
    # candidate counts of the staged tokens, from the library's own debug output
    ncand = torch.empty(1, dtype=torch.int32, device=dev)
    counts = []
    for i in range(32):
        N.maple_flashhead_forward(d, 1, hs[i], d_cen, d_rows, d_off, d_rt, tok[i:i + 1],
                                  lg[i:i + 1], ws, N.make_head_debug(n_cand=ncand))
        counts.append(int(ncand.item()))
    n_cand = float(np.mean(counts))
    prof = profile_kernels(N, lambda: [call(i) for i in range(32)], 4)
    per_kernel = {kn: dict(launches=n, avg_us=1000 * avg) for kn, (n, avg) in prof.items()}
    dom = max(prof, key=lambda kn: prof[kn][0] * prof[kn][1])
    dom_bytes = head_bytes(dom, H, C, P, n_cand)
    dom_avg_s = prof[dom][1] * 1e-3
    achieved = dom_bytes / dom_avg_s / 1e9
    tok_bytes = sum(head_bytes(k, H, C, P, n_cand) for k in ("head_scores", "head_select",
                                                              "head_search"))
    step_gbs = tok_bytes / (ms_per_step * 1e-3) / 1e9
    return dict(
        metric="output-head tok/s (clustered FlashHead search, one token per call)",
        value=1000.0 / ms_per_step, unit="tok/s", n_gpus=1, steps=n_tok, warmup=args.warmup,
        ms_per_step=ms_per_step, higher_is_better=True, scaling="weak", vs_baseline=None,
        dtype="bf16 rows, f32 sums", data="synthetic",
        config=dict(workload="flashhead_decode", hidden=H, vocab=V, clusters=C, probed=P,
                    mean_candidate_rows=n_cand, step="one head call for one token"),
        roofline=dict(bound="hbm", achieved=achieved, peak=HBM_PEAK_GBS, unit="GB/s",
                      frac=achieved / HBM_PEAK_GBS, traffic=traffic_for("flashhead_decode", dom),
                      kernel=dom, algorithmic_bytes_per_launch=dom_bytes,
                      avg_launch_us=dom_avg_s * 1e6),
        step_roofline=dict(algorithmic_bytes_per_step=tok_bytes, achieved_gbs=step_gbs,
                           frac_of_hbm_peak=step_gbs / HBM_PEAK_GBS,
                           dense_head_bytes=V * 2 * H,
                           fraction_of_dense_head_bytes=tok_bytes / (V * 2 * H)),
        kernels=per_kernel,
    ), (w, cen, rows, off, rt, hs.cpu().numpy())


def bench_attn(args, torch, N, S):
    """Attention of one decode step through the 24 layers of the hybrid
    pattern (layers 3, 7, .., 23 global, the other 18 sliding over 512
    positions), one sequence whose new token sits at position 131,071: 16
    query heads of 128 over 4 kv heads, bf16 caches.  Every global layer has
    its own 268 MB cache (the same history copied in), so each step streams
    1.6 GB from HBM.  Steps are replayed from captured HIP graphs of 4 steps;
    each call stores the new token at the same position, so steps repeat."""
    wg = S.ATTN_WORKLOADS["attn_global_decode"]
    wsw = S.ATTN_WORKLOADS["attn_swa_decode"]
    Hq, Hkv, D, W = wg.n_q, wg.n_kv, wg.head_dim, wsw.window
    L = 24
    is_global = [l % 4 == 3 for l in range(L)]
    p = wg.ctx - 1
    dev = "cuda"
    kg, vg = S.gen_attn_kv(wg, 0, wg.ctx)
    kw, vw = S.gen_attn_kv(wsw, p - W + 1, p + 1)
    q = S.gen_attn_q(wg)
    log(f"attention histories drawn: global {kg.nbytes * 2 / 1e6:.0f} MB, window "
        f"{kw.nbytes * 2 / 1e6:.1f} MB")

    def d16(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(dev)
    dims_g = N.make_attn_dims(Hq, Hkv, D, 0, wg.capacity)
    dims_w = N.make_attn_dims(Hq, Hkv, D, W, wsw.capacity)
    d_q, d_pos = d16(q), torch.tensor([p], dtype=torch.int32, device=dev)
    lin_g = (d16(kg[0, :, :p]), d16(vg[0, :, :p]))
    lin_w = (d16(kw[0, :, :-1]), d16(vw[0, :, :-1]))
    new_g = (d16(kg[:, :, p]), d16(vg[:, :, p]))
    new_w = (d16(kw[:, :, -1]), d16(vw[:, :, -1]))
    caches = []
    for l in range(L):
        dims = dims_g if is_global[l] else dims_w
        n = N.maple_attn_cache_bytes(dims, 1) // 2
        kc = torch.empty(n, dtype=torch.int16, device=dev)
        vc = torch.empty(n, dtype=torch.int16, device=dev)
        lk, lv = lin_g if is_global[l] else lin_w
        N.maple_attn_cache_fill(dims, 1, 0 if is_global[l] else p - W + 1, lk.shape[1], lk, lv,
                                kc, vc)
        caches.append((kc, vc))
    del lin_g, lin_w
    torch.cuda.synchronize()
    ws_g = torch.empty(N.maple_attn_workspace_bytes(dims_g, 1, wg.ctx), dtype=torch.uint8,
                       device=dev)
    ws_w = torch.empty(N.maple_attn_workspace_bytes(dims_w, 1, wg.ctx), dtype=torch.uint8,
                       device=dev)
    out = torch.empty(L, 1, Hq, D, dtype=torch.float32, device=dev)

    def step(s=None):
        for l in range(L):
            g = is_global[l]
            kn, vn = new_g if g else new_w
            N.maple_attn_decode(dims_g if g else dims_w, 1, wg.ctx, d_q, kn, vn, d_pos,
                                caches[l][0], caches[l][1], out[l], ws_g if g else ws_w,
                                stream=s)
    stream = torch.cuda.Stream()
    with torch.cuda.stream(stream):
        step(stream)
    torch.cuda.synchronize()
    G = 4
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=stream):
        for _ in range(G):
            step(stream)
    for _ in range(max(1, args.warmup // G)):
        graph.replay()
    torch.cuda.synchronize()
    replays = max(1, args.steps // G)
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record()
    for _ in range(replays):
        graph.replay()
    end.record()
    torch.cuda.synchronize()
    n_steps = replays * G
    ms_per_step = start.elapsed_time(end) / n_steps
    assert bool(torch.isfinite(out).all().item()), "non-finite attention output"
    log(f"hybrid attention: {1000 / ms_per_step:.0f} tok/s, {ms_per_step * 1000:.1f} us per step")
    prof = profile_kernels(N, step, 8)
    per_kernel = {kn: dict(launches=n, avg_us=1000 * avg) for kn, (n, avg) in prof.items()}
    gbytes = attn_bytes(Hq, Hkv, D, p + 1)
    wbytes = attn_bytes(Hq, Hkv, D, W)
    for kn, b in (("attn_global", gbytes), ("attn_window", wbytes)):
        if kn in per_kernel:
            per_kernel[kn]["algorithmic_bytes"] = b
            per_kernel[kn]["achieved_gbs"] = b / (per_kernel[kn]["avg_us"] * 1e-6) / 1e9
    dom = max(prof, key=lambda kn: prof[kn][0] * prof[kn][1])
    dom_bytes = {"attn_global": gbytes, "attn_window": wbytes}.get(dom)
    dom_avg_s = prof[dom][1] * 1e-3
    achieved = dom_bytes / dom_avg_s / 1e9 if dom_bytes else None
    step_bytes = 6 * gbytes + 18 * wbytes
    step_gbs = step_bytes / (ms_per_step * 1e-3) / 1e9
    return dict(
        metric="decode-attention tok/s (24-layer hybrid sliding-window/global pattern, one sequence "
               "at 131,072 positions)",
        value=1000.0 / ms_per_step, unit="tok/s", n_gpus=1, steps=n_steps, warmup=args.warmup,
        ms_per_step=ms_per_step, higher_is_better=True, scaling="weak", vs_baseline=None,
        dtype="bf16 MFMA, f32 softmax and sums", data="synthetic",
        config=dict(workload="hybrid_attn_decode", layers=L, global_layers=6, window=W,
                    position=p, batch=1, q_heads=Hq, kv_heads=Hkv, head_dim=D,
                    step="attention of one token through 24 layers"),
        roofline=dict(bound="hbm", achieved=achieved, peak=HBM_PEAK_GBS, unit="GB/s",
                      frac=achieved / HBM_PEAK_GBS if achieved else None,
                      traffic=traffic_for("hybrid_attn_decode", dom), kernel=dom,
                      algorithmic_bytes_per_launch=dom_bytes, avg_launch_us=dom_avg_s * 1e6),
        step_roofline=dict(algorithmic_bytes_per_step=step_bytes, achieved_gbs=step_gbs,
                           frac_of_hbm_peak=step_gbs / HBM_PEAK_GBS),
        kernels=per_kernel,
    ), (wg, wsw, q, kg, vg, kw, vw)


def cpu_baseline_attn(ctx, budget_s):
    """The oracle on a bounded sample: whole steps (6 global layers at 131,072
    positions and 18 sliding layers) until the budget is spent; tok/s."""
    import oracle
    wg, wsw, q, kg, vg, kw, vw = ctx
    p = wg.ctx - 1
    n, t_used = 0, 0.0
    while t_used < budget_s or n == 0:
        t0 = time.perf_counter()
        for l in range(24):
            if l % 4 == 3:
                oracle.attn_decode(q, kg, vg, [p], window=0)
            else:
                oracle.attn_decode(q, kw, vw, [wsw.window - 1], window=wsw.window)
        t_used += time.perf_counter() - t0
        n += 1
    return dict(value=n / t_used, unit="tok/s", cores=oracle.num_threads(), kind="oracle",
                sample=f"{n} whole steps of 24 layers ({t_used:.1f} s of oracle time)")


def convert_bytes(n_rows, cols):
    """Algorithmic HBM bytes of converting n_rows rows of cols bf16 values:
    the source read once, the 2-bit codes and one fp32 alpha per row written."""
    return n_rows * cols * 2 + n_rows * cols // 4 + 4 * n_rows


def bench_convert(args, torch, N, S):
    """BF16 -> ternary conversion of one whole MoE layer (256 experts, hidden
    2048, inter 512: 805M latent weights, 1.61 GB of bf16) into the layer blob
    and its alphas: two strided calls, the 512 gate/up rows of every expert
    (2048 columns) and its 2048 down rows (512 columns)."""
    w = S.WORKLOADS["decode_layer"]
    H, I, E = w.hidden, w.inter, w.n_experts
    n = 3 * H * I
    dev = "cuda"
    src = torch.empty(E * n, dtype=torch.int16, device=dev)
    for e in range(E):
        src[e * n:(e + 1) * n] = torch.from_numpy(S.gen_latent_expert(w, 0, e).view(np.int16)).to(dev)
    packed = torch.empty(E * n // 4, dtype=torch.uint8, device=dev)
    alpha = torch.empty(E * (2 * I + H), dtype=torch.float32, device=dev)
    bad = torch.empty(1, dtype=torch.int32, device=dev)
    log(f"latent layer drawn: {E * n * 2 / 1e9:.2f} GB of bf16")

    def step():
        N.maple_ternarize_bf16_device(src, E, 2 * I, H, n, n // 4, 2 * I + H, packed, alpha, bad)
        N.maple_ternarize_bf16_device(src[2 * I * H:], E, H, I, n, n // 4, 2 * I + H,
                                      packed[2 * I * H // 4:], alpha[2 * I:], bad)
    ms_per_step = timed(torch, step, args.steps, args.warmup)
    assert int(bad.item()) == 0, "bad rows in the latent layer"
    src_gb = E * n * 2 / 1e9
    log(f"ternarize: {src_gb / (ms_per_step * 1e-3):.0f} GB/s of bf16 source, {ms_per_step * 1000:.0f} us per layer")
    prof = profile_kernels(N, step, min(args.steps, 10))
    by = {"ternarize_w2": convert_bytes(E * 2 * I, H), "ternarize_g32": convert_bytes(E * H, I)}
    per_kernel = {kn: dict(launches=c, avg_us=1000 * avg, algorithmic_bytes=by.get(kn),
                           achieved_gbs=(by[kn] / (avg * 1e-3) / 1e9) if kn in by else None)
                  for kn, (c, avg) in prof.items()}
    dom = max((k for k in prof if k in by), key=lambda kn: prof[kn][0] * prof[kn][1])
    dom_avg_s = prof[dom][1] * 1e-3
    achieved = by[dom] / dom_avg_s / 1e9
    step_bytes = sum(by.values())
    return dict(
        metric="BF16 -> ternary weight conversion, GB/s of bf16 source (one whole MoE layer per step)",
        value=src_gb / (ms_per_step * 1e-3), unit="GB/s", n_gpus=1, steps=args.steps,
        warmup=args.warmup, ms_per_step=ms_per_step, higher_is_better=True, scaling="weak",
        vs_baseline=None, dtype="bf16 in, fp64 row sums, 2-bit codes + f32 alpha out",
        data="synthetic",
        config=dict(workload="ternary_convert", experts=E, hidden=H, inter=I,
                    weights=E * n, step="convert one layer (two calls)"),
        roofline=dict(bound="hbm", achieved=achieved, peak=HBM_PEAK_GBS, unit="GB/s",
                      frac=achieved / HBM_PEAK_GBS, traffic=traffic_for("ternary_convert", dom),
                      kernel=dom, algorithmic_bytes_per_launch=by[dom],
                      avg_launch_us=dom_avg_s * 1e6),
        step_roofline=dict(algorithmic_bytes_per_step=step_bytes,
                           achieved_gbs=step_bytes / (ms_per_step * 1e-3) / 1e9,
                           frac_of_hbm_peak=step_bytes / (ms_per_step * 1e-3) / 1e9 / HBM_PEAK_GBS),
        kernels=per_kernel,
    ), w


def cpu_baseline_convert(w, budget_s):
    """The oracle on a bounded sample: whole experts (gate/up rows, then down
    rows) until the budget is spent; GB/s of bf16 source."""
    import oracle
    from ternary_weight_moe_amd import synth as S
    H, I = w.hidden, w.inter
    n, t_used, e = 0, 0.0, 0
    while t_used < budget_s and e < w.n_experts:
        lat = S.gen_latent_expert(w, 0, e)
        t0 = time.perf_counter()
        oracle.ternarize(lat[:2 * I * H].reshape(2 * I, H))
        oracle.ternarize(lat[2 * I * H:].reshape(H, I))
        t_used += time.perf_counter() - t0
        n += lat.size
        e += 1
    return dict(value=n * 2 / t_used / 1e9, unit="GB/s", cores=oracle.num_threads(),
                kind="oracle", sample=f"{e} experts ({n} weights, {t_used:.1f} s of oracle time)")


def cpu_baseline_head(ctx, budget_s):
    """The oracle on a bounded sample: the staged tokens 16 per call (its
    threads take one token each) until the budget is spent; tok/s."""
    import oracle
    w, cen, rows, off, rt, h = ctx
    n, t_used = 0, 0.0
    while t_used < budget_s and n < h.shape[0]:
        t0 = time.perf_counter()
        oracle.flashhead(h[n:n + 16].astype(np.float64), cen, rows, off, rt, w.n_probe,
                         keep_cand=False)
        t_used += time.perf_counter() - t0
        n += 16
    return dict(value=n / t_used, unit="tok/s", cores=min(16, oracle.num_threads()),
                kind="oracle",
                sample=f"{n} staged tokens, 16 per call ({t_used:.2f} s of oracle time)")


def bench_prefill(args, torch, N, S):
    a8 = args.workload.endswith("_a8")
    wname = args.workload[:-3] if a8 else args.workload
    w = S.WORKLOADS[wname]
    H, E, k, I, T = w.hidden, w.n_experts, w.top_k, w.inter, w.n_tokens
    layer = build_layers(w, torch, N, S)[0]
    xs = S.gen_x(w, T)
    x = torch.from_numpy(xs.view(np.int16)).cuda().view(torch.bfloat16)
    d = N.make_dims(H, E, k, I, N.MAPLE_X_BF16 | (N.MAPLE_ACT_INT8 if a8 else 0))
    ws = torch.empty(N.maple_moe_workspace_bytes(d, T), dtype=torch.uint8, device="cuda")
    out = torch.empty(T, H, dtype=torch.float32, device="cuda")

    def step(st=None):
        N.maple_moe_layer_forward(d, T, x, layer["Wr"], layer["bias"], layer["packed"],
                                  layer["alpha"], out, ws, stream=st)
    ms_eager = timed(torch, step, args.steps, args.warmup)
    # the same call captured into a HIP graph: the host launches of the layer's
    # ten short kernels no longer pace it
    st = torch.cuda.Stream()
    with torch.cuda.stream(st):
        step(st)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=st):
        step(st)
    ms_per_step = timed(torch, graph.replay, args.steps, args.warmup)
    assert torch.isfinite(out).all().item(), "non-finite prefill output"
    log(f"{args.workload}: {T / ms_per_step * 1000:.0f} tok/s, {ms_per_step * 1000:.1f} us/layer "
        f"(graph replays; eager calls {ms_eager * 1000:.1f} us)")
    prof = profile_kernels(N, step, min(args.steps, 20))
    per_kernel = {kn: dict(launches=n, avg_us=1000 * avg, ops=prefill_ops(kn, H, k, I, T))
                  for kn, (n, avg) in prof.items()}
    dom = max(prof, key=lambda kn: prof[kn][0] * prof[kn][1])
    ops = prefill_ops(dom, H, k, I, T)
    dom_avg_s = prof[dom][1] * 1e-3
    # issued MFMA work: every expert's slots padded to whole 32-slot tiles (the
    # A8 kernels' 16 x 16 MFMAs skip the second half of a tile's columns when
    # its last tile holds at most 16 slots), and each product issued once per
    # digit plane (three in the fast form, one limb in A8); the routing is the
    # same call's, copied out
    idx = torch.empty(T, k, dtype=torch.int32, device="cuda")
    N.maple_moe_layer_forward(d, T, x, layer["Wr"], layer["bias"], layer["packed"],
                              layer["alpha"], out, ws, N.make_debug(idx=idx))
    counts = np.bincount(idx.cpu().numpy().reshape(-1), minlength=E)
    rem = counts % 32
    last = np.where(rem == 0, 0, np.where((rem <= 16) & a8, 16, 32))
    padded = int((32 * (counts // 32) + last).sum())
    issued_ratio = (1 if a8 else 3) * padded / (T * k)
    # the A8 variant runs int8 MFMAs; the default (fast) form fp4 x fp6 ones,
    # priced against that instruction's own peak
    peak, unit = (INT8_PEAK_TOPS, "TOP/s") if a8 else (FP6_PEAK_TFLOPS, "TFLOP/s")
    if ops:
        roof = dict(bound="mfma", achieved=ops / dom_avg_s / 1e12, peak=peak,
                    unit=unit, frac=ops / dom_avg_s / 1e12 / peak,
                    traffic=traffic_for(args.workload, dom),
                    kernel=dom, algorithmic_ops_per_launch=ops,
                    frac_of_int8_peak=ops / dom_avg_s / 1e12 / INT8_PEAK_TOPS,
                    issued_ops_per_launch=ops * issued_ratio,
                    issued_to_algorithmic=issued_ratio,
                    issued_frac=ops * issued_ratio / dom_avg_s / 1e12 / peak,
                    avg_launch_us=dom_avg_s * 1e6)
    else:
        roof = dict(bound="mfma", achieved=None, peak=peak, unit=unit, frac=None,
                    traffic=None, kernel=dom, avg_launch_us=dom_avg_s * 1e6)
    layer_ops = 2 * T * k * 3 * H * I
    return dict(
        metric=METRIC, value=T / ms_per_step * 1000.0, unit="tok/s", n_gpus=1, steps=args.steps,
        warmup=args.warmup, ms_per_step=ms_per_step, higher_is_better=True, scaling="weak",
        vs_baseline=None, data="synthetic",
        dtype=("int8 MFMA (int8 activations) + f32" if a8
               else "fp4 x fp6 MFMA (three six-bit digits) + f32"),
        config=dict(workload=args.workload, hidden=H, experts=E, top_k=k, inter=I, tokens=T,
                    layers=1, step="one layer call, replayed from a captured HIP graph",
                    eager_ms_per_step=ms_eager, padded_slots=padded,
                    activations=("int8 (one limb)" if a8
                                 else "fp32 coded in three fp6 digits (14-bit integers)")),
        roofline=roof,
        step_roofline=dict(algorithmic_ops_per_step=layer_ops,
                           achieved_tops=layer_ops / (ms_per_step * 1e-3) / 1e12,
                           frac_of_int8_peak=layer_ops / (ms_per_step * 1e-3) / 1e12 /
                           INT8_PEAK_TOPS),
        kernels=per_kernel,
    ), w


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None)
    ap.add_argument("--warmup", type=int, default=None)
    ap.add_argument("--workload", default="decode_stack",
                    choices=["decode_stack", "prefill_4096", "prefill_16384", "prefill_4096_a8",
                             "batched_stack_zipf", "flashhead_decode", "hybrid_attn_decode",
                             "ternary_convert"])
    ap.add_argument("--cpu-baseline-seconds", type=float, default=15.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-prefill", action="store_true",
                    help="decode_stack: leave out the prefill_4096 object")
    ap.add_argument("--no-batched", action="store_true",
                    help="decode_stack: leave out the batched_stack_zipf object")
    ap.add_argument("--copy-probe", type=int, default=0, metavar="MIB",
                    help="first run a plain copy of this many MiB (counter calibration)")
    ap.add_argument("--read-probe", action="store_true",
                    help="only run the read-bandwidth probe (built next to the library): the "
                         "plain read ceiling and the expert kernels' weight-fetch shapes")
    ap.add_argument("--mfma-probe", action="store_true",
                    help="only run the matrix-core probe (built next to the library): issue "
                         "rates of the MFMA kinds the kernels use, dependent-load latency")
    args = ap.parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU: the library has no multi-GPU path "
              "(every token is independent, so the path shards by tokens with no exchange). "
              "Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)
    if args.read_probe or args.mfma_probe:
        # a child process of its own; this one touches no GPU before it
        import subprocess
        probe = os.path.join(os.path.dirname(os.path.abspath(__file__)), "ternary_weight_moe_amd",
                             "read_probe" if args.read_probe else "mfma_probe")
        if not os.path.exists(probe):
            print(f"{probe} is missing: build first (python -c 'import __graft_entry__ as g; "
                  "g.build()')", file=sys.stderr)
            sys.exit(2)
        sys.exit(subprocess.run([probe]).returncode)
    decode = args.workload in ("decode_stack", "flashhead_decode", "hybrid_attn_decode")
    if args.steps is None:
        args.steps = 256 if decode else 20
    if args.warmup is None:
        args.warmup = 16 if decode else 3
    import torch
    from ternary_weight_moe_amd import _native as N
    from ternary_weight_moe_amd import synth as S
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    N.load()  # fails loudly if the HIP library is missing
    if args.copy_probe:
        copy_probe(torch, args.copy_probe)
    runner = {"decode_stack": bench_decode, "batched_stack_zipf": bench_batched,
              "flashhead_decode": bench_head,
              "hybrid_attn_decode": bench_attn,
              "ternary_convert": bench_convert}.get(args.workload, bench_prefill)
    res, w = runner(args, torch, N, S)
    if not args.no_cpu_baseline:
        base = {"decode_stack": cpu_baseline_decode, "batched_stack_zipf": cpu_baseline_batched,
                "flashhead_decode": cpu_baseline_head, "hybrid_attn_decode": cpu_baseline_attn,
                "ternary_convert": cpu_baseline_convert}
        if args.workload in base:
            res["cpu_baseline"] = base[args.workload](w, args.cpu_baseline_seconds)
        else:
            res["cpu_baseline"] = cpu_baseline_prefill(w, args.cpu_baseline_seconds,
                                                       a8=args.workload.endswith("_a8"))
    if args.workload == "decode_stack" and not args.no_prefill:
        # the third part of the metric: the 4096-token layer, timed like
        # --workload prefill_4096 (20 steps after 3 warm-up steps)
        torch.cuda.empty_cache()
        pargs = argparse.Namespace(**vars(args))
        pargs.workload, pargs.steps, pargs.warmup = "prefill_4096", 20, 3
        pres, pw = bench_prefill(pargs, torch, N, S)
        keep = ("value", "unit", "ms_per_step", "steps", "warmup", "dtype", "config", "roofline",
                "step_roofline", "kernels")
        res["prefill_4096"] = {kk: pres[kk] for kk in keep}
        if not args.no_cpu_baseline:
            res["prefill_4096"]["cpu_baseline"] = cpu_baseline_prefill(
                pw, args.cpu_baseline_seconds)
    if args.workload == "decode_stack" and not args.no_batched:
        # the batched-decode configuration (64 tokens per step through the
        # stack, Zipf-skewed routing), timed like --workload batched_stack_zipf
        torch.cuda.empty_cache()
        bargs = argparse.Namespace(**vars(args))
        bargs.workload, bargs.steps, bargs.warmup = "batched_stack_zipf", 20, 3
        bres, bw = bench_batched(bargs, torch, N, S)
        keep = ("value", "unit", "ms_per_step", "steps", "warmup", "dtype", "config", "roofline",
                "step_roofline", "routing", "kernels")
        res["batched_stack_zipf"] = {kk: bres[kk] for kk in keep}
        if not args.no_cpu_baseline:
            res["batched_stack_zipf"]["cpu_baseline"] = cpu_baseline_batched(
                bw, args.cpu_baseline_seconds)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
