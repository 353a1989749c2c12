#!/usr/bin/env python3
"""Benchmark of the svlm hot path on one MI355X at the LLaVA-OneVision-72B shape.

One step = one pass of the whole hot path over one synthetic request:
  score (80 layers, mean text->visual attention averaged into one row)
  -> select (Top-P 0.5 + spatially uniform fill to 10% = 2509 tokens)
  -> gather (all 80 layers in one call: kept visual + 128 text rows into the draft cache)
  -> draft decode attention (80 layers, 1 query over 2638 keys)
  -> dense verify decode attention (80 layers, gamma+1 = 6 queries over 25222 keys)
  -> acceptance (rejection sampling, gamma 5, vocabulary 152064).
All inputs are resident in HBM before timing; all 80 layers' KV (8.3 GB) are
allocated so no layer is served from the 256 MB Infinity Cache.

`value` is the decode-attention HBM throughput: algorithmic bytes (every
needed K and V row read once) of dense verify + 10% draft over the 80 layers,
divided by their summed launch time.  Each kernel sequence (e.g. the 80
dense-verify launches of one step) is captured once as a HIP graph and timed
by HIP events around its replays on the launch stream, so host-side launch
overhead is excluded and each figure is a per-launch average.
Prints one JSON line.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import workloads as W  # noqa: E402

METRIC = "decode-attn µs/step + HBM GB/s (dense verify γ+1, 10% draft) at 25k vis tokens"
HBM_PEAK_GBS = 8000.0
# rocprofv3 --pmc summary of the dense-verify call at this workload: HBM bytes per
# call, taken for the kernel source whose hash it records
VERIFY_PMC = os.path.join(ROOT, "profiles", "decode_attn_verify_llavaov72b_25k_pmc.txt")
KERNEL_SOURCES = ("visual_kv_pruning_amd/csrc/decode_attn.hip", "visual_kv_pruning_amd/csrc/svlm_internal.h")
CALIB_COPY_BYTES = 256 << 20   # plain device copy of known size that scales the PMC byte counters


def kernel_source_hash() -> str:
    import hashlib
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def measured_traffic():
    """HBM bytes per dense-verify call from the committed counter summary, or None
    when that summary is missing or was taken on a different kernel source."""
    try:
        fields = dict(line.split(":", 1) for line in open(VERIFY_PMC).read().splitlines() if ":" in line)
    except OSError:
        return None
    if fields.get("kernel_source_sha256", "").strip() != kernel_source_hash():
        return None
    try:
        return int(fields["hbm_bytes_per_call"].strip())
    except (KeyError, ValueError):
        return None


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=15.0, help="target length of the oracle sample")
    return ap.parse_args()


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}); the hot path here is the "
              "per-GPU kernel set, and multi-GPU runs are not part of this build.", file=sys.stderr)
        sys.exit(2)

    import torch
    from visual_kv_pruning_amd import ops
    from visual_kv_pruning_amd import _lib

    _lib.load()
    dev = torch.device("cuda:0")
    cfg = W.C3
    L, Hq, Hkv, D, T = cfg.layers, cfg.hq, cfg.hkv, cfg.d, cfg.n_text
    NV = cfg.n_vis
    gv = cfg.gamma_verify
    nqv = gv + 1
    N_full = cfg.n_ctx + nqv                 # 25222 keys in the verify pass
    B_keep = cfg.budget                      # 2509 kept visual tokens
    N_draft = B_keep + T + 1                 # 2638 keys in the draft pass
    V = cfg.vocab

    # ---------------- inputs (device-resident; values seeded)
    g = torch.Generator(device=dev)
    g.manual_seed(1000 * cfg.index)
    kv = torch.empty(2, L, Hkv, N_full, D, dtype=torch.bfloat16, device=dev)
    for l in range(L):
        kv[:, l].copy_(torch.randn(2, Hkv, N_full, D, generator=g, device=dev, dtype=torch.float32))
    K, Vv = kv[0], kv[1]
    qt = torch.randn(L, T, Hq, D, generator=g, device=dev, dtype=torch.float32).to(torch.bfloat16)
    # salient / sink structure on layer keys does not change the timing; the value model lives in the tests
    draft_kv = torch.zeros(2, L, Hkv, N_draft, D, dtype=torch.bfloat16, device=dev)
    qv = torch.randn(L, 1, nqv, Hq, D, generator=g, device=dev, dtype=torch.float32).to(torch.bfloat16)
    qd = torch.randn(L, 1, 1, Hq, D, generator=g, device=dev, dtype=torch.float32).to(torch.bfloat16)
    vi = W.verify_inputs(cfg.index, 1, gv, V)
    p_t = torch.from_numpy(vi.p).to(dev)
    q_t = torch.from_numpy(vi.q).to(dev)
    u_t = torch.from_numpy(vi.u).to(dev)
    d_t = torch.from_numpy(vi.draft_tok_sampled).to(dev)
    kv_len_v = torch.tensor([N_full], dtype=torch.int32, device=dev)
    kv_len_d = torch.tensor([N_draft], dtype=torch.int32, device=dev)

    row = torch.empty(1, NV, dtype=torch.float32, device=dev)
    ws_score = torch.empty(ops.score_workspace_bytes(T, Hq, Hkv, NV, NV), dtype=torch.uint8, device=dev)
    ws_score_l = torch.empty(ops.score_layers_workspace_bytes(L, T, Hq, Hkv, NV, NV), dtype=torch.uint8, device=dev)
    ws_v = torch.empty(max(256, ops.decode_attn_workspace_bytes(1, nqv, Hq, Hkv, D, N_full)), dtype=torch.uint8, device=dev)
    ws_d = torch.empty(max(256, ops.decode_attn_workspace_bytes(1, 1, Hq, Hkv, D, N_draft)), dtype=torch.uint8, device=dev)
    ws_di = torch.empty(max(256, ops.decode_attn_indexed_workspace_bytes(1, 1, Hq, Hkv, D, N_draft)),
                        dtype=torch.uint8, device=dev)
    # UV-Prune alternative to the attention score: hidden states of layers 0 and L at hidden size 8192
    d_model = W.HIDDEN[cfg.name]
    hv = torch.randn(2, NV, d_model, generator=g, device=dev, dtype=torch.float32).to(torch.bfloat16)
    hx = torch.randn(2, T, d_model, generator=g, device=dev, dtype=torch.float32).to(torch.bfloat16)
    uv_out = torch.empty(NV, dtype=torch.float32, device=dev)
    ws_uv = torch.empty(max(256, ops.uvprune_workspace_bytes(T, d_model)), dtype=torch.uint8, device=dev)
    # the draft's key list for the in-place variant: kept visual rows, then the text and newest rows
    draft_idx = torch.empty(N_draft, dtype=torch.int32, device=dev)
    draft_idx[B_keep:] = torch.arange(NV, NV + T + 1, dtype=torch.int32, device=dev)
    ws_acc = torch.zeros(ops.verify_workspace_bytes(1, gv, V), dtype=torch.uint8, device=dev)
    o_v = torch.empty(1, nqv, Hq, D, dtype=torch.float32, device=dev)
    l_v = torch.empty(1, nqv, Hq, dtype=torch.float32, device=dev)
    o_d = torch.empty(1, 1, Hq, D, dtype=torch.float32, device=dev)
    l_d = torch.empty(1, 1, Hq, dtype=torch.float32, device=dev)
    kept_box = {}

    # one plain copy of known size, untimed: under rocprofv3 --pmc its FETCH_SIZE and
    # WRITE_SIZE give the scale factor of those counters on this machine
    calib_src = torch.ones(CALIB_COPY_BYTES // 4, dtype=torch.float32, device=dev)
    calib_dst = torch.empty_like(calib_src)
    calib_dst.copy_(calib_src)
    torch.cuda.synchronize()
    del calib_src, calib_dst

    def k_score():
        # every layer in one call: the mean over layers and heads into one row
        ops.score_layers(qt, K, NV, NV, agg="all", layer_mean=True, out=row, ws=ws_score_l)

    def k_score_layer(l):
        ops.score(qt[l], K[l], NV, NV, agg="all", alpha=1.0 / L, beta=0.0 if l == 0 else 1.0, out=row, ws=ws_score)

    def k_select():
        kept_box["kept"] = ops.select(row, cfg.frames, cfg.gh, cfg.gw, cfg.top_p, B_keep)[0]
        draft_idx[:B_keep].copy_(kept_box["kept"][0])

    # one call gathers every layer: the layers' caches fold into the head axis
    # (uniform strides), and the selection row is shared by all of them
    K_all = K.reshape(L * Hkv, N_full, D)
    V_all = Vv.reshape(L * Hkv, N_full, D)
    dk_all = draft_kv[0, :, :, :B_keep + T].reshape(L * Hkv, B_keep + T, D)
    dv_all = draft_kv[1, :, :, :B_keep + T].reshape(L * Hkv, B_keep + T, D)
    assert dk_all.data_ptr() == draft_kv[0].data_ptr() and dk_all.stride(0) == N_draft * D

    def k_gather():
        ops.gather_kv(K_all, V_all, kept_box["kept"][0], NV, T, dk_all, dv_all)

    def k_draft(l):
        ops.decode_attn(qd[l], draft_kv[0, l], draft_kv[1, l], kv_len_d, False, out=o_d, lse=l_d, ws=ws_d)

    def k_draft_idx(l):
        ops.decode_attn_indexed(qd[l], K[l], Vv[l], draft_idx, kv_len_d, False, out=o_d, lse=l_d, ws=ws_di)

    def k_uvprune():
        ops.uvprune_score(hv[0], hv[1], hx[0], hx[1], 1.0 / (4 * T), 0.5, out=uv_out, ws=ws_uv)

    def k_verify_attn(l):
        ops.decode_attn(qv[l], K[l], Vv[l], kv_len_v, True, out=o_v, lse=l_v, ws=ws_v)

    def k_accept():
        ops.verify("reject", d_t, p_t, q_t, u_t, ws=ws_acc)

    seqs = {
        "score": k_score,
        "score_layer_calls": lambda: [k_score_layer(l) for l in range(L)],
        "select": k_select,
        "gather": k_gather,
        "draft_attn": lambda: [k_draft(l) for l in range(L)],
        "draft_attn_indexed": lambda: [k_draft_idx(l) for l in range(L)],
        "uvprune_score": k_uvprune,
        "verify_attn": lambda: [k_verify_attn(l) for l in range(L)],
        "accept": k_accept,
        # the same call 16 times in one graph: per-call time without the replay
        # overhead of a one-node graph (a decode loop runs it between other kernels)
        "accept_in_sequence": lambda: [k_accept() for _ in range(16)],
    }
    calls = {"score": 1, "score_layer_calls": L, "select": 1, "gather": 1, "draft_attn": L, "draft_attn_indexed": L, "uvprune_score": 1,
             "verify_attn": L, "accept": 1, "accept_in_sequence": 16}

    # warm up eagerly (also fills the library's device-property cache), then capture
    # each kernel sequence as a HIP graph so host launch overhead is out of the timings
    for _ in range(max(1, args.warmup)):
        for fn in seqs.values():
            fn()
    torch.cuda.synchronize()
    graphs = {}
    for kind, fn in seqs.items():
        gr = torch.cuda.CUDAGraph()
        with torch.cuda.graph(gr):
            fn()
        graphs[kind] = gr
    torch.cuda.synchronize()

    # one step of the path: every kind but the alternatives, timed on their own
    # below (the in-place draft instead of gather + compact draft; the UV-Prune
    # score instead of the attention score)
    step_kinds = [k for k in seqs if k not in ("draft_attn_indexed", "uvprune_score", "score_layer_calls",
                                                "accept_in_sequence")]

    def step():
        for kind in step_kinds:
            graphs[kind].replay()

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    # (1) whole-step time on the stream
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(args.steps):
        step()
    e1.record()
    torch.cuda.synchronize()
    ms_per_step = e0.elapsed_time(e1) / args.steps

    # (2) per-kind launch durations: events around each graph replay, on the launch stream
    per_us = {}
    spread = {}
    for kind in seqs:
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(args.steps):
            graphs[kind].replay()
        b.record()
        torch.cuda.synchronize()
        per_us[kind] = a.elapsed_time(b) * 1e3 / (args.steps * calls[kind])
        # the spread over replays: an event pair around each one
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
        ev[0].record()
        for i in range(args.steps):
            graphs[kind].replay()
            ev[i + 1].record()
        torch.cuda.synchronize()
        reps = np.array([ev[i].elapsed_time(ev[i + 1]) * 1e3 / calls[kind] for i in range(args.steps)])
        spread[kind] = {q: round(float(np.percentile(reps, p)), 3) for q, p in (("us_p10", 10), ("us_p50", 50),
                                                                             ("us_p90", 90))}

    # (2b) parallel decoding on one GPU (ParallelVLM notes, "parallel decoding":
    # the draft produces the next window while the target verifies the last):
    # the 80 verify launches and the 80 draft launches as two branches of one
    # graph on two streams (default priority), timed per replay
    side = torch.cuda.Stream()
    gpd = torch.cuda.CUDAGraph()
    with torch.cuda.graph(gpd):
        main = torch.cuda.current_stream()
        side.wait_stream(main)
        with torch.cuda.stream(side):
            for l in range(L):
                k_draft(l)
        for l in range(L):
            k_verify_attn(l)
        main.wait_stream(side)
    gpd.replay()
    torch.cuda.synchronize()
    a = torch.cuda.Event(enable_timing=True)
    b = torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(args.steps):
        gpd.replay()
    b.record()
    torch.cuda.synchronize()
    pd_us = a.elapsed_time(b) * 1e3 / args.steps     # both branches, all 80 layers

    # (2c) the hour-long shape (Sparse-to-Dense explainer, "problem statement"
    # and "KV cache selection"; Qwen2-VL-7B heads): dense verify of gamma + 1 = 10
    # queries over 141194 keys, and the draft over per-head lists of 1024 kept
    # visual rows + the 64 text rows + the newest row, read in place.  Reported
    # beside the workload above, not part of `value`.
    hour = measure_hour_shape(torch, ops, dev, g, args.steps)

    # (3) what this chip gives a launch: the in-tree streaming read (the
    # attention kernels' access pattern, nothing else) over the whole 80-layer
    # cache in one launch, over one layer's worth (103.3 MB, the verify
    # grid) per launch in a graph of 80 dependent launches, and an empty launch
    achievable = measure_achievable(torch, ops, dev, kv, args.steps)

    # (3b) the draft and dense verify at batch 2 .. 32 (independent sequences:
    # the data-parallel axis), and the 7B and 32B shapes
    batch_sweep = measure_batch_sweep(torch, ops, dev, g, args.steps)
    other_shapes = measure_other_shapes(torch, ops, dev, g, args.steps)

    bytes_row = Hkv * D * 2 * 2                       # K + V bytes per key
    verify_bytes = N_full * bytes_row                 # per layer
    draft_bytes = N_draft * bytes_row
    us_verify = per_us["verify_attn"]
    us_draft = per_us["draft_attn"]
    decode_us_step = L * (us_verify + us_draft)
    decode_gbs = L * (verify_bytes + draft_bytes) / (decode_us_step * 1e-6) / 1e9
    verify_gbs = verify_bytes / (us_verify * 1e-6) / 1e9
    draft_gbs = draft_bytes / (us_draft * 1e-6) / 1e9
    us_score = per_us["score"]
    # pass 1 over every visible (text row, key) pair + pass 2 over (text row, visual key), 2*D flop each
    score_flop = 2 * D * Hq * (T * NV + T * (T + 1) // 2) + 2 * D * Hq * T * NV

    kernels = {
        k: {"us_avg": round(per_us[k], 3), **spread[k], "calls_per_step": calls[k]} for k in seqs
    }
    kernels["verify_attn"].update(bytes=verify_bytes, gbs=round(verify_gbs, 1))
    kernels["draft_attn"].update(bytes=draft_bytes, gbs=round(draft_gbs, 1))
    kernels["draft_attn_indexed"].update(
        bytes=draft_bytes, gbs=round(draft_bytes / (per_us["draft_attn_indexed"] * 1e-6) / 1e9, 1),
        what="the same draft read in place from the full cache through the key list (no gather)")
    uv_bytes = 2 * (NV + T) * d_model * 2
    kernels["uvprune_score"].update(
        bytes=uv_bytes, gbs=round(uv_bytes / (per_us["uvprune_score"] * 1e-6) / 1e9, 1),
        what="UV-Prune score from layer-0 and layer-L hidden states (hidden 8192), once per prefill")
    kernels["score"].update(flop=L * score_flop, tflops=round(L * score_flop / (us_score * 1e-6) / 1e12, 1),
                            us_per_layer=round(us_score / L, 3),
                            what="svlm_score_layers: all 80 layers in one call, averaged into one row")
    kernels["score_layer_calls"].update(
        flop=score_flop, tflops=round(score_flop / (per_us["score_layer_calls"] * 1e-6) / 1e12, 1),
        what="the same score as 80 svlm_score calls (one per layer, accumulated with alpha/beta)")
    # acceptance: the gamma test probabilities, then the one row (p_n and q_n, or the bonus row p_gamma)
    # the draw scans; latency-bound (one launch, dependent loads).  The kernel reads every candidate
    # row's chunk up front to save a round trip; the algorithmic bytes are the two rows the draw needs
    acc_bytes = 2 * V * 4
    kernels["accept"].update(bytes=acc_bytes, gbs=round(acc_bytes / (per_us["accept"] * 1e-6) / 1e9, 1),
                             what="rejection acceptance, gamma 5, V 152064: bytes = the two probability rows "
                                  "the draw needs (p_n and q_n); one launch of dependent loads")
    kernels["accept_in_sequence"].update(
        bytes=acc_bytes, gbs=round(acc_bytes / (per_us["accept_in_sequence"] * 1e-6) / 1e9, 1),
        what="the same acceptance call, 16 calls in one graph (per call)")
    gather_bytes = L * 2 * 2 * (B_keep + T) * Hkv * D * 2  # every layer's kept K and V rows, read + write
    kernels["gather"].update(bytes=gather_bytes, gbs=round(gather_bytes / (per_us["gather"] * 1e-6) / 1e9, 1),
                             what="one call over all layers (their caches folded into the head axis)")

    result = {
        "metric": METRIC,
        "value": round(decode_gbs, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": "llavaov72b_25k: 80 layers, 64 q / 8 KV heads, D 128, 128 frames x 14x14 = 25088 visual "
                        "+ 128 text tokens, batch 1; dense verify gamma 5 (6 queries, 25222 keys), 10% draft "
                        "(1 query, 2638 keys), Top-P 0.5 + uniform fill to 2509, rejection acceptance over 152064",
            "layers": L, "hq": Hq, "hkv": Hkv, "head_dim": D, "n_vis": NV, "n_text": T,
            "verify_queries": nqv, "verify_keys": N_full, "draft_keys": N_draft, "batch": 1,
        },
        "decode_attn_us_per_step": round(decode_us_step, 2),
        "roofline": {
            "bound": "hbm",
            "achieved": round(verify_gbs, 1),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(verify_gbs / HBM_PEAK_GBS, 4),
            "traffic": measured_traffic(),
            "kernel": "svlm_decode_attn dense verify call (split-K kernel + combine; 25222 keys x 8 KV heads "
                      "x 512 B = 103.3 MB per call)",
            # the same bytes through svlm_stream_read (the attention read pattern and nothing else),
            # one launch per 103.3 MB in a graph through the whole cache, on the fastest of five
            # grids: what a launch of this size gets on this chip
            "achievable_gbs": achievable["stream_read_per_launch_best"]["gbs"],
            "frac_of_achievable": round(verify_gbs / achievable["stream_read_per_launch_best"]["gbs"], 4),
        },
        "kernels": kernels,
        "parallel_decoding": {
            "us_per_step": round(pd_us, 2),
            # ParallelVLM "parallel decoding": window gamma = c* = T_p / T_q(alpha), here with the
            # attention times alone (dense verify call over one draft call, per layer)
            "speed_ratio_attn": round(us_verify / us_draft, 2),
            "window_gamma_attn": max(1, round(us_verify / us_draft)),
            "gbs": round(L * (verify_bytes + draft_bytes) / (pd_us * 1e-6) / 1e9, 1),
            "what": "80 dense-verify and 80 draft launches overlapped on two streams (one graph, two branches); "
                    "decode_attn_us_per_step runs them one after the other"},
        "hour_shape": hour,
        "achievable": achievable,
        "batch_sweep": batch_sweep,
        "other_shapes": other_shapes,
    }

    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(cfg, N_full, N_draft, bytes_row, args.cpu_seconds)
    print(json.dumps(result), flush=True)


def graph_us(torch, fn, calls, reps):
    """Per-call microseconds of the launch sequence fn() (calls launches),
    captured once as a HIP graph and timed by events around `reps` replays."""
    fn()
    torch.cuda.synchronize()
    gr = torch.cuda.CUDAGraph()
    with torch.cuda.graph(gr):
        fn()
    gr.replay()
    torch.cuda.synchronize()
    a = torch.cuda.Event(enable_timing=True)
    b = torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(reps):
        gr.replay()
    b.record()
    torch.cuda.synchronize()
    return a.elapsed_time(b) * 1e3 / (reps * calls)


def measure_achievable(torch, ops, dev, kv, steps):
    """The streaming read of svlm_stream_read: the whole 80-layer K and V cache
    in one launch; 103.3 MB per launch (two adjacent layers of K or of V, the
    bytes of one dense-verify call), 80 dependent launches in a graph through
    the whole cache, over the verify grid and over a sweep of grids (the best
    one is the reference); and 80 empty launches (the per-launch floor)."""
    sink = torch.empty(4096, dtype=torch.float32, device=dev)
    whole = kv.view(-1)
    nb_whole = whole.numel() * whole.element_size()
    us_whole = graph_us(torch, lambda: ops.stream_read(whole, 2048, sink), 1, max(2, steps // 2))
    L = kv.shape[1]
    pairs = [kv[w, l:l + 2].reshape(-1) for w in range(2) for l in range(0, L - 1, 2)]
    nb_pair = pairs[0].numel() * pairs[0].element_size()
    sweep = {}
    for wg in (216, 256, 512, 1024, 2048):
        us = graph_us(torch, lambda: [ops.stream_read(t, wg, sink) for t in pairs], len(pairs), steps)
        sweep[f"wg{wg}"] = round(us, 3)
    us_pair = sweep["wg216"]
    best_wg = min(sweep, key=sweep.get)
    us_best = sweep[best_wg]
    us_empty = graph_us(torch, lambda: [ops.stream_read(None, 1, sink) for _ in range(80)], 80, steps)

    def rate(us):
        return round(nb_pair / (us * 1e-6) / 1e9, 1)
    return {
        "stream_read_whole": {"bytes": nb_whole, "us": round(us_whole, 1),
                              "gbs": round(nb_whole / (us_whole * 1e-6) / 1e9, 1),
                              "what": "one launch over the 80-layer K and V cache, 2048 workgroups"},
        "stream_read_per_launch": {"bytes": nb_pair, "us_avg": round(us_pair, 3), "gbs": rate(us_pair),
                                   "frac": round(rate(us_pair) / HBM_PEAK_GBS, 4),
                                   "what": "103.3 MB (one dense-verify call's bytes) per launch over the verify "
                                           "grid (216 workgroups), 80 dependent launches in a graph"},
        "stream_read_per_launch_best": {"bytes": nb_pair, "us_avg": us_best, "gbs": rate(us_best),
                                        "frac": round(rate(us_best) / HBM_PEAK_GBS, 4), "grid": best_wg,
                                        "us_by_grid": sweep,
                                        "what": "the same 80 launches over 216 to 2048 workgroups; the fastest"},
        "empty_launch_us": round(us_empty, 3),
        "what": "svlm_stream_read: the attention kernels' read pattern (1 KB LDS-DMA transfers, 16 KB in "
                "flight per wave) and nothing else",
    }


def measure_batch_sweep(torch, ops, dev, g, steps, layers=8):
    """The 10% draft (2638 keys) and the dense verify (6 queries over 25222
    keys) at the 72B shape for batches of independent sequences, rotating over
    `layers` layer buffers: per-call time, GB/s and fraction of peak."""
    cfg = W.C3
    Hq, Hkv, D = cfg.hq, cfg.hkv, cfg.d
    row = Hkv * D * 2 * 2
    out = {}
    for kind, nq, N, batches in (("draft_attn", 1, cfg.budget + cfg.n_text + 1, (1, 2, 4, 8, 16, 32)),
                                 ("verify_attn", cfg.gamma_verify + 1, cfg.n_ctx + cfg.gamma_verify + 1, (1, 2, 4, 8, 16))):
        res = {}
        for B in batches:
            kvb = torch.empty(2, layers, B, Hkv, N, D, dtype=torch.bfloat16, device=dev)
            kvb.normal_(generator=g)
            qb = torch.randn(layers, B, nq, Hq, D, generator=g, device=dev).to(torch.bfloat16)
            ob = torch.empty(B, nq, Hq, D, device=dev)
            lb = torch.empty(B, nq, Hq, device=dev)
            kl = torch.full((B,), N, dtype=torch.int32, device=dev)
            ws = torch.empty(max(256, ops.decode_attn_workspace_bytes(B, nq, Hq, Hkv, D, N)), dtype=torch.uint8,
                             device=dev)
            us = graph_us(torch, lambda: [ops.decode_attn(qb[l], kvb[0, l], kvb[1, l], kl, nq > 1, out=ob, lse=lb,
                                                          ws=ws) for l in range(layers)], layers, steps)
            nb = B * N * row
            res[f"B{B}"] = {"us_avg": round(us, 3), "bytes": nb, "gbs": round(nb / (us * 1e-6) / 1e9, 1),
                            "frac": round(nb / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)}
            del kvb
        out[kind] = res
    out["what"] = ("72B shape, batches of independent sequences (one cache each); draft 1 query over 2638 keys, "
                   "verify 6 queries over 25222 keys; 8 rotating layer buffers")
    return out


def measure_other_shapes(torch, ops, dev, g, steps):
    """Dense verify, 10% draft and the score per layer at the Qwen2-VL-7B shape
    (28 layers, 28 q / 4 KV heads, 8192 + 64 tokens, gamma 9) and the
    Qwen2.5-VL-32B shape (64 layers, 40 q / 8 KV heads, 20736 + 96 tokens,
    gamma 9), rotating over enough layers to exceed the Infinity Cache."""
    out = {}
    for cfg, layers in ((W.C2, 28), (W.C4, 16)):
        Hq, Hkv, D, T, NV = cfg.hq, cfg.hkv, cfg.d, cfg.n_text, cfg.n_vis
        nq = cfg.gamma_verify + 1
        Nv = cfg.n_ctx + nq
        Nd = cfg.budget + T + 1
        row = Hkv * D * 2 * 2
        kv = torch.empty(2, layers, Hkv, Nv, D, dtype=torch.bfloat16, device=dev)
        kv.normal_(generator=g)
        qv = torch.randn(layers, 1, nq, Hq, D, generator=g, device=dev).to(torch.bfloat16)
        qt = torch.randn(layers, T, Hq, D, generator=g, device=dev).to(torch.bfloat16)
        o = torch.empty(1, nq, Hq, D, device=dev)
        lse = torch.empty(1, nq, Hq, device=dev)
        klv = torch.tensor([Nv], dtype=torch.int32, device=dev)
        kld = torch.tensor([Nd], dtype=torch.int32, device=dev)
        wsv = torch.empty(max(256, ops.decode_attn_workspace_bytes(1, nq, Hq, Hkv, D, Nv)), dtype=torch.uint8,
                          device=dev)
        wsd = torch.empty(max(256, ops.decode_attn_workspace_bytes(1, 1, Hq, Hkv, D, Nd)), dtype=torch.uint8,
                          device=dev)
        # the draft reads the first Nd rows of each layer's cache (timing only)
        us_v = graph_us(torch, lambda: [ops.decode_attn(qv[l], kv[0, l], kv[1, l], klv, True, out=o, lse=lse,
                                                        ws=wsv) for l in range(layers)], layers, steps)
        us_d = graph_us(torch, lambda: [ops.decode_attn(qv[l][:, :1], kv[0, l, :, :Nd], kv[1, l, :, :Nd], kld,
                                                        False, out=o[:, :1], lse=lse[:, :1], ws=wsd)
                                        for l in range(layers)], layers, steps)
        # the shape's selection rows (one averaged row, one per layer, or one per
        # (layer, KV head)) from every rotated layer in one call
        agg = "kvhead" if cfg.rows == "layer_kvhead" else "all"
        mean = cfg.rows == "all"
        kl = kv[0, :, :, :NV + T]
        wss = torch.empty(ops.score_layers_workspace_bytes(layers, T, Hq, Hkv, NV, NV), dtype=torch.uint8,
                          device=dev)
        srow = ops.score_layers(qt, kl, NV, NV, agg=agg, layer_mean=mean, ws=wss)
        us_s = graph_us(torch, lambda: ops.score_layers(qt, kl, NV, NV, agg=agg, layer_mean=mean, out=srow, ws=wss),
                        layers, max(2, steps // 2))
        flop = 2 * D * Hq * (T * NV + T * (T + 1) // 2) + 2 * D * Hq * T * NV
        out[cfg.name] = {
            "verify_attn": {"us_avg": round(us_v, 3), "bytes": Nv * row, "keys": Nv, "queries": nq,
                            "gbs": round(Nv * row / (us_v * 1e-6) / 1e9, 1),
                            "frac": round(Nv * row / (us_v * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)},
            "draft_attn": {"us_avg": round(us_d, 3), "bytes": Nd * row, "keys": Nd,
                           "gbs": round(Nd * row / (us_d * 1e-6) / 1e9, 1),
                           "frac": round(Nd * row / (us_d * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)},
            "score": {"us_avg": round(us_s, 3), "flop": flop, "tflops": round(flop / (us_s * 1e-6) / 1e12, 1),
                      "frac_bf16_peak": round(flop / (us_s * 1e-6) / 1e12 / 2500.0, 4)},
            "layers_rotated": layers,
        }
        del kv
    return out


def measure_hour_shape(torch, ops, dev, g, steps, layers=8):
    """Verify and in-place draft attention at the hour-long shape, rotating over
    `layers` layer buffers (2.3 GB of KV, well past the 256 MB Infinity Cache),
    and the per-(layer, KV head) top-K selection; per-call times from HIP
    events around graph replays."""
    c5 = W.C5
    Hq, Hkv, D = c5.hq, c5.hkv, c5.d
    nq = c5.gamma_verify + 1
    N = c5.n_ctx + nq                                  # 141194 keys
    n_draft = c5.budget + c5.n_text + 1                # 1089 keys per head
    kv = torch.empty(2, layers, Hkv, N, D, dtype=torch.bfloat16, device=dev)
    for l in range(layers):
        kv[:, l].copy_(torch.randn(2, Hkv, N, D, generator=g, device=dev, dtype=torch.float32))
    qv = torch.randn(layers, 1, nq, Hq, D, generator=g, device=dev, dtype=torch.float32).to(torch.bfloat16)
    qd = torch.randn(layers, 1, 1, Hq, D, generator=g, device=dev, dtype=torch.float32).to(torch.bfloat16)
    idx = torch.empty(Hkv, n_draft, dtype=torch.int32, device=dev)
    for h in range(Hkv):
        pick = torch.randperm(c5.n_vis, generator=g, device=dev)[:c5.budget]
        idx[h, :c5.budget] = torch.sort(pick).values.to(torch.int32)
        idx[h, c5.budget:] = torch.arange(c5.n_vis, c5.n_vis + c5.n_text + 1, dtype=torch.int32, device=dev)
    len_v = torch.tensor([N], dtype=torch.int32, device=dev)
    len_d = torch.tensor([n_draft], dtype=torch.int32, device=dev)
    ws_v = torch.empty(max(256, ops.decode_attn_workspace_bytes(1, nq, Hq, Hkv, D, N)), dtype=torch.uint8, device=dev)
    ws_d = torch.empty(max(256, ops.decode_attn_indexed_workspace_bytes(1, 1, Hq, Hkv, D, n_draft)),
                       dtype=torch.uint8, device=dev)
    o_v = torch.empty(1, nq, Hq, D, dtype=torch.float32, device=dev)
    l_v = torch.empty(1, nq, Hq, dtype=torch.float32, device=dev)
    o_d = torch.empty(1, 1, Hq, D, dtype=torch.float32, device=dev)
    l_d = torch.empty(1, 1, Hq, dtype=torch.float32, device=dev)

    def verify():
        for l in range(layers):
            ops.decode_attn(qv[l], kv[0, l], kv[1, l], len_v, True, out=o_v, lse=l_v, ws=ws_v)

    def draft():
        for l in range(layers):
            ops.decode_attn_indexed(qd[l], kv[0, l], kv[1, l], idx, len_d, False, out=o_d, lse=l_d, ws=ws_d)

    # selection at this shape: one row per (layer, KV head), 28 x 4 = 112 rows of
    # 141120 scores, pure top-K = 1024 (Sparse-to-Dense explainer, "KV cache
    # selection"); heavy-tailed synthetic rows, each summing to 1
    R = c5.layers * Hkv
    srows = torch.rand(R, c5.n_vis, generator=g, device=dev, dtype=torch.float32).pow_(8.0)
    srows.div_(srows.sum(dim=1, keepdim=True))

    def select():
        ops.select(srows, c5.frames, c5.gh, c5.gw, c5.top_p, c5.budget)

    # greedy acceptance of a gamma = 9 window over vocabulary 152064 (the
    # hour-long configuration's acceptance): every row's argmax; the drafts
    # match the first five, so the walk stops at the sixth; 16 calls per graph
    gv = c5.gamma_verify
    V = 152064
    logits = torch.randn(1, gv + 1, V, generator=g, device=dev, dtype=torch.float32)
    dtok = torch.randint(0, V, (1, gv), generator=g, device=dev, dtype=torch.int32)
    dtok[0, :5] = logits[0, :5].argmax(dim=-1).to(torch.int32)
    ws_a = torch.zeros(ops.verify_workspace_bytes(1, gv, V), dtype=torch.uint8, device=dev)

    def accept_greedy():
        for _ in range(16):
            ops.verify("greedy", dtok, logits, ws=ws_a)

    out = {}
    row = Hkv * D * 2 * 2
    for name, fn, nbytes, n_calls in (("verify_attn", verify, N * row, layers),
                                      ("draft_attn_indexed", draft, n_draft * row, layers),
                                      ("select", select, R * (c5.n_vis + c5.budget) * 4, 1),
                                      ("accept_greedy", accept_greedy, (gv + 1) * V * 4, 16)):
        fn()
        torch.cuda.synchronize()
        gr = torch.cuda.CUDAGraph()
        with torch.cuda.graph(gr):
            fn()
        gr.replay()
        torch.cuda.synchronize()
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(steps):
            gr.replay()
        b.record()
        torch.cuda.synchronize()
        us = a.elapsed_time(b) * 1e3 / (steps * n_calls)
        gbs = nbytes / (us * 1e-6) / 1e9
        out[name] = {"us_avg": round(us, 3), "bytes": nbytes, "gbs": round(gbs, 1),
                     "frac": round(gbs / HBM_PEAK_GBS, 4)}
    out["select"]["what"] = ("112 rows (28 layers x 4 KV heads) x 141120 scores, top-K 1024; bytes = scores read "
                             "once + indices written")
    out["verify_attn"]["what"] = "dense verify, 10 queries x 141194 keys, 28 q / 4 KV heads, D 128"
    out["draft_attn_indexed"]["what"] = ("draft, 1 query over per-head lists of 1024 visual + 64 text + 1 rows "
                                         "read in place")
    out["accept_greedy"]["what"] = ("greedy acceptance, gamma 9, V 152064, one launch per call (16 calls per "
                                    "graph); bytes = the 10 logit rows, each read once")
    del kv, qv, qd, logits, ws_a
    torch.cuda.empty_cache()
    # the selection rows themselves: the score of all 28 layers in one call,
    # one row per (layer, KV head), over 141120 visual + 64 text keys
    T, NV, L = c5.n_text, c5.n_vis, c5.layers
    k = torch.empty(L, Hkv, NV + T, D, dtype=torch.bfloat16, device=dev)
    for l in range(L):
        k[l].copy_(torch.randn(Hkv, NV + T, D, generator=g, device=dev, dtype=torch.float32))
    qt = torch.randn(L, T, Hq, D, generator=g, device=dev, dtype=torch.float32).to(torch.bfloat16)
    ws_s = torch.empty(ops.score_layers_workspace_bytes(L, T, Hq, Hkv, NV, NV), dtype=torch.uint8, device=dev)
    rows = ops.score_layers(qt, k, NV, NV, agg="kvhead", layer_mean=False, ws=ws_s)
    us = graph_us(torch, lambda: ops.score_layers(qt, k, NV, NV, agg="kvhead", layer_mean=False, out=rows, ws=ws_s),
                  L, max(2, steps // 2))
    flop = 2 * D * Hq * (T * NV + T * (T + 1) // 2) + 2 * D * Hq * T * NV
    out["score"] = {"us_avg": round(us, 3), "flop": flop, "tflops": round(flop / (us * 1e-6) / 1e12, 1),
                    "frac_bf16_peak": round(flop / (us * 1e-6) / 1e12 / 2500.0, 4),
                    "what": "per layer: the 28 layers' score in one call, one row per (layer, KV head) = the 112 "
                            "rows the selection takes"}
    del k, qt, ws_s, rows
    return out


def cpu_baseline(cfg, N_full, N_draft, bytes_row, budget_s):
    """The fp64 NumPy oracle on a bounded sample of the same workload, on this host's cores."""
    import oracle
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        threads = 1
    nqv = cfg.gamma_verify + 1
    done_bytes = 0
    t_used = 0.0
    layers = 0
    while t_used < budget_s and layers < cfg.layers:
        k, v = W.random_kv(cfg.index, cfg.hkv, N_full, cfg.d, layer=layers)
        qv = W.decode_queries(cfg, layers, nqv)
        t0 = time.perf_counter()
        oracle.decode_attn(qv, k, v, [N_full], True)
        oracle.decode_attn(qv[:, :1], k[:, :N_draft], v[:, :N_draft], [N_draft], False)
        t_used += time.perf_counter() - t0
        done_bytes += (N_full + N_draft) * bytes_row
        layers += 1
    # one layer on one thread
    one_thread_s = None
    try:
        from threadpoolctl import threadpool_limits
        k, v = W.random_kv(cfg.index, cfg.hkv, N_full, cfg.d, layer=0)
        qv = W.decode_queries(cfg, 0, nqv)
        with threadpool_limits(limits=1):
            t0 = time.perf_counter()
            oracle.decode_attn(qv, k, v, [N_full], True)
            oracle.decode_attn(qv[:, :1], k[:, :N_draft], v[:, :N_draft], [N_draft], False)
            one_thread_s = time.perf_counter() - t0
    except Exception:  # pragma: no cover
        pass
    return {
        "value": round(done_bytes / t_used / 1e9, 3),
        "unit": "GB/s",
        "cores": int(threads),
        "kind": "oracle",
        "cpu_model": cpu_model(),
        "one_layer_1thread_s": round(one_thread_s, 3) if one_thread_s is not None else None,
        "one_layer_1thread_gbs": round((N_full + N_draft) * bytes_row / one_thread_s / 1e9, 4)
        if one_thread_s else None,
        "sample": f"{layers} layer(s) of dense verify (6 queries x 25222 keys) + 10% draft (1 x 2638 keys), "
                  f"64 q / 8 KV heads, fp64 NumPy, {t_used:.1f} s; per-step figures would be x80 extrapolations",
    }


def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    import platform
    return platform.processor() or "unknown"


if __name__ == "__main__":
    main()
