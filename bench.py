#!/usr/bin/env python3
"""Throughput benchmark of the Qwen3 decoder forward on one MI355X.

Default workload (the one the JSON line's value is quoted on): the 28-layer
Qwen3-0.6B-shaped stack, prefill of 4 sequences x 2048 tokens with the tied LM head on
every position (fp32 logits) and the greedy next token; one step = one forward pass.
Also measured, reported under "workloads": one decode step of the same stack at batch
64 against a 4096-token KV cache, the routed MoE FFN layer (8192 tokens, 128 experts,
top-8, skewed load), the 7B-shaped block at 32768 tokens and the 0.6B block at 128.

All inputs are seeded synthetic data generated directly in HBM; the timed region
contains only library calls.  Per-kernel durations come from HIP events the library
records around the launches of one kernel class (qwen3_profile_begin/end).  A short
breakdown run first times every kernel class; the timed region then records the events
of the dominant one (largest time per step), whose roofline uses algorithmic flops or
bytes per launch.  "traffic" is the HBM bytes per launch of that kernel from the
committed rocprofv3 counter table (profiles/traffic.json), null once the kernel's sources
differ from those the counters were taken with.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--workloads a,b,...]
"""
import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "prefill & decode tokens/s, Qwen3-0.6B-shape stack; % of bf16 MFMA / HBM peak"
PEAK_MFMA_TFLOPS = 2500.0  # MI355X dense fp16 / bf16 matrix-core peak
PEAK_HBM_GBS = 8000.0      # MI355X HBM3E peak


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def roofline_mfma(flops_per_launch, avg_ms, traffic=None):
    ach = flops_per_launch / (avg_ms * 1e-3) / 1e12
    return {"bound": "mfma", "achieved": round(ach, 2), "peak": PEAK_MFMA_TFLOPS,
            "unit": "TFLOP/s", "frac": round(ach / PEAK_MFMA_TFLOPS, 4), "traffic": traffic}


def roofline_hbm(bytes_per_launch, avg_ms, traffic=None):
    ach = bytes_per_launch / (avg_ms * 1e-3) / 1e9
    return {"bound": "hbm", "achieved": round(ach, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
            "frac": round(ach / PEAK_HBM_GBS, 4), "traffic": traffic}


class Timer:
    """Times K calls of fn on torch's current stream with HIP events; optionally has the
    library time one kernel class over the same region."""

    def __init__(self, torch, q3):
        self.torch, self.q3 = torch, q3

    def run(self, fn, steps, warmup, tag=None, launches_per_step=1, per_step=None):
        """Mean ms per step over `steps` back-to-back calls (events before the first and
        after the last); with a dict `per_step`, also the median and minimum of the
        per-call durations (an event between consecutive calls)."""
        torch, q3 = self.torch, self.q3
        for _ in range(warmup):
            fn()
        torch.cuda.synchronize()
        if tag:
            q3.qwen3_profile_begin(tag, steps * launches_per_step)
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
        ev[0].record()
        for i in range(steps):
            fn()
            ev[i + 1].record()
        torch.cuda.synchronize()
        total = ev[0].elapsed_time(ev[-1])
        if per_step is not None:
            d = sorted(ev[i].elapsed_time(ev[i + 1]) for i in range(steps))
            per_step["ms_per_step_median"] = d[len(d) // 2] if len(d) % 2 else \
                0.5 * (d[len(d) // 2 - 1] + d[len(d) // 2])
            per_step["ms_per_step_min"] = d[0]
        kernel = None
        if tag:
            kms, n = q3.qwen3_profile_end()
            kernel = {"tag": tag, "launches": n, "avg_ms": kms / max(n, 1)}
        return total / steps, kernel

    def run_cold(self, fn, steps, flush_bytes):
        """Per-call durations with the caches flushed before each call: a buffer of
        flush_bytes (larger than the 256 MB last-level cache) is written between calls,
        outside the timed events.  Returns (median, min) ms."""
        torch = self.torch
        buf = torch.empty(flush_bytes // 4, dtype=torch.float32, device="cuda")
        d = []
        for i in range(steps):
            buf.fill_(float(i))
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record()
            fn()
            e1.record()
            torch.cuda.synchronize()
            d.append(e0.elapsed_time(e1))
        del buf
        d.sort()
        return d[len(d) // 2], d[0]


# ------------------------------------------------------------------------- workloads

def setup_stack(torch, q3, recipes, dev, cfg, B, S, cap, seed_model, seed_in):
    model = recipes.model_device(seed_model, cfg, dev)
    mw, keep = q3.make_model_weights(model["embed"], model["norm"], model["layers"],
                                     model["lm_head"])
    rope = torch.empty(2 * cfg["max_position_embeddings"] * 64, dtype=torch.float32, device=dev)
    q3.qwen3_rope_table_init(cfg, rope)
    L, nkv = cfg["num_hidden_layers"], cfg["num_key_value_heads"]
    caches = []
    for _ in range(L):
        caches.append(q3.kv_cache_empty(B, nkv, cap, dev))
    return model, mw, keep, rope, caches


def wl_prefill(torch, q3, recipes, synth, dev, steps, warmup, timer, breakdown, routed=False):
    cfg = dict(recipes.QWEN3_0P6B)
    name = "stack_0p6b_prefill"
    if routed:
        # the two-expert variant of the 0.6B model: every layer's MLP is a top-1 routed
        # pair of experts of the dense MLP's shape, gated by bf16 probabilities
        cfg.update(recipes.MOE_2E)
        name = "stack_0p8b_2e_prefill"
    B, S = 4, 2048
    model, mw, keep, rope, caches = setup_stack(torch, q3, recipes, dev, cfg, B, S, S,
                                                recipes.MODEL_SEED_0P6B, 2)
    kvs = [q3.make_kv_layer(k, vt, S) for k, vt in caches]
    ids = torch.empty((B, S), dtype=torch.int32, device=dev)
    synth.uniform_i32_device(ids, 2, "input.ids", 0, cfg["vocab_size"])
    V = cfg["vocab_size"]
    logits = torch.empty((B, S, V), dtype=torch.float32, device=dev)
    nxt = torch.empty((B,), dtype=torch.int32, device=dev)
    ws = torch.empty(q3.qwen3_workspace_bytes(cfg, q3.QWEN3_OP_STACK_PREFILL, B, S),
                     dtype=torch.uint8, device=dev)

    def step():
        q3.qwen3_stack_forward(cfg, mw, rope, ids, B, S, 0, None, kvs, logits,
                               q3.QWEN3_LOGITS_ALL, nxt, ws)

    L, H, I = cfg["num_hidden_layers"], cfg["hidden_size"], cfg["intermediate_size"]
    T = B * S
    units = dense_units(cfg, B, S, L)
    units["lm_head_gemm"] = ("mfma", 2.0 * T * H * V, 1)
    units["argmax"] = ("hbm", 4.0 * B * V, 1)
    if routed:
        for tag in ("gate_up_gemm", "down_gemm"):
            del units[tag]
        units.update(moe_units(cfg, T, L))
    ms, dom, rf, kernels, stats = measure(timer, step, steps, warmup, name, units, "attn_prefill",
                                   breakdown)
    out = {"name": name, "tokens_per_s": T / (ms * 1e-3), "ms_per_step": ms,
           "config": {"workload": name, "batch": B, "seq_len": S, "layers": L,
                      "hidden": H, "heads": "16q/8kv x128", "intermediate": I, "vocab": V,
                      "lm_head": "tied, fp32 logits for all positions",
                      "greedy_next_token": True},
           "dominant_kernel": dom, "roofline": rf}
    if routed:
        out["config"].update(experts=cfg["num_experts"], top_k=cfg["num_experts_per_tok"],
                             expert_intermediate=cfg["moe_intermediate_size"],
                             gating="bf16 probabilities, not renormalised")
        del out["config"]["intermediate"]
    total_flops = stack_prefill_flops(cfg, B, S)
    out["whole_step_mfma_frac"] = round(total_flops / (ms * 1e-3) / 1e12 / PEAK_MFMA_TFLOPS, 4)
    out["algorithmic_tflop_per_step"] = round(total_flops / 1e12, 3)
    out.update({k: round(v, 4) for k, v in stats.items()})
    if kernels:
        out["kernels"] = kernels
    del logits, caches, kvs, model, ws
    torch.cuda.empty_cache()
    return out


def dense_units(cfg, B, S, launches):
    """Algorithmic work per launch of each dense-block kernel class for a prefill of B x S
    tokens from position 0 (causal pairs only).  Above 256 tokens the q/k-norm + RoPE +
    cache writes run in the QKV projection's epilogue; below, as a separate pass priced at
    the bytes it moves: fp16 q/k/v in, fp16 q and bf16 cache plus fp16 fresh K/V out."""
    H, nq, nkv, hd, I = (cfg["hidden_size"], cfg["num_attention_heads"],
                         cfg["num_key_value_heads"], cfg["head_dim"], cfg["intermediate_size"])
    T = B * S
    rope_bytes = T * (nq + 2 * nkv) * hd * 2 + T * nq * hd * 2 + 4.0 * T * nkv * hd * 2
    units = {
        "qkv_gemm": ("mfma", 2.0 * T * H * (nq + 2 * nkv) * hd, launches),
        "attn_prefill": ("mfma", 4.0 * hd * nq * B * S * (S + 1) / 2, launches),
        "o_proj_gemm": ("mfma", 2.0 * T * nq * hd * H, launches),
        "gate_up_gemm": ("mfma", 2.0 * T * H * 2 * I, launches),
        "down_gemm": ("mfma", 2.0 * T * I * H, launches),
    }
    if T <= 256:
        units["qk_norm_rope_cache"] = ("hbm", float(rope_bytes), launches)
    return units


def moe_units(cfg, T, launches):
    """Algorithmic work per launch of the routed-FFN kernel classes for T tokens."""
    H, E, k, I = (cfg["hidden_size"], cfg["num_experts"], cfg["num_experts_per_tok"],
                  cfg["moe_intermediate_size"])
    return {
        "moe_router_gemm": ("mfma", 2.0 * T * E * H, launches),
        "moe_route": ("hbm", 4.0 * T * E + 8.0 * T * k * 3, launches),
        "moe_gate_up_gemm": ("mfma", 2.0 * T * k * 2 * I * H, launches),
        "moe_down_gemm": ("mfma", 2.0 * T * k * I * H, launches),
        "moe_combine": ("hbm", 4.0 * T * k * H + 2.0 * T * H, launches),
    }


def stack_prefill_flops(cfg, B, S):
    H, nq, nkv, hd, I, L, V = (cfg["hidden_size"], cfg["num_attention_heads"],
                               cfg["num_key_value_heads"], cfg["head_dim"],
                               cfg["intermediate_size"], cfg["num_hidden_layers"],
                               cfg["vocab_size"])
    T = B * S
    ffn = 3 * I
    if cfg.get("num_experts", 0) > 0 and cfg.get("decoder_sparse_step", 0) == 1:
        ffn = cfg["num_experts"] + 3 * cfg["num_experts_per_tok"] * cfg["moe_intermediate_size"]
    gemm = 2.0 * T * H * ((nq + 2 * nkv) * hd + nq * hd + ffn)
    attn = 4.0 * hd * nq * B * S * (S + 1) / 2
    return L * (gemm + attn) + 2.0 * T * H * V


def kernel_breakdown(timer, step, units, steps):
    """Per kernel class: average launch duration (HIP events around each launch) and its
    roofline fraction from the algorithmic work per launch in `units`:
    tag -> (bound "mfma" | "hbm", flops or bytes per launch, launches per step)."""
    res = {}
    for tag, (bound, amount, per_step) in units.items():
        _, k = timer.run(step, steps, 1, tag=tag, launches_per_step=per_step)
        if not k["launches"]:
            continue  # this configuration does not launch that kernel
        e = {"avg_ms": round(k["avg_ms"], 4), "launches_per_step": per_step,
             "ms_per_step": round(k["avg_ms"] * per_step, 4), "bound": bound}
        if amount:
            rf = (roofline_mfma if bound == "mfma" else roofline_hbm)(amount, k["avg_ms"])
            e["frac"] = rf["frac"]
        res[tag] = e
    return res


# Products of at most 256 rows run on the decode-size GEMM kernel, whose counter entries
# carry their own tags (o_proj and down share one instantiation).
DECODE_SIZE_TAGS = {"qkv_gemm": "decode_qkv_gemm", "gate_up_gemm": "decode_gate_up_gemm",
                    "o_proj_gemm": "decode_res_gemm", "down_gemm": "decode_res_gemm"}


def measure(timer, step, steps, warmup, workload, units, default_tag, breakdown,
            traffic_tags=None):
    """Breakdown first (short runs), then the timed region with the dominant kernel class
    (largest time per step) recording its launch events live.  traffic_tags maps a kernel
    class to the tag of its counter entry where the two differ."""
    kernels = kernel_breakdown(timer, step, units, min(steps, 3)) if breakdown else None
    tag = default_tag
    if kernels:
        tag = max(kernels, key=lambda t: kernels[t]["ms_per_step"])
    bound, amount, per_step = units[tag]
    stats = {}
    ms, kern = timer.run(step, steps, warmup, tag=tag, launches_per_step=per_step,
                         per_step=stats)
    from decoder_only_forward_amd import profiling
    traffic = profiling.traffic_for(workload, (traffic_tags or {}).get(tag, tag))
    rf = (roofline_mfma if bound == "mfma" else roofline_hbm)(amount, kern["avg_ms"], traffic)
    dom = dict(kern, **({"flops_per_launch": amount} if bound == "mfma"
                        else {"bytes_per_launch": amount}))
    return ms, dom, rf, kernels, stats


def wl_decode(torch, q3, recipes, synth, dev, steps, warmup, timer, breakdown, S=1):
    """Decode of S new tokens per sequence (S = 1: one step; S > 1: the tokens of one
    sequence are decoded together, each seeing the cache and the new tokens before it)."""
    cfg = dict(recipes.QWEN3_0P6B)
    B, ctx = 64, 4096
    cap = 4160
    name = "stack_0p6b_decode" if S == 1 else f"stack_0p6b_decode_{S}tok"
    model, mw, keep, rope, caches = setup_stack(torch, q3, recipes, dev, cfg, B, 1, cap,
                                                recipes.MODEL_SEED_0P6B, 3)
    t0 = time.time()
    # the generator fills logical [B, nkv, cap, 128] tensors; copy them into the tiled cache
    k_log = torch.empty((B, cfg["num_key_value_heads"], cap, 128), dtype=torch.bfloat16,
                        device=dev)
    v_log = torch.empty_like(k_log)
    for l, (k, vt) in enumerate(caches):
        recipes.kv_fill_device(k_log, v_log, 3, l, ctx, ctx)
        q3.k_cache_from_logical(k_log, out=k)
        q3.v_cache_from_logical(v_log, out=vt)
    del k_log, v_log
    torch.cuda.synchronize()
    log(f"  decode: KV cache {len(caches)} x 2 x {tuple(caches[0][0].shape)} filled in "
        f"{time.time() - t0:.1f}s")
    kvs = [q3.make_kv_layer(k, vt, cap) for k, vt in caches]
    ids = torch.empty((B, S), dtype=torch.int32, device=dev)
    synth.uniform_i32_device(ids, 3, "input.ids", 0, cfg["vocab_size"])
    pos = torch.full((B,), ctx, dtype=torch.int32, device=dev)
    V = cfg["vocab_size"]
    mode = q3.QWEN3_LOGITS_LAST if S == 1 else q3.QWEN3_LOGITS_ALL
    logits = torch.empty((B * S, V), dtype=torch.float32, device=dev)
    nxt = torch.empty((B,), dtype=torch.int32, device=dev)
    ws = torch.empty(q3.qwen3_workspace_bytes(cfg, q3.QWEN3_OP_STACK_DECODE, B, S),
                     dtype=torch.uint8, device=dev)

    def step():
        q3.qwen3_stack_forward(cfg, mw, rope, ids, B, S, 0, pos, kvs, logits, mode, nxt, ws)

    L, nkv, nq = cfg["num_hidden_layers"], cfg["num_key_value_heads"], cfg["num_attention_heads"]
    H, hd, I = cfg["hidden_size"], cfg["head_dim"], cfg["intermediate_size"]
    T = B * S
    kv_bytes = 2.0 * B * nkv * (ctx + S) * hd * 2
    g = nq // nkv
    nqg = -(-(S * g) // 8)
    nsplit = min(-(-cap // 256), max(-(-cap // 8192), -(-512 // (B * nqg * nkv))))
    part_bytes = 4.0 * T * nq * nsplit * (hd + 2)  # split partials: design bytes, not algorithmic
    units = {
        # weights dominate the skinny GEMMs; activations in/out are counted too
        "qkv_gemm": ("hbm", 2.0 * H * (nq + 2 * nkv) * hd + 2.0 * T * H
                     + 2.0 * T * (nq + 2 * nkv) * hd, L),
        "qk_norm_rope_cache": ("hbm", 2.0 * T * (nq + 2 * nkv) * hd + 2.0 * T * nq * hd
                               + 2.0 * T * 2 * nkv * hd, L),
        "attn_decode": ("hbm", kv_bytes + 2.0 * T * nq * hd, L),
        "attn_decode_combine": ("hbm", part_bytes + 2.0 * T * nq * hd, L),
        "o_proj_gemm": ("hbm", 2.0 * nq * hd * H + 2.0 * T * nq * hd + 8.0 * T * H, L),
        "gate_up_gemm": ("hbm", 2.0 * 2 * I * H + 2.0 * T * H + 2.0 * T * I, L),
        "down_gemm": ("hbm", 2.0 * I * H + 2.0 * T * I + 8.0 * T * H, L),
        "lm_head_gemm": ("hbm", 2.0 * V * H + 4.0 * T * V, 1),
        "argmax": ("hbm", 4.0 * B * V, 1),
    }
    ms, dom, rf, kernels, stats = measure(timer, step, steps, warmup, name, units, "attn_decode",
                                   breakdown, DECODE_SIZE_TAGS if T <= 256 else None)
    step_bytes = decode_step_bytes(cfg, B, ctx, S)
    out = {"name": name, "tokens_per_s": T / (ms * 1e-3), "ms_per_step": ms,
           "config": {"workload": name, "batch": B, "context": ctx,
                      "new_tokens_per_seq": S, "layers": L, "greedy_next_token": True},
           "dominant_kernel": dom, "roofline": rf,
           "whole_step_hbm_frac": round(step_bytes / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
           "algorithmic_gb_per_step": round(step_bytes / 1e9, 3)}
    out.update({k: round(v, 4) for k, v in stats.items()})
    if kernels:
        out["kernels"] = kernels
    del caches, kvs, model, ws, logits
    torch.cuda.empty_cache()
    return out


def wl_generate(torch, q3, recipes, synth, dev, steps, warmup, timer, sampled):
    """Generation on the device: a 512-token prompt per sequence, then 64 new tokens each
    (prefill + 63 decode steps inside one qwen3_generate call), greedy or sampled."""
    cfg = dict(recipes.QWEN3_0P6B)
    B, S, n_new = 64, 512, 64
    cap = ((S + n_new - 1 + 63) // 64) * 64
    model, mw, keep, rope, caches = setup_stack(torch, q3, recipes, dev, cfg, B, S, cap,
                                                recipes.MODEL_SEED_0P6B, 4)
    kvs = [q3.make_kv_layer(k, vt, cap) for k, vt in caches]
    ids = torch.empty((B, S), dtype=torch.int32, device=dev)
    synth.uniform_i32_device(ids, 4, "input.ids", 0, cfg["vocab_size"])
    out = torch.empty((B, n_new), dtype=torch.int32, device=dev)
    ws = torch.empty(q3.qwen3_workspace_bytes(cfg, q3.QWEN3_OP_GENERATE, B, S),
                     dtype=torch.uint8, device=dev)
    T, top_p, uni = 0.0, 1.0, None
    if sampled:
        T, top_p = 0.8, 0.95
        gen = torch.Generator(device=dev)
        gen.manual_seed(4)
        uni = torch.rand((n_new, B), generator=gen, device=dev, dtype=torch.float32)

    def step():
        q3.qwen3_generate(cfg, mw, rope, ids, B, S, n_new, kvs, out, ws, temperature=T,
                          top_p=top_p, uniforms=uni)

    ms, _ = timer.run(step, steps, warmup)
    name = "generate_0p6b" + ("_sampled" if sampled else "_greedy")
    res = {"name": name, "tokens_per_s": B * n_new / (ms * 1e-3), "ms_per_step": ms,
           "config": {"workload": name, "batch": B, "prompt": S, "new_tokens_per_seq": n_new,
                      "layers": cfg["num_hidden_layers"],
                      "selection": (f"sampled (temperature {T}, top_p {top_p})" if sampled
                                    else "greedy")},
           "note": "tokens_per_s counts generated tokens; ms_per_step is one whole generation "
                   "(prompt prefill + 63 decode steps)"}
    del caches, kvs, model, ws, out
    torch.cuda.empty_cache()
    return res


def decode_step_bytes(cfg, B, ctx, S=1):
    H, nq, nkv, hd, I, L, V = (cfg["hidden_size"], cfg["num_attention_heads"],
                               cfg["num_key_value_heads"], cfg["head_dim"],
                               cfg["intermediate_size"], cfg["num_hidden_layers"],
                               cfg["vocab_size"])
    layer_w = 2.0 * (H * (nq + 2 * nkv) * hd + nq * hd * H + 3 * I * H + 2 * H + 2 * hd)
    kv_read = 2.0 * B * nkv * (ctx + S) * hd * 2
    kv_write = 2.0 * B * S * nkv * hd * 2
    logits = 4.0 * B * S * V if S > 1 else 4.0 * B * V
    return L * (layer_w + kv_read + kv_write) + 2.0 * V * H + logits


def wl_moe(torch, q3, recipes, synth, dev, steps, warmup, timer, breakdown):
    import numpy as np
    cfg = dict(recipes.MOE_2048)
    T = 8192
    router, gu, dn = recipes.moe_device(4, cfg, dev)
    w = q3.make_moe_weights(router, gu, dn)
    x = torch.empty((T, cfg["hidden_size"]), dtype=torch.bfloat16, device=dev)
    synth.normal_bf16_device(x, 4, recipes.activations_name(), 0.0, 1.0)
    y = torch.empty_like(x)
    E, k = cfg["num_experts"], cfg["num_experts_per_tok"]
    offsets = torch.empty((E + 1,), dtype=torch.int32, device=dev)
    ws = torch.empty(q3.qwen3_workspace_bytes(cfg, q3.QWEN3_OP_MOE_FFN, T), dtype=torch.uint8,
                     device=dev)

    def step():
        q3.qwen3_moe_ffn(cfg, w, x, y, T, None, None, None, offsets, None, None, ws)

    H, I = cfg["hidden_size"], cfg["moe_intermediate_size"]
    units = moe_units(cfg, T, 1)
    ms, dom, rf, kernels, stats = measure(timer, step, steps, warmup, "moe_ffn", units,
                                   "moe_gate_up_gemm", breakdown)
    counts = (offsets[1:] - offsets[:-1]).cpu().numpy()
    tile_rows = int(((counts + 255) // 256 * 256).sum())
    total = 2.0 * T * E * H + 2.0 * T * k * 2 * I * H + 2.0 * T * k * I * H
    # per expert: its rows' share of the 256-row tiles it occupies, and its own roofline time
    # (its gate|up and down flops at the MFMA peak, or its weights at the HBM peak, whichever
    # is longer); the sum over experts is the time a perfect kernel would need expert by expert
    live = counts[counts > 0]
    row_use = live / ((live + 255) // 256 * 256)
    t_exp = np.maximum(live * 6.0 * I * H / (PEAK_MFMA_TFLOPS * 1e12),
                       3.0 * I * H * 2 / (PEAK_HBM_GBS * 1e9))
    per_expert = {"tile_row_use_min": round(float(row_use.min()), 4),
                  "tile_row_use_median": round(float(np.median(row_use)), 4),
                  "below_ridge": int((live * 6.0 * I * H / (PEAK_MFMA_TFLOPS * 1e12) <
                                      3.0 * I * H * 2 / (PEAK_HBM_GBS * 1e9)).sum()),
                  "roofline_sum_ms": round(float(t_exp.sum()) * 1e3, 4),
                  "frac_of_roofline_sum": round(float(t_exp.sum()) * 1e3 / ms, 4)}
    out = {"name": "moe_ffn", "tokens_per_s": T / (ms * 1e-3), "ms_per_step": ms,
           "config": {"workload": "moe_ffn_2048x128e_top8", "tokens": T, "hidden": H,
                      "experts": E, "top_k": k, "expert_intermediate": I,
                      "load_max_over_mean": round(float(counts.max() / counts.mean()), 2),
                      "load_min": int(counts.min()), "load_max": int(counts.max()),
                      "experts_below_256_rows": int((counts < 256).sum()),
                      "grouped_tile_row_use": round(float(counts.sum()) / tile_rows, 4),
                      "per_expert": per_expert},
           "dominant_kernel": dom, "roofline": rf,
           "whole_step_mfma_frac": round(total / (ms * 1e-3) / 1e12 / PEAK_MFMA_TFLOPS, 4)}
    out.update({k: round(v, 4) for k, v in stats.items()})
    if kernels:
        out["kernels"] = kernels
    del router, gu, dn, ws
    torch.cuda.empty_cache()
    return out


def wl_block(torch, q3, recipes, synth, dev, steps, warmup, timer, breakdown, big,
             rope_interleaved=0):
    cfg = dict(recipes.QWEN_7B_BLOCK if big else recipes.QWEN3_0P6B)
    cfg["rope_interleaved"] = rope_interleaved
    B, S = (1, 32768) if big else (1, 128)
    seed = 5 if big else 1
    w = recipes.layer_device(seed, cfg, 0, dev)
    rope = torch.empty(2 * cfg["max_position_embeddings"] * 64, dtype=torch.float32, device=dev)
    q3.qwen3_rope_table_init(cfg, rope)
    nkv = cfg["num_key_value_heads"]
    cap = ((S + 63) // 64) * 64
    k, vt = q3.kv_cache_empty(B, nkv, cap, dev)
    kv = q3.make_kv_layer(k, vt, cap)
    H = cfg["hidden_size"]
    x = torch.empty((B, S, H), dtype=torch.bfloat16, device=dev)
    synth.normal_bf16_device(x, seed, recipes.activations_name(), 0.0, 1.0)
    xo = torch.empty_like(x)
    ws = torch.empty(q3.qwen3_workspace_bytes(cfg, q3.QWEN3_OP_BLOCK_PREFILL, B, S),
                     dtype=torch.uint8, device=dev)

    def step():
        q3.qwen3_block_prefill(cfg, w, rope, x, xo, B, S, 0, kv, ws)

    c1 = dict(cfg, num_hidden_layers=1, vocab_size=0)
    flops = stack_prefill_flops(c1, B, S)
    nq = cfg["num_attention_heads"]
    name = ("block_7b" if big else "block_0p6b") + ("_rope_interleaved" if rope_interleaved else "")
    units = dense_units(cfg, B, S, 1)
    ms, dom, rf, kernels, stats = measure(timer, step, steps, warmup, name, units, "attn_prefill",
                                   breakdown, DECODE_SIZE_TAGS if B * S <= 256 else None)
    out = {"name": name, "tokens_per_s": B * S / (ms * 1e-3), "ms_per_step": ms,
           "config": {"workload": name, "batch": B, "seq_len": S, "hidden": H,
                      "heads": f"{nq}q/{nkv}kv x128", "intermediate": cfg["intermediate_size"],
                      "rope": "interleaved pairs" if rope_interleaved else "rotate-half"},
           "dominant_kernel": dom, "roofline": rf,
           "whole_step_mfma_frac": round(flops / (ms * 1e-3) / 1e12 / PEAK_MFMA_TFLOPS, 4),
           "algorithmic_tflop_per_step": round(flops / 1e12, 3)}
    out.update({k: round(v, 4) for k, v in stats.items()})
    if not big:
        # the same call with every cache level cold: a 512 MB buffer (twice the 256 MB
        # last-level cache) is written before each call, outside the timed events
        med, mn = timer.run_cold(step, 10 * steps, 512 << 20)
        out["cold_cache_ms_median"] = round(med, 4)
        out["cold_cache_ms_min"] = round(mn, 4)
    if kernels:
        out["kernels"] = kernels
    del w, k, vt, x, xo, ws
    torch.cuda.empty_cache()
    return out


# ------------------------------------------------------------------------- CPU baseline

def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for ln in f:
                if ln.startswith("model name"):
                    return ln.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def cpu_baseline(n_tokens):
    """The oracle (as it stands) on a bounded sample of the prefill workload: the first
    n_tokens of sequence 0, all 28 layers, final norm and tied LM head on every row, with one
    thread per host core this process may run on."""
    import numpy as np
    import oracle
    import synth
    from synth import recipes
    threads = len(os.sched_getaffinity(0))
    oracle.set_threads(threads)
    cfg = dict(recipes.QWEN3_0P6B)
    model = recipes.model_host(recipes.MODEL_SEED_0P6B, cfg)
    ids = synth.uniform_i32(2, "input.ids", (4, 2048), 0, cfg["vocab_size"])[0, :n_tokens]
    t0 = time.time()
    oracle.stack_prefill(cfg, model, np.ascontiguousarray(ids))
    dt = time.time() - t0
    return {"value": round(n_tokens / dt, 3), "unit": "tokens/s", "cores": oracle.get_threads(),
            "kind": "oracle", "cpu_model": cpu_model(),
            "omp_num_threads": os.environ.get("OMP_NUM_THREADS"),
            "sample": f"sequence 0, first {n_tokens} tokens of the 4x2048 prefill workload; 28 "
                      f"layers + final norm + tied LM head on all {n_tokens} rows; fp64 C++ "
                      f"oracle, {dt:.1f}s wall"}


def cpu_workload_samples(wls):
    """The oracle (as it stands) beside the other workloads, each on a bounded sample of the
    same inputs, in that workload's own tokens/s: the whole 128-token 0.6B block, one
    sequence of the decode step (its 28 layers' caches regenerated, 4096 positions), 256 of
    the 8192 MoE tokens, and the first 512 rows of the 7B block."""
    import numpy as np
    import oracle
    import synth
    from synth import recipes
    oracle.set_threads(len(os.sched_getaffinity(0)))
    f64 = lambda u: synth.bf16_to_f32(u).astype(np.float64)
    out = {}

    def rec(w, n, dt, sample):
        out[w] = {"value": round(n / dt, 3), "unit": "tokens/s", "cores": oracle.get_threads(),
                  "kind": "oracle", "sample": f"{sample}; fp64 C++ oracle, {dt:.2f}s wall"}

    act = recipes.activations_name()
    if "block" in wls:
        cfg = dict(recipes.QWEN3_0P6B)
        layer = recipes.layer_host(1, cfg, 0)
        x = synth.normal_bf16(1, act, (1, 128, cfg["hidden_size"]))
        t0 = time.time()
        oracle.block(cfg, layer, f64(x[0]))
        rec("block", 128, time.time() - t0, "the whole workload (1 x 128 tokens, one block)")
    if "decode" in wls:
        cfg = dict(recipes.QWEN3_0P6B)
        L, ctx = cfg["num_hidden_layers"], 4096
        host = recipes.model_host(recipes.MODEL_SEED_0P6B, cfg)
        ids = synth.uniform_i32(3, "input.ids", (64, 1), 0, cfg["vocab_size"])
        ck, cv = zip(*[recipes.kv_host(3, cfg, l, 0, ctx, (cfg["num_key_value_heads"], ctx))
                       for l in range(L)])
        t0 = time.time()
        oracle.stack_decode(cfg, host, ids[0], ctx, list(ck), list(cv))
        rec("decode", 1, time.time() - t0,
            "sequence 0 of 64: one new token at position 4096, 28 layers + LM head")
        del host, ck, cv
    if "moe" in wls:
        cfg = dict(recipes.MOE_2048)
        router, gu, dn = recipes.moe_host(4, cfg)
        x = synth.normal_bf16(4, act, (8192, cfg["hidden_size"]))[:256]
        t0 = time.time()
        oracle.moe_ffn(cfg, router, gu, dn, f64(x))
        rec("moe", 256, time.time() - t0, "the first 256 of the 8192 tokens")
        del router, gu, dn
    if "block7b" in wls:
        cfg = dict(recipes.QWEN_7B_BLOCK)
        layer = recipes.layer_host(5, cfg, 0)
        x = synth.normal_bf16(5, act, (1, 32768, cfg["hidden_size"]))[0, :512]
        t0 = time.time()
        oracle.block(cfg, layer, f64(x))
        rec("block7b", 512, time.time() - t0, "the first 512 of the 32768 rows (causal prefix)")
    return out


# ------------------------------------------------------------------------- main

def device_info():
    """Compute units and engine clock of GPU agent 0 as rocminfo reports them (run before
    this process touches the GPU)."""
    import subprocess
    info = {}
    try:
        out = subprocess.run(["rocminfo"], capture_output=True, text=True, timeout=60).stdout
    except (OSError, subprocess.SubprocessError):
        return info
    agent = None
    for ln in out.splitlines():
        t = ln.strip()
        if t.startswith("Name:") and "gfx" in t:
            agent = t.split(":", 1)[1].strip()
            info["agent"] = agent
        elif agent and t.startswith("Max Clock Freq. (MHz):") and "max_clock_mhz" not in info:
            info["max_clock_mhz"] = int(t.split(":", 1)[1].split()[0])
        elif agent and t.startswith("Compute Unit:") and "compute_units" not in info:
            info["compute_units"] = int(t.split(":", 1)[1].split()[0])
        if len(info) == 3:
            break
    return info


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workloads",
                    default="prefill,decode,decode_4tok,moe,prefill_2e,block7b,block7b_irope,"
                            "block,generate,generate_sampled")
    ap.add_argument("--no-breakdown", action="store_true")
    ap.add_argument("--cpu-tokens", type=int, default=512,
                    help="prefix length for the oracle CPU baseline (0 = skip)")
    ap.add_argument("--copy-gib", type=float, default=0.0,
                    help="run a plain elementwise copy of this size first (calibrates the "
                         "HBM byte counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py: measures one GPU only (asked for --gpus {args.gpus}); "
              "each GPU would run these kernels on its own sequences", file=sys.stderr)
        sys.exit(2)

    dinfo = device_info()
    import torch
    import decoder_only_forward_amd as q3
    import synth
    from synth import recipes
    dev = torch.device("cuda:0")
    q3.lib()
    timer = Timer(torch, q3)
    if args.copy_gib > 0:
        n = int(args.copy_gib * (1 << 30)) // 4
        a = torch.ones(n, dtype=torch.float32, device=dev)
        b = torch.empty_like(a)
        torch.neg(a, out=b)  # elementwise: reads and writes copy_gib each
        torch.cuda.synchronize()
        del a, b
    wls = [w.strip() for w in args.workloads.split(",") if w.strip()]
    bd = not args.no_breakdown
    results = {}
    fns = {"prefill": lambda: wl_prefill(torch, q3, recipes, synth, dev, args.steps, args.warmup,
                                         timer, bd),
           "prefill_2e": lambda: wl_prefill(torch, q3, recipes, synth, dev, args.steps,
                                            args.warmup, timer, bd, routed=True),
           "decode": lambda: wl_decode(torch, q3, recipes, synth, dev, 2 * args.steps,
                                       args.warmup, timer, bd),
           "decode_4tok": lambda: wl_decode(torch, q3, recipes, synth, dev, 2 * args.steps,
                                            args.warmup, timer, bd, S=4),
           "moe": lambda: wl_moe(torch, q3, recipes, synth, dev, 2 * args.steps, args.warmup,
                                 timer, bd),
           "block7b": lambda: wl_block(torch, q3, recipes, synth, dev, max(2, args.steps // 3),
                                       1, timer, bd, True),
           "block7b_irope": lambda: wl_block(torch, q3, recipes, synth, dev,
                                             max(2, args.steps // 3), 1, timer, bd, True,
                                             rope_interleaved=1),
           "block": lambda: wl_block(torch, q3, recipes, synth, dev, 10 * args.steps,
                                     args.warmup, timer, bd, False),
           "generate": lambda: wl_generate(torch, q3, recipes, synth, dev, 3, 1, timer, False),
           "generate_sampled": lambda: wl_generate(torch, q3, recipes, synth, dev, 3, 1, timer,
                                                   True)}
    for w in wls:
        log(f"workload {w} ...")
        t0 = time.time()
        results[w] = fns[w]()
        log(f"  {w}: {results[w]['tokens_per_s']:.1f} tokens/s, "
            f"{results[w]['ms_per_step']:.3f} ms/step ({time.time() - t0:.1f}s)")

    main_wl = "prefill" if "prefill" in results else wls[0]
    m = results[main_wl]
    line = {"metric": METRIC, "value": round(m["tokens_per_s"], 1), "unit": "tokens/s",
            "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
            "ms_per_step": round(m["ms_per_step"], 4), "higher_is_better": True,
            "scaling": "weak", "vs_baseline": None, "dtype": "f16",
            "data": "synthetic (seeded counter-based generator, random-init weights)",
            "config": m["config"], "roofline": m.get("roofline")}
    for k in ("ms_per_step_median", "ms_per_step_min"):
        if k in m:
            line[k] = round(m[k], 4)
    line["device"] = dict(dinfo, peaks={"mfma_f16_bf16_tflops": PEAK_MFMA_TFLOPS,
                                        "hbm_gbs": PEAK_HBM_GBS})
    if "decode" in results:
        line["decode_tokens_per_s"] = round(results["decode"]["tokens_per_s"], 1)
    if args.cpu_tokens > 0 and main_wl == "prefill":
        log("cpu baseline (oracle) ...")
        line["cpu_baseline"] = cpu_baseline(args.cpu_tokens)
        log("cpu samples of the other workloads (oracle) ...")
        for w, r in cpu_workload_samples(set(results)).items():
            results[w]["cpu_baseline"] = r
    line["workloads"] = {k: {kk: (round(vv, 4) if isinstance(vv, float) else vv)
                             for kk, vv in v.items()} for k, v in results.items()}
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
