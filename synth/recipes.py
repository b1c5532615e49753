"""Synthetic workload recipes: shapes, tensor names, distributions and seeds.

Five workloads (all seeded; every tensor is drawn by the counter-based generator
from (seed, HF-style tensor name, element index)):

  1 block_0p6b   one Qwen3-0.6B-shaped block, prefill batch 1 x 128 tokens
  2 stack_0p6b   28-layer 0.6B-shaped stack + final norm + tied LM head,
                 prefill batch 4 x 2048, logits for every position
  3 decode_0p6b  one decode step of the same stack, batch 64, KV cache holding
                 positions 0..4095 (values ~N(0,1)), new token at position 4096
  4 moe_2048     routed MoE FFN: hidden 2048, 128 experts (SwiGLU, I=768),
                 top-8 with renormalised weights, 8192 tokens, Zipf-skewed load
  5 block_7b     one 7B-shaped block (hidden 3584, 28 q / 4 kv heads, I=18944),
                 prefill batch 1 x 32768
  and the two-expert stack: workload 2 with every layer's MLP replaced by a
                 top-1 pair of routed experts (I=3072 each, bf16 gating)

Distributions: linear weights ~N(0, 0.02) (routers of routed layers too); every RMSNorm weight (input, post,
final, q_norm, k_norm) ~1 + N(0, 0.05); activations ~N(0, 1); token ids
uniform in [0, vocab).  "N" is the generator's Irwin-Hall(12) normal.
"""
import json
import os

import numpy as np

from . import normal_bf16, uniform_i32

QWEN3_0P6B = dict(
    hidden_size=1024, num_attention_heads=16, num_key_value_heads=8, head_dim=128,
    intermediate_size=3072, num_hidden_layers=28, vocab_size=151936,
    max_position_embeddings=40960, rms_norm_eps=1e-6, rope_theta=1e6, qk_norm=1,
    tie_word_embeddings=1)

QWEN_7B_BLOCK = dict(
    hidden_size=3584, num_attention_heads=28, num_key_value_heads=4, head_dim=128,
    intermediate_size=18944, num_hidden_layers=1, vocab_size=152064,
    max_position_embeddings=40960, rms_norm_eps=1e-6, rope_theta=1e6, qk_norm=1,
    tie_word_embeddings=0)

MOE_2048 = dict(
    hidden_size=2048, num_experts=128, num_experts_per_tok=8, moe_intermediate_size=768,
    norm_topk_prob=1, rms_norm_eps=1e-6)

# Two-expert routed variant of the 0.6B model ([P1]: every layer's MLP replaced by two
# experts, top-1, weight = the bf16-rounded router probability, no renormalisation; the
# experts keep the dense MLP's shape)
MOE_2E = dict(num_experts=2, num_experts_per_tok=1, moe_intermediate_size=3072,
              norm_topk_prob=0, decoder_sparse_step=1, router_weights_bf16=1)

WORKLOADS = {
    1: dict(name="block_0p6b", cfg=QWEN3_0P6B, batch=1, seq_len=128, layers=1),
    2: dict(name="stack_0p6b_prefill", cfg=QWEN3_0P6B, batch=4, seq_len=2048, layers=28),
    3: dict(name="stack_0p6b_decode", cfg=QWEN3_0P6B, batch=64, seq_len=1, context=4096,
            layers=28),
    4: dict(name="moe_ffn_2048x128e_top8", cfg=MOE_2048, tokens=8192),
    5: dict(name="block_7b", cfg=QWEN_7B_BLOCK, batch=1, seq_len=32768, layers=1),
}

# The 28-layer stack's weights are one model shared by workloads 2 and 3.
MODEL_SEED_0P6B = 2

W_STD = 0.02
NORM_MEAN, NORM_STD = 1.0, 0.05

LAYER_FIELDS = ("in_norm", "q", "k", "v", "q_norm", "k_norm", "o", "post_norm", "gate", "up",
                "down")


def layer_specs(cfg, l):
    """(field, HF tensor name, shape, mean, std) for decoder layer ``l``."""
    H, nq, nkv, hd, I = (cfg["hidden_size"], cfg["num_attention_heads"],
                         cfg["num_key_value_heads"], cfg["head_dim"], cfg["intermediate_size"])
    p = f"model.layers.{l}."
    return [
        ("in_norm", p + "input_layernorm.weight", (H,), NORM_MEAN, NORM_STD),
        ("q", p + "self_attn.q_proj.weight", (nq * hd, H), 0.0, W_STD),
        ("k", p + "self_attn.k_proj.weight", (nkv * hd, H), 0.0, W_STD),
        ("v", p + "self_attn.v_proj.weight", (nkv * hd, H), 0.0, W_STD),
        ("q_norm", p + "self_attn.q_norm.weight", (hd,), NORM_MEAN, NORM_STD),
        ("k_norm", p + "self_attn.k_norm.weight", (hd,), NORM_MEAN, NORM_STD),
        ("o", p + "self_attn.o_proj.weight", (H, nq * hd), 0.0, W_STD),
        ("post_norm", p + "post_attention_layernorm.weight", (H,), NORM_MEAN, NORM_STD),
        ("gate", p + "mlp.gate_proj.weight", (I, H), 0.0, W_STD),
        ("up", p + "mlp.up_proj.weight", (I, H), 0.0, W_STD),
        ("down", p + "mlp.down_proj.weight", (H, I), 0.0, W_STD),
    ]


def model_specs(cfg):
    V, H = cfg["vocab_size"], cfg["hidden_size"]
    out = [("embed", "model.embed_tokens.weight", (V, H), 0.0, W_STD),
           ("norm", "model.norm.weight", (H,), NORM_MEAN, NORM_STD)]
    if not cfg.get("tie_word_embeddings", 1):
        out.append(("lm_head", "lm_head.weight", (V, H), 0.0, W_STD))
    return out


def has_experts(cfg, l):
    """Whether layer l's MLP is a routed expert set (the Hugging Face Qwen3-MoE layout:
    every decoder_sparse_step-th layer when num_experts > 0); such a layer has no dense
    gate/up/down projections."""
    step = cfg.get("decoder_sparse_step", 0)
    return cfg.get("num_experts", 0) > 0 and step > 0 and (l + 1) % step == 0


def layer_host(seed, cfg, l):
    routed = has_experts(cfg, l)
    d = {f: normal_bf16(seed, n, s, m, sd) for f, n, s, m, sd in layer_specs(cfg, l)
         if not (routed and f in ("gate", "up", "down"))}
    if routed:
        d["router"], d["experts_gate_up"], d["experts_down"] = moe_host(seed, cfg, l=l)
    return d


def model_host(seed, cfg, n_layers=None):
    n_layers = cfg["num_hidden_layers"] if n_layers is None else n_layers
    d = {f: normal_bf16(seed, n, s, m, sd) for f, n, s, m, sd in model_specs(cfg)}
    d.setdefault("lm_head", None)
    d["layers"] = [layer_host(seed, cfg, l) for l in range(n_layers)]
    return d


def activations_name():
    return "input.hidden_states"


def x_host(seed, shape):
    return normal_bf16(seed, activations_name(), shape, 0.0, 1.0)


def ids_host(seed, shape, vocab):
    return uniform_i32(seed, "input.ids", shape, 0, vocab)


def kv_names(l):
    return f"kv.{l}.k", f"kv.{l}.v"


def kv_host(seed, cfg, l, b, n_pos, batch_nkv_ctx):
    """Cache contents of sequence ``b`` for layer ``l`` as logical [nkv, n_pos, hd] (bf16
    bits).  Logical tensor is [batch, nkv, ctx, hd]; ``batch_nkv_ctx`` = (nkv, ctx)."""
    nkv, ctx = batch_nkv_ctx
    hd = cfg["head_dim"]
    kn, vn = kv_names(l)
    k = np.empty((nkv, n_pos, hd), np.uint16)
    v = np.empty((nkv, n_pos, hd), np.uint16)
    from . import normal_bf16_strided_host
    for h in range(nkv):
        off = ((b * nkv + h) * ctx) * hd
        normal_bf16_strided_host(seed, kn, k[h], (1, n_pos, hd), (0, hd, 1), 0.0, 1.0, off)
        normal_bf16_strided_host(seed, vn, v[h], (1, n_pos, hd), (0, hd, 1), 0.0, 1.0, off)
    return k, v


# ---- routed MoE (workload 4) ----------------------------------------------------------

SKEW_FILE = os.path.join(os.path.dirname(os.path.abspath(__file__)), "router_skew_e128_k8.json")


def router_row_scales(n_experts=128):
    """Per-expert router row scale g_e (geometric mean 1) giving a Zipf(1.1)-shaped load,
    from the committed calibration table; all ones when the table does not match."""
    if os.path.exists(SKEW_FILE):
        with open(SKEW_FILE) as f:
            t = json.load(f)
        if len(t["scale"]) == n_experts:
            return np.asarray(t["scale"], dtype=np.float64)
    return np.ones(n_experts)


def moe_specs(cfg, l=0):
    H, E, I = cfg["hidden_size"], cfg["num_experts"], cfg["moe_intermediate_size"]
    p = f"model.layers.{l}.mlp."
    return [("router", p + "gate.weight", (E, H)),
            ("gate_up", p + "experts.gate_up_proj", (E, 2 * I, H)),
            ("down", p + "experts.down_proj", (E, H, I))]


def moe_host(seed, cfg, skew=True, l=0):
    H, E = cfg["hidden_size"], cfg["num_experts"]
    specs = dict((f, (n, s)) for f, n, s in moe_specs(cfg, l))
    g = router_row_scales(E) if skew else np.ones(E)
    n, _ = specs["router"]
    router = np.empty((E, H), np.uint16)
    from . import normal_bf16_strided_host
    for e in range(E):
        normal_bf16_strided_host(seed, n, router[e], (1, 1, H), (0, 0, 1), 0.0,
                                 float(np.float32(W_STD * g[e])), e * H)
    gu = normal_bf16(seed, specs["gate_up"][0], specs["gate_up"][1], 0.0, W_STD)
    dn = normal_bf16(seed, specs["down"][0], specs["down"][1], 0.0, W_STD)
    return router, gu, dn


def param_count(cfg, tied=True):
    """Parameter count implied by the shapes (weights of every layer + embedding + norm
    (+ untied LM head))."""
    H, nq, nkv, hd, I, L, V = (cfg["hidden_size"], cfg["num_attention_heads"],
                               cfg["num_key_value_heads"], cfg["head_dim"],
                               cfg["intermediate_size"], cfg["num_hidden_layers"],
                               cfg["vocab_size"])
    per_layer = (H + nq * hd * H + 2 * nkv * hd * H + 2 * hd + H * nq * hd + H + 3 * I * H)
    total = L * per_layer + V * H + H
    if not tied:
        total += V * H
    return total


# ---- device-side generation (same values as the host recipes, written in HBM) ----------

LIB_LAYER_NAMES = {"in_norm": "input_layernorm", "q": "q_proj", "k": "k_proj", "v": "v_proj",
                   "q_norm": "q_norm", "k_norm": "k_norm", "o": "o_proj",
                   "post_norm": "post_attention_layernorm", "gate": "gate_proj",
                   "up": "up_proj", "down": "down_proj"}


def _dev_normal(shape, seed, name, mean, std, device):
    import torch
    from . import normal_bf16_device
    t = torch.empty(shape, dtype=torch.bfloat16, device=device)
    normal_bf16_device(t, seed, name, mean, std)
    return t


def layer_device(seed, cfg, l, device):
    """One layer's weights on the device, keyed by the library's field names."""
    routed = has_experts(cfg, l)
    d = {LIB_LAYER_NAMES[f]: _dev_normal(s, seed, n, m, sd, device)
         for f, n, s, m, sd in layer_specs(cfg, l)
         if not (routed and f in ("gate", "up", "down"))}
    if routed:
        d["router"], d["experts_gate_up_proj"], d["experts_down_proj"] = \
            moe_device(seed, cfg, device, l=l)
    return d


def model_device(seed, cfg, device, n_layers=None):
    n_layers = cfg["num_hidden_layers"] if n_layers is None else n_layers
    d = {f: _dev_normal(s, seed, n, m, sd, device) for f, n, s, m, sd in model_specs(cfg)}
    d.setdefault("lm_head", None)
    d["layers"] = [layer_device(seed, cfg, l, device) for l in range(n_layers)]
    return d


def kv_fill_device(k_log, v_log, seed, l, n_pos, ctx):
    """Fill positions [0, n_pos) of every (sequence, kv head) of one layer's logical K and V
    tensors, both [B, nkv, cap, hd], with the logical tensor [B, nkv, ctx, hd] named
    kv.{l}.k / kv.{l}.v."""
    from . import normal_bf16_device
    B, nkv, cap, hd = k_log.shape
    kn, vn = kv_names(l)
    if n_pos == ctx:
        for t, name in ((k_log, kn), (v_log, vn)):
            normal_bf16_device(t, seed, name, 0.0, 1.0, logical=(B * nkv, n_pos, hd),
                               strides=(cap * hd, hd, 1))
        return
    for i in range(B * nkv):
        b, h = divmod(i, nkv)
        for t, name in ((k_log, kn), (v_log, vn)):
            normal_bf16_device(t[b, h], seed, name, 0.0, 1.0, offset=i * ctx * hd,
                               logical=(1, n_pos, hd), strides=(0, hd, 1))


def moe_device(seed, cfg, device, skew=True, l=0):
    import torch
    from . import normal_bf16_device
    H, E = cfg["hidden_size"], cfg["num_experts"]
    specs = dict((f, (n, s)) for f, n, s in moe_specs(cfg, l))
    g = router_row_scales(E) if skew else np.ones(E)
    n, _ = specs["router"]
    router = torch.empty((E, H), dtype=torch.bfloat16, device=device)
    for e in range(E):
        normal_bf16_device(router[e], seed, n, 0.0, float(np.float32(W_STD * g[e])),
                           offset=e * H, logical=(1, 1, H), strides=(0, 0, 1))
    gu = _dev_normal(specs["gate_up"][1], seed, specs["gate_up"][0], 0.0, W_STD, device)
    dn = _dev_normal(specs["down"][1], seed, specs["down"][0], 0.0, W_STD, device)
    return router, gu, dn
