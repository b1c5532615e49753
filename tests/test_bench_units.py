"""Host checks of bench.py's algorithmic work counts, the numerators of every roofline
fraction it reports, against counts made here independently (brute force over small shapes,
parameter counts from the config) and against the page facts in
tests/golden/qwen3_0p6b_page_facts.json: the 0.6B parameter count ("测试与实测数字") and
the 4 KB of K/V per token and layer ("GQA 注意力")."""
import json
import os

import bench
from synth import recipes

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _cfg():
    return dict(recipes.QWEN3_0P6B)


def _layer_params(c):
    H, nq, nkv, hd, I = (c["hidden_size"], c["num_attention_heads"], c["num_key_value_heads"],
                         c["head_dim"], c["intermediate_size"])
    q, k, v, o = H * nq * hd, H * nkv * hd, H * nkv * hd, nq * hd * H
    mlp = 3 * H * I
    norms = 2 * H + 2 * hd  # input / post-attention RMSNorm, q / k RMSNorm
    return q + k + v + o + mlp + norms


def _tied_params(c):
    return c["num_hidden_layers"] * _layer_params(c) + c["vocab_size"] * c["hidden_size"] + \
        c["hidden_size"]


def test_parameter_count_matches_the_page():
    with open(os.path.join(GOLDEN, "qwen3_0p6b_page_facts.json")) as f:
        facts = json.load(f)
    c = _cfg()
    tied = _tied_params(c)
    untied = tied + c["vocab_size"] * c["hidden_size"]
    assert round(untied / 1e9, 3) == facts["params_untied_billion_rounded_3dp"]
    assert abs((untied - tied) - facts["untied_minus_tied_approx"]) < 0.05e8
    assert tied == 596_049_920


def test_decode_weight_bytes_are_the_tied_parameters_in_bf16():
    # with no sequences the step reads only the weights: every layer, the tied head (the
    # final norm's H values are not counted)
    c = _cfg()
    assert bench.decode_step_bytes(c, 0, 4096) == 2.0 * (_tied_params(c) - c["hidden_size"])


def test_decode_kv_bytes_per_token_and_layer_match_the_page():
    with open(os.path.join(GOLDEN, "qwen3_0p6b_page_facts.json")) as f:
        facts = json.load(f)
    c = _cfg()
    L = c["num_hidden_layers"]
    per_pos = bench.decode_step_bytes(c, 1, 4097) - bench.decode_step_bytes(c, 1, 4096)
    assert per_pos == L * 4096  # K and V of one position, all layers, read once
    assert per_pos / L / 1024 == facts["kv_cache_bytes_per_token_per_layer_approx_kb"]
    assert round(per_pos / 1024) == facts["kv_cache_bytes_per_token_all_layers_approx_kb"]


def test_prefill_gemm_flops_are_two_per_multiply_add():
    c = _cfg()
    B, S = 4, 2048
    T = B * S
    u = bench.dense_units(c, B, S, 1)
    assert u["gate_up_gemm"][1] == 2 * T * 1024 * 2 * 3072 == 103_079_215_104
    assert u["qkv_gemm"][1] == 2 * T * 1024 * (16 + 2 * 8) * 128
    assert u["o_proj_gemm"][1] == 2 * T * 16 * 128 * 1024
    assert u["down_gemm"][1] == 2 * T * 3072 * 1024
    assert all(kind == "mfma" for kind, _, _ in u.values())  # tiled: no separate q/k pass


def test_attention_flops_count_causal_pairs_only():
    c = _cfg()
    for B, S in [(1, 1), (2, 5), (3, 17), (1, 128)]:
        pairs = sum(1 for _b in range(B) for i in range(S) for j in range(S) if j <= i)
        # q.k and p.v: two multiply-adds per head dim per (query, key) pair and q head
        want = 2 * 2 * c["head_dim"] * c["num_attention_heads"] * pairs
        assert bench.dense_units(c, B, S, 1)["attn_prefill"][1] == want


def test_stack_prefill_flops_add_up_the_layers_and_the_head():
    c = _cfg()
    B, S = 4, 2048
    u = bench.dense_units(c, B, S, 1)
    per_layer = sum(u[k][1] for k in ("qkv_gemm", "attn_prefill", "o_proj_gemm",
                                      "gate_up_gemm", "down_gemm"))
    head = 2.0 * B * S * c["hidden_size"] * c["vocab_size"]
    total = bench.stack_prefill_flops(c, B, S)
    assert total == c["num_hidden_layers"] * per_layer + head
    assert round(total / 1e12, 2) == 11.69


def test_moe_units():
    c = dict(recipes.MOE_2048)
    T = 8192
    H, E, k, I = (c["hidden_size"], c["num_experts"], c["num_experts_per_tok"],
                  c["moe_intermediate_size"])
    u = bench.moe_units(c, T, 1)
    assert u["moe_router_gemm"][1] == 2 * T * H * E
    assert u["moe_gate_up_gemm"][1] == 2 * T * k * H * 2 * I
    assert u["moe_down_gemm"][1] == 2 * T * k * I * H
    # the combine reads k fp32 slot rows and writes one bf16 row per token
    assert u["moe_combine"][1] == T * (k * H * 4 + H * 2)
