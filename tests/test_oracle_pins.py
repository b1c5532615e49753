"""Pins for the CPU oracle: closed forms, invariants, special cases and page-printed values
that fix what each oracle function computes, independently of the oracle's own code.

Sources are the web pages on hand-building Qwen3 named in oracle/qwen3_oracle.h.
"""
import json
import math
import os

import numpy as np
import pytest

import oracle
import synth
from synth import recipes

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
rng = np.random.default_rng(1234)


def bf16(x):
    return synth.f32_to_bf16(np.asarray(x, np.float32))


def bf16_exact(x):
    """Values that are exactly representable in bf16, as (bits, float64)."""
    b = bf16(x)
    return b, synth.bf16_to_f32(b).astype(np.float64)


# ---------------------------------------------------------------- RMSNorm (rmsnorm_rows)

def test_rmsnorm_closed_form_constant_weight():
    # With w = c the output RMS is c * sqrt(ms / (ms + eps)).
    c = 1.5
    w = bf16(np.full(1024, c))
    for scale in (1.0, 1e-3, 37.0):
        x = rng.standard_normal((5, 1024)) * scale
        y = oracle.rmsnorm_rows(x, w, 1e-6)
        ms = (x * x).mean(axis=1)
        want = c * np.sqrt(ms / (ms + 1e-6))
        got = np.sqrt((y * y).mean(axis=1))
        np.testing.assert_allclose(got, want, rtol=1e-12)


def test_rmsnorm_eps_inside_root():
    # ms == eps makes the output RMS exactly c * sqrt(1/2): pins eps under the root.
    w = bf16(np.ones(64))
    x = np.full((1, 64), 1e-3)  # ms = 1e-6
    y = oracle.rmsnorm_rows(x, w, 1e-6)
    np.testing.assert_allclose(np.sqrt((y * y).mean()), math.sqrt(0.5), rtol=1e-12)


def test_rmsnorm_elementwise_weight_and_zero_input():
    wb, wf = bf16_exact(rng.standard_normal(256) * 0.05 + 1.0)
    x = rng.standard_normal((3, 256))
    y1 = oracle.rmsnorm_rows(x, bf16(np.ones(256)), 1e-6)
    yw = oracle.rmsnorm_rows(x, wb, 1e-6)
    np.testing.assert_allclose(yw, y1 * wf, rtol=1e-13)
    z = oracle.rmsnorm_rows(np.zeros((2, 256)), wb, 1e-6)
    assert np.all(z == 0.0)


def test_rmsnorm_worked_example():
    # x = (3, 4), unit weights, eps = 0: mean square 12.5, output (3, 4)/sqrt(12.5).
    y = oracle.rmsnorm_rows(np.array([[3.0, 4.0]]), bf16([1.0, 1.0]), 0.0)
    np.testing.assert_allclose(y[0], [0.848528137423857, 1.131370849898476], rtol=1e-13)


# ---------------------------------------------------------------- RoPE

def test_rope_identity_at_position_zero():
    x = rng.standard_normal((4, 128))
    np.testing.assert_array_equal(oracle.rope(x, 0, 1e6), x)


def test_rope_rotates_planes_i_and_i_plus_half():
    # A unit vector on dim i moves only within the plane (i, i + 64), by the angle
    # pos * theta_i with theta_i = base^(-2i/128): this pins the rotate-half pairing
    # and the frequency ladder of the pages' RoPE section.
    hd, base, pos = 128, 1e6, 7
    for i in (0, 1, 31, 63):
        e = np.zeros((1, hd))
        e[0, i] = 1.0
        y = oracle.rope(e, pos, base)[0]
        ang = pos * base ** (-2.0 * i / hd)
        want = np.zeros(hd)
        want[i] = math.cos(ang)
        want[i + hd // 2] = math.sin(ang)
        np.testing.assert_allclose(y, want, atol=1e-15)
        e2 = np.zeros((1, hd))
        e2[0, i + hd // 2] = 1.0
        y2 = oracle.rope(e2, pos, base)[0]
        want2 = np.zeros(hd)
        want2[i] = -math.sin(ang)
        want2[i + hd // 2] = math.cos(ang)
        np.testing.assert_allclose(y2, want2, atol=1e-15)


def test_rope_preserves_plane_norms_and_composes():
    x = rng.standard_normal((6, 128))
    y = oracle.rope(x, 1234, 1e6)
    n0 = x[:, :64] ** 2 + x[:, 64:] ** 2
    n1 = y[:, :64] ** 2 + y[:, 64:] ** 2
    np.testing.assert_allclose(n1, n0, rtol=1e-12)
    # R_a R_b = R_{a+b}
    np.testing.assert_allclose(oracle.rope(oracle.rope(x, 300, 1e6), 45, 1e6),
                               oracle.rope(x, 345, 1e6), atol=1e-11)


def test_rope_dot_product_depends_on_relative_position_only():
    q = rng.standard_normal((1, 128))
    k = rng.standard_normal((1, 128))
    d1 = (oracle.rope(q, 10, 1e6) @ oracle.rope(k, 3, 1e6).T).item()
    d2 = (oracle.rope(q, 1010, 1e6) @ oracle.rope(k, 1003, 1e6).T).item()
    d3 = (q @ oracle.rope(k, -7, 1e6).T).item()
    assert abs(d1 - d2) < 1e-10 and abs(d1 - d3) < 1e-10


def test_rope_interleaved_rotates_adjacent_planes():
    # Interleaved pairing (the complex-number form): a unit vector on dim 2i moves only
    # within the plane (2i, 2i + 1), by pos * theta_i with the same frequency ladder.
    hd, base, pos = 128, 1e6, 11
    for i in (0, 1, 31, 63):
        ang = pos * base ** (-2.0 * i / hd)
        e = np.zeros((1, hd))
        e[0, 2 * i] = 1.0
        want = np.zeros(hd)
        want[2 * i], want[2 * i + 1] = math.cos(ang), math.sin(ang)
        np.testing.assert_allclose(oracle.rope(e, pos, base, interleaved=True)[0], want,
                                   atol=1e-15)
        e2 = np.zeros((1, hd))
        e2[0, 2 * i + 1] = 1.0
        want2 = np.zeros(hd)
        want2[2 * i], want2[2 * i + 1] = -math.sin(ang), math.cos(ang)
        np.testing.assert_allclose(oracle.rope(e2, pos, base, interleaved=True)[0], want2,
                                   atol=1e-15)


def test_rope_interleaved_is_rotate_half_under_a_dim_permutation():
    # Moving dims (2i, 2i + 1) to (i, i + 64) turns one pairing into the other, so both
    # compute the same rotation of the same planes; identity at 0, composition and the
    # relative-position property carry over.
    hd = 128
    perm = np.empty(hd, dtype=np.int64)  # perm[rotate-half index] = interleaved index
    perm[:64] = np.arange(0, hd, 2)
    perm[64:] = np.arange(1, hd, 2)
    x = rng.standard_normal((5, hd))
    for pos in (0, 1, 777, 40000):
        yi = oracle.rope(x, pos, 1e6, interleaved=True)
        yh = oracle.rope(x[:, perm], pos, 1e6)
        np.testing.assert_allclose(yi[:, perm], yh, atol=1e-13)
    np.testing.assert_array_equal(oracle.rope(x, 0, 1e6, interleaved=True), x)
    q, k = rng.standard_normal((1, hd)), rng.standard_normal((1, hd))
    d1 = (oracle.rope(q, 10, 1e6, True) @ oracle.rope(k, 3, 1e6, True).T).item()
    d2 = (oracle.rope(q, 2010, 1e6, True) @ oracle.rope(k, 2003, 1e6, True).T).item()
    assert abs(d1 - d2) < 1e-10


# ---------------------------------------------------------------- attention

def _onehot_values(L, nkv, hd):
    # v_j = e_j on every kv head: the attention output row equals the weight row P[i, :].
    v = np.zeros((L, nkv, hd))
    for j in range(L):
        v[j, :, j] = 1.0
    return v


def test_attention_mask_matches_printed_17x17_pattern():
    with open(os.path.join(GOLDEN, "causal_mask_17.txt")) as f:
        rows = [ln.split() for ln in f if ln.strip() and not ln.startswith("#")]
    masked = np.array([[t == "-inf" for t in r] for r in rows])
    assert masked.shape == (17, 17)
    S, nq, nkv, hd = 17, 4, 2, 32
    q = rng.standard_normal((S, nq, hd))
    k = rng.standard_normal((S, nkv, hd))
    o = oracle.attention(q, k, _onehot_values(S, nkv, hd), np.arange(S))
    P = o[:, :, :S]  # [query, head, key]
    for h in range(nq):
        assert np.all(P[:, h][masked] == 0.0)
        assert np.all(P[:, h][~masked] > 0.0)
        np.testing.assert_allclose(P[:, h].sum(axis=1), 1.0, rtol=1e-13)


def test_attention_first_row_is_v0_and_equal_keys_average():
    S, nq, nkv, hd = 9, 2, 1, 16
    q = rng.standard_normal((S, nq, hd))
    v = rng.standard_normal((S, nkv, hd))
    k = np.repeat(rng.standard_normal((1, nkv, hd)), S, axis=0)
    o = oracle.attention(q, k, v, np.arange(S))
    np.testing.assert_allclose(o[0, 0], v[0, 0], rtol=1e-14)
    for i in range(S):
        np.testing.assert_allclose(o[i, 1], v[: i + 1, 0].mean(axis=0), atol=1e-13)


def test_attention_brute_force_with_explicit_mask_and_repeated_kv():
    # The pages' construction: repeat each kv head over its group of consecutive q
    # heads, scores / sqrt(hd) plus an additive -inf mask, softmax, times V.
    for S, nq, nkv, hd, L0 in ((12, 4, 2, 8, 0), (5, 6, 3, 8, 7), (16, 4, 4, 8, 3)):
        L = L0 + S
        q = rng.standard_normal((S, nq, hd))
        k = rng.standard_normal((L, nkv, hd))
        v = rng.standard_normal((L, nkv, hd))
        qpos = L0 + np.arange(S)
        got = oracle.attention(q, k, v, qpos)
        g = nq // nkv
        kr = np.repeat(k, g, axis=1)
        vr = np.repeat(v, g, axis=1)
        mask = np.where(np.arange(L)[None, :] > qpos[:, None], -np.inf, 0.0)
        want = np.empty_like(q)
        for h in range(nq):
            sc = q[:, h] @ kr[:, h].T / math.sqrt(hd) + mask
            p = np.exp(sc - sc.max(axis=1, keepdims=True))
            p /= p.sum(axis=1, keepdims=True)
            want[:, h] = p @ vr[:, h]
        np.testing.assert_allclose(got, want, atol=1e-12)


def test_gqa_equals_mha_with_copied_kv_heads():
    S, nq, nkv, hd = 10, 8, 2, 16
    q = rng.standard_normal((S, nq, hd))
    k = rng.standard_normal((S, nkv, hd))
    v = rng.standard_normal((S, nkv, hd))
    gqa = oracle.attention(q, k, v, np.arange(S))
    mha = oracle.attention(q, np.repeat(k, nq // nkv, axis=1), np.repeat(v, nq // nkv, axis=1),
                           np.arange(S))
    np.testing.assert_allclose(gqa, mha, rtol=1e-14)
    # head h uses kv head h // g: heads 0..3 must ignore kv head 1 entirely
    v2 = v.copy()
    v2[:, 1] += 100.0
    o2 = oracle.attention(q, k, v2, np.arange(S))
    np.testing.assert_array_equal(o2[:, :4], gqa[:, :4])
    assert not np.allclose(o2[:, 4:], gqa[:, 4:])


# ---------------------------------------------------------------- SwiGLU

def test_swiglu_worked_example():
    # H = 2, I = 1: gate picks x0, up picks x1, down writes only output 0:
    # y0 = silu(x0) * x1 with silu(ln 3) = 0.75 ln 3.
    gate, up = bf16([[1.0, 0.0]]), bf16([[0.0, 1.0]])
    down = bf16([[1.0], [0.0]])
    x = np.array([[math.log(3.0), 2.0]])
    y = oracle.swiglu_ffn(x, gate, up, down)
    np.testing.assert_allclose(y[0], [0.75 * math.log(3.0) * 2.0, 0.0], rtol=1e-14)


def test_swiglu_zero_gate_and_large_gate_limit():
    H, I = 64, 96
    x = rng.standard_normal((3, H))
    up, down = bf16(rng.standard_normal((I, H)) * 0.1), bf16(rng.standard_normal((H, I)) * 0.1)
    y = oracle.swiglu_ffn(x, bf16(np.zeros((I, H))), up, down)
    assert np.all(y == 0.0)
    # silu(z) -> z for large positive z: gate = up (scaled by 1e3 -> identical sign).
    wu = rng.standard_normal((I, H)) * 0.1
    xpos = np.abs(rng.standard_normal((1, H)))
    wpos = np.abs(wu)
    yb = oracle.swiglu_ffn(xpos * 1e3, bf16(wpos), bf16(wpos), down)
    z = (xpos * 1e3) @ synth.bf16_to_f32(bf16(wpos)).astype(np.float64).T
    want = (z * z) @ synth.bf16_to_f32(down).astype(np.float64).T
    np.testing.assert_allclose(yb, want, rtol=1e-12)


# ---------------------------------------------------------------- block (composition)

def _small_cfg(nq=4, nkv=2, H=64, hd=16, I=96, qk_norm=1):
    return dict(hidden_size=H, num_attention_heads=nq, num_key_value_heads=nkv, head_dim=hd,
                intermediate_size=I, num_hidden_layers=2, vocab_size=300,
                max_position_embeddings=4096, rms_norm_eps=1e-6, rope_theta=1e6,
                qk_norm=qk_norm, tie_word_embeddings=1)


def _layer(cfg, l, seed=9):
    return recipes.layer_host(seed, cfg, l)


def _f(u):
    return synth.bf16_to_f32(u).astype(np.float64)


def _block_by_composition(cfg, w, x, pos0, pk, pv):
    """The pre-norm block wired from separately pinned primitives (numpy matmuls for
    the bias-free projections)."""
    H, nq, nkv, hd = (cfg["hidden_size"], cfg["num_attention_heads"],
                      cfg["num_key_value_heads"], cfg["head_dim"])
    eps, th = cfg["rms_norm_eps"], cfg["rope_theta"]
    S = x.shape[0]
    n = oracle.rmsnorm_rows(x, w["in_norm"], eps)
    q = (n @ _f(w["q"]).T).reshape(S, nq, hd)
    k = (n @ _f(w["k"]).T).reshape(S, nkv, hd)
    v = (n @ _f(w["v"]).T).reshape(S, nkv, hd)
    if cfg["qk_norm"]:
        q = oracle.rmsnorm_rows(q, w["q_norm"], eps)
        k = oracle.rmsnorm_rows(k, w["k_norm"], eps)
    pos = pos0 + np.arange(S)
    q = oracle.rope(q, np.repeat(pos, nq), th)
    k = oracle.rope(k, np.repeat(pos, nkv), th)
    K = np.concatenate([pk.transpose(1, 0, 2), k], axis=0) if pos0 else k
    V = np.concatenate([pv.transpose(1, 0, 2), v], axis=0) if pos0 else v
    o = oracle.attention(q, K, V, pos)
    h1 = x + o.reshape(S, nq * hd) @ _f(w["o"]).T
    n2 = oracle.rmsnorm_rows(h1, w["post_norm"], eps)
    h2 = h1 + oracle.swiglu_ffn(n2, w["gate"], w["up"], w["down"])
    return h2, k.transpose(1, 0, 2), v.transpose(1, 0, 2)


@pytest.mark.parametrize("qk_norm", [1, 0])
def test_block_matches_composition_of_pinned_parts(qk_norm):
    cfg = _small_cfg(qk_norm=qk_norm)
    w = _layer(cfg, 0)
    x = rng.standard_normal((11, cfg["hidden_size"]))
    got, gk, gv = oracle.block(cfg, w, x)
    want, wk, wv = _block_by_composition(cfg, w, x, 0, None, None)
    np.testing.assert_allclose(got, want, atol=1e-11)
    np.testing.assert_allclose(gk, wk, atol=1e-12)
    np.testing.assert_allclose(gv, wv, atol=1e-12)


def test_block_chunked_prefill_and_decode_equal_one_prefill():
    cfg = _small_cfg()
    w = _layer(cfg, 1)
    x = rng.standard_normal((13, cfg["hidden_size"]))
    full, fk, fv = oracle.block(cfg, w, x)
    a, ak, av = oracle.block(cfg, w, x[:8])
    b, bk, bv = oracle.block(cfg, w, x[8:], pos0=8, past_k=ak, past_v=av)
    np.testing.assert_allclose(np.concatenate([a, b]), full, atol=1e-12)
    np.testing.assert_allclose(np.concatenate([ak, bk], axis=1), fk, atol=1e-13)
    # decode: token 12 alone against the cache of 0..11 equals row 12 of the prefill
    c, _, _ = oracle.block(cfg, w, x[12:], pos0=12, past_k=fk[:, :12], past_v=fv[:, :12])
    np.testing.assert_allclose(c[0], full[12], atol=1e-12)
    # row subset equals the same rows of the full call
    r, _, _ = oracle.block(cfg, w, x, rows=[0, 5, 12])
    np.testing.assert_allclose(r, full[[0, 5, 12]], atol=1e-13)


def test_block_single_token_reduces_to_value_path():
    # At one token attention returns v exactly, so q/k do not matter: replacing the
    # q/k weights must not change the output, and the result is x + o_proj(v) + ffn.
    cfg = _small_cfg()
    w = _layer(cfg, 0)
    x = rng.standard_normal((1, cfg["hidden_size"]))
    y1, _, _ = oracle.block(cfg, w, x)
    w2 = dict(w)
    w2["q"] = bf16(rng.standard_normal(w["q"].shape))
    w2["k"] = bf16(rng.standard_normal(w["k"].shape))
    y2, _, _ = oracle.block(cfg, w2, x)
    np.testing.assert_allclose(y1, y2, rtol=1e-14)


# ---------------------------------------------------------------- stack

def test_stack_equals_blocks_then_norm_then_tied_head():
    cfg = _small_cfg()
    model = recipes.model_host(5, cfg)
    ids = np.array([3, 17, 299, 0, 42, 42, 7], np.int32)
    lg = oracle.stack_prefill(cfg, model, ids)
    x = _f(model["embed"])[ids]
    for l in range(cfg["num_hidden_layers"]):
        x, _, _ = oracle.block(cfg, model["layers"][l], x)
    hf = oracle.rmsnorm_rows(x, model["norm"], cfg["rms_norm_eps"])
    np.testing.assert_allclose(lg, hf @ _f(model["embed"]).T, atol=1e-11)
    r = oracle.stack_prefill(cfg, model, ids, rows=[6])
    np.testing.assert_allclose(r[0], lg[6], atol=1e-12)


def test_stack_decode_equals_last_prefill_row():
    cfg = _small_cfg()
    model = recipes.model_host(6, cfg)
    ids = np.array([5, 9, 250, 1, 77, 13], np.int32)
    lg, ko, vo = oracle.stack_prefill(cfg, model, ids, want_kv=True)
    p = 5
    dec = oracle.stack_decode(cfg, model, ids[p], p, [k[:, :p] for k in ko],
                              [v[:, :p] for v in vo])
    np.testing.assert_allclose(dec, lg[p], atol=1e-11)


def test_multi_token_decode_equals_prefill_rows():
    # n new tokens decoded onto the cache of the first p positions give the full prefill's
    # rows p .. p + n - 1; and one step at a time (the cache grown by each step's own K/V)
    # gives the same rows
    cfg = _small_cfg()
    model = recipes.model_host(7, cfg)
    ids = np.array([5, 9, 250, 1, 77, 13, 40, 2, 211], np.int32)
    lg, ko, vo = oracle.stack_prefill(cfg, model, ids, want_kv=True)
    p, n = 4, 5
    dec = oracle.stack_decode(cfg, model, ids[p:p + n], p, [k[:, :p] for k in ko],
                              [v[:, :p] for v in vo])
    assert dec.shape == (n, cfg["vocab_size"])
    np.testing.assert_allclose(dec, lg[p:p + n], atol=1e-11)
    for i in range(n):
        one = oracle.stack_decode(cfg, model, ids[p + i], p + i, [k[:, :p + i] for k in ko],
                                  [v[:, :p + i] for v in vo])
        np.testing.assert_allclose(one, dec[i], atol=1e-11)
    # a later token changes nothing before it (causal), but does change its own row
    ids2 = ids.copy()
    ids2[p + n - 1] = 123
    dec2 = oracle.stack_decode(cfg, model, ids2[p:p + n], p, [k[:, :p] for k in ko],
                               [v[:, :p] for v in vo])
    np.testing.assert_array_equal(dec2[:n - 1], dec[:n - 1])
    assert np.abs(dec2[n - 1] - dec[n - 1]).max() > 1e-3


def test_config_shapes_match_page_facts():
    with open(os.path.join(GOLDEN, "qwen3_0p6b_page_facts.json")) as f:
        facts = json.load(f)
    cfg = recipes.QWEN3_0P6B
    for k, v in facts["config"].items():
        assert cfg[k] == v, k
    untied = recipes.param_count(cfg, tied=False)
    tied = recipes.param_count(cfg, tied=True)
    assert round(untied / 1e9, 3) == facts["params_untied_billion_rounded_3dp"]
    assert abs((untied - tied) - facts["untied_minus_tied_approx"]) < 0.05e8
    assert round(untied * 4 / 1e9, 2) == facts["fp32_weight_gb_untied_2dp"]
    kv = 2 * cfg["num_key_value_heads"] * cfg["head_dim"] * 2
    assert kv == facts["kv_cache_bytes_per_token_per_layer_approx_kb"] * 1024
    assert kv * cfg["num_hidden_layers"] == facts[
        "kv_cache_bytes_per_token_all_layers_approx_kb"] * 1024


# ---------------------------------------------------------------- MoE

def _moe_cfg(E=8, k=2, H=32, I=24, norm=1):
    return dict(hidden_size=H, num_experts=E, num_experts_per_tok=k, moe_intermediate_size=I,
                norm_topk_prob=norm, rms_norm_eps=1e-6)


def _moe_weights(cfg, seed=3):
    return recipes.moe_host(seed, cfg, skew=False)


def test_moe_weights_sum_to_one_and_topk_is_sorted_prefix():
    cfg = _moe_cfg(E=16, k=4)
    r, gu, dn = _moe_weights(cfg)
    x = rng.standard_normal((40, cfg["hidden_size"]))
    y, idx, w, lg = oracle.moe_ffn(cfg, r, gu, dn, x)
    np.testing.assert_allclose(w.sum(axis=1), 1.0, rtol=1e-14)
    order = np.argsort(-lg, axis=1, kind="stable")[:, :4]
    np.testing.assert_array_equal(idx, order)
    np.testing.assert_allclose(lg, x @ _f(r).T, rtol=1e-12)
    np.testing.assert_allclose(oracle.linear_rows(x, r), lg, rtol=1e-13)
    # the weights equal a softmax restricted to the selected logits
    sel = np.take_along_axis(lg, idx, axis=1)
    e = np.exp(sel - sel.max(axis=1, keepdims=True))
    np.testing.assert_allclose(w, e / e.sum(axis=1, keepdims=True), rtol=1e-12)


def test_moe_unnormalised_weights_are_full_softmax_probabilities():
    cfg = _moe_cfg(E=8, k=2, norm=0)
    r, gu, dn = _moe_weights(cfg)
    x = rng.standard_normal((10, cfg["hidden_size"]))
    y, idx, w, lg = oracle.moe_ffn(cfg, r, gu, dn, x)
    p = np.exp(lg - lg.max(axis=1, keepdims=True))
    p /= p.sum(axis=1, keepdims=True)
    np.testing.assert_allclose(w, np.take_along_axis(p, idx, axis=1), rtol=1e-12)
    assert np.all(w.sum(axis=1) < 1.0)


def test_moe_touches_only_selected_experts():
    cfg = _moe_cfg(E=16, k=2)
    r, gu, dn = _moe_weights(cfg)
    x = rng.standard_normal((6, cfg["hidden_size"]))
    y, idx, w, lg = oracle.moe_ffn(cfg, r, gu, dn, x)
    unused = sorted(set(range(16)) - set(idx.ravel().tolist()))
    assert unused
    gu2, dn2 = gu.copy(), dn.copy()
    nan = np.uint16(0x7FC0)
    gu2[unused] = nan
    dn2[unused] = nan
    y2, idx2, _, _ = oracle.moe_ffn(cfg, r, gu2, dn2, x)
    np.testing.assert_array_equal(idx2, idx)
    np.testing.assert_array_equal(y2, y)


def test_moe_identical_experts_equal_dense_swiglu_and_single_expert():
    cfg = _moe_cfg(E=6, k=3)
    H, I = cfg["hidden_size"], cfg["moe_intermediate_size"]
    r, _, _ = _moe_weights(cfg)
    g = bf16(rng.standard_normal((I, H)) * 0.2)
    u = bf16(rng.standard_normal((I, H)) * 0.2)
    d = bf16(rng.standard_normal((H, I)) * 0.2)
    gu = np.stack([np.concatenate([g, u])] * 6)
    dn = np.stack([d] * 6)
    x = rng.standard_normal((9, H))
    y, _, _, _ = oracle.moe_ffn(cfg, r, gu, dn, x)
    np.testing.assert_allclose(y, oracle.swiglu_ffn(x, g, u, d), atol=1e-13)
    one = _moe_cfg(E=1, k=1)
    y1, idx1, w1, _ = oracle.moe_ffn(one, r[:1], gu[:1], dn[:1], x)
    assert np.all(idx1 == 0) and np.all(w1 == 1.0)
    np.testing.assert_allclose(y1, oracle.swiglu_ffn(x, g, u, d), atol=1e-13)


def test_moe_tokenwise_equals_grouped_dispatch():
    cfg = _moe_cfg(E=8, k=3)
    H, I = cfg["hidden_size"], cfg["moe_intermediate_size"]
    r, gu, dn = _moe_weights(cfg)
    x = rng.standard_normal((25, H))
    y, idx, w, _ = oracle.moe_ffn(cfg, r, gu, dn, x)
    counts, offsets, perm, inv = oracle.permute(idx, 8)
    acc = np.zeros_like(x)
    for e in range(8):
        rows = np.arange(offsets[e], offsets[e + 1])
        toks = perm[rows]
        if len(toks) == 0:
            continue
        ye = oracle.swiglu_ffn(x[toks], gu[e][:I], gu[e][I:], dn[e])
        for rr, t in zip(rows, toks):
            j = int(np.nonzero(inv[t] == rr)[0][0])
            acc[t] += w[t, j] * ye[rr - offsets[e]]
    np.testing.assert_allclose(y, acc, atol=1e-13)


def test_permute_matches_stable_sort_by_expert():
    T, k, E = 300, 8, 128
    idx = np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
    counts, offsets, perm, inv = oracle.permute(idx, E)
    order = np.argsort(idx.ravel(), kind="stable")
    np.testing.assert_array_equal(perm, order // k)
    np.testing.assert_array_equal(counts, np.bincount(idx.ravel(), minlength=E))
    np.testing.assert_array_equal(offsets, np.concatenate([[0], np.cumsum(counts)]))
    flat = np.empty(T * k, np.int32)
    flat[order] = np.arange(T * k)
    np.testing.assert_array_equal(inv.ravel(), flat)


def test_topk_ties_go_to_lower_index():
    lg = np.array([[1.0, 3.0, 3.0, 2.0, 3.0, 0.5]], np.float32)
    np.testing.assert_array_equal(oracle.topk(lg, 4), [[1, 2, 4, 3]])


def test_argmax_ties_go_to_lowest_index():
    lg = np.array([[0.0, 5.0, 5.0, -1.0], [7.0, 7.0, 7.0, 7.0]], np.float32)
    np.testing.assert_array_equal(oracle.argmax(lg), [1, 0])
    np.testing.assert_array_equal(oracle.argmax(lg.astype(np.float64)), [1, 0])


# ---------------------------------------------------------------- sampling

def test_sample_inverse_cdf_on_a_worked_distribution():
    # logits 0, ln 2, ln 3, -inf at temperature 1: probabilities 1/6, 2/6, 3/6, 0; the
    # cumulative boundaries in index order are 1, 3, 6 (times 1/6)
    lg = np.array([0.0, math.log(2.0), math.log(3.0), -np.inf])
    cases = {0.0: 0, 0.16: 0, 0.17: 1, 0.49: 1, 0.51: 2, 0.99: 2}
    for u, want in cases.items():
        assert oracle.sample(lg, 1.0, 1.0, [u])[0][0] == want, u


def test_sample_top_p_cut_keeps_ties_and_renormalises():
    lg = np.log(np.array([1.0, 2.0, 3.0]))
    # top_p 0.5: the largest entry (3 of 6) already reaches the target -> only token 2
    for u in (0.0, 0.3, 0.9):
        assert oracle.sample(lg, 1.0, 0.5, [u])[0][0] == 2
    # top_p 0.6: target 3.6 needs 3 + 2 -> kept {1, 2}, mass 5, boundaries 2 and 5
    assert oracle.sample(lg, 1.0, 0.6, [0.39])[0][0] == 1
    assert oracle.sample(lg, 1.0, 0.6, [0.41])[0][0] == 2
    # ties at the cut are all kept: e = 2, 2, 1 with top_p 0.4 keeps tokens 0 and 1
    lt = np.log(np.array([2.0, 2.0, 1.0]))
    toks = [oracle.sample(lt, 1.0, 0.4, [u])[0][0] for u in np.linspace(0, 0.999, 50)]
    assert set(toks) == {0, 1}


def test_sample_frequencies_match_tempered_probabilities():
    # a regular grid of u gives each kept token a share equal to its probability
    lg = rng.standard_normal(40) * 2.0
    T = 0.7
    grid = (np.arange(20000) + 0.5) / 20000
    toks = oracle.sample(np.tile(lg, (len(grid), 1)), T, 1.0, grid)[0]
    p = np.exp((lg - lg.max()) / T)
    p /= p.sum()
    freq = np.bincount(toks, minlength=40) / len(grid)
    np.testing.assert_allclose(freq, p, atol=2.0 / len(grid) + 1e-12)


def test_sample_low_temperature_or_tiny_nucleus_is_greedy():
    lg = rng.standard_normal((5, 64))
    g = oracle.argmax(lg)
    lg[np.arange(5), g] += 1.0  # a clear maximum: at temperature 1e-4 the rest weigh e^-10^4
    for u in (0.0, 0.5, 0.999):
        np.testing.assert_array_equal(oracle.sample(lg, 1.0, 1e-9, [u] * 5)[0], g)
        np.testing.assert_array_equal(oracle.sample(lg, 1e-4, 1.0, [u] * 5)[0], g)


# ---------------------------------------------------------------- routed layers

def test_bf16_round_to_nearest_even():
    u = 2.0 ** -7  # bf16 spacing just above 1
    got = oracle.bf16_round([1.0, 1 + u / 2, 1 + 1.5 * u, 1 + u / 2 + 2.0 ** -20, -3.0, 0.0])
    np.testing.assert_array_equal(got, [1.0, 1.0, 1 + 2 * u, 1 + u, -3.0, 0.0])


def _two_expert_cfg(H=64, I=64, bf16_router=1, norm=0):
    return dict(hidden_size=H, num_experts=2, num_experts_per_tok=1, moe_intermediate_size=I,
                norm_topk_prob=norm, rms_norm_eps=1e-6, router_weights_bf16=bf16_router)


def test_router_bf16_tie_goes_to_the_lower_expert():
    # Router logits (0, d) with d = 0.0016: fp32 softmax gives 0.4996 / 0.5004, both rounding
    # to bf16 0.5.  The page's rule (argmax over the rounded probabilities, first on ties)
    # picks expert 0 with weight 0.5; the fp32 top-k rule picks expert 1 with 0.5004.
    H, I = 64, 64
    d = 0.0016
    x = np.zeros((1, H)); x[0, 0] = 1.0
    router = np.zeros((2, H), np.uint16)
    router[1, 0] = np.float32(d).view(np.uint32) >> 16  # bf16 bits of d (truncated)
    dval = float(np.array([int(router[1, 0]) << 16], np.uint32).view(np.float32)[0])
    gu = synth.normal_bf16(3, "t.gu", (2, 2 * I, H), 0.0, 0.05)
    dn = synth.normal_bf16(3, "t.dn", (2, H, I), 0.0, 0.05)
    y, idx, w, lg = oracle.moe_ffn(_two_expert_cfg(), router, gu, dn, x)
    assert idx[0, 0] == 0 and w[0, 0] == 0.5
    y2, idx2, w2, _ = oracle.moe_ffn(_two_expert_cfg(bf16_router=0), router, gu, dn, x)
    assert idx2[0, 0] == 1
    np.testing.assert_allclose(w2[0, 0], 1.0 / (1.0 + math.exp(-dval)), rtol=1e-12)
    # a clear winner is selected by both rules, the bf16 weight being its rounded probability
    router[1, 0] = np.float32(1.0).view(np.uint32) >> 16
    _, idx3, w3, _ = oracle.moe_ffn(_two_expert_cfg(), router, gu, dn, x)
    p1 = np.float32(1.0) / (np.float32(1.0) + np.exp(np.float32(-1.0)))
    assert idx3[0, 0] == 1 and w3[0, 0] == oracle.bf16_round(p1)[0]


def test_stack_routed_layers_with_one_expert_equal_the_dense_stack():
    # decoder_sparse_step = 1 routes every layer; with a single expert (k = 1, renormalised
    # weight 1) holding the dense FFN's weights, the routed stack is the dense stack.
    from q3_testutil import small_cfg
    cfg = small_cfg(L=2, V=300)
    model = recipes.model_host(5, cfg)
    ids = synth.uniform_i32(5, "input.ids", (9,), 0, 300)
    dense = oracle.stack_prefill(cfg, model, ids)
    rcfg = dict(cfg, num_experts=1, num_experts_per_tok=1,
                moe_intermediate_size=cfg["intermediate_size"], norm_topk_prob=1,
                decoder_sparse_step=1)
    H = cfg["hidden_size"]
    for lw in model["layers"]:
        lw["router"] = synth.normal_bf16(5, "t.router", (1, H), 0.0, 0.02)
        lw["experts_gate_up"] = np.concatenate([lw["gate"], lw["up"]])[None]
        lw["experts_down"] = lw["down"][None]
    routed, rl = oracle.stack_prefill(rcfg, model, ids, want_router=True)
    np.testing.assert_allclose(routed, dense, rtol=0, atol=1e-12)
    assert np.isfinite(rl).all()
    # sparse step 2: only layer 1 is routed
    _, rl2 = oracle.stack_prefill(dict(rcfg, decoder_sparse_step=2), model, ids, want_router=True)
    assert np.isnan(rl2[0]).all() and np.isfinite(rl2[1]).all()


def test_route_bf16_closed_form():
    # logits (0, ln 2, ln 2): probabilities 1/5, 2/5, 2/5; bf16 rounds 2/5 up to
    # 0.400390625 (fp32 0x3ECCCCCD, low half above the midpoint).  Top-1 takes the lower
    # index of the tie with that rounded weight; top-2 renormalised gives 1/2 each.
    lg = np.array([[0.0, math.log(2.0), math.log(2.0)]])
    idx, w = oracle.route_bf16(lg, 1)
    assert idx[0, 0] == 1 and w[0, 0] == 0.400390625
    idx, w = oracle.route_bf16(lg, 2, norm_topk=True)
    np.testing.assert_array_equal(idx[0], [1, 2])
    np.testing.assert_array_equal(w[0], [0.5, 0.5])
    # unrenormalised top-2 of (0, 0, -inf-like): bf16(1/2) each
    idx, w = oracle.route_bf16(np.array([[0.0, 0.0, -100.0]]), 2)
    np.testing.assert_array_equal(idx[0], [0, 1])
    np.testing.assert_array_equal(w[0], [0.5, 0.5])


# ---------------------------------------------------------------- MoE at a given selection

def test_moe_at_selection_equals_moe_ffn_and_single_expert_swiglu():
    # moe_ffn_at with moe_ffn's own selection and weights reproduces moe_ffn's y; one
    # selected expert at weight 1 is that expert's SwiGLU (gate = rows [0, I), up = the rest);
    # the output is linear in the weights (a dropped or doubled slot fails this)
    cfg = _moe_cfg(E=8, k=3)
    H, I = cfg["hidden_size"], cfg["moe_intermediate_size"]
    r, gu, dn = _moe_weights(cfg)
    x = rng.standard_normal((21, H))
    y, idx, w, _ = oracle.moe_ffn(cfg, r, gu, dn, x)
    np.testing.assert_allclose(oracle.moe_ffn_at(cfg, gu, dn, x, idx, w), y, atol=1e-14)
    e = 5
    one = dict(cfg, num_experts_per_tok=1)
    y1 = oracle.moe_ffn_at(one, gu, dn, x, np.full((21, 1), e), np.ones((21, 1)))
    np.testing.assert_allclose(y1, oracle.swiglu_ffn(x, gu[e][:I], gu[e][I:], dn[e]),
                               atol=1e-14)
    # another selection: each slot's expert output scaled by its own weight
    idx2 = np.stack([rng.permutation(8)[:3] for _ in range(21)]).astype(np.int32)
    w2 = rng.random((21, 3))
    want = np.zeros_like(x)
    for j in range(3):
        for t in range(21):
            ee = idx2[t, j]
            want[t] += w2[t, j] * oracle.swiglu_ffn(x[t:t + 1], gu[ee][:I], gu[ee][I:],
                                                     dn[ee])[0]
    np.testing.assert_allclose(oracle.moe_ffn_at(cfg, gu, dn, x, idx2, w2), want, atol=1e-13)


# ---------------------------------------------------------------- untied head, generation

def _untied(model, perm):
    """The same model with an untied head whose row v is embedding row perm[v]."""
    m = dict(model)
    m["lm_head"] = np.ascontiguousarray(model["embed"][perm])
    return m


def test_untied_head_reads_lm_head_rows():
    # lm_head = embedding rows permuted: logits column v must equal the tied model's column
    # perm[v] at every position, in prefill and decode (reading embed instead of lm_head for
    # the head, or lm_head instead of embed for the input lookup, breaks the identity)
    cfg = _small_cfg()
    V = cfg["vocab_size"]
    model = recipes.model_host(8, cfg)
    perm = rng.permutation(V)
    mu = _untied(model, perm)
    cu = dict(cfg, tie_word_embeddings=0)
    ids = np.array([4, 250, 31, 31, 7, 190], np.int32)
    tied, ko, vo = oracle.stack_prefill(cfg, model, ids, want_kv=True)
    unt = oracle.stack_prefill(cu, mu, ids)
    np.testing.assert_allclose(unt, tied[:, perm], rtol=0, atol=1e-13)
    p = 5
    dt = oracle.stack_decode(cfg, model, ids[p], p, [k[:, :p] for k in ko],
                             [v[:, :p] for v in vo])
    du = oracle.stack_decode(cu, mu, ids[p], p, [k[:, :p] for k in ko], [v[:, :p] for v in vo])
    np.testing.assert_allclose(du, dt[perm], rtol=0, atol=1e-13)
    # the permutation is not the identity on the argmax (the check has teeth)
    assert oracle.argmax(unt[-1])[0] != oracle.argmax(tied[-1])[0]


def _zero_layer_model(cfg, V, seed=11):
    """Every projection weight zero (each block is then the identity on the residual); the
    embedding rows are +-1/4 signs, so rmsnorm(E[t]) . E[u] is largest at u = t."""
    H = cfg["hidden_size"]
    g = np.random.default_rng(seed)
    model = recipes.model_host(seed, cfg)
    for lw in model["layers"]:
        for f in ("q", "k", "v", "o", "gate", "up", "down"):
            lw[f] = np.zeros_like(lw[f])
    model["embed"] = bf16(np.where(g.random((V, H)) < 0.5, -0.25, 0.25))
    return model


def test_generate_greedy_follows_the_head_permutation_with_zero_layers():
    # With zero projections every block returns its input, so the last hidden state is the
    # embedding row of the last token; with lm_head row v = E[perm[v]] the greedy next token
    # after t is the v with perm[v] = t.  Generation must therefore walk the inverse
    # permutation's cycle from the prompt's last token: a wrong feed-back (not the previous
    # token, or not at the end of the sequence) leaves that cycle.
    cfg = dict(_small_cfg(), tie_word_embeddings=0)
    V, H = cfg["vocab_size"], cfg["hidden_size"]
    model = _zero_layer_model(cfg, V)
    perm = rng.permutation(V)
    inv = np.argsort(perm)
    model = _untied(model, perm)
    # the next-token map from embed, norm and lm_head alone (numpy), against the closed form
    E = _f(model["embed"])
    wf = _f(model["norm"])
    hn = E / np.sqrt((E * E).mean(axis=1, keepdims=True) + cfg["rms_norm_eps"]) * wf
    nxt = np.argmax(hn @ _f(model["lm_head"]).T, axis=1)
    np.testing.assert_array_equal(nxt, inv)
    prompt = [17, 3, 250, 99]
    got = oracle.generate(cfg, model, prompt, 6)
    want, t = [], prompt[-1]
    for _ in range(6):
        t = int(inv[t])
        want.append(t)
    np.testing.assert_array_equal(got, want)
    assert len(set(want)) > 1
