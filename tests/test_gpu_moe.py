"""GPU parity: routed MoE FFN (router, top-k, dispatch order, grouped SwiGLU experts,
weighted combine) against the oracle.  Integer results (top-k indices, dispatch order)
must be bit-exact when computed from the same router logits."""
import numpy as np
import pytest

import decoder_only_forward_amd as q3
import oracle
import synth
from synth import recipes
from q3_testutil import bf16_host, f64, log, parity, to_dev_bf16

pytestmark = pytest.mark.gpu


def run_moe(cfg, router, gu, dn, x, dev):
    import torch
    T = x.shape[0]
    E, k, H = cfg["num_experts"], cfg["num_experts_per_tok"], cfg["hidden_size"]
    w = q3.make_moe_weights(to_dev_bf16(router, dev), to_dev_bf16(gu, dev), to_dev_bf16(dn, dev))
    keep = [to_dev_bf16(a, dev) for a in (router, gu, dn)]
    w = q3.make_moe_weights(*keep)
    xd = to_dev_bf16(x, dev)
    y = torch.empty_like(xd)
    out = dict(
        logits=torch.empty((T, E), dtype=torch.float32, device=dev),
        idx=torch.empty((T, k), dtype=torch.int32, device=dev),
        w=torch.empty((T, k), dtype=torch.float32, device=dev),
        offsets=torch.empty((E + 1,), dtype=torch.int32, device=dev),
        perm=torch.empty((T * k,), dtype=torch.int32, device=dev),
        inv=torch.empty((T, k), dtype=torch.int32, device=dev))
    ws = torch.empty(q3.qwen3_workspace_bytes(cfg, q3.QWEN3_OP_MOE_FFN, T), dtype=torch.uint8,
                     device=dev)
    q3.qwen3_moe_ffn(cfg, w, xd, y, T, out["logits"], out["idx"], out["w"], out["offsets"],
                     out["perm"], out["inv"], ws)
    torch.cuda.synchronize()
    res = {k_: v.cpu().numpy() for k_, v in out.items()}
    res["y"] = f64(bf16_host(y))
    return res


MOE_CASES = {
    "e16_k4_ragged": (dict(num_experts=16, num_experts_per_tok=4, moe_intermediate_size=128,
                           hidden_size=256), 300, False),
    "e128_k8_sparse": (dict(num_experts=128, num_experts_per_tok=8, moe_intermediate_size=256,
                            hidden_size=512), 200, True),
    "e8_k2_unnormalised": (dict(num_experts=8, num_experts_per_tok=2, moe_intermediate_size=128,
                                hidden_size=256, norm_topk_prob=0), 130, False),
    # bf16 router probabilities ([P1] section 11): two experts, top-1, unrenormalised
    "e2_k1_bf16_router": (dict(num_experts=2, num_experts_per_tok=1, moe_intermediate_size=192,
                               hidden_size=256, norm_topk_prob=0, router_weights_bf16=1), 150,
                          False),
    "e8_k2_bf16_router_norm": (dict(num_experts=8, num_experts_per_tok=2,
                                    moe_intermediate_size=128, hidden_size=256,
                                    router_weights_bf16=1), 170, False),
    # degenerate loads: one expert takes every token (three 256-row tiles, a ragged last
    # one) and the other fifteen none; with k = 2 the hot expert is every token's first
    "e16_k1_one_expert": (dict(num_experts=16, num_experts_per_tok=1, moe_intermediate_size=128,
                               hidden_size=256), 700, "hot"),
    "e8_k2_hot_expert": (dict(num_experts=8, num_experts_per_tok=2, moe_intermediate_size=128,
                              hidden_size=256), 300, "hot"),
    # the limits: 256 experts at top-8 (most experts get a few tokens or none), and top-k
    # equal to the expert count (every token uses every expert; the weights are the softmax)
    "e256_k8_max": (dict(num_experts=256, num_experts_per_tok=8, moe_intermediate_size=128,
                         hidden_size=256), 400, False),
    "e8_k8_all": (dict(num_experts=8, num_experts_per_tok=8, moe_intermediate_size=128,
                       hidden_size=192), 257, False),
}


def _make_hot(router, x):
    """Expert 0's logit gets +8 on every token (a constant input column of 8 that only its
    router row reads), far above the others' (about N(0, 0.3))."""
    router, x = router.copy(), x.copy()
    router[:, 0] = 0
    router[0, 0] = synth.f32_to_bf16(np.array([1.0], np.float32))[0]
    x[:, 0] = synth.f32_to_bf16(np.array([8.0], np.float32))[0]
    return router, x


def _near_bf16_midpoint(logits):
    """Rows whose fp32 softmax has a value within a few ulp of a bf16 rounding midpoint:
    there the two sides' fp32 exp and sum orders may round to different bf16 values."""
    lg = np.asarray(logits, np.float32)
    e = np.exp(lg - lg.max(axis=1, keepdims=True))
    p = (e / e.sum(axis=1, keepdims=True)).astype(np.float32)
    low = p.view(np.uint32) & 0xFFFF
    return np.any(np.abs(low.astype(np.int64) - 0x8000) <= 64, axis=1)


@pytest.mark.parametrize("name", list(MOE_CASES))
def test_moe_parity(gpu, name):
    kw, T, skew = MOE_CASES[name]
    cfg = dict(norm_topk_prob=1, rms_norm_eps=1e-6)
    cfg.update(kw)
    log(f"case moe/{name}: T={T} {kw}")
    _moe_case(gpu, cfg, T, skew)


def _moe_case(gpu, cfg, T, skew, seed=31):
    router, gu, dn = recipes.moe_host(seed, cfg, skew=skew is True)
    x = synth.normal_bf16(seed, recipes.activations_name(), (T, cfg["hidden_size"]))
    if skew == "hot":
        router, x = _make_hot(router, x)
    g = run_moe(cfg, router, gu, dn, x, gpu)
    if skew == "hot":
        assert np.all(g["idx"][:, 0] == 0) and g["offsets"][1] == T, g["offsets"]
    y_ref, idx_ref, w_ref, lg_ref = oracle.moe_ffn(cfg, router, gu, dn, f64(x))
    parity(g["logits"], lg_ref, "router_logits")
    k, E = cfg["num_experts_per_tok"], cfg["num_experts"]
    # integer work on the GPU's own logits: bit-exact
    if cfg.get("router_weights_bf16"):
        # selection and weights from the same logits; rows at a bf16 rounding midpoint of
        # the fp32 probabilities may round either way on the two sides
        idx_same, w_same = oracle.route_bf16(g["logits"], k, cfg["norm_topk_prob"])
        edge = _near_bf16_midpoint(g["logits"])
        log(f"  rows at a bf16 midpoint: {edge.sum()}/{T}")
        assert edge.mean() < 0.05
        np.testing.assert_array_equal(g["idx"][~edge], idx_same[~edge])
        np.testing.assert_allclose(g["w"][~edge], w_same[~edge], rtol=1e-6, atol=0)
    else:
        np.testing.assert_array_equal(g["idx"], oracle.topk(g["logits"], k))
        w_same = oracle.route_weights(g["logits"].astype(np.float64), g["idx"],
                                      cfg["norm_topk_prob"])
        np.testing.assert_allclose(g["w"], w_same, rtol=2e-6, atol=1e-7)
    counts, offsets, perm, inv = oracle.permute(g["idx"], E)
    np.testing.assert_array_equal(g["offsets"], offsets)
    np.testing.assert_array_equal(g["perm"], perm)
    np.testing.assert_array_equal(g["inv"], inv)
    # outputs of every token against the oracle evaluated at the GPU's own selection,
    # weighted as the oracle routes (fp64 softmax, or its bf16 rule) over that selection;
    # where the selections agree this is the oracle's own output
    agree = np.all(np.sort(g["idx"], axis=1) == np.sort(idx_ref, axis=1), axis=1)
    log(f"  routing equals the oracle's own on {agree.sum()}/{T} tokens")
    assert agree.mean() > 0.9
    if cfg.get("router_weights_bf16"):
        # the bf16 rule's weights at the GPU's selection: the rounded probabilities of the
        # chosen experts (all E of them from the rule with k = E), renormalised over the
        # chosen ones with norm_topk_prob
        idx_all, w_all = oracle.route_bf16(lg_ref, E, 0)
        p_bf = np.empty_like(lg_ref)
        np.put_along_axis(p_bf, idx_all.astype(np.int64), w_all, axis=1)
        w_at = np.take_along_axis(p_bf, g["idx"].astype(np.int64), axis=1)
        if cfg["norm_topk_prob"]:
            w_at = w_at / w_at.sum(axis=1, keepdims=True)
    else:
        w_at = oracle.route_weights(lg_ref, g["idx"], cfg["norm_topk_prob"])
    y_at = oracle.moe_ffn_at(cfg, gu, dn, f64(x), g["idx"], w_at)
    np.testing.assert_allclose(y_at[agree], y_ref[agree], rtol=0, atol=1e-12)
    parity(g["y"], y_at, "y (all tokens, at the GPU's selection)", stored_bf16=True)



# A seeded sweep over small valid routed layers beyond the hand-picked cases: 2-64 experts,
# top-1 to top-8, hidden and expert sizes at multiples of 64, 1-600 tokens (expert tiles
# from empty to several, ragged), renormalised or not.  The list is fixed by its seed.
def _moe_sweep(n=12, seed=2026):
    rng = np.random.default_rng(seed)
    out = []
    for _ in range(n):
        E = int(rng.integers(2, 65))
        kw = dict(num_experts=E, num_experts_per_tok=int(rng.integers(1, min(8, E) + 1)),
                  hidden_size=64 * int(rng.integers(1, 9)),
                  moe_intermediate_size=64 * int(rng.integers(1, 7)),
                  norm_topk_prob=int(rng.integers(0, 2)))
        out.append((kw, int(rng.integers(1, 601))))
    return out


MOE_SWEEP = _moe_sweep()


@pytest.mark.parametrize("i", range(len(MOE_SWEEP)))
def test_moe_shape_sweep(gpu, i):
    kw, T = MOE_SWEEP[i]
    cfg = dict(rms_norm_eps=1e-6)
    cfg.update(kw)
    log(f"case moe/sweep{i}: T={T} {kw}")
    _moe_case(gpu, cfg, T, False, seed=300 + i)

def test_moe_deterministic(gpu):
    kw, T, _ = MOE_CASES["e16_k4_ragged"]
    cfg = dict(norm_topk_prob=1, rms_norm_eps=1e-6, **kw)
    router, gu, dn = recipes.moe_host(32, cfg, skew=False)
    x = synth.normal_bf16(32, recipes.activations_name(), (T, cfg["hidden_size"]))
    a = run_moe(cfg, router, gu, dn, x, gpu)
    b = run_moe(cfg, router, gu, dn, x, gpu)
    for key in a:
        np.testing.assert_array_equal(a[key], b[key])
