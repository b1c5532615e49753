"""GPU parity: stacks whose layers include routed MoE FFNs (every decoder_sparse_step-th
layer, [P3] "MoE" and the Qwen3-MoE layer layout; the bf16-probability gating of [P1]
section 11), prefill and decode, against the oracle.

Routing is an integer decision taken from floating-point router logits, and the two sides'
logits differ by rounding.  A token whose routing the oracle finds within the logits parity
bar of a different selection may be routed differently on the GPU; it is left out of the
comparison together with what depends on it (the later positions of its sequence, unless the
layer is the last one).  Every other logits row must meet the parity bar, and most rows are
compared."""
import itertools

import numpy as np
import pytest

import decoder_only_forward_amd as q3
import oracle
import synth
from synth import recipes
from q3_testutil import layer_to_dev, log, new_cache, parity, small_cfg, \
    to_dev_bf16

pytestmark = pytest.mark.gpu

# routers drawn with a larger spread than the dense weights, so that most decisions are
# clear (router logits' standard deviation about ROUTER_STD * sqrt(hidden))
ROUTER_STD = 0.1
# bound on the GPU's router-logit error, relative to the logits' rms: fp16 activations and
# fp32 accumulation put it near 1e-3 (the mean-relative parity bar is 5e-3)
ROUTER_TOL = 5e-3

KINDS = {
    # top-2 of 4 with renormalised softmax weights; only the last of two layers is routed
    "e4_k2_step2": dict(num_experts=4, num_experts_per_tok=2, moe_intermediate_size=128,
                        norm_topk_prob=1, decoder_sparse_step=2, router_weights_bf16=0),
    # [P1] section 11: two experts, top-1, bf16 probabilities as weights, every layer routed
    "e2_k1_bf16_step1": dict(num_experts=2, num_experts_per_tok=1, moe_intermediate_size=192,
                             norm_topk_prob=0, decoder_sparse_step=1, router_weights_bf16=1),
    # top-4 of 16, every layer routed
    "e16_k4_step1": dict(num_experts=16, num_experts_per_tok=4, moe_intermediate_size=64,
                         norm_topk_prob=1, decoder_sparse_step=1, router_weights_bf16=0),
}


def _cfg(kind):
    cfg = small_cfg(L=2, V=600)
    cfg.update(KINDS[kind])
    return cfg


def _model(seed, cfg):
    model = recipes.model_host(seed, cfg)
    H, E = cfg["hidden_size"], cfg["num_experts"]
    n_routed = 0
    for l, lw in enumerate(model["layers"]):
        if "router" in lw:
            lw["router"] = synth.normal_bf16(seed, f"test.router.{l}", (E, H), 0.0, ROUTER_STD)
            n_routed += 1
    assert n_routed == sum(recipes.has_experts(cfg, l) for l in range(len(model["layers"])))
    return model


def _model_dev(model, dev):
    d = {"embed": to_dev_bf16(model["embed"], dev), "norm": to_dev_bf16(model["norm"], dev),
         "layers": [layer_to_dev(l, dev) for l in model["layers"]]}
    mw, keep = q3.make_model_weights(d["embed"], d["norm"], d["layers"], None)
    return mw, (d, keep)


def _rope(cfg, dev):
    import torch
    rope = torch.empty(2 * cfg["max_position_embeddings"] * 64, dtype=torch.float32, device=dev)
    q3.qwen3_rope_table_init(cfg, rope)
    return rope


def _unstable(cfg, lg, delta):
    """lg [S, E]: one routed layer's oracle router logits.  True where some perturbation of
    the logits by at most delta each could change the selected expert set."""
    k = cfg["num_experts_per_tok"]
    E = lg.shape[1]
    if not cfg.get("router_weights_bf16"):
        if k == E:
            return np.zeros(lg.shape[0], bool)
        s = -np.sort(-lg, axis=1)
        return (s[:, k - 1] - s[:, k]) <= 2 * delta
    # bf16 probabilities: the selection is a step function of the logits; try every corner
    # of the perturbation box (for two experts the selection depends on l1 - l0 alone and is
    # monotone in it, so the corners decide)
    assert E <= 4
    base = np.sort(oracle.route_bf16(lg, k)[0], axis=1)
    out = np.zeros(lg.shape[0], bool)
    for signs in itertools.product((-1.0, 0.0, 1.0), repeat=E):
        idx = np.sort(oracle.route_bf16(lg + delta * np.array(signs), k)[0], axis=1)
        out |= np.any(idx != base, axis=1)
    return out


def _comparable(cfg, rl):
    """rl [L, S, E] oracle router logits (NaN in dense layers) -> bool [S]: rows whose
    logits cannot depend on a routing decision taken within the parity bar of a tie."""
    L, S, _ = rl.shape
    ok = np.ones(S, bool)
    for l in range(L):
        if np.isnan(rl[l]).all():
            continue
        delta = ROUTER_TOL * float(np.sqrt(np.mean(rl[l] ** 2)))
        u = _unstable(cfg, rl[l], delta)
        if not u.any():
            continue
        if l == L - 1:
            ok &= ~u  # the FFN is per token: only that row depends on it
        else:
            ok[int(np.argmax(u)):] = False  # later layers attend to it
    return ok


@pytest.mark.parametrize("kind", list(KINDS))
def test_routed_stack_prefill_then_decode(gpu, kind):
    import torch
    cfg = _cfg(kind)
    L, V = cfg["num_hidden_layers"], cfg["vocab_size"]
    B, S, cap = 3, 29, 64
    log(f"case routed stack/{kind}: B={B} S={S} L={L}")
    model = _model(41, cfg)
    mw, keep = _model_dev(model, gpu)
    rope = _rope(cfg, gpu)
    ids = synth.uniform_i32(41, "input.ids", (B, S + 1), 0, V)
    caches = [new_cache(B, cfg["num_key_value_heads"], cap, gpu) for _ in range(L)]
    kvs = [q3.make_kv_layer(k, vt, cap) for k, vt in caches]
    logits = torch.empty((B, S, V), dtype=torch.float32, device=gpu)
    ws = torch.empty(q3.qwen3_workspace_bytes(cfg, q3.QWEN3_OP_STACK_PREFILL, B, S),
                     dtype=torch.uint8, device=gpu)
    q3.qwen3_stack_forward(cfg, mw, rope, torch.from_numpy(np.ascontiguousarray(ids[:, :S]))
                           .to(gpu), B, S, 0, None, kvs, logits, q3.QWEN3_LOGITS_ALL, None, ws)
    dec = torch.empty((B, V), dtype=torch.float32, device=gpu)
    wsd = torch.empty(q3.qwen3_workspace_bytes(cfg, q3.QWEN3_OP_STACK_DECODE, B),
                      dtype=torch.uint8, device=gpu)
    pos = torch.full((B,), S, dtype=torch.int32, device=gpu)
    last = torch.from_numpy(np.ascontiguousarray(ids[:, S])).to(gpu)
    q3.qwen3_stack_forward(cfg, mw, rope, last, B, 1, 0, pos, kvs, dec, q3.QWEN3_LOGITS_LAST,
                           None, wsd)
    torch.cuda.synchronize()
    got, got_dec = logits.cpu().numpy(), dec.cpu().numpy()
    compared = 0
    for b in range(B):
        ref, rl = oracle.stack_prefill(cfg, model, ids[b], want_router=True)
        ok = _comparable(cfg, rl)
        log(f"  b={b}: {ok.sum()}/{S + 1} rows clear of routing near-ties")
        if ok[:S].any():
            parity(got[b][ok[:S]], ref[:S][ok[:S]], f"prefill logits[b={b}]")
        if ok[S]:
            parity(got_dec[b], ref[S], f"decode logits[b={b}]")
        compared += int(ok.sum())
    assert compared >= 0.6 * B * (S + 1), compared


def test_routed_stack_without_sparse_step_is_dense(gpu):
    # num_experts > 0 with decoder_sparse_step = 0 routes no layer: the stack reads the
    # dense projections and gives the dense stack's logits bit for bit
    import torch
    dense = small_cfg(L=2, V=500)
    cfg = dict(dense, num_experts=4, num_experts_per_tok=2, moe_intermediate_size=128,
               norm_topk_prob=1, decoder_sparse_step=0)
    B, S, cap = 2, 17, 64
    log(f"case routed stack/no sparse step: B={B} S={S}")
    model = recipes.model_host(42, dense)
    mw, keep = _model_dev(model, gpu)
    rope = _rope(dense, gpu)
    ids = torch.from_numpy(synth.uniform_i32(42, "input.ids", (B, S), 0, 500)).to(gpu)
    outs = []
    for c in (dense, cfg):
        kvs_b = [new_cache(B, 2, cap, gpu) for _ in range(2)]
        lg = torch.empty((B, S, 500), dtype=torch.float32, device=gpu)
        ws = torch.empty(q3.qwen3_workspace_bytes(c, q3.QWEN3_OP_STACK_PREFILL, B, S),
                         dtype=torch.uint8, device=gpu)
        q3.qwen3_stack_forward(c, mw, rope, ids, B, S, 0, None,
                               [q3.make_kv_layer(k, vt, cap) for k, vt in kvs_b], lg,
                               q3.QWEN3_LOGITS_ALL, None, ws)
        torch.cuda.synchronize()
        outs.append(lg.cpu().numpy())
    np.testing.assert_array_equal(outs[0], outs[1])


def test_routed_stack_multi_token_decode_and_generation(gpu):
    # routed layers under the other entry points: a prefill of S tokens, then 4 new tokens
    # per sequence decoded together at position S (compared with the oracle's prefill over
    # the S + 4 tokens, rows clear of routing near-ties), and greedy generation whose first
    # token is the argmax of the prefill's last row
    import torch
    cfg = _cfg("e2_k1_bf16_step1")
    L, V = cfg["num_hidden_layers"], cfg["vocab_size"]
    B, S, n, cap = 2, 21, 4, 64
    log(f"case routed stack/multi-token decode + generation: B={B} S={S} n={n}")
    model = _model(43, cfg)
    mw, keep = _model_dev(model, gpu)
    rope = _rope(cfg, gpu)
    ids = synth.uniform_i32(43, "input.ids", (B, S + n), 0, V)
    caches = [new_cache(B, cfg["num_key_value_heads"], cap, gpu) for _ in range(L)]
    kvs = [q3.make_kv_layer(k, vt, cap) for k, vt in caches]
    ws = torch.empty(q3.qwen3_workspace_bytes(cfg, q3.QWEN3_OP_STACK_PREFILL, B, S),
                     dtype=torch.uint8, device=gpu)
    last = torch.empty((B, V), dtype=torch.float32, device=gpu)
    q3.qwen3_stack_forward(cfg, mw, rope, torch.from_numpy(np.ascontiguousarray(ids[:, :S]))
                           .to(gpu), B, S, 0, None, kvs, last, q3.QWEN3_LOGITS_LAST, None, ws)
    dec = torch.empty((B * n, V), dtype=torch.float32, device=gpu)
    wsd = torch.empty(q3.qwen3_workspace_bytes(cfg, q3.QWEN3_OP_STACK_DECODE, B, n),
                      dtype=torch.uint8, device=gpu)
    pos = torch.full((B,), S, dtype=torch.int32, device=gpu)
    q3.qwen3_stack_forward(cfg, mw, rope, torch.from_numpy(np.ascontiguousarray(ids[:, S:]))
                           .to(gpu), B, n, 0, pos, kvs, dec, q3.QWEN3_LOGITS_ALL, None, wsd)
    torch.cuda.synchronize()
    got_last, got_dec = last.cpu().numpy(), dec.cpu().numpy().reshape(B, n, V)
    first = []
    for b in range(B):
        ref, rl = oracle.stack_prefill(cfg, model, ids[b], want_router=True)
        ok = _comparable(cfg, rl)
        log(f"  b={b}: {ok.sum()}/{S + n} rows clear of routing near-ties")
        assert ok.sum() >= (S + n) // 2
        if ok[S - 1]:
            parity(got_last[b], ref[S - 1], f"prefill last row[b={b}]")
        if ok[S:].any():
            parity(got_dec[b][ok[S:]], ref[S:][ok[S:]], f"multi-token decode[b={b}]")
        first.append(int(oracle.argmax(got_last[b])[0]))
    # generation: token 0 is the argmax of the prefill's last row (same kernels, same logits)
    caches2 = [new_cache(B, cfg["num_key_value_heads"], cap, gpu) for _ in range(L)]
    out = torch.full((B, 3), -1, dtype=torch.int32, device=gpu)
    wsg = torch.empty(q3.qwen3_workspace_bytes(cfg, q3.QWEN3_OP_GENERATE, B, S),
                      dtype=torch.uint8, device=gpu)
    q3.qwen3_generate(cfg, mw, rope, torch.from_numpy(np.ascontiguousarray(ids[:, :S])).to(gpu),
                      B, S, 3, [q3.make_kv_layer(k, vt, cap) for k, vt in caches2], out, wsg)
    torch.cuda.synchronize()
    gen = out.cpu().numpy()
    np.testing.assert_array_equal(gen[:, 0], first)
    assert ((gen >= 0) & (gen < V)).all()
