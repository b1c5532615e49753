"""GPU parity: generation on the device (prefill, then decode steps that feed each chosen
token back), greedy and sampled, against the oracle."""
import numpy as np
import pytest

import decoder_only_forward_amd as q3
import oracle
import synth
from synth import recipes
from q3_testutil import layer_to_dev, log, new_cache, small_cfg, to_dev_bf16

pytestmark = pytest.mark.gpu


def _setup(gpu, cfg, seed, B, S, cap):
    import torch
    model = recipes.model_host(seed, cfg)
    d = {"embed": to_dev_bf16(model["embed"], gpu), "norm": to_dev_bf16(model["norm"], gpu),
         "layers": [layer_to_dev(l, gpu) for l in model["layers"]]}
    mw, keep = q3.make_model_weights(d["embed"], d["norm"], d["layers"], None)
    rope = torch.empty(2 * cfg["max_position_embeddings"] * 64, dtype=torch.float32, device=gpu)
    q3.qwen3_rope_table_init(cfg, rope)
    ids = synth.uniform_i32(seed, "input.ids", (B, S), 0, cfg["vocab_size"])
    return model, mw, (d, keep, rope), rope, ids


def _caches(cfg, B, cap, gpu):
    L, nkv = cfg["num_hidden_layers"], cfg["num_key_value_heads"]
    bufs = [new_cache(B, nkv, cap, gpu) for _ in range(L)]
    return bufs, [q3.make_kv_layer(k, vt, cap) for k, vt in bufs]


def _generate(gpu, cfg, mw, rope, ids, n_new, cap, temperature=0.0, top_p=1.0, uniforms=None):
    import torch
    B, S = ids.shape
    bufs, kvs = _caches(cfg, B, cap, gpu)
    out = torch.full((B, n_new), -1, dtype=torch.int32, device=gpu)
    ws = torch.empty(q3.qwen3_workspace_bytes(cfg, q3.QWEN3_OP_GENERATE, B, S),
                     dtype=torch.uint8, device=gpu)
    ud = None
    if uniforms is not None:
        ud = torch.from_numpy(np.ascontiguousarray(uniforms, np.float32)).to(gpu)
    q3.qwen3_generate(cfg, mw, rope, torch.from_numpy(ids).to(gpu), B, S, n_new, kvs, out, ws,
                      temperature=temperature, top_p=top_p, uniforms=ud)
    torch.cuda.synchronize()
    return out.cpu().numpy()


def test_generate_greedy_matches_oracle(gpu):
    # Each token must be the oracle's argmax given the GPU's own prefix (full recompute); a
    # different token is accepted only as a near-tie, within twice the logits parity bar.
    cfg = small_cfg(L=2, V=600)
    B, S, n_new, cap = 2, 21, 7, 64
    log(f"case generate greedy: B={B} prompt={S} n_new={n_new}")
    model, mw, keep, rope, ids = _setup(gpu, cfg, 31, B, S, cap)
    got = _generate(gpu, cfg, mw, rope, ids, n_new, cap)
    exact = 0
    for b in range(B):
        seq = list(ids[b])
        for i in range(n_new):
            lg = oracle.stack_prefill(cfg, model, np.array(seq, np.int32), rows=[len(seq) - 1])[0]
            want = int(oracle.argmax(lg)[0])
            g = int(got[b, i])
            assert 0 <= g < cfg["vocab_size"], (b, i, g)
            if g == want:
                exact += 1
            else:
                tol = 4e-2 * np.sqrt(np.mean(lg ** 2))
                assert lg[want] - lg[g] <= tol, (b, i, g, want, lg[want] - lg[g], tol)
            seq.append(g)
    assert exact >= B * n_new - 1, exact
    # with no near-ties the device loop reproduces the oracle's own generation
    if exact == B * n_new:
        for b in range(B):
            np.testing.assert_array_equal(got[b], oracle.generate(cfg, model, ids[b], n_new))


def _check_draw(tok, logits, temperature, top_p, u, where):
    """tok must be the oracle's draw on the same logits, or sit within a rounding distance of
    the drawn boundary (the kernel computes e_v in fp32 and sums them in 2^-44 fixed point)."""
    want, det = oracle.sample(logits, temperature, top_p, [u])
    want = int(want[0])
    if tok == want:
        return True
    d = det[0]
    K, r, cum, e, tau = d["K"], d["r"], d["cum"], d["e"], d["tau"]
    if d["kept"][tok]:
        # r falls on tok's interval of the kept running mass, up to rounding
        eps = 1e-4 * K
        assert cum[tok] - e[tok] - eps <= r <= cum[tok] + eps, (where, tok, want, r, cum[tok])
    else:
        # only a token at the nucleus cut may differ in membership
        assert e[tok] >= tau * (1 - 1e-4), (where, tok, want, e[tok], tau)
    return False


def _replay_draws(gpu, cfg, mw, rope, ids, got, temperature, top_p, uni, cap):
    """Replays the device loop step by step through qwen3_stack_forward (same kernels, same
    order, so the same logits) and checks every draw against the oracle's sampler on those
    logits with the same uniform.  Returns the number of draws equal to the oracle's."""
    import torch
    B, S = ids.shape
    n_new = got.shape[1]
    bufs, kvs = _caches(cfg, B, cap, gpu)
    V = cfg["vocab_size"]
    logits = torch.empty((B, V), dtype=torch.float32, device=gpu)
    ws_p = torch.empty(q3.qwen3_workspace_bytes(cfg, q3.QWEN3_OP_STACK_PREFILL, B, S),
                       dtype=torch.uint8, device=gpu)
    ws_d = torch.empty(q3.qwen3_workspace_bytes(cfg, q3.QWEN3_OP_STACK_DECODE, B, 1),
                       dtype=torch.uint8, device=gpu)
    q3.qwen3_stack_forward(cfg, mw, rope, torch.from_numpy(ids).to(gpu), B, S, 0, None, kvs,
                           logits, q3.QWEN3_LOGITS_LAST, None, ws_p)
    exact = 0
    for i in range(n_new):
        torch.cuda.synchronize()
        lg = logits.cpu().numpy().astype(np.float64)
        for b in range(B):
            exact += _check_draw(int(got[b, i]), lg[b], temperature, top_p, uni[i, b], (i, b))
        if i + 1 < n_new:
            cur = torch.from_numpy(np.ascontiguousarray(got[:, i])).to(gpu)
            pos = torch.full((B,), S + i, dtype=torch.int32, device=gpu)
            q3.qwen3_stack_forward(cfg, mw, rope, cur, B, 1, 0, pos, kvs, logits,
                                   q3.QWEN3_LOGITS_LAST, None, ws_d)
    return exact


def test_generate_sampling_matches_oracle_sampler(gpu):
    # Every draw must be the oracle's draw on the GPU's own logits with the same uniform.
    # The first tokens are also checked against the oracle's own logits through the greedy
    # path's parity, so the two checks together cover the loop.
    cfg = small_cfg(L=2, V=600)
    B, S, n_new, cap = 3, 19, 6, 64
    T, top_p = 0.8, 0.9
    log(f"case generate sampled: B={B} prompt={S} n_new={n_new} T={T} top_p={top_p}")
    model, mw, keep, rope, ids = _setup(gpu, cfg, 32, B, S, cap)
    rng = np.random.default_rng(7)
    uni = rng.random((n_new, B)).astype(np.float32)  # the values the device receives
    got = _generate(gpu, cfg, mw, rope, ids, n_new, cap, T, top_p, uni)
    exact = _replay_draws(gpu, cfg, mw, rope, ids, got, T, top_p, uni, cap)
    assert exact >= B * n_new - 1, exact


@pytest.mark.parametrize("T,top_p", [(0.7, 0.9), (1.0, 1.0), (1.3, 0.5), (0.05, 0.95)])
def test_generate_sampling_full_vocabulary(gpu, T, top_p):
    # The sampler at the full 151,936-token vocabulary: every chunk of every row holds
    # thousands of tokens, and the nucleus cut falls deep inside the radix histograms.
    cfg = small_cfg(L=1, V=151936)
    B, S, n_new, cap = 16, 8, 3, 64
    log(f"case generate sampled full vocabulary: B={B} prompt={S} n_new={n_new} T={T} "
        f"top_p={top_p}")
    model, mw, keep, rope, ids = _setup(gpu, cfg, 34, B, S, cap)
    rng = np.random.default_rng(9)
    uni = rng.random((n_new, B)).astype(np.float32)
    got = _generate(gpu, cfg, mw, rope, ids, n_new, cap, T, top_p, uni)
    exact = _replay_draws(gpu, cfg, mw, rope, ids, got, T, top_p, uni, cap)
    assert exact >= B * n_new - 1, exact



def test_generate_sampling_at_the_vocabulary_limit(gpu):
    # The largest vocabulary the sampler accepts (262,144 tokens: 16,384 per chunk of a row)
    cfg = small_cfg(L=1, V=262144)
    B, S, n_new, cap = 4, 8, 2, 64
    T, top_p = 1.0, 0.9
    log(f"case generate sampled vocabulary limit: V={cfg['vocab_size']} B={B} n_new={n_new}")
    model, mw, keep, rope, ids = _setup(gpu, cfg, 35, B, S, cap)
    rng = np.random.default_rng(10)
    uni = rng.random((n_new, B)).astype(np.float32)
    got = _generate(gpu, cfg, mw, rope, ids, n_new, cap, T, top_p, uni)
    exact = _replay_draws(gpu, cfg, mw, rope, ids, got, T, top_p, uni, cap)
    assert exact >= B * n_new - 1, exact

def test_generate_sampling_limits(gpu):
    # top_p -> 0 keeps only the largest logit: the draw is the greedy token whatever u is
    cfg = small_cfg(L=2, V=600)
    B, S, n_new, cap = 2, 10, 4, 64
    log(f"case generate sampling limit: B={B} prompt={S} n_new={n_new}")
    model, mw, keep, rope, ids = _setup(gpu, cfg, 33, B, S, cap)
    greedy = _generate(gpu, cfg, mw, rope, ids, n_new, cap)
    rng = np.random.default_rng(8)
    tiny = _generate(gpu, cfg, mw, rope, ids, n_new, cap, 1.0, 1e-7, rng.random((n_new, B)))
    np.testing.assert_array_equal(tiny, greedy)
