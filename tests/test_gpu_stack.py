"""GPU parity: the whole stack (embedding, layers, final norm, tied LM head, greedy
argmax) for prefill and decode, against the oracle."""
import numpy as np
import pytest

import decoder_only_forward_amd as q3
import oracle
import synth
from synth import recipes
from q3_testutil import fill_cache_synthetic, layer_to_dev, log, new_cache, parity, small_cfg, \
    to_dev_bf16

pytestmark = pytest.mark.gpu


def _model_dev(model, dev):
    d = {"embed": to_dev_bf16(model["embed"], dev), "norm": to_dev_bf16(model["norm"], dev),
         "lm_head": None if model.get("lm_head") is None else to_dev_bf16(model["lm_head"], dev),
         "layers": [layer_to_dev(l, dev) for l in model["layers"]]}
    mw, keep = q3.make_model_weights(d["embed"], d["norm"], d["layers"], d["lm_head"])
    return mw, (d, keep)


def _rope(cfg, dev):
    import torch
    rope = torch.empty(2 * cfg["max_position_embeddings"] * 64, dtype=torch.float32, device=dev)
    q3.qwen3_rope_table_init(cfg, rope)
    return rope


@pytest.mark.parametrize("tied", [1, 0])
def test_stack_prefill_all_logits_and_argmax(gpu, tied):
    import torch
    cfg = small_cfg(L=3, V=1000)
    cfg["tie_word_embeddings"] = tied
    B, S = 2, 77
    log(f"case stack_prefill tied={tied}: B={B} S={S} L=3 V=1000")
    model = recipes.model_host(21, cfg)
    mw, keep = _model_dev(model, gpu)
    ids = synth.uniform_i32(21, "input.ids", (B, S), 0, cfg["vocab_size"])
    idd = torch.from_numpy(ids).to(gpu)
    cap = 128
    caches = [new_cache(B, 2, cap, gpu) for _ in range(3)]
    kvs = [q3.make_kv_layer(k, vt, cap) for k, vt in caches]
    logits = torch.empty((B, S, cfg["vocab_size"]), dtype=torch.float32, device=gpu)
    nxt = torch.empty((B,), dtype=torch.int32, device=gpu)
    ws = torch.empty(q3.qwen3_workspace_bytes(cfg, q3.QWEN3_OP_STACK_PREFILL, B, S),
                     dtype=torch.uint8, device=gpu)
    q3.qwen3_stack_forward(cfg, mw, _rope(cfg, gpu), idd, B, S, 0, None, kvs, logits,
                           q3.QWEN3_LOGITS_ALL, nxt, ws)
    torch.cuda.synchronize()
    got = logits.cpu().numpy()
    for b in range(B):
        ref = oracle.stack_prefill(cfg, model, ids[b])
        parity(got[b], ref, f"logits[b={b}]")
    # same-input rule: argmax of the GPU's own logits, lowest index on ties
    np.testing.assert_array_equal(nxt.cpu().numpy(), oracle.argmax(got[:, -1, :]))
    # LAST mode equals the last rows of ALL
    last = torch.empty((B, cfg["vocab_size"]), dtype=torch.float32, device=gpu)
    caches2 = [new_cache(B, 2, cap, gpu) for _ in range(3)]
    q3.qwen3_stack_forward(cfg, mw, _rope(cfg, gpu), idd, B, S, 0, None,
                           [q3.make_kv_layer(k, vt, cap) for k, vt in caches2], last,
                           q3.QWEN3_LOGITS_LAST, None, ws)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(last.cpu().numpy(), got[:, -1, :])


def test_stack_decode_step(gpu):
    import torch
    cfg = small_cfg(L=2, V=700)
    positions = [50, 127, 3]
    B = len(positions)
    ctx = max(positions)
    log(f"case stack_decode: pos={positions}")
    model = recipes.model_host(22, cfg)
    mw, keep = _model_dev(model, gpu)
    ids = synth.uniform_i32(22, "input.ids", (B,), 0, cfg["vocab_size"])
    cap = 128
    caches = []
    for l in range(2):
        k, vt = new_cache(B, 2, cap, gpu)
        fill_cache_synthetic(k, vt, 22, l, ctx, ctx)
        caches.append((k, vt))
    logits = torch.empty((B, cfg["vocab_size"]), dtype=torch.float32, device=gpu)
    nxt = torch.empty((B,), dtype=torch.int32, device=gpu)
    ws = torch.empty(q3.qwen3_workspace_bytes(cfg, q3.QWEN3_OP_STACK_DECODE, B),
                     dtype=torch.uint8, device=gpu)
    pos = torch.tensor(positions, dtype=torch.int32, device=gpu)
    q3.qwen3_stack_forward(cfg, mw, _rope(cfg, gpu), torch.from_numpy(ids).to(gpu), B, 1, 0,
                           pos, [q3.make_kv_layer(k, vt, cap) for k, vt in caches], logits,
                           q3.QWEN3_LOGITS_LAST, nxt, ws)
    torch.cuda.synchronize()
    got = logits.cpu().numpy()
    for b, p in enumerate(positions):
        ck, cv = [], []
        for l in range(2):
            k, v = recipes.kv_host(22, cfg, l, b, p, (2, ctx))
            ck.append(k)
            cv.append(v)
        ref = oracle.stack_decode(cfg, model, ids[b], p, ck, cv)
        parity(got[b], ref, f"decode logits[b={b}]")
    np.testing.assert_array_equal(nxt.cpu().numpy(), oracle.argmax(got))


def test_prefill_then_decode_matches_longer_prefill(gpu):
    """Cache written by a GPU prefill, then one GPU decode step: the decode logits match
    the oracle's prefill over the longer sequence (row S)."""
    import torch
    cfg = small_cfg(L=2, V=600)
    B, S = 2, 40
    model = recipes.model_host(23, cfg)
    mw, keep = _model_dev(model, gpu)
    ids = synth.uniform_i32(23, "input.ids", (B, S + 1), 0, cfg["vocab_size"])
    cap = 64
    caches = [new_cache(B, 2, cap, gpu) for _ in range(2)]
    kvs = [q3.make_kv_layer(k, vt, cap) for k, vt in caches]
    ws = torch.empty(q3.qwen3_workspace_bytes(cfg, q3.QWEN3_OP_STACK_PREFILL, B, S),
                     dtype=torch.uint8, device=gpu)
    rope = _rope(cfg, gpu)
    idd = torch.from_numpy(np.ascontiguousarray(ids[:, :S])).to(gpu)
    q3.qwen3_stack_forward(cfg, mw, rope, idd, B, S, 0, None, kvs, None, q3.QWEN3_LOGITS_NONE,
                           None, ws)
    logits = torch.empty((B, cfg["vocab_size"]), dtype=torch.float32, device=gpu)
    wsd = torch.empty(q3.qwen3_workspace_bytes(cfg, q3.QWEN3_OP_STACK_DECODE, B),
                      dtype=torch.uint8, device=gpu)
    pos = torch.full((B,), S, dtype=torch.int32, device=gpu)
    last = torch.from_numpy(np.ascontiguousarray(ids[:, S])).to(gpu)
    q3.qwen3_stack_forward(cfg, mw, rope, last, B, 1, 0, pos, kvs, logits, q3.QWEN3_LOGITS_LAST,
                           None, wsd)
    torch.cuda.synchronize()
    got = logits.cpu().numpy()
    for b in range(B):
        ref = oracle.stack_prefill(cfg, model, ids[b], rows=[S])
        parity(got[b], ref[0], f"prefill+decode logits[b={b}]")


# A seeded sweep of whole-stack prefills over small valid shapes: vocabularies of any size
# (the LM head's last column tile and the argmax chunks ragged), one or two layers, tied or
# untied head, 1-8 q heads per kv head, ragged B x S.  Every logit is compared, the argmax on
# the GPU's own logits, and LAST mode bit for bit against ALL's last rows.
def _stack_sweep(n=8, seed=2027):
    rng = np.random.default_rng(seed)
    out = []
    for _ in range(n):
        nkv = int(rng.choice([1, 2, 4]))
        kw = dict(H=64 * int(rng.integers(1, 7)), nq=nkv * int(rng.choice([1, 2, 3, 7, 8])),
                  nkv=nkv, I=64 * int(rng.integers(1, 9)), L=int(rng.integers(1, 3)),
                  V=int(rng.integers(64, 3001)), qk_norm=int(rng.integers(0, 2)),
                  rope_interleaved=int(rng.integers(0, 2)))
        out.append((kw, int(rng.integers(0, 2)), int(rng.integers(1, 4)),
                    int(rng.integers(1, 200))))
    return out


STACK_SWEEP = _stack_sweep()


@pytest.mark.parametrize("i", range(len(STACK_SWEEP)))
def test_stack_prefill_shape_sweep(gpu, i):
    import torch
    kw, tied, B, S = STACK_SWEEP[i]
    cfg = small_cfg(**kw)
    cfg["tie_word_embeddings"] = tied
    L, V, nkv = cfg["num_hidden_layers"], cfg["vocab_size"], cfg["num_key_value_heads"]
    log(f"case stack_prefill/sweep{i}: {kw} tied={tied} B={B} S={S}")
    model = recipes.model_host(400 + i, cfg)
    mw, keep = _model_dev(model, gpu)
    ids = synth.uniform_i32(400 + i, "input.ids", (B, S), 0, V)
    idd = torch.from_numpy(ids).to(gpu)
    cap = ((S + 63) // 64) * 64
    ws = torch.empty(q3.qwen3_workspace_bytes(cfg, q3.QWEN3_OP_STACK_PREFILL, B, S),
                     dtype=torch.uint8, device=gpu)
    logits = torch.empty((B, S, V), dtype=torch.float32, device=gpu)
    nxt = torch.empty((B,), dtype=torch.int32, device=gpu)
    caches = [new_cache(B, nkv, cap, gpu) for _ in range(L)]
    q3.qwen3_stack_forward(cfg, mw, _rope(cfg, gpu), idd, B, S, 0, None,
                           [q3.make_kv_layer(k, vt, cap) for k, vt in caches], logits,
                           q3.QWEN3_LOGITS_ALL, nxt, ws)
    last = torch.empty((B, V), dtype=torch.float32, device=gpu)
    caches2 = [new_cache(B, nkv, cap, gpu) for _ in range(L)]
    q3.qwen3_stack_forward(cfg, mw, _rope(cfg, gpu), idd, B, S, 0, None,
                           [q3.make_kv_layer(k, vt, cap) for k, vt in caches2], last,
                           q3.QWEN3_LOGITS_LAST, None, ws)
    torch.cuda.synchronize()
    got = logits.cpu().numpy()
    for b in range(B):
        parity(got[b], oracle.stack_prefill(cfg, model, ids[b]), f"logits[b={b}]")
    np.testing.assert_array_equal(nxt.cpu().numpy(), oracle.argmax(got[:, -1, :]))
    np.testing.assert_array_equal(last.cpu().numpy(), got[:, -1, :])
