"""GPU parity: decode of several new tokens per sequence (qwen3_stack_forward with seq_len > 1
and device positions): sequence b's tokens take positions pos[b] .. pos[b] + S - 1 on a cache
that holds positions 0 .. pos[b] - 1, each seeing the cache and the new tokens up to itself
([P3] "prefill 与 decode"; [P2] section 4's mask slice), against the oracle's decode of the
same tokens on the same cache."""
import numpy as np
import pytest

import decoder_only_forward_amd as q3
import oracle
import synth
from synth import recipes
from q3_testutil import (cache_logical_host, fill_cache_synthetic, layer_to_dev, log, new_cache,
                         parity, small_cfg, to_dev_bf16)

pytestmark = pytest.mark.gpu


def _run(gpu, cfg, seed, positions, S, cap, mode):
    import torch
    L, V = cfg["num_hidden_layers"], cfg["vocab_size"]
    nkv = cfg["num_key_value_heads"]
    B = len(positions)
    ctx = cap
    model = recipes.model_host(seed, cfg)
    d = {"embed": to_dev_bf16(model["embed"], gpu), "norm": to_dev_bf16(model["norm"], gpu),
         "layers": [layer_to_dev(l, gpu) for l in model["layers"]]}
    mw, keep = q3.make_model_weights(d["embed"], d["norm"], d["layers"], None)
    rope = torch.empty(2 * cfg["max_position_embeddings"] * 64, dtype=torch.float32, device=gpu)
    q3.qwen3_rope_table_init(cfg, rope)
    caches = []
    for l in range(L):
        k, vt = new_cache(B, nkv, cap, gpu)
        fill_cache_synthetic(k, vt, seed, l, 0, ctx,
                             rows={b: min(max(p, 0), cap) for b, p in enumerate(positions)})
        caches.append((k, vt))
    before = [cache_logical_host(k, vt) for k, vt in caches]
    ids = synth.uniform_i32(seed, "input.ids", (B, S), 0, V)
    rows = B * S if mode == q3.QWEN3_LOGITS_ALL else B
    logits = torch.empty((rows, V), dtype=torch.float32, device=gpu)
    nxt = torch.empty((B,), dtype=torch.int32, device=gpu)
    ws = torch.empty(q3.qwen3_workspace_bytes(cfg, q3.QWEN3_OP_STACK_DECODE, B, S),
                     dtype=torch.uint8, device=gpu)
    pos = torch.tensor(positions, dtype=torch.int32, device=gpu)
    q3.qwen3_stack_forward(cfg, mw, rope, torch.from_numpy(ids).to(gpu), B, S, 0, pos,
                           [q3.make_kv_layer(k, vt, cap) for k, vt in caches], logits, mode,
                           nxt, ws)
    torch.cuda.synchronize()
    got = logits.cpu().numpy()
    after = [cache_logical_host(k, vt) for k, vt in caches]
    return model, ids, got, nxt.cpu().numpy(), before, after


def _oracle(cfg, model, seed, ids_b, b, p, ctx):
    ck, cv = [], []
    for l in range(cfg["num_hidden_layers"]):
        k, v = recipes.kv_host(seed, cfg, l, b, p, (cfg["num_key_value_heads"], ctx))
        ck.append(k)
        cv.append(v)
    return oracle.stack_decode(cfg, model, ids_b, p, ck, cv)


CASES = {
    # positions per sequence, new tokens per sequence, cache capacity, config overrides
    "s5_ragged": ([50, 120, 0], 5, 128, {}),
    "s20_tile_gemms": ([7, 64, 33, 90], 20, 128, {}),   # 80 rows: tiled projections
    "g8_three_groups": ([70, 3], 3, 128, dict(nq=8, nkv=1)),  # 24 queries per kv head
    "g16_six_groups": ([70, 3], 3, 128, dict(nq=16, nkv=1)),  # 48 queries per kv head
}


@pytest.mark.parametrize("name", list(CASES))
def test_multi_token_decode_matches_oracle(gpu, name):
    positions, S, cap, over = CASES[name]
    cfg = small_cfg(L=2, V=600, **over)
    log(f"case multi-token decode/{name}: pos={positions} S={S} cap={cap}")
    _check_all_rows(gpu, cfg, 51, positions, S, cap)


def _check_all_rows(gpu, cfg, seed, positions, S, cap):
    model, ids, got, nxt, before, after = _run(gpu, cfg, seed, positions, S, cap,
                                               q3.QWEN3_LOGITS_ALL)
    got = got.reshape(len(positions), S, -1)
    for b, p in enumerate(positions):
        ref = _oracle(cfg, model, seed, ids[b], b, p, cap)
        parity(got[b], ref, f"logits[b={b}, pos={p}]")
    np.testing.assert_array_equal(nxt, oracle.argmax(np.ascontiguousarray(got[:, -1, :])))
    # each sequence's new positions were written, nothing else
    for l, ((k0, v0), (k1, v1)) in enumerate(zip(before, after)):
        for b, p in enumerate(positions):
            kd = np.any(k0[b] != k1[b], axis=(0, 2))  # per position
            changed = np.nonzero(kd)[0]
            assert changed.min() >= p and changed.max() < p + S, (l, b, changed)



# A seeded sweep over small valid shapes: 1-5 sequences at ragged positions with 1-12 new
# tokens each (at most 60 rows: decode-size products; above 256 rows the tiled ones, covered
# by the cases above), 1-8 q heads per kv head, hidden and FFN sizes at multiples of 64, one
# or two layers, any vocabulary size, both norm and RoPE settings.
def _multitoken_sweep(n=10, seed=2028):
    rng = np.random.default_rng(seed)
    out = []
    for _ in range(n):
        nkv = int(rng.choice([1, 2, 4]))
        kw = dict(H=64 * int(rng.integers(1, 7)), nq=nkv * int(rng.choice([1, 2, 3, 7, 8])),
                  nkv=nkv, I=64 * int(rng.integers(1, 9)), L=int(rng.integers(1, 3)),
                  V=int(rng.integers(64, 2001)), qk_norm=int(rng.integers(0, 2)),
                  rope_interleaved=int(rng.integers(0, 2)))
        cap = 64 * int(rng.integers(1, 5))
        S = int(rng.integers(1, min(12, cap) + 1))
        positions = [int(p) for p in rng.integers(0, cap - S + 1, size=int(rng.integers(1, 6)))]
        out.append((kw, positions, S, cap))
    return out


MULTITOKEN_SWEEP = _multitoken_sweep()


@pytest.mark.parametrize("i", range(len(MULTITOKEN_SWEEP)))
def test_multi_token_decode_shape_sweep(gpu, i):
    kw, positions, S, cap = MULTITOKEN_SWEEP[i]
    log(f"case multi-token decode/sweep{i}: {kw} pos={positions} S={S} cap={cap}")
    _check_all_rows(gpu, small_cfg(**kw), 500 + i, positions, S, cap)

def test_multi_token_decode_last_rows_and_out_of_range(gpu):
    # LAST mode gives each sequence's last new row; a sequence whose last new position is
    # outside the cache gets NaN logits and leaves its cache untouched
    cap, S = 64, 4
    positions = [10, cap - 2, 31]
    cfg = small_cfg(L=2, V=500)
    log(f"case multi-token decode/last + out of range: pos={positions} S={S}")
    model, ids, got, nxt, before, after = _run(gpu, cfg, 52, positions, S, cap,
                                               q3.QWEN3_LOGITS_LAST)
    for b in (0, 2):
        ref = _oracle(cfg, model, 52, ids[b], b, positions[b], cap)
        parity(got[b], ref[-1], f"last logits[b={b}]")
    assert np.isnan(got[1]).all()
    for (k0, v0), (k1, v1) in zip(before, after):
        np.testing.assert_array_equal(k1[1], k0[1])
        np.testing.assert_array_equal(v1[1], v0[1])


def test_single_token_rows_equal_multi_token_first_row(gpu):
    # token 0 of a multi-token decode sees exactly what a one-token decode sees
    cap = 128
    positions = [40, 77]
    cfg = small_cfg(L=2, V=500)
    log("case multi-token decode/first row vs one token")
    _, ids, got, _, _, _ = _run(gpu, cfg, 53, positions, 6, cap, q3.QWEN3_LOGITS_ALL)
    model = recipes.model_host(53, cfg)
    got = got.reshape(2, 6, -1)
    for b, p in enumerate(positions):
        one = _oracle(cfg, model, 53, ids[b, 0], b, p, cap)
        parity(got[b, 0], one, f"first row[b={b}]")


def test_decode_single_split_many_sequences(gpu):
    # 256 sequences x 2 kv heads fill the GPU with one block per (sequence, kv head): the
    # decode attention then normalises in the kernel with no combine pass; sampled sequences
    # (ragged positions, one token and two tokens per sequence) against the oracle
    cap = 128
    B = 256
    rng = np.random.default_rng(5)
    positions = [int(p) for p in rng.integers(0, cap - 2, B)]
    cfg = small_cfg(L=2, V=300)
    for S in (1, 2):
        log(f"case single-split decode: B={B} S={S}")
        model, ids, got, nxt, _, _ = _run(gpu, cfg, 54, positions, S, cap, q3.QWEN3_LOGITS_ALL)
        got = got.reshape(B, S, -1)
        for b in (0, 1, 77, 128, 255):
            ref = _oracle(cfg, model, 54, ids[b], b, positions[b], cap)
            parity(got[b], ref, f"logits[b={b}, pos={positions[b]}, S={S}]")


def test_decode_at_the_last_positions_of_cache_and_rope_table(gpu):
    # capacity == max_position_embeddings: the new tokens take the very last cache slots and
    # RoPE table rows (one token at position 255, three tokens at 253..255)
    cap = 256
    cfg = small_cfg(L=2, V=300, max_pos=cap)
    for S, positions in ((1, [cap - 1, 100]), (3, [cap - 3, 0])):
        log(f"case decode at the table end: S={S} pos={positions}")
        model, ids, got, nxt, _, _ = _run(gpu, cfg, 55, positions, S, cap, q3.QWEN3_LOGITS_ALL)
        got = got.reshape(len(positions), S, -1)
        for b, p in enumerate(positions):
            parity(got[b], _oracle(cfg, model, 55, ids[b], b, p, cap), f"logits[b={b}, pos={p}]")
