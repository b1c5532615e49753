"""GPU parity: one decoder block (prefill, chunked prefill, decode) against the oracle."""
import numpy as np
import pytest

import decoder_only_forward_amd as q3
import oracle
import synth
from synth import recipes
from q3_testutil import (bf16_host, cache_k_logical, cache_v_logical, f64, fill_cache_synthetic,
                         layer_to_dev, log, new_cache, parity, small_cfg, to_dev_bf16)

pytestmark = pytest.mark.gpu


def _rope(cfg, dev):
    import torch
    rope = torch.empty(2 * cfg["max_position_embeddings"] * 64, dtype=torch.float32, device=dev)
    q3.qwen3_rope_table_init(cfg, rope)
    return rope


PREFILL_CASES = {
    # name: (cfg kwargs, B, S, pos0)
    "small_ragged": (dict(), 2, 200, 0),
    "small_chunked": (dict(), 2, 93, 70),
    "group7": (dict(nq=7, nkv=1), 1, 130, 0),
    "no_qk_norm": (dict(qk_norm=0), 1, 64, 0),
    "one_token": (dict(), 3, 1, 0),
    "interleaved_rope": (dict(rope_interleaved=1), 2, 150, 0),
    "interleaved_rope_chunked": (dict(rope_interleaved=1), 1, 70, 60),
    "cfg1_0p6b": (None, 1, 128, 0),
    # above 256 rows the projections are tiled and the QKV epilogue does q/k-norm, RoPE and
    # the cache writes; 128-row tiles then straddle sequences when S is not a multiple of 128
    "tiled_chunked": (dict(), 3, 130, 70),
    "tiled_group7": (dict(nq=7, nkv=1), 3, 100, 0),
    "tiled_no_qk_norm": (dict(qk_norm=0), 2, 160, 0),
    # longer sequences: several causal row blocks of very different lengths
    "long_sequence": (dict(), 1, 1000, 0),
    "long_group7": (dict(nq=7, nkv=1), 2, 450, 0),
    # sixteen q heads per kv head (a 64 q / 4 kv model's grouping), tiled and small
    "group16_tiled": (dict(nq=16, nkv=1), 2, 160, 0),
    "group16_chunked": (dict(nq=16, nkv=1), 1, 40, 30),
    # a hidden size that is a multiple of 64 but not of 128: the o_proj and down products end
    # in a partly filled column tile (and, at 300 rows, a partly filled row tile), so their
    # residual epilogues take both the full-tile and the bounds-checked path
    "tiled_h320": (dict(H=320), 2, 150, 0),
    "tiled_h320_chunked": (dict(H=320), 3, 100, 40),
    "small_h320": (dict(H=320), 1, 90, 0),
}


@pytest.mark.parametrize("name", list(PREFILL_CASES))
def test_block_prefill_parity(gpu, name):
    kw, B, S, pos0 = PREFILL_CASES[name]
    cfg = dict(recipes.QWEN3_0P6B) if kw is None else small_cfg(**kw)
    log(f"case block_prefill/{name}: B={B} S={S} pos0={pos0}")
    _block_prefill_case(gpu, cfg, B, S, pos0)


def _block_prefill_case(gpu, cfg, B, S, pos0, seed=11):
    import torch
    H, nkv = cfg["hidden_size"], cfg["num_key_value_heads"]
    layer = recipes.layer_host(seed, cfg, 0)
    x = synth.normal_bf16(seed, recipes.activations_name(), (B, S, H))
    lw = layer_to_dev(layer, gpu)
    rope = _rope(cfg, gpu)
    cap = ((pos0 + S + 63) // 64) * 64
    k, vt = new_cache(B, nkv, cap, gpu)
    if pos0:
        fill_cache_synthetic(k, vt, seed, 0, pos0, pos0)
    xd = to_dev_bf16(x, gpu)
    out = torch.empty_like(xd)
    ws = torch.empty(q3.qwen3_workspace_bytes(cfg, q3.QWEN3_OP_BLOCK_PREFILL, B, S),
                     dtype=torch.uint8, device=gpu)
    kv = q3.make_kv_layer(k, vt, cap)
    q3.qwen3_block_prefill(cfg, lw, rope, xd, out, B, S, pos0, kv, ws)
    torch.cuda.synchronize()
    got = f64(bf16_host(out))
    for b in range(B):
        pk = pv = None
        if pos0:
            pk, pv = recipes.kv_host(seed, cfg, 0, b, pos0, (nkv, pos0))
            pk, pv = f64(pk), f64(pv)
        ref, nk, nv = oracle.block(cfg, layer, f64(x[b]), pos0, pk, pv)
        parity(got[b], ref, f"x_out[b={b}]")
        parity(cache_k_logical(k, b, pos0 + S)[:, pos0:], nk, f"cache_k[b={b}]")
        parity(cache_v_logical(vt, b, pos0 + S)[:, pos0:], nv, f"cache_v[b={b}]")
        if pos0:  # the past must be left untouched
            np.testing.assert_array_equal(cache_k_logical(k, b, pos0), pk)


def test_block_prefill_deterministic(gpu):
    import torch
    cfg = small_cfg()
    B, S = 2, 150
    layer = layer_to_dev(recipes.layer_host(3, cfg, 0), gpu)
    x = to_dev_bf16(synth.normal_bf16(3, recipes.activations_name(), (B, S, 256)), gpu)
    rope = _rope(cfg, gpu)
    outs = []
    for _ in range(2):
        k, vt = new_cache(B, 2, 192, gpu)
        out = torch.empty_like(x)
        ws = torch.empty(q3.qwen3_workspace_bytes(cfg, q3.QWEN3_OP_BLOCK_PREFILL, B, S),
                         dtype=torch.uint8, device=gpu)
        q3.qwen3_block_prefill(cfg, layer, rope, x, out, B, S, 0, q3.make_kv_layer(k, vt, 192),
                               ws)
        torch.cuda.synchronize()
        outs.append(bf16_host(out))
    np.testing.assert_array_equal(outs[0], outs[1])


@pytest.mark.parametrize("B,S", [(2, 150), (1, 40)])
def test_block_prefill_without_cache_equals_with_cache(gpu, B, S):
    # With no cache the call keeps its keys and values in the workspace: the output must be
    # the same bits as with a caller cache (tiled projections at 300 rows, decode-size ones
    # at 40), and every output row must still match the oracle.
    import torch
    cfg = small_cfg()
    log(f"case block prefill without cache: B={B} S={S}")
    host = recipes.layer_host(5, cfg, 0)
    layer = layer_to_dev(host, gpu)
    xh = synth.normal_bf16(5, recipes.activations_name(), (B, S, 256))
    x = to_dev_bf16(xh, gpu)
    rope = _rope(cfg, gpu)
    ws = torch.empty(q3.qwen3_workspace_bytes(cfg, q3.QWEN3_OP_BLOCK_PREFILL, B, S),
                     dtype=torch.uint8, device=gpu)
    cap = ((S + 63) // 64) * 64
    k, vt = new_cache(B, 2, cap, gpu)
    with_cache = torch.empty_like(x)
    q3.qwen3_block_prefill(cfg, layer, rope, x, with_cache, B, S, 0,
                           q3.make_kv_layer(k, vt, cap), ws)
    without = torch.empty_like(x)
    q3.qwen3_block_prefill(cfg, layer, rope, x, without, B, S, 0, None, ws)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(bf16_host(without), bf16_host(with_cache))
    got = synth.bf16_to_f32(bf16_host(without)).astype(np.float64)
    for b in range(B):
        ref, _, _ = oracle.block(cfg, host, f64(xh[b]))
        parity(got[b], ref, f"x_out[{b}] without cache")


DECODE_CASES = {
    "small": (dict(), [0, 100, 255, 37], 256),
    "group7": (dict(nq=7, nkv=1), [300, 5], 320),
    # two 8-query blocks per (sequence, kv head)
    "group16": (dict(nq=16, nkv=1), [200, 63, 0], 256),
    "interleaved_rope": (dict(rope_interleaved=1), [0, 77, 200], 256),
    "cfg_0p6b": (None, [4096, 1000], 4160),
    # the 7B-shaped block: K = 3584 and 18944 decode products, 7 q heads per kv head
    "cfg_7b": ("7b", [2000, 37], 2048),
}


@pytest.mark.parametrize("name", list(DECODE_CASES))
def test_block_decode_parity(gpu, name):
    kw, positions, cap = DECODE_CASES[name]
    if kw is None:
        cfg = dict(recipes.QWEN3_0P6B)
    elif kw == "7b":
        cfg = dict(recipes.QWEN_7B_BLOCK)
    else:
        cfg = small_cfg(**kw)
    log(f"case block_decode/{name}: pos={positions} cap={cap}")
    _block_decode_case(gpu, cfg, positions, cap)


def _block_decode_case(gpu, cfg, positions, cap, seed=12):
    import torch
    B = len(positions)
    H, nkv = cfg["hidden_size"], cfg["num_key_value_heads"]
    layer = recipes.layer_host(seed, cfg, 0)
    x = synth.normal_bf16(seed, recipes.activations_name(), (B, H))
    ctx = max(positions)
    k, vt = new_cache(B, nkv, cap, gpu)
    fill_cache_synthetic(k, vt, seed, 0, ctx, ctx)  # every sequence: positions < ctx
    pos = torch.tensor(positions, dtype=torch.int32, device=gpu)
    xd = to_dev_bf16(x, gpu)
    out = torch.empty_like(xd)
    ws = torch.empty(q3.qwen3_workspace_bytes(cfg, q3.QWEN3_OP_BLOCK_DECODE, B),
                     dtype=torch.uint8, device=gpu)
    q3.qwen3_block_decode(cfg, layer_to_dev(layer, gpu), _rope(cfg, gpu), xd, out, B, pos,
                          q3.make_kv_layer(k, vt, cap), ws)
    torch.cuda.synchronize()
    got = f64(bf16_host(out))
    for b, p in enumerate(positions):
        pk, pv = recipes.kv_host(seed, cfg, 0, b, p, (nkv, ctx))
        ref, nk, nv = oracle.block(cfg, layer, f64(x[b:b + 1]), p, f64(pk), f64(pv))
        parity(got[b:b + 1], ref, f"x_out[b={b}]")
        parity(cache_k_logical(k, b, p + 1)[:, p:], nk, f"cache_k[b={b}]")
        parity(cache_v_logical(vt, b, p + 1)[:, p:], nv, f"cache_v[b={b}]")


def test_block_decode_out_of_range_position_gives_nan_row(gpu):
    import torch
    cfg = small_cfg()
    B, cap = 2, 128
    layer = layer_to_dev(recipes.layer_host(5, cfg, 0), gpu)
    x = to_dev_bf16(synth.normal_bf16(5, recipes.activations_name(), (B, 256)), gpu)
    k, vt = new_cache(B, 2, cap, gpu)
    k.zero_()
    vt.zero_()
    pos = torch.tensor([10, cap], dtype=torch.int32, device=gpu)
    out = torch.empty_like(x)
    ws = torch.empty(q3.qwen3_workspace_bytes(cfg, q3.QWEN3_OP_BLOCK_DECODE, B),
                     dtype=torch.uint8, device=gpu)
    q3.qwen3_block_decode(cfg, layer, _rope(cfg, gpu), x, out, B, pos,
                          q3.make_kv_layer(k, vt, cap), ws)
    torch.cuda.synchronize()
    o = out.float().cpu().numpy()
    assert np.all(np.isfinite(o[0])) and np.all(np.isnan(o[1]))


# A seeded sweep over small valid shapes, beyond the hand-picked cases: hidden and
# intermediate sizes at every multiple of 64 up to 512 / 768, 1-4 kv heads with 1-8 q heads
# each, ragged lengths, prefills onto a past, both q/k-norm settings and both RoPE pairings;
# decode steps at ragged positions.  The list is fixed by its seed.
def _sweep_cfg(rng):
    nkv = int(rng.choice([1, 2, 4]))
    g = int(rng.choice([1, 2, 3, 5, 7, 8]))
    return dict(H=64 * int(rng.integers(1, 9)), nq=nkv * g, nkv=nkv,
                I=64 * int(rng.integers(1, 13)), qk_norm=int(rng.integers(0, 2)),
                rope_interleaved=int(rng.integers(0, 2)))


def _prefill_sweep(n=16, seed=2024):
    rng = np.random.default_rng(seed)
    out = []
    for _ in range(n):
        kw = _sweep_cfg(rng)
        B, S = int(rng.integers(1, 4)), int(rng.integers(1, 300))
        pos0 = 0 if rng.integers(0, 2) == 0 else int(rng.integers(1, 150))
        out.append((kw, B, S, pos0))
    return out


def _decode_sweep(n=12, seed=2025):
    rng = np.random.default_rng(seed)
    out = []
    for _ in range(n):
        kw = _sweep_cfg(rng)
        cap = 64 * int(rng.integers(1, 9))
        positions = [int(p) for p in rng.integers(0, cap, size=int(rng.integers(1, 6)))]
        out.append((kw, positions, cap))
    return out


PREFILL_SWEEP = _prefill_sweep()
DECODE_SWEEP = _decode_sweep()


@pytest.mark.parametrize("i", range(len(PREFILL_SWEEP)))
def test_block_prefill_shape_sweep(gpu, i):
    kw, B, S, pos0 = PREFILL_SWEEP[i]
    log(f"case block_prefill/sweep{i}: {kw} B={B} S={S} pos0={pos0}")
    _block_prefill_case(gpu, small_cfg(**kw), B, S, pos0, seed=100 + i)


@pytest.mark.parametrize("i", range(len(DECODE_SWEEP)))
def test_block_decode_shape_sweep(gpu, i):
    kw, positions, cap = DECODE_SWEEP[i]
    log(f"case block_decode/sweep{i}: {kw} pos={positions} cap={cap}")
    _block_decode_case(gpu, small_cfg(**kw), positions, cap, seed=200 + i)
