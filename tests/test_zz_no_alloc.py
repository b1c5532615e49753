"""GPU check of the allocation-free block decode (qwen3_block_decode_static) against the
workspace entry point (qwen3_block_decode): the same inputs and caches must give bit-identical
outputs and cache writes, on two calls in a row, the second with a smaller batch (the static
scratch keeps the first call's contents, which must not leak into the second)."""
import numpy as np
import pytest

import decoder_only_forward_amd as q3
import synth
from synth import recipes
from q3_testutil import bf16_host, layer_to_dev, log, new_cache, fill_cache_synthetic, to_dev_bf16

pytestmark = pytest.mark.gpu


def test_block_decode_static_equals_workspace_entry(gpu):
    import torch
    cfg = dict(recipes.QWEN3_0P6B)
    H, nkv, cap = cfg["hidden_size"], cfg["num_key_value_heads"], 1024
    seed = 41
    layer = recipes.layer_host(seed, cfg, 0)
    lw = layer_to_dev(layer, gpu)
    rope = torch.empty(2 * cfg["max_position_embeddings"] * 64, dtype=torch.float32, device=gpu)
    q3.qwen3_rope_table_init(cfg, rope)
    for call, (B, positions) in enumerate(((8, [0, 5, 100, 511, 700, 1023, 64, 300]),
                                           (3, [900, 17, 255]))):
        log(f"case no_alloc/call{call}: B={B} pos={positions} cap={cap}")
        need = q3.qwen3_workspace_bytes(cfg, q3.QWEN3_OP_BLOCK_DECODE, B)
        assert need <= q3.QWEN3_STATIC_SCRATCH_BYTES
        x = synth.normal_bf16(seed + call, recipes.activations_name(), (B, H))
        xd = to_dev_bf16(x, gpu)
        pos = torch.tensor(positions, dtype=torch.int32, device=gpu)
        caches = []
        for _ in range(2):
            k, vt = new_cache(B, nkv, cap, gpu)
            fill_cache_synthetic(k, vt, seed, 0, 0, cap, rows={b: p for b, p in enumerate(positions)})
            caches.append((k, vt))
        assert torch.equal(caches[0][0].view(torch.int16), caches[1][0].view(torch.int16))
        out_ws = torch.empty_like(xd)
        out_st = torch.empty_like(xd)
        ws = torch.empty(need, dtype=torch.uint8, device=gpu)
        q3.qwen3_block_decode(cfg, lw, rope, xd, out_ws, B, pos,
                              q3.make_kv_layer(*caches[0], cap), ws)
        q3.qwen3_block_decode_static(cfg, lw, rope, xd, out_st, B, pos,
                                     q3.make_kv_layer(*caches[1], cap))
        torch.cuda.synchronize()
        a, b = bf16_host(out_ws), bf16_host(out_st)
        assert np.all(np.isfinite(synth.bf16_to_f32(a)))
        np.testing.assert_array_equal(b, a)
        for (ka, va), (kb, vb) in [(caches[0], caches[1])]:
            np.testing.assert_array_equal(bf16_host(kb), bf16_host(ka))
            np.testing.assert_array_equal(bf16_host(vb), bf16_host(va))
        log(f"  call {call}: outputs and cache writes bit-identical")
