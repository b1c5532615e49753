"""GPU checks of the library's stream contract: every entry point only enqueues work on the
stream it is given, allocates nothing and never synchronises, so (1) independent calls on two
streams give the same bits as the same calls one after the other, and (2) a decode step
captured in a HIP graph and replayed gives, on every replay, the bits of the eager call."""
import numpy as np
import pytest

import decoder_only_forward_amd as q3
import synth
from synth import recipes
from q3_testutil import (bf16_host, fill_cache_synthetic, layer_to_dev, log, new_cache,
                         small_cfg, to_dev_bf16)

pytestmark = pytest.mark.gpu


def _rope(cfg, dev):
    import torch
    rope = torch.empty(2 * cfg["max_position_embeddings"] * 64, dtype=torch.float32, device=dev)
    q3.qwen3_rope_table_init(cfg, rope)
    return rope


def test_block_decodes_on_two_streams_equal_sequential_calls(gpu):
    import torch
    cfg = dict(recipes.QWEN3_0P6B)
    H, nkv, cap, B = cfg["hidden_size"], cfg["num_key_value_heads"], 1024, 8
    log(f"case streams: two block decodes B={B} cap={cap} on two streams")
    layer = layer_to_dev(recipes.layer_host(51, cfg, 0), gpu)
    rope = _rope(cfg, gpu)
    jobs = []
    for j in range(2):
        positions = [int(p) for p in synth.uniform_i32(52 + j, "input.pos", (B,), 0, cap)]
        x = to_dev_bf16(synth.normal_bf16(53 + j, recipes.activations_name(), (B, H)), gpu)
        pos = torch.tensor(positions, dtype=torch.int32, device=gpu)
        jobs.append((x, pos, positions))

    def run(streams):
        outs = []
        for j, (x, pos, positions) in enumerate(jobs):
            k, vt = new_cache(B, nkv, cap, gpu)
            fill_cache_synthetic(k, vt, 54 + j, 0, 0, cap,
                                 rows={b: p for b, p in enumerate(positions)})
            out = torch.empty_like(x)
            ws = torch.empty(q3.qwen3_workspace_bytes(cfg, q3.QWEN3_OP_BLOCK_DECODE, B),
                             dtype=torch.uint8, device=gpu)
            outs.append((out, k, vt, ws))
        torch.cuda.synchronize()
        for j, (x, pos, _) in enumerate(jobs):
            out, k, vt, ws = outs[j]
            s = streams[j] if streams else None
            q3.qwen3_block_decode(cfg, layer, rope, x, out, B, pos,
                                  q3.make_kv_layer(k, vt, cap), ws, stream=s)
        torch.cuda.synchronize()
        return [(bf16_host(o), bf16_host(k), bf16_host(vt)) for o, k, vt, _ in outs]

    ref = run(None)
    got = run([torch.cuda.Stream(), torch.cuda.Stream()])
    for (a, ka, va), (b, kb, vb) in zip(ref, got):
        np.testing.assert_array_equal(b, a)
        np.testing.assert_array_equal(kb, ka)
        np.testing.assert_array_equal(vb, va)


def test_stack_decode_step_replayed_from_a_graph_equals_eager(gpu):
    import torch
    cfg = small_cfg(L=2, V=700)
    positions = [50, 127, 3, 90]
    B, cap = len(positions), 128
    log(f"case graph: stack decode step pos={positions}, captured and replayed 3 times")
    model = recipes.model_host(61, cfg)
    d = {"embed": to_dev_bf16(model["embed"], gpu), "norm": to_dev_bf16(model["norm"], gpu),
         "layers": [layer_to_dev(l, gpu) for l in model["layers"]]}
    mw, keep = q3.make_model_weights(d["embed"], d["norm"], d["layers"], None)
    rope = _rope(cfg, gpu)
    caches = []
    for l in range(2):
        k, vt = new_cache(B, 2, cap, gpu)
        fill_cache_synthetic(k, vt, 62, l, max(positions), max(positions))
        caches.append((k, vt))
    kvs = [q3.make_kv_layer(k, vt, cap) for k, vt in caches]
    ids = torch.from_numpy(synth.uniform_i32(63, "input.ids", (B,), 0, cfg["vocab_size"])).to(gpu)
    pos = torch.tensor(positions, dtype=torch.int32, device=gpu)
    logits = torch.empty((B, cfg["vocab_size"]), dtype=torch.float32, device=gpu)
    nxt = torch.empty((B,), dtype=torch.int32, device=gpu)
    ws = torch.empty(q3.qwen3_workspace_bytes(cfg, q3.QWEN3_OP_STACK_DECODE, B),
                     dtype=torch.uint8, device=gpu)

    def step():
        q3.qwen3_stack_forward(cfg, mw, rope, ids, B, 1, 0, pos, kvs, logits,
                               q3.QWEN3_LOGITS_LAST, nxt, ws)

    step()
    torch.cuda.synchronize()
    eager = logits.cpu().numpy().copy()
    eager_ids = nxt.cpu().numpy().copy()
    eager_k = [bf16_host(k) for k, _ in caches]

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        step()
    torch.cuda.synchronize()
    for r in range(3):
        # the program's own eager work between the replays: clobber the outputs first
        logits.fill_(float("nan"))
        nxt.fill_(-1)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        np.testing.assert_array_equal(logits.cpu().numpy(), eager, err_msg=f"replay {r}")
        np.testing.assert_array_equal(nxt.cpu().numpy(), eager_ids, err_msg=f"replay {r}")
        for l, (k, _) in enumerate(caches):
            np.testing.assert_array_equal(bf16_host(k), eager_k[l], err_msg=f"replay {r}")
    del g
