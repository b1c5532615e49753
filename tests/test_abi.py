"""CPU checks of the C ABI: the library loads, exports every declared entry point, and
rejects bad arguments on the host (nothing reaches the GPU on these paths)."""
import ctypes
import os
import re

import pytest

import decoder_only_forward_amd as q3
from synth import recipes

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_functions():
    with open(os.path.join(ROOT, "include", "qwen3.h")) as f:
        src = f.read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(qwen3_[a-z_]+)\s*\(", src)))


def test_header_and_binding_agree():
    decl = declared_functions()
    assert set(decl) == set(q3.EXPORTS), decl


def test_library_exports_every_declared_symbol():
    lib = q3.lib()
    for name in declared_functions():
        assert hasattr(lib, name), name
        assert ctypes.cast(getattr(lib, name), ctypes.c_void_p).value


def test_status_strings():
    lib = q3.lib()
    for code in (0, -1, -2, -3, -4, -5):
        assert lib.qwen3_status_string(code)


def _fake_layer():
    return {k: 0x1000 * (i + 1) for i, k in enumerate(q3.LAYER_FIELDS)}


def _expect(rc_fn, code, text):
    with pytest.raises(RuntimeError) as ei:
        rc_fn()
    msg = str(ei.value)
    assert q3.lib().qwen3_status_string(code).decode() in msg, msg
    assert text in msg, msg


def test_workspace_bytes_scale_with_tokens():
    cfg = recipes.QWEN3_0P6B
    a = q3.qwen3_workspace_bytes(cfg, q3.QWEN3_OP_BLOCK_PREFILL, 1, 128)
    b = q3.qwen3_workspace_bytes(cfg, q3.QWEN3_OP_BLOCK_PREFILL, 4, 2048)
    assert 0 < a < b
    assert q3.qwen3_workspace_bytes(cfg, q3.QWEN3_OP_STACK_DECODE, 64) > 0
    assert q3.qwen3_workspace_bytes(recipes.MOE_2048, q3.QWEN3_OP_MOE_FFN, 8192) > 0
    bad = dict(cfg, head_dim=64)
    assert q3.qwen3_workspace_bytes(bad, q3.QWEN3_OP_BLOCK_PREFILL, 1, 8) == 0
    assert b"head_dim" in q3.lib().qwen3_last_error()


def test_block_prefill_rejects_bad_arguments():
    cfg = dict(recipes.QWEN3_0P6B)
    lw = _fake_layer()
    cache = q3.make_kv_layer(0x10000, 0x20000, 128, regions=64)
    args = dict(rope=0x3000, x_in=0x4000, x_out=0x5000, batch=1, seq_len=64, pos0=0,
                cache=cache, workspace=None)

    def call(c=cfg, w=lw, **kw):
        a = dict(args, **kw)
        return q3.qwen3_block_prefill(c, w, a["rope"], a["x_in"], a["x_out"], a["batch"],
                                      a["seq_len"], a["pos0"], a["cache"], a["workspace"],
                                      stream=0)

    _expect(lambda: call(c=dict(cfg, head_dim=64)), q3.QWEN3_EUNSUPPORTED, "head_dim")
    _expect(lambda: call(c=dict(cfg, num_key_value_heads=3)), q3.QWEN3_EINVAL,
            "num_key_value_heads")
    _expect(lambda: call(c=dict(cfg, rope_interleaved=2)), q3.QWEN3_EINVAL, "rope_interleaved")
    _expect(lambda: call(w=dict(lw, o_proj=0)), q3.QWEN3_EINVAL, "o_proj")
    _expect(lambda: call(w=dict(lw, q_proj=0x1001)), q3.QWEN3_EINVAL, "q_proj")
    _expect(lambda: call(x_out=0x4000), q3.QWEN3_EINVAL, "alias")
    _expect(lambda: call(seq_len=129), q3.QWEN3_ERANGE, "capacity")
    _expect(lambda: call(pos0=-1), q3.QWEN3_ERANGE, "pos0")
    _expect(lambda: call(cache=q3.make_kv_layer(0x10000, 0x20000, 100, regions=64)), q3.QWEN3_EINVAL,
            "capacity")
    big = dict(cfg, max_position_embeddings=100)
    _expect(lambda: call(c=big, seq_len=101, cache=q3.make_kv_layer(0x10000, 0x20000, 128, regions=64)),
            q3.QWEN3_ERANGE, "max_position_embeddings")
    # a cache holding fewer (sequence, kv head) regions than batch x num_key_value_heads
    _expect(lambda: call(cache=q3.make_kv_layer(0x10000, 0x20000, 128, regions=7)),
            q3.QWEN3_EINVAL, "regions")
    _expect(lambda: call(batch=2, cache=q3.make_kv_layer(0x10000, 0x20000, 128, regions=15)),
            q3.QWEN3_EINVAL, "regions")
    _expect(lambda: call(), q3.QWEN3_EWORKSPACE, "workspace")
    # no cache: a prefill from position 0 only, bounded by max_position_embeddings
    _expect(lambda: call(cache=None, pos0=64), q3.QWEN3_EINVAL, "pos0")
    _expect(lambda: call(c=big, seq_len=101, cache=None), q3.QWEN3_ERANGE,
            "max_position_embeddings")
    _expect(lambda: call(cache=None, seq_len=129), q3.QWEN3_EWORKSPACE, "workspace")


def test_moe_rejects_bad_arguments():
    w = q3.make_moe_weights(0x1000, 0x2000, 0x3000)
    base = dict(recipes.MOE_2048)

    def call(c=base, n=16):
        q3.qwen3_moe_ffn(c, w, 0x4000, 0x5000, n, stream=0)

    _expect(lambda: call(c=dict(base, num_experts_per_tok=9)), q3.QWEN3_EUNSUPPORTED,
            "num_experts_per_tok")
    _expect(lambda: call(c=dict(base, num_experts=300)), q3.QWEN3_EUNSUPPORTED, "num_experts")
    _expect(lambda: call(c=dict(base, moe_intermediate_size=100)), q3.QWEN3_EUNSUPPORTED,
            "moe_intermediate_size")
    _expect(lambda: call(n=0), q3.QWEN3_EINVAL, "n_tokens")
    _expect(lambda: call(), q3.QWEN3_EWORKSPACE, "workspace")


def test_stack_rejects_bad_arguments():
    cfg = dict(recipes.QWEN3_0P6B, num_hidden_layers=2)
    layers = [_fake_layer(), _fake_layer()]
    mw, keep = q3.make_model_weights(0x7000, 0x8000, layers)
    caches = [q3.make_kv_layer(0x10000, 0x20000, 128, regions=64)] * 2

    def call(c=cfg, mode=q3.QWEN3_LOGITS_ALL, logits=0x9000, seq_len=16, cs=caches):
        q3.qwen3_stack_forward(c, mw, 0x3000, 0x6000, 1, seq_len, 0, None, cs, logits, mode,
                               None, None, stream=0)

    _expect(lambda: call(mode=7), q3.QWEN3_EINVAL, "logits_mode")
    _expect(lambda: call(logits=0), q3.QWEN3_EINVAL, "logits")
    _expect(lambda: call(seq_len=200), q3.QWEN3_ERANGE, "capacity")
    _expect(lambda: call(cs=[caches[0], q3.make_kv_layer(0x10000, 0x20000, 192, regions=64)]),
            q3.QWEN3_EINVAL, "capacity")
    _expect(lambda: call(cs=[caches[0], q3.make_kv_layer(0x10000, 0x20000, 128, regions=4)]),
            q3.QWEN3_EINVAL, "regions")
    _expect(lambda: call(), q3.QWEN3_EWORKSPACE, "workspace")


def test_routed_stack_multi_token_and_generation_reject_bad_arguments():
    # validation happens on the host before anything is enqueued (no GPU needed)
    cfg = dict(recipes.QWEN3_0P6B, num_hidden_layers=2, num_experts=2, num_experts_per_tok=1,
               moe_intermediate_size=3072, norm_topk_prob=0, decoder_sparse_step=1,
               router_weights_bf16=1)
    full = _fake_layer()
    no_router = dict(full, router=0)
    caches = [q3.make_kv_layer(0x10000, 0x20000, 128, regions=64)] * 2

    def stack(c=cfg, layers=(full, full), seq_len=16, pos=None):
        mw, keep = q3.make_model_weights(0x7000, 0x8000, list(layers))
        q3.qwen3_stack_forward(c, mw, 0x3000, 0x6000, 1, seq_len, 0, pos, caches, 0x9000,
                               q3.QWEN3_LOGITS_ALL, None, None, stream=0)

    _expect(lambda: stack(layers=(full, no_router)), q3.QWEN3_EINVAL, "router")
    _expect(lambda: stack(c=dict(cfg, decoder_sparse_step=-1)), q3.QWEN3_EINVAL,
            "decoder_sparse_step")
    _expect(lambda: stack(c=dict(cfg, router_weights_bf16=2)), q3.QWEN3_EINVAL,
            "router_weights_bf16")
    # the routed layers need no dense FFN weights; a dense stack needs them
    dense_only = dict(cfg, num_experts=0)
    _expect(lambda: stack(c=dense_only, layers=(dict(full, gate_proj=0), full)),
            q3.QWEN3_EINVAL, "gate_proj")
    _expect(lambda: stack(layers=(dict(full, gate_proj=0), full)), q3.QWEN3_EWORKSPACE,
            "workspace")
    # decode of several tokens per sequence: seq_len must fit the cache
    _expect(lambda: stack(seq_len=200, pos=0x4000), q3.QWEN3_ERANGE, "capacity")
    _expect(lambda: stack(seq_len=8, pos=0x4000), q3.QWEN3_EWORKSPACE, "workspace")

    def gen(temperature=0.5, top_p=0.9, uniforms=0x5000, n_new=4, c=cfg):
        mw, keep = q3.make_model_weights(0x7000, 0x8000, [full, full])
        q3.qwen3_generate(c, mw, 0x3000, 0x6000, 1, 16, n_new, caches, 0x9000, None,
                          temperature=temperature, top_p=top_p, uniforms=uniforms, stream=0)

    _expect(lambda: gen(temperature=-1.0), q3.QWEN3_EINVAL, "temperature")
    _expect(lambda: gen(top_p=1.5), q3.QWEN3_EINVAL, "top_p")
    _expect(lambda: gen(uniforms=None), q3.QWEN3_EINVAL, "uniforms")
    _expect(lambda: gen(n_new=200), q3.QWEN3_ERANGE, "capacity")
    _expect(lambda: gen(c=dict(cfg, vocab_size=300000)), q3.QWEN3_EINVAL, "vocab_size")


def test_block_decode_static_rejects_calls_beyond_its_scratch():
    # the allocation-free entry validates like qwen3_block_decode and refuses a call whose
    # scratch need exceeds the static buffer before touching the device
    with open(os.path.join(ROOT, "include", "qwen3.h")) as f:
        m = re.search(r"#define QWEN3_STATIC_SCRATCH_BYTES \((\d+)u << (\d+)\)", f.read())
    assert m and int(m.group(1)) << int(m.group(2)) == q3.QWEN3_STATIC_SCRATCH_BYTES
    cfg = dict(recipes.QWEN3_0P6B)
    lw = _fake_layer()

    def call(batch, cache):
        q3.qwen3_block_decode_static(cfg, lw, 0x3000, 0x4000, 0x5000, batch, 0x6000, cache,
                                     stream=0)

    big = 4096
    assert q3.qwen3_workspace_bytes(cfg, q3.QWEN3_OP_BLOCK_DECODE, big) > \
        q3.QWEN3_STATIC_SCRATCH_BYTES
    _expect(lambda: call(big, q3.make_kv_layer(0x10000, 0x20000, 128, regions=big * 8)),
            q3.QWEN3_EWORKSPACE, "static scratch")
    _expect(lambda: call(2, q3.make_kv_layer(0x10000, 0x20000, 128, regions=8)),
            q3.QWEN3_EINVAL, "regions")
    _expect(lambda: call(1, q3.make_kv_layer(0x10000, 0x20000, 100, regions=8)),
            q3.QWEN3_EINVAL, "capacity")
