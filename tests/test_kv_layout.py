"""The tiled KV-cache layout helpers of the Python binding against the element offsets the
C header states for K(b, h, pos, d) and V(b, h, pos, d) (CPU only)."""
import numpy as np
import torch

import decoder_only_forward_amd as q3


def _k_off(b, h, pos, d, nkv, cap):
    tile = (b * nkv + h) * (cap // 32) + pos // 32
    return (tile * 4 + d // 32) * 1024 + (pos % 32) * 32 + d % 32


def _v_off(b, h, pos, d, nkv, cap):
    return (((b * nkv + h) * (cap // 32) + pos // 32) * 128 + d) * 32 + pos % 32


def test_tiled_cache_offsets_and_round_trip():
    B, nkv, cap = 2, 3, 128
    g = torch.Generator().manual_seed(0)
    k_log = torch.randn((B, nkv, cap, 128), generator=g).to(torch.bfloat16)
    v_log = torch.randn((B, nkv, cap, 128), generator=g).to(torch.bfloat16)
    k, vt = q3.kv_cache_from_logical(k_log, v_log)
    assert k.shape == (B, nkv, cap // 32, 4, 32, 32) and vt.shape == (B, nkv, cap // 32, 128, 32)
    kf = k.reshape(-1).view(torch.int16).numpy()
    vf = vt.reshape(-1).view(torch.int16).numpy()
    kl = k_log.view(torch.int16).numpy()
    vl = v_log.view(torch.int16).numpy()
    rng = np.random.default_rng(1)
    for _ in range(2000):
        b, h = int(rng.integers(B)), int(rng.integers(nkv))
        pos, d = int(rng.integers(cap)), int(rng.integers(128))
        assert kf[_k_off(b, h, pos, d, nkv, cap)] == kl[b, h, pos, d]
        assert vf[_v_off(b, h, pos, d, nkv, cap)] == vl[b, h, pos, d]
    k2, v2 = q3.kv_cache_to_logical(k, vt)
    assert torch.equal(k2, k_log) and torch.equal(v2, v_log)
    # in-place variant writes the same bytes into a preallocated cache
    ko, vo = q3.kv_cache_empty(B, nkv, cap, "cpu")
    q3.k_cache_from_logical(k_log, out=ko)
    q3.v_cache_from_logical(v_log, out=vo)
    assert torch.equal(ko, k) and torch.equal(vo, vt)


def test_tiled_cache_rejects_bad_capacity():
    import pytest
    with pytest.raises(ValueError):
        q3.kv_cache_empty(1, 1, 96, "cpu")


def test_make_kv_layer_checks_region_sizes():
    import pytest
    k, vt = q3.kv_cache_empty(2, 1, 64, "cpu")
    q3.make_kv_layer(k, vt, 64)  # whole regions: accepted
    with pytest.raises(ValueError):
        q3.make_kv_layer(k, vt, 192)  # 2 x 64 positions is not a multiple of 192


def test_make_kv_layer_records_regions():
    import pytest
    k, vt = q3.kv_cache_empty(3, 2, 64, "cpu")
    assert q3.make_kv_layer(k, vt, 64).regions == 6
    assert q3.make_kv_layer(k, vt, 64, regions=4).regions == 4
    with pytest.raises(ValueError):
        q3.make_kv_layer(k, vt, 64, regions=7)  # more than the tensors hold
    with pytest.raises(ValueError):
        q3.make_kv_layer(0x10000, 0x20000, 64)  # raw pointers must state it


def test_kv_pack_rejects_bad_arguments():
    import pytest
    from synth import recipes
    cfg = dict(recipes.QWEN3_0P6B)  # 8 kv heads
    cache = q3.make_kv_layer(0x10000, 0x20000, 128, regions=16)

    def expect(fn, code, word):
        with pytest.raises(RuntimeError) as e:
            fn()
        msg = str(e.value)
        assert q3.lib().qwen3_status_string(code).decode() in msg and word in msg, msg

    expect(lambda: q3.qwen3_kv_pack(cfg, 0x4000, 0x5000, 2, 129, cache, stream=0),
           q3.QWEN3_ERANGE, "len")
    expect(lambda: q3.qwen3_kv_unpack(cfg, cache, 2, -1, 0x4000, 0x5000, stream=0),
           q3.QWEN3_ERANGE, "len")
    expect(lambda: q3.qwen3_kv_pack(cfg, 0x4000, 0x5000, 3, 64, cache, stream=0),
           q3.QWEN3_EINVAL, "regions")
    expect(lambda: q3.qwen3_kv_pack(cfg, 0x4008, 0x5000, 2, 64, cache, stream=0),
           q3.QWEN3_EINVAL, "aligned")
    expect(lambda: q3.qwen3_kv_unpack(cfg, None, 2, 64, 0x4000, 0x5000, stream=0),
           q3.QWEN3_EINVAL, "cache")
