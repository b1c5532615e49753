"""GPU check of qwen3_kv_pack / qwen3_kv_unpack: plain [B][nkv][len][128] bf16 K / V into the
tiled cache at the element offsets the C header states, positions past len left untouched,
and back again bit for bit."""
import numpy as np
import pytest

import decoder_only_forward_amd as q3
from synth import recipes
from q3_testutil import log

pytestmark = pytest.mark.gpu


def _k_off(b, h, pos, d, nkv, cap):
    tile = (b * nkv + h) * (cap // 32) + pos // 32
    return (tile * 4 + d // 32) * 1024 + (pos % 32) * 32 + d % 32


def _v_off(b, h, pos, d, nkv, cap):
    return (((b * nkv + h) * (cap // 32) + pos // 32) * 128 + d) * 32 + pos % 32


@pytest.mark.parametrize("B,length,cap", [(2, 100, 128), (3, 64, 64), (1, 1, 192), (2, 0, 64)])
def test_kv_pack_unpack_follow_the_header_offsets(gpu, B, length, cap):
    import torch
    cfg = dict(recipes.QWEN3_0P6B, num_key_value_heads=4)
    nkv = cfg["num_key_value_heads"]
    log(f"case kv pack/unpack: B={B} len={length} cap={cap}")
    rng = np.random.default_rng(B * 1000 + length)
    kp = rng.integers(0, 1 << 16, size=(B, nkv, length, 128), dtype=np.uint16)
    vp = rng.integers(0, 1 << 16, size=(B, nkv, length, 128), dtype=np.uint16)
    sentinel = 0x7F7F
    k, vt = q3.kv_cache_empty(B, nkv, cap, gpu)
    k.view(torch.int16).fill_(sentinel)
    vt.view(torch.int16).fill_(sentinel)
    cache = q3.make_kv_layer(k, vt, cap)
    kd = torch.from_numpy(kp.view(np.int16)).to(gpu)
    vd = torch.from_numpy(vp.view(np.int16)).to(gpu)
    q3.qwen3_kv_pack(cfg, kd, vd, B, length, cache)
    torch.cuda.synchronize()
    kf = k.reshape(-1).view(torch.int16).cpu().numpy().view(np.uint16)
    vf = vt.reshape(-1).view(torch.int16).cpu().numpy().view(np.uint16)
    want_k = np.full(kf.shape, sentinel, np.uint16)
    want_v = np.full(vf.shape, sentinel, np.uint16)
    b, h, p, d = np.meshgrid(np.arange(B), np.arange(nkv), np.arange(length), np.arange(128),
                             indexing="ij")
    want_k[_k_off(b, h, p, d, nkv, cap)] = kp
    want_v[_v_off(b, h, p, d, nkv, cap)] = vp
    np.testing.assert_array_equal(kf, want_k)
    np.testing.assert_array_equal(vf, want_v)
    k2 = torch.zeros_like(kd)
    v2 = torch.zeros_like(vd)
    q3.qwen3_kv_unpack(cfg, cache, B, length, k2, v2)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(k2.cpu().numpy().view(np.uint16), kp)
    np.testing.assert_array_equal(v2.cpu().numpy().view(np.uint16), vp)
