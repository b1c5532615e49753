"""GPU check of the library's stated numeric contract for its fp16 intermediates.

Activations passed between the kernels (normalised rows, q/k/v projections, attention
output, SwiGLU output) are fp16.  A value whose magnitude rounds past fp16's largest finite
value (65504) becomes an infinity there, and the output rows computed from it are
non-finite; rows that stay inside the range are unaffected.  This test drives one token's
SwiGLU activation far past the range (its input row is constant and one gate/up column pair
has large weights) and checks exactly that outcome on the tiled and the decode-size paths.
"""
import numpy as np
import pytest

import decoder_only_forward_amd as q3
import oracle
import synth
from synth import recipes
from q3_testutil import bf16_host, f64, layer_to_dev, log, new_cache, parity, small_cfg, to_dev_bf16

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("S", [300, 40])
def test_swiglu_activation_beyond_fp16_range_gives_nonfinite_row_only(gpu, S):
    import torch
    cfg = small_cfg()
    H, nkv = cfg["hidden_size"], cfg["num_key_value_heads"]
    seed, hot = 21, 17
    log(f"case numerics/fp16_range S={S}: row {hot} constant, gate/up row 0 = 2.0, down column 0 = 0")
    layer = recipes.layer_host(seed, cfg, 0)
    layer["gate"] = layer["gate"].copy()
    layer["up"] = layer["up"].copy()
    layer["gate"][0, :] = synth.f32_to_bf16(np.float32(2.0))
    layer["up"][0, :] = synth.f32_to_bf16(np.float32(2.0))
    # the down projection ignores that activation column, so the in-range rows keep their
    # usual magnitudes; the hot row's infinity still reaches every output (inf * 0 is NaN)
    layer["down"] = layer["down"].copy()
    layer["down"][:, 0] = 0
    x = synth.normal_bf16(seed, recipes.activations_name(), (1, S, H)).copy()
    x[0, hot, :] = synth.f32_to_bf16(np.float32(1.0))
    xf = f64(x[0])
    # the hot row's gate and up sums are about 2 * H = 512: silu(g) * u is near 2.6e5, past
    # fp16's range; every other row stays far inside it (checked on the oracle's side below)
    ref, _, _ = oracle.block(cfg, layer, xf)
    n = oracle.rmsnorm_rows(xf, layer["in_norm"], cfg["rms_norm_eps"])
    assert abs(n[hot].sum() * 2.0) > 400
    rope = torch.empty(2 * cfg["max_position_embeddings"] * 64, dtype=torch.float32, device=gpu)
    q3.qwen3_rope_table_init(cfg, rope)
    cap = ((S + 63) // 64) * 64
    k, vt = new_cache(1, nkv, cap, gpu)
    xd = to_dev_bf16(x, gpu)
    out = torch.empty_like(xd)
    ws = torch.empty(q3.qwen3_workspace_bytes(cfg, q3.QWEN3_OP_BLOCK_PREFILL, 1, S),
                     dtype=torch.uint8, device=gpu)
    q3.qwen3_block_prefill(cfg, layer_to_dev(layer, gpu), rope, xd, out, 1, S, 0,
                           q3.make_kv_layer(k, vt, cap), ws)
    torch.cuda.synchronize()
    got = synth.bf16_to_f32(bf16_host(out[0])).astype(np.float64)
    assert not np.isfinite(got[hot]).any(), "the out-of-range row must come out non-finite"
    rest = np.arange(S) != hot
    parity(got[rest], ref[rest], f"x_out of the {S - 1} in-range rows")
