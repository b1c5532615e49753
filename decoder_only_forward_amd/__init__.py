"""Python binding of libqwen3 (MI355X / gfx950 Qwen3 decoder forward).

Argument marshalling only: every step of the forward pass runs in the library's HIP
kernels.  The functions carry the C entry points' names and signatures
(``include/qwen3.h``); tensors are torch tensors on the GPU (torch supplies device
memory and the current stream), configs are dicts with Hugging Face field names.
A nonzero status raises ``RuntimeError`` with the library's message.  There is no
fallback: if ``libqwen3.so`` cannot be loaded, importing the binding's functions fails.
"""
import ctypes
import os

from . import build as _build

LIB_PATH = _build.SO

QWEN3_OK = 0
QWEN3_EINVAL = -1
QWEN3_EUNSUPPORTED = -2
QWEN3_ERANGE = -3
QWEN3_EWORKSPACE = -4
QWEN3_EHIP = -5

QWEN3_OP_BLOCK_PREFILL = 1
QWEN3_OP_BLOCK_DECODE = 2
QWEN3_OP_MOE_FFN = 3
QWEN3_OP_STACK_PREFILL = 4
QWEN3_OP_STACK_DECODE = 5
QWEN3_OP_GENERATE = 6

QWEN3_LOGITS_NONE = 0
QWEN3_LOGITS_ALL = 1
QWEN3_LOGITS_LAST = 2

EXPORTS = ("qwen3_workspace_bytes", "qwen3_rope_table_init", "qwen3_block_prefill",
           "qwen3_block_decode", "qwen3_block_decode_static", "qwen3_moe_ffn",
           "qwen3_stack_forward", "qwen3_generate", "qwen3_kv_pack", "qwen3_kv_unpack",
           "qwen3_status_string", "qwen3_last_error", "qwen3_profile_begin",
           "qwen3_profile_end")

# qwen3_block_decode_static's device scratch per GPU (QWEN3_STATIC_SCRATCH_BYTES)
QWEN3_STATIC_SCRATCH_BYTES = 16 << 20


class Config(ctypes.Structure):
    _fields_ = [("hidden_size", ctypes.c_int32), ("num_attention_heads", ctypes.c_int32),
                ("num_key_value_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("intermediate_size", ctypes.c_int32), ("num_hidden_layers", ctypes.c_int32),
                ("vocab_size", ctypes.c_int32), ("max_position_embeddings", ctypes.c_int32),
                ("rms_norm_eps", ctypes.c_float), ("rope_theta", ctypes.c_float),
                ("qk_norm", ctypes.c_int32), ("tie_word_embeddings", ctypes.c_int32),
                ("num_experts", ctypes.c_int32), ("num_experts_per_tok", ctypes.c_int32),
                ("moe_intermediate_size", ctypes.c_int32), ("norm_topk_prob", ctypes.c_int32),
                ("rope_interleaved", ctypes.c_int32), ("decoder_sparse_step", ctypes.c_int32),
                ("router_weights_bf16", ctypes.c_int32)]


LAYER_FIELDS = ("input_layernorm", "q_proj", "k_proj", "v_proj", "q_norm", "k_norm", "o_proj",
                "post_attention_layernorm", "gate_proj", "up_proj", "down_proj", "router",
                "experts_gate_up_proj", "experts_down_proj")


class LayerWeights(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in LAYER_FIELDS]


class ModelWeights(ctypes.Structure):
    _fields_ = [("embed_tokens", ctypes.c_void_p), ("norm", ctypes.c_void_p),
                ("lm_head", ctypes.c_void_p), ("layers", ctypes.POINTER(LayerWeights))]


class MoeWeights(ctypes.Structure):
    _fields_ = [("router", ctypes.c_void_p), ("gate_up_proj", ctypes.c_void_p),
                ("down_proj", ctypes.c_void_p)]


class KVLayer(ctypes.Structure):
    _fields_ = [("k", ctypes.c_void_p), ("vt", ctypes.c_void_p), ("capacity", ctypes.c_int32),
                ("regions", ctypes.c_int32)]


_lib = None


def lib():
    """Load libqwen3.so (building it in-tree first if it was never built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            _build.build()
        L = ctypes.CDLL(LIB_PATH)
        vp, i32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
        L.qwen3_workspace_bytes.restype = sz
        L.qwen3_workspace_bytes.argtypes = [vp, i32, i32, i32]
        L.qwen3_rope_table_init.restype = ctypes.c_int
        L.qwen3_rope_table_init.argtypes = [vp, vp, vp]
        L.qwen3_block_prefill.restype = ctypes.c_int
        L.qwen3_block_prefill.argtypes = [vp, vp, vp, vp, vp, i32, i32, i32, vp, vp, sz, vp]
        L.qwen3_block_decode.restype = ctypes.c_int
        L.qwen3_block_decode.argtypes = [vp, vp, vp, vp, vp, i32, vp, vp, vp, sz, vp]
        L.qwen3_block_decode_static.restype = ctypes.c_int
        L.qwen3_block_decode_static.argtypes = [vp, vp, vp, vp, vp, i32, vp, vp, vp]
        L.qwen3_moe_ffn.restype = ctypes.c_int
        L.qwen3_moe_ffn.argtypes = [vp, vp, vp, vp, i32, vp, vp, vp, vp, vp, vp, vp, sz, vp]
        L.qwen3_stack_forward.restype = ctypes.c_int
        L.qwen3_stack_forward.argtypes = [vp, vp, vp, vp, i32, i32, i32, vp, vp, vp, i32, vp, vp,
                                          sz, vp]
        L.qwen3_generate.restype = ctypes.c_int
        L.qwen3_generate.argtypes = [vp, vp, vp, vp, i32, i32, i32, vp, ctypes.c_float,
                                     ctypes.c_float, vp, vp, vp, sz, vp]
        L.qwen3_kv_pack.restype = ctypes.c_int
        L.qwen3_kv_pack.argtypes = [vp, vp, vp, i32, i32, vp, vp]
        L.qwen3_kv_unpack.restype = ctypes.c_int
        L.qwen3_kv_unpack.argtypes = [vp, vp, i32, i32, vp, vp, vp]
        L.qwen3_status_string.restype = ctypes.c_char_p
        L.qwen3_status_string.argtypes = [ctypes.c_int]
        L.qwen3_last_error.restype = ctypes.c_char_p
        L.qwen3_last_error.argtypes = []
        L.qwen3_profile_begin.restype = ctypes.c_int
        L.qwen3_profile_begin.argtypes = [ctypes.c_char_p, i32]
        L.qwen3_profile_end.restype = ctypes.c_int
        L.qwen3_profile_end.argtypes = [vp, vp]
        _lib = L
    return _lib


# ------------------------------------------------------------------ marshalling helpers

def make_config(d):
    """qwen3_config from a dict with Hugging Face config names."""
    c = Config()
    for name, _ in Config._fields_:
        if name in d:
            setattr(c, name, d[name])
    if "qk_norm" not in d:
        c.qk_norm = 1
    if "tie_word_embeddings" not in d:
        c.tie_word_embeddings = 1
    if "norm_topk_prob" not in d:
        c.norm_topk_prob = 1
    return c


def _ptr(t):
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def make_layer_weights(w):
    """qwen3_layer_weights from a dict of device tensors keyed by LAYER_FIELDS."""
    return LayerWeights(**{k: _ptr(w.get(k)) for k in LAYER_FIELDS})


def make_kv_layer(k, vt, capacity, regions=None):
    """qwen3_kv_layer for one layer's tiled K and V caches (see kv_cache_empty).  For
    tensors the region count (sequence x kv head regions of capacity x 128 elements) is
    taken from their sizes; raw pointers must state it."""
    counts = []
    for name, t in (("k", k), ("vt", vt)):
        n = getattr(t, "numel", None)
        if n is None:
            continue
        if n() == 0 or n() % (int(capacity) * 128):
            raise ValueError(f"{name}: {n()} elements is not a whole number of "
                             f"capacity x 128 = {int(capacity) * 128} regions")
        counts.append(n() // (int(capacity) * 128))
    if regions is None:
        if len(counts) != 2:
            raise ValueError("regions must be given for raw cache pointers")
        regions = min(counts)
    elif counts and regions > min(counts):
        raise ValueError(f"regions={regions} exceeds what the tensors hold ({min(counts)})")
    return KVLayer(_ptr(k), _ptr(vt), int(capacity), int(regions))


# ---- KV-cache layout (data movement only: conversions for setting up or inspecting a cache)
# Per layer and (sequence, kv head), positions are grouped in tiles of KV_TILE:
#   K: [cap / 32][4][32][32]   tile, 32-dim chunk, position in the tile, dim in the chunk
#   V: [cap / 32][128][32]     tile, dim, position in the tile
KV_TILE = 32


def kv_cache_empty(batch, nkv, capacity, device, head_dim=128):
    """Uninitialised K and V caches of one layer in the library's tiled layout."""
    import torch
    if capacity % 64 or head_dim != 128:
        raise ValueError("capacity must be a multiple of 64 and head_dim 128")
    nt = capacity // KV_TILE
    k = torch.empty((batch, nkv, nt, 4, KV_TILE, 32), dtype=torch.bfloat16, device=device)
    vt = torch.empty((batch, nkv, nt, head_dim, KV_TILE), dtype=torch.bfloat16, device=device)
    return k, vt


def k_cache_from_logical(k_log, out=None):
    """Tiled K cache from a logical [B, nkv, cap, 128] tensor (a copy, into ``out`` if given)."""
    B, nkv, cap, _ = k_log.shape
    nt = cap // KV_TILE
    src = k_log.reshape(B, nkv, nt, KV_TILE, 4, 32).permute(0, 1, 2, 4, 3, 5)
    if out is None:
        return src.contiguous()
    return out.view(B, nkv, nt, 4, KV_TILE, 32).copy_(src)


def v_cache_from_logical(v_log, out=None):
    """Tiled V cache from a logical [B, nkv, cap, 128] tensor (a copy, into ``out`` if given)."""
    B, nkv, cap, hd = v_log.shape
    nt = cap // KV_TILE
    src = v_log.reshape(B, nkv, nt, KV_TILE, hd).permute(0, 1, 2, 4, 3)
    if out is None:
        return src.contiguous()
    return out.view(B, nkv, nt, hd, KV_TILE).copy_(src)


def k_cache_to_logical(k):
    """Logical [B, nkv, cap, 128] view-copy of a tiled K cache."""
    B, nkv, nt = k.shape[:3]
    return (k.reshape(B, nkv, nt, 4, KV_TILE, 32).permute(0, 1, 2, 4, 3, 5)
            .reshape(B, nkv, nt * KV_TILE, 128))


def v_cache_to_logical(vt):
    """Logical [B, nkv, cap, 128] view-copy of a tiled V cache."""
    B, nkv, nt = vt.shape[:3]
    return (vt.reshape(B, nkv, nt, 128, KV_TILE).permute(0, 1, 2, 4, 3)
            .reshape(B, nkv, nt * KV_TILE, 128))


def kv_cache_from_logical(k_log, v_log):
    return k_cache_from_logical(k_log), v_cache_from_logical(v_log)


def kv_cache_to_logical(k, vt):
    return k_cache_to_logical(k), v_cache_to_logical(vt)


def make_model_weights(embed_tokens, norm, layers, lm_head=None):
    """layers: list of dicts (or LayerWeights).  Returns (ModelWeights, keepalive)."""
    structs = [x if isinstance(x, LayerWeights) else make_layer_weights(x) for x in layers]
    arr = (LayerWeights * len(structs))(*structs)
    m = ModelWeights(_ptr(embed_tokens), _ptr(norm), _ptr(lm_head),
                     ctypes.cast(arr, ctypes.POINTER(LayerWeights)))
    return m, arr


def make_moe_weights(router, gate_up_proj, down_proj):
    return MoeWeights(_ptr(router), _ptr(gate_up_proj), _ptr(down_proj))


def _stream(stream):
    if stream is not None:
        return stream if isinstance(stream, int) else stream.cuda_stream
    import torch
    return torch.cuda.current_stream().cuda_stream


def _cfg(cfg):
    return cfg if isinstance(cfg, Config) else make_config(cfg)


def _check(rc):
    if rc != QWEN3_OK:
        L = lib()
        raise RuntimeError("libqwen3: %s: %s" % (L.qwen3_status_string(rc).decode(),
                                                 L.qwen3_last_error().decode()))


def _ws(workspace):
    if workspace is None:
        return None, 0
    return _ptr(workspace), workspace.numel() * workspace.element_size()


def _byref(x):
    return ctypes.byref(x) if x is not None else None


# ------------------------------------------------------------------ entry points

def qwen3_workspace_bytes(cfg, op, batch, seq_len=1):
    return int(lib().qwen3_workspace_bytes(ctypes.byref(_cfg(cfg)), op, batch, seq_len))


def qwen3_rope_table_init(cfg, rope, stream=None):
    _check(lib().qwen3_rope_table_init(ctypes.byref(_cfg(cfg)), _ptr(rope), _stream(stream)))


def qwen3_block_prefill(cfg, w, rope, x_in, x_out, batch, seq_len, pos0, cache, workspace,
                        stream=None):
    lw = w if isinstance(w, LayerWeights) else make_layer_weights(w)
    wp, wb = _ws(workspace)
    _check(lib().qwen3_block_prefill(ctypes.byref(_cfg(cfg)), ctypes.byref(lw), _ptr(rope),
                                     _ptr(x_in), _ptr(x_out), batch, seq_len, pos0,
                                     _byref(cache), wp, wb, _stream(stream)))


def qwen3_block_decode(cfg, w, rope, x_in, x_out, batch, pos, cache, workspace, stream=None):
    lw = w if isinstance(w, LayerWeights) else make_layer_weights(w)
    wp, wb = _ws(workspace)
    _check(lib().qwen3_block_decode(ctypes.byref(_cfg(cfg)), ctypes.byref(lw), _ptr(rope),
                                    _ptr(x_in), _ptr(x_out), batch, _ptr(pos), _byref(cache),
                                    wp, wb, _stream(stream)))


def qwen3_block_decode_static(cfg, w, rope, x_in, x_out, batch, pos, cache, stream=None):
    """qwen3_block_decode with the library's static device scratch instead of a workspace
    (no allocation; calls that may overlap on one GPU must be serialised by the caller)."""
    lw = w if isinstance(w, LayerWeights) else make_layer_weights(w)
    _check(lib().qwen3_block_decode_static(ctypes.byref(_cfg(cfg)), ctypes.byref(lw), _ptr(rope),
                                           _ptr(x_in), _ptr(x_out), batch, _ptr(pos),
                                           _byref(cache), _stream(stream)))


def qwen3_moe_ffn(cfg, w, x, y, n_tokens, router_logits=None, topk_idx=None, topk_w=None,
                  expert_offsets=None, perm_token=None, inv_row=None, workspace=None,
                  stream=None):
    wp, wb = _ws(workspace)
    _check(lib().qwen3_moe_ffn(ctypes.byref(_cfg(cfg)), ctypes.byref(w), _ptr(x), _ptr(y),
                               n_tokens, _ptr(router_logits), _ptr(topk_idx), _ptr(topk_w),
                               _ptr(expert_offsets), _ptr(perm_token), _ptr(inv_row), wp, wb,
                               _stream(stream)))


def qwen3_stack_forward(cfg, w, rope, ids, batch, seq_len, pos0, pos, caches, logits,
                        logits_mode, next_ids, workspace, stream=None):
    """caches: list of KVLayer (one per layer)."""
    arr = (KVLayer * len(caches))(*caches)
    wp, wb = _ws(workspace)
    _check(lib().qwen3_stack_forward(ctypes.byref(_cfg(cfg)), ctypes.byref(w), _ptr(rope),
                                     _ptr(ids), batch, seq_len, pos0, _ptr(pos), arr,
                                     _ptr(logits), logits_mode, _ptr(next_ids), wp, wb,
                                     _stream(stream)))


def qwen3_generate(cfg, w, rope, prompt_ids, batch, prompt_len, n_new, caches, out_ids,
                   workspace, temperature=0.0, top_p=1.0, uniforms=None, stream=None):
    """caches: list of KVLayer (one per layer); out_ids: device int32 [batch][n_new];
    uniforms: device float32 [n_new][batch] when temperature > 0."""
    arr = (KVLayer * len(caches))(*caches)
    wp, wb = _ws(workspace)
    _check(lib().qwen3_generate(ctypes.byref(_cfg(cfg)), ctypes.byref(w), _ptr(rope),
                                _ptr(prompt_ids), batch, prompt_len, n_new, arr,
                                float(temperature), float(top_p), _ptr(uniforms),
                                _ptr(out_ids), wp, wb, _stream(stream)))


def qwen3_kv_pack(cfg, k_plain, v_plain, batch, length, cache, stream=None):
    _check(lib().qwen3_kv_pack(ctypes.byref(_cfg(cfg)), _ptr(k_plain), _ptr(v_plain), batch,
                               length, _byref(cache), _stream(stream)))


def qwen3_kv_unpack(cfg, cache, batch, length, k_plain, v_plain, stream=None):
    _check(lib().qwen3_kv_unpack(ctypes.byref(_cfg(cfg)), _byref(cache), batch, length,
                                 _ptr(k_plain), _ptr(v_plain), _stream(stream)))


def qwen3_profile_begin(tag, max_launches):
    _check(lib().qwen3_profile_begin(tag.encode(), max_launches))


def qwen3_profile_end():
    """Returns (total_ms, launches); synchronise the stream first."""
    ms = ctypes.c_float()
    n = ctypes.c_int32()
    _check(lib().qwen3_profile_end(ctypes.byref(ms), ctypes.byref(n)))
    return float(ms.value), int(n.value)
