"""CPU oracle for the Qwen3 decoder forward -- TEST INFRASTRUCTURE ONLY.

A plain, slow, fp64 C++ implementation (``qwen3_oracle.cpp``) of what the GPU
library computes, written from the pages' definitions (see the header of
``qwen3_oracle.h`` for the sources).  Only ``tests/``, ``__graft_entry__.smoke``
and the CPU-baseline leg of ``bench.py`` may import this package.  It shares no
code with the GPU path; inputs come from the ``synth`` generator.

bf16 tensors are numpy ``uint16`` arrays holding the bf16 bits.
"""
import ctypes
import os

import numpy as np

from . import build as _build

_lib = None

_D = ctypes.POINTER(ctypes.c_double)


class OracleCfg(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in (
        "hidden", "n_heads", "n_kv_heads", "head_dim", "inter", "n_layers", "vocab", "max_pos")] + [
        ("eps", ctypes.c_double), ("theta", ctypes.c_double), ("qk_norm", ctypes.c_int32),
        ("n_experts", ctypes.c_int32), ("top_k", ctypes.c_int32), ("moe_inter", ctypes.c_int32),
        ("norm_topk", ctypes.c_int32), ("rope_interleaved", ctypes.c_int32),
        ("sparse_step", ctypes.c_int32), ("router_bf16", ctypes.c_int32)]


LAYER_FIELDS = ("in_norm", "q", "k", "v", "q_norm", "k_norm", "o", "post_norm", "gate", "up",
                "down")


MOE_LAYER_FIELDS = ("router", "experts_gate_up", "experts_down")


class OracleLayer(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in LAYER_FIELDS + MOE_LAYER_FIELDS]


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_build.SO):
            _build.build()
        L = ctypes.CDLL(_build.SO)
        L.oracle_get_threads.restype = ctypes.c_int
        _lib = L
    return _lib


def set_threads(n):
    lib().oracle_set_threads(int(n))


def get_threads():
    return lib().oracle_get_threads()


def make_cfg(c):
    """``c``: dict with HF config names (hidden_size, num_attention_heads, ...)."""
    return OracleCfg(
        hidden=c.get("hidden_size", 0), n_heads=c.get("num_attention_heads", 0),
        n_kv_heads=c.get("num_key_value_heads", 0), head_dim=c.get("head_dim", 0),
        inter=c.get("intermediate_size", 0), n_layers=c.get("num_hidden_layers", 0),
        vocab=c.get("vocab_size", 0), max_pos=c.get("max_position_embeddings", 0),
        eps=c.get("rms_norm_eps", 1e-6), theta=c.get("rope_theta", 1e6),
        qk_norm=int(c.get("qk_norm", 1)), n_experts=c.get("num_experts", 0),
        top_k=c.get("num_experts_per_tok", 0), moe_inter=c.get("moe_intermediate_size", 0),
        norm_topk=int(c.get("norm_topk_prob", 1)),
        rope_interleaved=int(c.get("rope_interleaved", 0)),
        sparse_step=int(c.get("decoder_sparse_step", 0)),
        router_bf16=int(c.get("router_weights_bf16", 0)))


def _p(a):
    return ctypes.c_void_p(a.ctypes.data) if a is not None else ctypes.c_void_p(0)


def _f64(a):
    return np.ascontiguousarray(a, dtype=np.float64)


def _u16(a):
    return np.ascontiguousarray(a, dtype=np.uint16)


def make_layer(w):
    """``w``: dict with keys LAYER_FIELDS (and, for routed layers, MOE_LAYER_FIELDS) ->
    uint16 arrays.  Returns (struct, keepalive)."""
    keep = {k: _u16(w[k]) for k in LAYER_FIELDS + MOE_LAYER_FIELDS if w.get(k) is not None}
    return OracleLayer(**{k: keep[k].ctypes.data for k in keep}), keep


def rmsnorm_rows(x, w, eps):
    x = _f64(x)
    n = x.shape[-1]
    y = np.empty_like(x)
    w = _u16(w)
    lib().oracle_rmsnorm_rows(_p(x), ctypes.c_int64(x.size // n), n, _p(w), ctypes.c_double(eps),
                              _p(y))
    return y


def rope(x, pos, theta, interleaved=False):
    x = _f64(x)
    hd = x.shape[-1]
    pos = np.ascontiguousarray(np.broadcast_to(pos, (x.size // hd,)), dtype=np.int64)
    y = np.empty_like(x)
    lib().oracle_rope(_p(x), ctypes.c_int64(x.size // hd), hd, _p(pos), ctypes.c_double(theta),
                      int(interleaved), _p(y))
    return y


def attention(q, k, v, qpos):
    """q [S, nq, hd]; k, v [L, nkv, hd] (key index = absolute position); qpos [S]."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    S, nq, hd = q.shape
    L, nkv, _ = k.shape
    qpos = np.ascontiguousarray(qpos, dtype=np.int64)
    o = np.empty_like(q)
    lib().oracle_attention(_p(q), _p(k), _p(v), _p(qpos), ctypes.c_int64(S), ctypes.c_int64(L),
                           nq, nkv, hd, _p(o))
    return o


def linear_rows(x, W):
    """y = x W^T for x [T, K] (float) and bf16 weights W [N, K]."""
    x = _f64(x)
    T, K = x.shape
    W = _u16(W)
    N = W.shape[0]
    y = np.empty((T, N), dtype=np.float64)
    lib().oracle_linear_rows(_p(x), ctypes.c_int64(T), ctypes.c_int64(K), _p(W),
                             ctypes.c_int64(N), _p(y))
    return y


def swiglu_ffn(x, gate, up, down):
    x = _f64(x)
    T, H = x.shape
    I = gate.shape[0]
    gate, up, down = _u16(gate), _u16(up), _u16(down)
    y = np.empty((T, H), dtype=np.float64)
    lib().oracle_swiglu_ffn(_p(x), ctypes.c_int64(T), H, I, _p(gate), _p(up), _p(down), _p(y))
    return y


def block(cfg, layer, x, pos0=0, past_k=None, past_v=None, rows=None, routed=False):
    """One decoder block on one sequence.  x [S, H] (float); past_k/v [nkv, pos0, hd].
    routed: the FFN is the layer's routed MoE.
    Returns (x_out [len(rows) or S, H], new_k [nkv, S, hd], new_v)."""
    c = make_cfg(cfg)
    lw, keep = make_layer(layer)
    x = _f64(x)
    S, H = x.shape
    nkv, hd = c.n_kv_heads, c.head_dim
    pk = _f64(past_k) if pos0 > 0 else None
    pv = _f64(past_v) if pos0 > 0 else None
    if rows is not None:
        rows = np.ascontiguousarray(rows, dtype=np.int64)
        nr = len(rows)
    else:
        nr = S
    out = np.empty((nr, H), dtype=np.float64)
    nk = np.empty((nkv, S, hd), dtype=np.float64)
    nv = np.empty((nkv, S, hd), dtype=np.float64)
    lib().oracle_block(ctypes.byref(c), ctypes.byref(lw), _p(x), ctypes.c_int64(S),
                       ctypes.c_int64(pos0), _p(pk), _p(pv), _p(rows), ctypes.c_int64(nr), _p(out),
                       _p(nk), _p(nv), int(routed), ctypes.c_void_p(0))
    return out, nk, nv


def _layers(model):
    structs, keep = [], []
    for lw in model["layers"]:
        s, k = make_layer(lw)
        structs.append(s)
        keep.append(k)
    arr = (OracleLayer * len(structs))(*structs)
    return arr, keep


def _check_ids(ids, cfg):
    """Token ids index the embedding rows: each must lie in [0, vocab_size)."""
    if ids.size and (ids.min() < 0 or ids.max() >= cfg["vocab_size"]):
        raise ValueError(f"token id outside [0, {cfg['vocab_size']})")


def stack_prefill(cfg, model, ids, rows=None, want_kv=False, want_router=False):
    """Whole model on one sequence from position 0.  model: dict(embed, norm, lm_head or None,
    layers=[layer dicts]).  Returns logits [len(rows), V] (and per-layer k, v when asked;
    with want_router also the routed layers' router logits [L, S, E], NaN elsewhere)."""
    c = make_cfg(cfg)
    arr, keep = _layers(model)
    ids = np.ascontiguousarray(ids, dtype=np.int32)
    _check_ids(ids, cfg)
    S = ids.shape[0]
    rows = np.arange(S, dtype=np.int64) if rows is None else np.ascontiguousarray(rows, np.int64)
    embed, norm = _u16(model["embed"]), _u16(model["norm"])
    head = _u16(model["lm_head"]) if model.get("lm_head") is not None else None
    logits = np.empty((len(rows), c.vocab), dtype=np.float64)
    ko = vo = None
    if want_kv:
        ko = np.empty((c.n_layers, c.n_kv_heads, S, c.head_dim), dtype=np.float64)
        vo = np.empty_like(ko)
    ro = np.full((c.n_layers, S, c.n_experts), np.nan) if want_router else None
    lib().oracle_stack_prefill(ctypes.byref(c), _p(embed), _p(norm), _p(head), arr, _p(ids),
                               ctypes.c_int64(S), _p(rows), ctypes.c_int64(len(rows)), _p(logits),
                               _p(ko), _p(vo), _p(ro))
    out = (logits, ko, vo) if want_kv else (logits,)
    if want_router:
        out = out + (ro,)
    return out if len(out) > 1 else out[0]


def stack_decode(cfg, model, token_id, pos, cache_k, cache_v, want_router=False):
    """Decode of one sequence: token_id (an int: one token, or a sequence of n tokens taking
    positions pos .. pos + n - 1, each seeing the cache and the new tokens up to itself).
    cache_k/v: per-layer arrays [nkv, pos, hd], uint16 (bf16 bits) or float64.  Returns
    logits [V] for an int, [n, V] for a sequence (and, with want_router, the routed layers'
    router logits [L, E] or [L, n, E], NaN elsewhere)."""
    c = make_cfg(cfg)
    arr, keep = _layers(model)
    embed, norm = _u16(model["embed"]), _u16(model["norm"])
    head = _u16(model["lm_head"]) if model.get("lm_head") is not None else None
    L = c.n_layers
    single = np.ndim(token_id) == 0
    ids = np.ascontiguousarray(np.atleast_1d(token_id), dtype=np.int32)
    _check_ids(ids, cfg)
    n = ids.shape[0]
    f64 = cache_k[0].dtype == np.float64
    ck = [(_f64(a) if f64 else _u16(a)) for a in cache_k]
    cv = [(_f64(a) if f64 else _u16(a)) for a in cache_v]
    pk = (ctypes.c_void_p * L)(*[a.ctypes.data for a in ck])
    pv = (ctypes.c_void_p * L)(*[a.ctypes.data for a in cv])
    null = ctypes.c_void_p(0)
    logits = np.empty((n, c.vocab), dtype=np.float64)
    ro = np.full((L, n, c.n_experts), np.nan) if want_router else None
    lib().oracle_stack_decode(ctypes.byref(c), _p(embed), _p(norm), _p(head), arr, _p(ids),
                              ctypes.c_int64(n), ctypes.c_int64(pos),
                              null if f64 else pk, null if f64 else pv,
                              pk if f64 else null, pv if f64 else null, _p(logits), _p(ro))
    if single:
        logits = logits[0]
        ro = ro[:, 0] if ro is not None else None
    return (logits, ro) if want_router else logits


def moe_ffn(cfg, router, gate_up, down, x):
    """Routed MoE FFN, token by token.  x [T, H] float.  Returns y [T, H], idx [T, k] int32,
    w [T, k], router logits [T, E]."""
    c = make_cfg(cfg)
    x = _f64(x)
    T, H = x.shape
    router, gate_up, down = _u16(router), _u16(gate_up), _u16(down)
    y = np.empty((T, H), dtype=np.float64)
    idx = np.empty((T, c.top_k), dtype=np.int32)
    w = np.empty((T, c.top_k), dtype=np.float64)
    lg = np.empty((T, c.n_experts), dtype=np.float64)
    lib().oracle_moe_ffn(ctypes.byref(c), _p(router), _p(gate_up), _p(down), _p(x),
                         ctypes.c_int64(T), _p(y), _p(idx), _p(w), _p(lg))
    return y, idx, w, lg


def moe_ffn_at(cfg, gate_up, down, x, idx, w):
    """Routed MoE FFN at a given selection: y[t] = sum_j w[t, j] expert_{idx[t, j]}(x[t]).
    x [T, H] float; idx [T, k] int; w [T, k] float.  Returns y [T, H]."""
    c = make_cfg(cfg)
    x = _f64(x)
    T, H = x.shape
    idx = np.ascontiguousarray(idx, dtype=np.int32)
    w = _f64(w)
    if idx.shape != (T, c.top_k) or w.shape != (T, c.top_k):
        raise ValueError("idx and w must be [T, num_experts_per_tok]")
    if idx.size and (idx.min() < 0 or idx.max() >= c.n_experts):
        raise ValueError("expert index outside [0, num_experts)")
    gate_up, down = _u16(gate_up), _u16(down)
    y = np.empty((T, H), dtype=np.float64)
    lib().oracle_moe_ffn_at(ctypes.byref(c), _p(gate_up), _p(down), _p(x), ctypes.c_int64(T),
                            _p(idx), _p(w), _p(y))
    return y


def topk(logits, k):
    lg = np.ascontiguousarray(logits, dtype=np.float32)
    T, E = lg.shape
    idx = np.empty((T, k), dtype=np.int32)
    lib().oracle_topk(_p(lg), ctypes.c_int64(T), E, k, _p(idx))
    return idx


def route_weights(logits, idx, norm_topk=True):
    lg = _f64(logits)
    idx = np.ascontiguousarray(idx, dtype=np.int32)
    T, E = lg.shape
    k = idx.shape[1]
    w = np.empty((T, k), dtype=np.float64)
    lib().oracle_route_weights(_p(lg), _p(idx), ctypes.c_int64(T), E, k, int(norm_topk), _p(w))
    return w


def route_bf16(logits, k, norm_topk=False):
    """Routing with bf16-rounded probabilities ([P1] section 11) on given router logits
    [T, E]: fp32 softmax rounded to bf16, the k largest rounded values (lower index first
    on ties), weights = rounded probabilities (renormalised with norm_topk).
    Returns idx [T, k] int32, w [T, k]."""
    lg = _f64(logits)
    T, E = lg.shape
    idx = np.empty((T, k), np.int32)
    w = np.empty((T, k), np.float64)
    lib().oracle_route_bf16(_p(lg), ctypes.c_int64(T), E, k, int(norm_topk), _p(idx), _p(w))
    return idx, w


def permute(idx, E):
    idx = np.ascontiguousarray(idx, dtype=np.int32)
    T, k = idx.shape
    counts = np.empty((E,), np.int32)
    offsets = np.empty((E + 1,), np.int32)
    perm = np.empty((T * k,), np.int32)
    inv = np.empty((T, k), np.int32)
    lib().oracle_permute(_p(idx), ctypes.c_int64(T), k, E, _p(counts), _p(offsets), _p(perm),
                         _p(inv))
    return counts, offsets, perm, inv


def sample(logits, temperature, top_p, u):
    """One draw per row by the sampling rule of the generation loops ([P3] generation and
    [P4] sampling sections: softmax of logits / temperature, optionally cut to the top-p
    nucleus, then a multinomial draw), made exact so that two implementations agree:
      e_v = exp((l_v - max) / temperature), non-finite logits give e_v = 0;
      sort e descending (ties by index); the nucleus is cut at the first sorted entry where
      the running sum reaches top_p * sum(e), and every e_v >= that entry's value is kept
      (top_p >= 1 keeps every e_v > 0);
      K = kept mass; r = u K; the token is the smallest index v whose running kept mass over
      tokens <= v (ascending index order) exceeds r, else the last kept index.
    logits [rows, V] (or [V]); u [rows] in [0, 1).  Returns (tokens int32 [rows], details),
    details per row: dict(e, tau, kept, K, r, cum) for tolerance checks."""
    lg = np.asarray(logits, dtype=np.float64)
    if lg.ndim == 1:
        lg = lg[None]
    u = np.broadcast_to(np.asarray(u, dtype=np.float64), (lg.shape[0],))
    toks = np.empty((lg.shape[0],), np.int32)
    details = []
    for r_i in range(lg.shape[0]):
        l = lg[r_i]
        fin = np.isfinite(l)
        if not fin.any():
            toks[r_i] = 0
            details.append(None)
            continue
        m = l[fin].max()
        e = np.zeros_like(l)
        e[fin] = np.exp((l[fin] - m) / temperature)
        if top_p < 1.0:
            order = np.argsort(-e, kind="stable")
            cs = np.cumsum(e[order])
            k = int(np.argmax(cs >= top_p * e.sum()))
            tau = e[order[k]]
        else:
            tau = e[e > 0].min()
        kept = (e >= tau) & (e > 0)
        K = e[kept].sum()
        r = min(max(float(u[r_i]), 0.0), 1.0) * K
        cum = np.cumsum(np.where(kept, e, 0.0))
        hit = np.nonzero(kept & (cum > r))[0]
        toks[r_i] = hit[0] if hit.size else np.nonzero(kept)[0][-1]
        details.append(dict(e=e, tau=tau, kept=kept, K=K, r=r, cum=cum))
    return toks, details


def generate(cfg, model, prompt, n_new, temperature=0.0, top_p=1.0, uniforms=None):
    """Generation by full recompute, as in the pages' generation loops ([P1] section 13,
    [P3] generation): every step runs the whole model over prompt + tokens so far and takes
    the last row's logits; greedy (argmax, lowest index on ties) when temperature == 0, else
    sample() with uniforms[i].  prompt: int sequence.  Returns int32 [n_new]."""
    seq = [int(t) for t in prompt]
    out = []
    for i in range(n_new):
        lg = stack_prefill(cfg, model, np.array(seq, np.int32), rows=[len(seq) - 1])[0]
        if temperature == 0.0:
            t = int(argmax(lg)[0])
        else:
            t = int(sample(lg, temperature, top_p, [uniforms[i]])[0][0])
        out.append(t)
        seq.append(t)
    return np.array(out, np.int32)


def bf16_round(x):
    """fp32 values rounded to bf16 (round to nearest, ties to even), returned as float64."""
    a = np.atleast_1d(np.asarray(x, dtype=np.float32))
    lib().oracle_bf16_round.restype = ctypes.c_float
    lib().oracle_bf16_round.argtypes = [ctypes.c_float]
    return np.array([lib().oracle_bf16_round(float(v)) for v in a], dtype=np.float64)


def argmax(logits):
    lg = np.asarray(logits)
    if lg.ndim == 1:
        lg = lg[None]
    out = np.empty((lg.shape[0],), np.int32)
    if lg.dtype == np.float32:
        lg = np.ascontiguousarray(lg)
        lib().oracle_argmax_f32(_p(lg), ctypes.c_int64(lg.shape[0]), ctypes.c_int64(lg.shape[1]),
                                _p(out))
    else:
        lg = _f64(lg)
        lib().oracle_argmax_f64(_p(lg), ctypes.c_int64(lg.shape[0]), ctypes.c_int64(lg.shape[1]),
                                _p(out))
    return out
