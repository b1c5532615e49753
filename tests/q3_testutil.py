"""Shared helpers for the GPU parity tests: upload synthetic inputs, build caches, compare
against the oracle with the parity bar.

Parity bar (floating point): max |gpu - oracle| <= 2e-2 * rms(oracle) and
sum |gpu - oracle| / sum |oracle| <= 5e-3 (bf16 storage, fp32 accumulation).
Integer outputs are compared exactly.
"""
import sys

import numpy as np

import decoder_only_forward_amd as q3
import synth
from synth import recipes

MAX_ABS_REL_RMS = 2e-2
MEAN_REL = 5e-3


def log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


# Every comparison made by parity() in this process: the test that made it, what was
# compared, the element count and both error measures against their bars.  The session
# hook in conftest.py writes them to the JSON file named by Q3_PARITY_LOG.
RECORDS = []


def _current_test():
    import os
    return os.environ.get("PYTEST_CURRENT_TEST", "").split(" ")[0]


def parity(got, ref, what="", max_abs_rel=MAX_ABS_REL_RMS, mean_rel=MEAN_REL, stored_bf16=False):
    """Compare a GPU tensor with the oracle's: max |got - ref| <= max_abs_rel * rms(ref) and
    sum |got - ref| / sum |ref| <= mean_rel.  With stored_bf16 (the GPU output is bf16) the
    error against the oracle rounded to bf16 is reported too: it separates the output
    rounding from the computation's own error."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    assert got.shape == ref.shape, (what, got.shape, ref.shape)
    assert np.all(np.isfinite(got)), f"{what}: non-finite GPU output"
    err = np.abs(got - ref)
    rms = float(np.sqrt(np.mean(ref * ref)))
    max_abs = float(err.max()) if err.size else 0.0
    l1 = float(err.sum() / max(np.abs(ref).sum(), 1e-300))
    rec = dict(test=_current_test(), what=what, n=int(ref.size), rms=rms, max_abs=max_abs,
               max_abs_bar=max_abs_rel * rms, mean_rel=l1, mean_rel_bar=mean_rel)
    extra = ""
    if stored_bf16 and err.size:
        rb = synth.bf16_to_f32(synth.f32_to_bf16(ref.astype(np.float32))).astype(np.float64)
        rec["max_abs_vs_bf16_ref"] = float(np.abs(got - rb).max())
        extra = f" [vs bf16(oracle) {rec['max_abs_vs_bf16_ref']:.3e}]"
    RECORDS.append(rec)
    log(f"  parity {what}: max_abs={max_abs:.3e} (bar {max_abs_rel * rms:.3e}, "
        f"{max_abs / max(max_abs_rel * rms, 1e-300):.2f} of it) mean_rel={l1:.3e} "
        f"(bar {mean_rel:.1e}, {l1 / mean_rel:.2f}){extra}")
    assert max_abs <= max_abs_rel * rms, f"{what}: max_abs {max_abs} > {max_abs_rel} * rms {rms}"
    assert l1 <= mean_rel, f"{what}: mean relative error {l1} > {mean_rel}"
    return max_abs, l1


class ParityAccumulator:
    """parity() over a tensor compared in pieces: the error sums and maxima of each piece
    are accumulated and the bar is applied once to the whole tensor (rms and L1 norm of the
    whole oracle tensor), exactly as one parity() call on the concatenation would.  With
    stored_bf16 the largest error against the oracle rounded to bf16 is reported as well."""

    def __init__(self, what, max_abs_rel=MAX_ABS_REL_RMS, mean_rel=MEAN_REL, stored_bf16=False):
        self.what, self.max_abs_rel, self.mean_rel = what, max_abs_rel, mean_rel
        self.stored_bf16 = stored_bf16
        self.n = 0
        self.sq = self.abs_ref = self.abs_err = self.max_err = 0.0
        self.max_err_bf16 = 0.0  # against the oracle rounded to bf16 (stored_bf16 only)

    def add(self, got, ref):
        got = np.asarray(got, np.float64)
        ref = np.asarray(ref, np.float64)
        assert got.shape == ref.shape, (self.what, got.shape, ref.shape)
        assert np.all(np.isfinite(got)), f"{self.what}: non-finite GPU output"
        err = np.abs(got - ref)
        self.n += ref.size
        self.sq += float(np.sum(ref * ref))
        self.abs_ref += float(np.abs(ref).sum())
        self.abs_err += float(err.sum())
        self.max_err = max(self.max_err, float(err.max()) if err.size else 0.0)
        if self.stored_bf16 and err.size:
            rb = synth.bf16_to_f32(synth.f32_to_bf16(ref.astype(np.float32))).astype(np.float64)
            self.max_err_bf16 = max(self.max_err_bf16, float(np.abs(got - rb).max()))

    def check(self):
        rms = float(np.sqrt(self.sq / max(self.n, 1)))
        l1 = self.abs_err / max(self.abs_ref, 1e-300)
        bar = self.max_abs_rel * rms
        rec = dict(test=_current_test(), what=self.what, n=self.n, rms=rms,
                   max_abs=self.max_err, max_abs_bar=bar, mean_rel=l1, mean_rel_bar=self.mean_rel)
        extra = ""
        if self.stored_bf16:
            rec["max_abs_vs_bf16_ref"] = self.max_err_bf16
            extra = f" [vs bf16(oracle) {self.max_err_bf16:.3e}]"
        RECORDS.append(rec)
        log(f"  parity {self.what}: max_abs={self.max_err:.3e} (bar {bar:.3e}, "
            f"{self.max_err / max(bar, 1e-300):.2f} of it) mean_rel={l1:.3e} "
            f"(bar {self.mean_rel:.1e}, {l1 / self.mean_rel:.2f}) over {self.n} elements{extra}")
        assert self.max_err <= bar, f"{self.what}: max_abs {self.max_err} > {bar}"
        assert l1 <= self.mean_rel, f"{self.what}: mean relative error {l1} > {self.mean_rel}"


def f64(u16):
    return synth.bf16_to_f32(u16).astype(np.float64)


def to_dev_bf16(u16, device):
    import torch
    return torch.from_numpy(np.ascontiguousarray(u16)).view(torch.bfloat16).to(device)


def bf16_host(t):
    import torch
    return t.detach().contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def layer_to_dev(layer_host, device):
    """Oracle-side field names -> library field names, on the device."""
    m = {"in_norm": "input_layernorm", "q": "q_proj", "k": "k_proj", "v": "v_proj",
         "q_norm": "q_norm", "k_norm": "k_norm", "o": "o_proj",
         "post_norm": "post_attention_layernorm", "gate": "gate_proj", "up": "up_proj",
         "down": "down_proj", "router": "router", "experts_gate_up": "experts_gate_up_proj",
         "experts_down": "experts_down_proj"}
    return {m[k]: to_dev_bf16(v, device) for k, v in layer_host.items()}


def new_cache(B, nkv, cap, device):
    """One layer's K and V caches in the library's tiled layout, every slot NaN (untouched
    slots must never be read)."""
    k, vt = q3.kv_cache_empty(B, nkv, cap, device)
    k.fill_(float("nan"))
    vt.fill_(float("nan"))
    return k, vt


def fill_cache_synthetic(k, vt, seed, l, n_pos, ctx, rows=None):
    """Positions [0, n_pos) of every (sequence, kv head) from the generator, logical tensor
    [B, nkv, ctx, hd] named kv.{l}.k / kv.{l}.v; other slots keep their contents.  With
    ``rows`` = {b: n_pos_b} only those sequences are filled, each to its own length."""
    k_log, v_log = q3.kv_cache_to_logical(k, vt)
    B, nkv = k_log.shape[:2]
    kn, vn = recipes.kv_names(l)
    for b in range(B):
        n = n_pos if rows is None else rows.get(b, 0)
        if n <= 0:
            continue
        for h in range(nkv):
            off = ((b * nkv + h) * ctx) * 128
            for t, name in ((k_log, kn), (v_log, vn)):
                synth.normal_bf16_device(t[b, h], seed, name, 0.0, 1.0, offset=off,
                                         logical=(1, n, 128), strides=(0, 128, 1))
    kt, vtt = q3.kv_cache_from_logical(k_log, v_log)
    k.copy_(kt)
    vt.copy_(vtt)


def cache_logical_host(k, vt):
    """(K, V) of a device cache as logical [B, nkv, cap, hd] bf16 bit arrays."""
    k_log, v_log = q3.kv_cache_to_logical(k, vt)
    return bf16_host(k_log), bf16_host(v_log)


def cache_k_logical(k, b, n_pos):
    """[nkv, n_pos, hd] float64 from the device K cache."""
    return f64(bf16_host(q3.k_cache_to_logical(k)[b, :, :n_pos, :]))


def cache_v_logical(vt, b, n_pos):
    """[nkv, n_pos, hd] float64 from the device V cache."""
    return f64(bf16_host(q3.v_cache_to_logical(vt)[b, :, :n_pos, :]))


def small_cfg(H=256, nq=4, nkv=2, I=512, L=2, V=512, qk_norm=1, max_pos=4096,
              rope_interleaved=0):
    return dict(hidden_size=H, num_attention_heads=nq, num_key_value_heads=nkv, head_dim=128,
                intermediate_size=I, num_hidden_layers=L, vocab_size=V,
                max_position_embeddings=max_pos, rms_norm_eps=1e-6, rope_theta=1e6,
                qk_norm=qk_norm, tie_word_embeddings=1, rope_interleaved=rope_interleaved)
