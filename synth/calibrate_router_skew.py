"""Calibrate per-expert router row scales for the skewed-load MoE workload.

Input recipe only (no decoder arithmetic).  With token activations ~N(0, I) and random
router rows w_e ~ N(0, (0.02 g_e)^2 I), the router logits are (nearly) independent
normals with standard deviations proportional to g_e, so an expert with a larger g_e
lands in a token's top-k more often.  A fixed-point iteration on Monte-Carlo draws of
independent normals picks g_e so that the expected number of tokens per expert follows
a Zipf(s = 1.1) profile over expert ranks.

An expert can never take more than half of the tokens here (the logits are
sign-symmetric and there is no router bias, so P(e in top-k) <= P(e in bottom-k) + ...
<= 1/2), so the Zipf profile is capped at CAP_FRACTION of the tokens and renormalised
to T * k.  Ranks are mapped to expert ids by a seeded permutation.

Writes router_skew_e128_k8.json next to this file.
"""
import json
import os

import numpy as np

E, K, T = 128, 8, 8192
ZIPF_S = 1.1
CAP_FRACTION = 0.40
SEED = 4
HERE = os.path.dirname(os.path.abspath(__file__))
OUT = os.path.join(HERE, "router_skew_e128_k8.json")


def target_counts():
    r = np.arange(1, E + 1, dtype=np.float64)
    cap = CAP_FRACTION * T
    lo, hi = 0.0, 1e9
    for _ in range(200):
        c = 0.5 * (lo + hi)
        n = np.minimum(cap, c * r ** -ZIPF_S)
        if n.sum() > T * K:
            hi = c
        else:
            lo = c
    return np.minimum(cap, lo * r ** -ZIPF_S)


def expected_counts(g, rng, draws=65536):
    z = rng.standard_normal((draws, E)) * g[None, :]
    top = np.argpartition(-z, K, axis=1)[:, :K]
    return np.bincount(top.ravel(), minlength=E) * (T / draws)


def calibrate(iters=60):
    rng = np.random.default_rng(SEED)
    target = target_counts()  # by rank
    g = np.ones(E)
    for it in range(iters):
        n = expected_counts(g, rng)
        step = 0.5 if it < 40 else 0.25
        g *= (target / np.maximum(n, 1e-3)) ** step
        g /= np.exp(np.mean(np.log(g)))  # geometric mean 1
        g = np.clip(g, 1e-3, 1e3)
    n = expected_counts(g, np.random.default_rng(SEED + 1), draws=262144)
    perm = np.random.default_rng(SEED).permutation(E)  # rank -> expert id
    scale = np.empty(E)
    scale[perm] = g
    return scale, target, n, perm


def main():
    scale, target, n, perm = calibrate()
    out = {
        "description": "router row scale per expert (index = expert id); Zipf(1.1) load "
                       "capped at 0.40 of the tokens, k=8 of 128 experts, 8192 tokens",
        "zipf_s": ZIPF_S, "cap_fraction": CAP_FRACTION, "seed": SEED,
        "scale": [float(x) for x in scale],
        "rank_to_expert": [int(x) for x in perm],
        "target_tokens_by_rank": [float(x) for x in target],
        "expected_tokens_by_rank": [float(x) for x in n],
    }
    with open(OUT, "w") as f:
        json.dump(out, f, indent=1)
    print("max/mean expected load %.2f, top-4 %s, rank64 %.0f, rank128 %.0f" % (
        n.max() / n.mean(), np.round(n[:4]).tolist(), n[63], n[127]))


if __name__ == "__main__":
    main()
