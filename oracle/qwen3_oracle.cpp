// Qwen3 decoder forward -- CPU ORACLE (test infrastructure only; see header).
// Every function states the passage it follows.  All arithmetic is double.
#include "qwen3_oracle.h"

#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstring>
#include <functional>
#include <limits>
#include <thread>
#include <vector>

namespace {

int g_threads = 0;

int threads() {
  if (g_threads > 0) return g_threads;
  unsigned n = std::thread::hardware_concurrency();
  return n ? (int)n : 1;
}

// Run fn(i) for i in [0, n) on the worker threads (independent items only).
void parallel_for(int64_t n, const std::function<void(int64_t)> &fn) {
  int nt = (int)std::min<int64_t>(threads(), n);
  if (nt <= 1) {
    for (int64_t i = 0; i < n; ++i) fn(i);
    return;
  }
  std::atomic<int64_t> next(0);
  std::vector<std::thread> pool;
  for (int t = 0; t < nt; ++t)
    pool.emplace_back([&]() {
      for (;;) {
        int64_t i = next.fetch_add(1);
        if (i >= n) break;
        fn(i);
      }
    });
  for (auto &th : pool) th.join();
}

inline double bf(uint16_t u) {
  uint32_t bits = (uint32_t)u << 16;
  float f;
  std::memcpy(&f, &bits, 4);
  return (double)f;
}

// y[n] = sum_k x[k] * W[n][k]: a linear layer without bias, weights in the HF
// [out, in] layout, i.e. x @ W.T ([P1] section 7; [P3] "GQA 注意力": all
// projections bias=False).
void linear_row(const double *x, const uint16_t *W, int64_t N, int64_t K, double *y) {
  for (int64_t n = 0; n < N; ++n) {
    const uint16_t *w = W + n * K;
    double acc = 0.0;
    for (int64_t k = 0; k < K; ++k) acc += x[k] * bf(w[k]);
    y[n] = acc;
  }
}

// RMSNorm of one vector: y_i = x_i / sqrt(mean_j x_j^2 + eps) * w_i
// ([P3] "RMSNorm" formula; [P1] section 6; [P4] 3.1).
void rmsnorm_vec(const double *x, int n, const uint16_t *w, double eps, double *y) {
  double ss = 0.0;
  for (int i = 0; i < n; ++i) ss += x[i] * x[i];
  double inv = 1.0 / std::sqrt(ss / n + eps);
  for (int i = 0; i < n; ++i) y[i] = x[i] * inv * bf(w[i]);
}

// RoPE of one head vector at absolute position pos: theta_i = base^(-2i/hd), i < hd/2;
// plane i is rotated by pos theta_i: [a, b] -> [a cos - b sin, a sin + b cos].
// Rotate-half pairing (the default): plane i = dims (i, i + hd/2) ([P3] "RoPE" formula
// and apply_rope; [P4] 3.4).  Interleaved pairing: plane i = dims (2i, 2i + 1), the
// complex-number form of [P1] section 8.
void rope_vec(const double *x, int hd, int64_t pos, double theta, int interleaved, double *y) {
  int half = hd / 2;
  for (int i = 0; i < half; ++i) {
    double inv_freq = std::pow(theta, -(2.0 * i) / hd);
    double ang = (double)pos * inv_freq;
    double c = std::cos(ang), s = std::sin(ang);
    int ia = interleaved ? 2 * i : i, ib = interleaved ? 2 * i + 1 : i + half;
    double a = x[ia], b = x[ib];
    y[ia] = a * c - b * s;
    y[ib] = a * s + b * c;
  }
}

// fp32 -> bf16 -> fp32 with round-to-nearest-even: keep the top 16 bits of the fp32
// pattern, rounding on the dropped 16 (a NaN stays a NaN).
float bf16_round_impl(float x) {
  uint32_t u;
  std::memcpy(&u, &x, 4);
  if ((u & 0x7f800000u) == 0x7f800000u && (u & 0x007fffffu)) return x;
  const uint32_t dropped = u & 0xffffu, keep = u & 0xffff0000u;
  const uint32_t half = 0x8000u;
  uint32_t r = keep;
  if (dropped > half || (dropped == half && (keep & 0x10000u))) r += 0x10000u;
  float y;
  std::memcpy(&y, &r, 4);
  return y;
}

// silu(z) = z / (1 + e^-z) ([P3] "SwiGLU FFN"; [P1] section 11).
inline double silu(double z) { return z / (1.0 + std::exp(-z)); }

// One query row of causal scaled-dot-product attention for one q head:
// s_j = q . k_j / sqrt(hd) for keys j <= qpos, softmax over those j,
// o = sum_j p_j v_j ([P3] "GQA 注意力" formula with mask M_ij = -inf for j > i;
// [P1] section 9).  The max subtraction leaves the softmax unchanged.
void attend_row(const double *q, const double *k, const double *v, int64_t qpos, int kvh,
                int nkv, int hd, double *o, std::vector<double> &s) {
  int64_t n = qpos + 1;
  s.resize(n);
  double scale = 1.0 / std::sqrt((double)hd);
  double m = -std::numeric_limits<double>::infinity();
  for (int64_t j = 0; j < n; ++j) {
    const double *kj = k + (j * nkv + kvh) * hd;
    double d = 0.0;
    for (int e = 0; e < hd; ++e) d += q[e] * kj[e];
    s[j] = d * scale;
    m = std::max(m, s[j]);
  }
  double sum = 0.0;
  for (int64_t j = 0; j < n; ++j) {
    s[j] = std::exp(s[j] - m);
    sum += s[j];
  }
  for (int e = 0; e < hd; ++e) o[e] = 0.0;
  for (int64_t j = 0; j < n; ++j) {
    const double *vj = v + (j * nkv + kvh) * hd;
    double p = s[j] / sum;
    for (int e = 0; e < hd; ++e) o[e] += p * vj[e];
  }
}

}  // namespace

extern "C" {

void oracle_set_threads(int n) { g_threads = n; }
int oracle_get_threads(void) { return threads(); }

void oracle_rmsnorm_rows(const double *x, int64_t rows, int n, const uint16_t *w, double eps,
                         double *y) {
  parallel_for(rows, [&](int64_t r) { rmsnorm_vec(x + r * n, n, w, eps, y + r * n); });
}

void oracle_rope(const double *x, int64_t nvec, int hd, const int64_t *pos, double theta,
                 int interleaved, double *y) {
  parallel_for(nvec, [&](int64_t i) {
    rope_vec(x + i * hd, hd, pos[i], theta, interleaved, y + i * hd);
  });
}

// Grouped-query attention: q head h reads kv head h / (nq / nkv)
// ([P3] "GQA 注意力": repeat_interleave of each kv group over its q heads;
// [P1] section 10).  Keys are indexed by absolute position 0..L-1.
void oracle_attention(const double *q, const double *k, const double *v, const int64_t *qpos,
                      int64_t S, int64_t L, int nq, int nkv, int hd, double *o) {
  int g = nq / nkv;
  parallel_for(S * nq, [&](int64_t i) {
    int64_t s = i / nq;
    int h = (int)(i % nq);
    int64_t p = std::min<int64_t>(qpos[s], L - 1);
    std::vector<double> sc;
    attend_row(q + i * hd, k, v, p, h / g, nkv, hd, o + i * hd, sc);
  });
}

// Bias-free linear layer over rows: y[t] = x[t] W^T ([P1] section 7; [P3] "MoE": the
// router is such a linear map from hidden to experts).
void oracle_linear_rows(const double *x, int64_t T, int64_t K, const uint16_t *W, int64_t N,
                        double *y) {
  parallel_for(T, [&](int64_t t) { linear_row(x + t * K, W, N, K, y + t * N); });
}

// SwiGLU FFN: down(silu(gate x) * up x) ([P3] "SwiGLU FFN" formula; [P4] 3.8).
void oracle_swiglu_ffn(const double *x, int64_t T, int H, int I, const uint16_t *gate,
                       const uint16_t *up, const uint16_t *down, double *y) {
  parallel_for(T, [&](int64_t t) {
    std::vector<double> g(I), u(I);
    linear_row(x + t * H, gate, I, H, g.data());
    linear_row(x + t * H, up, I, H, u.data());
    for (int i = 0; i < I; ++i) g[i] = silu(g[i]) * u[i];
    linear_row(g.data(), down, H, I, y + t * H);
  });
}

static void moe_row(const oracle_cfg *c, const uint16_t *router, const uint16_t *gate_up,
                    const uint16_t *down, const double *xt, double *y, int32_t *idx, double *w,
                    double *r);

// One pre-norm decoder block for one sequence ([P3] "TransformerBlock" and
// "GQA 注意力"; [P4] decoder layer):
//   n  = rmsnorm(x, in_norm)
//   q, k, v = n Wq^T, n Wk^T, n Wv^T, reshaped into heads
//   q, k  = per-head rmsnorm(q_norm / k_norm) when qk_norm, then RoPE at
//           absolute position pos0 + s (the offset is the cached length)
//   keys/values = past cache (positions < pos0) followed by the new k, v
//   h1 = x + attention(q, keys, values) Wo^T
//   h2 = h1 + swiglu(rmsnorm(h1, post_norm))   (routed: h1 + moe(rmsnorm(h1, post_norm)))
// rows != NULL restricts the attention/FFN outputs to those token rows (the K/V
// of every row are still produced, as every later row needs them).  routed selects the
// routed MoE FFN ([P1] section 11, [P3] "MoE") with the layer's router and experts;
// router_logits (nullable) then receives each output row's router logits [n_rows][E].
void oracle_block(const oracle_cfg *c, const oracle_layer *w, const double *x, int64_t S,
                  int64_t pos0, const double *past_k, const double *past_v, const int64_t *rows,
                  int64_t n_rows, double *x_out, double *new_k, double *new_v, int routed,
                  double *router_logits) {
  const int H = c->hidden, nq = c->n_heads, nkv = c->n_kv_heads, hd = c->head_dim;
  const int64_t L = pos0 + S;
  std::vector<int64_t> all;
  if (!rows) {
    all.resize(S);
    for (int64_t s = 0; s < S; ++s) all[s] = s;
    rows = all.data();
    n_rows = S;
  }
  // keys and values for every absolute position 0..L-1, layout [L][nkv][hd]
  std::vector<double> K((size_t)L * nkv * hd), V((size_t)L * nkv * hd);
  for (int h = 0; h < nkv; ++h)
    for (int64_t p = 0; p < pos0; ++p)
      for (int e = 0; e < hd; ++e) {
        K[(p * nkv + h) * hd + e] = past_k[((int64_t)h * pos0 + p) * hd + e];
        V[(p * nkv + h) * hd + e] = past_v[((int64_t)h * pos0 + p) * hd + e];
      }
  parallel_for(S, [&](int64_t s) {
    std::vector<double> n(H), kr((size_t)nkv * hd), vr((size_t)nkv * hd), t(hd);
    rmsnorm_vec(x + s * H, H, w->in_norm, c->eps, n.data());
    linear_row(n.data(), w->k, (int64_t)nkv * hd, H, kr.data());
    linear_row(n.data(), w->v, (int64_t)nkv * hd, H, vr.data());
    for (int h = 0; h < nkv; ++h) {
      double *kh = kr.data() + (size_t)h * hd;
      if (c->qk_norm) {
        rmsnorm_vec(kh, hd, w->k_norm, c->eps, t.data());
        std::copy(t.begin(), t.end(), kh);
      }
      rope_vec(kh, hd, pos0 + s, c->theta, c->rope_interleaved, t.data());
      for (int e = 0; e < hd; ++e) {
        K[((pos0 + s) * nkv + h) * hd + e] = t[e];
        V[((pos0 + s) * nkv + h) * hd + e] = vr[(size_t)h * hd + e];
      }
    }
  });
  if (new_k)
    for (int h = 0; h < nkv; ++h)
      for (int64_t s = 0; s < S; ++s)
        for (int e = 0; e < hd; ++e) {
          new_k[((int64_t)h * S + s) * hd + e] = K[((pos0 + s) * nkv + h) * hd + e];
          new_v[((int64_t)h * S + s) * hd + e] = V[((pos0 + s) * nkv + h) * hd + e];
        }
  const int g = nq / nkv;
  const int I = c->inter;
  parallel_for(n_rows, [&](int64_t ri) {
    int64_t s = rows[ri];
    std::vector<double> n(H), q((size_t)nq * hd), t(hd), o((size_t)nq * hd), h1(H), n2(H),
        gg(I), uu(I), y(H), sc;
    rmsnorm_vec(x + s * H, H, w->in_norm, c->eps, n.data());
    linear_row(n.data(), w->q, (int64_t)nq * hd, H, q.data());
    for (int h = 0; h < nq; ++h) {
      double *qh = q.data() + (size_t)h * hd;
      if (c->qk_norm) {
        rmsnorm_vec(qh, hd, w->q_norm, c->eps, t.data());
        std::copy(t.begin(), t.end(), qh);
      }
      rope_vec(qh, hd, pos0 + s, c->theta, c->rope_interleaved, t.data());
      std::copy(t.begin(), t.end(), qh);
      attend_row(qh, K.data(), V.data(), pos0 + s, h / g, nkv, hd, o.data() + (size_t)h * hd, sc);
    }
    linear_row(o.data(), w->o, H, (int64_t)nq * hd, h1.data());
    for (int i = 0; i < H; ++i) h1[i] += x[s * H + i];
    rmsnorm_vec(h1.data(), H, w->post_norm, c->eps, n2.data());
    if (routed) {
      const int E = c->n_experts, k = c->top_k;
      std::vector<int32_t> idx(k);
      std::vector<double> wt(k), r(E);
      moe_row(c, w->router, w->experts_gate_up, w->experts_down, n2.data(), y.data(),
              idx.data(), wt.data(), r.data());
      if (router_logits) std::copy(r.begin(), r.end(), router_logits + ri * E);
    } else {
      linear_row(n2.data(), w->gate, I, H, gg.data());
      linear_row(n2.data(), w->up, I, H, uu.data());
      for (int i = 0; i < I; ++i) gg[i] = silu(gg[i]) * uu[i];
      linear_row(gg.data(), w->down, H, I, y.data());
    }
    for (int i = 0; i < H; ++i) x_out[ri * H + i] = h1[i] + y[i];
  });
}

// Whole model for one sequence starting at position 0 ([P3] "骨架" forward;
// [P1] sections 12-13): embedding lookup, every block in order, final RMSNorm,
// LM head (lm_head == NULL means tied: the embedding matrix is reused).
// logits are produced for the requested token rows; k_out / v_out (nullable)
// receive each layer's new keys / values, layout [layer][nkv][S][hd].  Layer l is routed
// when the config has experts and (l + 1) % sparse_step == 0 (the Qwen-MoE convention
// behind [P1]'s decoder_sparse_step); router_out (nullable) receives the routed layers'
// router logits [layer][S][E].
static bool routed_layer(const oracle_cfg *c, int l) {
  return c->n_experts > 0 && c->sparse_step > 0 && (l + 1) % c->sparse_step == 0;
}

void oracle_stack_prefill(const oracle_cfg *c, const uint16_t *embed, const uint16_t *final_norm,
                          const uint16_t *lm_head, const oracle_layer *layers, const int32_t *ids,
                          int64_t S, const int64_t *rows, int64_t n_rows, double *logits,
                          double *k_out, double *v_out, double *router_out) {
  const int H = c->hidden, nkv = c->n_kv_heads, hd = c->head_dim;
  std::vector<double> x((size_t)S * H), y((size_t)S * H);
  for (int64_t s = 0; s < S; ++s)
    for (int i = 0; i < H; ++i) x[s * H + i] = bf(embed[(int64_t)ids[s] * H + i]);
  for (int l = 0; l < c->n_layers; ++l) {
    double *kk = k_out ? k_out + (int64_t)l * nkv * S * hd : nullptr;
    double *vv = v_out ? v_out + (int64_t)l * nkv * S * hd : nullptr;
    double *ro = router_out ? router_out + (int64_t)l * S * c->n_experts : nullptr;
    oracle_block(c, &layers[l], x.data(), S, 0, nullptr, nullptr, nullptr, 0, y.data(), kk, vv,
                 routed_layer(c, l), ro);
    x.swap(y);
  }
  const uint16_t *head = lm_head ? lm_head : embed;
  std::vector<double> hf((size_t)n_rows * H);
  for (int64_t r = 0; r < n_rows; ++r) rmsnorm_vec(&x[rows[r] * H], H, final_norm, c->eps, &hf[r * H]);
  const int64_t V = c->vocab;
  const int64_t chunk = 1024;
  const int64_t nchunk = (V + chunk - 1) / chunk;
  parallel_for(n_rows * nchunk, [&](int64_t i) {
    int64_t r = i / nchunk, v0 = (i % nchunk) * chunk;
    int64_t n = std::min(chunk, V - v0);
    linear_row(&hf[r * H], head + v0 * H, n, H, logits + r * V + v0);
  });
}

// One decode step for one sequence: the new token at absolute position pos
// attends to cached keys/values 0..pos-1 plus its own ([P3] "prefill 与
// decode": the last mask row sees all history).  Caches per layer are
// [nkv][pos][hd], either bf16 (cache_k/cache_v) or double (cache_k64/...).
// Decode of n new tokens of one sequence at positions pos .. pos + n - 1 ([P3] "prefill 与
// decode"; [P2] section 4's mask slice: token i sees the cached positions and new tokens
// 0..i): every layer is the block over the n rows with the given cache as its past, then
// the final norm and the LM head on each row.  logits [n][V]; router_out [L][n][E].
void oracle_stack_decode(const oracle_cfg *c, const uint16_t *embed, const uint16_t *final_norm,
                         const uint16_t *lm_head, const oracle_layer *layers, const int32_t *ids,
                         int64_t n, int64_t pos, const uint16_t *const *cache_k,
                         const uint16_t *const *cache_v, const double *const *cache_k64,
                         const double *const *cache_v64, double *logits, double *router_out) {
  const int H = c->hidden, nkv = c->n_kv_heads, hd = c->head_dim;
  std::vector<double> x((size_t)n * H), y((size_t)n * H), pk((size_t)nkv * pos * hd),
      pv((size_t)nkv * pos * hd);
  for (int64_t t = 0; t < n; ++t)
    for (int i = 0; i < H; ++i) x[t * H + i] = bf(embed[(int64_t)ids[t] * H + i]);
  for (int l = 0; l < c->n_layers; ++l) {
    for (size_t i = 0; i < pk.size(); ++i) {
      pk[i] = cache_k64 ? cache_k64[l][i] : bf(cache_k[l][i]);
      pv[i] = cache_v64 ? cache_v64[l][i] : bf(cache_v[l][i]);
    }
    oracle_block(c, &layers[l], x.data(), n, pos, pk.data(), pv.data(), nullptr, 0, y.data(),
                 nullptr, nullptr, routed_layer(c, l),
                 router_out ? router_out + (int64_t)l * n * c->n_experts : nullptr);
    x.swap(y);
  }
  const uint16_t *head = lm_head ? lm_head : embed;
  const int64_t V = c->vocab, chunk = 1024, nchunk = (V + chunk - 1) / chunk;
  std::vector<double> hf(H);
  for (int64_t t = 0; t < n; ++t) {
    rmsnorm_vec(x.data() + t * H, H, final_norm, c->eps, hf.data());
    double *lg = logits + t * V;
    parallel_for(nchunk, [&](int64_t i) {
      int64_t v0 = i * chunk, m = std::min(chunk, V - v0);
      linear_row(hf.data(), head + v0 * H, m, H, lg + v0);
    });
  }
}

// Top-k selection on given scores: the k largest, in descending order, ties
// broken toward the lower expert index.  (The pages call topk on the fp32
// softmax probabilities; softmax is monotone, so selecting on logits is the
// same selection.)
void oracle_topk(const float *logits, int64_t T, int E, int k, int32_t *idx) {
  parallel_for(T, [&](int64_t t) {
    std::vector<int> order(E);
    for (int e = 0; e < E; ++e) order[e] = e;
    const float *r = logits + t * E;
    std::stable_sort(order.begin(), order.end(), [&](int a, int b) { return r[a] > r[b]; });
    for (int j = 0; j < k; ++j) idx[t * k + j] = order[j];
  });
}

// Routing weights ([P3] "MoE" router): p = softmax over all experts, in full
// precision; w_j = p_{idx_j}, divided by the sum of the selected p when
// norm_topk_prob is set.
void oracle_route_weights(const double *logits, const int32_t *idx, int64_t T, int E, int k,
                          int norm_topk, double *w) {
  for (int64_t t = 0; t < T; ++t) {
    const double *r = logits + t * E;
    double m = -std::numeric_limits<double>::infinity();
    for (int e = 0; e < E; ++e) m = std::max(m, r[e]);
    double z = 0.0;
    for (int e = 0; e < E; ++e) z += std::exp(r[e] - m);
    double sel = 0.0;
    for (int j = 0; j < k; ++j) {
      w[t * k + j] = std::exp(r[idx[t * k + j]] - m) / z;
      sel += w[t * k + j];
    }
    if (norm_topk)
      for (int j = 0; j < k; ++j) w[t * k + j] /= sel;
  }
}

// Routing with bf16 probabilities ([P1] section 11): the softmax over all experts, in
// fp32 as that page computes it, is rounded to bf16; the k experts with the largest
// rounded probabilities are taken (the lower index first among equal values) and each
// weight is its rounded probability, divided by the selection's sum with norm_topk.
void oracle_route_bf16(const double *logits, int64_t T, int E, int k, int norm_topk,
                       int32_t *idx, double *w) {
  std::vector<int> order(E);
  std::vector<double> p(E);
  for (int64_t t = 0; t < T; ++t) {
    const double *r = logits + t * E;
    float m = -std::numeric_limits<float>::infinity();
    for (int e = 0; e < E; ++e) m = std::max(m, (float)r[e]);
    float z = 0.f;
    for (int e = 0; e < E; ++e) z += std::exp((float)r[e] - m);
    for (int e = 0; e < E; ++e) p[e] = oracle_bf16_round(std::exp((float)r[e] - m) / z);
    for (int e = 0; e < E; ++e) order[e] = e;
    std::stable_sort(order.begin(), order.end(), [&](int a, int b) { return p[a] > p[b]; });
    double sel = 0.0;
    for (int j = 0; j < k; ++j) {
      idx[t * k + j] = order[j];
      w[t * k + j] = p[order[j]];
      sel += w[t * k + j];
    }
    if (norm_topk)
      for (int j = 0; j < k; ++j) w[t * k + j] /= sel;
  }
}

// The selected experts of one token, mixed: y = sum_j w_j down_e(silu(gate_e x) * up_e x) with
// e = idx[j]; each expert is a SwiGLU whose fused gate_up_proj [2I, H] splits into gate =
// rows [0, I) and up = rows [I, 2I) ([P3] "MoE": chunk(2) of gate_up_proj, the expert
// outputs weighted and summed per token).
static void expert_mix(int H, int I, int k, const uint16_t *gate_up, const uint16_t *down,
                       const double *xt, const int32_t *idx, const double *w, double *y) {
  std::vector<double> g(I), u(I), o(H);
  for (int i = 0; i < H; ++i) y[i] = 0.0;
  for (int j = 0; j < k; ++j) {
    int e = idx[j];
    const uint16_t *gu = gate_up + (int64_t)e * 2 * I * H;
    linear_row(xt, gu, I, H, g.data());
    linear_row(xt, gu + (int64_t)I * H, I, H, u.data());
    for (int i = 0; i < I; ++i) g[i] = silu(g[i]) * u[i];
    linear_row(g.data(), down + (int64_t)e * H * I, H, I, o.data());
    for (int i = 0; i < H; ++i) y[i] += w[j] * o[i];
  }
}

// Routed MoE FFN of one token ([P3] "MoE": router linear, fp32 softmax, top-k, optional
// renormalisation; each selected expert is a SwiGLU whose fused gate_up_proj [2I, H]
// splits into gate = rows [0, I) and up = rows [I, 2I) (chunk(2)); outputs are summed with
// the routing weights).  With router_bf16 the selection follows [P1] section 11 instead:
// the softmax (fp32, as that page computes it) is rounded to bf16, the experts with the
// largest rounded probabilities are taken (lower index first on ties) and each weight is
// its rounded probability (renormalised over the selection only with norm_topk).
static void moe_row(const oracle_cfg *c, const uint16_t *router, const uint16_t *gate_up,
                    const uint16_t *down, const double *xt, double *y, int32_t *idx, double *w,
                    double *r) {
  const int H = c->hidden, E = c->n_experts, k = c->top_k, I = c->moe_inter;
  linear_row(xt, router, E, H, r);
  std::vector<int> order(E);
  for (int e = 0; e < E; ++e) order[e] = e;
  if (c->router_bf16) {
    oracle_route_bf16(r, 1, E, k, c->norm_topk, idx, w);
  } else {
    std::stable_sort(order.begin(), order.end(), [&](int a, int b) { return r[a] > r[b]; });
    for (int j = 0; j < k; ++j) idx[j] = order[j];
    oracle_route_weights(r, idx, 1, E, k, c->norm_topk, w);
  }
  expert_mix(H, I, k, gate_up, down, xt, idx, w, y);
}

// Routed MoE FFN over T tokens, token by token (see moe_row).
void oracle_moe_ffn(const oracle_cfg *c, const uint16_t *router, const uint16_t *gate_up,
                    const uint16_t *down, const double *x, int64_t T, double *y, int32_t *idx,
                    double *w, double *logits) {
  const int H = c->hidden, E = c->n_experts, k = c->top_k;
  parallel_for(T, [&](int64_t t) {
    moe_row(c, router, gate_up, down, x + t * H, y + t * H, idx + t * k, w + t * k,
            logits + t * E);
  });
}

// Routed MoE FFN evaluated at a given selection: token t mixes experts idx[t][0..k) with
// weights w[t][0..k) (see expert_mix).  This is the token-wise reference of [P3] "MoE" with
// the routing taken as an input, so that a device's output can be checked at the device's
// own expert choice for tokens whose top-k sits on a near-tie of router logits.
void oracle_moe_ffn_at(const oracle_cfg *c, const uint16_t *gate_up, const uint16_t *down,
                       const double *x, int64_t T, const int32_t *idx, const double *w,
                       double *y) {
  const int H = c->hidden, k = c->top_k, I = c->moe_inter;
  parallel_for(T, [&](int64_t t) {
    expert_mix(H, I, k, gate_up, down, x + t * H, idx + t * k, w + t * k, y + t * H);
  });
}

// Dispatch order of (token, slot) pairs: grouped by expert in ascending
// expert id, tokens ascending within an expert ([P3] "MoE": each hit expert
// gathers its token rows; the order within the group is not fixed by the
// pages, ascending token order is the reading taken).  counts[e] rows per
// expert, offsets = exclusive prefix (E + 1 entries), perm_token[row] = token,
// inv_row[t * k + j] = row of token t's j-th choice.
void oracle_permute(const int32_t *idx, int64_t T, int k, int E, int32_t *counts,
                    int32_t *offsets, int32_t *perm_token, int32_t *inv_row) {
  int32_t row = 0;
  for (int e = 0; e < E; ++e) {
    offsets[e] = row;
    for (int64_t t = 0; t < T; ++t)
      for (int j = 0; j < k; ++j)
        if (idx[t * k + j] == e) {
          perm_token[row] = (int32_t)t;
          inv_row[t * k + j] = row;
          ++row;
        }
    counts[e] = row - offsets[e];
  }
  offsets[E] = row;
}

// Greedy next token: index of the largest logit, lowest index on ties
// ([P1] section 13 argmax; [P4] greedy generation).
void oracle_argmax_f32(const float *logits, int64_t rows, int64_t V, int32_t *out) {
  for (int64_t r = 0; r < rows; ++r) {
    const float *x = logits + r * V;
    int64_t best = 0;
    for (int64_t v = 1; v < V; ++v)
      if (x[v] > x[best]) best = v;
    out[r] = (int32_t)best;
  }
}

float oracle_bf16_round(float x) { return bf16_round_impl(x); }

void oracle_argmax_f64(const double *logits, int64_t rows, int64_t V, int32_t *out) {
  for (int64_t r = 0; r < rows; ++r) {
    const double *x = logits + r * V;
    int64_t best = 0;
    for (int64_t v = 1; v < V; ++v)
      if (x[v] > x[best]) best = v;
    out[r] = (int32_t)best;
  }
}

}  // extern "C"
