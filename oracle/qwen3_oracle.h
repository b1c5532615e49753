/*
 * Qwen3 decoder forward -- CPU ORACLE (test infrastructure only).
 *
 * Plain, slow, obviously-correct reference used to check the GPU library.
 * Only the tests, the smoke check and the benchmark's CPU-baseline leg may
 * load it; the product path never does.  It shares no code with the GPU path.
 *
 * Arithmetic: every intermediate is IEEE double.  bf16 inputs (weights,
 * activations, KV-cache contents) are widened exactly.  No blocking, fusion or
 * reordering beyond what each definition states; threads only split
 * independent rows / heads / tokens.
 *
 * Sources (web pages on hand-building Qwen3; sections named as on the pages):
 *   [P1] "Building Qwen-3 MoE from scratch" (adg.csdn.net), sections 6-13.
 *   [P2] "手搓一个Qwen3" (news.43b.com.cn), sections 4-6.
 *   [P3] "从零实现 Qwen3：拆解 mini-qwen3 的 0.6B Dense 架构" (quarkcode.cn),
 *        sections "RMSNorm", "GQA 注意力", "RoPE", "SwiGLU FFN",
 *        "TransformerBlock", "骨架", "prefill 与 decode", "MoE".
 *   [P4] "从0实现SGLang" part 3 (wmrh.cn), sections 3.1-3.8.
 *
 * Layouts (row-major, HF [out_features, in_features] weights):
 *   x [S][H]; q [S][nq][hd]; k, v [L][nkv][hd] with key index = absolute
 *   position; past caches [nkv][pos0][hd].
 */
#ifndef QWEN3_ORACLE_H
#define QWEN3_ORACLE_H
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct {
  int32_t hidden, n_heads, n_kv_heads, head_dim, inter, n_layers, vocab, max_pos;
  double eps, theta;
  int32_t qk_norm;
  int32_t n_experts, top_k, moe_inter, norm_topk;
  int32_t rope_interleaved; /* 1: planes (2i, 2i + 1); 0: planes (i, i + hd/2) */
  int32_t sparse_step;      /* stack: layer l is routed when n_experts > 0 and
                               (l + 1) % sparse_step == 0; 0: no routed layers */
  int32_t router_bf16;      /* 1: routing probabilities rounded to bf16 before selection */
} oracle_cfg;

typedef struct { /* bf16 bits */
  const uint16_t *in_norm, *q, *k, *v, *q_norm, *k_norm, *o, *post_norm, *gate, *up, *down;
  /* routed layers: router [E][H], experts' fused gate|up [E][2I][H], down [E][H][I] */
  const uint16_t *router, *experts_gate_up, *experts_down;
} oracle_layer;

void oracle_set_threads(int n);
int oracle_get_threads(void);

void oracle_rmsnorm_rows(const double *x, int64_t rows, int n, const uint16_t *w, double eps,
                         double *y);
void oracle_rope(const double *x, int64_t nvec, int hd, const int64_t *pos, double theta,
                 int interleaved, double *y);
void oracle_attention(const double *q, const double *k, const double *v, const int64_t *qpos,
                      int64_t S, int64_t L, int nq, int nkv, int hd, double *o);
void oracle_linear_rows(const double *x, int64_t T, int64_t K, const uint16_t *W, int64_t N,
                        double *y);
void oracle_swiglu_ffn(const double *x, int64_t T, int H, int I, const uint16_t *gate,
                       const uint16_t *up, const uint16_t *down, double *y);
void oracle_block(const oracle_cfg *c, const oracle_layer *w, const double *x, int64_t S,
                  int64_t pos0, const double *past_k, const double *past_v, const int64_t *rows,
                  int64_t n_rows, double *x_out, double *new_k, double *new_v, int routed,
                  double *router_logits);
void oracle_stack_prefill(const oracle_cfg *c, const uint16_t *embed, const uint16_t *final_norm,
                          const uint16_t *lm_head, const oracle_layer *layers, const int32_t *ids,
                          int64_t S, const int64_t *rows, int64_t n_rows, double *logits,
                          double *k_out, double *v_out, double *router_out);
void oracle_stack_decode(const oracle_cfg *c, const uint16_t *embed, const uint16_t *final_norm,
                         const uint16_t *lm_head, const oracle_layer *layers, const int32_t *ids,
                         int64_t n, int64_t pos, const uint16_t *const *cache_k,
                         const uint16_t *const *cache_v, const double *const *cache_k64,
                         const double *const *cache_v64, double *logits, double *router_out);
void oracle_moe_ffn(const oracle_cfg *c, const uint16_t *router, const uint16_t *gate_up,
                    const uint16_t *down, const double *x, int64_t T, double *y, int32_t *idx,
                    double *w, double *logits);
void oracle_moe_ffn_at(const oracle_cfg *c, const uint16_t *gate_up, const uint16_t *down,
                       const double *x, int64_t T, const int32_t *idx, const double *w,
                       double *y);
void oracle_topk(const float *logits, int64_t T, int E, int k, int32_t *idx);
void oracle_route_weights(const double *logits, const int32_t *idx, int64_t T, int E, int k,
                          int norm_topk, double *w);
void oracle_route_bf16(const double *logits, int64_t T, int E, int k, int norm_topk,
                       int32_t *idx, double *w);
void oracle_permute(const int32_t *idx, int64_t T, int k, int E, int32_t *counts,
                    int32_t *offsets, int32_t *perm_token, int32_t *inv_row);
void oracle_argmax_f32(const float *logits, int64_t rows, int64_t V, int32_t *out);
void oracle_argmax_f64(const double *logits, int64_t rows, int64_t V, int32_t *out);
float oracle_bf16_round(float x);

#ifdef __cplusplus
}
#endif
#endif
