/*
 * qwen3.h -- C ABI of the MI355X (gfx950) Qwen3 decoder-forward library (libqwen3.so).
 *
 * The operations follow the hand-built Qwen3 described on these web pages
 * (sections named as on the pages):
 *   [P1] "Building Qwen-3 MoE from scratch" (adg.csdn.net), sections 5-13.
 *   [P2] "手搓一个Qwen3" (news.43b.com.cn), section 4 (KV cache and offset mask).
 *   [P3] "从零实现 Qwen3：拆解 mini-qwen3 的 0.6B Dense 架构" (quarkcode.cn):
 *        config table, "骨架", "prefill 与 decode", "RMSNorm", "GQA 注意力",
 *        "RoPE", "SwiGLU FFN", "TransformerBlock", "MoE".
 *   [P4] "从0实现SGLang" part 3 (wmrh.cn), sections 3.1-3.8 and 六.
 *
 * General conventions
 *   - Every tensor pointer is a DEVICE pointer unless stated otherwise; tensors are
 *     dense row-major.  "bf16" means IEEE bfloat16 bits (uint16).
 *   - Weights use the Hugging Face [out_features, in_features] layout: a projection
 *     computes y = x W^T without bias ([P1] section 7; [P3] "GQA 注意力").
 *   - Ownership: the caller owns all memory.  The library never allocates, frees or
 *     synchronises; it enqueues kernels on `stream` (a hipStream_t; NULL = default
 *     stream) and returns while they run.  Scratch space is the caller's `workspace`,
 *     sized by qwen3_workspace_bytes().
 *   - Errors: arguments are validated on the host before anything is enqueued; on a
 *     failure nothing is enqueued, a negative QWEN3_E* code is returned and
 *     qwen3_last_error() names the offending field.  A failed kernel launch returns
 *     QWEN3_EHIP.  Device faults surface at the caller's next synchronisation.
 *   - Alignment: every pointer must be 16-byte aligned.
 *   - Precision: weights, the embedding and the KV cache are bf16 in memory; matrix-core
 *     products accumulate in fp32; norms, softmax and RoPE run in fp32; inside
 *     qwen3_stack_forward the residual stream is fp32, and logits are fp32.  The activations
 *     passed between kernels (normalised rows, q/k/v projections, attention output, SwiGLU
 *     output) are IEEE fp16: 11-bit significand (8x finer than bf16), largest finite
 *     magnitude 65504.  A value whose magnitude rounds past 65504 becomes an infinity, and
 *     every output computed from it is non-finite: in the block entry points that token's
 *     output row; in the stack also later layers' rows of that sequence that attend to it.
 *     Rows that stay inside the range are unaffected.  On the fp16 path bf16 weights are
 *     converted to fp16 after loading: exact for magnitudes in [2^-14, 65504]; smaller ones
 *     keep fp16-subnormal precision (absolute error at most 2^-25); larger ones are not
 *     supported.  qwen3_moe_ffn reads its bf16 input x as bf16 matrix-core operands.
 *   - Supported shapes: head_dim == 128; hidden_size and the intermediate sizes
 *     multiples of 64; num_attention_heads a multiple of num_key_value_heads (any group
 *     size: decode steps serve a group's queries eight per block); MoE: at most 256
 *     experts and 8 experts per token.
 *
 * KV cache (per layer, caller-owned, bf16), tiled by 32 positions (head_dim = 128):
 *   k  [batch][num_key_value_heads][capacity/32][4][32][32]
 *        tile, 32-dim chunk, position in the tile, dim in the chunk:
 *        K(b, h, pos, d) at (((b*nkv + h)*(capacity/32) + pos/32)*4 + d/32)*1024
 *                           + (pos%32)*32 + d%32
 *   vt [batch][num_key_value_heads][capacity/32][128][32]
 *        tile, dim, position in the tile:
 *        V(b, h, pos, d) at (((b*nkv + h)*(capacity/32) + pos/32)*128 + d)*32 + pos%32
 *   Keys are stored after q/k-norm and RoPE, values as projected ([P3] "GQA 注意力":
 *   the cache keeps normalised, rotated K).  A 32-position tile is 8 KB of K and 8 KB of
 *   V in the operand order of the decode attention's matrix-core loads, so each of its
 *   loads reads whole 128-byte lines.
 *   capacity must be a multiple of 64 and at most max_position_embeddings rounded
 *   up to 64.
 */
#ifndef QWEN3_H
#define QWEN3_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes. */
#define QWEN3_OK 0
#define QWEN3_EINVAL (-1)       /* bad pointer, shape or size */
#define QWEN3_EUNSUPPORTED (-2) /* valid but not implemented (e.g. head_dim != 128) */
#define QWEN3_ERANGE (-3)       /* positions beyond the cache or max_position_embeddings */
#define QWEN3_EWORKSPACE (-4)   /* workspace missing or too small */
#define QWEN3_EHIP (-5)         /* a HIP launch failed */

/* Model configuration; field names follow the Hugging Face config.json
 * ([P3] config table; [P1] section 2 config; [P4] Qwen3Config). */
typedef struct qwen3_config {
  int32_t hidden_size;             /* H, e.g. 1024 */
  int32_t num_attention_heads;     /* nq, e.g. 16 */
  int32_t num_key_value_heads;     /* nkv, e.g. 8; nq % nkv == 0 */
  int32_t head_dim;                /* hd, independent of H; must be 128 */
  int32_t intermediate_size;       /* dense SwiGLU width I, e.g. 3072 */
  int32_t num_hidden_layers;       /* L (stack only) */
  int32_t vocab_size;              /* V (stack only) */
  int32_t max_position_embeddings; /* largest position + 1, e.g. 40960 */
  float rms_norm_eps;              /* 1e-6 */
  float rope_theta;                /* RoPE base, 1e6 */
  int32_t qk_norm;                 /* 1: per-head RMSNorm of q and k before RoPE */
  int32_t tie_word_embeddings;     /* 1: LM head reuses embed_tokens */
  int32_t num_experts;             /* E (MoE only) */
  int32_t num_experts_per_tok;     /* k (MoE only), 1 <= k <= min(E, 8) */
  int32_t moe_intermediate_size;   /* I_moe (MoE only) */
  int32_t norm_topk_prob;          /* 1: renormalise the k selected probabilities */
  int32_t rope_interleaved;        /* RoPE pairing. 0: planes (i, i + hd/2) (rotate-half,
                                      Qwen3 "RoPE" section of the build-it-yourself pages);
                                      1: planes (2i, 2i + 1) (the complex-number form of
                                      the first page's RoPE section). Other values: EINVAL */
  int32_t decoder_sparse_step;     /* stack: layer l runs the routed MoE FFN (num_experts,
                                      num_experts_per_tok, moe_intermediate_size,
                                      norm_topk_prob) when num_experts > 0 and
                                      (l + 1) % decoder_sparse_step == 0 (the first page's
                                      Qwen-MoE config); 0: every layer dense. The block entry
                                      points always run the dense FFN. */
  int32_t router_weights_bf16;     /* routed FFN: 1 rounds the fp32 softmax probabilities to
                                      bf16, selects the largest rounded values (lower expert
                                      first on ties) and uses them as the weights (the first
                                      page's MoE section); 0: fp32 selection and weights */
} qwen3_config;

/* One decoder layer's weights (device, bf16). */
typedef struct qwen3_layer_weights {
  const void *input_layernorm;          /* [H] */
  const void *q_proj;                   /* [nq*hd, H] */
  const void *k_proj;                   /* [nkv*hd, H] */
  const void *v_proj;                   /* [nkv*hd, H] */
  const void *q_norm;                   /* [hd]  (read only when qk_norm) */
  const void *k_norm;                   /* [hd] */
  const void *o_proj;                   /* [H, nq*hd] */
  const void *post_attention_layernorm; /* [H] */
  const void *gate_proj;                /* [I, H] */
  const void *up_proj;                  /* [I, H] */
  const void *down_proj;                /* [H, I] */
  /* routed layers of the stack (see decoder_sparse_step); such a layer needs only these
     three for its FFN (gate_proj, up_proj, down_proj may be NULL there) */
  const void *router;                   /* [E, H] */
  const void *experts_gate_up_proj;     /* [E, 2*I_moe, H]; rows [0, I_moe) gate, rest up */
  const void *experts_down_proj;        /* [E, H, I_moe] */
} qwen3_layer_weights;

/* Whole-model weights. `layers` is a HOST array of num_hidden_layers entries. */
typedef struct qwen3_model_weights {
  const void *embed_tokens;              /* [V, H] bf16 */
  const void *norm;                      /* [H] final RMSNorm weight */
  const void *lm_head;                   /* [V, H]; ignored when tie_word_embeddings */
  const qwen3_layer_weights *layers;     /* host array [L] */
} qwen3_model_weights;

/* Routed-MoE FFN weights ([P3] "MoE": fused gate_up_proj, experts along dim 0). */
typedef struct qwen3_moe_weights {
  const void *router;       /* [E, H] bf16 (the MoE "gate" linear) */
  const void *gate_up_proj; /* [E, 2*I_moe, H] bf16; rows [0, I_moe) gate, [I_moe, 2 I_moe) up */
  const void *down_proj;    /* [E, H, I_moe] bf16 */
} qwen3_moe_weights;

/* One layer's KV cache (see layout above). */
typedef struct qwen3_kv_layer {
  void *k;          /* [B][nkv][capacity/32][4][32][32] bf16 (tiled, see above) */
  void *vt;         /* [B][nkv][capacity/32][hd][32] bf16 (tiled, see above) */
  int32_t capacity; /* positions per sequence, multiple of 64 */
  int32_t regions;  /* (sequence, kv head) regions of capacity * hd elements that k and vt
                       each hold; a call on `batch` sequences needs batch * num_key_value_heads
                       of them (else QWEN3_EINVAL, nothing enqueued) */
} qwen3_kv_layer;

/* Operation selector for qwen3_workspace_bytes. */
#define QWEN3_OP_BLOCK_PREFILL 1
#define QWEN3_OP_BLOCK_DECODE 2
#define QWEN3_OP_MOE_FFN 3
#define QWEN3_OP_STACK_PREFILL 4
#define QWEN3_OP_STACK_DECODE 5
#define QWEN3_OP_GENERATE 6 /* qwen3_generate: batch, seq_len = prompt length */

/* Logits selection for qwen3_stack_forward. */
#define QWEN3_LOGITS_NONE 0 /* no logits (next_ids still allowed) */
#define QWEN3_LOGITS_ALL 1  /* [B][S][V]: every position */
#define QWEN3_LOGITS_LAST 2 /* [B][V]: last position of each sequence */

/* Bytes of workspace needed by `op` for `batch` sequences of `seq_len` new tokens
 * (QWEN3_OP_MOE_FFN: batch = number of tokens, seq_len ignored; QWEN3_OP_BLOCK_DECODE: one
 * token per sequence; QWEN3_OP_STACK_DECODE: seq_len new tokens per sequence, at least 1;
 * decode sizes hold for any cache capacity up to max_position_embeddings).  Returns 0 for
 * an invalid configuration (qwen3_last_error() says why). */
size_t qwen3_workspace_bytes(const qwen3_config *cfg, int32_t op, int32_t batch,
                             int32_t seq_len);

/* Fill the RoPE table ([P3] "RoPE": per-position cos/sin of pos * theta_i with
 * theta_i = rope_theta^(-2i/hd), i < hd/2, precomputed up to max_position_embeddings).
 * rope: device fp32 [2][max_position_embeddings][hd/2]; cos block first, then sin.
 * Values are computed in fp64 on the device and rounded once to fp32. */
int qwen3_rope_table_init(const qwen3_config *cfg, float *rope, void *stream);

/* Copies between plain K / V tensors of one layer, bf16 [batch][num_key_value_heads][len][128]
 * (one row of head_dim values per position, the pages' cache tensors: [P3] "prefill 与
 * decode"), and the tiled cache above.  Positions [0, len) of each (sequence, kv head)
 * region are copied; the cache's other positions are not touched.
 *   qwen3_kv_pack:   k_plain, v_plain -> cache
 *   qwen3_kv_unpack: cache -> k_plain, v_plain
 * All pointers are device memory, 16-byte aligned (k_plain / v_plain may be NULL when
 * len is 0); 0 <= len <= capacity (ERANGE otherwise); the cache needs batch *
 * num_key_value_heads regions.  Enqueued on `stream`. */
int qwen3_kv_pack(const qwen3_config *cfg, const void *k_plain, const void *v_plain,
                  int32_t batch, int32_t len, const qwen3_kv_layer *cache, void *stream);
int qwen3_kv_unpack(const qwen3_config *cfg, const qwen3_kv_layer *cache, int32_t batch,
                    int32_t len, void *k_plain, void *v_plain, void *stream);

/* One pre-norm decoder block, prefill of `seq_len` new tokens for each of `batch`
 * sequences that all start at absolute position pos0 ([P3] "TransformerBlock",
 * "GQA 注意力", "prefill 与 decode"; [P4] decoder layer):
 *   h1 = x + o_proj(attn(rope(qk_norm(split_heads(rmsnorm(x) W_qkv^T)))))
 *   x_out = h1 + down(silu(gate(rmsnorm(h1))) * up(rmsnorm(h1)))
 * Query row s (absolute position pos0+s) attends to keys 0..pos0+s: positions < pos0 are
 * read from `cache`, the new keys/values are written into it at [pos0, pos0+seq_len).
 *   x_in, x_out: bf16 [batch][seq_len][H] (may not alias)
 *   rope: table from qwen3_rope_table_init
 *   cache: holds the new K/V; pos0 + seq_len <= capacity and <= max_position_embeddings,
 *          else QWEN3_ERANGE.  NULL: no earlier positions and nothing kept (pos0 must be 0,
 *          else QWEN3_EINVAL; seq_len <= max_position_embeddings): the call's keys and
 *          values live in the workspace, which qwen3_workspace_bytes sizes for this. */
int qwen3_block_prefill(const qwen3_config *cfg, const qwen3_layer_weights *w,
                        const float *rope, const void *x_in, void *x_out, int32_t batch,
                        int32_t seq_len, int32_t pos0, const qwen3_kv_layer *cache,
                        void *workspace, size_t workspace_bytes, void *stream);

/* One decoder block, decode step: one new token per sequence at its own position
 * ([P3] "prefill 与 decode": the new token sees all cached positions and itself).
 *   x_in, x_out: bf16 [batch][H]
 *   pos: DEVICE int32 [batch]; the token of sequence b is written to cache slot pos[b]
 *        and attends to slots 0..pos[b].  A position outside [0, min(capacity,
 *        max_position_embeddings)) is not written and yields a NaN output row. */
int qwen3_block_decode(const qwen3_config *cfg, const qwen3_layer_weights *w,
                       const float *rope, const void *x_in, void *x_out, int32_t batch,
                       const int32_t *pos, const qwen3_kv_layer *cache, void *workspace,
                       size_t workspace_bytes, void *stream);

/* Allocation-free block decode, for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid allocation): the same
 * operation, arguments and results as qwen3_block_decode, but its scratch memory is the
 * library's static device buffer of QWEN3_STATIC_SCRATCH_BYTES per GPU instead of a caller
 * workspace.  It calls no allocator.  A call whose scratch need (qwen3_workspace_bytes
 * with QWEN3_OP_BLOCK_DECODE for this batch and cache capacity) exceeds the buffer returns
 * QWEN3_EWORKSPACE with nothing enqueued.  The buffer is looked up on the current device
 * on its first call there.  Every call on one GPU shares that GPU's buffer: calls that
 * may overlap in time on one GPU (other streams, other threads) race and must be
 * serialised by the caller.  The kernels write every scratch byte before reading it
 * within a call, so nothing needs clearing between calls. */
#define QWEN3_STATIC_SCRATCH_BYTES (16u << 20)
int qwen3_block_decode_static(const qwen3_config *cfg, const qwen3_layer_weights *w,
                              const float *rope, const void *x_in, void *x_out, int32_t batch,
                              const int32_t *pos, const qwen3_kv_layer *cache, void *stream);

/* Routed MoE FFN sub-layer on already-normalised inputs ([P3] "MoE"):
 *   r = x Wr^T (fp32); the k experts with the largest r are chosen (descending, ties to
 *   the lower index); w = their softmax probabilities, renormalised over the k when
 *   norm_topk_prob; y = sum_j w_j down_e(silu(gate_e x) * up_e x).  No residual.
 *   x: bf16 [n_tokens][H]; y: bf16 [n_tokens][H]
 * Optional outputs (device, may be NULL):
 *   router_logits fp32 [T][E]; topk_idx int32 [T][k]; topk_w fp32 [T][k];
 *   expert_offsets int32 [E+1] (rows of expert e are [off[e], off[e+1]) of the
 *   dispatch order); perm_token int32 [T*k] (token of each dispatch row; experts
 *   ascending, tokens ascending within an expert); inv_row int32 [T][k]. */
int qwen3_moe_ffn(const qwen3_config *cfg, const qwen3_moe_weights *w, const void *x, void *y,
                  int32_t n_tokens, float *router_logits, int32_t *topk_idx, float *topk_w,
                  int32_t *expert_offsets, int32_t *perm_token, int32_t *inv_row,
                  void *workspace, size_t workspace_bytes, void *stream);

/* Whole model ([P3] "骨架"; [P1] sections 12-13): embedding gather, num_hidden_layers
 * blocks with an fp32 residual stream, final RMSNorm, LM head (tied unless
 * tie_word_embeddings == 0), optional greedy argmax.
 *   ids: device int32 [batch][seq_len], each in [0, V) (an out-of-range id gives a NaN row)
 *   pos == NULL: prefill of every sequence from position pos0 (pos0 + seq_len <= capacity,
 *     <= max_position_embeddings).
 *   pos != NULL: decode of seq_len new tokens per sequence; token s of sequence b takes
 *     position pos[b] + s (device int32 [batch]) and sees cache slots 0 .. pos[b] - 1 and
 *     the new tokens 0 .. s ([P3] "prefill 与 decode", [P2] section 4's mask slice).  A
 *     sequence with pos[b] < 0 or pos[b] + seq_len beyond the capacity or
 *     max_position_embeddings is not written and yields NaN rows; seq_len itself must fit
 *     the capacity (ERANGE).
 *   caches: HOST array [L] of per-layer caches (required).
 *   logits: fp32, layout by logits_mode (NULL only with QWEN3_LOGITS_NONE).
 *   next_ids: device int32 [batch] (nullable): argmax of each sequence's last-position
 *             logits, lowest index on ties ([P1] section 13; [P4] greedy generation). */
int qwen3_stack_forward(const qwen3_config *cfg, const qwen3_model_weights *w,
                        const float *rope, const int32_t *ids, int32_t batch, int32_t seq_len,
                        int32_t pos0, const int32_t *pos, const qwen3_kv_layer *caches,
                        float *logits, int32_t logits_mode, int32_t *next_ids, void *workspace,
                        size_t workspace_bytes, void *stream);

/* Generation on the device (the pages' generation loops, [P3] and [P4]; [P1] section 13):
 * a prefill of prompt_ids [batch][prompt_len] (device int32, positions 0..prompt_len-1)
 * picks token 0 of each sequence from its last-position logits; then n_new - 1 decode steps
 * each feed the previous token back at position prompt_len + i - 1 and pick token i.
 * All steps run on `stream` without host synchronisation.
 *   temperature == 0: greedy, the largest logit, lowest index on ties (uniforms unused).
 *   temperature > 0: e_v = exp((l_v - max) / temperature); the nucleus keeps every token with
 *     e_v >= tau, tau the largest value whose kept mass reaches top_p (in (0, 1]) of the
 *     total; r = u * kept mass; the token is the smallest index v whose running kept mass
 *     over tokens <= v exceeds r.  uniforms: device float [n_new][batch] in [0, 1), the
 *     caller's random numbers (u for step i, sequence b at uniforms[i * batch + b]).
 *     e_v is computed in fp32 and the masses are summed exactly in fixed point (units of
 *     2^-44, e_v <= 1), so the draw does not depend on the order of any sum.
 *   caches: HOST array [L] of per-layer caches (one capacity, >= prompt_len + n_new - 1,
 *     <= max_position_embeddings); positions 0 .. prompt_len + n_new - 2 are written.
 *   out_ids: device int32 [batch][n_new].
 *   workspace: qwen3_workspace_bytes(cfg, QWEN3_OP_GENERATE, batch, prompt_len) bytes.
 * Errors as for qwen3_stack_forward; EINVAL for temperature < 0, top_p outside (0, 1],
 * missing uniforms, or vocab_size above 262144 when sampling. */
int qwen3_generate(const qwen3_config *cfg, const qwen3_model_weights *w, const float *rope,
                   const int32_t *prompt_ids, int32_t batch, int32_t prompt_len, int32_t n_new,
                   const qwen3_kv_layer *caches, float temperature, float top_p,
                   const float *uniforms, int32_t *out_ids, void *workspace,
                   size_t workspace_bytes, void *stream);

/* Opt-in kernel timing for measurement tools.  qwen3_profile_begin(tag, n) makes the
 * next (up to n) launches of the kernel class `tag` record a pair of HIP events on their
 * launch stream (tags: "qkv_gemm", "qk_norm_rope_cache", "attn_prefill", "attn_decode",
 * "attn_decode_combine", "o_proj_gemm", "gate_up_gemm", "down_gemm", "lm_head_gemm", "argmax",
 * "moe_router_gemm", "moe_route", "moe_gate_up_gemm", "moe_down_gemm", "moe_combine",
 * "sample").
 * It creates 2n host-side event objects once (not on the forward path).
 * qwen3_profile_end() stops recording; after the caller has synchronised the stream it
 * returns the summed duration (ms) and the number of timed launches. */
int qwen3_profile_begin(const char *tag, int32_t max_launches);
int qwen3_profile_end(float *total_ms, int32_t *launches);

/* Text for a status code. */
const char *qwen3_status_string(int status);

/* Description of the last failure on the calling thread ("" if none). */
const char *qwen3_last_error(void);

#ifdef __cplusplus
}
#endif
#endif
