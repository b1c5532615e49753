// libqwen3 C ABI: argument validation, workspace layout and launch sequencing.
// Nothing here allocates or synchronises; every kernel goes on the caller's stream.
#include <stdarg.h>
#include <stdio.h>

#include <algorithm>
#include <mutex>
#include <string>

#include "../../include/qwen3.h"
#include "launch.h"

using namespace q3;
using gemm::Args;

namespace {

thread_local std::string g_err;

// ---------------------------------------------------------------- opt-in kernel timing
// When enabled for a tag, every launch carrying that tag is bracketed by a pair of HIP
// events recorded on the launch stream.  Events are created once, when enabled.
struct Profiler {
  std::string tag;
  int cap = 0, used = 0;
  bool on = false;
  hipEvent_t* ev = nullptr;  // 2 * cap events
};
Profiler g_prof;

struct ProfScope {
  hipStream_t s;
  bool active;
  ProfScope(const char* tag, hipStream_t st) : s(st), active(false) {
    if (g_prof.on && g_prof.used < g_prof.cap && g_prof.tag == tag) {
      hipEventRecord(g_prof.ev[2 * g_prof.used], s);
      active = true;
    }
  }
  ~ProfScope() {
    if (active) {
      hipEventRecord(g_prof.ev[2 * g_prof.used + 1], s);
      ++g_prof.used;
    }
  }
};

int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return code;
}

#define CHECK_HIP(expr)                                                                  \
  do {                                                                                   \
    hipError_t e_ = (expr);                                                              \
    if (e_ != hipSuccess) return fail(QWEN3_EHIP, "%s: %s", #expr, hipGetErrorString(e_)); \
  } while (0)

bool aligned16(const void* p) { return p && ((uintptr_t)p & 15u) == 0; }

#define REQ_PTR(p, name)                                                                  \
  do {                                                                                    \
    if (!aligned16(p)) return fail(QWEN3_EINVAL, "%s is NULL or not 16-byte aligned", name); \
  } while (0)

// ---------------------------------------------------------------- workspace layout
struct Bump {
  size_t off = 0;
  size_t take(size_t bytes) {
    size_t o = off;
    off += (bytes + 255) & ~(size_t)255;
    return o;
  }
};

struct MoeLayout {
  size_t logits, idx, w, chunk_counts, counts, offsets, perm, inv, tile_e, tile_r, tile_n, act,
      yrows;
  size_t total;
  int max_tiles, tile_m;
};

MoeLayout moe_layout(const qwen3_config* c, int T) {
  MoeLayout L{};
  const int E = c->num_experts, k = c->num_experts_per_tok, H = c->hidden_size,
            I = c->moe_intermediate_size;
  L.tile_m = 256;
  L.max_tiles = (int)(((int64_t)T * k + L.tile_m - 1) / L.tile_m) + E;
  Bump b;
  L.logits = b.take((size_t)T * E * 4);
  L.idx = b.take((size_t)T * k * 4);
  L.w = b.take((size_t)T * k * 4);
  L.chunk_counts = b.take((size_t)moe_route_chunks(T) * E * 4);
  L.counts = b.take((size_t)E * 4);
  L.offsets = b.take((size_t)(E + 1) * 4);
  L.perm = b.take((size_t)T * k * 4);
  L.inv = b.take((size_t)T * k * 4);
  L.tile_e = b.take((size_t)L.max_tiles * 4);
  L.tile_r = b.take((size_t)L.max_tiles * 4);
  L.tile_n = b.take(4);
  L.act = b.take((size_t)T * k * I * 2);
  L.yrows = b.take((size_t)T * k * H * 4);
  L.total = b.off;
  return L;
}

// Stack layer l runs the routed MoE FFN when the config has experts and
// (l + 1) % decoder_sparse_step == 0.
bool has_routed(const qwen3_config* c) { return c->num_experts > 0 && c->decoder_sparse_step > 0; }
bool routed_layer(const qwen3_config* c, int l) {
  return has_routed(c) && (l + 1) % c->decoder_sparse_step == 0;
}

struct DenseLayout {
  size_t xn, qkv, q, attn, h1, act, res, hf, part_attn, part_res, am_val, am_idx, lg_scratch;
  size_t moe;      // stack with routed layers: the MoE FFN's workspace (layout ml)
  MoeLayout ml;
  size_t kf, vtf;  // prefill: fp16 copies of the new keys / values
  size_t own_k, own_vt;  // block prefill without a caller cache: a cache of own_cap positions
  int own_cap;
  size_t total;
  int T, rows_out, attn_splits, attn_chunk, am_chunks, fresh_w_max;
};

constexpr int kArgmaxChunks = 64;


// op: block prefill / decode (bf16 block I/O) or stack prefill / decode
DenseLayout dense_layout(const qwen3_config* c, int op, int B, int S, int cap_hint) {
  DenseLayout L{};
  const bool decode = op == QWEN3_OP_BLOCK_DECODE || op == QWEN3_OP_STACK_DECODE;
  const bool stack = op == QWEN3_OP_STACK_PREFILL || op == QWEN3_OP_STACK_DECODE;
  const int T = B * S;  // decode: S new tokens per sequence
  const int H = c->hidden_size, nq = c->num_attention_heads, nkv = c->num_key_value_heads,
            hd = c->head_dim, I = c->intermediate_size;
  L.T = T;
  Bump b;
  L.xn = b.take((size_t)T * H * 2);
  L.qkv = b.take((size_t)T * (nq + 2 * nkv) * hd * 2);
  L.q = b.take((size_t)T * nq * hd * 2);
  L.attn = b.take((size_t)T * nq * hd * 2);
  L.act = b.take((size_t)T * I * 2);
  L.h1 = stack ? 0 : b.take((size_t)T * H * 4);
  L.res = stack ? b.take((size_t)T * H * 4) : 0;
  if (!decode) {
    L.fresh_w_max = ((S + 63 + 63) / 64) * 64;
    L.kf = b.take((size_t)B * nkv * L.fresh_w_max * hd * 2);
    L.vtf = b.take((size_t)B * nkv * L.fresh_w_max * hd * 2);
  }
  if (op == QWEN3_OP_BLOCK_PREFILL) {
    L.own_cap = ((S + 63) / 64) * 64;
    L.own_k = b.take((size_t)B * nkv * L.own_cap * hd * 2);
    L.own_vt = b.take((size_t)B * nkv * L.own_cap * hd * 2);
  }
  if (decode) {
    attn_decode_plan(cap_hint, B * attn_decode_groups(S, nq / nkv), nkv, L.attn_splits,
                     L.attn_chunk);
    L.part_attn = b.take((size_t)T * nq * L.attn_splits * (hd + 2) * 4);
  }
  {
    // K-split partial sums of the residual projections (decode sizes only)
    const int so = gemm_plan(T, H, nq * hd, gemm::B_DENSE, gemm::E_RES_F32, false).k_splits;
    const int sd = gemm_plan(T, H, I, gemm::B_DENSE, gemm::E_RES_F32, false).k_splits;
    const int sm = std::max(so, sd);
    L.part_res = sm > 1 ? b.take((size_t)sm * T * H * 4) : 0;
  }
  if (stack && has_routed(c)) {
    L.ml = moe_layout(c, T);
    L.moe = b.take(L.ml.total);
  }
  if (stack) {
    L.rows_out = T;  // upper bound: ALL mode needs every row normalised
    L.hf = b.take((size_t)T * H * 2);
    L.am_chunks = kArgmaxChunks;
    L.am_val = b.take((size_t)B * kArgmaxChunks * 4);
    L.am_idx = b.take((size_t)B * kArgmaxChunks * 4);
    L.lg_scratch = b.take((size_t)B * c->vocab_size * 4);
  }
  L.total = b.off;
  return L;
}

// Generation workspace: per-step buffers, then one region shared by the prefill and the
// decode steps of the stack.
struct GenLayout {
  size_t logits, ids, pos, samp, stack, total;
  DenseLayout prefill, decode;
};

GenLayout gen_layout(const qwen3_config* c, int B, int S, int cap) {
  GenLayout G{};
  Bump b;
  G.logits = b.take((size_t)B * c->vocab_size * 4);
  G.ids = b.take((size_t)B * 4);
  G.pos = b.take((size_t)B * 4);
  G.samp = b.take(sample_ws_bytes(B));
  G.stack = b.off;
  G.prefill = dense_layout(c, QWEN3_OP_STACK_PREFILL, B, S, cap);
  G.decode = dense_layout(c, QWEN3_OP_STACK_DECODE, B, 1, cap);
  G.total = G.stack + std::max(G.prefill.total, G.decode.total);
  return G;
}


// ---------------------------------------------------------------- validation
int check_dense_cfg(const qwen3_config* c) {
  if (!c) return fail(QWEN3_EINVAL, "cfg is NULL");
  if (c->head_dim != 128)
    return fail(QWEN3_EUNSUPPORTED, "head_dim=%d: only 128 is supported", c->head_dim);
  if (c->hidden_size <= 0 || c->hidden_size % 64)
    return fail(QWEN3_EUNSUPPORTED, "hidden_size=%d must be a positive multiple of 64",
                c->hidden_size);
  if (c->intermediate_size <= 0 || c->intermediate_size % 64)
    return fail(QWEN3_EUNSUPPORTED, "intermediate_size=%d must be a positive multiple of 64",
                c->intermediate_size);
  if (c->num_attention_heads <= 0 || c->num_key_value_heads <= 0)
    return fail(QWEN3_EINVAL, "num_attention_heads and num_key_value_heads must be positive");
  if (c->num_attention_heads % c->num_key_value_heads)
    return fail(QWEN3_EINVAL, "num_attention_heads=%d is not a multiple of num_key_value_heads=%d",
                c->num_attention_heads, c->num_key_value_heads);
  if (c->max_position_embeddings <= 0)
    return fail(QWEN3_EINVAL, "max_position_embeddings=%d", c->max_position_embeddings);
  if (!(c->rms_norm_eps >= 0.f)) return fail(QWEN3_EINVAL, "rms_norm_eps must be >= 0");
  if (!(c->rope_theta > 0.f)) return fail(QWEN3_EINVAL, "rope_theta must be > 0");
  if (c->rope_interleaved != 0 && c->rope_interleaved != 1)
    return fail(QWEN3_EINVAL, "rope_interleaved=%d must be 0 or 1", c->rope_interleaved);
  return QWEN3_OK;
}

int check_layer(const qwen3_config* c, const qwen3_layer_weights* w, bool routed = false) {
  if (!w) return fail(QWEN3_EINVAL, "layer weights are NULL");
  REQ_PTR(w->input_layernorm, "input_layernorm");
  REQ_PTR(w->q_proj, "q_proj");
  REQ_PTR(w->k_proj, "k_proj");
  REQ_PTR(w->v_proj, "v_proj");
  if (c->qk_norm) {
    REQ_PTR(w->q_norm, "q_norm");
    REQ_PTR(w->k_norm, "k_norm");
  }
  REQ_PTR(w->o_proj, "o_proj");
  REQ_PTR(w->post_attention_layernorm, "post_attention_layernorm");
  if (routed) {
    REQ_PTR(w->router, "router");
    REQ_PTR(w->experts_gate_up_proj, "experts_gate_up_proj");
    REQ_PTR(w->experts_down_proj, "experts_down_proj");
  } else {
    REQ_PTR(w->gate_proj, "gate_proj");
    REQ_PTR(w->up_proj, "up_proj");
    REQ_PTR(w->down_proj, "down_proj");
  }
  return QWEN3_OK;
}

int check_moe_cfg(const qwen3_config* c) {
  const int E = c->num_experts, k = c->num_experts_per_tok, H = c->hidden_size,
            I = c->moe_intermediate_size;
  if (E <= 0 || E > 256) return fail(QWEN3_EUNSUPPORTED, "num_experts=%d must be in [1, 256]", E);
  if (k <= 0 || k > 8 || k > E)
    return fail(QWEN3_EUNSUPPORTED, "num_experts_per_tok=%d must be in [1, min(E, 8)]", k);
  if (H <= 0 || H % 64) return fail(QWEN3_EUNSUPPORTED, "hidden_size=%d must be a multiple of 64", H);
  if (I <= 0 || I % 64)
    return fail(QWEN3_EUNSUPPORTED, "moe_intermediate_size=%d must be a multiple of 64", I);
  if (c->router_weights_bf16 != 0 && c->router_weights_bf16 != 1)
    return fail(QWEN3_EINVAL, "router_weights_bf16=%d must be 0 or 1", c->router_weights_bf16);
  return QWEN3_OK;
}

int check_cache(const qwen3_config* c, const qwen3_kv_layer* kv, const char* what, int batch) {
  if (!kv) return fail(QWEN3_EINVAL, "%s: cache is NULL", what);
  if ((int64_t)batch * c->num_key_value_heads > kv->regions)
    return fail(QWEN3_EINVAL,
                "%s: regions=%d is fewer than batch x num_key_value_heads = %lld "
                "(sequence, kv head) regions", what, kv->regions,
                (long long)batch * c->num_key_value_heads);
  if (!aligned16(kv->k) || !aligned16(kv->vt))
    return fail(QWEN3_EINVAL, "%s: cache k/vt NULL or not 16-byte aligned", what);
  if (kv->capacity <= 0 || kv->capacity % 64)
    return fail(QWEN3_EINVAL, "%s: capacity=%d must be a positive multiple of 64", what,
                kv->capacity);
  if (kv->capacity > ((c->max_position_embeddings + 63) / 64) * 64)
    return fail(QWEN3_EINVAL, "%s: capacity=%d exceeds max_position_embeddings rounded up to 64",
                what, kv->capacity);
  return QWEN3_OK;
}

int check_range(const qwen3_config* c, const qwen3_kv_layer* kv, int pos0, int S) {
  if (pos0 < 0) return fail(QWEN3_ERANGE, "pos0=%d is negative", pos0);
  if ((int64_t)pos0 + S > kv->capacity)
    return fail(QWEN3_ERANGE, "pos0 + seq_len = %lld exceeds cache capacity %d",
                (long long)pos0 + S, kv->capacity);
  if ((int64_t)pos0 + S > c->max_position_embeddings)
    return fail(QWEN3_ERANGE, "pos0 + seq_len = %lld exceeds max_position_embeddings %d",
                (long long)pos0 + S, c->max_position_embeddings);
  return QWEN3_OK;
}

#define TRY(x)                  \
  do {                          \
    int rc_ = (x);              \
    if (rc_ != QWEN3_OK) return rc_; \
  } while (0)

// ---------------------------------------------------------------- one layer
struct LayerIO {
  int T, B, S, pos0;
  const int32_t* pos;  // decode positions (device) or nullptr
  const bf16_t* x_bf16;  // block API input (nullptr in the stack)
  float* res;            // stack residual (in/out) (nullptr in the block API)
  bf16_t* x_out;         // block API output
  bool input_normed;        // stack: xn already holds this layer's normalised input
  const bf16_t* next_norm;  // stack: next layer's input RMSNorm weight (nullptr: none)
};

// Routed MoE FFN ([P3] "MoE"; [P1] section 11 with router_weights_bf16): router GEMM,
// top-k routing and dispatch order, grouped gate|up + SwiGLU, grouped down, weighted
// combine (plus the residual when given).  Arguments are checked by the callers.
struct MoeIO {
  const void* x;  // [T][H] input rows: the caller's bf16 tokens or fp16 normalised rows
  bool x_f16;
  int T;
  const float* residual;  // nullable: out = residual + moe(x)
  void* out;              // [T][H], fp32 or bf16 (may be the residual itself)
  bool out_f32;
  // optional outputs (nullptr: workspace)
  float* lg;
  int32_t* idx;
  float* wt;
  int32_t* offs;
  int32_t* perm;
  int32_t* inv;
};

int moe_run(const qwen3_config* c, const void* router, const void* gate_up, const void* down,
            const MoeIO& io, char* ws, const MoeLayout& L, hipStream_t s) {
  const int T = io.T;
  const int E = c->num_experts, k = c->num_experts_per_tok, H = c->hidden_size,
            I = c->moe_intermediate_size;
  float* lg = io.lg ? io.lg : (float*)(ws + L.logits);
  int32_t* idx = io.idx ? io.idx : (int32_t*)(ws + L.idx);
  float* wt = io.wt ? io.wt : (float*)(ws + L.w);
  int32_t* offs = io.offs ? io.offs : (int32_t*)(ws + L.offsets);
  int32_t* perm = io.perm ? io.perm : (int32_t*)(ws + L.perm);
  int32_t* inv = io.inv ? io.inv : (int32_t*)(ws + L.inv);
  int32_t* tile_e = (int32_t*)(ws + L.tile_e);
  int32_t* tile_r = (int32_t*)(ws + L.tile_r);
  int32_t* tile_n = (int32_t*)(ws + L.tile_n);
  f16_t* act = (f16_t*)(ws + L.act);
  float* yrows = (float*)(ws + L.yrows);

  // router logits (fp32); with few experts the routing kernel forms them itself
  const bool small_router = E <= kRouteSmallE;
  if (!small_router) {
    Args a{};
    a.M = T; a.N = E; a.K = H;
    a.A = (const uint16_t*)io.x; a.lda = H;
    a.B0 = (const bf16_t*)router; a.ldb = H;
    a.C = lg; a.ldc = E;
    GemmPlan p = gemm_plan(a.M, a.N, a.K, gemm::B_DENSE, gemm::E_F32, false);
    ProfScope ps("moe_router_gemm", s);
    CHECK_HIP(gemm_run(a, io.x_f16, gemm::B_DENSE, gemm::E_F32, false, p, s));
  }
  // top-k, weights, dispatch order, tile table
  {
    MoeRouteArgs r{};
    r.logits = lg; r.T = T; r.E = E; r.k = k; r.norm_topk = c->norm_topk_prob;
    r.router_bf16 = c->router_weights_bf16;
    if (small_router) {
      r.x = io.x; r.x_f16 = io.x_f16; r.router = (const bf16_t*)router; r.H = H;
    }
    r.idx = idx; r.w = wt;
    r.chunk_counts = (int32_t*)(ws + L.chunk_counts);
    r.counts = (int32_t*)(ws + L.counts);
    r.offsets = offs; r.perm_token = perm; r.inv_row = inv;
    r.tile_expert = tile_e; r.tile_row0 = tile_r; r.tile_count = tile_n;
    r.max_tiles = L.max_tiles; r.tile_m = L.tile_m;
    ProfScope ps("moe_route", s);
    CHECK_HIP(moe_route(r, s));
  }
  // grouped gate|up + SwiGLU over gathered token rows
  {
    Args a{};
    a.M = T * k; a.N = 2 * I; a.K = H;
    a.A = (const uint16_t*)io.x; a.lda = H; a.a_rows = perm;
    a.B0 = (const bf16_t*)gate_up;
    a.B1 = (const bf16_t*)gate_up + (int64_t)I * H;
    a.ldb = H;
    a.g_offsets = offs; a.g_tile_expert = tile_e; a.g_tile_row0 = tile_r;
    a.g_tile_count = tile_n;
    a.g_b_stride = (int64_t)2 * I * H;
    a.m_tiles = L.max_tiles;
    a.C = act; a.ldc = I;
    GemmPlan p{kBig};
    ProfScope ps("moe_gate_up_gemm", s);
    CHECK_HIP(gemm_run(a, io.x_f16, gemm::B_SWIGLU, gemm::E_SWIGLU, true, p, s));
  }
  // grouped down -> per-row fp32 outputs in dispatch order
  {
    Args a{};
    a.M = T * k; a.N = H; a.K = I;
    a.A = act; a.lda = I;
    a.B0 = (const bf16_t*)down; a.B1 = a.B0; a.ldb = I;
    a.g_offsets = offs; a.g_tile_expert = tile_e; a.g_tile_row0 = tile_r;
    a.g_tile_count = tile_n;
    a.g_b_stride = (int64_t)H * I;
    a.m_tiles = L.max_tiles;
    a.C = yrows; a.ldc = H;
    GemmPlan p{kBig};
    ProfScope ps("moe_down_gemm", s);
    CHECK_HIP(gemm_run(a, true, gemm::B_DENSE, gemm::E_F32, true, p, s));
  }
  {
    ProfScope ps("moe_combine", s);
    CHECK_HIP(moe_combine(yrows, inv, wt, io.residual, io.out, io.out_f32, T, k, H, s));
  }
  return QWEN3_OK;
}

// *next_normed is set when the layer's last reduction also wrote the next layer's
// normalised input into xn (decode sizes, stack only).
int run_layer(const qwen3_config* c, const qwen3_layer_weights* w, const float* rope,
              const qwen3_kv_layer* kv, const LayerIO& io, char* ws, const DenseLayout& L,
              hipStream_t s, bool* next_normed = nullptr, bool routed = false) {
  if (next_normed) *next_normed = false;
  const int H = c->hidden_size, nq = c->num_attention_heads, nkv = c->num_key_value_heads,
            hd = c->head_dim, I = c->intermediate_size, T = io.T;
  // transient activations feeding the matrix cores are fp16
  f16_t* xn = (f16_t*)(ws + L.xn);
  f16_t* qkv = (f16_t*)(ws + L.qkv);
  f16_t* q = (f16_t*)(ws + L.q);
  f16_t* attn = (f16_t*)(ws + L.attn);
  f16_t* act = (f16_t*)(ws + L.act);
  float* h1 = io.res ? io.res : (float*)(ws + L.h1);
  const float eps = c->rms_norm_eps;

  float* part_res = L.part_res ? (float*)(ws + L.part_res) : nullptr;

  // input RMSNorm (unless the previous layer's last reduction produced it)
  if (io.res) {
    if (!io.input_normed)
      CHECK_HIP(rmsnorm_f32(io.res, 1, 0, (const bf16_t*)w->input_layernorm, xn, T, H, eps, s));
  } else {
    CHECK_HIP(rmsnorm_bf16(io.x_bf16, 1, 0, (const bf16_t*)w->input_layernorm, xn, T, H, eps, s));
  }

  // QKV projection (q, k, v weights stacked along N without a copy), rounded to fp16 (4x
  // finer than the bf16 cache the keys end in), then q/k RMSNorm + RoPE and the K/V cache
  // writes: fused into the projection's epilogue for prefill tiles, a separate pass for
  // decode-size products
  RopeCacheArgs r{};
  r.qkv = qkv; r.rope = rope;
  r.q_norm = (const bf16_t*)w->q_norm; r.k_norm = (const bf16_t*)w->k_norm;
  r.q_out = q; r.k_cache = (bf16_t*)kv->k; r.vt_cache = (bf16_t*)kv->vt;
  r.pos = io.pos; r.pos0 = io.pos0; r.B = io.B; r.S = io.S;
  r.nq = nq; r.nkv = nkv; r.cap = kv->capacity; r.max_pos = c->max_position_embeddings;
  r.qk_norm = c->qk_norm; r.eps = eps;
  r.interleaved = c->rope_interleaved;
  if (!io.pos) {
    r.k_fresh = (f16_t*)(ws + L.kf);
    r.vt_fresh = (f16_t*)(ws + L.vtf);
    r.fresh_base = io.pos0 & ~63;
    r.fresh_w = ((io.pos0 + io.S - r.fresh_base + 63) / 64) * 64;
  }
  {
    Args a{};
    a.M = T; a.N = (nq + 2 * nkv) * hd; a.K = H;
    a.A = xn; a.lda = H;
    a.B0 = (const bf16_t*)w->q_proj; a.B1 = (const bf16_t*)w->k_proj;
    a.B2 = (const bf16_t*)w->v_proj; a.ldb = H;
    a.seg1 = nq * hd; a.seg2 = (nq + nkv) * hd;
    a.C = qkv; a.ldc = a.N;
    GemmPlan p = gemm_plan(a.M, a.N, a.K, gemm::B_QKV, gemm::E_F16, false);
    const bool fused = !io.pos && p.tile != kDecode;
    if (fused) {
      gemm::RopeEpi& e = a.re;
      e.table = rope; e.q_norm = r.q_norm; e.k_norm = r.k_norm;
      e.q_out = q; e.k_cache = r.k_cache; e.vt_cache = r.vt_cache;
      e.k_fresh = r.k_fresh; e.vt_fresh = r.vt_fresh;
      e.fresh_base = r.fresh_base; e.fresh_w = r.fresh_w; e.pos0 = io.pos0; e.S = io.S;
      e.nq = nq; e.nkv = nkv; e.cap = kv->capacity; e.max_pos = c->max_position_embeddings;
      e.qk_norm = c->qk_norm; e.interleaved = c->rope_interleaved; e.eps = eps;
      ProfScope ps("qkv_gemm", s);
      CHECK_HIP(gemm_run(a, true, gemm::B_QKV, gemm::E_QKROPE, false, p, s));
    } else {
      {
        ProfScope ps("qkv_gemm", s);
        CHECK_HIP(gemm_run(a, true, gemm::B_QKV, gemm::E_F16, false, p, s));
      }
      ProfScope ps("qk_norm_rope_cache", s);
      CHECK_HIP(qkv_rope_cache(r, s));
    }
  }
  // attention
  if (io.pos) {
    AttnDecodeArgs d{};
    d.q = q; d.k_cache = (const bf16_t*)kv->k; d.vt_cache = (const bf16_t*)kv->vt;
    d.pos = io.pos; d.out = attn; d.part = (float*)(ws + L.part_attn);
    d.B = io.B; d.S = io.S; d.nq = nq; d.nkv = nkv; d.cap = kv->capacity;
    d.max_pos = c->max_position_embeddings;
    d.nqg = attn_decode_groups(io.S, nq / nkv);
    attn_decode_plan(kv->capacity, io.B * d.nqg, nkv, d.splits, d.chunk);
    {
      ProfScope ps("attn_decode", s);
      CHECK_HIP(attn_decode(d, s));
    }
    if (d.splits > 1) {
      ProfScope ps("attn_decode_combine", s);
      CHECK_HIP(attn_decode_combine(d, s));
    }
  } else {
    AttnPrefillArgs p{};
    p.q = q; p.k_cache = (const bf16_t*)kv->k; p.vt_cache = (const bf16_t*)kv->vt;
    p.out = attn; p.B = io.B; p.S = io.S; p.pos0 = io.pos0; p.nq = nq; p.nkv = nkv;
    p.cap = kv->capacity;
    p.k_fresh = (const f16_t*)(ws + L.kf);
    p.vt_fresh = (const f16_t*)(ws + L.vtf);
    p.fresh_base = io.pos0 & ~63;
    p.fresh_w = ((io.pos0 + io.S - p.fresh_base + 63) / 64) * 64;
    ProfScope ps("attn_prefill", s);
    CHECK_HIP(attn_prefill(p, s));
  }
  // o_proj + residual -> h1 (fp32)
  {
    Args a{};
    a.M = T; a.N = H; a.K = nq * hd;
    a.A = attn; a.lda = nq * hd;
    a.B0 = (const bf16_t*)w->o_proj; a.ldb = nq * hd;
    a.C = h1; a.ldc = H;
    int epi = io.res ? gemm::E_RES_F32 : gemm::E_RESB_F32;
    a.R = io.res ? (const void*)io.res : (const void*)io.x_bf16; a.ldr = H;
    GemmPlan p = gemm_plan(a.M, a.N, a.K, gemm::B_DENSE, epi, false);
    if (p.k_splits > 1) {
      // partial sums; then residual add and the post-attention RMSNorm in one pass
      a.partial = part_res;
      {
        ProfScope ps("o_proj_gemm", s);
        CHECK_HIP(gemm_run(a, true, gemm::B_DENSE, epi, false, p, s));
      }
      CHECK_HIP(splitk_res_norm(part_res, p.k_splits, T, H, a.R, io.res == nullptr, h1, false,
                                (const bf16_t*)w->post_attention_layernorm, xn, eps, s));
    } else {
      {
        ProfScope ps("o_proj_gemm", s);
        CHECK_HIP(gemm_run(a, true, gemm::B_DENSE, epi, false, p, s));
      }
      // post-attention RMSNorm
      CHECK_HIP(rmsnorm_f32(h1, 1, 0, (const bf16_t*)w->post_attention_layernorm, xn, T, H,
                            eps, s));
    }
  }
  if (routed) {
    // routed MoE FFN on the normalised rows; the combine adds the residual h1
    MoeIO m{};
    m.x = xn; m.x_f16 = true; m.T = T;
    m.residual = h1;
    m.out = io.res ? (void*)io.res : (void*)io.x_out;
    m.out_f32 = io.res != nullptr;
    return moe_run(c, w->router, w->experts_gate_up_proj, w->experts_down_proj, m,
                   ws + L.moe, L.ml, s);
  }
  // gate | up with SwiGLU
  {
    Args a{};
    a.M = T; a.N = 2 * I; a.K = H;
    a.A = xn; a.lda = H;
    a.B0 = (const bf16_t*)w->gate_proj; a.B1 = (const bf16_t*)w->up_proj; a.ldb = H;
    a.C = act; a.ldc = I;
    GemmPlan p = gemm_plan(a.M, a.N, a.K, gemm::B_SWIGLU, gemm::E_SWIGLU, false);
    ProfScope ps("gate_up_gemm", s);
    CHECK_HIP(gemm_run(a, true, gemm::B_SWIGLU, gemm::E_SWIGLU, false, p, s));
  }
  // down + residual
  {
    Args a{};
    a.M = T; a.N = H; a.K = I;
    a.A = act; a.lda = I;
    a.B0 = (const bf16_t*)w->down_proj; a.ldb = I;
    a.R = h1; a.ldr = H;
    int epi;
    if (io.res) {
      epi = gemm::E_RES_F32;
      a.C = io.res;
    } else {
      epi = gemm::E_RESF_B16;
      a.C = io.x_out;
    }
    a.ldc = H;
    GemmPlan p = gemm_plan(a.M, a.N, a.K, gemm::B_DENSE, epi, false);
    if (p.k_splits > 1) {
      // partial sums; then residual add (and the next layer's input RMSNorm) in one pass
      a.partial = part_res;
      {
        ProfScope ps("down_gemm", s);
        CHECK_HIP(gemm_run(a, true, gemm::B_DENSE, epi, false, p, s));
      }
      const bf16_t* nn = io.res ? io.next_norm : nullptr;
      CHECK_HIP(splitk_res_norm(part_res, p.k_splits, T, H, h1, false, a.C, io.res == nullptr,
                                nn, xn, eps, s));
      if (next_normed) *next_normed = nn != nullptr;
    } else {
      ProfScope ps("down_gemm", s);
      CHECK_HIP(gemm_run(a, true, gemm::B_DENSE, epi, false, p, s));
    }
  }
  return QWEN3_OK;
}

}  // namespace

extern "C" {

const char* qwen3_status_string(int status) {
  switch (status) {
    case QWEN3_OK: return "ok";
    case QWEN3_EINVAL: return "invalid argument";
    case QWEN3_EUNSUPPORTED: return "unsupported configuration";
    case QWEN3_ERANGE: return "position out of range";
    case QWEN3_EWORKSPACE: return "workspace too small";
    case QWEN3_EHIP: return "HIP launch failure";
    default: return "unknown status";
  }
}

const char* qwen3_last_error(void) { return g_err.c_str(); }

int qwen3_profile_begin(const char* tag, int32_t max_launches) {
  g_err.clear();
  if (!tag || max_launches <= 0) return fail(QWEN3_EINVAL, "tag / max_launches");
  if (g_prof.cap < max_launches) {
    for (int i = 0; i < 2 * g_prof.cap; ++i) hipEventDestroy(g_prof.ev[i]);
    delete[] g_prof.ev;
    g_prof.ev = new hipEvent_t[2 * max_launches];
    for (int i = 0; i < 2 * max_launches; ++i) CHECK_HIP(hipEventCreate(&g_prof.ev[i]));
    g_prof.cap = max_launches;
  }
  g_prof.tag = tag;
  g_prof.used = 0;
  g_prof.on = true;
  return QWEN3_OK;
}

int qwen3_profile_end(float* total_ms, int32_t* launches) {
  g_err.clear();
  g_prof.on = false;
  float total = 0.f;
  for (int i = 0; i < g_prof.used; ++i) {
    float ms = 0.f;
    CHECK_HIP(hipEventElapsedTime(&ms, g_prof.ev[2 * i], g_prof.ev[2 * i + 1]));
    total += ms;
  }
  if (total_ms) *total_ms = total;
  if (launches) *launches = g_prof.used;
  return QWEN3_OK;
}

size_t qwen3_workspace_bytes(const qwen3_config* c, int32_t op, int32_t batch, int32_t seq_len) {
  g_err.clear();
  if (batch <= 0) { fail(QWEN3_EINVAL, "batch=%d", batch); return 0; }
  if (op == QWEN3_OP_MOE_FFN) {
    if (!c || c->num_experts <= 0 || c->num_experts_per_tok <= 0) {
      fail(QWEN3_EINVAL, "MoE configuration missing");
      return 0;
    }
    return moe_layout(c, batch).total;
  }
  if (check_dense_cfg(c) != QWEN3_OK) return 0;
  if (op == QWEN3_OP_GENERATE) {
    if (seq_len <= 0) { fail(QWEN3_EINVAL, "seq_len=%d", seq_len); return 0; }
    if (c->vocab_size <= 0) { fail(QWEN3_EINVAL, "vocab_size=%d", c->vocab_size); return 0; }
    int cap = ((c->max_position_embeddings + 63) / 64) * 64;
    return gen_layout(c, batch, seq_len, cap).total;
  }
  if (op == QWEN3_OP_BLOCK_DECODE || op == QWEN3_OP_STACK_DECODE) {
    // decode partials scale with the cache capacity; size for max_position_embeddings.
    // The stack decodes seq_len new tokens per sequence (at least one).
    int cap = ((c->max_position_embeddings + 63) / 64) * 64;
    const int S = op == QWEN3_OP_STACK_DECODE ? std::max(1, (int)seq_len) : 1;
    return dense_layout(c, op, batch, S, cap).total;
  }
  if (op != QWEN3_OP_BLOCK_PREFILL && op != QWEN3_OP_STACK_PREFILL) {
    fail(QWEN3_EINVAL, "unknown op %d", op);
    return 0;
  }
  if (seq_len <= 0) { fail(QWEN3_EINVAL, "seq_len=%d", seq_len); return 0; }
  if (op == QWEN3_OP_STACK_PREFILL && c->vocab_size <= 0) {
    fail(QWEN3_EINVAL, "vocab_size=%d", c->vocab_size);
    return 0;
  }
  return dense_layout(c, op, batch, seq_len, 64).total;
}

int qwen3_rope_table_init(const qwen3_config* c, float* rope, void* stream) {
  g_err.clear();
  if (!c) return fail(QWEN3_EINVAL, "cfg is NULL");
  if (c->head_dim <= 0 || c->head_dim % 2)
    return fail(QWEN3_EINVAL, "head_dim=%d must be positive and even", c->head_dim);
  if (c->max_position_embeddings <= 0)
    return fail(QWEN3_EINVAL, "max_position_embeddings=%d", c->max_position_embeddings);
  if (!(c->rope_theta > 0.f)) return fail(QWEN3_EINVAL, "rope_theta must be > 0");
  REQ_PTR(rope, "rope");
  CHECK_HIP(q3::rope_table(rope, c->max_position_embeddings, c->head_dim, (double)c->rope_theta,
                           (hipStream_t)stream));
  return QWEN3_OK;
}

int qwen3_kv_pack(const qwen3_config* c, const void* k_plain, const void* v_plain,
                  int32_t batch, int32_t len, const qwen3_kv_layer* cache, void* stream) {
  g_err.clear();
  TRY(check_dense_cfg(c));
  if (batch <= 0) return fail(QWEN3_EINVAL, "batch=%d must be positive", batch);
  TRY(check_cache(c, cache, "cache", batch));
  if (len < 0 || len > cache->capacity)
    return fail(QWEN3_ERANGE, "len=%d outside [0, capacity %d]", len, cache->capacity);
  if (len > 0 && (!aligned16(k_plain) || !aligned16(v_plain)))
    return fail(QWEN3_EINVAL, "k_plain / v_plain NULL or not 16-byte aligned");
  CHECK_HIP(kv_copy(const_cast<void*>(k_plain), const_cast<void*>(v_plain), cache->k, cache->vt,
                    batch * c->num_key_value_heads, len, cache->capacity, true,
                    (hipStream_t)stream));
  return QWEN3_OK;
}

int qwen3_kv_unpack(const qwen3_config* c, const qwen3_kv_layer* cache, int32_t batch,
                    int32_t len, void* k_plain, void* v_plain, void* stream) {
  g_err.clear();
  TRY(check_dense_cfg(c));
  if (batch <= 0) return fail(QWEN3_EINVAL, "batch=%d must be positive", batch);
  TRY(check_cache(c, cache, "cache", batch));
  if (len < 0 || len > cache->capacity)
    return fail(QWEN3_ERANGE, "len=%d outside [0, capacity %d]", len, cache->capacity);
  if (len > 0 && (!aligned16(k_plain) || !aligned16(v_plain)))
    return fail(QWEN3_EINVAL, "k_plain / v_plain NULL or not 16-byte aligned");
  CHECK_HIP(kv_copy(k_plain, v_plain, cache->k, cache->vt, batch * c->num_key_value_heads, len,
                    cache->capacity, false, (hipStream_t)stream));
  return QWEN3_OK;
}

int qwen3_block_prefill(const qwen3_config* c, const qwen3_layer_weights* w, const float* rope,
                        const void* x_in, void* x_out, int32_t batch, int32_t seq_len,
                        int32_t pos0, const qwen3_kv_layer* cache, void* workspace,
                        size_t workspace_bytes, void* stream) {
  g_err.clear();
  TRY(check_dense_cfg(c));
  TRY(check_layer(c, w));
  if (batch <= 0 || seq_len <= 0)
    return fail(QWEN3_EINVAL, "batch=%d seq_len=%d must be positive", batch, seq_len);
  REQ_PTR(rope, "rope");
  REQ_PTR(x_in, "x_in");
  REQ_PTR(x_out, "x_out");
  if (x_in == x_out) return fail(QWEN3_EINVAL, "x_in and x_out may not alias");
  if ((int64_t)batch * seq_len > (1 << 30)) return fail(QWEN3_EINVAL, "too many tokens");
  if (cache) {
    TRY(check_cache(c, cache, "cache", batch));
    TRY(check_range(c, cache, pos0, seq_len));
  } else {
    // no cache: the keys and values of this call only, kept in the workspace
    if (pos0 != 0) return fail(QWEN3_EINVAL, "cache is NULL: pos0=%d must be 0", pos0);
    if (seq_len > c->max_position_embeddings)
      return fail(QWEN3_ERANGE, "seq_len=%d exceeds max_position_embeddings %d", seq_len,
                  c->max_position_embeddings);
  }
  DenseLayout L = dense_layout(c, QWEN3_OP_BLOCK_PREFILL, batch, seq_len,
                               cache ? cache->capacity : 0);
  if (!aligned16(workspace) || workspace_bytes < L.total)
    return fail(QWEN3_EWORKSPACE, "workspace needs %zu bytes (got %zu)", L.total,
                workspace_bytes);
  qwen3_kv_layer own{};
  if (!cache) {
    own.k = (char*)workspace + L.own_k;
    own.vt = (char*)workspace + L.own_vt;
    own.capacity = L.own_cap;
    own.regions = batch * c->num_key_value_heads;
  }
  LayerIO io{};
  io.T = batch * seq_len; io.B = batch; io.S = seq_len; io.pos0 = pos0;
  io.x_bf16 = (const bf16_t*)x_in; io.x_out = (bf16_t*)x_out;
  return run_layer(c, w, rope, cache ? cache : &own, io, (char*)workspace, L,
                   (hipStream_t)stream);
}

}  // extern "C"

namespace {

// Argument checks of the block decode entry points; *L receives the workspace layout.
int check_block_decode(const qwen3_config* c, const qwen3_layer_weights* w, const float* rope,
                       const void* x_in, const void* x_out, int32_t batch, const int32_t* pos,
                       const qwen3_kv_layer* cache, DenseLayout* L) {
  TRY(check_dense_cfg(c));
  TRY(check_layer(c, w));
  if (batch <= 0) return fail(QWEN3_EINVAL, "batch=%d must be positive", batch);
  REQ_PTR(rope, "rope");
  REQ_PTR(x_in, "x_in");
  REQ_PTR(x_out, "x_out");
  if (!pos) return fail(QWEN3_EINVAL, "pos is NULL");
  if (x_in == x_out) return fail(QWEN3_EINVAL, "x_in and x_out may not alias");
  TRY(check_cache(c, cache, "cache", batch));
  *L = dense_layout(c, QWEN3_OP_BLOCK_DECODE, batch, 1, cache->capacity);
  return QWEN3_OK;
}

int run_block_decode(const qwen3_config* c, const qwen3_layer_weights* w, const float* rope,
                     const void* x_in, void* x_out, int32_t batch, const int32_t* pos,
                     const qwen3_kv_layer* cache, char* ws, const DenseLayout& L,
                     hipStream_t s) {
  LayerIO io{};
  io.T = batch; io.B = batch; io.S = 1; io.pos = pos;
  io.x_bf16 = (const bf16_t*)x_in; io.x_out = (bf16_t*)x_out;
  return run_layer(c, w, rope, cache, io, ws, L, s);
}

// Scratch of the allocation-free decode entry point: one copy per GPU, resident while the
// library is loaded.  Host code never passes `scratch` itself to a kernel (on the host it
// is only a stand-in for the symbol); it uses the device address that hipGetSymbolAddress
// returns, looked up once per device on the first call there.
static __device__ __align__(256) char scratch[QWEN3_STATIC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

int static_scratch(char** out) {
  int dev = -1;
  CHECK_HIP(hipGetDevice(&dev));
  if (dev < 0 || dev >= kMaxDevices)
    return fail(QWEN3_EUNSUPPORTED, "device %d: at most %d devices", dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    CHECK_HIP(hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)));
    if (!p) return fail(QWEN3_EHIP, "hipGetSymbolAddress(scratch) returned NULL");
    g_scratch_ptr[dev] = p;
  }
  *out = (char*)g_scratch_ptr[dev];
  return QWEN3_OK;
}

}  // namespace

extern "C" {

int qwen3_block_decode(const qwen3_config* c, const qwen3_layer_weights* w, const float* rope,
                       const void* x_in, void* x_out, int32_t batch, const int32_t* pos,
                       const qwen3_kv_layer* cache, void* workspace, size_t workspace_bytes,
                       void* stream) {
  g_err.clear();
  DenseLayout L;
  TRY(check_block_decode(c, w, rope, x_in, x_out, batch, pos, cache, &L));
  if (!aligned16(workspace) || workspace_bytes < L.total)
    return fail(QWEN3_EWORKSPACE, "workspace needs %zu bytes (got %zu)", L.total,
                workspace_bytes);
  return run_block_decode(c, w, rope, x_in, x_out, batch, pos, cache, (char*)workspace, L,
                          (hipStream_t)stream);
}

int qwen3_block_decode_static(const qwen3_config* c, const qwen3_layer_weights* w,
                              const float* rope, const void* x_in, void* x_out, int32_t batch,
                              const int32_t* pos, const qwen3_kv_layer* cache, void* stream) {
  g_err.clear();
  DenseLayout L;
  TRY(check_block_decode(c, w, rope, x_in, x_out, batch, pos, cache, &L));
  if (L.total > (size_t)QWEN3_STATIC_SCRATCH_BYTES)
    return fail(QWEN3_EWORKSPACE,
                "this call needs %zu bytes of scratch; the static scratch holds %zu (use "
                "qwen3_block_decode with a workspace)", L.total,
                (size_t)QWEN3_STATIC_SCRATCH_BYTES);
  char* ws = nullptr;
  TRY(static_scratch(&ws));
  return run_block_decode(c, w, rope, x_in, x_out, batch, pos, cache, ws, L,
                          (hipStream_t)stream);
}

}  // extern "C"

namespace {

// Model-level argument checks shared by the stack forward and generation.
int check_stack(const qwen3_config* c, const qwen3_model_weights* w, const float* rope,
                const qwen3_kv_layer* caches, int batch) {
  TRY(check_dense_cfg(c));
  if (!w) return fail(QWEN3_EINVAL, "model weights are NULL");
  if (c->num_hidden_layers <= 0 || !w->layers)
    return fail(QWEN3_EINVAL, "num_hidden_layers=%d / layers array missing",
                c->num_hidden_layers);
  if (c->vocab_size <= 0) return fail(QWEN3_EINVAL, "vocab_size=%d", c->vocab_size);
  REQ_PTR(w->embed_tokens, "embed_tokens");
  REQ_PTR(w->norm, "norm");
  if (!c->tie_word_embeddings) REQ_PTR(w->lm_head, "lm_head");
  if (c->decoder_sparse_step < 0)
    return fail(QWEN3_EINVAL, "decoder_sparse_step=%d must be >= 0", c->decoder_sparse_step);
  if (has_routed(c)) TRY(check_moe_cfg(c));
  for (int l = 0; l < c->num_hidden_layers; ++l) {
    int rc = check_layer(c, &w->layers[l], routed_layer(c, l));
    if (rc) return fail(rc, "layer %d: %s", l, g_err.c_str());
  }
  REQ_PTR(rope, "rope");
  if (!caches) return fail(QWEN3_EINVAL, "caches is NULL");
  for (int l = 0; l < c->num_hidden_layers; ++l) {
    TRY(check_cache(c, &caches[l], "caches[l]", batch));
    if (caches[l].capacity != caches[0].capacity)
      return fail(QWEN3_EINVAL, "all layers' caches must share one capacity");
  }
  return QWEN3_OK;
}

// Embedding, the layers, final norm, LM head and optional argmax (arguments checked).
int stack_run(const qwen3_config* c, const qwen3_model_weights* w, const float* rope,
              const int32_t* ids, int32_t batch, int32_t seq_len, int32_t pos0,
              const int32_t* pos, const qwen3_kv_layer* caches, float* logits,
              int32_t logits_mode, int32_t* next_ids, char* ws, const DenseLayout& L,
              hipStream_t s) {
  const bool decode = pos != nullptr;
  const int H = c->hidden_size, V = c->vocab_size, T = L.T;
  float* res = (float*)(ws + L.res);
  CHECK_HIP(embed_gather(ids, (const bf16_t*)w->embed_tokens, res, T, H, V, s));
  LayerIO io{};
  io.T = T; io.B = batch; io.S = seq_len; io.pos0 = decode ? 0 : pos0;
  io.pos = pos; io.res = res;
  bool normed = false;
  for (int l = 0; l < c->num_hidden_layers; ++l) {
    io.input_normed = normed;
    io.next_norm = l + 1 < c->num_hidden_layers
                       ? (const bf16_t*)w->layers[l + 1].input_layernorm : nullptr;
    TRY(run_layer(c, &w->layers[l], rope, &caches[l], io, ws, L, s, &normed,
                  routed_layer(c, l)));
  }

  // final RMSNorm on the rows that need logits, LM head (tied: embed_tokens)
  const bf16_t* head = (const bf16_t*)(c->tie_word_embeddings ? w->embed_tokens : w->lm_head);
  f16_t* hf = (f16_t*)(ws + L.hf);
  const int S = io.S;
  int rows;
  float* out;
  if (logits_mode == QWEN3_LOGITS_ALL) {
    rows = T;
    out = logits;
    CHECK_HIP(rmsnorm_f32(res, 1, 0, (const bf16_t*)w->norm, hf, rows, H, c->rms_norm_eps, s));
  } else {
    if (logits_mode == QWEN3_LOGITS_NONE && !next_ids) return QWEN3_OK;
    rows = batch;
    out = logits_mode == QWEN3_LOGITS_LAST ? logits : (float*)(ws + L.lg_scratch);
    CHECK_HIP(rmsnorm_f32(res, S, S - 1, (const bf16_t*)w->norm, hf, rows, H, c->rms_norm_eps, s));
  }
  {
    Args a{};
    a.M = rows; a.N = V; a.K = H;
    a.A = hf; a.lda = H;
    a.B0 = head; a.ldb = H;
    a.C = out; a.ldc = V;
    GemmPlan p = gemm_plan(a.M, a.N, a.K, gemm::B_DENSE, gemm::E_F32, false);
    ProfScope ps("lm_head_gemm", s);
    CHECK_HIP(gemm_run(a, true, gemm::B_DENSE, gemm::E_F32, false, p, s));
  }
  if (next_ids) {
    const float* last = out;
    int64_t stride = V;
    if (logits_mode == QWEN3_LOGITS_ALL) {
      last = out + (int64_t)(S - 1) * V;
      stride = (int64_t)S * V;
    }
    ProfScope ps("argmax", s);
    CHECK_HIP(argmax_rows(last, stride, batch, V, next_ids, (float*)(ws + L.am_val),
                          (int32_t*)(ws + L.am_idx), L.am_chunks, s));
  }
  return QWEN3_OK;
}

}  // namespace

extern "C" {

int qwen3_stack_forward(const qwen3_config* c, const qwen3_model_weights* w, const float* rope,
                        const int32_t* ids, int32_t batch, int32_t seq_len, int32_t pos0,
                        const int32_t* pos, const qwen3_kv_layer* caches, float* logits,
                        int32_t logits_mode, int32_t* next_ids, void* workspace,
                        size_t workspace_bytes, void* stream) {
  g_err.clear();
  if (batch <= 0 || seq_len <= 0)
    return fail(QWEN3_EINVAL, "batch=%d seq_len=%d must be positive", batch, seq_len);
  TRY(check_stack(c, w, rope, caches, batch));
  if (!ids) return fail(QWEN3_EINVAL, "ids is NULL");
  if (logits_mode != QWEN3_LOGITS_NONE && logits_mode != QWEN3_LOGITS_ALL &&
      logits_mode != QWEN3_LOGITS_LAST)
    return fail(QWEN3_EINVAL, "logits_mode=%d", logits_mode);
  if (logits_mode != QWEN3_LOGITS_NONE) REQ_PTR(logits, "logits");
  const bool decode = pos != nullptr;
  if (decode) {
    // the positions live on the device: the kernels check them (NaN rows, no writes)
    if (seq_len > std::min(caches[0].capacity, c->max_position_embeddings))
      return fail(QWEN3_ERANGE, "seq_len=%d exceeds the cache capacity %d", seq_len,
                  caches[0].capacity);
  } else {
    for (int l = 0; l < c->num_hidden_layers; ++l) TRY(check_range(c, &caches[l], pos0, seq_len));
  }
  const int op = decode ? QWEN3_OP_STACK_DECODE : QWEN3_OP_STACK_PREFILL;
  DenseLayout L = dense_layout(c, op, batch, seq_len, caches[0].capacity);
  if (!aligned16(workspace) || workspace_bytes < L.total)
    return fail(QWEN3_EWORKSPACE, "workspace needs %zu bytes (got %zu)", L.total,
                workspace_bytes);
  return stack_run(c, w, rope, ids, batch, seq_len, pos0, pos, caches, logits, logits_mode,
                   next_ids, (char*)workspace, L, (hipStream_t)stream);
}

int qwen3_generate(const qwen3_config* c, const qwen3_model_weights* w, const float* rope,
                   const int32_t* prompt_ids, int32_t batch, int32_t prompt_len, int32_t n_new,
                   const qwen3_kv_layer* caches, float temperature, float top_p,
                   const float* uniforms, int32_t* out_ids, void* workspace,
                   size_t workspace_bytes, void* stream) {
  g_err.clear();
  if (batch <= 0 || prompt_len <= 0 || n_new <= 0)
    return fail(QWEN3_EINVAL, "batch=%d prompt_len=%d n_new=%d must be positive", batch,
                prompt_len, n_new);
  TRY(check_stack(c, w, rope, caches, batch));
  if (!prompt_ids) return fail(QWEN3_EINVAL, "prompt_ids is NULL");
  if (!out_ids) return fail(QWEN3_EINVAL, "out_ids is NULL");
  const bool sampling = temperature != 0.f;
  if (sampling) {
    if (!(temperature > 0.f)) return fail(QWEN3_EINVAL, "temperature must be >= 0");
    if (!(top_p > 0.f && top_p <= 1.f)) return fail(QWEN3_EINVAL, "top_p must be in (0, 1]");
    if (!uniforms) return fail(QWEN3_EINVAL, "uniforms is NULL (needed when temperature > 0)");
    if (c->vocab_size > (1 << 18))
      return fail(QWEN3_EINVAL, "sampling supports vocab_size <= 262144 (got %d)", c->vocab_size);
  }
  // the prompt and every generated token but the last take a cache position
  for (int l = 0; l < c->num_hidden_layers; ++l)
    TRY(check_range(c, &caches[l], 0, prompt_len + n_new - 1));
  const GenLayout G = gen_layout(c, batch, prompt_len, caches[0].capacity);
  if (!aligned16(workspace) || workspace_bytes < G.total)
    return fail(QWEN3_EWORKSPACE, "workspace needs %zu bytes (got %zu)", G.total,
                workspace_bytes);
  hipStream_t s = (hipStream_t)stream;
  char* ws = (char*)workspace;
  float* logits = (float*)(ws + G.logits);
  int32_t* ids = (int32_t*)(ws + G.ids);
  int32_t* pos = (int32_t*)(ws + G.pos);
  char* sws = ws + G.stack;
  const int V = c->vocab_size;
  for (int i = 0; i < n_new; ++i) {
    // step 0: prefill of the prompt; step i: decode of token i - 1 at prompt_len + i - 1
    if (i == 0)
      TRY(stack_run(c, w, rope, prompt_ids, batch, prompt_len, 0, nullptr, caches, logits,
                    QWEN3_LOGITS_LAST, sampling ? nullptr : ids, sws, G.prefill, s));
    else
      TRY(stack_run(c, w, rope, ids, batch, 1, 0, pos, caches, logits, QWEN3_LOGITS_LAST,
                    sampling ? nullptr : ids, sws, G.decode, s));
    if (sampling) {
      ProfScope ps("sample", s);
      CHECK_HIP(sample_rows(logits, V, batch, V, temperature, top_p,
                            uniforms + (int64_t)i * batch, ids, ws + G.samp, s));
    }
    CHECK_HIP(gen_feed(ids, out_ids, n_new, i, pos, prompt_len + i, batch, s));
  }
  return QWEN3_OK;
}

int qwen3_moe_ffn(const qwen3_config* c, const qwen3_moe_weights* w, const void* x, void* y,
                  int32_t n_tokens, float* router_logits, int32_t* topk_idx, float* topk_w,
                  int32_t* expert_offsets, int32_t* perm_token, int32_t* inv_row,
                  void* workspace, size_t workspace_bytes, void* stream) {
  g_err.clear();
  if (!c) return fail(QWEN3_EINVAL, "cfg is NULL");
  TRY(check_moe_cfg(c));
  const int k = c->num_experts_per_tok;
  if (n_tokens <= 0) return fail(QWEN3_EINVAL, "n_tokens=%d must be positive", n_tokens);
  if ((int64_t)n_tokens * k > (1 << 30)) return fail(QWEN3_EINVAL, "too many tokens");
  if (!w) return fail(QWEN3_EINVAL, "MoE weights are NULL");
  REQ_PTR(w->router, "router");
  REQ_PTR(w->gate_up_proj, "gate_up_proj");
  REQ_PTR(w->down_proj, "down_proj");
  REQ_PTR(x, "x");
  REQ_PTR(y, "y");
  MoeLayout L = moe_layout(c, n_tokens);
  if (!aligned16(workspace) || workspace_bytes < L.total)
    return fail(QWEN3_EWORKSPACE, "workspace needs %zu bytes (got %zu)", L.total,
                workspace_bytes);
  MoeIO m{};
  m.x = x; m.x_f16 = false; m.T = n_tokens;
  m.out = y; m.out_f32 = false;
  m.lg = router_logits; m.idx = topk_idx; m.wt = topk_w; m.offs = expert_offsets;
  m.perm = perm_token; m.inv = inv_row;
  return moe_run(c, w->router, w->gate_up_proj, w->down_proj, m, (char*)workspace, L,
                 (hipStream_t)stream);
}

}  // extern "C"
