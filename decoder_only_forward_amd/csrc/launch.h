// Internal launch interface of libqwen3 (host side).  Every launcher enqueues on `s`
// and returns hipSuccess or the launch error; none allocates or synchronises.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "gemm_kernel.h"

namespace q3 {

// ---- GEMM (gemm.hip)
// Tile families; kAuto picks by problem size.
enum GemmTile { kAuto = 0, kBig = 1, kMid = 2, kSkinny = 3, kDecode = 4, kTall = 5 };

struct GemmPlan {
  int tile;      // GemmTile actually used
  int k_splits;  // decode residual projections: > 1 means fp32 partial sums
                 // [k_splits][M][N] in a.partial, reduced by splitk_res_norm()
};

// Chooses the tile family for an (M, N, K) problem: for M <= 64 the decode kernel (the
// 64x128 tile for fp32 outputs), else 256x256 when that gives >= 512 tiles, else
// 128x128 (grouped problems always 128x128).
GemmPlan gemm_plan(int M, int N, int K, int bmode, int epi, bool grouped);

// Runs C = A . B^T with the given B source and epilogue.
// f16: A holds fp16 activations and the bf16 weights are converted to fp16 (otherwise
// both operands are bf16).
hipError_t gemm_run(const gemm::Args& a, bool f16, int bmode, int epi, bool grouped,
                    const GemmPlan& plan, hipStream_t s);

// ---- norms, embedding, RoPE (norm_rope.hip)
// out[r] = f16(rmsnorm(in[r_in])) with r_in = r * in_row_stride + in_row_offset.
hipError_t rmsnorm_f32(const float* in, int64_t in_row_stride, int64_t in_row_offset,
                       const bf16_t* w, f16_t* out, int rows, int H, float eps, hipStream_t s);
hipError_t rmsnorm_bf16(const bf16_t* in, int64_t in_row_stride, int64_t in_row_offset,
                        const bf16_t* w, f16_t* out, int rows, int H, float eps, hipStream_t s);
// out[m] = residual[m] + sum_s part[s][m] (fixed order), then, if norm_w is given,
// xn[m] = rmsnorm(out[m]) * norm_w (fp16).  residual / out may be fp32 or bf16; N <= 2048.
hipError_t splitk_res_norm(const float* part, int splits, int M, int N, const void* residual,
                           bool residual_bf16, void* out, bool out_bf16, const bf16_t* norm_w,
                           f16_t* xn, float eps, hipStream_t s);
hipError_t embed_gather(const int32_t* ids, const bf16_t* table, float* out, int T, int H, int V,
                        hipStream_t s);
hipError_t rope_table(float* rope, int max_pos, int hd, double theta, hipStream_t s);

struct RopeCacheArgs {
  const f16_t* qkv;  // [T][(nq + 2 nkv) * hd] fp16 projections, token t = b * S + s
  const float* rope;  // [2][max_pos][hd/2]
  const bf16_t* q_norm;
  const bf16_t* k_norm;
  f16_t* q_out;  // [T][nq][hd] fp16, pre-scaled by log2(e) / sqrt(hd)
  bf16_t* k_cache;  // [B][nkv] regions of cap * hd, 32-position tiles (kcache_idx)
  bf16_t* vt_cache; // [B][nkv] regions of cap * hd, 32-position tiles (vcache_idx)
  const int32_t* pos;  // decode: device [B], token s at pos[b] + s; prefill: nullptr
  // prefill only: fp16 copies of the new keys / values (not rounded to bf16) for the attention,
  // indexed by absolute position - fresh_base; k_fresh [B][nkv][fresh_w][hd],
  // vt_fresh [B][nkv][hd][fresh_w] (nullptr: not written)
  f16_t* k_fresh;
  f16_t* vt_fresh;
  int fresh_base, fresh_w;
  int pos0, B, S, nq, nkv, cap, max_pos, qk_norm;
  int interleaved;  // RoPE planes (2i, 2i + 1) instead of (i, i + hd/2)
  float eps;
};
hipError_t qkv_rope_cache(const RopeCacheArgs& a, hipStream_t s);

// ---- attention (attention.hip)
struct AttnPrefillArgs {
  const f16_t* q;        // [B][S][nq][hd] fp16
  const bf16_t* k_cache; // [B][nkv] regions of cap * hd, 32-position tiles
  const bf16_t* vt_cache;// [B][nkv] regions of cap * hd, 32-position tiles
  f16_t* out;            // [B][S][nq][hd] fp16
  // keys / values at positions >= pos0 come from these fp16 copies (see RopeCacheArgs)
  const f16_t* k_fresh;
  const f16_t* vt_fresh;
  int fresh_base, fresh_w;
  int B, S, pos0, nq, nkv, cap;
};
hipError_t attn_prefill(const AttnPrefillArgs& a, hipStream_t s);

struct AttnDecodeArgs {
  const f16_t* q;   // [B][S][nq][hd] fp16
  const bf16_t* k_cache;
  const bf16_t* vt_cache;
  const int32_t* pos;  // device [B]: token s of sequence b sits at pos[b] + s
  f16_t* out;          // [B][S][nq][hd] fp16
  float* part;         // [B][S][nq][splits][hd + 2]
  int B, S, nq, nkv, cap, max_pos, splits, chunk;
  int nqg;  // query groups of 8 per (sequence, kv head): attn_decode_groups(S, nq / nkv)
};
int attn_decode_groups(int S, int g);
// blocks: B * attn_decode_groups(S, g) per kv head
void attn_decode_plan(int cap, int B, int nkv, int& splits, int& chunk);
hipError_t attn_decode(const AttnDecodeArgs& a, hipStream_t s);
hipError_t attn_decode_combine(const AttnDecodeArgs& a, hipStream_t s);

// ---- sampling (argmax.hip)
hipError_t argmax_rows(const float* logits, int64_t row_stride, int rows, int V, int32_t* out,
                       float* part_val, int32_t* part_idx, int chunks, hipStream_t s);

// ---- sampling and generation bookkeeping (sample.hip)
// temperature > 0, top_p in (0, 1]; u: device [rows] uniforms in [0, 1); ws: device scratch
// of sample_ws_bytes(rows) bytes, 16-byte aligned (its contents need no initialisation)
size_t sample_ws_bytes(int rows);
hipError_t sample_rows(const float* logits, int64_t row_stride, int rows, int V,
                       float temperature, float top_p, const float* u, int32_t* out, void* ws,
                       hipStream_t s);
// out_ids[b][col] = ids[b] (out_ids [B][n_new]); pos[b] = next_pos
hipError_t gen_feed(const int32_t* ids, int32_t* out_ids, int n_new, int col, int32_t* pos,
                    int next_pos, int B, hipStream_t s);

// ---- cache layout copies (kv_layout.hip)
// regions (sequence, kv head) pairs of positions [0, len): plain [regions][len][128] bf16
// K / V <-> tiled cache regions of cap * 128 (to_tiled: plain -> tiled)
hipError_t kv_copy(void* k_plain, void* v_plain, void* k_tiled, void* vt_tiled, int regions,
                   int len, int cap, bool to_tiled, hipStream_t s);

// ---- MoE (moe.hip)
struct MoeRouteArgs {
  float* logits;  // [T][E]: read, or written when x is set
  int T, E, k, norm_topk;
  // few experts (E <= kRouteSmallE): the routing kernel forms the logits itself,
  // logits[t][e] = x[t] . router[e] (fp32 accumulation), instead of reading a GEMM's
  const void* x;           // [T][H] fp16 (x_f16) or bf16 rows; nullptr: read logits
  bool x_f16;
  const bf16_t* router;    // [E][H]
  int H;
  int router_bf16;  // select on (and weight by) bf16-rounded softmax probabilities
  int32_t* idx;   // [T][k]
  float* w;       // [T][k]
  int32_t* chunk_counts;  // [nchunks][E]
  int32_t* counts;        // [E]
  int32_t* offsets;       // [E + 1]
  int32_t* perm_token;    // [T*k]
  int32_t* inv_row;       // [T][k]
  int32_t* tile_expert;   // [max_tiles]
  int32_t* tile_row0;     // [max_tiles]
  int32_t* tile_count;    // [1] number of tiles in use (the first entries of the table)
  int max_tiles, tile_m;
};
constexpr int kRouteSmallE = 16;
int moe_route_chunks(int T);
hipError_t moe_route(const MoeRouteArgs& a, hipStream_t s);
// out[t] = (residual[t] +) sum_j w[t][j] y_rows[inv_row[t][j]]; out fp32 or bf16
// (residual nullable; out may be the residual itself)
hipError_t moe_combine(const float* y_rows, const int32_t* inv_row, const float* w,
                       const float* residual, void* out, bool out_f32, int T, int k, int H,
                       hipStream_t s);

}  // namespace q3
