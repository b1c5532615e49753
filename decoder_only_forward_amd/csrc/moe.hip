// Routed MoE: top-k routing, deterministic dispatch order, weighted combine
// ([P3] "MoE": fp32 router softmax, top-k, renormalisation, hit experts only,
// weighted index_add back to the token rows).  With router_bf16 the selection follows
// [P1] section 11: the fp32 softmax over all experts is rounded to bf16, the largest
// rounded probabilities are selected (lower index first on ties) and serve as the weights.
//
// Dispatch order: experts ascending, tokens ascending within an expert.  It is a counting
// sort over fixed token chunks whose result does not depend on thread timing (the only
// atomics are order-free bit sets), so it is bit-reproducible:
//   hist    per chunk, per-expert token bitmasks in LDS; counts are popcounts
//   scan    per expert: chunk bases, totals, offsets, and the m-tile table the grouped
//           GEMM walks (tile -> expert, first row)
//   scatter per chunk, one thread per token: its row for expert e is the expert's base
//           plus the popcount of e's mask bits below the token
#include <algorithm>

#include "launch.h"

namespace q3 {
namespace {

constexpr int kChunk = 256;  // tokens per routing chunk
constexpr int kMaxK = 8;
constexpr int kMaxE = 256;

// One wave per token: k rounds of a wave-wide (value desc, index asc) argmax.
__global__ void __launch_bounds__(256) topk_kernel(MoeRouteArgs a) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= a.T) return;
  float v[4];
  int e_of[4];
  if (a.x) {
    // few experts: each logit is one wave-wide dot product (lanes take 8-element chunks)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      e_of[i] = lane + 64 * i;
      v[i] = -INFINITY;
    }
    float acc[kRouteSmallE];
#pragma unroll
    for (int e = 0; e < kRouteSmallE; ++e) acc[e] = 0.f;
    for (int c = lane; c < a.H / 8; c += 64) {
      float xf[8];
      const int64_t xo = (int64_t)t * a.H + c * 8;
      if (a.x_f16) unpack8_f16(ld16((const f16_t*)a.x + xo), xf);
      else unpack8(ld16((const bf16_t*)a.x + xo), xf);
#pragma unroll
      for (int e = 0; e < kRouteSmallE; ++e) {
        if (e >= a.E) break;
        float wf[8];
        unpack8(ld16(a.router + (int64_t)e * a.H + c * 8), wf);
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[e] = fmaf(xf[i], wf[i], acc[e]);
      }
    }
#pragma unroll
    for (int e = 0; e < kRouteSmallE; ++e) {
      if (e >= a.E) break;
      const float lg = warp_sum(acc[e]);
      if (lane == 0) a.logits[(int64_t)t * a.E + e] = lg;
      if (lane == e) v[0] = lg;
    }
  } else {
    const float* r = a.logits + (int64_t)t * a.E;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      int e = lane + 64 * i;
      e_of[i] = e;
      v[i] = e < a.E ? r[e] : -INFINITY;
    }
  }
  if (a.router_bf16) {
    // selection keys: the bf16-rounded fp32 softmax probabilities
    float m = fmaxf(fmaxf(v[0], v[1]), fmaxf(v[2], v[3]));
    for (int o = 32; o > 0; o >>= 1) m = fmaxf(m, __shfl_xor(m, o, 64));
    float ex[4], s = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      ex[i] = e_of[i] < a.E ? expf(v[i] - m) : 0.f;
      s += ex[i];
    }
    s = warp_sum(s);
#pragma unroll
    for (int i = 0; i < 4; ++i) v[i] = e_of[i] < a.E ? bf2f(f2bf(ex[i] / s)) : -INFINITY;
  }
  bool taken[4] = {false, false, false, false};
  float sel_v[kMaxK];
  int sel_e[kMaxK];
#pragma unroll
  for (int j = 0; j < kMaxK; ++j) {
    if (j >= a.k) break;
    float bv = -INFINITY;
    int be = 0x7FFFFFFF;
#pragma unroll
    for (int i = 0; i < 4; ++i)
      if (!taken[i] && e_of[i] < a.E && (v[i] > bv || (v[i] == bv && e_of[i] < be))) {
        bv = v[i];
        be = e_of[i];
      }
    for (int o = 32; o > 0; o >>= 1) {
      float ov = __shfl_xor(bv, o, 64);
      int oe = __shfl_xor(be, o, 64);
      if (ov > bv || (ov == bv && oe < be)) { bv = ov; be = oe; }
    }
#pragma unroll
    for (int i = 0; i < 4; ++i)
      if (e_of[i] == be) taken[i] = true;
    sel_v[j] = bv;
    sel_e[j] = be;
  }
  if (a.router_bf16) {  // the selected rounded probabilities are the weights
    float sel = 0.f;
#pragma unroll
    for (int j = 0; j < kMaxK; ++j)
      if (j < a.k) sel += sel_v[j];
    if (lane < a.k) {
      float sv = sel_v[0];
      int se = sel_e[0];
#pragma unroll
      for (int j = 1; j < kMaxK; ++j)
        if (j == lane && j < a.k) { sv = sel_v[j]; se = sel_e[j]; }
      a.idx[(int64_t)t * a.k + lane] = se;
      a.w[(int64_t)t * a.k + lane] = a.norm_topk ? sv / sel : sv;
    }
    return;
  }
  // probabilities: softmax over all experts (max = sel_v[0]); renormalised over the k
  float denom = 0.f;
  if (a.norm_topk) {
#pragma unroll
    for (int j = 0; j < kMaxK; ++j)
      if (j < a.k) denom += __expf(sel_v[j] - sel_v[0]);
  } else {
    float s = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i)
      if (e_of[i] < a.E) s += __expf(v[i] - sel_v[0]);
    denom = warp_sum(s);
  }
  if (lane < a.k) {
    float sv = sel_v[0];
    int se = sel_e[0];
#pragma unroll
    for (int j = 1; j < kMaxK; ++j)
      if (j == lane && j < a.k) { sv = sel_v[j]; se = sel_e[j]; }
    a.idx[(int64_t)t * a.k + lane] = se;
    a.w[(int64_t)t * a.k + lane] = __expf(sv - sel_v[0]) / denom;
  }
}

// Per 256-token chunk: bit t of word w of expert e's mask says token 32 w + t of the chunk
// selected e.  Counts are popcounts; the stable (token-ascending) rank of an entry among
// its expert's entries in the chunk is the popcount of the bits below its token.
constexpr int kMaskWords = kChunk / 32;

DEV void build_masks(const MoeRouteArgs& a, int t0, int nt, uint32_t (*smask)[kMaskWords]) {
  for (int i = threadIdx.x; i < a.E * kMaskWords; i += 256) smask[i / kMaskWords][i % kMaskWords] = 0u;
  __syncthreads();
  const int tl = threadIdx.x;
  if (tl < nt) {
    for (int j = 0; j < a.k; ++j) {
      const int e = a.idx[(int64_t)(t0 + tl) * a.k + j];
      if (e >= 0 && e < a.E) atomicOr(&smask[e][tl >> 5], 1u << (tl & 31));
    }
  }
  __syncthreads();
}

__global__ void __launch_bounds__(256) hist_kernel(MoeRouteArgs a) {
  __shared__ uint32_t smask[kMaxE][kMaskWords];
  const int c = blockIdx.x;
  const int t0 = c * kChunk, nt = min(kChunk, a.T - t0);
  build_masks(a, t0, nt, smask);
  const int e = threadIdx.x;
  if (e >= a.E) return;
  int cnt = 0;
#pragma unroll
  for (int w = 0; w < kMaskWords; ++w) cnt += __popc(smask[e][w]);
  a.chunk_counts[(int64_t)c * a.E + e] = cnt;
}

__global__ void __launch_bounds__(256) scan_kernel(MoeRouteArgs a, int nchunks) {
  __shared__ int s_tot[kMaxE], s_tiles[kMaxE];
  const int e = threadIdx.x;
  int tot = 0;
  if (e < a.E) {
    for (int c = 0; c < nchunks; ++c) {
      int v = a.chunk_counts[(int64_t)c * a.E + e];
      a.chunk_counts[(int64_t)c * a.E + e] = tot;  // exclusive base within the expert
      tot += v;
    }
  }
  s_tot[e] = e < a.E ? tot : 0;
  s_tiles[e] = e < a.E ? (tot + a.tile_m - 1) / a.tile_m : 0;
  __syncthreads();
  if (e == 0) {
    int off = 0, toff = 0;
    for (int i = 0; i < a.E; ++i) {
      int n = s_tot[i], tl = s_tiles[i];
      a.counts[i] = n;
      a.offsets[i] = off;
      s_tot[i] = off;
      s_tiles[i] = toff;
      off += n;
      toff += tl;
    }
    a.offsets[a.E] = off;
    a.tile_count[0] = toff;
  }
  __syncthreads();
  // tile table: each expert's tiles in order (tile_count of them), then idle entries
  for (int i = e; i < a.max_tiles; i += 256) {
    a.tile_expert[i] = -1;
    a.tile_row0[i] = 0;
  }
  __syncthreads();
  if (e < a.E) {
    int first = s_tiles[e];
    int ntl = (tot + a.tile_m - 1) / a.tile_m;
    for (int i = 0; i < ntl; ++i) {
      a.tile_expert[first + i] = e;
      a.tile_row0[first + i] = i * a.tile_m;
    }
  }
}

__global__ void __launch_bounds__(256) scatter_kernel(MoeRouteArgs a) {
  __shared__ uint32_t smask[kMaxE][kMaskWords];
  const int c = blockIdx.x;
  const int t0 = c * kChunk, nt = min(kChunk, a.T - t0);
  build_masks(a, t0, nt, smask);
  const int tl = threadIdx.x;
  if (tl >= nt) return;
  const int t = t0 + tl, w0 = tl >> 5;
  const uint32_t below = (1u << (tl & 31)) - 1u;
  for (int j = 0; j < a.k; ++j) {
    const int e = a.idx[(int64_t)t * a.k + j];
    if (e < 0 || e >= a.E) continue;
    int rank = __popc(smask[e][w0] & below);
    for (int w = 0; w < w0; ++w) rank += __popc(smask[e][w]);
    const int row = a.offsets[e] + a.chunk_counts[(int64_t)c * a.E + e] + rank;
    a.perm_token[row] = t;
    a.inv_row[(int64_t)t * a.k + j] = row;
  }
}

// y[t] = sum_j w[t][j] * y_rows[inv_row[t][j]], in slot order, rounded once to bf16.
__global__ void __launch_bounds__(256)
combine_kernel(const float* __restrict__ y_rows, const int32_t* __restrict__ inv_row,
               const float* __restrict__ w, const float* residual, void* out, bool out_f32,
               int T, int k, int H) {
  const int nchunk = H / 8;
  const int64_t total = (int64_t)T * nchunk;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total;
       i += (int64_t)gridDim.x * blockDim.x) {
    int t = (int)(i / nchunk), c = (int)(i % nchunk);
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    for (int j = 0; j < k; ++j) {
      float wj = w[(int64_t)t * k + j];
      const float* src = y_rows + (int64_t)inv_row[(int64_t)t * k + j] * H + c * 8;
      f32x4_t a0 = *(const f32x4_t*)src, a1 = *(const f32x4_t*)(src + 4);
      for (int e = 0; e < 4; ++e) {
        acc[e] += wj * a0[e];
        acc[4 + e] += wj * a1[e];
      }
    }
    const int64_t off = (int64_t)t * H + c * 8;
    if (residual) {  // out = residual + sum (in place allowed: read before written)
      const f32x4_t r0 = *(const f32x4_t*)(residual + off);
      const f32x4_t r1 = *(const f32x4_t*)(residual + off + 4);
      for (int e = 0; e < 4; ++e) {
        acc[e] = r0[e] + acc[e];
        acc[4 + e] = r1[e] + acc[4 + e];
      }
    }
    if (out_f32) {
      *(f32x4_t*)((float*)out + off) = f32x4_t{acc[0], acc[1], acc[2], acc[3]};
      *(f32x4_t*)((float*)out + off + 4) = f32x4_t{acc[4], acc[5], acc[6], acc[7]};
    } else {
      u32x4_t o;
      for (int e = 0; e < 4; ++e) o[e] = pack_bf16x2(acc[2 * e], acc[2 * e + 1]);
      st16((bf16_t*)out + off, o);
    }
  }
}

}  // namespace

int moe_route_chunks(int T) { return (T + kChunk - 1) / kChunk; }

hipError_t moe_route(const MoeRouteArgs& a, hipStream_t s) {
  if (a.T <= 0) return hipSuccess;
  hipLaunchKernelGGL(topk_kernel, dim3((a.T + 3) / 4), dim3(256), 0, s, a);
  const int nchunks = moe_route_chunks(a.T);
  hipLaunchKernelGGL(hist_kernel, dim3(nchunks), dim3(256), 0, s, a);
  hipLaunchKernelGGL(scan_kernel, dim3(1), dim3(256), 0, s, a, nchunks);
  hipLaunchKernelGGL(scatter_kernel, dim3(nchunks), dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t moe_combine(const float* y_rows, const int32_t* inv_row, const float* w,
                       const float* residual, void* out, bool out_f32, int T, int k, int H,
                       hipStream_t s) {
  if (T <= 0) return hipSuccess;
  int64_t work = (int64_t)T * H / 8;
  int blocks = (int)std::min<int64_t>(65536, (work + 255) / 256);
  hipLaunchKernelGGL(combine_kernel, dim3(blocks), dim3(256), 0, s, y_rows, inv_row, w, residual,
                     out, out_f32, T, k, H);
  return hipGetLastError();
}

}  // namespace q3
