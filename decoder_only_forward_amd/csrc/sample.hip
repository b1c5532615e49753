// Next-token selection by sampling, and the per-step bookkeeping of device-side generation.
//
// Sampling rule (temperature t > 0, nucleus mass top_p in (0, 1], one uniform u in [0, 1)
// per row; the pages' generation loops draw from softmax(logits / t), optionally cut to the
// top-p nucleus, [P3] generation and [P4] sampling sections):
//   e_v = exp((l_v - max_l) / t)                 (non-finite logits count as e_v = 0)
//   tau = the largest value such that the e_v >= tau sum to at least top_p * sum_v e_v
//         (top_p = 1: every token with e_v > 0), so ties at the cut are all kept;
//   kept mass K = sum of e_v >= tau; r = u K (u clamped to [0, 1), r kept below K);
//   the token is the smallest index v whose running sum of kept e_w (w <= v, ascending
//   token order) exceeds r (should rounding leave no such v in the range that holds r,
//   that range's last kept index).
// One block of 512 threads per row.  tau is found by bisection on the fp32 bit pattern
// (the e_v are positive, so the order of their bit patterns is their numeric order); each
// step is one block reduction with the e_v recomputed, which is cheaper than storing them.
// All passes read the row lane-strided (coalesced).  Every reduction has a fixed order, so
// the result is deterministic.
#include "launch.h"

namespace q3 {
namespace {

constexpr int kSampThreads = 512;

DEV float block_sum(float v, float* red) {
  v = warp_sum(v);
  const int w = threadIdx.x >> 6, l = threadIdx.x & 63;
  __syncthreads();
  if (l == 0) red[w] = v;
  __syncthreads();
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < kSampThreads / 64; ++i) s += red[i];
  return s;
}

DEV float block_max(float v, float* red) {
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  const int w = threadIdx.x >> 6, l = threadIdx.x & 63;
  __syncthreads();
  if (l == 0) red[w] = v;
  __syncthreads();
  float m = -INFINITY;
#pragma unroll
  for (int i = 0; i < kSampThreads / 64; ++i) m = fmaxf(m, red[i]);
  return m;
}

__global__ void __launch_bounds__(kSampThreads)
sample_kernel(const float* __restrict__ logits, int64_t row_stride, int V, float inv_t,
              float top_p, const float* __restrict__ u, int32_t* __restrict__ out) {
  constexpr int kTile = 1024;            // tokens per tile of the ascending-order prefix
  constexpr int kMaxTiles = 256;         // V <= 262144
  __shared__ float red[kSampThreads / 64];
  __shared__ float tile_sum[kMaxTiles];
  __shared__ int s_tile;
  __shared__ float s_off;
  const int row = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const float* x = logits + (int64_t)row * row_stride;

  // passes over the row are lane-strided (coalesced); their sums have a fixed order
  float m = -INFINITY;
  for (int v = tid; v < V; v += kSampThreads) {
    const float l = x[v];
    if (l == l && l != INFINITY) m = fmaxf(m, l);
  }
  m = block_max(m, red);
  if (m == -INFINITY) {  // no finite logit
    if (tid == 0) out[row] = 0;
    return;
  }
  const float inv_t2 = inv_t * 1.4426950408889634f;  // e^y = 2^(y log2 e)
  auto ev = [&](int v) {
    const float l = x[v];
    return (l == l && l != INFINITY) ? __builtin_amdgcn_exp2f((l - m) * inv_t2) : 0.f;
  };
  float tau = 0.f;  // keep every e_v > 0
  if (top_p < 1.f) {
    // masses of e_v >= t_k for kProbe thresholds at once (one pass over the row), each a
    // fixed-order block sum
    constexpr int kProbe = 15;
    __shared__ float probe_red[kSampThreads / 64][kProbe];
    auto masses = [&](const float* t, float* outm) {
      float acc[kProbe];
#pragma unroll
      for (int k = 0; k < kProbe; ++k) acc[k] = 0.f;
#pragma unroll 4
      for (int v = tid; v < V; v += kSampThreads) {
        const float e = ev(v);
#pragma unroll
        for (int k = 0; k < kProbe; ++k)
          if (e >= t[k] && e > 0.f) acc[k] += e;
      }
      __syncthreads();
#pragma unroll
      for (int k = 0; k < kProbe; ++k) {
        const float w = warp_sum(acc[k]);
        if (lane == 0) probe_red[wave][k] = w;
      }
      __syncthreads();
#pragma unroll
      for (int k = 0; k < kProbe; ++k) {
        float sum = 0.f;
        for (int i = 0; i < kSampThreads / 64; ++i) sum += probe_red[i][k];
        outm[k] = sum;
      }
    };
    float t[kProbe], mk[kProbe];
    t[0] = 0.f;
    for (int k = 1; k < kProbe; ++k) t[k] = 2.f;  // above every e_v: mass 0
    masses(t, mk);
    const float target = top_p * mk[0];  // mk[0]: the total
    // largest bit pattern b in [0, bits(1.0)] with mass(float(b)) >= target, by a 16-way
    // search: mass(lo) >= target and mass(hi) < target throughout; every e_v <= 1
    uint32_t lo = 0, hi = 0x3F800001u;
    while (hi - lo > 1) {
      const uint32_t span = hi - lo;
      uint32_t pt[kProbe];
#pragma unroll
      for (int k = 0; k < kProbe; ++k) {
        pt[k] = lo + (uint32_t)(((uint64_t)span * (k + 1)) / (kProbe + 1));
        t[k] = __uint_as_float(pt[k]);
      }
      masses(t, mk);
      uint32_t nlo = lo, nhi = hi;
#pragma unroll
      for (int k = 0; k < kProbe; ++k) {
        if (pt[k] <= lo || pt[k] >= hi) continue;  // duplicate point on a small span
        if (mk[k] >= target) nlo = pt[k] > nlo ? pt[k] : nlo;
        else nhi = pt[k] < nhi ? pt[k] : nhi;
      }
      lo = nlo;
      hi = nhi;
    }
    tau = __uint_as_float(lo);
  }
  auto kept = [&](int v) {
    const float e = v < V ? ev(v) : 0.f;
    return (e >= tau && e > 0.f) ? e : 0.f;
  };

  // inverse CDF in ascending token order, two levels: kept mass of each 1024-token tile
  // (one wave per tile, 16 coalesced loads), then a running sum over the tiles in order
  const int ntiles = (V + kTile - 1) / kTile;
  for (int t = wave; t < ntiles; t += kSampThreads / 64) {
    float sum = 0.f;
    for (int j = 0; j < kTile; j += 64) sum += kept(t * kTile + j + lane);
    sum = warp_sum(sum);
    if (lane == 0) tile_sum[t] = sum;
  }
  __syncthreads();
  if (tid == 0) {
    float K = 0.f;
    for (int t = 0; t < ntiles; ++t) K += tile_sum[t];  // > 0: the largest logit gives 1
    const float uu = fminf(fmaxf(u[row], 0.f), 1.f);
    const float r = fminf(uu * K, __uint_as_float(__float_as_uint(K) - 1u));  // r < K
    float c = 0.f;
    int tsel = -1;
    for (int t = 0; t < ntiles; ++t) {
      if (tile_sum[t] > 0.f) tsel = t;
      if (c + tile_sum[t] > r && tile_sum[t] > 0.f) break;
      c += tile_sum[t];
    }
    s_tile = tsel;     // the tile holding r (rounding past the end: the last kept tile)
    s_off = r - c;     // r within that tile's kept mass
  }
  __syncthreads();
  if (wave == 0) {
    // one wave scans the chosen tile 64 tokens at a time in ascending order
    const int t = s_tile;
    const float r = s_off;
    float c = 0.f;
    int pick = -1, last = -1;
    for (int j = 0; j < kTile && pick < 0; j += 64) {
      const int v = t * kTile + j + lane;
      const float e = kept(v);
      float inc = e;  // inclusive prefix over the 64 lanes (fixed order)
      for (int o = 1; o < 64; o <<= 1) {
        const float y = __shfl_up(inc, o, 64);
        if (lane >= o) inc += y;
      }
      const unsigned long long hit = __ballot(e > 0.f && c + inc > r);
      const unsigned long long any = __ballot(e > 0.f);
      if (any) last = t * kTile + j + 63 - __builtin_clzll(any);
      if (hit) pick = t * kTile + j + __builtin_ctzll(hit);
      c += __shfl(inc, 63, 64);
    }
    if (lane == 0) out[row] = pick >= 0 ? pick : (last >= 0 ? last : 0);
  }
}

// out_ids[b][col] = ids[b]; pos[b] = next_pos (the position the fed-back token takes)
__global__ void gen_feed_kernel(const int32_t* __restrict__ ids, int32_t* __restrict__ out_ids,
                                int n_new, int col, int32_t* __restrict__ pos, int next_pos,
                                int B) {
  const int b = blockIdx.x * blockDim.x + threadIdx.x;
  if (b >= B) return;
  out_ids[(int64_t)b * n_new + col] = ids[b];
  pos[b] = next_pos;
}

}  // namespace

hipError_t sample_rows(const float* logits, int64_t row_stride, int rows, int V,
                       float temperature, float top_p, const float* u, int32_t* out,
                       hipStream_t s) {
  if (rows <= 0) return hipSuccess;
  if (!(temperature > 0.f) || !(top_p > 0.f) || top_p > 1.f) return hipErrorInvalidValue;
  if (V <= 0 || V > 256 * 1024) return hipErrorInvalidValue;
  hipLaunchKernelGGL(sample_kernel, dim3(rows), dim3(kSampThreads), 0, s, logits, row_stride, V,
                     1.f / temperature, top_p, u, out);
  return hipGetLastError();
}

hipError_t gen_feed(const int32_t* ids, int32_t* out_ids, int n_new, int col, int32_t* pos,
                    int next_pos, int B, hipStream_t s) {
  if (B <= 0) return hipSuccess;
  hipLaunchKernelGGL(gen_feed_kernel, dim3((B + 255) / 256), dim3(256), 0, s, ids, out_ids,
                     n_new, col, pos, next_pos, B);
  return hipGetLastError();
}

}  // namespace q3
