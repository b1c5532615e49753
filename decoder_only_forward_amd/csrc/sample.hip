// Next-token selection by sampling, and the per-step bookkeeping of device-side generation.
//
// Sampling rule (temperature t > 0, nucleus mass top_p in (0, 1], one uniform u in [0, 1)
// per row; the pages' generation loops draw from softmax(logits / t), optionally cut to the
// top-p nucleus, [P3] generation and [P4] sampling sections):
//   e_v = exp((l_v - max_l) / t)                 (non-finite logits count as e_v = 0)
//   tau = the largest value such that the e_v >= tau sum to at least top_p * sum_v e_v
//         (top_p = 1: every token with e_v > 0), so ties at the cut are all kept;
//   kept mass K = sum of e_v >= tau; r = u K (u clamped to [0, 1), r below K);
//   the token is the smallest index v whose running sum of kept e_w (w <= v, ascending
//   token order) exceeds r.
// Masses are summed in 64-bit fixed point, q_v = floor(e_v * 2^44) (every e_v <= 1, so a row
// of up to 2^18 tokens sums below 2^62): integer sums are exact, so every partial sum, in any
// order and over any split of the row, gives the same result (deterministic without a fixed
// reduction order), and the running mass of the inverse CDF is exact.  Tokens with
// e_v < 2^-44 carry no mass; an fp32 running sum of the row would drop them as well.
//
// Each row is split over kChunks blocks.  Launches, in stream order:
//   1. max of each chunk (and zeroing of the row's histograms);
//   2. (top_p < 1) three histogram passes: tau is the largest fp32 bit pattern b with
//      mass(e >= float(b)) >= top_p * total (the e_v are >= 0, so bit order is value
//      order); the 30-bit pattern is found 10 bits per pass from 1024-bin mass histograms
//      (a radix select), each pass counting only the tokens whose higher bits match;
//   3. the kept mass of each 64-token tile and of each chunk;
//   4. one wave per row: the chunk holding r, then its tile, then the token.
// Every pass reads the logits lane-strided (coalesced) and recomputes e_v with the same
// code, so all passes see bit-identical e_v.
#include "launch.h"

namespace q3 {
namespace {

constexpr int kThreads = 256;
constexpr int kChunks = 16;            // blocks per row
constexpr int kBins = 1024;            // 10 bits per radix pass
constexpr int kMaxV = 256 * 1024;
constexpr int kMaxTiles = (kMaxV / kChunks + 63) / 64;  // 64-token tiles per chunk
constexpr float kQScale = 17592186044416.0f;            // 2^44
static_assert(3 * kBins <= kChunks * kThreads, "the first pass zeroes one histogram word per thread");
static_assert(kBins == 4 * kThreads, "a radix scan gives each thread four bins");

// per-row workspace
constexpr int kOffMax = 0;                              // float [kChunks]
constexpr int kOffMass = 64;                            // uint64 [kChunks]
constexpr int kOffTau = 192;                            // uint32: tau's bit pattern
constexpr int kOffHist = 256;                           // uint64 [3][kBins]
constexpr int kOffTiles = kOffHist + 3 * kBins * 8;     // uint64 [kChunks][kMaxTiles]
constexpr int64_t kRowBytes = kOffTiles + kChunks * kMaxTiles * 8;
static_assert(kRowBytes % 256 == 0, "rows keep the alignment of the workspace");

struct RowWs {
  char* base;
  __device__ __forceinline__ float* pmax() const { return (float*)(base + kOffMax); }
  __device__ __forceinline__ uint64_t* mass() const { return (uint64_t*)(base + kOffMass); }
  __device__ __forceinline__ uint32_t* tau() const { return (uint32_t*)(base + kOffTau); }
  __device__ __forceinline__ uint64_t* hist(int level) const { return (uint64_t*)(base + kOffHist) + level * kBins; }
  __device__ __forceinline__ uint64_t* tiles(int c) const { return (uint64_t*)(base + kOffTiles) + c * kMaxTiles; }
};

DEV RowWs row_ws(void* ws, int row) { return RowWs{(char*)ws + (int64_t)row * kRowBytes}; }

DEV void chunk_range(int V, int c, int& v0, int& v1) {
  const int cs = (V + kChunks - 1) / kChunks;
  v0 = min(V, c * cs);
  v1 = min(V, v0 + cs);
}

DEV bool finite_logit(float l) { return l == l && l != INFINITY; }

// e_v in [0, 1]; inv_t2 = log2(e) / t
DEV float weight(float l, float m, float inv_t2) {
  return finite_logit(l) ? fminf(__builtin_amdgcn_exp2f((l - m) * inv_t2), 1.f) : 0.f;
}

DEV uint64_t fixed_mass(float e) { return (uint64_t)(e * kQScale); }

DEV uint64_t shfl_u64(uint64_t v, int src) {
  const uint32_t lo = __shfl((uint32_t)v, src, 64), hi = __shfl((uint32_t)(v >> 32), src, 64);
  return ((uint64_t)hi << 32) | lo;
}
DEV uint64_t shfl_up_u64(uint64_t v, int d) {
  const uint32_t lo = __shfl_up((uint32_t)v, d, 64), hi = __shfl_up((uint32_t)(v >> 32), d, 64);
  return ((uint64_t)hi << 32) | lo;
}
DEV uint64_t shfl_down_u64(uint64_t v, int d) {
  const uint32_t lo = __shfl_down((uint32_t)v, d, 64),
                 hi = __shfl_down((uint32_t)(v >> 32), d, 64);
  return ((uint64_t)hi << 32) | lo;
}
DEV uint64_t wave_sum_u64(uint64_t v) {
  for (int o = 32; o > 0; o >>= 1) {
    const uint32_t lo = __shfl_xor((uint32_t)v, o, 64),
                   hi = __shfl_xor((uint32_t)(v >> 32), o, 64);
    v += ((uint64_t)hi << 32) | lo;
  }
  return v;
}

DEV float block_max(float v, float* red) {
  v = warp_max(v);
  const int w = threadIdx.x >> 6;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[w] = v;
  __syncthreads();
  float m = -INFINITY;
#pragma unroll
  for (int i = 0; i < kThreads / 64; ++i) m = fmaxf(m, red[i]);
  return m;
}

DEV uint64_t block_sum_u64(uint64_t v, uint64_t* red) {
  v = wave_sum_u64(v);
  const int w = threadIdx.x >> 6;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[w] = v;
  __syncthreads();
  uint64_t s = 0;
#pragma unroll
  for (int i = 0; i < kThreads / 64; ++i) s += red[i];
  return s;
}

DEV float row_max(const RowWs& r) {
  float m = -INFINITY;
#pragma unroll
  for (int c = 0; c < kChunks; ++c) m = fmaxf(m, r.pmax()[c]);
  return m;
}

// One radix level: the largest bin b with base + sum_{j >= b} h[j] >= target (one exists by
// construction); *above = base + sum_{j > b} h[j].  Thread t owns bins 4t .. 4t + 3.
struct ScanShared {
  uint64_t wave_tot[kThreads / 64];
  int best[kThreads / 64];
  uint64_t above;
};

DEV int radix_level(const uint64_t* h, uint64_t base, uint64_t target, uint64_t& above,
                    ScanShared& sh) {
  const int t = threadIdx.x, lane = t & 63, w = t >> 6;
  uint64_t b[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) b[j] = h[4 * t + j];
  const uint64_t own = b[0] + b[1] + b[2] + b[3];
  // inclusive suffix sum over the lanes of the wave, then the waves above
  uint64_t inc = own;
  for (int d = 1; d < 64; d <<= 1) {
    const uint64_t y = shfl_down_u64(inc, d);
    if (lane + d < 64) inc += y;
  }
  __syncthreads();
  if (lane == 0) sh.wave_tot[w] = inc;
  __syncthreads();
  uint64_t suf = inc - own;  // mass of the bins above 4t + 3
  for (int i = w + 1; i < kThreads / 64; ++i) suf += sh.wave_tot[i];
  int best = -1;
  uint64_t above_best = 0;
#pragma unroll
  for (int j = 3; j >= 0; --j) {
    if (best < 0 && base + suf + b[j] >= target) {
      best = 4 * t + j;
      above_best = base + suf;
    }
    suf += b[j];
  }
  int wb = best;
  for (int o = 32; o > 0; o >>= 1) wb = max(wb, __shfl_xor(wb, o, 64));
  if (lane == 0) sh.best[w] = wb;
  __syncthreads();
  int bb = -1;
#pragma unroll
  for (int i = 0; i < kThreads / 64; ++i) bb = max(bb, sh.best[i]);
  if (best == bb && bb >= 0) sh.above = above_best;
  __syncthreads();
  above = sh.above;
  return bb;
}

// The bits of tau fixed by the first `levels` radix passes (levels = 3: tau's whole pattern;
// top_p < 1).  Every block of a row computes the same value from the same histograms.
DEV uint32_t tau_prefix(const RowWs& r, int levels, float top_p, ScanShared& sh,
                        uint64_t* red) {
  uint64_t own = 0;
#pragma unroll
  for (int j = 0; j < 4; ++j) own += r.hist(0)[4 * threadIdx.x + j];
  const uint64_t total = block_sum_u64(own, red);
  uint64_t target = (uint64_t)ceil((double)top_p * (double)total);
  target = min(max(target, (uint64_t)1), total);
  uint64_t base = 0, above = 0;
  uint32_t bits = 0;
  for (int l = 0; l < levels; ++l) {
    const int b = radix_level(r.hist(l), base, target, above, sh);
    bits = (bits << 10) | (uint32_t)max(b, 0);
    base = above;
  }
  return bits;
}

__global__ void __launch_bounds__(kThreads)
samp_max_kernel(const float* __restrict__ logits, int64_t row_stride, int V, void* ws) {
  __shared__ float red[kThreads / 64];
  const int c = blockIdx.x, row = blockIdx.y;
  const RowWs r = row_ws(ws, row);
  const float* x = logits + (int64_t)row * row_stride;
  int v0, v1;
  chunk_range(V, c, v0, v1);
  float m = -INFINITY;
  for (int v = v0 + threadIdx.x; v < v1; v += kThreads) {
    const float l = x[v];
    if (finite_logit(l)) m = fmaxf(m, l);
  }
  m = block_max(m, red);
  if (threadIdx.x == 0) r.pmax()[c] = m;
  const int z = c * kThreads + threadIdx.x;
  if (z < 3 * kBins) r.hist(0)[z] = 0;  // hist(0..2) are contiguous
}

__global__ void __launch_bounds__(kThreads)
samp_hist_kernel(const float* __restrict__ logits, int64_t row_stride, int V, float inv_t2,
                 float top_p, int level, void* ws) {
  __shared__ uint64_t h[kBins];
  __shared__ ScanShared sh;
  __shared__ uint64_t red[kThreads / 64];
  const int c = blockIdx.x, row = blockIdx.y;
  const RowWs r = row_ws(ws, row);
  const float m = row_max(r);
  if (m == -INFINITY) return;
  const uint32_t prefix = level > 0 ? tau_prefix(r, level, top_p, sh, red) : 0u;
  const int shift = 20 - 10 * level;
  for (int i = threadIdx.x; i < kBins; i += kThreads) h[i] = 0;
  __syncthreads();
  const float* x = logits + (int64_t)row * row_stride;
  int v0, v1;
  chunk_range(V, c, v0, v1);
  for (int v = v0 + threadIdx.x; v < v1; v += kThreads) {
    const float e = weight(x[v], m, inv_t2);
    const uint32_t bits = __float_as_uint(e);
    const uint64_t q = fixed_mass(e);
    if (q != 0 && (level == 0 || (bits >> (shift + 10)) == prefix))
      atomicAdd((unsigned long long*)&h[(bits >> shift) & (kBins - 1)], (unsigned long long)q);
  }
  __syncthreads();
  uint64_t* g = r.hist(level);
  for (int i = threadIdx.x; i < kBins; i += kThreads)
    if (h[i] != 0) atomicAdd((unsigned long long*)&g[i], (unsigned long long)h[i]);
}

// kept mass of every 64-token tile of the chunk (one wave per tile) and of the whole chunk
__global__ void __launch_bounds__(kThreads)
samp_kept_kernel(const float* __restrict__ logits, int64_t row_stride, int V, float inv_t2,
                 float top_p, void* ws) {
  __shared__ ScanShared sh;
  __shared__ uint64_t red[kThreads / 64];
  const int c = blockIdx.x, row = blockIdx.y, lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const RowWs r = row_ws(ws, row);
  const float m = row_max(r);
  if (m == -INFINITY) return;
  const uint32_t tau_bits = top_p < 1.f ? tau_prefix(r, 3, top_p, sh, red) : 0u;
  const float tau = __uint_as_float(tau_bits);
  const float* x = logits + (int64_t)row * row_stride;
  int v0, v1;
  chunk_range(V, c, v0, v1);
  const int ntiles = (v1 - v0 + 63) / 64;
  uint64_t* ts = r.tiles(c);
  uint64_t s = 0;
  constexpr int kW = kThreads / 64;
  for (int t0 = wave; t0 < ntiles; t0 += 4 * kW) {
    uint64_t q[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {  // four tiles' loads in flight before the reductions
      const int v = v0 + (t0 + i * kW) * 64 + lane;
      const float e = v < v1 ? weight(x[v], m, inv_t2) : 0.f;
      q[i] = e >= tau ? fixed_mass(e) : 0;
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int t = t0 + i * kW;
      const uint64_t tsum = wave_sum_u64(q[i]);
      if (t < ntiles && lane == 0) ts[t] = tsum;
      s += q[i];
    }
  }
  s = block_sum_u64(s, red);
  if (threadIdx.x == 0) {
    r.mass()[c] = s;
    if (c == 0) *r.tau() = tau_bits;
  }
}

// one wave per row: the chunk holding r, its tile, the token
__global__ void __launch_bounds__(64)
samp_pick_kernel(const float* __restrict__ logits, int64_t row_stride, int V, float inv_t2,
                 const float* __restrict__ u, const void* ws_, int32_t* __restrict__ out) {
  const int row = blockIdx.x, lane = threadIdx.x;
  const RowWs r = row_ws(const_cast<void*>(ws_), row);
  const float m = row_max(r);
  if (m == -INFINITY) {  // no finite logit
    if (lane == 0) out[row] = 0;
    return;
  }
  const float tau = __uint_as_float(*r.tau());
  uint64_t K = 0;
#pragma unroll
  for (int c = 0; c < kChunks; ++c) K += r.mass()[c];  // >= 2^44: the largest logit has e = 1
  const float uu = fminf(fmaxf(u[row], 0.f), 1.f);
  uint64_t rq = (uint64_t)((double)uu * (double)K);
  rq = min(rq, K - 1);
  // the chunk: the first whose running kept mass exceeds rq (values uniform over the wave)
  int c = 0;
  for (; c < kChunks - 1; ++c) {
    const uint64_t mc = r.mass()[c];
    if (mc > rq) break;
    rq -= mc;
  }
  int v0, v1;
  chunk_range(V, c, v0, v1);
  const int ntiles = (v1 - v0 + 63) / 64;
  // the tile: lane l holds tiles 4l .. 4l + 3
  const uint64_t* ts = r.tiles(c);
  uint64_t tv[4], own = 0;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    tv[j] = 4 * lane + j < ntiles ? ts[4 * lane + j] : 0;
    own += tv[j];
  }
  uint64_t inc = own;
  for (int d = 1; d < 64; d <<= 1) {
    const uint64_t y = shfl_up_u64(inc, d);
    if (lane >= d) inc += y;
  }
  const unsigned long long lhit = __ballot(inc > rq);  // lane 63 holds the chunk's mass > rq
  const int L = lhit ? __builtin_ctzll(lhit) : 63;
  uint64_t acc = shfl_u64(inc - own, L);  // kept mass of the tiles before 4L
  int tile = -1;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const uint64_t tj = shfl_u64(tv[j], L);
    if (tile < 0) {
      if (acc + tj > rq) tile = 4 * L + j;
      else acc += tj;
    }
  }
  if (tile < 0) tile = ntiles - 1;
  const uint64_t off = rq - acc;  // < the tile's kept mass
  // the token: inclusive running mass over the tile's 64 tokens
  const int v = v0 + tile * 64 + lane;
  uint64_t q = 0;
  if (v < v1) {
    const float e = weight(logits[(int64_t)row * row_stride + v], m, inv_t2);
    q = e >= tau ? fixed_mass(e) : 0;
  }
  uint64_t run = q;
  for (int d = 1; d < 64; d <<= 1) {
    const uint64_t y = shfl_up_u64(run, d);
    if (lane >= d) run += y;
  }
  const unsigned long long hit = __ballot(q != 0 && run > off);
  if (lane == 0) out[row] = hit ? v + __builtin_ctzll(hit) : v1 - 1;
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

size_t sample_ws_bytes(int rows) { return rows > 0 ? (size_t)rows * kRowBytes : 0; }

hipError_t sample_rows(const float* logits, int64_t row_stride, int rows, int V,
                       float temperature, float top_p, const float* u, int32_t* out, void* ws,
                       hipStream_t s) {
  if (rows <= 0) return hipSuccess;
  if (!(temperature > 0.f) || !(top_p > 0.f) || top_p > 1.f) return hipErrorInvalidValue;
  if (V <= 0 || V > kMaxV) return hipErrorInvalidValue;
  if (((uintptr_t)ws & 15) != 0) return hipErrorInvalidValue;
  const float inv_t2 = 1.4426950408889634f / temperature;  // e^y = 2^(y log2 e)
  const dim3 grid(kChunks, rows);
  hipLaunchKernelGGL(samp_max_kernel, grid, dim3(kThreads), 0, s, logits, row_stride, V, ws);
  if (top_p < 1.f)
    for (int level = 0; level < 3; ++level)
      hipLaunchKernelGGL(samp_hist_kernel, grid, dim3(kThreads), 0, s, logits, row_stride, V,
                         inv_t2, top_p, level, ws);
  hipLaunchKernelGGL(samp_kept_kernel, grid, dim3(kThreads), 0, s, logits, row_stride, V,
                     inv_t2, top_p, ws);
  hipLaunchKernelGGL(samp_pick_kernel, dim3(rows), dim3(64), 0, s, logits, row_stride, V,
                     inv_t2, u, ws, out);
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
