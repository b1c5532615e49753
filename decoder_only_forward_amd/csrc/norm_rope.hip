// RMSNorm, embedding gather, RoPE table, and the fused q/k RMSNorm + RoPE + KV-cache
// write that follows the QKV projection.
#include "launch.h"

namespace q3 {
namespace {

// RMSNorm of one row per wave: y = x * rsqrt(mean(x^2) + eps) * w, fp32 math, one
// rounding to the fp16 GEMM operand ([P3] "RMSNorm": computed in fp32; [P1] section 6).
DEV void load8(const float* p, float* f) {
  f32x4_t a = *(const f32x4_t*)p, b = *(const f32x4_t*)(p + 4);
  for (int i = 0; i < 4; ++i) { f[i] = a[i]; f[4 + i] = b[i]; }
}
DEV void load8(const bf16_t* p, float* f) { unpack8(ld16(p), f); }

template <typename InT>
__global__ void __launch_bounds__(256)
rmsnorm_kernel(const InT* __restrict__ in, int64_t in_row_stride, int64_t in_row_offset,
               const bf16_t* __restrict__ w, f16_t* __restrict__ out, int rows, int H,
               float eps) {
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= rows) return;
  const InT* x = in + ((int64_t)row * in_row_stride + in_row_offset) * H;
  const int nchunk = H / 8;
  float ss = 0.f;
  for (int c = lane; c < nchunk; c += 64) {
    float f[8];
    load8(x + c * 8, f);
#pragma unroll
    for (int i = 0; i < 8; ++i) ss += f[i] * f[i];
  }
  ss = warp_sum(ss);
  const float inv = rsqrtf(ss / (float)H + eps);
  f16_t* y = out + (int64_t)row * H;
  for (int c = lane; c < nchunk; c += 64) {
    float f[8], g[8];
    load8(x + c * 8, f);
    unpack8(ld16(w + c * 8), g);
    u32x4_t o;
#pragma unroll
    for (int i = 0; i < 4; ++i)
      o[i] = pack_f16x2(f[2 * i] * inv * g[2 * i], f[2 * i + 1] * inv * g[2 * i + 1]);
    st16(y + c * 8, o);
  }
}

// h[t] = E[id[t]] widened to fp32 ([P1] section 5; [P3] "骨架": nn.Embedding).  An id
// outside [0, V) yields a NaN row instead of an out-of-bounds read.
__global__ void __launch_bounds__(256)
embed_kernel(const int32_t* __restrict__ ids, const bf16_t* __restrict__ table,
             float* __restrict__ out, int T, int H, int V) {
  const int nchunk = H / 8;
  const int64_t total = (int64_t)T * nchunk;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total;
       i += (int64_t)gridDim.x * blockDim.x) {
    int t = (int)(i / nchunk), c = (int)(i % nchunk);
    int id = ids[t];
    float f[8];
    if (id >= 0 && id < V) {
      unpack8(ld16(table + (int64_t)id * H + c * 8), f);
    } else {
      for (int j = 0; j < 8; ++j) f[j] = __int_as_float(0x7FC00000);
    }
    float* o = out + (int64_t)t * H + c * 8;
    *(f32x4_t*)o = f32x4_t{f[0], f[1], f[2], f[3]};
    *(f32x4_t*)(o + 4) = f32x4_t{f[4], f[5], f[6], f[7]};
  }
}

// cos/sin of pos * theta^(-2i/hd) in fp64, rounded once to fp32 ([P3] "RoPE":
// the table is precomputed per position up to the maximum context).
__global__ void __launch_bounds__(256)
rope_table_kernel(float* __restrict__ rope, int max_pos, int half, double theta, int hd) {
  const int64_t total = (int64_t)max_pos * half;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total;
       i += (int64_t)gridDim.x * blockDim.x) {
    int pos = (int)(i / half), j = (int)(i % half);
    double inv = exp(-(2.0 * j / (double)hd) * log(theta));
    double ang = (double)pos * inv;
    rope[i] = (float)cos(ang);
    rope[total + i] = (float)sin(ang);
  }
}

// Per (64-token tile, sequence, head slot):
//   q heads:  q = rope(rmsnorm_hd(q)) * log2(e)/sqrt(hd) -> q_out [T][nq][hd] (fp16)
//   k heads:  k = rope(rmsnorm_hd(k)) -> k_cache[b][h][pos][:]
//   v heads:  v -> vt_cache[b][h][:][pos]  (transposed through LDS)
// ([P3] "GQA 注意力": per-head q/k RMSNorm before RoPE, offset = cached length;
// "RoPE": pairs (i, i + hd/2) rotated by pos * theta_i.)
// Lane l of a wave holds dims l and l + 64 of one token: exactly one RoPE plane.
constexpr int kRopeTile = 64;

__global__ void __launch_bounds__(256) qkv_rope_cache_kernel(RopeCacheArgs a) {
  const int HD = 128;
  const int tile = blockIdx.x, b = blockIdx.y, slot = blockIdx.z;
  const int s0 = tile * kRopeTile;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int row_elems = (a.nq + 2 * a.nkv) * HD;
  const int half = HD / 2;

  // The fp16 copies are read in whole 64-position tiles: the last token tile of each
  // k / v head zeroes their tail, from the last new position to the padded width.
  if (a.k_fresh && slot >= a.nq && tile == gridDim.x - 1) {
    const bool is_k = slot < a.nq + a.nkv;
    const int h = is_k ? slot - a.nq : slot - a.nq - a.nkv;
    const int t0 = a.pos0 + a.S - a.fresh_base, nt = a.fresh_w - t0;
    for (int i = threadIdx.x; i < nt * HD; i += 256) {
      const int r = t0 + i / HD, d = i % HD;
      if (is_k)
        a.k_fresh[(((int64_t)b * a.nkv + h) * a.fresh_w + r) * HD + d] = 0;
      else
        a.vt_fresh[(((int64_t)b * a.nkv + h) * HD + d) * a.fresh_w + r] = 0;
    }
  }

  if (slot < a.nq + a.nkv) {
    const bool is_q = slot < a.nq;
    const int h = is_q ? slot : slot - a.nq;
    const bf16_t* nw = is_q ? a.q_norm : a.k_norm;
    const float w0 = a.qk_norm ? bf2f(nw[lane]) : 1.f;
    const float w1 = a.qk_norm ? bf2f(nw[lane + half]) : 1.f;
    for (int j = wave; j < kRopeTile; j += 4) {
      const int s = s0 + j;
      if (s >= a.S) break;
      const int64_t t = (int64_t)b * a.S + s;
      const int pos = a.pos ? a.pos[b] : a.pos0 + s;
      const bool ok = pos >= 0 && pos < a.cap && pos < a.max_pos;
      const float* src = a.qkv + t * row_elems + slot * HD;
      float x0 = src[lane], x1 = src[lane + half];
      if (a.qk_norm) {
        float ss = warp_sum(x0 * x0 + x1 * x1);
        float inv = rsqrtf(ss / (float)HD + a.eps);
        x0 = x0 * inv * w0;
        x1 = x1 * inv * w1;
      }
      float c = 0.f, sn = 0.f;
      if (ok) {
        c = a.rope[(int64_t)pos * half + lane];
        sn = a.rope[(int64_t)a.max_pos * half + (int64_t)pos * half + lane];
      }
      float y0 = x0 * c - x1 * sn;
      float y1 = x0 * sn + x1 * c;
      if (is_q) {
        // q carries the softmax scale log2(e) / sqrt(hd) for the attention kernels
        const float qs = 0.08838834764831845f * kLog2e;
        y0 *= qs;
        y1 *= qs;
        if (!ok) y0 = y1 = __int_as_float(0x7FC00000);
        f16_t* dst = a.q_out + (t * a.nq + h) * HD;
        dst[lane] = f2h(y0);
        dst[lane + half] = f2h(y1);
      } else if (ok) {
        bf16_t* dst = a.k_cache + (((int64_t)b * a.nkv + h) * a.cap + pos) * HD;
        dst[lane] = f2bf(y0);
        dst[lane + half] = f2bf(y1);
        if (a.k_fresh) {
          f16_t* kf = a.k_fresh +
                      (((int64_t)b * a.nkv + h) * a.fresh_w + (pos - a.fresh_base)) * HD;
          kf[lane] = f2h(y0);
          kf[lane + half] = f2h(y1);
        }
      }
    }
    return;
  }

  // value head: stage [64 tokens][128] in LDS, write 64 consecutive positions per d row
  __shared__ float sv[kRopeTile][HD + 1];
  const int h = slot - a.nq - a.nkv;
  for (int i = threadIdx.x; i < kRopeTile * (HD / 2); i += 256) {
    int j = i / (HD / 2), d2 = (i % (HD / 2)) * 2;
    int s = s0 + j;
    float v0 = 0.f, v1 = 0.f;
    if (s < a.S) {
      const int64_t t = (int64_t)b * a.S + s;
      const float* src = a.qkv + t * row_elems + slot * HD + d2;
      v0 = src[0];
      v1 = src[1];
    }
    sv[j][d2] = v0;
    sv[j][d2 + 1] = v1;
  }
  __syncthreads();
  const int s = s0 + lane;
  if (s < a.S) {
    const int pos = a.pos ? a.pos[b] : a.pos0 + s;
    if (pos >= 0 && pos < a.cap && pos < a.max_pos) {
      bf16_t* base = a.vt_cache + ((int64_t)b * a.nkv + h) * HD * a.cap + pos;
      for (int d = wave; d < HD; d += 4) base[(int64_t)d * a.cap] = f2bf(sv[lane][d]);
      if (a.vt_fresh) {
        f16_t* fb = a.vt_fresh + ((int64_t)b * a.nkv + h) * HD * a.fresh_w + (pos - a.fresh_base);
        for (int d = wave; d < HD; d += 4) fb[(int64_t)d * a.fresh_w] = f2h(sv[lane][d]);
      }
    }
  }
}

int blocks_for(int64_t work, int per_block, int cap = 65536) {
  int64_t b = (work + per_block - 1) / per_block;
  if (b < 1) b = 1;
  if (b > cap) b = cap;
  return (int)b;
}

}  // namespace

hipError_t rmsnorm_f32(const float* in, int64_t in_row_stride, int64_t in_row_offset,
                       const bf16_t* w, f16_t* out, int rows, int H, float eps, hipStream_t s) {
  if (rows <= 0) return hipSuccess;
  hipLaunchKernelGGL(rmsnorm_kernel<float>, dim3((rows + 3) / 4), dim3(256), 0, s, in,
                     in_row_stride, in_row_offset, w, out, rows, H, eps);
  return hipGetLastError();
}

hipError_t rmsnorm_bf16(const bf16_t* in, int64_t in_row_stride, int64_t in_row_offset,
                        const bf16_t* w, f16_t* out, int rows, int H, float eps,
                        hipStream_t s) {
  if (rows <= 0) return hipSuccess;
  hipLaunchKernelGGL(rmsnorm_kernel<bf16_t>, dim3((rows + 3) / 4), dim3(256), 0, s, in,
                     in_row_stride, in_row_offset, w, out, rows, H, eps);
  return hipGetLastError();
}

hipError_t embed_gather(const int32_t* ids, const bf16_t* table, float* out, int T, int H, int V,
                        hipStream_t s) {
  if (T <= 0) return hipSuccess;
  hipLaunchKernelGGL(embed_kernel, dim3(blocks_for((int64_t)T * H / 8, 256)), dim3(256), 0, s,
                     ids, table, out, T, H, V);
  return hipGetLastError();
}

hipError_t rope_table(float* rope, int max_pos, int hd, double theta, hipStream_t s) {
  hipLaunchKernelGGL(rope_table_kernel, dim3(blocks_for((int64_t)max_pos * hd / 2, 256)),
                     dim3(256), 0, s, rope, max_pos, hd / 2, theta, hd);
  return hipGetLastError();
}

hipError_t qkv_rope_cache(const RopeCacheArgs& a, hipStream_t s) {
  if (a.B <= 0 || a.S <= 0) return hipSuccess;
  dim3 grid((a.S + kRopeTile - 1) / kRopeTile, a.B, a.nq + 2 * a.nkv);
  hipLaunchKernelGGL(qkv_rope_cache_kernel, grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace q3
