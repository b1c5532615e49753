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
  constexpr int kKeep = 4;  // chunks of 8 a lane keeps in registers (rows up to 2048 wide)
  if (nchunk <= 64 * kKeep) {
    // one pass over the row: every load is issued before the reduction
    float f[kKeep][8];
    float ss = 0.f;
#pragma unroll
    for (int k = 0; k < kKeep; ++k) {
      const int c = lane + 64 * k;
      if (c < nchunk) {
        load8(x + c * 8, f[k]);
      } else {
#pragma unroll
        for (int i = 0; i < 8; ++i) f[k][i] = 0.f;
      }
    }
#pragma unroll
    for (int k = 0; k < kKeep; ++k)
#pragma unroll
      for (int i = 0; i < 8; ++i) ss += f[k][i] * f[k][i];
    ss = warp_sum(ss);
    const float inv = rsqrtf(ss / (float)H + eps);
    f16_t* y = out + (int64_t)row * H;
#pragma unroll
    for (int k = 0; k < kKeep; ++k) {
      const int c = lane + 64 * k;
      if (c >= nchunk) break;
      float g[8];
      unpack8(ld16(w + c * 8), g);
      u32x4_t o;
#pragma unroll
      for (int i = 0; i < 4; ++i)
        o[i] = pack_f16x2(f[k][2 * i] * inv * g[2 * i], f[k][2 * i + 1] * inv * g[2 * i + 1]);
      st16(y + c * 8, o);
    }
    return;
  }
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
//   k heads:  k = rope(rmsnorm_hd(k)) -> K cache of (b, h) at pos
//   v heads:  v -> V cache of (b, h) at pos  (dim-major inside each 32-position tile,
//             transposed through LDS)
// ([P3] "GQA 注意力": per-head q/k RMSNorm before RoPE, offset = cached length;
// "RoPE": pairs (i, i + hd/2) rotated by pos * theta_i; with a.interleaved the planes are
// (2i, 2i + 1) instead, the complex-number form of [P1] section 8.)
// q / k heads: 16 lanes per token row, lane j holding dims 8j .. 8j + 7 (16-byte loads and
// stores); the rotate-half partner of dim d is dim d ^ 64, held by lane j ^ 8 of the same
// 16-lane row, so the exchange and the sum of squares are row-local DPP rotations; the
// interleaved partner d ^ 1 is in the same lane.
constexpr int kRopeTile = 64;

// rotate within 16-lane rows by n (n in 1..15)

// Prefill: tokens of sequence b at positions pos0 .. pos0 + S - 1 (decode steps use
// qkv_rope_decode_kernel below).
__global__ void __launch_bounds__(256) qkv_rope_cache_kernel(RopeCacheArgs a) {
  const int HD = 128;
  const int tile = blockIdx.x, b = blockIdx.y, slot = blockIdx.z;
  const int s0 = tile * kRopeTile;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int row_elems = (a.nq + 2 * a.nkv) * HD;
  const int half = HD / 2;

  // The fp16 copies are read in whole 64-position tiles: the last token tile of each
  // k / v head zeroes their tail, from the last new position to the padded width.
  if (a.k_fresh && slot >= a.nq && tile == gridDim.x - 1) {
    const bool is_k = slot < a.nq + a.nkv;
    const int h = is_k ? slot - a.nq : slot - a.nq - a.nkv;
    const int t0 = a.pos0 + a.S - a.fresh_base, nt = a.fresh_w - t0;
    for (int i = tid; i < nt * HD; i += 256) {
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
    const int j = lane & 15, sub = lane >> 4;  // 4 token rows per wave step
    const int d0 = 8 * j;                       // first dim of this lane
    // first RoPE frequency index of this lane's dims: 8 consecutive (rotate-half) or the
    // 4 planes (2i, 2i + 1) its 8 dims form (interleaved)
    const int i0 = a.interleaved ? d0 / 2 : d0 & (half - 1);
    const float sgn = d0 < half ? -1.f : 1.f;   // y = x c + sgn * partner * s
    float w[8];
    if (a.qk_norm) {
      unpack8(ld16((is_q ? a.q_norm : a.k_norm) + d0), w);
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) w[e] = 1.f;
    }
    // all rows' loads (activations and RoPE table) are issued before any is used
    constexpr int RPL = kRopeTile / 16;  // token rows per lane
    u32x4_t raw[RPL];
    f32x4_t tc[RPL][2], ts[RPL][2];
    int pos_r[RPL];
    bool ok_r[RPL], live_r[RPL];
#pragma unroll
    for (int k = 0; k < RPL; ++k) {
      const int s = s0 + wave * 4 + sub + 16 * k;
      live_r[k] = s < a.S;
      const int sc = live_r[k] ? s : a.S - 1;
      const int64_t t = (int64_t)b * a.S + sc;
      const int pos = a.pos0 + sc;
      ok_r[k] = pos >= 0 && pos < a.cap && pos < a.max_pos;
      pos_r[k] = pos;
      // rows past the end load a clamped row so that every load is unconditional
      raw[k] = ld16(a.qkv + t * row_elems + slot * HD + d0);
      const int pc = ok_r[k] ? pos : 0;
      const float* cp = a.rope + (int64_t)pc * half + i0;
      const float* sp = a.rope + ((int64_t)a.max_pos + pc) * half + i0;
      tc[k][0] = *(const f32x4_t*)cp;
      ts[k][0] = *(const f32x4_t*)sp;
      if (!a.interleaved) {
        tc[k][1] = *(const f32x4_t*)(cp + 4);
        ts[k][1] = *(const f32x4_t*)(sp + 4);
      }
    }
#pragma unroll
    for (int k = 0; k < RPL; ++k) {
      if (!live_r[k]) break;
      const int s = s0 + wave * 4 + sub + 16 * k;
      const int64_t t = (int64_t)b * a.S + s;
      const int pos = pos_r[k];
      const bool ok = ok_r[k];
      float x[8];
      unpack8_f16(raw[k], x);
      if (a.qk_norm) {
        float ss = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) ss += x[e] * x[e];
        ss += ror16<8>(ss);
        ss += ror16<4>(ss);
        ss += ror16<2>(ss);
        ss += ror16<1>(ss);
        const float inv = rsqrtf(ss / (float)HD + a.eps);
#pragma unroll
        for (int e = 0; e < 8; ++e) x[e] = x[e] * inv * w[e];
      }
      float y[8];
      if (a.interleaved) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float c = ok ? tc[k][0][e] : 0.f, sn = ok ? ts[k][0][e] : 0.f;
          y[2 * e] = x[2 * e] * c - x[2 * e + 1] * sn;
          y[2 * e + 1] = x[2 * e] * sn + x[2 * e + 1] * c;
        }
      } else {
        float c[8], sn[8];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          c[e] = ok ? tc[k][0][e] : 0.f;
          c[e + 4] = ok ? tc[k][1][e] : 0.f;
          sn[e] = ok ? ts[k][0][e] : 0.f;
          sn[e + 4] = ok ? ts[k][1][e] : 0.f;
        }
#pragma unroll
        for (int e = 0; e < 8; ++e) y[e] = x[e] * c[e] + sgn * ror16<8>(x[e]) * sn[e];
      }
      if (is_q) {
        // q carries the softmax scale log2(e) / sqrt(hd) for the attention kernels
        const float qs = 0.08838834764831845f * kLog2e;
        u32x4_t o;
#pragma unroll
        for (int e = 0; e < 4; ++e)
          o[e] = ok ? pack_f16x2(y[2 * e] * qs, y[2 * e + 1] * qs) : 0x7E007E00u;
        st16(a.q_out + (t * a.nq + h) * HD + d0, o);
      } else if (ok) {
        u32x4_t kb, kh;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          kb[e] = pack_bf16x2(y[2 * e], y[2 * e + 1]);
          kh[e] = pack_f16x2(y[2 * e], y[2 * e + 1]);
        }
        st16(a.k_cache + ((int64_t)b * a.nkv + h) * a.cap * HD + kcache_idx(pos, d0), kb);
        if (a.k_fresh)
          st16(a.k_fresh + (((int64_t)b * a.nkv + h) * a.fresh_w + (pos - a.fresh_base)) * HD + d0,
               kh);
      }
    }
    return;
  }

  // value head: stage [64 tokens][128] in LDS (fp32, padded rows), then write V^T rows of
  // 8 consecutive positions per lane (16-byte stores)
  __shared__ float sv[kRopeTile][HD + 1];
  const int h = slot - a.nq - a.nkv;
  {
    constexpr int PER = kRopeTile * (HD / 8) / 256;  // 16-byte chunks per thread
    u32x4_t raw[PER];
#pragma unroll
    for (int k = 0; k < PER; ++k) {
      const int i = tid + 256 * k;
      const int r = i / (HD / 8), d = (i % (HD / 8)) * 8;
      const int s = min(s0 + r, a.S - 1);
      raw[k] = ld16(a.qkv + ((int64_t)b * a.S + s) * row_elems + slot * HD + d);
    }
#pragma unroll
    for (int k = 0; k < PER; ++k) {
      const int i = tid + 256 * k;
      const int r = i / (HD / 8), d = (i % (HD / 8)) * 8;
      float v[8];
      unpack8_f16(raw[k], v);
      const bool live = s0 + r < a.S;
#pragma unroll
      for (int e = 0; e < 8; ++e) sv[r][d + e] = live ? v[e] : 0.f;
    }
  }
  __syncthreads();
  // positions pos0 + s0 .. contiguous
  for (int i = tid; i < HD * (kRopeTile / 8); i += 256) {
    const int d = i / (kRopeTile / 8), r0 = (i % (kRopeTile / 8)) * 8;
    const int s = s0 + r0;
    if (s >= a.S) continue;
    const int pos = a.pos0 + s;
    const int n = min(8, a.S - s);  // valid tokens in this group
    bf16_t* const vreg = a.vt_cache + ((int64_t)b * a.nkv + h) * a.cap * HD;
    f16_t* vf = a.vt_fresh ? a.vt_fresh + (((int64_t)b * a.nkv + h) * HD + d) * a.fresh_w +
                                 (pos - a.fresh_base)
                           : nullptr;
    if (n == 8 && (pos & 7) == 0 && (!vf || ((pos - a.fresh_base) & 7) == 0)) {
      u32x4_t ob, oh;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        ob[e] = pack_bf16x2(sv[r0 + 2 * e][d], sv[r0 + 2 * e + 1][d]);
        oh[e] = pack_f16x2(sv[r0 + 2 * e][d], sv[r0 + 2 * e + 1][d]);
      }
      st16(vreg + vcache_idx(pos, d), ob);
      if (vf) st16(vf, oh);
    } else {
      for (int e = 0; e < n; ++e) {
        vreg[vcache_idx(pos + e, d)] = f2bf(sv[r0 + e][d]);
        if (vf) vf[e] = f2h(sv[r0 + e][d]);
      }
    }
  }
}

// Decode residual projections split over K: one block per row sums the partials in a fixed
// order, adds the residual, writes the residual stream and (optionally) the RMSNorm of the
// new row that the next projection consumes ([P3] "TransformerBlock": x + sublayer(x),
// then the next pre-norm).  Thread t owns columns 4 t .. 4 t + 3 (+ 1024 for N > 1024).
constexpr int kResMaxIter = 2;  // N <= 2048

__global__ void __launch_bounds__(256)
splitk_res_norm_kernel(const float* __restrict__ part, int splits, int M, int N,
                       const void* residual, bool residual_bf16, void* out, bool out_bf16,
                       const bf16_t* __restrict__ norm_w, f16_t* __restrict__ xn, float eps) {
  __shared__ float sred[4];
  const int m = blockIdx.x, tid = threadIdx.x;
  float v[kResMaxIter][4];
  float ss = 0.f;
#pragma unroll
  for (int it = 0; it < kResMaxIter; ++it) {
    const int c = (it * 256 + tid) * 4;
    if (c >= N) continue;
    const int64_t o = (int64_t)m * N + c;
    f32x4_t acc;
    if (residual_bf16) {
      const u32x2_t r = *(const u32x2_t*)((const bf16_t*)residual + o);
      acc = f32x4_t{__uint_as_float(r[0] << 16), __uint_as_float(r[0] & 0xffff0000u),
                    __uint_as_float(r[1] << 16), __uint_as_float(r[1] & 0xffff0000u)};
    } else {
      acc = *(const f32x4_t*)((const float*)residual + o);
    }
    for (int sp = 0; sp < splits; ++sp) {
      const f32x4_t pv = *(const f32x4_t*)(part + ((int64_t)sp * M + m) * N + c);
#pragma unroll
      for (int e = 0; e < 4; ++e) acc[e] += pv[e];
    }
    if (out_bf16)
      *(u32x2_t*)((bf16_t*)out + o) = u32x2_t{pack_bf16x2(acc[0], acc[1]), pack_bf16x2(acc[2], acc[3])};
    else
      *(f32x4_t*)((float*)out + o) = acc;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      v[it][e] = acc[e];
      ss += acc[e] * acc[e];
    }
  }
  if (norm_w == nullptr) return;
  ss = warp_sum(ss);
  if ((tid & 63) == 0) sred[tid >> 6] = ss;
  __syncthreads();
  const float inv = rsqrtf((sred[0] + sred[1] + sred[2] + sred[3]) / (float)N + eps);
#pragma unroll
  for (int it = 0; it < kResMaxIter; ++it) {
    const int c = (it * 256 + tid) * 4;
    if (c >= N) continue;
    const u32x2_t wv = *(const u32x2_t*)(norm_w + c);
    const float w0 = __uint_as_float(wv[0] << 16), w1 = __uint_as_float(wv[0] & 0xffff0000u);
    const float w2 = __uint_as_float(wv[1] << 16), w3 = __uint_as_float(wv[1] & 0xffff0000u);
    *(u32x2_t*)(xn + (int64_t)m * N + c) =
        u32x2_t{pack_f16x2(v[it][0] * inv * w0, v[it][1] * inv * w1),
                pack_f16x2(v[it][2] * inv * w2, v[it][3] * inv * w3)};
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

hipError_t splitk_res_norm(const float* part, int splits, int M, int N, const void* residual,
                           bool residual_bf16, void* out, bool out_bf16, const bf16_t* norm_w,
                           f16_t* xn, float eps, hipStream_t s) {
  if (M <= 0) return hipSuccess;
  if (N % 4 || N > 256 * 4 * kResMaxIter) return hipErrorInvalidValue;
  hipLaunchKernelGGL(splitk_res_norm_kernel, dim3(M), dim3(256), 0, s, part, splits, M, N,
                     residual, residual_bf16, out, out_bf16, norm_w, xn, eps);
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

// Decode: 16 lanes per (token row, head slot), 16 such items per block, so a step of a few
// tokens per sequence launches as many blocks as it has work (one (64-token tile, sequence,
// head) block each would leave 15 of 16 lane groups idle).  q/k heads: RMSNorm and RoPE as
// above; v heads: 8 dims per lane written into their V^T rows at the token's position.
__global__ void __launch_bounds__(256) qkv_rope_decode_kernel(RopeCacheArgs a) {
  const int HD = 128, half = HD / 2;
  const int slots = a.nq + 2 * a.nkv;
  const int item = blockIdx.x * 16 + (threadIdx.x >> 4);
  const int T = a.B * a.S;
  if (item >= T * slots) return;  // whole 16-lane groups leave together
  const int t = item / slots, slot = item % slots;
  const int b = t / a.S, sq = t % a.S;
  const int p0 = a.pos[b];
  const bool ok = p0 >= 0 && p0 + a.S <= a.cap && p0 + a.S <= a.max_pos;
  const int pos = p0 + sq;
  const int j = threadIdx.x & 15, d0 = 8 * j;
  const int row_elems = slots * HD;
  float x[8];
  unpack8_f16(ld16(a.qkv + (int64_t)t * row_elems + slot * HD + d0), x);
  if (slot >= a.nq + a.nkv) {  // v head
    if (!ok) return;
    const int h = slot - a.nq - a.nkv;
    bf16_t* const vreg = a.vt_cache + ((int64_t)b * a.nkv + h) * a.cap * HD;
#pragma unroll
    for (int e = 0; e < 8; ++e) vreg[vcache_idx(pos, d0 + e)] = f2bf(x[e]);
    return;
  }
  const bool is_q = slot < a.nq;
  const int h = is_q ? slot : slot - a.nq;
  if (a.qk_norm) {
    float w[8];
    unpack8(ld16((is_q ? a.q_norm : a.k_norm) + d0), w);
    float ss = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) ss += x[e] * x[e];
    ss += ror16<8>(ss);
    ss += ror16<4>(ss);
    ss += ror16<2>(ss);
    ss += ror16<1>(ss);
    const float inv = rsqrtf(ss / (float)HD + a.eps);
#pragma unroll
    for (int e = 0; e < 8; ++e) x[e] = x[e] * inv * w[e];
  }
  const int pc = ok ? pos : 0;
  const int i0 = a.interleaved ? d0 / 2 : d0 & (half - 1);
  const float* cp = a.rope + (int64_t)pc * half + i0;
  const float* sp = a.rope + ((int64_t)a.max_pos + pc) * half + i0;
  float y[8];
  if (a.interleaved) {
    const f32x4_t c4 = *(const f32x4_t*)cp, s4 = *(const f32x4_t*)sp;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float c = ok ? c4[e] : 0.f, sn = ok ? s4[e] : 0.f;
      y[2 * e] = x[2 * e] * c - x[2 * e + 1] * sn;
      y[2 * e + 1] = x[2 * e] * sn + x[2 * e + 1] * c;
    }
  } else {
    const float sgn = d0 < half ? -1.f : 1.f;
    const f32x4_t c0 = *(const f32x4_t*)cp, c1 = *(const f32x4_t*)(cp + 4);
    const f32x4_t s0 = *(const f32x4_t*)sp, s1 = *(const f32x4_t*)(sp + 4);
    float c[8], sn[8];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      c[e] = ok ? c0[e] : 0.f;
      c[e + 4] = ok ? c1[e] : 0.f;
      sn[e] = ok ? s0[e] : 0.f;
      sn[e + 4] = ok ? s1[e] : 0.f;
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) y[e] = x[e] * c[e] + sgn * ror16<8>(x[e]) * sn[e];
  }
  if (is_q) {
    const float qs = 0.08838834764831845f * kLog2e;
    u32x4_t o;
#pragma unroll
    for (int e = 0; e < 4; ++e)
      o[e] = ok ? pack_f16x2(y[2 * e] * qs, y[2 * e + 1] * qs) : 0x7E007E00u;
    st16(a.q_out + ((int64_t)t * a.nq + h) * HD + d0, o);
  } else if (ok) {
    u32x4_t kb;
#pragma unroll
    for (int e = 0; e < 4; ++e) kb[e] = pack_bf16x2(y[2 * e], y[2 * e + 1]);
    st16(a.k_cache + ((int64_t)b * a.nkv + h) * a.cap * HD + kcache_idx(pos, d0), kb);
  }
}

hipError_t qkv_rope_cache(const RopeCacheArgs& a, hipStream_t s) {
  if (a.B <= 0 || a.S <= 0) return hipSuccess;
  if (a.pos) {
    const int64_t items = (int64_t)a.B * a.S * (a.nq + 2 * a.nkv);
    hipLaunchKernelGGL(qkv_rope_decode_kernel, dim3((unsigned)((items + 15) / 16)), dim3(256), 0,
                       s, a);
    return hipGetLastError();
  }
  dim3 grid((a.S + kRopeTile - 1) / kRopeTile, a.B, a.nq + 2 * a.nkv);
  hipLaunchKernelGGL(qkv_rope_cache_kernel, grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace q3
