// Copies between plain per-layer K / V tensors [B][nkv][len][128] (the pages' cache: one row
// of head_dim values per position, [P3] "prefill 与 decode") and the library's 32-position
// tiled cache.  Plumbing for callers that fill or read a cache themselves; nothing of the
// decoder's arithmetic.  One thread per 16-byte piece:
//   K: 8 consecutive dims of one position, contiguous on both sides;
//   V: 8 consecutive positions of one dim, contiguous in the tiled V^T rows, 128 elements
//      apart in the plain tensor.
#include <algorithm>

#include "launch.h"

namespace q3 {
namespace {

constexpr int HD = 128;

// pieces per (sequence, kv head): len * 16 for K, (len / 8 rounded up) * 128 for V
__global__ void __launch_bounds__(256)
kv_copy_kernel(bf16_t* __restrict__ k_plain, bf16_t* __restrict__ v_plain,
               bf16_t* __restrict__ k_tiled, bf16_t* __restrict__ vt_tiled, int regions,
               int len, int cap, bool to_tiled) {
  const int64_t kp = (int64_t)len * (HD / 8), vp = (int64_t)((len + 7) / 8) * HD;
  const int64_t per = kp + vp, total = (int64_t)regions * per;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total;
       i += (int64_t)gridDim.x * blockDim.x) {
    const int64_t r = i / per, j = i % per;
    bf16_t* const kt = k_tiled + r * cap * HD;
    bf16_t* const vt = vt_tiled + r * cap * HD;
    bf16_t* const kl = k_plain + r * len * HD;
    bf16_t* const vl = v_plain + r * len * HD;
    if (j < kp) {
      const int pos = (int)(j / (HD / 8)), d = (int)(j % (HD / 8)) * 8;
      if (to_tiled) st16(kt + kcache_idx(pos, d), ld16(kl + (int64_t)pos * HD + d));
      else st16(kl + (int64_t)pos * HD + d, ld16(kt + kcache_idx(pos, d)));
    } else {
      const int64_t jv = j - kp;
      const int d = (int)(jv % HD), p0 = (int)(jv / HD) * 8, n = min(8, len - p0);
      if (to_tiled) {
        if (n == 8 && (p0 & 31) + 8 <= 32) {
          u32x4_t o;
#pragma unroll
          for (int e = 0; e < 4; ++e)
            o[e] = (uint32_t)vl[(int64_t)(p0 + 2 * e) * HD + d] |
                   ((uint32_t)vl[(int64_t)(p0 + 2 * e + 1) * HD + d] << 16);
          st16(vt + vcache_idx(p0, d), o);
        } else {
          for (int e = 0; e < n; ++e) vt[vcache_idx(p0 + e, d)] = vl[(int64_t)(p0 + e) * HD + d];
        }
      } else {
        for (int e = 0; e < n; ++e) vl[(int64_t)(p0 + e) * HD + d] = vt[vcache_idx(p0 + e, d)];
      }
    }
  }
}

}  // namespace

hipError_t kv_copy(void* k_plain, void* v_plain, void* k_tiled, void* vt_tiled, int regions,
                   int len, int cap, bool to_tiled, hipStream_t s) {
  if (regions <= 0 || len <= 0) return hipSuccess;
  const int64_t per = (int64_t)len * (HD / 8) + (int64_t)((len + 7) / 8) * HD;
  const int64_t total = per * regions;
  const int blocks = (int)std::min<int64_t>((total + 255) / 256, 65536);
  hipLaunchKernelGGL(kv_copy_kernel, dim3(blocks), dim3(256), 0, s, (bf16_t*)k_plain,
                     (bf16_t*)v_plain, (bf16_t*)k_tiled, (bf16_t*)vt_tiled, regions, len, cap,
                     to_tiled);
  return hipGetLastError();
}

}  // namespace q3
