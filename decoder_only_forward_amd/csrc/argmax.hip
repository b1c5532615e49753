// Greedy next-token selection: index of the largest logit per row, lowest index on ties
// ([P1] section 13 argmax; [P4] greedy generation).  Two deterministic passes: per-chunk
// (value, index) candidates, then one wave per row merges them.  NaN never wins.
#include "launch.h"

namespace q3 {
namespace {

DEV void better(float v, int i, float& bv, int& bi) {
  if (v > bv || (v == bv && i < bi)) { bv = v; bi = i; }
}

__global__ void __launch_bounds__(256)
argmax_chunk_kernel(const float* __restrict__ logits, int64_t row_stride, int V, int chunks,
                    float* __restrict__ pv, int32_t* __restrict__ pi) {
  const int chunk = blockIdx.x, row = blockIdx.y;
  const int cs = (V + chunks - 1) / chunks;
  const int v0 = chunk * cs, v1 = min(V, v0 + cs);
  const float* x = logits + (int64_t)row * row_stride;
  float bv = -INFINITY;
  int bi = 0x7FFFFFFF;
  // 16-byte loads over the aligned middle of the chunk, single elements at its ends (the
  // result does not depend on the visiting order: larger value, then lower index, wins)
  const int a0 = min(v1, v0 + (int)(((16 - ((uintptr_t)(x + v0) & 15)) & 15) >> 2));
  const int a1 = a0 + ((v1 - a0) & ~3);
  for (int v = v0 + threadIdx.x; v < a0; v += 256) better(x[v], v, bv, bi);
  for (int v = a0 + 4 * threadIdx.x; v < a1; v += 4 * 256) {
    const f32x4_t q = *(const f32x4_t*)(x + v);
#pragma unroll
    for (int e = 0; e < 4; ++e) better(q[e], v + e, bv, bi);
  }
  for (int v = a1 + threadIdx.x; v < v1; v += 256) better(x[v], v, bv, bi);
  for (int o = 32; o > 0; o >>= 1) {
    float ov = __shfl_xor(bv, o, 64);
    int oi = __shfl_xor(bi, o, 64);
    better(ov, oi, bv, bi);
  }
  __shared__ float sv[4];
  __shared__ int si[4];
  if ((threadIdx.x & 63) == 0) { sv[threadIdx.x >> 6] = bv; si[threadIdx.x >> 6] = bi; }
  __syncthreads();
  if (threadIdx.x == 0) {
    for (int w = 1; w < 4; ++w) better(sv[w], si[w], bv, bi);
    pv[(int64_t)row * chunks + chunk] = bv;
    pi[(int64_t)row * chunks + chunk] = bi;
  }
}

__global__ void __launch_bounds__(64)
argmax_final_kernel(const float* __restrict__ pv, const int32_t* __restrict__ pi, int chunks,
                    int32_t* __restrict__ out) {
  const int row = blockIdx.x;
  float bv = -INFINITY;
  int bi = 0x7FFFFFFF;
  for (int c = threadIdx.x; c < chunks; c += 64)
    better(pv[(int64_t)row * chunks + c], pi[(int64_t)row * chunks + c], bv, bi);
  for (int o = 32; o > 0; o >>= 1) {
    float ov = __shfl_xor(bv, o, 64);
    int oi = __shfl_xor(bi, o, 64);
    better(ov, oi, bv, bi);
  }
  if (threadIdx.x == 0) out[row] = bi == 0x7FFFFFFF ? 0 : bi;
}

}  // namespace

hipError_t argmax_rows(const float* logits, int64_t row_stride, int rows, int V, int32_t* out,
                       float* part_val, int32_t* part_idx, int chunks, hipStream_t s) {
  if (rows <= 0) return hipSuccess;
  hipLaunchKernelGGL(argmax_chunk_kernel, dim3(chunks, rows), dim3(256), 0, s, logits,
                     row_stride, V, chunks, part_val, part_idx);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(argmax_final_kernel, dim3(rows), dim3(64), 0, s, part_val, part_idx,
                     chunks, out);
  return hipGetLastError();
}

}  // namespace q3
