// Device side of the seeded input generator (definition in synth_core.h).
// Produces the same bits as synth_host.c, directly in device memory, so large
// synthetic inputs (weights, a pre-filled KV cache) never cross PCIe.
// Same logical->physical layout rule as the host side:
//   counter = offset + (b*rows + r)*cols + c,  address = b*ld_b + r*ld_r + c*ld_c.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "synth_core.h"

namespace {

__global__ void __launch_bounds__(256)
normal_bf16_kernel(uint64_t key, uint64_t offset, int64_t batch, int64_t rows, int64_t cols,
                   float mean, float stdv, uint16_t* __restrict__ out, int64_t ld_b,
                   int64_t ld_r, int64_t ld_c) {
  const int64_t total = batch * rows * cols;
  const int64_t step = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total; i += step) {
    int64_t c = i % cols;
    int64_t br = i / cols;
    int64_t r = br % rows;
    int64_t b = br / rows;
    out[b * ld_b + r * ld_r + c * ld_c] = synth_normal_bf16_at(key, offset + (uint64_t)i, mean, stdv);
  }
}

__global__ void __launch_bounds__(256)
uniform_i32_kernel(uint64_t key, uint64_t offset, int64_t batch, int64_t rows, int64_t cols,
                   int32_t lo, int32_t hi, int32_t* __restrict__ out, int64_t ld_b, int64_t ld_r,
                   int64_t ld_c) {
  const int64_t total = batch * rows * cols;
  const int64_t step = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total; i += step) {
    int64_t c = i % cols;
    int64_t br = i / cols;
    int64_t r = br % rows;
    int64_t b = br / rows;
    out[b * ld_b + r * ld_r + c * ld_c] = synth_uniform_at(key, offset + (uint64_t)i, lo, hi);
  }
}

int grid_for(int64_t total) {
  int64_t blocks = (total + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  if (blocks < 1) blocks = 1;
  return (int)blocks;
}

}  // namespace

extern "C" int synth_normal_bf16_3d_device(uint64_t seed, uint64_t stream, uint64_t offset,
                                           int64_t batch, int64_t rows, int64_t cols, float mean,
                                           float stdv, void* out, int64_t ld_b, int64_t ld_r,
                                           int64_t ld_c, void* hip_stream) {
  int64_t total = batch * rows * cols;
  if (total <= 0) return 0;
  hipLaunchKernelGGL(normal_bf16_kernel, dim3(grid_for(total)), dim3(256), 0,
                     (hipStream_t)hip_stream, synth_key(seed, stream), offset, batch, rows, cols,
                     mean, stdv, (uint16_t*)out, ld_b, ld_r, ld_c);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

extern "C" int synth_uniform_i32_3d_device(uint64_t seed, uint64_t stream, uint64_t offset,
                                           int64_t batch, int64_t rows, int64_t cols, int32_t lo,
                                           int32_t hi, void* out, int64_t ld_b, int64_t ld_r,
                                           int64_t ld_c, void* hip_stream) {
  int64_t total = batch * rows * cols;
  if (total <= 0) return 0;
  hipLaunchKernelGGL(uniform_i32_kernel, dim3(grid_for(total)), dim3(256), 0,
                     (hipStream_t)hip_stream, synth_key(seed, stream), offset, batch, rows, cols,
                     lo, hi, (int32_t*)out, ld_b, ld_r, ld_c);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}
