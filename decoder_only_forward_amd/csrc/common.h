// Device helpers shared by the gfx950 kernels of libqwen3.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

typedef uint16_t bf16_t;  // bfloat16 bits
typedef uint16_t f16_t;   // IEEE binary16 bits (transient activations)
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

#define DEV static __device__ __forceinline__

DEV float bf2f(bf16_t h) { return __uint_as_float((uint32_t)h << 16); }

// fp32 -> bf16, round to nearest even; a NaN input stays a (quiet) NaN.  One conversion
// instruction (v_cvt_pk_bf16_f32), with no per-element branch for the NaN case.
DEV bf16_t f2bf(float f) { return __builtin_bit_cast(bf16_t, (__bf16)f); }

// two floats -> packed bf16 pair, round to nearest even, NaN stays NaN (v_cvt_pk_bf16_f32)
DEV uint32_t pack_bf16x2(float lo, float hi) {
  typedef __bf16 b2 __attribute__((ext_vector_type(2)));
  typedef float f2 __attribute__((ext_vector_type(2)));
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f2{lo, hi}), b2));
}

// fp16 <-> fp32 (round to nearest even)
DEV float h2f(f16_t h) { return (float)__builtin_bit_cast(_Float16, h); }
DEV f16_t f2h(float f) { return __builtin_bit_cast(f16_t, (_Float16)f); }
// two floats -> packed fp16 pair, round to nearest even (one v_cvt_pk_f16_f32)
DEV uint32_t pack_f16x2(float lo, float hi) {
  typedef _Float16 h2 __attribute__((ext_vector_type(2)));
  typedef float f2 __attribute__((ext_vector_type(2)));
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f2{lo, hi}), h2));
}
DEV void unpack8_f16(const u32x4_t v, float* f) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    f[2 * i] = h2f((f16_t)(v[i] & 0xFFFFu));
    f[2 * i + 1] = h2f((f16_t)(v[i] >> 16));
  }
}
// Two bf16 -> two fp16.  Exact for magnitudes in fp16's normal range
// [6.1e-5, 65504]; smaller values become fp16 subnormals (error <= 6e-8).
DEV uint32_t bf16x2_to_f16x2(uint32_t v) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(__uint_as_float(v << 16),
                                                                 __uint_as_float(v & 0xFFFF0000u)));
}
DEV u32x4_t bf16x8_to_f16x8(u32x4_t v) {
  return u32x4_t{bf16x2_to_f16x2(v[0]), bf16x2_to_f16x2(v[1]), bf16x2_to_f16x2(v[2]),
                 bf16x2_to_f16x2(v[3])};
}

// Unpack 8 bf16 held in a 16-byte vector into floats.
DEV void unpack8(const u32x4_t v, float* f) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    f[2 * i] = __uint_as_float(v[i] << 16);
    f[2 * i + 1] = __uint_as_float(v[i] & 0xFFFF0000u);
  }
}

DEV float warp_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

DEV float warp_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}

// Reductions over the four 16-lane rows of a wave (lanes r, r + 16, r + 32, r + 48) with
// the gfx950 row-swap permutes (VALU only, no LDS round trip).  Every lane receives the
// same result, formed in the same order.
DEV float rows4_max(float x) {
  auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
DEV float rows4_sum(float x) {
  auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// silu(z) = z / (1 + e^-z), the division taken as the hardware reciprocal (about one fp32
// ulp): every caller rounds silu(g) * u to fp16 next, 2^13 times coarser, and the IEEE
// division sequence would cost nine vector instructions per element in the SwiGLU epilogues.
DEV float silu(float z) { return z * __builtin_amdgcn_rcpf(1.0f + __expf(-z)); }

// Reinterpret 4 dwords as 8 bf16 / 8 fp16 for the MFMA builtins.
DEV bf16x8_t as_bf16x8(u32x4_t v) { return __builtin_bit_cast(bf16x8_t, v); }
DEV f16x8_t as_f16x8(u32x4_t v) { return __builtin_bit_cast(f16x8_t, v); }

DEV u32x4_t ld16(const void* p) { return *(const u32x4_t*)p; }
DEV void st16(void* p, u32x4_t v) { *(u32x4_t*)p = v; }

constexpr float kLog2e = 1.4426950408889634f;

// KV-cache layout (bf16, per layer).  Each (sequence, kv head) owns a region of cap * 128
// elements; positions are grouped in tiles of 32 (cap is a multiple of 64):
//   K: [cap / 32][4][32][32]  tile, 32-dim chunk, position in the tile, dim in the chunk
//   V: [cap / 32][128][32]    tile, dim, position in the tile
// so one 32-position tile is 8 KB of K and 8 KB of V, and every 128-byte line a decode
// fragment load touches is read whole by that load.  Element offsets inside a region:
DEV int kcache_idx(int pos, int d) {
  return ((((pos >> 5) << 2) + (d >> 5)) << 10) + ((pos & 31) << 5) + (d & 31);
}
DEV int vcache_idx(int pos, int d) { return ((((pos >> 5) << 7) + d) << 5) + (pos & 31); }

// x from the lane N places round the same 16-lane row (DPP row_ror)
template <int N>
DEV float ror16(float x) {
  return __int_as_float(
      __builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x120 + N, 0xf, 0xf, false));
}

// Asynchronous 16-byte global -> LDS copy (global_load_lds_dwordx4): the 64 lanes of the
// wave write 1 KB at lds_base + 16 * lane (lds_base must be wave-uniform).  It is issued
// from inline asm so that the compiler does not make every later LDS read wait for it
// (it cannot tell that the copy targets the other half of a double buffer); the caller
// publishes the data with wait_dma() before the barrier that precedes its use.  The copy
// writes only LDS (no destination registers) and reads its address registers at issue;
// M0 is saved and restored inside the block.
DEV void lds_dma16(const void* gptr, void* lds_base) {
  uint32_t lds = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)lds_base);
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %2\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %1, off\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "v"(gptr), "s"(lds)
      : "memory");
}
// vmcnt(0) (expcnt and lgkmcnt left at their maxima), through the builtin so that the
// compiler's own wait-count bookkeeping sees it: loads issued before it are known complete
// afterwards, and no later vmcnt wait is inserted for them.
DEV void wait_dma() { __builtin_amdgcn_s_waitcnt(0x0F70); }
