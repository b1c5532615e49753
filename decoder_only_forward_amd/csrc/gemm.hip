// GEMM launchers: tile-family choice, split-K reduction, template instantiations.
#include <algorithm>

#include "launch.h"

namespace q3 {
namespace {

using namespace gemm;

using TBig = Tile<256, 256, 2, 4>;   // 8 waves (2 per SIMD), 128x64 per wave, 128 KB LDS
using TMid = Tile<128, 128, 2, 2>;   // 4 waves, 64x64 per wave, 32 KB LDS
using TSkin = Tile<64, 128, 2, 2>;   // 4 waves, 32x64 per wave: decode (M <= 64)

template <class T>
int tiles_m(int M) { return (M + T::BM - 1) / T::BM; }
template <class T>
int tiles_n(int N, int bmode) {
  return (N + T::BN - 1) / T::BN;
}

template <class T, bool F16, int BMODE, int EPI, bool G, bool SK>
hipError_t launch_t(Args a, int splits, hipStream_t s) {
  if (!G) a.m_tiles = tiles_m<T>(a.M);
  a.n_tiles = tiles_n<T>(a.N, BMODE);
  a.k_splits = splits;
  dim3 grid(a.m_tiles * a.n_tiles, SK ? splits : 1);
  hipLaunchKernelGGL((gemm_kernel<T, F16, BMODE, EPI, G, SK>), grid, dim3(T::THREADS), 0, s, a);
  return hipGetLastError();
}

// Sum the split-K partials and apply the epilogue.
__global__ void __launch_bounds__(256)
splitk_reduce_kernel(const float* __restrict__ part, int splits, int M, int N, int epi,
                     void* C, int64_t ldc, const void* R, int64_t ldr, int BN, int WN) {
  const int ncols = epi == E_SWIGLU ? N / 2 : N;
  const int64_t total = (int64_t)M * ncols;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total;
       i += (int64_t)gridDim.x * blockDim.x) {
    int m = (int)(i / ncols), c = (int)(i % ncols);
    if (epi == E_SWIGLU) {
      int half = WN / 2;
      int vg = (c / (BN / 2)) * BN + ((c % (BN / 2)) / half) * WN + (c % half);
      int vu = vg + half;
      float g = 0.f, u = 0.f;
      for (int z = 0; z < splits; ++z) {
        g += part[((int64_t)z * M + m) * N + vg];
        u += part[((int64_t)z * M + m) * N + vu];
      }
      ((f16_t*)C)[m * ldc + c] = f2h(silu(g) * u);
      continue;
    }
    float v = 0.f;
    for (int z = 0; z < splits; ++z) v += part[((int64_t)z * M + m) * N + c];
    switch (epi) {
      case E_F32: ((float*)C)[m * ldc + c] = v; break;
      case E_F16: ((f16_t*)C)[m * ldc + c] = f2h(v); break;
      case E_RES_F32: ((float*)C)[m * ldc + c] = ((const float*)R)[m * ldr + c] + v; break;
      case E_RESB_F32:
        ((float*)C)[m * ldc + c] = bf2f(((const bf16_t*)R)[m * ldr + c]) + v;
        break;
      case E_RESF_B16:
        ((bf16_t*)C)[m * ldc + c] = f2bf(((const float*)R)[m * ldr + c] + v);
        break;
      default: break;
    }
  }
}

}  // namespace

GemmPlan gemm_plan(int M, int N, int K, int bmode, int epi, bool grouped) {
  GemmPlan p{kMid, 1, 0};
  if (grouped) return p;
  const int nk = K / 64;
  if (M <= 64) {
    p.tile = kSkinny;
    int tiles = (N + TSkin::BN - 1) / TSkin::BN;
    if (epi == E_F32 && tiles >= 512) return p;  // wide output (LM head): no split
    int splits = (512 + tiles - 1) / tiles;
    splits = std::min(splits, std::max(1, nk / 2));
    p.k_splits = std::max(1, splits);
    p.partial_bytes = (size_t)p.k_splits * M * N * sizeof(float);
    return p;
  }
  int big_tiles = ((M + 255) / 256) * ((N + 255) / 256);
  p.tile = big_tiles >= 512 ? kBig : kMid;
  return p;
}

#define GEMM_CASE(TT, TCFG, F16, BM, EP, G)                                          \
  if (plan.tile == TT && f16 == F16 && bmode == BM && epi == EP && grouped == G)        \
    return launch_t<TCFG, F16, BM, EP, G, false>(a, plan.k_splits, s);

hipError_t gemm_run(const Args& a_in, bool f16, int bmode, int epi, bool grouped,
                    const GemmPlan& plan, float* partial, hipStream_t s) {
  Args a = a_in;
  if (plan.tile == kSkinny && !(epi == E_F32 && plan.k_splits == 1)) {
    // split-K: fp32 partial sums, then one reduce + epilogue pass
    if (grouped || partial == nullptr || !f16) return hipErrorInvalidValue;
    a.partial = partial;
    hipError_t e;
    if (bmode == B_QKV)
      e = launch_t<TSkin, true, B_QKV, E_PARTIAL, false, true>(a, plan.k_splits, s);
    else if (bmode == B_SWIGLU)
      e = launch_t<TSkin, true, B_SWIGLU, E_PARTIAL, false, true>(a, plan.k_splits, s);
    else
      e = launch_t<TSkin, true, B_DENSE, E_PARTIAL, false, true>(a, plan.k_splits, s);
    if (e != hipSuccess) return e;
    const int ncols = epi == E_SWIGLU ? a.N / 2 : a.N;
    const int64_t total = (int64_t)a.M * ncols;
    const int blocks = (int)std::min<int64_t>(4096, (total + 255) / 256);
    hipLaunchKernelGGL(splitk_reduce_kernel, dim3(blocks), dim3(256), 0, s, partial,
                       plan.k_splits, a.M, a.N, epi, a.C, a.ldc, a.R, a.ldr, TSkin::BN,
                       TSkin::WN);
    return hipGetLastError();
  }
  // dense layers: fp16 activations x bf16->fp16 weights
  GEMM_CASE(kBig, TBig, true, B_QKV, E_F16, false)
  GEMM_CASE(kBig, TBig, true, B_DENSE, E_RES_F32, false)
  GEMM_CASE(kBig, TBig, true, B_DENSE, E_RESB_F32, false)
  GEMM_CASE(kBig, TBig, true, B_DENSE, E_RESF_B16, false)
  GEMM_CASE(kBig, TBig, true, B_SWIGLU, E_SWIGLU, false)
  GEMM_CASE(kBig, TBig, true, B_DENSE, E_F32, false)
  GEMM_CASE(kMid, TMid, true, B_QKV, E_F16, false)
  GEMM_CASE(kMid, TMid, true, B_DENSE, E_RES_F32, false)
  GEMM_CASE(kMid, TMid, true, B_DENSE, E_RESB_F32, false)
  GEMM_CASE(kMid, TMid, true, B_DENSE, E_RESF_B16, false)
  GEMM_CASE(kMid, TMid, true, B_SWIGLU, E_SWIGLU, false)
  GEMM_CASE(kMid, TMid, true, B_DENSE, E_F32, false)
  GEMM_CASE(kSkinny, TSkin, true, B_DENSE, E_F32, false)
  // routed MoE: router and gate|up read the caller's bf16 tokens; down reads fp16
  GEMM_CASE(kBig, TBig, false, B_DENSE, E_F32, false)
  GEMM_CASE(kMid, TMid, false, B_DENSE, E_F32, false)
  GEMM_CASE(kSkinny, TSkin, false, B_DENSE, E_F32, false)
  GEMM_CASE(kMid, TMid, false, B_SWIGLU, E_SWIGLU, true)
  GEMM_CASE(kMid, TMid, true, B_DENSE, E_F32, true)
  return hipErrorInvalidValue;
}

}  // namespace q3
