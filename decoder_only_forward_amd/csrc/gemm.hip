// GEMM launchers: tile-family choice, split-K reduction, template instantiations.
#include <algorithm>

#include "launch.h"

namespace q3 {
namespace {

using namespace gemm;

using TBig = Tile<256, 256, 2, 4>;   // 8 waves (2 per SIMD), 128x64 per wave, 128 KB LDS
using TMid = Tile<128, 128, 2, 2>;   // 4 waves, 64x64 per wave, 64 KB LDS
using TTall = Tile<256, 128, 4, 2>;  // 8 waves, 64x64 per wave, 96 KB LDS: narrow outputs
using TSkin = Tile<64, 128, 2, 2>;   // 4 waves, 32x64 per wave: decode (M <= 64)

template <class T>
int tiles_m(int M) { return (M + T::BM - 1) / T::BM; }
template <class T>
int tiles_n(int N, int bmode) {
  return (N + T::BN - 1) / T::BN;
}

template <class T, bool F16, int BMODE, int EPI, bool G>
hipError_t launch_t(Args a, hipStream_t s) {
  if (!G) a.m_tiles = tiles_m<T>(a.M);
  a.n_tiles = tiles_n<T>(a.N, BMODE);
  dim3 grid(a.m_tiles * a.n_tiles);
  hipLaunchKernelGGL((gemm_kernel<T, F16, BMODE, EPI, G>), grid, dim3(T::THREADS), 0, s, a);
  return hipGetLastError();
}

// Decode-size products (M <= 256 rows): one block per 16 output columns (SwiGLU: 16 gate
// columns and the matching 16 up columns) and 64 rows (blockIdx.z), the K range split
// across the block's 8 waves.  Each wave streams its slice of the weights straight from memory into
// 16x16x32 fp16 MFMAs (every weight is read once; bf16 -> fp16 is exact in fp16's normal
// range); the activations come through L2.  The waves' partial sums are added in LDS in a
// fixed order and the epilogue applied once: no partial sums in memory, one launch.
// MFMA layouts (lane l, r = l % 16, g = l / 16): A row r, B column r, k = 8 g .. 8 g + 7;
// the accumulator holds column r, rows 4 g .. 4 g + 3.
constexpr int kDecWaves = 8;
constexpr int kDecBatch = 4;  // k-steps of 32 loaded per batch
constexpr int kDecMaxRows = 256;
constexpr int kSplitMaxN = 2048;  // the split-K reduction handles rows of up to 2048

DEV f32x4_t mfma16h(u32x4_t a, u32x4_t b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(as_f16x8(a), as_f16x8(b), c, 0, 0, 0);
}

// With PART the K range is further split over gridDim.y blocks, each writing its fp32
// partial sums to p.partial[blockIdx.y] for a separate reduction (used when N alone gives
// too few blocks).
template <int BMODE, int EPI, bool PART>
__global__ void __launch_bounds__(64 * kDecWaves) decode_gemm_kernel(Args p) {
  constexpr int NT = BMODE == B_SWIGLU ? 2 : 1;
  __shared__ float red[kDecWaves][4][NT][256];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int r16 = lane & 15, grp = lane >> 4;
  const int c0 = blockIdx.x * 16;
  const int ncols = BMODE == B_SWIGLU ? p.N / 2 : p.N;

  const bf16_t* bp[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    const int col = min(c0 + r16, ncols - 1);
    if (BMODE == B_SWIGLU) {
      bp[nt] = (nt == 0 ? p.B0 : p.B1) + (int64_t)col * p.ldb;
    } else if (BMODE == B_QKV) {
      bp[nt] = col < p.seg1 ? p.B0 + (int64_t)col * p.ldb
             : col < p.seg2 ? p.B1 + (int64_t)(col - p.seg1) * p.ldb
                            : p.B2 + (int64_t)(col - p.seg2) * p.ldb;
    } else {
      bp[nt] = p.B0 + (int64_t)col * p.ldb;
    }
  }
  const int row0 = blockIdx.z * 64;
  const uint16_t* ap[4];
#pragma unroll
  for (int mt = 0; mt < 4; ++mt)
    ap[mt] = p.A + (int64_t)min(row0 + mt * 16 + r16, p.M - 1) * p.lda;

  const int nks_all = p.K / 32;
  const int per_split = (nks_all + gridDim.y - 1) / gridDim.y;
  const int kbase = min(nks_all, (int)blockIdx.y * per_split);
  const int nks = min(nks_all, kbase + per_split) - kbase;
  const int per = (nks + kDecWaves - 1) / kDecWaves;
  const int ks0 = kbase + min(nks, wave * per), ks1 = kbase + min(nks, min(nks, wave * per) + per);
  f32x4_t acc[4][NT];
#pragma unroll
  for (int mt = 0; mt < 4; ++mt)
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) acc[mt][nt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  for (int kb = ks0; kb < ks1; kb += kDecBatch) {
    u32x4_t fa[kDecBatch][4], fb[kDecBatch][NT];
#pragma unroll
    for (int u = 0; u < kDecBatch; ++u) {
      if (kb + u < ks1) {
        const int ko = (kb + u) * 32 + grp * 8;
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) fb[u][nt] = ld16(bp[nt] + ko);
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) fa[u][mt] = ld16(ap[mt] + ko);
      }
    }
#pragma unroll
    for (int u = 0; u < kDecBatch; ++u) {
      if (kb + u < ks1) {
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
          const u32x4_t b = bf16x8_to_f16x8(fb[u][nt]);
#pragma unroll
          for (int mt = 0; mt < 4; ++mt) acc[mt][nt] = mfma16h(fa[u][mt], b, acc[mt][nt]);
        }
      }
    }
  }
#pragma unroll
  for (int mt = 0; mt < 4; ++mt)
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
      *(f32x4_t*)&red[wave][mt][nt][lane * 4] = acc[mt][nt];
  __syncthreads();
  for (int o = tid; o < 64 * 16; o += 64 * kDecWaves) {
    const int ml = o >> 4, n = o & 15, m = row0 + ml;
    if (m >= p.M) continue;
    const int col = c0 + n;
    if (col >= ncols) continue;
    const int mt = ml >> 4, rr = ml & 15;
    const int slot = (n + 16 * (rr >> 2)) * 4 + (rr & 3);
    float v[NT];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      float sum = 0.f;
#pragma unroll
      for (int w = 0; w < kDecWaves; ++w) sum += red[w][mt][nt][slot];
      v[nt] = sum;
    }
    if (PART) {
      p.partial[((int64_t)blockIdx.y * p.M + m) * ncols + col] = v[0];
      continue;
    }
    const int64_t ci = (int64_t)m * p.ldc + col, ri = (int64_t)m * p.ldr + col;
    if (EPI == E_SWIGLU) ((f16_t*)p.C)[ci] = f2h(silu(v[0]) * v[NT - 1]);
    else if (EPI == E_F16) ((f16_t*)p.C)[ci] = f2h(v[0]);
    else if (EPI == E_RES_F32) ((float*)p.C)[ci] = ((const float*)p.R)[ri] + v[0];
    else if (EPI == E_RESB_F32) ((float*)p.C)[ci] = bf2f(((const bf16_t*)p.R)[ri]) + v[0];
    else if (EPI == E_RESF_B16) ((bf16_t*)p.C)[ci] = f2bf(((const float*)p.R)[ri] + v[0]);
  }
}

template <int BMODE, int EPI>
hipError_t launch_decode(const Args& a, int splits, hipStream_t s) {
  const int ncols = BMODE == B_SWIGLU ? a.N / 2 : a.N;
  const int chunks = (a.M + 63) / 64;
  if (splits > 1)
    hipLaunchKernelGGL((decode_gemm_kernel<BMODE, EPI, true>),
                       dim3((ncols + 15) / 16, splits, chunks), dim3(64 * kDecWaves), 0, s, a);
  else
    hipLaunchKernelGGL((decode_gemm_kernel<BMODE, EPI, false>), dim3((ncols + 15) / 16, 1, chunks),
                       dim3(64 * kDecWaves), 0, s, a);
  return hipGetLastError();
}

}  // namespace

GemmPlan gemm_plan(int M, int N, int K, int bmode, int epi, bool grouped) {
  GemmPlan p{kMid, 1};
  if (grouped) return p;
  if (M <= 64 || (M <= kDecMaxRows && epi != E_F32)) {
    // fp32 outputs (LM head, router) keep the 64x128 tile (the larger tiles above 64
    // rows): its k order is that of the larger tiles, so last-position logits equal the
    // corresponding rows of a full pass
    p.tile = epi == E_F32 ? kSkinny : kDecode;
    // residual projections with fewer than 256 blocks of 16 columns split K over extra
    // blocks; the caller reduces the partials (fused with the residual add and the
    // following RMSNorm)
    const bool res = epi == E_RES_F32 || epi == E_RESB_F32 || epi == E_RESF_B16;
    const int blocks = (N + 15) / 16 * ((M + 63) / 64);
    if (p.tile == kDecode && res && blocks < 256 && N <= kSplitMaxN) {
      const int want = (256 + blocks - 1) / blocks;
      p.k_splits = std::max(1, std::min(want, K / (32 * kDecWaves)));
    }
    return p;
  }
  // the largest tile that still gives every CU a block: 256x256 moves the fewest bytes per
  // flop through the copy path, 256x128 a third more, 128x128 twice as many
  const int big_tiles = ((M + 255) / 256) * ((N + 255) / 256);
  const int tall_tiles = ((M + 255) / 256) * ((N + 127) / 128);
  p.tile = big_tiles >= 512 ? kBig : tall_tiles >= 256 ? kTall : kMid;
  return p;
}

#define GEMM_CASE(TT, TCFG, F16, BM, EP, G)                                          \
  if (pl.tile == TT && f16 == F16 && bmode == BM && epi == EP && grouped == G)          \
    return launch_t<TCFG, F16, BM, EP, G>(a, s);

hipError_t gemm_run(const Args& a_in, bool f16, int bmode, int epi, bool grouped,
                    const GemmPlan& plan, hipStream_t s) {
  Args a = a_in;
  const GemmPlan& pl = plan;
  if (pl.tile == kDecode) {
    if (grouped || !f16 || a.M > kDecMaxRows) return hipErrorInvalidValue;
    if (pl.k_splits > 1) {  // partial sums only (bmode dense, any residual epilogue)
      if (bmode != B_DENSE || a.partial == nullptr) return hipErrorInvalidValue;
      return launch_decode<B_DENSE, E_RES_F32>(a, pl.k_splits, s);
    }
    if (bmode == B_QKV && epi == E_F16) return launch_decode<B_QKV, E_F16>(a, 1, s);
    if (bmode == B_SWIGLU && epi == E_SWIGLU) return launch_decode<B_SWIGLU, E_SWIGLU>(a, 1, s);
    if (bmode == B_DENSE && epi == E_RES_F32) return launch_decode<B_DENSE, E_RES_F32>(a, 1, s);
    if (bmode == B_DENSE && epi == E_RESB_F32) return launch_decode<B_DENSE, E_RESB_F32>(a, 1, s);
    if (bmode == B_DENSE && epi == E_RESF_B16) return launch_decode<B_DENSE, E_RESF_B16>(a, 1, s);
    return hipErrorInvalidValue;
  }
  // dense layers: fp16 activations x bf16->fp16 weights
  GEMM_CASE(kBig, TBig, true, B_QKV, E_F16, false)
  GEMM_CASE(kBig, TBig, true, B_QKV, E_QKROPE, false)
  GEMM_CASE(kMid, TMid, true, B_QKV, E_QKROPE, false)
  GEMM_CASE(kBig, TBig, true, B_DENSE, E_RES_F32, false)
  GEMM_CASE(kBig, TBig, true, B_DENSE, E_RESB_F32, false)
  GEMM_CASE(kBig, TBig, true, B_DENSE, E_RESF_B16, false)
  GEMM_CASE(kBig, TBig, true, B_SWIGLU, E_SWIGLU, false)
  GEMM_CASE(kBig, TBig, true, B_DENSE, E_F32, false)
  GEMM_CASE(kTall, TTall, true, B_QKV, E_F16, false)
  GEMM_CASE(kTall, TTall, true, B_QKV, E_QKROPE, false)
  GEMM_CASE(kTall, TTall, true, B_DENSE, E_RES_F32, false)
  GEMM_CASE(kTall, TTall, true, B_DENSE, E_RESB_F32, false)
  GEMM_CASE(kTall, TTall, true, B_DENSE, E_RESF_B16, false)
  GEMM_CASE(kTall, TTall, true, B_SWIGLU, E_SWIGLU, false)
  GEMM_CASE(kTall, TTall, true, B_DENSE, E_F32, false)
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
  GEMM_CASE(kBig, TBig, false, B_SWIGLU, E_SWIGLU, true)
  // routed layers inside the stack read fp16 normalised rows
  GEMM_CASE(kBig, TBig, true, B_SWIGLU, E_SWIGLU, true)
  GEMM_CASE(kBig, TBig, true, B_DENSE, E_F32, true)
  return hipErrorInvalidValue;
}

}  // namespace q3
