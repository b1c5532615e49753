// GEMM on the gfx950 matrix cores: C[M, N] = A[M, K] . B[N, K]^T, fp32 accumulate.
//
// Both operands are K-contiguous (activations [tokens, in], weights in the HF
// [out, in] layout), which is the operand order of v_mfma_f32_32x32x16_{bf16,f16}.
// Operand precision: weights are always bf16 in memory.  When the activations are
// bf16 exactly (a caller's bf16 input) the bf16 MFMA is used; when they are computed
// activations they are kept in fp16 (8x finer rounding than bf16) and the weight tile
// is converted bf16 -> fp16 on its way into LDS (exact in fp16's normal range), so the
// fp16 MFMA runs at the same rate.
// Block tile BM x BN x BK staged through a ring of STAGES LDS slots filled by direct
// global -> LDS copies issued STAGES - 1 k-steps ahead (one barrier per k-step).  Tile
// rows are stored with their 16-byte chunks XOR-swizzled (lds_off), so the 16-byte
// fragment reads of consecutive lanes (consecutive rows, same chunk) hit distinct banks,
// and each copy instruction still fills 1 KB of contiguous LDS.
// Every wave owns a WM x WN sub-tile made of 32x32 MFMA tiles.
//
// Fused epilogues (one per projection of the decoder block):
//   E_F32       fp32 streaming store                     (LM head, router, MoE down)
//   E_F16       fp16 store                               (QKV projections)
//   E_RES_F32   out_f32 = res_f32 + acc (in place ok)    (o_proj / down in the stack)
//   E_RESB_F32  out_f32 = float(res_bf16) + acc          (o_proj in the block API)
//   E_RESF_B16  out_bf16 = bf16(res_f32 + acc)           (down in the block API)
//   E_SWIGLU    out_f16[:, c] = f16(silu(g) * u)         (gate|up with SwiGLU)
//   E_QKROPE    QKV projections of a prefill: the tile is rounded to fp16 and staged in
//               LDS, then per (token, head): q/k RMSNorm, RoPE, q to q_out (pre-scaled
//               fp16), k to the bf16 cache and its fp16 copy, v transposed to the V^T
//               cache and its fp16 copy; the copies' tails past the last position are
//               zeroed (see RopeEpi)
// B row sources:
//   B_DENSE   one matrix;  B_QKV  q/k/v weights stacked along N without a copy;
//   B_SWIGLU  gate and up rows interleaved per wave so that a lane holds the gate and
//             up accumulators of the same output element.
// Grouped mode (routed MoE): the m-tile index selects (expert, first row) from a
// device tile table; A rows may be gathered through a row-index list.
#pragma once

#include <type_traits>

#include "common.h"

namespace gemm {

enum BMode { B_DENSE = 0, B_QKV = 1, B_SWIGLU = 2 };
enum EpiMode { E_F32 = 1, E_RES_F32, E_RESB_F32, E_RESF_B16, E_SWIGLU, E_F16, E_QKROPE };

// Destination of the E_QKROPE epilogue (a prefill of B sequences of S tokens from pos0;
// output row t is token t % S of sequence t / S at position pos0 + t % S).
struct RopeEpi {
  const float* table;  // [2][max_pos][hd/2]: cos, then sin
  const bf16_t* q_norm;
  const bf16_t* k_norm;
  f16_t* q_out;      // [T][nq][hd], pre-scaled by log2(e) / sqrt(hd)
  bf16_t* k_cache;   // [B][nkv] regions, 32-position tiles (kcache_idx)
  bf16_t* vt_cache;  // [B][nkv] regions, 32-position tiles (vcache_idx)
  f16_t* k_fresh;    // [B][nkv][fresh_w][hd], position - fresh_base
  f16_t* vt_fresh;   // [B][nkv][hd][fresh_w]
  int fresh_base, fresh_w, pos0, S, nq, nkv, cap, max_pos, qk_norm, interleaved;
  float eps;
};

struct Args {
  int M, N, K;  // N counts virtual columns (gate|up: 2 * I)
  const uint16_t* A;  // bf16 or fp16 bits (see F16)
  int64_t lda;
  const int32_t* a_rows;  // optional: A row of output row r is a_rows[r]
  const bf16_t* B0;
  const bf16_t* B1;
  const bf16_t* B2;
  int64_t ldb;
  int seg1, seg2;  // B_QKV: virtual columns [0,seg1) from B0, [seg1,seg2) B1, rest B2
  void* C;
  int64_t ldc;
  const void* R;  // residual input
  int64_t ldr;
  float* partial;  // decode K-split: fp32 partial sums [splits][M][N] (no epilogue)
  int m_tiles, n_tiles;
  // grouped mode
  const int32_t* g_offsets;      // [E + 1] first output row of each expert
  const int32_t* g_tile_expert;  // [m_tiles] expert of each m tile (-1: idle)
  const int32_t* g_tile_row0;    // [m_tiles] first row within the expert
  const int32_t* g_tile_count;   // [1] m tiles in use (nullptr: all m_tiles)
  int64_t g_b_stride;            // elements between experts' B matrices
  RopeEpi re;                    // E_QKROPE only
};

template <int BM_, int BN_, int WAVES_M_, int WAVES_N_, int BK_ = 64, int STAGES_ = 2>
struct Tile {
  static constexpr int BM = BM_, BN = BN_, BK = BK_, STAGES = STAGES_;
  static constexpr int ROWS_PER_COPY = 1024 / (2 * BK);  // tile rows per 1 KB copy
  static constexpr int WAVES_M = WAVES_M_, WAVES_N = WAVES_N_;
  static constexpr int WM = BM / WAVES_M, WN = BN / WAVES_N;
  static constexpr int TM = WM / 32, TN = WN / 32;
  static constexpr int NWAVES = WAVES_M * WAVES_N;
  static constexpr int THREADS = NWAVES * 64;
  static_assert(WM % 32 == 0 && WN % 32 == 0, "wave tile must be a multiple of 32");
  static_assert(BK == 32 || BK == 64, "k-step");
  static_assert(BM % (ROWS_PER_COPY * NWAVES) == 0 && BN % (ROWS_PER_COPY * NWAVES) == 0,
                "whole copies per wave");
};

// Blocks are dispatched round-robin over the 8 XCDs; give each XCD a contiguous run of
// tile ids so neighbouring tiles (which share A row panels / B column panels) share an
// L2.  Then order tiles in groups of 8 m-tiles for panel reuse.
DEV int xcd_remap(int b, int nblocks) {
  int q = nblocks >> 3, r = nblocks & 7;
  int xcd = b & 7, idx = b >> 3;
  int base = xcd < r ? xcd * (q + 1) : r * (q + 1) + (xcd - r) * q;
  return base + idx;
}

DEV void tile_coords(int t, int m_tiles, int n_tiles, int& tm, int& tn) {
  const int G = 8;
  int group = t / (G * n_tiles);
  int first_m = group * G;
  int gm = min(G, m_tiles - first_m);
  int rem = t - group * G * n_tiles;
  tm = first_m + rem % gm;
  tn = rem / gm;
}

// 16-byte chunk c of tile row `row`.
// 128-byte rows (BK = 64): the XOR spreads any 16 consecutive rows' fragment reads (same
// logical chunk) over distinct banks whether the LDS serves 8 lanes (128 B) or 16 lanes
// (256 B) of a 16-byte read per cycle: rows r and r+8 differ in bit 0 of the swizzle and
// rows of opposite parity sit in opposite 128-byte halves.
// 64-byte rows (BK = 32, four rows per 256-byte bank line): rows r, r+4, r+8, r+12 share
// bank positions; XOR-ing the chunk with (r / 4) % 4 gives them distinct chunks.
template <int BK>
DEV int lds_swz(int row) {
  return BK == 64 ? ((row & 7) ^ ((row >> 3) & 1)) : ((row >> 2) & 3);
}
template <int BK>
DEV int lds_off(int row, int chunk) { return row * BK + ((chunk ^ lds_swz<BK>(row)) << 3); }

// s_waitcnt vmcnt(N) through the builtin (expcnt and lgkmcnt at their maxima).
template <int N>
DEV void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | (((N >> 4) & 3) << 14) | 0x0F70);
}

// E_QKROPE epilogue.  Columns n0 .. n0 + BN of the B_QKV product lie in one segment (q, k or
// v heads: BN divides the segment boundaries), each 128 columns one head.  The block's fp16
// tile is staged in LDS ([BM][BN + 8], rows padded by 16 bytes), then
//   q / k heads: 16 lanes per (token, head), 8 dims each: RMSNorm over the head (sum of
//     squares by row-local DPP rotations), RoPE (rotate-half: dim d pairs with d ^ 64, held
//     by lane j ^ 8; interleaved: planes (2i, 2i + 1) inside a lane), 16-byte stores;
//   v heads: one lane per (dim, 8 consecutive tokens), transposed 16-byte stores where the
//     8 tokens are one sequence's aligned positions, element stores otherwise.
// The attention reads the fp16 copies in whole 64-position tiles: zero each sequence's
// tail, from its last new position to the padded width, for the tile whose rows hold the
// sequence's last token (k heads: rows of k_fresh; v heads: columns of vt_fresh).
template <int THREADS>
DEV void zero_fresh_tail(const RopeEpi& e, int out_row0, int rows_valid, int head0, int heads,
                         bool is_k) {
  const int HD = 128;
  const int t0 = e.pos0 + e.S - e.fresh_base, nt = e.fresh_w - t0;
  if (!e.k_fresh || nt <= 0) return;
  const int b_lo = out_row0 / e.S, b_hi = (out_row0 + rows_valid) / e.S - 1;
  const int nh = min(heads, e.nkv - head0);
  if (b_hi < b_lo || nh <= 0) return;
  const int per_seq = nh * nt * HD;
  for (int i = threadIdx.x; i < (b_hi - b_lo + 1) * per_seq; i += THREADS) {
    const int b = b_lo + i / per_seq, j = i % per_seq;
    const int h = head0 + j / (nt * HD), r = t0 + (j / HD) % nt, d = j % HD;
    if (is_k)
      e.k_fresh[(((int64_t)b * e.nkv + h) * e.fresh_w + r) * HD + d] = 0;
    else
      e.vt_fresh[(((int64_t)b * e.nkv + h) * HD + d) * e.fresh_w + r] = 0;
  }
}

template <class T>
DEV void qkrope_epilogue(const Args& p, const f32x16_t (&acc)[T::TM][T::TN], f16_t* st,
                         int out_row0, int rows_valid, int n0, int wm, int wn, int lane,
                         int wave) {
  constexpr int HD = 128, LDT = T::BN + 8, HEADS = T::BN / HD;
  const RopeEpi& e = p.re;
  const int ccol = lane & 31, rsub = (lane >> 5) * 4;
  __syncthreads();  // every wave is done with the operand ring
#pragma unroll
  for (int i = 0; i < T::TM; ++i)
#pragma unroll
    for (int j = 0; j < T::TN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int lr = wm * T::WM + i * 32 + (r >> 2) * 8 + rsub + (r & 3);
        st[lr * LDT + wn * T::WN + j * 32 + ccol] = f2h(acc[i][j][r]);
      }
  __syncthreads();
  const int tid = threadIdx.x;
  // Output row out_row0 + lr is token (s_first + lr) % S of sequence b_first +
  // (s_first + lr) / S: one division per tile, then a 32-bit one per row (rows < 2^30)
  const unsigned S_u = (unsigned)e.S;
  const int b_first = out_row0 / e.S, s_first = out_row0 % e.S;
  auto seq_of = [&](int lr, int& b, int& s) {
    const unsigned a = (unsigned)(s_first + lr), q = a / S_u;
    b = b_first + (int)q;
    s = (int)(a - q * S_u);
  };
  if (n0 < p.seg2) {
    const bool is_q = n0 < p.seg1;
    const int head0 = is_q ? n0 / HD : (n0 - p.seg1) / HD;
    const int nh = is_q ? e.nq : e.nkv;
    const int j16 = lane & 15, sub = lane >> 4, d0 = 8 * j16;
    const int half = HD / 2;
    const int i0 = e.interleaved ? d0 / 2 : d0 & (half - 1);
    const float sgn = d0 < half ? -1.f : 1.f;
    const float qs = 0.08838834764831845f * kLog2e;
    float w[8];
    if (e.qk_norm) {
      unpack8(ld16((is_q ? e.q_norm : e.k_norm) + d0), w);
    } else {
#pragma unroll
      for (int k = 0; k < 8; ++k) w[k] = 1.f;
    }
    // 16 lanes per token row handle all HEADS heads of the row with one RoPE-table load; NB
    // rows per lane at a time, all their LDS reads and table loads issued before any is used
    constexpr int NB = 4, STEP = T::NWAVES * 4;
    for (int base = wave * 4 + sub; base < rows_valid; base += NB * STEP) {
      u32x4_t raw[NB][HEADS];
      f32x4_t tc[NB][2], ts[NB][2];
      int pos_k[NB], b_k[NB];
      bool ok_k[NB];
#pragma unroll
      for (int u = 0; u < NB; ++u) {
        const int lr = min(base + u * STEP, rows_valid - 1);
        int sq;
        seq_of(lr, b_k[u], sq);
        const int pos = e.pos0 + sq;
        pos_k[u] = pos;
        ok_k[u] = pos >= 0 && pos < e.cap && pos < e.max_pos;
#pragma unroll
        for (int hl = 0; hl < HEADS; ++hl) raw[u][hl] = ld16(st + lr * LDT + hl * HD + d0);
        const int pc = ok_k[u] ? pos : 0;
        const float* cp = e.table + (int64_t)pc * half + i0;
        const float* sp = e.table + ((int64_t)e.max_pos + pc) * half + i0;
        tc[u][0] = *(const f32x4_t*)cp;
        ts[u][0] = *(const f32x4_t*)sp;
        if (!e.interleaved) {
          tc[u][1] = *(const f32x4_t*)(cp + 4);
          ts[u][1] = *(const f32x4_t*)(sp + 4);
        }
      }
#pragma unroll
      for (int u = 0; u < NB; ++u) {
        const int lr = base + u * STEP;
        if (lr >= rows_valid) break;
        const int64_t t = out_row0 + lr;
        const int b = b_k[u];
        const int pos = pos_k[u];
        const bool ok = ok_k[u];
        float c[8], sn[8];
        if (e.interleaved) {
#pragma unroll
          for (int k = 0; k < 4; ++k) {
            c[k] = ok ? tc[u][0][k] : 0.f;
            sn[k] = ok ? ts[u][0][k] : 0.f;
          }
        } else {
#pragma unroll
          for (int k = 0; k < 4; ++k) {
            c[k] = ok ? tc[u][0][k] : 0.f;
            c[k + 4] = ok ? tc[u][1][k] : 0.f;
            sn[k] = ok ? ts[u][0][k] : 0.f;
            sn[k + 4] = ok ? ts[u][1][k] : 0.f;
          }
        }
#pragma unroll
        for (int hl = 0; hl < HEADS; ++hl) {
          const int h = head0 + hl;
          float x[8];
          unpack8_f16(raw[u][hl], x);
          if (e.qk_norm) {
            float ss = 0.f;
#pragma unroll
            for (int k = 0; k < 8; ++k) ss += x[k] * x[k];
            ss += ror16<8>(ss);
            ss += ror16<4>(ss);
            ss += ror16<2>(ss);
            ss += ror16<1>(ss);
            const float inv = rsqrtf(ss / (float)HD + e.eps);
#pragma unroll
            for (int k = 0; k < 8; ++k) x[k] = x[k] * inv * w[k];
          }
          float y[8];
          if (e.interleaved) {
#pragma unroll
            for (int k = 0; k < 4; ++k) {
              y[2 * k] = x[2 * k] * c[k] - x[2 * k + 1] * sn[k];
              y[2 * k + 1] = x[2 * k] * sn[k] + x[2 * k + 1] * c[k];
            }
          } else {
#pragma unroll
            for (int k = 0; k < 8; ++k) y[k] = x[k] * c[k] + sgn * ror16<8>(x[k]) * sn[k];
          }
          if (h >= nh) continue;
          if (is_q) {
            u32x4_t o;
#pragma unroll
            for (int k = 0; k < 4; ++k)
              o[k] = ok ? pack_f16x2(y[2 * k] * qs, y[2 * k + 1] * qs) : 0x7E007E00u;
            st16(e.q_out + (t * e.nq + h) * HD + d0, o);
          } else if (ok) {
            u32x4_t kb, kh;
#pragma unroll
            for (int k = 0; k < 4; ++k) {
              kb[k] = pack_bf16x2(y[2 * k], y[2 * k + 1]);
              kh[k] = pack_f16x2(y[2 * k], y[2 * k + 1]);
            }
            st16(e.k_cache + ((int64_t)b * e.nkv + h) * e.cap * HD + kcache_idx(pos, d0), kb);
            if (e.k_fresh)
              st16(e.k_fresh + (((int64_t)b * e.nkv + h) * e.fresh_w + (pos - e.fresh_base)) *
                                   HD + d0, kh);
          }
        }
      }
    }
    if (!is_q) zero_fresh_tail<T::THREADS>(e, out_row0, rows_valid, head0, HEADS, true);
    return;
  }
  // v heads: item = (32-row group, column c, group of 8 rows); four consecutive lanes take
  // the four 8-row groups of one column, the next lanes the next columns, so that with
  // tile-aligned positions a wave's 16-byte stores cover 16 whole dims of a cache tile
  const int head0 = (n0 - p.seg2) / HD;
  for (int item = tid; item < T::BN * (T::BM / 8); item += T::THREADS) {
    const int c = (item >> 2) % T::BN, r0 = ((item >> 2) / T::BN) * 32 + (item & 3) * 8;
    const int h = head0 + c / HD, d = c % HD;
    if (h >= e.nkv || r0 >= rows_valid) continue;
    int b, s0;
    seq_of(r0, b, s0);
    const int pos = e.pos0 + s0;
    const int n = min(8, rows_valid - r0);
    float v[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) v[k] = h2f(st[(r0 + (k < n ? k : 0)) * LDT + c]);
    bf16_t* const vreg = e.vt_cache + ((int64_t)b * e.nkv + h) * e.cap * HD;
    f16_t* vf = e.vt_fresh ? e.vt_fresh + (((int64_t)b * e.nkv + h) * HD + d) * e.fresh_w +
                                 (pos - e.fresh_base)
                           : nullptr;
    if (n == 8 && s0 + 8 <= e.S && (pos & 7) == 0 && pos + 8 <= e.cap &&
        (!vf || ((pos - e.fresh_base) & 7) == 0)) {
      u32x4_t ob, oh;
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        ob[k] = pack_bf16x2(v[2 * k], v[2 * k + 1]);
        oh[k] = pack_f16x2(v[2 * k], v[2 * k + 1]);
      }
      st16(vreg + vcache_idx(pos, d), ob);
      if (vf) st16(vf, oh);
    } else {
      // rows may cross into the next sequence: place each token by its own (b, s)
      for (int k = 0; k < n; ++k) {
        int bk, sk;
        seq_of(r0 + k, bk, sk);
        const int pk = e.pos0 + sk;
        if (pk < 0 || pk >= e.cap || pk >= e.max_pos) continue;
        const int64_t bh = (int64_t)bk * e.nkv + h;
        e.vt_cache[bh * e.cap * HD + vcache_idx(pk, d)] = f2bf(v[k]);
        if (e.vt_fresh) e.vt_fresh[(bh * HD + d) * e.fresh_w + (pk - e.fresh_base)] = f2h(v[k]);
      }
    }
  }
  zero_fresh_tail<T::THREADS>(e, out_row0, rows_valid, head0, T::BN / HD, false);
}

template <class T, bool F16, int BMODE, int EPI, bool GROUPED>
__global__ void __launch_bounds__(T::THREADS) gemm_kernel(Args p) {
  // operand ring; the E_QKROPE epilogue reuses it (and more) for the fp16 output tile
  constexpr int kRing = T::STAGES * (T::BM + T::BN) * T::BK * 2;
  constexpr int kEpiLds = EPI == E_QKROPE ? T::BM * (T::BN + 8) * 2 : 0;
  __shared__ __attribute__((aligned(16))) char smem[kRing > kEpiLds ? kRing : kEpiLds];
  bf16_t* const sA = (bf16_t*)smem;                            // [STAGES][BM * BK]
  bf16_t* const sB = sA + T::STAGES * T::BM * T::BK;           // [STAGES][BN * BK]

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int wm = wave / T::WAVES_N, wn = wave % T::WAVES_N;

  // Grouped mode: the grid covers every possible m tile, but only the first tile_count
  // are in use; the used tiles are spread over the XCDs and surplus blocks leave at once.
  const int m_tiles = GROUPED && p.g_tile_count ? min(p.m_tiles, *p.g_tile_count) : p.m_tiles;
  const int nblocks_mn = m_tiles * p.n_tiles;
  if ((int)blockIdx.x >= nblocks_mn) return;
  const int t = xcd_remap(blockIdx.x, nblocks_mn);
  int tm, tn;
  tile_coords(t, m_tiles, p.n_tiles, tm, tn);

  // rows handled by this block
  int out_row0, rows_valid;
  const bf16_t* B0 = p.B0;
  const bf16_t* B1 = p.B1;
  if (GROUPED) {
    int e = p.g_tile_expert[tm];
    if (e < 0) return;
    int r0 = p.g_tile_row0[tm];
    int ne = p.g_offsets[e + 1] - p.g_offsets[e];
    out_row0 = p.g_offsets[e] + r0;
    rows_valid = min(T::BM, ne - r0);
    B0 += (int64_t)e * p.g_b_stride;
    B1 += (int64_t)e * p.g_b_stride;
  } else {
    out_row0 = tm * T::BM;
    rows_valid = min(T::BM, p.M - out_row0);
  }
  const int n0 = tn * T::BN;

  const int kt0 = 0, nk = p.K / T::BK;

  // ---- operand tiles go global -> LDS directly (lds_dma16): lane L of a
  // wave instruction lands at 16 L bytes past that instruction's 1 KB LDS slot, i.e. at
  // row R q + L / C, physical chunk L % C of the tile (R rows of C chunks per copy), so
  // each lane fetches the logical chunk the swizzle stores there.  Rows past the valid
  // range are clamped to the last valid row: they only feed accumulator rows / columns
  // the epilogue never stores.
  constexpr int RPC = T::ROWS_PER_COPY, CPR = T::BK / 8;
  constexpr int A_INSTS = T::BM / (RPC * T::NWAVES), B_INSTS = T::BN / (RPC * T::NWAVES);
  constexpr int STAGE_INSTS = A_INSTS + B_INSTS;  // copies per wave per stage
  const int lrow = lane / CPR, pchunk = lane % CPR;
  const uint16_t* aptr[A_INSTS];
  const bf16_t* bptr[B_INSTS];
#pragma unroll
  for (int i = 0; i < A_INSTS; ++i) {
    int r = RPC * (wave * A_INSTS + i) + lrow;
    int rc = min(r, rows_valid - 1);
    int orow = out_row0 + rc;
    int64_t arow = p.a_rows ? (int64_t)p.a_rows[orow] : (int64_t)orow;
    int c = pchunk ^ lds_swz<T::BK>(r);
    aptr[i] = p.A + arow * p.lda + c * 8;
  }
#pragma unroll
  for (int i = 0; i < B_INSTS; ++i) {
    int r = RPC * (wave * B_INSTS + i) + lrow;
    int c = pchunk ^ lds_swz<T::BK>(r);
    const bf16_t* ptr;
    if (BMODE == B_SWIGLU) {
      const int half = T::WN / 2;
      int w = r / T::WN, j = r % T::WN;
      int col = min(tn * (T::BN / 2) + w * half + (j % half), p.N / 2 - 1);
      ptr = (j < half ? B0 : B1) + (int64_t)col * p.ldb;
    } else {
      int n = min(n0 + r, p.N - 1);
      if (BMODE == B_QKV) {
        if (n < p.seg1) ptr = B0 + (int64_t)n * p.ldb;
        else if (n < p.seg2) ptr = B1 + (int64_t)(n - p.seg1) * p.ldb;
        else ptr = p.B2 + (int64_t)(n - p.seg2) * p.ldb;
      } else {
        ptr = B0 + (int64_t)n * p.ldb;
      }
    }
    bptr[i] = ptr + c * 8;
  }

  f32x16_t acc[T::TM][T::TN];
#pragma unroll
  for (int i = 0; i < T::TM; ++i)
#pragma unroll
    for (int j = 0; j < T::TN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

  // Grouped tiles are often partly filled (an expert's last rows): copies of A rows wholly
  // past rows_valid and the MFMAs of 32-row groups wholly past it are skipped (those LDS rows
  // then hold stale data, which only reaches accumulator rows the epilogue never stores).
  // The waits below count copies per stage, which skipped copies would throw off unless
  // every wait is for all copies (two stages).
  static_assert(!GROUPED || T::STAGES == 2, "grouped tiles skip copies: two stages only");
  auto a_live = [&](int i) { return !GROUPED || RPC * (wave * A_INSTS + i) < rows_valid; };
  const int tm_live =
      GROUPED ? max(0, min(T::TM, (rows_valid - wm * T::WM + 31) / 32)) : T::TM;
  auto load_stage = [&](int kt, int st) {
    const int koff = kt * T::BK;
#pragma unroll
    for (int i = 0; i < A_INSTS; ++i)
      if (a_live(i))
        lds_dma16(aptr[i] + koff, sA + st * (T::BM * T::BK) + (wave * A_INSTS + i) * 512);
#pragma unroll
    for (int i = 0; i < B_INSTS; ++i)
      lds_dma16(bptr[i] + koff, sB + st * (T::BN * T::BK) + (wave * B_INSTS + i) * 512);
  };

  // prologue: the first STAGES - 1 k-steps in flight, then wait for the first one
#pragma unroll
  for (int j = 0; j < T::STAGES - 1; ++j)
    if (j < nk) load_stage(kt0 + j, j);
  if (nk >= T::STAGES - 1) wait_vm<(T::STAGES - 2) * STAGE_INSTS>();
  else wait_vm<0>();
  __syncthreads();

  const int frow = lane & 31, fhalf = lane >> 5;
  // Inside a stage the fragments of k-slice kk+1 are read from LDS while the MFMAs of
  // k-slice kk run; later stages stream into the other ring slots meanwhile.  bf16 weight
  // fragments are converted to fp16 after the LDS read when the activations are fp16.
  u32x4_t fa[2][T::TM], fb[2][T::TN];
  auto read = [&](int s, int kk, int slot) {
    const int c = 2 * kk + fhalf;
#pragma unroll
    for (int i = 0; i < T::TM; ++i)
      fa[slot][i] = ld16(sA + s * (T::BM * T::BK) + lds_off<T::BK>(wm * T::WM + i * 32 + frow, c));
#pragma unroll
    for (int j = 0; j < T::TN; ++j) {
      u32x4_t v = ld16(sB + s * (T::BN * T::BK) + lds_off<T::BK>(wn * T::WN + j * 32 + frow, c));
      fb[slot][j] = F16 ? bf16x8_to_f16x8(v) : v;
    }
  };
  auto mma = [&](int slot) {
#pragma unroll
    for (int i = 0; i < T::TM; ++i)
#pragma unroll
      for (int j = 0; j < T::TN; ++j) {
        if (GROUPED && i >= tm_live) continue;
        if (F16)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(as_f16x8(fa[slot][i]),
                                                             as_f16x8(fb[slot][j]), acc[i][j],
                                                             0, 0, 0);
        else
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(fa[slot][i]),
                                                              as_bf16x8(fb[slot][j]), acc[i][j],
                                                              0, 0, 0);
      }
  };
  constexpr int KK = T::BK / 16;  // MFMA k-slices per stage
  for (int it = 0; it < nk; ++it) {
    const int s = it % T::STAGES;
    // ring slot (it - 1) % STAGES was last read before the previous barrier
    const bool issue = it + T::STAGES - 1 < nk;
    if (issue) load_stage(kt0 + it + T::STAGES - 1, (it + T::STAGES - 1) % T::STAGES);
    read(s, 0, 0);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
      if (kk + 1 < KK) read(s, kk + 1, (kk + 1) & 1);
      mma(kk & 1);
      __builtin_amdgcn_sched_barrier(0);
    }
    // k-step it + 1 must have landed: at most the copies issued after it may be pending
    if (issue) wait_vm<(T::STAGES - 2) * STAGE_INSTS>();
    else wait_vm<0>();
    __syncthreads();
  }

  // ---------------- epilogue
  // 32x32 accumulator layout: lane l, register r -> row 8*(r/4) + 4*(l/32) + r%4,
  // column l%32 of the MFMA tile.
  const int ccol = lane & 31;
  const int rsub = (lane >> 5) * 4;
  if constexpr (EPI == E_QKROPE) {
    qkrope_epilogue<T>(p, acc, (f16_t*)smem, out_row0, rows_valid, n0, wm, wn, lane, wave);
    return;
  }
  if constexpr (EPI == E_SWIGLU) {
    // silu(gate) * up rounded to fp16, staged in LDS ([BM][BN / 2 + 8]) so that the global
    // stores go out as 16-byte chunks of whole rows instead of 2-byte scatters
    constexpr int HALF_TN = T::TN / 2, OBN = T::BN / 2, LDO = OBN + 8, CPR = OBN / 8;
    static_assert(T::BM * LDO * 2 <= (int)sizeof(smem), "SwiGLU staging exceeds the ring");
    f16_t* const so = (f16_t*)smem;
    __syncthreads();  // every wave is done with the operand ring
#pragma unroll
    for (int i = 0; i < T::TM; ++i)
#pragma unroll
      for (int j = 0; j < HALF_TN; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int lr = wm * T::WM + i * 32 + (r >> 2) * 8 + rsub + (r & 3);
          const float g = acc[i][j][r], u = acc[i][j + HALF_TN][r];
          so[lr * LDO + wn * (T::WN / 2) + j * 32 + ccol] = f2h(silu(g) * u);
        }
    __syncthreads();
    for (int c = threadIdx.x; c < T::BM * CPR; c += T::THREADS) {
      const int lr = c / CPR, col = tn * OBN + (c % CPR) * 8;
      if (lr >= rows_valid || col >= p.N / 2) continue;
      st16((f16_t*)p.C + (int64_t)(out_row0 + lr) * p.ldc + col,
           ld16(so + lr * LDO + (c % CPR) * 8));
    }
    return;
  }
  // Residual modes walk the accumulator groups (i, j) as a pipeline: the residual values
  // of group g + 1 are loaded before group g is stored, so only the first load latency is
  // exposed.  The output may be the residual buffer itself: each element is read before it
  // is written and distinct elements never overlap.
  // A lane's 16 elements of a group lie in rows row0 + roff(r) of one column, roff(r) =
  // 8 (r / 4) + r % 4: in a full tile (every row and column valid, all tiles but the last
  // row / column of a product) each element is the group's base address plus a row offset
  // that is the same for every lane, with no bounds logic.  Otherwise rows / columns past
  // the valid range are clamped to the last valid one for the residual loads (every load in
  // bounds and unconditional, so they issue back to back) and those elements are not stored.
  constexpr bool RES = EPI == E_RES_F32 || EPI == E_RESB_F32 || EPI == E_RESF_B16;
  constexpr int NG = T::TM * T::TN;
  auto walk = [&](auto full_c) {
    constexpr bool FULL = decltype(full_c)::value;
    auto load_res = [&](int gi, float* res) {
      const int i = gi / T::TN, j = gi % T::TN;
      const int col = FULL ? n0 + wn * T::WN + j * 32 + ccol
                           : min(n0 + wn * T::WN + j * 32 + ccol, p.N - 1);
      const int64_t row0 = out_row0 + wm * T::WM + i * 32 + rsub;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int roff = (r >> 2) * 8 + (r & 3);
        const int64_t row =
            FULL ? row0 + roff : out_row0 + min((int)(row0 - out_row0) + roff, rows_valid - 1);
        if (EPI == E_RESB_F32) {
          // the aligned 32-bit word holding this bf16 and its neighbour's
          const uint32_t w = *(const uint32_t*)((const bf16_t*)p.R + row * p.ldr + (col & ~1));
          res[r] = __uint_as_float((col & 1) ? (w & 0xffff0000u) : (w << 16));
        } else {
          res[r] = ((const float*)p.R)[row * p.ldr + col];
        }
      }
    };
    float res_cur[16], res_next[16];
    if (RES) load_res(0, res_next);
#pragma unroll
    for (int gi = 0; gi < NG; ++gi) {
      const int i = gi / T::TN, j = gi % T::TN;
      if (RES) {
#pragma unroll
        for (int r = 0; r < 16; ++r) res_cur[r] = res_next[r];
        if (gi + 1 < NG) load_res(gi + 1, res_next);
      }
      const int col = n0 + wn * T::WN + j * 32 + ccol;
      if (!FULL && col >= p.N) continue;
      const int lr0 = wm * T::WM + i * 32 + rsub;
      const int64_t row0 = out_row0 + lr0;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int roff = (r >> 2) * 8 + (r & 3);
        if (!FULL && lr0 + roff >= rows_valid) continue;
        const int64_t row = row0 + roff;
        const float v = acc[i][j][r];
        if (EPI == E_F32) {
          // fp32 outputs (logits, MoE slot rows) are far larger than the caches and read
          // once by a later pass: streaming stores (measured: LM head -1%, MoE down -5%,
          // and the combine that reads the slot rows -17%)
          __builtin_nontemporal_store(v, (float*)p.C + row * p.ldc + col);
        } else if (EPI == E_F16) {
          ((f16_t*)p.C)[row * p.ldc + col] = f2h(v);
        } else if (EPI == E_RES_F32 || EPI == E_RESB_F32) {
          ((float*)p.C)[row * p.ldc + col] = res_cur[r] + v;
        } else if (EPI == E_RESF_B16) {
          ((bf16_t*)p.C)[row * p.ldc + col] = f2bf(res_cur[r] + v);
        }
      }
    }
  };
  if (rows_valid == T::BM && n0 + T::BN <= p.N) walk(std::true_type{});
  else walk(std::false_type{});
}

}  // namespace gemm
