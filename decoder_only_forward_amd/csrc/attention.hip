// Causal grouped-query attention over the KV cache.
//
// Definition ([P3] "GQA 注意力" formula; [P1] sections 9-10): for q head h of a
// sequence, query row at absolute position p, kv head h / (nq / nkv):
//     o = sum_{j <= p} softmax_j(q . k_j / sqrt(hd)) v_j
//
// Operands: q arrives in fp16; keys/values produced by this call come from unrounded fp16
// copies, older ones from the bf16 cache (converted to fp16, exact in fp16's normal range,
// as they are staged); P is rounded to fp16.  Both products run on
// v_mfma_f32_16x16x32_f16.
// Prefill (flash-style, matrix cores):
//   one block = 128 query rows of one q head, 4 waves x 32 rows; K tiles of 64 keys
//   [64][128] and the matching V^T tile [128][64] are staged in LDS (double buffered).
//   Scores are formed transposed, S^T = K . Q^T, so each lane owns one query column:
//   the row max needs only two cross-lane steps and the rescale is per lane.  The
//   probabilities P^T then sit in registers exactly in the B-operand order of
//   O^T = V^T . P^T (k-slots permuted consistently with the V^T reads), so P never
//   leaves registers; this is why the cache keeps V transposed.  Tiles entirely above
//   a wave's rows are skipped; heavy row blocks are dispatched first.
// Decode (bandwidth bound): split-K over the cache positions, one block per
// (sequence, kv head, 256-position chunk) serving all q heads of the group from one
// read of K and V; a second kernel merges the partial (max, sum, output) triples.
#include "launch.h"

namespace q3 {
namespace {

constexpr int HD = 128;
constexpr int WROWS = 64;   // query rows per wave (two 32-column MFMA tiles)
constexpr int PF_WAVES = 4;
constexpr int BQ = WROWS * PF_WAVES;  // query rows per block
constexpr int BKV = 64;     // keys per tile

// LDS layouts (16-byte chunks, XOR-swizzled so that the fragment reads of 16 consecutive
// rows at one logical chunk hit distinct banks):
//   K tile   [64 keys][128 dims]  = 16 chunks per row, chunk ^ (row & 15)
//   V^T tile [128 dims][64 keys]  =  8 chunks per row, chunk ^ (row & 7) ^ (row >> 3 & 1)
DEV int k_off(int row, int chunk) { return row * HD + ((chunk ^ (row & 15)) << 3); }
DEV int v_swz(int row) { return (row & 7) ^ ((row >> 3) & 1); }
DEV int v_off(int row, int chunk) { return row * BKV + ((chunk ^ v_swz(row)) << 3); }

DEV float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

DEV f32x16_t mfma32(f16x8_t a, f16x8_t b, f32x16_t c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
}

// Key order inside a 32-key MFMA tile: A-operand row rho reads key pi(rho), pi swapping
// bits 2 and 3.  With the 32x32 accumulator layout (lane l, h = l / 32, register i ->
// row 8(i/4) + 4h + i%4) this puts keys 16(i/8) + 8h + i%8 in register i of lane half h:
// each 8-register group holds 8 consecutive keys, which is the B-operand k-slot order of
// the P^T.V product, and the matching V^T fragment is one contiguous 16-byte read.
DEV int key_perm(int r) { return (r & ~12) | ((r & 4) << 1) | ((r & 8) >> 1); }

// 32x32x16 MFMA operand layouts (lane l, h = l / 32): A row l % 32 and B column l % 32,
// k = 8h .. 8h + 7 for both.  S^T = K . Q^T puts one query in each lane's column, so the
// row max needs one cross-lane step and the rescale is per lane.
template <bool HAS_PAST>
__global__ void __launch_bounds__(256) attn_prefill_kernel(AttnPrefillArgs a) {
  __shared__ __attribute__((aligned(16))) f16_t sK[2][BKV * HD];
  __shared__ __attribute__((aligned(16))) f16_t sV[2][HD * BKV];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, hh = lane >> 5;
  const int nmb = (a.S + BQ - 1) / BQ;
  const int nblocks = nmb * a.B * a.nq;
  // contiguous work ranges per XCD; heavy (late) row blocks first
  int wid;
  {
    int q = nblocks >> 3, r = nblocks & 7, x = blockIdx.x & 7, i = blockIdx.x >> 3;
    wid = (x < r ? x * (q + 1) : r * (q + 1) + (x - r) * q) + i;
  }
  const int mb = nmb - 1 - wid / (a.B * a.nq);
  const int rem = wid % (a.B * a.nq);
  const int b = rem / a.nq, h = rem % a.nq;
  const int g = a.nq / a.nkv, kvh = h / g;

  const int row0 = mb * BQ;                          // first query row (token index)
  const int kv_len = a.pos0 + min(a.S, row0 + BQ);   // keys this block may need
  const int ntiles = (kv_len + BKV - 1) / BKV;
  const int wrow0 = row0 + wave * WROWS;
  const int wave_max_pos = a.pos0 + min(a.S - 1, wrow0 + WROWS - 1);
  const int wave_min_pos = a.pos0 + wrow0;

  const f16_t* kfbase = a.k_fresh + ((int64_t)b * a.nkv + kvh) * a.fresh_w * HD;
  const f16_t* vfbase = a.vt_fresh + ((int64_t)b * a.nkv + kvh) * HD * a.fresh_w;

  // Q^T fragments (B operand): column = query row, k = head dims
  f16x8_t qf[2][8];
  int qpos[2];
#pragma unroll
  for (int nt = 0; nt < 2; ++nt) {
    int s = wrow0 + nt * 32 + l32;
    bool valid = s < a.S;
    int sc = valid ? s : a.S - 1;
    qpos[nt] = valid ? a.pos0 + s : kv_len - 1;
    const f16_t* qp = a.q + (((int64_t)b * a.S + sc) * a.nq + h) * HD;
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) qf[nt][ks] = as_f16x8(ld16(qp + ks * 16 + hh * 8));
  }

  f32x16_t oacc[4][2];
#pragma unroll
  for (int md = 0; md < 4; ++md)
#pragma unroll
    for (int nt = 0; nt < 2; ++nt)
#pragma unroll
      for (int i = 0; i < 16; ++i) oacc[md][nt][i] = 0.f;
  // q arrives pre-scaled by log2(e) / sqrt(hd): scores are in log2 units
  float m_run[2] = {-INFINITY, -INFINITY}, l_run[2] = {0.f, 0.f};

  // ---- tile staging
  // No past (pos0 == 0): every key/value of the block comes from the fp16 copies written
  // by this call (zero beyond the last position), loaded straight into LDS with
  // lds_dma16: lane L of a wave instruction lands at base + 16 L, so each
  // lane fetches the logical chunk that the swizzle places at its physical slot.
  // With a past: keys/values < pos0 come from the bf16 cache (converted to fp16 in
  // registers), the rest from the fp16 copies; rows/columns >= kv_len are zero.
  auto direct_load = [&](int t, int st) {
    const int j0 = t * BKV;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int o = (wave * 4 + i) * 1024 + lane * 16;  // byte offset in the K tile
      const int row = o >> 8, p = (o >> 4) & 15;
      const f16_t* src = kfbase + (int64_t)(j0 + row - a.fresh_base) * HD + ((p ^ (row & 15)) << 3);
      lds_dma16(src, &sK[st][(wave * 4 + i) * 512]);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int o = (wave * 4 + i) * 1024 + lane * 16;  // byte offset in the V^T tile
      const int d = o >> 7, p = (o >> 4) & 7;
      const f16_t* src = vfbase + (int64_t)d * a.fresh_w + (j0 - a.fresh_base) + ((p ^ v_swz(d)) << 3);
      lds_dma16(src, &sV[st][(wave * 4 + i) * 512]);
    }
  };
  const bf16_t* kbase = a.k_cache + ((int64_t)b * a.nkv + kvh) * a.cap * HD;
  const bf16_t* vbase = a.vt_cache + ((int64_t)b * a.nkv + kvh) * HD * a.cap;
  u32x4_t rk[HAS_PAST ? 4 : 1], rv[HAS_PAST ? 4 : 1];
  const u32x4_t zero4 = {0u, 0u, 0u, 0u};
  auto gload = [&](int t) {
    const int j0 = t * BKV;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      int c = tid & 15, r = (tid >> 4) + 16 * i;
      int key = j0 + r;
      u32x4_t v = zero4;
      if (key < a.pos0)
        v = bf16x8_to_f16x8(ld16(kbase + (int64_t)key * HD + c * 8));
      else if (key < kv_len)
        v = ld16(kfbase + (int64_t)(key - a.fresh_base) * HD + c * 8);
      rk[i] = v;
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      int c = tid & 7, d = (tid >> 3) + 32 * i;
      int key = j0 + c * 8;
      u32x4_t v = zero4;
      if (key < kv_len) {
        if (key + 8 <= a.pos0) {
          v = bf16x8_to_f16x8(ld16(vbase + (int64_t)d * a.cap + key));
        } else if (key >= a.pos0) {
          v = ld16(vfbase + (int64_t)d * a.fresh_w + (key - a.fresh_base));
        } else {  // chunk straddles pos0: element-wise choice
          u32x4_t vc = bf16x8_to_f16x8(ld16(vbase + (int64_t)d * a.cap + key));
          u32x4_t vf = ld16(vfbase + (int64_t)d * a.fresh_w + (key - a.fresh_base));
          int ncache = a.pos0 - key;  // 1..7 elements from the cache
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            uint32_t mc = (2 * e + 1 < ncache) ? 0xFFFFFFFFu : (2 * e < ncache ? 0xFFFFu : 0u);
            v[e] = (vc[e] & mc) | (vf[e] & ~mc);
          }
        }
        if (key + 8 > kv_len) {
          int nvalid = kv_len - key;  // 1..7 keys valid in this chunk
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            uint32_t keep = (2 * e + 1 < nvalid) ? 0xFFFFFFFFu : (2 * e < nvalid ? 0xFFFFu : 0u);
            v[e] &= keep;
          }
        }
      }
      rv[i] = v;
    }
  };
  auto sstore = [&](int st) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      int c = tid & 15, r = (tid >> 4) + 16 * i;
      st16(&sK[st][k_off(r, c)], rk[i]);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      int c = tid & 7, d = (tid >> 3) + 32 * i;
      st16(&sV[st][v_off(d, c)], rv[i]);
    }
  };

  if (HAS_PAST) {
    gload(0);
    sstore(0);
  } else {
    direct_load(0, 0);
    wait_dma();
  }
  __syncthreads();

  const int krow0 = key_perm(l32);
  for (int t = 0; t < ntiles; ++t) {
    const int st = t & 1;
    if (t + 1 < ntiles) {
      if (HAS_PAST) gload(t + 1);
      else direct_load(t + 1, st ^ 1);
    }
    const int j0 = t * BKV;
    if (j0 <= wave_max_pos) {
      // S^T[key][qrow]: 64 keys (mt) x 64 query rows (nt)
      f32x16_t sacc[2][2];
#pragma unroll
      for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int nt = 0; nt < 2; ++nt)
#pragma unroll
          for (int i = 0; i < 16; ++i) sacc[mt][nt][i] = 0.f;
#pragma unroll
      for (int ks = 0; ks < 8; ++ks) {
#pragma unroll
        for (int mt = 0; mt < 2; ++mt) {
          f16x8_t kf = as_f16x8(ld16(&sK[st][k_off(mt * 32 + krow0, ks * 2 + hh)]));
#pragma unroll
          for (int nt = 0; nt < 2; ++nt) sacc[mt][nt] = mfma32(kf, qf[nt][ks], sacc[mt][nt]);
        }
      }
      const bool need_mask = j0 + BKV - 1 > wave_min_pos;
      f16x8_t pf[2][4];
#pragma unroll
      for (int nt = 0; nt < 2; ++nt) {
        float tmax = -INFINITY;
        if (need_mask) {
#pragma unroll
          for (int mt = 0; mt < 2; ++mt)
#pragma unroll
            for (int i = 0; i < 16; ++i) {
              int key = j0 + mt * 32 + (i >> 3) * 16 + hh * 8 + (i & 7);
              if (key > qpos[nt]) sacc[mt][nt][i] = -INFINITY;
            }
        }
#pragma unroll
        for (int mt = 0; mt < 2; ++mt)
#pragma unroll
          for (int i = 0; i < 16; ++i) tmax = fmaxf(tmax, sacc[mt][nt][i]);
        tmax = fmaxf(tmax, __shfl_xor(tmax, 32, 64));
        // Lazy rescaling: the running max is only raised when a score exceeds it by more
        // than 8 (log2 units), so P <= 2^8 stays exact enough in fp16 and the output
        // accumulators are rescaled only when some lane's max moved that far.
        const bool raise = tmax > m_run[nt] + 8.0f;
        if (__any(raise)) {
          const float m_new = raise ? tmax : m_run[nt];
          const float alpha = exp2_fast(m_run[nt] - m_new);
          m_run[nt] = m_new;
          l_run[nt] *= alpha;
#pragma unroll
          for (int md = 0; md < 4; ++md)
#pragma unroll
            for (int i = 0; i < 16; ++i) oacc[md][nt][i] *= alpha;
        }
        const float m_use = m_run[nt] == -INFINITY ? 0.f : m_run[nt];
        float psum = 0.f;
#pragma unroll
        for (int s2 = 0; s2 < 4; ++s2) {
          const int mt = s2 >> 1, i0 = (s2 & 1) * 8;
          u32x4_t u;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            float p0 = exp2_fast(sacc[mt][nt][i0 + 2 * e] - m_use);
            float p1 = exp2_fast(sacc[mt][nt][i0 + 2 * e + 1] - m_use);
            psum += p0 + p1;
            u[e] = pack_f16x2(p0, p1);
          }
          pf[nt][s2] = as_f16x8(u);
        }
        l_run[nt] += psum;
      }
      // O^T[d][qrow] += V^T[d][keys] . P^T[keys][qrow]; keys 16 s2 + 8h .. +8 per lane half
#pragma unroll
      for (int s2 = 0; s2 < 4; ++s2) {
#pragma unroll
        for (int md = 0; md < 4; ++md) {
          f16x8_t vf = as_f16x8(ld16(&sV[st][v_off(md * 32 + l32, s2 * 2 + hh)]));
#pragma unroll
          for (int nt = 0; nt < 2; ++nt) oacc[md][nt] = mfma32(vf, pf[nt][s2], oacc[md][nt]);
        }
      }
    }
    if (t + 1 < ntiles) {
      if (HAS_PAST) sstore(st ^ 1);
      else wait_dma();
    }
    __syncthreads();
  }

  // normalise and store: lane owns query column l32 of n-tile nt, dims 32md + 8g + 4hh + i
#pragma unroll
  for (int nt = 0; nt < 2; ++nt) {
    float l = l_run[nt];
    l += __shfl_xor(l, 32, 64);
    const float inv = 1.0f / l;
    const int s = wrow0 + nt * 32 + l32;
    if (s >= a.S) continue;
    f16_t* op = a.out + (((int64_t)b * a.S + s) * a.nq + h) * HD;
#pragma unroll
    for (int md = 0; md < 4; ++md)
#pragma unroll
      for (int gq = 0; gq < 4; ++gq) {
        u32x2_t v;
        v[0] = pack_f16x2(oacc[md][nt][4 * gq] * inv, oacc[md][nt][4 * gq + 1] * inv);
        v[1] = pack_f16x2(oacc[md][nt][4 * gq + 2] * inv, oacc[md][nt][4 * gq + 3] * inv);
        *(u32x2_t*)(op + md * 32 + gq * 8 + hh * 4) = v;
      }
  }
}

// ------------------------------------------------------------------ decode
constexpr int kDecChunk = 256;
constexpr int kMaxGroup = 8;

__global__ void __launch_bounds__(256) attn_decode_kernel(AttnDecodeArgs a) {
  __shared__ float sp[kMaxGroup][kDecChunk];
  __shared__ float sm[kMaxGroup], sl[kMaxGroup];
  const int split = blockIdx.x, kvh = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = a.nq / a.nkv;
  const int pos = a.pos[b];
  const bool ok = pos >= 0 && pos < a.cap && pos < a.max_pos;
  const int kv_len = ok ? pos + 1 : 0;
  const int j0 = split * kDecChunk;
  const int n = max(0, min(kDecChunk, kv_len - j0));
  float* part = a.part + (((int64_t)b * a.nq + kvh * g) * a.splits + split) * (HD + 2);
  const int64_t hstride = (int64_t)a.splits * (HD + 2);

  if (n == 0) {
    for (int i = tid; i < g * (HD + 2); i += 256) {
      int hh = i / (HD + 2), e = i % (HD + 2);
      part[hh * hstride + e] = e == HD ? -INFINITY : 0.f;
    }
    return;
  }
  const bf16_t* kbase = a.k_cache + (((int64_t)b * a.nkv + kvh) * a.cap + j0) * HD;
  const bf16_t* vbase = a.vt_cache + ((int64_t)b * a.nkv + kvh) * HD * a.cap + j0;

  // phase 1: scores (log2 domain).  16 lanes per key row, 4 keys per wave step.
  const int kg = lane >> 4, dc = lane & 15;
  // q arrives pre-scaled by log2(e) / sqrt(hd): scores are in log2 units
  float qv[kMaxGroup][8];
#pragma unroll
  for (int hh = 0; hh < kMaxGroup; ++hh) {
    if (hh < g) {
      float f[8];
      unpack8_f16(ld16(a.q + ((int64_t)b * a.nq + kvh * g + hh) * HD + dc * 8), f);
#pragma unroll
      for (int e = 0; e < 8; ++e) qv[hh][e] = f[e];
    }
  }
  for (int j = wave * 4 + kg; j < n; j += 16) {
    float kf[8];
    unpack8(ld16(kbase + (int64_t)j * HD + dc * 8), kf);
#pragma unroll
    for (int hh = 0; hh < kMaxGroup; ++hh) {
      if (hh < g) {
        float d = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) d += qv[hh][e] * kf[e];
        d += __shfl_xor(d, 1, 64);
        d += __shfl_xor(d, 2, 64);
        d += __shfl_xor(d, 4, 64);
        d += __shfl_xor(d, 8, 64);
        if (dc == 0) sp[hh][j] = d;
      }
    }
  }
  __syncthreads();
  // phase 2: per-head max and exponentials
  for (int hh = wave; hh < g; hh += 4) {
    float m = -INFINITY;
    for (int j = lane; j < n; j += 64) m = fmaxf(m, sp[hh][j]);
    m = warp_max(m);
    float s = 0.f;
    for (int j = lane; j < kDecChunk; j += 64) {
      float p = j < n ? exp2_fast(sp[hh][j] - m) : 0.f;
      sp[hh][j] = p;
      s += p;
    }
    s = warp_sum(s);
    if (lane == 0) { sm[hh] = m; sl[hh] = s; }
  }
  __syncthreads();
  // phase 3: o[hh][d] = sum_j p[hh][j] vt[d][j]; 16 lanes per d row, 16 keys per lane
  const int rg = tid >> 4, kl = tid & 15;
  float pv[kMaxGroup][16];
#pragma unroll
  for (int hh = 0; hh < kMaxGroup; ++hh)
    if (hh < g)
#pragma unroll
      for (int e = 0; e < 16; ++e) pv[hh][e] = sp[hh][kl * 16 + e];
  for (int r = 0; r < HD / 16; ++r) {
    const int d = rg + 16 * r;
    const int key = kl * 16;
    float vf[16];
    if (key + 16 <= n) {
      unpack8(ld16(vbase + (int64_t)d * a.cap + key), vf);
      unpack8(ld16(vbase + (int64_t)d * a.cap + key + 8), vf + 8);
    } else {
#pragma unroll
      for (int e = 0; e < 16; ++e)
        vf[e] = key + e < n ? bf2f(vbase[(int64_t)d * a.cap + key + e]) : 0.f;
    }
#pragma unroll
    for (int hh = 0; hh < kMaxGroup; ++hh) {
      if (hh < g) {
        float acc = 0.f;
#pragma unroll
        for (int e = 0; e < 16; ++e) acc += pv[hh][e] * vf[e];
        acc += __shfl_xor(acc, 1, 64);
        acc += __shfl_xor(acc, 2, 64);
        acc += __shfl_xor(acc, 4, 64);
        acc += __shfl_xor(acc, 8, 64);
        if (kl == 0) part[hh * hstride + d] = acc;
      }
    }
  }
  if (tid < g) {
    part[tid * hstride + HD] = sm[tid];
    part[tid * hstride + HD + 1] = sl[tid];
  }
}

__global__ void __launch_bounds__(128) attn_decode_combine_kernel(AttnDecodeArgs a) {
  const int bh = blockIdx.x;
  const int b = bh / a.nq;
  const int d = threadIdx.x;
  const int pos = a.pos[b];
  const bool ok = pos >= 0 && pos < a.cap && pos < a.max_pos;
  const float* part = a.part + (int64_t)bh * a.splits * (HD + 2);
  float M = -INFINITY;
  for (int s = 0; s < a.splits; ++s) M = fmaxf(M, part[s * (HD + 2) + HD]);
  float L = 0.f, O = 0.f;
  for (int s = 0; s < a.splits; ++s) {
    const float* p = part + s * (HD + 2);
    float m = p[HD];
    if (m == -INFINITY) continue;
    float f = exp2_fast(m - M);
    L += p[HD + 1] * f;
    O += p[d] * f;
  }
  float o = ok ? O / L : __int_as_float(0x7FC00000);
  a.out[(int64_t)bh * HD + d] = f2h(o);
}

}  // namespace

hipError_t attn_prefill(const AttnPrefillArgs& a, hipStream_t s) {
  if (a.B <= 0 || a.S <= 0) return hipSuccess;
  const int nmb = (a.S + BQ - 1) / BQ;
  if (a.pos0 > 0)
    hipLaunchKernelGGL(attn_prefill_kernel<true>, dim3(nmb * a.B * a.nq), dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL(attn_prefill_kernel<false>, dim3(nmb * a.B * a.nq), dim3(256), 0, s, a);
  return hipGetLastError();
}

void attn_decode_plan(int cap, int& splits, int& chunk) {
  chunk = kDecChunk;
  splits = (cap + kDecChunk - 1) / kDecChunk;
}

hipError_t attn_decode(const AttnDecodeArgs& a, hipStream_t s) {
  if (a.B <= 0) return hipSuccess;
  hipLaunchKernelGGL(attn_decode_kernel, dim3(a.splits, a.nkv, a.B), dim3(256), 0, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(attn_decode_combine_kernel, dim3(a.B * a.nq), dim3(128), 0, s, a);
  return hipGetLastError();
}

}  // namespace q3
