// Causal grouped-query attention over the KV cache.
//
// Definition ([P3] "GQA 注意力" formula; [P1] sections 9-10): for q head h of a
// sequence, query row at absolute position p, kv head h / (nq / nkv):
//     o = sum_{j <= p} softmax_j(q . k_j / sqrt(hd)) v_j
//
// Prefill operands: q arrives in fp16; keys/values produced by this call come from
// unrounded fp16 copies, older ones from the bf16 cache (converted to fp16, exact in fp16's
// normal range, as they are staged); P is rounded to fp16.  Both products run on
// v_mfma_f32_16x16x32_f16.
// Prefill (flash-style, matrix cores):
//   one block = 192 query rows of one q head, 4 waves x 48 rows; K tiles of 64 keys
//   [64][128] and the matching V^T tile [128][64] are staged in LDS (double buffered).
//   Scores are formed transposed, S^T = K . Q^T, so each lane owns one query column:
//   the row max needs two cross-lane steps and the rescale is per lane.  The
//   probabilities P^T then sit in registers exactly in the B-operand order of
//   O^T = V^T . P^T (k-slots permuted consistently with the V^T reads), so P never
//   leaves registers; this is why the cache keeps V transposed.  Tiles entirely above
//   a wave's rows are skipped; heavy row blocks are dispatched first.
// Decode (bandwidth bound): the positions of each (sequence, kv head) are split evenly
// over the waves of several blocks; each wave streams its run of 32-position tiles
// straight from the bf16 cache into 16x16x32 bf16 MFMAs serving all q heads of the group,
// with the next tile's loads in flight.  q and P enter as exact bf16 high + low pairs
// (fp16 q is exactly representable that way), so no operand rounding is added.  The
// block merges its waves in LDS; a second kernel merges the blocks' (max, sum, output)
// partials.
#include "launch.h"

namespace q3 {
namespace {

constexpr int HD = 128;
constexpr int NT = 3;                 // 16-query MFMA column tiles per wave
constexpr int WROWS = 16 * NT;        // query rows per wave
constexpr int PF_WAVES = 4;
constexpr int PF_THREADS = 64 * PF_WAVES;
constexpr int BQ = WROWS * PF_WAVES;  // query rows per block
constexpr int STAGE_WAVES = 4;        // waves that copy K/V tiles (16 KB = 4 x 4 x 1 KB each)
constexpr int BKV = 64;               // keys per LDS tile (two 32-key halves)

// LDS layouts, 16-byte chunks XOR-swizzled so that each 16-lane group of a fragment read
// touches 16 distinct 4-bank groups:
//   K tile   [64 keys][128 dims], 16 chunks per row.  A fragment read takes rows
//            8 (r / 4) + 4 mt + r % 4 (+ 32 in the upper half), r = 0..15, at one logical
//            chunk; row bits 0-1 and 3-4 select the swizzle, which is then r itself.
//   V^T tile [128 dims][64 keys], 8 chunks per row, two rows per bank line.  A fragment
//            read takes 16 consecutive rows at one chunk; rows of one parity get distinct
//            chunks from row bits 1-3.
DEV int k_swz(int row) { return (row & 3) | (((row >> 3) & 3) << 2); }
DEV int k_off(int row, int chunk) { return row * HD + ((chunk ^ k_swz(row)) << 3); }
DEV int v_swz(int row) { return (row >> 1) & 7; }
DEV int v_off(int row, int chunk) { return row * BKV + ((chunk ^ v_swz(row)) << 3); }

DEV float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

DEV f32x4_t mfma16_f16(f16x8_t a, f16x8_t b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

// 16x16x32 MFMA operand layouts (lane l, r = l % 16, grp = l / 16): A row r and B column r,
// k = 8 grp .. 8 grp + 7 for both; the accumulator holds column r, rows 4 grp .. 4 grp + 3.
// S^T = K . Q^T puts one query in each lane's column, so the row max needs two cross-lane
// steps and the rescale is per lane.  Key order: in 32-key half h2 and 16-key m-tile mt,
// A row r reads key 8 (r / 4) + 4 mt + r % 4, so a lane's two accumulators hold keys
// 8 grp .. 8 grp + 7, which is the B-operand k order of O^T = V^T . P^T; P^T never leaves
// registers and the matching V^T fragment is one 16-byte read.  48 query rows per wave keep
// the live state (Q^T 48, O^T 96, S^T 24, P^T 12 registers) small enough for two waves per
// SIMD, so one wave's softmax overlaps the other's matrix work.  (32 rows per wave at three
// waves per SIMD measured slower: less reuse of each K/V fragment, more per-wave overhead.)
// Work placement of the prefill blocks.  A work item is (row level, sequence, q head);
// heavy (late) row levels go first.  Workgroups reach the eight XCDs round-robin (block
// id mod 8), and each XCD has its own L2, so the items are arranged for each XCD to keep
// whole (sequence, kv head) groups: the q heads of a group read the same K/V, which then
// stays in one L2.  With G = B * nkv groups:
//   G a multiple of 8: XCD x owns groups x, x + 8, ...; its i-th block takes level
//     i / n_x, then group and head in order (n_x = G / 8 * g items per level);
//   G dividing 8: R = 8 / G XCDs share one group; XCD x serves group x / R and takes the
//     group's items n = i R + x % R (n = level * g + head), so the levels stay balanced;
//   otherwise: block id = level * (B * nq) + b * nq + h, every XCD receiving every eighth
//     item of each level.
// The block-id -> item map is a bijection onto the items plus idle ids (mode two pads
// the grid to 8 P blocks), so results do not depend on the placement; only locality does.
DEV bool prefill_item(int wid, int nmb, int B, int nq, int nkv, int& mb, int& b, int& h) {
  const int g = nq / nkv, G = B * nkv;
  int level, grpi, head;
  if (G % 8 == 0) {
    const int x = wid & 7, i = wid >> 3, nx = (G / 8) * g;
    level = i / nx;
    const int j = i % nx;
    grpi = x + 8 * (j / g);
    head = j % g;
  } else if (8 % G == 0) {
    const int R = 8 / G, x = wid & 7, i = wid >> 3;
    const int n = i * R + x % R;
    if (n >= nmb * g) return false;
    grpi = x / R;
    level = n / g;
    head = n % g;
  } else {
    level = wid / (B * nq);
    const int rem = wid % (B * nq);
    grpi = (rem / nq) * nkv + (rem % nq) / g;
    head = rem % g;
  }
  if (level >= nmb) return false;
  mb = nmb - 1 - level;
  b = grpi / nkv;
  h = (grpi % nkv) * g + head;
  return true;
}

int prefill_blocks(int nmb, int B, int nq, int nkv) {
  const int g = nq / nkv, G = B * nkv;
  if (G % 8 == 0) return nmb * B * nq;
  if (8 % G == 0) {
    const int R = 8 / G;
    return 8 * ((nmb * g + R - 1) / R);
  }
  return nmb * B * nq;
}

template <bool HAS_PAST>
__global__ void __launch_bounds__(PF_THREADS, HAS_PAST ? 1 : 2) attn_prefill_kernel(AttnPrefillArgs a) {
  __shared__ __attribute__((aligned(16))) f16_t sK[2][BKV * HD];
  __shared__ __attribute__((aligned(16))) f16_t sV[2][HD * BKV];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int r16 = lane & 15, grp = lane >> 4;
  const int nmb = (a.S + BQ - 1) / BQ;
  int mb, b, h;
  if (!prefill_item(blockIdx.x, nmb, a.B, a.nq, a.nkv, mb, b, h)) return;
  const int g = a.nq / a.nkv, kvh = h / g;

  const int row0 = mb * BQ;                          // first query row (token index)
  const int kv_len = a.pos0 + min(a.S, row0 + BQ);   // keys this block may need
  const int ntiles = (kv_len + BKV - 1) / BKV;
  const int wrow0 = row0 + wave * WROWS;
  // a wave whose rows all lie past the sequence end computes nothing
  const int wave_max_pos = wrow0 < a.S ? a.pos0 + min(a.S - 1, wrow0 + WROWS - 1) : -1;
  const int wave_min_pos = a.pos0 + wrow0;

  const f16_t* kfbase = a.k_fresh + ((int64_t)b * a.nkv + kvh) * a.fresh_w * HD;
  const f16_t* vfbase = a.vt_fresh + ((int64_t)b * a.nkv + kvh) * HD * a.fresh_w;

  // Q^T fragments (B operand): column = query row, k = head dims
  f16x8_t qf[NT][4];
  int qpos[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    const int s = wrow0 + nt * 16 + r16;
    const bool valid = s < a.S;
    const int sc = valid ? s : a.S - 1;
    qpos[nt] = valid ? a.pos0 + s : kv_len - 1;
    const f16_t* qp = a.q + (((int64_t)b * a.S + sc) * a.nq + h) * HD + grp * 8;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) qf[nt][ks] = as_f16x8(ld16(qp + ks * 32));
  }

  f32x4_t oacc[8][NT];
#pragma unroll
  for (int md = 0; md < 8; ++md)
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) oacc[md][nt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  // q arrives pre-scaled by log2(e) / sqrt(hd): scores are in log2 units.  m_ref is the
  // reference max the exponentials are taken against (set on the wave's first half).
  // lacc accumulates the softmax denominators with the matrix cores (ones . P^T).
  float m_ref[NT];
  f32x4_t lacc[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    m_ref[nt] = 0.f;
    lacc[nt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  }
  bool first = true;
  const f16x8_t ones = as_f16x8(u32x4_t{0x3C003C00u, 0x3C003C00u, 0x3C003C00u, 0x3C003C00u});

  // ---- tile staging
  // No past (pos0 == 0): every key/value of the block comes from the fp16 copies written
  // by this call (zero beyond the last position), loaded straight into LDS with
  // lds_dma16: lane L of a wave instruction lands at base + 16 L, so each lane fetches
  // the logical chunk that the swizzle places at its physical slot.
  // With a past: keys/values < pos0 come from the bf16 cache (converted to fp16 in
  // registers), the rest from the fp16 copies; rows/columns >= kv_len are zero.
  auto direct_load = [&](int t, int st) {
    if (wave >= STAGE_WAVES) return;
    const int j0 = t * BKV;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int o = (wave * 4 + i) * 1024 + lane * 16;  // byte offset in the K tile
      const int row = o >> 8, p = (o >> 4) & 15;
      const f16_t* src = kfbase + (int64_t)(j0 + row - a.fresh_base) * HD + ((p ^ k_swz(row)) << 3);
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
  const bf16_t* vbase = a.vt_cache + ((int64_t)b * a.nkv + kvh) * a.cap * HD;
  u32x4_t rk[HAS_PAST ? 4 : 1], rv[HAS_PAST ? 4 : 1];
  const u32x4_t zero4 = {0u, 0u, 0u, 0u};
  auto gload = [&](int t) {
    if (tid >= 64 * STAGE_WAVES) return;
    const int j0 = t * BKV;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      int c = tid & 15, r = (tid >> 4) + 16 * i;
      int key = j0 + r;
      u32x4_t v = zero4;
      if (key < a.pos0)
        v = bf16x8_to_f16x8(ld16(kbase + kcache_idx(key, c * 8)));
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
          v = bf16x8_to_f16x8(ld16(vbase + vcache_idx(key, d)));
        } else if (key >= a.pos0) {
          v = ld16(vfbase + (int64_t)d * a.fresh_w + (key - a.fresh_base));
        } else {  // chunk straddles pos0: element-wise choice
          u32x4_t vc = bf16x8_to_f16x8(ld16(vbase + vcache_idx(key, d)));
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
    if (tid >= 64 * STAGE_WAVES) return;
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

  const int krow = 8 * (r16 >> 2) + (r16 & 3);  // K row of A-operand row r16 (mt = 0, h2 = 0)
  for (int t = 0; t < ntiles; ++t) {
    const int st = t & 1;
    if (t + 1 < ntiles) {
      if (HAS_PAST) gload(t + 1);
      else direct_load(t + 1, st ^ 1);
    }
#pragma unroll
    for (int h2 = 0; h2 < 2; ++h2) {
      const int k0 = t * BKV + 32 * h2;
      if (k0 > wave_max_pos) continue;
      // S^T[key][query] - m: 32 keys (two 16-key m-tiles) x 48 queries.  The running
      // reference max enters as the accumulator's initial value, so the scores come out
      // already shifted.
      f32x4_t sacc[2][NT];
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        const f32x4_t negm = {-m_ref[nt], -m_ref[nt], -m_ref[nt], -m_ref[nt]};
#pragma unroll
        for (int mt = 0; mt < 2; ++mt) {
          const f16x8_t kf = as_f16x8(ld16(&sK[st][k_off(32 * h2 + 4 * mt + krow, grp)]));
          sacc[mt][nt] = mfma16_f16(kf, qf[nt][0], negm);
        }
      }
#pragma unroll
      for (int ks = 1; ks < 4; ++ks) {
#pragma unroll
        for (int mt = 0; mt < 2; ++mt) {
          const f16x8_t kf = as_f16x8(ld16(&sK[st][k_off(32 * h2 + 4 * mt + krow, 4 * ks + grp)]));
#pragma unroll
          for (int nt = 0; nt < NT; ++nt) sacc[mt][nt] = mfma16_f16(kf, qf[nt][ks], sacc[mt][nt]);
        }
      }
      if (k0 + 31 > wave_min_pos) {  // the causal diagonal crosses this half
#pragma unroll
        for (int nt = 0; nt < NT; ++nt)
#pragma unroll
          for (int mt = 0; mt < 2; ++mt)
#pragma unroll
            for (int i = 0; i < 4; ++i)
              if (k0 + 8 * grp + 4 * mt + i > qpos[nt]) sacc[mt][nt][i] = -INFINITY;
      }
      // Lazy rescaling: the reference max moves (to this half's column max) only on a
      // wave's first half or when a score exceeds it by more than 8 (log2 units), so
      // P <= 2^8 stays exact enough in fp16 and the accumulators are rescaled rarely.  The
      // test needs only each lane's own maximum; column maxima are formed in the rare path.
      float lmax = sacc[0][0][0];
#pragma unroll
      for (int nt = 0; nt < NT; ++nt)
#pragma unroll
        for (int mt = 0; mt < 2; ++mt)
#pragma unroll
          for (int i = 0; i < 4; ++i) lmax = fmaxf(lmax, sacc[mt][nt][i]);
      if (first || __any(lmax > 8.0f)) {
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
          float x = sacc[0][nt][0];
#pragma unroll
          for (int mt = 0; mt < 2; ++mt)
#pragma unroll
            for (int i = 0; i < 4; ++i) x = fmaxf(x, sacc[mt][nt][i]);
          const float tmax = rows4_max(x);
          const bool mv = (first && tmax > -INFINITY) || tmax > 8.0f;
          const float delta = mv ? tmax : 0.f;
          const float alpha = exp2_fast(-delta);
          m_ref[nt] += delta;
#pragma unroll
          for (int i = 0; i < 4; ++i) lacc[nt][i] *= alpha;
#pragma unroll
          for (int md = 0; md < 8; ++md)
#pragma unroll
            for (int i = 0; i < 4; ++i) oacc[md][nt][i] *= alpha;
#pragma unroll
          for (int mt = 0; mt < 2; ++mt)
#pragma unroll
            for (int i = 0; i < 4; ++i) sacc[mt][nt][i] -= delta;
        }
        first = false;
      }
      f16x8_t pf[NT];
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        u32x4_t u;
#pragma unroll
        for (int e = 0; e < 4; ++e)
          u[e] = pack_f16x2(exp2_fast(sacc[e >> 1][nt][2 * (e & 1)]),
                            exp2_fast(sacc[e >> 1][nt][2 * (e & 1) + 1]));
        pf[nt] = as_f16x8(u);
        // row sums of the rounded P (every accumulator row gets the column's sum)
        lacc[nt] = mfma16_f16(ones, pf[nt], lacc[nt]);
      }
      // O^T[d][query] += V^T[d][keys] . P^T[keys][query]; keys 8 grp .. +8 per lane group
#pragma unroll
      for (int md = 0; md < 8; ++md) {
        const f16x8_t vf = as_f16x8(ld16(&sV[st][v_off(md * 16 + r16, 4 * h2 + grp)]));
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) oacc[md][nt] = mfma16_f16(vf, pf[nt], oacc[md][nt]);
      }
    }
    if (t + 1 < ntiles) {
      if (HAS_PAST) sstore(st ^ 1);
      else wait_dma();
    }
    __syncthreads();
  }

  // normalise and store: lane owns query column r16 of n-tile nt, dims 16 md + 4 grp + i
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    const float inv = 1.0f / lacc[nt][0];
    const int s = wrow0 + nt * 16 + r16;
    if (s >= a.S) continue;
    f16_t* op = a.out + (((int64_t)b * a.S + s) * a.nq + h) * HD + grp * 4;
#pragma unroll
    for (int md = 0; md < 8; ++md) {
      u32x2_t v;
      v[0] = pack_f16x2(oacc[md][nt][0] * inv, oacc[md][nt][1] * inv);
      v[1] = pack_f16x2(oacc[md][nt][2] * inv, oacc[md][nt][3] * inv);
      *(u32x2_t*)(op + md * 16) = v;
    }
  }
}

// ------------------------------------------------------------------ decode
// One wave streams a contiguous run of 32-key tiles of one (sequence, kv head) through
// v_mfma_f32_16x16x32_bf16, reading the bf16 cache as-is.  Operand layouts (lane l,
// r = l % 16, grp = l / 16): A row r, B column r, k = 8 grp .. 8 grp + 7 for both; the
// accumulator holds column r, rows 4 grp .. 4 grp + 3.
//   S^T = K . Q^T: columns 0..7 carry the bf16 high parts of the group's (pre-scaled)
//   q heads, columns 8..15 the bf16 low parts (q - hi), so one MFMA per 32 dims gives
//   both halves and a row_ror:8 DPP add forms the exact fp16 q . k in fp32.
//   O^T = V^T . P^T: likewise P's high part in columns 0..7, its remainder in 8..15.
// Key order: sub-tile s (16 keys) row rho holds key 8 (rho / 4) + 4 s + rho % 4, so the
// two accumulators of a lane hold keys 8 grp .. 8 grp + 7 in B-operand k order and the
// V^T fragment for them is one 16-byte read.
constexpr int kDecWaves = 4;
constexpr int kDecTile = 32;
constexpr int kMaxGroup = 8;

struct DecTile {
  u32x4_t k[8];  // [sub-tile][32-dim chunk]
  u32x4_t v[8];  // [16-dim row tile]
};

// The cache region of one (sequence, kv head) is addressed through buffer descriptors:
// one 32-bit lane offset per operand and the tile's byte offset as a uniform add, so the
// loads need no 64-bit address registers.  In the tiled cache layout a 32-position tile is
// 8 KB of K ([4 chunks][32 positions][32 dims]) and 8 KB of V ([128 dims][32 positions]):
// each K load takes four runs of four positions x 64 bytes (whole 128-byte lines), each V
// load 16 dims x 64 bytes (1 KB in one piece).
struct DecSrc {
  __amdgpu_buffer_rsrc_t k, v;
  uint32_t k_lane;  // bytes: K position 8 (r / 4) + r % 4 of the tile, chunk 0 dims 8 grp ..
  uint32_t v_lane;  // bytes: V dim r of the tile, positions 8 grp ..
};

// Cache-policy bits of the buffer loads: nt (streaming).  The cache is read once per step,
// so its lines are not kept for reuse.  Measured on gfx950 with these whole-line loads, it
// raises the decode attention's read rate by about a tenth; with loads that take half
// lines it costs a quarter instead (the other half is fetched again).
constexpr int kStreamPolicy = 2;

DEV void dec_load(DecTile& t, const DecSrc& src, int key0) {
  const uint32_t tb = (uint32_t)(key0 >> 5) * 8192u;  // key0 is a multiple of 32
#pragma unroll
  for (int s = 0; s < 2; ++s)
#pragma unroll
    for (int c = 0; c < 4; ++c)
      t.k[s * 4 + c] = __builtin_amdgcn_raw_buffer_load_b128(
          src.k, tb + src.k_lane + s * 256 + c * 2048, 0, kStreamPolicy);
#pragma unroll
  for (int rt = 0; rt < 8; ++rt)
    t.v[rt] = __builtin_amdgcn_raw_buffer_load_b128(src.v, tb + src.v_lane + rt * 1024, 0,
                                                    kStreamPolicy);
}

DEV f32x4_t mfma16_bf16(u32x4_t a, u32x4_t b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(a), as_bf16x8(b), c, 0, 0, 0);
}

// x + x from the lane 8 places round the same 16-lane row
DEV float add_ror8(float x) {
  int y = __builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x128, 0xf, 0xf, false);
  return x + __int_as_float(y);
}

DEV uint32_t cvt_bf16x2(float lo, float hi) {
  typedef __bf16 bf16x2v __attribute__((ext_vector_type(2)));
  typedef float f32x2v __attribute__((ext_vector_type(2)));
  f32x2v v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2v));
}

// high part (columns 0..7) or remainder (columns 8..15) of x, rounded to bf16
DEV float split_part(float x, bool low) {
  float hi = __uint_as_float(__float_as_uint(x) & 0xffff0000u);
  return low ? x - hi : hi;
}

struct DecState {
  f32x4_t o[8];  // O^T row tiles: dims 16 rt + 4 grp + i, column r
  float m, l;    // running max (log2 units) and sum for column r's head
};

// Keys at or past kv_len (the last new token's limit) hold anything and are zeroed in V;
// column r's query sees keys below col_len (<= kv_len; mask_from is the smallest col_len
// of the block, so tiles wholly below it need no masking).
DEV void dec_tile(DecState& st, const DecTile& t, const u32x4_t* qb, int key0, int kv_len,
                  int col_len, int mask_from, int lane) {
  const int grp = lane >> 4;
  const bool low = (lane & 15) >= 8;
  f32x4_t sc[2];
#pragma unroll
  for (int s = 0; s < 2; ++s) {
    f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int c = 0; c < 4; ++c) acc = mfma16_bf16(t.k[s * 4 + c], qb[c], acc);
#pragma unroll
    for (int i = 0; i < 4; ++i) acc[i] = add_ror8(acc[i]);
    sc[s] = acc;
  }
  const bool masked = key0 + kDecTile > mask_from;
  if (masked) {
#pragma unroll
    for (int s = 0; s < 2; ++s)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (key0 + 8 * grp + 4 * s + i >= col_len) sc[s][i] = -INFINITY;
  }
  const bool tail = key0 + kDecTile > kv_len;
  float mx = sc[0][0];
#pragma unroll
  for (int s = 0; s < 2; ++s)
#pragma unroll
    for (int i = 0; i < 4; ++i) mx = fmaxf(mx, sc[s][i]);
  mx = rows4_max(mx);
  // lazy rescale: move the reference max only when a score exceeds it by 2^8
  if (__any(mx > st.m + 8.f)) {
    const float mn = fmaxf(st.m, mx);
    const float f = st.m == -INFINITY ? 0.f : exp2_fast(st.m - mn);
    st.m = mn;
    st.l *= f;
#pragma unroll
    for (int rt = 0; rt < 8; ++rt)
#pragma unroll
      for (int i = 0; i < 4; ++i) st.o[rt][i] *= f;
  }
  // a column with no visible key yet keeps m = -inf; its weights are all zero
  const float mref = st.m == -INFINITY ? 0.f : st.m;
  float p[8];
#pragma unroll
  for (int s = 0; s < 2; ++s)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      p[4 * s + i] = exp2_fast(sc[s][i] - mref);
      st.l += p[4 * s + i];
    }
  u32x4_t pb;
#pragma unroll
  for (int e = 0; e < 4; ++e)
    pb[e] = cvt_bf16x2(split_part(p[2 * e], low), split_part(p[2 * e + 1], low));
  if (!tail) {
#pragma unroll
    for (int rt = 0; rt < 8; ++rt) st.o[rt] = mfma16_bf16(t.v[rt], pb, st.o[rt]);
  } else {
    // values past the sequence end may hold anything (NaN included): zero them
    u32x4_t keep;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int k = key0 + 8 * grp + 2 * e;
      keep[e] = (k < kv_len ? 0xffffu : 0u) | (k + 1 < kv_len ? 0xffff0000u : 0u);
    }
#pragma unroll
    for (int rt = 0; rt < 8; ++rt) st.o[rt] = mfma16_bf16(t.v[rt] & keep, pb, st.o[rt]);
  }
}

// Queries of one (sequence, kv head): its S new tokens times the g q heads of the group,
// listed token-major (query i = token i / g, head i % g), eight per block (blockIdx.z
// = sequence * nqg + query group).  Token s of the sequence sees keys 0 .. pos + s.
__global__ void __launch_bounds__(256) attn_decode_kernel(AttnDecodeArgs a) {
  __shared__ float so[kDecWaves][kMaxGroup][HD];
  __shared__ float sm[kDecWaves][kMaxGroup], sl[kDecWaves][kMaxGroup];
  const int split = blockIdx.x, kvh = blockIdx.y, b = blockIdx.z / a.nqg;
  const int qg = blockIdx.z % a.nqg;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = a.nq / a.nkv;
  const int nqry = a.S * g;                           // queries of this (sequence, kv head)
  const int ncols = min(kMaxGroup, nqry - qg * kMaxGroup);  // in this block
  const int pos = a.pos[b];
  const bool ok = pos >= 0 && pos + a.S <= a.cap && pos + a.S <= a.max_pos;
  const int kv_len = ok ? pos + a.S : 0;
  // 64-key units spread evenly over the blocks serving this (sequence, kv head); the
  // block's waves take its 32-key tiles in turn, so at any time the block reads one
  // contiguous window of its cache region (3% faster than a run per wave)
  const int n64 = (kv_len + 63) / 64;
  const int kbeg = (int)((int64_t)split * n64 / a.splits) * 64 + wave * kDecTile;
  const int kend = min((int)((int64_t)(split + 1) * n64 / a.splits) * 64, kv_len);
  constexpr int kStep = kDecWaves * kDecTile;

  const int r = lane & 15, grp = lane >> 4;
  const int hh = r & 7;  // query column within the block
  const bool low = r >= 8;
  const int qi = qg * kMaxGroup + hh;
  const bool qlive = hh < ncols;
  const int q_tok = qlive ? qi / g : 0, q_head = qlive ? qi % g : 0;
  const int col_len = qlive ? pos + 1 + q_tok : kv_len;
  DecState st;
  st.m = -INFINITY;
  st.l = 0.f;
#pragma unroll
  for (int rt = 0; rt < 8; ++rt) st.o[rt] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  if (kbeg < kend) {
    const int64_t region = (int64_t)a.cap * HD;  // elements per (sequence, kv head)
    DecSrc src;
    src.k = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(a.k_cache + ((int64_t)b * a.nkv + kvh) * region), 0, (int)(region * 2), 0x00020000);
    src.v = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(a.vt_cache + ((int64_t)b * a.nkv + kvh) * region), 0, (int)(region * 2),
        0x00020000);
    src.k_lane = (uint32_t)(8 * (r >> 2) + (r & 3)) * 64 + grp * 16;
    src.v_lane = (uint32_t)r * 64 + grp * 16;
    // two register buffers: the wave's next tile is in flight while one is consumed.
    // Past the wave's last tile the "next" load repeats the current tile (one spare 16 KB
    // read per wave) so that the wait counts are the same on every path.
    DecTile t0, t1;
    int key = kbeg;
    dec_load(t0, src, key);
    dec_load(t1, src, key + kStep < kend ? key + kStep : key);
    // q after the first two tiles' loads: all arrive within one memory latency
    u32x4_t qb[4];
    const f16_t* qrow =
        a.q + (((int64_t)b * a.S + q_tok) * a.nq + kvh * g + q_head) * HD + grp * 8;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      float f[8];
      if (qlive) {
        unpack8_f16(ld16(qrow + c * 32), f);
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) f[e] = 0.f;
      }
#pragma unroll
      for (int e = 0; e < 4; ++e)
        qb[c][e] = cvt_bf16x2(split_part(f[2 * e], low), split_part(f[2 * e + 1], low));
    }
    // t0 holds the tile at key, t1 the wave's next tile (in flight)
    for (;;) {
      dec_tile(st, t0, qb, key, kv_len, col_len, pos + 1, lane);
      key += kStep;
      if (key >= kend) break;
      dec_load(t0, src, key + kStep < kend ? key + kStep : key);
      dec_tile(st, t1, qb, key, kv_len, col_len, pos + 1, lane);
      key += kStep;
      if (key >= kend) break;
      dec_load(t1, src, key + kStep < kend ? key + kStep : key);
    }
  }
  // fold the low-part columns into the high ones and the four row groups of the sum
  st.l = rows4_sum(st.l);
#pragma unroll
  for (int rt = 0; rt < 8; ++rt)
#pragma unroll
    for (int i = 0; i < 4; ++i) st.o[rt][i] = add_ror8(st.o[rt][i]);
  if (r < ncols) {
#pragma unroll
    for (int rt = 0; rt < 8; ++rt)
#pragma unroll
      for (int i = 0; i < 4; ++i) so[wave][r][rt * 16 + 4 * grp + i] = st.o[rt][i];
    if (grp == 0) {
      sm[wave][r] = st.m;
      sl[wave][r] = st.l;
    }
  }
  __syncthreads();
  // merge the block's four waves into one (max, sum, output) partial per query; with a
  // single split that is the result: normalise and store it (NaN rows for a sequence
  // outside the cache, as the combine kernel does)
  for (int i = tid; i < ncols * HD; i += 256) {
    const int h = i / HD, d = i % HD;
    const int qh = qg * kMaxGroup + h;
    float* part = a.part + ((((int64_t)b * a.S + qh / g) * a.nq + kvh * g + qh % g) * a.splits +
                            split) * (HD + 2);
    float M = -INFINITY;
#pragma unroll
    for (int v = 0; v < kDecWaves; ++v) M = fmaxf(M, sm[v][h]);
    float O = 0.f, L = 0.f;
    if (M != -INFINITY) {
#pragma unroll
      for (int v = 0; v < kDecWaves; ++v) {
        if (sm[v][h] == -INFINITY) continue;
        const float f = exp2_fast(sm[v][h] - M);
        O += so[v][h][d] * f;
        L += sl[v][h] * f;
      }
    }
    if (a.splits == 1) {
      const int64_t row = (int64_t)b * a.S + qh / g;
      a.out[(row * a.nq + kvh * g + qh % g) * HD + d] =
          f2h(ok ? O / L : __int_as_float(0x7FC00000));
      continue;
    }
    part[d] = O;
    if (d == 0) {
      part[HD] = M;
      part[HD + 1] = L;
    }
  }
}

__global__ void __launch_bounds__(128) attn_decode_combine_kernel(AttnDecodeArgs a) {
  const int bh = blockIdx.x;  // (token row, q head)
  const int b = bh / a.nq / a.S;
  const int d = threadIdx.x;
  const int pos = a.pos[b];
  const bool ok = pos >= 0 && pos + a.S <= a.cap && pos + a.S <= a.max_pos;
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
  const int blocks = prefill_blocks(nmb, a.B, a.nq, a.nkv);
  if (a.pos0 > 0)
    hipLaunchKernelGGL(attn_prefill_kernel<true>, dim3(blocks), dim3(PF_THREADS), 0, s, a);
  else
    hipLaunchKernelGGL(attn_prefill_kernel<false>, dim3(blocks), dim3(PF_THREADS), 0, s, a);
  return hipGetLastError();
}

void attn_decode_plan(int cap, int B, int nkv, int& splits, int& chunk) {
  // up to 8192 positions per block (2048 per wave), more blocks when the batch is too
  // small for one round of resident blocks (two per CU), never fewer than 64 positions per
  // wave.  With one split the kernel normalises and stores the output itself.
  const int by_len = (cap + 8191) / 8192;
  const int fill = (512 + B * nkv - 1) / (B * nkv);
  splits = std::min((cap + 255) / 256, std::max(by_len, fill));
  chunk = (cap + splits - 1) / splits;
}

int attn_decode_groups(int S, int g) { return (S * g + kMaxGroup - 1) / kMaxGroup; }

hipError_t attn_decode(const AttnDecodeArgs& a, hipStream_t s) {
  if (a.B <= 0) return hipSuccess;
  if (a.S <= 0 || a.nqg != attn_decode_groups(a.S, a.nq / a.nkv)) return hipErrorInvalidValue;
  hipLaunchKernelGGL(attn_decode_kernel, dim3(a.splits, a.nkv, a.B * a.nqg), dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t attn_decode_combine(const AttnDecodeArgs& a, hipStream_t s) {
  if (a.B <= 0) return hipSuccess;
  hipLaunchKernelGGL(attn_decode_combine_kernel, dim3(a.B * a.S * a.nq), dim3(128), 0, s, a);
  return hipGetLastError();
}

}  // namespace q3
