// Tree attention for the verification forward on gfx950.
//
// The target verifies the whole draft tree in one forward pass: node i of
// sequence b attends to the committed keys 0..L-1 and to the tree keys L+j of
// its ancestors j (EAGLE, paperlayer.ai summary, §2 Preliminaries; §3 EAGLE:
// tree attention).  This is decode-shaped attention: M = G*N query rows per
// KV head against L+N keys, HBM-bound on the bf16 K/V stream.
//
// Work decomposition
//   unit  = (b, kv head, query group of <= RW rows); split = a contiguous range
//   of KV tiles.  One 256-thread workgroup per (unit, split).  Workgroup ids
//   are laid out so every split of a unit lands on one XCD (blocks go to XCDs
//   round robin), keeping its partials and counter in that XCD's L2.
//   Inside a workgroup the 4 waves form a WQ x WK grid: WQ waves over query
//   blocks of 16 rows, WK waves over 32-key chunks of each tile.
//
// Per tile (KT keys): all 256 threads stream K and V with 16-byte coalesced
// loads into registers (issued one tile ahead), then store K row-major and V
// transposed into LDS, so every wave of the workgroup (all G*N queries of the
// KV head) reuses one copy of the tile.  Each wave computes
//   S^T[32 keys x 16 queries] = K Q^T   with v_mfma_f32_16x16x32_bf16
//   (keys on MFMA rows; the K rows are permuted so that each lane ends up
//    holding 8 consecutive keys of one query column),
// applies the tree mask, runs the online softmax with cross-lane shuffles,
// packs P^T to bf16 in registers and accumulates
//   O^T[d x 16 queries] += V^T P^T      with the same MFMA.
// Splits write (m, l, O) partials; the last workgroup of a unit to finish
// (atomic ticket) merges them with log-sum-exp weights and writes bf16 output.
#include <stdlib.h>

#include "common.h"
#include "launch.h"

namespace eagle {

template <int D_, int QBW_, int WQ_, int KC_>
struct AttnShape {
  static constexpr int D = D_;
  static constexpr int QBW = QBW_;          // 16-row query blocks per wave
  static constexpr int WQ = WQ_;            // waves across query blocks
  static constexpr int WK = 4 / WQ_;        // waves across keys
  static constexpr int KC = KC_;            // 32-key chunks per wave per tile
  static constexpr int KT = 32 * KC * WK;   // keys per tile
  static constexpr int RW = 16 * QBW * WQ;  // query rows per workgroup
  static constexpr int KS = D + 8;          // K tile row stride (bf16 elements)
  static constexpr int VS = KT + 8;         // V^T tile row stride (bf16 elements)
  static constexpr int CPR = D / 8;         // 16-byte chunks per key row
  static constexpr int KG = 256 / CPR;      // key quads per staging pass
  static constexpr int NQ = KT / 4;         // key quads per tile
  static constexpr int PASSES = (NQ + KG - 1) / KG;
  static constexpr int NKS = D / 32;        // MFMA k-steps over d
  static constexpr int NDB = D / 16;        // 16-wide d blocks of the output
  static constexpr int LDS_TILE = (KT * KS + D * VS) * 2;        // bytes
  static constexpr int LDS_MERGE = WK > 1 ? 4 * (QBW * NDB * 256 + QBW * 32) * 4 : 0;
  static constexpr int LDS_WEIGHTS = RW * 32 * 4;  // split-merge weights, <= 32 splits
  static constexpr int LDS_BYTES0 = LDS_TILE > LDS_MERGE ? LDS_TILE : LDS_MERGE;
  static constexpr int LDS_BYTES = LDS_BYTES0 > LDS_WEIGHTS ? LDS_BYTES0 : LDS_WEIGHTS;
  static_assert(NQ >= 8 && (NQ & (NQ - 1)) == 0, "V^T swizzle needs >= 8 key quads, power of 2");
};

struct AttnArgs {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  const int32_t* kv_len;
  const uint64_t* anc;
  uint16_t* out;
  float* part_o;     // [units * splits * RW * D]
  float2* part_ml;   // [units * splits * RW]
  int32_t* counters; // [units]
  int32_t* flags;
  int B, N, Hq, Hkv, Lmax, G, M, qgroups, units, splits;
  float scale_log2;
};

__device__ __forceinline__ uint32_t pick_half(uint32_t w, int hi) {
  return hi ? (w >> 16) : (w & 0xffffu);
}

template <class S>
__global__ __launch_bounds__(256) void tree_attn_kernel(AttnArgs a) {
  constexpr int D = S::D, QBW = S::QBW, WQ = S::WQ, KC = S::KC, KT = S::KT, RW = S::RW;
  constexpr int KS = S::KS, VS = S::VS, CPR = S::CPR, KG = S::KG, NQ = S::NQ;
  constexpr int NKS = S::NKS, NDB = S::NDB;
  __shared__ __attribute__((aligned(16))) uint8_t lds_raw[S::LDS_BYTES];
  __shared__ int s_ticket;
  uint16_t* Ks = reinterpret_cast<uint16_t*>(lds_raw);
  uint16_t* Vt = Ks + KT * KS;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wq = wave % WQ;
  const int wk = wave / WQ;
  const int g = lane >> 4;   // lane group: MFMA k-slot group / output row quad
  const int c = lane & 15;   // MFMA row (A) / column (B, C)

  // ---- workgroup -> (unit, split), XCD-aware --------------------------------
  const int w = blockIdx.x;
  const int xcd = w % kNumXCDs;
  const int slot = w / kNumXCDs;
  const int split = slot % a.splits;
  const int unit = (slot / a.splits) * kNumXCDs + xcd;
  if (unit >= a.units) return;
  const int qgroup = unit % a.qgroups;
  const int pair = unit / a.qgroups;
  const int kvh = pair % a.Hkv;
  const int b = pair / a.Hkv;
  const int N = a.N, G = a.G, M = a.M;

  int L = a.kv_len[b];
  const bool bad = L < 0 || L > a.Lmax - N;
  if (bad) {
    L = 0;
    if (a.flags && split == 0 && qgroup == 0 && kvh == 0 && tid == 0)
      atomicOr(a.flags + b, EAGLE_FLAG_BAD_KV_LEN);
  }
  const int total = L + N;
  const int n_tiles = (total + KT - 1) / KT;
  const int t_begin = (int)((long long)split * n_tiles / a.splits);
  const int t_end = (int)((long long)(split + 1) * n_tiles / a.splits);

  const size_t kv_base = ((size_t)b * a.Hkv + kvh) * (size_t)a.Lmax * D;
  const uint16_t* kp = a.k + kv_base;
  const uint16_t* vp = a.v + kv_base;

  // ---- this wave's query rows: Q fragments (MFMA B operand) and tree masks ----
  const int row0 = qgroup * RW + wq * QBW * 16;
  bf16x8 qf[QBW][NKS];
  uint64_t anc_q[QBW];
#pragma unroll
  for (int qb = 0; qb < QBW; ++qb) {
    const int row = row0 + qb * 16 + c;
    if (row < M) {
      const int i = row / G;
      const int h = kvh * G + (row - i * G);
      const uint16_t* qrow = a.q + (((size_t)b * N + i) * a.Hq + h) * D;
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks)
        qf[qb][ks] = *reinterpret_cast<const bf16x8*>(qrow + ks * 32 + g * 8);
      anc_q[qb] = a.anc[(size_t)b * N + i] & (N == 64 ? ~0ull : (1ull << N) - 1ull);
    } else {
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) qf[qb][ks] = bf16x8{};
      anc_q[qb] = 0;
    }
  }

  f32x4 acc[QBW][NDB];
  float m_run[QBW], l_run[QBW];
#pragma unroll
  for (int qb = 0; qb < QBW; ++qb) {
    m_run[qb] = -INFINITY;
    l_run[qb] = 0.f;
#pragma unroll
    for (int db = 0; db < NDB; ++db) acc[qb][db] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  // ---- staging: thread -> (16-byte chunk dc of a key row, key quad kq) -------
  const int dc = tid % CPR;
  const int kq0 = tid / CPR;
  u32x4 kreg[S::PASSES][4], vreg[S::PASSES][4];

  auto load_tile = [&](int t) {
    const int base = t * KT;
#pragma unroll
    for (int p = 0; p < S::PASSES; ++p) {
      const int kq = kq0 + p * KG;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int key = base + 4 * kq + i;
        if (kq < NQ && key < total) {
          const size_t off = (size_t)key * D + dc * 8;
          kreg[p][i] = *reinterpret_cast<const u32x4*>(kp + off);
          vreg[p][i] = *reinterpret_cast<const u32x4*>(vp + off);
        } else {
          kreg[p][i] = u32x4{0, 0, 0, 0};
          vreg[p][i] = u32x4{0, 0, 0, 0};
        }
      }
    }
  };

  auto store_tile = [&]() {
#pragma unroll
    for (int p = 0; p < S::PASSES; ++p) {
      const int kq = kq0 + p * KG;
      if (kq < NQ) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
          *reinterpret_cast<u32x4*>(Ks + (4 * kq + i) * KS + dc * 8) = kreg[p][i];
        // V^T: element (d, key) at row d, key quad kq stored at quad kq ^ (d >> 4).
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const int d = dc * 8 + j;
          const int pq = kq ^ (d >> 4);
          const int wsel = j >> 1, hi = j & 1;
          const uint32_t lo = pick_half(vreg[p][0][wsel], hi) | (pick_half(vreg[p][1][wsel], hi) << 16);
          const uint32_t up = pick_half(vreg[p][2][wsel], hi) | (pick_half(vreg[p][3][wsel], hi) << 16);
          *reinterpret_cast<u32x2*>(Vt + d * VS + pq * 4) = u32x2{lo, up};
        }
      }
    }
  };

  if (t_begin < t_end) load_tile(t_begin);

  for (int t = t_begin; t < t_end; ++t) {
    __syncthreads();  // every wave is done reading the previous tile
    store_tile();
    __syncthreads();
    if (t + 1 < t_end) load_tile(t + 1);  // in flight while this tile is computed

    const int tile_base = t * KT;
    const bool need_mask = tile_base + KT > L;
#pragma unroll
    for (int kc = 0; kc < KC; ++kc) {
      const int chunk = wk * KC + kc;  // 32-key chunk within the tile
      f32x4 s[QBW][2];
#pragma unroll
      for (int qb = 0; qb < QBW; ++qb) s[qb][0] = s[qb][1] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int hlf = 0; hlf < 2; ++hlf) {
        // MFMA row c holds key 8*(c/4) + 4*hlf + c%4, so output row 4g+r is key 8g+4*hlf+r.
        const int krow = chunk * 32 + 8 * (c >> 2) + 4 * hlf + (c & 3);
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) {
          const bf16x8 kf = *reinterpret_cast<const bf16x8*>(Ks + krow * KS + ks * 32 + g * 8);
#pragma unroll
          for (int qb = 0; qb < QBW; ++qb)
            s[qb][hlf] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf, qf[qb][ks], s[qb][hlf], 0, 0, 0);
        }
      }
      // Lane (g, c) now holds scores of query column c for keys chunk*32 + 8g + j, j = 4*hlf + r.
      const int key0 = tile_base + chunk * 32 + 8 * g;
      bf16x8 pf[QBW];
#pragma unroll
      for (int qb = 0; qb < QBW; ++qb) {
        float x[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) x[j] = s[qb][j >> 2][j & 3] * a.scale_log2;
        if (need_mask) {
          // Valid keys among key0..key0+7 as an 8-bit mask, built without branches:
          // committed keys (< L) plus the ancestor bits of this query's node.
          const int below = L - key0;  // how many of the 8 keys are committed
          const uint32_t pre = below >= 8 ? 0xffu : below <= 0 ? 0u : (1u << below) - 1u;
          const int tk0 = -below;      // tree index of key0
          const uint64_t am = anc_q[qb];
          const uint32_t tre = tk0 >= 0 ? (tk0 < 64 ? (uint32_t)(am >> tk0) & 0xffu : 0u)
                                        : (tk0 > -8 ? (uint32_t)(am << -tk0) & 0xffu : 0u);
          const uint32_t ok = pre | tre;
#pragma unroll
          for (int j = 0; j < 8; ++j) x[j] = ((ok >> j) & 1u) ? x[j] : -INFINITY;
        }
        float mx = x[0];
#pragma unroll
        for (int j = 1; j < 8; ++j) mx = fmaxf(mx, x[j]);
        mx = fmaxf(mx, __shfl_xor(mx, 16));
        mx = fmaxf(mx, __shfl_xor(mx, 32));
        const float m_new = fmaxf(m_run[qb], mx);
        const float m_use = m_new == -INFINITY ? 0.f : m_new;
        const float alpha = __builtin_amdgcn_exp2f(m_run[qb] - m_use);
        float psum = 0.f;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const float pj = __builtin_amdgcn_exp2f(x[j] - m_use);
          psum += pj;
          pf[qb][j] = (__bf16)pj;
        }
        l_run[qb] = l_run[qb] * alpha + psum;
        m_run[qb] = m_new;
#pragma unroll
        for (int db = 0; db < NDB; ++db) acc[qb][db] *= alpha;
      }
      // O^T[d, q] += V^T[d, keys] P^T[keys, q]; lane (g, c) supplies d = db*16 + c and
      // keys chunk*32 + 8g .. +7 (quads 2g, 2g+1 of the chunk, swizzled by d >> 4 = db).
#pragma unroll
      for (int db = 0; db < NDB; ++db) {
        const int d = db * 16 + c;
        const int q0 = chunk * 8 + 2 * g;
        const int pq = (q0 ^ db) & ~1;
        bf16x8 vf = *reinterpret_cast<const bf16x8*>(Vt + d * VS + pq * 4);
        if (db & 1) vf = __builtin_shufflevector(vf, vf, 4, 5, 6, 7, 0, 1, 2, 3);
#pragma unroll
        for (int qb = 0; qb < QBW; ++qb)
          acc[qb][db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf, pf[qb], acc[qb][db], 0, 0, 0);
      }
    }
  }

  // ---- per-query totals across the four lanes of a column ---------------------
#pragma unroll
  for (int qb = 0; qb < QBW; ++qb) {
    l_run[qb] += __shfl_xor(l_run[qb], 16);
    l_run[qb] += __shfl_xor(l_run[qb], 32);
  }

  // ---- merge the WK key-waves of each query group through LDS ---------------
  if constexpr (S::WK > 1) {
    __syncthreads();  // tile buffers are free
    float* mb = reinterpret_cast<float*>(lds_raw);
    constexpr int PER_WAVE = QBW * NDB * 256 + QBW * 32;
    if (wk > 0) {
      float* my = mb + wave * PER_WAVE;
#pragma unroll
      for (int qb = 0; qb < QBW; ++qb) {
#pragma unroll
        for (int db = 0; db < NDB; ++db)
          *reinterpret_cast<f32x4*>(my + ((qb * NDB + db) * 64 + lane) * 4) = acc[qb][db];
        if (g == 0) {
          my[QBW * NDB * 256 + qb * 32 + c] = m_run[qb];
          my[QBW * NDB * 256 + qb * 32 + 16 + c] = l_run[qb];
        }
      }
    }
    __syncthreads();
    if (wk == 0) {
#pragma unroll
      for (int qb = 0; qb < QBW; ++qb) {
        float mt = m_run[qb];
#pragma unroll
        for (int o = 1; o < S::WK; ++o)
          mt = fmaxf(mt, mb[(o * WQ + wq) * PER_WAVE + QBW * NDB * 256 + qb * 32 + c]);
        const float mu = mt == -INFINITY ? 0.f : mt;
        const float fs = __builtin_amdgcn_exp2f(m_run[qb] - mu);
        float lt = l_run[qb] * fs;
#pragma unroll
        for (int db = 0; db < NDB; ++db) acc[qb][db] *= fs;
#pragma unroll
        for (int o = 1; o < S::WK; ++o) {
          const float* other = mb + (o * WQ + wq) * PER_WAVE;
          const float fo = __builtin_amdgcn_exp2f(other[QBW * NDB * 256 + qb * 32 + c] - mu);
          lt += other[QBW * NDB * 256 + qb * 32 + 16 + c] * fo;
#pragma unroll
          for (int db = 0; db < NDB; ++db)
            acc[qb][db] += *reinterpret_cast<const f32x4*>(other + ((qb * NDB + db) * 64 + lane) * 4) * fo;
        }
        m_run[qb] = mt;
        l_run[qb] = lt;
      }
    }
  }

  // ---- output ----------------------------------------------------------------
  if (a.splits == 1) {
    if (wk == 0) {
#pragma unroll
      for (int qb = 0; qb < QBW; ++qb) {
        const int row = row0 + qb * 16 + c;
        if (row >= M) continue;
        const int i = row / G;
        const int h = kvh * G + (row - i * G);
        uint16_t* orow = a.out + (((size_t)b * N + i) * a.Hq + h) * D;
        const float inv = bad ? 0.f : 1.f / l_run[qb];
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
          const f32x4 o = acc[qb][db] * inv;
          const uint32_t lo = float_to_bf16_bits(o[0]) | ((uint32_t)float_to_bf16_bits(o[1]) << 16);
          const uint32_t up = float_to_bf16_bits(o[2]) | ((uint32_t)float_to_bf16_bits(o[3]) << 16);
          *reinterpret_cast<u32x2*>(orow + db * 16 + 4 * g) = u32x2{lo, up};
        }
      }
    }
    return;
  }

  const size_t pbase = ((size_t)unit * a.splits + split) * RW;
  if (wk == 0) {
#pragma unroll
    for (int qb = 0; qb < QBW; ++qb) {
      const int rl = wq * QBW * 16 + qb * 16 + c;  // row within the unit
      if (qgroup * RW + rl >= M) continue;
      float* po = a.part_o + (pbase + rl) * D;
#pragma unroll
      for (int db = 0; db < NDB; ++db) *reinterpret_cast<f32x4*>(po + db * 16 + 4 * g) = acc[qb][db];
      if (g == 0) a.part_ml[pbase + rl] = make_float2(m_run[qb], l_run[qb]);
    }
  }
  __threadfence();
  __syncthreads();
  if (tid == 0) s_ticket = atomicAdd(a.counters + unit, 1);
  __syncthreads();
  if (s_ticket != a.splits - 1) return;

  // Last split of this unit: merge all partials.
  __threadfence();
  const int rows = min(RW, M - qgroup * RW);
  const int S_ = a.splits;
  float* wts = reinterpret_cast<float*>(lds_raw);  // [rows][S_] merge weights
  for (int r = tid; r < rows; r += 256) {
    const size_t ub = (size_t)unit * S_ * RW;
    float mt = -INFINITY;
    for (int sp = 0; sp < S_; ++sp) mt = fmaxf(mt, a.part_ml[ub + (size_t)sp * RW + r].x);
    const float mu = mt == -INFINITY ? 0.f : mt;
    float lt = 0.f;
    for (int sp = 0; sp < S_; ++sp) {
      const float2 ml = a.part_ml[ub + (size_t)sp * RW + r];
      const float f = __builtin_amdgcn_exp2f(ml.x - mu);
      wts[r * S_ + sp] = f;
      lt += ml.y * f;
    }
    const float inv = (bad || lt == 0.f) ? 0.f : 1.f / lt;
    for (int sp = 0; sp < S_; ++sp) wts[r * S_ + sp] *= inv;
  }
  __syncthreads();
  constexpr int D4 = D / 4;
  for (int it = tid; it < rows * D4; it += 256) {
    const int r = it / D4;
    const int d4 = it - r * D4;
    f32x4 o = f32x4{0.f, 0.f, 0.f, 0.f};
    for (int sp = 0; sp < S_; ++sp) {
      const f32x4 po = *reinterpret_cast<const f32x4*>(
          a.part_o + (((size_t)unit * S_ + sp) * RW + r) * D + d4 * 4);
      o += po * wts[r * S_ + sp];
    }
    const int row = qgroup * RW + r;
    const int i = row / G;
    const int h = kvh * G + (row - i * G);
    uint16_t* orow = a.out + (((size_t)b * N + i) * a.Hq + h) * D + d4 * 4;
    const uint32_t lo = float_to_bf16_bits(o[0]) | ((uint32_t)float_to_bf16_bits(o[1]) << 16);
    const uint32_t up = float_to_bf16_bits(o[2]) | ((uint32_t)float_to_bf16_bits(o[3]) << 16);
    *reinterpret_cast<u32x2*>(orow) = u32x2{lo, up};
  }
  if (tid == 0) atomicExch(a.counters + unit, 0);
}

// ---- variants ----------------------------------------------------------------
// index: 0 = 1 query block/WG (4 key waves), 1 = 2 blocks (4 key waves),
//        2 = 4 blocks (2x2), 3 = 8 blocks (4 query waves x 2), 4 = 16 blocks (4x4)
struct VariantInfo {
  int rw;
  int kt;
};

static VariantInfo variant_info(int variant, int d) {
  (void)d;
  switch (variant) {
    case 0: return {16, 128};
    case 1: return {32, 128};
    case 2: return {64, 64};
    case 3: return {128, 64};
    default: return {256, 64};
  }
}

template <int D>
static void* variant_kernel(int variant) {
  switch (variant) {
    case 0: return (void*)tree_attn_kernel<AttnShape<D, 1, 1, 1>>;
    case 1: return (void*)tree_attn_kernel<AttnShape<D, 2, 1, 1>>;
    case 2: return (void*)tree_attn_kernel<AttnShape<D, 2, 2, 1>>;
    case 3: return (void*)tree_attn_kernel<AttnShape<D, 2, 4, 2>>;
    default: return (void*)tree_attn_kernel<AttnShape<D, 4, 4, 2>>;
  }
}

static int env_int(const char* name, int dflt) {
  const char* s = getenv(name);
  if (!s || !*s) return dflt;
  return atoi(s);
}

AttnPlan plan_tree_attn(int B, int N, int Hq, int Hkv, int d, int Lmax) {
  AttnPlan p{};
  p.d = d;
  p.G = Hq / Hkv;
  p.M = p.G * N;
  const int nqb = (p.M + 15) / 16;
  int variant = nqb <= 1 ? 0 : nqb <= 2 ? 1 : nqb <= 4 ? 2 : nqb <= 8 ? 3 : 4;
  variant = env_int("EAGLE_ATTN_VARIANT", variant);
  if (variant < 0 || variant > 4) variant = 4;
  const VariantInfo vi = variant_info(variant, d);
  p.variant = variant;
  p.rows_per_wg = vi.rw;
  p.kt = vi.kt;
  p.qgroups = (p.M + vi.rw - 1) / vi.rw;
  p.units = B * Hkv * p.qgroups;
  const int tiles = (Lmax + vi.kt - 1) / vi.kt;
  const int padded_units = ((p.units + kNumXCDs - 1) / kNumXCDs) * kNumXCDs;
  int splits = (2 * kNumCUs + padded_units - 1) / padded_units;
  splits = env_int("EAGLE_ATTN_SPLITS", splits);
  if (splits > tiles) splits = tiles;
  if (splits > 32) splits = 32;  // the merge keeps rows x splits weights in LDS
  if (splits < 1) splits = 1;
  p.splits = splits;
  p.ws_partials = splits > 1 ? (size_t)p.units * splits * vi.rw * (d * 4 + 8) : 0;
  p.ws_counters = splits > 1 ? (size_t)p.units * 4 : 0;
  return p;
}

hipError_t launch_tree_attn(const AttnPlan& plan, const uint16_t* q, const uint16_t* k,
                            const uint16_t* v, const int32_t* kv_len, const uint64_t* anc,
                            int B, int N, int Hq, int Hkv, int Lmax, float scale_log2,
                            uint16_t* out, void* ws, int32_t* flags, hipStream_t s) {
  AttnArgs a{};
  a.q = q;
  a.k = k;
  a.v = v;
  a.kv_len = kv_len;
  a.anc = anc;
  a.out = out;
  uint8_t* w = static_cast<uint8_t*>(ws);
  a.counters = reinterpret_cast<int32_t*>(w);
  const size_t cnt_bytes = (plan.ws_counters + 255) & ~size_t(255);
  a.part_ml = reinterpret_cast<float2*>(w + cnt_bytes);
  const size_t ml_bytes = ((size_t)plan.units * plan.splits * plan.rows_per_wg * 8 + 255) & ~size_t(255);
  a.part_o = reinterpret_cast<float*>(w + cnt_bytes + ml_bytes);
  a.flags = flags;
  a.B = B;
  a.N = N;
  a.Hq = Hq;
  a.Hkv = Hkv;
  a.Lmax = Lmax;
  a.G = plan.G;
  a.M = plan.M;
  a.qgroups = plan.qgroups;
  a.units = plan.units;
  a.splits = plan.splits;
  a.scale_log2 = scale_log2;
  const int padded_units = ((plan.units + kNumXCDs - 1) / kNumXCDs) * kNumXCDs;
  const dim3 grid((unsigned)(padded_units * plan.splits));
  void* fn = plan.d == 64 ? variant_kernel<64>(plan.variant) : variant_kernel<128>(plan.variant);
  void* args[] = {&a};
  return hipLaunchKernel(fn, grid, dim3(256), args, 0, s);
}

size_t tree_attn_workspace_bytes(const AttnPlan& p) {
  if (p.splits <= 1) return 0;
  const size_t cnt_bytes = (p.ws_counters + 255) & ~size_t(255);
  const size_t ml_bytes = ((size_t)p.units * p.splits * p.rows_per_wg * 8 + 255) & ~size_t(255);
  const size_t o_bytes = (size_t)p.units * p.splits * p.rows_per_wg * p.d * 4;
  return cnt_bytes + ml_bytes + o_bytes;
}

}  // namespace eagle
