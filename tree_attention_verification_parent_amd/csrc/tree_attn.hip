// Tree attention for the verification forward on gfx950.
//
// The target verifies the whole draft tree in one forward pass: node i of
// sequence b attends to the committed keys 0..L-1 and to the tree keys L+j of
// its ancestors j (EAGLE, paperlayer.ai summary, §2 Preliminaries; §3 EAGLE:
// tree attention).  This is decode-shaped attention: M = G*N query rows per
// KV head against L+N keys, HBM-bound on the bf16 K/V stream.
//
// Work decomposition
//   unit  = (b, kv head, group of RW query rows); split = a contiguous range of
//   32-key chunks.  One 256-thread workgroup per (unit, split).  Workgroup ids
//   are laid out so that all splits of a unit run on one XCD (blocks go to XCDs
//   round robin), keeping a unit's partials in that XCD's caches.
//
// Two kernels, picked by the number of query rows per KV head:
//   ring  (M <= 32, e.g. multi-head attention): every wave owns a private ring
//         of 32-key chunk slots in LDS, filled by direct-to-LDS loads
//         (global_load_lds_dwordx4) issued ahead, so the whole split is in
//         flight from the start with no staging registers and no barriers in
//         the main loop.  Each wave computes all query rows against its own
//         chunks; the four waves merge at the end.
//   tile  (larger M, grouped-query attention): the 256 threads stage each tile
//         of keys into LDS (K row-major, V transposed) and the waves split the
//         query rows, so one copy of the tile serves all G*N queries.
// Both compute S^T = K Q^T and O^T += V^T P^T with v_mfma_f32_16x16x32_bf16
// (keys on MFMA rows: the K rows are permuted so each lane ends up holding 8
// consecutive keys of one query column, exactly the k-slots of P^T), apply the
// tree mask, and run the online softmax with cross-lane shuffles.
//
// With more than one split, every split writes its normalised rows O / l and
// log2-sum-exp with coalesced stores.  Ring variants combine them in the
// kernel: the unit's last split to finish (a per-unit ticket) reads the other
// splits' partials from the XCD's L2 and writes the output.  Tile variants
// leave them to a small merge kernel on the same stream (one wave per query
// row), whose kernel boundary makes the partials visible.
#include <stdlib.h>

#include "common.h"
#include "launch.h"

namespace eagle {

typedef short short4_t __attribute__((ext_vector_type(4)));

struct AttnArgs {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  const int32_t* kv_len;
  const uint64_t* anc;       // ancestor masks [B, N], or null: built from parents
  const int32_t* parents;    // [B, N] when anc is null
  uint64_t* anc_out;         // optional tree outputs written when built here
  int32_t* depth_out;
  int32_t* pos_out;
  uint16_t* out;
  float* part_o;     // [units * splits * RW * D]  O / l of each split
  float* part_lse;   // [units * splits * RW]      m + log2(l) of each split
  int32_t* flags;
  int32_t* tickets;  // [units] splits finished (ring variants; zero between calls)
  int B, N, Hq, Hkv, Lmax, G, M, qgroups, units, splits;
  float scale_log2;
};

// Swizzle of 16-byte slots within a key row of a 32-key chunk: slot p of row r
// holds the global slot p ^ swz(r).  gfx950's LDS has 64 banks of 4 bytes; a
// 16-byte read serves 16 lanes per cycle, an 8-byte transposed read 32.  The
// K fragment reads of 16 lanes take rows {0-3, 8-11, 16-19, 24-27} (or the
// same + 4) at one global slot: swz is distinct over them.  The transposed V
// reads of 32 lanes take 8 rows {0-3, 8-11} (+4, +16) at two adjacent slots
// each: swz >> 1 is distinct over them.  (D = 64: two rows share a 256-byte
// bank row, so the conditions hold per row parity.)  Measured against the
// earlier 2 (r & 3) + ((r >> 3) & 1), conflict-free only for half as many
// lanes per cycle: bank-conflict cycles 48 % -> 32 % of the LDS-active
// cycles in the grouped-query kernel (llama2-70b shape), 20 % -> 10 % in the
// ring kernel (llama2-7b); the kernels' times did not change.
template <int D>
__device__ __forceinline__ int swz(int r) {
  if constexpr (D == 128)
    return 8 * ((r >> 3) & 1) + 2 * (r & 3) + ((r >> 4) & 1);
  else
    return 4 * ((r >> 3) & 1) + 2 * ((r >> 1) & 1) + ((r >> 4) & 1);
}

__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  return float_to_bf16_bits(a) | ((uint32_t)float_to_bf16_bits(b) << 16);
}

// Online softmax update of one 16-query block from this lane's 8 scores
// (already scaled to the log2 domain and masked).  Returns the bf16 P^T
// fragment.  The running max m_run is shared by the four lanes of a query
// column (the MFMA sums their keys) and is raised lazily: only when some
// lane of the wave sees a score more than LAZY above it does the wave take
// the column max with cross-lane shuffles and rescale its accumulators, so
// in the common case a chunk needs no shuffles and no rescale.  Exponents
// stay below 2^LAZY, far inside fp32 and bf16 range; the result is the same
// softmax whichever reference max is used.
constexpr float LAZY = 8.f;

template <int NDB>
__device__ __forceinline__ bf16x8 softmax_step(const float (&x)[8], float& m_run, float& l_run,
                                               f32x4 (&acc)[NDB]) {
  float mx = x[0];
#pragma unroll
  for (int j = 1; j < 8; ++j) mx = fmaxf(mx, x[j]);
  if (__ballot(mx > m_run + LAZY)) {  // wave-uniform
    mx = fmaxf(mx, __shfl_xor(mx, 16));
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float m_new = fmaxf(m_run, mx);
    if (m_new > m_run) {
      const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);  // 0 when m_run = -inf
      l_run *= alpha;
#pragma unroll
      for (int db = 0; db < NDB; ++db) acc[db] *= alpha;
      m_run = m_new;
    }
  }
  const float m_use = m_run == -INFINITY ? 0.f : m_run;
  float psum = 0.f;
  bf16x8 pf;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const float pj = __builtin_amdgcn_exp2f(x[j] - m_use);
    psum += pj;
    pf[j] = (__bf16)pj;
  }
  l_run += psum;
  return pf;
}

// Valid keys among key0..key0+7 as an 8-bit mask, without branches: committed
// keys (< L) plus the ancestor bits of the query's node.  (A branchy form of
// this test was miscompiled for the first of the eight scores.)
__device__ __forceinline__ uint32_t key_mask8(int key0, int L, uint64_t anc) {
  const int below = L - key0;
  const uint32_t pre = below >= 8 ? 0xffu : below <= 0 ? 0u : (1u << below) - 1u;
  const int tk0 = -below;
  const uint32_t tre = tk0 >= 0 ? (tk0 < 64 ? (uint32_t)(anc >> tk0) & 0xffu : 0u)
                                : (tk0 > -8 ? (uint32_t)(anc << -tk0) & 0xffu : 0u);
  return pre | tre;
}

// Write the final bf16 rows (one split) or this split's partial (O / l and
// log2-sum-exp).  acc/m/l hold the lane's query column for QBW blocks starting
// at row r0 of the unit.
template <int D, int RW, int QBW>
__device__ void finish_split(const AttnArgs& a, int unit, int split, int qgroup, int b, int kvh,
                             bool bad, bool active, int r0, f32x4 (&acc)[QBW][D / 16],
                             float (&m_run)[QBW], float (&l_run)[QBW], uint8_t* lds) {
  constexpr int NDB = D / 16;
  const int tid = threadIdx.x, lane = tid & 63, g = lane >> 4, c = lane & 15;
  const int N = a.N, G = a.G, M = a.M;
  if (a.splits == 1) {
    if (active) {
#pragma unroll
      for (int qb = 0; qb < QBW; ++qb) {
        const int row = qgroup * RW + r0 + qb * 16 + c;
        if (row >= M) continue;
        const int i = row / G;
        const int h = kvh * G + (row - i * G);
        uint16_t* orow = a.out + (((size_t)b * N + i) * a.Hq + h) * D;
        const float inv = (bad || l_run[qb] == 0.f) ? 0.f : 1.f / l_run[qb];
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
          const f32x4 o = acc[qb][db] * inv;
          *reinterpret_cast<u32x2*>(orow + db * 16 + 4 * g) =
              u32x2{pack_bf16x2(o[0], o[1]), pack_bf16x2(o[2], o[3])};
        }
      }
    }
    return;
  }

  // Stage this split's normalised rows in LDS (row-major fp32) so that the
  // partial stores are coalesced 16-byte stores; the merge kernel that
  // follows on the stream combines the splits.
  const int rows = min(RW, M - qgroup * RW);
  float* stage = reinterpret_cast<float*>(lds);  // [RW][D + 4]: column D = log2-sum-exp
  constexpr int SD = D + 4;
  if (active) {
#pragma unroll
    for (int qb = 0; qb < QBW; ++qb) {
      const int rl = r0 + qb * 16 + c;
      const float inv = l_run[qb] == 0.f ? 0.f : 1.f / l_run[qb];
#pragma unroll
      for (int db = 0; db < NDB; ++db)
        *reinterpret_cast<f32x4*>(stage + rl * SD + db * 16 + 4 * g) = acc[qb][db] * inv;
      if (g == 0) stage[rl * SD + D] = l_run[qb] == 0.f ? -INFINITY : m_run[qb] + __log2f(l_run[qb]);
    }
  }
  __syncthreads();
  const size_t pbase = ((size_t)unit * a.splits + split) * RW;
  constexpr int D4 = D / 4;
  for (int it = tid; it < rows * D4; it += 256) {
    const int rl = it / D4, d4 = it - rl * D4;
    *reinterpret_cast<f32x4*>(a.part_o + (pbase + rl) * D + 4 * d4) =
        *reinterpret_cast<const f32x4*>(stage + rl * SD + 4 * d4);
  }
  for (int rl = tid; rl < rows; rl += 256) a.part_lse[pbase + rl] = stage[rl * SD + D];
}

// Workgroup -> (unit, split), XCD-aware; validates kv_len.
struct UnitCtx {
  int unit, split, qgroup, pair, kvh, b, L, total;
  bool bad;
};

__device__ __forceinline__ bool decode_unit(const AttnArgs& a, UnitCtx& u) {
  const int w = blockIdx.x;
  const int xcd = w % kNumXCDs;
  const int slot = w / kNumXCDs;
  u.split = slot % a.splits;
  u.unit = (slot / a.splits) * kNumXCDs + xcd;
  if (u.unit >= a.units) return false;
  u.qgroup = u.unit % a.qgroups;
  u.pair = u.unit / a.qgroups;
  u.kvh = u.pair % a.Hkv;
  u.b = u.pair / a.Hkv;
  int L = a.kv_len[u.b];
  u.bad = L < 0 || L > a.Lmax - a.N;
  if (u.bad) {
    L = 0;
    if (a.flags && u.split == 0 && u.qgroup == 0 && u.kvh == 0 && threadIdx.x == 0)
      atomicOr(a.flags + u.b, EAGLE_FLAG_BAD_KV_LEN);
  }
  u.L = L;
  u.total = L + a.N;
  return true;
}

// The tree-mask builder's outputs (ancestor masks, depths, position ids
// kv_len + depth) of sequence b, written by the one wave per sequence that
// the kernel picks, when the masks were built from the parent links.
__device__ __forceinline__ void write_tree_outputs(const AttnArgs& a, int b, const TreeLinks& t) {
  const int lane = threadIdx.x & 63;
  const size_t o = (size_t)b * a.N + lane;
  if (lane < a.N) {
    if (a.anc_out) a.anc_out[o] = t.anc;
    if (a.depth_out) a.depth_out[o] = t.depth;
    if (a.pos_out) a.pos_out[o] = a.kv_len[b] + t.depth;
  }
  if (__ballot(t.bad) && lane == 0 && a.flags) atomicOr(a.flags + b, EAGLE_FLAG_BAD_PARENT);
}

// Q fragments (MFMA B operand) and tree masks of QBW query blocks at unit row r0.
template <int D, int QBW, int RW>
__device__ __forceinline__ void load_queries(const AttnArgs& a, const UnitCtx& u, int r0,
                                             bf16x8 (&qf)[QBW][D / 32], uint64_t (&anc_q)[QBW]) {
  const int lane = threadIdx.x & 63, g = lane >> 4, c = lane & 15;
  const int N = a.N, G = a.G;
  const uint64_t nmask = N == 64 ? ~0ull : (1ull << N) - 1ull;
  // masks built from the parent links: every wave derives its sequence's
  // tree (lane = node); wave 0 of the unit's last split for KV head 0 and
  // query group 0 writes the builder's outputs
  uint64_t anc_w = 0;
  if (a.parents) {
    const TreeLinks t = tree_links_wave(a.parents + (size_t)u.b * N, N);
    anc_w = t.anc;
    if (u.kvh == 0 && u.qgroup == 0 && u.split == a.splits - 1 && threadIdx.x < 64)
      write_tree_outputs(a, u.b, t);
  }
#pragma unroll
  for (int qb = 0; qb < QBW; ++qb) {
    const int row = u.qgroup * RW + r0 + qb * 16 + c;
    const uint64_t built = a.parents ? __shfl(anc_w, row < a.M ? row / G : 0) : 0ull;
    if (row < a.M) {
      const int i = row / G;
      const int h = u.kvh * G + (row - i * G);
      const uint16_t* qrow = a.q + (((size_t)u.b * N + i) * a.Hq + h) * D;
#pragma unroll
      for (int ks = 0; ks < D / 32; ++ks)
        qf[qb][ks] = *reinterpret_cast<const bf16x8*>(qrow + ks * 32 + g * 8);
      anc_q[qb] = (a.parents ? built : a.anc[(size_t)u.b * N + i]) & nmask;
    } else {
#pragma unroll
      for (int ks = 0; ks < D / 32; ++ks) qf[qb][ks] = bf16x8{};
      anc_q[qb] = 0;
    }
  }
}

// Merge the states of the waves that hold the same query rows (o-th such wave
// at index base + o * stride), into wave 0 of the group, through LDS.
template <int QBW, int NDB, int NW>
__device__ __forceinline__ void merge_waves(f32x4 (&acc)[QBW][NDB], float (&m_run)[QBW],
                                            float (&l_run)[QBW], float* mb, int me, int first,
                                            int stride) {
  constexpr int PER_WAVE = QBW * NDB * 256 + QBW * 32;
  const int lane = threadIdx.x & 63, g = lane >> 4, c = lane & 15;
  __syncthreads();
  if (me != first) {
    float* my = mb + me * PER_WAVE;
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
  if (me == first) {
#pragma unroll
    for (int qb = 0; qb < QBW; ++qb) {
      float mt = m_run[qb];
#pragma unroll
      for (int o = 1; o < NW; ++o)
        mt = fmaxf(mt, mb[(first + o * stride) * PER_WAVE + QBW * NDB * 256 + qb * 32 + c]);
      const float mu = mt == -INFINITY ? 0.f : mt;
      const float fs = __builtin_amdgcn_exp2f(m_run[qb] - mu);
      float lt = l_run[qb] * fs;
#pragma unroll
      for (int db = 0; db < NDB; ++db) acc[qb][db] *= fs;
#pragma unroll
      for (int o = 1; o < NW; ++o) {
        const float* other = mb + (first + o * stride) * PER_WAVE;
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
  __syncthreads();  // the merge buffers may now be reused
}

// ============================================================================
// ring kernel: committed prefix only, one direct-to-LDS chunk slot per wave
// ============================================================================
// Eight waves, each with one 32-key K/V slot in LDS.  The chunks of a split
// are dealt to them round robin; a wave waits for its chunk, computes it and
// refills the slot with its next chunk, while the other seven keep theirs in
// flight (two waves per SIMD hide each other's MFMA and softmax latency).
// The split ranges are laid over the cache capacity Lmax - N, not over
// kv_len, so the first loads go out before anything else is read; keys at or
// past kv_len are masked.  The tree keys (each query's ancestors and itself,
// N <= 64 of them) are one or two more chunks, masked by the ancestor bits,
// for one wave of the last split.
//
// A workgroup holds RW query rows.  With more rows per KV head (grouped-query
// attention, G*N > RW) the rows are cut into query groups, each a unit of its
// own that streams the same K/V; those units sit on one XCD so that the
// repeats come from its L2, and their loads use the default cache policy
// instead of the non-temporal one.
constexpr int kRingThreads = 64 * 8;
constexpr int kNonTemporal = 2;  // cache-policy bits of a load: nt

// One lane's 16-byte direct-to-LDS load; the cache policy is a literal in
// each branch (a template-dependent policy argument made hipcc drop the
// kernel instantiations without a diagnostic).
template <int POLICY>
__device__ __forceinline__ void load_lds16(const uint16_t* src, uint8_t* dst) {
  if constexpr (POLICY == kNonTemporal)
    __builtin_amdgcn_global_load_lds(src, (__attribute__((address_space(3))) void*)dst, 16, 0, kNonTemporal);
  else
    __builtin_amdgcn_global_load_lds(src, (__attribute__((address_space(3))) void*)dst, 16, 0, 0);
}

template <int D_, int QBW_, int POLICY_ = kNonTemporal>
struct RingShape {
  static constexpr int D = D_;
  static constexpr int QBW = QBW_;
  static constexpr int POLICY = POLICY_;  // cache-policy bits of the K/V loads
  static constexpr int NWAVE = 8;
  static constexpr int THREADS = 64 * NWAVE;
  static constexpr int MAT_BYTES = 32 * D * 2;    // K (or V) of one 32-key chunk
  static constexpr int SLOT_BYTES = 2 * MAT_BYTES;
  static constexpr int SPR = D / 8;               // 16-byte slots per key row
  static constexpr int RPL = 64 / SPR;            // key rows per wave-wide direct load
  static constexpr int LPM = 32 / RPL;            // direct loads per matrix
  static constexpr int NKS = D / 32, NDB = D / 16;
  static constexpr int RW = 16 * QBW;
  static constexpr int ACC_BYTES = QBW * NDB * 256 * 4;  // one wave's accumulators
  static_assert(ACC_BYTES <= SLOT_BYTES, "a wave's state is parked in its own slot");
  static constexpr int LDS_RING = NWAVE * SLOT_BYTES;
  static constexpr int LDS_ML = NWAVE * QBW * 32 * 4;   // each wave's m and l
  static constexpr int LDS_BYTES = LDS_RING + LDS_ML;
};

// The NWAVE waves' online-softmax states for the same query rows combined in
// one round: every wave parks its accumulators (rows below `rows` only) in its
// own (now idle) slot and its m, l beside the ring; after one barrier the
// waves share out the (query block, d block) tiles of the result, each
// combining all NWAVE states of its tiles, and hand every normalised tile
// straight from registers to emit(row, d block, O / l, log2-sum-exp).
template <int QBW, int NDB, int NWAVE, int SLOT_BYTES, typename Emit>
__device__ __forceinline__ void fold_waves(const f32x4 (&acc)[QBW][NDB], const float (&m_run)[QBW],
                                           const float (&l_run)[QBW], uint8_t* lds, float* ml,
                                           int wave, int rows, Emit&& emit) {
  const int lane = threadIdx.x & 63, g = lane >> 4, c = lane & 15;
  float* mine = reinterpret_cast<float*>(lds + wave * SLOT_BYTES);
#pragma unroll
  for (int qb = 0; qb < QBW; ++qb) {
    if (qb * 16 + c >= rows) continue;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
      *reinterpret_cast<f32x4*>(mine + ((qb * NDB + db) * 64 + lane) * 4) = acc[qb][db];
    if (g == 0) {
      ml[(wave * QBW + qb) * 32 + c] = m_run[qb];
      ml[(wave * QBW + qb) * 32 + 16 + c] = l_run[qb];
    }
  }
  __syncthreads();
  for (int it = wave; it < QBW * NDB; it += NWAVE) {
    const int qb = it / NDB, db = it - qb * NDB;
    const int rl = qb * 16 + c;
    if (rl >= rows) continue;
    float ms[NWAVE], mt = -INFINITY;
#pragma unroll
    for (int w = 0; w < NWAVE; ++w) {
      ms[w] = ml[(w * QBW + qb) * 32 + c];
      mt = fmaxf(mt, ms[w]);
    }
    const float mu = mt == -INFINITY ? 0.f : mt;
    float lt = 0.f;
    f32x4 o = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int w = 0; w < NWAVE; ++w) {
      const float f = __builtin_amdgcn_exp2f(ms[w] - mu);
      lt += ml[(w * QBW + qb) * 32 + 16 + c] * f;
      o += *reinterpret_cast<const f32x4*>(reinterpret_cast<const float*>(lds + w * SLOT_BYTES) +
                                           ((qb * NDB + db) * 64 + lane) * 4) * f;
    }
    const float inv = lt == 0.f ? 0.f : 1.f / lt;
    emit(rl, db, o * inv, lt == 0.f ? -INFINITY : mt + __log2f(lt));
  }
}

// A wave-uniform 32-bit value read with a scalar load (constant address
// space), which the compiler tracks apart from the vector loads in flight.
__device__ __forceinline__ int32_t load_uniform(const int32_t* p) {
  return *(const __attribute__((address_space(4))) int32_t*)p;
}

// Valid committed keys among key0..key0+7 (keys below L) as an 8-bit mask.
__device__ __forceinline__ uint32_t prefix_mask8(int key0, int L) {
  const int below = L - key0;
  return below >= 8 ? 0xffu : below <= 0 ? 0u : (1u << below) - 1u;
}

// One 32-key chunk in LDS: K then V, 32 rows of D bf16 each, the 16-byte
// slots of row r permuted by swz(r).  The chunk is computed in three parts
// (so that a caller can overlap one chunk's softmax with another's MFMAs):
//   chunk_qk:   S^T = K Q^T for QBW 16-row query blocks (keys on MFMA rows,
//               permuted so lane (g, c) holds keys 8g..8g+7 of column c);
//   chunk_soft: the tree or prefix mask and the online softmax, giving the
//               bf16 P^T fragments (a tree chunk admits key 8g + j of the
//               lane's column when ancestor bit tree_bit0 + 8g + j of its
//               row's node is set, a prefix chunk by the 8-bit ok_prefix);
//   chunk_pv:   O^T += V^T P^T with V^T fragments from transposed LDS reads.
template <int D, int QBW>
__device__ __forceinline__ void chunk_qk(const uint8_t* slot, const bf16x8 (&qf)[QBW][D / 32],
                                         f32x4 (&sc)[QBW][2]) {
  constexpr int NKS = D / 32;
  const int lane = threadIdx.x & 63, g = lane >> 4, c = lane & 15;
  const uint16_t* Kc = reinterpret_cast<const uint16_t*>(slot);
#pragma unroll
  for (int qb = 0; qb < QBW; ++qb) sc[qb][0] = sc[qb][1] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int hlf = 0; hlf < 2; ++hlf) {
    // MFMA row c holds key 8*(c/4) + 4*hlf + c%4, so output row 4g+r is key 8g+4*hlf+r.
    const int kr = 8 * (c >> 2) + 4 * hlf + (c & 3);
    const int sw = swz<D>(kr);
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
      const bf16x8 kf = *reinterpret_cast<const bf16x8*>(Kc + kr * D + (((ks * 4 + g) ^ sw) * 8));
#pragma unroll
      for (int qb = 0; qb < QBW; ++qb)
        sc[qb][hlf] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf, qf[qb][ks], sc[qb][hlf], 0, 0, 0);
    }
  }
}

template <int D, int QBW>
__device__ __forceinline__ void chunk_soft(const f32x4 (&sc)[QBW][2], const uint64_t (&anc_q)[QBW],
                                           f32x4 (&acc)[QBW][D / 16], float (&m_run)[QBW],
                                           float (&l_run)[QBW], bf16x8 (&pf)[QBW], float scale_log2,
                                           bool need_mask, bool tree_chunk, int tree_bit0,
                                           uint32_t ok_prefix) {
  const int g = (threadIdx.x & 63) >> 4;
#pragma unroll
  for (int qb = 0; qb < QBW; ++qb) {
    float x[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) x[j] = sc[qb][j >> 2][j & 3] * scale_log2;
    if (need_mask) {
      const uint32_t ok =
          tree_chunk ? (uint32_t)(anc_q[qb] >> (tree_bit0 + 8 * g)) & 0xffu : ok_prefix;
#pragma unroll
      for (int j = 0; j < 8; ++j) x[j] = ((ok >> j) & 1u) ? x[j] : -INFINITY;
    }
    pf[qb] = softmax_step<D / 16>(x, m_run[qb], l_run[qb], acc[qb]);
  }
}

template <int D, int QBW>
__device__ __forceinline__ void chunk_pv(const uint8_t* slot, const bf16x8 (&pf)[QBW],
                                         f32x4 (&acc)[QBW][D / 16]) {
  constexpr int NDB = D / 16, MAT_BYTES = 32 * D * 2;
  const int lane = threadIdx.x & 63, g = lane >> 4, c = lane & 15;
  const uint8_t* Vb = slot + MAT_BYTES;
  // V^T fragments by transposed LDS reads: lane (g, c) gets V[8g + j][16db + c],
  // j = 0..7, as two 4-element halves.
#pragma unroll
  for (int db = 0; db < NDB; ++db) {
    short4_t h2[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int vr = 8 * g + 4 * h + (c >> 2);
      const int ps = (2 * db + ((c & 3) >> 1)) ^ swz<D>(vr);
      const uint8_t* src = Vb + vr * D * 2 + ps * 16 + (c & 1) * 8;
      h2[h] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (__attribute__((address_space(3))) short4_t*)(src));
    }
    const bf16x8 vf =
        __builtin_bit_cast(bf16x8, __builtin_shufflevector(h2[0], h2[1], 0, 1, 2, 3, 4, 5, 6, 7));
#pragma unroll
    for (int qb = 0; qb < QBW; ++qb)
      acc[qb][db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf, pf[qb], acc[qb][db], 0, 0, 0);
  }
}

// The three parts of one chunk in order.
template <int D, int QBW>
__device__ __forceinline__ void chunk_step(const uint8_t* slot, const bf16x8 (&qf)[QBW][D / 32],
                                           const uint64_t (&anc_q)[QBW], f32x4 (&acc)[QBW][D / 16],
                                           float (&m_run)[QBW], float (&l_run)[QBW],
                                           float scale_log2, bool need_mask, bool tree_chunk,
                                           int tree_bit0, uint32_t ok_prefix) {
  f32x4 sc[QBW][2];
  bf16x8 pf[QBW];
  chunk_qk<D, QBW>(slot, qf, sc);
  chunk_soft<D, QBW>(sc, anc_q, acc, m_run, l_run, pf, scale_log2, need_mask, tree_chunk,
                     tree_bit0, ok_prefix);
  chunk_pv<D, QBW>(slot, pf, acc);
}

template <class S>
__global__ __launch_bounds__(S::THREADS) void tree_attn_ring_kernel(AttnArgs a) {
  constexpr int D = S::D, QBW = S::QBW, RW = S::RW, NKS = S::NKS, NDB = S::NDB;
  constexpr int SPR = S::SPR, RPL = S::RPL, LPM = S::LPM, NWAVE = S::NWAVE;
  __shared__ __attribute__((aligned(16))) uint8_t lds[S::LDS_BYTES];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 4, c = lane & 15;

  // workgroup -> (unit, split): all splits of a unit on one XCD
  const int xcd = blockIdx.x % kNumXCDs, slotw = blockIdx.x / kNumXCDs;
  const int split = slotw % a.splits;
  const int unit = (slotw / a.splits) * kNumXCDs + xcd;
  if (unit >= a.units) return;
  // unit -> (pair = b * Hkv + kvh, query group of RW rows).  The query groups
  // of a pair are consecutive units of one XCD, so they are resident together
  // and stream the same K/V through that XCD's L2 (read from HBM about once).
  const int ux = unit / kNumXCDs;
  const int qgroup = ux % a.qgroups;
  const int pair = (ux / a.qgroups) * kNumXCDs + xcd;
  if (pair >= a.B * a.Hkv) return;
  const int kvh = pair % a.Hkv;
  const int b = pair / a.Hkv;
  const int row0 = qgroup * RW;  // first query row (of the pair's G*N) of this unit

  // this split's chunks of the capacity prefix; wave w takes cb + w, cb + w + NWAVE, ...
  const int Lp = a.Lmax - a.N;
  const int n_chunks = (Lp + 31) / 32;
  const int cb = (int)((long long)split * n_chunks / a.splits);
  const int ce = (int)((long long)(split + 1) * n_chunks / a.splits);
  const int my_first = cb + wave;
  const int my_n = my_first < ce ? (ce - my_first + NWAVE - 1) / NWAVE : 0;

  const size_t kv_base = ((size_t)b * a.Hkv + kvh) * (size_t)a.Lmax * D;
  const uint16_t* kp = a.k + kv_base;
  const uint16_t* vp = a.v + kv_base;
  uint8_t* slot = lds + wave * S::SLOT_BYTES;

  // Direct-to-LDS fill of 32 keys from key0: lane l writes 16 bytes at load
  // base + 16 l, i.e. row t*RPL + l/SPR, slot l%SPR, which receives global
  // slot (l%SPR)^swz(row).  Rows past key_max re-read it (finite data, masked
  // later).  The stream is read once: non-temporal loads (nt) keep it from
  // evicting the split partials that the unit's last split reads back from
  // this XCD's L2 (the stream per XCD is about the size of its L2).
  const int r_in = lane / SPR, p_in = lane % SPR;
  auto issue_keys = [&](int key0, int key_max) {
#pragma unroll
    for (int t = 0; t < LPM; ++t) {
      const int r = t * RPL + r_in;
      const int key = min(key0 + r, key_max);
      const size_t off = (size_t)key * D + (p_in ^ swz<D>(r)) * 8;
      load_lds16<S::POLICY>(kp + off, slot + t * RPL * D * 2);
    }
#pragma unroll
    for (int t = 0; t < LPM; ++t) {
      const int r = t * RPL + r_in;
      const int key = min(key0 + r, key_max);
      const size_t off = (size_t)key * D + (p_in ^ swz<D>(r)) * 8;
      load_lds16<S::POLICY>(vp + off, slot + S::MAT_BYTES + t * RPL * D * 2);
    }
  };
  auto issue = [&](int gc) { issue_keys(gc * 32, Lp - 1); };
  if (my_n > 0) issue(my_first);
  // The tree keys [L, L + N) are one or two more masked chunks (N <= 64),
  // taken by the wave of the last split with the fewest prefix chunks.
  const bool tree_wave = split == a.splits - 1 && wave == (ce - cb) % NWAVE;

  // A wave with three or more chunks loads its second one into registers
  // right away, so that it is in flight with the first instead of requested
  // once the first has been computed (the slot is busy until then); it is
  // written to the slot in the layout a direct-to-LDS load gives.  (Measured
  // on MI355X: llama2-13b shape, ~5 chunks per wave, 60.9 us against 62.7;
  // with only two chunks, as at the llama2-7b shape, waiting for both before
  // the first is computed costs more than it saves: 15.2 us against 14.2.)
  const int my_chunks = my_n + (tree_wave ? (a.N + 31) / 32 : 0);
  const bool pre2 = my_chunks >= 3;  // wave-uniform
  u32x4 pre[2 * LPM];
  auto load_pre = [&](int key0, int key_max) {
#pragma unroll
    for (int t = 0; t < LPM; ++t) {
      const int r = t * RPL + r_in;
      const size_t off = (size_t)min(key0 + r, key_max) * D + (p_in ^ swz<D>(r)) * 8;
      pre[t] = *reinterpret_cast<const u32x4*>(kp + off);
      pre[LPM + t] = *reinterpret_cast<const u32x4*>(vp + off);
    }
  };
  if (pre2 && 1 < my_n) load_pre((my_first + NWAVE) * 32, Lp - 1);

  // committed length (a scalar load: waiting for it does not wait for the
  // chunks' vector loads), then the queries, needed once the first chunk is in
  int L = load_uniform(a.kv_len + b);
  const bool bad = L < 0 || L > Lp;
  if (bad) {
    L = 0;
    if (a.flags && split == 0 && kvh == 0 && qgroup == 0 && tid == 0)
      atomicOr(a.flags + b, EAGLE_FLAG_BAD_KV_LEN);
  }
  if (tree_wave && my_n == 0) issue_keys(L, L + a.N - 1);
  if (pre2 && my_n <= 1) load_pre(L + 32 * (1 - my_n), L + a.N - 1);  // a tree chunk second
  // the tree wave's rows' ancestor masks: bit t of anc[row] admits key L + t
  uint64_t anc_q[QBW];
  if (tree_wave) {
    const uint64_t nmask = a.N == 64 ? ~0ull : (1ull << a.N) - 1ull;
    if (a.parents) {
      // masks built here from the parent links (lane = node); the tree wave
      // of KV head 0 also writes the builder's outputs
      const TreeLinks t = tree_links_wave(a.parents + (size_t)b * a.N, a.N);
#pragma unroll
      for (int qb = 0; qb < QBW; ++qb) {
        const int row = row0 + qb * 16 + c;
        const uint64_t m = __shfl(t.anc, row < a.M ? row / a.G : 0);
        anc_q[qb] = row < a.M ? m & nmask : 0ull;
      }
      if (kvh == 0 && qgroup == 0) write_tree_outputs(a, b, t);
    } else {
#pragma unroll
      for (int qb = 0; qb < QBW; ++qb) {
        const int row = row0 + qb * 16 + c;
        anc_q[qb] = row < a.M ? a.anc[(size_t)b * a.N + row / a.G] & nmask : 0ull;
      }
    }
  }
  const int rows = min(RW, a.M - row0);
  bf16x8 qf[QBW][NKS];
#pragma unroll
  for (int qb = 0; qb < QBW; ++qb) {
    const int row = row0 + qb * 16 + c;
    if (row < a.M) {
      const int i = row / a.G;
      const int h = kvh * a.G + (row - i * a.G);
      const uint16_t* qrow = a.q + (((size_t)b * a.N + i) * a.Hq + h) * D;
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks)
        qf[qb][ks] = *reinterpret_cast<const bf16x8*>(qrow + ks * 32 + g * 8);
    } else {
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) qf[qb][ks] = bf16x8{};
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

  for (int i = 0; i < my_chunks; ++i) {
    const bool tree_chunk = i >= my_n;
    const int tree_bit0 = 32 * (i - my_n);  // anc bit of the tree chunk's first key
    const int gc = my_first + NWAVE * i;
    if (i == 1 && pre2) {
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // the first chunk's reads are done
#pragma unroll
      for (int t = 0; t < LPM; ++t) {
        *reinterpret_cast<u32x4*>(slot + t * RPL * D * 2 + lane * 16) = pre[t];
        *reinterpret_cast<u32x4*>(slot + S::MAT_BYTES + t * RPL * D * 2 + lane * 16) = pre[LPM + t];
      }
    } else {
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // this wave's chunk has landed
    }
    const bool need_mask = tree_chunk || gc * 32 + 32 > L;
    chunk_step<D, QBW>(slot, qf, anc_q, acc, m_run, l_run, a.scale_log2, need_mask, tree_chunk,
                       tree_bit0, prefix_mask8(gc * 32 + 8 * g, L));
    if (i + 1 < my_chunks && !(i == 0 && pre2)) {
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // this slot's reads are done
      if (i + 1 < my_n)
        issue(gc + NWAVE);
      else
        issue_keys(L + 32 * (i + 1 - my_n), L + a.N - 1);
    }
  }

#pragma unroll
  for (int qb = 0; qb < QBW; ++qb) {
    l_run[qb] += __shfl_xor(l_run[qb], 16);
    l_run[qb] += __shfl_xor(l_run[qb], 32);
  }
  // the folded rows go from registers to the output (one split) or to this
  // split's partial (O / l and log2-sum-exp)
  float* ml = reinterpret_cast<float*>(lds + S::LDS_RING);
  constexpr int D4 = D / 4;
  auto out_row = [&](int rl) {
    const int row = row0 + rl;
    const int i = row / a.G;
    const int h = kvh * a.G + (row - i * a.G);
    return a.out + (((size_t)b * a.N + i) * a.Hq + h) * D;
  };
  if (a.splits == 1) {
    fold_waves<QBW, NDB, NWAVE, S::SLOT_BYTES>(
        acc, m_run, l_run, lds, ml, wave, rows, [&](int rl, int db, f32x4 o, float) {
          if (bad) o = f32x4{0.f, 0.f, 0.f, 0.f};
          *reinterpret_cast<u32x2*>(out_row(rl) + db * 16 + 4 * g) =
              u32x2{pack_bf16x2(o[0], o[1]), pack_bf16x2(o[2], o[3])};
        });
    return;
  }
  const size_t pbase = ((size_t)unit * a.splits + split) * RW;
  fold_waves<QBW, NDB, NWAVE, S::SLOT_BYTES>(
      acc, m_run, l_run, lds, ml, wave, rows, [&](int rl, int db, f32x4 o, float lse) {
        *reinterpret_cast<f32x4*>(a.part_o + (pbase + rl) * D + db * 16 + 4 * g) = o;
        if (db == 0 && g == 0) a.part_lse[pbase + rl] = lse;
      });

  // The unit's last split to finish combines the partials.  All splits of a
  // unit run on one XCD, so its L2 is where they meet: each workgroup's
  // stores have reached it (vmcnt) before the workgroup takes its ticket,
  // and the combining workgroup's loads miss its own L1, which held none of
  // these lines since the kernel started.
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  int* last = reinterpret_cast<int*>(ml);
  if (tid == 0) {
    const int done = __hip_atomic_fetch_add(a.tickets + unit, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    *last = done == a.splits - 1;
    if (done == a.splits - 1) __hip_atomic_store(a.tickets + unit, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  __syncthreads();
  if (!*last) return;
  // (row, 4 columns) items: w_s = 2^(lse_s - max), o = sum w_s O_s / sum w_s.
  // The splits go in batches of 8, and a thread's two items share a batch,
  // so that every load of a batch is issued before any is used.
  const size_t ub = (size_t)unit * a.splits * RW;
  const int total = rows * D4;
  for (int it0 = tid; it0 < total; it0 += 2 * S::THREADS) {
    const int its[2] = {it0, it0 + S::THREADS};
    float mt[2] = {-INFINITY, -INFINITY}, lt[2] = {0.f, 0.f};
    f32x4 o[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
    for (int s0 = 0; s0 < a.splits; s0 += 8) {
      float ls[2][8];
      f32x4 os[2][8];
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int it = its[u] < total ? its[u] : it0;  // a duplicate item is never stored
        const int rl = it / D4, d4 = it - rl * D4;
#pragma unroll
        for (int q = 0; q < 8; ++q) {
          const bool in = s0 + q < a.splits;
          const size_t r = ub + (size_t)(in ? s0 + q : 0) * RW + rl;  // in range either way
          ls[u][q] = in ? a.part_lse[r] : -INFINITY;
          os[u][q] = in ? *reinterpret_cast<const f32x4*>(a.part_o + r * D + 4 * d4)
                        : f32x4{0.f, 0.f, 0.f, 0.f};
        }
      }
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        float mb = mt[u];
#pragma unroll
        for (int q = 0; q < 8; ++q) mb = fmaxf(mb, ls[u][q]);
        if (mb == -INFINITY) continue;
        const float f = mt[u] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(mt[u] - mb);
        lt[u] *= f;
        o[u] *= f;
#pragma unroll
        for (int q = 0; q < 8; ++q) {
          const float w = ls[u][q] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(ls[u][q] - mb);
          lt[u] += w;
          o[u] += os[u][q] * w;
        }
        mt[u] = mb;
      }
    }
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      if (its[u] >= total) continue;
      const int rl = its[u] / D4, d4 = its[u] - rl * D4;
      const float inv = (bad || lt[u] == 0.f) ? 0.f : 1.f / lt[u];
      *reinterpret_cast<u32x2*>(out_row(rl) + 4 * d4) =
          u32x2{pack_bf16x2(o[u][0] * inv, o[u][1] * inv), pack_bf16x2(o[u][2] * inv, o[u][3] * inv)};
    }
  }
}

// ============================================================================
// tile kernel: shared LDS tiles, waves split the query rows (grouped queries)
// ============================================================================
template <int D_, int QBW_, int WQ_, int KC_>
struct TileShape {
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
  static constexpr int NKS = D / 32;
  static constexpr int NDB = D / 16;
  static constexpr int LDS_TILE = (KT * KS + D * VS) * 2;
  static constexpr int LDS_MERGE = WK > 1 ? 4 * (QBW * NDB * 256 + QBW * 32) * 4 : 0;
  static constexpr int LDS_STAGE = RW * (D + 4) * 4;
  static constexpr int LDS_A = LDS_TILE > LDS_MERGE ? LDS_TILE : LDS_MERGE;
  static constexpr int LDS_BYTES = LDS_A > LDS_STAGE ? LDS_A : LDS_STAGE;
  static_assert(NQ >= 8 && (NQ & (NQ - 1)) == 0, "V^T swizzle needs >= 8 key quads, power of 2");
};

__device__ __forceinline__ uint32_t pick_half(uint32_t w, int hi) {
  return hi ? (w >> 16) : (w & 0xffffu);
}

template <class S>
__global__ __launch_bounds__(256) void tree_attn_tile_kernel(AttnArgs a) {
  constexpr int D = S::D, QBW = S::QBW, WQ = S::WQ, KC = S::KC, KT = S::KT, RW = S::RW;
  constexpr int KS = S::KS, VS = S::VS, CPR = S::CPR, KG = S::KG, NQ = S::NQ;
  constexpr int NKS = S::NKS, NDB = S::NDB;
  __shared__ __attribute__((aligned(16))) uint8_t lds_raw[S::LDS_BYTES];
  uint16_t* Ks = reinterpret_cast<uint16_t*>(lds_raw);
  uint16_t* Vt = Ks + KT * KS;

  UnitCtx u;
  if (!decode_unit(a, u)) return;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wq = wave % WQ;
  const int wk = wave / WQ;
  const int g = lane >> 4;
  const int c = lane & 15;
  const int L = u.L, total = u.total;
  const int n_tiles = (total + KT - 1) / KT;
  const int t_begin = (int)((long long)u.split * n_tiles / a.splits);
  const int t_end = (int)((long long)(u.split + 1) * n_tiles / a.splits);

  const size_t kv_base = ((size_t)u.b * a.Hkv + u.kvh) * (size_t)a.Lmax * D;
  const uint16_t* kp = a.k + kv_base;
  const uint16_t* vp = a.v + kv_base;

  const int r0 = wq * QBW * 16;
  bf16x8 qf[QBW][NKS];
  uint64_t anc_q[QBW];
  load_queries<D, QBW, RW>(a, u, r0, qf, anc_q);

  f32x4 acc[QBW][NDB];
  float m_run[QBW], l_run[QBW];
#pragma unroll
  for (int qb = 0; qb < QBW; ++qb) {
    m_run[qb] = -INFINITY;
    l_run[qb] = 0.f;
#pragma unroll
    for (int db = 0; db < NDB; ++db) acc[qb][db] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  // staging: thread -> (16-byte chunk dc of a key row, key quad kq)
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
      const int chunk = wk * KC + kc;
      f32x4 s[QBW][2];
#pragma unroll
      for (int qb = 0; qb < QBW; ++qb) s[qb][0] = s[qb][1] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int hlf = 0; hlf < 2; ++hlf) {
        const int krow = chunk * 32 + 8 * (c >> 2) + 4 * hlf + (c & 3);
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) {
          const bf16x8 kf = *reinterpret_cast<const bf16x8*>(Ks + krow * KS + ks * 32 + g * 8);
#pragma unroll
          for (int qb = 0; qb < QBW; ++qb)
            s[qb][hlf] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf, qf[qb][ks], s[qb][hlf], 0, 0, 0);
        }
      }
      const int key0 = tile_base + chunk * 32 + 8 * g;
      bf16x8 pf[QBW];
#pragma unroll
      for (int qb = 0; qb < QBW; ++qb) {
        float x[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) x[j] = s[qb][j >> 2][j & 3] * a.scale_log2;
        if (need_mask) {
          const uint32_t ok = key_mask8(key0, L, anc_q[qb]);
#pragma unroll
          for (int j = 0; j < 8; ++j) x[j] = ((ok >> j) & 1u) ? x[j] : -INFINITY;
        }
        pf[qb] = softmax_step<NDB>(x, m_run[qb], l_run[qb], acc[qb]);
      }
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

#pragma unroll
  for (int qb = 0; qb < QBW; ++qb) {
    l_run[qb] += __shfl_xor(l_run[qb], 16);
    l_run[qb] += __shfl_xor(l_run[qb], 32);
  }
  if constexpr (S::WK > 1) {
    merge_waves<QBW, NDB, S::WK>(acc, m_run, l_run, reinterpret_cast<float*>(lds_raw), wave, wq, WQ);
  } else {
    __syncthreads();  // tile buffers may be reused for the split weights
  }
  finish_split<D, RW, QBW>(a, u.unit, u.split, u.qgroup, u.b, u.kvh, u.bad, wk == 0, r0, acc,
                           m_run, l_run, lds_raw);
}

// ============================================================================
// group kernel: a head group's query rows share a ring of K/V tiles in LDS
// ============================================================================
// Grouped-query attention with up to 256 query rows per (b, KV head): eight
// waves, each owning 32 of the rows, compute every 64-key tile of the split
// against their own rows, so a tile is read from HBM once for the whole
// head group and no wave has to merge with another.  The tiles stream
// through NBUF LDS buffers, NBUF - 1 of them in flight while one is
// computed; each wave issues a quarter of every tile's direct-to-LDS loads.
// Those loads are inline assembly: the compiler treats a direct-to-LDS load
// of its own as a pending LDS write that every later LDS read waits for,
// which would drain all buffers before each tile.  Their completion is
// tracked here instead: before tile i a wave waits until at most its own
// loads of the tiles after i are outstanding (vector loads complete in
// order), and one LDS-only barrier then makes tile i whole for all waves and
// frees the buffer of tile i - 1 for tile i + NBUF - 1.  The last split
// also computes the tree keys [L, L + N) as one more tile.  Rows O / l and
// log2-sum-exp of a split go straight from registers to the partials (the
// merge kernel combines splits: the unit's last split combining them, as the
// ring kernel does, took longer, 63 against 59 us at the llama2-70b shape,
// one workgroup reading 4 x 208 rows), or the bf16 rows to the output.
template <int D_>
struct GroupShape {
  static constexpr int D = D_;
  static constexpr int QBW = 2;                        // 16-row query blocks per wave
  static constexpr int NWAVE = 8;
  static constexpr int THREADS = 64 * NWAVE;
  static constexpr int RW = 16 * QBW * NWAVE;          // 256 query rows per workgroup
  static constexpr int MAT_BYTES = 32 * D * 2;         // K (or V) of a 32-key chunk
  static constexpr int SLOT_BYTES = 2 * MAT_BYTES;
  static constexpr int TILE_KEYS = 64;
  static constexpr int TILE_BYTES = 2 * SLOT_BYTES;    // two chunks
  static constexpr int NBUF = 4;
  static constexpr int SPR = D / 8;                    // 16-byte slots per key row
  static constexpr int RPL = 64 / SPR;                 // key rows per wave-wide load
  static constexpr int LPM = 32 / RPL;                 // wave-wide loads per matrix
  static constexpr int LPW = 2 * 2 * LPM / NWAVE;      // loads per wave per tile
  static constexpr int LDS_BYTES = NBUF * TILE_BYTES;
  static_assert(LPW * NWAVE == 4 * LPM, "a tile's loads split evenly over the waves");
};

// One lane's 16 bytes of global memory into LDS at lds_addr + 16 * lane (lds_addr
// wave-uniform), issued as inline assembly (M0 saved and restored around it).
__device__ __forceinline__ void lds_dma16(const uint16_t* src, uint32_t lds_addr) {
  uint32_t save;
  asm volatile(
      "s_mov_b32 %0, m0\n\ts_mov_b32 m0, %1\n\ts_nop 0\n\t"
      "global_load_lds_dwordx4 %2, off nt\n\ts_mov_b32 m0, %0"
      : "=&s"(save)
      : "s"(lds_addr), "v"(src)
      : "memory");
}

// Waits until at most n of this wave's vector loads are outstanding.
template <int LPW>
__device__ __forceinline__ void wait_tiles_after(int tiles_after) {
  if (tiles_after <= 0)
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  else if (tiles_after == 1)
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(LPW) : "memory");
  else
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(2 * LPW) : "memory");
}

template <class S>
__global__ __launch_bounds__(S::THREADS) void tree_attn_group_kernel(AttnArgs a) {
  constexpr int D = S::D, QBW = S::QBW, RW = S::RW, NBUF = S::NBUF, LPW = S::LPW;
  constexpr int SPR = S::SPR, RPL = S::RPL, LPM = S::LPM, NKS = D / 32, NDB = D / 16;
  static_assert(NBUF == 4, "wait_tiles_after covers up to NBUF - 2 = 2 tiles");
  __shared__ __attribute__((aligned(16))) uint8_t lds[S::LDS_BYTES];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 4, c = lane & 15;

  // workgroup -> (unit, split) as for the shared-tile kernel: the splits of a
  // unit share an XCD; unit = pair * qgroups + qgroup
  UnitCtx u;
  {
    const int xcd = blockIdx.x % kNumXCDs, slotw = blockIdx.x / kNumXCDs;
    u.split = slotw % a.splits;
    u.unit = (slotw / a.splits) * kNumXCDs + xcd;
    if (u.unit >= a.units) return;
    u.qgroup = u.unit % a.qgroups;
    u.pair = u.unit / a.qgroups;
    u.kvh = u.pair % a.Hkv;
    u.b = u.pair / a.Hkv;
  }
  const int r0 = wave * QBW * 16;                  // this wave's first row in the unit
  const bool active = u.qgroup * RW + r0 < a.M;   // wave-uniform: the wave has rows

  // this split's 64-key tiles of the capacity prefix; the last split adds the tree tile
  const int Lp = a.Lmax - a.N;
  const int n_tiles = (Lp + S::TILE_KEYS - 1) / S::TILE_KEYS;
  const int tb = (int)((long long)u.split * n_tiles / a.splits);
  const int te = (int)((long long)(u.split + 1) * n_tiles / a.splits);
  const int n_pre = te - tb;
  const bool tree_split = u.split == a.splits - 1;
  const int n_my = n_pre + (tree_split ? 1 : 0);

  const size_t kv_base = ((size_t)u.b * a.Hkv + u.kvh) * (size_t)a.Lmax * D;
  const uint16_t* kp = a.k + kv_base;
  const uint16_t* vp = a.v + kv_base;
  const uint32_t lds_base = (uint32_t)(size_t)(__attribute__((address_space(3))) uint8_t*)lds;
  const int r_in = lane / SPR, p_in = lane % SPR;
  // tile position j: keys key0.. (chunk h at key0 + 32 h), rows past key_max re-read it
  auto issue_tile = [&](int j, int key0, int key_max) {
#pragma unroll
    for (int e = 0; e < LPW; ++e) {
      const int li = wave * LPW + e;
      const int ch = li / (2 * LPM), mat = (li / LPM) & 1, t = li % LPM;
      const int r = t * RPL + r_in;
      const int key = min(key0 + ch * 32 + r, key_max);
      const uint16_t* src = (mat ? vp : kp) + (size_t)key * D + (p_in ^ swz<D>(r)) * 8;
      const uint32_t dst = lds_base + (uint32_t)((j % NBUF) * S::TILE_BYTES + ch * S::SLOT_BYTES +
                                                 mat * S::MAT_BYTES + t * RPL * D * 2);
      lds_dma16(src, __builtin_amdgcn_readfirstlane(dst));
    }
  };
  int L = 0;
  auto issue = [&](int j) {
    if (j < n_pre)
      issue_tile(j, (tb + j) * S::TILE_KEYS, Lp - 1);
    else
      issue_tile(j, L, L + a.N - 1);  // the tree tile
  };
  // prefix tiles go out first; the tree tile needs kv_len
  const int n_pro = min(NBUF - 1, n_my);
  for (int j = 0; j < min(n_pro, n_pre); ++j) issue(j);
  L = load_uniform(a.kv_len + u.b);  // scalar: no wait for the tiles in flight
  u.bad = L < 0 || L > Lp;
  if (u.bad) {
    L = 0;
    if (a.flags && u.split == 0 && u.qgroup == 0 && u.kvh == 0 && tid == 0)
      atomicOr(a.flags + u.b, EAGLE_FLAG_BAD_KV_LEN);
  }
  u.L = L;
  u.total = L + a.N;
  for (int j = n_pre; j < n_pro; ++j) issue(j);

  // every wave computes (rows past M hold zero queries and no tree bits):
  // a wave-uniform skip inside the tile loop made the compiler copy the
  // accumulators at every join, and the barrier paces all waves alike anyway
  bf16x8 qf[QBW][NKS];
  uint64_t anc_q[QBW];
  load_queries<D, QBW, RW>(a, u, r0, qf, anc_q);

  f32x4 acc[QBW][NDB];
  float m_run[QBW], l_run[QBW];
#pragma unroll
  for (int qb = 0; qb < QBW; ++qb) {
    m_run[qb] = -INFINITY;
    l_run[qb] = 0.f;
#pragma unroll
    for (int db = 0; db < NDB; ++db) acc[qb][db] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  // prefix tiles; the tree tile (position n_pre, if this split has it) after
  // the loop, so that the loop body has no join for the compiler to copy at
  for (int i = 0; i < n_pre; ++i) {
    wait_tiles_after<LPW>(min(NBUF - 2, n_my - 1 - i));
    barrier_lds();  // tile i is whole; every wave is done with tile i - 1
    if (i + NBUF - 1 < n_my) issue(i + NBUF - 1);
    const uint8_t* tile = lds + (i % NBUF) * S::TILE_BYTES;
    const int key0 = (tb + i) * S::TILE_KEYS;
    // both chunks' S first, so each softmax overlaps MFMAs still in flight
    f32x4 s0[QBW][2], s1[QBW][2];
    bf16x8 pf[QBW];
    chunk_qk<D, QBW>(tile, qf, s0);
    chunk_qk<D, QBW>(tile + S::SLOT_BYTES, qf, s1);
    chunk_soft<D, QBW>(s0, anc_q, acc, m_run, l_run, pf, a.scale_log2, key0 + 32 > L, false, 0,
                       prefix_mask8(key0 + 8 * g, L));
    chunk_pv<D, QBW>(tile, pf, acc);
    chunk_soft<D, QBW>(s1, anc_q, acc, m_run, l_run, pf, a.scale_log2, key0 + 64 > L, false, 0,
                       prefix_mask8(key0 + 32 + 8 * g, L));
    chunk_pv<D, QBW>(tile + S::SLOT_BYTES, pf, acc);
  }
  if (tree_split) {
    wait_tiles_after<LPW>(0);
    barrier_lds();
    const uint8_t* tile = lds + (n_pre % NBUF) * S::TILE_BYTES;
    for (int h = 0; h < 2 && 32 * h < a.N; ++h)
      chunk_step<D, QBW>(tile + h * S::SLOT_BYTES, qf, anc_q, acc, m_run, l_run, a.scale_log2,
                         true, true, 32 * h, 0u);
  }
  if (!active) return;

#pragma unroll
  for (int qb = 0; qb < QBW; ++qb) {
    l_run[qb] += __shfl_xor(l_run[qb], 16);
    l_run[qb] += __shfl_xor(l_run[qb], 32);
  }
  const size_t pbase = ((size_t)u.unit * a.splits + u.split) * RW;
#pragma unroll
  for (int qb = 0; qb < QBW; ++qb) {
    const int rl = r0 + qb * 16 + c;
    const int row = u.qgroup * RW + rl;
    if (row >= a.M) continue;
    if (a.splits == 1) {
      const int i = row / a.G;
      const int h = u.kvh * a.G + (row - i * a.G);
      uint16_t* orow = a.out + (((size_t)u.b * a.N + i) * a.Hq + h) * D;
      const float inv = (u.bad || l_run[qb] == 0.f) ? 0.f : 1.f / l_run[qb];
#pragma unroll
      for (int db = 0; db < NDB; ++db) {
        const f32x4 o = acc[qb][db] * inv;
        *reinterpret_cast<u32x2*>(orow + db * 16 + 4 * g) =
            u32x2{pack_bf16x2(o[0], o[1]), pack_bf16x2(o[2], o[3])};
      }
    } else {
      const float inv = l_run[qb] == 0.f ? 0.f : 1.f / l_run[qb];
#pragma unroll
      for (int db = 0; db < NDB; ++db)
        *reinterpret_cast<f32x4*>(a.part_o + (pbase + rl) * D + db * 16 + 4 * g) = acc[qb][db] * inv;
      if (g == 0)
        a.part_lse[pbase + rl] = l_run[qb] == 0.f ? -INFINITY : m_run[qb] + __log2f(l_run[qb]);
    }
  }
}

// ============================================================================
// merge (group and tile kernels): the splits' partials of a query row combined
// ============================================================================
// A thread per 16-byte column of a row (D / 4 threads per row): it loads the
// log2-sum-exp and the O / l column of every split, eight splits at a time
// with every load of a batch issued before any is used, rescales online, and
// writes four bf16 outputs.
template <int D>
__global__ __launch_bounds__(256) void tree_attn_merge_kernel(AttnArgs a, int RW) {
  constexpr int C4 = D / 4;        // 16-byte columns per row
  constexpr int RPB = 256 / C4;    // rows per workgroup
  // a unit's RW / RPB workgroups run on the XCD whose workgroups wrote its
  // partials (unit mod 8), so its reads can hit that XCD's L2
  const int bpu = RW / RPB;
  const int x = blockIdx.x % kNumXCDs, q = blockIdx.x / kNumXCDs;
  const int unit = (q / bpu) * kNumXCDs + x;
  if (unit >= a.units) return;
  const int rl = (q % bpu) * RPB + threadIdx.x / C4;
  const int d4 = threadIdx.x % C4;
  const int qgroup = unit % a.qgroups;
  const int pair = unit / a.qgroups;
  const int kvh = pair % a.Hkv;
  const int b = pair / a.Hkv;
  const int row = qgroup * RW + rl;
  if (row >= a.M) return;
  const int i = row / a.G;
  const int h = kvh * a.G + (row - i * a.G);
  const int S = a.splits;
  const size_t base = (size_t)unit * S * RW + rl;
  const int L = a.kv_len[b];
  const bool bad = L < 0 || L > a.Lmax - a.N;
  float mt = -INFINITY, lt = 0.f;
  f32x4 o = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int s0 = 0; s0 < S; s0 += 8) {
    float ls[8];
    f32x4 os[8];
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      const bool in = s0 + q < S;
      const size_t r = base + (size_t)(in ? s0 + q : 0) * RW;  // in range either way
      ls[q] = in ? a.part_lse[r] : -INFINITY;
      os[q] = in ? *reinterpret_cast<const f32x4*>(a.part_o + r * D + 4 * d4)
                 : f32x4{0.f, 0.f, 0.f, 0.f};
    }
    float mb = mt;
#pragma unroll
    for (int q = 0; q < 8; ++q) mb = fmaxf(mb, ls[q]);
    if (mb == -INFINITY) continue;
    const float f = mt == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(mt - mb);
    lt *= f;
    o *= f;
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      const float w = ls[q] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(ls[q] - mb);
      lt += w;
      o += os[q] * w;
    }
    mt = mb;
  }
  const float inv = (bad || lt == 0.f) ? 0.f : 1.f / lt;
  uint16_t* orow = a.out + (((size_t)b * a.N + i) * a.Hq + h) * D + 4 * d4;
  *reinterpret_cast<u32x2*>(orow) =
      u32x2{pack_bf16x2(o[0] * inv, o[1] * inv), pack_bf16x2(o[2] * inv, o[3] * inv)};
}

// ---- variants ----------------------------------------------------------------
// 0: ring, 1 query block      1: ring, 2 query blocks
// 2: tile, 4 blocks (2x2)     3: tile, 8 blocks (4 query waves)   4: tile, 16 blocks
// 5: ring, 2 query blocks per query group, default cache policy (grouped queries)
// 6: group kernel, 256 rows per workgroup sharing a ring of 64-key tiles
struct VariantInfo {
  int rw;
  int keys_per_piece;  // split granularity in keys
};

static VariantInfo variant_info(int variant) {
  switch (variant) {
    case 0: return {16, 32};
    case 1: return {32, 32};
    case 2: return {64, 64};
    case 3: return {128, 64};
    case 5: return {32, 32};
    case 6: return {256, 64};
    default: return {256, 64};
  }
}

template <int D>
static void* variant_kernel(int variant) {
  static_assert(RingShape<D, 1>::THREADS == kRingThreads && RingShape<D, 2>::THREADS == kRingThreads &&
                    RingShape<D, 2, 0>::THREADS == kRingThreads,
                "ring launch size");
  switch (variant) {
    case 0: return (void*)tree_attn_ring_kernel<RingShape<D, 1>>;
    case 1: return (void*)tree_attn_ring_kernel<RingShape<D, 2>>;
    case 2: return (void*)tree_attn_tile_kernel<TileShape<D, 2, 2, 1>>;
    case 3: return (void*)tree_attn_tile_kernel<TileShape<D, 2, 4, 2>>;
    case 5: return (void*)tree_attn_ring_kernel<RingShape<D, 2, 0>>;
    case 6: return (void*)tree_attn_group_kernel<GroupShape<D>>;
    default: return (void*)tree_attn_tile_kernel<TileShape<D, 4, 4, 2>>;
  }
}

static bool is_ring(int variant) { return variant <= 1 || variant == 5; }

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
  const int pairs = B * Hkv;
  int variant = nqb <= 1 ? 0 : nqb <= 2 ? 1 : nqb <= 4 ? 2 : nqb <= 8 ? 3 : 4;
  // Grouped queries: the group kernel, whose 256 rows per workgroup share a
  // ring of K/V tiles (measured on MI355X: llama2-70b shape 67 us against 79
  // for ring query groups and 85 for the shared-tile kernel; mixtral shape
  // 206 us against 266 and 249).
  if (variant >= 2) variant = 6;
  variant = env_int("EAGLE_ATTN_VARIANT", variant);
  if (variant < 0 || variant > 6) variant = 4;
  const VariantInfo vi = variant_info(variant);
  p.variant = variant;
  p.rows_per_wg = vi.rw;
  p.kt = vi.keys_per_piece;
  p.qgroups = (p.M + vi.rw - 1) / vi.rw;
  // ring variants: the query groups of a (b, kv head) pair are consecutive
  // units of the pair's XCD (pair mod 8), so the pairs are padded to a
  // multiple of 8 and the padding units exit at once
  p.units = is_ring(variant) ? ((pairs + kNumXCDs - 1) / kNumXCDs) * kNumXCDs * p.qgroups
                             : pairs * p.qgroups;
  const int pieces = (Lmax + vi.keys_per_piece - 1) / vi.keys_per_piece;
  const int padded_units = ((p.units + kNumXCDs - 1) / kNumXCDs) * kNumXCDs;
  // Aim for one workgroup per CU: a ring workgroup keeps up to eight 32-key
  // chunks in flight and fills its CU's LDS; more splits only lengthen the
  // merge, whose cost grows with splits x query rows.
  const int target = kNumCUs;
  int splits = (target + padded_units - 1) / padded_units;
  if (is_ring(variant) && p.qgroups == 1) {
    // One ring workgroup per CU (its LDS): workgroups beyond kNumCUs run in
    // another round, so a half-empty last round costs as much as a full one.
    // Pick the split count s minimising rounds(s) * chunks per split plus a
    // merge cost of 1.75 chunk-times per split (fitted on MI355X: llama2-7b
    // 6 splits, 14.9 us against 16.0 us at 8; llama2-13b 3 splits, 64 us
    // against 85 us at 2).
    const int n_chunks = (Lmax - N + 31) / 32;
    float best = 0.f;
    for (int sc = 1; sc <= 16 && sc <= n_chunks; ++sc) {
      const int rounds = (padded_units * sc + kNumCUs - 1) / kNumCUs;
      const float cost = (float)(rounds * ((n_chunks + sc - 1) / sc)) + 1.75f * sc;
      if (sc == 1 || cost < best) {
        best = cost;
        splits = sc;
      }
    }
  }
  splits = env_int("EAGLE_ATTN_SPLITS", splits);
  if (splits > pieces) splits = pieces;
  if (splits > 64) splits = 64;  // the merge keeps one split weight per lane
  if (splits < 1) splits = 1;
  p.splits = splits;
  return p;
}

static size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

// Workspace: [unit tickets (ring variants) | split log2-sum-exp | split O].
static size_t ticket_bytes(const AttnPlan& p) {
  return is_ring(p.variant) && p.splits > 1 ? align256((size_t)p.units * 4) : 0;
}

size_t tree_attn_workspace_bytes(const AttnPlan& p) {
  if (p.splits <= 1) return 0;
  const size_t lse = align256((size_t)p.units * p.splits * p.rows_per_wg * 4);
  const size_t o = (size_t)p.units * p.splits * p.rows_per_wg * p.d * 4;
  return ticket_bytes(p) + lse + o;
}

hipError_t launch_tree_attn(const AttnPlan& plan, const uint16_t* q, const uint16_t* k,
                            const uint16_t* v, const int32_t* kv_len, const uint64_t* anc,
                            const int32_t* parents, uint64_t* anc_out, int32_t* depth_out,
                            int32_t* pos_out,
                            int B, int N, int Hq, int Hkv, int Lmax, float scale_log2,
                            uint16_t* out, void* ws, int32_t* flags, hipStream_t s) {
  AttnArgs a{};
  a.q = q;
  a.k = k;
  a.v = v;
  a.kv_len = kv_len;
  a.anc = anc;
  a.parents = anc ? nullptr : parents;
  a.anc_out = anc_out;
  a.depth_out = depth_out;
  a.pos_out = pos_out;
  a.out = out;
  const bool ring = is_ring(plan.variant);
  uint8_t* w = static_cast<uint8_t*>(ws);
  const size_t tk = ticket_bytes(plan);
  const size_t lse = align256((size_t)plan.units * plan.splits * plan.rows_per_wg * 4);
  a.tickets = reinterpret_cast<int32_t*>(w);
  a.part_lse = reinterpret_cast<float*>(w + tk);
  a.part_o = reinterpret_cast<float*>(w + tk + lse);
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
  const int threads = ring ? kRingThreads : plan.variant == 6 ? GroupShape<128>::THREADS : 256;
  hipError_t err = hipLaunchKernel(fn, grid, dim3(threads), args, 0, s);
  // ring variants combine their splits in the kernel
  if (err != hipSuccess || plan.splits == 1 || ring) return err;
  const int rw = plan.rows_per_wg;
  const int rows_per_block = 256 / (plan.d / 4);
  const dim3 mgrid((unsigned)(((plan.units + kNumXCDs - 1) / kNumXCDs) * kNumXCDs *
                               (rw / rows_per_block)));
  if (plan.d == 64)
    tree_attn_merge_kernel<64><<<mgrid, 256, 0, s>>>(a, rw);
  else
    tree_attn_merge_kernel<128><<<mgrid, 256, 0, s>>>(a, rw);
  return hipGetLastError();
}

}  // namespace eagle
