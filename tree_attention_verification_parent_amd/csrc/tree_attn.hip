// Tree attention for the verification forward on gfx950.
//
// The target verifies the whole draft tree in one forward pass: node i of
// sequence b attends to the committed keys 0..L-1 and to the tree keys L+j of
// its ancestors j (EAGLE, paperlayer.ai summary, §2 Preliminaries; §3 EAGLE:
// tree attention; A.1 Tree Structure).  This is decode-shaped attention:
// M = G*N query rows per KV head against L+N keys, HBM-bound on the bf16 K/V
// stream.
//
// Only the keys of J are ever read: the committed keys [0, L) of the
// sequence and its tree keys [L, L+N).  Chunks are laid over [0, L), not over
// the cache capacity, and a load past the end of its range re-reads the last
// key of that range (masked afterwards), so cache slots at or past L+N, which
// may hold anything (a preallocated cache, the unused tail of a shorter
// sequence in a ragged batch), never reach the scores or the V products.
//
// Work decomposition
//   unit  = (b, KV head, group of RW query rows); piece = a contiguous range
//   of key chunks of one unit.  The launch has a fixed number of workgroup
//   slots (a multiple of 8, sized on the host from the cache capacity); every
//   workgroup reads the batch's committed lengths and shares the slots out:
//   each unit gets one, the rest go to the sequences in proportion to their
//   lengths, so a ragged batch costs about the sum of its lengths.  Slots are
//   numbered so that consecutive ones (the pieces of a unit) run on one XCD
//   (workgroup i is dispatched to XCD i mod 8).
//
// Two kernels, picked by the number of query rows per KV head:
//   ring  (M <= 32, e.g. multi-head attention): every wave owns a 32-key
//         chunk slot in LDS, filled by direct-to-LDS loads, so a piece's
//         chunks are in flight from the start with no staging registers and
//         no barriers in the main loop; the waves' states are folded at the
//         end, and the unit's last piece to finish combines the pieces'
//         partials (written and read with device-coherent accesses, so the
//         combine does not depend on where the pieces ran).
//   group (M > 32, grouped-query attention): eight waves each own 32 of up to
//         256 query rows and compute every 64-key tile of the piece against
//         them, so a tile is read from HBM once for the whole head group; a
//         merge kernel combines the pieces.
// Both compute S^T = K Q^T and O^T += V^T P^T with v_mfma_f32_16x16x32_bf16
// (keys on MFMA rows: the K rows are permuted so each lane ends up holding 8
// consecutive keys of one query column, exactly the k-slots of P^T), apply
// the tree mask, and run the online softmax with cross-lane shuffles.
#include <limits.h>

#include <algorithm>
#include <mutex>

#include "common.h"
#include "launch.h"

namespace eagle {

typedef short short4_t __attribute__((ext_vector_type(4)));
typedef uint64_t u64x2 __attribute__((ext_vector_type(2)));

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
  float* part_o;      // [slots * RW * D]  O / l of each piece, by slot
  float* part_lse;    // [slots * RW]      m + log2(l) of each piece
  int32_t* tickets;   // [units] pieces finished (ring kernel; zero between calls)
  int32_t* unit_info; // [units * 2] first slot and piece count (group kernel -> merge)
  int32_t* flags;
  int B, N, Hq, Hkv, Lmax, G, M, qgroups, slots, kg, max_pieces;
  int full_pieces;  // pieces per unit when every sequence fills the cache (see the ring kernel)
  int ring_cost;    // 1: pick the piece length by the ring kernel's order (else the smallest that fits)
  float scale_log2;
  // multipliers for div_magic by full_pieces, Hkv, qgroups and G
  uint32_t fp_magic, hkv_magic, qg_magic, g_magic;
  int xcd_group;  // 1: a unit's full_pieces slots share one XCD (logical_slot)
};

// n / d without a division, for n * d <= 2^32: the high half of n * m with
// m = floor((2^32 - 1) / d) + 1 = (2^32 + e) / d, 0 <= e < d, is
// floor(n / d + n e / (d 2^32)), and n e < 2^32 keeps the added fraction
// below the distance 1/d to the next integer (Granlund and Montgomery,
// division by invariant integers).  d = 1 passes n through (m would need 33
// bits).  The host computes m once per launch.
__device__ __forceinline__ int div_magic(int n, uint32_t m, int d) {
  return d == 1 ? n : (int)__umulhi((uint32_t)n, m);
}
__host__ inline uint32_t magic_of(int d) {
  return d <= 1 ? 0u : (uint32_t)(0xffffffffull / (unsigned long long)d + 1ull);
}

// a * b / c for non-negative ints, in 32 bits when a * b fits (wave-uniform
// operands: a uniform branch)
__device__ __forceinline__ int mul_div(int a, int b, int c) {
  const unsigned long long p = (unsigned long long)(unsigned)a * (unsigned)b;
  if ((p >> 32) == 0) return (int)((uint32_t)p / (uint32_t)c);
  return (int)(p / (unsigned long long)c);
}

// ---- decomposition -------------------------------------------------------------
// A unit's piece: which (sequence, KV head, query group), which of its
// nsplit pieces, the slot of its first piece, and the committed length.
struct Piece {
  int b, kvh, qgroup, unit, split, nsplit, first, L;
  bool bad;
};

// Slot of this workgroup.  Workgroup ids go to the XCDs round robin (id mod
// 8).  With xcd_group (the ring kernel, units a multiple of 8, slots = units
// x full_pieces) id 8 (q P + p) + x takes piece p of unit 8 q + x, so that at
// full length the P pieces of a unit run on one XCD: measured faster on
// MI355X (llama2-7b shape 14.8 against 15.3 us, llama2-13b 62.8 against
// 63.4), though nothing depends on it, since the partials meet through
// device-coherent memory whatever the placement.  Otherwise the slot is the
// id: the used slots (0 .. pieces - 1 when the committed lengths leave some
// unused) spread over all XCDs.
__device__ __forceinline__ int div_magic(int n, uint32_t m, int d);
__device__ __forceinline__ int logical_slot(const AttnArgs& a) {
  const int bid = (int)blockIdx.x;
  if (!a.xcd_group) return bid;
  const int x = bid & (kNumXCDs - 1), j = bid / kNumXCDs;
  const int q = div_magic(j, a.fp_magic, a.full_pieces);
  return (kNumXCDs * q + x) * a.full_pieces + (j - q * a.full_pieces);
}

// A wave-uniform 32-bit value read with a scalar load (constant address
// space), which the compiler tracks apart from the vector loads in flight.
__device__ __forceinline__ int32_t load_uniform(const int32_t* p) {
  return *(const __attribute__((address_space(4))) int32_t*)p;
}

// The committed lengths of sequences 0..63 in lanes 0..63 (0 past B).  For
// B <= 16 they are read with scalar loads (addresses clamped into the array),
// which a wave can wait for without waiting for its vector loads in flight:
// the kernels issue their first K/V loads before they know the plan.
__device__ __forceinline__ int kv_len_lanes(const AttnArgs& a) {
  const int lane = threadIdx.x & 63;
  if (a.B <= 16) {
    int x[16];
#pragma unroll
    for (int b = 0; b < 16; ++b) x[b] = load_uniform(a.kv_len + min(b, a.B - 1));
    int v = 0;
#pragma unroll
    for (int b = 0; b < 16; ++b) v = lane == b ? x[b] : v;
    return lane < a.B ? v : 0;
  }
  const int v = a.kv_len[min(lane, a.B - 1)];
  return lane < a.B ? v : 0;
}

// Sum over the wave of a non-negative int (DPP within rows of 16, then the
// four rows); every lane receives it.
__device__ __forceinline__ int wave_allsum_i(int v) {
  v += dpp_i<kDppXor1>(v);
  v += dpp_i<kDppXor2>(v);
  v += dpp_i<kDppHalfMirror>(v);
  v += dpp_i<kDppMirror>(v);
  return (lane_i(v, 0) + lane_i(v, 16)) + (lane_i(v, 32) + lane_i(v, 48));
}

// The ring kernel's order of decompositions (pieces of at most T chunks,
// n_pieces of them in all, the longest sequence of cmax chunks): first the
// fewest rounds of workgroups (a ring workgroup fills its CU's LDS, so
// workgroups beyond the CU count wait for a whole round), then the shortest
// piece, but no shorter than 8 chunks, one per wave (a shorter piece leaves
// waves idle and only adds partials to combine).  Within one round a shorter
// piece puts more CUs on the stream; measured on MI355X against the earlier
// model (a round costing T chunk-times, each piece 1.75 more for its merge,
// which took more pieces over two rounds): llama2-13b 61.8 -> 59.4 us with
// one piece per head instead of three, four 8192-key sequences 128.8 ->
// 106.1, a ragged batch of 512, 1024, 2048, 8192 keys 63.0 -> 52.4, the
// llama2-7b shape 15.2 -> 14.8 with 8 pieces of 8 chunks instead of 6 of 11.
// The host (at full cache length) and the device (at the committed lengths)
// apply the same order, so at full length both choose the same pieces.
__host__ __device__ inline int ring_rounds(long long n_pieces) {
  const long long slots = (n_pieces + kNumXCDs - 1) / kNumXCDs * kNumXCDs;
  return (int)((slots + kNumCUs - 1) / kNumCUs);
}
__host__ __device__ inline int ring_piece_len(int T, int cmax) {
  const int floor8 = cmax < 8 ? cmax : 8;
  return T > floor8 ? T : floor8;
}

// Committed length of sequence b (given as read) -> chunks of kg keys; a
// length that leaves no room for the tree (or is negative) counts as 0.
__device__ __forceinline__ int seq_chunks(const AttnArgs& a, bool in, int Lraw, int& L, bool& bad) {
  bad = in && (Lraw < 0 || Lraw > a.Lmax - a.N);
  L = in && !bad ? Lraw : 0;
  return (L + a.kg - 1) / a.kg;
}

// Pieces of all units at 16 candidate piece lengths at once, B <= 64: lane j
// holds candidate j & 15's length t and adds the pieces of sequences
// j >> 4, (j >> 4) + 4, ... (c0: chunks by lane, as in plan_piece); the four
// partial sums of a candidate meet across lanes j, j ^ 16, j ^ 32, j ^ 48.
// Every lane returns its candidate's total.
__device__ __forceinline__ long long count_pieces_x16(const AttnArgs& a, int c0, int t) {
  const int part = (threadIdx.x & 63) >> 4;
  int n = 0;
  for (int b0 = 0; b0 < a.B; b0 += 4) {  // wave-uniform
    const int b = b0 + part;
    const int cb = __shfl(c0, b & 63);
    if (b < a.B) n += max(1, min(a.max_pieces, (cb + t - 1) / t));
  }
  n += __shfl_xor(n, 16);
  n += __shfl_xor(n, 32);
  return (long long)(a.Hkv * a.qgroups) * n;
}

// Shares the launch's slots out and finds a piece.  Every unit of sequence b
// gets s_b = ceil(c_b / T) pieces (at least one, at most max_pieces), where
// c_b is its number of chunks of kg committed keys and T is the largest piece
// in chunks.  Ring kernel: T = ceil(c_max / k) for the k in 1..16 first in
// the order of ring_rounds, ring_piece_len among those whose pieces fit the
// launch's slots (so short committed lengths take fewer, not shorter, rounds
// of workgroups).
// Otherwise T is the smallest value for which all pieces fit the slots: in
// closed form when every sequence has the same length, else by bisection
// (the count only falls as T grows, and T = max c_b fits since the host
// launches at least one slot per unit).  With B <= 64 the 16 candidates of
// the ring order are counted at once, one per group of lanes, and the
// bisection becomes a 16-way search; both give the same T as the serial
// forms (the first candidate first in the order; the least fitting T), at a
// fraction of the instructions, which every workgroup spends before its
// first loads when the lengths are not the full ones.  Slots are numbered sequence by
// sequence, unit by unit, piece by piece; slots past the last piece are
// unused.  Finds the piece in slot `key`; kvl0 holds the committed lengths of
// sequences 0..63 by lane (kv_len_lanes).  A function of the committed
// lengths and the launch shape alone, so every wave finds the same
// decomposition.  All 64 lanes of the wave call it; the result is
// wave-uniform.  Returns false for an unused slot.
__device__ bool plan_piece(const AttnArgs& a, int key, int kvl0, Piece& p) {
  const int lane = threadIdx.x & 63;
  const int U = a.Hkv * a.qgroups;
  int L0;
  bool bad0;
  const int c0 = seq_chunks(a, lane < a.B, kvl0, L0, bad0);
  auto block_chunks = [&](int b0, int& L, bool& bad) {
    const int b = b0 + lane;
    const int raw = a.kv_len[min(b, a.B - 1)];
    return seq_chunks(a, b < a.B, raw, L, bad);
  };
  int cmax = wave_allmax_i(c0);
  int cmin = wave_allmin_i(lane < a.B ? c0 : INT_MAX);
  for (int b0 = 64; b0 < a.B; b0 += 64) {
    int L;
    bool bad;
    const int c = block_chunks(b0, L, bad);
    cmax = max(cmax, wave_allmax_i(c));
    cmin = min(cmin, wave_allmin_i(b0 + lane < a.B ? c : INT_MAX));
  }
  auto pieces_of = [&](int c, int t) { return max(1, min(a.max_pieces, (c + t - 1) / t)); };
  // all pieces at piece length t (capped just past the slots)
  auto count_at = [&](int t) {
    long long n = wave_allsum_i(lane < a.B ? min(U * pieces_of(c0, t), a.slots + 1) : 0);
    for (int b0 = 64; b0 < a.B && n <= a.slots; b0 += 64) {
      int L;
      bool bad;
      const int c = block_chunks(b0, L, bad);
      n += wave_allsum_i(b0 + lane < a.B ? min(U * pieces_of(c, t), a.slots + 1) : 0);
    }
    return n;
  };
  int T = 0;
  if (a.B <= 64 && a.ring_cost) {
    const int cm = max(cmax, 1);
    const int k = (lane & 15) + 1;
    const int t = (cm + k - 1) / k;
    const long long n = count_pieces_x16(a, c0, t);
    const bool ok = k <= cm && n <= a.slots;
    const int r = ok ? ring_rounds(n) : INT_MAX;
    const int best_r = wave_allmin_i(r);
    const int te = ok && r == best_r ? ring_piece_len(t, cm) : INT_MAX;
    const int best_t = wave_allmin_i(te);
    const uint64_t m = __ballot(lane < 16 && ok && r == best_r && te == best_t);  // k = 1 always fits
    T = m ? lane_i(t, __ffsll((unsigned long long)m) - 1) : cm;
  } else if (a.B <= 64 && cmin != cmax) {
    // least fitting T in [lo, hi] (hi fits): candidate j = lo + (j + 1) step - 1,
    // the last one hi; the first that fits bounds the next range
    int lo = 1, hi = max(cmax, 1);
    const int j = lane & 15;
    while (lo < hi) {  // wave-uniform
      const int step = (hi - lo + 16) / 16;
      const int t = min(hi, lo + (j + 1) * step - 1);
      const bool fit = count_pieces_x16(a, c0, t) <= a.slots;
      const uint64_t m = __ballot(lane < 16 && fit);  // candidate 15 (= hi) fits
      const int jf = m ? __ffsll((unsigned long long)m) - 1 : 15;
      const int prev = lane_i(t, max(jf - 1, 0));
      hi = lane_i(t, jf);
      lo = jf > 0 ? prev + 1 : lo;
    }
    T = lo;
  } else if (a.ring_cost) {
    const int cm = max(cmax, 1);
    int best_r = 0, best_t = 0;
    for (int k = 1; k <= min(16, cm); ++k) {  // wave-uniform
      const int t = (cm + k - 1) / k;
      const long long n = count_at(t);
      if (n > a.slots) continue;
      const int r = ring_rounds(n), te = ring_piece_len(t, cm);
      if (T == 0 || r < best_r || (r == best_r && te < best_t)) {
        best_r = r;
        best_t = te;
        T = t;
      }
    }
  }
  if (T > 0) {
    // chosen by the ring order
  } else if (cmin == cmax) {
    // every unit alike: ceil(c / T) <= slots / units
    const int per_unit = (int)((long long)a.slots / ((long long)a.B * U));
    T = per_unit >= a.max_pieces ? 1 : max(1, (cmax + per_unit - 1) / per_unit);
  } else {
    auto fits = [&](int t) { return count_at(t) <= a.slots; };
    int lo = 1, hi = max(cmax, 1);
    while (lo < hi) {  // wave-uniform
      const int mid = (lo + hi) >> 1;
      if (fits(mid))
        hi = mid;
      else
        lo = mid + 1;
    }
    T = lo;
  }
  long long base = 0;  // slots of the sequences before this block
  for (int b0 = 0; b0 < a.B; b0 += 64) {
    const int b = b0 + lane;
    int L = L0, c = c0;
    bool bad = bad0;
    if (b0 > 0) c = block_chunks(b0, L, bad);
    const int s = pieces_of(c, T);
    const int n = b < a.B ? U * s : 0;
    int incl = n;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int o = __shfl_up(incl, off);
      if (lane >= off) incl += o;
    }
    const long long lo_slot = base + (incl - n);
    const bool mine = b < a.B && key >= lo_slot && key < lo_slot + n;
    const uint64_t m = __ballot(mine);
    if (m) {
      const int src = __ffsll((unsigned long long)m) - 1;
      const int sb = __shfl(b, src), ss = __shfl(s, src);
      p.L = __shfl(L, src);
      p.bad = __shfl((int)bad, src) != 0;
      const long long slo = __shfl(lo_slot, src);
      const int r = (int)(key - slo);
      const int uis = r / ss;  // unit within the sequence
      p.b = sb;
      p.nsplit = ss;
      p.split = r - uis * ss;
      p.kvh = uis / a.qgroups;
      p.qgroup = uis - p.kvh * a.qgroups;
      p.unit = sb * U + uis;
      p.first = (int)(slo + (long long)uis * ss);
      return true;
    }
    base += lane_i(incl, 63);
  }
  return false;
}

// Device-coherent 16- and 4-byte accesses (agent scope, the sc1 bit): they
// bypass the caches that are not coherent between XCDs, so a partial stored
// by a piece on one XCD is seen by the combining workgroup on any other once
// the store has completed and the ticket that follows it has been taken.
// The 16-byte store is a single instruction (inline assembly: a store has no
// outputs); the caller's s_waitcnt vmcnt(0) covers it before the ticket.
__device__ __forceinline__ void store_coherent(float* p, f32x4 v) {
  asm volatile("global_store_dwordx4 %0, %1, off sc1" ::"v"(p), "v"(v) : "memory");
}
__device__ __forceinline__ void store_coherent(float* p, float v) {
  __hip_atomic_store(reinterpret_cast<uint32_t*>(p), __float_as_uint(v), __ATOMIC_RELAXED,
                     __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ f32x4 load_coherent4(__amdgpu_buffer_rsrc_t r, uint32_t byte_off) {
  return __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(r, (int)byte_off, 0, 16));
}
__device__ __forceinline__ float load_coherent(const float* p) {
  return __uint_as_float(__hip_atomic_load(reinterpret_cast<uint32_t*>(const_cast<float*>(p)),
                                           __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
}

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

// Q fragments (MFMA B operand) and tree masks of QBW query blocks at unit row
// r0.  Rows past M hold zero queries and no tree bits.
template <int D, int QBW, int RW>
__device__ __forceinline__ void load_queries(const AttnArgs& a, const Piece& u, int r0,
                                             bf16x8 (&qf)[QBW][D / 32], uint64_t (&anc_q)[QBW]) {
  const int lane = threadIdx.x & 63, g = lane >> 4, c = lane & 15;
  const int N = a.N, G = a.G;
  const uint64_t nmask = N == 64 ? ~0ull : (1ull << N) - 1ull;
  // masks built from the parent links: every wave derives its sequence's
  // tree (lane = node); wave 0 of the last piece of KV head 0, query group 0
  // writes the builder's outputs
  uint64_t anc_w = 0;
  if (a.parents) {
    const TreeLinks t = tree_links_wave(a.parents + (size_t)u.b * N, N);
    anc_w = t.anc;
    if (u.kvh == 0 && u.qgroup == 0 && u.split == u.nsplit - 1 && threadIdx.x < 64)
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

// ============================================================================
// ring kernel: one direct-to-LDS chunk slot per wave
// ============================================================================
// Eight waves, each with one 32-key K/V slot in LDS.  The chunks of a piece
// are dealt to them round robin; a wave waits for its chunk, computes it and
// refills the slot with its next chunk, while the other seven keep theirs in
// flight (two waves per SIMD hide each other's MFMA and softmax latency).
// The tree keys (each query's ancestors and itself, N <= 64 of them) are one
// or two more chunks, masked by the ancestor bits, for the wave of the last
// piece with the fewest committed chunks.
constexpr int kRingThreads = 64 * 8;

// One lane's 16 bytes of global memory into LDS at lds_addr + 16 * lane
// (lds_addr wave-uniform), non-temporal (the K/V stream is read once, and per
// XCD it is about the size of the L2).  Inline assembly (M0 saved and restored
// around it): the compiler treats a direct-to-LDS load of its own as a pending
// LDS write that every later LDS read waits for, which would hold each chunk's
// computation up behind every load issued after it.  The kernels track the
// loads' completion themselves with s_waitcnt (vector loads complete in
// order).
__device__ __forceinline__ void lds_dma16(const uint16_t* src, uint32_t lds_addr) {
  uint32_t save;
  asm volatile(
      "s_mov_b32 %0, m0\n\ts_mov_b32 m0, %1\n\ts_nop 0\n\t"
      "global_load_lds_dwordx4 %2, off nt\n\ts_mov_b32 m0, %0"
      : "=&s"(save)
      : "s"(lds_addr), "v"(src)
      : "memory");
}
__device__ __forceinline__ uint32_t lds_addr(const uint8_t* p) {
  return __builtin_amdgcn_readfirstlane(
      (uint32_t)(size_t)(const __attribute__((address_space(3))) uint8_t*)p);
}

template <int D_, int QBW_>
struct RingShape {
  static constexpr int D = D_;
  static constexpr int QBW = QBW_;
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

  const int slot_w = logical_slot(a);
  const int r_in = lane / SPR, p_in = lane % SPR;
  uint8_t* slot = lds + wave * S::SLOT_BYTES;
  // Direct-to-LDS fill of 32 keys from key0: lane l writes 16 bytes at load
  // base + 16 l, i.e. row t*RPL + l/SPR, slot l%SPR, which receives global
  // slot (l%SPR)^swz(row).  Rows past key_max re-read it (a key of J, masked
  // later).
  auto issue_keys_at = [&](const uint16_t* kp, const uint16_t* vp, int key0, int key_max) {
#pragma unroll
    for (int t = 0; t < LPM; ++t) {
      const int r = t * RPL + r_in;
      const int key = min(key0 + r, key_max);
      const size_t off = (size_t)key * D + (p_in ^ swz<D>(r)) * 8;
      lds_dma16(kp + off, lds_addr(slot + t * RPL * D * 2));
    }
#pragma unroll
    for (int t = 0; t < LPM; ++t) {
      const int r = t * RPL + r_in;
      const int key = min(key0 + r, key_max);
      const size_t off = (size_t)key * D + (p_in ^ swz<D>(r)) * 8;
      lds_dma16(vp + off, lds_addr(slot + S::MAT_BYTES + t * RPL * D * 2));
    }
  };

  // The query rows of a unit (b, kvh): lane (c, g) holds row qb * 16 + c's
  // 8 dims at ks * 32 + g * 8.  Rows past M load row 0 again: each query row
  // is a column of its own through the MFMAs, the softmax and the fold, and
  // those rows are never stored.  (Zeroing them with a select made the
  // compiler wait for every load in flight at the start of a piece, the
  // second chunk's included, before anything else.)
  bf16x8 qf[QBW][NKS];
  auto load_q = [&](int b, int kvh) {
#pragma unroll
    for (int qb = 0; qb < QBW; ++qb) {
      const int row = qb * 16 + c;
      const int rr = row < a.M ? row : 0;
      const int i = div_magic(rr, a.g_magic, a.G);
      const int h = kvh * a.G + (rr - i * a.G);
      const uint16_t* qrow = a.q + (((size_t)b * a.N + i) * a.Hq + h) * D;
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks)
        qf[qb][ks] = *reinterpret_cast<const bf16x8*>(qrow + ks * 32 + g * 8);
    }
  };

  // A piece's chunks for this wave: 32-key chunks of [0, L), wave w taking
  // cb + w, cb + w + NWAVE, ..., then (for the wave of the last piece with
  // the fewest committed chunks) the tree keys [L, L + N) as one or two more
  // masked chunks (N <= 64).
  struct Run {
    int L, my_first, my_n, my_chunks;
    bool tree_wave;
    const uint16_t* kp;
    const uint16_t* vp;
  };
  // (cb, ce: the piece's chunks of [0, L))
  auto run_at = [&](const Piece& p, int cb, int ce) {
    Run r;
    r.L = p.L;
    r.my_first = cb + wave;
    r.my_n = r.my_first < ce ? (ce - r.my_first + NWAVE - 1) / NWAVE : 0;  // NWAVE: a power of 2
    r.tree_wave = p.split == p.nsplit - 1 && wave == (ce - cb) % NWAVE;
    r.my_chunks = r.my_n + (r.tree_wave ? (a.N + 31) / 32 : 0);
    const size_t kv_base = ((size_t)p.b * a.Hkv + p.kvh) * (size_t)a.Lmax * D;
    r.kp = a.k + kv_base;
    r.vp = a.v + kv_base;
    return r;
  };
  auto run_of = [&](const Piece& p) {
    const int n_chunks = (p.L + 31) >> 5;
    return run_at(p, mul_div(p.split, n_chunks, p.nsplit), mul_div(p.split + 1, n_chunks, p.nsplit));
  };
  auto chunk_key0 = [&](const Run& r, int i) {
    return i < r.my_n ? (r.my_first + NWAVE * i) * 32 : r.L + 32 * (i - r.my_n);
  };
  auto chunk_kmax = [&](const Run& r, int i) { return i < r.my_n ? r.L - 1 : r.L + a.N - 1; };
  // The start of a piece: its query rows, then its first chunk into the slot
  // and (a wave with two or more chunks) its second into registers, so that
  // the second is in flight with the first instead of requested once the
  // first has been computed (the slot is busy until then); it goes to the
  // slot later in the layout a direct-to-LDS load gives.  Vector loads
  // complete in order: the rows land before the chunk that needs them, and
  // the first chunk can be waited for with the second's loads outstanding.
  u32x4 pre[2 * LPM];
  auto start = [&](const Piece& p, const Run& r) __attribute__((always_inline)) {
    load_q(p.b, p.kvh);
    if (r.my_chunks > 0) issue_keys_at(r.kp, r.vp, chunk_key0(r, 0), chunk_kmax(r, 0));
    if (r.my_chunks >= 2) {
      const int key0 = chunk_key0(r, 1), key_max = chunk_kmax(r, 1);
#pragma unroll
      for (int t = 0; t < LPM; ++t) {
        const int rr = t * RPL + r_in;
        const size_t off = (size_t)min(key0 + rr, key_max) * D + (p_in ^ swz<D>(rr)) * 8;
        pre[t] = *reinterpret_cast<const u32x4*>(r.kp + off);
        pre[LPM + t] = *reinterpret_cast<const u32x4*>(r.vp + off);
      }
    }
  };

  const int Lcap = a.Lmax - a.N;
  // When every sequence fills the cache (the common case) the planner gives
  // this slot piece slot % full_pieces of unit slot / full_pieces: the wave
  // starts that piece before the lengths are read, and the plan reduces to
  // checking that every length is the full one.  Otherwise the started loads
  // are waited for and dropped, and the planner finds the piece.
  // Only the first round of workgroups (one per CU) guesses: when the lengths
  // are not the full ones the launch's later slots are mostly unused, and a
  // guess there costs an unused workgroup its loads' latency (llama2-13b
  // heads, four sequences of 2944 keys in a 8192-key cache: 60.8 us against
  // 95.8 when every slot guesses), while a later workgroup that plans first
  // starts about 1.5 us later at full length (62.7 against 61.1 us).
  // A later workgroup still takes the closed form once the lengths are known
  // to be the full ones, instead of planning.
  const bool guessable = a.full_pieces > 0 && a.B <= 64 && slot_w < a.B * a.Hkv * a.full_pieces;
  const bool spec = guessable && (int)blockIdx.x < kNumCUs;
  // (no division on the way to the first loads: a wave issues them about
  // 0.5 us sooner at the llama2-7b shape than with the divisions)
  Piece pc{};
  Run R{};
  auto guess = [&]() __attribute__((always_inline)) {
    pc.unit = div_magic(slot_w, a.fp_magic, a.full_pieces);
    pc.b = div_magic(pc.unit, a.hkv_magic, a.Hkv);
    pc.kvh = pc.unit - pc.b * a.Hkv;
    pc.qgroup = 0;
    pc.nsplit = a.full_pieces;
    pc.split = slot_w - pc.unit * a.full_pieces;
    pc.first = pc.unit * a.full_pieces;
    pc.L = Lcap;
    pc.bad = false;
    const int n_chunks = (Lcap + 31) >> 5;
    R = run_at(pc, div_magic(pc.split * n_chunks, a.fp_magic, a.full_pieces),
               div_magic((pc.split + 1) * n_chunks, a.fp_magic, a.full_pieces));
  };
  if (spec) {
    guess();
    start(pc, R);
  }
  // The committed lengths, lane b holding sequence b's, read once the guess's
  // loads are issued: scalar loads for B <= 16, so that waiting for them does
  // not wait for those vector loads (vector loads complete in order).
  const int kvl0 = kv_len_lanes(a);
  const bool full = guessable && wave_allmin_i(lane < a.B ? (kvl0 == Lcap ? 1 : 0) : 1) == 1;
  if (!full) {
    // slot -> piece (every wave finds it; the committed lengths decide it),
    // while the guessed piece's loads are still in flight; they are waited
    // for and dropped before the slot is used again or the wave ends
    const bool used = plan_piece(a, slot_w, kvl0, pc);
    if (spec) asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    if (!used) return;
    if (pc.bad && a.flags && pc.split == 0 && pc.kvh == 0 && tid == 0)
      atomicOr(a.flags + pc.b, EAGLE_FLAG_BAD_KV_LEN);
    R = run_of(pc);
  } else if (!spec) {
    guess();
  }
  if (!(full && spec)) start(pc, R);
  const int b = pc.b, kvh = pc.kvh, L = pc.L;
  const bool bad = pc.bad;
  const int my_n = R.my_n, my_chunks = R.my_chunks;
  const bool tree_wave = R.tree_wave;
  const bool pre2 = my_chunks >= 2;  // wave-uniform

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
        const int row = qb * 16 + c;
        const uint64_t m = __shfl(t.anc, row < a.M ? row / a.G : 0);
        anc_q[qb] = row < a.M ? m & nmask : 0ull;
      }
      if (kvh == 0) write_tree_outputs(a, b, t);
    } else {
#pragma unroll
      for (int qb = 0; qb < QBW; ++qb) {
        const int row = qb * 16 + c;
        anc_q[qb] = row < a.M ? a.anc[(size_t)b * a.N + row / a.G] & nmask : 0ull;
      }
    }
  }
  const int rows = a.M;  // <= RW

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
    const int key0 = chunk_key0(R, i);
    if (i == 1 && pre2) {
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // the first chunk's reads are done
#pragma unroll
      for (int t = 0; t < LPM; ++t) {
        *reinterpret_cast<u32x4*>(slot + t * RPL * D * 2 + lane * 16) = pre[t];
        *reinterpret_cast<u32x4*>(slot + S::MAT_BYTES + t * RPL * D * 2 + lane * 16) = pre[LPM + t];
      }
    } else if (i == 0 && pre2) {
      // the first chunk has landed: at most the 2 * LPM loads of the second
      // (and any issued after them) are outstanding
      asm volatile("s_waitcnt vmcnt(%0)" ::"n"(2 * LPM) : "memory");
    } else {
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // this wave's chunk has landed
    }
    const bool need_mask = tree_chunk || key0 + 32 > L;
    chunk_step<D, QBW>(slot, qf, anc_q, acc, m_run, l_run, a.scale_log2, need_mask, tree_chunk,
                       tree_bit0, prefix_mask8(key0 + 8 * g, L));
    if (i + 1 < my_chunks && !(i == 0 && pre2)) {
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // this slot's reads are done
      issue_keys_at(R.kp, R.vp, chunk_key0(R, i + 1), chunk_kmax(R, i + 1));
    }
  }

#pragma unroll
  for (int qb = 0; qb < QBW; ++qb) {
    l_run[qb] += __shfl_xor(l_run[qb], 16);
    l_run[qb] += __shfl_xor(l_run[qb], 32);
  }
  // the folded rows go from registers to the output (one piece) or to this
  // piece's partial (O / l and log2-sum-exp)
  float* ml = reinterpret_cast<float*>(lds + S::LDS_RING);
  constexpr int D4 = D / 4;
  auto out_row = [&](int row) {
    const int i = row / a.G;
    const int h = kvh * a.G + (row - i * a.G);
    return a.out + (((size_t)b * a.N + i) * a.Hq + h) * D;
  };
  if (pc.nsplit == 1) {
    fold_waves<QBW, NDB, NWAVE, S::SLOT_BYTES>(
        acc, m_run, l_run, lds, ml, wave, rows, [&](int rl, int db, f32x4 o, float) {
          if (bad) o = f32x4{0.f, 0.f, 0.f, 0.f};
          *reinterpret_cast<u32x2*>(out_row(rl) + db * 16 + 4 * g) =
              u32x2{pack_bf16x2(o[0], o[1]), pack_bf16x2(o[2], o[3])};
        });
    return;
  }
  const size_t pbase = (size_t)slot_w * RW;
  fold_waves<QBW, NDB, NWAVE, S::SLOT_BYTES>(
      acc, m_run, l_run, lds, ml, wave, rows, [&](int rl, int db, f32x4 o, float lse) {
        store_coherent(a.part_o + (pbase + rl) * D + db * 16 + 4 * g, o);
        if (db == 0 && g == 0) store_coherent(a.part_lse + pbase + rl, lse);
      });

  // The unit's last piece to finish combines the partials: each workgroup's
  // coherent stores have completed (vmcnt) before it takes the unit's ticket,
  // and the combining workgroup reads them with coherent loads issued after
  // its ticket returned.
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  int* last = reinterpret_cast<int*>(ml);
  if (tid == 0) {
    const int done =
        __hip_atomic_fetch_add(a.tickets + pc.unit, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    *last = done == pc.nsplit - 1;
    if (done == pc.nsplit - 1)
      __hip_atomic_store(a.tickets + pc.unit, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  __syncthreads();
  if (!*last) return;
  // (row, 4 columns) items: w_s = 2^(lse_s - max), o = sum w_s O_s / sum w_s.
  // The pieces go in batches of 8, and a thread's two items share a batch,
  // so that every load of a batch is issued before any is used.
  const size_t ub = (size_t)pc.first * RW;
  const int total = rows * D4;
  const int S_ = pc.nsplit;
  // the unit's partials as one buffer range (its pieces' slots are consecutive)
  const __amdgpu_buffer_rsrc_t po = buffer_rsrc(a.part_o + ub * D, (size_t)S_ * RW * D * 4);
  for (int it0 = tid; it0 < total; it0 += 2 * S::THREADS) {
    const int its[2] = {it0, it0 + S::THREADS};
    float mt[2] = {-INFINITY, -INFINITY}, lt[2] = {0.f, 0.f};
    f32x4 o[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
    for (int s0 = 0; s0 < S_; s0 += 8) {
      float ls[2][8];
      f32x4 os[2][8];
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int it = its[u] < total ? its[u] : it0;  // a duplicate item is never stored
        const int rl = it / D4, d4 = it - rl * D4;
#pragma unroll
        for (int q = 0; q < 8; ++q) {
          const bool in = s0 + q < S_;
          const int sq = in ? s0 + q : 0;  // in range either way
          ls[u][q] = in ? load_coherent(a.part_lse + ub + (size_t)sq * RW + rl) : -INFINITY;
          os[u][q] = in ? load_coherent4(po, (uint32_t)(((sq * RW + rl) * D + 4 * d4) * 4))
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
          const float wq = ls[u][q] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(ls[u][q] - mb);
          lt[u] += wq;
          o[u] += os[u][q] * wq;
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
// group kernel: a head group's query rows share a ring of K/V tiles in LDS
// ============================================================================
// Grouped-query attention with up to 256 query rows per (b, KV head): eight
// waves, each owning 32 of the rows, compute every 64-key tile of the piece
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
// frees the buffer of tile i - 1 for tile i + NBUF - 1.  The last piece also
// computes the tree keys [L, L + N) as one more tile.  Rows O / l and
// log2-sum-exp of a piece go straight from registers to the partials, which
// the merge kernel combines (the unit's last piece combining them, as the
// ring kernel does, took longer: 63 against 59 us at the llama2-70b shape,
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

  const int slot_w = logical_slot(a);
  const uint32_t lds_base = (uint32_t)(size_t)(__attribute__((address_space(3))) uint8_t*)lds;
  const int r_in = lane / SPR, p_in = lane % SPR;
  // tile position j: keys key0.. (chunk h at key0 + 32 h), rows past key_max
  // re-read it (a key of J, masked later)
  auto issue_tile_at = [&](const uint16_t* kp, const uint16_t* vp, int j, int key0, int key_max) {
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

  // As in the ring kernel: the first tiles of the piece this slot would hold
  // if every sequence filled the cache go out before the plan is known, and
  // are kept only if the real plan agrees (else waited for and discarded).
  // (no division before those loads, and the lengths read after them)
  const int Lcap = a.Lmax - a.N;
  const int cap_tiles = (Lcap + S::TILE_KEYS - 1) / S::TILE_KEYS;
  const int U = a.Hkv * a.qgroups;
  int spec_unit = -1, spec_split = 0, spec_n = 0;
  if (a.full_pieces > 0 && slot_w < a.B * U * a.full_pieces) {
    spec_unit = div_magic(slot_w, a.fp_magic, a.full_pieces);
    spec_split = slot_w - spec_unit * a.full_pieces;
    const int stb = div_magic(spec_split * cap_tiles, a.fp_magic, a.full_pieces);
    const int ste = div_magic((spec_split + 1) * cap_tiles, a.fp_magic, a.full_pieces);
    spec_n = min(NBUF - 1, ste - stb);
    const int pair = div_magic(spec_unit, a.qg_magic, a.qgroups);  // b * Hkv + kvh
    const size_t sbase = (size_t)pair * (size_t)a.Lmax * D;
    for (int j = 0; j < spec_n; ++j)
      issue_tile_at(a.k + sbase, a.v + sbase, j, (stb + j) * S::TILE_KEYS, Lcap - 1);
  }
  const int kvl0 = kv_len_lanes(a);
  Piece u;
  if (!plan_piece(a, slot_w, kvl0, u)) {
    if (spec_n > 0) asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    return;
  }
  const int L = u.L;
  if (tid == 0) {
    if (u.bad && a.flags && u.split == 0 && u.qgroup == 0 && u.kvh == 0)
      atomicOr(a.flags + u.b, EAGLE_FLAG_BAD_KV_LEN);
    if (u.split == 0 && a.unit_info) {  // for the merge kernel (absent: one piece per unit)
      a.unit_info[2 * u.unit] = u.first;
      a.unit_info[2 * u.unit + 1] = u.nsplit;
    }
  }
  const int r0 = wave * QBW * 16;                 // this wave's first row in the unit
  const bool active = u.qgroup * RW + r0 < a.M;  // wave-uniform: the wave has rows

  // this piece's 64-key tiles of [0, L); the last piece adds the tree tile
  const int n_tiles = (L + S::TILE_KEYS - 1) / S::TILE_KEYS;
  const int tb = (int)((long long)u.split * n_tiles / u.nsplit);
  const int te = (int)((long long)(u.split + 1) * n_tiles / u.nsplit);
  const int n_pre = te - tb;
  const bool tree_split = u.split == u.nsplit - 1;
  const int n_my = n_pre + (tree_split ? 1 : 0);

  const size_t kv_base = ((size_t)u.b * a.Hkv + u.kvh) * (size_t)a.Lmax * D;
  const uint16_t* kp = a.k + kv_base;
  const uint16_t* vp = a.v + kv_base;
  auto issue = [&](int j) {
    if (j < n_pre)
      issue_tile_at(kp, vp, j, (tb + j) * S::TILE_KEYS, L - 1);
    else
      issue_tile_at(kp, vp, j, L, L + a.N - 1);  // the tree tile
  };
  // the tiles the speculation issued are those of positions 0..spec_n - 1
  // when the plans agree (then spec_n <= n_pre)
  const bool spec_kept = spec_n > 0 && spec_unit == u.unit && spec_split == u.split &&
                         u.nsplit == a.full_pieces && L == Lcap;
  if (spec_n > 0 && !spec_kept) asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // discarded
  const int n_pro = min(NBUF - 1, n_my);
  for (int j = spec_kept ? spec_n : 0; j < n_pro; ++j) issue(j);

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

  // committed tiles; the tree tile (position n_pre, if this piece has it)
  // after the loop, so that the loop body has no join for the compiler to copy at
  for (int i = 0; i < n_pre; ++i) {
    wait_tiles_after<LPW>(min(NBUF - 2, n_my - 1 - i));
    barrier_lds();  // tile i is whole; every wave is done with tile i - 1
    if (i + NBUF - 1 < n_my) issue(i + NBUF - 1);
    const uint8_t* tile = lds + (i % NBUF) * S::TILE_BYTES;
    const int key0 = (tb + i) * S::TILE_KEYS;
    // one chunk after the other (measured against both chunks' S first:
    // llama2-70b 58.3 against 59.4 us, Mixtral shape 181.3 against 184.9)
    f32x4 s0[QBW][2], s1[QBW][2];
    bf16x8 pf[QBW];
    chunk_qk<D, QBW>(tile, qf, s0);
    chunk_soft<D, QBW>(s0, anc_q, acc, m_run, l_run, pf, a.scale_log2, key0 + 32 > L, false, 0,
                       prefix_mask8(key0 + 8 * g, L));
    chunk_pv<D, QBW>(tile, pf, acc);
    chunk_qk<D, QBW>(tile + S::SLOT_BYTES, qf, s1);
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
  const size_t pbase = (size_t)slot_w * RW;
#pragma unroll
  for (int qb = 0; qb < QBW; ++qb) {
    const int rl = r0 + qb * 16 + c;
    const int row = u.qgroup * RW + rl;
    if (row >= a.M) continue;
    if (u.nsplit == 1) {
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
// merge (group kernel): the pieces' partials of a query row combined
// ============================================================================
// A thread per 16-byte column of a row (D / 4 threads per row): it loads the
// log2-sum-exp and the O / l column of every piece, eight pieces at a time
// with every load of a batch issued before any is used, rescales online, and
// writes four bf16 outputs.  The pieces of a unit (first slot, count) come
// from the group kernel through the workspace (scalar loads); the kernel
// boundary makes them and the partials visible.  The first batch is loaded
// for the pieces the unit has when every sequence fills the cache while the
// piece table is read, and again only if the table disagrees.  A unit's
// workgroups are consecutive ids of one XCD (ids go to the XCDs round robin),
// the units spread evenly over the XCDs.
template <int D>
__global__ __launch_bounds__(256) void tree_attn_merge_kernel(AttnArgs a, int RW, int units) {
  constexpr int C4 = D / 4;        // 16-byte columns per row
  constexpr int RPB = 256 / C4;    // rows per workgroup
  const int bpu = RW / RPB;
  const int per_xcd = (units + kNumXCDs - 1) / kNumXCDs;
  const int q = (int)blockIdx.x / kNumXCDs;
  const int unit = ((int)blockIdx.x % kNumXCDs) * per_xcd + q / bpu;
  if (unit >= units || q / bpu >= per_xcd) return;
  const int first = load_uniform(a.unit_info + 2 * unit);
  const int S = load_uniform(a.unit_info + 2 * unit + 1);
  const int rl = (q % bpu) * RPB + threadIdx.x / C4;
  const int d4 = threadIdx.x % C4;
  const int qgroup = unit % a.qgroups;
  const int pair = unit / a.qgroups;
  const int kvh = pair % a.Hkv;
  const int b = pair / a.Hkv;
  const int row = qgroup * RW + rl;
  const bool has_row = row < a.M;
  float ls[8];
  f32x4 os[8];
  auto load_batch = [&](int fst, int cnt, int s0) {
    const size_t base = (size_t)fst * RW + rl;
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const bool in = s0 + k < cnt;
      const size_t r = base + (size_t)(in ? s0 + k : 0) * RW;  // in range either way
      ls[k] = in ? a.part_lse[r] : -INFINITY;
      os[k] = in ? *reinterpret_cast<const f32x4*>(a.part_o + r * D + 4 * d4)
                 : f32x4{0.f, 0.f, 0.f, 0.f};
    }
  };
  const int fp = a.full_pieces;
  const bool guess = fp > 1 && (long long)(unit + 1) * fp <= a.slots;
  if (guess && has_row) load_batch(unit * fp, fp, 0);
  if (S <= 1 || !has_row) return;  // a single piece wrote the output itself
  if (!guess || first != unit * fp || S != fp) load_batch(first, S, 0);
  const int Lb = a.kv_len[b];
  const bool bad = Lb < 0 || Lb > a.Lmax - a.N;
  const int i = row / a.G;
  const int h = kvh * a.G + (row - i * a.G);
  float mt = -INFINITY, lt = 0.f;
  f32x4 o = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int s0 = 0; s0 < S; s0 += 8) {
    if (s0 > 0) load_batch(first, S, s0);
    float mb = mt;
#pragma unroll
    for (int k = 0; k < 8; ++k) mb = fmaxf(mb, ls[k]);
    if (mb == -INFINITY) continue;
    const float f = mt == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(mt - mb);
    lt *= f;
    o *= f;
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const float w = ls[k] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(ls[k] - mb);
      lt += w;
      o += os[k] * w;
    }
    mt = mb;
  }
  const float inv = (bad || lt == 0.f) ? 0.f : 1.f / lt;
  uint16_t* orow = a.out + (((size_t)b * a.N + i) * a.Hq + h) * D + 4 * d4;
  *reinterpret_cast<u32x2*>(orow) =
      u32x2{pack_bf16x2(o[0] * inv, o[1] * inv), pack_bf16x2(o[2] * inv, o[3] * inv)};
}

// ---- host plan -------------------------------------------------------------------
namespace {
constexpr int kMaxPiecesPerUnit = 1024;

// Test-only override of the planner's choices (eagle_testing_attn_plan).
struct PlanOverride {
  int kernel;  // 0: planner's choice, 1: ring, 2: group
  int pieces;  // 0: planner's choice, else pieces per unit at full length
};
PlanOverride g_plan_override{0, 0};

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }
int round8(long long x) { return (int)((x + kNumXCDs - 1) / kNumXCDs * kNumXCDs); }
}  // namespace

void set_attn_plan_override(int kernel, int pieces) {
  g_plan_override.kernel = kernel;
  g_plan_override.pieces = pieces;
}

AttnPlan plan_tree_attn(int B, int N, int Hq, int Hkv, int d, int Lmax) {
  AttnPlan p{};
  p.d = d;
  p.G = Hq / Hkv;
  p.M = p.G * N;
  int kernel = p.M <= 32 ? 1 : 2;
  if (g_plan_override.kernel == 1 || g_plan_override.kernel == 2) kernel = g_plan_override.kernel;
  if (kernel == 1 && p.M > 32) {
    p.kernel = -1;  // the ring kernel holds at most 32 query rows per KV head
    return p;
  }
  p.kernel = kernel;
  if (kernel == 1) {
    p.rows_per_wg = p.M <= 16 ? 16 : 32;
    p.kg = 32;
    p.qgroups = 1;
  } else {
    p.rows_per_wg = 256;
    p.kg = 64;
    p.qgroups = (p.M + 255) / 256;
  }
  p.units = B * Hkv * p.qgroups;
  p.max_pieces = kMaxPiecesPerUnit;
  // Pieces per unit at full length (the cache capacity); the device shares
  // the resulting slots out by the actual committed lengths.
  const int cap_chunks = std::max(1, (Lmax - N + p.kg - 1) / p.kg);
  int pieces;
  if (kernel == 1) {
    // The ring kernel's order of decompositions at full cache length (the
    // device applies the same one to the committed lengths, see plan_piece).
    pieces = 1;
    int best_r = 0, best_t = 0;
    for (int k = 1; k <= 16 && k <= cap_chunks; ++k) {
      const int t = (cap_chunks + k - 1) / k;
      const int s = std::min((cap_chunks + t - 1) / t, kMaxPiecesPerUnit);
      const int r = ring_rounds((long long)p.units * s), te = ring_piece_len(t, cap_chunks);
      if (best_t == 0 || r < best_r || (r == best_r && te < best_t)) {
        best_r = r;
        best_t = te;
        pieces = s;
      }
    }
  } else {
    // grouped queries: about one workgroup per CU (measured on MI355X:
    // llama2-70b 4 pieces, 59.3 us against 68.2 at 3 and 74.9 at 8;
    // mixtral shape 2 pieces, 186.8 us against 220.7 at 3)
    pieces = (kNumCUs + round8(p.units) - 1) / round8(p.units);
  }
  // the ring kernel's device planner applies its order to the committed
  // lengths unless a test fixed the piece count
  p.ring_cost = kernel == 1 && g_plan_override.pieces <= 0 ? 1 : 0;
  if (g_plan_override.pieces > 0) pieces = g_plan_override.pieces;
  pieces = std::max(1, std::min(pieces, std::min(cap_chunks, kMaxPiecesPerUnit)));
  p.slots = round8((long long)p.units * pieces);
  // the ring kernel launches at least a round of workgroups (up to 16 pieces
  // per unit) even when the units fill fewer CUs at full length: committed
  // lengths below the capacity then cut their longest sequences into more
  // pieces on the idle CUs (unused slots plan and return)
  if (p.ring_cost)
    p.slots = std::max(p.slots, round8(std::min<long long>(
                                    kNumCUs, (long long)p.units * std::min(16, cap_chunks))));
  if (p.ring_cost) {
    // at full length the device's order makes the same choice
    p.full_pieces = pieces;
  } else {
    // what the device planner gives every unit when all sequences fill the
    // cache: the smallest piece T (in chunks) with units * ceil(C / T) <= slots
    const int per_unit = p.slots / p.units;
    const int T =
        per_unit >= kMaxPiecesPerUnit ? 1 : std::max(1, (cap_chunks + per_unit - 1) / per_unit);
    p.full_pieces = std::max(1, std::min(kMaxPiecesPerUnit, (cap_chunks + T - 1) / T));
  }
  return p;
}

size_t tree_attn_workspace_bytes(const AttnPlan& p) {
  if (p.kernel < 0 || p.slots <= p.units) return 0;
  return align256((size_t)p.units * 8) + align256((size_t)p.slots * p.rows_per_wg * 4) +
         (size_t)p.slots * p.rows_per_wg * p.d * 4;
}

template <int D>
static void* attn_kernel(int kernel, int rows_per_wg) {
  if (kernel == 2) return (void*)tree_attn_group_kernel<GroupShape<D>>;
  return rows_per_wg == 16 ? (void*)tree_attn_ring_kernel<RingShape<D, 1>>
                           : (void*)tree_attn_ring_kernel<RingShape<D, 2>>;
}

// ---- scratch of the entry point that allocates nothing ------------------------------
// eagle_tree_attn_parents_noalloc keeps its workspace (piece tickets or table,
// partials) here instead of in a caller's buffer.  Each device holds its own
// copy for the life of the process; host code reaches it only through the
// address hipGetSymbolAddress returns with that device current, recorded
// once per device.
static __device__ __align__(256) uint8_t scratch[kStaticScratchBytes];

namespace {
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxScratchDevices];
}  // namespace

hipError_t static_scratch(void** ptr) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxScratchDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return hipSuccess;
}

size_t tree_attn_zeroed_bytes(const AttnPlan& p) {
  return p.kernel == 1 && p.slots > p.units ? align256((size_t)p.units * 8) : 0;
}

hipError_t launch_tree_attn(const AttnPlan& plan, const uint16_t* q, const uint16_t* k,
                            const uint16_t* v, const int32_t* kv_len, const uint64_t* anc,
                            const int32_t* parents, uint64_t* anc_out, int32_t* depth_out,
                            int32_t* pos_out,
                            int B, int N, int Hq, int Hkv, int Lmax, float scale_log2,
                            uint16_t* out, void* ws, int32_t* flags, hipStream_t s) {
  static_assert(RingShape<64, 1>::THREADS == kRingThreads && RingShape<128, 2>::THREADS == kRingThreads &&
                    GroupShape<128>::THREADS == kRingThreads && GroupShape<64>::THREADS == kRingThreads,
                "launch size");
  if (plan.kernel < 0) return hipErrorInvalidValue;
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
  const bool pieces = plan.slots > plan.units;
  uint8_t* w = static_cast<uint8_t*>(ws);
  if (pieces) {
    const size_t head = align256((size_t)plan.units * 8);
    const size_t lse = align256((size_t)plan.slots * plan.rows_per_wg * 4);
    a.tickets = plan.kernel == 1 ? reinterpret_cast<int32_t*>(w) : nullptr;
    a.unit_info = plan.kernel == 2 ? reinterpret_cast<int32_t*>(w) : nullptr;
    a.part_lse = reinterpret_cast<float*>(w + head);
    a.part_o = reinterpret_cast<float*>(w + head + lse);
  }
  a.flags = flags;
  a.B = B;
  a.N = N;
  a.Hq = Hq;
  a.Hkv = Hkv;
  a.Lmax = Lmax;
  a.G = plan.G;
  a.M = plan.M;
  a.qgroups = plan.qgroups;
  a.slots = plan.slots;
  a.kg = plan.kg;
  a.max_pieces = plan.max_pieces;
  a.full_pieces = Lmax > N ? plan.full_pieces : 0;
  a.ring_cost = plan.ring_cost;
  {
    // the guessed piece's quotients by div_magic need n * d <= 2^32: slot and
    // piece bounds times the piece count, the unit times Hkv or qgroups
    const long long P = std::max(1, a.full_pieces);
    const long long cap = (long long)(Lmax - N) + 64;  // keys (chunks or tiles are fewer)
    const long long units = (long long)B * Hkv * plan.qgroups;
    const long long lim = 1ll << 32;
    if ((long long)plan.slots * P > lim || cap * P * P > lim ||
        units * std::max(Hkv, plan.qgroups) > lim)
      a.full_pieces = 0;  // plan first instead of guessing
  }
  a.fp_magic = magic_of(a.full_pieces);
  a.hkv_magic = magic_of(Hkv);
  a.qg_magic = magic_of(plan.qgroups);
  a.g_magic = magic_of(plan.G);
  a.xcd_group = plan.kernel == 1 && a.full_pieces > 1 && plan.units % kNumXCDs == 0 &&
                        (long long)plan.slots == (long long)plan.units * a.full_pieces
                    ? 1
                    : 0;
  a.scale_log2 = scale_log2;
  void* fn = plan.d == 64 ? attn_kernel<64>(plan.kernel, plan.rows_per_wg)
                          : attn_kernel<128>(plan.kernel, plan.rows_per_wg);
  void* args[] = {&a};
  hipError_t err = hipLaunchKernel(fn, dim3((unsigned)plan.slots), dim3(kRingThreads), args, 0, s);
  // the ring kernel combines its pieces itself
  if (err != hipSuccess || !pieces || plan.kernel == 1) return err;
  const int rw = plan.rows_per_wg;
  const int rows_per_block = 256 / (plan.d / 4);
  const int per_xcd = (plan.units + kNumXCDs - 1) / kNumXCDs;
  const dim3 mgrid((unsigned)(kNumXCDs * per_xcd * (rw / rows_per_block)));
  if (plan.d == 64)
    tree_attn_merge_kernel<64><<<mgrid, 256, 0, s>>>(a, rw, plan.units);
  else
    tree_attn_merge_kernel<128><<<mgrid, 256, 0, s>>>(a, rw, plan.units);
  return hipGetLastError();
}

}  // namespace eagle
