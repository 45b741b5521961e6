// Acceptance walk of the verification step: temperature softmax, multi-round
// speculative sampling over the draft tree, final-token draw.
//
// Speculative sampling accepts a drafted token t with probability
// min(1, p(t)/p_hat(t)) and, after a rejection, draws from an adjusted
// distribution (EAGLE, paperlayer.ai summary, §2 Preliminaries); for a tree the
// procedure is applied recursively over each node's candidates and returns a
// sample of the target distribution (A.2 Multi-Round Speculative Sampling;
// B, the inputs of the procedure).  At temperature 0 the target emits its most
// probable token (EAGLE-2 overview blog, §1).
//
// Layout of the work: one workgroup per tree node, all nodes at once.  The
// outcome at a node (which candidate it accepts, or which token it would emit
// if none) depends only on that node's own row, its candidates' draft rows
// and the uniforms, never on the rest of the walk, so every node computes it
// speculatively in parallel; the last node of a sequence to finish (atomic
// ticket) then follows the accepted candidates from the root, a scalar walk.
//
// Per node j with candidates c_1..c_k (ascending) and T > 0:
//   U_0 = exp((l_j - max) / T) (unnormalised target), C_0 = sum U_0
//   ratio_s = U_{s-1}[t_s] / (C_{s-1} q_s[t_s])       (accept iff u_s < ratio_s)
//   U_s = max(0, U_{s-1} - C_{s-1} q_s),  C_s = sum U_s  (kept if C_s = 0)
// U_s / C_s is the adjusted distribution norm(max(0, r - q)) after s
// rejections.
//
// A node's critical path is a sequence of full-vocabulary passes, each ending
// in a workgroup reduction, so the kernel is built around short passes:
//   * the row lives in registers across the 1024-thread workgroup (8 float4
//     per thread at V <= 32768), entries past V padded so no pass needs a
//     bounds check;
//   * a candidate's draft row is prefetched into LDS with direct-to-LDS loads
//     (each thread's float4 lands where that thread reads it back, so no
//     barrier guards the buffer) and is read once: the pass builds the updated
//     row W = max(0, U - C q) in a second register row (the two rows swap
//     roles each candidate), and the next row's prefetch is issued as soon as
//     this thread's reads are done;
//   * wave reductions use DPP within rows of 16 lanes and readlane across the
//     four rows; a workgroup reduction takes one barrier (two alternating
//     LDS slot sets);
//   * masses: fp32 pairwise sums per thread, fp64 across threads, in a fixed
//     order (deterministic).  The final draw scans in fp64.
#include <float.h>
#include <limits.h>
#include <stdlib.h>

#include <utility>

#include "common.h"
#include "launch.h"

namespace eagle {

// Per-node results published for the walk (device-coherent stores/loads).
struct NodeResults {
  int32_t* acc;      // [B*N] accepted candidate, -1 if none
  int32_t* bonus;    // [B*N] token drawn if the walk ends here
  float* ratio;      // [B*N] ratio of node c as tested by its parent's chain
  int32_t* ntested;  // [B*N] candidates of the node that its chain tested
  int32_t* nphase;   // [B*N] exchange phases the node used (split rows)
  int32_t* counter;  // [B] per-sequence tickets (zero between calls)
};

struct VArgs {
  const int32_t* tokens;
  const float* draft;
  const float* logits;
  const int32_t* parents;
  const int32_t* kv_len;
  const float* uniforms;
  int32_t* accept_len;
  int32_t* path;
  int32_t* acc_tokens;
  int32_t* bonus;
  int32_t* kv_src;
  float* out_probs;
  float* out_final;
  float* out_ratio;
  int32_t* flags;
  NodeResults nr;
  VerifyCompact kc;            // compaction fused into the walk (kc.k == nullptr: none)
  unsigned long long* xwords;  // [B*N][kXPhases][kXWords] exchange words (split rows; zero between calls)
  int N, V;
  int nodes;  // B * N
  int P;      // workgroups per node (split rows when > 1)
  float T;
};

__device__ __forceinline__ void st_c(int32_t* p, int32_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_c(float* p, float v) {
  __hip_atomic_store(reinterpret_cast<uint32_t*>(p), __float_as_uint(v), __ATOMIC_RELAXED,
                     __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ int32_t ld_c(int32_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float ld_c(float* p) {
  return __uint_as_float(
      __hip_atomic_load(reinterpret_cast<uint32_t*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
}

constexpr int kMaxParts = 8;  // split rows: workgroups per node

template <int BLOCK, int NPT>
struct Shared {
  static constexpr int NW = BLOCK / 64;
  int par[64], tok[64], kids[64];
  float u[64];
  float ratio[64];
  float qt[64 * 64];  // qt[k*64 + i] = q_{kid k}(t_{kid i}) for k <= i (T > 0)
  int nk;
  // workgroup reductions: two slot sets, used alternately (see rb below)
  double rd[2][NW];
  float rf[2][NW];
  int ri[2][NW];
  double sel_before;
  int sel_entry;
  int pick;
  double gd[2];  // split rows: broadcast of the cross-workgroup results
  float gf[2];
  double pm[kMaxParts];  // split rows: each part's mass of the current row
  float mp[kMaxParts];   // split rows: each part's own logit maximum
  float fp[kMaxParts];   // split rows: exp((m_p - max) / T), each part's scale
  int xabort;    // split rows: a wait timed out, later waits are skipped
  int last, term;
  int wacc[64], wbonus[64], wnt[64], wph[64];
  int mv[64];      // fused compaction: the path positions whose K/V move
  int nmv, Lkv;
  float l2sink[64];  // split rows: destination of the L2 prefetch (never read)
  int path[64];
};

// Workgroup reductions over the BLOCK row threads (a split-row workgroup's
// extra exchange and prefetch waves hold no row data: they take part in the
// barriers and read the result).  `rb` selects the slot set and flips on every call;
// all threads make the same sequence of calls, so a slot set is rewritten
// only after the barrier of the reduction in between, which every reader of
// its previous contents has passed: one barrier per reduction suffices.
template <int BLOCK, int NPT>
__device__ __forceinline__ double block_sum(double v, Shared<BLOCK, NPT>& sh, int& rb) {
  v = wave_allsum(v);
  const int buf = rb;
  rb ^= 1;
  if ((threadIdx.x & 63) == 0 && threadIdx.x < BLOCK) sh.rd[buf][threadIdx.x >> 6] = v;
  barrier_lds();
  double t = 0.0;
#pragma unroll
  for (int i = 0; i < BLOCK / 64; ++i) t += sh.rd[buf][i];
  return t;
}

template <int BLOCK, int NPT>
__device__ __forceinline__ float block_max(float v, Shared<BLOCK, NPT>& sh, int& rb) {
  v = wave_allmax(v);
  const int buf = rb;
  rb ^= 1;
  if ((threadIdx.x & 63) == 0 && threadIdx.x < BLOCK) sh.rf[buf][threadIdx.x >> 6] = v;
  barrier_lds();
  float t = -INFINITY;
#pragma unroll
  for (int i = 0; i < BLOCK / 64; ++i) t = fmaxf(t, sh.rf[buf][i]);
  return t;
}

template <int BLOCK, int NPT>
__device__ __forceinline__ int block_min_i(int v, Shared<BLOCK, NPT>& sh, int& rb) {
  v = wave_allmin_i(v);
  const int buf = rb;
  rb ^= 1;
  if ((threadIdx.x & 63) == 0 && threadIdx.x < BLOCK) sh.ri[buf][threadIdx.x >> 6] = v;
  barrier_lds();
  int t = INT_MAX;
#pragma unroll
  for (int i = 0; i < BLOCK / 64; ++i) t = min(t, sh.ri[buf][i]);
  return t;
}

template <int BLOCK, int NPT>
__device__ __forceinline__ int block_max_i(int v, Shared<BLOCK, NPT>& sh, int& rb) {
  v = wave_allmax_i(v);
  const int buf = rb;
  rb ^= 1;
  if ((threadIdx.x & 63) == 0 && threadIdx.x < BLOCK) sh.ri[buf][threadIdx.x >> 6] = v;
  barrier_lds();
  int t = INT_MIN;
#pragma unroll
  for (int i = 0; i < BLOCK / 64; ++i) t = max(t, sh.ri[buf][i]);
  return t;
}

// ---- split rows ----------------------------------------------------------------
// With P > 1 the P workgroups of a node each hold a slice of the row and every
// workgroup reduction is completed across them through exchange words in the
// workspace (64-bit atomics, then polling; the P workgroups run on one XCD
// and are all resident, which the host checks).  A split workgroup has two
// waves beyond its BLOCK row threads.  One does the exchange: its polling
// loads never queue behind a row prefetch (a wave's vector loads complete in
// order), so the prefetch of the next draft row stays in flight across the
// exchange.  The other only brings the node's later draft rows into L2 at
// the start, for the same reason.
// Sums travel as fixed point relative to a known bound: every row wave of
// every part writes its partial (value << 8 | 1, never zero) to a slot of its
// own, and the exchange wave reads the P x 4 slots until all are written, so
// every part forms the same exact integer total, and the same per-part
// masses, which the final draw uses to find the part that holds its crossing
// without another exchange.  A max travels as an order-preserving 32-bit
// key with a separate count.  A wait that exceeds kSpinCap polls sets
// EAGLE_FLAG_TIMEOUT and skips later waits.
constexpr int kXWords = kMaxParts * 5;  // words per phase: one per (part, row wave), one per part
constexpr int kXPhases = 72;            // phases per node: row statistics, candidates
constexpr int kSpinCap = 1 << 20;
constexpr double kFix = 1125899906842624.0;  // 2^50

// round(x) for 0 <= x < 2^51 as an integer: adding 1.5 * 2^52 leaves a sum
// whose last mantissa bit weighs 1, so the addition itself rounds to nearest
// (even), and the integer is the difference of the bit patterns.
__device__ __forceinline__ unsigned long long fix_round(double x) {
  constexpr double kMagic = 6755399441055744.0;  // 1.5 * 2^52
  return (unsigned long long)(__double_as_longlong(x + kMagic) - __double_as_longlong(kMagic));
}

struct Grp {
  unsigned long long* words;  // this node's exchange words
  int P, part, phase;
  int base, len;              // this part's slice of the row: ids [base, base + len)
  int32_t* flags;
  int b;
  int xt;                     // the thread that exchanges (lane 0 of the exchange wave)
};

__device__ __forceinline__ unsigned long long* grp_phase_words(Grp& g) {
  return g.words + (size_t)g.phase * kXWords;
}

// Polls *w until its low 8 bits reach `need`; returns the last value read.
template <int BLOCK, int NPT>
__device__ __forceinline__ unsigned long long grp_wait(unsigned long long* w, unsigned long long cur,
                                                       int need, Grp& g, Shared<BLOCK, NPT>& sh) {
  int it = 0;
#pragma nounroll
  while ((int)(cur & 0xffull) < need && !sh.xabort) {
    if (++it > kSpinCap) {
      sh.xabort = 1;
      if (g.flags) atomicOr(g.flags + g.b, EAGLE_FLAG_TIMEOUT);
      break;
    }
    cur = __hip_atomic_load(w, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  return cur;
}

// Sum over the node's workgroups of v >= 0, with 0 <= total <= scale; inv is
// kFix / scale (computed by the caller ahead of the reduction).  mid() runs on
// every thread while the exchange is in flight (after the workgroup reduction
// when P = 1); it must issue no memory access from the exchange wave.
// Split rows: every row wave adds its own partial (fixed point, count 1) to
// the phase word of its wave index without waiting, so no workgroup barrier
// precedes the exchange; the exchange wave polls the BLOCK / 64 words until
// each holds P arrivals, and their integer total is the same in every
// workgroup.
template <int BLOCK, int NPT, typename F>
__device__ __forceinline__ double grp_sum(double v, double scale, double inv, Grp& g,
                                          Shared<BLOCK, NPT>& sh, int& rb, F&& mid) {
  constexpr int NW = BLOCK / 64;
  // (split rows run 256-thread workgroups; wider ones always have P = 1)
  if (NW != 4 || g.P == 1) {
    v = block_sum<BLOCK, NPT>(v, sh, rb);
    mid();
    return v;
  }
  const int tid = threadIdx.x, lane = tid & 63;
  const int slot = g.phase & 1;
  unsigned long long* w = grp_phase_words(g);
  if (tid < BLOCK) {
    v = wave_allsum(v);
    if (lane == 0)  // an add into a zero word: atomics meet at the memory side, as the polls do
      __hip_atomic_fetch_add(w + g.part * NW + (tid >> 6), (fix_round(v * inv) << 8) | 1ull,
                             __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  mid();  // guarded by the caller: no loads from the exchange wave
  if ((tid >> 6) == (g.xt >> 6)) {
    // the exchange wave: lane l < P * NW reads slot l (part l / NW)
    const int nslots = g.P * NW;
    unsigned long long x = 1ull;
    int it = 0;
#pragma nounroll
    for (;;) {
      if (lane < nslots) x = __hip_atomic_load(w + lane, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      if (__all(x != 0ull) || sh.xabort) break;
      if (++it > kSpinCap) {
        if (lane == 0) {
          sh.xabort = 1;
          if (g.flags) atomicOr(g.flags + g.b, EAGLE_FLAG_TIMEOUT);
        }
        break;
      }
    }
    // integers below 2^53: exact in fp64, in any order
    double q = lane < nslots ? (double)(x >> 8) : 0.0;
    q += dpp_d<kDppXor1>(q);  // the NW = 4 waves of a part are one quad
    q += dpp_d<kDppXor2>(q);
    const double tot = wave_allsum(lane < nslots && (lane & 3) == 0 ? q : 0.0);
    const double unit = scale / kFix;
    if (tot > 0.0 && lane < nslots && (lane & 3) == 0) sh.pm[lane >> 2] = q * unit;
    if (lane == 0) sh.gd[slot] = tot * unit;
  }
  ++g.phase;
  barrier_lds();
  return sh.gd[slot];
}
template <int BLOCK, int NPT>
__device__ __forceinline__ double grp_sum(double v, double scale, double inv, Grp& g,
                                          Shared<BLOCK, NPT>& sh, int& rb) {
  return grp_sum<BLOCK, NPT>(v, scale, inv, g, sh, rb, [] {});
}

template <int BLOCK, int NPT>
__device__ __forceinline__ float grp_max(float v, Grp& g, Shared<BLOCK, NPT>& sh, int& rb) {
  v = block_max<BLOCK, NPT>(v, sh, rb);
  if (g.P == 1) return v;
  const int slot = g.phase & 1;
  if (threadIdx.x == g.xt) {
    unsigned long long* w = grp_phase_words(g);
    const uint32_t bits = __float_as_uint(v);
    const uint32_t key = (bits & 0x80000000u) ? ~bits : (bits | 0x80000000u);
    __hip_atomic_fetch_max(reinterpret_cast<uint32_t*>(w), key, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // the key is in before the count
    unsigned long long cur = __hip_atomic_fetch_add(w + 1, 1ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) + 1ull;
    grp_wait<BLOCK, NPT>(w + 1, cur, g.P, g, sh);
    const uint32_t k = __hip_atomic_load(reinterpret_cast<uint32_t*>(w), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    sh.gf[slot] = __uint_as_float((k & 0x80000000u) ? (k & 0x7fffffffu) : ~k);
  }
  ++g.phase;
  barrier_lds();
  return sh.gf[slot];
}

// True in the waves that hold row data (all but a split workgroup's exchange
// wave).  Read from the first lane so the compiler sees a wave-uniform
// branch: loads issued under it then land in their destination registers
// without a merge copy that would wait for them.
template <int BLOCK>
__device__ __forceinline__ bool row_wave() {
  return __builtin_amdgcn_readfirstlane(threadIdx.x) < BLOCK;
}

// ---- rows --------------------------------------------------------------------
// A vocabulary row across the workgroup: thread t owns elements
// (k * BLOCK + t) * 4 + e, k < NPT, e < 4 ("slab" k, coalesced float4 loads).
template <int BLOCK, int NPT>
struct Row {
  float4 v[NPT];
};

__device__ __forceinline__ float comp(const float4& f, int e) {
  return e == 0 ? f.x : e == 1 ? f.y : e == 2 ? f.z : f.w;
}

// Logit row into registers; entries past V read as -FLT_MAX (no mass, never
// the maximum of a row that has a finite entry).
template <int BLOCK, int NPT>
__device__ __forceinline__ void load_logits(Row<BLOCK, NPT>& r, const float* src, int V) {
  const int tid = threadIdx.x;
  // every load is issued at an in-range address and the padding selected
  // afterwards, so the loads need no branches
  const bool row = tid < BLOCK;  // not an extra wave of a split workgroup
  if ((V & 3) == 0) {
#pragma unroll
    for (int k = 0; k < NPT; ++k) {
      const int e0 = (k * BLOCK + tid) * 4;
      const bool in = row && e0 < V;
      const float4 x = *reinterpret_cast<const float4*>(src + (in ? e0 : 0));
      r.v[k] = in ? x : make_float4(-FLT_MAX, -FLT_MAX, -FLT_MAX, -FLT_MAX);
    }
  } else {
#pragma unroll
    for (int k = 0; k < NPT; ++k) {
      const int e0 = (k * BLOCK + tid) * 4;
      const float x0 = src[min(e0 + 0, V - 1)], x1 = src[min(e0 + 1, V - 1)];
      const float x2 = src[min(e0 + 2, V - 1)], x3 = src[min(e0 + 3, V - 1)];
      r.v[k].x = row && e0 + 0 < V ? x0 : -FLT_MAX;
      r.v[k].y = row && e0 + 1 < V ? x1 : -FLT_MAX;
      r.v[k].z = row && e0 + 2 < V ? x2 : -FLT_MAX;
      r.v[k].w = row && e0 + 3 < V ? x3 : -FLT_MAX;
    }
  }
}

// exp(z) for z <= 0 as 2^(z log2 e) with the rounding error of the product
// carried as a first-order correction (relative error ~2 ulp).  Arguments
// below -110 (results below the fp32 range) are clamped, which keeps the
// correction finite for the -FLT_MAX padding.
__device__ __forceinline__ float exp_neg(float z) {
  z = fmaxf(z, -110.f);
  constexpr float kL2E = 1.44269502162933349609375f;  // log2(e), fp32 head
  constexpr float kL2ELo = 1.925963033500011e-08f;    // log2(e) - kL2E
  constexpr float kLn2 = 0.693147180559945309f;
  const float t = z * kL2E;
  const float err = fmaf(z, kL2ELo, fmaf(z, kL2E, -t));
  const float r = __builtin_amdgcn_exp2f(t);
  return fmaf(r, err * kLn2, r);
}

__device__ __forceinline__ float sum4(const float4& f) { return (f.x + f.y) + (f.z + f.w); }

template <int NPT>
__device__ __forceinline__ float pairwise(const float (&s)[NPT]) {
  if constexpr (NPT == 16) {
    return (((s[0] + s[1]) + (s[2] + s[3])) + ((s[4] + s[5]) + (s[6] + s[7]))) +
           (((s[8] + s[9]) + (s[10] + s[11])) + ((s[12] + s[13]) + (s[14] + s[15])));
  } else if constexpr (NPT == 8) {
    return ((s[0] + s[1]) + (s[2] + s[3])) + ((s[4] + s[5]) + (s[6] + s[7]));
  } else {
    static_assert(NPT == 4, "rows of 4, 8 or 16 float4 per thread");
    return (s[0] + s[1]) + (s[2] + s[3]);
  }
}

// The scaled exponent of one logit, exactly as the row pass computes it
// (non-finite logits have no mass).
__device__ __forceinline__ float target_entry(float x, float m, bool unit, float invT) {
  x = isfinite(x) ? x : -FLT_MAX;
  return exp_neg(unit ? x - m : (x - m) * invT);
}

// Split rows: a row's maximum and mass in one exchange.  Each part has
// scaled its slice by its own maximum m_loc (U = exp((l - m_loc) / T),
// entries <= 1, 1024 per row wave).  Every row wave adds its partial mass to
// its slot and wave 0 also posts m_loc (an order-preserving key); every part
// then forms, with the same operations, the maximum M, the factors
// f_p = exp((m_p - M) / T), each part's mass f_p S_p and the total in a fixed
// order.  The caller rescales its slice by f_part.  Returns the total.
template <int BLOCK, int NPT>
__device__ __forceinline__ double grp_stats(double v, float m_loc, bool unit, float invT, Grp& g,
                                            Shared<BLOCK, NPT>& sh) {
  constexpr int NW = BLOCK / 64;
  static_assert(NW == 4, "split rows: four row waves");
  const int tid = threadIdx.x, lane = tid & 63;
  const int slot = g.phase & 1;
  unsigned long long* w = grp_phase_words(g);
  const int nsum = g.P * NW;
  if (tid < BLOCK) {
    v = wave_allsum(v);
    if (lane == 0) {
      __hip_atomic_fetch_add(w + g.part * NW + (tid >> 6), (fix_round(v * (kFix / 1024.0)) << 8) | 1ull,
                             __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      if (tid == 0) {
        const uint32_t bits = __float_as_uint(m_loc);
        const uint32_t key = (bits & 0x80000000u) ? ~bits : (bits | 0x80000000u);
        __hip_atomic_fetch_add(w + nsum + g.part, ((unsigned long long)key << 8) | 1ull,
                               __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
    }
  }
  if ((tid >> 6) == (g.xt >> 6)) {
    // the exchange wave: lanes [0, nsum) read the mass slots, lanes
    // [nsum, nsum + P) the maxima
    const int nslots = nsum + g.P;
    unsigned long long x = 1ull;
    int it = 0;
#pragma nounroll
    for (;;) {
      if (lane < nslots) x = __hip_atomic_load(w + lane, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      if (__all(x != 0ull) || sh.xabort) break;
      if (++it > kSpinCap) {
        if (lane == 0) {
          sh.xabort = 1;
          if (g.flags) atomicOr(g.flags + g.b, EAGLE_FLAG_TIMEOUT);
        }
        break;
      }
    }
    const bool is_max = lane >= nsum && lane < nslots;
    const uint32_t k = (uint32_t)(x >> 8);
    const float mp = is_max ? __uint_as_float((k & 0x80000000u) ? (k & 0x7fffffffu) : ~k) : -INFINITY;
    const float M = wave_allmax(mp);
    const float f = is_max ? exp_neg(unit ? mp - M : (mp - M) * invT) : 0.f;
    if (is_max) {
      sh.mp[lane - nsum] = mp;
      sh.fp[lane - nsum] = f;
    }
    // integers below 2^53: exact in fp64, in any order
    double q = lane < nsum ? (double)(x >> 8) : 0.0;
    q += dpp_d<kDppXor1>(q);  // the NW = 4 waves of a part are one quad
    q += dpp_d<kDppXor2>(q);
    const float fq = __shfl(f, nsum + (lane >> 2));  // the factor of this lane's part
    const double mass = lane < nsum && (lane & 3) == 0 ? (double)fq * q * (1024.0 / kFix) : 0.0;
    const double tot = wave_allsum(mass);
    if (lane < nsum && (lane & 3) == 0) sh.pm[lane >> 2] = mass;
    if (lane == 0) sh.gd[slot] = tot;
  }
  ++g.phase;
  barrier_lds();
  return sh.gd[slot];
}

// Target row statistics of one node from its logits (already in U): flags
// non-finite logits (they are given no mass); T = 0 returns the lowest-index
// argmax; T > 0 turns U into exp((l - max)/T) and returns its mass in C.
// before_sum(buf, m, unit, invT) runs before the mass reduction, whose
// barrier (slot set buf, also returned in sum_buf) publishes what it writes.
template <int BLOCK, int NPT, bool GREEDY, typename F>
__device__ __forceinline__ int target_stats(Row<BLOCK, NPT>& U, float T, int b, int32_t* flags,
                                            double& C, int& sum_buf, F&& before_sum, Grp& grp,
                                            Shared<BLOCK, NPT>& sh, int& rb) {
  const int tid = threadIdx.x;
  // x * 0 is NaN exactly for non-finite x: one fma per entry
  float bad = 0.f;
#pragma unroll
  for (int k = 0; k < NPT; ++k) {
    bad = fmaf(U.v[k].x, 0.f, bad);
    bad = fmaf(U.v[k].y, 0.f, bad);
    bad = fmaf(U.v[k].z, 0.f, bad);
    bad = fmaf(U.v[k].w, 0.f, bad);
  }
  const bool nonfinite = bad != bad;
  if (nonfinite) {
#pragma unroll
    for (int k = 0; k < NPT; ++k) {
      float4& f = U.v[k];
      f.x = isfinite(f.x) ? f.x : -FLT_MAX;
      f.y = isfinite(f.y) ? f.y : -FLT_MAX;
      f.z = isfinite(f.z) ? f.z : -FLT_MAX;
      f.w = isfinite(f.w) ? f.w : -FLT_MAX;
    }
  }
  if (__ballot(nonfinite) && (tid & 63) == 0 && flags) atomicOr(flags + b, EAGLE_FLAG_NONFINITE);

  if constexpr (GREEDY) {
    float lm = -INFINITY;
    int li = INT_MAX;
#pragma unroll
    for (int k = 0; k < NPT; ++k)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float x = comp(U.v[k], e);
        const bool gt = x > lm;  // ids increase with (k, e): first maximum kept
        lm = gt ? x : lm;
        li = gt ? (k * BLOCK + tid) * 4 + e : li;
      }
    const float mx = block_max<BLOCK, NPT>(lm, sh, rb);
    const int am = block_min_i<BLOCK, NPT>(lm == mx ? li : INT_MAX, sh, rb);
    C = 1.0;
    sum_buf = 0;
    return am == INT_MAX ? 0 : am;
  } else {
    float lm = -INFINITY;
#pragma unroll
    for (int k = 0; k < NPT; ++k)
      lm = fmaxf(lm, fmaxf(fmaxf(U.v[k].x, U.v[k].y), fmaxf(U.v[k].z, U.v[k].w)));
    const bool split = BLOCK == 256 && grp.P > 1;
    // split rows: this part's own maximum (the global one comes with the mass)
    const float m = split ? block_max<BLOCK, NPT>(lm, sh, rb) : grp_max<BLOCK, NPT>(lm, grp, sh, rb);
    const bool unit = T == 1.f;
    const float invT = 1.f / T;
    float s[NPT];
#pragma unroll
    for (int k = 0; k < NPT; ++k) {
      float4& f = U.v[k];
      f.x = exp_neg(unit ? f.x - m : (f.x - m) * invT);  // already finite
      f.y = exp_neg(unit ? f.y - m : (f.y - m) * invT);
      f.z = exp_neg(unit ? f.z - m : (f.z - m) * invT);
      f.w = exp_neg(unit ? f.w - m : (f.w - m) * invT);
      s[k] = sum4(f);
    }
    sum_buf = rb;
    before_sum(sum_buf, m, unit, invT);
    if constexpr (BLOCK == 256) {
      if (split) {
        C = grp_stats<BLOCK, NPT>((double)pairwise<NPT>(s), m, unit, invT, grp, sh);
        const float f = sh.fp[grp.part];
#pragma unroll
        for (int k = 0; k < NPT; ++k) {
          U.v[k].x *= f;
          U.v[k].y *= f;
          U.v[k].z *= f;
          U.v[k].w *= f;
        }
        return 0;
      }
    }
    // entries <= 1, V <= 32768
    C = grp_sum<BLOCK, NPT>((double)pairwise<NPT>(s), 32768.0, kFix / 32768.0, grp, sh, rb);
    return 0;
  }
}

// Children of node j in ascending order into sh.kids / sh.nk.  Wave 0 only;
// the caller synchronises.
template <int BLOCK, int NPT>
__device__ __forceinline__ void find_kids(int N, int j, Shared<BLOCK, NPT>& sh) {
  const int lane = threadIdx.x & 63;
  if (threadIdx.x >= 64) return;
  const bool kid = lane < N && lane > j && sh.par[lane] == j;
  const uint64_t mask = __ballot(kid);
  if (kid) sh.kids[__popcll(mask & ((1ull << lane) - 1ull))] = lane;
  if (lane == 0) sh.nk = __popcll(mask);
}

// f(std::integral_constant<int, J>) for J = 0..N-1, unrolled.
template <typename F, int... J>
__device__ __forceinline__ void unroll_seq(F&& f, std::integer_sequence<int, J...>) {
  (f(std::integral_constant<int, J>{}), ...);
}
template <int N, typename F>
__device__ __forceinline__ void unroll(F&& f) {
  unroll_seq(f, std::make_integer_sequence<int, N>{});
}

// Position of q_{kid k}(t_{kid i}), k <= i < nk, in sh.qt.
__device__ __forceinline__ int tri(int k, int i, int) { return k * 64 + i; }

// A draft row -> LDS with direct-to-LDS loads: thread t's float4 k lands at
// LDS float4 k*BLOCK + t, where only thread t reads it back.  Slots past V are
// not loaded (zeroed once by node_setup).  V % 4 == 0.
template <int BLOCK, int NPT>
__device__ __forceinline__ void issue_row_lds(const float* row, int V, float4* qlds) {
  const int tid = threadIdx.x, wave = tid >> 6;
#pragma unroll
  for (int k = 0; k < NPT; ++k) {
    const int e0 = (k * BLOCK + tid) * 4;
    if (e0 < V)
      __builtin_amdgcn_global_load_lds(row + e0,
          (__attribute__((address_space(3))) void*)(qlds + k * BLOCK + wave * 64), 16, 0, 0);
  }
}

// The candidates of a node, one per lane (lane i < nk holds candidate i, in
// every wave; lanes past nk hold tok = -1): node id, drafted token (-1 if
// outside the vocabulary), its uniform and q_i(t_i).  Read with readlane, so
// a chain step needs no LDS lookups to test its candidate.
struct Cand {
  int kid, tok;
  float u, q;
};

// Brings rows into this XCD's L2 ahead of use: one 4-byte direct-to-LDS load
// per 128-byte line, into a scratch LDS word nothing reads.  Written as
// inline assembly (M0 saved and restored around it) so the compiler does not
// treat the transfer as a pending LDS write that every later LDS read must
// wait for; the hardware counts it like any vector load, so later waits can
// only become longer, never too short.
__device__ __forceinline__ void l2_touch(const float* p, uint32_t sink_lds) {
  uint32_t save;
  asm volatile(
      "s_mov_b32 %0, m0\n\ts_mov_b32 m0, %1\n\ts_nop 0\n\t"
      "global_load_lds_dword %2, off\n\ts_mov_b32 m0, %0"
      : "=&s"(save)
      : "s"(sink_lds), "v"(p)
      : "memory");
}

// True in a split workgroup's prefetch wave (the last one).
template <int BLOCK>
__device__ __forceinline__ bool prefetch_wave() {
  return __builtin_amdgcn_readfirstlane(threadIdx.x) >= BLOCK + 64;
}

// Draft rows touched ahead of the chain by the prefetch wave: few enough that
// its transfers are issued quickly (its workgroup's barriers wait for it).
constexpr int kL2Ahead = 3;

// One wave brings a row slice of len floats into L2 (one touch per line).
__device__ __forceinline__ void l2_touch_slice(const float* row, int len, float* sink) {
  const int lines = (len + 31) / 32;
  const uint32_t lds = (uint32_t)(size_t)(__attribute__((address_space(3))) float*)sink;
  for (int l = threadIdx.x & 63; l < lines; l += 64) l2_touch(row + l * 32, lds);
}

// One candidate of the multi-round chain at a node: the ratio test of
// candidate s against the current row `cur` (mass C, entry ut at the
// candidate's token) and, on rejection, the adjusted row into `nxt`.
// Returns true if the candidate is accepted; otherwise `nxt` holds the current
// row afterwards (the update, or a copy of `cur` in the rare case that the
// update leaves no mass).  Lane i < nk of every wave carries `val`, the
// current row's entry at candidate i's token, updated with the same fp32
// operations as the row (so bit-identical to it) from the gathered sh.qt
// table.  The next candidate's draft row is prefetched while this one's
// reduction runs: with RP into the registers qn (split rows; row s is in qn
// on entry and row s + 1 is loaded into it once read), else with VEC into
// qlds by direct-to-LDS loads.
template <int BLOCK, int NPT, bool VEC, bool RP, bool RATIO>
__device__ __forceinline__ bool chain_step(const VArgs& a, size_t ob, const Row<BLOCK, NPT>& cur,
                                           Row<BLOCK, NPT>& nxt, double& C, float& ut, float& val,
                                           const Cand& cd, float4 (&qn)[NPT], int s, int nk,
                                           bool stop_at_accept, Grp& grp, Shared<BLOCK, NPT>& sh,
                                           float4* qlds, int& rb) {
  const int tid = threadIdx.x, lane = tid & 63, V = a.V;
  // this workgroup's slice of candidate i's draft row (the whole row when P = 1)
  auto qrow = [&](int i) { return a.draft + (ob + lane_i(cd.kid, i)) * V + grp.base; };
  const int len = grp.len;
  const bool tok_ok = lane_i(cd.tok, s) >= 0;
  const double qt = tok_ok ? (double)lane_f(cd.q, s) : 0.0;
  const double num = tok_ok ? (double)ut : 0.0;
  // ratio = num / (C qt); accept iff u < ratio, tested without the division
  // (q = 0: ratio is +inf when num > 0, else 0)
  const double den = C * qt;
  const bool accept = qt > 0.0 ? (double)lane_f(cd.u, s) * den < num : num > 0.0;
  const double inv = kFix / C;  // for the mass exchange; its latency hides behind the pass
  if (RATIO && tid == 0)
    sh.ratio[s] = qt > 0.0 ? (float)(num / den) : (num > 0.0 ? INFINITY : 0.f);
  if (stop_at_accept && accept) return true;
  // rejection: nxt = max(0, cur - C q_s) and its mass, one read of q_s
  const float q_lane = sh.qt[tri(s, lane, nk)];  // q_s at candidate `lane`'s token
  if (VEC && !RP) asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // own prefetch landed
  const float cf = (float)C;
  const bool more = s + 1 < nk;
  float ps[NPT];
  float4 qv[NPT];
#pragma unroll
  for (int k = 0; k < NPT; ++k) {
    const int e0 = (k * BLOCK + tid) * 4;
    if constexpr (RP) {
      qv[k] = tid < BLOCK && e0 < len ? qn[k] : make_float4(0.f, 0.f, 0.f, 0.f);
    } else if constexpr (VEC) {
      qv[k] = qlds[k * BLOCK + tid];
    } else {
      const float* qs = qrow(s);
      const float x0 = qs[min(e0 + 0, len - 1)], x1 = qs[min(e0 + 1, len - 1)];
      const float x2 = qs[min(e0 + 2, len - 1)], x3 = qs[min(e0 + 3, len - 1)];
      qv[k] = make_float4(e0 + 0 < len ? x0 : 0.f, e0 + 1 < len ? x1 : 0.f, e0 + 2 < len ? x2 : 0.f,
                          e0 + 3 < len ? x3 : 0.f);
    }
  }
#pragma unroll
  for (int k = 0; k < NPT; ++k) {
    const float4 q = qv[k];
    float4& w = nxt.v[k];
    w.x = fmaxf(0.f, fmaf(-cf, q.x, cur.v[k].x));
    w.y = fmaxf(0.f, fmaf(-cf, q.y, cur.v[k].y));
    w.z = fmaxf(0.f, fmaf(-cf, q.z, cur.v[k].z));
    w.w = fmaxf(0.f, fmaf(-cf, q.w, cur.v[k].w));
    ps[k] = sum4(w);
  }
  const float vnew = fmaxf(0.f, fmaf(-cf, q_lane, val));
  if constexpr (VEC && !RP) {
    if (more) {
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // own reads of q_s done
      issue_row_lds<BLOCK, NPT>(qrow(s + 1), len, qlds);
    }
  }
  // RP: row s + 1's loads are issued once this workgroup's partial mass is
  // handed to the exchange, so they overlap it (addresses clamped into the
  // slice, len >= 4; the tail is zeroed on use)
  const double Cn = grp_sum<BLOCK, NPT>((double)pairwise<NPT>(ps), C, inv, grp, sh, rb, [&] {
    if constexpr (RP) {
      if (more && row_wave<BLOCK>()) {
        const float* qs = qrow(s + 1);
#pragma unroll
        for (int k = 0; k < NPT; ++k)
          qn[k] = *reinterpret_cast<const float4*>(qs + min((k * BLOCK + tid) * 4, len - 4));
      } else if (s + 1 + kL2Ahead < nk && prefetch_wave<BLOCK>()) {
        l2_touch_slice(qrow(s + 1 + kL2Ahead), len, sh.l2sink);
      }
    }
  });  // Cn <= C
  const bool commit = Cn > 0.0;
  if (commit) {
    C = Cn;
    if (lane > s) val = vnew;
  } else {
#pragma unroll
    for (int k = 0; k < NPT; ++k) nxt.v[k] = cur.v[k];
  }
  if (more) ut = lane_f(val, s + 1);
  return false;
}

// The multi-round chain at one node: tests its candidates in order (stopping
// at the first acceptance when `stop_at_accept`), leaving the adjusted row in
// U (unnormalised, mass C).  ut is U's entry at the first candidate's token,
// val the per-lane candidate entries (see chain_step).  Candidate s's ratio
// goes to sh.ratio[s] (RATIO).  Returns the index of the accepted candidate,
// or -1.  The first candidate's row prefetch (RP: into qn) must already be
// issued.  One copy of the step's code (the loop is not unrolled: the step
// is long, and a kernel that starts with a cold instruction cache pays for
// every line of straight code once); the next row is moved into U after each
// step.
template <int BLOCK, int NPT, bool VEC, bool RP, bool RATIO>
__device__ __forceinline__ int run_chain(const VArgs& a, size_t ob, Row<BLOCK, NPT>& U, double& C,
                                         float ut, float val, const Cand& cd, float4 (&qn)[NPT],
                                         int nk, bool stop_at_accept, Grp& grp,
                                         Shared<BLOCK, NPT>& sh, float4* qlds, int& rb) {
  Row<BLOCK, NPT> W;
#pragma nounroll
  for (int s = 0; s < nk; ++s) {
    if (chain_step<BLOCK, NPT, VEC, RP, RATIO>(a, ob, U, W, C, ut, val, cd, qn, s, nk,
                                               stop_at_accept, grp, sh, qlds, rb))
      return s;
#pragma unroll
    for (int k = 0; k < NPT; ++k) U.v[k] = W.v[k];
  }
  return -1;
}

// Set-up of one node's chain after the tree is in LDS and the node's logits
// were issued into U: its children (sh.kids, and per lane in cd), the first
// candidate's row prefetch, the table qt[k][i] = q_{kid k}(t_{kid i}) and
// each candidate's own logit (gathered while the row pass runs), then the
// row statistics.  Returns the argmax (T = 0); sets C, ut (U at the first
// candidate's token) and, on lane i < nk, val = U at candidate i's token.
template <int BLOCK, int NPT, bool GREEDY, bool VEC, bool RP>
__device__ __forceinline__ int node_setup(const VArgs& a, size_t ob, int node, int b,
                                          int32_t* flags, Row<BLOCK, NPT>& U, double& C, float& ut,
                                          float& val, Cand& cd, float4 (&qn)[NPT], Grp& grp,
                                          Shared<BLOCK, NPT>& sh, float4* qlds, int& rb) {
  const int tid = threadIdx.x, lane = tid & 63, V = a.V;
  find_kids<BLOCK, NPT>(a.N, node, sh);
  barrier_lds();
  const int nk = sh.nk;
  int sum_buf = 0;
  ut = 0.f;
  val = 0.f;
  if constexpr (GREEDY) {
    return target_stats<BLOCK, NPT, true>(U, a.T, b, flags, C, sum_buf,
                                          [](int, float, bool, float) {}, grp, sh, rb);
  } else {
    cd.kid = 0;
    cd.tok = -1;
    cd.u = 0.f;
    cd.q = 0.f;
    if (lane < nk) {
      cd.kid = sh.kids[lane];
      const int t = sh.tok[cd.kid];
      cd.tok = t >= 0 && t < V ? t : -1;
      cd.u = sh.u[cd.kid];
    }
    if (nk > 0) {
      const float* q0 = a.draft + (ob + lane_i(cd.kid, 0)) * V + grp.base;
      if constexpr (RP) {
        if (row_wave<BLOCK>()) {
#pragma unroll
          for (int k = 0; k < NPT; ++k)
            qn[k] = *reinterpret_cast<const float4*>(q0 + min((k * BLOCK + tid) * 4, grp.len - 4));
        }
      } else if constexpr (VEC) {
        // slots past the slice are never loaded: zero this thread's (the pass reads them)
#pragma unroll
        for (int k = 0; k < NPT; ++k)
          if ((k * BLOCK + tid) * 4 >= grp.len) qlds[k * BLOCK + tid] = make_float4(0.f, 0.f, 0.f, 0.f);
        issue_row_lds<BLOCK, NPT>(q0, grp.len, qlds);
      }
    }
    constexpr int G = (64 * 64 + BLOCK - 1) / BLOCK;
    float g[G];
#pragma unroll
    for (int r = 0; r < G; ++r) {
      const int f = r * BLOCK + tid;
      const int k = f / 64, i = f & 63;
      g[r] = 0.f;
      if (tid < BLOCK && k <= i && i < nk) {
        const int t = sh.tok[sh.kids[i]];
        if (t >= 0 && t < V) g[r] = a.draft[(ob + sh.kids[k]) * V + t];
      }
    }
    float lt = 0.f;
    if (cd.tok >= 0) lt = a.logits[(ob + node) * V + cd.tok];
    target_stats<BLOCK, NPT, false>(
        U, a.T, b, flags, C, sum_buf,
        [&](int, float m, bool unit, float invT) {
#pragma unroll
          for (int r = 0; r < G; ++r) {
            const int f = r * BLOCK + tid;
            const int k = f / 64, i = f & 63;
            if (tid < BLOCK && k <= i && i < nk) sh.qt[tri(k, i, nk)] = g[r];
          }
          if (lane < nk) val = target_entry(lt, m, unit, invT);  // (split rows: redone below)
        },
        grp, sh, rb);
    if (RP && grp.P > 1 && lane < nk && cd.tok >= 0) {
      // split rows: the entry as the part that holds the token computed it,
      // from that part's maximum and scale
      const int slice = (((V >> 2) + grp.P - 1) / grp.P) * 4;
      const int pt = cd.tok / slice;
      val = target_entry(lt, sh.mp[pt], a.T == 1.f, 1.f / a.T) * sh.fp[pt];
    }
    // the table is published by the mass reduction's barrier
    if (lane < nk) cd.q = sh.qt[tri(lane, lane, nk)];
    if (RP && prefetch_wave<BLOCK>()) {
      // the prefetch wave: the next candidates' slices into L2, so that each
      // step's one-row-ahead register prefetch finds them there; issued once
      // this wave's own loads are consumed (a wave's transfers complete in
      // order), and kept kL2Ahead rows ahead by the chain steps
      for (int c = 1; c <= kL2Ahead && c < nk; ++c)
        l2_touch_slice(a.draft + (ob + lane_i(cd.kid, c)) * V + grp.base, grp.len, sh.l2sink);
    }
    ut = lane_f(val, 0);
    return 0;
  }
}

// Inverse-CDF draw from U / sum(U) with uniform u: the smallest id whose
// cumulative mass exceeds u * sum; if rounding leaves none, the last id with
// mass.  fp64 cumulative sums in id order.  The masses of the 4-id groups are
// laid out in LDS in id order (`part`, NPT*BLOCK doubles, free memory); each
// thread then owns NPT consecutive groups, each wave 64 threads of them: the
// wave totals locate the wave, a lane scan the thread, its groups the group
// and the group's owner the id.
// With `given`, the row is one slice of a split row: the search starts at
// mass `start` and stops at threshold `thr_given` instead of u * sum.
template <int BLOCK, int NPT>
__device__ __forceinline__ int inverse_cdf(const Row<BLOCK, NPT>& U, float u, int V,
                                           Shared<BLOCK, NPT>& sh, double* part, int& rb,
                                           bool given = false, double start = 0.0,
                                           double thr_given = 0.0) {
  constexpr int NW = BLOCK / 64;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const bool row = tid < BLOCK;  // not an extra wave of a split workgroup (no mass)
  if (row) {
#pragma unroll
    for (int k = 0; k < NPT; ++k)
      part[k * BLOCK + tid] =
          (((double)U.v[k].x + (double)U.v[k].y) + (double)U.v[k].z) + (double)U.v[k].w;
  }
  barrier_lds();
  double e[NPT];
#pragma unroll
  for (int i = 0; i < NPT; ++i) e[i] = row ? part[tid * NPT + i] : 0.0;
  double own = 0.0;
#pragma unroll
  for (int i = 0; i < NPT; ++i) own += e[i];
  const double wt = wave_allsum(own);
  const int wbuf = rb;
  rb ^= 1;
  if (lane == 0 && row) sh.rd[wbuf][wave] = wt;
  if (tid == 0) sh.pick = -1;
  barrier_lds();
  double Z = 0.0;
#pragma unroll
  for (int i = 0; i < NW; ++i) Z += sh.rd[wbuf][i];
  const double thr = given ? thr_given : (double)u * Z;
  int ws = NW - 1;  // rounding may leave no crossing: then the last wave
  double before_w = start, run = start;
#pragma unroll
  for (int i = 0; i < NW; ++i) {
    const double nx = run + sh.rd[wbuf][i];
    if (ws == NW - 1 && i < NW - 1 && nx > thr) {
      ws = i;
      before_w = run;
    }
    if (i == NW - 1 && ws == NW - 1) before_w = run;
    run = nx;
  }
  if (wave == ws) {
    double incl = own;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const double o = __shfl_up(incl, off);
      if (lane >= off) incl += o;
    }
    const uint64_t hm = __ballot(before_w + incl > thr);
    const int L = hm ? __ffsll((unsigned long long)hm) - 1 : 63;
    if (lane == L) {
      double f = before_w + (incl - own);
      int sel = -1;
      double before_e = 0.0;
#pragma unroll
      for (int i = 0; i < NPT; ++i) {
        if (sel < 0 && f + e[i] > thr) {
          sel = i;
          before_e = f;
        }
        f += e[i];
      }
      if (sel < 0) {  // rounding: the lane's last group
        sel = NPT - 1;
        before_e = f - e[NPT - 1];
      }
      sh.sel_entry = tid * NPT + sel;
      sh.sel_before = before_e;
    }
  }
  barrier_lds();
  {
    const int entry = sh.sel_entry;
    const int ks = entry / BLOCK, ts = entry - ks * BLOCK;
    if (tid == ts) {
      float4 rv = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
      for (int k = 0; k < NPT; ++k)
        if (k == ks) rv = U.v[k];
      const int id0 = entry * 4;
      double f = sh.sel_before;
      int cand = -1, lastpos = -1;
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const float x = comp(rv, c);
        f += (double)x;
        if (id0 + c < V && x > 0.f) {
          lastpos = id0 + c;
          if (cand < 0 && f > thr) cand = id0 + c;
        }
      }
      sh.pick = cand >= 0 ? cand : lastpos;
    }
  }
  barrier_lds();
  int pick = sh.pick;
  if (pick < 0) {
    int last = -1;
#pragma unroll
    for (int k = 0; k < NPT; ++k)
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const int idx = (k * BLOCK + tid) * 4 + c;
        if (row && idx < V && comp(U.v[k], c) > 0.f) last = idx;
      }
    pick = block_max_i<BLOCK, NPT>(last, sh, rb);
    if (pick < 0) pick = 0;
  }
  return pick;
}

// Final draw over a split row.  The exchange that produced the row's mass
// left every part's mass of it in sh.pm, identical in every part, so each
// part knows the mass before its slice and the total without another
// exchange; the one part whose slice holds u * total searches its slice.
// Returns the drawn id in the owning part, -1 in the others.
template <int BLOCK, int NPT>
__device__ __forceinline__ int split_draw(const Row<BLOCK, NPT>& U, float u, Grp& g,
                                          Shared<BLOCK, NPT>& sh, double* part, int& rb) {
  double tot = 0.0, lo = 0.0;
  for (int p = 0; p < g.P; ++p) {  // fixed order: the same sums in every part
    if (p == g.part) lo = tot;
    tot += sh.pm[p];
  }
  const double thr = (double)u * tot;
  const bool own = lo <= thr && (thr < lo + sh.pm[g.part] || g.part == g.P - 1);
  if (!own) return -1;
  const int pick = inverse_cdf<BLOCK, NPT>(U, u, g.len, sh, part, rb, true, lo, thr);
  return g.base + pick;
}

// KV compaction fused into the walk (the effect of eagle_kv_compact with this
// call's kv_src_slots and accept_len): the K/V of path node path[j] move from
// slot L + path[j] to slot L + j, j = 1..m (the root stays).  Each thread owns
// whole 16-byte columns (one matrix, head and chunk) and moves the moving rows
// of its columns in increasing j, reading a batch of rows before writing them.
// No other thread touches those addresses, and in increasing j no read can
// see an earlier write: the source L + path[j'] of a later row lies past every
// destination L + j, j < j', already written (path[j'] >= j').  A destination
// may be the source of an earlier row of the same batch, whose read is done.
template <int BLOCK, int NPT>
__device__ inline void fused_compact(const VerifyCompact& kc, int b, int N, int m,
                                     int32_t* flags, Shared<BLOCK, NPT>& sh) {
  const int tid = threadIdx.x;
  const int L = sh.Lkv;
  const bool ok = L >= 0 && L <= kc.Lmax - N;
  if (tid == 0) {
    kc.new_len[b] = ok ? L + m + 1 : L;
    if (!ok && flags) atomicOr(flags + b, EAGLE_FLAG_BAD_KV_LEN);
    int n = 0;
    for (int j = 1; ok && j <= m; ++j)
      if (sh.path[j] != j) sh.mv[n++] = j;
    sh.nmv = n;
  }
  __syncthreads();
  const int nmv = sh.nmv;
  if (nmv == 0) return;
  const int cpr = kc.d / 8;                      // 16-byte chunks per key row
  const int cols = 2 * kc.Hkv * cpr;             // K columns, then V columns
  constexpr int kRows = 8;                       // rows per batch
  for (int c = tid; c < cols; c += (int)blockDim.x) {
    const int which = c >= kc.Hkv * cpr;
    const int c2 = c - which * kc.Hkv * cpr;
    const int h = c2 / cpr, ch = c2 - h * cpr;
    uint16_t* col = (which ? kc.v : kc.k) +
                    (((size_t)b * kc.Hkv + h) * (size_t)kc.Lmax + L) * kc.d + ch * 8;
    for (int r0 = 0; r0 < nmv; r0 += kRows) {
      u32x4 buf[kRows];
#pragma unroll
      for (int i = 0; i < kRows; ++i)
        if (r0 + i < nmv)
          buf[i] = *reinterpret_cast<const u32x4*>(col + (size_t)sh.path[sh.mv[r0 + i]] * kc.d);
#pragma unroll
      for (int i = 0; i < kRows; ++i)
        if (r0 + i < nmv)
          *reinterpret_cast<u32x4*>(col + (size_t)sh.mv[r0 + i] * kc.d) = buf[i];
    }
  }
}

// BLOCK row threads; split rows add an exchange wave and a prefetch wave.
template <int BLOCK, int NPT, bool GREEDY, bool PARITY, bool VEC, bool SPLIT>
__global__ __launch_bounds__(SPLIT ? BLOCK + 128 : BLOCK) void verify_node_kernel(VArgs a) {
  static_assert(!SPLIT || (!GREEDY && !PARITY && VEC), "split rows: sampling path only");
  __shared__ Shared<BLOCK, NPT> sh;
  __shared__ float4 qlds[GREEDY ? 1 : NPT * BLOCK];  // draft-row prefetch
  const int N = a.N, V = a.V;
  const int tid = threadIdx.x;
  // Workgroup -> (node, part).  Split rows: workgroup i runs on XCD i % 8, and
  // the P parts of a node take slots with the same i % 8 (one L2 for their
  // exchange words); slots past the last node exit at once.
  int node = blockIdx.x, part = 0;
  if constexpr (SPLIT) {
    const int xcd = blockIdx.x & 7, slot = blockIdx.x >> 3;
    part = slot % a.P;
    node = (slot / a.P) * 8 + xcd;
    if (node >= a.nodes) return;
  }
  const int b = node / N;
  const int j = node - b * N;
  const size_t ob = (size_t)b * N;
  int rb = 0;
  Grp grp{nullptr, 1, 0, 0, 0, V, a.flags, b, 0};
  if constexpr (SPLIT) {
    const int s4 = ((V >> 2) + a.P - 1) / a.P;  // float4 per part
    grp.words = a.xwords + (size_t)node * kXPhases * kXWords;
    grp.P = a.P;
    grp.part = part;
    grp.base = part * s4 * 4;
    grp.len = min(V - grp.base, s4 * 4);
    grp.xt = BLOCK;
    if (tid == 0) sh.xabort = 0;
  }

  // the node's logit row (this part's slice) first: its latency overlaps the
  // tree set-up
  Row<BLOCK, NPT> U;
  load_logits<BLOCK, NPT>(U, a.logits + (ob + j) * V + grp.base, grp.len);

  // tree, tokens, uniforms; the committed length too (only the walk needs it,
  // and it would be a round trip of its own there)
  bool tok_bad = false;
  int Lkv = 0;
  if (tid < N) {
    Lkv = a.kv_len[b];
    if (tid == 0) sh.Lkv = Lkv;
    int par = a.parents[ob + tid];
    if (tid == 0)
      par = -1;
    else if (par != -1 && (par < 0 || par >= tid))
      par = 0;  // a bad link hangs off the root; -1 (absent node) is nobody's child
    const int tk = a.tokens[ob + tid];
    sh.par[tid] = par;
    sh.tok[tid] = tk;
    sh.u[tid] = a.uniforms[ob + tid];
    tok_bad = tid > 0 && par != -1 && (tk < 0 || tk >= V);
  }
  if (j == 0 && part == 0 && __ballot(tok_bad) && (tid & 63) == 0 && a.flags)
    atomicOr(a.flags + b, EAGLE_FLAG_BAD_TOKEN);
  barrier_lds();
  double C = 1.0;
  float ut = 0.f, val = 0.f;
  Cand cd{0, -1, 0.f, 0.f};
  float4 qn[NPT];  // split rows: draft-row prefetch registers
  const int am = node_setup<BLOCK, NPT, GREEDY, VEC, SPLIT>(a, ob, j, b, a.flags, U, C, ut, val, cd,
                                                             qn, grp, sh, qlds, rb);
  const int nk = sh.nk;

  if (PARITY && a.out_probs) {
    float* po = a.out_probs + (ob + j) * V;
#pragma unroll
    for (int k = 0; k < NPT; ++k)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int idx = (k * BLOCK + tid) * 4 + e;
        if (idx < V) po[idx] = GREEDY ? (idx == am ? 1.f : 0.f) : (float)((double)comp(U.v[k], e) / C);
      }
  }

  int acc = -1, bonus = am, ntested = nk;
  if constexpr (GREEDY) {
    for (int s = 0; s < nk; ++s) {
      const int c = sh.kids[s];
      const bool ok = sh.tok[c] == am;
      if (tid == 0) sh.ratio[s] = ok ? 1.f : 0.f;
      if (ok) {
        acc = c;
        ntested = s + 1;
        break;
      }
    }
  } else {
    const int si = run_chain<BLOCK, NPT, VEC, SPLIT, PARITY>(a, ob, U, C, ut, val, cd, qn, nk, true,
                                                             grp, sh, qlds, rb);
    if (si >= 0) {
      acc = sh.kids[si];
      ntested = si + 1;
    } else if constexpr (SPLIT) {
      bonus = split_draw<BLOCK, NPT>(U, sh.u[0], grp, sh, reinterpret_cast<double*>(qlds), rb);
    } else {
      bonus = inverse_cdf<BLOCK, NPT>(U, sh.u[0], V, sh, reinterpret_cast<double*>(qlds), rb);
    }
  }
  // a prefetch left in flight by an early acceptance must land before exit
  if (!GREEDY && VEC) asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();

  // publish this node's outcome (split rows: part 0, and the part that drew
  // the final token); the last workgroup of the sequence walks the tree
  if (tid == 0) {
    if (part == 0) {
      st_c(a.nr.acc + ob + j, acc);
      st_c(a.nr.ntested + ob + j, ntested);
    }
    if (!SPLIT || (acc >= 0 ? part == 0 : bonus >= 0)) st_c(a.nr.bonus + ob + j, bonus);
    if (SPLIT)
      __hip_atomic_fetch_max(a.nr.nphase + ob + j, grp.phase, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  if (PARITY && tid < ntested) st_c(a.nr.ratio + ob + sh.kids[tid], sh.ratio[tid]);  // read by out_ratio only
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  if (tid == 0) {
    const int ticket = __hip_atomic_fetch_add(a.nr.counter + b, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    sh.last = ticket == N * grp.P - 1;
  }
  __syncthreads();
  if (!sh.last) return;

  // ---- walk (last workgroup of sequence b) -----------------------------------
  if (tid < N) {
    // all four loads in flight before any result is used
    const int r0 = ld_c(a.nr.acc + ob + tid);
    const int r1 = ld_c(a.nr.bonus + ob + tid);
    const int r2 = ld_c(a.nr.ntested + ob + tid);
    const int r3 = SPLIT ? ld_c(a.nr.nphase + ob + tid) : 0;
    sh.wacc[tid] = r0;
    sh.wbonus[tid] = r1;
    sh.wnt[tid] = r2;
    if (SPLIT) sh.wph[tid] = min(r3, kXPhases);
  }
  __syncthreads();
  if (tid == 0) {
    int cur = 0, m_acc = 0;
    sh.path[0] = 0;
    for (;;) {
      const int nx = sh.wacc[cur];
      if (nx < 0 || nx <= cur || nx >= N) break;  // nx > cur for any valid walk
      sh.path[++m_acc] = nx;
      cur = nx;
    }
    sh.term = cur;
    // in range even if a timed-out exchange left the slot unwritten
    sh.pick = min(max(sh.wbonus[cur], 0), V - 1);
    sh.nk = m_acc;
    __hip_atomic_store(a.nr.counter + b, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  if constexpr (SPLIT) {
    // every workgroup of the sequence is past its last exchange: zero the
    // words its nodes used, and the phase counts, for the next call.  Wide
    // streaming stores (a store instruction is slow to issue, so few and
    // wide ones); the kernel's end makes them visible to the next call,
    // whose exchanges read the words only with device-coherent atomics.
    // Each wave takes whole nodes, so a lane issues only the stores of the
    // nodes of its wave.
    static_assert(kXWords % 2 == 0, "16-byte stores");
    const int nwaves = (int)blockDim.x >> 6, wave = tid >> 6, lane = tid & 63;
    for (int n = wave; n < N; n += nwaves) {
      u32x4* w = reinterpret_cast<u32x4*>(a.xwords + (ob + n) * kXPhases * kXWords);
      for (int i = lane; i < sh.wph[n] * (kXWords / 2); i += 64)
        __builtin_nontemporal_store(u32x4{0u, 0u, 0u, 0u}, w + i);
    }
    if (tid < N) st_c(a.nr.nphase + ob + tid, 0);
  }
  __syncthreads();
  const int m_acc = sh.nk;
  if (tid < N) {
    const size_t o = ob + tid;
    const bool on = tid <= m_acc;
    const int pn = on ? sh.path[tid] : -1;
    a.path[o] = pn;
    a.kv_src[o] = on ? Lkv + pn : -1;
    a.acc_tokens[o] = tid < m_acc ? sh.tok[sh.path[tid + 1]] : -1;
  }
  if (tid == 0) {
    a.accept_len[b] = m_acc;
    a.bonus[b] = sh.pick;
  }
  if (a.kc.k) fused_compact(a.kc, b, N, m_acc, a.flags, sh);
  if (PARITY && a.out_ratio) {
    // tested nodes: the candidates each path node's chain tested
    if (tid < N) {
      const int c = tid;
      float r = __int_as_float(0x7fc00000);
      if (c > 0) {
        const int p = sh.par[c];
        bool on_path = false;
        for (int k = 0; k <= m_acc; ++k) on_path |= sh.path[k] == p;
        if (on_path) {
          int rank = 0;
          for (int x = p + 1; x < c; ++x) rank += sh.par[x] == p;
          if (rank < sh.wnt[p]) r = ld_c(a.nr.ratio + ob + c);
        }
      }
      a.out_ratio[ob + c] = r;
    }
  }
  if (PARITY && a.out_final) {
    // the distribution of the final token: recompute the terminal's chain
    const int term = sh.term;
    const int bt = sh.pick;
    __syncthreads();
    float* fo = a.out_final + (size_t)b * V;
    if constexpr (GREEDY) {
      for (int v = tid; v < V; v += BLOCK) fo[v] = v == bt ? 1.f : 0.f;
    } else {
      Grp whole{nullptr, 1, 0, 0, 0, V, nullptr, b, 0};
      load_logits<BLOCK, NPT>(U, a.logits + (ob + term) * V, V);
      node_setup<BLOCK, NPT, false, VEC, false>(a, ob, term, b, nullptr, U, C, ut, val, cd, qn, whole,
                                                sh, qlds, rb);
      run_chain<BLOCK, NPT, VEC, false, false>(a, ob, U, C, ut, val, cd, qn, sh.nk, false, whole, sh,
                                               qlds, rb);
#pragma unroll
      for (int k = 0; k < NPT; ++k)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int idx = (k * BLOCK + tid) * 4 + e;
          if (idx < V) fo[idx] = (float)((double)comp(U.v[k], e) / C);
        }
    }
  }
}

// ---------------------------------------------------------------------------
// Split rows pay off where a node's chain is long per workgroup: large
// vocabularies with few nodes, so that all B * N * P workgroups are resident
// at once (one per CU at most), which the exchange waits rely on.
static int verify_parts(int B, int N, int V) {
  const size_t nodes = (size_t)B * N;
  if ((V & 3) != 0 || V <= 28672 || V > 32768) return 1;
  if (nodes * kMaxParts > (size_t)kNumCUs) return 1;
  return kMaxParts;
}

VerifyPlan plan_verify(int B, int N, int V) {
  VerifyPlan p{};
  p.V = V;
  p.parts = verify_parts(B, N, V);
  p.walk_threads = p.parts > 1 ? 256 : V > 4096 ? 1024 : 256;
  const size_t nodes = (size_t)B * N;
  p.ws_stats = nodes * 20;  // acc, bonus, ratio, ntested, nphase
  p.ws_counters = (size_t)B * 4;
  p.ws_partials = p.parts > 1 ? nodes * kXPhases * kXWords * 8 : 0;  // exchange words
  p.chunks = 1;
  return p;
}

static size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

size_t verify_workspace_bytes(const VerifyPlan& p) {
  return align256(p.ws_counters) + align256(p.ws_stats) + align256(p.ws_partials);
}

hipError_t launch_verify(const VerifyPlan& plan, const int32_t* tokens, const float* draft,
                         const float* logits, const int32_t* parents, const int32_t* kv_len,
                         int B, int N, float T, const float* uniforms, int32_t* accept_len,
                         int32_t* path, int32_t* acc_tokens, int32_t* bonus, int32_t* kv_src,
                         float* out_probs, float* out_final, float* out_ratio, void* ws,
                         int32_t* flags, const VerifyCompact& kc, hipStream_t s) {
  uint8_t* w = static_cast<uint8_t*>(ws);
  const size_t nodes = (size_t)B * N;
  VArgs a{};
  a.tokens = tokens;
  a.draft = draft;
  a.logits = logits;
  a.parents = parents;
  a.kv_len = kv_len;
  a.uniforms = uniforms;
  a.accept_len = accept_len;
  a.path = path;
  a.acc_tokens = acc_tokens;
  a.bonus = bonus;
  a.kv_src = kv_src;
  a.out_probs = out_probs;
  a.out_final = out_final;
  a.out_ratio = out_ratio;
  a.flags = flags;
  a.kc = kc;
  a.nr.counter = reinterpret_cast<int32_t*>(w);
  uint8_t* nb = w + align256(plan.ws_counters);
  a.nr.acc = reinterpret_cast<int32_t*>(nb);
  a.nr.bonus = reinterpret_cast<int32_t*>(nb + nodes * 4);
  a.nr.ratio = reinterpret_cast<float*>(nb + nodes * 8);
  a.nr.ntested = reinterpret_cast<int32_t*>(nb + nodes * 12);
  a.nr.nphase = reinterpret_cast<int32_t*>(nb + nodes * 16);
  a.xwords = reinterpret_cast<unsigned long long*>(nb + align256(plan.ws_stats));
  a.N = N;
  a.V = plan.V;
  a.nodes = (int)nodes;
  a.P = 1;
  a.T = T;
  const unsigned grid = (unsigned)nodes;
  const bool greedy = T == 0.f;
  const bool parity = out_probs || out_final || out_ratio;
  const bool vec = (plan.V & 3) == 0;
  if (plan.parts > 1 && !greedy && !parity && vec) {
    // node slots rounded up to a multiple of the 8 XCDs, P parts each
    a.P = plan.parts;
    const unsigned sgrid = (unsigned)(((nodes + 7) / 8) * 8 * plan.parts);
    verify_node_kernel<256, 4, false, false, true, true><<<sgrid, 256 + 128, 0, s>>>(a);
    return hipGetLastError();
  }
#define EAGLE_LAUNCH_VERIFY(BLK, NPT)                                                        \
  do {                                                                                      \
    if (greedy && parity) verify_node_kernel<BLK, NPT, true, true, true, false><<<grid, BLK, 0, s>>>(a);    \
    else if (greedy) verify_node_kernel<BLK, NPT, true, false, true, false><<<grid, BLK, 0, s>>>(a);        \
    else if (parity && vec) verify_node_kernel<BLK, NPT, false, true, true, false><<<grid, BLK, 0, s>>>(a); \
    else if (parity) verify_node_kernel<BLK, NPT, false, true, false, false><<<grid, BLK, 0, s>>>(a);       \
    else if (vec) verify_node_kernel<BLK, NPT, false, false, true, false><<<grid, BLK, 0, s>>>(a);          \
    else verify_node_kernel<BLK, NPT, false, false, false, false><<<grid, BLK, 0, s>>>(a);                  \
  } while (0)
  // the row must fit one workgroup unless it is split
  if (plan.V > 4096)
    EAGLE_LAUNCH_VERIFY(1024, 8);
  else
    EAGLE_LAUNCH_VERIFY(256, 4);
#undef EAGLE_LAUNCH_VERIFY
  return hipGetLastError();
}

}  // namespace eagle
