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
// No workgroup ever waits for another: a sequence's nodes only meet at the
// ticket, and the one that draws the last ticket walks.
//
// Per node j with candidates c_1..c_k (ascending) and T > 0:
//   U_0 = exp((l_j - max) / T) (unnormalised target), C_0 = sum U_0
//   ratio_s = U_{s-1}[t_s] / (C_{s-1} q_s[t_s])       (accept iff u_s < ratio_s)
//   U_s = max(0, U_{s-1} - C_{s-1} q_s),  C_s = sum U_s  (kept if C_s = 0)
// U_s / C_s is the adjusted distribution norm(max(0, r - q)) after s
// rejections.  When the candidates share one draft row q (siblings drawn
// i.i.d. from their parent's draft distribution) the recursion has a closed
// form: with S_0 = 0 and S_s = S_{s-1} + C_{s-1},
//   U_s = max(0, U_0 - S_s q),  C_s = F(S_s),  F(S) = sum_v max(0, U_v - S q_v)
// (by induction: where U_{s-1} > 0 it equals U_0 - S_{s-1} q, and where it is
// 0, U_0 - S_s q <= U_0 - S_{s-1} q <= 0).  Each rejection is then one pass
// over the two rows held in registers and one workgroup reduction, with no
// row reloaded and no residual row written.
//
// A node's critical path is a sequence of full-vocabulary passes, each ending
// in a workgroup reduction, so the kernel is built around short passes:
//   * the rows live in registers across the 512-thread workgroup (16 float4
//     per thread at V <= 32768), entries past V padded so no pass needs a
//     bounds check;
//   * without a shared row, a candidate's draft row is prefetched into LDS
//     with direct-to-LDS loads (each thread's float4 lands where that thread
//     reads it back, so no barrier guards the buffer) and is read once: the
//     pass builds the updated row W = max(0, U - C q) in a second register
//     row, and the next row's prefetch is issued as soon as this thread's
//     reads are done;
//   * wave reductions use DPP within rows of 16 lanes and readlane across the
//     four rows; a workgroup reduction takes one barrier (two alternating
//     LDS slot sets);
//   * masses: fp32 pairwise sums per thread, fp64 across threads (across
//     waves for the chain's per-rejection mass, fp32 within a wave), in a
//     fixed order (deterministic).  The final draw scans in fp64.
// At T = 0 a node's outcome needs only its row's argmax: rows are split over
// several workgroups that each publish their part's (value, lowest index) as
// one 64-bit atomic maximum, and the walk reads the maxima.
#include <float.h>
#include <limits.h>
#include <stdlib.h>

#include <utility>

#include "common.h"
#include "launch.h"

namespace eagle {

// Per-node results published for the walk (device-coherent stores/loads).
struct NodeResults {
  int32_t* acc;       // [B*N] accepted candidate, -1 if none
  int32_t* bonus;     // [B*N] token drawn if the walk ends here
  float* ratio;       // [B*N] ratio of node c as tested by its parent's chain
  int32_t* ntested;   // [B*N] candidates of the node that its chain tested
  int32_t* counter;   // [B] per-sequence tickets (zero between calls)
  unsigned long long* amax;  // [B*N] packed (value, lowest id) maxima (zero between calls)
};

struct VArgs {
  const int32_t* tokens;
  const float* draft;
  const int32_t* draft_row;  // [B*N] row of `draft` node i was drawn from, or null: row i
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
  VerifyCompact kc;  // compaction fused into the walk (kc.k == nullptr: none)
  int N, V;
  int nodes;  // B * N
  int P;      // workgroups per node (T = 0 split argmax)
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

template <int BLOCK, int NPT>
struct Shared {
  static constexpr int NW = BLOCK / 64;
  int par[64], tok[64], kids[64], row[64];
  float u[64];
  float ratio[64];
  float qt[64 * 64];  // qt[k*64 + i] = q_{kid k}(t_{kid i}) for k <= i (T > 0, rows not shared)
  int nk;
  // workgroup reductions: two slot sets, used alternately (see rb below)
  double rd[2][NW];
  float rf[2][NW];
  int ri[2][NW];
  double sel_before;
  int sel_entry;
  int pick;
  int last, term;
  int wacc[64], wbonus[64], wnt[64];
  int mv[64];      // fused compaction: the path positions whose K/V move
  int nmv, Lkv;
  int path[64];
};

// Workgroup reductions over the BLOCK threads.  `rb` selects the slot set and
// flips on every call; all threads make the same sequence of calls, so a slot
// set is rewritten only after the barrier of the reduction in between, which
// every reader of its previous contents has passed: one barrier per reduction
// suffices.  The sum takes the wave's partial from its last lane (DPP row
// broadcasts); the maximum and minimum keep the readlane form, which the
// node kernel at T = 0 ran faster with (7B step: 7.7 against 7.9 us).
template <int BLOCK, int NPT>
__device__ __forceinline__ double block_sum(double v, Shared<BLOCK, NPT>& sh, int& rb) {
  v = wave_sum_last(v);
  const int buf = rb;
  rb ^= 1;
  if ((threadIdx.x & 63) == 63) sh.rd[buf][threadIdx.x >> 6] = v;
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
  if ((threadIdx.x & 63) == 0) sh.rf[buf][threadIdx.x >> 6] = v;
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
  if ((threadIdx.x & 63) == 0) sh.ri[buf][threadIdx.x >> 6] = v;
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
  if ((threadIdx.x & 63) == 0) sh.ri[buf][threadIdx.x >> 6] = v;
  barrier_lds();
  int t = INT_MIN;
#pragma unroll
  for (int i = 0; i < BLOCK / 64; ++i) t = max(t, sh.ri[buf][i]);
  return t;
}

// max(0, x) for the entries of an adjusted row.  Such an entry is the target
// entry (at most 1: the row is exp((l - max) / T)) less a non-negative
// multiple of a probability, so it never exceeds 1 and clamping to [0, 1]
// gives the same value; the clamp folds into the FMA that produces x as its
// output modifier, saving the separate max.
__device__ __forceinline__ float pos01(float x) { return __builtin_amdgcn_fmed3f(x, 0.f, 1.f); }

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

// `len` floats of a row into registers, len % 4 == 0: straight-line buffer
// loads (no branches, so the compiler can count them and later waits name only
// the loads they need); entries past len read 0 from the buffer without a
// memory access and are then set to `pad`.  len = 0 loads nothing.
template <int BLOCK, int NPT>
__device__ __forceinline__ void load_row_vec(Row<BLOCK, NPT>& r, const float* src, int len,
                                             float pad) {
  const int tid = threadIdx.x;
  const __amdgpu_buffer_rsrc_t rs = buffer_rsrc(src, (size_t)len * 4);
#pragma unroll
  for (int k = 0; k < NPT; ++k)
    r.v[k] = __builtin_bit_cast(float4, __builtin_amdgcn_raw_buffer_load_b128(
                                            rs, (k * BLOCK + tid) * 16, 0, 0));
  if (pad != 0.f) {
#pragma unroll
    for (int k = 0; k < NPT; ++k)
      if ((k + 1) * BLOCK * 4 > len && (k * BLOCK + tid) * 4 >= len)
        r.v[k] = make_float4(pad, pad, pad, pad);
  }
}

// `len` floats of a row into registers (len >= 1); entries past len read as
// `pad` (-FLT_MAX for logits: no mass, never the maximum of a row that has a
// finite entry; 0 for draft rows).  Every load is issued at an in-range
// address and the padding selected afterwards, so the loads need no branches.
template <int BLOCK, int NPT>
__device__ __forceinline__ void load_row(Row<BLOCK, NPT>& r, const float* src, int len, float pad) {
  const int tid = threadIdx.x;
  if ((len & 3) == 0) {
#pragma unroll
    for (int k = 0; k < NPT; ++k) {
      const int e0 = (k * BLOCK + tid) * 4;
      const bool in = e0 < len;
      const float4 x = *reinterpret_cast<const float4*>(src + (in ? e0 : 0));
      r.v[k] = in ? x : make_float4(pad, pad, pad, pad);
    }
  } else {
    // one-dword buffer loads (the row need not be 16-byte aligned): offsets
    // from the thread id and immediates, so no per-entry address registers;
    // dwords past len read 0 and are then set to pad
    const __amdgpu_buffer_rsrc_t rs = buffer_rsrc(src, (size_t)len * 4);
#pragma unroll
    for (int k = 0; k < NPT; ++k) {
      const int e0 = (k * BLOCK + tid) * 4;
      float x[4];
#pragma unroll
      for (int e = 0; e < 4; ++e)
        x[e] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rs, (e0 + e) * 4, 0, 0));
      if ((k + 1) * BLOCK * 4 > len) {
#pragma unroll
        for (int e = 0; e < 4; ++e) x[e] = e0 + e < len ? x[e] : pad;
      }
      r.v[k] = make_float4(x[0], x[1], x[2], x[3]);
    }
  }
}

// exp(z) for z <= 0, computed as 2^t with t = z log2(e) rounded to fp32 and
// the rest of the exponent carried in natural units: e = z - t ln 2, with
// ln 2 split into an fp32 head and tail, is formed by two FMAs (the first
// exact: its product is exact in the FMA and the difference, about 2^-24 z,
// fits in fp32), and e^z = 2^t e^e = 2^t (1 + e) to within e^2/2 (below
// 1e-11 relative over the range).  The hardware exp2 is within 1 ulp, so the
// whole is within about 2 ulp of exp(z) (checked against fp64 on the device
// in the tests).  One instruction fewer per entry than carrying the rounding
// of t in log2 units (and scaling it by ln 2).  Arguments below -110
// (results below the fp32 range) are clamped, which keeps the correction
// finite for the -FLT_MAX padding.
__device__ __forceinline__ float exp_neg(float z) {
  z = fmaxf(z, -110.f);
  constexpr float kL2E = 1.44269502162933349609375f;  // log2(e), fp32
  constexpr float kLn2Hi = 0.693147182464599609375f;  // ln 2, fp32 head
  constexpr float kLn2Lo = -1.9046542121259336e-09f;  // ln 2 - kLn2Hi
  const float t = z * kL2E;
  const float e = fmaf(-t, kLn2Lo, fmaf(-t, kLn2Hi, z));
  const float r = __builtin_amdgcn_exp2f(t);
  return fmaf(r, e, r);
}

__device__ __forceinline__ float sum4(const float4& f) { return (f.x + f.y) + (f.z + f.w); }

template <int NPT>
__device__ __forceinline__ float pairwise(const float (&s)[NPT]) {
  if constexpr (NPT == 16) {
    return (((s[0] + s[1]) + (s[2] + s[3])) + ((s[4] + s[5]) + (s[6] + s[7]))) +
           (((s[8] + s[9]) + (s[10] + s[11])) + ((s[12] + s[13]) + (s[14] + s[15])));
  } else if constexpr (NPT == 8) {
    return ((s[0] + s[1]) + (s[2] + s[3])) + ((s[4] + s[5]) + (s[6] + s[7]));
  } else if constexpr (NPT == 4) {
    return (s[0] + s[1]) + (s[2] + s[3]);
  } else if constexpr (NPT == 2) {
    return s[0] + s[1];
  } else {
    static_assert(NPT == 1, "rows of 1, 2, 4, 8 or 16 float4 per thread");
    return s[0];
  }
}

// The scaled exponent of one logit, exactly as the row pass computes it
// (non-finite logits have no mass); nmi = -(m * invT).
__device__ __forceinline__ float target_entry(float x, float nmi, float invT) {
  x = isfinite(x) ? x : -FLT_MAX;
  return exp_neg(fmaf(x, invT, nmi));
}

// Non-finite logits (NaN, +-Inf) are reported and given no mass: replaced by
// -FLT_MAX in the row.  x * 0 is NaN exactly for non-finite x: one fma per
// entry to detect them.
template <int BLOCK, int NPT>
__device__ __forceinline__ void sanitize_logits(Row<BLOCK, NPT>& U, int b, int32_t* flags) {
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
  if (__ballot(nonfinite) && (threadIdx.x & 63) == 0 && flags) atomicOr(flags + b, EAGLE_FLAG_NONFINITE);
}

// The lowest index of the row's maximum (this workgroup's row or slice):
// every thread's first maximum in id order, then the workgroup's.
template <int BLOCK, int NPT>
__device__ __forceinline__ void row_argmax(const Row<BLOCK, NPT>& U, float& mx, int& am,
                                           Shared<BLOCK, NPT>& sh, int& rb) {
  const int tid = threadIdx.x;
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
  // each wave's maximum and the lowest index holding it, then one barrier:
  // the row's maximum over the waves and the lowest index among the waves
  // that hold it (one barrier fewer than a maximum and then a minimum
  // across the workgroup: verification at T = 0, 7B step 7.7 -> 6.8 us,
  // 70B 12.6 -> 11.7 us)
  const float wm = wave_allmax(lm);
  const int wi = wave_allmin_i(lm == wm ? li : INT_MAX);
  const int buf = rb;
  rb ^= 1;
  if ((tid & 63) == 0) {
    sh.rf[buf][tid >> 6] = wm;
    sh.ri[buf][tid >> 6] = wi;
  }
  barrier_lds();
  float m = -INFINITY;
#pragma unroll
  for (int i = 0; i < BLOCK / 64; ++i) m = fmaxf(m, sh.rf[buf][i]);
  int a = INT_MAX;
#pragma unroll
  for (int i = 0; i < BLOCK / 64; ++i) a = sh.rf[buf][i] == m ? min(a, sh.ri[buf][i]) : a;
  mx = m;
  am = a;
}

// Target row statistics of one node from its logits (already in U): T = 0
// returns the lowest-index argmax; T > 0 turns U into exp((l - max)/T) and
// returns its mass in C.  after_max() runs once the row's maximum is known
// (U has arrived: loads it issues no longer share the CU's bandwidth with
// U's); before_sum(nmi, invT), nmi = -(m * invT), runs before the mass
// reduction, whose barrier publishes what it writes to LDS.
template <int BLOCK, int NPT, bool GREEDY, typename G, typename F>
__device__ __forceinline__ int target_stats(Row<BLOCK, NPT>& U, float T, int b, int32_t* flags,
                                            double& C, G&& after_max, F&& before_sum,
                                            Shared<BLOCK, NPT>& sh, int& rb) {
  sanitize_logits<BLOCK, NPT>(U, b, flags);
  if constexpr (GREEDY) {
    float mx;
    int am;
    row_argmax<BLOCK, NPT>(U, mx, am, sh, rb);
    C = 1.0;
    return am == INT_MAX ? 0 : am;
  } else {
    float lm = -INFINITY;
#pragma unroll
    for (int k = 0; k < NPT; ++k)
      lm = fmaxf(lm, fmaxf(fmaxf(U.v[k].x, U.v[k].y), fmaxf(U.v[k].z, U.v[k].w)));
    const float m = block_max<BLOCK, NPT>(lm, sh, rb);
    after_max();
    // (x - m) / T as one FMA, x (1 / T) - m (1 / T): at T = 1 it is x - m
    // exactly, so one form serves every temperature (a select between two
    // forms cost an instruction per entry)
    const float invT = 1.f / T;
    const float nmi = -(m * invT);
    float s[NPT];
#pragma unroll
    for (int k = 0; k < NPT; ++k) {
      float4& f = U.v[k];
      f.x = exp_neg(fmaf(f.x, invT, nmi));  // already finite
      f.y = exp_neg(fmaf(f.y, invT, nmi));
      f.z = exp_neg(fmaf(f.z, invT, nmi));
      f.w = exp_neg(fmaf(f.w, invT, nmi));
      s[k] = sum4(f);
    }
    before_sum(nmi, invT);
    C = block_sum<BLOCK, NPT>((double)pairwise<NPT>(s), sh, rb);  // entries <= 1
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

// Position of q_{kid k}(t_{kid i}), k <= i < nk, in sh.qt.
__device__ __forceinline__ int tri(int k, int i) { return k * 64 + i; }

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
// outside the vocabulary), the draft row it was drawn from, its uniform, the
// draft probability q_i(t_i) and (shared row) the target entry U_0(t_i).
// Read with readlane, so a chain step needs no LDS lookups to test its
// candidate.
struct Cand {
  int kid, tok, row;
  float u, q, ut;
};

// ---- candidates with their own draft rows: the recursion step by step --------
// One candidate of the multi-round chain at a node: the ratio test of
// candidate s against the current row `cur` (mass C, entry ut at the
// candidate's token) and, on rejection, the adjusted row into `nxt`.
// Returns true if the candidate is accepted; otherwise `nxt` holds the current
// row afterwards (the update, or a copy of `cur` in the rare case that the
// update leaves no mass).  Lane i < nk of every wave carries `val`, the
// current row's entry at candidate i's token, updated with the same fp32
// operations as the row (so bit-identical to it) from the gathered sh.qt
// table.  With VEC the next candidate's draft row is prefetched into qlds by
// direct-to-LDS loads while this one's reduction runs.
template <int BLOCK, int NPT, bool VEC, bool RATIO>
__device__ __forceinline__ bool chain_step(const VArgs& a, size_t ob, const Row<BLOCK, NPT>& cur,
                                           Row<BLOCK, NPT>& nxt, double& C, float& ut, float& val,
                                           const Cand& cd, int s, int nk, bool stop_at_accept,
                                           Shared<BLOCK, NPT>& sh, float4* qlds, int& rb) {
  const int tid = threadIdx.x, lane = tid & 63, V = a.V;
  auto qrow = [&](int i) { return a.draft + (ob + lane_i(cd.row, i)) * V; };
  const bool tok_ok = lane_i(cd.tok, s) >= 0;
  const double qt = tok_ok ? (double)lane_f(cd.q, s) : 0.0;
  const double num = tok_ok ? (double)ut : 0.0;
  // ratio = num / (C qt); accept iff u < ratio, tested without the division
  // (q = 0: ratio is +inf when num > 0, else 0)
  const double den = C * qt;
  const bool accept = qt > 0.0 ? (double)lane_f(cd.u, s) * den < num : num > 0.0;
  if (RATIO && tid == 0)
    sh.ratio[s] = qt > 0.0 ? (float)(num / den) : (num > 0.0 ? INFINITY : 0.f);
  if (stop_at_accept && accept) return true;
  // rejection: nxt = max(0, cur - C q_s) and its mass, one read of q_s
  const float q_lane = sh.qt[tri(s, lane)];  // q_s at candidate `lane`'s token
  if (VEC) asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // own prefetch landed
  const float cf = (float)C;
  const bool more = s + 1 < nk;
  float ps[NPT];
  // the draft row: from this thread's own LDS slots (VEC), or loaded into
  // the output row first and consumed in place
  if constexpr (!VEC) load_row<BLOCK, NPT>(nxt, qrow(s), V, 0.f);
#pragma unroll
  for (int k = 0; k < NPT; ++k) {
    float4 q;
    if constexpr (VEC)
      q = qlds[k * BLOCK + tid];
    else
      q = nxt.v[k];
    float4& w = nxt.v[k];
    w.x = pos01(fmaf(-cf, q.x, cur.v[k].x));
    w.y = pos01(fmaf(-cf, q.y, cur.v[k].y));
    w.z = pos01(fmaf(-cf, q.z, cur.v[k].z));
    w.w = pos01(fmaf(-cf, q.w, cur.v[k].w));
    ps[k] = sum4(w);
  }
  const float vnew = pos01(fmaf(-cf, q_lane, val));
  if constexpr (VEC) {
    if (more) {
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // own reads of q_s done
      issue_row_lds<BLOCK, NPT>(qrow(s + 1), V, qlds);
    }
  }
  const double Cn = block_sum<BLOCK, NPT>((double)pairwise<NPT>(ps), sh, rb);  // Cn <= C
  if (Cn > 0.0) {
    C = Cn;
    if (lane > s) val = vnew;
  } else {
#pragma unroll
    for (int k = 0; k < NPT; ++k) nxt.v[k] = cur.v[k];
  }
  if (more) ut = lane_f(val, s + 1);
  return false;
}

// The multi-round chain at one node, candidates with their own rows: tests
// them in order (stopping at the first acceptance when `stop_at_accept`),
// leaving the adjusted row in U (unnormalised, mass C).  ut is U's entry at
// the first candidate's token, val the per-lane candidate entries.  Candidate
// s's ratio goes to sh.ratio[s] (RATIO).  Returns the index of the accepted
// candidate, or -1.  The first candidate's row prefetch (VEC) must already be
// issued.  W is a second row buffer.  One copy of the step's code (the loop is
// not unrolled: the step is long, and a kernel that starts with a cold
// instruction cache pays for every line of straight code once).
template <int BLOCK, int NPT, bool VEC, bool RATIO>
__device__ __forceinline__ int run_chain(const VArgs& a, size_t ob, Row<BLOCK, NPT>& U,
                                         Row<BLOCK, NPT>& W, double& C, float ut, float val,
                                         const Cand& cd, int nk, bool stop_at_accept,
                                         Shared<BLOCK, NPT>& sh, float4* qlds, int& rb) {
#pragma nounroll
  for (int s = 0; s < nk; ++s) {
    if (chain_step<BLOCK, NPT, VEC, RATIO>(a, ob, U, W, C, ut, val, cd, s, nk, stop_at_accept, sh,
                                           qlds, rb))
      return s;
#pragma unroll
    for (int k = 0; k < NPT; ++k) U.v[k] = W.v[k];
  }
  return -1;
}

// ---- candidates sharing one draft row: the closed form --------------------------
// After s rejections the adjusted row is max(0, U - S q) with mass F(S)
// (S = S_s, see the top of the file).  S is carried in fp64 and applied as an
// fp32 pair (head + tail), so the row entry is exact to about one rounding
// however large S grows relative to an entry; every entry and every
// candidate's entry come from the same two FMAs, so a candidate's numerator
// is bit-identical to its entry of the row.
__device__ __forceinline__ float residual(float u, float q, float hs, float ls) {
  return pos01(fmaf(-ls, q, fmaf(-hs, q, u)));
}
__device__ __forceinline__ float4 residual4(const float4& u, const float4& q, float hs, float ls) {
  return make_float4(residual(u.x, q.x, hs, ls), residual(u.y, q.y, hs, ls),
                     residual(u.z, q.z, hs, ls), residual(u.w, q.w, hs, ls));
}

template <int BLOCK, int NPT>
__device__ __forceinline__ void split_s(double S, float& hs, float& ls) {
  hs = (float)S;
  ls = (float)(S - (double)hs);
}

// F(S): one pass over the two rows and one workgroup reduction.  The sum
// applies S through its fp32 head alone: one clamped FMA per entry instead of
// two.  Leaving out the tail moves each term by at most |S - hs| q <= 2^-24 S q,
// under one ulp of a live entry (S q < U there), and an entry within that of
// zero (S within 2^-24 of its ratio U/q) by no more, so the mass keeps the
// accuracy of the fp32 sums; the entries themselves (a candidate's numerator,
// the row of the final draw) keep both parts.
template <int BLOCK, int NPT>
__device__ __forceinline__ double residual_mass(const Row<BLOCK, NPT>& U, const Row<BLOCK, NPT>& Q,
                                                float hs, Shared<BLOCK, NPT>& sh, int& rb) {
  float ps[NPT];
#pragma unroll
  for (int k = 0; k < NPT; ++k) {
    const float4 u = U.v[k], q = Q.v[k];
    ps[k] = (pos01(fmaf(-hs, q.x, u.x)) + pos01(fmaf(-hs, q.y, u.y))) +
            (pos01(fmaf(-hs, q.z, u.z)) + pos01(fmaf(-hs, q.w, u.w)));
  }
  // fp32 within the wave, fp64 across the waves; the wave's sum lands in its
  // last lane (DPP row broadcasts, no readlanes).  Per rejection this is on
  // the critical path: whole verification of the 7B step 20.7 -> 20.35 us for
  // the fp32 wave sum, -> 19.8 us with the broadcasts
  const float v = wave_sum_last(pairwise<NPT>(ps));
  const int buf = rb;
  rb ^= 1;
  if ((threadIdx.x & 63) == 63) sh.rd[buf][threadIdx.x >> 6] = (double)v;
  barrier_lds();
  double t = 0.0;
#pragma unroll
  for (int i = 0; i < BLOCK / 64; ++i) t += sh.rd[buf][i];
  return t;
}

// The adjusted row max(0, U - S q) materialised (for the final distribution output).
template <int BLOCK, int NPT>
__device__ __forceinline__ void residual_row(const Row<BLOCK, NPT>& U, const Row<BLOCK, NPT>& Q,
                                             double S, Row<BLOCK, NPT>& W) {
  float hs, ls;
  split_s<BLOCK, NPT>(S, hs, ls);
#pragma unroll
  for (int k = 0; k < NPT; ++k) W.v[k] = residual4(U.v[k], Q.v[k], hs, ls);
}

// The chain over candidates that share the draft row Q: S, C start at 0,
// sum U; on a rejection S <- S + C and C <- F(S) (kept if F(S) = 0, as the
// step-by-step form keeps the previous row).  Returns the accepted
// candidate's index or -1; S and C describe the adjusted row afterwards.
// With stop_at_accept (the walk's chain, whose row is then only drawn from)
// the last candidate's rejection skips the pass for F: S becomes S + C and
// Sprev keeps the previous S, C is left stale, and the draw, which sums the
// row itself, goes back to Sprev if the row at S has no mass (the sums are
// of non-negative entries: zero exactly when F would be).
template <int BLOCK, int NPT, bool RATIO>
__device__ __forceinline__ int run_chain_shared(const Row<BLOCK, NPT>& U, const Row<BLOCK, NPT>& Q,
                                                double& S, double& Sprev, double& C, const Cand& cd,
                                                int nk, bool stop_at_accept, Shared<BLOCK, NPT>& sh,
                                                int& rb) {
  Sprev = S;
  const int tid = threadIdx.x;
#pragma nounroll
  for (int s = 0; s < nk; ++s) {
    // the next row's S (and its fp32 pair) does not depend on the test: it
    // is formed alongside it, and the test's operands are read without
    // branches (selects after unconditional lane reads)
    const double Sn = S + C;
    float hs, ls, hn;
    split_s<BLOCK, NPT>(S, hs, ls);
    hn = (float)Sn;
    const float wl = residual(cd.ut, cd.q, hs, ls);  // each lane's candidate entry
    const bool tok_ok = lane_i(cd.tok, s) >= 0;
    const double qraw = (double)lane_f(cd.q, s), nraw = (double)lane_f(wl, s);
    const double uu = (double)lane_f(cd.u, s);
    const double qt = tok_ok ? qraw : 0.0;
    const double num = tok_ok ? nraw : 0.0;
    const double den = C * qt;
    const bool accept = (qt > 0.0 && uu * den < num) || (!(qt > 0.0) && num > 0.0);
    if (RATIO && tid == 0)
      sh.ratio[s] = qt > 0.0 ? (float)(num / den) : (num > 0.0 ? INFINITY : 0.f);
    if (stop_at_accept && accept) return s;
    if (stop_at_accept && s == nk - 1) {
      Sprev = S;
      S = Sn;
      return -1;
    }
    const double Cn = residual_mass<BLOCK, NPT>(U, Q, hn, sh, rb);
    if (Cn > 0.0) {
      S = Sn;
      C = Cn;
    }
  }
  return -1;
}

// Set-up of one node's chain after the tree is in LDS and the node's logits
// were issued into U: its children (sh.kids, and per lane in cd), whether
// they share one draft row (`shared`) and then that row into Q, issued once U
// has arrived: the stats, which need all of U first, no longer wait for a
// second row sharing the CU's bandwidth, and the row still lands in time for
// the chain (whole verification, 32000-entry vocabulary: 26.3 -> 25.1 us at
// 1 x 26 nodes, 21.4 -> 17.8 us at 8 x 26, 63.6 -> 57.2 us at 16 x 60); or else the
// first candidate's row prefetch and the table qt[k][i] = q_{kid k}(t_{kid i});
// each candidate's own logit (gathered while the row pass runs), then the row
// statistics.  Returns the argmax (T = 0); sets C, ut (U at the first
// candidate's token) and, on lane i < nk, val = U at candidate i's token.
template <int BLOCK, int NPT, bool GREEDY, bool VEC>
__device__ __forceinline__ int node_setup(const VArgs& a, size_t ob, int node, int b,
                                          int32_t* flags, Row<BLOCK, NPT>& U,
                                          Row<BLOCK, NPT>& Q, double& C, float& ut,
                                          float& val, Cand& cd, bool& shared,
                                          Shared<BLOCK, NPT>& sh, float4* qlds, int& rb) {
  const int tid = threadIdx.x, lane = tid & 63, V = a.V;
  find_kids<BLOCK, NPT>(a.N, node, sh);
  barrier_lds();
  const int nk = sh.nk;
  ut = 0.f;
  val = 0.f;
  shared = false;
  if constexpr (GREEDY) {
    return target_stats<BLOCK, NPT, true>(U, a.T, b, flags, C, [] {}, [](float, float) {}, sh,
                                          rb);
  } else {
    cd.kid = 0;
    cd.tok = -1;
    cd.row = 0;
    cd.u = 0.f;
    cd.q = 0.f;
    cd.ut = 0.f;
    if (lane < nk) {
      cd.kid = sh.kids[lane];
      const int t = sh.tok[cd.kid];
      cd.tok = t >= 0 && t < V ? t : -1;
      cd.u = sh.u[cd.kid];
      cd.row = sh.row[cd.kid];
    }
    const int r0 = lane_i(cd.row, 0);
    shared = nk > 0 && __ballot(lane < nk && cd.row != r0) == 0;  // wave-uniform
    if (shared) {
      // each candidate's probability in the one draft row
      if (cd.tok >= 0) cd.q = a.draft[(ob + r0) * V + cd.tok];
    } else if (nk > 0 && VEC) {
      // slots past V are never loaded: zero this thread's (the pass reads them)
#pragma unroll
      for (int k = 0; k < NPT; ++k)
        if ((k * BLOCK + tid) * 4 >= V) qlds[k * BLOCK + tid] = make_float4(0.f, 0.f, 0.f, 0.f);
      issue_row_lds<BLOCK, NPT>(a.draft + (ob + lane_i(cd.row, 0)) * V, V, qlds);
    }
    constexpr int G = (64 * 64 + BLOCK - 1) / BLOCK;
    float g[G];
    if (!shared) {
#pragma unroll
      for (int r = 0; r < G; ++r) {
        const int f = r * BLOCK + tid;
        const int k = f / 64, i = f & 63;
        g[r] = 0.f;
        if (k <= i && i < nk) {
          const int t = sh.tok[sh.kids[i]];
          if (t >= 0 && t < V) g[r] = a.draft[(ob + sh.row[sh.kids[k]]) * V + t];
        }
      }
    }
    float lt = 0.f;
    if (cd.tok >= 0) lt = a.logits[(ob + node) * V + cd.tok];
    target_stats<BLOCK, NPT, false>(
        U, a.T, b, flags, C,
        [&] {
          if (shared) {
            if constexpr (VEC)
              load_row_vec<BLOCK, NPT>(Q, a.draft + (ob + r0) * V, V, 0.f);
            else
              load_row<BLOCK, NPT>(Q, a.draft + (ob + r0) * V, V, 0.f);
          }
        },
        [&](float nmi, float invT) {
          if (!shared) {
#pragma unroll
            for (int r = 0; r < G; ++r) {
              const int f = r * BLOCK + tid;
              const int k = f / 64, i = f & 63;
              if (k <= i && i < nk) sh.qt[tri(k, i)] = g[r];
            }
          }
          if (lane < nk) val = target_entry(lt, nmi, invT);
        },
        sh, rb);
    // the table is published by the mass reduction's barrier
    if (!shared && lane < nk) cd.q = sh.qt[tri(lane, lane)];
    cd.ut = val;
    ut = lane_f(val, 0);
    return 0;
  }
}

// Inclusive prefix sum over the wave in lane order: shifts by 1, 2, 4, 8
// within each row of 16, then the last lane of row 0 (of row 2) added to row 1
// (row 3), then lane 31 added to rows 2 and 3.
__device__ __forceinline__ double wave_incl_scan_d(double v) {
  v += dpp_d<0x111>(v);  // row_shr:1
  v += dpp_d<0x112>(v);  // row_shr:2
  v += dpp_d<0x114>(v);  // row_shr:4
  v += dpp_d<0x118>(v);  // row_shr:8
  v += __hiloint2double(__builtin_amdgcn_update_dpp(0, __double2hiint(v), 0x142, 0xa, 0xf, false),
                        __builtin_amdgcn_update_dpp(0, __double2loint(v), 0x142, 0xa, 0xf, false));
  v += __hiloint2double(__builtin_amdgcn_update_dpp(0, __double2hiint(v), 0x143, 0xc, 0xf, false),
                        __builtin_amdgcn_update_dpp(0, __double2loint(v), 0x143, 0xc, 0xf, false));
  return v;
}

// Inverse-CDF draw from the row W / sum(W) with uniform u: the smallest id
// whose cumulative mass exceeds u * sum, accumulated in id order.  `ent(k)`
// gives this thread's four entries of slab k (ids (k * BLOCK + tid) * 4 + e,
// entries past V zero), so the row can be the adjusted row computed on the
// fly.  The cumulative sums are built in levels over consecutive ids: a
// group (one thread's four entries, summed left to right in fp32), a lane
// group (BLOCK / 64 consecutive groups, fp64), a slab (2048 or 1024 ids, a
// wave's prefix scan of its lane groups), the row (a scan of the slab
// totals over one lane each, done alike by every wave).  The draw
// descends the levels: the first slab whose end exceeds the threshold, in it
// the first lane group, in that the first group (its lane group's sums read
// at once, then walked without further LDS round trips: whole verification
// at the 7B shape 24.4 -> 23.4 us), in that the first entry; an
// entry's cumulative sum is its group's start plus the group's own fp32
// prefix, which ends exactly at the group's sum.  Where the levels' fp64
// roundings leave no crossing inside the chosen lane group (a window of about
// 1e-16 of the mass), or u rounds to the whole mass, the last entry with mass
// in the chosen range (else the row) is taken; a row without mass gives -1.
// `scratch` holds NPT * BLOCK floats and NPT * 64 doubles of free LDS.
template <int BLOCK, int NPT, typename E>
__device__ __forceinline__ int inverse_cdf(E&& ent, float u, int V, Shared<BLOCK, NPT>& sh,
                                           void* scratch, int& rb) {
  constexpr int NW = BLOCK / 64;
  constexpr int GPL = BLOCK / 64;  // groups per lane group
  static_assert(NPT % NW == 0, "whole slabs per wave");
  static_assert(GPL % 4 == 0 && NPT <= 64, "lane groups read as float4; slab totals one per lane");
  constexpr int SPW = NPT / NW;    // slabs per wave
  float* gbuf = static_cast<float*>(scratch);                       // [NPT][BLOCK]
  double* lsc = reinterpret_cast<double*>(gbuf + NPT * BLOCK);      // [NPT][64]
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
#pragma unroll
  for (int k = 0; k < NPT; ++k) {
    const float4 w = ent(k);
    gbuf[k * BLOCK + tid] = ((w.x + w.y) + w.z) + w.w;
  }
  if (tid == 0) sh.pick = -1;
  barrier_lds();
#pragma unroll
  for (int i = 0; i < SPW; ++i) {
    const int k = wave * SPW + i;
    double ls = 0.0;
#pragma unroll
    for (int g = 0; g < GPL; ++g) ls += (double)gbuf[k * BLOCK + lane * GPL + g];
    lsc[k * 64 + lane] = wave_incl_scan_d(ls);
  }
  barrier_lds();
  // every wave takes the same decisions from the same LDS values: the slab
  // totals' prefix by a scan over lanes 0..NPT-1, the crossing slab, then
  // its crossing lane group and group
  const double tot = lane < NPT ? lsc[lane * 64 + 63] : 0.0;
  const double tinc = wave_incl_scan_d(tot);
  const double Z = lane_d(tinc, NPT - 1);
  const double thr = (double)u * Z;
  const uint64_t over = __ballot(lane < NPT && tinc > thr);
  int ks = over ? __ffsll((unsigned long long)over) - 1 : -1;
  if (ks >= 0) {
    const double bk = ks > 0 ? lane_d(tinc, ks - 1) : 0.0;
    const double incl = lsc[ks * 64 + lane];
    const uint64_t cross = __ballot(bk + incl > thr);
    const int L = cross ? __ffsll((unsigned long long)cross) - 1 : 63;
    double base = bk + (L > 0 ? lane_d(incl, L - 1) : 0.0);
    // the lane group's GPL group sums, read before any is used
    float gm[GPL];
#pragma unroll
    for (int h = 0; h < GPL / 4; ++h) {
      const float4 q4 = reinterpret_cast<const float4*>(gbuf + ks * BLOCK + L * GPL)[h];
      gm[4 * h] = q4.x;
      gm[4 * h + 1] = q4.y;
      gm[4 * h + 2] = q4.z;
      gm[4 * h + 3] = q4.w;
    }
    int gsel = -1, glast = -1;
    double gbase = base;
#pragma unroll
    for (int g = 0; g < GPL; ++g) {
      const double nb = base + (double)gm[g];
      const bool hit = gsel < 0 && nb > thr;
      gbase = hit ? base : gbase;
      gsel = hit ? g : gsel;
      glast = gm[g] > 0.f ? g : glast;
      base = nb;
    }
    const bool fallback = gsel < 0;
    if (fallback) gsel = glast;
    if (gsel >= 0 && tid == L * GPL + gsel) {
      float4 w = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
      for (int k = 0; k < NPT; ++k)
        if (k == ks) w = ent(k);
      const int id0 = (ks * BLOCK + tid) * 4;
      float pre = 0.f;
      int cand = -1, lastpos = -1;
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const float x = comp(w, c);
        pre = c == 0 ? x : pre + x;
        if (id0 + c < V && x > 0.f) {
          lastpos = id0 + c;
          if (cand < 0 && !fallback && gbase + (double)pre > thr) cand = id0 + c;
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
    for (int k = 0; k < NPT; ++k) {
      const float4 w = ent(k);
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const int idx = (k * BLOCK + tid) * 4 + c;
        if (idx < V && comp(w, c) > 0.f) last = idx;
      }
    }
    pick = block_max_i<BLOCK, NPT>(last, sh, rb);  // -1: the row has no mass
  }
  return pick;
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

// Per-sequence set-up shared by the kernels, in two halves so that the
// tree's few loads can be issued ahead of a row's: fetch_tree reads the tree
// (parent links, tokens, uniforms, draft rows of sequence b, threads < N)
// into registers; store_tree sanitises it into LDS and reports data errors
// (bad token, draft row out of range).
struct TreeRegs {
  int par, tok, row, L;
  float u;
};

__device__ __forceinline__ TreeRegs fetch_tree(const VArgs& a, int b) {
  const int tid = threadIdx.x, N = a.N;
  const size_t ob = (size_t)b * N;
  TreeRegs t{-1, 0, 0, 0, 0.f};
  if (tid < N) {
    t.par = a.parents[ob + tid];
    t.tok = a.tokens[ob + tid];
    t.u = a.uniforms[ob + tid];
    t.row = a.draft_row ? a.draft_row[ob + tid] : tid;
    if (tid == 0) t.L = a.kv_len[b];
  }
  return t;
}

template <int BLOCK, int NPT>
__device__ __forceinline__ void store_tree(const VArgs& a, int b, const TreeRegs& t, bool flag_here,
                                           Shared<BLOCK, NPT>& sh) {
  const int tid = threadIdx.x, N = a.N, V = a.V;
  bool tok_bad = false, row_bad = false;
  if (tid < N) {
    if (tid == 0) sh.Lkv = t.L;
    int par = t.par;
    if (tid == 0)
      par = -1;
    else if (par != -1 && (par < 0 || par >= tid))
      par = 0;  // a bad link hangs off the root; -1 (absent node) is nobody's child
    const bool present = tid > 0 && par != -1;
    tok_bad = present && (t.tok < 0 || t.tok >= V);
    row_bad = present && (t.row < 0 || t.row >= N);
    sh.par[tid] = par;
    sh.tok[tid] = t.tok;
    sh.u[tid] = t.u;
    sh.row[tid] = t.row >= 0 && t.row < N ? t.row : tid;  // in range whatever the input
  }
  if (tid < 64) {  // N <= 64: the whole tree sits in wave 0
    const uint64_t tb = __ballot(tok_bad), rbm = __ballot(row_bad);
    if (flag_here && tid == 0 && a.flags) {
      if (tb) atomicOr(a.flags + b, EAGLE_FLAG_BAD_TOKEN);
      if (rbm && a.draft_row && a.T > 0.f) atomicOr(a.flags + b, EAGLE_FLAG_BAD_ROW);
    }
  }
}

// The walk's outputs for sequence b once sh.path[0..m] and the final token
// are known: path, KV source slots, accepted tokens, accept length, final
// token, then the compaction when fused.
template <int BLOCK, int NPT>
__device__ __forceinline__ void write_walk(const VArgs& a, int b, int m_acc, int pick,
                                           Shared<BLOCK, NPT>& sh) {
  const int tid = threadIdx.x, N = a.N;
  const size_t ob = (size_t)b * N;
  const int Lkv = sh.Lkv;
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
    a.bonus[b] = pick;
  }
  if (a.kc.k) fused_compact(a.kc, b, N, m_acc, a.flags, sh);
}

template <int BLOCK, int NPT, bool GREEDY, bool PARITY, bool VEC>
__global__ __launch_bounds__(BLOCK) void verify_node_kernel(VArgs a) {
  __shared__ Shared<BLOCK, NPT> sh;
  __shared__ float4 qlds[GREEDY ? 1 : NPT * BLOCK];  // draft-row prefetch / final-draw scratch
  const int N = a.N, V = a.V;
  const int tid = threadIdx.x;
  const int node = blockIdx.x;
  const int b = node / N;
  const int j = node - b * N;
  const size_t ob = (size_t)b * N;
  int rb = 0;

  // the tree's few loads first, then the node's logit row (vector loads
  // complete in order: the tree is not held up behind the row)
  const TreeRegs tr = fetch_tree(a, b);
  asm volatile("" ::: "memory");
  Row<BLOCK, NPT> U;
  Row<BLOCK, NPT> Q;  // the shared draft row, or the second row of the step-by-step chain
  if constexpr (VEC)
    load_row_vec<BLOCK, NPT>(U, a.logits + (ob + j) * V, V, -FLT_MAX);
  else
    load_row<BLOCK, NPT>(U, a.logits + (ob + j) * V, V, -FLT_MAX);
  store_tree<BLOCK, NPT>(a, b, tr, j == 0, sh);
  barrier_lds();
  double C = 1.0;
  float ut = 0.f, val = 0.f;
  Cand cd{0, -1, 0, 0.f, 0.f, 0.f};
  bool shared;
  const int am = node_setup<BLOCK, NPT, GREEDY, VEC>(a, ob, j, b, a.flags, U, Q, C, ut, val, cd,
                                                     shared, sh, qlds, rb);
  const int nk = sh.nk;

  if (PARITY && a.out_probs) {
    // p = U / C through one fp64 reciprocal (within an fp64 ulp of the
    // quotient, far below the fp32 result's rounding)
    float* po = a.out_probs + (ob + j) * V;
    const double inv = 1.0 / C;
#pragma unroll
    for (int k = 0; k < NPT; ++k)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int idx = (k * BLOCK + tid) * 4 + e;
        if (idx < V) po[idx] = GREEDY ? (idx == am ? 1.f : 0.f) : (float)((double)comp(U.v[k], e) * inv);
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
    int si;
    if (shared) {
      double S = 0.0, Sprev = 0.0;
      si = run_chain_shared<BLOCK, NPT, PARITY>(U, Q, S, Sprev, C, cd, nk, true, sh, rb);
      if (si < 0) {  // the final token from the adjusted row, computed on the fly
        float hs, ls;
        split_s<BLOCK, NPT>(S, hs, ls);
        bonus = inverse_cdf<BLOCK, NPT>(
            [&](int k) { return residual4(U.v[k], Q.v[k], hs, ls); }, sh.u[0], V, sh, qlds, rb);
        if (bonus < 0 && nk > 0) {  // the last rejection left no mass: the row before it
          split_s<BLOCK, NPT>(Sprev, hs, ls);
          bonus = inverse_cdf<BLOCK, NPT>(
              [&](int k) { return residual4(U.v[k], Q.v[k], hs, ls); }, sh.u[0], V, sh, qlds, rb);
        }
        bonus = max(bonus, 0);
      }
    } else {
      si = run_chain<BLOCK, NPT, VEC, PARITY>(a, ob, U, Q, C, ut, val, cd, nk, true, sh, qlds, rb);
      if (si < 0)
        bonus = max(0, inverse_cdf<BLOCK, NPT>([&](int k) { return U.v[k]; }, sh.u[0], V, sh, qlds,
                                               rb));
    }
    if (si >= 0) {
      acc = sh.kids[si];
      ntested = si + 1;
    }
  }
  // a prefetch left in flight by an early acceptance must land before exit
  if (!GREEDY && VEC) asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();

  // publish this node's outcome; the last workgroup of the sequence walks the tree
  if (tid == 0) {
    st_c(a.nr.acc + ob + j, acc);
    st_c(a.nr.ntested + ob + j, ntested);
    st_c(a.nr.bonus + ob + j, bonus);
  }
  if (PARITY && tid < ntested) st_c(a.nr.ratio + ob + sh.kids[tid], sh.ratio[tid]);  // read by out_ratio only
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  if (tid == 0) {
    const int ticket = __hip_atomic_fetch_add(a.nr.counter + b, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    sh.last = ticket == N - 1;
  }
  __syncthreads();
  if (!sh.last) return;

  // ---- walk (last workgroup of sequence b) -----------------------------------
  // The walk starts at the root: when the last workgroup is the root's own and
  // it accepted none of its children, the walk ends there and needs no other
  // node's published outcome (the 7B step, whose root rejects all 15
  // children, saves the loads' round trip: whole verification 23.5 -> 22.8 us)
  const bool root_only = !PARITY && j == 0 && acc < 0;
  if (!root_only && tid < N) {
    // all three loads in flight before any result is used
    const int r0 = ld_c(a.nr.acc + ob + tid);
    const int r1 = ld_c(a.nr.bonus + ob + tid);
    const int r2 = ld_c(a.nr.ntested + ob + tid);
    sh.wacc[tid] = r0;
    sh.wbonus[tid] = r1;
    sh.wnt[tid] = r2;
  }
  __syncthreads();
  if (tid == 0) {
    int cur = 0, m_acc = 0;
    sh.path[0] = 0;
    for (; !root_only;) {
      const int nx = sh.wacc[cur];
      if (nx < 0 || nx <= cur || nx >= N) break;  // nx > cur for any valid walk
      sh.path[++m_acc] = nx;
      cur = nx;
    }
    sh.term = cur;
    sh.pick = min(max(root_only ? bonus : sh.wbonus[cur], 0), V - 1);
    sh.nk = m_acc;
    __hip_atomic_store(a.nr.counter + b, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  __syncthreads();
  const int m_acc = sh.nk;
  write_walk<BLOCK, NPT>(a, b, m_acc, sh.pick, sh);
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
      if constexpr (VEC)
        load_row_vec<BLOCK, NPT>(U, a.logits + (ob + term) * V, V, -FLT_MAX);
      else
        load_row<BLOCK, NPT>(U, a.logits + (ob + term) * V, V, -FLT_MAX);
      node_setup<BLOCK, NPT, false, VEC>(a, ob, term, b, nullptr, U, Q, C, ut, val, cd, shared, sh,
                                         qlds, rb);
      if (shared) {
        double S = 0.0;
        double Sprev = 0.0;
        run_chain_shared<BLOCK, NPT, false>(U, Q, S, Sprev, C, cd, sh.nk, false, sh, rb);
        residual_row<BLOCK, NPT>(U, Q, S, U);
      } else {
        run_chain<BLOCK, NPT, VEC, false>(a, ob, U, Q, C, ut, val, cd, sh.nk, false, sh, qlds, rb);
      }
      const double inv = 1.0 / C;
#pragma unroll
      for (int k = 0; k < NPT; ++k)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int idx = (k * BLOCK + tid) * 4 + e;
          if (idx < V) fo[idx] = (float)((double)comp(U.v[k], e) * inv);
        }
    }
  }
}

// ---- temperature 0: the argmax over a split row ---------------------------------
// At T = 0 a node's outcome is fixed by its row's argmax.  Each of the node's
// P workgroups takes a slice of the row, finds the slice's maximum and its
// lowest index, and posts them as one 64-bit key (order-preserving value bits
// above the inverted index) with an atomic maximum, so the word ends up with
// the row's maximum and its lowest index whatever the order of arrival.  No
// workgroup waits for another: every workgroup then takes the sequence's
// ticket, and the one that draws the last (of N * P) walks, reading the words
// and zeroing them and the ticket for the next call.  Every workgroup fetches
// the sequence's tree at its start (a few bytes), so the walker has it.
__device__ __forceinline__ uint32_t order_key(float v) {
  const uint32_t bits = __float_as_uint(v);
  return (bits & 0x80000000u) ? ~bits : (bits | 0x80000000u);
}

template <int NPT>
__global__ __launch_bounds__(256) void verify_argmax_kernel(VArgs a) {
  constexpr int BLOCK = 256, NW = BLOCK / 64;
  __shared__ Shared<BLOCK, NPT> sh;
  __shared__ uint32_t wkey[NW], widx[NW];
  const int N = a.N, V = a.V, P = a.P;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int node = blockIdx.x / P, part = blockIdx.x - node * P;
  const int b = node / N;
  const int j = node - b * N;
  const size_t ob = (size_t)b * N;
  const int s4 = ((V + 3) / 4 + P - 1) / P;  // float4 per part (the host keeps every slice non-empty)
  const int base = part * s4 * 4;
  const int len = min(V - base, s4 * 4);
  const TreeRegs tr = fetch_tree(a, b);
  asm volatile("" ::: "memory");
  Row<BLOCK, NPT> U;
  load_row<BLOCK, NPT>(U, a.logits + (ob + j) * V + base, len, -FLT_MAX);
  sanitize_logits<BLOCK, NPT>(U, b, a.flags);
  // the slice's maximum and its lowest index: per thread (ids increase with
  // (k, e)), per wave (maximum key, then the lowest index holding it), then
  // across the waves in one barrier
  float lm = -INFINITY;
  int li = INT_MAX;
#pragma unroll
  for (int k = 0; k < NPT; ++k)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float x = comp(U.v[k], e);
      const bool gt = x > lm;
      lm = gt ? x : lm;
      li = gt ? (k * BLOCK + tid) * 4 + e : li;
    }
  const int sk = (int)(order_key(lm) ^ 0x80000000u);  // order-preserving as a signed int
  const int wk = wave_allmax_i(sk);
  const int wi = wave_allmin_i(sk == wk ? li : INT_MAX);
  if (lane == 0) {
    wkey[wave] = (uint32_t)wk;
    widx[wave] = (uint32_t)wi;
  }
  barrier_lds();
  if (tid == 0) {
    int bk = (int)wkey[0], bi = (int)widx[0];
#pragma unroll
    for (int w = 1; w < NW; ++w) {
      const int k = (int)wkey[w], i = (int)widx[w];
      if (k > bk || (k == bk && i < bi)) {
        bk = k;
        bi = i;
      }
    }
    const uint64_t key = ((uint64_t)((uint32_t)bk ^ 0x80000000u) << 32) |
                         (uint64_t)(0xffffffffu - (uint32_t)(base + bi));
    __hip_atomic_fetch_max(a.nr.amax + node, (unsigned long long)key, __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // the maximum is in before the ticket
    const int ts = __hip_atomic_fetch_add(a.nr.counter + b, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const int last = ts == N * P - 1;
    if (last) __hip_atomic_store(a.nr.counter + b, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    sh.last = last;
  }
  barrier_lds();
  if (!sh.last) return;

  // ---- walk (last workgroup of sequence b) -----------------------------------
  store_tree<BLOCK, NPT>(a, b, tr, true, sh);
  if (tid < N) {
    unsigned long long* w = a.nr.amax + ob + tid;
    const unsigned long long k = __hip_atomic_load(w, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_store(w, 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    sh.wbonus[tid] = (int)(0xffffffffu - (uint32_t)(k & 0xffffffffull));  // the node's argmax
  }
  __syncthreads();
  if (tid == 0) {
    int cur = 0, m_acc = 0;
    sh.path[0] = 0;
    for (;;) {
      const int am_cur = sh.wbonus[cur];
      int nx = -1;
      for (int c = cur + 1; c < N && nx < 0; ++c)
        if (sh.par[c] == cur && sh.tok[c] == am_cur) nx = c;
      if (nx < 0) break;
      sh.path[++m_acc] = nx;
      cur = nx;
    }
    sh.pick = min(max(sh.wbonus[cur], 0), V - 1);
    sh.nk = m_acc;
  }
  __syncthreads();
  write_walk<BLOCK, NPT>(a, b, sh.nk, sh.pick, sh);
}

// ---------------------------------------------------------------------------
// T = 0 without parity outputs may split each row over P workgroups of 256
// threads (at most 8 float4 per thread).  The P slices of a row meet on one
// packed maximum before the sequence's ticket, a second round trip to memory
// that the unsplit node kernel (one 512-thread workgroup per row, its
// argmax published with the ticket) does not pay, so splitting pays only for
// a handful of nodes (graph-timed, V = 32000, 7B layer: 8 nodes 5.8 us split
// against 6.6 unsplit; 16 nodes 7.2 against 6.8; 26 nodes 9.1 against 7.7;
// 52 nodes 9.3 either way).  About 128 workgroups in all is the target, and
// a row needing more slices than that gives reads in one workgroup instead.
static int argmax_parts(int B, int N, int V) {
  const long long nodes = (long long)B * N;
  if (V <= 4096 || nodes > 8) return 1;
  const int v4 = (V + 3) / 4;
  const int min_parts = (v4 + 8 * 256 - 1) / (8 * 256);
  const long long want = 128 / std::max<long long>(nodes, 1);
  if (want < 2 || want < min_parts) return 1;
  int P = (int)std::min<long long>(want, 16);
  while (P > 1 && (long long)(P - 1) * ((v4 + P - 1) / P) >= v4) --P;  // no empty slice
  return P < min_parts ? 1 : P;
}

static int argmax_npt(int V, int P) {
  const int per = (((V + 3) / 4 + P - 1) / P + 255) / 256;
  return per <= 1 ? 1 : per <= 2 ? 2 : per <= 4 ? 4 : 8;
}

VerifyPlan plan_verify(int B, int N, int V) {
  VerifyPlan p{};
  p.V = V;
  p.parts = argmax_parts(B, N, V);
  const size_t nodes = (size_t)B * N;
  p.ws_counters = (size_t)B * 4;
  p.ws_amax = nodes * 8;
  p.ws_stats = nodes * 16;  // acc, bonus, ratio, ntested
  return p;
}

static size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

size_t verify_workspace_bytes(const VerifyPlan& p) {
  return align256(p.ws_counters) + align256(p.ws_amax) + align256(p.ws_stats);
}

hipError_t launch_verify(const VerifyPlan& plan, const int32_t* tokens, const float* draft,
                         const int32_t* draft_row, const float* logits, const int32_t* parents,
                         const int32_t* kv_len, int B, int N, float T, const float* uniforms,
                         int32_t* accept_len, int32_t* path, int32_t* acc_tokens, int32_t* bonus,
                         int32_t* kv_src, float* out_probs, float* out_final, float* out_ratio,
                         void* ws, int32_t* flags, const VerifyCompact& kc, hipStream_t s) {
  uint8_t* w = static_cast<uint8_t*>(ws);
  const size_t nodes = (size_t)B * N;
  VArgs a{};
  a.tokens = tokens;
  a.draft = draft;
  a.draft_row = draft_row;
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
  size_t off = 0;
  a.nr.counter = reinterpret_cast<int32_t*>(w + off);
  off += align256(plan.ws_counters);
  a.nr.amax = reinterpret_cast<unsigned long long*>(w + off);
  off += align256(plan.ws_amax);
  a.nr.acc = reinterpret_cast<int32_t*>(w + off);
  a.nr.bonus = reinterpret_cast<int32_t*>(w + off + nodes * 4);
  a.nr.ratio = reinterpret_cast<float*>(w + off + nodes * 8);
  a.nr.ntested = reinterpret_cast<int32_t*>(w + off + nodes * 12);
  a.N = N;
  a.V = plan.V;
  a.nodes = (int)nodes;
  a.P = plan.parts;
  // a small batch is latency-bound: fetching a row that turns out unused
  // (a leaf's) costs bandwidth, not time
  a.T = T;
  const unsigned grid = (unsigned)nodes;
  const bool greedy = T == 0.f;
  const bool parity = out_probs || out_final || out_ratio;
  const bool vec = (plan.V & 3) == 0;
  if (greedy && !parity && plan.parts > 1) {
    const unsigned sgrid = (unsigned)(nodes * plan.parts);
    switch (argmax_npt(plan.V, plan.parts)) {
      case 1: verify_argmax_kernel<1><<<sgrid, 256, 0, s>>>(a); break;
      case 2: verify_argmax_kernel<2><<<sgrid, 256, 0, s>>>(a); break;
      case 4: verify_argmax_kernel<4><<<sgrid, 256, 0, s>>>(a); break;
      default: verify_argmax_kernel<8><<<sgrid, 256, 0, s>>>(a); break;
    }
    return hipGetLastError();
  }
#define EAGLE_LAUNCH_VERIFY(BLK, NPT)                                                        \
  do {                                                                                      \
    if (greedy && parity && vec) verify_node_kernel<BLK, NPT, true, true, true><<<grid, BLK, 0, s>>>(a); \
    else if (greedy && parity) verify_node_kernel<BLK, NPT, true, true, false><<<grid, BLK, 0, s>>>(a); \
    else if (greedy && vec) verify_node_kernel<BLK, NPT, true, false, true><<<grid, BLK, 0, s>>>(a);  \
    else if (greedy) verify_node_kernel<BLK, NPT, true, false, false><<<grid, BLK, 0, s>>>(a);        \
    else if (parity && vec) verify_node_kernel<BLK, NPT, false, true, true><<<grid, BLK, 0, s>>>(a); \
    else if (parity) verify_node_kernel<BLK, NPT, false, true, false><<<grid, BLK, 0, s>>>(a);       \
    else if (vec) verify_node_kernel<BLK, NPT, false, false, true><<<grid, BLK, 0, s>>>(a);          \
    else verify_node_kernel<BLK, NPT, false, false, false><<<grid, BLK, 0, s>>>(a);                  \
  } while (0)
  // the row must fit one workgroup: 512 threads of 16 float4 leave 256 VGPRs
  // per thread for the two resident rows (1024 threads would leave 128)
  if (plan.V > 4096)
    EAGLE_LAUNCH_VERIFY(512, 16);
  else
    EAGLE_LAUNCH_VERIFY(256, 4);
#undef EAGLE_LAUNCH_VERIFY
  return hipGetLastError();
}

}  // namespace eagle
