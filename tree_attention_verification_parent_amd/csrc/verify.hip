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
// rejections.  The rows live in registers across the workgroup (V <= 32768);
// the next candidate's draft row is prefetched while the current one is
// consumed; each candidate costs one workgroup barrier, which publishes the
// partial masses and the next candidate's U element together.  Masses and the
// inverse-CDF scan of the final draw accumulate in fp64.
#include <limits.h>
#include <stdlib.h>

#include "common.h"
#include "launch.h"

namespace eagle {

__device__ __forceinline__ float scaled_exp(float x, float m, float T, bool unit_T) {
  const float z = unit_T ? (x - m) : (x - m) / T;
  return expf(z);
}

// Per-node results published for the walk (device-coherent stores/loads).
struct NodeResults {
  int32_t* acc;      // [B*N] accepted candidate, -1 if none
  int32_t* bonus;    // [B*N] token drawn if the walk ends here
  float* ratio;      // [B*N] ratio of node c as tested by its parent's chain
  int32_t* ntested;  // [B*N] candidates of the node that its chain tested
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
  int N, V;
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

template <int BLOCK>
struct Shared {
  int par[64], tok[64], kids[64];
  float u[64], qt[64];
  float ratio[64];
  int nk;
  double red[BLOCK / 64];
  float redf[BLOCK / 64];
  int redi[BLOCK / 64];
  double gsum[8];
  float next_u[2];  // next candidate's U element: [0] after the update, [1] before
  int acc, bonus, term;
  int path[64];
};

template <int BLOCK>
__device__ __forceinline__ double block_sum(double v, Shared<BLOCK>& sh) {
  v = wave_sum(v);
  __syncthreads();
  if ((threadIdx.x & 63) == 0) sh.red[threadIdx.x >> 6] = v;
  __syncthreads();
  double t = 0.0;
#pragma unroll
  for (int i = 0; i < BLOCK / 64; ++i) t += sh.red[i];
  return t;
}

template <int BLOCK>
__device__ __forceinline__ float block_max(float v, Shared<BLOCK>& sh) {
  v = wave_max(v);
  __syncthreads();
  if ((threadIdx.x & 63) == 0) sh.redf[threadIdx.x >> 6] = v;
  __syncthreads();
  float t = -INFINITY;
#pragma unroll
  for (int i = 0; i < BLOCK / 64; ++i) t = fmaxf(t, sh.redf[i]);
  return t;
}

template <int BLOCK>
__device__ __forceinline__ int block_min_i(int v, Shared<BLOCK>& sh) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v = min(v, __shfl_xor(v, off));
  __syncthreads();
  if ((threadIdx.x & 63) == 0) sh.redi[threadIdx.x >> 6] = v;
  __syncthreads();
  int t = INT_MAX;
#pragma unroll
  for (int i = 0; i < BLOCK / 64; ++i) t = min(t, sh.redi[i]);
  return t;
}

template <int BLOCK>
__device__ __forceinline__ int block_max_i(int v, Shared<BLOCK>& sh) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v = max(v, __shfl_xor(v, off));
  __syncthreads();
  if ((threadIdx.x & 63) == 0) sh.redi[threadIdx.x >> 6] = v;
  __syncthreads();
  int t = INT_MIN;
#pragma unroll
  for (int i = 0; i < BLOCK / 64; ++i) t = max(t, sh.redi[i]);
  return t;
}

// Exclusive prefix over the workgroup in thread order, fp64.
template <int BLOCK>
__device__ __forceinline__ double block_excl_scan(double v, Shared<BLOCK>& sh) {
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  double incl = v;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const double o = __shfl_up(incl, off);
    if (lane >= off) incl += o;
  }
  __syncthreads();
  if (lane == 63) sh.red[wv] = incl;
  __syncthreads();
  double before = 0.0;
  for (int i = 0; i < wv; ++i) before += sh.red[i];
  return before + incl - v;
}

// A vocabulary row across the workgroup: thread t owns elements
// (k * BLOCK + t) * 4 + e, k < NPT, e < 4.
template <int BLOCK, int NPT>
struct Row {
  float4 v[NPT];
};

template <int BLOCK, int NPT>
__device__ __forceinline__ void load_row(Row<BLOCK, NPT>& r, const float* src, int V) {
  const int tid = threadIdx.x;
  if ((V & 3) == 0) {
#pragma unroll
    for (int k = 0; k < NPT; ++k) {
      const int e0 = (k * BLOCK + tid) * 4;
      r.v[k] = e0 < V ? *reinterpret_cast<const float4*>(src + e0) : make_float4(0.f, 0.f, 0.f, 0.f);
    }
  } else {
#pragma unroll
    for (int k = 0; k < NPT; ++k) {
      const int e0 = (k * BLOCK + tid) * 4;
      r.v[k].x = e0 + 0 < V ? src[e0 + 0] : 0.f;
      r.v[k].y = e0 + 1 < V ? src[e0 + 1] : 0.f;
      r.v[k].z = e0 + 2 < V ? src[e0 + 2] : 0.f;
      r.v[k].w = e0 + 3 < V ? src[e0 + 3] : 0.f;
    }
  }
}

__device__ __forceinline__ float comp(const float4& f, int e) {
  return e == 0 ? f.x : e == 1 ? f.y : e == 2 ? f.z : f.w;
}

template <int BLOCK, int NPT>
__device__ __forceinline__ float row_elem(const Row<BLOCK, NPT>& r, int k, int e) {
  float out = 0.f;
#pragma unroll
  for (int kk = 0; kk < NPT; ++kk)
    if (kk == k) out = comp(r.v[kk], e);
  return out;
}

// Target row of node j: U = exp((x - m)/T) with its mass C (T > 0), or the
// argmax (T = 0).  Flags non-finite logits.  Returns the argmax (T = 0).
template <int BLOCK, int NPT>
__device__ __forceinline__ int target_row(const VArgs a, int b, int node, Row<BLOCK, NPT>& U, double& C, float& m,
                          Shared<BLOCK>& sh) {
  const int tid = threadIdx.x, V = a.V;
  const float T = a.T;
  const bool unit_T = T == 1.f;
  load_row<BLOCK, NPT>(U, a.logits + ((size_t)b * a.N + node) * V, V);
  bool nonfinite = false;
  float lm = -INFINITY;
  int li = INT_MAX;
#pragma unroll
  for (int k = 0; k < NPT; ++k) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int idx = (k * BLOCK + tid) * 4 + e;
      const float x = comp(U.v[k], e);
      if (idx < V) {
        if (!isfinite(x)) nonfinite = true;
        else if (x > lm) {  // ids visited in increasing order within a thread
          lm = x;
          li = idx;
        }
      }
    }
  }
  if (__ballot(nonfinite) && (tid & 63) == 0 && a.flags) atomicOr(a.flags + b, EAGLE_FLAG_NONFINITE);
  if (T == 0.f) {
    // argmax: max value, then the lowest id holding it
    const float mx = block_max<BLOCK>(lm, sh);
    const int am = block_min_i<BLOCK>(lm == mx ? li : INT_MAX, sh);
    m = mx;
    return am == INT_MAX ? 0 : am;
  }
  m = block_max<BLOCK>(lm, sh);
  double part = 0.0;
#pragma unroll
  for (int k = 0; k < NPT; ++k) {
    float4& f = U.v[k];
    const int e0 = (k * BLOCK + tid) * 4;
    f.x = e0 + 0 < V && isfinite(f.x) ? scaled_exp(f.x, m, T, unit_T) : 0.f;
    f.y = e0 + 1 < V && isfinite(f.y) ? scaled_exp(f.y, m, T, unit_T) : 0.f;
    f.z = e0 + 2 < V && isfinite(f.z) ? scaled_exp(f.z, m, T, unit_T) : 0.f;
    f.w = e0 + 3 < V && isfinite(f.w) ? scaled_exp(f.w, m, T, unit_T) : 0.f;
    part += (double)f.x + (double)f.y + ((double)f.z + (double)f.w);
  }
  C = block_sum<BLOCK>(part, sh);
  return 0;
}

// Inverse-CDF draw from U / sum(U) with uniform u: the smallest id whose
// cumulative mass exceeds u * sum; if rounding leaves none, the last id with
// mass.  fp64 accumulation.
template <int BLOCK, int NPT>
__device__ __forceinline__ int inverse_cdf(const Row<BLOCK, NPT>& U, float u, int V, Shared<BLOCK>& sh) {
  const int tid = threadIdx.x;
#pragma unroll
  for (int k = 0; k < NPT; ++k) {
    const double t = block_sum<BLOCK>(
        (double)U.v[k].x + (double)U.v[k].y + ((double)U.v[k].z + (double)U.v[k].w), sh);
    if (tid == 0) sh.gsum[k] = t;
  }
  __syncthreads();
  double ztot = 0.0;
#pragma unroll
  for (int k = 0; k < NPT; ++k) ztot += sh.gsum[k];
  const double thr = (double)u * ztot;
  double run = 0.0;
  int kstar = -1;
#pragma unroll
  for (int k = 0; k < NPT; ++k) {
    if (kstar < 0 && run + sh.gsum[k] > thr) kstar = k;
    if (kstar < 0) run += sh.gsum[k];
  }
  int cand = INT_MAX;
  if (kstar >= 0) {
    float4 rv = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
    for (int k = 0; k < NPT; ++k)
      if (k == kstar) rv = U.v[k];
    const double before =
        run + block_excl_scan<BLOCK>((double)rv.x + (double)rv.y + ((double)rv.z + (double)rv.w), sh);
    const int base = (kstar * BLOCK + tid) * 4;
    double f = before;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      f += (double)comp(rv, e);
      if (cand == INT_MAX && f > thr && base + e < V) cand = base + e;
    }
  }
  int pick = block_min_i<BLOCK>(cand, sh);
  if (pick == INT_MAX) {
    int last = -1;
#pragma unroll
    for (int k = 0; k < NPT; ++k)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int idx = (k * BLOCK + tid) * 4 + e;
        if (idx < V && comp(U.v[k], e) > 0.f) last = idx;
      }
    pick = block_max_i<BLOCK>(last, sh);
    if (pick < 0) pick = 0;
  }
  return pick;
}

// Draft rows are prefetched into LDS with direct-to-LDS loads: thread t's
// float4 k lands at LDS float4 k*BLOCK + t, the same place it would occupy in
// the row, so each thread reads back only what it loaded itself (its own
// vmcnt wait suffices, no barrier).  Rows whose length is not a multiple of 4
// are loaded straight into registers instead.
template <int BLOCK, int NPT>
__device__ __forceinline__ void issue_row_lds(const float* src, int V, float4* qlds) {
  const int tid = threadIdx.x, wave = tid >> 6;
#pragma unroll
  for (int k = 0; k < NPT; ++k) {
    const int e0 = (k * BLOCK + tid) * 4;
    if (e0 < V)
      __builtin_amdgcn_global_load_lds(src + e0,
          (__attribute__((address_space(3))) void*)(qlds + k * BLOCK + wave * 64), 16, 0, 0);
  }
}

// The multi-round chain at one node: tests its candidates in order (stopping
// at the first acceptance when `stop_at_accept`), leaving the adjusted row in
// U (unnormalised, mass C).  Candidate s's ratio goes to sh.ratio[s].  Returns
// the index (into sh.kids) of the accepted candidate, or -1.
template <int BLOCK, int NPT>
__device__ __forceinline__ int run_chain(const VArgs a, int b, Row<BLOCK, NPT>& U, double& C, int nk,
                         bool stop_at_accept, Shared<BLOCK>& sh, float4* qlds) {
  const int tid = threadIdx.x, V = a.V, N = a.N;
  if (nk == 0) return -1;
  const bool vec = (V & 3) == 0;
  auto qrow = [&](int s) { return a.draft + ((size_t)b * N + sh.kids[s]) * V; };
  auto owner_of = [&](int t, int& k, int& e) {
    const int quad = t >> 2;
    k = quad / BLOCK;
    e = t & 3;
    return quad - k * BLOCK;
  };
  if (vec) issue_row_lds<BLOCK, NPT>(qrow(0), V, qlds);
  float ut = 0.f;
  {
    const int t = sh.tok[sh.kids[0]];
    if (t >= 0 && t < V) {
      int k, e;
      if (owner_of(t, k, e) == tid) sh.next_u[0] = row_elem<BLOCK, NPT>(U, k, e);
    }
    __syncthreads();
    ut = (t >= 0 && t < V) ? sh.next_u[0] : 0.f;
    __syncthreads();
  }
  // this thread's float4 k of the current draft row
  auto qv = [&](int k, int s) -> float4 {
    const int e0 = (k * BLOCK + tid) * 4;
    if (e0 >= V) return make_float4(0.f, 0.f, 0.f, 0.f);
    if (vec) return qlds[k * BLOCK + tid];
    const float* src = qrow(s) + e0;
    float4 q;
    q.x = src[0];
    q.y = e0 + 1 < V ? src[1] : 0.f;
    q.z = e0 + 2 < V ? src[2] : 0.f;
    q.w = e0 + 3 < V ? src[3] : 0.f;
    return q;
  };
  for (int s = 0; s < nk; ++s) {
    const int c = sh.kids[s];
    const int t = sh.tok[c];
    const bool tok_ok = t >= 0 && t < V;
    const double qt = tok_ok ? (double)sh.qt[c] : 0.0;
    const double num = tok_ok ? (double)ut : 0.0;
    double ratio;
    if (qt > 0.0)
      ratio = num / (C * qt);
    else
      ratio = num > 0.0 ? (double)INFINITY : 0.0;
    if (tid == 0) sh.ratio[s] = (float)ratio;
    if (stop_at_accept && (double)sh.u[c] < ratio) return s;
    // rejection: U <- max(0, U - C q_s).  Mass first (U kept until it is known
    // to be non-zero), then the update; q_s is read from LDS both times.
    if (vec) asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // own prefetch landed
    const float cf = (float)C;
    double part = 0.0;
#pragma unroll
    for (int k = 0; k < NPT; ++k) {
      const float4 q = qv(k, s);
      const float4 w = U.v[k];
      part += (double)fmaxf(0.f, w.x - cf * q.x) + (double)fmaxf(0.f, w.y - cf * q.y) +
              ((double)fmaxf(0.f, w.z - cf * q.z) + (double)fmaxf(0.f, w.w - cf * q.w));
    }
    // next candidate's element, after and before this update
    int tn = -1;
    if (s + 1 < nk) {
      int kn, en;
      tn = sh.tok[sh.kids[s + 1]];
      if (tn >= 0 && tn < V && owner_of(tn, kn, en) == tid) {
        const float w = row_elem<BLOCK, NPT>(U, kn, en);
        float q = 0.f;
#pragma unroll
        for (int k = 0; k < NPT; ++k)
          if (k == kn) q = comp(qv(k, s), en);
        sh.next_u[0] = fmaxf(0.f, w - cf * q);
        sh.next_u[1] = w;
      }
    }
    const double Cn = block_sum<BLOCK>(part, sh);  // its barriers publish next_u too
    const bool commit = Cn > 0.0;
    if (commit) {
#pragma unroll
      for (int k = 0; k < NPT; ++k) {
        const float4 q = qv(k, s);
        U.v[k].x = fmaxf(0.f, U.v[k].x - cf * q.x);
        U.v[k].y = fmaxf(0.f, U.v[k].y - cf * q.y);
        U.v[k].z = fmaxf(0.f, U.v[k].z - cf * q.z);
        U.v[k].w = fmaxf(0.f, U.v[k].w - cf * q.w);
      }
      C = Cn;
    }
    if (s + 1 < nk) {
      ut = (tn >= 0 && tn < V) ? sh.next_u[commit ? 0 : 1] : 0.f;
      if (vec) {
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // own reads done before the refill
        issue_row_lds<BLOCK, NPT>(qrow(s + 1), V, qlds);
      }
    }
    __syncthreads();  // next_u may be rewritten in the next round
  }
  return -1;
}

template <int BLOCK, int NPT, bool GREEDY, bool PARITY>
__global__ __launch_bounds__(BLOCK) void verify_node_kernel(VArgs a) {
  __shared__ Shared<BLOCK> sh;
  __shared__ float4 qlds[NPT * BLOCK];
  const int N = a.N, V = a.V;
  const int b = blockIdx.x / N;
  const int j = blockIdx.x - b * N;
  const int tid = threadIdx.x;
  constexpr bool greedy = GREEDY;
  const size_t ob = (size_t)b * N;

  // tree, tokens, uniforms, gathered draft mass of each node's own token
  bool tok_bad = false;
  if (tid < N) {
    int par = a.parents[ob + tid];
    if (tid == 0 || par < 0 || par >= tid) par = tid == 0 ? -1 : 0;
    const int tk = a.tokens[ob + tid];
    sh.par[tid] = par;
    sh.tok[tid] = tk;
    sh.u[tid] = a.uniforms[ob + tid];
    float qt = 0.f;
    if (tid > 0) {
      if (tk < 0 || tk >= V)
        tok_bad = true;
      else if (!greedy && par == j)
        qt = a.draft[(ob + tid) * V + tk];
    }
    sh.qt[tid] = qt;
  }
  if (j == 0 && __ballot(tok_bad) && (tid & 63) == 0 && a.flags)
    atomicOr(a.flags + b, EAGLE_FLAG_BAD_TOKEN);
  __syncthreads();
  if (tid == 0) {
    int nk = 0;
    for (int c = j + 1; c < N; ++c)
      if (sh.par[c] == j) sh.kids[nk++] = c;
    sh.nk = nk;
  }
  __syncthreads();
  const int nk = sh.nk;

  Row<BLOCK, NPT> U;
  double C = 1.0;
  float m = 0.f;
  const int am = target_row<BLOCK, NPT>(a, b, j, U, C, m, sh);

  if (PARITY && a.out_probs) {
    float* po = a.out_probs + (ob + j) * V;
    const float inv = greedy ? 0.f : (float)(1.0 / C);
#pragma unroll
    for (int k = 0; k < NPT; ++k)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int idx = (k * BLOCK + tid) * 4 + e;
        if (idx < V) po[idx] = greedy ? (idx == am ? 1.f : 0.f) : (float)((double)comp(U.v[k], e) / C);
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
    const int si = run_chain<BLOCK, NPT>(a, b, U, C, nk, true, sh, qlds);
    if (si >= 0) {
      acc = sh.kids[si];
      ntested = si + 1;
    } else {
      bonus = inverse_cdf<BLOCK, NPT>(U, sh.u[0], V, sh);
    }
  }
  __syncthreads();

  // publish this node's outcome; the last node of the sequence walks the tree
  if (tid == 0) {
    st_c(a.nr.acc + ob + j, acc);
    st_c(a.nr.bonus + ob + j, bonus);
    st_c(a.nr.ntested + ob + j, ntested);
  }
  if (tid < ntested) st_c(a.nr.ratio + ob + sh.kids[tid], sh.ratio[tid]);
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  if (tid == 0) {
    const int ticket = __hip_atomic_fetch_add(a.nr.counter + b, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    sh.acc = ticket == N - 1;
  }
  __syncthreads();
  if (!sh.acc) return;

  // ---- walk (last node workgroup of sequence b) ------------------------------
  if (tid == 0) {
    int cur = 0, m_acc = 0;
    sh.path[0] = 0;
    for (;;) {
      const int nx = ld_c(a.nr.acc + ob + cur);
      if (nx < 0 || nx <= cur || nx >= N) break;  // nx > cur for any valid walk
      sh.path[++m_acc] = nx;
      cur = nx;
    }
    sh.term = cur;
    sh.bonus = ld_c(a.nr.bonus + ob + cur);
    sh.nk = m_acc;
    __hip_atomic_store(a.nr.counter + b, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  __syncthreads();
  const int m_acc = sh.nk;
  if (tid < N) {
    const size_t o = ob + tid;
    const bool on = tid <= m_acc;
    const int node = on ? sh.path[tid] : -1;
    a.path[o] = node;
    a.kv_src[o] = on ? a.kv_len[b] + node : -1;
    a.acc_tokens[o] = tid < m_acc ? sh.tok[sh.path[tid + 1]] : -1;
  }
  if (tid == 0) {
    a.accept_len[b] = m_acc;
    a.bonus[b] = sh.bonus;
  }
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
          if (rank < ld_c(a.nr.ntested + ob + p)) r = ld_c(a.nr.ratio + ob + c);
        }
      }
      a.out_ratio[ob + c] = r;
    }
  }
  if (PARITY && a.out_final) {
    // the distribution of the final token: recompute the terminal's chain
    const int term = sh.term;
    __syncthreads();
    if (tid == 0) {
      int nk2 = 0;
      for (int c = term + 1; c < N; ++c)
        if (sh.par[c] == term) sh.kids[nk2++] = c;
      sh.nk = nk2;
    }
    if (tid < N) {
      const int tk = sh.tok[tid];
      sh.qt[tid] = (!greedy && tid > 0 && sh.par[tid] == term && tk >= 0 && tk < V)
                       ? a.draft[(ob + tid) * V + tk] : 0.f;
    }
    __syncthreads();
    float* fo = a.out_final + (size_t)b * V;
    if constexpr (GREEDY) {
      const int bt = sh.bonus;
      for (int v = tid; v < V; v += BLOCK) fo[v] = v == bt ? 1.f : 0.f;
    } else {
      target_row<BLOCK, NPT>(a, b, term, U, C, m, sh);
      run_chain<BLOCK, NPT>(a, b, U, C, sh.nk, false, sh, qlds);
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
VerifyPlan plan_verify(int B, int N, int V) {
  VerifyPlan p{};
  p.V = V;
  p.walk_threads = V > 4096 ? 1024 : 256;
  const size_t nodes = (size_t)B * N;
  p.ws_stats = nodes * 16;  // acc, bonus, ratio, ntested
  p.ws_counters = (size_t)B * 4;
  p.ws_partials = 0;
  p.chunks = 1;
  return p;
}

static size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

size_t verify_workspace_bytes(const VerifyPlan& p) {
  return align256(p.ws_counters) + align256(p.ws_stats);
}

hipError_t launch_verify(const VerifyPlan& plan, const int32_t* tokens, const float* draft,
                         const float* logits, const int32_t* parents, const int32_t* kv_len,
                         int B, int N, float T, const float* uniforms, int32_t* accept_len,
                         int32_t* path, int32_t* acc_tokens, int32_t* bonus, int32_t* kv_src,
                         float* out_probs, float* out_final, float* out_ratio, void* ws,
                         int32_t* flags, hipStream_t s) {
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
  a.nr.counter = reinterpret_cast<int32_t*>(w);
  uint8_t* nb = w + align256(plan.ws_counters);
  a.nr.acc = reinterpret_cast<int32_t*>(nb);
  a.nr.bonus = reinterpret_cast<int32_t*>(nb + nodes * 4);
  a.nr.ratio = reinterpret_cast<float*>(nb + nodes * 8);
  a.nr.ntested = reinterpret_cast<int32_t*>(nb + nodes * 12);
  a.N = N;
  a.V = plan.V;
  a.T = T;
  const unsigned grid = (unsigned)nodes;
  const bool greedy = T == 0.f;
  const bool parity = out_probs || out_final || out_ratio;
#define EAGLE_LAUNCH_VERIFY(BLK, NPT)                                                   \
  do {                                                                                 \
    if (greedy && parity) verify_node_kernel<BLK, NPT, true, true><<<grid, BLK, 0, s>>>(a);     \
    else if (greedy) verify_node_kernel<BLK, NPT, true, false><<<grid, BLK, 0, s>>>(a);         \
    else if (parity) verify_node_kernel<BLK, NPT, false, true><<<grid, BLK, 0, s>>>(a);         \
    else verify_node_kernel<BLK, NPT, false, false><<<grid, BLK, 0, s>>>(a);                    \
  } while (0)
  if (plan.walk_threads == 1024)
    EAGLE_LAUNCH_VERIFY(1024, 8);
  else
    EAGLE_LAUNCH_VERIFY(256, 4);
#undef EAGLE_LAUNCH_VERIFY
  return hipGetLastError();
}

}  // namespace eagle
