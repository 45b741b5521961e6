// Vocabulary statistics and the acceptance walk of the verification step.
//
// Speculative sampling accepts a drafted token t with probability
// min(1, p(t)/p_hat(t)) and, after a rejection, draws from an adjusted
// distribution (EAGLE, paperlayer.ai summary, §2 Preliminaries); for a tree the
// procedure is applied recursively over each node's candidates and returns a
// sample of the target distribution (A.2 Multi-Round Speculative Sampling;
// B, the inputs of the procedure).  At temperature 0 the target emits its most
// probable token (EAGLE-2 overview blog, §1).
//
// Two kernels:
//   vocab_stats  row-parallel over every (sequence, node) target row and
//                vocabulary chunk: running max and sum of exp((x - max)/T)
//                (or the argmax at T = 0) per chunk, merged by the last chunk
//                of each row to finish; flags non-finite logits.
//   walk         one workgroup per sequence.  The scalar walk reads the row
//                statistics; a rejection streams the candidate's draft row
//                once and updates the residual r <- max(0, r/Z - q), held in
//                registers across the workgroup (V <= 32768), with its mass
//                summed in fp64.  The final token is an fp64 inverse-CDF scan.
// A third kernel writes the normalised target rows when the caller asks for
// them (parity checks only).
#include <limits.h>
#include <stdlib.h>

#include "common.h"
#include "launch.h"

namespace eagle {

struct RowStat {
  float m;     // row max (T > 0) or max value (T = 0)
  int amax;    // argmax, lowest id on ties
  double S;    // sum_v exp((x_v - m) / T)
};

__device__ __forceinline__ float scaled_exp(float x, float m, float T, bool unit_T) {
  const float z = unit_T ? (x - m) : (x - m) / T;
  return expf(z);
}

// Combine (m, s) partial softmax statistics.
__device__ __forceinline__ void ms_combine(float& m, double& s, float mo, double so, float T,
                                           bool unit_T) {
  const float mn = fmaxf(m, mo);
  if (mn == -INFINITY) {
    m = mn;
    s = 0.0;
    return;
  }
  const double a = s == 0.0 ? 0.0 : s * (double)scaled_exp(m, mn, T, unit_T);
  const double bb = so == 0.0 ? 0.0 : so * (double)scaled_exp(mo, mn, T, unit_T);
  m = mn;
  s = a + bb;
}

// Argmax combine: greater value wins, equal values keep the lower id.
__device__ __forceinline__ void am_combine(float& v, int& i, float vo, int io) {
  if (vo > v || (vo == v && io < i)) {
    v = vo;
    i = io;
  }
}

struct StatsArgs {
  const float* logits;
  RowStat* stats;
  RowStat* part;
  int32_t* counters;
  int32_t* flags;
  int rows, N, V, chunks;
  float T;
};

__global__ __launch_bounds__(256) void vocab_stats_kernel(StatsArgs a) {
  const int tid = threadIdx.x;
  const int row = blockIdx.x / a.chunks;
  const int ch = blockIdx.x - row * a.chunks;
  const int V = a.V;
  const bool vec = (V & 3) == 0;
  const int V4 = V >> 2;
  // chunk boundaries in units of 4 elements when vectorised
  int v0, v1;
  if (vec) {
    v0 = (int)((long long)ch * V4 / a.chunks) * 4;
    v1 = (int)((long long)(ch + 1) * V4 / a.chunks) * 4;
  } else {
    v0 = (int)((long long)ch * V / a.chunks);
    v1 = (int)((long long)(ch + 1) * V / a.chunks);
  }
  const float* x = a.logits + (size_t)row * V;
  const float T = a.T;
  const bool greedy = T == 0.f;
  const bool unit_T = T == 1.f;
  bool nonfinite = false;

  float m = -INFINITY;
  double s = 0.0;
  float sf = 0.f;
  int am = INT_MAX;
  auto visit = [&](float xv, int v) {
    if (!isfinite(xv)) {
      nonfinite = true;
      return;
    }
    if (greedy) {
      if (xv > m) {  // ids visited in increasing order per thread: first max kept
        m = xv;
        am = v;
      }
    } else if (xv > m) {
      sf = sf * scaled_exp(m, xv, T, unit_T) + 1.f;
      m = xv;
    } else {
      sf += scaled_exp(xv, m, T, unit_T);
    }
  };
  if (vec) {
    for (int v = v0 + 4 * tid; v < v1; v += 4 * 256) {
      const float4 q = *reinterpret_cast<const float4*>(x + v);
      visit(q.x, v);
      visit(q.y, v + 1);
      visit(q.z, v + 2);
      visit(q.w, v + 3);
    }
  } else {
    for (int v = v0 + tid; v < v1; v += 256) visit(x[v], v);
  }
  s = sf;

  // wave reduction
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) {
    const float mo = __shfl_xor(m, off);
    const double so = __shfl_xor(s, off);
    const int io = __shfl_xor(am, off);
    if (greedy)
      am_combine(m, am, mo, io);
    else
      ms_combine(m, s, mo, so, T, unit_T);
  }
  __shared__ float sm[4];
  __shared__ double ss[4];
  __shared__ int si[4];
  __shared__ int s_last;
  const int lane = tid & 63, wv = tid >> 6;
  const uint64_t bad = __ballot(nonfinite);
  if (lane == 0) {
    sm[wv] = m;
    ss[wv] = s;
    si[wv] = am;
    if (bad && a.flags) atomicOr(a.flags + row / a.N, EAGLE_FLAG_NONFINITE);
  }
  __syncthreads();
  if (tid == 0) {
    for (int k = 1; k < 4; ++k) {
      if (greedy)
        am_combine(m, am, sm[k], si[k]);
      else
        ms_combine(m, s, sm[k], ss[k], T, unit_T);
    }
    RowStat r;
    r.m = m;
    r.amax = am == INT_MAX ? 0 : am;
    r.S = s;
    if (a.chunks == 1) {
      a.stats[row] = r;
    } else {
      a.part[(size_t)row * a.chunks + ch] = r;
      __threadfence();
      s_last = atomicAdd(a.counters + row, 1) == a.chunks - 1;
    }
  }
  if (a.chunks == 1) return;
  __syncthreads();
  if (!s_last || tid != 0) return;
  __threadfence();
  RowStat acc = a.part[(size_t)row * a.chunks];
  float mm = acc.m;
  double S = acc.S;
  int ai = acc.amax;
  for (int k = 1; k < a.chunks; ++k) {
    const RowStat p = a.part[(size_t)row * a.chunks + k];
    if (greedy)
      am_combine(mm, ai, p.m, p.amax);
    else
      ms_combine(mm, S, p.m, p.S, T, unit_T);
  }
  RowStat out;
  out.m = mm;
  out.amax = ai;
  out.S = S;
  a.stats[row] = out;
  atomicExch(a.counters + row, 0);
}

// ---------------------------------------------------------------------------
struct WalkArgs {
  const int32_t* tokens;
  const float* draft;
  const float* logits;
  const int32_t* parents;
  const int32_t* kv_len;
  const float* uniforms;
  const RowStat* stats;
  int32_t* accept_len;
  int32_t* path;
  int32_t* acc_tokens;
  int32_t* bonus;
  int32_t* kv_src;
  float* out_final;
  float* out_ratio;
  int32_t* flags;
  int N, V;
  float T;
};

template <int BLOCK>
__device__ double block_sum_d(double v, double* red) {
  v = wave_sum(v);
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  double t = 0.0;
#pragma unroll
  for (int i = 0; i < BLOCK / 64; ++i) t += red[i];
  return t;
}

template <int BLOCK>
__device__ int block_min_i(int v, int* red) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v = min(v, __shfl_xor(v, off));
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  int t = INT_MAX;
#pragma unroll
  for (int i = 0; i < BLOCK / 64; ++i) t = min(t, red[i]);
  return t;
}

template <int BLOCK>
__device__ int block_max_i(int v, int* red) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v = max(v, __shfl_xor(v, off));
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  int t = INT_MIN;
#pragma unroll
  for (int i = 0; i < BLOCK / 64; ++i) t = max(t, red[i]);
  return t;
}

// Exclusive prefix over the workgroup (thread order), fp64.
template <int BLOCK>
__device__ double block_excl_scan_d(double v, double* red) {
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  double incl = v;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const double o = __shfl_up(incl, off);
    if (lane >= off) incl += o;
  }
  __syncthreads();
  if (lane == 63) red[wv] = incl;
  __syncthreads();
  double before = 0.0;
  for (int i = 0; i < wv; ++i) before += red[i];
  return before + incl - v;
}

// Element layout of a vocabulary row across the workgroup: group k, thread t
// owns elements (k * BLOCK + t) * 4 + e, e = 0..3.
template <int BLOCK, int NPT>
__global__ __launch_bounds__(BLOCK) void walk_kernel(WalkArgs a) {
  const int b = blockIdx.x;
  const int tid = threadIdx.x;
  const int N = a.N, V = a.V;
  const float T = a.T;
  const bool greedy = T == 0.f;
  const bool unit_T = T == 1.f;
  const bool vec = (V & 3) == 0;

  __shared__ int s_par[64], s_tok[64], s_am[64];
  __shared__ float s_m[64], s_lt[64], s_qt[64], s_u[64], s_ratio[64];
  __shared__ double s_S[64];
  __shared__ double red[BLOCK / 64];
  __shared__ int redi[BLOCK / 64];
  __shared__ double s_gsum[NPT];
  __shared__ float s_rt;
  __shared__ int s_path[64];

  const int L = a.kv_len[b];
  bool tok_bad = false;
  if (tid < N) {
    const size_t o = (size_t)b * N + tid;
    int par = a.parents[o];
    if (tid == 0 || par < 0 || par >= tid) par = tid == 0 ? -1 : 0;
    const int tk = a.tokens[o];
    s_par[tid] = par;
    s_tok[tid] = tk;
    s_u[tid] = a.uniforms[o];
    s_ratio[tid] = __int_as_float(0x7fc00000);  // NaN: untested
    const RowStat st = a.stats[o];
    s_m[tid] = st.m;
    s_S[tid] = st.S;
    s_am[tid] = st.amax;
    float lt = 0.f, qt = 0.f;
    if (tid > 0) {
      if (tk < 0 || tk >= V) {
        tok_bad = true;
      } else if (!greedy) {
        lt = a.logits[((size_t)b * N + par) * V + tk];
        qt = a.draft[o * V + tk];
      }
    }
    s_lt[tid] = lt;
    s_qt[tid] = qt;
  }
  if (__ballot(tok_bad) && (tid & 63) == 0 && a.flags) atomicOr(a.flags + b, EAGLE_FLAG_BAD_TOKEN);
  __syncthreads();

  float4 r[NPT];
  double Z = 0.0;
  bool have_r = false;

  auto load4 = [&](const float* rowp, int k) -> float4 {
    const int e0 = (k * BLOCK + tid) * 4;
    if (vec) {
      if (e0 < V) return *reinterpret_cast<const float4*>(rowp + e0);
      return make_float4(0.f, 0.f, 0.f, 0.f);
    }
    float4 o;
    o.x = e0 + 0 < V ? rowp[e0 + 0] : 0.f;
    o.y = e0 + 1 < V ? rowp[e0 + 1] : 0.f;
    o.z = e0 + 2 < V ? rowp[e0 + 2] : 0.f;
    o.w = e0 + 3 < V ? rowp[e0 + 3] : 0.f;
    return o;
  };
  auto valid = [&](int k, int e) { return (k * BLOCK + tid) * 4 + e < V; };

  // r <- exp((logits[node] - m) / T) (unnormalised p_node), Z <- its sum.
  auto materialize = [&](int node) {
    const float* rowp = a.logits + ((size_t)b * N + node) * V;
    const float m = s_m[node];
#pragma unroll
    for (int k = 0; k < NPT; ++k) {
      const float4 x = load4(rowp, k);
      r[k].x = valid(k, 0) ? scaled_exp(x.x, m, T, unit_T) : 0.f;
      r[k].y = valid(k, 1) ? scaled_exp(x.y, m, T, unit_T) : 0.f;
      r[k].z = valid(k, 2) ? scaled_exp(x.z, m, T, unit_T) : 0.f;
      r[k].w = valid(k, 3) ? scaled_exp(x.w, m, T, unit_T) : 0.f;
    }
    Z = s_S[node];
    have_r = true;
  };

  // r <- max(0, r/Z - q_c), Z <- sum; kept unchanged if the new mass is zero.
  auto residual = [&](int cnode) {
    const float* qrow = a.draft + ((size_t)b * N + cnode) * V;
    const float zf = (float)Z;
    float4 rn[NPT];
    double part = 0.0;
#pragma unroll
    for (int k = 0; k < NPT; ++k) {
      const float4 q = load4(qrow, k);
      rn[k].x = fmaxf(0.f, r[k].x / zf - q.x);
      rn[k].y = fmaxf(0.f, r[k].y / zf - q.y);
      rn[k].z = fmaxf(0.f, r[k].z / zf - q.z);
      rn[k].w = fmaxf(0.f, r[k].w / zf - q.w);
      part += (double)rn[k].x + (double)rn[k].y + ((double)rn[k].z + (double)rn[k].w);
    }
    const double Zn = block_sum_d<BLOCK>(part, red);
    if (Zn > 0.0) {
#pragma unroll
      for (int k = 0; k < NPT; ++k) r[k] = rn[k];
      Z = Zn;
    }
  };

  // r[t] broadcast through LDS.
  auto fetch_r = [&](int t) -> float {
    __syncthreads();
    const int quad = t >> 2, e = t & 3;
    const int k = quad / BLOCK, owner = quad - k * BLOCK;
    if (owner == tid) {
#pragma unroll
      for (int kk = 0; kk < NPT; ++kk)
        if (kk == k) s_rt = e == 0 ? r[kk].x : e == 1 ? r[kk].y : e == 2 ? r[kk].z : r[kk].w;
    }
    __syncthreads();
    return s_rt;
  };

  int cur = 0;
  int m_acc = 0;
  if (tid == 0) s_path[0] = 0;
  for (;;) {
    int accepted = -1;
    for (int cnode = cur + 1; cnode < N; ++cnode) {
      if (s_par[cnode] != cur) continue;
      const int tk = s_tok[cnode];
      const bool tok_ok = tk >= 0 && tk < V;
      double ratio;
      if (greedy) {
        ratio = (tok_ok && tk == s_am[cur]) ? 1.0 : 0.0;
      } else {
        double rt;
        if (!tok_ok) {
          rt = 0.0;
        } else if (!have_r) {
          rt = (double)scaled_exp(s_lt[cnode], s_m[cur], T, unit_T) / s_S[cur];
        } else {
          rt = (double)fetch_r(tk) / Z;
        }
        const double qt = s_qt[cnode];
        ratio = qt > 0.0 ? rt / qt : (rt > 0.0 ? (double)INFINITY : 0.0);
      }
      if (tid == 0) s_ratio[cnode] = (float)ratio;
      const bool ok = greedy ? ratio == 1.0 : (double)s_u[cnode] < ratio;
      if (ok) {
        accepted = cnode;
        break;
      }
      if (!greedy) {
        if (!have_r) materialize(cur);
        residual(cnode);
      }
    }
    if (accepted < 0) break;
    ++m_acc;
    if (tid == 0) s_path[m_acc] = accepted;
    cur = accepted;
    have_r = false;
  }

  // ---- final token -------------------------------------------------------------
  int bonus;
  if (greedy) {
    bonus = s_am[cur];
    if (a.out_final) {
      float* fo = a.out_final + (size_t)b * V;
      for (int v = tid; v < V; v += BLOCK) fo[v] = v == bonus ? 1.f : 0.f;
    }
  } else {
    if (!have_r) materialize(cur);
    double gs[NPT];
#pragma unroll
    for (int k = 0; k < NPT; ++k)
      gs[k] = (double)r[k].x + (double)r[k].y + ((double)r[k].z + (double)r[k].w);
    // group totals in fixed order
#pragma unroll
    for (int k = 0; k < NPT; ++k) {
      const double t = block_sum_d<BLOCK>(gs[k], red);
      if (tid == 0) s_gsum[k] = t;
    }
    __syncthreads();
    double ztot = 0.0;
#pragma unroll
    for (int k = 0; k < NPT; ++k) ztot += s_gsum[k];
    const double thr = (double)s_u[0] * ztot;
    double run = 0.0;
    int kstar = -1;
#pragma unroll
    for (int k = 0; k < NPT; ++k) {
      if (kstar < 0 && run + s_gsum[k] > thr) kstar = k;
      if (kstar < 0) run += s_gsum[k];
    }
    int cand = INT_MAX;
    if (kstar >= 0) {
      float4 rv = make_float4(0.f, 0.f, 0.f, 0.f);
      double tsum = 0.0;
#pragma unroll
      for (int k = 0; k < NPT; ++k)
        if (k == kstar) {
          rv = r[k];
          tsum = gs[k];
        }
      (void)tsum;
      const double before = run + block_excl_scan_d<BLOCK>(
                                      (double)rv.x + (double)rv.y + ((double)rv.z + (double)rv.w), red);
      const int base = (kstar * BLOCK + tid) * 4;
      double f = before;
      const float ev[4] = {rv.x, rv.y, rv.z, rv.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        f += (double)ev[e];
        if (cand == INT_MAX && f > thr && base + e < V) cand = base + e;
      }
    }
    int pick = block_min_i<BLOCK>(cand, redi);
    if (pick == INT_MAX) {  // rounding left no crossing: last id with mass
      int last = -1;
#pragma unroll
      for (int k = 0; k < NPT; ++k) {
        const int base = (k * BLOCK + tid) * 4;
        if (r[k].x > 0.f && base + 0 < V) last = max(last, base + 0);
        if (r[k].y > 0.f && base + 1 < V) last = max(last, base + 1);
        if (r[k].z > 0.f && base + 2 < V) last = max(last, base + 2);
        if (r[k].w > 0.f && base + 3 < V) last = max(last, base + 3);
      }
      pick = block_max_i<BLOCK>(last, redi);
      if (pick < 0) pick = 0;
    }
    bonus = pick;
    if (a.out_final) {
      float* fo = a.out_final + (size_t)b * V;
      const float zf = (float)Z;
#pragma unroll
      for (int k = 0; k < NPT; ++k) {
        const int base = (k * BLOCK + tid) * 4;
        if (base + 0 < V) fo[base + 0] = r[k].x / zf;
        if (base + 1 < V) fo[base + 1] = r[k].y / zf;
        if (base + 2 < V) fo[base + 2] = r[k].z / zf;
        if (base + 3 < V) fo[base + 3] = r[k].w / zf;
      }
    }
  }

  __syncthreads();
  if (tid < N) {
    const size_t o = (size_t)b * N + tid;
    const bool on = tid <= m_acc;
    const int node = on ? s_path[tid] : -1;
    a.path[o] = node;
    a.kv_src[o] = on ? L + node : -1;
    a.acc_tokens[o] = tid < m_acc ? s_tok[s_path[tid + 1]] : -1;
    if (a.out_ratio) a.out_ratio[o] = s_ratio[tid];
  }
  if (tid == 0) {
    a.accept_len[b] = m_acc;
    a.bonus[b] = bonus;
  }
}

// Normalised target rows for parity checks: p = exp((x - m)/T) / S, or one-hot.
__global__ __launch_bounds__(256) void probs_kernel(const float* __restrict__ logits,
                                                    const RowStat* __restrict__ stats, int V,
                                                    int chunks, float T, float* __restrict__ out) {
  const int row = blockIdx.x / chunks;
  const int ch = blockIdx.x - row * chunks;
  const int v0 = (int)((long long)ch * V / chunks), v1 = (int)((long long)(ch + 1) * V / chunks);
  const RowStat st = stats[row];
  const float* x = logits + (size_t)row * V;
  float* o = out + (size_t)row * V;
  const bool unit_T = T == 1.f;
  for (int v = v0 + threadIdx.x; v < v1; v += 256) {
    if (T == 0.f)
      o[v] = v == st.amax ? 1.f : 0.f;
    else
      o[v] = (float)((double)scaled_exp(x[v], st.m, T, unit_T) / st.S);
  }
}

// ---------------------------------------------------------------------------
VerifyPlan plan_verify(int B, int N, int V) {
  VerifyPlan p{};
  p.V = V;
  const int rows = B * N;
  int chunks = (2 * kNumCUs + rows - 1) / rows;
  const int max_chunks = (V + 1023) / 1024;
  if (chunks > max_chunks) chunks = max_chunks;
  if (chunks < 1) chunks = 1;
  const char* e = getenv("EAGLE_VOCAB_CHUNKS");
  if (e && *e) chunks = atoi(e) < 1 ? 1 : atoi(e);
  p.chunks = chunks;
  p.walk_threads = V > 4096 ? 1024 : 256;
  p.ws_stats = (size_t)rows * sizeof(RowStat);
  p.ws_partials = chunks > 1 ? (size_t)rows * chunks * sizeof(RowStat) : 0;
  p.ws_counters = chunks > 1 ? (size_t)rows * 4 : 0;
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
                         int32_t* flags, hipStream_t s) {
  uint8_t* w = static_cast<uint8_t*>(ws);
  int32_t* counters = reinterpret_cast<int32_t*>(w);
  RowStat* stats = reinterpret_cast<RowStat*>(w + align256(plan.ws_counters));
  RowStat* part = reinterpret_cast<RowStat*>(w + align256(plan.ws_counters) + align256(plan.ws_stats));
  const int rows = B * N;

  StatsArgs sa{};
  sa.logits = logits;
  sa.stats = stats;
  sa.part = part;
  sa.counters = counters;
  sa.flags = flags;
  sa.rows = rows;
  sa.N = N;
  sa.V = plan.V;
  sa.chunks = plan.chunks;
  sa.T = T;
  vocab_stats_kernel<<<rows * plan.chunks, 256, 0, s>>>(sa);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;

  if (out_probs) {
    const int pchunks = (plan.V + 4095) / 4096;
    probs_kernel<<<rows * pchunks, 256, 0, s>>>(logits, stats, plan.V, pchunks, T, out_probs);
    err = hipGetLastError();
    if (err != hipSuccess) return err;
  }

  WalkArgs wa{};
  wa.tokens = tokens;
  wa.draft = draft;
  wa.logits = logits;
  wa.parents = parents;
  wa.kv_len = kv_len;
  wa.uniforms = uniforms;
  wa.stats = stats;
  wa.accept_len = accept_len;
  wa.path = path;
  wa.acc_tokens = acc_tokens;
  wa.bonus = bonus;
  wa.kv_src = kv_src;
  wa.out_final = out_final;
  wa.out_ratio = out_ratio;
  wa.flags = flags;
  wa.N = N;
  wa.V = plan.V;
  wa.T = T;
  if (plan.walk_threads == 1024)
    walk_kernel<1024, 8><<<B, 1024, 0, s>>>(wa);
  else
    walk_kernel<256, 4><<<B, 256, 0, s>>>(wa);
  return hipGetLastError();
}

}  // namespace eagle
