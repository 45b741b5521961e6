// EAGLE-2 dynamic draft tree on the GPU.
//
// EAGLE-2 grows the draft tree from the draft model's confidences (EAGLE-2
// overview blog, §1 and §4 EAGLE vs EAGLE-2): a node's value is the product
// of the draft probabilities along its path; each layer expands the k most
// valuable nodes of the layer before into their k most probable next tokens,
// and a final rerank keeps the most valuable nodes as the tree to verify.
// Nodes are numbered in creation order (root 0; an expansion's children
// follow their parent rows in order, each row's by decreasing probability);
// ties go to the lower token id (expansion) or node id (selection, rerank).
//
// All three steps are top-k selections over (value, id) pairs, compared as
// 64-bit keys that order by value, then by lower id.  Over a vocabulary row
// (expansion) the keys at or above a threshold (the k-th largest of the
// waves' maxima) are ranked among themselves; where that does not apply,
// every wave finds its own k largest keys in k rounds of a wave maximum (no
// barrier: every lane keeps the largest of its keys below the last one
// taken, and only the lane whose key was taken looks again), and the row's
// k largest are the keys of rank below k among the waves' k each.  Over at most 2048 created
// nodes (selection, rerank) each key's rank is counted against all the keys
// in LDS, and the keys of rank below k are the selection.
#include "common.h"
#include "launch.h"

namespace eagle {

constexpr int kTreeBlock = 1024;   // selection and rerank
// expansion: 16 waves of 32 keys per thread; against 8 waves of 64 the k
// rounds of each wave overlap four to a SIMD and a winner's rescan covers
// half the keys (the 12-launch build at the Mixtral shape: 125 -> 109 us)
constexpr int kExpandBlock = 1024;

// Larger value first, then lower id (ids below 2^31); key 0 is below every
// real key and marks "none".
__device__ __forceinline__ unsigned long long vkey(float v, int id) {
  const uint32_t bits = __float_as_uint(v);
  const uint32_t ord = (bits & 0x80000000u) ? ~bits : (bits | 0x80000000u);
  return ((unsigned long long)ord << 32) | (uint32_t)(0x7fffffff - id);
}
__device__ __forceinline__ float key_value(unsigned long long key) {
  const uint32_t ord = (uint32_t)(key >> 32);
  return __uint_as_float((ord & 0x80000000u) ? (ord & 0x7fffffffu) : ~ord);
}
__device__ __forceinline__ int key_id(unsigned long long key) {
  return 0x7fffffff - (int)(uint32_t)key;
}

// One DPP step of a 64-bit maximum (both halves moved by the same lane
// permutation, compared as one key).
template <int CTRL>
__device__ __forceinline__ unsigned long long dpp_max_u64(unsigned long long x) {
  const uint32_t hi = (uint32_t)dpp_i<CTRL>((int)(uint32_t)(x >> 32));
  const uint32_t lo = (uint32_t)dpp_i<CTRL>((int)(uint32_t)x);
  const unsigned long long y = ((unsigned long long)hi << 32) | lo;
  return y > x ? y : x;
}
__device__ __forceinline__ unsigned long long lane_u64(unsigned long long x, int l) {
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(x >> 32), l);
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)x, l);
  return ((unsigned long long)hi << 32) | lo;
}

// Wave maximum: DPP row steps, then the four rows' lanes.
__device__ __forceinline__ unsigned long long wave_max_key(unsigned long long x) {
  x = dpp_max_u64<kDppXor1>(x);
  x = dpp_max_u64<kDppXor2>(x);
  x = dpp_max_u64<kDppHalfMirror>(x);
  x = dpp_max_u64<kDppMirror>(x);
  const unsigned long long a = lane_u64(x, 0), b = lane_u64(x, 16);
  const unsigned long long c = lane_u64(x, 32), d = lane_u64(x, 48);
  const unsigned long long ab = a > b ? a : b, cd = c > d ? c : d;
  return ab > cd ? ab : cd;
}

// Wave maximum of 32-bit values (the same row steps).
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t x) {
  x = max(x, (uint32_t)dpp_i<kDppXor1>((int)x));
  x = max(x, (uint32_t)dpp_i<kDppXor2>((int)x));
  x = max(x, (uint32_t)dpp_i<kDppHalfMirror>((int)x));
  x = max(x, (uint32_t)dpp_i<kDppMirror>((int)x));
  const uint32_t a = (uint32_t)__builtin_amdgcn_readlane((int)x, 0);
  const uint32_t b = (uint32_t)__builtin_amdgcn_readlane((int)x, 16);
  const uint32_t c = (uint32_t)__builtin_amdgcn_readlane((int)x, 32);
  const uint32_t d = (uint32_t)__builtin_amdgcn_readlane((int)x, 48);
  return max(max(a, b), max(c, d));
}

// Largest key of the wave: the maximum of the value halves (nonzero for
// every real key), then, if one lane holds that value, its key; only a tie
// between lanes needs the 64-bit maximum.
__device__ __forceinline__ unsigned long long wave_best_key(unsigned long long m) {
  const uint32_t hi = (uint32_t)(m >> 32);
  const uint32_t vmax = wave_max_u32(hi);
  if (vmax == 0u) return 0ull;  // uniform: no key left
  const unsigned long long lanes = __ballot(hi == vmax);
  if (__popcll(lanes) == 1) return lane_u64(m, __ffsll((long long)lanes) - 1);
  return wave_max_key(hi == vmax ? m : 0ull);
}

// The k largest keys of the workgroup (keys distinct, k <= 64): each wave
// writes its own k largest to cand[wave * k ..] (0 where it has fewer), in k
// rounds of a wave maximum; a lane offers its largest key not yet taken (m1)
// and keeps its second largest (m2) ready, so it rescans its keys only when
// it wins a third time or more.  After one barrier, emit(rank, key) runs on
// the thread holding each of the k largest of the waves' candidates, rank
// 0 the largest: the row's k largest are all among them.
template <int BLOCK, int EPT, typename KeyAt, typename Emit>
__device__ __forceinline__ void block_topk(KeyAt&& key_at, int k, unsigned long long* cand,  // 16-byte aligned
                                           Emit&& emit) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  unsigned long long m1 = 0, m2 = 0;
#pragma unroll
  for (int e = 0; e < EPT; ++e) {
    const unsigned long long x = key_at(e);
    if (x > m1) {
      m2 = m1;
      m1 = x;
    } else if (x > m2) {
      m2 = x;
    }
  }
  bool m2_ready = true;
  for (int j = 0; j < k; ++j) {
    const unsigned long long best = wave_best_key(m1);  // 0: the wave has no key left
    if (lane == 0) cand[wave * k + j] = best;
    // keys are distinct, so one lane at most holds best; the other lanes skip
    // the update with a wave-uniform branch (predicated, every lane paid for
    // the rescan)
    const bool won = best != 0ull && m1 == best;
    if (__ballot(won)) {
      if (won) {
        if (m2_ready) {
          m1 = m2;  // the largest below best
          m2_ready = false;
        } else {
          m1 = 0;
#pragma unroll
          for (int e = 0; e < EPT; ++e) {
            const unsigned long long x = key_at(e);
            if (x < best && x > m1) m1 = x;
          }
        }
      }
    }
  }
  barrier_lds();
  // nc is a multiple of 8: eight keys per step, their LDS reads issued together
  const int nc = (BLOCK / 64) * k;
  for (int t = threadIdx.x; t < nc; t += BLOCK) {
    const unsigned long long mine = cand[t];
    if (mine == 0ull) continue;
    int rank = 0;
    for (int i = 0; i < nc; i += 8) {
      const ulonglong2* c2 = reinterpret_cast<const ulonglong2*>(cand + i);
      const ulonglong2 a = c2[0], b = c2[1], c = c2[2], d = c2[3];
      rank += (a.x > mine) + (a.y > mine) + (b.x > mine) + (b.y > mine) + (c.x > mine) +
              (c.y > mine) + (d.x > mine) + (d.y > mine);
    }
    if (rank < k) emit(rank, mine);
  }
}

// The k largest keys of the workgroup through a threshold: every wave's
// largest value (ord_at gives the keys' value halves, 0 for no key), then
// tau, the k-th largest of those NW maxima (counted with multiplicity).  At
// least k keys have a value half >= tau (one per wave whose maximum is), so
// the k largest keys all do: only those survive, appended to cand, and each
// survivor's rank among them is its rank in the row.  With random or peaked
// rows a few dozen keys survive; when k > NW, when tau is 0 (fewer than k
// keys) or when more than the list holds survive (many equal values), the
// rounds of block_topk take over.  One wave maximum replaces k rounds of
// them (the 12-launch build at the Mixtral shape, graph-timed: 108 -> 76.5
// us).
template <int BLOCK, int EPT, typename OrdAt, typename KeyAt, typename Emit>
__device__ __forceinline__ void block_topk_filtered(OrdAt&& ord_at, KeyAt&& key_at, int k,
                                                    unsigned long long* cand, int cap,
                                                    uint32_t* wmax, int* nsurv, Emit&& emit) {
  constexpr int NW = BLOCK / 64;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  uint32_t vm = 0;
#pragma unroll
  for (int e = 0; e < EPT; ++e) vm = max(vm, ord_at(e));
  const uint32_t wv = wave_max_u32(vm);
  if (lane == 0) wmax[wave] = wv;
  if (threadIdx.x == 0) *nsurv = 0;
  barrier_lds();
  uint32_t tau = 0;
  if (k <= NW) {
    // lane i < NW: wave i's maximum is the k-th largest iff fewer than k
    // maxima exceed it and at least k reach it; every wave finds the same
    const uint32_t mine = lane < NW ? wmax[lane] : 0u;
    int gt = 0, ge = 0;
#pragma unroll
    for (int j = 0; j < NW; ++j) {
      const uint32_t w = wmax[j];
      gt += w > mine;
      ge += w >= mine;
    }
    const unsigned long long hit = __ballot(lane < NW && gt < k && k <= ge);
    if (hit) tau = (uint32_t)__builtin_amdgcn_readlane((int)mine, __ffsll((long long)hit) - 1);
  }
  if (tau != 0u) {  // uniform
#pragma unroll
    for (int e = 0; e < EPT; ++e)
      if (ord_at(e) >= tau) {
        const int pos = atomicAdd(nsurv, 1);
        if (pos < cap) cand[pos] = key_at(e);
      }
    barrier_lds();
    const int n = *nsurv;
    if (n <= cap) {  // uniform
      for (int t = threadIdx.x; t < n; t += BLOCK) {
        const unsigned long long mine = cand[t];
        int rank = 0;
        for (int i = 0; i < n; ++i) rank += cand[i] > mine;
        if (rank < k) emit(rank, mine);
      }
      return;
    }
    barrier_lds();  // every thread has read the count before the rounds rewrite cand
  }
  block_topk<BLOCK, EPT>(key_at, k, cand, emit);
}

// Expansion: one workgroup per (sequence, row); the row's V <= 32768
// probabilities in registers (32 per thread), their keys formed as needed.
__global__ __launch_bounds__(kExpandBlock) void eagle2_expand_kernel(
    const float* __restrict__ q, int R, int V, int k, const int32_t* __restrict__ parent_node,
    const float* __restrict__ parent_value, int32_t* __restrict__ cpar,
    int32_t* __restrict__ ctok, float* __restrict__ cval, int T, int base) {
  constexpr int EPT = 32768 / kExpandBlock;
  __shared__ __attribute__((aligned(16))) unsigned long long cand[(kExpandBlock / 64) * 64];
  __shared__ unsigned long long taken[64];
  __shared__ uint32_t wmax[kExpandBlock / 64];
  __shared__ int nsurv;
  const int row = blockIdx.x;
  const int b = row / R, r = row - b * R;
  const float* qr = q + (size_t)row * V;
  // 16-byte buffer loads, every one in flight before any is used (ids past
  // V read 0 and get no key); thread t holds ids 4 (f * BLOCK + t) + c
  const __amdgpu_buffer_rsrc_t rs = buffer_rsrc(qr, (size_t)V * 4);
  f32x4 x4[EPT / 4];
#pragma unroll
  for (int f = 0; f < EPT / 4; ++f)
    x4[f] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                          rs, (f * kExpandBlock + (int)threadIdx.x) * 16, 0, 0));
  // the keys' value halves (0: no key), the id half formed when a key is needed
  uint32_t ord[EPT];
#pragma unroll
  for (int f = 0; f < EPT / 4; ++f)
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const int t = 4 * (f * kExpandBlock + (int)threadIdx.x) + c;
      ord[4 * f + c] = t < V ? (uint32_t)(vkey(x4[f][c], t) >> 32) : 0u;
    }
  auto ord_at = [&](int e) { return ord[e]; };
  auto key_at = [&](int e) -> unsigned long long {
    const int t = 4 * ((e >> 2) * kExpandBlock + (int)threadIdx.x) + (e & 3);
    return t < V ? ((unsigned long long)ord[e] << 32) | (uint32_t)(0x7fffffff - t) : 0ull;
  };
  const float pv = parent_value[row];
  const int pn = parent_node[row];
  block_topk_filtered<kExpandBlock, EPT>(
      ord_at, key_at, k, cand, (kExpandBlock / 64) * 64, wmax, &nsurv,
      [&](int rank, unsigned long long key) { taken[rank] = key; });
  barrier_lds();
  // the children, written once all are known (k <= 64)
  if (threadIdx.x < k) {
    const unsigned long long best = taken[threadIdx.x];
    const size_t c = (size_t)b * T + base + r * k + threadIdx.x;
    cpar[c] = pn;
    ctok[c] = key_id(best);
    cval[c] = pv * key_value(best);
  }
}

// The keys of ids [first, first + M) (M <= 2048) of one sequence's values
// into LDS, then emit(rank, key) for every key of rank below k (its rank =
// the number of larger keys; keys are distinct).
template <typename Emit>
__device__ __forceinline__ void rank_select(const float* vals, int first, int M, int k,
                                            unsigned long long* skey, Emit&& emit) {
  for (int i = threadIdx.x; i < M; i += kTreeBlock) skey[i] = vkey(vals[first + i], first + i);
  __syncthreads();
  for (int i = threadIdx.x; i < M; i += kTreeBlock) {
    const unsigned long long mine = skey[i];
    int rank = 0;
    for (int j = 0; j < M; ++j) rank += skey[j] > mine;
    if (rank < k) emit(rank, mine);
  }
}

// Selection: one workgroup per sequence over ids [first, first + M), M <= 2048.
__global__ __launch_bounds__(kTreeBlock) void eagle2_select_kernel(
    const float* __restrict__ cval, int T, int first, int M, int k, int32_t* __restrict__ out_node,
    float* __restrict__ out_value) {
  __shared__ unsigned long long skey[2048];
  const int b = blockIdx.x;
  rank_select(cval + (size_t)b * T, first, M, k, skey, [&](int rank, unsigned long long key) {
    out_node[(size_t)b * k + rank] = key_id(key);
    out_value[(size_t)b * k + rank] = key_value(key);
  });
}

// Rerank: the root and the N - 1 most valuable of ids [1, T_used), renumbered
// in creation order by one wave (lane = new id).
__global__ __launch_bounds__(kTreeBlock) void eagle2_rerank_kernel(
    const int32_t* __restrict__ cpar, const int32_t* __restrict__ ctok,
    const float* __restrict__ cval, int T, int T_used, int N, int32_t* __restrict__ parents,
    int32_t* __restrict__ tokens, int32_t* __restrict__ kept_node, int32_t* __restrict__ flags) {
  __shared__ unsigned long long skey[2048];
  __shared__ int sel[64];
  __shared__ int order[64];
  const int b = blockIdx.x;
  const size_t cb = (size_t)b * T;
  if (threadIdx.x == 0) sel[0] = 0;  // the root
  rank_select(cval + cb, 1, T_used - 1, N - 1, skey,
              [&](int rank, unsigned long long key) { sel[1 + rank] = key_id(key); });
  __syncthreads();
  const int lane = threadIdx.x;
  // new id = number of kept ids below this one (kept ids are distinct)
  if (lane < N) {
    const int mine = sel[lane];
    int rank = 0;
    for (int i = 0; i < N; ++i) rank += sel[i] < mine;
    order[rank] = mine;
  }
  __syncthreads();
  if (lane >= N) return;
  const int id = order[lane];
  int par = -1;
  bool bad = false;
  if (lane > 0) {
    const int p = cpar[cb + id];
    par = 0;
    bad = true;
    for (int i = 0; i < N; ++i)
      if (order[i] == p) {
        par = i;
        bad = false;
      }
  }
  parents[(size_t)b * N + lane] = par;
  tokens[(size_t)b * N + lane] = ctok[cb + id];
  kept_node[(size_t)b * N + lane] = id;
  if (bad && flags) atomicOr(flags + b, EAGLE_FLAG_BAD_PARENT);
}

hipError_t launch_eagle2_expand(const float* q, int B, int R, int V, int k,
                                const int32_t* parent_node, const float* parent_value,
                                int32_t* cpar, int32_t* ctok, float* cval, int T, int base,
                                hipStream_t s) {
  eagle2_expand_kernel<<<dim3((unsigned)(B * R)), kExpandBlock, 0, s>>>(
      q, R, V, k, parent_node, parent_value, cpar, ctok, cval, T, base);
  return hipGetLastError();
}

hipError_t launch_eagle2_select(const float* cval, int B, int T, int first, int M, int k,
                                int32_t* out_node, float* out_value, hipStream_t s) {
  eagle2_select_kernel<<<dim3((unsigned)B), kTreeBlock, 0, s>>>(cval, T, first, M, k, out_node,
                                                                  out_value);
  return hipGetLastError();
}

hipError_t launch_eagle2_rerank(const int32_t* cpar, const int32_t* ctok, const float* cval,
                                int B, int T, int T_used, int N, int32_t* parents,
                                int32_t* tokens, int32_t* kept_node, int32_t* flags,
                                hipStream_t s) {
  eagle2_rerank_kernel<<<dim3((unsigned)B), kTreeBlock, 0, s>>>(cpar, ctok, cval, T, T_used, N,
                                                                  parents, tokens, kept_node,
                                                                  flags);
  return hipGetLastError();
}

}  // namespace eagle
