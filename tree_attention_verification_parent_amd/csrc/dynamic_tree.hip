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
// All three steps are top-k selections over (value, id) pairs, done as k
// rounds of a workgroup maximum over 64-bit keys that order by value, then
// by lower id: every thread keeps the largest of its keys below the last one
// taken, and only the thread whose key was taken looks again.
#include "common.h"
#include "launch.h"

namespace eagle {

constexpr int kTreeBlock = 1024;

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

// Workgroup maximum; `red` holds two sets of per-wave slots used in turn, so
// one barrier per call suffices.
__device__ __forceinline__ unsigned long long block_max_key(unsigned long long x,
                                                            unsigned long long* red, int turn) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    const unsigned long long y = __shfl_xor(x, o);
    x = y > x ? y : x;
  }
  constexpr int NW = kTreeBlock / 64;
  unsigned long long* slot = red + (turn & 1) * NW;
  if ((threadIdx.x & 63) == 0) slot[threadIdx.x >> 6] = x;
  __syncthreads();
  unsigned long long m = slot[0];
#pragma unroll
  for (int i = 1; i < NW; ++i) m = slot[i] > m ? slot[i] : m;
  return m;
}

// The k largest keys of the workgroup, largest first: emit(j, key) on every
// thread for j = 0.. until k keys or no key is left.
template <int EPT, typename Emit>
__device__ __forceinline__ void block_topk(const unsigned long long (&key)[EPT], int k,
                                           unsigned long long* red, Emit&& emit) {
  unsigned long long m = 0;
#pragma unroll
  for (int e = 0; e < EPT; ++e) m = key[e] > m ? key[e] : m;
  for (int j = 0; j < k; ++j) {
    const unsigned long long best = block_max_key(m, red, j);
    if (best == 0) break;  // uniform: fewer than k keys
    emit(j, best);
    if (m == best) {  // keys are distinct: only this thread held it
      m = 0;
#pragma unroll
      for (int e = 0; e < EPT; ++e)
        if (key[e] < best && key[e] > m) m = key[e];
    }
  }
}

// Expansion: one workgroup per (sequence, row); the row's V <= 32768
// probabilities in registers (32 per thread).
__global__ __launch_bounds__(kTreeBlock) void eagle2_expand_kernel(
    const float* __restrict__ q, int R, int V, int k, const int32_t* __restrict__ parent_node,
    const float* __restrict__ parent_value, int32_t* __restrict__ cpar,
    int32_t* __restrict__ ctok, float* __restrict__ cval, int T, int base) {
  constexpr int EPT = 32768 / kTreeBlock;
  __shared__ unsigned long long red[2 * kTreeBlock / 64];
  const int row = blockIdx.x;
  const int b = row / R, r = row - b * R;
  const float* qr = q + (size_t)row * V;
  unsigned long long key[EPT];
#pragma unroll
  for (int e = 0; e < EPT; ++e) {
    const int t = e * kTreeBlock + threadIdx.x;
    key[e] = t < V ? vkey(qr[t], t) : 0ull;
  }
  const float pv = parent_value[row];
  const int pn = parent_node[row];
  block_topk<EPT>(key, k, red, [&](int j, unsigned long long best) {
    if (threadIdx.x == 0) {
      const size_t c = (size_t)b * T + base + r * k + j;
      cpar[c] = pn;
      ctok[c] = key_id(best);
      cval[c] = pv * key_value(best);
    }
  });
}

// Selection: one workgroup per sequence over ids [first, first + M), M <= 2048.
__global__ __launch_bounds__(kTreeBlock) void eagle2_select_kernel(
    const float* __restrict__ cval, int T, int first, int M, int k, int32_t* __restrict__ out_node,
    float* __restrict__ out_value) {
  __shared__ unsigned long long red[2 * kTreeBlock / 64];
  const int b = blockIdx.x;
  unsigned long long key[2];
#pragma unroll
  for (int e = 0; e < 2; ++e) {
    const int i = e * kTreeBlock + threadIdx.x;
    key[e] = i < M ? vkey(cval[(size_t)b * T + first + i], first + i) : 0ull;
  }
  block_topk<2>(key, k, red, [&](int j, unsigned long long best) {
    if (threadIdx.x == 0) {
      out_node[(size_t)b * k + j] = key_id(best);
      out_value[(size_t)b * k + j] = key_value(best);
    }
  });
}

// Rerank: the root and the N - 1 most valuable of ids [1, T_used), renumbered
// in creation order by one wave (lane = new id).
__global__ __launch_bounds__(kTreeBlock) void eagle2_rerank_kernel(
    const int32_t* __restrict__ cpar, const int32_t* __restrict__ ctok,
    const float* __restrict__ cval, int T, int T_used, int N, int32_t* __restrict__ parents,
    int32_t* __restrict__ tokens, int32_t* __restrict__ kept_node, int32_t* __restrict__ flags) {
  __shared__ unsigned long long red[2 * kTreeBlock / 64];
  __shared__ int sel[64];
  __shared__ int order[64];
  const int b = blockIdx.x;
  const size_t cb = (size_t)b * T;
  const int M = T_used - 1;
  unsigned long long key[2];
#pragma unroll
  for (int e = 0; e < 2; ++e) {
    const int i = e * kTreeBlock + threadIdx.x;
    key[e] = i < M ? vkey(cval[cb + 1 + i], 1 + i) : 0ull;
  }
  if (threadIdx.x < 64) sel[threadIdx.x] = 0;  // the root, and padding if fewer nodes
  __syncthreads();
  block_topk<2>(key, N - 1, red, [&](int j, unsigned long long best) {
    if (threadIdx.x == 0) sel[1 + j] = key_id(best);
  });
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
  eagle2_expand_kernel<<<dim3((unsigned)(B * R)), kTreeBlock, 0, s>>>(
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
