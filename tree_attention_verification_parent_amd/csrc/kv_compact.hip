// KV compaction: move the accepted path's keys/values to the front of the
// tree segment of the cache, recording the accepted tokens for the next round
// (EAGLE, paperlayer.ai summary, §3 EAGLE: accepted tokens are recorded).
//
// Slot L+j takes slot L+path[j], j = 0..m.  Because path[j] >= j a source slot
// can be another pair's destination (path = [0, 2, 3]: slot L+2 is read for
// j = 1 and written for j = 2), so a workgroup reads every row it moves into
// registers, synchronises, and only then writes.  One workgroup per (b, KV
// head) owns all rows of that head, so workgroups never overlap.
#include <algorithm>

#include "common.h"
#include "launch.h"

namespace eagle {

template <int D>
__global__ __launch_bounds__(256) void kv_compact_kernel(uint16_t* __restrict__ k,
                                                         uint16_t* __restrict__ v,
                                                         const int32_t* __restrict__ kv_len,
                                                         const int32_t* __restrict__ kv_src,
                                                         const int32_t* __restrict__ accept_len,
                                                         int N, int Hkv, int Lmax,
                                                         int32_t* __restrict__ new_len,
                                                         int32_t* __restrict__ flags) {
  constexpr int CPR = D / 8;                  // 16-byte chunks per row
  constexpr int MAX_ITEMS = 64 * CPR * 2 / 256;  // K and V rows of a full path
  __shared__ int s_src[64];
  __shared__ int s_ok;
  const int b = blockIdx.x / Hkv;
  const int h = blockIdx.x - b * Hkv;
  const int tid = threadIdx.x;
  const int L = kv_len[b];
  const int m = accept_len[b];
  if (tid < 64) s_src[tid] = tid < N ? kv_src[(size_t)b * N + tid] : -1;
  __syncthreads();
  if (tid == 0) {
    bool ok = L >= 0 && L <= Lmax - N && m >= 0 && m < N;
    int prev = -1;
    for (int j = 0; ok && j <= m; ++j) {
      const int sj = s_src[j];
      ok = sj >= L + j && sj < Lmax && sj > prev;
      prev = sj;
    }
    s_ok = ok;
    if (h == 0) {
      new_len[b] = ok ? L + m + 1 : L;
      if (!ok && flags) atomicOr(flags + b, EAGLE_FLAG_BAD_KV_LEN);
    }
  }
  __syncthreads();
  if (!s_ok) return;

  // rows already in place (source slot L + j, e.g. the root, and every node
  // of a chain-shaped path) are neither read nor written; if none moves the
  // workgroup is done
  int first_move = m + 1;
  for (int j = m; j >= 0; --j)
    if (s_src[j] != L + j) first_move = j;
  if (first_move > m) return;
  const size_t head = ((size_t)b * Hkv + h) * (size_t)Lmax * D;
  const int items = (m + 1) * CPR * 2;
  u32x4 buf[MAX_ITEMS];
#pragma unroll
  for (int n = 0; n < MAX_ITEMS; ++n) {
    const int it = tid + n * 256;
    if (it < items) {
      const int which = it / ((m + 1) * CPR);   // 0: K, 1: V
      const int rem = it - which * (m + 1) * CPR;
      const int j = rem / CPR, ch = rem - j * CPR;
      const uint16_t* base = which ? v : k;
      if (s_src[j] != L + j)
        buf[n] = *reinterpret_cast<const u32x4*>(base + head + (size_t)s_src[j] * D + ch * 8);
    }
  }
  __syncthreads();
#pragma unroll
  for (int n = 0; n < MAX_ITEMS; ++n) {
    const int it = tid + n * 256;
    if (it < items) {
      const int which = it / ((m + 1) * CPR);
      const int rem = it - which * (m + 1) * CPR;
      const int j = rem / CPR, ch = rem - j * CPR;
      if (s_src[j] == L + j) continue;  // already in place
      uint16_t* base = which ? v : k;
      *reinterpret_cast<u32x4*>(base + head + (size_t)(L + j) * D + ch * 8) = buf[n];
    }
  }
}

hipError_t launch_kv_compact(uint16_t* k, uint16_t* v, const int32_t* kv_len,
                             const int32_t* kv_src, const int32_t* accept_len, int B, int N,
                             int Hkv, int d, int Lmax, int32_t* new_len, int32_t* flags,
                             hipStream_t s) {
  const dim3 grid((unsigned)(B * Hkv));
  if (d == 64)
    kv_compact_kernel<64><<<grid, 256, 0, s>>>(k, v, kv_len, kv_src, accept_len, N, Hkv, Lmax,
                                               new_len, flags);
  else
    kv_compact_kernel<128><<<grid, 256, 0, s>>>(k, v, kv_len, kv_src, accept_len, N, Hkv, Lmax,
                                                new_len, flags);
  return hipGetLastError();
}

// Feature gather: out[b, j] = features[b, path[b, j]] for j = 0..m, the rows
// copied as 16-byte columns.  Out of place, so rows can be copied in any
// order.  A sequence's rows are spread over `nb` workgroups (ids b * nb ..),
// each thread taking (row, column) items strided over them, so that loads
// and stores run along a row.  Every workgroup of a sequence checks the path
// the same way; the first one flags a bad path.
__global__ __launch_bounds__(256) void feature_gather_kernel(const u32x4* __restrict__ feat,
                                                             const int32_t* __restrict__ path,
                                                             const int32_t* __restrict__ accept_len,
                                                             int N, int cols, int nb,
                                                             u32x4* __restrict__ out,
                                                             int32_t* __restrict__ flags) {
  __shared__ int s_src[64];
  __shared__ int s_ok;
  const int b = blockIdx.x / nb;
  const int part = blockIdx.x - b * nb;
  const int tid = threadIdx.x;
  const int m = accept_len[b];
  if (tid < 64) s_src[tid] = tid < N ? path[(size_t)b * N + tid] : -1;
  __syncthreads();
  if (tid == 0) {
    bool ok = m >= 0 && m < N && s_src[0] == 0;
    for (int j = 1; ok && j <= m; ++j) ok = s_src[j] > s_src[j - 1] && s_src[j] < N;
    s_ok = ok;
    if (!ok && part == 0 && flags) atomicOr(flags + b, EAGLE_FLAG_BAD_PATH);
  }
  __syncthreads();
  if (!s_ok) return;
  const int total = (m + 1) * cols;
  const size_t base = (size_t)b * N * cols;
  for (int it = part * 256 + tid; it < total; it += nb * 256) {
    const int j = it / cols;
    const int col = it - j * cols;
    out[base + (size_t)j * cols + col] = feat[base + (size_t)s_src[j] * cols + col];
  }
}

hipError_t launch_feature_gather(const void* features, const int32_t* path,
                                 const int32_t* accept_len, int B, int N, int64_t row_bytes,
                                 void* out, int32_t* flags, hipStream_t s) {
  const int cols = (int)(row_bytes / 16);
  // enough workgroups per sequence for a full path, at most 64
  const long long items = (long long)N * cols;
  const int nb = (int)std::min<long long>(64, (items + 255) / 256);
  feature_gather_kernel<<<dim3((unsigned)(B * nb)), 256, 0, s>>>(
      static_cast<const u32x4*>(features), path, accept_len, N, cols, nb,
      static_cast<u32x4*>(out), flags);
  return hipGetLastError();
}

}  // namespace eagle
