// Tree-mask builder: parent array -> ancestor bitmask, depth, position id.
//
// Each drafted node attends to its own ancestors (EAGLE, paperlayer.ai
// summary, §3 EAGLE: tree attention; A.1 Tree Structure).  One wavefront per
// sequence, lane i owning node i (N <= 64); the ancestor sets come from
// pointer jumping over the parent links (tree_links_wave).
#include "common.h"
#include "launch.h"

namespace eagle {

__global__ __launch_bounds__(256) void tree_build_kernel(
    const int32_t* __restrict__ parents, const int32_t* __restrict__ kv_len, int B, int N,
    uint64_t* __restrict__ anc, int32_t* __restrict__ depth, int32_t* __restrict__ pos,
    int32_t* __restrict__ flags) {
  const int lane = threadIdx.x & (kWave - 1);
  const int b = blockIdx.x * (blockDim.x / kWave) + threadIdx.x / kWave;
  if (b >= B) return;  // uniform per wavefront
  const bool live = lane < N;
  // issued before the parent links: the position ids need the committed length
  const int L = pos && live ? kv_len[b] : 0;
  const TreeLinks t = tree_links_wave(parents + (size_t)b * N, N);
  if (live) {
    const size_t o = (size_t)b * N + lane;
    anc[o] = t.anc;
    if (depth) depth[o] = t.depth;
    if (pos) pos[o] = L + t.depth;
  }
  const uint64_t any_bad = __ballot(t.bad);
  if (flags && any_bad && lane == 0) atomicOr(flags + b, EAGLE_FLAG_BAD_PARENT);
}

__global__ __launch_bounds__(256) void fill_zero_kernel(uint8_t* __restrict__ p, size_t bytes) {
  const size_t tid = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  const size_t head = (16 - ((uintptr_t)p & 15)) & 15;
  const size_t h = head < bytes ? head : bytes;
  for (size_t i = tid; i < h; i += stride) p[i] = 0;
  uint4* q = reinterpret_cast<uint4*>(p + h);
  const size_t n16 = (bytes - h) / 16;
  for (size_t i = tid; i < n16; i += stride) q[i] = make_uint4(0, 0, 0, 0);
  for (size_t i = h + n16 * 16 + tid; i < bytes; i += stride) p[i] = 0;
}

// Read floor of the attention's load structure: `workgroups` workgroups of
// 8 waves, workgroup w reading its own contiguous `per_wg` bytes in 16 KB
// chunks (wave i taking chunks i, i + 8, ...), one chunk in flight per wave,
// and nothing else: the time the ring kernel's stream would take if the
// chunks cost no compute, fold or combine.  Each thread XORs what it read
// into sink[w * 512 + thread] so the loads are kept.  Buffer loads past the
// region read 0 without touching memory.
__global__ __launch_bounds__(512) void read_floor_kernel(const uint8_t* src, size_t per_wg,
                                                         uint32_t* sink) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const uint8_t* base = src + (size_t)blockIdx.x * per_wg;
  const __amdgpu_buffer_rsrc_t r =
      buffer_rsrc(reinterpret_cast<const float*>(base), per_wg);
  const size_t chunks = (per_wg + 16383) / 16384;
  uint32_t acc = 0;
  for (size_t c = wave; c < chunks; c += 8) {
    u32x4 v[16];
#pragma unroll
    for (int k = 0; k < 16; ++k)
      v[k] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                           r, (int)(c * 16384 + k * 1024 + lane * 16), 0, 2));
#pragma unroll
    for (int k = 0; k < 16; ++k) acc ^= v[k].x ^ v[k].y ^ v[k].z ^ v[k].w;
  }
  sink[(size_t)blockIdx.x * 512 + tid] = acc;
}

hipError_t launch_read_floor(const void* src, size_t bytes, int workgroups, uint32_t* sink,
                             hipStream_t s) {
  const size_t per_wg = bytes / (size_t)workgroups;
  read_floor_kernel<<<workgroups, 512, 0, s>>>(static_cast<const uint8_t*>(src), per_wg, sink);
  return hipGetLastError();
}

hipError_t launch_tree_build(const int32_t* parents, const int32_t* kv_len, int B, int N,
                             uint64_t* anc, int32_t* depth, int32_t* pos, int32_t* flags,
                             hipStream_t s) {
  const int per_block = 4;
  const int grid = (B + per_block - 1) / per_block;
  tree_build_kernel<<<grid, per_block * kWave, 0, s>>>(parents, kv_len, B, N, anc, depth, pos,
                                                       flags);
  return hipGetLastError();
}

hipError_t launch_fill_zero(void* ptr, size_t bytes, hipStream_t s) {
  if (bytes == 0) return hipSuccess;
  size_t blocks = (bytes / 16 + 255) / 256;
  if (blocks < 1) blocks = 1;
  if (blocks > 4096) blocks = 4096;
  fill_zero_kernel<<<(unsigned)blocks, 256, 0, s>>>(static_cast<uint8_t*>(ptr), bytes);
  return hipGetLastError();
}

}  // namespace eagle
