// Device-side helpers shared by the gfx950 kernels of the verification step.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "eagle_verify.h"

namespace eagle {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// Raw buffer over `bytes` bytes at `base`: loads at offsets past the end read
// 0 without touching memory.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_rsrc(const float* base, size_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(base), 0,
                                           (int)(bytes < 0x7fffffffu ? bytes : 0x7fffffffu),
                                           0x00020000);
}
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;

// Workgroup barrier that orders LDS accesses only.  __syncthreads() also
// waits for every outstanding global load of the wave (a workgroup-scope
// release covers global memory), which would pull a prefetch issued before
// the barrier onto the critical path; this one lets such loads stay in
// flight.  Loads that land in LDS (global_load_lds) are not ordered by it:
// their data is only read back by the thread that issued them, after its own
// vmcnt wait.
__device__ __forceinline__ void barrier_lds() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

__device__ __forceinline__ float bf16_bits_to_float(uint32_t bits16) {
  return __uint_as_float(bits16 << 16);
}

// Round to nearest even, NaN kept quiet.
__device__ __forceinline__ uint16_t float_to_bf16_bits(float f) {
  __bf16 h = (__bf16)f;
  return __builtin_bit_cast(uint16_t, h);
}

template <typename T>
__device__ __forceinline__ T wave_max(T v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v = fmaxf(v, __shfl_xor(v, off));
  return v;
}

__device__ __forceinline__ double wave_sum(double v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off);
  return v;
}

__device__ __forceinline__ float wave_sum_f(float v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off);
  return v;
}

// ---- wave reductions ---------------------------------------------------------
// DPP lane permutations within a row of 16: swap neighbours, swap pairs, mirror
// each half row, mirror the row.  After the four steps every lane of a row
// holds the row's result (the operations are commutative, so both lanes of a
// pair compute the same value bit for bit); readlane combines the four rows in
// a fixed order, giving every lane the same wave result.
constexpr int kDppXor1 = 0xB1;       // quad_perm [1,0,3,2]
constexpr int kDppXor2 = 0x4E;       // quad_perm [2,3,0,1]
constexpr int kDppHalfMirror = 0x141;
constexpr int kDppMirror = 0x140;

template <int CTRL>
__device__ __forceinline__ int dpp_i(int v) {
  return __builtin_amdgcn_update_dpp(0, v, CTRL, 0xf, 0xf, false);
}
template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
  return __int_as_float(dpp_i<CTRL>(__float_as_int(v)));
}
template <int CTRL>
__device__ __forceinline__ double dpp_d(double v) {
  return __hiloint2double(dpp_i<CTRL>(__double2hiint(v)), dpp_i<CTRL>(__double2loint(v)));
}
__device__ __forceinline__ int lane_i(int v, int l) { return __builtin_amdgcn_readlane(v, l); }
__device__ __forceinline__ float lane_f(float v, int l) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), l));
}
__device__ __forceinline__ double lane_d(double v, int l) {
  return __hiloint2double(__builtin_amdgcn_readlane(__double2hiint(v), l),
                          __builtin_amdgcn_readlane(__double2loint(v), l));
}

__device__ __forceinline__ double wave_allsum(double v) {
  v += dpp_d<kDppXor1>(v);
  v += dpp_d<kDppXor2>(v);
  v += dpp_d<kDppHalfMirror>(v);
  v += dpp_d<kDppMirror>(v);
  return (lane_d(v, 0) + lane_d(v, 16)) + (lane_d(v, 32) + lane_d(v, 48));
}
__device__ __forceinline__ float wave_allmax(float v) {
  v = fmaxf(v, dpp_f<kDppXor1>(v));
  v = fmaxf(v, dpp_f<kDppXor2>(v));
  v = fmaxf(v, dpp_f<kDppHalfMirror>(v));
  v = fmaxf(v, dpp_f<kDppMirror>(v));
  return fmaxf(fmaxf(lane_f(v, 0), lane_f(v, 16)), fmaxf(lane_f(v, 32), lane_f(v, 48)));
}
__device__ __forceinline__ int wave_allmin_i(int v) {
  v = min(v, dpp_i<kDppXor1>(v));
  v = min(v, dpp_i<kDppXor2>(v));
  v = min(v, dpp_i<kDppHalfMirror>(v));
  v = min(v, dpp_i<kDppMirror>(v));
  return min(min(lane_i(v, 0), lane_i(v, 16)), min(lane_i(v, 32), lane_i(v, 48)));
}
__device__ __forceinline__ int wave_allmax_i(int v) {
  v = max(v, dpp_i<kDppXor1>(v));
  v = max(v, dpp_i<kDppXor2>(v));
  v = max(v, dpp_i<kDppHalfMirror>(v));
  v = max(v, dpp_i<kDppMirror>(v));
  return max(max(lane_i(v, 0), lane_i(v, 16)), max(lane_i(v, 32), lane_i(v, 48)));
}

// Sums whose result one lane needs (a workgroup sum's partial per wave):
// after the four row steps, row_bcast:15 adds the last lane of rows 0
// and 2 into rows 1 and 3, then row_bcast:31 adds the last lane of row 1 into
// rows 2 and 3, so the lanes of row 3 (48..63) hold the wave's result.  Two
// DPP operations replace four readlanes whose results pass through scalar
// registers.  Rows a broadcast skips keep `old`: the operation's identity.
constexpr int kDppBcast15 = 0x142;
constexpr int kDppBcast31 = 0x143;
template <int CTRL, int ROWS>
__device__ __forceinline__ int dpp_rows_i(int old, int v) {
  return __builtin_amdgcn_update_dpp(old, v, CTRL, ROWS, 0xf, false);
}
__device__ __forceinline__ float wave_sum_last(float v) {
  v += dpp_f<kDppXor1>(v);
  v += dpp_f<kDppXor2>(v);
  v += dpp_f<kDppHalfMirror>(v);
  v += dpp_f<kDppMirror>(v);
  v += __int_as_float(dpp_rows_i<kDppBcast15, 0xa>(0, __float_as_int(v)));
  v += __int_as_float(dpp_rows_i<kDppBcast31, 0xc>(0, __float_as_int(v)));
  return v;
}
__device__ __forceinline__ double wave_sum_last(double v) {
  v += dpp_d<kDppXor1>(v);
  v += dpp_d<kDppXor2>(v);
  v += dpp_d<kDppHalfMirror>(v);
  v += dpp_d<kDppMirror>(v);
  v += __hiloint2double(dpp_rows_i<kDppBcast15, 0xa>(0, __double2hiint(v)),
                        dpp_rows_i<kDppBcast15, 0xa>(0, __double2loint(v)));
  v += __hiloint2double(dpp_rows_i<kDppBcast31, 0xc>(0, __double2hiint(v)),
                        dpp_rows_i<kDppBcast31, 0xc>(0, __double2loint(v)));
  return v;
}
// Sums of M values over the wave at once (the M reductions interleave, so
// their latencies overlap); every lane receives every sum.
template <int M>
__device__ __forceinline__ void wave_allsum_n(float (&v)[M]) {
#pragma unroll
  for (int i = 0; i < M; ++i) v[i] += dpp_f<kDppXor1>(v[i]);
#pragma unroll
  for (int i = 0; i < M; ++i) v[i] += dpp_f<kDppXor2>(v[i]);
#pragma unroll
  for (int i = 0; i < M; ++i) v[i] += dpp_f<kDppHalfMirror>(v[i]);
#pragma unroll
  for (int i = 0; i < M; ++i) v[i] += dpp_f<kDppMirror>(v[i]);
#pragma unroll
  for (int i = 0; i < M; ++i)
    v[i] = (lane_f(v[i], 0) + lane_f(v[i], 16)) + (lane_f(v[i], 32) + lane_f(v[i], 48));
}

// Ancestor set, depth and link check of one tree node per lane (lane i owns
// node i, N <= 64), from the sequence's parent array (EAGLE, paperlayer.ai
// summary, A.1 Tree Structure: each node attends to its ancestors).  Pointer
// jumping: after r rounds a lane has OR-ed in the masks of its 2^r nearest
// ancestors, so 6 rounds cover any depth below 64.  Parent -1 marks an absent
// node (padding of a smaller tree in a ragged batch): its set is itself
// alone, depth 0.  A malformed link (root with a parent, a parent not below
// the node) is reported in `bad` and replaced by the root, keeping every mask
// in range; a present node under an absent one is reported too.  Every lane of the wave
// must call it (cross-lane shuffles); lanes >= N return an empty set.
struct TreeLinks {
  uint64_t anc;
  int depth;
  bool bad;
};

__device__ __forceinline__ TreeLinks tree_links_wave(const int32_t* parents_b, int N) {
  const int lane = threadIdx.x & (kWave - 1);
  const bool live = lane < N;
  int par = live ? parents_b[lane] : -1;
  bool bad = false;
  if (live) {
    if (lane == 0) {
      bad = par != -1;
      par = -1;
    } else if (par != -1 && (par < 0 || par >= lane)) {
      bad = true;
      par = 0;
    }  // par == -1: an absent node (ragged batch padding), its own ancestor only
  }
  uint64_t a = live ? (1ull << lane) : 0ull;
  int cnt = par >= 0 ? 1 : 0;
  int jump = par;
#pragma unroll
  for (int r = 0; r < 6; ++r) {
    const int src = jump >= 0 ? jump : lane;
    const uint64_t a_j = __shfl(a, src);
    const int cnt_j = __shfl(cnt, src);
    const int jump_j = __shfl(jump, src);
    if (jump >= 0) {
      a |= a_j;
      cnt += cnt_j;
      jump = jump_j;
    }
  }
  // a present node must reach the root; one under an absent node does not
  if (live && lane > 0 && par >= 0 && !(a & 1ull)) bad = true;
  return TreeLinks{a, cnt, bad};
}

// Number of compute units the grids are shaped for (MI355X: 8 XCDs x 32 CUs).
constexpr int kNumCUs = 256;
constexpr int kNumXCDs = 8;

}  // namespace eagle
