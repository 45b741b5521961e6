// Host-side launchers of the gfx950 kernels (one per .hip file); the C ABI in
// abi.cpp validates arguments and calls these.  All return a hipError_t from
// the launch and never synchronise.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace eagle {

hipError_t launch_tree_build(const int32_t* parents, const int32_t* kv_len, int B, int N,
                             uint64_t* anc, int32_t* depth, int32_t* pos, int32_t* flags,
                             hipStream_t s);

hipError_t launch_fill_zero(void* ptr, size_t bytes, hipStream_t s);
hipError_t launch_read_floor(const void* src, size_t bytes, int workgroups, uint32_t* sink,
                             hipStream_t s);

// Tree attention -----------------------------------------------------------
struct AttnPlan {
  int d;
  int G;           // query heads per KV head
  int M;           // query rows per (b, kv head) = G * N
  int kernel;      // 1: ring (M <= 32), 2: group; -1: shape not supported by the forced kernel
  int rows_per_wg; // query rows per workgroup
  int qgroups;     // ceil(M / rows_per_wg)
  int units;       // B * Hkv * qgroups
  int slots;       // workgroups launched (a multiple of 8)
  int kg;          // keys per planning chunk
  int max_pieces;  // pieces per unit at most
  int full_pieces; // pieces per unit the device gives when every sequence fills the cache
  int ring_cost;   // 1: the device picks pieces by the ring kernel's order of decompositions
};

// Test-only: force the kernel (0 planner, 1 ring, 2 group) and the pieces per
// unit (0 planner) of later plans.
void set_attn_plan_override(int kernel, int pieces);
AttnPlan plan_tree_attn(int B, int N, int Hq, int Hkv, int d, int Lmax);
size_t tree_attn_workspace_bytes(const AttnPlan& p);
// Leading workspace bytes that must be zero when a call starts (the ring
// kernel's piece tickets, which every call leaves zero again).
size_t tree_attn_zeroed_bytes(const AttnPlan& p);

// Static scratch of eagle_tree_attn_parents_noalloc: its device address on
// the current device (looked up once per device).
constexpr size_t kStaticScratchBytes = size_t(64) << 20;
constexpr int kMaxScratchDevices = 64;
hipError_t static_scratch(void** ptr);

hipError_t launch_tree_attn(const AttnPlan& plan, const uint16_t* q, const uint16_t* k,
                            const uint16_t* v, const int32_t* kv_len, const uint64_t* anc,
                            const int32_t* parents, uint64_t* anc_out, int32_t* depth_out,
                            int32_t* pos_out,
                            int B, int N, int Hq, int Hkv, int Lmax, float scale_log2,
                            uint16_t* out, void* ws, int32_t* flags, hipStream_t s);

// Verification (vocabulary statistics + acceptance walk) -------------------
struct VerifyPlan {
  int V;
  int parts;                 // workgroups per node of the T = 0 argmax (1: one per node)
  size_t ws_counters;        // per-sequence tickets
  size_t ws_amax;            // per-node packed argmax words
  size_t ws_stats;           // per-node outcomes
};

VerifyPlan plan_verify(int B, int N, int V);
size_t verify_workspace_bytes(const VerifyPlan& p);

// Compaction fused into the walk (eagle_verify_accept_compact); k == nullptr: none.
struct VerifyCompact {
  uint16_t* k;
  uint16_t* v;
  int32_t* new_len;
  int Hkv, d, Lmax;
};

hipError_t launch_verify(const VerifyPlan& plan, const int32_t* tokens, const float* draft,
                         const int32_t* draft_row, const float* logits, const int32_t* parents, const int32_t* kv_len,
                         int B, int N, float T, const float* uniforms, int32_t* accept_len,
                         int32_t* path, int32_t* acc_tokens, int32_t* bonus, int32_t* kv_src,
                         float* out_probs, float* out_final, float* out_ratio, void* ws,
                         int32_t* flags, const VerifyCompact& kc, hipStream_t s);

// KV compaction ------------------------------------------------------------
hipError_t launch_kv_compact(uint16_t* k, uint16_t* v, const int32_t* kv_len,
                             const int32_t* kv_src, const int32_t* accept_len, int B, int N,
                             int Hkv, int d, int Lmax, int32_t* new_len, int32_t* flags,
                             hipStream_t s);

// Feature gather (out-of-place, rows as 16-byte columns) ----------------------
hipError_t launch_feature_gather(const void* features, const int32_t* path,
                                 const int32_t* accept_len, int B, int N, int64_t row_bytes,
                                 void* out, int32_t* flags, hipStream_t s);

// EAGLE-2 dynamic tree --------------------------------------------------------
hipError_t launch_eagle2_expand(const float* q, int B, int R, int V, int k,
                                const int32_t* parent_node, const float* parent_value,
                                int32_t* cpar, int32_t* ctok, float* cval, int T, int base,
                                hipStream_t s);
hipError_t launch_eagle2_select(const float* cval, int B, int T, int first, int M, int k,
                                int32_t* out_node, float* out_value, hipStream_t s);
hipError_t launch_eagle2_rerank(const int32_t* cpar, const int32_t* ctok, const float* cval,
                                int B, int T, int T_used, int N, int32_t* parents,
                                int32_t* tokens, int32_t* kept_node, int32_t* flags,
                                hipStream_t s);

}  // namespace eagle
