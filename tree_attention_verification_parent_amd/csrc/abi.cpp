// C ABI of the verification step: argument validation, workspace sizing and
// dispatch to the gfx950 kernels.  Every check here happens before anything
// is enqueued; the kernels themselves guard what only the device can see.
#include <math.h>
#include <stdarg.h>
#include <stdio.h>

#include <string>

#include "eagle_verify.h"
#include "launch.h"

namespace {

thread_local std::string g_last_error;

eagle_status_t fail(eagle_status_t st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return st;
}

eagle_status_t hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return EAGLE_OK;
  return fail(EAGLE_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

hipStream_t as_stream(void* s) { return reinterpret_cast<hipStream_t>(s); }

bool tree_size_ok(int N) { return N >= 1 && N <= 64; }

}  // namespace

extern "C" {

const char* eagle_last_error(void) { return g_last_error.c_str(); }

int eagle_abi_version(void) { return 2; }

eagle_status_t eagle_validate_tree_host(const int32_t* parents, int B, int N) {
  if (B < 0) return fail(EAGLE_ERR_INVALID_ARGUMENT, "B must be >= 0 (got %d)", B);
  if (!tree_size_ok(N)) return fail(EAGLE_ERR_INVALID_ARGUMENT, "N must be in [1, 64] (got %d)", N);
  if (B > 0 && !parents) return fail(EAGLE_ERR_INVALID_ARGUMENT, "parents is NULL");
  for (int b = 0; b < B; ++b) {
    const int32_t* p = parents + (size_t)b * N;
    if (p[0] != -1) return fail(EAGLE_ERR_INVALID_ARGUMENT, "parents[%d, 0] = %d, expected -1", b, p[0]);
    for (int i = 1; i < N; ++i) {
      if (p[i] == -1) continue;  // absent node (ragged batch padding)
      if (p[i] < 0 || p[i] >= i)
        return fail(EAGLE_ERR_INVALID_ARGUMENT, "parents[%d, %d] = %d violates 0 <= parent < %d", b,
                    i, p[i], i);
      if (p[i] > 0 && p[p[i]] == -1)
        return fail(EAGLE_ERR_INVALID_ARGUMENT, "parents[%d, %d] = %d is an absent node", b, i, p[i]);
    }
  }
  return EAGLE_OK;
}

eagle_status_t eagle_workspace_clear(void* ptr, size_t bytes, void* stream) {
  if (bytes == 0) return EAGLE_OK;
  if (!ptr) return fail(EAGLE_ERR_INVALID_ARGUMENT, "workspace pointer is NULL");
  return hip_status(eagle::launch_fill_zero(ptr, bytes, as_stream(stream)), "workspace clear");
}

eagle_status_t eagle_testing_attn_plan(int kernel, int pieces_per_unit) {
  if (kernel < 0 || kernel > 2)
    return fail(EAGLE_ERR_INVALID_ARGUMENT, "kernel must be 0 (planner), 1 (ring) or 2 (group)");
  if (pieces_per_unit < 0 || pieces_per_unit > 1024)
    return fail(EAGLE_ERR_INVALID_ARGUMENT, "pieces_per_unit must be in [0, 1024]");
  eagle::set_attn_plan_override(kernel, pieces_per_unit);
  return EAGLE_OK;
}

eagle_status_t eagle_testing_read_floor(const void* src, size_t bytes, int workgroups,
                                        uint32_t* sink, void* stream) {
  if (!src || !sink) return fail(EAGLE_ERR_INVALID_ARGUMENT, "src and sink must be non-NULL");
  if (workgroups < 1 || workgroups > 65535)
    return fail(EAGLE_ERR_INVALID_ARGUMENT, "workgroups must be in [1, 65535] (got %d)", workgroups);
  if (bytes / (size_t)workgroups > 0x7fffffffu)
    return fail(EAGLE_ERR_INVALID_ARGUMENT, "at most 2^31 - 1 bytes per workgroup");
  if (bytes < (size_t)workgroups * 16)
    return fail(EAGLE_ERR_INVALID_ARGUMENT, "at least 16 bytes per workgroup");
  return hip_status(eagle::launch_read_floor(src, bytes, workgroups, sink, as_stream(stream)),
                    "read floor launch");
}

eagle_status_t eagle_tree_build(const int32_t* parents, const int32_t* kv_len, int B, int N,
                                uint64_t* anc, int32_t* depth, int32_t* pos, int32_t* seq_flags,
                                void* stream) {
  if (B < 0) return fail(EAGLE_ERR_INVALID_ARGUMENT, "B must be >= 0 (got %d)", B);
  if (!tree_size_ok(N)) return fail(EAGLE_ERR_INVALID_ARGUMENT, "N must be in [1, 64] (got %d)", N);
  if (B == 0) return EAGLE_OK;
  if (!parents || !anc) return fail(EAGLE_ERR_INVALID_ARGUMENT, "parents and anc must be non-NULL");
  if (pos && !kv_len) return fail(EAGLE_ERR_INVALID_ARGUMENT, "pos needs kv_len");
  return hip_status(eagle::launch_tree_build(parents, kv_len, B, N, anc, depth, pos, seq_flags,
                                             as_stream(stream)),
                    "tree build launch");
}

static eagle_status_t check_attn_shape(int B, int N, int Hq, int Hkv, int d, int Lmax) {
  if (B < 0) return fail(EAGLE_ERR_INVALID_ARGUMENT, "B must be >= 0 (got %d)", B);
  if (!tree_size_ok(N)) return fail(EAGLE_ERR_INVALID_ARGUMENT, "N must be in [1, 64] (got %d)", N);
  if (Hkv < 1 || Hq < 1) return fail(EAGLE_ERR_INVALID_ARGUMENT, "head counts must be >= 1");
  if (Hq % Hkv) return fail(EAGLE_ERR_UNSUPPORTED, "Hq (%d) must be a multiple of Hkv (%d)", Hq, Hkv);
  if (d != 64 && d != 128) return fail(EAGLE_ERR_UNSUPPORTED, "head dim %d not in {64, 128}", d);
  if (Lmax < N) return fail(EAGLE_ERR_INVALID_ARGUMENT, "Lmax (%d) must be >= N (%d)", Lmax, N);
  const double wgs = (double)B * Hkv * (((double)Hq / Hkv * N + 15) / 16) * 64;
  if (wgs > 2.0e9) return fail(EAGLE_ERR_UNSUPPORTED, "problem too large for one launch");
  return EAGLE_OK;
}

size_t eagle_tree_attn_workspace(int B, int N, int Hq, int Hkv, int d, int Lmax) {
  if (check_attn_shape(B, N, Hq, Hkv, d, Lmax) != EAGLE_OK || B == 0) return 0;
  return eagle::tree_attn_workspace_bytes(eagle::plan_tree_attn(B, N, Hq, Hkv, d, Lmax));
}

// Shared by both attention entry points: the tree comes either as ancestor
// masks (anc) or as parent links (parents, masks built in the kernel).
static eagle_status_t tree_attn_call(const uint16_t* q, const uint16_t* k_cache,
                                     const uint16_t* v_cache, const int32_t* kv_len,
                                     const uint64_t* anc, const int32_t* parents, int B, int N,
                                     int Hq, int Hkv, int d, int Lmax, float sm_scale,
                                     uint16_t* out, uint64_t* anc_out, int32_t* depth_out,
                                     int32_t* pos_out, void* workspace, size_t workspace_bytes,
                                     int32_t* seq_flags, void* stream) {
  const eagle::AttnPlan plan = eagle::plan_tree_attn(B, N, Hq, Hkv, d, Lmax);
  if (plan.kernel < 0)
    return fail(EAGLE_ERR_UNSUPPORTED, "the forced ring kernel holds at most 32 query rows per KV head (G * N = %d)",
                plan.M);
  const size_t need = eagle::tree_attn_workspace_bytes(plan);
  if (need > 0 && (!workspace || workspace_bytes < need))
    return fail(EAGLE_ERR_WORKSPACE, "tree attention needs %zu workspace bytes (got %zu)", need,
                workspace ? workspace_bytes : (size_t)0);
  const float scale = sm_scale > 0.f ? sm_scale : 1.0f / sqrtf((float)d);
  const float scale_log2 = scale * 1.4426950408889634f;
  return hip_status(eagle::launch_tree_attn(plan, q, k_cache, v_cache, kv_len, anc, parents,
                                            anc_out, depth_out, pos_out, B, N, Hq, Hkv, Lmax,
                                            scale_log2, out, workspace, seq_flags,
                                            as_stream(stream)),
                    "tree attention launch");
}

eagle_status_t eagle_tree_attn(const uint16_t* q, const uint16_t* k_cache, const uint16_t* v_cache,
                               const int32_t* kv_len, const uint64_t* anc, int B, int N, int Hq,
                               int Hkv, int d, int Lmax, float sm_scale, uint16_t* out,
                               void* workspace, size_t workspace_bytes, int32_t* seq_flags,
                               void* stream) {
  eagle_status_t st = check_attn_shape(B, N, Hq, Hkv, d, Lmax);
  if (st != EAGLE_OK) return st;
  if (B == 0) return EAGLE_OK;
  if (!q || !k_cache || !v_cache || !kv_len || !anc || !out)
    return fail(EAGLE_ERR_INVALID_ARGUMENT, "q, k_cache, v_cache, kv_len, anc and out must be non-NULL");
  if (!isfinite(sm_scale)) return fail(EAGLE_ERR_INVALID_ARGUMENT, "sm_scale must be finite");
  return tree_attn_call(q, k_cache, v_cache, kv_len, anc, nullptr, B, N, Hq, Hkv, d, Lmax,
                        sm_scale, out, nullptr, nullptr, nullptr, workspace, workspace_bytes,
                        seq_flags, stream);
}

eagle_status_t eagle_tree_attn_parents(const uint16_t* q, const uint16_t* k_cache,
                                       const uint16_t* v_cache, const int32_t* kv_len,
                                       const int32_t* parents, int B, int N, int Hq, int Hkv,
                                       int d, int Lmax, float sm_scale, uint16_t* out,
                                       uint64_t* anc, int32_t* depth, int32_t* pos,
                                       void* workspace, size_t workspace_bytes,
                                       int32_t* seq_flags, void* stream) {
  eagle_status_t st = check_attn_shape(B, N, Hq, Hkv, d, Lmax);
  if (st != EAGLE_OK) return st;
  if (B == 0) return EAGLE_OK;
  if (!q || !k_cache || !v_cache || !kv_len || !parents || !out)
    return fail(EAGLE_ERR_INVALID_ARGUMENT,
                "q, k_cache, v_cache, kv_len, parents and out must be non-NULL");
  if (!isfinite(sm_scale)) return fail(EAGLE_ERR_INVALID_ARGUMENT, "sm_scale must be finite");
  return tree_attn_call(q, k_cache, v_cache, kv_len, nullptr, parents, B, N, Hq, Hkv, d, Lmax,
                        sm_scale, out, anc, depth, pos, workspace, workspace_bytes, seq_flags,
                        stream);
}

eagle_status_t eagle_tree_attn_parents_noalloc(const uint16_t* q, const uint16_t* k_cache,
                                               const uint16_t* v_cache, const int32_t* kv_len,
                                               const int32_t* parents, int B, int N, int Hq,
                                               int Hkv, int d, int Lmax, float sm_scale,
                                               uint16_t* out, uint64_t* anc, int32_t* depth,
                                               int32_t* pos, int32_t* seq_flags, void* stream) {
  eagle_status_t st = check_attn_shape(B, N, Hq, Hkv, d, Lmax);
  if (st != EAGLE_OK) return st;
  if (B == 0) return EAGLE_OK;
  if (!q || !k_cache || !v_cache || !kv_len || !parents || !out)
    return fail(EAGLE_ERR_INVALID_ARGUMENT,
                "q, k_cache, v_cache, kv_len, parents and out must be non-NULL");
  if (!isfinite(sm_scale)) return fail(EAGLE_ERR_INVALID_ARGUMENT, "sm_scale must be finite");
  const eagle::AttnPlan plan = eagle::plan_tree_attn(B, N, Hq, Hkv, d, Lmax);
  if (plan.kernel < 0)
    return fail(EAGLE_ERR_UNSUPPORTED, "the forced ring kernel holds at most 32 query rows per KV head (G * N = %d)",
                plan.M);
  const size_t need = eagle::tree_attn_workspace_bytes(plan);
  if (need > eagle::kStaticScratchBytes)
    return fail(EAGLE_ERR_UNSUPPORTED,
                "this shape needs %zu scratch bytes; eagle_tree_attn_parents_noalloc holds at most "
                "%zu (use eagle_tree_attn_parents with a workspace)",
                need, eagle::kStaticScratchBytes);
  void* ws = nullptr;
  if (need > 0) {
    st = hip_status(eagle::static_scratch(&ws), "static scratch lookup");
    if (st != EAGLE_OK) return st;
    // the tickets must start at zero: a fill kernel (no memset node)
    const size_t zeroed = eagle::tree_attn_zeroed_bytes(plan);
    if (zeroed > 0) {
      st = hip_status(eagle::launch_fill_zero(ws, zeroed, as_stream(stream)), "scratch clear");
      if (st != EAGLE_OK) return st;
    }
  }
  const float scale = sm_scale > 0.f ? sm_scale : 1.0f / sqrtf((float)d);
  return hip_status(eagle::launch_tree_attn(plan, q, k_cache, v_cache, kv_len, nullptr, parents,
                                            anc, depth, pos, B, N, Hq, Hkv, Lmax,
                                            scale * 1.4426950408889634f, out, ws, seq_flags,
                                            as_stream(stream)),
                    "tree attention launch");
}

static eagle_status_t check_verify_shape(int B, int N, int V) {
  if (B < 0) return fail(EAGLE_ERR_INVALID_ARGUMENT, "B must be >= 0 (got %d)", B);
  if (!tree_size_ok(N)) return fail(EAGLE_ERR_INVALID_ARGUMENT, "N must be in [1, 64] (got %d)", N);
  if (V < 1) return fail(EAGLE_ERR_INVALID_ARGUMENT, "V must be >= 1 (got %d)", V);
  if (V > 32768) return fail(EAGLE_ERR_UNSUPPORTED, "V = %d exceeds 32768", V);
  if ((double)B * N > 1.0e8) return fail(EAGLE_ERR_UNSUPPORTED, "B * N too large");
  return EAGLE_OK;
}

size_t eagle_verify_accept_workspace(int B, int N, int V) {
  if (check_verify_shape(B, N, V) != EAGLE_OK || B == 0) return 0;
  return eagle::verify_workspace_bytes(eagle::plan_verify(B, N, V));
}

eagle_status_t eagle_verify_accept(const int32_t* draft_tokens, const float* draft_probs,
                                   const int32_t* draft_row,
                                   const float* target_logits, const int32_t* parents,
                                   const int32_t* kv_len, int B, int N, int V, float temperature,
                                   const float* uniforms, int32_t* accept_len, int32_t* path,
                                   int32_t* accepted_tokens, int32_t* bonus_token,
                                   int32_t* kv_src_slots, float* out_probs, float* out_final_dist,
                                   float* out_ratio, void* workspace, size_t workspace_bytes,
                                   int32_t* seq_flags, void* stream) {
  eagle_status_t st = check_verify_shape(B, N, V);
  if (st != EAGLE_OK) return st;
  if (!isfinite(temperature) || temperature < 0.f)
    return fail(EAGLE_ERR_INVALID_ARGUMENT, "temperature must be finite and >= 0");
  if (B == 0) return EAGLE_OK;
  if (!draft_tokens || !target_logits || !parents || !kv_len || !uniforms)
    return fail(EAGLE_ERR_INVALID_ARGUMENT, "draft_tokens, target_logits, parents, kv_len and uniforms must be non-NULL");
  if (temperature > 0.f && !draft_probs)
    return fail(EAGLE_ERR_INVALID_ARGUMENT, "draft_probs is required when temperature > 0");
  if (!accept_len || !path || !accepted_tokens || !bonus_token || !kv_src_slots)
    return fail(EAGLE_ERR_INVALID_ARGUMENT, "accept_len, path, accepted_tokens, bonus_token and kv_src_slots must be non-NULL");
  const eagle::VerifyPlan plan = eagle::plan_verify(B, N, V);
  const size_t need = eagle::verify_workspace_bytes(plan);
  if (!workspace || workspace_bytes < need)
    return fail(EAGLE_ERR_WORKSPACE, "verification needs %zu workspace bytes (got %zu)", need,
                workspace ? workspace_bytes : (size_t)0);
  return hip_status(eagle::launch_verify(plan, draft_tokens, draft_probs, draft_row, target_logits, parents,
                                         kv_len, B, N, temperature, uniforms, accept_len, path,
                                         accepted_tokens, bonus_token, kv_src_slots, out_probs,
                                         out_final_dist, out_ratio, workspace, seq_flags,
                                         eagle::VerifyCompact{}, as_stream(stream)),
                    "verification launch");
}

static eagle_status_t check_compact_shape(int N, int Hkv, int d, int Lmax) {
  if (Hkv < 1) return fail(EAGLE_ERR_INVALID_ARGUMENT, "Hkv must be >= 1");
  if (d != 64 && d != 128) return fail(EAGLE_ERR_UNSUPPORTED, "head dim %d not in {64, 128}", d);
  if (Lmax < N) return fail(EAGLE_ERR_INVALID_ARGUMENT, "Lmax (%d) must be >= N (%d)", Lmax, N);
  return EAGLE_OK;
}

eagle_status_t eagle_verify_accept_compact(
    const int32_t* draft_tokens, const float* draft_probs, const int32_t* draft_row,
    const float* target_logits,
    const int32_t* parents, const int32_t* kv_len, int B, int N, int V, float temperature,
    const float* uniforms, int32_t* accept_len, int32_t* path, int32_t* accepted_tokens,
    int32_t* bonus_token, int32_t* kv_src_slots, uint16_t* k_cache, uint16_t* v_cache, int Hkv,
    int d, int Lmax, int32_t* new_kv_len, void* workspace, size_t workspace_bytes,
    int32_t* seq_flags, void* stream) {
  eagle_status_t st = check_verify_shape(B, N, V);
  if (st != EAGLE_OK) return st;
  st = check_compact_shape(N, Hkv, d, Lmax);
  if (st != EAGLE_OK) return st;
  if (!isfinite(temperature) || temperature < 0.f)
    return fail(EAGLE_ERR_INVALID_ARGUMENT, "temperature must be finite and >= 0");
  if (B == 0) return EAGLE_OK;
  if (!draft_tokens || !target_logits || !parents || !kv_len || !uniforms)
    return fail(EAGLE_ERR_INVALID_ARGUMENT, "draft_tokens, target_logits, parents, kv_len and uniforms must be non-NULL");
  if (temperature > 0.f && !draft_probs)
    return fail(EAGLE_ERR_INVALID_ARGUMENT, "draft_probs is required when temperature > 0");
  if (!accept_len || !path || !accepted_tokens || !bonus_token || !kv_src_slots)
    return fail(EAGLE_ERR_INVALID_ARGUMENT, "accept_len, path, accepted_tokens, bonus_token and kv_src_slots must be non-NULL");
  if (!k_cache || !v_cache || !new_kv_len)
    return fail(EAGLE_ERR_INVALID_ARGUMENT, "k_cache, v_cache and new_kv_len must be non-NULL");
  if (new_kv_len == kv_len) return fail(EAGLE_ERR_INVALID_ARGUMENT, "new_kv_len must not alias kv_len");
  if ((double)B * Hkv > 2.0e9) return fail(EAGLE_ERR_UNSUPPORTED, "B * Hkv too large");
  const eagle::VerifyPlan plan = eagle::plan_verify(B, N, V);
  const size_t need = eagle::verify_workspace_bytes(plan);
  if (!workspace || workspace_bytes < need)
    return fail(EAGLE_ERR_WORKSPACE, "verification needs %zu workspace bytes (got %zu)", need,
                workspace ? workspace_bytes : (size_t)0);
  const eagle::VerifyCompact kc{k_cache, v_cache, new_kv_len, Hkv, d, Lmax};
  return hip_status(eagle::launch_verify(plan, draft_tokens, draft_probs, draft_row, target_logits, parents,
                                         kv_len, B, N, temperature, uniforms, accept_len, path,
                                         accepted_tokens, bonus_token, kv_src_slots, nullptr,
                                         nullptr, nullptr, workspace, seq_flags, kc,
                                         as_stream(stream)),
                    "verification launch");
}

eagle_status_t eagle_kv_compact(uint16_t* k_cache, uint16_t* v_cache, const int32_t* kv_len,
                                const int32_t* kv_src_slots, const int32_t* accept_len, int B,
                                int N, int Hkv, int d, int Lmax, int32_t* new_kv_len,
                                int32_t* seq_flags, void* stream) {
  if (B < 0) return fail(EAGLE_ERR_INVALID_ARGUMENT, "B must be >= 0 (got %d)", B);
  if (!tree_size_ok(N)) return fail(EAGLE_ERR_INVALID_ARGUMENT, "N must be in [1, 64] (got %d)", N);
  if (Hkv < 1) return fail(EAGLE_ERR_INVALID_ARGUMENT, "Hkv must be >= 1");
  if (d != 64 && d != 128) return fail(EAGLE_ERR_UNSUPPORTED, "head dim %d not in {64, 128}", d);
  if (Lmax < N) return fail(EAGLE_ERR_INVALID_ARGUMENT, "Lmax (%d) must be >= N (%d)", Lmax, N);
  if (B == 0) return EAGLE_OK;
  if (!k_cache || !v_cache || !kv_len || !kv_src_slots || !accept_len || !new_kv_len)
    return fail(EAGLE_ERR_INVALID_ARGUMENT, "cache, kv_len, kv_src_slots, accept_len and new_kv_len must be non-NULL");
  if (new_kv_len == kv_len) return fail(EAGLE_ERR_INVALID_ARGUMENT, "new_kv_len must not alias kv_len");
  if ((double)B * Hkv > 2.0e9) return fail(EAGLE_ERR_UNSUPPORTED, "B * Hkv too large");
  return hip_status(eagle::launch_kv_compact(k_cache, v_cache, kv_len, kv_src_slots, accept_len, B, N,
                                             Hkv, d, Lmax, new_kv_len, seq_flags, as_stream(stream)),
                    "kv compaction launch");
}

eagle_status_t eagle_feature_gather(const void* features, const int32_t* path,
                                    const int32_t* accept_len, int B, int N, int64_t row_bytes,
                                    void* out, int32_t* seq_flags, void* stream) {
  if (B < 0) return fail(EAGLE_ERR_INVALID_ARGUMENT, "B must be >= 0 (got %d)", B);
  if (!tree_size_ok(N)) return fail(EAGLE_ERR_INVALID_ARGUMENT, "N must be in [1, 64] (got %d)", N);
  if (row_bytes <= 0 || row_bytes % 16 != 0)
    return fail(EAGLE_ERR_INVALID_ARGUMENT, "row_bytes must be a positive multiple of 16 (got %lld)",
                (long long)row_bytes);
  if ((double)N * (double)(row_bytes / 16) >= 2147483648.0)
    return fail(EAGLE_ERR_INVALID_ARGUMENT, "N * row_bytes must be below 2^35");
  if (B == 0) return EAGLE_OK;
  if ((double)B * 64.0 > 2.0e9) return fail(EAGLE_ERR_INVALID_ARGUMENT, "B too large for one launch");
  if (!features || !path || !accept_len || !out)
    return fail(EAGLE_ERR_INVALID_ARGUMENT, "features, path, accept_len and out must be non-NULL");
  const uintptr_t f0 = reinterpret_cast<uintptr_t>(features);
  const uintptr_t o0 = reinterpret_cast<uintptr_t>(out);
  const uintptr_t bytes = (uintptr_t)B * (uintptr_t)N * (uintptr_t)row_bytes;
  if (f0 < o0 + bytes && o0 < f0 + bytes)
    return fail(EAGLE_ERR_INVALID_ARGUMENT, "out must not overlap features");
  return hip_status(eagle::launch_feature_gather(features, path, accept_len, B, N, row_bytes, out,
                                                 seq_flags, as_stream(stream)),
                    "feature gather launch");
}

eagle_status_t eagle_dtree_expand(const float* q, int B, int R, int V, int k, const int32_t* parent_node,
                             const float* parent_value, int32_t* created_parent,
                             int32_t* created_token, float* created_value, int T, int base,
                             void* stream) {
  if (B < 0 || R < 1 || V < 1 || V > 32768 || k < 1 || k > V || k > 64 || base < 0 || T < 1)
    return fail(EAGLE_ERR_INVALID_ARGUMENT,
                "eagle_dtree_expand: need B >= 0, R >= 1, 1 <= V <= 32768, 1 <= k <= min(V, 64), base >= 0 "
                "(got B=%d R=%d V=%d k=%d base=%d)", B, R, V, k, base);
  if ((long long)base + (long long)R * k > T)
    return fail(EAGLE_ERR_INVALID_ARGUMENT, "eagle_dtree_expand: base + R*k = %lld exceeds T = %d",
                (long long)base + (long long)R * k, T);
  if ((double)B * R > 2.0e9) return fail(EAGLE_ERR_INVALID_ARGUMENT, "eagle_dtree_expand: B * R too large");
  if (B == 0) return EAGLE_OK;
  if (!q || !parent_node || !parent_value || !created_parent || !created_token || !created_value)
    return fail(EAGLE_ERR_INVALID_ARGUMENT, "eagle_dtree_expand: NULL pointer");
  return hip_status(eagle::launch_eagle2_expand(q, B, R, V, k, parent_node, parent_value,
                                                created_parent, created_token, created_value, T,
                                                base, as_stream(stream)),
                    "eagle_dtree_expand launch");
}

eagle_status_t eagle_dtree_select(const float* created_value, int B, int T, int first, int M, int k,
                             int32_t* out_node, float* out_value, void* stream) {
  if (B < 0 || first < 0 || M < 1 || M > 2048 || k < 1 || k > M || (long long)first + M > T)
    return fail(EAGLE_ERR_INVALID_ARGUMENT,
                "eagle_dtree_select: need B >= 0, 1 <= k <= M <= 2048, 0 <= first, first + M <= T "
                "(got B=%d T=%d first=%d M=%d k=%d)", B, T, first, M, k);
  if (B == 0) return EAGLE_OK;
  if (!created_value || !out_node || !out_value)
    return fail(EAGLE_ERR_INVALID_ARGUMENT, "eagle_dtree_select: NULL pointer");
  return hip_status(eagle::launch_eagle2_select(created_value, B, T, first, M, k, out_node,
                                                out_value, as_stream(stream)),
                    "eagle_dtree_select launch");
}

eagle_status_t eagle_dtree_rerank(const int32_t* created_parent, const int32_t* created_token,
                             const float* created_value, int B, int T, int T_used, int N,
                             int32_t* parents, int32_t* tokens, int32_t* kept_node,
                             int32_t* seq_flags, void* stream) {
  if (B < 0 || !tree_size_ok(N) || T_used < N || T_used > T || T_used > 2049)
    return fail(EAGLE_ERR_INVALID_ARGUMENT,
                "eagle_dtree_rerank: need B >= 0, 1 <= N <= 64, N <= T_used <= min(T, 2049) "
                "(got B=%d T=%d T_used=%d N=%d)", B, T, T_used, N);
  if (B == 0) return EAGLE_OK;
  if (!created_parent || !created_token || !created_value || !parents || !tokens || !kept_node)
    return fail(EAGLE_ERR_INVALID_ARGUMENT, "eagle_dtree_rerank: NULL pointer");
  return hip_status(eagle::launch_eagle2_rerank(created_parent, created_token, created_value, B, T,
                                                T_used, N, parents, tokens, kept_node, seq_flags,
                                                as_stream(stream)),
                    "eagle_dtree_rerank launch");
}

}  // extern "C"
