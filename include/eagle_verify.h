/*
 * eagle_verify.h — C ABI of the tree-verification step of EAGLE-style
 * speculative sampling, for AMD Instinct MI355X (gfx950).
 *
 * The step verifies a tree-structured draft with one target forward (tree
 * attention) and then walks the tree, accepting drafted tokens with
 * probability min(1, p/p_hat) and resampling from the adjusted distribution
 * on rejection (EAGLE: Speculative Sampling Requires Rethinking Feature
 * Uncertainty, paperlayer.ai summary of arXiv 2401.15077: §2 Preliminaries,
 * §3 EAGLE, A.1 Tree Structure, A.2 Multi-Round Speculative Sampling).
 *
 * Conventions shared by every entry point
 *   - All pointers marked "device" are device (HBM) addresses on the current
 *     HIP device; pointers marked "host" are host memory.  The caller owns
 *     every buffer; the library never allocates device memory.
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream).
 *     Calls only enqueue work on it and return; none synchronises the host.
 *   - bf16 tensors are passed as uint16_t bit patterns.
 *   - Layouts are row-major and contiguous, as annotated [outer, ..., inner].
 *   - Tree topology: node 0 is the root (parent -1); for i >= 1,
 *     0 <= parent[i] < i.  N counts the root, 1 <= N <= 64.  A batch of
 *     trees of different sizes (ragged batch) pads each smaller tree with
 *     absent nodes, parent[i] = -1 for i >= 1: an absent node is nobody's
 *     parent or child, is never tested and never on a path; its ancestor set
 *     is itself (depth 0), so its attention row is that of a lone node and
 *     its token, draft row and uniform are not read by the walk.  A present
 *     node whose parent is absent is a data error (EAGLE_FLAG_BAD_PARENT).
 *   - Host-detectable errors (null pointers, bad sizes, unsupported shapes,
 *     a too-small workspace) return a non-zero status before anything is
 *     enqueued; eagle_last_error() then describes it (thread-local).
 *   - Data errors only visible on the device (a bad parent, a kv_len that
 *     leaves no room for the tree, a token outside the vocabulary, a
 *     non-finite logit) never fault: the kernels stay in bounds, OR a bit
 *     into seq_flags[b] (when seq_flags is non-NULL) and produce defined
 *     but meaningless results for that sequence.
 */
#ifndef EAGLE_VERIFY_H
#define EAGLE_VERIFY_H

#include <stddef.h>
#include <stdint.h>

#if defined(__GNUC__) || defined(__clang__)
#define EAGLE_API __attribute__((visibility("default")))
#else
#define EAGLE_API
#endif

#ifdef __cplusplus
extern "C" {
#endif

typedef int eagle_status_t;

#define EAGLE_OK                    0
#define EAGLE_ERR_INVALID_ARGUMENT  1  /* null pointer, size out of range       */
#define EAGLE_ERR_UNSUPPORTED       2  /* shape outside what the kernels cover  */
#define EAGLE_ERR_HIP               3  /* HIP runtime error (no device, launch) */
#define EAGLE_ERR_WORKSPACE         4  /* workspace NULL or too small           */

/* Bits OR-ed into seq_flags[b] by the kernels. */
#define EAGLE_FLAG_BAD_PARENT   1  /* parent array violates the tree rules  */
#define EAGLE_FLAG_BAD_KV_LEN   2  /* kv_len[b] < 0 or kv_len[b] + N > Lmax */
#define EAGLE_FLAG_BAD_TOKEN    4  /* a drafted token outside [0, V)        */
#define EAGLE_FLAG_NONFINITE    8  /* NaN or Inf in a target logit row      */
/* 16 is unused (no kernel waits for another workgroup) */
#define EAGLE_FLAG_BAD_PATH    32  /* accepted path not as the walk emits  */
                                   /* it (eagle_feature_gather)            */
#define EAGLE_FLAG_BAD_ROW     64  /* draft_row outside [0, N) on a tested */
                                   /* node (eagle_verify_accept*)          */

/* Message for the last non-zero status returned on this thread. */
EAGLE_API const char* eagle_last_error(void);

/* Version of this ABI (incremented on any signature change; 2: draft_row). */
EAGLE_API int eagle_abi_version(void);

/*
 * Host-only check of parent arrays (host [B, N] int32).  Returns EAGLE_OK or
 * EAGLE_ERR_INVALID_ARGUMENT naming the first offending (b, i).  Touches no
 * device.
 */
EAGLE_API eagle_status_t eagle_validate_tree_host(const int32_t* parents, int B, int N);

/*
 * Zero-fill `bytes` of device memory at `ptr` with a kernel (no memset node,
 * so it may be captured in a HIP graph).  eagle_verify_accept's workspace
 * must be zero before its first use; each call leaves its tickets and argmax
 * words zero again (the rest holds per-call scratch), so it is cleared once.
 */
EAGLE_API eagle_status_t eagle_workspace_clear(void* ptr, size_t bytes, void* stream);

/*
 * Tree mask builder.  Each drafted node attends to its ancestors (EAGLE,
 * paperlayer.ai summary, §3 EAGLE: tree attention; A.1 Tree Structure).
 *
 *   parents  device [B, N] int32
 *   kv_len   device [B] int32 or NULL: committed length L of each sequence
 *   anc      device [B, N] uint64 out: bit j of anc[b, i] set iff node j lies
 *            on the path root..i (i included)
 *   depth    device [B, N] int32 out or NULL: depth of node i (root 0)
 *   pos      device [B, N] int32 out or NULL: L + depth (position id of node
 *            i, for the caller's rotary embedding); needs kv_len
 *   seq_flags device [B] int32 or NULL (EAGLE_FLAG_BAD_PARENT)
 * A bad parent is treated as the root, so anc stays within [0, N).
 */
EAGLE_API eagle_status_t eagle_tree_build(const int32_t* parents, const int32_t* kv_len, int B, int N,
                                uint64_t* anc, int32_t* depth, int32_t* pos,
                                int32_t* seq_flags, void* stream);

/*
 * Workspace bytes eagle_tree_attn needs for this shape (a function of the
 * shape alone, so it can be sized once per model).
 */
EAGLE_API size_t eagle_tree_attn_workspace(int B, int N, int Hq, int Hkv, int d, int Lmax);

/*
 * Tree attention: every draft node against the committed KV cache and its
 * own ancestors, in one pass (EAGLE, paperlayer.ai summary, §2 Preliminaries
 * and §3 EAGLE: the target verifies the whole tree in a single forward).
 *
 * For sequence b, node i, query head h (KV head g = h * Hkv / Hq):
 *   keys  J = {0 .. L-1} U {L + j : bit j of anc[b, i]},  L = kv_len[b]
 *   out[b, i, h] = sum_{k in J} softmax_k(sm_scale * q.K[g, k]) V[g, k]
 *
 *   q        device [B, N, Hq, d] bf16
 *   k_cache  device [B, Hkv, Lmax, d] bf16; slots [L, L+N) hold the tree's
 *   v_cache           own keys/values (written by the caller)
 *   kv_len   device [B] int32; needs 0 <= L and L + N <= Lmax
 *   anc      device [B, N] uint64 from eagle_tree_build
 *   sm_scale softmax scale; <= 0 selects 1/sqrt(d)
 *   out      device [B, N, Hq, d] bf16 (round to nearest even); fp32 inside
 *   workspace device, eagle_tree_attn_workspace() bytes (per-head tickets
 *            and split partials; zero before its first use, left with zero
 *            tickets; calls that overlap must not share it; 0 bytes when no
 *            split is needed)
 *   seq_flags device [B] int32 or NULL (EAGLE_FLAG_BAD_KV_LEN; that
 *            sequence's output is zero)
 * Supported: d in {64, 128}; Hq % Hkv == 0; 1 <= N <= 64; Lmax >= N.
 */
EAGLE_API eagle_status_t eagle_tree_attn(const uint16_t* q, const uint16_t* k_cache, const uint16_t* v_cache,
                               const int32_t* kv_len, const uint64_t* anc,
                               int B, int N, int Hq, int Hkv, int d, int Lmax, float sm_scale,
                               uint16_t* out, void* workspace, size_t workspace_bytes,
                               int32_t* seq_flags, void* stream);

/*
 * Tree mask builder and tree attention in one launch (EAGLE, paperlayer.ai
 * summary, A.1 Tree Structure and §3 EAGLE: the mask follows the tree's
 * parent links).  Computes what eagle_tree_build followed by eagle_tree_attn
 * computes: the kernel derives every node's ancestor set from `parents`
 * itself, so `out` is bit-identical to eagle_tree_attn with the masks that
 * eagle_tree_build returns for the same parents.
 *
 *   parents  device [B, N] int32 (root parent -1, 0 <= parents[i] < i,
 *            or -1 for an absent node)
 *   anc, depth, pos  device [B, N] out or NULL each: the builder's outputs,
 *            as eagle_tree_build defines them (pos = kv_len + depth), written
 *            once per sequence by the kernel
 *   seq_flags device [B] int32 or NULL (EAGLE_FLAG_BAD_KV_LEN as
 *            eagle_tree_attn, EAGLE_FLAG_BAD_PARENT as eagle_tree_build; a
 *            bad link is treated as the root)
 * Every other argument, the workspace (eagle_tree_attn_workspace bytes) and
 * the supported shapes are those of eagle_tree_attn.
 */
EAGLE_API eagle_status_t eagle_tree_attn_parents(const uint16_t* q, const uint16_t* k_cache,
                               const uint16_t* v_cache, const int32_t* kv_len,
                               const int32_t* parents, int B, int N, int Hq, int Hkv, int d,
                               int Lmax, float sm_scale, uint16_t* out, uint64_t* anc,
                               int32_t* depth, int32_t* pos, void* workspace,
                               size_t workspace_bytes, int32_t* seq_flags, void* stream);

/*
 * eagle_tree_attn_parents without a workspace argument, for callers that
 * cannot allocate device memory: code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc.  Same arguments (minus workspace),
 * same kernels and bit-identical results.  The scratch the kernels need
 * (piece tickets or piece table, split partials) lives in a static device
 * array of the library, 64 MiB per GPU, held by each GPU the library runs on
 * until the process ends; no hipMalloc, hipFree or other allocation happens
 * on any call.  The first call on a device looks the array's address up
 * (hipGetSymbolAddress); each call that needs the tickets clears them with a
 * small fill kernel on `stream` (no memset node).  A shape whose scratch
 * would exceed 64 MiB (eagle_tree_attn_workspace above 67108864) returns
 * EAGLE_ERR_UNSUPPORTED before anything is enqueued.  All calls on one GPU
 * share the array: calls that overlap on that GPU (other streams or threads)
 * race and must be serialised by the caller.
 */
EAGLE_API eagle_status_t eagle_tree_attn_parents_noalloc(const uint16_t* q, const uint16_t* k_cache,
                               const uint16_t* v_cache, const int32_t* kv_len,
                               const int32_t* parents, int B, int N, int Hq, int Hkv, int d,
                               int Lmax, float sm_scale, uint16_t* out, uint64_t* anc,
                               int32_t* depth, int32_t* pos, int32_t* seq_flags, void* stream);

/* Workspace bytes eagle_verify_accept needs for this shape. */
EAGLE_API size_t eagle_verify_accept_workspace(int B, int N, int V);

/*
 * Acceptance walk over the draft tree (multi-round speculative sampling:
 * EAGLE, paperlayer.ai summary, §2 Preliminaries and A.2; Algorithm 1's
 * inputs are the target distribution, the candidates and their draft
 * distributions, B Detailed results).
 *
 * Target distribution of node i: p_i = softmax(target_logits[b, i] / T) for
 * T > 0, one-hot of its argmax (lowest id on ties) for T = 0.  Starting at
 * the root, the candidates c of the current node j are tested in ascending
 * node order against the current distribution r (initially p_j):
 *   T > 0: ratio = r(t_c) / q_c(t_c); accept iff uniforms[b, c] < ratio
 *          (ratio = +inf if q_c(t_c) = 0 < r(t_c)); on rejection
 *          r <- norm(max(0, r - q_c)) (kept unchanged if that has no mass)
 *   T = 0: accept iff t_c == argmax p_j
 * On acceptance the walk descends to c; when a node has no candidate left
 * the final token is drawn from r by inverse CDF with uniforms[b, 0]
 * (T = 0: the argmax).
 *
 *   draft_tokens  device [B, N] int32; [b, 0] is the root token (not tested)
 *   draft_probs   device [B, N, V] fp32 draft distributions; may be NULL when
 *                 T == 0
 *   draft_row     device [B, N] int32 or NULL: node i's token was drawn from
 *                 row draft_row[b, i] of draft_probs[b] (0 <= row < N).  NULL
 *                 means row i (each node its own row; row 0 unused).  Siblings
 *                 drawn i.i.d. from their parent's draft distribution name the
 *                 same row (e.g. draft_row = parents, with row j holding the
 *                 draft distribution after node j), and a node whose
 *                 candidates all name one row is evaluated in closed form: each
 *                 rejection costs one pass over the two rows in registers and
 *                 no row is re-read.  A row outside [0, N) on a tested node sets
 *                 EAGLE_FLAG_BAD_ROW and that node's own row is used instead.
 *   target_logits device [B, N, V] fp32; row i = target logits after node i
 *   parents       device [B, N] int32
 *   kv_len        device [B] int32 (for kv_src_slots)
 *   temperature   >= 0, finite
 *   uniforms      device [B, N] fp32 in [0, 1)
 * Outputs (device):
 *   accept_len      [B]    m = accepted draft nodes (root and final token excluded)
 *   path            [B, N] accepted node ids, path[b, 0] = 0; -1 after m
 *   accepted_tokens [B, N] draft_tokens of path[1..m]; -1 after m - 1
 *   bonus_token     [B]    the final token drawn at the last accepted node
 *   kv_src_slots    [B, N] kv_len[b] + path[b, j] for j <= m; -1 after
 *   out_probs       [B, N, V] or NULL: p_i for every node (parity checks)
 *   out_final_dist  [B, V] or NULL: the distribution the final token came from
 *   out_ratio       [B, N] or NULL: ratio used for each tested node, NaN for
 *                   untested ones (T = 0: 1 for a match, 0 otherwise)
 *   seq_flags       [B] int32 or NULL (BAD_TOKEN, BAD_ROW, NONFINITE)
 *   workspace       device, eagle_verify_accept_workspace() bytes: per-sequence
 *                   and per-node tickets and maxima, which must be zero before
 *                   the first call (eagle_workspace_clear) and are left zero by
 *                   every call, and per-node scratch; calls that overlap must
 *                   not share it
 * Supported: 1 <= V <= 32768; 1 <= N <= 64.
 * No workgroup waits for another (the nodes of a sequence meet only at an
 * atomic ticket), so the results never depend on how many run at once.  At
 * T = 0 without out_* buffers and V > 4096 each row's argmax is split over
 * several workgroups; results are identical to the unsplit argmax.
 */
EAGLE_API eagle_status_t eagle_verify_accept(const int32_t* draft_tokens, const float* draft_probs,
                                   const int32_t* draft_row,
                                   const float* target_logits, const int32_t* parents,
                                   const int32_t* kv_len, int B, int N, int V, float temperature,
                                   const float* uniforms,
                                   int32_t* accept_len, int32_t* path, int32_t* accepted_tokens,
                                   int32_t* bonus_token, int32_t* kv_src_slots,
                                   float* out_probs, float* out_final_dist, float* out_ratio,
                                   void* workspace, size_t workspace_bytes,
                                   int32_t* seq_flags, void* stream);

/*
 * eagle_verify_accept followed by eagle_kv_compact on the result, in one
 * launch: the workgroup that walks a sequence's tree also moves the K/V of
 * its accepted path (EAGLE, paperlayer.ai summary, §2 Preliminaries and A.2
 * for the walk; §3 EAGLE: accepted tokens are recorded for the next round).
 * Outputs and effects are exactly those of the two calls in sequence with
 * the same arguments (no out_probs / out_final_dist / out_ratio here); the
 * cache, Hkv, d, Lmax, new_kv_len and their rules are those of
 * eagle_kv_compact, the rest those of eagle_verify_accept (same workspace).
 * A kv_len out of range sets EAGLE_FLAG_BAD_KV_LEN and leaves that
 * sequence's cache unchanged (new_kv_len = kv_len).
 */
EAGLE_API eagle_status_t eagle_verify_accept_compact(
    const int32_t* draft_tokens, const float* draft_probs, const int32_t* draft_row,
    const float* target_logits,
    const int32_t* parents, const int32_t* kv_len, int B, int N, int V, float temperature,
    const float* uniforms, int32_t* accept_len, int32_t* path, int32_t* accepted_tokens,
    int32_t* bonus_token, int32_t* kv_src_slots, uint16_t* k_cache, uint16_t* v_cache, int Hkv,
    int d, int Lmax, int32_t* new_kv_len, void* workspace, size_t workspace_bytes,
    int32_t* seq_flags, void* stream);

/*
 * KV compaction: record the accepted path in the cache (EAGLE, paperlayer.ai
 * summary, §3 EAGLE: accepted tokens are recorded for the next round).  For
 * every sequence b, KV head and j = 0..accept_len[b], slot kv_len[b] + j of
 * k_cache and v_cache takes the contents of slot kv_src_slots[b, j]
 * (in place); new_kv_len[b] = kv_len[b] + accept_len[b] + 1.
 *
 *   k_cache, v_cache device [B, Hkv, Lmax, d] bf16, updated in place
 *   kv_len, kv_src_slots, accept_len: device, as produced above; source
 *            slots must satisfy kv_len + j <= src < Lmax and increase with j
 *            (true for every path the walk emits); others set
 *            EAGLE_FLAG_BAD_KV_LEN and leave that sequence unchanged
 *   new_kv_len device [B] int32 out; must not alias kv_len
 * Supported: d in {64, 128}; 1 <= N <= 64.
 */
EAGLE_API eagle_status_t eagle_kv_compact(uint16_t* k_cache, uint16_t* v_cache, const int32_t* kv_len,
                                const int32_t* kv_src_slots, const int32_t* accept_len,
                                int B, int N, int Hkv, int d, int Lmax,
                                int32_t* new_kv_len, int32_t* seq_flags, void* stream);

/*
 * Feature gather: the features of the accepted path, in path order, for the
 * next round's draft (EAGLE, paperlayer.ai summary, §3 EAGLE: the accepted
 * tokens and their features are recorded, and the draft head extrapolates
 * from the target's features).  For every sequence b and j = 0..accept_len[b],
 * row j of out takes row path[b, j] of features; rows of out past
 * accept_len[b] are not written.
 *
 *   features device [B, N, row_bytes], one row per tree node in node order
 *            (e.g. the target's last hidden state of every node); rows are
 *            copied as bytes, so any element type works
 *   path, accept_len device [B, N] / [B] int32 as eagle_verify_accept emits
 *            them: path[b, 0] = 0 and path[b, j] increasing and below N for
 *            j <= accept_len[b] < N; a sequence that breaks this sets
 *            EAGLE_FLAG_BAD_PATH and has no row written
 *   row_bytes bytes per row: a positive multiple of 16, N * row_bytes < 2^35
 *   out      device [B, N, row_bytes]; must not overlap features
 *   seq_flags device [B] int32 or NULL
 * Errors: EAGLE_ERR_INVALID_ARGUMENT for a bad size, NULL pointer or
 * overlapping buffers; nothing is enqueued then.
 * Supported: 1 <= N <= 64.
 */
EAGLE_API eagle_status_t eagle_feature_gather(const void* features, const int32_t* path,
                                              const int32_t* accept_len, int B, int N,
                                              int64_t row_bytes, void* out, int32_t* seq_flags,
                                              void* stream);

/*
 * EAGLE-2 dynamic draft tree (EAGLE-2 overview blog, §1 and §4 EAGLE vs
 * EAGLE-2): the tree grows layer by layer from the draft model's
 * confidences.  A node's value is the product of the draft probabilities
 * along its path; each layer expands the k most valuable nodes of the layer
 * before into their k most probable next tokens, and a final rerank keeps
 * the N most valuable nodes (the root always) as the tree to verify.
 *
 * The created nodes of a sequence live in caller-owned device arrays of T
 * entries each: created_parent [B, T] int32, created_token [B, T] int32,
 * created_value [B, T] fp32.  Node 0 is the root (parent -1, value 1, token
 * = the last committed token, written by the caller); nodes are numbered in
 * creation order.  A driver runs: expand the root (R = 1), then per layer
 * select the layer's k best, run the draft model on them, expand them; then
 * rerank.  Values are fp32 products, ties go to the lower token id
 * (expansion) or node id (selection, rerank).  Asynchronous on `stream`;
 * argument errors return before anything is enqueued.
 */

/*
 * Expansion: for sequence b and row r < R, the k tokens with the largest
 * q[b, r, :] (ties: lower token id) become created nodes base + r*k + j,
 * j = 0..k-1 in decreasing probability, with parent parent_node[b, r], that
 * token, and value parent_value[b, r] * q[b, r, token].
 *   q device [B, R, V] fp32 draft distributions (finite), V <= 32768
 *   parent_node, parent_value device [B, R]
 *   1 <= k <= min(V, 64), base + R * k <= T
 */
EAGLE_API eagle_status_t eagle_dtree_expand(const float* q, int B, int R, int V, int k,
                                       const int32_t* parent_node, const float* parent_value,
                                       int32_t* created_parent, int32_t* created_token,
                                       float* created_value, int T, int base, void* stream);

/*
 * Selection: out_node[b, 0..k-1] = the k created nodes among ids
 * [first, first + M) with the largest value (ties: lower id), most valuable
 * first; out_value their values.  1 <= k <= M <= 2048, first + M <= T.
 */
EAGLE_API eagle_status_t eagle_dtree_select(const float* created_value, int B, int T, int first, int M,
                                       int k, int32_t* out_node, float* out_value, void* stream);

/*
 * Rerank: keep node 0 and the N - 1 nodes of ids [1, T_used) with the
 * largest value (ties: lower id), renumbered in creation order (so parents
 * precede children and shallower nodes come first).  Writes parents [B, N]
 * (new numbering, parents[b, 0] = -1), tokens [B, N] and kept_node [B, N]
 * (each kept node's created id, to gather its draft row or features).  A
 * kept node whose parent was not kept (impossible when values never grow
 * down a path) is hung off the root and sets EAGLE_FLAG_BAD_PARENT in
 * seq_flags (device [B] int32 or NULL).  1 <= N <= 64, N <= T_used <= T,
 * T_used <= 2049.
 */
EAGLE_API eagle_status_t eagle_dtree_rerank(const int32_t* created_parent, const int32_t* created_token,
                                       const float* created_value, int B, int T, int T_used,
                                       int N, int32_t* parents, int32_t* tokens,
                                       int32_t* kept_node, int32_t* seq_flags, void* stream);

/*
 * Testing hook, not for production use: forces the attention kernel and the
 * work split of every later eagle_tree_attn / eagle_tree_attn_parents call
 * and workspace query in this process, so that tests can run each kernel and
 * piece count on the same inputs.  kernel: 0 = the planner's choice, 1 = the
 * ring kernel (at most 32 query rows per KV head; larger shapes then return
 * EAGLE_ERR_UNSUPPORTED), 2 = the group kernel.  pieces_per_unit: 0 = the
 * planner's choice, else the number of key ranges per (sequence, KV head) at
 * full cache length, 1..1024 (sequences shorter than the cache get fewer).
 * Results are the same for every setting up to the rounding of the split
 * merge.  Not thread-safe: set it while no attention call is being made.
 * Returns EAGLE_ERR_INVALID_ARGUMENT for values out of range.
 */
EAGLE_API eagle_status_t eagle_testing_attn_plan(int kernel, int pieces_per_unit);

/*
 * Measurement only (the roofline's context): reads `bytes` of device memory
 * at `src` with the ring attention kernel's load structure and nothing else:
 * `workgroups` workgroups of 512 threads, workgroup w reading its contiguous
 * share bytes / workgroups (the remainder is not read) in 16 KB chunks, one
 * chunk in flight per wave.  Its time is the floor of the attention's stream
 * at that size and workgroup count.  sink: device, workgroups * 512 uint32
 * written (the XOR of what each thread read).  Asynchronous on `stream`.
 * EAGLE_ERR_INVALID_ARGUMENT for NULL pointers, workgroups outside
 * [1, 65535], fewer than 16 or more than 2^31 - 1 bytes per workgroup.
 */
EAGLE_API eagle_status_t eagle_testing_read_floor(const void* src, size_t bytes, int workgroups,
                                                  uint32_t* sink, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* EAGLE_VERIFY_H */
