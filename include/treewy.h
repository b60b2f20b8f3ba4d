/*
 * treewy.h -- C ABI of the TreeWY verify/commit path on MI355X (gfx950).
 *
 * Method: "TreeWY: Speculative Verification for Gated DeltaNet Hybrids"
 * (arXiv 2608.20961).  A Gated DeltaNet head keeps a state S in R^{dv x dk} that
 * follows the gated delta rule (Eq. 1, §1):
 *     S_t = a_t S_{t-1} (I - b_t k_t k_t^T) + b_t v_t k_t^T,    o_t = S_t q_t.
 * A draft tree of N nodes hangs off the committed state S0; node t's "previous
 * state" is its parent's (§3 "Verifying a draft").
 *
 * Conventions shared by every call
 *   d = dk = dv = 128 (fixed).  1 <= N <= 64.  B >= 1, 1 <= H <= 65536.
 *   All pointers are DEVICE pointers owned by the caller; the library never
 *   allocates, frees or retains them.  Between calls it keeps only each device's
 *   compute-unit count, queried once (and, for the one entry point that takes no
 *   workspace, the address of its fixed device array; see below).
 *   Layouts are dense and C-contiguous:
 *     S0, S   [B, H, 128, 128] float32, row v contiguous over k (S[v][k])
 *     Q, K    [B, N, H, 128]   element type given by in_dtype
 *     V       [B, N, H, 128]   element type given by in_dtype
 *     alpha, beta, gamma [B, N, H] float32
 *     O, U    [B, N, H, 128]   float32
 *     parent  [B, N] int32: parent[b][t] in [-1, t-1]; -1 = child of S0.  Several
 *             children of S0 are allowed.  Any topological numbering works (DFS
 *             pre-order, as in the paper, is one).
 *     accepted [B] int32: accepted node in [-1, N-1]; -1 = nothing accepted.
 *     Snap    [B, H, N, 128, 128] float32 (one full state per draft node).
 *   in_dtype: TREEWY_F32 (float) or TREEWY_BF16 (bfloat16 bit patterns, uint16).
 *   stream: a hipStream_t (NULL = the default stream).  Every call only enqueues
 *   work on it and returns without synchronising; no call reads device data on the
 *   host, so every call can be captured into a HIP graph.
 *
 * Errors
 *   The return value reports what the host can check: TREEWY_EINVAL for a null
 *   required pointer, N outside [1, 64], B < 1, H outside [1, 65536], an unknown in_dtype, or sizes
 *   whose element counts overflow; TREEWY_EHIP when the launch fails.  Nothing is
 *   enqueued when the return value is not TREEWY_OK.
 *   What only the device can see is written to the optional device word `status`
 *   (first error wins; the caller zeroes it beforehand): TREEWY_ETREE for a parent
 *   outside [-1, t-1], TREEWY_EACCEPT for an accepted node outside [-1, N-1].  The
 *   outputs of an offending sequence are then unspecified; other sequences are
 *   computed normally, and no access leaves the documented buffers.
 *
 * Thread safety: calls are re-entrant; calls on different streams may overlap
 * as long as their output buffers do not.
 */
#ifndef TREEWY_H
#define TREEWY_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define TREEWY_VERSION 4

enum {
    TREEWY_OK = 0,
    TREEWY_EINVAL = 1,
    TREEWY_EHIP = 2,
    TREEWY_ETREE = 3,
    TREEWY_EACCEPT = 4,
    TREEWY_ELOG = 5,
    TREEWY_ECTX = 6,
    TREEWY_ESCRATCH = 7
};

/* Size of the fixed device array behind treewy_tree_attention_noalloc (48 MiB per GPU). */
#define TREEWY_NOALLOC_SCRATCH_BYTES ((size_t)48 << 20)

enum { TREEWY_F32 = 0, TREEWY_BF16 = 1 };

/*
 * Tree verification (paper §3, "Verifying a draft", Eq. 2, and its readout).
 * For every (sequence b, head h) computes, for all N draft nodes t:
 *   gamma[t] = g_t, the product of alpha over t and all its ancestors;
 *   U[t]     = the pseudo-value vt~_t = b_t (v_t - a_t S_parent(t) k_t) (§3 "Key rewrite"),
 *              obtained from the unit lower-triangular system
 *              (I + diag(b) G) U = R,  G[t,i] = (g_t/g_i)(k_t . k_i) for strict ancestors i,
 *              R[t] = b_t v_t - b_t g_t S0 k_t;
 *   O[t]     = S_t q_t = g_t S0 q_t + sum over i ancestor-or-self of t of (g_t/g_i)(k_i . q_t) U[i].
 * Optional outputs (NULL to skip): anc_out [B, N] uint64 with bit i set for every
 * ancestor-or-self i of t; depth_out [B, N] int32 with depth 1 for children of S0.
 * S0 is only read.
 */
int treewy_verify(const float* S0, const void* Q, const void* K, const void* V,
                  const float* alpha, const float* beta, const int32_t* parent,
                  int B, int H, int N, int in_dtype,
                  float* O, float* U, float* gamma,
                  uint64_t* anc_out, int32_t* depth_out, int32_t* status, void* stream);

/*
 * Commit (paper §3, "Reconstruct on commit", Eq. 3).  In place, for every sequence b
 * with a = accepted[b] >= 0 and every head h:
 *   S <- g_a S + sum over i ancestor-or-self of a of (g_a/g_i) U[i] k_i^T,
 * i.e. the state after node a, which becomes the next committed state.  a = -1 leaves
 * S untouched (not read, not written).  U and gamma are treewy_verify's outputs for the
 * same S, K and tree; K's element type is in_dtype.
 */
int treewy_commit(float* S, const float* U, const void* K, const float* gamma,
                  const int32_t* parent, const int32_t* accepted,
                  int B, int H, int N, int in_dtype, int32_t* status, void* stream);

/*
 * The previous step's commit fused into this step's verify (paper §4 "Implementation":
 * on chains verify and commit run as one fused kernel; its Conclusion names fusion for
 * trees as the next step).  Equivalent to
 *     treewy_commit(S, U_prev, K_prev, gamma_prev, parent_prev, accepted_prev,
 *                   B, H, N_prev, in_dtype, status, stream);
 *     treewy_verify(S, Q, K, V, alpha, beta, parent, B, H, N, in_dtype,
 *                   O, U, gamma, anc_out, depth_out, status, stream);
 * but it runs as one kernel that reads and writes each state once: the committed rows are
 * formed on the way into the contractions (bf16 and fp32 inputs alike).
 *   S                     [B, H, 128, 128] float32, in place: in, the state before the
 *                         previous step's commit; out, the committed state (the state this
 *                         step verified against).  Rows of sequences with
 *                         accepted_prev[b] = -1 are not written.
 *   U_prev, K_prev, gamma_prev, parent_prev, accepted_prev
 *                         the previous step's U, keys, gamma, tree and accepted node, laid
 *                         out with N_prev nodes (1 <= N_prev <= 64); K_prev has in_dtype.
 *   Q, K, V, alpha, beta, parent, O, U, gamma, anc_out, depth_out
 *                         this step's, as in treewy_verify, with N nodes.
 * O, U and gamma must not overlap U_prev, K_prev or gamma_prev (TREEWY_EINVAL when they do):
 * keep two sets of per-step buffers and alternate.  Device-side errors of either step go to
 * `status`; a sequence whose previous accepted node or path is invalid keeps its S.
 */
int treewy_commit_verify(float* S, const float* U_prev, const void* K_prev,
                         const float* gamma_prev, const int32_t* parent_prev,
                         const int32_t* accepted_prev, int N_prev,
                         const void* Q, const void* K, const void* V,
                         const float* alpha, const float* beta, const int32_t* parent,
                         int B, int H, int N, int in_dtype,
                         float* O, float* U, float* gamma,
                         uint64_t* anc_out, int32_t* depth_out, int32_t* status, void* stream);

/*
 * The commit deferred into a log (the deferred state writes the paper's Conclusion names as
 * a next step; §3 "Reconstruct on commit", Eq. 3, for what a commit adds).  Between writes,
 * each (sequence b, head h) keeps its committed state as
 *     S_committed = scale[b][h] * (S[b][h] + sum over j < len[b] of logU[b][h][j] logK[b][h][j]^T),
 * with at most Lmax (1..16) rank-one terms.  One call does the work of
 * treewy_commit_verify: it folds the previous step's commit into that representation and
 * verifies this step's tree against the committed state.  When the log can take the accepted
 * path's terms they are appended (u~ = (g_a/g_i) U_prev[i] / new scale) and S is not written;
 * otherwise the committed state is written to S and the log is emptied.  The log can take them
 * when, for N <= 16, len + depth(a) <= Lmax and depth(a) is small enough to stage (4 for
 * N <= 4, else 8); for 16 < N <= 48, when len + depth(a) <= Lmax; for 48 < N <= 64, when
 * len + depth(a) <= min(Lmax, 8) (the log's and the path's rows share one staged chunk of
 * 16 terms up to 48 nodes, of 8 above; a longer list, on a step that writes S, is fetched
 * chunk by chunk).
 *   S                       [B, H, 128, 128] float32, in place (written only when emptying)
 *   logU                    [B, H, Lmax, 128] float32 (rows past len are ignored)
 *   logK                    [B, H, Lmax, 128] bfloat16
 *   scale_in, scale_out     [B, H] float32 } the log header before and after this step.  They
 *   len_in, len_out         [B] int32      } must not overlap; alternate them between steps.
 *                           A fresh log is len 0, scale 1 (S is then the committed state).
 *   the rest                as treewy_commit_verify.
 * Only bf16 inputs are supported (TREEWY_EINVAL otherwise), N up to 64.  A header length
 * outside [0, Lmax] is reported as TREEWY_ELOG on `status` and clamped.
 */
int treewy_commit_verify_deferred(float* S, float* logU, void* logK,
                                  const float* scale_in, float* scale_out,
                                  const int32_t* len_in, int32_t* len_out, int Lmax,
                                  const float* U_prev, const void* K_prev,
                                  const float* gamma_prev, const int32_t* parent_prev,
                                  const int32_t* accepted_prev, int N_prev,
                                  const void* Q, const void* K, const void* V,
                                  const float* alpha, const float* beta, const int32_t* parent,
                                  int B, int H, int N, int in_dtype,
                                  float* O, float* U, float* gamma,
                                  uint64_t* anc_out, int32_t* depth_out, int32_t* status,
                                  void* stream);

/*
 * Writes the committed state a deferred-commit log stands for into S (S <- scale (S + sum of
 * the logged terms)) and empties the log into the output header (scale 1, length 0).  Used
 * before the state is read by anything else (another kernel, a checkpoint).  Arguments as in
 * treewy_commit_verify_deferred; in_dtype must be TREEWY_BF16.
 */
int treewy_deferred_flush(float* S, const float* logU, const void* logK,
                          const float* scale_in, float* scale_out,
                          const int32_t* len_in, int32_t* len_out, int Lmax,
                          int B, int H, int in_dtype, int32_t* status, void* stream);

/*
 * Full-state snapshotting, the comparison scheme of the paper's §2 ("full-state
 * snapshotting", store-all): every node's state S_t = Eq. (1) applied to its parent's
 * state is materialised in Snap[b][h][t], and O[t] = S_t q_t.  S0 is only read.
 */
int treewy_verify_snapshot(const float* S0, const void* Q, const void* K, const void* V,
                           const float* alpha, const float* beta, const int32_t* parent,
                           int B, int H, int N, int in_dtype,
                           float* O, float* Snap, int32_t* status, void* stream);

/*
 * Store-all rollback (paper §2): S[b][h] <- Snap[b][h][accepted[b]] for every sequence
 * with accepted[b] >= 0; a = -1 leaves S untouched.
 */
int treewy_commit_snapshot(float* S, const float* Snap, const int32_t* accepted,
                           int B, int H, int N, int32_t* status, void* stream);

/*
 * Tree-aware softmax-attention verify: the softmax layers' half of a tree verify pass (the
 * technical review "TreeWY: Removing the Memory Wall in Speculative Decoding for Gated
 * DeltaNet Hybrids", §2.3 "KV cache attention", Eq. (2); tree-structured drafting, §2.2).
 * For every sequence b, draft node t and query head hq:
 *   O[b][t][hq] = softmax(q K^T / 16) V,  q = Qd[b][t][hq],
 * over the keys/values of head hq / G: the committed cache rows 0 .. ctx[b]-1 followed by the
 * draft tokens that are ancestors-or-self of t (the GDN path's ancestor sets).
 * Head dimension 256 (the modelled softmax layers', paper §2), bf16 inputs only.
 *   Kc, Vc   [B, Hkv, T_max, 256] bf16   committed cache (rows >= ctx[b] are never read)
 *   ctx      [B] int32                  committed lengths, 0 <= ctx[b] <= T_max
 *   Qd       [B, N, Hkv*G, 256] bf16    draft queries (query head hq reads KV head hq / G)
 *   Kd, Vd   [B, N, Hkv, 256] bf16      draft keys and values
 *   parent   [B, N] int32               the draft tree, as for treewy_verify
 *   O        [B, N, Hkv*G, 256] float32
 *   workspace  device scratch of at least treewy_tree_attention_workspace(B, Hkv, G, N, T_max)
 *              bytes, owned by the caller; contents need no initialisation and are not kept.
 * 1 <= N <= 64, B, Hkv, G >= 1.  TREEWY_EINVAL for bad sizes or a short workspace; on
 * `status`: TREEWY_ETREE for a malformed parent, TREEWY_ECTX for ctx outside [0, T_max].
 */
int treewy_tree_attention(const void* Kc, const void* Vc, const int32_t* ctx, int T_max,
                          const void* Qd, const void* Kd, const void* Vd,
                          const int32_t* parent, int B, int Hkv, int G, int N, float* O,
                          void* workspace, size_t workspace_bytes, int32_t* status,
                          void* stream);

/* Bytes of workspace treewy_tree_attention needs for these sizes (0 for invalid sizes). */
size_t treewy_tree_attention_workspace(int B, int Hkv, int G, int N, int T_max);

/*
 * treewy_tree_attention without a workspace argument, for callers that cannot allocate
 * (code under HIP graph capture, tight serving loops, harnesses that forbid allocation): the
 * split partials go to a fixed device array of TREEWY_NOALLOC_SCRATCH_BYTES that the library
 * holds on each GPU it runs on until the process ends.  Arguments, results and `status` are
 * those of treewy_tree_attention.  This call allocates nothing: on its first call on a device
 * it looks up that device's array once.  Returns TREEWY_ESCRATCH (nothing enqueued) when
 * treewy_tree_attention_workspace(B, Hkv, G, N, T_max) exceeds the array.
 * Every call on one GPU shares that GPU's array: calls whose executions overlap on one GPU
 * (different streams, different host threads) race on it and their outputs are undefined;
 * serialise them (one stream, or events).  The array's contents are not kept between calls
 * and need no initialisation.
 */
int treewy_tree_attention_noalloc(const void* Kc, const void* Vc, const int32_t* ctx, int T_max,
                                  const void* Qd, const void* Kd, const void* Vd,
                                  const int32_t* parent, int B, int Hkv, int G, int N, float* O,
                                  int32_t* status, void* stream);

/*
 * Cache commit of the softmax layers: the accepted node's root-to-node path (keys and values
 * of every KV head) is appended after each sequence's committed rows, rejected branches are
 * dropped (review page §2.3: rejected drafts are discarded, no recomputation), and
 * ctx_out[b] = ctx_in[b] + depth(accepted[b]).  accepted[b] = -1 appends nothing.
 * ctx_in and ctx_out must not overlap.  On `status`: TREEWY_EACCEPT, TREEWY_ETREE, and
 * TREEWY_ECTX when the path would not fit in T_max rows (that sequence is left unchanged).
 */
int treewy_kv_commit(void* Kc, void* Vc, const int32_t* ctx_in, int32_t* ctx_out, int T_max,
                     const void* Kd, const void* Vd, const int32_t* parent,
                     const int32_t* accepted, int B, int Hkv, int N, int32_t* status,
                     void* stream);

/* Static, NUL-terminated description of an error code (never NULL). */
const char* treewy_strerror(int code);

/* TREEWY_VERSION of the built library. */
int treewy_version(void);

#ifdef __cplusplus
}
#endif

#endif /* TREEWY_H */
