/*
 * reformer_lsh.h -- C ABI of the shared-QK LSH self-attention forward pass
 * for AMD MI355X (gfx950).
 *
 * The operation is the Reformer's LSH attention as summarised on the page
 * "Reformer: The Efficient Transformer" (research summary):
 *   - Summary: queries and keys come from one shared projection, are hashed
 *     with random rotations, sorted by bucket, and attention runs only inside
 *     small fixed-size chunks; several hash rounds are combined.
 *   - Key points, LSH attention bullet: h(x) = argmax([xR; -xR]) for a random
 *     matrix R; once sorted, the positions are cut into chunks of m and a
 *     chunk's queries see the keys of that chunk and of the one preceding it.
 *   - Key points, Shared-QK bullet: a position's own key is excluded from
 *     its window; it is used only when nothing else is left to attend to.
 *
 * Readings taken where the page is silent (each one is also what the test
 * oracle implements):
 *   - rotations are float32 [n_rounds, d_head, n_buckets/2], one matrix per
 *     round shared by every batch row and head; bucket k < b/2 is +(xR)_k and
 *     bucket b/2 + k is -(xR)_k; argmax ties go to the lowest bucket index;
 *     n_buckets == 1 puts every position in bucket 0 (rotations unused).
 *   - the sort is stable: key (bucket, original position) within each
 *     (batch, head, round).
 *   - chunk length m' = min(chunk_len, seq_len), seq_len a multiple of m';
 *     chunk 0 of a round has no predecessor.  Every key of the window is
 *     eligible (no same-bucket mask).  Score s_ij = x_i . x_j / sqrt(d_head).
 *   - causal (optional): key j is allowed for query i only if j < i in the
 *     original order.
 *   - a round in which a position has no valid non-self key contributes
 *     nothing; if no round has one the output row is the position's own v.
 *   - rounds are combined with logsumexp weights:
 *     out_i = sum_r exp(z_r(i) - Z_i) o_r(i), Z_i = logsumexp_r z_r(i).
 *
 * Conventions for every entry point
 *   - All tensor pointers are DEVICE pointers to contiguous row-major memory,
 *     owned by the caller; qk, v, out, o_rounds and workspace must be 16-byte
 *     aligned (rows move as 16-byte vectors).  The library never allocates or frees device
 *     memory and never synchronises; all work is enqueued in order on
 *     `stream` (0 = the null stream).  Outputs must not alias inputs.
 *   - Layouts: qk, v, out [batch, heads, seq_len, d_head] in `dtype`;
 *     buckets, perm, inv_perm [batch, heads, n_rounds, seq_len] int32;
 *     o_rounds [batch, heads, n_rounds, seq_len, d_head] float32 and
 *     z_rounds [batch, heads, n_rounds, seq_len] float32, both indexed by
 *     ORIGINAL position (not sorted slot).
 *   - Arguments are validated on the host before any HIP call.  Invalid
 *     arguments return RLSH_ERR_INVALID_ARGUMENT, shapes the kernels are not
 *     built for return RLSH_ERR_UNSUPPORTED, a short workspace returns
 *     RLSH_ERR_WORKSPACE_TOO_SMALL, and a failed launch returns RLSH_ERR_HIP;
 *     in every error case nothing was enqueued (launch failures aside) and
 *     reformer_lsh_last_error() describes the problem.  No C++ exception
 *     crosses the ABI.
 *   - Size limits: batch, heads, seq_len, n_rounds >= 1; d_head in {64, 128};
 *     n_buckets == 1 or even, at most 16384; chunk_len >= 1;
 *     batch*heads*n_rounds*seq_len < 2^31.
 */
#ifndef REFORMER_LSH_H
#define REFORMER_LSH_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum rlsh_status {
  RLSH_OK = 0,
  RLSH_ERR_INVALID_ARGUMENT = 1,
  RLSH_ERR_UNSUPPORTED = 2,
  RLSH_ERR_WORKSPACE_TOO_SMALL = 3,
  RLSH_ERR_HIP = 4
} rlsh_status_t;

typedef enum rlsh_dtype {
  RLSH_F32 = 0,  /* float32 qk / v / out */
  RLSH_BF16 = 1  /* bfloat16 qk / v / out, float32 accumulation */
} rlsh_dtype_t;

/* Human-readable name of a status code (static string). */
const char* reformer_lsh_status_string(rlsh_status_t status);

/* Detail of the last error returned on the calling thread ("" if none). */
const char* reformer_lsh_last_error(void);

/* Library version as MAJOR*10000 + MINOR*100 + PATCH. */
int reformer_lsh_version(void);

/* ---------------------------------------------------------------- hash ----
 * Bucket ids h(x) = argmax([xR_r; -xR_r]) for every (batch, head, round,
 * position)  (Key points, LSH attention bullet).
 *
 * qk         [B, H, L, d] in dtype (bf16 values are used exactly).
 * rotations  float32 [n_rounds, d, n_buckets/2]; may be NULL if n_buckets == 1.
 * buckets    int32 [B, H, n_rounds, L], written.
 * workspace  device scratch of at least reformer_lsh_hash_workspace_bytes().
 * n_near_ties (optional, may be NULL) DEVICE pointer to one int32 that
 *            receives the number of (position, round) pairs whose float32
 *            top-two gap was too small to trust and were re-decided in
 *            float64 (diagnostic).
 *
 * Projections are computed approximately -- bf16 MFMA on R rounded to bf16
 * plus an fp6 MFMA pass on the rounding residue (bf16 inputs), float32 FMA
 * (float32 inputs) -- with a rigorous per-token bound tau on the error of a
 * gap between two projections (Cauchy-Schwarz on the operand residues plus
 * float32 accumulation plus the key truncation).  A (position, round) whose
 * leader is within tau of the runner-up is re-decided in float64: between the
 * two leading candidates when every other candidate is provably more than tau
 * below the leader, otherwise over all n_buckets/2 columns.  Bucket ids
 * therefore equal the argmax of exact arithmetic (ties to the lowest bucket)
 * except where the exact top-two gap is below the float64 rounding of a
 * d-term dot product (about 1e-13 of |x| max_j |R_j|).
 */
size_t reformer_lsh_hash_workspace_bytes(int batch, int heads, int seq_len, int d_head,
                                         int n_rounds, int n_buckets);
rlsh_status_t reformer_lsh_hash(const void* qk, rlsh_dtype_t dtype, const float* rotations,
                                int batch, int heads, int seq_len, int d_head, int n_rounds,
                                int n_buckets, int32_t* buckets, int32_t* n_near_ties,
                                void* workspace, size_t workspace_bytes, hipStream_t stream);

/* ------------------------------------------------- hash, no allocation ----
 * For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the same
 * computation and results as reformer_lsh_hash, with the hash scratch in a
 * static device array of RLSH_NOALLOC_SCRATCH_BYTES that the library holds on
 * every GPU it runs on until the process ends.  No workspace argument; the
 * function calls no hipMalloc/hipFree.  Shapes whose scratch
 * (reformer_lsh_hash_workspace_bytes) exceeds the array are rejected with
 * RLSH_ERR_UNSUPPORTED before any launch; 160 MiB holds every shape up to
 * 2^20 positions x 8 rounds at 8192 buckets, d = 64 (110 MiB).
 *
 * All calls on one GPU share that GPU's array: calls that overlap in time on
 * one GPU (different streams, or host threads) race and must be serialised
 * by the caller.  Nothing in the array needs to start at zero.
 */
#define RLSH_NOALLOC_SCRATCH_BYTES (160u * 1024u * 1024u)
rlsh_status_t reformer_lsh_hash_noalloc(const void* qk, rlsh_dtype_t dtype, const float* rotations,
                                        int batch, int heads, int seq_len, int d_head, int n_rounds,
                                        int n_buckets, int32_t* buckets, int32_t* n_near_ties,
                                        hipStream_t stream);

/* ---------------------------------------------------------------- sort ----
 * Stable sort of each (batch, head, round) segment by bucket id; ties keep
 * position order ("Reformer: The Efficient Transformer" research summary,
 * Summary: positions are ordered by their bucket).
 *
 * workspace  device scratch of reformer_lsh_sort_workspace_bytes(...) bytes,
 *            16-byte aligned, caller-owned; no contents need to be set.  The
 *            size is 0 (workspace may be NULL) when one workgroup sorts each
 *            segment (at most 12288 positions and 256 buckets).
 *
 * buckets   int32 [B, H, n_rounds, L], values in [0, n_buckets); a value
 *           outside that range is clamped into it (sorted as 0 or
 *           n_buckets - 1), so the output is always a permutation.
 * perm      int32 [B, H, n_rounds, L], written: perm[.., s] = original
 *           position at sorted slot s.
 * inv_perm  int32 [B, H, n_rounds, L], written: inv_perm[.., perm[.., s]] = s.
 *           May be NULL.
 */
size_t reformer_lsh_sort_workspace_bytes(int batch, int heads, int seq_len, int n_rounds,
                                         int n_buckets);
rlsh_status_t reformer_lsh_sort(const int32_t* buckets, int batch, int heads, int seq_len,
                                int n_rounds, int n_buckets, int32_t* perm, int32_t* inv_perm,
                                void* workspace, size_t workspace_bytes, hipStream_t stream);

/* -------------------------------------------------------- chunk attend ----
 * For every round: gather the sorted rows, let each chunk of m' sorted slots
 * attend to itself and the previous chunk with the self and (optional)
 * causal masks, and write per-position results (Key points, LSH attention
 * and Shared-QK bullets):
 *   z_r(i) = log sum_{j in T_r(i)} exp(s_ij),
 *   o_r(i) = sum_{j in T_r(i)} exp(s_ij - z_r(i)) v_j,
 * or o_r(i) = 0, z_r(i) = -inf when T_r(i) is empty.
 *
 * perm      int32 [B, H, n_rounds, L], a permutation of 0..L-1 per segment
 *           (any permutation is accepted; the sort's output is the usual one).
 * o_rounds  float32 [B, H, n_rounds, L, d], written (position order).
 * z_rounds  float32 [B, H, n_rounds, L], written (position order).
 */
rlsh_status_t reformer_lsh_chunk_attend(const void* qk, const void* v, rlsh_dtype_t dtype,
                                        const int32_t* perm, int batch, int heads, int seq_len,
                                        int d_head, int n_rounds, int chunk_len, int causal,
                                        float* o_rounds, float* z_rounds, hipStream_t stream);

/* ------------------------------------------------------------- combine ----
 * out_i = sum_r exp(z_r(i) - Z_i) o_r(i), Z_i = logsumexp_r z_r(i); rows
 * whose z_r(i) are all -inf get out_i = v_i (self fallback, Shared-QK bullet).
 * out is written in dtype (round to nearest even for bf16).
 */
rlsh_status_t reformer_lsh_combine(const float* o_rounds, const float* z_rounds, const void* v,
                                   rlsh_dtype_t dtype, int batch, int heads, int seq_len,
                                   int d_head, int n_rounds, void* out, hipStream_t stream);

/* -------------------------------------------------------------- attend ----
 * chunk_attend followed by combine, given a permutation.  workspace holds the
 * per-round results: at least reformer_lsh_attend_workspace_bytes().  For
 * bf16 inputs with 64-slot chunks the workspace keeps them compact (o as
 * float16 scaled by a per-row power of two, with the row's log normaliser and
 * scale carried in the lowest mantissa bit of 48 of its values: 10 or 11
 * significant bits); otherwise as float32 (the layout of
 * reformer_lsh_chunk_attend).
 */
size_t reformer_lsh_attend_workspace_bytes(rlsh_dtype_t dtype, int batch, int heads, int seq_len,
                                           int d_head, int n_rounds, int chunk_len);
rlsh_status_t reformer_lsh_attend(const void* qk, const void* v, rlsh_dtype_t dtype,
                                  const int32_t* perm, int batch, int heads, int seq_len,
                                  int d_head, int n_rounds, int chunk_len, int causal, void* out,
                                  void* workspace, size_t workspace_bytes, hipStream_t stream);

/* reformer_lsh_attend that also writes lse: float32 [B, H, L], device memory,
 * 4-byte aligned; lse_i = Z_i = logsumexp_r z_r(i) (natural log), the log of
 * the combined softmax normaliser of position i over every round's targets,
 * -inf on self-fallback rows.  It is what reformer_lsh_attend_backward_lse
 * takes to skip recomputing the normalisers.  A null lse is
 * RLSH_ERR_INVALID_ARGUMENT; everything else as reformer_lsh_attend.
 */
rlsh_status_t reformer_lsh_attend_lse(const void* qk, const void* v, rlsh_dtype_t dtype,
                                      const int32_t* perm, int batch, int heads, int seq_len,
                                      int d_head, int n_rounds, int chunk_len, int causal, void* out,
                                      float* lse, void* workspace, size_t workspace_bytes,
                                      hipStream_t stream);

/* ----------------------------------------------------------- attention ----
 * The whole forward pass: hash -> sort -> chunk attention -> combine and
 * un-sort, out [B, H, L, d] in dtype.  workspace: at least
 * reformer_lsh_workspace_bytes() bytes (it holds buckets, perm, sort and hash
 * scratch and the per-round o/z).
 */
size_t reformer_lsh_workspace_bytes(rlsh_dtype_t dtype, int batch, int heads, int seq_len,
                                    int d_head, int n_rounds, int n_buckets, int chunk_len);
rlsh_status_t reformer_lsh_attention(const void* qk, const void* v, const float* rotations,
                                     rlsh_dtype_t dtype, int batch, int heads, int seq_len,
                                     int d_head, int n_rounds, int n_buckets, int chunk_len,
                                     int causal, void* out, void* workspace,
                                     size_t workspace_bytes, hipStream_t stream);

/* ----------------------------------------------------- instrumentation ----
 * reformer_lsh_attention with hipEventRecord calls at kernel boundaries, for
 * measuring the launches of the real pipeline on the caller's stream.
 * events: RLSH_TIMED_EVENTS caller-created events (hipEventCreate), recorded on
 * `stream` in this order:
 *   0 start            1 after the hash set-up kernels (rotation preparation)
 *   2 after the projection/argmax kernel (which also re-decides its near-ties)
 *   3 the same point as 2 (kept so the event layout is stable)
 *   4 after the sort   5 after chunk attention 6 after the round combine
 * (with n_buckets == 1 events 1..3 are recorded where the hash would run; for
 * bf16 inputs with 64-slot chunks the last round's attention launch does the
 * combine, so event 5 follows rounds 0..r-2 and event 6 the last round).
 * Arguments and errors otherwise as reformer_lsh_attention; a null events
 * array or fewer than RLSH_TIMED_EVENTS entries is RLSH_ERR_INVALID_ARGUMENT.
 */
#define RLSH_TIMED_EVENTS 7
rlsh_status_t reformer_lsh_attention_timed(const void* qk, const void* v, const float* rotations,
                                           rlsh_dtype_t dtype, int batch, int heads, int seq_len,
                                           int d_head, int n_rounds, int n_buckets, int chunk_len,
                                           int causal, void* out, void* workspace,
                                           size_t workspace_bytes, hipEvent_t* events, int n_events,
                                           hipStream_t stream);

/* ------------------------------------------------------------ backward ----
 * Gradients of reformer_lsh_attend (chunk attention + logsumexp combine +
 * self fallback) with respect to qk and v, for a given sorted order.  The
 * bucket ids are piecewise constant in the inputs, so the order is held
 * fixed and gradients flow through the scores and values only (Key points,
 * LSH attention and Shared-QK bullets; the pages give no backward).
 *
 * qk, v, dtype, perm, sizes, chunk_len, causal: as for reformer_lsh_attend;
 *          chunks must be exactly 64 slots (min(chunk_len, L) == 64), else
 *          RLSH_ERR_UNSUPPORTED.
 * out      [B, H, L, d] in dtype: the forward output for these inputs.
 * dout     [B, H, L, d] in dtype: gradient of the loss with respect to out.
 * dqk, dv  [B, H, L, d] float32, written (not accumulated): dqk sums the
 *          query and key roles of each shared vector.
 * workspace: at least reformer_lsh_attend_backward_workspace_bytes() bytes.
 * All pointers device memory, 16-byte aligned; asynchronous on `stream`.
 */
size_t reformer_lsh_attend_backward_workspace_bytes(int batch, int heads, int seq_len, int d_head,
                                                    int n_rounds, int chunk_len);
rlsh_status_t reformer_lsh_attend_backward(const void* qk, const void* v, rlsh_dtype_t dtype,
                                           const int32_t* perm, int batch, int heads, int seq_len,
                                           int d_head, int n_rounds, int chunk_len, int causal,
                                           const void* out, const void* dout, float* dqk, float* dv,
                                           void* workspace, size_t workspace_bytes,
                                           hipStream_t stream);

/* reformer_lsh_attend_backward given the forward's lse (float32 [B, H, L], as
 * written by reformer_lsh_attend_lse for the same inputs and perm): the
 * per-round normaliser pass is skipped.  Same workspace size; a null lse is
 * RLSH_ERR_INVALID_ARGUMENT; everything else as reformer_lsh_attend_backward.
 */
rlsh_status_t reformer_lsh_attend_backward_lse(const void* qk, const void* v, rlsh_dtype_t dtype,
                                               const int32_t* perm, int batch, int heads,
                                               int seq_len, int d_head, int n_rounds, int chunk_len,
                                               int causal, const void* out, const void* dout,
                                               const float* lse, float* dqk, float* dv,
                                               void* workspace, size_t workspace_bytes,
                                               hipStream_t stream);

/* -------------------------------------------------------- feed-forward ----
 * Position-wise feed-forward layer applied to chunk_tokens positions at a time
 * ("Reformer: The Efficient Transformer" (research summary), Summary and Key
 * points, reversible layers bullet: running the feed-forward layers a chunk
 * of positions at a time takes the d_ff-wide activation out of the memory
 * bound without changing any result):
 *   out = relu(x W1^T + b1) W2^T + b2   (the pages name no activation; ReLU)
 *
 * x, out   [n_tokens, d_model] bf16 row-major.
 * w1       [d_ff, d_model] bf16, w2 [d_model, d_ff] bf16 (linear-layer layout).
 * b1 [d_ff], b2 [d_model] float32.
 * chunk_tokens: positions per chunk (0 = all at once); the result does not
 *          depend on it, bit for bit.  The bf16 intermediate of one chunk
 *          ([chunk, d_ff]) lives in the workspace: at least
 *          reformer_lsh_feed_forward_workspace_bytes() bytes.
 * Limits: d_model and d_ff multiples of 128.  All pointers device memory,
 * 16-byte aligned; asynchronous on `stream`.
 */
size_t reformer_lsh_feed_forward_workspace_bytes(int n_tokens, int d_model, int d_ff, int chunk_tokens);
rlsh_status_t reformer_lsh_feed_forward(const void* x, const void* w1, const float* b1, const void* w2,
                                        const float* b2, int n_tokens, int d_model, int d_ff,
                                        int chunk_tokens, void* out, void* workspace,
                                        size_t workspace_bytes, hipStream_t stream);

/* ---------------------------------------------------- local attention ----
 * Local (sliding-chunk) self-attention ("The Reformer - Pushing the limits of
 * language modeling" (summary page), Approach / What changed and Takeaways:
 * chunks of length l_c attend to themselves plus an overlap of preceding and
 * following chunks).
 *
 * q, k, v  [B, H, L, d] row-major in dtype, device memory, 16-byte aligned;
 *          q may alias k (shared projection).
 * Query i in chunk c = i / m', m' = min(chunk_len, L) (L a multiple of m'),
 * attends to the keys j of chunks c - n_before .. c + n_after that exist (no
 * wrap-around), restricted to j <= i when causal != 0, with one softmax of
 * q_i . k_j / sqrt(d) over that window.  There is no self-mask: position i is
 * always in its own window, so every query has a key.
 * out      [B, H, L, d] in dtype (round to nearest even for bf16).
 * Limits: d in {64, 128}; B*H <= 65535; B*H*L < 2^31; n_before, n_after >= 0
 * (values beyond the number of chunks act as "all chunks").
 * No workspace; asynchronous on `stream`.
 */
rlsh_status_t reformer_lsh_local_attention(const void* q, const void* k, const void* v,
                                           rlsh_dtype_t dtype, int batch, int heads, int seq_len,
                                           int d_head, int chunk_len, int n_before, int n_after,
                                           int causal, void* out, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* REFORMER_LSH_H */
