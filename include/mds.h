/*
 * mds.h - C-ABI of the MI355X (gfx950) Markov draft-sampling library (libmds.so).
 *
 * The library runs the hot path of DSpark speculative decoding on one GPU:
 *   1. the sequential Markov draft loop (DSparkSpeculator API page, methods
 *      _sample_markov_chain / _sample_logits; vLLM PR #65007 "vocab-parallel
 *      DSpark Markov sampling", section Part 1), and
 *   2. rejection-sampling verification of the drafts, with optional exact
 *      top-p on the target (PR #65007, Overview and Part 2; PR #63554 Notes
 *      for greedy requests).
 *
 * Conventions for every entry point:
 *   - All array arguments are DEVICE pointers owned by the caller. The library
 *     allocates nothing, never synchronises the device, keeps no pointer after
 *     returning, and enqueues all its work on `stream` (a hipStream_t passed
 *     as void*; NULL means the default stream). Calls can be captured in a
 *     HIP graph.
 *   - Scalars (sizes, strides, dtypes) are validated on the host before
 *     anything is launched; device memory is never dereferenced by the host.
 *     On a validation failure nothing is enqueued and a negative MDS_ERR_*
 *     code is returned; mds_last_error() then holds a message (per thread).
 *   - Strides are in ELEMENTS of the array's dtype. Vector (16-byte) access is
 *     used when pointers and strides allow it; any stride >= V works.
 *   - Values derived from device data that are out of contract (an anchor or
 *     draft token outside [0, V)) cannot be rejected on the host. The kernels
 *     then substitute token 0 and set a bit in the workspace's sticky status
 *     word (the first 4 bytes of the workspace, see MDS_STATUS_*). The
 *     library never clears that word: the caller zeroes the workspace once
 *     when allocating it and reads the word after a synchronisation.
 *   - Logits (base, target, cache) are finite, -inf (a masked column) or NaN;
 *     +inf is outside the contract (NaN in target rows too). A row with no
 *     finite logit (all -inf) is a legal input: its winner is column 0 (the
 *     first of equal maxima), and verification takes its distribution (p of
 *     a target row, with top-p its kept set {0}; q of a draft cache row) to
 *     be the one-hot at column 0.
 *   - Outputs must not alias inputs; the cache must not alias base or target.
 *   - Calls that share a workspace must be ordered (same stream).
 */
#ifndef MDS_H_
#define MDS_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MDS_ABI_VERSION 2

/* return codes */
#define MDS_OK 0
#define MDS_ERR_INVALID_ARG (-1)      /* a size, stride, pointer or dtype is invalid */
#define MDS_ERR_UNSUPPORTED (-2)      /* valid but not supported by this library (e.g. r not a multiple of 32) */
#define MDS_ERR_WORKSPACE (-3)        /* workspace smaller than the matching *_workspace_bytes() */
#define MDS_ERR_HIP (-4)              /* a HIP runtime call or kernel launch failed */

/* element types */
#define MDS_F32 0
#define MDS_BF16 1

/* sticky status bits (workspace word 0) */
#define MDS_STATUS_BAD_ANCHOR 1u      /* an anchor token was outside [0, V); token 0 was used */
#define MDS_STATUS_BAD_DRAFT 2u       /* a draft token given to verification was outside [0, V); token 0 was used */
/* bit 4u is reserved (unused) */
#define MDS_STATUS_BAD_INDEX 8u       /* an indexed call met a state slot >= n_slots or a cache row outside
                                         [0, n_cache_rows); that row was treated as padding */

/* sampling salts: the draft salt is the pages' draft-noise salt (1 << 30) */
#define MDS_SALT_DRAFT (1u << 30)
#define MDS_SALT_ACCEPT 1u
#define MDS_SALT_RESAMPLE 2u

/* Version of this ABI (MDS_ABI_VERSION of the build). */
int mds_abi_version(void);

/* Static description of a return code. */
const char* mds_status_string(int status);

/* Message of the last failed call on this thread ("" if none). */
const char* mds_last_error(void);

/*
 * Workspace sizes (bytes) for the two calls at the given sizes. Pure host
 * functions: they need no GPU. Limits: 1 <= B <= 65535, 1 <= K <= 32,
 * 2 <= V < 2^24, 32 <= r <= 512 with r % 32 == 0.
 */
int mds_draft_workspace_bytes(int B, int K, int V, int r, size_t* out_bytes);
int mds_verify_workspace_bytes(int B, int K, int V, int has_top_p, int has_draft_lse, size_t* out_bytes);

/*
 * mds_markov_draft_loop - the K sequential Markov draft steps for B requests.
 *
 * For request b, with prev_0 = anchor_tokens[b] and P0 = anchor_pos[b], step
 * k = 0..K-1 computes, for every column v < V
 * (DSparkSpeculator API page, _sample_markov_chain and _sample_logits):
 *   e          = w1[prev_k, 0:r]                          (Markov embedding)
 *   bias[v]    = sum_j w2[v, j] * e[j]                    (Markov bias, fp32 accumulation)
 *   z[v]       = float(base[b, k, v]) + bias[v]           (fp32)
 *   cache[b,k,v] = z[v] rounded to the cache dtype         (pre-temperature biased logits)
 *   s[v]       = z[v] / T_b + Gumbel(seed_b, P0 + k, v)   if T_b > 0; s[v] = z[v] if T_b == 0
 *   token      = first NaN column of s, else first maximum (PR #65007, Part 1)
 * and feeds token back as prev_{k+1}. The draw for the token at position
 * P0+1+k is keyed by the position before it, P0+k; the Gumbel variate of
 * column v is -log(-log u) with u = (2*(w >> 9) + 1) * 2^-24 and w = word
 * (v & 3) of Philox4x32-10(counter = (v >> 2, lo32(P0+k), hi32(P0+k),
 * MDS_SALT_DRAFT), key = (lo32(seed), hi32(seed))).
 *
 * Arguments (device pointers unless stated):
 *   B, K, V, r            batch, draft steps, vocabulary, Markov rank (host ints)
 *   base, base_dtype      base draft logits, MDS_F32 or MDS_BF16; element (b, k, v) at
 *                         b*base_req_stride + k*base_step_stride + v
 *   w1, w2                bf16 [V, r] row-major (row stride r), 16-byte aligned
 *                         (else MDS_ERR_INVALID_ARG)
 *   anchor_tokens         int32 [B]   previous token of step 0
 *   anchor_pos            int64 [B]   position P0 of the anchor token
 *   temperature           float [B]   > 0 sampled request, == 0 greedy request
 *   seeds                 int64 [B]   per-request seed
 *   cache, cache_dtype    draft-logits cache (written), MDS_F32 or MDS_BF16; element
 *                         (b, k, v) at b*cache_req_stride + k*cache_step_stride + v
 *   draft_tokens          int32 [B, K] (written), row-major
 *   draft_lse             float [B, K] (written, nullable): log-sum-exp over v of
 *                         cache[b,k,v] / T_b, the normaliser of the draft distribution
 *                         q_k that verification needs (NaN if the row holds NaN,
 *                         unspecified for greedy requests)
 *   workspace             >= mds_draft_workspace_bytes(B, K, V, r) bytes, 256-byte aligned,
 *                         zeroed when allocated; the library keeps part of it at zero
 *                         between calls (so a call needs no clearing launch), so the
 *                         caller must not write it between calls (it may be shared
 *                         with top-k drafting calls); after a call that returned
 *                         MDS_ERR_HIP, zero it again before the next call
 *   stream                hipStream_t as void*
 *
 * Kernels: one launch per step (each streams w2 once; rank <= 256 and larger
 * ranks use different step kernels), then one launch that writes the tokens
 * and draft_lse; a call with K*B > 4096 also clears its winner keys first.
 * The kernel sequence depends only on the arguments, never on global state.
 */
int mds_markov_draft_loop(int B, int K, int V, int r,
                          const void* base, int base_dtype, int64_t base_req_stride, int64_t base_step_stride,
                          const void* w1, const void* w2,
                          const int32_t* anchor_tokens, const int64_t* anchor_pos,
                          const float* temperature, const int64_t* seeds,
                          void* cache, int cache_dtype, int64_t cache_req_stride, int64_t cache_step_stride,
                          int32_t* draft_tokens, float* draft_lse,
                          void* workspace, size_t workspace_bytes, void* stream);

/*
 * mds_rejection_verify - verify the K drafts of B requests against the target.
 *
 * Target row j of request b (position P0+1+j) is at
 * target + (b*(K+1) + j)*target_row_stride, j = 0..K.
 * Greedy request (T_b == 0), PR #63554 Notes: a_j = first-NaN-else-first-max
 * of target row j; drafts are accepted while draft[b,k] == a_k; the final
 * token is a_n at the first mismatch n (a_K if all match); the cache is not read.
 * Sampled request (T_b > 0), PR #65007 Overview/Part 2:
 *   p_j = softmax(target row j / T_b), restricted when top_p[b] < 1 to the
 *         smallest prefix in (logit desc, token id asc) order whose mass
 *         reaches top_p[b], plus the row maximum, and renormalised;
 *   q_k = softmax(cache[b,k,:] / T_b) (q from draft_lse when given);
 *   draft k is accepted iff p_k(x) >= u_k * q_k(x), u_k = uniform of column 0
 *         of the MDS_SALT_ACCEPT stream keyed (seed_b, P0+k);
 *   at the first rejection j the final token is drawn from
 *         max(0, p_j - q_j) normalised (from p_j if that is all zero, or if
 *         q_j is NaN) and when all K are accepted from p_K: Gumbel-max over
 *         log of that distribution plus noise of the MDS_SALT_RESAMPLE
 *         stream keyed (seed_b, P0+j).
 * A draft token of -1 is a placeholder (PR #65007, Tests: rejection sampling
 * with -1 placeholder drafts): the request's drafts end at its first -1, and
 * when all drafts before it are accepted the final token is drawn from p of
 * that row (the argmax of that row for a greedy request). Any other token
 * outside [0, V) is out of contract (token 0 is used, MDS_STATUS_BAD_DRAFT).
 * Outputs: out_tokens int32 [B, K+1] = accepted drafts, the final token, then
 * -1 padding; num_accepted int32 [B].
 *
 * Arguments:
 *   target                float [B*(K+1), V] rows as above, target_row_stride >= V
 *   cache, cache_dtype    as written by mds_markov_draft_loop (strides in elements)
 *   draft_lse             float [B, K] from mds_markov_draft_loop, or NULL to recompute
 *                         it from the cache (one extra read of the cache)
 *   draft_tokens          int32 [B, K]
 *   temperature, seeds, anchor_pos   as for the draft loop
 *   top_p                 float [B] or NULL (off); a value >= 1 turns it off for that request
 *   workspace             >= mds_verify_workspace_bytes(B, K, V, top_p != NULL,
 *                         draft_lse != NULL) bytes, 256-byte aligned, zero-filled
 *                         before its first use. Bytes [256, 256 + 1 MiB) hold one
 *                         arrival counter and one winner key per request (see
 *                         mds_verify_slot_offsets) that every call leaves at zero;
 *                         the caller must not write the workspace between calls
 *                         (nor use the same memory as a draft-loop workspace).
 */
int mds_rejection_verify(int B, int K, int V,
                         const float* target, int64_t target_row_stride,
                         const void* cache, int cache_dtype, int64_t cache_req_stride, int64_t cache_step_stride,
                         const float* draft_lse, const int32_t* draft_tokens,
                         const float* temperature, const float* top_p,
                         const int64_t* seeds, const int64_t* anchor_pos,
                         int32_t* out_tokens, int32_t* num_accepted,
                         void* workspace, size_t workspace_bytes, void* stream);

/* flags of mds_markov_draft_loop_ex */
#define MDS_DRAFT_FP64_GUMBEL 1u /* the API page's use_fp64_gumbel: Gumbel variate and score in float64 */
#define MDS_DRAFT_W2_TILED 2u    /* w2 given in the tiled order of mds_tile_markov_w2 (r <= 256) */

/*
 * mds_markov_draft_loop_ex - mds_markov_draft_loop with the pages'
 * request-state indexing and options (DSparkSpeculator API page,
 * _sample_logits and _sample_markov_chain: per-row idx_map and sample_pos,
 * the cache's row_mapping, use_fp64_gumbel; _sample_sequential_sharded:
 * padding slots are inert, with no draft-logits cache writes).
 *
 * Batch row b at step k uses state slot s = idx_map[b*K + k] (s = b when
 * idx_map is NULL; then row_mapping must be NULL and n_slots, n_cache_rows
 * >= B):
 *   temperature[s], seeds[s]   its temperature and seed (arrays of n_slots);
 *   sample_pos[b*K + k]        the position P of the predicted token; the draw
 *                              is keyed by P - 1 (the plain call's P0 + k);
 *   cache row                  row_mapping[s] (s itself if row_mapping is NULL)
 *                              of a [n_cache_rows, K, V] cache, written at
 *                              column k (strides as in the plain call).
 * base rows, anchor_tokens, draft_tokens and draft_lse stay batch-indexed.
 * s < 0 makes the row inert at that step: no cache write, draft token -1,
 * draft_lse NaN; a later step of that row that is not inert has no previous
 * token and uses token 0 (MDS_STATUS_BAD_ANCHOR). A slot >= n_slots or a
 * mapped row outside [0, n_cache_rows) is treated as inert and sets
 * MDS_STATUS_BAD_INDEX.
 * flags: MDS_DRAFT_FP64_GUMBEL computes g = -ln(-ln u) (same u) and the score
 * z/T + g in float64; the winner is the first NaN, else the first maximum of
 * the float64 scores at a resolution of 2^-28 relative (candidates closer
 * than that go to the lower column); needs r <= 256.
 * flags: MDS_DRAFT_W2_TILED: w2 points to the output of mds_tile_markov_w2
 * for (V, r) instead of the row-major [V, r] matrix; the results are those
 * of the row-major call on the matrix it was made from. Needs r <= 256
 * (else MDS_ERR_UNSUPPORTED).
 * Workspace and errors as for mds_markov_draft_loop.
 * ev_begin / ev_end (hipEvent_t as void*, or NULL) are recorded on `stream`
 * around the Markov step launches and *n_step_launches (if not NULL) gets
 * their count, as in mds_markov_draft_loop_timed.
 */
int mds_markov_draft_loop_ex(int B, int K, int V, int r,
                             const void* base, int base_dtype, int64_t base_req_stride, int64_t base_step_stride,
                             const void* w1, const void* w2,
                             const int32_t* anchor_tokens, const int32_t* idx_map, const int64_t* sample_pos,
                             int n_slots, const float* temperature, const int64_t* seeds,
                             const int32_t* row_mapping, int n_cache_rows,
                             void* cache, int cache_dtype, int64_t cache_row_stride, int64_t cache_step_stride,
                             int32_t* draft_tokens, float* draft_lse, uint32_t flags,
                             void* workspace, size_t workspace_bytes, void* stream,
                             void* ev_begin, void* ev_end, int* n_step_launches);

/*
 * mds_draft_topk_workspace_bytes - workspace size of mds_markov_draft_loop_topk:
 * 256 bytes of status, 8 * B*K*ceil(V/8192)*topk bytes of per-chunk
 * candidates and 4 * B*K*topk bytes of candidate columns (each 256-aligned).
 * Errors as for mds_markov_draft_loop_topk's size checks.
 */
int mds_draft_topk_workspace_bytes(int B, int K, int V, int r, int topk, size_t* out_bytes);

/*
 * mds_markov_w2_tiled_bytes / mds_tile_markov_w2 - markov_w2, the Markov
 * head's [V, r] bias factor (DSparkSpeculator API page, _sample_markov_chain),
 * stored once in the order in which the Markov step kernel reads it, for
 * callers that keep the weights resident between calls
 * (mds_markov_draft_loop_ex with MDS_DRAFT_W2_TILED).
 *
 * Tiled order: with T = ceil(V / 16) tiles of 16 rows, element (v, j) of w2
 * (v < V, j < r) is at index
 *   (v / 16) * 16 r + (j / 32) * 512 + ((v % 16) + 16 * ((j % 32) / 8)) * 8 + j % 8
 * of the tiled array (T * 16 * r bf16 elements; the rows v in [V, 16 T) of
 * the last tile are zero). Each 1 KB block then holds one wave's operand of
 * one 16-row, 32-rank matrix-core product.
 *
 * mds_markov_w2_tiled_bytes: *out_bytes = 32 * r * ceil(V / 16) (host only).
 * mds_tile_markov_w2: w2 bf16 [V, r] row-major (device), w2_tiled (device,
 * w2_tiled_bytes >= mds_markov_w2_tiled_bytes, written), both 16-byte
 * aligned and not overlapping; one kernel on `stream` (hipStream_t as void*).
 * Errors: V outside [2, 2^24), r not a multiple of 32 in [32, 512], NULL,
 * misaligned or overlapping pointers or a short w2_tiled give
 * MDS_ERR_INVALID_ARG / MDS_ERR_UNSUPPORTED as for the draft calls, with
 * nothing enqueued.
 */
int mds_markov_w2_tiled_bytes(int V, int r, size_t* out_bytes);
int mds_tile_markov_w2(int V, int r, const void* w2, void* w2_tiled, size_t w2_tiled_bytes, void* stream);

/*
 * mds_markov_draft_loop_topk - top-k Markov drafting (DSparkSpeculator API
 * page, _sample_sequential_topk): the draft loop of mds_markov_draft_loop_ex
 * with the Markov bias applied only to each step's topk candidates.
 *
 * For every (b, k) that is not inert, the candidates are the topk largest of
 * base[b, k, :], chosen once from the base logits alone: ordered by value
 * with NaN above every number, -0 equal to +0, and the lower column first
 * among equal values. The cache row (b, k) (mapped as in _ex) is then written
 * in full: -inf at every other column and, at candidate v,
 *   z_v = fp32(base[b,k,v]) + sum_j w2[v,j] * w1[prev_b, j]
 * (float32 accumulation), rounded to the cache dtype. The draft token is the
 * Gumbel-max winner of that row exactly as in the dense loop (noise keyed by
 * column, (seed, sample_pos - 1), MDS_SALT_DRAFT; temperature; the first NaN,
 * else the first maximum, so a row of -inf only gives token 0), and draft_lse
 * is the log-sum-exp of the row / T over the candidates (NaN for greedy and
 * inert rows). Verification reads the cache unchanged.
 *
 * Arguments as for mds_markov_draft_loop_ex, plus:
 *   topk        1 <= topk <= min(256, V), and ceil(V/8192) * topk <= 7168
 *               (else MDS_ERR_INVALID_ARG / MDS_ERR_UNSUPPORTED);
 *   flags       MDS_DRAFT_FP64_GUMBEL: float64 variates and scores, winner
 *               taken exactly over the float64 scores (MDS_DRAFT_W2_TILED is
 *               not supported here: MDS_ERR_UNSUPPORTED);
 *   workspace   >= mds_draft_topk_workspace_bytes(B, K, V, r, topk) bytes,
 *               256-byte aligned, zeroed when allocated and not written by the
 *               caller between calls (it may be shared with the dense draft
 *               calls, whose zero-kept region it leaves untouched);
 *   ev_begin / ev_end  hipEvent_t (as void*) or NULL: recorded around the
 *               candidate-selection launch (the kernel that streams the base
 *               logits and writes the -inf cache rows).
 * Launches three kernels on `stream`: selection (one work-group per
 * 8192-column chunk of a row), merge (one per row) and the K-step chain (one
 * per request).
 */
int mds_markov_draft_loop_topk(int B, int K, int V, int r, int topk,
                               const void* base, int base_dtype, int64_t base_req_stride,
                               int64_t base_step_stride, const void* w1, const void* w2,
                               const int32_t* anchor_tokens, const int32_t* idx_map, const int64_t* sample_pos,
                               int n_slots, const float* temperature, const int64_t* seeds,
                               const int32_t* row_mapping, int n_cache_rows,
                               void* cache, int cache_dtype, int64_t cache_row_stride, int64_t cache_step_stride,
                               int32_t* draft_tokens, float* draft_lse, uint32_t flags,
                               void* workspace, size_t workspace_bytes, void* stream,
                               void* ev_begin, void* ev_end);

/*
 * mds_draft_lm_head - the draft model's LM head ahead of the loop
 * (DSparkSpeculator API page, _sample_sequential: compute_draft_logits on the
 * gathered hidden states, ordered (request, step)).
 *   out[b, k, v] = sum_h hidden[b*K + k, h] * lm_head[v, h]
 * bf16 inputs, float32 accumulation (any order), rounded to out_dtype (bf16:
 * round to nearest even). The output is the base-logit layout the draft loop
 * reads: row (b, k) at out + b*out_req_stride + k*out_step_stride (elements).
 * Arguments:
 *   B, K, V      as for the draft loop (B*K rows)
 *   H            hidden size, a multiple of 256 (else MDS_ERR_UNSUPPORTED)
 *   hidden       bf16 [B*K, H], row stride hidden_row_stride >= H elements, a
 *                multiple of 8; 16-byte aligned
 *   lm_head      bf16 [V, H] contiguous, 16-byte aligned
 *   out          MDS_F32 or MDS_BF16, rows as above (must not overlap)
 *   ev_begin / ev_end  hipEvent_t (as void*) or NULL, recorded around the launch
 * One kernel launch on `stream`; lm_head is read once from HBM while
 * B*K <= 256 (each further 256 rows read it again). No workspace.
 */
int mds_draft_lm_head(int B, int K, int V, int H, const void* hidden, int64_t hidden_row_stride,
                      const void* lm_head, void* out, int out_dtype, int64_t out_req_stride,
                      int64_t out_step_stride, void* stream, void* ev_begin, void* ev_end);

/*
 * mds_markov_draft_loop_from_hidden - the draft LM head followed by the
 * K-step Markov draft loop (DSparkSpeculator API page, _sample_sequential:
 * compute_draft_logits gives the base draft logits of every (request, step)
 * row, which the sequential loop then consumes).
 *   hidden, lm_head, H    as for mds_draft_lm_head
 *   base                  MDS_F32 or MDS_BF16 rows [B, >=K, V] as the out of
 *                         mds_draft_lm_head: receives the base logits of steps
 *                         1 .. K-1; its step-0 rows are scratch (left unwritten
 *                         when step 0 runs fused)
 *   the other arguments   as for mds_markov_draft_loop (workspace of
 *                         mds_draft_workspace_bytes(B, K, V, r))
 *   ev_begin / ev_end     hipEvent_t (as void*) or NULL, recorded before the
 *                         first and after the last launch of the call
 * The results equal those of mds_draft_lm_head followed by
 * mds_markov_draft_loop on the same buffers: draft tokens, the cache and base
 * rows 1 .. K-1 bit for bit, draft_lse up to the order of float32 sums. When
 * B <= 32, B*K <= 256 and r <= 256, step 0 runs inside the LM head's
 * work-groups (its base row is neither stored nor read back, and one launch
 * fewer); otherwise the two run one after the other. Errors as for the two.
 */
int mds_markov_draft_loop_from_hidden(int B, int K, int V, int r, int H, const void* hidden,
                                      int64_t hidden_row_stride, const void* lm_head, void* base,
                                      int base_dtype, int64_t base_req_stride, int64_t base_step_stride,
                                      const void* w1, const void* w2, const int32_t* anchor_tokens,
                                      const int64_t* anchor_pos, const float* temperature,
                                      const int64_t* seeds, void* cache, int cache_dtype,
                                      int64_t cache_req_stride, int64_t cache_step_stride,
                                      int32_t* draft_tokens, float* draft_lse, void* workspace,
                                      size_t workspace_bytes, void* stream, void* ev_begin, void* ev_end);

/*
 * mds_rejection_verify_indexed - mds_rejection_verify with request-state
 * indexing: request b uses state slot s = idx_map[b] (temperature[s],
 * seeds[s], top_p[s], arrays of n_slots) and draft-logits cache rows
 * row_mapping[s] (s itself if row_mapping is NULL) of a [n_cache_rows, K, V]
 * cache. target rows, draft_tokens, draft_lse, anchor_pos and the outputs
 * stay batch-indexed. s < 0 is a padding request: nothing is read, every
 * output token is -1 and num_accepted 0. A slot >= n_slots or a mapped row
 * outside [0, n_cache_rows) is treated as padding and sets
 * MDS_STATUS_BAD_INDEX. Workspace: mds_verify_workspace_bytes(B, ...).
 */
int mds_rejection_verify_indexed(int B, int K, int V,
                                 const float* target, int64_t target_row_stride,
                                 const void* cache, int cache_dtype, int64_t cache_row_stride,
                                 int64_t cache_step_stride, int n_cache_rows,
                                 const float* draft_lse, const int32_t* draft_tokens,
                                 const int32_t* idx_map, int n_slots,
                                 const float* temperature, const float* top_p, const int64_t* seeds,
                                 const int32_t* row_mapping, const int64_t* anchor_pos,
                                 int32_t* out_tokens, int32_t* num_accepted,
                                 void* workspace, size_t workspace_bytes, void* stream);

/*
 * mds_markov_draft_loop_timed - mds_markov_draft_loop that also records
 * ev_begin just before the first and ev_end just after the last launch of the
 * Markov step kernel on `stream` (the init and finalize kernels stay outside),
 * and writes to *n_step_launches how many launches that span held (K).
 * ev_begin, ev_end: hipEvent_t (as void*) created by the caller;
 * n_step_launches: host pointer, nullable.
 */
int mds_markov_draft_loop_timed(int B, int K, int V, int r,
                                const void* base, int base_dtype, int64_t base_req_stride, int64_t base_step_stride,
                                const void* w1, const void* w2,
                                const int32_t* anchor_tokens, const int64_t* anchor_pos,
                                const float* temperature, const int64_t* seeds,
                                void* cache, int cache_dtype, int64_t cache_req_stride, int64_t cache_step_stride,
                                int32_t* draft_tokens, float* draft_lse,
                                void* workspace, size_t workspace_bytes, void* stream,
                                void* ev_begin, void* ev_end, int* n_step_launches);

/*
 * mds_debug_noise - test hook: writes for n columns cols[i] the Philox word
 * and the float32 Gumbel variate of the stream (seed, pos_key, salt) exactly as
 * the sampling kernels compute them. cols int32 [n], words uint32 [n],
 * gumbel float [n] (device pointers). Used by the tests to compare the device
 * noise with an independent implementation.
 */
int mds_debug_noise(int n, const int32_t* cols, int64_t seed, int64_t pos_key, uint32_t salt,
                    uint32_t* words, float* gumbel, void* stream);

/*
 * mds_debug_top_p - test hook: the exact top-p kept set of `rows` independent
 * rows (row i at target + i*row_stride, temperature[i] > 0, top_p[i]) as
 * verification computes it: column v is kept iff ord(t_v) > tau[i], or
 * ord(t_v) == tau[i] and v <= cut[i], where ord maps a float to an unsigned key
 * in the same order (NaN above all, -0 == +0); log_z[i] is the log of the kept
 * mass sum exp(x - max x), x = t / T. on[i] = 0 means nothing was filtered
 * (top_p >= 1). workspace >= mds_verify_workspace_bytes(rows, 1, V, 1, 1).
 */
int mds_debug_top_p(int rows, int V, const float* target, int64_t row_stride, const float* temperature,
                    const float* top_p, uint32_t* tau, int32_t* cut, float* log_z, int32_t* on,
                    void* workspace, size_t workspace_bytes, void* stream);

/*
 * mds_markov_draft_loop_noalloc - mds_markov_draft_loop without a workspace
 * argument, for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc): the
 * loop's scratch (winner keys and per-slab partials) lives in a fixed
 * 8.5 MiB + 256 B array inside the library, one copy per device, held until
 * the process ends. The call allocates nothing and launches the same kernels
 * as mds_markov_draft_loop (plus, on its first call on a device, one clearing
 * launch), so its outputs are identical.
 *   K * B must be <= 1024 (else MDS_ERR_UNSUPPORTED, nothing enqueued).
 *   status   device uint32 (written): the sticky status word that the plain
 *            call keeps in its workspace (MDS_STATUS_* bits are OR-ed in);
 *            the caller zeroes it and reads it after a synchronisation.
 * Every call on one device shares that device's array and leaves its winner
 * keys at zero: calls that may overlap on one device (different streams
 * without ordering, or concurrent host threads' work on unordered streams)
 * race on it and must be serialised by the caller. Other arguments, limits
 * and errors as for mds_markov_draft_loop.
 */
int mds_markov_draft_loop_noalloc(int B, int K, int V, int r,
                                  const void* base, int base_dtype, int64_t base_req_stride, int64_t base_step_stride,
                                  const void* w1, const void* w2,
                                  const int32_t* anchor_tokens, const int64_t* anchor_pos,
                                  const float* temperature, const int64_t* seeds,
                                  void* cache, int cache_dtype, int64_t cache_req_stride, int64_t cache_step_stride,
                                  int32_t* draft_tokens, float* draft_lse, uint32_t* status, void* stream);

/*
 * mds_verify_slot_offsets - layout hook (pure host function, no GPU needed):
 * byte offsets, from the start of a verification workspace, of request b's
 * 32-bit arrival counter and of its 64-bit final-draw winner key, for
 * 0 <= b < 65535 (else MDS_ERR_INVALID_ARG). Both lie in the fixed block
 * [256, 256 + 1 MiB) whatever B, K or V a call uses; no two requests share a
 * counter or a key, and no key overlaps a counter.
 */
int mds_verify_slot_offsets(int b, size_t* counter_offset, size_t* key_offset);

/*
 * mds_debug_gumbel - test hook: the float32 Gumbel variate the kernels derive
 * from each given 32-bit word (device arrays of n elements). Only the top 23
 * bits of a word matter, so 2^23 words cover every possible variate.
 */
int mds_debug_gumbel(int n, const uint32_t* words, float* gumbel, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* MDS_H_ */
