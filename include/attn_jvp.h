/*
 * attn_jvp.h -- C ABI of the MI355X (gfx950) forward-mode JVP of masked
 * scaled-dot-product attention.
 *
 * Operation ("Causal-rCM: A Unified Teacher-Forcing and Self-Forcing Open
 * Recipe ..." summary, Appendix B "FlashAttention-2 JVP Kernel with Custom
 * Masks"): given Q, K, V and their tangents dQ, dK, dV, compute in one
 * online-softmax pass the primal masked attention output O, its row
 * log-sum-exp LSE and the tangent dO, the directional derivative of exactly
 * the same masked operator.  Masked-out pairs contribute no tangent (the mask
 * is discrete).  For query row i with admissible keys J_i:
 *
 *   s_j = scale <q_i,k_j>,  p = softmax_{J_i}(s),  O_i = sum_j p_j v_j,
 *   LSE_i = ln sum_{j in J_i} exp(s_j),
 *   ds_j = scale (<dq_i,k_j> + <q_i,dk_j>),  mu_i = sum_j p_j ds_j,
 *   dO_i = sum_j p_j (ds_j - mu_i) v_j + sum_j p_j dv_j,
 *   dLSE_i = mu_i (the tangent of LSE, an optional output).
 *
 * Around it: a split-key variant of the same pass (attn_jvp_fwd_split) and
 * the backward of the primal, the gradients of sum(g * O) with respect to Q,
 * K and V reusing the forward's LSE (attn_jvp_bwd).
 *
 * Masks are query groups with admissible key ranges (Appendix B: custom masks
 * as query-key rectangles, one sparse schedule shared by the primal and the
 * tangent scores).  The teacher-forcing builder packs [clean | noisy] tokens
 * (Section 3 of the same page: the TF-masked packed forward; "Causal Forcing:
 * Autoregressive Diffusion Distillation Done Right ..." summary, Section 2:
 * clean and noisy videos concatenated under a causal attention mask).
 *
 * Conventions for every entry point:
 *   - returns ATTN_JVP_OK (0) or a negative status; never throws, never
 *     aborts, never writes through a pointer after returning an error;
 *   - all int32/int64 sizes are element counts;
 *   - host pointers are read during the call only; nothing is retained.
 */
#ifndef ATTN_JVP_H
#define ATTN_JVP_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define ATTN_JVP_API_VERSION 2

enum attn_jvp_status {
  ATTN_JVP_OK = 0,
  ATTN_JVP_ERR_NULL = -1,        /* a required pointer is NULL */
  ATTN_JVP_ERR_SHAPE = -2,       /* sizes inconsistent or out of range */
  ATTN_JVP_ERR_DTYPE = -3,       /* unknown dtype code */
  ATTN_JVP_ERR_ALIGN = -4,       /* pointer or stride not 16-byte aligned, or
                                    last dimension not contiguous */
  ATTN_JVP_ERR_MASK = -5,        /* malformed mask description, or mask size
                                    differs from the tensors */
  ATTN_JVP_ERR_UNSUPPORTED = -6, /* valid but not implemented (head dim,
                                    aliasing outputs, the LSE tangent
                                    without any input tangent) */
  ATTN_JVP_ERR_HIP = -7,         /* no usable HIP device, or a HIP call failed */
  ATTN_JVP_ERR_OOM = -8,         /* host or device allocation failed */
  ATTN_JVP_ERR_NOT_READY = -9,   /* allocation-free call: the mask's schedule
                                    for this device and split count is not
                                    resident yet */
  ATTN_JVP_ERR_SCRATCH = -10     /* allocation-free call: the launch needs more
                                    than the fixed scratch buffer */
};

enum attn_jvp_dtype {
  ATTN_JVP_BF16 = 0, /* inputs and O/dO in bfloat16; bf16 MFMA, fp32 accumulate */
  ATTN_JVP_F32 = 1   /* inputs and O/dO in fp32; fp32 arithmetic throughout */
};

/* Opaque, immutable mask descriptor: a partition of the query rows [0, n_q)
 * into contiguous groups, each with a sorted list of disjoint key intervals
 * [k_begin, k_end) in [0, n_k).  Library-owned host memory plus lazily built
 * per-device tile schedules.  Safe to share between threads once built. */
typedef struct attn_jvp_mask attn_jvp_mask;

/* Teacher-forcing mask over the packed sequence [clean | noisy], each stream
 * n_frames * tokens_per_frame tokens (N = 2 * n_frames * tokens_per_frame).
 * A unit is frames_per_chunk consecutive frames (1 = frame-wise).  A clean
 * token of unit u sees clean units <= u; a noisy token of unit u sees clean
 * units < u and the noisy tokens of unit u (all of them, in both directions).
 * Errors: ERR_NULL (out == NULL); ERR_SHAPE (a size <= 0, n_frames not a
 * multiple of frames_per_chunk, or N > 2^30); ERR_OOM.  On success *out owns a
 * new mask; release it with attn_jvp_mask_free. */
int attn_jvp_mask_tf(int32_t n_frames, int32_t tokens_per_frame,
                     int32_t frames_per_chunk, attn_jvp_mask **out);

/* Generic query-key rectangles in CSR form.
 *   group_q_begin[n_groups + 1]: strictly increasing, group_q_begin[0] = 0,
 *                                group_q_begin[n_groups] = n_q;
 *   range_ptr[n_groups + 1]:     non-decreasing, range_ptr[0] = 0; group g owns
 *                                ranges range_ptr[g] .. range_ptr[g+1]-1;
 *   k_begin[r], k_end[r]:        0 <= k_begin <= k_end <= n_k; within a group
 *                                sorted by k_begin and non-overlapping
 *                                (touching ranges are merged, empty ones
 *                                dropped).
 * Errors: ERR_NULL; ERR_SHAPE (n_q, n_k <= 0 or > 2^30, n_groups <= 0);
 * ERR_MASK (any rule above broken); ERR_OOM.  The stored form is canonical:
 * adjacent groups with identical key sets are merged. */
int attn_jvp_mask_rects(int32_t n_q, int32_t n_k, int32_t n_groups,
                        const int32_t *group_q_begin, const int32_t *range_ptr,
                        const int32_t *k_begin, const int32_t *k_end,
                        attn_jvp_mask **out);

/* Block-causal mask over one stream of n_units units of unit_tokens tokens
 * (N = n_units * unit_tokens): a token of unit u sees every token of units
 * <= u.  This is the diffusion-forcing layout ("Causal Forcing ..." summary,
 * Section 2: a noisy frame attends directly to the noisy prefix, with no
 * clean copy); unit_tokens = 1 gives plain causal attention.
 * Errors: ERR_NULL, ERR_SHAPE (a size <= 0 or N > 2^30), ERR_OOM. */
int attn_jvp_mask_block_causal(int32_t n_units, int32_t unit_tokens,
                               attn_jvp_mask **out);

/* Every query sees every key (plain attention): one group, one range. */
int attn_jvp_mask_dense(int32_t n_q, int32_t n_k, attn_jvp_mask **out);

/* Sizes of a mask; any output pointer may be NULL.  n_visible_pairs is the
 * number of admissible (query, key) pairs. Errors: ERR_NULL (m == NULL). */
int attn_jvp_mask_info(const attn_jvp_mask *m, int32_t *n_q, int32_t *n_k,
                       int32_t *n_groups, int32_t *n_ranges,
                       int64_t *n_visible_pairs);

/* Copy the canonical CSR form out (arrays sized from attn_jvp_mask_info:
 * n_groups + 1, n_groups + 1, n_ranges, n_ranges).  Errors: ERR_NULL. */
int attn_jvp_mask_export(const attn_jvp_mask *m, int32_t *group_q_begin,
                         int32_t *range_ptr, int32_t *k_begin, int32_t *k_end);

/* Host copy of the block schedule the kernels use for a tile shape
 * (block_m query rows x block_n keys, block_n a multiple of 32).  For query
 * tile t (rows [t*block_m, (t+1)*block_m)), entries tile_offsets[t] ..
 * tile_offsets[t+1]-1 list the key blocks b (keys [b*block_n, (b+1)*block_n))
 * holding at least one admissible pair of the tile: first the full blocks in
 * increasing order, then the partial ones in increasing order.
 * entry_partial[e] is -1 for a full block (every (row, key) of the block is
 * admissible for every row of the tile that exists), else an index p into
 * partial_bits, where word
 *   partial_bits[(p * block_m + r) * (block_n / 32) + w]
 * bit i says whether row t*block_m + r may see key b*block_n + 32*w + i.
 * tile_order[n_tiles] lists the tiles by decreasing entry count (ties by
 * index): the kernels launch heavy tiles first.
 * Call with all array pointers NULL to get n_tiles / n_entries / n_partial,
 * then again with arrays of those sizes.  Errors: ERR_NULL (m or a size
 * pointer), ERR_SHAPE (block_m <= 0, block_n <= 0 or not a multiple of 32),
 * ERR_OOM. */
int attn_jvp_mask_schedule(const attn_jvp_mask *m, int32_t block_m,
                           int32_t block_n, int32_t *n_tiles,
                           int64_t *n_entries, int64_t *n_partial,
                           int32_t *tile_offsets, int32_t *tile_order,
                           int32_t *entry_block, int32_t *entry_partial,
                           uint32_t *partial_bits);

/* Host copy of the unit list attn_jvp_fwd_split launches for max_splits
 * (for tests and tools).  With L = max(1, ceil(longest / max_splits)),
 * longest the largest entry count of any tile of the (block_m, block_n)
 * schedule, tile t with n entries becomes k = max(1, ceil(n / L)) units,
 * entries tile_offsets[t] + floor(n*u/k) .. tile_offsets[t] + floor(n*(u+1)/k)
 * - 1 for u = 0 .. k-1, listed tile by tile: unit_offsets[n_units + 1] holds
 * these boundaries, unit_tile[n_units] the tile, unit_part[n_units] the
 * partial slot (consecutive from 0 over the units of tiles with k > 1; -1 for
 * a tile's only unit), unit_order[n_units] the units by decreasing entry
 * count (ties by index).  *n_parts counts the slots.  Call with NULL arrays
 * for the sizes first.  Errors: ERR_NULL, ERR_SHAPE (as for
 * attn_jvp_mask_schedule, or max_splits < 1), ERR_OOM. */
int attn_jvp_mask_split_schedule(const attn_jvp_mask *m, int32_t block_m,
                                 int32_t block_n, int32_t max_splits,
                                 int32_t *n_units, int32_t *n_parts,
                                 int32_t *unit_offsets, int32_t *unit_order,
                                 int32_t *unit_tile, int32_t *unit_part);

/* The transposed mask: key and query roles swapped (its n_q is m's n_k):
 * key j admits query i exactly when query i admits key j under m.  The
 * backward pass walks it (key tiles over query blocks).  On success *out owns
 * a new canonical mask; release it with attn_jvp_mask_free.
 * Errors: ERR_NULL, ERR_OOM. */
int attn_jvp_mask_transpose(const attn_jvp_mask *m, attn_jvp_mask **out);

/* Release a mask and its device schedules.  The caller must make sure no
 * launched work still uses it (synchronise the streams first).  NULL is a
 * no-op. */
void attn_jvp_mask_free(attn_jvp_mask *m);

/* Arguments of one forward call.  Tensors are caller-owned device memory in
 * [B, N, H, D] order with element strides (the last dimension contiguous):
 * Q, dQ, O, dO use the q_stride_* strides and n_q rows; K, V, dK, dV use the
 * k_stride_* strides and n_k rows.  LSE is [B, H, n_q] fp32, contiguous,
 * natural log.  Every tensor pointer and every stride in bytes must be a
 * multiple of 16. */
typedef struct attn_jvp_args {
  int32_t dtype;       /* enum attn_jvp_dtype */
  int32_t B, H;        /* batch, heads (> 0) */
  int32_t n_q, n_k;    /* query rows, key rows: must equal the mask's */
  int32_t D;           /* head dim: 64 or 128 */
  const void *q, *k, *v;
  const void *dq, *dk, *dv; /* tangents; any of them NULL: that tangent is zero
                               (e.g. dK = dV = 0 for detached cached keys);
                               all NULL: primal only (d_o untouched) */
  void *o, *d_o;            /* outputs; must not alias any input */
  float *lse;               /* output, required */
  int64_t q_stride_b, q_stride_n, q_stride_h;
  int64_t k_stride_b, k_stride_n, k_stride_h;
  float scale;              /* softmax scale; <= 0 selects 1/sqrt(D) */
  float *d_lse;             /* optional output: the tangent of LSE, [B, H, n_q]
                               fp32 contiguous, sum_j p_ij ds_ij (0 for rows
                               without keys); NULL = not written.  Needs at
                               least one tangent (ERR_UNSUPPORTED otherwise). */
} attn_jvp_args;

/* Launch the fused primal + tangent pass on hip_stream (a hipStream_t; NULL
 * means the default stream) of the current device.  Asynchronous: argument
 * errors are returned before anything is launched; a failed launch returns
 * ERR_HIP; faults inside the kernel surface at the caller's next
 * synchronisation.  The first call for a (mask, device, tile shape) builds and
 * uploads the tile schedule (a blocking device allocation and copy); later
 * calls launch only, so they can be captured into a HIP graph (the same holds
 * for attn_jvp_fwd_split and attn_jvp_bwd once their schedules are uploaded).
 * Deterministic: no atomics, fixed reduction order.
 * Errors: ERR_NULL, ERR_DTYPE, ERR_SHAPE, ERR_ALIGN, ERR_MASK (mask sizes
 * differ from n_q/n_k), ERR_UNSUPPORTED, ERR_HIP, ERR_OOM. */
int attn_jvp_fwd(const attn_jvp_args *a, const attn_jvp_mask *m,
                 void *hip_stream);

/* Split-key variant of attn_jvp_fwd, same arguments and results ("Causal-rCM
 * ..." Appendix B: the kernel works through a tile's admissible key ranges in
 * parallel).  Each query tile's list of key blocks (attn_jvp_mask_schedule) is
 * cut into consecutive pieces of at most ceil(max_blocks / max_splits) blocks,
 * max_blocks being the longest list of any tile, and every piece runs as a
 * workgroup of its own, so long rows no longer serialise on one compute unit
 * (few query tiles against many keys, e.g. one chunk of queries against a
 * cached prefix).  The pieces of a tile that was cut write their running max,
 * sums l and mu and unnormalised accumulators to the workspace; a second
 * kernel merges them (rescaled to their common max) into O, dO, LSE and d_lse.
 * Tiles left whole finish as in attn_jvp_fwd.  max_splits = 1 gives exactly
 * attn_jvp_fwd's results; otherwise results agree with it up to fp32
 * rounding of the reordered sums.  Deterministic.
 *
 * workspace: caller-owned device memory, 16-byte aligned, of at least the
 * size attn_jvp_fwd_split_workspace reports for the same arguments, mask and
 * max_splits (0 bytes, and NULL allowed, when no tile is cut).  It holds
 * scratch only: nothing needs clearing, and calls sharing one workspace must
 * be ordered on one stream.  Errors: those of attn_jvp_fwd, ERR_SHAPE
 * (max_splits < 1, or workspace_bytes below the required size), ERR_NULL
 * (workspace NULL while bytes are needed), ERR_ALIGN (workspace). */
int attn_jvp_fwd_split_workspace(const attn_jvp_args *a, const attn_jvp_mask *m,
                                 int32_t max_splits, uint64_t *bytes);
int attn_jvp_fwd_split(const attn_jvp_args *a, const attn_jvp_mask *m,
                       int32_t max_splits, void *workspace,
                       uint64_t workspace_bytes, void *hip_stream);

/* attn_jvp_fwd_split without any allocation, for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation.  Same arguments (less the workspace) and
 * results, bit for bit, as attn_jvp_fwd_split with the same max_splits: the
 * partial sums of cut tiles go to a fixed scratch array of
 * ATTN_JVP_NOALLOC_SCRATCH_BYTES bytes that the library holds on every device
 * it runs on until the process ends.  The call allocates nothing, host or
 * device, and builds and uploads nothing: the mask's schedule and unit list
 * for this device, tile shape and max_splits must already be resident, which
 * one earlier attn_jvp_fwd_split call with the same max_splits on this device
 * (any arguments with the same dtype and D) makes them.  Nothing in the
 * scratch needs clearing.  All calls on one device share its scratch array:
 * calls that may overlap in time (on different streams, or from several
 * threads without ordering) race and give wrong results; order them on one
 * stream.  Errors: those of attn_jvp_fwd_split, ERR_NOT_READY (schedule not
 * resident), ERR_SCRATCH (the workspace attn_jvp_fwd_split_workspace reports
 * for these arguments exceeds ATTN_JVP_NOALLOC_SCRATCH_BYTES), ERR_HIP (the
 * scratch array's address could not be obtained). */
#define ATTN_JVP_NOALLOC_SCRATCH_BYTES (64ull << 20)
int attn_jvp_fwd_split_noalloc(const attn_jvp_args *a, const attn_jvp_mask *m,
                               int32_t max_splits, void *hip_stream);

/* A max_splits for attn_jvp_fwd_split on a device with n_cu compute units
 * (host-only: nothing is launched).  Returns 1 when the unsplit grid has at
 * least two workgroups per resident slot; otherwise, among 1 .. 16, the count
 * whose unit list has the smallest predicted makespan (units heaviest first
 * on the slot that frees up first, cost = key blocks + a fixed start-up cost,
 * plus a partial-sum cost for units of cut tiles), if it beats the unsplit
 * prediction by more than 15 %, else 1.  Errors: those of attn_jvp_fwd's
 * argument checks, ERR_NULL (max_splits), ERR_SHAPE (n_cu < 1), ERR_OOM. */
int attn_jvp_split_choose(const attn_jvp_args *a, const attn_jvp_mask *m,
                          int32_t n_cu, int32_t *max_splits);

/* Arguments of one backward call: the gradients of L = sum(g_o * O) with
 * respect to Q, K and V for the masked attention O = attn(Q, K, V) of the
 * forward (the forward returns LSE so that this pass can reuse it).
 * Layouts as in attn_jvp_args: Q, O, g_o, g_q use the q_stride_* strides and
 * n_q rows; K, V, g_k, g_v the k_stride_* strides and n_k rows; lse (input,
 * the forward's) and delta (output) are [B, H, n_q] fp32, contiguous.  delta
 * receives D_i = <g_o_i, O_i>, the row sums the pass needs; it is returned so
 * the caller owns all memory.  Every pointer and stride in bytes a multiple
 * of 16; outputs alias nothing.  Supported: both dtypes (bf16: MFMA products,
 * fp32 accumulation, bf16 outputs; fp32: fp32 throughout), D = 64 or 128. */
typedef struct attn_jvp_bwd_args {
  int32_t dtype;
  int32_t B, H;
  int32_t n_q, n_k;     /* must equal the mask's */
  int32_t D;
  const void *q, *k, *v;
  const void *o;        /* the forward's output O */
  const void *g_o;      /* gradient flowing into O */
  const float *lse;     /* the forward's LSE (natural log) */
  void *g_q, *g_k, *g_v;
  float *delta;
  int64_t q_stride_b, q_stride_n, q_stride_h;
  int64_t k_stride_b, k_stride_n, k_stride_h;
  float scale;          /* the forward's scale; <= 0 selects 1/sqrt(D) */
} attn_jvp_bwd_args;

/* Launch the backward on hip_stream: a dQ pass over query tiles (which also
 * writes delta) then a dK/dV pass over key tiles of the transposed mask
 * (built and uploaded on first use, cached with the mask).  Asynchronous,
 * deterministic (no atomics).  Errors: ERR_NULL, ERR_DTYPE, ERR_SHAPE,
 * ERR_ALIGN, ERR_MASK, ERR_UNSUPPORTED (D other than 64 or 128, aliasing),
 * ERR_HIP, ERR_OOM. */
int attn_jvp_bwd(const attn_jvp_bwd_args *a, const attn_jvp_mask *m,
                 void *hip_stream);

/* Tile shape (query rows, keys per block) of the forward kernel for (dtype,
 * D) with (tangent != 0) or without (tangent == 0) input tangents; these are
 * the block_m / block_n of the schedule that kernel walks (the bf16 primal-only
 * kernel at D = 128 takes 64-key blocks, every other bf16 kernel 32).
 * Errors: ERR_NULL, ERR_DTYPE, ERR_UNSUPPORTED (D not 64 or 128). */
int attn_jvp_tile_shape(int32_t dtype, int32_t D, int32_t tangent, int32_t *block_m,
                        int32_t *block_n);

/* Static English text for a status code (never NULL). */
const char *attn_jvp_status_str(int status);

/* ATTN_JVP_API_VERSION of the built library. */
int attn_jvp_version(void);

#ifdef __cplusplus
}
#endif

#endif /* ATTN_JVP_H */
