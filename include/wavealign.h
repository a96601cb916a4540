/*
 * wavealign.h - C ABI of the MI355X (gfx950) cache-aware block-sparse attention library.
 *
 * The library computes the hot path described by two pages:
 *   [WA]   "WaveAlign: Cache-Aware Query-Row Scheduling for Sparse Attention in
 *           Long-Video Generation"
 *   [GSRS] "Sparse Attention for Video Generation Acceleration via Growing Sparsity
 *           and Reduced Search"
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - All array arguments are DEVICE pointers owned by the caller (allocated with
 *    hipMalloc or by PyTorch) unless the comment says "host".  The library never
 *    allocates or frees device memory and keeps no state between calls.
 *  - Every call only validates its scalar arguments on the host and enqueues work
 *    on `stream` (a hipStream_t, passed as void*; NULL means the null stream).  No
 *    call synchronises.  Results are valid once the stream has reached the point
 *    after the call.
 *  - Return value: WA_OK (0) or a negative WA_ERR_* code.  On error nothing was
 *    enqueued and wa_last_error() returns a message (thread-local, valid until the
 *    next call from the same thread).
 *  - Tensors are row-major.  bf16 values are stored as uint16_t bit patterns.
 *  - Shapes: H heads, block size b, L valid tokens, L_pad = MB * b with
 *    MB = NB = ceil(L / b) query and key/value blocks.  Token rows >= L are padding:
 *    the caller zero-fills them in Q, K and V; their outputs are unspecified.
 *  - Calls issued on different streams may run concurrently as long as they do not
 *    write the same buffers.
 */
#ifndef WAVEALIGN_H
#define WAVEALIGN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define WA_OK 0
#define WA_ERR_INVALID_ARG (-1) /* null pointer, negative size, bad flag */
#define WA_ERR_UNSUPPORTED (-2) /* shape the kernels do not implement (head_dim, block, > limits) */
#define WA_ERR_CAPACITY (-3)    /* a workspace or output buffer is too small */
#define WA_ERR_HIP (-4)         /* the HIP runtime reported an error at launch */

/* Largest number of query/key blocks per head the reorder kernel handles. */
#define WA_MAX_BLOCKS 4096

/* Attention schedules (how workgroups map to query blocks). */
#define WA_SCHED_NATURAL 0     /* workgroup w runs position w of the head-major order      */
#define WA_SCHED_XCD_SLICED 1  /* XCD x runs the x-th contiguous slice of each head's order */
#define WA_SCHED_HEADS_INTERLEAVED 2 /* workgroup w runs position w / H of head w % H: all heads
                                        at once, the concurrent-head execution that WaveAlign
                                        VI-B contrasts with sequential heads */
#define WA_SCHED_AUTO 3 /* the schedule wa_attn_schedule_select wrote into the workspace:
                           XCD-sliced if some head was reordered, WA_SCHED_DEFAULT (the
                           default path) if every head kept its order */
#define WA_SCHED_DEFAULT 4 /* the default path for heads that all keep their original order
                              (perm is not read): all heads at once when one head's K and V,
                              MB * block * head_dim * 4 bytes, take at most
                              WA_ALL_HEADS_MAX_KV_BYTES, XCD-sliced in the original order
                              otherwise (wa_default_schedule) */

/* Per-head K + V bytes up to which WA_SCHED_DEFAULT runs all heads at once.  Measured on
   MI355X over Top-k, banded, Top-p and random masks: all heads at once is faster (up to
   9%) while a head's K and V take at most 8.4 MB (128 blocks of 128 x 128), and slower
   (4 to 37%) from 16.6 MB (254 blocks) on, where the XCD-sliced order lets the
   workgroups of one XCD share one head's K/V blocks in its L2. */
#define WA_ALL_HEADS_MAX_KV_BYTES (12u << 20)

/* Skip modes of wa_reorder_rows. */
#define WA_SKIP_ADAPTIVE 0
#define WA_SKIP_NEVER 1
#define WA_SKIP_ALWAYS 2

typedef uint16_t wa_bf16;

/* ABI version of this header; bumps on incompatible change. */
int wa_abi_version(void);

/* Message of the last failed call on this thread ("" if none). */
const char* wa_last_error(void);

/*
 * wa_schedule_info - hardware figures the reorder needs (host outputs).
 *   n_xcd        number of XCDs (L2 domains) of `device`
 *   cus_per_xcd  compute units per XCD
 *   wave         [WA §II-C, §VI-A] the dispatch wave per XCD: compute units per XCD
 *                times the attention workgroups resident per compute unit for
 *                head_dim (the WaveAlign bucket size W on one L2 domain)
 * Errors: WA_ERR_INVALID_ARG for null outputs, WA_ERR_UNSUPPORTED for head_dim not
 * 64/128, WA_ERR_HIP if the device cannot be queried.
 */
int wa_schedule_info(int device, int32_t head_dim, int32_t* n_xcd, int32_t* cus_per_xcd,
                     int32_t* wave);

/*
 * wa_build_block_index - [WA §II-B, §II-C] block mask -> per-query-block K/V lists.
 * Mask row i of head h lists the K/V blocks query block i visits; its row sum is
 * the query block's workload (NNZ).
 *   mask      uint8 [H][MB][NB], non-zero = selected
 *   row_ptr   int32 [H*MB + 1]  exclusive prefix sum of the row counts in head-major
 *                               row order; row_ptr[H*MB] = total NNZ (always written)
 *   col_idx   int32 [col_capacity]  ascending K/V block ids of each row, in row order
 *   row_nnz   int32 [H*MB]      per-row counts
 *   csc_ptr   int32 [H*NB + 1] or NULL  the same for the transposed mask (columns in
 *                                       head-major order); NULL skips the CSC
 *   csc_idx   int32 [csc_capacity] or NULL  ascending query block ids per column
 * Entries that would land at an index >= capacity are not written; row_ptr[H*MB]
 * and csc_ptr[H*NB] still hold the true totals, so a caller whose capacity is
 * below H*MB*NB detects truncation by reading them.  Integer work, bit-exact.
 * Errors: WA_ERR_INVALID_ARG (null required pointer, H/MB/NB < 1, negative capacity).
 */
int wa_build_block_index(const uint8_t* mask, int32_t H, int32_t MB, int32_t NB,
                         int32_t* row_ptr, int32_t* col_idx, int64_t col_capacity,
                         int32_t* row_nnz, int32_t* csc_ptr, int32_t* csc_idx,
                         int64_t csc_capacity, void* stream);

/* Parameters of wa_reorder_rows (host struct). */
typedef struct wa_reorder_params {
  int32_t wave;        /* W, rows per wave bucket (>= 1)                                */
  int32_t n_slices;    /* contiguous slices of the order, one per L2 domain (1..64);
                          1 reproduces [WA Algorithm 2] exactly; the XCD-sliced
                          attention schedule needs the device's XCD count here and
                          checks it (wa_sparse_attn_fwd perm_slices)                     */
  int32_t iters;       /* T of [WA Algorithm 1] (0..1000)                                */
  int32_t stage1;      /* 1: spectral polar order, 0: keep the row order                 */
  int32_t stage2;      /* 1: NNZ-descending order inside buckets, 0: off                  */
  int32_t skip_mode;   /* WA_SKIP_ADAPTIVE / WA_SKIP_NEVER / WA_SKIP_ALWAYS              */
  double ws_min_bytes; /* reorder only if the head's K/V bytes exceed this               */
  double flops_min;    /* ... and the selected FLOP of the heaviest head of the call
                          are at least this (the heads are reordered side by side, so
                          the call costs what its slowest head costs)                    */
  double jaccard_max;  /* ... and its adjacent-row Jaccard similarity is below this      */
} wa_reorder_params;

/*
 * wa_reorder_rows - [WA §IV, Algorithms 1 and 2] per-head query-block permutation.
 * Per head: statistics and the adaptive skip [WA §IV-E]; if not skipped, the rank-2
 * embedding of the column-centered mask by matrix-free centered subspace iteration
 * [WA §IV-C-2, Algorithm 1] from the start block x0, the optional Ritz rotation,
 * polar angles a_i = atan2(u2, u1) in [0, 2pi] [WA eq. (4)], a stable ascending
 * sort (Stage 1), buckets of at most `wave` positions inside `n_slices` contiguous
 * slices, and a stable NNZ-descending sort inside each bucket (Stage 2) [WA §IV-D].
 * Arithmetic is fp64.  Readings of open points: the start block is orthonormalised
 * by modified Gram-Schmidt; a second basis vector whose norm falls to <= 1e-12 of
 * the first is set to zero; each basis vector's sign makes its sum of cubes
 * positive (first entry > 1e-6 positive if |sum| < 1e-6); a mask whose rows are
 * all identical keeps the identity Stage-1 order; the skip rule reorders a head only
 * if K/V bytes NB*b*d*4 > ws_min_bytes, 4*b*b*d*max_h(nnz_h) >= flops_min (the work
 * of the call's heaviest head: one head's work pays for the call, and the other
 * heads are reordered alongside it at no extra cost) and the head's pooled Jaccard
 * similarity of adjacent rows < jaccard_max.
 *   row_ptr, col_idx, csc_ptr, csc_idx  from wa_build_block_index.  The CSC may be
 *             NULL when the head's mask fits in LDS as column bitmasks:
 *             (MB+NB)*16 + (NB*ceil(MB/32) + NB)*4 <= 155648 bytes (about
 *             MB = NB <= 972); the reorder then reads only the CSR
 *   capacity  number of entries col_idx and csc_idx hold; list entries at or beyond it
 *             are ignored (a truncated index never causes an out-of-bounds read)
 *   x0        float [H][MB][2]  raw start values (the random block of Algorithm 1)
 *   perm      int32 [H][MB] out  perm[h][pos] = query block executed at position pos
 *   inv_perm  int32 [H][MB] out  inv_perm[h][perm[h][pos]] = pos
 *   skipped   uint8 [H]     out  1 if the head kept the identity order
 *   angles    double [H][MB] out or NULL  polar angle per query block (NaN where
 *                                         Stage 1 did not run)
 *   stats     double [H][5] out or NULL  nnz, density, K/V bytes, selected FLOP,
 *                                        adjacent-row Jaccard (NaN when the skip was
 *                                        decided without it: WA_SKIP_ALWAYS, or the
 *                                        adaptive rule failing on bytes or FLOP, which
 *                                        skips the head before its mask is read)
 *   params    host pointer
 * Errors: WA_ERR_INVALID_ARG (null pointer, bad params, CSC missing where it is
 * required), WA_ERR_UNSUPPORTED (MB or NB > WA_MAX_BLOCKS, head_dim/block < 1),
 * WA_ERR_HIP.
 */
int wa_reorder_rows(const int32_t* row_ptr, const int32_t* col_idx, const int32_t* csc_ptr,
                    const int32_t* csc_idx, int64_t capacity, const float* x0, int32_t H,
                    int32_t MB, int32_t NB,
                    int32_t block, int32_t head_dim, const wa_reorder_params* params,
                    int32_t* perm, int32_t* inv_perm, uint8_t* skipped, double* angles,
                    double* stats, void* stream);

/*
 * wa_minhash_order - the MinHash comparator row order of [WA §VI, Table II
 * (comparison with other reordering algorithms)], from min-wise hashing of sets:
 * per head, row u's signature is sig_i(u) = min over the K/V blocks v of its list of
 * (hash_a[i] * v + hash_b[i]) mod (2^31 - 1), i < n_hash (an empty row gets 2^31 - 1
 * in each); rows are sorted by (sig_1, ..., sig_n_hash, row); with stage2 = 1 the
 * order then goes through the same wave buckets and NNZ-descending Stage 2 as
 * wa_reorder_rows [WA §IV-D].  No skip rule: every head is reordered.  Integer work,
 * bit-exact.
 *   row_ptr, col_idx, capacity  the CSR from wa_build_block_index
 *   hash_a, hash_b  host arrays of n_hash (1 or 2) coefficients, 1 <= a < 2^31 - 1,
 *                   0 <= b < 2^31 - 1 (drawn by the caller)
 *   wave, n_slices  the bucket geometry, as in wa_reorder_params
 *   perm, inv_perm  int32 [H][MB] out, as in wa_reorder_rows
 * Errors: WA_ERR_INVALID_ARG (null pointer, sizes, coefficients, n_hash, wave,
 * n_slices, stage2), WA_ERR_UNSUPPORTED (MB or NB > WA_MAX_BLOCKS), WA_ERR_HIP.
 */
int wa_minhash_order(const int32_t* row_ptr, const int32_t* col_idx, int64_t capacity, int32_t H,
                     int32_t MB, int32_t NB, const uint32_t* hash_a, const uint32_t* hash_b,
                     int32_t n_hash, int32_t wave, int32_t n_slices, int32_t stage2,
                     int32_t* perm, int32_t* inv_perm, void* stream);

/*
 * wa_lsh_order - the banded locality-sensitive-hashing comparator row order of
 * [WA §VI, Table II (comparison with other reordering algorithms)]: per head, band b
 * (b < n_bands <= 4) puts row u in the bucket (sig_2b(u), sig_2b+1(u)) of its MinHash
 * values (as in wa_minhash_order, hash functions 2b and 2b+1); each row is labelled
 * with the lowest row it shares a bucket with in any band (itself if none is lower,
 * no transitive closure) and rows are ordered by (label, row): a row and the higher
 * rows directly similar to it run together, groups in the order of their first row,
 * and a row that shares no bucket keeps its place relative to the others.  With
 * stage2 = 1 the same wave buckets and NNZ-descending Stage 2 follow [WA §IV-D].  No
 * skip rule.  Integer work, bit-exact.
 *   hash_a, hash_b  host arrays of 2 * n_bands coefficients, 1 <= a < 2^31 - 1,
 *                   0 <= b < 2^31 - 1 (drawn by the caller)
 *   other arguments as wa_minhash_order
 * Errors: WA_ERR_INVALID_ARG (null pointer, sizes, coefficients, n_bands, wave,
 * n_slices, stage2), WA_ERR_UNSUPPORTED (MB or NB > WA_MAX_BLOCKS), WA_ERR_HIP.
 */
int wa_lsh_order(const int32_t* row_ptr, const int32_t* col_idx, int64_t capacity, int32_t H,
                 int32_t MB, int32_t NB, const uint32_t* hash_a, const uint32_t* hash_b,
                 int32_t n_bands, int32_t wave, int32_t n_slices, int32_t stage2,
                 int32_t* perm, int32_t* inv_perm, void* stream);

/* 1 if wa_reorder_rows needs the CSC (csc_ptr, csc_idx) for an MB x NB mask,
 * 0 if it reads only the CSR (see wa_reorder_rows), negative on bad sizes. */
int wa_reorder_needs_csc(int32_t MB, int32_t NB);

/* Workspace bytes wa_sparse_attn_fwd needs for these sizes (host output): 256 bytes,
 * which hold the schedule wa_attn_schedule_select chooses for WA_SCHED_AUTO (K and V
 * are read in place). */
int wa_sparse_attn_workspace_size(int32_t H, int32_t L, int32_t head_dim, int32_t block,
                                  size_t* bytes);

/*
 * wa_sparse_attn_fwd - [WA §II-C; GSRS §3] block-sparse attention forward.
 * Query block u of head h attends to the tokens j < L of the K/V blocks listed in
 * col_idx[row_ptr[h*MB+u] .. row_ptr[h*MB+u+1]), in ascending order:
 *   LSE_i = ln sum_j exp(scale * q_i.k_j),  O_i = sum_j exp(scale * q_i.k_j - LSE_i) v_j.
 * A query block with no K/V block gets O = 0 and LSE = -inf [GSRS, fully masked rows].
 * Inputs are bf16; products accumulate in fp32 (bf16 MFMA); the softmax is fp32 and
 * the probabilities are rounded to bf16 before the P*V product.
 *   q, k, v   bf16 [H][L_pad][head_dim]; head_dim 64 or 128; block 64 or 128
 *   capacity  entries col_idx holds (and rows g holds); entries at or beyond it are
 *             skipped, as are block ids outside [0, MB): such an entry evaluates no
 *             key and its G row is -inf; a query block whose entries are all skipped
 *             gets O = 0 and LSE = -inf, like an empty one
 *   perm      int32 [H][MB] or NULL  execution order [WA §V]: position p of head h runs
 *             query block perm[h][p]; O, LSE and G stay in the original order (the
 *             permutation is applied by indexing, the inverse reorder is implicit)
 *   perm_slices  the n_slices the permutation's wave buckets were cut into (the
 *             reorder's parameter), 0 if unknown.  With perm != NULL and the
 *             XCD-sliced (or AUTO) schedule it must equal the device's XCD count
 *             (wa_schedule_info): slice x of each head's order runs on XCD x.
 *             Ignored when perm is NULL or the schedule is WA_SCHED_DEFAULT.
 *   schedule  WA_SCHED_NATURAL, WA_SCHED_XCD_SLICED, WA_SCHED_HEADS_INTERLEAVED,
 *             WA_SCHED_AUTO (reads the choice of wa_attn_schedule_select from workspace)
 *             or WA_SCHED_DEFAULT (resolved from the sizes, perm not read).
 *             XCD-sliced: workgroup w runs on XCD w mod n_xcd (round-robin dispatch,
 *             n_xcd = the device's XCD count, checked by wa_xcd_placement) and takes
 *             position floor(w / n_xcd) of slice (w mod n_xcd) of its head's order
 *   o         bf16 [H][L_pad][head_dim] out
 *   lse       float [H][L_pad] out, natural log
 *   g         float [row_ptr[H*MB]][block] out or NULL  [GSRS §5.3 Phase 1] for CSR
 *             entry e = (u, v) and row r of u, the block log-sum-exp
 *             G = m + ln sum_{j in v, j < L} exp(z_rj - m), m the block maximum
 *   workspace device buffer of at least wa_sparse_attn_workspace_size bytes
 * Errors: WA_ERR_INVALID_ARG (including perm_slices != the XCD count under the
 * XCD-sliced schedule), WA_ERR_UNSUPPORTED (head_dim/block), WA_ERR_CAPACITY
 * (workspace too small), WA_ERR_HIP.
 */
int wa_sparse_attn_fwd(const wa_bf16* q, const wa_bf16* k, const wa_bf16* v, int32_t H,
                       int32_t L, int32_t head_dim, int32_t block, const int32_t* row_ptr,
                       const int32_t* col_idx, int64_t capacity, const int32_t* perm,
                       int32_t perm_slices, int32_t schedule, float scale, wa_bf16* o,
                       float* lse, float* g, void* workspace, size_t workspace_bytes,
                       void* stream);

/*
 * wa_sparse_attn_fwd_noalloc - wa_sparse_attn_fwd for callers that cannot allocate
 * device memory or pass a workspace: code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc.  It allocates nothing: the 256-byte
 * schedule word that WA_SCHED_AUTO reads lives in a static device array of the
 * library (one copy per GPU, held until the process ends, its address looked up once
 * per device on the first call there).
 *   skipped   uint8 [H] (wa_reorder_rows) with WA_SCHED_AUTO: the call then enqueues
 *             the schedule choice of wa_attn_schedule_select into the static array
 *             before the attention; ignored (may be NULL) for the other schedules
 * Every other argument, the results and the errors are those of wa_sparse_attn_fwd,
 * plus WA_ERR_CAPACITY if these sizes needed more scratch than the static 256 bytes
 * (none does at present).  Calls that overlap on one GPU share its array and race:
 * enqueue them on one stream, or let one finish before the next starts.
 */
int wa_sparse_attn_fwd_noalloc(const wa_bf16* q, const wa_bf16* k, const wa_bf16* v, int32_t H,
                               int32_t L, int32_t head_dim, int32_t block, const int32_t* row_ptr,
                               const int32_t* col_idx, int64_t capacity, const int32_t* perm,
                               int32_t perm_slices, int32_t schedule, const uint8_t* skipped,
                               float scale, wa_bf16* o, float* lse, float* g, void* stream);

/*
 * wa_xcd_placement - [WA §II-C: a wave is the set of row tasks resident at once on
 * processors that share one L2] checks the dispatch the XCD-sliced schedule relies
 * on: launches n_wg workgroups of the attention kernel's size for `block` and writes,
 * for each, the XCD (L2 domain) it ran on, read from the XCC_ID hardware register.
 *   xcd_out  int32 [n_wg] out
 * Errors: WA_ERR_INVALID_ARG (null pointer, n_wg < 1), WA_ERR_UNSUPPORTED (block not
 * 64/128), WA_ERR_HIP.
 */
int wa_xcd_placement(int32_t n_wg, int32_t block, int32_t* xcd_out, void* stream);

/*
 * wa_attn_schedule_select - [WA §VI-F, Fig. 13: when the adaptive skip leaves every
 * head in its order, execution falls back to the default sparse-attention path]
 * writes into workspace the schedule WA_SCHED_AUTO runs: WA_SCHED_XCD_SLICED (in the
 * reordered order) if some skipped[h] is 0, WA_SCHED_DEFAULT (the permutation, all
 * identity, is then not read) if every one is non-zero.  One small kernel on the
 * device, so the choice follows the reorder without a host synchronisation.
 *   skipped   uint8 [H] from wa_reorder_rows
 *   workspace device buffer of at least wa_sparse_attn_workspace_size bytes, passed to
 *             the wa_sparse_attn_fwd calls that use WA_SCHED_AUTO afterwards
 * Errors: WA_ERR_INVALID_ARG (null pointer, H < 1), WA_ERR_CAPACITY (workspace too
 * small), WA_ERR_HIP.
 */
int wa_attn_schedule_select(const uint8_t* skipped, int32_t H, void* workspace,
                            size_t workspace_bytes, void* stream);

/*
 * wa_default_schedule - [WA §VI-F: the default path when no head is reordered] the
 * schedule WA_SCHED_DEFAULT runs for these sizes (host only, no device work):
 * WA_SCHED_HEADS_INTERLEAVED if MB * block * head_dim * 4 <= WA_ALL_HEADS_MAX_KV_BYTES
 * (MB = ceil(L / block)), else WA_SCHED_XCD_SLICED.
 *   schedule  int32 host out
 * Errors: WA_ERR_INVALID_ARG (null pointer, L < 1), WA_ERR_UNSUPPORTED (head_dim or
 * block not 64/128).
 */
int wa_default_schedule(int32_t L, int32_t head_dim, int32_t block, int32_t* schedule);

/*
 * wa_sparse_attn_fwd_diag - wa_sparse_attn_fwd that also writes per-row attention
 * statistics from the same pass [GSRS §4, Fig. 1 (attention entropy and mean
 * attention distance across denoising steps), and its appendix on computing both
 * inside the attention kernel with two running sums rescaled like the output]:
 *   entropy[h][i]  = -sum_j A_ij ln A_ij, computed as LSE_i - E[z_ij] (E under A,
 *                    z = scale * q.k)
 *   distance[h][i] = sum_j A_ij |i - j|, i and j token positions in the stored order
 * over the row's attended keys.  A row with no keys gets 0 in both.  Values for rows
 * >= L are unspecified.  All other arguments and errors as wa_sparse_attn_fwd, plus
 * WA_ERR_INVALID_ARG when both outputs are NULL.
 *   entropy   float [H][L_pad] out or NULL
 *   distance  float [H][L_pad] out or NULL
 */
int wa_sparse_attn_fwd_diag(const wa_bf16* q, const wa_bf16* k, const wa_bf16* v, int32_t H,
                            int32_t L, int32_t head_dim, int32_t block, const int32_t* row_ptr,
                            const int32_t* col_idx, int64_t capacity, const int32_t* perm,
                            int32_t perm_slices, int32_t schedule, float scale, wa_bf16* o,
                            float* lse, float* g, float* entropy, float* distance,
                            void* workspace, size_t workspace_bytes, void* stream);

/*
 * wa_block_importance - [GSRS §5.3 Phase 2, Appendix A.2] block weights.
 * For CSR entry e = (h, u, v): W[e] = (1/B_u) sum over the valid rows i of query
 * block u of exp(G[e][i] - LSE_i), B_u = number of rows of u below L; rows with
 * LSE = -inf add nothing.  Each non-empty row of W sums to 1.
 *   g    float [capacity][block], lse float [H][L_pad], w float [capacity] out; entries
 *        at or beyond capacity are skipped
 * Errors: WA_ERR_INVALID_ARG, WA_ERR_HIP.
 */
int wa_block_importance(const float* g, const float* lse, const int32_t* row_ptr,
                        int64_t capacity, int32_t H, int32_t MB, int32_t L, int32_t block,
                        float* w, void* stream);

/*
 * wa_topp_select - [GSRS Algorithm 3] Top-p block selection per query block.
 * The candidates of a row (its CSR entries) are sorted by descending W, equal W by
 * ascending block id; their W are summed in fp64 in that order and a block is kept
 * while the sum before it is <= p (the block that takes the sum above p is the last
 * one kept).  Restricting a second selection to the first selection's index gives
 * the reduced search of GSRS.
 *   w        float [capacity], col_idx int32 [capacity]; entries at or beyond capacity
 *            are not candidates
 *   mask_out uint8 [H][MB][NB] out (fully overwritten)
 * Errors: WA_ERR_INVALID_ARG (p outside (0, 1], null pointers), WA_ERR_UNSUPPORTED
 * (NB > WA_MAX_BLOCKS), WA_ERR_HIP.
 */
int wa_topp_select(const float* w, const int32_t* row_ptr, const int32_t* col_idx,
                   int64_t capacity, int32_t H, int32_t MB, int32_t NB, double p,
                   uint8_t* mask_out, void* stream);

/*
 * wa_mask_recall - [GSRS §3, attention recall] the share of the attention weight
 * that a block mask keeps, per query block.  With w the block weights of a pass
 * over the evaluated blocks (wa_block_importance after a wa_sparse_attn_fwd with
 * g, e.g. over all blocks for the full attention), recall[h][u] is the sum of
 * w[e] over the CSR entries e = (h, u, v) whose block v the mask keeps: the mean,
 * over the valid rows of u, of the attention those rows put on the kept blocks.
 * The sum runs in fp64 in a fixed order.  A row with no entries gets 0.
 *   w          float [capacity], row_ptr int32 [H*MB+1], col_idx int32 [capacity]:
 *              the index and weights of the evaluated pass
 *   mask       uint8 [H][MB][NB], non-zero = kept
 *   recall_out float [H][MB] out
 * Errors: WA_ERR_INVALID_ARG, WA_ERR_UNSUPPORTED (NB > WA_MAX_BLOCKS), WA_ERR_HIP.
 */
int wa_mask_recall(const float* w, const int32_t* row_ptr, const int32_t* col_idx,
                   int64_t capacity, int32_t H, int32_t MB, int32_t NB, const uint8_t* mask,
                   float* recall_out, void* stream);

/*
 * wa_gather_blocks / wa_scatter_blocks - [WA §V] explicit reorder operators.
 * Row blocks of block_bytes bytes: gather dst[h][s] = src[h][perm[h][s]];
 * scatter dst[h][perm[h][s]] = src[h][s].  Used for Q blocks, mask rows, O and
 * LSE when the permutation is applied as copies instead of by indexing.
 * src and dst must not overlap; perm entries outside [0, MB) are skipped.
 * Errors: WA_ERR_INVALID_ARG, WA_ERR_HIP.
 */
int wa_gather_blocks(const void* src, void* dst, const int32_t* perm, int32_t H, int32_t MB,
                     int64_t block_bytes, void* stream);
int wa_scatter_blocks(const void* src, void* dst, const int32_t* perm, int32_t H, int32_t MB,
                      int64_t block_bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* WAVEALIGN_H */
