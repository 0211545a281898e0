/*
 * sparse_attn.h -- C ABI of the MI355X (gfx950) sparse attention library.
 *
 * Operations, all launched asynchronously on the caller's HIP stream:
 *
 *   sparse_attn_build_mask   block mask -> CSR key-block lists on the device
 *   sparse_attn_fwd          block-sparse attention over a CSR mask
 *   offset_attn_fwd          token-level attention over a table of distances
 *
 * with the offset_attn_fwd_interp variant, the backward passes
 * (sparse_attn_mask_transpose, sparse_attn_bwd, offset_attn_bwd) and host helpers
 * (sparse_attn_mask_capacity, sparse_attn_literal_flags, offset_attn_make_table,
 * offset_attn_make_table_ratio, offset_attn_make_interp).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - Pointers are DEVICE pointers unless documented as HOST.
 *  - The caller owns all memory.  The library never allocates, frees or
 *    synchronises; every kernel goes on `stream` (NULL = the null stream).
 *  - Argument errors are detected on the host before anything is launched and
 *    nothing is written.  A failed launch returns SA_ERR_HIP and
 *    sa_last_hip_error() describes it (thread-local text).  The library never
 *    prints and never aborts.
 *  - Tensors are [B, H, N, d] (K and V: [B, H_kv, N, d]) with d contiguous.
 *    `strides` (HOST, may be NULL) gives for q, k, v, o in that order the
 *    batch, head and sequence strides in ELEMENTS (int64 [4][3]); NULL means
 *    contiguous.  Rows must be 16-byte aligned: every stride must be a
 *    multiple of 8 elements (bf16) or 4 elements (fp32), and base pointers
 *    16-byte aligned.
 *  - Head h reads K/V head h / (H / H_kv) (grouped-query attention).
 *  - lse is fp32 [B, H, N], contiguous, natural-log log-sum-exp of the scaled
 *    logits of each query row; a query with no allowed key gets o = 0 and
 *    lse = -inf.
 *  - O is written in the input dtype, rounded to nearest even.
 *  - Thread safety: the library keeps no state besides the thread-local error
 *    text; calls are reentrant.  Calls that write the same buffers race.
 */
#ifndef SPARSE_ATTN_H
#define SPARSE_ATTN_H

#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef int32_t sa_status;
enum {
  SA_OK = 0,
  SA_ERR_NULL = -1,        /* a required pointer is NULL                       */
  SA_ERR_INVALID = -2,     /* a size, stride, flag or list is out of range     */
  SA_ERR_UNSUPPORTED = -3, /* valid, but outside the compiled kernel set       */
  SA_ERR_CAPACITY = -4,    /* an output buffer is smaller than required        */
  SA_ERR_HIP = -5          /* the HIP runtime reported an error                */
};

enum { SA_F32 = 0, SA_BF16 = 1 };

/* Long-range "literal" component of the block mask. */
enum {
  SA_LIT_NONE = 0,
  SA_LIT_PAIR = 1, /* row i attends literal block j iff l_i = l_j = 1 (both literal) */
  SA_LIT_ANYQ = 2  /* row i attends every literal block j (query flag ignored)      */
};

#define SA_MAX_GLOBAL 64   /* global blocks per mask                       */
#define SA_MAX_RANDOM 32   /* random blocks per row                        */
#define SA_MAX_BLOCKS 16384 /* blocks per sequence (num_blocks)            */
#define SA_MAX_OFFSETS 128 /* distances per offset table                   */
#define SA_MAX_RUNGS 64    /* interpolated rungs per offset call            */
#define SA_MAX_SPLIT_WAYS 16 /* workgroups sharing one split forward row    */
#define SA_SPLIT_COUNTERS 16384 /* split forward rows per launch (B * H * split_rows) */

/*
 * Block mask description (HOST struct, passed by host pointer).
 *
 * Row i of group g lists, ascending and without repeats, the key blocks j of
 *
 *    I    {i}                        -- "Parameter-free Adaptive Sparse
 *                                       Attention via Compression-Based Content
 *                                       Selection", Sec. 3.2 Eq. 3
 *    W    local window:  causal  {j : i - win_before <= j <= i}
 *                        non-causal, win_clamp = 0: [i - win_before, i + win_after]
 *                        non-causal, win_clamp = 1: the same width shifted inside
 *                           [0, num_blocks) so every row keeps exactly
 *                           win_before + win_after + 1 blocks ("BigBird" Sec. 2,
 *                           |G_W| = N w)
 *    G    global: every row attends the global blocks, a global row attends
 *         every block ("BigBird" Sec. 2, |G_G| = 2gN - g^2)
 *    R    num_random distinct uniform draws ("BigBird" Sec. 2, |G_R| = N r),
 *         from [0, i) when causal (earlier blocks only) else [0, num_blocks)
 *    L    literal blocks outside the window band [i - win_before, i + win_after]
 *         (compression paper Sec. 3.2, M^lit), per literal_mode
 *
 * intersected with j <= i when causal.
 *
 * Random draws: `random_blocks` (DEVICE int32 [G][num_blocks][num_random]) gives
 * them explicitly; entries outside the allowed range are ignored and repeats
 * count once.  If NULL they are drawn with the library's counter-based
 * SplitMix64 scheme keyed by (seed, 2, g, i, k): candidate k is
 * ((key >> 32) * n) >> 32, repeats skipped, stop at min(r, n) values or 64 r
 * candidates.
 *
 * Literal flags: `literal_flags` (DEVICE uint8 [F][num_blocks], nonzero =
 * literal; F = G, or ceil(G / P) with a group period P) gives them explicitly;
 * if NULL, block j of flag group f is literal iff
 * (key(seed, 1, f, j, 0) >> 32) < floor(literal_p * 2^32).  Group g reads flag
 * group f = g (f = g / P with a period).
 * key(seed, t, a, b, c) = sm(sm(sm(sm(sm(seed) ^ t) ^ a) ^ b) ^ c) with sm the
 * SplitMix64 output function (Steele, Lea & Flood, OOPSLA 2014).
 */
/* Components of the union that a mask may leave out (sa_mask_desc.exclude_parts,
 * and per group through group_period / period_exclude).  The identity is always
 * kept.  The compression paper's head groups (Sec. 3.3) are: local heads =
 * window U I (exclude SA_PART_LITERAL), long-range heads = literal U I (exclude
 * SA_PART_WINDOW; the literal component still skips the window band
 * |i - j| <= w), hybrid heads = the full mask.  With one mask group per
 * (sequence, head), g = b * H + h, group_period = H and period_exclude[h] = the
 * head's exclusions, every head of a sequence shares that sequence's literal
 * flags (row b) and sparse_attn_fwd takes mask_batch_stride = H,
 * mask_head_stride = 1. */
#define SA_MAX_PERIOD 64
enum {
  SA_PART_WINDOW = 1,
  SA_PART_GLOBAL = 2,
  SA_PART_RANDOM = 4,
  SA_PART_LITERAL = 8,
};

typedef struct sa_mask_desc {
  int32_t num_blocks;           /* N_b = N / block, 1..SA_MAX_BLOCKS              */
  int32_t num_groups;           /* G >= 1 independent masks                        */
  int32_t causal;               /* 0 or 1                                          */
  int32_t win_before;           /* >= 0                                            */
  int32_t win_after;            /* >= 0; must be 0 when causal                     */
  int32_t win_clamp;            /* 0 or 1 (non-causal only)                        */
  const int32_t* global_blocks; /* HOST, ascending, unique, in [0, N_b); NULL if 0 */
  int32_t num_global;           /* 0..SA_MAX_GLOBAL                                */
  int32_t num_random;           /* 0..SA_MAX_RANDOM                                */
  const int32_t* random_blocks; /* DEVICE [G][N_b][num_random] or NULL             */
  int32_t literal_mode;         /* SA_LIT_*                                        */
  const uint8_t* literal_flags; /* DEVICE [G][N_b] or NULL                         */
  double literal_p;             /* in [0, 1]; used when literal_flags is NULL      */
  uint64_t seed;
  int32_t exclude_parts;        /* SA_PART_* bits left out of every group's union  */
  int32_t group_period;         /* P, 0..SA_MAX_PERIOD; 0 = no per-group pattern    */
  int32_t period_exclude[SA_MAX_PERIOD]; /* when P > 0: group g also leaves out
                                   period_exclude[g % P], and reads its literal
                                   flags (explicit or drawn) as group g / P     */
} sa_mask_desc;

/* Entries col_idx must hold for sparse_attn_build_mask: the largest number of
 * CSR entries the mask can have (G * N_b * (N_b + 1) / 2 when causal,
 * G * N_b * N_b otherwise) plus G * N_b entries of scratch (the row lengths,
 * kept past the CSR while it is built).
 * Returns a negative sa_status if the description is invalid. */
int64_t sparse_attn_mask_capacity(const sa_mask_desc* desc);

/* Check a mask description without launching anything. */
sa_status sparse_attn_check_mask_desc(const sa_mask_desc* desc);

/*
 * Build the CSR form of the mask on the device.
 *   row_ptr  DEVICE int32 [G * N_b + 1]: row (g, i) is entries
 *            [row_ptr[g*N_b + i], row_ptr[g*N_b + i + 1]) of col_idx.
 *   col_idx  DEVICE int32 [col_capacity]; col_capacity must be at least
 *            sparse_attn_mask_capacity(desc) (SA_ERR_CAPACITY otherwise).
 *   sched    DEVICE int32 [G][N_b] or NULL: per group, the row ids ordered by
 *            decreasing row length, ties by increasing row id (a longest-first
 *            launch order for sparse_attn_fwd).
 * Kernels on `stream`: count, then fill with the prefix sum folded in (up to
 * 8192 rows; larger masks take a separate prefix-sum kernel between them).
 * The result is unique (bit-exact for a given description); col_idx entries
 * past the CSR are scratch.
 */
sa_status sparse_attn_build_mask(const sa_mask_desc* desc, int32_t* row_ptr, int32_t* col_idx,
                                 int64_t col_capacity, int32_t* sched, hipStream_t stream);

/*
 * Literal flags from byte content (compression paper, Sec. 3.1, Eq. 1-2;
 * Appendix B, Algorithm 1 steps 1-2).  Host only: no GPU work.
 * Each of G sequences of n_bytes bytes is cut into B = n_bytes / block_bytes
 * blocks; c_i = size in bytes of block i compressed on its own by gzip at
 * `level` (zlib deflate, gzip container, window 15, memory level 8, default
 * strategy); block i is literal iff c_i * B > sum_j c_j, i.e. its compression
 * ratio c_i / block_bytes is above the sequence mean.
 *   bytes      HOST uint8 [G][n_bytes]
 *   flags_out  HOST uint8 [G][B] (1 = literal); copy to the device to use as
 *              sa_mask_desc.literal_flags
 *   sizes_out  HOST int32 [G][B] or NULL: the compressed sizes c_i
 *   level      1..9 (the paper uses 1)
 * SA_ERR_INVALID if n_bytes % block_bytes != 0 or a size is out of range;
 * SA_ERR_UNSUPPORTED if B > SA_MAX_BLOCKS; argument errors return before
 * anything is written.
 */
sa_status sparse_attn_literal_flags(const uint8_t* bytes, int32_t G, int64_t n_bytes, int32_t block_bytes,
                                    int32_t level, uint8_t* flags_out, int32_t* sizes_out);

/*
 * Block-sparse attention forward.
 *
 * For token t in query block qb = t / block of (b, h), with mask row
 * r = g * N_b + qb, g = b * mask_batch_stride + h * mask_head_stride:
 *   K(t) = tokens of the key blocks col_idx[row_ptr[r] .. row_ptr[r+1]),
 *          restricted to s <= t when causal (the diagonal block is partially
 *          masked; blocks after the query block contribute nothing);
 *   o_t  = softmax_s(scale * <q_t, k_s>) . v_s over s in K(t);
 *   lse_t = ln sum_s exp(scale * <q_t, k_s>).
 * This is the block mask expanded to tokens and ANDed with the causal triangle
 * (compression paper Sec. 3.4 and Appendix B Algorithm 1 step 4), evaluated
 * without materialising it.
 *
 *   dtype      SA_BF16 (MFMA path) or SA_F32
 *   d, block   each 64 or 128; N % block == 0
 *   row_ptr/col_idx  as built by sparse_attn_build_mask (any canonical CSR:
 *              rows ascending and unique).  Column ids outside [0, N_b) are
 *              skipped; entries beyond col_capacity are never read.
 *   sched      DEVICE int32 [num_groups][N_b] launch order or NULL.
 *   num_groups G; (B-1)*mask_batch_stride + (H-1)*mask_head_stride < G,
 *              strides >= 0.
 *   scale      logit scale, e.g. 1/sqrt(d) (any finite value, 0 and < 0 included)
 *   row_split  1 or 2 (else SA_ERR_INVALID): wave groups sharing one mask row
 *              in the bf16 path.  2 splits every row's key tiles over two
 *              groups whose softmax states are merged at the end: shorter
 *              critical path when a few rows are much longer than the rest
 *              (global rows of a non-causal mask), more waves per row
 *              otherwise.  Same results up to fp32 summation order; the fp32
 *              path ignores it.
 *   split_rows 0 .. N_b (else SA_ERR_INVALID), bf16 with row_split = 1 only
 *              (SA_ERR_INVALID otherwise; the fp32 path ignores it): the rows
 *              at the first split_rows launch positions of every (b, h) --
 *              the longest ones when sched is the longest-first order -- are
 *              each run by split_ways workgroups, part p taking the row's key
 *              tiles p, p + split_ways, ...; the last part to finish merges
 *              the partial softmax states.  Shortens the critical path of rows
 *              much longer than the rest (the global rows of a non-causal
 *              mask); results equal those of whole rows up to fp32 summation
 *              order (bit-identical from launch to launch).
 *   split_ways 2 .. SA_MAX_SPLIT_WAYS when split_rows > 0 (else ignored).
 *   workspace  DEVICE, 16-byte aligned, when split_rows > 0 (else ignored,
 *              may be NULL): workspace_bytes >= sparse_attn_fwd_workspace_bytes
 *              (B, H, d, block, split_rows, split_ways) (SA_ERR_CAPACITY
 *              otherwise; SA_ERR_NULL when NULL).  Its first
 *              SA_SPLIT_COUNTERS int32 (64 KiB, the same for every split
 *              shape) are arrival counters that must be zero when the
 *              workspace is first used; every launch leaves them zero, so a
 *              workspace zeroed once serves later launches of any shape
 *              whose size it covers.  Launches that share a workspace must
 *              not overlap in time.
 *              SA_ERR_UNSUPPORTED when B * H * split_rows > SA_SPLIT_COUNTERS.
 *   SA_ERR_UNSUPPORTED for bf16 when a K or V sequence stride is >= 2^24
 *              elements.
 */
sa_status sparse_attn_fwd(int32_t dtype, const void* q, const void* k, const void* v, void* o,
                          float* lse, int32_t B, int32_t H, int32_t H_kv, int32_t N, int32_t d,
                          int32_t block, const int64_t* strides, const int32_t* row_ptr,
                          const int32_t* col_idx, int64_t col_capacity, const int32_t* sched,
                          int32_t num_groups, int64_t mask_batch_stride, int64_t mask_head_stride,
                          int32_t causal, float scale, int32_t row_split, int32_t split_rows,
                          int32_t split_ways, void* workspace, int64_t workspace_bytes,
                          hipStream_t stream);

/*
 * sparse_attn_fwd without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc).  It allocates nothing: the split-row
 * workspace is a static device array of SA_NOALLOC_SCRATCH_BYTES held by every
 * device the library runs on until the process ends.  Arguments, results and
 * errors as for sparse_attn_fwd (workspace and workspace_bytes left out), plus
 * SA_ERR_CAPACITY when sparse_attn_fwd_workspace_bytes(B, H, d, block,
 * split_rows, split_ways) exceeds SA_NOALLOC_SCRATCH_BYTES (for example the
 * BigBird workload's split, 2 rows x 8 ways of 24 heads at d = 64, needs
 * 6.8 MB).  With split_rows > 0 (bf16) each call first zeroes the arrival
 * counters it uses with a small kernel on `stream`, then launches the
 * forward.  All calls on one device share its array: calls that overlap in
 * time on one device (other streams, other threads) race and must not be
 * issued; calls with split_rows = 0 or fp32 touch no scratch.
 */
#define SA_NOALLOC_SCRATCH_BYTES (16 << 20)
sa_status sparse_attn_fwd_noalloc(int32_t dtype, const void* q, const void* k, const void* v, void* o,
                                  float* lse, int32_t B, int32_t H, int32_t H_kv, int32_t N, int32_t d,
                                  int32_t block, const int64_t* strides, const int32_t* row_ptr,
                                  const int32_t* col_idx, int64_t col_capacity, const int32_t* sched,
                                  int32_t num_groups, int64_t mask_batch_stride, int64_t mask_head_stride,
                                  int32_t causal, float scale, int32_t row_split, int32_t split_rows,
                                  int32_t split_ways, hipStream_t stream);

/* Bytes of the split-row workspace of sparse_attn_fwd: 0 when split_rows = 0,
 * else 4 * SA_SPLIT_COUNTERS bytes of counters followed by the partial
 * states; SA_ERR_INVALID / SA_ERR_UNSUPPORTED (negative) for invalid sizes
 * (SA_ERR_UNSUPPORTED when B * H * split_rows > SA_SPLIT_COUNTERS). */
int64_t sparse_attn_fwd_workspace_bytes(int32_t B, int32_t H, int32_t d, int32_t block, int32_t split_rows,
                                        int32_t split_ways);

/*
 * Offset table of "Depth-Staggered Fibonacci Spacing for Sparse Attention",
 * Sec. 2 ("Attended set"): the distinct distances
 *   {0, 1, ..., W}  U  {floor(alpha * base[k] + 1/2) : k < K}
 * that lie in [0, N), ascending.  Host only.
 *   base       HOST int64 [K], each >= 0 (e.g. 1, 2, 3, 5, 8, ... below N)
 *   table_out  HOST int32 [capacity]; count_out HOST int32 receives the size.
 * SA_ERR_CAPACITY if the table does not fit (nothing written).
 */
sa_status offset_attn_make_table(int32_t W, double alpha, const int64_t* base, int32_t K, int32_t N,
                                 int32_t* table_out, int32_t capacity, int32_t* count_out);

/*
 * The same table with alpha = num / den held exactly (e.g. the linear stagger
 * alpha = 0.5 + l / (L - 1) of the same page, Sec. 2, "The per-layer
 * scalar", as (L - 1 + 2 l) / (2 (L - 1))): each rung is
 * floor(num * base[k] / den + 1/2) computed in integers, so rungs that land
 * exactly on a half round up, which a double-precision alpha cannot promise.
 *   0 <= num < 2^31, 1 <= den < 2^31, 0 <= base[k] < 2^31 (else SA_ERR_INVALID)
 */
sa_status offset_attn_make_table_ratio(int32_t W, int64_t num, int64_t den, const int64_t* base,
                                       int32_t K, int32_t N, int32_t* table_out, int32_t capacity,
                                       int32_t* count_out);

/*
 * Split of the key set for the interpolated gather of continuous distances
 * d_k = alpha * base[k] (same page, Sec. 2, "Attended set" and
 * "Implementation note": the key / value of a rung is the linear
 * interpolation between the rows at distances floor(d_k) and floor(d_k) + 1).
 * Host only.
 *   table_out  HOST int32 [capacity]: ascending distinct integer distances:
 *              {0..W} and every rung whose d_k (double) is an integer, in [0, N)
 *   rung_floor HOST int32 [rung_capacity], rung_weight HOST float
 *              [rung_capacity]: the other rungs in base order as
 *              (a, w) = (floor(d_k), d_k - floor(d_k)), 0 < w < 1; a rung with
 *              a + 1 > N - 1 reaches no query and is dropped, and so is a
 *              negative d_k
 *   count_out, rung_count  HOST int32: sizes written
 * With every d_k an integer the table equals offset_attn_make_table's.
 * SA_ERR_CAPACITY if either output does not fit (nothing written).
 */
sa_status offset_attn_make_interp(int32_t W, double alpha, const int64_t* base, int32_t K, int32_t N,
                                  int32_t* table_out, int32_t capacity, int32_t* count_out,
                                  int32_t* rung_floor, float* rung_weight, int32_t rung_capacity,
                                  int32_t* rung_count);

/*
 * Offset attention forward: query t attends keys {t - delta : delta in
 * offsets, t - delta >= 0} (same page, Sec. 2: shifted gathers shared by all
 * queries; the self distance 0 keeps every key set non-empty).
 *   offsets    HOST int32 [num_offsets], ascending, unique, 0 <= delta < N,
 *              1 <= num_offsets <= SA_MAX_OFFSETS
 *   dtype      SA_BF16 or SA_F32; d 64 or 128; any N >= 1
 */
sa_status offset_attn_fwd(int32_t dtype, const void* q, const void* k, const void* v, void* o,
                          float* lse, int32_t B, int32_t H, int32_t H_kv, int32_t N, int32_t d,
                          const int64_t* strides, const int32_t* offsets, int32_t num_offsets,
                          float scale, hipStream_t stream);

/*
 * Offset attention with interpolated rungs (same page, Sec. 2, "Attended
 * set"): query t attends keys {t - delta : delta in offsets, t - delta >= 0}
 * and, for each rung r with t >= rung_floor[r] + 1, one more key / value
 *   (1 - w) row[t - a] + w row[t - a - 1],  a = rung_floor[r], w = rung_weight[r]
 * of K and V (each rung is its own key, also where it meets an integer
 * distance).  Rungs may come in any order.
 *   offsets     HOST int32 [num_offsets] as for offset_attn_fwd, but
 *               0 <= num_offsets <= SA_MAX_OFFSETS
 *   rung_floor  HOST int32 [num_rungs], 0 <= a and a + 1 <= N - 1
 *   rung_weight HOST float [num_rungs], 0 <= w <= 1
 *   0 <= num_rungs <= SA_MAX_RUNGS, num_offsets + num_rungs >= 1
 * Other arguments, outputs and errors as for offset_attn_fwd.
 */
sa_status offset_attn_fwd_interp(int32_t dtype, const void* q, const void* k, const void* v, void* o,
                                 float* lse, int32_t B, int32_t H, int32_t H_kv, int32_t N, int32_t d,
                                 const int64_t* strides, const int32_t* offsets, int32_t num_offsets,
                                 const int32_t* rung_floor, const float* rung_weight, int32_t num_rungs,
                                 float scale, hipStream_t stream);

/*
 * Backward pass (gradients of the loss L through o): given dO = dL/do, the
 * gradients of masked softmax attention, from the saved lse,
 *     D_t = <dO_t, o_t>,  p_ts = exp(scale <q_t, k_s> - lse_t),
 *     dv_s = sum_t p_ts dO_t,  ds_ts = p_ts (<dO_t, v_s> - D_t),
 *     dq_t = scale sum_s ds_ts k_s,  dk_s = scale sum_t ds_ts q_t
 * over the allowed pairs (every page trains through the forward; the lse it
 * returns is kept for this).  Grouped-query heads add into their K/V head.
 */

/*
 * Transpose of a block mask: for every group g and key block j, the query
 * blocks i whose CSR row lists j, ascending (rows must be ascending, as the
 * builder writes them).  Entries outside [0, N_b) are ignored.
 *   row_ptr, col_idx  DEVICE, as written by sparse_attn_build_mask
 *   col_ptr           DEVICE int32 [G * N_b + 1] (written)
 *   row_idx           DEVICE int32 [row_capacity] (written; row_capacity >=
 *                     the number of mask entries keeps every entry)
 */
sa_status sparse_attn_mask_transpose(int32_t num_groups, int32_t num_blocks, const int32_t* row_ptr,
                                     const int32_t* col_idx, int64_t col_capacity, int32_t* col_ptr,
                                     int32_t* row_idx, int64_t row_capacity, hipStream_t stream);

/*
 * Block-sparse attention backward over the mask used by sparse_attn_fwd
 * (row_ptr / col_idx) and its transpose (col_ptr / row_idx from
 * sparse_attn_mask_transpose).
 *   q, k, v, o, lse  the forward's inputs and outputs; dout = dO [B, H, N, d]
 *   dq [B, H, N, d], dk, dv [B, H_kv, N, d]  DEVICE, written (input dtype)
 *   workspace        DEVICE, 16-byte aligned, workspace_bytes >=
 *                    sparse_attn_bwd_workspace_bytes(B, H, H_kv, N, d, block)
 *                    (else SA_ERR_CAPACITY): per-row {lse log2(e), D}, the
 *                    dK/dV work list, and fp32 partial dK/dV of key blocks
 *                    listed by more than L (query block, q head) pairs of
 *                    their K/V head, L = the mask's entries per resident
 *                    dK/dV workgroup, clamped to 16 .. 64; those are split
 *                    over several workgroups and their partial sums added
 *                    with fp32 atomics, so their low-order bits may differ
 *                    from run to run
 *   sched            DEVICE int32 [num_groups][N_b] or NULL: the launch order
 *                    of the dQ rows, as for sparse_attn_fwd (the
 *                    longest-first order of sparse_attn_build_mask shortens
 *                    the tail when a few rows are much longer than the rest);
 *                    each group's list must be a permutation of 0 .. N_b - 1
 *                    (a row id outside [0, N_b) leaves a dQ block unwritten).
 *                    Results do not depend on it; the fp32 path ignores it.
 *   strides          HOST int64 [8][3] for q, k, v, o, dout, dq, dk, dv
 *                    (batch, head, sequence strides in elements) or NULL; for
 *                    bf16 the sequence strides of q, k, v, dout must be below
 *                    2^24 elements (else SA_ERR_UNSUPPORTED)
 * Other arguments, layouts, supported sizes and errors as for sparse_attn_fwd.
 */
int64_t sparse_attn_bwd_workspace_bytes(int32_t B, int32_t H, int32_t H_kv, int32_t N, int32_t d,
                                        int32_t block);
sa_status sparse_attn_bwd(int32_t dtype, const void* q, const void* k, const void* v, const void* o,
                          const float* lse, const void* dout, void* dq, void* dk, void* dv, void* workspace,
                          int64_t workspace_bytes, int32_t B, int32_t H, int32_t H_kv, int32_t N, int32_t d,
                          int32_t block,
                          const int64_t* strides, const int32_t* row_ptr, const int32_t* col_idx,
                          int64_t col_capacity, const int32_t* sched, const int32_t* col_ptr,
                          const int32_t* row_idx, int64_t row_capacity, int32_t num_groups,
                          int64_t mask_batch_stride,
                          int64_t mask_head_stride, int32_t causal, float scale, hipStream_t stream);

/*
 * Offset attention backward over the table used by offset_attn_fwd.
 * Tensors and strides as for sparse_attn_bwd; delta is a DEVICE fp32
 * [B, H, N] workspace (written with D); offsets as for offset_attn_fwd.
 */
sa_status offset_attn_bwd(int32_t dtype, const void* q, const void* k, const void* v, const void* o,
                          const float* lse, const void* dout, void* dq, void* dk, void* dv, float* delta,
                          int32_t B, int32_t H, int32_t H_kv, int32_t N, int32_t d, const int64_t* strides,
                          const int32_t* offsets, int32_t num_offsets, float scale, hipStream_t stream);

/*
 * The library's counter-based draws, evaluated on the host by the same code
 * the mask kernels run (for checks without a GPU; no page fixes a generator,
 * this is the library's convention).  sm = SplitMix64 output function (Steele,
 * Lea & Flood, OOPSLA 2014).
 *   sa_rng_key            key(seed, tag, a, b, c) = sm(sm(sm(sm(sm(seed) ^ tag) ^ a) ^ b) ^ c)
 *   sa_rng_literal        the drawn literal flag of block `block` of flag group
 *                         `group`: (key(seed, 1, group, block, 0) >> 32) <
 *                         floor(p * 2^32) (clamped to [0, 2^32]) -> 1 / 0
 *   sa_rng_random_blocks  the drawn random blocks of row `row` of group
 *                         `group` over [0, n): candidate k = ((key(seed, 2,
 *                         group, row, k) >> 32) * n) >> 32, repeats skipped,
 *                         stop at min(r, n) values or 64 r candidates; writes
 *                         them in draw order to `out` (HOST int32 [r]) and
 *                         returns their count, or SA_ERR_NULL / SA_ERR_INVALID
 *                         (n < 0, r < 0 or r > SA_MAX_RANDOM)
 * sparse_attn_build_mask (literal_flags / random_blocks NULL) uses exactly these
 * draws, with n = i (causal) or N_b (non-causal).
 */
uint64_t sa_rng_key(uint64_t seed, uint64_t tag, uint64_t a, uint64_t b, uint64_t c);
int32_t sa_rng_literal(uint64_t seed, uint64_t group, uint64_t block, double p);
int32_t sa_rng_random_blocks(uint64_t seed, uint64_t group, uint64_t row, int32_t n, int32_t r, int32_t* out);

/*
 * Shader-clock probe (measurement aid, not part of the attention path): one
 * wave on `stream` counts shader-clock cycles (s_memtime) while at least
 * `ticks` ticks of the constant-rate counter (s_memrealtime, the device's wall
 * clock, 100 MHz on MI355X) pass, and writes out[0] = cycles, out[1] = ticks
 * (DEVICE int64 [2]).  Run beside a workload on another stream, cycles / ticks
 * x the wall-clock rate is the clock the workload ran at.
 * 0 <= ticks <= 6e9 (else SA_ERR_INVALID).
 */
sa_status sa_clock_probe(int64_t* out, int64_t ticks, hipStream_t stream);

const char* sa_status_string(sa_status s);
const char* sa_last_hip_error(void);
int32_t sa_version(void);

/* Layout of sa_mask_desc for bindings: writes min(n, 18) values -- sizeof,
 * then the offset of each field in declaration order -- and returns 18. */
int32_t sa_mask_desc_layout(int64_t* out, int32_t n);

#ifdef __cplusplus
}
#endif
#endif /* SPARSE_ATTN_H */
