/*
 * pdattn.h -- paged split-KV grouped-query decode attention for AMD Instinct
 * MI355X (gfx950). C ABI; every pointer is a plain host or device address.
 *
 * The operation (FlashQuant wiki "CUDA Kernels": flash_attention.cu Online
 * Softmax and GQA Support, paged_decode.cu Page Table Addressing and Partial
 * Output, split_k_reduce.cu Algorithm; AstrAI "CUDA Kernels": Python
 * Wrappers; OASR "Kernel Layer": Fused attention and FP8 KV variants):
 *
 *   for each sequence b < B and query head h < Hq, with G = Hq / Hkv,
 *   kv head kvh = h / G and L = context_lens[b]:
 *     page(t) = block_table[b * max_pages_per_seq + t / P],  slot(t) = t mod P
 *     s_t = scale * sum_d q[b][h][d] * K[page(t)][slot(t)][kvh][d],  t < L
 *     out[b][h][:] = sum_t softmax(s)_t * V[page(t)][slot(t)][kvh][:]
 *     lse[b][h]    = ln sum_t exp(s_t)            (natural log)
 *   L == 0 gives out = 0 and lse = -inf.
 *
 * Multi-query decode (problem->q_len = n > 1; speculative decoding's next_n
 * tokens, DeepGEMM documentation section 6.1: paged q of shape
 * [batch, next_n, heads, d]): each sequence has n query rows, the last n
 * positions of its context, already in the cache. Query row i (0 <= i < n)
 * attends causally, to the positions t < L - (n - 1 - i); a row that sees
 * no position gets out = 0 and lse = -inf. q, out and lse then carry a row
 * axis: q [B][n][Hq][d], out [B][n][Hq][d], lse [B][n][Hq]. The kernel
 * treats the n * G (row, head) pairs of a kv head as the columns of one
 * MFMA operand, so n * G must be at most 16; the K/V bytes read are those
 * of one decode step. Static plans only (not PDATTN_PLAN_BALANCED).
 *
 * Work decomposition (flash-decoding): the (b, kvh) pairs are laid end to
 * end, each cut into 16-token tiles, and a persistent grid of
 * plan->num_workers waves streams that tile list. A wave computes all G
 * query heads of a kv head with an online softmax (running max and sum in
 * base 2, fp32 accumulators); pieces of a pair computed by different waves
 * leave (m, l, acc) partials in the workspace and are merged with the
 * log-sum-exp rule. Two modes (plan flags):
 *   default   each wave takes a contiguous range of the tile list, sized by
 *             the plan's worker weights (split_weights);
 *             pdattn_decode writes the pairs one wave covers and
 *             pdattn_reduce merges the others. Bitwise reproducible for a
 *             fixed plan.
 *   BALANCED  the split points are decided on the device while the kernel
 *             runs (each wave streams a static share, then takes further
 *             tiles from atomic counters as it gets ahead), and the merge
 *             runs in the same kernel: pdattn_decode alone produces every
 *             output; pdattn_reduce enqueues nothing. Results agree with the
 *             default mode to fp32 rounding but may differ between calls in
 *             the last bits; the workspace needs pdattn_workspace_init.
 *
 * Layouts (all contiguous, row-major):
 *   q            bf16 [B][Hq][d]
 *   k_pages,     bf16 or OCP e4m3fn bytes, [num_pages][P][Hkv][d] (NHD) or
 *   v_pages      [num_pages][Hkv][P][d] (HND), per problem->kv_layout
 *   k_scale,     fp32 [num_pages][P][Hkv] (NHD) or [num_pages][Hkv][P] (HND),
 *   v_scale      fp8 pools only (NULL for bf16): the stored value of
 *                element d is e4m3fn(code) * scale
 *   block_table  int32 [B][max_pages_per_seq]; only entries < ceil(L_b / P)
 *                are read; a page may appear in several rows
 *   context_lens int32 [B], device copy, read by the kernels
 *   out          fp32 [B][Hq][d]
 *   lse          fp32 [B][Hq], optional (NULL to skip)
 *
 * Supported: d in {64, 128, 256} (256: static plans); any G <= 16 (and
 * n * G <= 16; a G that is not a power of two: static plans): the kernel
 * instance has the next power of two of columns, the rest padding;
 * P a power of two in [8, 128]; q / k / v / out bases 16-byte aligned;
 * B <= 65535.
 *
 * Ownership and execution: the caller allocates and owns every buffer,
 * including the workspace (size from the plan). The library allocates
 * nothing, keeps no device state and never synchronises; decode and reduce
 * are enqueued on the caller's stream and are safe to capture in a graph
 * (no allocation, no memset, no capture-dependent choice).
 *
 * Errors: every call validates its arguments before launching anything and
 * returns a status; an invalid call enqueues no work. The last error message
 * of the calling thread is available from pdattn_last_error(). On the
 * device, a context length that is negative or beyond the block table
 * (max_pages_per_seq * P), and a block_table entry outside [0, num_pages),
 * are not read through: the affected outputs are set to NaN instead.
 */
#ifndef PDATTN_H
#define PDATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define PDATTN_API __attribute__((visibility("default")))

typedef enum pdattn_status {
  PDATTN_OK = 0,
  PDATTN_ERR_INVALID_ARGUMENT = 1, /* null or misaligned pointer, bad shape or length */
  PDATTN_ERR_UNSUPPORTED = 2,      /* head_dim, group size, page size, dtype or mode not built */
  PDATTN_ERR_WORKSPACE = 3,        /* workspace missing or smaller than plan->workspace_bytes */
  PDATTN_ERR_PLAN_MISMATCH = 4,    /* plan not produced by pdattn_plan */
  PDATTN_ERR_DEVICE = 5            /* HIP runtime error; detail in pdattn_last_error() */
} pdattn_status;

typedef enum pdattn_kv_dtype {
  PDATTN_KV_BF16 = 0,
  PDATTN_KV_FP8_E4M3 = 1, /* OCP e4m3fn codes with one fp32 scale per (token, kv head) */
  PDATTN_KV_FP8_E4M3_INLINE = 2, /* the same codes and scales, each row's scale stored after its codes */
  PDATTN_KV_TQ4 = 3 /* TQ4 compressed rows (pdattn_tq4_* calls only; see below) */
} pdattn_kv_dtype;

/*
 * PDATTN_KV_FP8_E4M3_INLINE (DeepGEMM documentation section 6.1: the paged
 * cache of its indexer keeps each token's fp32 scale in the byte cache,
 * after the token's value bytes): a pool row is d e4m3fn code bytes followed
 * by 4 bytes holding the row's fp32 scale (little-endian), so rows are
 * d + 4 bytes apart and 4-byte aligned; the row order inside a page is
 * problem->kv_layout's, as for the other dtypes. k_scale and v_scale are
 * NULL. The stored value of element i is e4m3fn(code_i) * scale, as for
 * PDATTN_KV_FP8_E4M3. Served by static decode plans (one-token and
 * multi-query), by pdattn_kv_append and by the prefill calls; balanced
 * plans return PDATTN_ERR_UNSUPPORTED.
 */

/* The order of the (slot, kv head) rows inside one page of the K and V
 * pools (and of the fp8 scales). The paged addressing (FlashQuant wiki "CUDA
 * Kernels", paged_decode.cu Page Table Addressing) fixes the page and the
 * slot of a position, not this order; both are served:
 *   NHD  rows [page][slot][kv head]: a token's kv heads are adjacent
 *   HND  rows [page][kv head][slot]: one kv head's P rows of a page are one
 *        contiguous block (for P = 16, d = 128, bf16: 4 KB), which the decode
 *        streams measurably faster on MI355X. */
typedef enum pdattn_kv_layout {
  PDATTN_LAYOUT_NHD = 0,
  PDATTN_LAYOUT_HND = 1
} pdattn_kv_layout;

/* The problem shape (AstrAI "CUDA Kernels", Python Wrappers: blhd layout,
 * scale 1/sqrt(head_dim); OASR "Kernel Layer", Fused attention: paged mode
 * takes block_table and per-sequence lengths). */
typedef struct pdattn_problem {
  int32_t batch;             /* B */
  int32_t num_q_heads;       /* Hq */
  int32_t num_kv_heads;      /* Hkv; Hq % Hkv == 0 */
  int32_t head_dim;          /* d */
  int32_t page_size;         /* P */
  int32_t max_pages_per_seq; /* block_table row stride, in entries */
  int32_t num_pages;         /* pool size, in pages */
  int32_t kv_dtype;          /* pdattn_kv_dtype */
  float scale;               /* softmax scale; <= 0 selects 1/sqrt(head_dim) */
  int32_t kv_layout;         /* pdattn_kv_layout: the order of rows inside a page */
  int32_t q_len;             /* query rows per sequence n (0 or 1: one-token decode) */
} pdattn_problem;

/* A launch plan: a pure function of the problem, the host copy of the
 * context lengths and the compute-unit count (OASR "Kernel Layer", Fused
 * attention: the split count depends on shape and machine only; Atlas
 * "CUDA Kernel Engineering", kernel inventory: adaptive split count). The
 * kernels re-derive the split points from the device context_lens, so the
 * workspace size does not depend on the lengths. */
typedef struct pdattn_plan_t {
  pdattn_problem problem;   /* copy of the problem, scale resolved */
  int32_t num_cus;          /* compute units the plan was sized for */
  int32_t num_workgroups;   /* grid of the decode kernel (4 waves each) */
  int32_t num_workers;      /* worker waves, <= 4 * num_workgroups */
  int32_t flags;            /* PDATTN_PLAN_* flags the plan was made with */
  int64_t total_tiles;      /* Hkv * sum_b ceil(L_b / 16) over the host lengths */
  int64_t max_context_len;  /* largest host context length planned for */
  uint64_t workspace_bytes; /* partial records and the tile prefix, or counters */
  uint32_t magic;           /* set by pdattn_plan; checked by decode / reduce */
  uint32_t split_weights;   /* default mode: worker weights wa << 16 | wb; the first half of
                               the workers takes wa shares of the tile list each, the rest wb
                               (1:1, or 5:4 for fp8 pools at the full grid); set by pdattn_plan */
} pdattn_plan_t;

/* Plan flags (0: static equal ranges + pdattn_reduce; bitwise reproducible). */
#define PDATTN_PLAN_BALANCED 2 /* on-device balancing, merge inside pdattn_decode */

/*
 * Plan one decode step.
 *   problem            shape; validated here (supported set above)
 *   context_lens_host  host int32 [batch]; each 0 <= L <= max_pages_per_seq * P
 *   num_cus            compute units to size for; 0 queries the current device
 *   force_workers      0 = adaptive (fill the device's resident capacity, at
 *                      least 4 tiles per worker); > 0 forces this number of
 *                      worker waves (tests use it to move the split points)
 *   flags              0 or PDATTN_PLAN_BALANCED
 *   out                receives the plan (caller-owned POD)
 * Pure host computation apart from the optional device query (cached per
 * device after the first call).
 */
PDATTN_API pdattn_status pdattn_plan(const pdattn_problem* problem, const int32_t* context_lens_host,
                                     int32_t num_cus, int32_t force_workers, int32_t flags, pdattn_plan_t* out);

/*
 * Prepare a workspace of plan->workspace_bytes bytes (or more) for balanced-
 * mode decodes: zero its counters and stamp it with the counter layout, with
 * one small kernel on `stream` (no memset, so it can be captured). Every
 * decode leaves the counters zero again, so one preparation serves every
 * later plan with the same counter layout (the same batch, num_kv_heads,
 * page_size and max_pages_per_seq; any lengths and worker counts) whose
 * workspace_bytes fits in the buffer; a plan with another layout needs the
 * workspace prepared again. A decode that finds the workspace unprepared, or
 * prepared for another layout, writes NaN to every output. Concurrent
 * decodes on one workspace race; give each stream its own. No-op for
 * default-mode plans.
 */
PDATTN_API pdattn_status pdattn_workspace_init(const pdattn_plan_t* plan, void* workspace, uint64_t workspace_bytes,
                                               void* stream);

/*
 * Enqueue the decode step on `stream` (a hipStream_t; NULL = the null
 * stream). Pointers and layouts as described above; k_scale / v_scale must
 * be NULL for bf16 pools and non-NULL for fp8 pools; `workspace` holds
 * plan->workspace_bytes bytes, prepared by pdattn_workspace_init for
 * balanced plans (default-mode plans need no preparation). Default mode:
 * writes `out` (and `lse`) for every (b, kvh) pair that one worker covers
 * and for empty or invalid sequences, and leaves partials and the tile prefix
 * in the workspace for the cut pairs, which pdattn_reduce completes.
 * Balanced mode: writes every output.
 */
PDATTN_API pdattn_status pdattn_decode(const pdattn_plan_t* plan, const void* q, const void* k_pages,
                                       const void* v_pages, const float* k_scale, const float* v_scale,
                                       const int32_t* block_table, const int32_t* context_lens,
                                       void* workspace, uint64_t workspace_bytes, float* out, float* lse,
                                       void* stream);

/*
 * Enqueue the split reduce (FlashQuant wiki "CUDA Kernels", split_k_reduce.cu
 * Algorithm and Numerical Stability) on `stream`: for each pair cut into
 * pieces s, out = sum_s 2^(m_s - M) acc_s / sum_s 2^(m_s - M) l_s with
 * M = max_s m_s, and lse = ln 2 * (M + log2 sum_s 2^(m_s - M) l_s). Must
 * follow pdattn_decode with the same plan and workspace on the same stream.
 * Balanced plans merge inside pdattn_decode: this call then validates its
 * arguments and enqueues nothing.
 */
PDATTN_API pdattn_status pdattn_reduce(const pdattn_plan_t* plan, const void* workspace,
                                       uint64_t workspace_bytes, float* out, float* lse, void* stream);

/* Bytes of device scratch behind pdattn_decode_noalloc, per device. */
#define PDATTN_NOALLOC_SCRATCH_BYTES (64ull << 20)

/*
 * For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the
 * default-mode decode followed by its reduce, as pdattn_decode then
 * pdattn_reduce, with the workspace taken from a static device array of
 * PDATTN_NOALLOC_SCRATCH_BYTES bytes that the library holds on each device
 * it runs on until the process ends (no workspace argument). Arguments as for
 * pdattn_decode; writes every output. Allocates nothing: no hipMalloc, no
 * hipFree. Errors: PDATTN_ERR_UNSUPPORTED for balanced plans,
 * PDATTN_ERR_WORKSPACE when plan->workspace_bytes exceeds the scratch,
 * PDATTN_ERR_DEVICE when the scratch's device address cannot be resolved.
 * Every call on one device shares that device's scratch: calls that overlap
 * on one device (on different streams, or from different threads) race and
 * must be serialised by the caller.
 */
PDATTN_API pdattn_status pdattn_decode_noalloc(const pdattn_plan_t* plan, const void* q, const void* k_pages,
                                               const void* v_pages, const float* k_scale, const float* v_scale,
                                               const int32_t* block_table, const int32_t* context_lens, float* out,
                                               float* lse, void* stream);

/* Append flags. */
#define PDATTN_APPEND_POW2_SCALES 1 /* fp8 pools: power-of-two scales */

/*
 * Enqueue the KV append on `stream`: write the K and V rows of num_tokens
 * new tokens into the paged pools (FlashQuant wiki "CUDA Kernels",
 * paged_decode.cu Page Table Addressing: the slot of position t of sequence
 * b is page block_table[b][t / P], row t mod P; Atlas "CUDA Kernel
 * Engineering", kernel inventory: per-token K/V write into the paged cache;
 * OASR "Kernel Layer", FP8 KV variants: the quantise-and-scatter that fills
 * an FP8 cache, with power-of-two scales).
 *   problem      the pools' shape: batch, num_kv_heads, head_dim,
 *                page_size, max_pages_per_seq, num_pages and kv_dtype are
 *                used (num_q_heads and scale are validated, not used)
 *   k_new, v_new bf16 [num_tokens][Hkv][d], device, 16-byte aligned
 *   token_seq    int32 [num_tokens], device: the sequence b of each token
 *   token_pos    int32 [num_tokens], device: its position t in that sequence
 *   block_table  int32 [B][max_pages_per_seq], device
 *   k_pages,     the pools, layouts as for pdattn_decode (problem->kv_layout);
 *   v_pages      written in place
 *   k_scale,     fp32, one per row as for pdattn_decode, for fp8 pools
 *   v_scale      (written in place); NULL for bf16 pools
 *   flags        0 or PDATTN_APPEND_POW2_SCALES (fp8 pools only)
 * A bf16 pool receives the rows bit for bit. An fp8 pool receives, for each
 * (token, kv head) and separately for K and V, a scale s and the codes
 * code_i = e4m3fn(clamp(x_i / s, -448, 448)), rounded to the nearest code,
 * ties to even, every division a correctly rounded fp32 division: s =
 * absmax / 448 by default, or with PDATTN_APPEND_POW2_SCALES the smallest
 * power of two s with 448 * s >= absmax (then x_i / s is exact and so is the
 * decode's product code * s); an all-zero row gets s = 1. Non-finite inputs
 * give unspecified codes.
 * A token whose sequence is outside [0, B), whose position is outside
 * [0, max_pages_per_seq * P), or whose block_table entry is outside
 * [0, num_pages) is skipped: nothing is written for it. Tokens must name
 * distinct slots (two tokens writing one slot race). Nothing else in the
 * pools changes. The library allocates nothing and never synchronises; the
 * call is safe to capture in a graph. Errors: validated before launch as
 * for pdattn_decode; an invalid call enqueues nothing.
 */
PDATTN_API pdattn_status pdattn_kv_append(const pdattn_problem* problem, int32_t num_tokens, const void* k_new,
                                          const void* v_new, const int32_t* token_seq, const int32_t* token_pos,
                                          const int32_t* block_table, void* k_pages, void* v_pages, float* k_scale,
                                          float* v_scale, int32_t flags, void* stream);

/*
 * Enqueue the merge of exported partial attention states on `stream`: for
 * each row r (a (sequence, query head) pair) and pieces s over disjoint key
 * sets, each a normalised output o_s and a natural-log lse_s as
 * pdattn_decode exports them (FlashQuant wiki "CUDA Kernels",
 * split_k_reduce.cu Algorithm and Numerical Stability):
 *   M = max_s lse_s,  w_s = exp(lse_s - M),
 *   out = sum_s w_s o_s / sum_s w_s,  lse = M + ln sum_s w_s
 * i.e. attention over the union of the pieces' keys (a shared prefix and a
 * per-request suffix decoded separately; or the pages of one sequence split
 * across devices, each decoding its share).
 *   num_partials  S >= 1
 *   num_rows      R, e.g. batch * num_q_heads (0: nothing to do)
 *   head_dim      d in {64, 128, 256}
 *   partial_out   fp32 [S][R][d], device, 16-byte aligned
 *   partial_lse   fp32 [S][R], device (natural log)
 *   out           fp32 [R][d], device, 16-byte aligned; may be the same
 *                 buffer as piece 0 of partial_out (no other overlap)
 *   lse           fp32 [R], device, optional (NULL to skip); may be piece 0
 *                 of partial_lse
 * A piece with lse = -inf is empty and weighs nothing; a row whose pieces
 * are all empty gets out = 0, lse = -inf; a NaN or +inf lse in any piece
 * makes the row's out and lse NaN. fp32 arithmetic, one pass over the
 * pieces. Allocates nothing, never synchronises, graph-capturable;
 * validated before launch.
 */
PDATTN_API pdattn_status pdattn_merge(int32_t num_partials, int64_t num_rows, int32_t head_dim,
                                      const float* partial_out, const float* partial_lse, float* out, float* lse,
                                      void* stream);

/*
 * Diagnostic, not part of the path: enqueue a comparison of the hardware
 * float -> e4m3fn conversion the fp8 append uses with the format's
 * definition (nearest code, ties to even, sign kept, subnormals m * 2^-9),
 * over every fp32 value y with |y| <= 448, both signs (about 2.3e9 values;
 * milliseconds on the device). `mismatches` (device, one uint64, zeroed by
 * the caller) receives the number of values where the two differ; 0 means
 * the conversion is exact on everything the append can feed it.
 */
PDATTN_API pdattn_status pdattn_fp8_conversion_check(uint64_t* mismatches, void* stream);

/*
 * Ragged paged prefill (AstrAI "CUDA Kernels": the paged prefill entry over a
 * ragged batch, qo_indptr plus the cache's own lengths; section "Q
 * Scheduling and KV Addressing" for the tile map). Request b owns the packed
 * query rows qo_indptr[b] .. qo_indptr[b+1] - 1 (n_b of them), the last n_b
 * positions of its context of L_b = context_lens[b] positions, whose keys
 * and values are already in the pools (pdattn_kv_append writes them). The
 * pages leave that placement open; it is the reading under which a prompt
 * prefilled in chunks gives the rows a whole-prompt prefill gives. Query
 * row i of request b and head h (kv head h / G):
 *   causal:      positions t < L_b - n_b + i + 1 (clamped to [0, L_b])
 *   non-causal:  positions t < L_b
 *   out[qo_indptr[b] + i][h][:] = softmax over those t of
 *                scale * q . K[page(t)][slot(t)][kvh], times V, as for decode
 *   lse[qo_indptr[b] + i][h]    = ln sum_t exp(s_t)
 * A row that sees no position gets out = 0 and lse = -inf.
 *
 * The work is cut into query tiles of rows_per_tile rows of one request
 * (pdattn_prefill_rows_per_tile: the (row, head) columns one workgroup of
 * the kernel holds, divided by G), each paired with every kv head. The
 * host builds the tile map once per batch (pdattn_prefill_tiles) and copies
 * it to the device; the kernel finds a tile's request and rows in O(1).
 */

/* rows_per_tile for `problem` (head_dim and group size; q_len is not used):
 * 128 / G for d in {64, 128}, 64 / G for d = 256. */
PDATTN_API pdattn_status pdattn_prefill_rows_per_tile(const pdattn_problem* problem, int32_t* rows_per_tile);

/* Tile-map flags. */
#define PDATTN_TILES_LONGEST_FIRST 1 /* order tiles by positions read, most first */

/*
 * Build the tile map on the host. qo_indptr: host int32 [batch + 1],
 * non-decreasing from a value >= 0. Without flags the tiles are listed
 * request by request, tile by tile: tile_batch[t] = b, tile_index[t] = j
 * covers rows qo_indptr[b] + j * rows_per_tile .. (the pages' worked
 * example: Q lengths 70, 10, 130 at 64 rows give batch 0 0 1 2 2 2 and
 * index 0 1 0 0 1 2). PDATTN_TILES_LONGEST_FIRST reorders them by the
 * number of context positions their rows reach (causal: L_b - n_b + last
 * row + 1; else L_b), most first, ties kept in order, so that the longest
 * tiles start first; it needs context_lens (host int32 [batch]; otherwise
 * ignored, may be NULL). *num_tiles receives the tile count; with
 * tile_batch or tile_index NULL nothing else is written (a count query);
 * else both must hold `capacity` >= *num_tiles entries. Host memory only.
 */
PDATTN_API pdattn_status pdattn_prefill_tiles(const int32_t* qo_indptr, const int32_t* context_lens, int32_t batch,
                                              int32_t rows_per_tile, int32_t causal, int32_t flags,
                                              int32_t* tile_batch, int32_t* tile_index, int32_t capacity,
                                              int32_t* num_tiles);

/*
 * Enqueue the prefill on `stream`.
 *   problem      pools and heads as for decode (q_len is not used; any G
 *                up to 16, d in {64, 128, 256}, both layouts, bf16 or fp8
 *                with separate or inline scales)
 *   causal       1: causal mask as above; 0: every row sees all L_b positions
 *   q            bf16 [total_q][Hq][d], device, 16-byte aligned
 *   qo_indptr    int32 [batch + 1], device: the same values the tile map
 *                was built from
 *   tile_batch,  int32 [num_tiles], device: from pdattn_prefill_tiles with
 *   tile_index   this problem's rows_per_tile
 *   k_pages ...  pools, scales, block_table and context_lens as for decode
 *   out          fp32 [total_q][Hq][d], device, 16-byte aligned
 *   lse          fp32 [total_q][Hq], device, optional (NULL to skip)
 * Rows that no tile covers are not written. On the device, a context length
 * outside [0, max_pages_per_seq * P] makes its request's rows NaN, and a
 * block_table entry outside [0, num_pages) makes NaN the rows of every tile
 * that reads it. Allocates nothing, never synchronises, graph-capturable;
 * validated before launch (an invalid call enqueues nothing).
 */
PDATTN_API pdattn_status pdattn_prefill(const pdattn_problem* problem, int32_t causal, const void* q,
                                        const int32_t* qo_indptr, const int32_t* tile_batch,
                                        const int32_t* tile_index, int32_t num_tiles, const void* k_pages,
                                        const void* v_pages, const float* k_scale, const float* v_scale,
                                        const int32_t* block_table, const int32_t* context_lens, float* out,
                                        float* lse, void* stream);

/*
 * Split-KV prefill. A query tile reads its context positions in order, one
 * kernel tile after another, so a grid whose tiles differ much in length
 * (one long causal prompt: the last tile of 32 rows reads 2048 positions,
 * the first 32) runs as long as its longest tile. Splitting the K/V range
 * when the grid cannot fill the machine is the flash-decoding remedy,
 * applied to fused attention too (OASR "Kernel Layer", section "Fused
 * attention", where the number of splits depends only on the shape and the
 * device; FlashQuant wiki "CUDA Kernels", paged_decode.cu and
 * split_k_reduce.cu, for the per-split (m, l, acc) states and their
 * log-sum-exp merge). Here a long tile is cut into parts over consecutive
 * position ranges; each part is one workgroup per kv head, which keeps its
 * unnormalised state in a record of the caller's workspace, and the last
 * part of a tile to finish merges the records in part order (the result does
 * not depend on which part finished last) and writes the rows. The outputs
 * are those of pdattn_prefill up to rounding.
 */

/*
 * Build the split tile map on the host. problem: as for pdattn_prefill
 * (batch = number of requests). qo_indptr: host int32 [batch + 1],
 * non-decreasing from >= 0; context_lens: host int32 [batch], each within
 * the block table (PDATTN_ERR_INVALID_ARGUMENT otherwise). slots: the
 * workgroups the device runs at once, 0 for the current device's (compute
 * units x resident prefill workgroups per unit; PDATTN_ERR_DEVICE without a
 * device).
 *
 * A tile reads ceil(reach / T) kernel tiles (reach as for
 * PDATTN_TILES_LONGEST_FIRST; T = 64 positions, 32 at d 256). For a cap c,
 * a tile of more than c kernel tiles is cut into min(ceil(count / c), 16,
 * floor(units / m)) parts, units = ceil(reach / 64) and m = the 64-position
 * units of 4 kernel tiles: part q covers units [q units / parts, (q + 1)
 * units / parts) (integer division), times 64, the last ending at reach.
 * An entry's cost, in quarter kernel tiles: 4 per tile read, plus 1 per tile
 * at or past the first row's causal limit, plus 20, plus 12 for a part;
 * entries are listed by cost, most first (ties in request, tile, part
 * order). The device starts workgroups in grid order as slots free up, so
 * the planner simulates that list schedule (each entry's num_kv_heads
 * workgroups in turn, each on the slot free first) for no cut and for
 * c = ceil(k x longest / 16), k = 15 down to 3 (at least 4), and keeps the
 * first that ends soonest. Outputs, for entry t < *num_tiles:
 *   tile_batch[t], tile_index[t]  the query tile, as in pdattn_prefill_tiles
 *   tile_kv[4t + 0], [4t + 1]     its positions [first, end)
 *   tile_kv[4t + 2]               -1 for a whole tile; for a part, the first
 *                                 of the tile's consecutive workspace slots
 *   tile_kv[4t + 3]               part | parts << 16 (1 << 16 when whole)
 * *num_slots receives the slots the parts use and *workspace_bytes the
 * workspace pdattn_prefill_split needs for them (0 when nothing is cut).
 * With any of tile_batch, tile_index, tile_kv NULL only the three counts
 * are written; else tile_batch and tile_index hold `capacity` entries and
 * tile_kv 4 * capacity, capacity >= *num_tiles. Host memory only.
 */
PDATTN_API pdattn_status pdattn_prefill_split_tiles(const pdattn_problem* problem, const int32_t* qo_indptr,
                                                    const int32_t* context_lens, int32_t causal, int32_t slots,
                                                    int32_t* tile_batch, int32_t* tile_index, int32_t* tile_kv,
                                                    int32_t capacity, int32_t* num_tiles, int32_t* num_slots,
                                                    uint64_t* workspace_bytes);

/*
 * Enqueue the split-KV prefill on `stream`: num_tiles x num_kv_heads
 * workgroups. pdattn_prefill's arguments, plus
 *   tile_kv      int32 [num_tiles][4], device, 16-byte aligned: from
 *                pdattn_prefill_split_tiles with the same problem and lengths
 *   num_slots    that call's *num_slots (0: nothing cut, workspace unused)
 *   workspace    device, 256-byte aligned, at least that call's
 *                *workspace_bytes: num_slots x num_kv_heads 32-bit counters
 *                (the region rounded up to 256 bytes), then as many part
 *                records. The counters must be zero before the first call
 *                that uses the workspace (e.g. hipMemset once after
 *                allocation); each call leaves them zero. Calls that share a
 *                workspace must not overlap (order them on one stream).
 * A part entry whose slots lie outside num_slots makes its tile's rows NaN
 * without touching the workspace (the tile's other parts then leave their
 * counter nonzero: zero the workspace again before reusing it). Bad lengths
 * and page entries poison rows as in pdattn_prefill, across all parts of a
 * tile. Allocates nothing, never synchronises, graph-capturable; validated
 * before launch.
 */
PDATTN_API pdattn_status pdattn_prefill_split(const pdattn_problem* problem, int32_t causal, const void* q,
                                              const int32_t* qo_indptr, const int32_t* tile_batch,
                                              const int32_t* tile_index, const int32_t* tile_kv, int32_t num_tiles,
                                              int32_t num_slots, void* workspace, uint64_t workspace_bytes,
                                              const void* k_pages, const void* v_pages, const float* k_scale,
                                              const float* v_scale, const int32_t* block_table,
                                              const int32_t* context_lens, float* out, float* lse, void* stream);

/*
 * ---- TQ4 compressed KV cache (FlashQuant wiki "CUDA Kernels": compress.cu,
 * decompress.cu, fused_tq_attention.cu, paged_decode.cu, split_k_reduce.cu)
 *
 * Codec. R is a d x d orthogonal rotation (float32, row-major, 16-byte
 * aligned), the same for K and V; K and V each have 16 centroids and 15
 * sorted boundaries (float32). A row x (bf16) is stored as its norm
 * ||x||_2 (fp32) and d 4-bit codes: x_hat = x / (||x|| + 1e-10), y = R x_hat,
 * code_i = #{boundaries b : b <= y_i}, byte j = code_2j << 4 | code_2j+1
 * (compress.cu, What It Replaces and Algorithm). The row it stands for is
 * R_seq^T c where c_j = centroid[high nibble of byte j] * norm and
 * c_{d/2 + j} = centroid[low nibble of byte j] * norm (decompress.cu,
 * Sequential Layout), R_seq being R with row j = R[2j], row d/2 + j =
 * R[2j + 1].
 *
 * Cache (paged_decode.cu, KV Cache Byte Layout): problem->kv_dtype =
 * PDATTN_KV_TQ4, kv_layout = PDATTN_LAYOUT_HND; one uint8 pool of
 * num_pages * Hkv * P rows of d + 8 bytes, row (page * Hkv + kvh) * P + slot:
 * [K codes d/2 | K norm fp32 | V codes d/2 | V norm fp32]. The pool is 16-byte
 * aligned. Page sizes: powers of two in [8, 128]; q_len 0 or 1.
 */

/* The codebook pdattn_tq4_append / pdattn_tq4_decode expect for rotated
 * unit vectors of head_dim coordinates (FlashQuant wiki index, Algorithm
 * Deep Dive, Lloyd-Max via erfinv): the 16-level Lloyd-Max quantiser of
 * N(0, 1/head_dim), by Lloyd's iteration in double precision from the
 * Gaussian quantiles; centroids (16) and boundaries (15, the midpoints)
 * written as float32 to host arrays. Any head_dim >= 1. Host only. */
PDATTN_API pdattn_status pdattn_tq4_codebook(int32_t head_dim, float* centroids, float* boundaries);

/* Compress num_tokens new rows per kv head (k_new, v_new: bf16
 * [num_tokens][Hkv][d], 16-byte aligned) and write them at page
 * block_table[token_seq[t]][token_pos[t] / P], slot token_pos[t] % P, of
 * `cache` (compress.cu, fused into the scatter). Tokens whose sequence,
 * position or page falls outside the tables are skipped. Rows that two
 * tokens name race. rotation, k_boundaries, v_boundaries: device float32
 * (rotation 16-byte aligned). One kernel on `stream`. */
PDATTN_API pdattn_status pdattn_tq4_append(const pdattn_problem* problem, int32_t num_tokens, const void* k_new,
                                           const void* v_new, const int32_t* token_seq, const int32_t* token_pos,
                                           const int32_t* block_table, const float* rotation,
                                           const float* k_boundaries, const float* v_boundaries, void* cache,
                                           void* stream);

/* A TQ4 decode plan: every (sequence, kv head) pair is cut into work items
 * of about chunk_tiles 16-token tiles (paged_decode.cu, split-K; the count
 * per pair from the plan, not fixed), one wave each on a persistent grid. */
typedef struct pdattn_tq4_plan_t {
  pdattn_problem problem;   /* copy of the problem, scale resolved */
  int32_t num_cus;          /* compute units the plan was sized for */
  int32_t num_workgroups;   /* grid of the decode kernel (8 waves each) */
  int32_t chunk_tiles;      /* tiles per work item (a pair takes ceil(tiles / chunk_tiles) items, evenly split) */
  int32_t max_chunks;       /* work items per pair at most (longer pairs split their tiles over this many) */
  int64_t total_tiles;      /* Hkv * sum_b ceil(L_b / 16) over the host lengths */
  int64_t max_context_len;  /* largest host context length planned for */
  uint64_t workspace_bytes; /* rotated queries, then the work items' records */
  uint32_t magic;
  uint32_t reserved1;
} pdattn_tq4_plan_t;

/* Plan a TQ4 decode step (problem->kv_dtype = PDATTN_KV_TQ4). num_cus: 0
 * queries the current device; chunk_tiles: 0 = adaptive, > 0 forces it
 * (tests move the split points with it). Host only apart from the device
 * query. */
PDATTN_API pdattn_status pdattn_tq4_plan(const pdattn_problem* problem, const int32_t* context_lens_host,
                                         int32_t num_cus, int32_t chunk_tiles, pdattn_tq4_plan_t* out);

/* Enqueue a TQ4 decode step on `stream`: q (bf16 [B][Hq][d], model space,
 * 16-byte aligned) is rotated into the codes' space and rounded to fp16
 * (fused_tq_attention.cu, Input/Output: the rotated queries are 16-bit), so
 * its rotated values must stay below 65504 in magnitude;
 * attention runs there over the cache (fused_tq_attention.cu, Decode Path;
 * paged_decode.cu), each work item leaving (m, l, acc) in the workspace;
 * the merge (split_k_reduce.cu) then writes out (fp32 [B][Hq][d], rotated
 * back to model space: R_seq^T o) and lse (fp32 [B][Hq], natural log, or
 * NULL). Empty sequences give out = 0, lse = -inf; a length beyond the
 * block table or a block-table entry outside [0, num_pages) gives NaN.
 * workspace: plan->workspace_bytes, 16-byte aligned; concurrent calls on one
 * workspace race. Three kernels on `stream`. */
PDATTN_API pdattn_status pdattn_tq4_decode(const pdattn_tq4_plan_t* plan, const void* q, const void* cache,
                                           const float* rotation, const float* k_centroids,
                                           const float* v_centroids, const int32_t* block_table,
                                           const int32_t* context_lens, void* workspace, uint64_t workspace_bytes,
                                           float* out, float* lse, void* stream);

/* The same step at the fused attention's own boundary (fused_tq_attention.cu,
 * Input/Output: the queries arrive pre-rotated, the output stays in the
 * rotated space and the caller rotates it back; a caller can fold R into its
 * q and output projections). q_rot: fp16 [B][Hq][d], 16-byte aligned, in the
 * rotation's natural order, q_rot = R q (y_i = sum_k R[i][k] q_k; row i of the
 * `rotation` given to pdattn_tq4_append). out: fp32 [B][Hq][d] in that same
 * order (the attention output o_rot, with R^T o_rot the model-space output);
 * lse as in pdattn_tq4_decode. Same plan, workspace, errors and empty /
 * invalid sequence results as pdattn_tq4_decode. Two kernels on `stream`
 * (the decode and the merge; no rotation). */
PDATTN_API pdattn_status pdattn_tq4_decode_rotated(const pdattn_tq4_plan_t* plan, const void* q_rot,
                                                   const void* cache, const float* k_centroids,
                                                   const float* v_centroids, const int32_t* block_table,
                                                   const int32_t* context_lens, void* workspace,
                                                   uint64_t workspace_bytes, float* out, float* lse, void* stream);

/* Static description of a status code. */
PDATTN_API const char* pdattn_status_string(pdattn_status status);

/* The last error message of the calling thread ("" if none). */
PDATTN_API const char* pdattn_last_error(void);

/*
 * Measurement aid, not part of the decode path: enqueue a plain streaming
 * read of `bytes` bytes at `buffer` (16-byte aligned, a multiple of 4096)
 * with the same non-temporal 16-byte loads the decode kernel streams K/V
 * with, on 2 * num_cus workgroups. `sink` (device, pdattn_stream_read_sink_
 * words(num_cus) uint32 words, caller-owned) receives one folded word per
 * thread. Timing it gives the read bandwidth the device sustains for this
 * size, the ceiling the decode kernel is compared against.
 */
PDATTN_API pdattn_status pdattn_stream_read(const void* buffer, uint64_t bytes, uint32_t* sink, int32_t num_cus,
                                            void* stream);
PDATTN_API uint64_t pdattn_stream_read_sink_words(int32_t num_cus);

/* sizeof(pdattn_problem), sizeof(pdattn_plan_t) and sizeof(pdattn_tq4_plan_t),
 * for binding checks. */
PDATTN_API uint64_t pdattn_problem_size(void);
PDATTN_API uint64_t pdattn_plan_size(void);
PDATTN_API uint64_t pdattn_tq4_plan_size(void);

#ifdef __cplusplus
}
#endif

#endif /* PDATTN_H */
