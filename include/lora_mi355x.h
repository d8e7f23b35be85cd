/*
 * lora_mi355x.h -- C ABI of the multi-LoRA batched adapter path on MI355X
 * (gfx950, CDNA4).
 *
 * The operation.  For every token t of a batch, with adapter i = a(t) chosen
 * per token from a pool of adapters resident in device memory:
 *
 *     y[t] += (alpha_i / r_i) * (x[t] A_i) B_i
 *
 * "Multi-LoRA Serving in Production: Comparing S-LoRA, Punica, LoRAX, and
 * vLLM ..." (llms.blog), section "Mathematical Formulation and the Batching
 * Challenge" gives the layer equation (base x W0 plus (alpha/r)(x A) B) and,
 * in section "Kernel Architectures: SGMV, MBGMV, and Grouped GEMMs", the two
 * stages: a shrink x A_i (d_in -> r_i) over contiguous segments of tokens that
 * share an adapter, found "via pointer array lookups", then an expand
 * (r_i -> d_out) that scales and accumulates into the base output.  Ranks may
 * differ between adapters and are never padded (same page, "S-LoRA: MBGMV and
 * MBGMM Kernels": r in [1, 256]).  "Multi-LoRA serving: the single translator
 * with a thousand glossaries" (blog.lo0.es), section "SGMV: the kernel that
 * holds it all up", defines the per-token adapter a(t).
 *
 * Storage (row-major everywhere; element type per lora_dtype):
 *   x   [T, ldx]          activations, row pitch ldx elements
 *   A_i [r_i, d_in]       stored contiguously, row pitch d_in (the pages' A^T)
 *   B_i [d_out, r_i]      stored contiguously, row pitch r_i  (the pages' B^T)
 *   W0  [d_out, d_in]     base weight of the fused entry, row pitch d_in
 *   y   [T, ldy]          output, row pitch ldy elements
 *   v   [rows, ldv] fp32  the shrink result (the pages' h), row pitch ldv
 * Accumulation is fp32; bf16 outputs are rounded to nearest-even once.
 *
 * Ownership and ordering.  The caller owns every buffer (activations, pool,
 * plans, v, workspace).  The library never frees or synchronises;
 * every GPU call is enqueued on the caller's stream (a hipStream_t passed as
 * void*, NULL = the null stream) and returns before the work runs.  Buffers
 * must stay alive until the stream has passed the call.  x, v and y must not
 * overlap.  The library allocates no device memory and keeps no mutable
 * global state; per thread it keeps the last error message, a pending
 * launch-timing request (lora_profile_launches) and a host scratch array for
 * the plan builder's counts, so it may be used from several threads.
 *
 * Errors.  Every call returns LORA_OK (0) or a negative lora_status, after
 * checking every argument the host can see and before enqueuing anything;
 * lora_last_error() then describes the failure.  A call with T = 0 (or no
 * segments) is a successful no-op.  Device-resident tables (the BGMV id and
 * pool tables) cannot be read by the host: their contents are a precondition
 * (ids in [-1, n_adapters), ranks in [1, max_rank]); a BGMV kernel treats a
 * token whose id or rank breaks it as having no adapter.
 */
#ifndef LORA_MI355X_H
#define LORA_MI355X_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum lora_status {
    LORA_OK = 0,
    LORA_ERR_ARG = -1,        /* null pointer, negative size, bad op code */
    LORA_ERR_RANK = -2,       /* a rank outside [1, 256], or ldv < max rank */
    LORA_ERR_ADAPTER_ID = -3, /* an id < -1 or >= n_adapters (host-visible ids) */
    LORA_ERR_ALIGN = -4,      /* pointer not 16-byte aligned, or row pitch not a multiple of 16 bytes */
    LORA_ERR_DTYPE = -5,      /* unknown lora_dtype */
    LORA_ERR_WORKSPACE = -6,  /* workspace or plan buffer smaller than required */
    LORA_ERR_HIP = -7,        /* a HIP runtime call or kernel launch failed */
    LORA_ERR_PLAN = -8        /* plan buffer does not hold a valid plan */
} lora_status;

typedef enum lora_dtype {
    LORA_F32 = 0,  /* x, A, B, W0, y in fp32 */
    LORA_BF16 = 1  /* x, A, B, W0, y in bf16 (stored as 16-bit patterns) */
} lora_dtype;

#define LORA_MAX_RANK 256     /* largest adapter rank accepted */
#define LORA_PLAN_ROW_BLOCK 16 /* rows per block in a plan's block list */

/* ------------------------------------------------------------------ segments
 * The grouping of one batch's tokens into segments: tokens sorted by adapter
 * id (ascending), the original order kept inside a segment, tokens with id -1
 * left out.  The pages fix the grouping but not its order; the ascending
 * stable order makes it unique.  ("Multi-LoRA Serving in Production ...",
 * section "Punica and Segmented Gather Matrix-Vector Multiplication (SGMV)":
 * the batch is split into contiguous segments whose tokens reference one
 * adapter id, given by segment start indices; the adapters are reached through
 * a pointer array, with a rank per adapter.)
 *
 * lora_build_segments emits, for S segments over the T' adapted tokens:
 *   perm[T']          original token index at each sorted position (then the
 *                     T - T' tokens without an adapter, in their order)
 *   seg_indptr[S + 1] segment s covers sorted positions [seg_indptr[s], seg_indptr[s+1])
 *   seg_adapter[S], seg_A[S], seg_B[S], seg_rank[S], seg_scale[S] (alpha / r, fp32)
 * All of it lives in one buffer, with the same layout on the host and the
 * device, so one copy moves it (lora_segments_upload).  The buffer also holds
 * the descriptors the kernels start from (below), so that a workgroup reads
 * one record before it fetches activations and adapter weights.
 *
 * Buffer layout (a "plan"):
 *   [lora_plan_header][lora_seg_desc x S][lora_blk_desc x n_blocks][int32 perm x T]
 *   [lora_chunk_desc x n_chunks][int32 segidx x T'][segment arrays]
 *
 * perm[p] is the original token index at sorted position p (p < T'); the
 * tokens without an adapter follow in their original order (perm[T' .. T)),
 * for the fused entry, which writes every row.  segidx[p] is the segment of
 * sorted position p.  Segment s covers
 * sorted positions [start, start + len).  The block list cuts every segment
 * into blocks of LORA_PLAN_ROW_BLOCK rows (the last one ragged); segment s
 * owns blocks [blk0, blk0 + ceil(len/16)).  A block descriptor repeats what a
 * kernel needs about its segment and lists its rows, so a workgroup reads one
 * 128-byte record before it can fetch activations and adapter weights.
 */
typedef struct lora_seg_desc {
    uint64_t A;      /* device address of A_i, [rank, d_in] */
    uint64_t B;      /* device address of B_i, [d_out, rank] */
    int32_t start;   /* first sorted position */
    int32_t len;     /* number of tokens (>= 1) */
    int32_t rank;    /* r_i in [1, 256] */
    int32_t adapter; /* adapter id i */
    float scale;     /* alpha_i / r_i, fp32 */
    int32_t blk0;    /* first block of this segment */
} lora_seg_desc;

typedef struct lora_blk_desc {
    uint64_t A;       /* as the segment's descriptor */
    uint64_t B;
    float scale;
    int32_t rank;
    int32_t n;        /* rows in this block, 1..16 */
    int32_t p0;       /* sorted position of the block's first row (rows are p0 .. p0+n-1) */
    int32_t seg;      /* segment index */
    int32_t reserved[7];
    int32_t rows[LORA_PLAN_ROW_BLOCK]; /* original token index of each row; -1 past n */
} lora_blk_desc; /* 128 bytes */

typedef struct lora_plan_header {
    uint32_t magic;       /* LORA_PLAN_MAGIC when valid */
    int32_t num_tokens;   /* T of the batch */
    int32_t num_sorted;   /* T' = tokens that have an adapter */
    int32_t num_segments; /* S */
    int32_t num_blocks;   /* sum over segments of ceil(len / 16) */
    int32_t max_rank;     /* largest rank among the segments (0 if S = 0) */
    int32_t max_len;      /* longest segment */
    int32_t num_chunks;   /* sum over segments of ceil(blocks / LORA_PLAN_CHUNK_BLOCKS) */
    uint64_t seg_offset;  /* byte offset of the lora_seg_desc array */
    uint64_t blk_offset;  /* byte offset of the lora_blk_desc array (128-byte aligned) */
    uint64_t perm_offset; /* byte offset of perm */
    uint64_t bytes_used;  /* bytes from the start of the buffer that hold the plan */
    uint64_t chunk_offset; /* byte offset of the lora_chunk_desc array (64-byte aligned) */
    uint64_t segidx_offset; /* byte offset of segidx (16-byte aligned) */
    uint64_t soa_offset;  /* byte offset of the segment arrays (16-byte aligned): seg_A[S],
                             seg_B[S] (uint64), seg_indptr[S + 1], seg_adapter[S], seg_rank[S]
                             (int32), seg_scale[S] (float) */
    uint64_t reserved;
} lora_plan_header; /* 96 bytes */

/* A chunk is up to this many consecutive blocks of one segment (64 rows): the
 * unit of expand work that reuses one adapter's B tile across its rows.  Like a
 * block descriptor it is self-contained. */
#define LORA_PLAN_CHUNK_BLOCKS 4
#define LORA_PLAN_CHUNK_ROWS (LORA_PLAN_ROW_BLOCK * LORA_PLAN_CHUNK_BLOCKS)

typedef struct lora_chunk_desc {
    uint64_t A;
    uint64_t B;
    float scale;
    int32_t rank;
    int32_t n;          /* rows in this chunk, 1..64 */
    int32_t p0;         /* sorted position of the first row (rows are p0 .. p0+n-1) */
    int32_t seg;
    int32_t first_blk;  /* first of the chunk's blocks */
    int32_t nblk;       /* blocks in the chunk, 1..4 */
    int32_t reserved[5];
    int32_t rows[LORA_PLAN_CHUNK_ROWS]; /* original token index of each row; -1 past n */
} lora_chunk_desc; /* 320 bytes */

#define LORA_PLAN_MAGIC 0x4C6F5241u

/* A batch's segments, on the host or on the device: counts, and pointers into
 * the buffer the struct is bound to (host addresses in a host struct, device
 * addresses in a device struct).  The first eleven fields are the segment
 * table; the rest tie the struct to its buffer. */
typedef struct lora_segments {
    int32_t num_segments;  /* S */
    int32_t num_tokens;    /* T' = seg_indptr[S], tokens that have an adapter */
    int32_t max_rank;      /* largest r_s (0 when S = 0) */
    int32_t capacity;      /* largest batch the bound buffer holds */
    int32_t *perm;         /* [batch_tokens] */
    int32_t *seg_indptr;   /* [S + 1] */
    int32_t *seg_adapter;  /* [S] */
    int32_t *seg_rank;     /* [S] */
    uint64_t *seg_A;       /* [S] device addresses of A_s */
    uint64_t *seg_B;       /* [S] device addresses of B_s */
    float *seg_scale;      /* [S] alpha_s / r_s */
    int32_t batch_tokens;  /* T of the batch, tokens without an adapter included */
    int32_t reserved0;
    void *buf;             /* the bound buffer (holds the plan) */
    const void *host;      /* device struct: the host buffer it was uploaded from (the calls read the
                              launch geometry there); NULL in a host struct */
} lora_segments;

/* Bytes a segments buffer needs for batches of up to `capacity` tokens (>= 0). */
size_t lora_segments_bytes(int32_t capacity);

/* Bind a caller buffer (host or device memory, 16-byte aligned, at least
 * lora_segments_bytes(capacity) bytes) to *out; counts and pointers are set by
 * lora_build_segments (host) or lora_segments_upload (device).  The buffer
 * stays the caller's.  Errors: LORA_ERR_ARG, LORA_ERR_ALIGN. */
int lora_segments_bind(void *buf, int32_t capacity, lora_segments *out);

/* Build the segments of one batch into a host-bound struct (no GPU call),
 * O(T + n_adapters).
 *   ids        [T] host, adapter per token, -1 = none; T <= out_host->capacity
 *   pool_A/B   [n_adapters] host, device addresses of A_i / B_i (16-byte aligned)
 *   pool_rank  [n_adapters] host, r_i in [1, 256]
 *   pool_alpha [n_adapters] host, alpha_i; seg_scale = alpha_i / r_i in fp32
 * Only the adapters the batch uses are looked at.
 * Errors: LORA_ERR_ARG, LORA_ERR_ADAPTER_ID, LORA_ERR_RANK, LORA_ERR_ALIGN,
 * LORA_ERR_WORKSPACE (batch larger than the capacity). */
int lora_build_segments(int32_t T, const int32_t *ids, int32_t n_adapters,
                        const uint64_t *pool_A, const uint64_t *pool_B,
                        const int32_t *pool_rank, const float *pool_alpha,
                        lora_segments *out_host);

/* Enqueue one host-to-device copy of a built host struct's buffer into the
 * buffer `dev` is bound to, and set dev's counts and device pointers; dev
 * remembers host's buffer.  host's buffer should be pinned memory and must stay
 * unchanged while the copy is pending and while dev is passed to the calls
 * below (they read the launch geometry from it).
 * Errors: LORA_ERR_ARG, LORA_ERR_PLAN, LORA_ERR_WORKSPACE (dev too small),
 * LORA_ERR_HIP. */
int lora_segments_upload(const lora_segments *host, lora_segments *dev, void *stream);

/* ------------------------------------------------------------------ SGMV
 * Segmented shrink, the pages' "Shrink Stage" ("Multi-LoRA Serving in
 * Production ...", section "Punica and Segmented Gather Matrix-Vector
 * Multiplication (SGMV)"):
 *     v[p, j] = sum_k x[perm[p], k] * A_s[j, k]    for j < r_s,
 * for every sorted position p of segment s.  v rows are in sorted order; the
 * columns j >= r_s of a row are left untouched.  Overwrites v.
 *   seg                   the batch's segments, uploaded (a device struct; the
 *                         call reads the launch geometry, and the expand the
 *                         chunk descriptors it passes in the kernel arguments,
 *                         from its host copy)
 *   v                     device fp32 [seg->num_tokens, ldv], ldv >= max_rank,
 *                         ldv a multiple of 4
 * Errors: LORA_ERR_ARG, LORA_ERR_DTYPE, LORA_ERR_RANK, LORA_ERR_ALIGN,
 * LORA_ERR_PLAN, LORA_ERR_HIP. */
int lora_sgmv_shrink(void *stream, int dtype, const void *x, int64_t ldx, int32_t d_in,
                     const lora_segments *seg, float *v, int64_t ldv, void *ws, size_t ws_bytes);

/* Segmented expand, the pages' "Expand Stage" (same section): scale and
 * accumulate into the base output,
 *     y[perm[p], n] += scale_s * sum_{j < r_s} v[p, j] * B_s[n, j]   for n < d_out.
 * Rows of tokens without an adapter are not touched.  Precision (every
 * expand of the library, SGMV and BGMV): bf16 calls multiply on bf16 MFMA with
 * fp32 accumulation, each fp32 v value fed as its two bf16 halves hi = bf16(v)
 * and lo = bf16(v - hi) (16 significant bits, a residual below 2^-17 of v);
 * the sum is scaled in fp32 and rounded to bf16 once.  fp32 calls multiply
 * exactly in fp32.
 * Errors: as lora_sgmv_shrink. */
int lora_sgmv_expand(void *stream, int dtype, const float *v, int64_t ldv,
                     const lora_segments *seg, void *y, int64_t ldy, int32_t d_out, void *ws, size_t ws_bytes);

/* One call for the whole correction of a batch from its segments, shrink then
 * expand (same section): y[perm[p], :] += scale_s (x[perm[p], :] A_s) B_s.
 * The low-rank intermediate stays in the workspace as fp32 partial sums over
 * slices of d_in (summed in a fixed order by the expand, so results are
 * reproducible run to run).  Small plans (grids of up to 1536 workgroups)
 * with x and y rows 16-byte aligned, d_out % 16 == 0 and every rank <= 32
 * run in one kernel launch: the shrink workgroups, then the expand workgroups
 * of every (64-row chunk, 256 columns), which wait for their chunk's partial
 * sums, stored as tagged words in the workspace (as lora_bgmv).  Other plans
 * run as two launches.  Both forms give the same result.  The int32 at the
 * start of the workspace is the same sticky status word as lora_bgmv's.
 * Needs ws_bytes >= lora_workspace_bytes(LORA_OP_SGMV, T, d_in, d_out, max_rank)
 * with T >= seg->num_tokens and max_rank >= seg->max_rank.
 * Errors: as lora_sgmv_shrink, plus LORA_ERR_WORKSPACE. */
int lora_sgmv(void *stream, int dtype, const void *x, int64_t ldx, int32_t d_in,
              const lora_segments *seg, void *y, int64_t ldy, int32_t d_out, void *ws, size_t ws_bytes);

/* ------------------------------------------------------------------ BGMV
 * Decode-shaped gather (one row per request, "Multi-LoRA Serving in
 * Production ...", section "S-LoRA: MBGMV and MBGMM Kernels": single-token
 * vectors, heterogeneous ranks, no padding).  No plan: the adapter of token t
 * is read from ids_dev[t] on the device, its A/B addresses and rank from the
 * device pool tables.  v rows are in token order.
 *   ids_dev        [T] device int32, -1 = none
 *   pool_A_dev     [n_adapters] device uint64 addresses
 *   pool_rank_dev  [n_adapters] device int32
 *   max_rank       an upper bound of every rank used (host), in [1, 256]
 * Shrink: v[t, j] = sum_k x[t, k] A_{ids[t]}[j, k]; rows of tokens without an
 * adapter are left untouched.  T must be <= 65536.
 * Errors: LORA_ERR_ARG, LORA_ERR_DTYPE, LORA_ERR_RANK, LORA_ERR_ALIGN, LORA_ERR_HIP. */
int lora_bgmv_shrink(void *stream, int dtype, int32_t T, const void *x, int64_t ldx, int32_t d_in,
                     const int32_t *ids_dev, const uint64_t *pool_A_dev,
                     const int32_t *pool_rank_dev, int32_t n_adapters, int32_t max_rank,
                     float *v, int64_t ldv, void *ws, size_t ws_bytes);

/* Expand: y[t, n] += (alpha_i / r_i) * sum_j v[t, j] B_i[n, j], i = ids[t]
 * (alpha_i / r_i formed in fp32 on the device).
 *   pool_B_dev [n_adapters] device uint64; pool_alpha_dev [n_adapters] device fp32. */
int lora_bgmv_expand(void *stream, int dtype, int32_t T, const float *v, int64_t ldv,
                     const int32_t *ids_dev, const uint64_t *pool_B_dev,
                     const int32_t *pool_rank_dev, const float *pool_alpha_dev,
                     int32_t n_adapters, int32_t max_rank,
                     void *y, int64_t ldy, int32_t d_out, void *ws, size_t ws_bytes);

/* Decode correction in one call: the shrink then the expand, with the
 * intermediate kept in the workspace as fp32 partial sums over slices of d_in
 * (fixed summation order).  Needs ws_bytes >=
 * lora_workspace_bytes(LORA_OP_BGMV, T, d_in, d_out, max_rank).
 *
 * One kernel launch when x and y rows are 16-byte aligned, d_out % 16 == 0
 * and max_rank <= 64 (else two): its first workgroups compute the partial
 * sums of (adapter, d_in slice) and store each as one 64-bit word, the value
 * in the low half and the launch's tag in the high half (the top bit set,
 * then 31 bits of a key made from the launch's dispatch id and queue); the
 * others load their B tile and y rows, then load their partial sums until
 * every word holds the tag, then expand (the per-launch cost the pages put on
 * naive per-adapter launches, "Multi-LoRA Serving in Production ...", section
 * "Mathematical Formulation and the Batching Challenge", paid once).  Both
 * forms compute the same sums in the same order, so their outputs are equal.
 *
 * Workspace: a 256-byte status block, the two-launch form's fp32 partial
 * sums, then the one-launch form's tagged words (a region of their own, twice
 * the bytes of the fp32 sums).  Nothing needs
 * preparation or reset between calls: a word left by an earlier launch holds
 * another tag (tags differ between any two of 2^31 consecutive launches on a
 * queue, and never equal the zero of a cleared workspace).  Calls that share a
 * workspace must be ordered on one stream.  The int32 at the start of the
 * workspace is a status word, sticky: nonzero once a wait of the one-launch
 * form gave up (see lora_debug_wait_limit; that call's output is incomplete);
 * lora_workspace_clear resets it.  Allocate the workspace zero-filled (or
 * clear it) so that the status word starts at zero.
 * Errors: as lora_bgmv_shrink, plus LORA_ERR_WORKSPACE. */
int lora_bgmv(void *stream, int dtype, int32_t T, const void *x, int64_t ldx, int32_t d_in,
              const int32_t *ids_dev, const uint64_t *pool_A_dev, const uint64_t *pool_B_dev,
              const int32_t *pool_rank_dev, const float *pool_alpha_dev,
              int32_t n_adapters, int32_t max_rank,
              void *y, int64_t ldy, int32_t d_out, void *ws, size_t ws_bytes);

/* Enqueue a kernel that zero-fills ws_bytes of a workspace (16-byte aligned
 * device memory), which resets lora_bgmv's status word.  A kernel, not a
 * memset, so that it can be recorded in a graph.
 * Errors: LORA_ERR_ARG, LORA_ERR_ALIGN, LORA_ERR_HIP. */
int lora_workspace_clear(void *stream, void *ws, size_t ws_bytes);

/* Diagnostic: polls the one-launch BGMV's wait makes before it gives up, for
 * the calls this thread makes from now on: 0 = the default (about 4 million
 * polls, seconds), > 0 = that many, < 0 = give up at once (used to test the
 * give-up path; the call's output is then incomplete).  Always LORA_OK. */
int lora_debug_wait_limit(int32_t polls);

/* ------------------------------------------------------------ grouped BGMV
 * Several projections of a layer in one kernel launch (or one shrink launch
 * and one expand launch), after the pages' grouped invocation that serves
 * every active adapter of all projections at once instead of one launch per
 * projection ("Multi-LoRA Serving in Production ...", section "Ragged Batching
 * and FlashInfer Grouped GEMM"; the per-launch cost it removes is in section
 * "Kernel Architectures: SGMV, MBGMV, and Grouped GEMMs").  Every projection p applies
 *     y_p[t, :] += (alpha_{i,p} / r_{i,p}) (x_p[t, :] A_{i,p}) B_{i,p},  i = ids[t],
 * with one adapter id per token for all projections and its own x, y, sizes
 * and adapter tables.  Projections whose inputs are the same tensor (q, k, v;
 * gate, up) may pass the same x.  Each projection gives the same result as a
 * lora_bgmv call with its arguments (same d_in split and summation order). */
#define LORA_MAX_PROJ 8 /* projections per grouped call */

typedef struct lora_proj {
    const void *x;              /* device [T, ldx] of the call's dtype */
    void *y;                    /* device [T, ldy]; the y of two projections share no element */
    const uint64_t *pool_A_dev; /* [n_adapters] device addresses of A_{i,p}, [r, d_in] */
    const uint64_t *pool_B_dev; /* [n_adapters] device addresses of B_{i,p}, [d_out, r] */
    const int32_t *pool_rank_dev; /* [n_adapters] device r_{i,p} */
    const float *pool_alpha_dev;  /* [n_adapters] device alpha_{i,p} */
    int64_t ldx, ldy;
    int32_t d_in, d_out;
    int32_t max_rank;           /* upper bound of the projection's ranks, [1, 256] */
    int32_t reserved;           /* 0 */
} lora_proj;

/* Workspace bytes of lora_bgmv_grouped for T tokens and these projections
 * (host array of n_proj, 1 <= n_proj <= LORA_MAX_PROJ); 0 if the arguments
 * are invalid.  Layout: lora_bgmv's 256-byte status block, then for each
 * projection its two-launch fp32 partial sums and its one-launch tagged words
 * (twice those bytes). */
size_t lora_bgmv_grouped_workspace_bytes(int32_t T, const lora_proj *projs, int32_t n_proj);

/*   ids_dev  [T] device int32, -1 = none; n_adapters entries in every table
 *   projs    host array of n_proj projections (read during the call)
 *   ws       device, 16-byte aligned, >= lora_bgmv_grouped_workspace_bytes
 * One kernel launch when every projection has 16-byte aligned x and y rows,
 * d_out % 16 == 0 and max_rank <= 64: the shrink workgroups of all
 * projections first, then their expand workgroups, with lora_bgmv's hand-over
 * (tagged partial sums, no flags, nothing reset between calls) and its sticky
 * status word at the start of the workspace (nonzero once a wait gave up; see
 * lora_debug_wait_limit); allocate the workspace zero-filled or clear it with
 * lora_workspace_clear.  Otherwise one shrink and one expand launch.  Calls
 * that share a workspace must be ordered on one stream.
 * Errors: LORA_ERR_ARG (also: two projections with the same y), LORA_ERR_DTYPE,
 * LORA_ERR_RANK, LORA_ERR_ALIGN, LORA_ERR_WORKSPACE, LORA_ERR_HIP. */
int lora_bgmv_grouped(void *stream, int dtype, int32_t T, const int32_t *ids_dev, int32_t n_adapters,
                      const lora_proj *projs, int32_t n_proj, void *ws, size_t ws_bytes);

/* ------------------------------------------------------------ grouped SGMV
 * The prefill form of the grouped invocation (same sections as grouped BGMV):
 * several projections of a layer, each with its own plan, x, y and sizes, in
 * one shrink launch and one expand launch.  Each projection's plan is built
 * (lora_build_segments) from the batch's ids with that projection's adapter
 * tables, so every projection applies
 *     y_p[t, :] += (alpha_{i,p} / r_{i,p}) (x_p[t, :] A_{i,p}) B_{i,p},  i = ids[t].
 * Projections whose inputs are the same tensor (q, k, v; gate, up) may pass the
 * same x.  The expand takes the 64-row chunk form when every projection's
 * ranks are <= 32 and the projections together give at least 1024 (chunk,
 * 256-column tile) items, else the 16-row block form; a projection's result
 * equals that of a lora_sgmv call that takes the same kernel variants (same
 * expand form and d_in split), and is within the stated tolerance of the exact
 * result in every case. */
typedef struct lora_sgmv_proj {
    const void *x;          /* device [T, ldx] of the call's dtype */
    void *y;                /* device [T, ldy]; the y of two projections share no element */
    const lora_segments *seg; /* this projection's segments, uploaded (device struct) */
    int64_t ldx, ldy;
    int32_t d_in, d_out;
} lora_sgmv_proj;

/* Workspace bytes of lora_sgmv_grouped for these projections (host array of
 * n_proj, 1 <= n_proj <= LORA_MAX_PROJ, plans already built); 0 if the
 * arguments are invalid. */
size_t lora_sgmv_grouped_workspace_bytes(const lora_sgmv_proj *projs, int32_t n_proj);

/*   projs    host array of n_proj projections (read during the call)
 *   ws       device, 16-byte aligned, >= lora_sgmv_grouped_workspace_bytes
 * Projections whose plan has no adapted token are skipped.
 * Errors: LORA_ERR_ARG (also: two projections with the same y), LORA_ERR_DTYPE,
 * LORA_ERR_RANK, LORA_ERR_ALIGN, LORA_ERR_PLAN, LORA_ERR_WORKSPACE, LORA_ERR_HIP. */
int lora_sgmv_grouped(void *stream, int dtype, const lora_sgmv_proj *projs, int32_t n_proj, void *ws,
                      size_t ws_bytes);

/* ------------------------------------------------------------ adapter residency
 * The GPU and host tiers of the pages' adapter storage ("Multi-LoRA Serving:
 * Many Adapters on One GPU" (gpusmith.com), section "Swap latency and cache
 * policy"; "Multi-LoRA Serving in Production ..." (llms.blog), sections
 * "Tiered Storage Hierarchy and Asynchronous Streaming" and "Eviction and
 * Replacement Policies"): adapters live in pinned host memory and are copied
 * into HBM on a copy stream when a batch needs them; when HBM is full the
 * least recently used adapter that is neither pinned nor in the batch is
 * evicted.
 *
 * The cache manages a caller-owned device buffer: the first
 * lora_cache_table_bytes(n_adapters) bytes hold the device tables the kernels
 * read (pool_A, pool_B, rank, alpha, indexed by adapter id; zero for an adapter
 * that is not resident), the rest holds adapter extents (A [r, d_in] then
 * B [d_out, r], 256-byte aligned, not padded to a maximum rank).  One cache
 * serves one projection shape (d_in, d_out) and dtype.  It never allocates
 * device memory; it allocates a few pinned host staging buffers and events.
 * Not thread-safe: one host thread drives a cache.
 */
typedef struct lora_cache lora_cache;

#define LORA_CACHE_DRY 1u /* placement and statistics only: no GPU call, no copy (host-side tests) */

typedef struct lora_cache_stats {
    int64_t batches;        /* lora_cache_prepare calls that succeeded */
    int64_t hits;           /* adapters of a batch that were already resident */
    int64_t misses;         /* adapters copied in */
    int64_t evictions;
    int64_t bytes_copied;   /* adapter bytes copied host -> device */
    int64_t resident_bytes; /* bytes of the extents resident now */
    int32_t resident;       /* adapters resident now */
    int32_t reserved;
} lora_cache_stats;

typedef struct lora_cache_view {
    const uint64_t *pool_A_dev; /* device tables [n_adapters], for the BGMV calls */
    const uint64_t *pool_B_dev;
    const int32_t *rank_dev;
    const float *alpha_dev;
    const uint64_t *pool_A_host; /* host mirrors, current after the last prepare: the */
    const uint64_t *pool_B_host; /* inputs of lora_build_segments for the batch */
    const int32_t *rank_host;
    const float *alpha_host;
    int32_t n_adapters;
    int32_t max_rank; /* largest registered rank */
} lora_cache_view;

/* Bytes at the start of the device buffer that hold the tables. */
size_t lora_cache_table_bytes(int32_t n_adapters);

/* dev_buf: device memory, 256-byte aligned, dev_bytes > table bytes; it must
 * outlive the cache.  flags: 0 or LORA_CACHE_DRY.  Zeroes the tables (a
 * synchronous hipMemset) unless dry.
 * Errors: LORA_ERR_ARG, LORA_ERR_DTYPE, LORA_ERR_ALIGN, LORA_ERR_WORKSPACE, LORA_ERR_HIP. */
int lora_cache_create(void *dev_buf, size_t dev_bytes, int32_t n_adapters, int dtype, int32_t d_in,
                      int32_t d_out, unsigned flags, lora_cache **out);

/* Waits for the cache's own staging copies, then frees its host resources. */
void lora_cache_destroy(lora_cache *cache);

/* Host copy of adapter `adapter`: A_host [rank, d_in], B_host [d_out, rank]
 * row-major of the cache's dtype; pinned memory (hipHostMalloc) for copies that
 * overlap compute.  The memory must stay valid while the adapter may be loaded.
 * Errors: LORA_ERR_ARG (also: adapter resident), LORA_ERR_ADAPTER_ID, LORA_ERR_RANK. */
int lora_cache_register(lora_cache *cache, int32_t adapter, const void *A_host, const void *B_host,
                        int32_t rank, float alpha);

/* A pinned adapter is never evicted (the pages' priority tiers). */
int lora_cache_pin(lora_cache *cache, int32_t adapter, int pinned);

/* Make every adapter of a batch (ids_host [T], -1 = none) resident before the
 * work enqueued next on compute_stream.  Copies of missing adapters and the
 * table update are enqueued on copy_stream, after the compute work that last
 * read any space they reuse; compute_stream then waits for them (only when a
 * copy was needed).  No host synchronisation.  Build the batch's plan from the
 * view's host mirrors after this call.
 * Errors: LORA_ERR_ARG, LORA_ERR_ADAPTER_ID (id out of range or not
 * registered), LORA_ERR_WORKSPACE (the batch does not fit, or the free space is
 * too fragmented once every evictable adapter is gone), LORA_ERR_HIP.  After an
 * error the batch must not run; the cache stays consistent. */
int lora_cache_prepare(lora_cache *cache, const int32_t *ids_host, int32_t T, void *copy_stream,
                       void *compute_stream);

int lora_cache_view_get(const lora_cache *cache, lora_cache_view *out);
int lora_cache_stats_get(const lora_cache *cache, lora_cache_stats *out);

/* ------------------------------------------------------------ paged adapter storage
 * The pages' unified paging ("Multi-LoRA Serving in Production ..."
 * (llms.blog), section "Unified Paged Memory"; "Multi-LoRA serving: the single
 * translator with a thousand glossaries" (blog.lo0.es), section "Operational
 * pitfalls", on memory fragmentation): adapter matrices are cut into fixed-size pages held in
 * non-contiguous frames of one device pool, and a page table per matrix maps
 * its logical pages to frames, so adapters of any rank come and go without
 * fragmenting HBM.
 *
 * Layout.  `pages` is a caller-owned device buffer of n_frames * page_bytes
 * bytes, 16-byte aligned; page_bytes is a power of two in [64, 2^24] (the
 * pages name 16 KB and 64 KB).  A matrix of `bytes` bytes (A_i [r_i, d_in] or
 * B_i [d_out, r_i], row-major, as in the dense pool) occupies
 * lora_pages_needed(bytes, page_bytes) frames; its page table is a device
 * int32 array whose entry p is the frame of logical page p, so byte b of the
 * matrix lives at pages + table[b / page_bytes] * page_bytes + b % page_bytes.
 * Each page table must start on a 16-byte boundary.  Frame numbers are device
 * data: that every entry is in [0, n_frames) is a precondition (like the BGMV
 * ids); the kernels do not check it.
 *
 * The paged calls take the same plans and tables as the dense ones, with the
 * address of each adapter's A and B page tables where the dense pool has the
 * address of A and B.  They run the same kernels with the element address
 * looked up through the page table, so for the same inputs they return the
 * same bits as lora_sgmv / lora_bgmv. */

/* Frames a matrix of `bytes` bytes needs: ceil(bytes / page_bytes); -1 if
 * bytes < 0 or page_bytes is not a power of two in [64, 2^24]. */
int64_t lora_pages_needed(int64_t bytes, int64_t page_bytes);

/* Host allocator of the frames of one pool: a free list, so any request for at
 * most lora_page_alloc_free_count() frames succeeds whatever the order of
 * earlier allocations and frees (no fragmentation).  Frames come back in the
 * order they were freed last-in first-out.  Host memory only; not
 * thread-safe: one thread drives an allocator. */
typedef struct lora_page_alloc lora_page_alloc;

/* n_frames in [1, 2^31 - 1].  Errors: LORA_ERR_ARG. */
int lora_page_alloc_create(int32_t n_frames, lora_page_alloc **out);
void lora_page_alloc_destroy(lora_page_alloc *alloc);

/* Takes n frames into frames_out (host int32 [n]), all or nothing.
 * Errors: LORA_ERR_ARG (n < 0, NULL), LORA_ERR_WORKSPACE (fewer than n free). */
int lora_page_alloc_take(lora_page_alloc *alloc, int32_t n, int32_t *frames_out);

/* Returns n frames (host int32 [n]) to the free list, all or nothing.
 * Errors: LORA_ERR_ARG (a frame out of range, not taken, or repeated). */
int lora_page_alloc_give(lora_page_alloc *alloc, const int32_t *frames, int32_t n);

/* Free frames now; -1 for NULL. */
int32_t lora_page_alloc_free_count(const lora_page_alloc *alloc);

/* Copies `bytes` bytes of a matrix from src (device memory, or host memory
 * the device can read, 16-byte aligned) into its frames:
 * logical page p goes to pages + table_dev[p] * page_bytes.  One kernel on
 * `stream`.  table_dev: device int32 [lora_pages_needed(bytes, page_bytes)].
 * Errors: LORA_ERR_ARG, LORA_ERR_ALIGN, LORA_ERR_HIP. */
int lora_pages_write(void *stream, void *pages, int64_t page_bytes, const int32_t *table_dev,
                     const void *src, int64_t bytes);

/* lora_sgmv over paged adapters: the segments were built (lora_build_segments)
 * with pool_A[i] / pool_B[i] = device addresses of adapter i's A and B page
 * tables.
 * Errors: as lora_sgmv, plus LORA_ERR_ARG / LORA_ERR_ALIGN for pages or
 * page_bytes. */
int lora_sgmv_paged(void *stream, int dtype, const void *x, int64_t ldx, int32_t d_in,
                    const lora_segments *seg, const void *pages, int64_t page_bytes,
                    void *y, int64_t ldy, int32_t d_out, void *ws, size_t ws_bytes);

/* lora_bgmv over paged adapters: pool_A_dev[i] / pool_B_dev[i] are the
 * device addresses of adapter i's A and B page tables.  Same workspace,
 * one-launch condition, hand-over and status word as lora_bgmv.
 * Errors: as lora_bgmv, plus LORA_ERR_ARG / LORA_ERR_ALIGN for pages or
 * page_bytes. */
int lora_bgmv_paged(void *stream, int dtype, int32_t T, const void *x, int64_t ldx, int32_t d_in,
                    const int32_t *ids_dev, const uint64_t *pool_A_dev, const uint64_t *pool_B_dev,
                    const int32_t *pool_rank_dev, const float *pool_alpha_dev,
                    int32_t n_adapters, int32_t max_rank, const void *pages, int64_t page_bytes,
                    void *y, int64_t ldy, int32_t d_out, void *ws, size_t ws_bytes);

/* ------------------------------------------------------------------ fused layer
 * The whole adapted layer: the shared base product once for every token plus
 * each token's correction, y = x W0 + scale_s (x A_s) B_s, overwriting y
 * ("Multi-LoRA Serving" (fp-ai-systems.pages.dev), section "Serving it: batch
 * across adapters": one shared matmul for all requests plus a per-request
 * low-rank correction; "Multi-LoRA Serving in Production ...", layer equation).
 * Tokens without an adapter get x W0 only.  bf16 only; W0 is [d_out, d_in]
 * with row pitch d_in.  x, W0, y and the workspace must be 16-byte aligned,
 * ldx and ldy multiples of 8 elements and d_in a multiple of 8 (d_out is
 * free).  Enqueues three kernels: the SGMV shrink into the workspace, a pass
 * that writes scale_s * v as two bf16 halves (hi + lo, 16 significant bits),
 * and one GEMM over the plan's rows whose bf16 MFMA accumulators also take the
 * correction (fp32 accumulation, one rounding to bf16).  The plan must come
 * from the same batch (its perm also lists the tokens without an adapter).
 * Needs ws_bytes >= lora_workspace_bytes(LORA_OP_FUSED, T, d_in, d_out, max_rank)
 * (the shrink's slice partials plus T * 2 * round16(max_rank) bf16).
 * x (T rows at pitch ldx) and W0 must each span less than 4 GiB: the GEMM
 * addresses their rows with 32-bit byte offsets.
 * Errors: as lora_sgmv_shrink; LORA_ERR_DTYPE for fp32; LORA_ERR_ALIGN for
 * the alignment rules above; LORA_ERR_ARG for x or W0 of 4 GiB or more;
 * LORA_ERR_WORKSPACE. */
int lora_fused_linear(void *stream, int dtype, const void *x, int64_t ldx, int32_t d_in,
                      const void *W0, int32_t d_out, const lora_segments *seg,
                      void *y, int64_t ldy, void *ws, size_t ws_bytes);

/* The fused layer over an FP8 base: W0 holds one OCP E4M3 code per element
 * (sign, 4-bit exponent of bias 7, 3-bit mantissa; subnormals; the two codes
 * 0x7F and 0xFF are NaN; largest finite 448) and stands for w0_scale * code,
 * one fp32 scale for the whole matrix; x, y and the adapters are bf16
 * ("Multi-LoRA serving: the single translator with a thousand glossaries"
 * (blog.lo0.es), section "Combined pattern with quantisation and
 * disaggregated serving": BF16 adapters over an FP8 base; the pages fix no
 * scale granularity, one per matrix is the plainest reading).
 * y = x (w0_scale q)^T + scale_s (x A_s) B_s, overwriting y.  The codes are
 * widened to bf16 exactly (an E4M3 value has 4 significant bits) and
 * multiplied on bf16 MFMA with fp32 accumulation; the accumulator holds
 * x q^T + (scale_s / w0_scale) v B_s and is multiplied by w0_scale once
 * before the single rounding to bf16.  Same launches, plan, workspace
 * (lora_workspace_bytes(LORA_OP_FUSED, ...)) and rules as lora_fused_linear,
 * except: W0 is [d_out, d_in] bytes with row pitch d_in, 16-byte aligned,
 * d_in a multiple of 16, and W0 must span less than 4 GiB.
 * Errors: as lora_fused_linear; LORA_ERR_ARG also for a w0_scale that is zero,
 * infinite or NaN; LORA_ERR_ALIGN for d_in % 16 != 0. */
int lora_fused_linear_e4m3(void *stream, const void *x, int64_t ldx, int32_t d_in,
                           const void *W0, float w0_scale, int32_t d_out,
                           const lora_segments *seg, void *y, int64_t ldy,
                           void *ws, size_t ws_bytes);

/* ------------------------------------------------------------------ helpers */
enum {
    LORA_OP_SGMV_SHRINK = 0,
    LORA_OP_SGMV_EXPAND = 1,
    LORA_OP_BGMV_SHRINK = 2,
    LORA_OP_BGMV_EXPAND = 3,
    LORA_OP_FUSED = 4,
    LORA_OP_SGMV = 5,
    LORA_OP_BGMV = 6
};

/* Workspace bytes an op needs (0 = none; ws may then be NULL); -1 cast to
 * size_t on a bad op code. */
size_t lora_workspace_bytes(int op, int32_t T, int32_t d_in, int32_t d_out, int32_t max_rank);

/* Adapter parameters of one adapted d_in -> d_out projection at rank r:
 * r (d_in + d_out) ("Multi-LoRA Serving: Many Adapters on One GPU"
 * (gpusmith.com), section "LoRA recap and why adapters are small").
 * Returns -1 for a negative argument. */
int64_t lora_adapter_numel(int32_t r, int32_t d_in, int32_t d_out);

/* Static text for a status code; never NULL. */
const char *lora_status_string(int status);

/* Message of the last failed call on this thread ("" if none). */
const char *lora_last_error(void);

/* Timing of the library's own kernels, for benchmarks: the next `count`
 * kernels this thread enqueues through the library record start_events[i]
 * when kernel i begins and stop_events[i] when it ends (hipEvent_t handles
 * created by the caller with hipEventCreate; the arrays and events must stay
 * valid until those launches have been enqueued).  count = 0 cancels a
 * pending request.  The request is per thread.
 * Errors: LORA_ERR_ARG (negative count, NULL array or event). */
int lora_profile_launches(void **start_events, void **stop_events, int32_t count);

/* Number of events of the current lora_profile_launches request that kernels
 * have taken so far on this thread (how many kernels a call enqueued). */
int32_t lora_profile_launches_used(void);

/* ------------------------------------------------------------ no allocation
 * lora_bgmv for callers that cannot allocate device memory or pass a
 * workspace (code under graph capture, tight serving loops, harnesses that
 * forbid allocation).  The arguments are lora_bgmv's without the workspace: the
 * fp32 slice partial sums live in a static array the library holds on every
 * device it runs on (LORA_NOALLOC_SCRATCH_BYTES each, until the process ends),
 * and the call runs lora_bgmv's shrink and expand kernels (two launches) on
 * the current device.  The shrink writes every partial sum the expand reads,
 * so the array needs no clearing between calls.  Calls on one device share
 * the array: calls that may overlap on one device (streams without an
 * ordering between them) race.  The call allocates and frees nothing.
 * Errors: as lora_bgmv; LORA_ERR_WORKSPACE when the batch's partial sums
 * (lora_workspace_bytes(LORA_OP_SGMV, T, d_in, d_out, max_rank)) exceed the
 * array; LORA_ERR_HIP when the array's device address cannot be found. */
#define LORA_NOALLOC_SCRATCH_BYTES (4u << 20)
int lora_bgmv_noalloc(void *stream, int dtype, int32_t T, const void *x, int64_t ldx, int32_t d_in,
                      const int32_t *ids_dev, const uint64_t *pool_A_dev, const uint64_t *pool_B_dev,
                      const int32_t *pool_rank_dev, const float *pool_alpha_dev, int32_t n_adapters,
                      int32_t max_rank, void *y, int64_t ldy, int32_t d_out);

/* ------------------------------------------------------------ measurement aids
 * Reference kernels a benchmark times beside the adapter kernels, so that each
 * adapter kernel can be read against what the chip achieves for the same
 * bytes without the method's dependent loads.  None of them is part of the
 * adapter path.
 *
 * lora_probe_empty: an empty kernel of `workgroups` workgroups of 256 threads
 * (the per-launch floor).  Errors: LORA_ERR_ARG, LORA_ERR_HIP. */
int lora_probe_empty(void *stream, int32_t workgroups);

/* One kernel that reads read_bytes of src and reads, modifies and writes back
 * rmw_bytes of rmw (the data written equals the data read), with 16-byte
 * accesses, over at most max_workgroups workgroups split in proportion to the
 * bytes each part moves.  Both counts are multiples of 16, the buffers are
 * 16-byte aligned device memory; sink is a device buffer of max_workgroups
 * uint32 that the kernel may write.  Errors: LORA_ERR_ARG, LORA_ERR_ALIGN,
 * LORA_ERR_HIP. */
int lora_probe_stream(void *stream, const void *src, int64_t read_bytes, void *rmw, int64_t rmw_bytes, void *sink,
                      int32_t max_workgroups);

/* One lane of one workgroup follows `steps` dependent loads i = next[i] from
 * i = 0 (the cost of a global-memory round trip), then writes i to sink[0].
 * Every next[i] reached must index inside the caller's array.
 * Errors: LORA_ERR_ARG, LORA_ERR_HIP. */
int lora_probe_chase(void *stream, const uint32_t *next, int32_t steps, uint32_t *sink);

/* Library version string. */
const char *lora_version(void);

#ifdef __cplusplus
}
#endif

#endif /* LORA_MI355X_H */
