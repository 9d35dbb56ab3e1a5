/*
 * blasst.h -- C ABI of the MI355X (gfx950) block-skipping attention library
 * (libblasst.so).
 *
 * The method: "BLASST: Dynamic BLocked Attention Sparsity via Softmax
 * Thresholding" (gist.science/pt/paper/2512.12087, section 2 "Metodologia:
 * BLASST"; the same in gist.science/hi/paper/2512.12087, section 2).  A
 * FlashAttention-style blockwise online-softmax forward pass keeps a running
 * row max m; for every key block it forms the block-local row max m~ and skips
 * the block when m~ - m < ln(lambda).  A skipped block does no exponential, no
 * V-block load and no P.V product.  The threshold follows lambda = a / L, with
 * a fitted per target sparsity (BLASST summary, gist.science/pt/paper/2512.12087,
 * section 2 "Calibração Automática"; BLASST reading
 * notes, papers.lqhl.me/papers/BLASST-MLSys26, "关键观察" observation 2).
 *
 * Conventions shared by every entry point
 *  - Tensors are described by blasst_tensor: a DEVICE pointer, an element type
 *    and strides IN ELEMENTS for the batch, head and token dimensions; the
 *    last (feature) dimension is always contiguous.  Every device buffer is
 *    allocated and owned by the caller; the library allocates no device
 *    memory in any call and keeps no pointer after a call returns (the one
 *    array it owns, the scratch of blasst_decode_noalloc, exists from the
 *    loading of its device code).
 *  - Calls are asynchronous: they validate their arguments on the host,
 *    enqueue kernels on the given HIP stream (a hipStream_t passed as void*;
 *    NULL = the default stream) and return.  Outputs are valid once the stream
 *    has been synchronised.
 *  - Validation happens before any launch, so a call that returns an error
 *    has written nothing.  blasst_last_error() then holds a message naming the
 *    offending argument (per calling thread).
 *  - "Query tile" and "key block": decisions are taken per (query tile, key
 *    block) pair.  A query tile skips a key block only if EVERY valid row of
 *    the tile meets the criterion (the pages decide per block, see the BLASST
 *    reading notes, "设计取舍": block rather than token granularity).
 *  - Skip map entries: 0 = executed, 1 = skipped, 255 = not visited (no
 *    unmasked (row, key) entry in the pair).  Gap map entries: the tile gap
 *    g = max over valid rows of (m~ - m) in natural-log units of the scaled
 *    scores; +inf for a unit's first visited block (m = -inf there); -inf for
 *    pairs that are not visited.  Every entry of both maps is written.
 *  - Counters (optional, device, two uint64): [0] += visited pairs,
 *    [1] += skipped pairs.  They are accumulated atomically; the caller zeroes
 *    them.  Block sparsity = counters[1] / counters[0].
 *  - Arithmetic: bf16 inputs, fp32 scores and accumulation; the skip test is
 *    evaluated in fp32 on the scaled scores (scale applied in fp32, never folded
 *    into the bf16 query).
 */
#ifndef BLASST_H
#define BLASST_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define BLASST_ABI_VERSION 3

typedef enum {
    BLASST_OK = 0,
    BLASST_ERR_INVALID_ARG = 1, /* bad pointer, size, stride, lambda, ... */
    BLASST_ERR_UNSUPPORTED = 2, /* valid request with no compiled kernel (head dim, tile, dtype) */
    BLASST_ERR_WORKSPACE = 3,   /* workspace missing or smaller than blasst_decode_plan() asked */
    BLASST_ERR_LAUNCH = 4       /* the HIP runtime refused the launch */
} blasst_status;

typedef enum { BLASST_BF16 = 0, BLASST_FP32 = 1 } blasst_dtype;

typedef struct {
    void *ptr;          /* device pointer to element [0,0,0,0] */
    blasst_dtype dtype;
    int64_t sb, sh, st; /* strides in elements: batch, head, token (token unused for 3-D tensors) */
} blasst_tensor;

/* ------------------------------------------------------------------ prefill
 * blasst_prefill(Q, K, V, causal, lambda, tile sizes): the blockwise skip
 * forward for a whole sequence (Lq = Lk = L; with causal masking query i sees
 * keys 0..i).  Query head h reads KV head h / (Hq / Hkv) (MHA when Hq = Hkv,
 * GQA, MQA when Hkv = 1).  Key blocks are visited in ascending order.
 *
 *   q  [B, Hq, L, d]   bf16          k [B, Hkv, L, d]  bf16
 *   v  [B, Hkv, L, dv] bf16          o [B, Hq, L, dv]  fp32 or bf16 (written)
 *   d = dv in {64, 128}; tile_q in {64, 128}; block_k = 64.
 *   scale   : multiplies q.k; <= 0 selects 1/sqrt(d).
 *   lambda  : in [0, 1).  0 disables skipping and runs the dense kernel.
 *   skip_map: optional device uint8 [B, Hq, nQT, nKB], nQT = ceil(L/tile_q),
 *             nKB = ceil(L/block_k), contiguous.
 *   gap_map : optional device float [B, Hq, nQT, nKB], contiguous.
 *   counters: optional device uint64 [2].
 *   window  : 0 = none; W > 0 (causal only) = sliding window: query i sees
 *             keys i - W < c <= i.  The BLASST reading notes
 *             (papers.lqhl.me/papers/BLASST-MLSys26, "问题与动机") list
 *             sliding-window attention among the supported forms.  Key blocks
 *             with no key inside any row's window are not visited (255 in the
 *             skip map); the skip test runs unchanged on the others.
 * Errors: INVALID_ARG for null q/k/v/o, L < 0, B < 0, Hq or Hkv <= 0,
 * Hq % Hkv != 0, lambda outside [0,1) or NaN, window < 0 or a window without
 * causal masking, a non-positive stride or a
 * pointer not aligned to 16 bytes with a token stride not a multiple of 8
 * elements; UNSUPPORTED for other d, dv, tile or dtype, for L > 2^30, for
 * B * Hq * nQT above (2^32 - 1) / (2 tile_q) (one workgroup of 2 tile_q
 * threads each; a launch counts threads in 32 bits), and for k or v token
 * strides above 2^24 elements; LAUNCH if HIP fails.
 * L = 0 or B = 0 is a valid no-op: only the scalar arguments are checked and
 * the tensor pointers may be null.
 */
typedef struct {
    blasst_tensor q, k, v, o;
    int64_t B, Hq, Hkv, L, d, dv;
    int causal;
    double scale;
    double lambda;
    int tile_q;
    int block_k;
    uint8_t *skip_map;
    float *gap_map;
    unsigned long long *counters;
    int64_t window;
} blasst_prefill_params;

blasst_status blasst_prefill(const blasst_prefill_params *p, void *hip_stream);

/* The gap pass of blasst_prefill, for calibration (BLASST summary,
 * gist.science/pt/paper/2512.12087, section 2 "Calibração Automática": the
 * threshold for a target sparsity is found by a search over the sparsity it
 * achieves; BLASST reading notes, "核心方法": automatic lambda search).  It
 * forms the same scores, block maxima, running max and decisions (at
 * p->lambda) as blasst_prefill and writes the same skip map, gap map and
 * counters, with no exponential, no V load, no P.V product and no output:
 * p->o is neither read nor written and may be null.  The running max never
 * depends on the decisions (a skipped block has m~ < m + ln(lambda) <= m), so
 * the gap map is blasst_prefill's at any lambda and the lambda of a target
 * sparsity is a quantile of it (blasst_calibrate_search).
 * Errors: as blasst_prefill, plus INVALID_ARG when gap_map, skip_map and
 * counters are all null. */
blasst_status blasst_prefill_gaps(const blasst_prefill_params *p, void *hip_stream);

/* ------------------------------------------------------------------- decode
 * blasst_decode(q, KV cache, seq lens, lambda): one query token per sequence
 * against a KV cache.  A query tile is the group of G = Hq / Hkv query heads
 * that share one KV head (GQA; MQA when Hkv = 1; MHA when G = 1); MLA in its
 * absorbed form is Hkv = 1 with a latent cache whose first dv columns are the
 * values (pass v_cache.ptr == k_cache.ptr with the same strides).
 *
 * Split-K: the nkb = ceil(seq_len/block_k) key blocks of a sequence are cut
 * into num_splits contiguous runs of ceil(nkb/num_splits) blocks; each run is
 * processed from m = -inf (so its first block is always executed) and the run
 * partials are merged with the log-sum-exp rule.  Decisions therefore depend
 * on num_splits; the value used is reported by blasst_decode_plan().
 *
 *   q       [B, Hq, dqk] bf16 (sb, sh)       o [B, Hq, dv] fp32 or bf16 (sb, sh)
 *   k_cache [B, Hkv, Lmax, dqk] bf16         v_cache [B, Hkv, Lmax, dv] bf16
 *   seq_lens: device int32 [B], each in 1..Lmax (the kernel clamps other
 *             values into 0..Lmax; a length of 0 yields O = 0).
 *   Supported: (dqk = dv in {64, 128}, G in 1..64: MHA, GQA and MQA) and the latent form
 *   (dqk = 576, dv = 512, Hkv = 1, G in 1..128 -- all heads of a model, or
 *   a shard of them when heads are split across GPUs -- v aliasing k).
 *   block_k = 64.
 *   num_splits: 0 lets the library choose; otherwise 1..nKB.
 *   skip_map / gap_map: optional device [B, Hkv, nKB], nKB = ceil(Lmax/64).
 *   B = 0 is a valid no-op: only the scalar arguments are checked, the
 *             pointers may be null and the planned workspace is 0 bytes.
 *   window  : 0 = none; W > 0 = sliding window (see blasst_prefill): the
 *             query, at position seq_len-1, sees the last W keys.  The splits
 *             then cut the blocks from the first one holding such a key,
 *             j0 = max(0, seq_len - W) / 64, into runs of
 *             ceil((nkb - j0) / num_splits) blocks.
 *   sink_seed: 0 = every split starts its running max from -inf.  Nonzero:
 *             splits after the first start it from the row maxima of the
 *             sequence's first visible block (block j0; the sink block 0
 *             without a window), so a cold split may skip even its first
 *             blocks, or all of them.  This applies the pseudo-maximum of
 *             the FFD summary (gist.science/pt/paper/2609.00097, section 2,
 *             top-delta selection: a max estimated from sink and local
 *             tokens) to the split start.  The seed is a real score of a
 *             visible key, so the skip test keeps its bound on the dropped
 *             mass.  It costs one extra block of scores per seeded split.
 */
typedef struct {
    blasst_tensor q, k_cache, v_cache, o;
    const int32_t *seq_lens;
    int64_t B, Hq, Hkv, Lmax, dqk, dv;
    double scale;
    double lambda;
    int block_k;
    int num_splits;
    uint8_t *skip_map;
    float *gap_map;
    unsigned long long *counters;
    int64_t window;
    int sink_seed;
} blasst_decode_params;

/* Host-only: the split count a call with *p will use and the device workspace
 * (bytes) it needs; either output pointer may be NULL.  Same validation as
 * blasst_decode.  With more than one split the workspace holds each split's
 * fp32 partial output, max and sum per query head, and each split's block
 * counts (merged into counters by the combine step); with one split it is 0. */
blasst_status blasst_decode_plan(const blasst_decode_params *p, int *num_splits_used,
                                 size_t *workspace_bytes);

/* workspace: caller-owned device buffer of at least the planned size (may be
 * NULL when the planned size is 0).  Calls that share one workspace must be
 * ordered on one stream.
 * Errors: INVALID_ARG for null q/k_cache/v_cache/o/seq_lens, B < 0, Lmax < 1,
 * Hq or Hkv <= 0, Hq % Hkv != 0, lambda outside [0,1) or NaN, a non-finite
 * scale, window < 0,
 * num_splits outside 0..nKB, a non-positive stride or a pointer or stride not
 * aligned to 16 bytes; UNSUPPORTED for other head shapes or dtypes, a latent
 * cache whose v_cache does not alias k_cache, a latent cache with
 * Lmax * token stride * 2 >= 2^31 bytes, Lmax > 2^30, or B or Hkv > 65535;
 * WORKSPACE for a missing or too small workspace; LAUNCH if HIP fails. */
blasst_status blasst_decode(const blasst_decode_params *p, void *workspace, size_t workspace_bytes,
                            void *hip_stream);

/* The gap pass of blasst_decode, for calibration (see blasst_prefill_gaps):
 * the same split plan (blasst_decode_plan), scores, decisions at p->lambda,
 * skip map, gap map and counters, with no V load, no exponential, no P.V
 * product, no split partials and no output.  Needs no workspace; p->o is
 * neither read nor written and may be null.
 * Errors: as blasst_decode (without WORKSPACE), plus INVALID_ARG when gap_map,
 * skip_map and counters are all null. */
blasst_status blasst_decode_gaps(const blasst_decode_params *p, void *hip_stream);

/* ------------------------------------------------------------ paged decode
 * blasst_decode over a paged KV cache, the layout of serving engines: the
 * cache rows of every sequence live in fixed-size pages of one shared pool,
 * found through a per-sequence page table.  The pages name integration into
 * serving stacks (TensorRT-LLM, FlashInfer: gist.science/pt/paper/2512.12087,
 * section 3, contribution 4) and end-to-end runs with PagedAttention serving
 * (BLASST reading notes, papers.lqhl.me/papers/BLASST-MLSys26, "局限与后续工作"
 * future work 2).  The result equals blasst_decode on the contiguous cache
 * obtained by gathering every sequence's pages in table order: the method,
 * the split rule, the decisions and the outputs are the same; only the
 * address of a cache row changes.
 *
 *   d            : the decode parameters, with d.k_cache / d.v_cache
 *                  describing the page POOLS instead of per-sequence caches:
 *                  k pool [num_pages, Hkv, page_size, dqk], strides
 *                  (sb = page stride, sh = head stride, st = row stride);
 *                  likewise the v pool (dv columns).  Any stride order works
 *                  ([page, row, head, d] pools pass sh = d, st = Hkv * d).
 *                  d.Lmax is the largest sequence length of the call (it
 *                  sizes the skip and gap maps as in blasst_decode).
 *   page_table   : device int32 [B, page_table_stride]; entry i of row b is
 *                  the pool page holding rows [i * page_size, (i+1) *
 *                  page_size) of sequence b.  Only entries
 *                  i < ceil(seq_lens[b] / page_size) are read.  An id outside
 *                  [0, num_pages) is clamped into that range (it reads a wrong
 *                  page but never outside the pool).  K and V share the table.
 *   page_table_stride : elements between table rows, >= ceil(Lmax/page_size).
 *   num_pages    : pages in each pool (>= 1).
 *   page_size    : rows per page, a power of two >= 16.
 * Errors: as blasst_decode, plus INVALID_ARG for a null table, num_pages < 1,
 * a page size that is not a power of two >= 16, or a table stride below
 * ceil(Lmax/page_size); UNSUPPORTED for the latent form when one page spans
 * 2^31 bytes or more.
 */
typedef struct {
    blasst_decode_params d;
    const int32_t *page_table;
    int64_t page_table_stride;
    int64_t num_pages;
    int64_t page_size;
} blasst_decode_paged_params;

/* Host-only planner of blasst_decode_paged (same contract as
 * blasst_decode_plan). */
blasst_status blasst_decode_paged_plan(const blasst_decode_paged_params *p, int *num_splits_used,
                                       size_t *workspace_bytes);

blasst_status blasst_decode_paged(const blasst_decode_paged_params *p, void *workspace,
                                  size_t workspace_bytes, void *hip_stream);

/* ---------------------------------------------------- no-allocation decode
 * For callers that cannot allocate device memory: code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc.
 * blasst_decode_noalloc is blasst_decode (same parameters, kernels, split plan,
 * decisions and outputs) with the split partials kept in a device array that
 * the library owns instead of a caller workspace.  Each GPU the library runs
 * on holds its own array of BLASST_NOALLOC_SCRATCH_BYTES from the loading of
 * the library's device code until the process ends; the call itself allocates
 * nothing.  Its device address is looked up on the first call on each device
 * (the current device, which must be the device of hip_stream).
 *
 * Every call on one GPU shares that GPU's array and leaves its partials in
 * it.  Calls ordered on one stream are safe; calls that overlap on one GPU
 * (several streams, or threads without ordering) race and give wrong outputs.
 * The caller still passes every input and output buffer.
 * Errors: as blasst_decode, plus WORKSPACE when the split partials of the
 * planned split count (blasst_decode_plan) exceed BLASST_NOALLOC_SCRATCH_BYTES
 * (pass a smaller num_splits), and LAUNCH when no current device exists or the
 * array's address cannot be found.
 */
#define BLASST_NOALLOC_SCRATCH_BYTES (96u * 1024u * 1024u)

blasst_status blasst_decode_noalloc(const blasst_decode_params *p, void *hip_stream);

/* ---------------------------------------------------------------- calibrate
 * blasst_calibrate(target_sparsity, L) -> lambda = a(target) / L.  The table
 * holds a fitted per target sparsity (strictly increasing targets, a > 0); ln a
 * is interpolated linearly in the target between rows.  Host only.
 *
 * A fitted a is not a universal constant (BLASST reading notes,
 * papers.lqhl.me/papers/BLASST-MLSys26, "关键观察" observation 2: it is fitted
 * on calibration data), and the decisions it was fitted on depend on the
 * tiling: a tile skips a block only when all of its rows meet the test, and a
 * decode split restarts the running max.  So the table records the tiling it
 * was fitted with -- query tile (prefill), key block, and decode split count
 * (0 for prefill) -- and a call states the tiling it will run with; a table
 * fitted with another tiling is refused.
 * Errors: INVALID_ARG for a null or empty table, non-increasing targets,
 * a <= 0, L <= 0, a target outside [targets[0], targets[n-1]], a result
 * lambda >= 1, or a tiling (tile_q, block_k, num_splits) other than the
 * table's.
 */
typedef struct {
    int n;
    const double *target;
    const double *a;
    int tile_q;     /* query tile rows the table was fitted with (prefill; 0 for decode) */
    int block_k;    /* key block (64) */
    int num_splits; /* decode split count it was fitted with (0 for prefill) */
} blasst_calib_table;

blasst_status blasst_calibrate(const blasst_calib_table *table, double target_sparsity, int64_t L, int tile_q,
                               int block_k, int num_splits, double *lambda_out);

/* The calibration search at one length, host only.  gaps: host copy of a gap
 * map (entries of -inf, i.e. unvisited pairs, are ignored).  Because the
 * running max never depends on the decisions, the sparsity at lambda is the
 * fraction of gaps below ln(lambda); the returned lambda puts ln(lambda)
 * halfway between the k-th and (k+1)-th smallest gap, k = ceil(target * N).
 * *reached_out (optional) gets the sparsity that lambda gives on these gaps;
 * when the target needs lambda >= 1 the largest lambda below 1 is returned and
 * *reached_out says what it reaches.  INVALID_ARG for null pointers, n < 1,
 * no visited pair, or a target outside [0, 1]. */
blasst_status blasst_calibrate_search(const float *gaps, int64_t n, double target,
                                      double *lambda_out, double *reached_out);

/* Fit of the law lambda = a / L over n lengths: ln a = mean(ln(lambda_i * L_i)).
 * INVALID_ARG for null pointers, n < 1, lambda_i outside (0, 1) or L_i <= 0. */
blasst_status blasst_calibrate_fit(const double *lambda_at_L, const int64_t *L, int n, double *a_out);

/* ------------------------------------------------------------------ helpers */
const char *blasst_status_str(blasst_status s); /* static string, never NULL */
const char *blasst_last_error(void);            /* message of this thread's last failed call */
int blasst_abi_version(void);                   /* BLASST_ABI_VERSION */

#ifdef __cplusplus
}
#endif

#endif /* BLASST_H */
