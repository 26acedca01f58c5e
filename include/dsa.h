/*
 * libdsa: the decode step of a DSA sparse-attention layer on one MI355X (gfx950).
 *
 * One step through one layer does three things (ds4 glm53-m3ultra branch post,
 * 2026-09-09 "rising" page, paragraph on very long context):
 *   1. a lightweight indexer scores every cached position of the row;
 *   2. the k best positions (about 2,048) are selected, always the same positions
 *      in the same order;
 *   3. attention runs over only the selected positions.
 * The pages fix the behaviour, not the arithmetic. The arithmetic implemented here
 * (the plainest reading, stated once for every entry point below):
 *   score[b][s] = sum_h iw[b][h] * max(0, sum_d iq[b][h][d] * ik[s][d])     (int32, exact)
 *   order       = score descending, ties to the lower position
 *   out[b][h][:] = sum_i softmax_i(scale * q[b][h][:] . kv[i][:]) * kv[i][0:Dv]
 * with one shared latent row per position serving as key (all Dk values: latent +
 * rope) and as value (its first Dv values): the MQA fold of the
 * GLM-5.3-Flash-Alis-MLX-4bit model card (Speed section) and the latent (absorbed
 * MLA) KV cache of the glm53-tensorfold-spark README (introduction).
 *
 * Conventions shared by every call:
 *  - All array arguments are DEVICE pointers to caller-owned, contiguous, row-major
 *    memory, except ctx_len, which is a HOST array of B int32 values read during
 *    the call (its values are passed to the kernels by value, so a captured HIP
 *    graph keeps them).
 *  - Calls are asynchronous on `stream` (0 = the null stream): no host
 *    synchronisation, no readback, no device allocation. The caller must keep the
 *    buffers alive until the stream has executed the work.
 *  - Arguments are validated on the host before anything is enqueued; a rejected
 *    call enqueues nothing and returns an error code. Nothing aborts and no C++
 *    exception crosses this interface.
 *  - Row validity comes from ctx_len[b] alone: positions ctx_len[b] .. N-1 of row b
 *    are never read as scores, never selected and never attended (model card,
 *    "What changed" list, FIXED item on left-padded batches).
 *  - Indexer scores are exact when every true score lies in int32 (it does when
 *    sum_h |iw[b][h]| * sum_d |iq[b][h][d]| * 128 < 2^31); otherwise they wrap.
 *  - Results are run-to-run bit-identical: no floating-point atomics anywhere.
 *  - Different calls may run concurrently on different streams when they use
 *    different workspaces; a workspace serves one call at a time.
 */
#ifndef LIBDSA_DSA_H
#define LIBDSA_DSA_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum dsa_status {
  DSA_OK = 0,
  DSA_ERR_INVALID_ARG = 1, /* a shape, pointer, k or ctx_len value is out of range */
  DSA_ERR_UNSUPPORTED = 2, /* valid, but outside the shapes the kernels are built for */
  DSA_ERR_WORKSPACE = 3,   /* workspace missing, misaligned or smaller than dsa_workspace_size() */
  DSA_ERR_HIP = 4          /* the HIP runtime refused a launch or a copy */
} dsa_status;

typedef enum dsa_dtype {
  DSA_F32 = 0,      /* q and kv hold float32 */
  DSA_BF16 = 1,     /* q and kv hold bfloat16 */
  DSA_FP8_E4M3 = 2  /* q holds bfloat16; kv holds FP8 E4M3 ("e4m3fn": 1 sign, 4 exponent bits
                       with bias 7, 3 mantissa bits, no infinities, 0x7F/0xFF NaN), one byte
                       per value, no scale: the FP8 KV storage of the glm53-tensorfold-spark
                       README (introduction, patch list); a per-tensor dequantisation scale
                       folds into `scale` for K and into the output for V. Matrix-core
                       path only: Dk a multiple of 32 up to 1024, Dv a multiple of 16 up to
                       512, Hq <= 64 (else DSA_ERR_UNSUPPORTED) */
} dsa_dtype;

/* Limits checked by the validators. */
#define DSA_MAX_BATCH 16
#define DSA_MAX_K 4096
#define DSA_MAX_INDEX_HEADS 64   /* Hi */
#define DSA_MAX_INDEX_DIM 256    /* Di, a multiple of 16 (larger: DSA_ERR_UNSUPPORTED) */
#define DSA_MAX_ATTN_HEADS 64    /* Hq */
#define DSA_MAX_ATTN_DIM 1024    /* Dk */
#define DSA_PAGE_SIZE 256        /* positions per page of a paged cache pool */
#define DSA_MAX_PAGES 8192       /* page-table entries of one paged call (N <= 2,097,152) */

/* flags for dsa_topk_select / dsa_decode_step */
#define DSA_FLAG_FORCE_FALLBACK 1u /* testing: take the exhaustive path for every row */
#define DSA_FLAG_TABLE_IN_MEMORY 2u /* dsa_decode_step_paged, testing: the selection kernel reads
                                       the page table from memory, as it does when the table
                                       does not fit in its LDS */

/* Per-row record of what the selection did, kept in the workspace. */
typedef struct dsa_row_stats {
  int32_t path;        /* 0 = candidate path, 1 = exhaustive fallback */
  int32_t reason;      /* 0 = none, 1 = forced by flag, 2 = per-chunk candidates did not
                          provably contain the top k (threshold ties), 3 = chunks too long
                          for the candidate pass */
  int32_t selected;    /* min(k, ctx_len[b]) */
  int32_t kth_score;   /* score of the last selected position */
  int32_t candidates;  /* valid candidate keys examined on the candidate path */
  int32_t tied_at_kth; /* selected positions whose score equals kth_score */
  int32_t bad_indices; /* dsa_sparse_attn: idx entries outside [0, N) other than -1 (skipped) */
  int32_t reserved;
} dsa_row_stats;

/*
 * Human-readable name and meaning of a status code (static storage; never NULL;
 * unknown codes give a string naming them unknown). Every call reports a rejected
 * argument as a code, never as a failure of the engine: the error discipline of the
 * glm53-tensorfold-spark README ("What's new (W19)": malformed requests get a
 * clean client error instead of an engine error; "What's new (2026-09-30)": patch
 * 0490's OpenAI-style errors).
 */
const char* dsa_status_string(dsa_status status);

/*
 * The selection's working memory is sized once, up front, and reused by every call:
 * the pre-grown selection scratch the glm53-tensorfold-spark README adopts in
 * "What's new (W19)" (patch 0550, one pre-grown buffer instead of growth during
 * the run).
 *
 * Bytes of device workspace that dsa_topk_select, dsa_sparse_attn and
 * dsa_decode_step need for these sizes (B rows, N cached positions, k selected,
 * Hq attention heads, Dv output values per head). The caller allocates it (any
 * device allocation aligned to 256 bytes), need not clear it, and owns it; the
 * library never allocates or frees device memory. Returns 0 for sizes the
 * validators would reject.
 */
size_t dsa_workspace_size(int B, int64_t N, int k, int Hq, int Dv);

/*
 * Stage 1, the indexer (the "lightweight indexer" that scores every cached
 * position: rising post, long-context paragraph; the fused indexer-score kernel
 * of the MLX model card's cluster notes).
 *   iq      [B][Hi][Di] int8   indexer query heads of each row
 *   iw      [B][Hi]     int8   per-head weights of each row
 *   ik      [N][Di]     int8   indexer key cache, one shared key per position
 *   ctx_len host [B]           1 <= ctx_len[b] <= N
 *   scores  [B][N]      int32  out: scores[b][s] for s < ctx_len[b]; the rest of
 *                              the row is left untouched
 * Limits: 1 <= B <= 16, N < 2^31, Di a multiple of 16 (else DSA_ERR_INVALID_ARG);
 * Hi <= 64 and Di <= 256 are what the kernels are built for (beyond them:
 * DSA_ERR_UNSUPPORTED).
 */
dsa_status dsa_index_scores(const int8_t* iq, const int8_t* iw, const int8_t* ik,
                            const int32_t* ctx_len, int B, int Hi, int Di, int64_t N,
                            int32_t* scores, hipStream_t stream);

/*
 * Stage 2, exact top-k with a fixed order (rising post, long-context paragraph:
 * scans that narrow the candidates before a small sort, the original algorithm
 * for ambiguous cases, the same positions in the same order).
 *   scores  [B][N] int32   as written by dsa_index_scores (only s < ctx_len[b] is read)
 *   ctx_len host [B]
 *   idx     [B][k] int32   out: the first min(k, ctx_len[b]) positions of row b in
 *                          (score descending, position ascending) order, then -1
 *   ws, ws_bytes           workspace of at least dsa_workspace_size(B, N, k, 1, 1) bytes
 *   flags                  0 or DSA_FLAG_FORCE_FALLBACK
 * Limits: 1 <= k <= 4096; the rest as above.
 */
dsa_status dsa_topk_select(const int32_t* scores, const int32_t* ctx_len, int B, int64_t N,
                           int k, int32_t* idx, void* ws, size_t ws_bytes, unsigned flags,
                           hipStream_t stream);

/*
 * Stage 3, attention over the selected positions only (rising post, long-context
 * paragraph; MQA fold of the MLX model card; latent KV cache of the TensorFold
 * README).
 *   q    [B][Hq][Dk]  dt       query heads of each row (bfloat16 for DSA_FP8_E4M3)
 *   kv   [N][Dk]      dt       latent cache: row i = [Dv latent values | Dk-Dv rope values];
 *                              K is the whole row, V its first Dv values (one byte per
 *                              value for DSA_FP8_E4M3, 16-byte aligned rows: Dk % 16 == 0)
 *   idx  [B][k]       int32    positions to attend; -1 entries are skipped, and so are
 *                              (with a count in the row's stats) entries outside [0, N)
 *   out  [B][Hq][Dv]  float32  out: softmax(scale * q.K) @ V over the valid entries;
 *                              a row with no valid entry gets zeros
 *   ws, ws_bytes               at least dsa_workspace_size(B, N, k, Hq, Dv) bytes
 * Limits: 1 <= Hq <= 64, Dv <= Dk <= 1024, Dk and Dv multiples of 32 (bf16, fp8) or
 * of 4 (f32, Dk <= 256).
 */
dsa_status dsa_sparse_attn(const void* q, const void* kv, const int32_t* idx, int B, int Hq,
                           int Dk, int Dv, int64_t N, int k, float scale, dsa_dtype dt,
                           float* out, void* ws, size_t ws_bytes, hipStream_t stream);

/*
 * The whole step through one layer: stage 1, then 2, then 3, in three kernel
 * launches on `stream`. Arguments as for the three calls above; scores and idx
 * are written as those calls write them, out as dsa_sparse_attn writes it.
 * Workspace: dsa_workspace_size(B, N, k, Hq, Dv) bytes.
 */
dsa_status dsa_decode_step(const int8_t* iq, const int8_t* iw, const int8_t* ik, const void* q,
                           const void* kv, const int32_t* ctx_len, int B, int Hi, int Di, int Hq,
                           int Dk, int Dv, int64_t N, int k, float scale, dsa_dtype dt,
                           int32_t* scores, int32_t* idx, float* out, void* ws,
                           size_t ws_bytes, unsigned flags, hipStream_t stream);

/*
 * dsa_decode_step with per-kernel timing: when kernel_events is not NULL it must
 * point to 6 events created on the current device. Events 2i and 2i+1 receive
 * the start and end timestamps of stage i's kernel dispatch (i = 0: indexer
 * scores with per-chunk candidates; 1: selection and attention splits, one
 * launch; 2: combine of the splits), so hipEventElapsedTime(e[2i], e[2i+1]) is
 * that kernel's own duration without queueing or launch gaps. When the indexer
 * stage needs several launches (many query rows), the pair spans all of them.
 * Everything else is as for dsa_decode_step, which is this call with
 * kernel_events = NULL. Returns DSA_ERR_INVALID_ARG if any of the 6 is NULL.
 */
dsa_status dsa_decode_step_timed(const int8_t* iq, const int8_t* iw, const int8_t* ik,
                                 const void* q, const void* kv, const int32_t* ctx_len, int B,
                                 int Hi, int Di, int Hq, int Dk, int Dv, int64_t N, int k,
                                 float scale, dsa_dtype dt, int32_t* scores, int32_t* idx,
                                 float* out, void* ws, size_t ws_bytes, unsigned flags,
                                 hipStream_t stream, hipEvent_t* kernel_events);

/*
 * dsa_decode_step for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid allocation): the same
 * step with no workspace argument. Its workspace is a static device array of
 * DSA_NOALLOC_SCRATCH_BYTES per device, part of the library's code object and held
 * until the process ends; its address is looked up once per device (the first call
 * on it). Nothing is allocated or freed, here or later.
 *  - Sizes whose dsa_workspace_size exceeds DSA_NOALLOC_SCRATCH_BYTES return
 *    DSA_ERR_WORKSPACE (B=1, k=2048, Hq=16, Dv=512 needs about 2.2 MB; B=16 about
 *    34 MB); other arguments are checked as for dsa_decode_step.
 *  - Every call on a device shares that device's scratch, and the scratch keeps the
 *    last call's contents: calls that overlap on one device (other streams, other
 *    host threads) race and must be ordered by the caller. dsa_read_stats cannot
 *    read these calls' statistics.
 *  - DSA_ERR_HIP if the scratch address cannot be resolved on the current device.
 */
#define DSA_NOALLOC_SCRATCH_BYTES (64u << 20)
dsa_status dsa_decode_step_noalloc(const int8_t* iq, const int8_t* iw, const int8_t* ik, const void* q,
                                   const void* kv, const int32_t* ctx_len, int B, int Hi, int Di, int Hq,
                                   int Dk, int Dv, int64_t N, int k, float scale, dsa_dtype dt,
                                   int32_t* scores, int32_t* idx, float* out, unsigned flags,
                                   hipStream_t stream);

/*
 * Paged caches: the three stages over a pool of fixed-size pages shared by many
 * sequences, read through one sequence's page table (the glm53-tensorfold-spark
 * README: a 1,048,576-token KV pool held in 4,096 pages, in the introduction and the
 * "What's new (2026-09-30)" note on 1M-context fixes; 1,048,576 / 4,096 gives
 * DSA_PAGE_SIZE = 256 positions a page). Logical position s of the sequence lives
 * in pool row page_table[s / 256] * 256 + s % 256 of both pools, so one table serves
 * the indexer keys and the latent rows. The results are those of the contiguous
 * calls on the caches the table describes (ik[s] = ik_pool[that row], and the same
 * for kv), bit for bit: scores and idx hold logical positions.
 *   ik_pool    [pool_pages * 256][Di]  int8   indexer key pool
 *   kv_pool    [pool_pages * 256][Dk]  dt     latent pool (layout of kv above)
 *   page_table [ceil(N / 256)]         int32  DEVICE array: pool page of each logical
 *                                             page of the sequence, shared by its B
 *                                             rows (ctx_len[b] <= N as before)
 *   pool_pages                                pages in each pool (>= 1)
 * Entries outside [0, pool_pages) are clamped into the pool (no read leaves it; the
 * results for those pages are unspecified). Limits, beyond those of the contiguous
 * calls: N <= DSA_MAX_PAGES * 256, pool_pages * 256 <= INT32_MAX, and
 * pool_pages * 256 * Di < 2^31 for calls that read ik_pool (else
 * DSA_ERR_UNSUPPORTED); page_table NULL or misaligned, or pool_pages < 1, give
 * DSA_ERR_INVALID_ARG. Workspace sizes are those of the contiguous calls.
 */
dsa_status dsa_index_scores_paged(const int8_t* iq, const int8_t* iw, const int8_t* ik_pool,
                                  const int32_t* page_table, int64_t pool_pages, const int32_t* ctx_len,
                                  int B, int Hi, int Di, int64_t N, int32_t* scores, hipStream_t stream);

dsa_status dsa_sparse_attn_paged(const void* q, const void* kv_pool, const int32_t* page_table,
                                 int64_t pool_pages, const int32_t* idx, int B, int Hq, int Dk, int Dv,
                                 int64_t N, int k, float scale, dsa_dtype dt, float* out, void* ws,
                                 size_t ws_bytes, hipStream_t stream);

/* kernel_events: NULL, or 6 events as for dsa_decode_step_timed. */
dsa_status dsa_decode_step_paged(const int8_t* iq, const int8_t* iw, const int8_t* ik_pool, const void* q,
                                 const void* kv_pool, const int32_t* page_table, int64_t pool_pages,
                                 const int32_t* ctx_len, int B, int Hi, int Di, int Hq, int Dk, int Dv,
                                 int64_t N, int k, float scale, dsa_dtype dt, int32_t* scores, int32_t* idx,
                                 float* out, void* ws, size_t ws_bytes, unsigned flags, hipStream_t stream,
                                 hipEvent_t* kernel_events);

/*
 * Copies the per-row stats of the last call that used `ws` into stats[0..B): which
 * selection path each row took and why (the rising post's long-context paragraph:
 * the narrowing scans handle the common case and the original algorithm the
 * ambiguous ones), with the threshold score and its ties. Arguments: ws as passed
 * to that call, ws_bytes its size (at least the stats region), B <= 16 rows,
 * stats a HOST array of B records. DSA_ERR_INVALID_ARG for a null pointer or B out
 * of range, DSA_ERR_WORKSPACE when ws_bytes cannot hold B records, DSA_ERR_HIP if
 * the copy fails. Synchronises `stream` (call it outside timed regions).
 */
dsa_status dsa_read_stats(const void* ws, size_t ws_bytes, int B, dsa_row_stats* stats,
                          hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* LIBDSA_DSA_H */
