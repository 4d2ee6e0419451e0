/*
 * idx.h — C ABI of the MI355X (gfx950) DSA lightning-indexer top-k library (libidx.so).
 *
 * The operation (LiteTopK prefill indexer page, sgl-project/sglang#47469, introduction
 * and section 1; ROCm DSA indexer top-k page, sgl-project/sglang#37591):
 *
 *   For every query row r and every key s the row can see (ks[r] <= s < ke[r]):
 *       score[r, s] = kscale[s] * sum_h w[r, h] * max(q[r, h] . k[s], 0)
 *   (MQA: one key vector per position shared by all heads), then return the exact
 *   top-k keys of the row: fp32 value descending, -0.0 == +0.0, ties to the lower key
 *   index.  Indices are relative to ks[r]; rows that see fewer than k keys return all
 *   of them followed by -1.  The order of the indices inside a row is unspecified.
 *
 * Conventions for every entry point:
 *   - Pointers are DEVICE pointers unless marked (host).  The library never frees,
 *     keeps or allocates device memory: the caller owns every buffer, including the
 *     workspace, whose size comes from the matching *_workspace query.
 *   - Alignment (error IDX_EALIGN): q and k 16 bytes (they are read as 16-byte vectors),
 *     workspaces 256 bytes, every other device pointer its element size.
 *   - `stream` is a hipStream_t (NULL = the legacy default stream).  All work is
 *     enqueued on it, asynchronously; the call returns before the GPU finishes unless
 *     stated otherwise.  The device used is the current HIP device of the calling thread.
 *   - Return value: IDX_OK (0) or a negative error code; idx_strerror() gives text.
 *     Argument errors are detected on the host before anything is enqueued, so a
 *     failed call leaves outputs untouched.  The boundary never throws or aborts.
 *   - Sizes: rows up to 2^31-1, keys per row up to 2^31-1, pitches and offsets int64.
 */
#ifndef IDX_H_
#define IDX_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ------------------------------------------------------------------ error codes */
#define IDX_OK 0
#define IDX_EINVAL (-1) /* null pointer, bad size, k out of range, heads/head_dim unsupported */
#define IDX_EFMT (-2)   /* format and pointers disagree (e.g. MXFP4 without block scales) */
#define IDX_EALIGN (-3) /* a device pointer is misaligned (see Alignment above) */
#define IDX_EWS (-4)    /* workspace smaller than the *_workspace query returned */
#define IDX_EHIP (-5)   /* a HIP runtime call or kernel launch failed */
#define IDX_ENODEV (-6) /* no usable gfx950 device is current */
#define IDX_ESCRATCH (-7) /* the problem needs more workspace than the library's fixed scratch
                             (idx_fused_topk_noalloc) */

/* ------------------------------------------------------------------ limits */
#define IDX_HEAD_DIM 128  /* head_dim of q and k */
#define IDX_MAX_TOPK 2048 /* largest k (the DSA indexers keep 512..2048 keys) */
#define IDX_PAGE 64       /* tokens per page of a paged K cache */

/* Operand format, shared by q and k. */
typedef enum idx_fmt {
  IDX_FMT_E4M3 = 1,  /* OCP FP8 E4M3FN, one byte per element */
  IDX_FMT_MXFP4 = 2  /* OCP MXFP4: e2m1 codes, two per byte (element 2i in the low
                        nibble), plus one e8m0 scale per 32 consecutive head_dim
                        elements (4 per head or key) */
} idx_fmt;

/* Test hooks that force the rare paths of idx_fused_topk from the host (NULL in
 * production).  None of them changes the result, only the route to it. */
typedef struct idx_debug {
  int32_t cap;            /* > 0: candidate-slab capacity per row instead of 4*k */
  int32_t threshold_mode; /* 0 sampled; 1 = +inf (no candidates: every sampled row
                             underflows and falls back); 2 = -inf (every visible key is a
                             candidate: rows with more than cap keys overflow) */
  int32_t threshold_row_mod; /* > 0: apply threshold_mode only to rows r with
                                r % threshold_row_mod == 0 */
  int32_t tie_cap;        /* 1..4096: tie-buffer capacity of the slab select and the exact
                             fallback (0 = 4096, the ROCm top-k page's kTieCap); a
                             boundary bin with more elements is resolved by rescanning
                             the row instead of refining it in LDS */
} idx_debug;

/* One indexer problem.  Layouts are row-major and densely packed.
 *   q        E4M3: u8 [rows][heads][128];  MXFP4: u8 [rows][heads][64]
 *   q_sf     MXFP4 only: e8m0 u8 [rows][heads][4]; must be NULL for E4M3
 *   k        contiguous: E4M3 u8 [num_keys][128] / MXFP4 u8 [num_keys][64]
 *            paged (E4M3 only): u8 [num_keys/64][64][128] (num_keys = pages * 64)
 *   k_sf     MXFP4 only: e8m0 u8 [num_keys][4]; must be NULL for E4M3
 *   k_scale  optional fp32 [num_keys] (per key, or per physical slot when paged),
 *            > 0; NULL means 1.0.  Multiplies the score (equivalently the key).
 *   w        bf16 bits [rows][heads], >= 0
 *   ks, ke   int32 [rows]: row r sees logical keys [ks[r], ke[r]), 0 <= ks <= ke.
 *            Contiguous: ke <= num_keys.  Paged: ke <= max_pages * 64.
 *   page_table  NULL = contiguous K.  Else int32 [num_req][max_pages]: logical key s of
 *            request q lives in physical slot page_table[q][s / 64] * 64 + s % 64
 *            (LiteTopK page, section 3).  Entries past a request's last visible page are
 *            never read.
 *   row_req  paged only: int32 [rows], request of each row, in [0, num_req).
 *   num_keys must be > 0 when rows > 0 (IDX_EINVAL otherwise).
 *   Values the library cannot check on the host (ranges inside device arrays, NaN
 *   codes, page ids) must be valid; invalid ones give undefined results, but key reads
 *   stay inside k and the page table (out-of-range keys and slots are clamped), a range
 *   with ke < ks counts as empty, and writes stay inside the outputs: out_idx[rows][k]
 *   of the top-k entry points, out[rows][ld] of idx_score (a row's scores past ld are
 *   not written).
 */
typedef struct idx_problem {
  int32_t rows;
  int32_t heads;    /* 32 or 64 */
  int32_t head_dim; /* must be IDX_HEAD_DIM */
  int32_t fmt;      /* idx_fmt */
  const void* q;
  const uint8_t* q_sf;
  const void* k;
  const uint8_t* k_sf;
  const float* k_scale;
  const uint16_t* w;
  const int32_t* ks;
  const int32_t* ke;
  int64_t num_keys;
  const int32_t* page_table;
  const int32_t* row_req;
  int32_t num_req;
  int32_t max_pages;
  const idx_debug* debug; /* (host) NULL in production */
} idx_problem;

/* Route taken by idx_fused_topk (host struct, filled when a pointer is passed). */
typedef struct idx_stats {
  int32_t rows;            /* rows of the problem */
  int32_t rows_store_all;  /* rows that see <= cap keys: every key is a candidate */
  int32_t rows_sampled;    /* rows filtered by a sampled threshold */
  int32_t fallback_rows;   /* rows re-scored and selected over the whole row because the
                              slab under- or overflowed */
  int32_t max_count;       /* largest candidate count of a row (may exceed cap) */
  int32_t min_count;       /* smallest candidate count among sampled rows */
  int64_t total_count;     /* sum of candidate counts */
  int32_t cap;             /* slab capacity per row */
  int32_t sample_stride;   /* odd sample stride S */
  int32_t sample_keys;     /* sample slots per row (one every S keys) */
  int32_t reserved;
} idx_stats;

/* ------------------------------------------------------------------ scoring
 * idx_score — materialised scores (the role of DeepGEMM mqa_logits, LiteTopK page,
 * introduction).  Writes out[r * ld + (s - ks[r])] (fp32) for every visible key s of
 * row r and nothing else.  ld >= max over rows of (ke - ks); out: fp32 [rows][ld].
 *   ws   workspace of idx_score_workspace(p) bytes (may be NULL when that is 0: e4m3);
 *        for MXFP4 it holds per-row constants the scoring kernels derive from q and w.
 * Scores are bitwise identical to those idx_fused_topk selects from (same scoring
 * core; LiteTopK page, section 1: only the epilogue differs), and never negative (-0.0
 * is stored as +0.0).
 * Numerics.  Head dots come from the gfx950 scaled MFMAs with fp32 results.  The fp8
 * (e4m3) MFMA drops products that lie far below the largest product of their group of 8
 * head_dim elements, so an e4m3 head dot can differ from the exact one by about 2^-12 of
 * that group's largest |q_d k_d| per group; e2m1 products are exact.  e4m3: score =
 * kscale * sum_h w_h max(x_h, 0) in fp32 (a key whose every head dot is negative scores
 * exactly 0).  MXFP4: the sum is evaluated as (sum_h w_h |x_h| + u . k) / 2 with
 * u = sum_h w_h q_h on the matrix cores; its rounding error is bounded relative to the
 * score's magnitude B = kscale * sum_h w_h sum_d |q_hd k_d|, not to the score, so a key
 * whose exact score is 0 can score a small positive value instead (and does not then
 * tie with other zeros by index).  On the workloads' inputs (N(0,1)-scale values, w of
 * order 1/H) every score is within 1e-4 + 1e-5 |exact| of the exact score.          */
int idx_score(const idx_problem* p, float* out, int64_t ld, void* ws, size_t ws_bytes, void* stream);

/* Bytes of workspace idx_score needs for this problem (host only; scalar fields only).
 * Returns 0 when none is needed or the arguments are invalid.                       */
size_t idx_score_workspace(const idx_problem* p);

/* ------------------------------------------------------------------ selection
 * idx_select — exact top-k over materialised fp32 rows (ROCm DSA indexer top-k page:
 * fp32 radix histogram, exact tie refinement, full-row rescan when the tie buffer
 * overflows, rows split over several workgroups at low batch).
 *   scores   fp32 [rows][ld]; row r's candidates are scores[r*ld + row_start[r] + j],
 *            0 <= j < len[r]  (row_start may be NULL = 0; row_start + len <= ld)
 *   len      int32 [rows], 0 <= len <= ld
 *   k        1 .. IDX_MAX_TOPK
 *   out_idx  int32 [rows][k]: the selected j (relative to row_start), -1 padded
 *   ws       workspace of idx_select_workspace(rows, ld, k) bytes (may be NULL when
 *            that is 0).  The row split keeps one counter per row in it and every call
 *            leaves those at 0; on a workspace whose contents are not yet the library's
 *            (say a fresh allocation) a split row may take the multi-pass route once, with
 *            the same result.  Calls that share a workspace must not overlap.
 * NaN scores give undefined results.  Device-side row_start and len outside those bounds
 * are clamped into the row ([0, ld)), so reads stay inside scores[rows][ld] and writes
 * inside out_idx[rows][k].                                                            */
int idx_select(const float* scores, int64_t ld, const int32_t* row_start, const int32_t* len,
               int32_t rows, int32_t k, int32_t* out_idx, void* ws, size_t ws_bytes,
               void* stream);

/* Same as idx_select with the number of workgroups per row forced: split = 0 one
 * workgroup per row, split >= 2 that many (at most 32).  The result is identical. */
int idx_select_split(const float* scores, int64_t ld, const int32_t* row_start,
                     const int32_t* len, int32_t rows, int32_t k, int32_t* out_idx, void* ws,
                     size_t ws_bytes, int32_t split, void* stream);

/* Workgroups per row idx_select uses for `rows` rows of pitch `row_len` on a device
 * with `cu_count` compute units: g = min(cu_count / rows, 32), or 0 (one workgroup per
 * row) when g < 4 or row_len < 65536 (ROCm top-k page, row_split).  Host only.     */
int32_t idx_row_split(int32_t rows, int64_t row_len, int32_t cu_count);

/* Bytes of workspace idx_select / idx_select_split need (the larger of both routes). */
size_t idx_select_workspace(int32_t rows, int64_t ld, int32_t k);

/* ------------------------------------------------------------------ fused top-k
 * idx_fused_topk — the no-logits path (LiteTopK page, "sampled threshold", sections
 * 1-2; exactness as in the ROCm top-k page).  Per row: a threshold T_r from an
 * odd-stride single-key sample of the row's own scores; one pass scores every visible
 * key and appends only (score, key) with score >= T_r to a per-row candidate slab with
 * a count (rows that see <= cap keys keep every key); an exact radix select over the
 * slab; rows whose slab under- or overflowed are re-scored and selected exactly.  The
 * result equals idx_select over idx_score's output, bit for bit.
 *   out_idx  int32 [rows][k], indices relative to ks[r], -1 padded
 *   ws       workspace of idx_fused_workspace(p, k) bytes
 *   stats    (host) optional; when non-NULL the call waits for the stream and fills it.
 */
int idx_fused_topk(const idx_problem* p, int32_t k, int32_t* out_idx, void* ws, size_t ws_bytes,
                   idx_stats* stats, void* stream);

/* Bytes of workspace idx_fused_topk needs for this problem shape and k (host only;
 * reads only the scalar fields of p).  Returns 0 for invalid arguments.            */
size_t idx_fused_workspace(const idx_problem* p, int32_t k);

/* idx_fused_topk_noalloc — idx_fused_topk for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid hipMalloc):
 * the workspace is a fixed device array inside the library, IDX_NOALLOC_SCRATCH_BYTES per
 * GPU it runs on, held until the process ends.  The caller still passes the inputs and
 * out_idx.  The call itself allocates nothing (its first call on a device resolves that
 * device's copy of the array).  Problems whose idx_fused_workspace(p, k) exceeds the
 * array return IDX_ESCRATCH (the decode/MTP batch of 512 rows over 256K-token contexts at
 * k = 2048 needs about 72 MiB; 4096 prefill rows of 64K keys need about 282 MiB and do
 * not fit).  All calls on one GPU share its array: calls that overlap on one GPU (other
 * streams or threads) race and must be serialised by the caller.  It reports no
 * statistics (no host read-back); the result is identical to idx_fused_topk's.      */
#define IDX_NOALLOC_SCRATCH_BYTES (128u << 20)
int idx_fused_topk_noalloc(const idx_problem* p, int32_t k, int32_t* out_idx, void* stream);

/* ------------------------------------------------------------------ paged output
 * idx_page_slots — selected logical positions to physical KV slots for a paged cache
 * (LiteTopK page, section 3, topk_page_table_transform: a position pos >= 0 of request q
 * becomes page_table[q][pos / 64] * 64 + pos % 64, and -1 passes through).
 *   idx        int32 [rows][k]: indices relative to ks[r] (as idx_fused_topk and
 *              idx_select return them), -1 for empty entries
 *   ks         int32 [rows] first visible key of each row, or NULL for 0
 *   page_table int32 [num_req][max_pages]; row_req int32 [rows] (as in idx_problem)
 *   out        int32 [rows][k]; may equal idx (in place)
 * For idx >= 0 the logical position is pos = ks[r] + idx; a pos whose page lies past
 * max_pages yields -1 (no read outside the table).  Page entries the positions name must
 * be valid.  One flat 1-D grid over rows * k; four entries per thread when k % 4 == 0
 * and idx, out are 16-byte aligned.  Errors: IDX_EINVAL (null pointer with rows > 0,
 * rows < 0, k < 1, max_pages < 1), IDX_EALIGN (idx or out not 4-byte aligned).       */
int idx_page_slots(const int32_t* idx, int32_t rows, int32_t k, const int32_t* ks, const int32_t* page_table,
                   const int32_t* row_req, int32_t max_pages, int32_t* out, void* stream);

/* ------------------------------------------------------------------ consumer
 * idx_sparse_attn — attention of each query row over only the KV slots its indexer
 * selected (QSA sparse paged attention page, vllm-project/vllm#66512: about 2048 tokens
 * per row chosen by the indexer; slots are physical, as idx_page_slots returns them;
 * QK in bf16 and PV in fp16 with the e4m3 cache values converted exactly, fp32
 * accumulation):
 *     s_j      = softmax_scale * q[r, h] . k_cache[slot_j, g],   g = h / (hq / hkv)
 *     out[r,h] = output_scale * sum_j exp(s_j - max) v_cache[slot_j, g] / sum_j exp(s_j - max)
 * over the valid slots of row r.
 *   q        bf16 bit patterns [rows][hq][128]
 *   k_cache, v_cache  e4m3 (OCP E4M3FN) [num_slots][hkv][128]
 *   slots    int32 [rows][width]; an entry outside [0, num_slots) (such as the -1 of a
 *            short selection) takes no part; a row with no valid entry gives zeros
 *   out      fp32 [rows][hq][128]
 * The softmax weights enter the PV product rounded to fp16 (relative error <= 2^-11 per
 * weight).  One workgroup per (row, KV head); no workspace.  Errors: IDX_EINVAL (rows < 0,
 * width < 0, hkv < 1, hq not a multiple of hkv, hq / hkv > 32, num_slots < 1, rows * hkv
 * >= 2^31, a non-finite scale, a null pointer with rows > 0), IDX_EALIGN (q, k_cache,
 * v_cache not 16-byte aligned; out or slots not 4-byte aligned).                     */
int idx_sparse_attn(const uint16_t* q, const uint8_t* k_cache, const uint8_t* v_cache, int64_t num_slots,
                    const int32_t* slots, int32_t rows, int32_t hq, int32_t hkv, int32_t width, float softmax_scale,
                    float output_scale, float* out, void* stream);

/* ------------------------------------------------------------------ measurement
 * Stage timing of idx_fused_topk for benchmarks.  While enabled, every idx_fused_topk
 * call (any thread) records six HIP events on its own stream at its stage boundaries,
 * without synchronising; the records of up to max_calls calls are kept (later calls are
 * not timed).  idx_timing_read waits for the recorded events and writes, per timed call,
 * the milliseconds of the five stages in order — threshold samples, thresholds, fused
 * score + filter, slab select, fallback — to ms (host, [calls][5]); it returns the number
 * of calls written (<= max_calls) or a negative error code, and starts a new record.
 * idx_timing_disable stops recording and releases the events.                       */
int idx_timing_enable(int32_t max_calls);
int idx_timing_read(float* ms, int32_t max_calls);
int idx_timing_disable(void);

/* ------------------------------------------------------------------ misc */
const char* idx_strerror(int code);
/* Library version as MAJOR*10000 + MINOR*100 + PATCH. */
int32_t idx_version(void);

#ifdef __cplusplus
}
#endif
#endif /* IDX_H_ */
