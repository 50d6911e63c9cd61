/*
 * csa.h -- C ABI of the compressed sparse attention (CSA / HCA) step for gfx950.
 *
 * Sources (web pages; cited by title and section):
 *   [P1] "Token 的一生：DSV4 架构与 DSpark" (security.zone.ci):
 *        §1 (DSA -> DSV4 pipeline), §2.1 (C4 compressor), §2.2 (C4 KV cache
 *        size, PagedIndexerMetadata), §3.1 (FP8/FP4 indexer query),
 *        §3.2 (top-512 transform), §4 (Hadamard rotation).
 *   [P2] "DeepSeek-V4 的交錯壓縮注意力（CSA/HCA）：將百萬標記長上下文變為可用資源"
 *        (agents-report.net): section "架構突破" (CSA and HCA paragraphs) and
 *        section "低精度與儲存策略的配合" (FP8 KV, BF16 RoPE dims, FP4 indexer).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - Every pointer argument is DEVICE memory owned by the caller, unless the
 *    argument's comment says otherwise. The library never allocates, frees or
 *    synchronises; it only enqueues kernels on the given stream and returns.
 *    (indexer_topk512_noalloc alone uses a fixed array of the library's own,
 *    in device memory, instead of a caller's workspace; see there.)
 *  - All shape / format / null checks run on the host before any launch. On a
 *    failed check the call returns CSA_ERR_INVALID (or CSA_ERR_UNSUPPORTED for a
 *    well-formed but unimplemented combination) and touches no buffer.
 *    A launch error reported by the runtime returns CSA_ERR_HIP.
 *  - Device-resident integers (page tables, lengths, positions, indices) are
 *    int32; -1 marks an empty selection slot. Values read from device memory
 *    cannot be checked on the host: a page id outside [0, num_pages), a length
 *    beyond the row's capacity or a position beyond the pool is a breach of
 *    the caller's contract and its result is undefined.
 *  - Apart from that array, the library holds no mutable global state: calls on
 *    different streams are independent and every call can be captured into a
 *    HIP graph.
 *
 * KV entry (one compressed or raw token), 576 dims = 512 latent + 64 RoPE
 * ([P2] "低精度與儲存策略的配合": most KV dims in FP8, RoPE dims in BF16):
 *    CSA_FP8_E4M3 pool: latent  uint8  [num_pages][page_size][512]  OCP e4m3fn codes
 *                       scale   float  [num_pages][page_size]       one scale per entry,
 *                                                                  value = code * scale
 *                       rope    bf16   [num_pages][page_size][64]
 *    CSA_F32 pool:      latent  float  [num_pages][page_size][512]
 *                       rope    float  [num_pages][page_size][64]   (scale unused)
 *  Slot of logical entry j of sequence s:
 *      page_table[s * pt_stride + j / page_size] * page_size + j % page_size
 *  ([P1] §2.2: raw pages hold 256 tokens, a C4 page page_size/4 = 64 entries.)
 *
 * Index-K pool (one row per compressed entry, dim = indexer head dim):
 *    CSA_F32:      data float [num_pages][page_size][dim]                 (scale unused)
 *    CSA_FP8_E4M3: data uint8 [num_pages][page_size][dim], scale float [num_pages][page_size]
 *    CSA_MXFP4:    data uint8 [num_pages][page_size][dim/2]  two e2m1 codes per byte,
 *                  element 2i in the low nibble; scale uint8 [num_pages][page_size][dim/32]
 *                  e8m0 exponents (value = code * 2^(byte-127)), OCP MX v1.0.
 */
#ifndef CSA_H_
#define CSA_H_

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Fixed sizes of the method. */
#define CSA_TOPK        512   /* [P1] §3.2: top-512 compressed entries per query   */
#define CSA_TOPK_MAX    2048  /* largest k of topk_page_select (DSA-style top-k)   */
#define CSA_C4_RATIO    4     /* [P1] §2.1: 4 raw tokens -> 1 compressed entry     */
#define CSA_HCA_RATIO   128   /* [P2] HCA paragraph: about 128x compression        */
#define CSA_RAW_PAGE    256   /* [P1] §2.2: page_size = 256 raw tokens            */
#define CSA_C4_PAGE     64    /* [P1] §2.2: c4_page_size = page_size / 4          */
#define CSA_KV_DIM      576   /* latent 512 + RoPE 64                              */
#define CSA_LATENT_DIM  512
#define CSA_ROPE_DIM    64

typedef enum {
  CSA_OK = 0,
  CSA_ERR_INVALID = 1,      /* bad argument; nothing launched, nothing written  */
  CSA_ERR_UNSUPPORTED = 2,  /* valid but unimplemented format / shape combo     */
  CSA_ERR_WORKSPACE = 3,    /* workspace too small (see csa_workspace_size)     */
  CSA_ERR_HIP = 4,          /* the HIP runtime reported a launch error          */
  CSA_ERR_BOUNDS = 5        /* debug mode: a device-resident page id, length,
                               position or slot is out of range; the call's own
                               kernels were not launched (see csa_set_debug)   */
} csa_status;

typedef enum {
  CSA_F32 = 0,
  CSA_BF16 = 1,
  CSA_FP8_E4M3 = 2,  /* OCP e4m3fn: bias 7, max 448, no infinities */
  CSA_MXFP4 = 3      /* OCP MX v1.0: e2m1 elements, one e8m0 scale per 32 */
} csa_fmt;

/* Index preparation flags ([P1] §4: q and K go rope -> hadamard -> quant). */
#define CSA_PREP_HADAMARD 1u  /* v <- H_D v / sqrt(D), Sylvester order */
#define CSA_PREP_QUANT    2u  /* quantise to the index pool's format   */
#define CSA_PREP_ROPE     4u  /* rotary embedding first (see csa_rope)  */
/*
 * Rows-per-sequence hint for indexer_score / indexer_topk512 (OR-ed into
 * `prep`; n in 0..255, 0 = no hint): the query rows come in consecutive groups
 * of n that share a sequence, row_seq[t] == row_seq[n * (t / n)], as the q_len
 * query tokens of each sequence in multi-token (speculative-verify) decode.
 * Results are the same with or without it. When n has a divisor r in 2..8
 * (the largest is taken) and the pool has 64-entry pages, each index-K page is
 * read once per r rows of a group instead of once per row (a row whose
 * sequence differs from its group's first row is still scored correctly,
 * from its own pages).
 */
#define CSA_ROWS_PER_SEQ(n) ((((uint32_t)(n)) & 0xFFu) << 8)

/*
 * Rotary position embedding of indexer rows ([P1] §3.1: the fused query
 * preparation takes a cos/sin table `freqs_cis` and the token positions; §4:
 * rope -> hadamard -> quant for q and for the index-K rows). The last `dim`
 * dims of a row are rotated in adjacent pairs: pair i = (x[D-dim+2i],
 * x[D-dim+2i+1]) at position p becomes (x c - y s, x s + y c) with
 * (c, s) = (cos_sin[(p * dim/2 + i) * 2], cos_sin[(p * dim/2 + i) * 2 + 1]).
 * The caller owns the table (float32, any frequencies it chooses; e.g. the
 * textbook theta^(-2i/dim) angles) and guarantees every position used is a
 * row of it.
 *   pos           device int32: the position of each group of rows
 *   cos_sin       device float [positions][dim/2][2]
 *   dim           even, 2 <= dim <= the row dim
 *   rows_per_pos  csa_index_prep: rows r of the call use pos[r / rows_per_pos]
 *                 (1 for index-K rows, H_I for [T][H_I] query rows)
 */
typedef struct {
  const int32_t* pos;
  const float*   cos_sin;
  int32_t dim;
  int32_t rows_per_pos;
} csa_rope;

typedef struct {
  void*   latent;        /* see the KV entry layout above */
  float*  latent_scale;  /* FP8 pools only; NULL for F32 */
  void*   rope;
  int32_t fmt;           /* CSA_FP8_E4M3 or CSA_F32 */
  int32_t page_size;     /* entries per page (64 compressed, 256 raw) */
  int64_t num_pages;
} csa_kv_pool;

typedef struct {
  void*   data;
  void*   scale;         /* float [P][ps] for FP8, uint8 [P][ps][dim/32] for MXFP4, NULL for F32 */
  int32_t fmt;           /* CSA_F32, CSA_FP8_E4M3 or CSA_MXFP4 */
  int32_t dim;           /* indexer head dim: 64 or 128 (multiple of 32 for MXFP4) */
  int32_t page_size;
  int64_t num_pages;
} csa_index_pool;

/*
 * c4_compress -- softmax-gated pooling of each block of `ratio` raw KV rows into
 * one compressed entry, then quantised into a KV pool.
 * Defined by [P1] §2.1 (block k covers raw positions [4k, 4k+3] and is emitted
 * once position 4k+3 exists; output is seqlen//4 entries) and [P2] CSA paragraph
 * (softmax-gated pooling with a learned positional bias); HCA uses the same
 * form with ratio 128 ([P2] HCA paragraph).
 * For block k of sequence b with rows x_i (i = 0..ratio-1, raw position ratio*k+i):
 *     g_i = sum_d gate_w[d] * x_i[d] + gate_b[i],  a = softmax(g),  c = sum_i a_i x_i.
 * c (576 dims) is stored at logical entry k of sequence b in `out`:
 *   FP8 pool: scale = max(amax(c[0:512]), FLT_MIN) / 448, latent code = e4m3_rne(c/scale)
 *   saturated at +-448, rope = bf16_rne(c[512:576]); F32 pool: stored as is.
 * ratio == 1 stores each row unchanged apart from that quantisation (used to
 * append raw tokens to the window pool).
 *
 *  x         [cu_rows[B]][576], CSA_BF16 or CSA_F32, row-major.
 *  cu_rows   int32[B+1]: rows of sequence b are x[cu_rows[b] .. cu_rows[b+1]).
 *  start_pos int32[B]: raw position of the first row of sequence b. Every
 *            complete aligned block [ratio*k, ratio*k + ratio) inside the rows
 *            is emitted; rows of a partial block at either end are skipped.
 *  max_rows  HOST: an upper bound of cu_rows[b+1] - cu_rows[b] over b (sizes the grid).
 *  gate_w    float[576]; gate_b float[ratio].
 *  page_table int32 [B][pt_stride] over out.page_size-entry pages.
 * Returns CSA_ERR_INVALID if ratio is outside [1, 1024], B or max_rows is
 * negative, a pointer is NULL, or the pool format is not FP8 / F32.
 */
csa_status c4_compress(const void* x, csa_fmt x_fmt, const int32_t* cu_rows,
                       const int32_t* start_pos, int32_t B, int32_t max_rows, int32_t ratio,
                       const float* gate_w, const float* gate_b,
                       const int32_t* page_table, int32_t pt_stride,
                       csa_kv_pool out, hipStream_t stream);

/*
 * csa_index_prep -- rotary embedding, Hadamard rotation and quantisation of
 * indexer rows (q rows or index-K rows): [P1] §3.1 and §4 (rope -> hadamard ->
 * FP8/FP4 quant).
 *   v       [rows][dim] CSA_BF16 or CSA_F32.
 *   flags   CSA_PREP_ROPE: first rotate the last rope.dim dims of each row by
 *           its position (csa_rope), in fp32.
 *           CSA_PREP_HADAMARD: v <- H v / sqrt(dim), H the Sylvester Hadamard
 *           matrix (dim a power of two, <= 128), computed in fp32.
 *   out_fmt CSA_FP8_E4M3: out uint8 [*][dim] + out_scale float[*], per row
 *                         scale = max(amax, FLT_MIN)/448, code = e4m3_rne(v/scale).
 *           CSA_MXFP4:    out uint8 [*][dim/2] + out_scale uint8 [*][dim/32]; per 32
 *                         elements X = floor(log2 amax) - 2 (X = -127 if amax == 0),
 *                         code = e2m1_rne(v / 2^X) saturated at +-6, byte = X + 127.
 *           CSA_F32:      out float [*][dim] (out_scale unused).
 *   dst_rows optional int32[rows]: row i is written to output row dst_rows[i]
 *           (e.g. a pool slot), and not written at all when dst_rows[i] < 0 (a
 *           decode step where a sequence completes no block); NULL writes row i
 *           to output row i.
 *   rope    used with CSA_PREP_ROPE (ignored otherwise); rope.pos / cos_sin
 *           must be set and rope.dim, rope.rows_per_pos valid, else
 *           CSA_ERR_INVALID.
 */
csa_status csa_index_prep(const void* v, csa_fmt v_fmt, int64_t rows, int32_t dim,
                          uint32_t flags, csa_fmt out_fmt, void* out, void* out_scale,
                          const int32_t* dst_rows, csa_rope rope, hipStream_t stream);

/*
 * csa_decode_prep -- every per-sequence write and the query preparation of one
 * decode step, in one launch ([P1] §1: the new token updates the compressed
 * cache, the raw window and the indexer's K cache before the indexer runs).
 * For sequence b with p = pos[b], the raw position of its current token:
 *   - if (p + 1) % ratio == 0 (the token completes block kb = (p+1)/ratio - 1),
 *     rows x[b][0 .. ratio) (positions p+1-ratio .. p) are compressed exactly
 *     as c4_compress does and stored at entry kb of c4, and, if k_rows is set,
 *     k_rows[b] is prepared exactly as csa_index_prep does and stored at entry
 *     kb of kpool;
 *   - row x[b][ratio-1] (the token) is stored at position p of raw, exactly as
 *     c4_compress with ratio 1 stores it;
 *   - if q_rows is set, q_rows[b][h] (h < H_I) are prepared as csa_index_prep
 *     does into q_out [B*H_I][...] and q_out_scale, in kpool.fmt.
 *  x        [B][ratio][576], CSA_BF16 or CSA_F32; ratio in [1, 128].
 *  pos      int32 [B].
 *  gate_w   float[576]; gate_b float[ratio].
 *  page_table int32 [B][pt_stride]: pages of c4 and of kpool (both page_size
 *           entries per page: kpool.page_size must equal c4.page_size).
 *  raw_page_table int32 [B][raw_pt_stride] over raw.page_size-token pages.
 *  k_rows, q_rows  [B][dim] and [B][H_I][dim] in kq_fmt (CSA_BF16 / CSA_F32),
 *           dim = kpool.dim; either may be NULL.
 *  flags    CSA_PREP_HADAMARD and / or CSA_PREP_ROPE, for both k and q rows;
 *           with CSA_PREP_ROPE both are rotated at the token's position pos[b]
 *           (the block's index-K row takes the position of the token that
 *           completes it), from rope.cos_sin; rope.pos and rope.rows_per_pos
 *           are not used.
 * c4 and raw must have the same format (FP8 or F32). Returns CSA_ERR_INVALID
 * on a bad pointer, size or format, CSA_OK (nothing enqueued) when B == 0.
 */
csa_status csa_decode_prep(const void* x, csa_fmt x_fmt, const int32_t* pos, int32_t B,
                           int32_t ratio, const float* gate_w, const float* gate_b,
                           const int32_t* page_table, int32_t pt_stride, csa_kv_pool c4,
                           const int32_t* raw_page_table, int32_t raw_pt_stride,
                           csa_kv_pool raw, const void* k_rows, const void* q_rows,
                           csa_fmt kq_fmt, int32_t H_I, uint32_t flags, csa_rope rope,
                           csa_index_pool kpool, void* q_out, void* q_out_scale,
                           hipStream_t stream);

/*
 * indexer_score -- lightning-indexer logits of every visible compressed entry
 * ([P1] §3 C4Indexer, §3.2 `logits [bs, c4_seqlen]`; [P2] CSA paragraph: a light
 * low-precision indexer scores compressed blocks for each query):
 *     logits[t*ld + j] = sum_h w[t][h] * ReLU(qhat[t][h] . khat[j]),   0 <= j < row_len[t]
 * with khat the dequantised index-K row of logical entry j of sequence row_seq[t]
 * and qhat the dequantised query. Entries j >= row_len[t] are not written.
 *   q        [T][H_I][D_I]. q_fmt CSA_BF16 / CSA_F32 (raw; prep flags decide what
 *            happens before scoring) or CSA_FP8_E4M3 / CSA_MXFP4 (already
 *            prepared, scales in q_scale: float [T][H_I] for FP8, uint8
 *            [T][H_I][D_I/32] e8m0 for MXFP4). A prepared q must match k.fmt.
 *   prep     0 or CSA_PREP_HADAMARD | CSA_PREP_QUANT for raw q: rotate and
 *            quantise q exactly as csa_index_prep does, to k.fmt. An F32 pool takes
 *            raw F32 q with prep 0. Either may be OR-ed with CSA_ROWS_PER_SEQ(n).
 *   w        float [T][H_I] head weights (w >= 0).
 *   row_seq, row_len  int32 [T]: sequence and visible length of each query row
 *            (decode: row_len = c4 length; prefill: row_len = min(N, (p+1)/4)).
 *   max_row_len HOST: an upper bound of row_len (sizes the grid); ld >= max_row_len.
 *   logits   float, row stride ld >= max row_len.
 *   q_used, q_used_scale  optional (NULL or both set): the prepared q codes and
 *            scales in q_scale's layout, for inspection.
 * Supported: F32 pool with D_I in {64,128}; FP8 / MXFP4 pools with D_I = 128.
 */
csa_status indexer_score(const void* q, csa_fmt q_fmt, const void* q_scale, uint32_t prep,
                         const float* w, int32_t T, int32_t H_I, int32_t D_I,
                         const int32_t* row_seq, const int32_t* row_len, int32_t max_row_len,
                         const int32_t* page_table, int32_t pt_stride, csa_index_pool k,
                         float* logits, int64_t ld, void* q_used, void* q_used_scale,
                         void* ws, size_t ws_bytes, hipStream_t stream);

/*
 * indexer_topk512 -- indexer_score followed by topk512_page_select on its
 * logits, in one call ([P1] §3 C4Indexer logits feeding §3.2's top-512
 * transform): phys_idx / logical_idx are exactly what
 *     indexer_score(..., logits, ld, ...);
 *     topk512_page_select(logits, ld, T, row_len, row_seq, page_table,
 *                         pt_stride, k.page_size, phys_idx, logical_idx, ...)
 * would produce. The index-K pool and the c4 KV pool share page_table and the
 * page size (k.page_size is the translation's c4_page_size), as in
 * csa_decode_prep. For FP8 / MXFP4 pools with few rows the logits are not
 * materialised: each scan workgroup selects the top-512 candidates of its
 * chunk from the logits it holds on chip. Rows of 9 to 64 scan chunks finish
 * inside the same launch: the last-arriving workgroup of each group of chunks
 * merges the group and the last group of a row selects the row; shorter rows
 * take one final pass per row, longer ones one merge and one final pass (exact
 * either way: an entry of a row's top-512 is in its chunk's top-512). Other shapes (many rows, rows
 * grouped by CSA_ROWS_PER_SEQ, an F32 pool) run the two calls through the
 * workspace.
 *   Arguments as indexer_score and topk512_page_select; max_row_len up to
 *   2097152.
 *   ws   csa_workspace_size(CSA_OP_INDEXER_TOPK, T, max_row_len, H_I) bytes
 *        (always needed). Its first 9216 bytes are counters that the fused
 *        selection finds at zero and leaves at zero: they must be zero before
 *        the first call with a workspace (a zero-filled allocation), and stay
 *        untouched between calls.
 *   scan_done  NULL, or an event recorded on `stream` right after the scan
 *        launch (before the final selection), so that a caller can time the
 *        scan alone or start dependent work early.
 */
csa_status indexer_topk512(const void* q, csa_fmt q_fmt, const void* q_scale, uint32_t prep,
                           const float* w, int32_t T, int32_t H_I, int32_t D_I,
                           const int32_t* row_seq, const int32_t* row_len, int32_t max_row_len,
                           const int32_t* page_table, int32_t pt_stride, csa_index_pool k,
                           int32_t* phys_idx, int32_t* logical_idx, void* q_used,
                           void* q_used_scale, void* ws, size_t ws_bytes, hipEvent_t scan_done,
                           hipStream_t stream);

/*
 * indexer_topk512_noalloc -- indexer_topk512 for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc): the same arguments and results, without `ws` and
 * `scan_done`. The workspace is the library's own array in device memory,
 * CSA_NOALLOC_SCRATCH_BYTES per GPU, which the library holds until the process
 * ends; the call itself allocates and frees nothing.
 *   Limit: calls whose workspace, csa_workspace_size(CSA_OP_INDEXER_TOPK, T,
 *   max_row_len, H_I), exceeds CSA_NOALLOC_SCRATCH_BYTES return
 *   CSA_ERR_WORKSPACE and launch nothing (decode shapes fit: 32 rows x 128K,
 *   4 rows x 1M, 128 multi-token rows x 128K; a 4096-row prefill does not).
 *   Every call on one GPU uses that GPU's single array, so calls that overlap
 *   on one GPU (different streams, or different host threads without ordering)
 *   race on it and their results are undefined; calls ordered on one stream
 *   are fine. `stream` must belong to the current device. The array keeps the
 *   last call's contents; nothing in it needs to start cleared.
 *   Returns CSA_ERR_HIP if the array's device address cannot be looked up.
 */
#define CSA_NOALLOC_SCRATCH_BYTES ((size_t)32 << 20)
csa_status indexer_topk512_noalloc(const void* q, csa_fmt q_fmt, const void* q_scale,
                                   uint32_t prep, const float* w, int32_t T, int32_t H_I,
                                   int32_t D_I, const int32_t* row_seq, const int32_t* row_len,
                                   int32_t max_row_len, const int32_t* page_table,
                                   int32_t pt_stride, csa_index_pool k, int32_t* phys_idx,
                                   int32_t* logical_idx, void* q_used, void* q_used_scale,
                                   hipStream_t stream);

/*
 * topk512_page_select -- the fixed top-512 transform ([P1] §3.2): per row, the
 * 512 largest logits among j < row_len[r], translated through the page table
 * to physical slots page_table[row_seq[r]][j / c4_page_size] * c4_page_size
 * + j % c4_page_size.
 * Order: by logit descending, equal logits by lower j; -0 equals +0; NaN ranks
 * below -inf. If row_len <= 512 every entry is selected. The selected entries are
 * written in ascending j; the unused tail of a row is -1.
 *   phys_idx    int32 [R][512] (required); logical_idx int32 [R][512] or NULL.
 *   ws          csa_workspace_size(CSA_OP_TOPK, R, ld, 1) bytes: when ld > 16384,
 *               or ld > 8192 and R < 128, rows are reduced in two launches through
 *               it (chunk candidates, then the row); otherwise 0 bytes. ld up to
 *               2097152.
 */
csa_status topk512_page_select(const float* logits, int64_t ld, int32_t R,
                               const int32_t* row_len, const int32_t* row_seq,
                               const int32_t* page_table, int32_t pt_stride,
                               int32_t c4_page_size, int32_t* phys_idx,
                               int32_t* logical_idx, void* ws, size_t ws_bytes,
                               hipStream_t stream);

/*
 * topk_page_select -- the generic top-k transform, k in [1, CSA_TOPK_MAX]: the
 * selection DSA makes over raw tokens ([P1] §1: in DSA the indexer picks the
 * top-k tokens and attention reads only their KV; §3.2 contrasts the fixed-k
 * transform with a generic top-k; §2.2: DSA pages hold 64 tokens). Same rules
 * as topk512_page_select with k in place of 512: per row the k largest logits
 * among j < row_len[r] (larger first, equal logits by lower j, -0 == +0, NaN
 * below -inf; all of them if row_len <= k), in ascending j, translated through
 * the page table with `page_size` entries per page; rows of phys_idx /
 * logical_idx hold k entries, the unused tail -1.
 *   ws   csa_workspace_size(CSA_OP_TOPK_K, R, ld, k) bytes.
 *   ld   up to (32768 / k) * 32768 (k = 2048: 524288), else CSA_ERR_UNSUPPORTED.
 */
csa_status topk_page_select(const float* logits, int64_t ld, int32_t R, const int32_t* row_len,
                            const int32_t* row_seq, const int32_t* page_table, int32_t pt_stride,
                            int32_t page_size, int32_t k, int32_t* phys_idx,
                            int32_t* logical_idx, void* ws, size_t ws_bytes, hipStream_t stream);

/*
 * hisparse_swap_in -- HiSparse staging of each step's selected compressed
 * entries in a near (hot) KV pool ([P1] §5: the coordinator swaps the step's
 * top-512 compressed tokens into fast storage, keyed by the top-k result's raw
 * (logical) indices, and attention reads them there; entries selected again
 * stay resident). Sequence s owns the near-pool slots [s * hot_slots,
 * (s + 1) * hot_slots). For query row r of sequence s = row_seq[r], with its
 * selection logical_idx[r][0..k) (-1 = empty):
 *   - an entry already resident (slot_of[s][j] = h >= 0) is used in place;
 *   - the m entries that are not are assigned, in selection order, the m
 *     least recently used hot slots of s that no entry of this step uses
 *     (empty slots first, then the smallest last_use, equal stamps by lower
 *     slot), in ascending slot order; the slot's previous entry is unmapped;
 *     the entry (latent, scale, RoPE dims) is copied from `far` (logical entry
 *     j at far_page_table[s][j / page] * page + j % page, page = far.page_size);
 *   - every used slot gets last_use = step; near_idx[r][i] is the near-pool
 *     slot s * hot_slots + h of logical_idx[r][i] (-1 where it is -1).
 * Attention then runs as csa_sparse_attn(..., near_idx, k, near pool, ...).
 * State, owned by the caller (device int32): slot_of [S][max_entries]
 * (logical entry -> hot slot or -1), owner [S][hot_slots] (hot slot ->
 * logical entry or -1) and last_use [S][hot_slots]; start with slot_of and
 * owner all -1. `far` may be any memory the device can read (an HBM pool, or
 * host memory mapped for the device).
 * Requires 1 <= k <= 512, k <= hot_slots <= 4096, step >= 0, pools of the same
 * format; rows of one call must belong to different sequences (rows of one
 * sequence in one call race), the near pool must hold S * hot_slots slots and
 * max_entries cover every selected index (caller's contract).
 */
csa_status hisparse_swap_in(const int32_t* logical_idx, int32_t R, int32_t k,
                            const int32_t* row_seq, csa_kv_pool far,
                            const int32_t* far_page_table, int32_t far_pt_stride,
                            csa_kv_pool near, int32_t hot_slots, int32_t* slot_of,
                            int64_t max_entries, int32_t* owner, int32_t* last_use, int32_t step,
                            int32_t* near_idx, hipStream_t stream);

/*
 * csa_sparse_attn -- MLA-style sparse attention of each query over its selected
 * compressed entries plus a sliding window of raw tokens ([P1] §1: attention
 * reads the 512 selected compressed KV; [P2] CSA paragraph: a sliding-window
 * branch keeps recent uncompressed tokens). For query t at raw position
 * p = q_pos[t] of sequence s = q_seq[t], head h:
 *   E = { c4 slot phys_idx[t][i] : i < k_sel, != -1 }
 *       U { raw slot of positions max(0, p-window+1) .. p via raw_page_table[s] }
 *   score_e = softmax_scale * sum_{d<576} q[t][h][d] * kv_e[d]
 *   out[t][h][:] = sum_e softmax(score)_e * kv_e[0:512]
 * kv_e is the dequantised entry. All H heads share the KV (MQA).
 *   q    [T][H][576]: CSA_BF16 with FP8 pools (H a multiple of 16, <= 128), or
 *        CSA_F32 with F32 pools (any H; lists of up to 32768 entries). out [T][H][512] CSA_BF16 or CSA_F32
 *        (F32 pools: CSA_F32 only).
 *   c4 and raw pools must have the same fmt; raw.page_size is the raw page size.
 *   Requires 0 <= window <= 4096, 0 <= k_sel <= CSA_TOPK_MAX and
 *   k_sel + window >= 1. k_sel up to 2048 with window 0 is the DSA mode: the
 *   selection is over raw tokens (topk_page_select over an index pool of raw
 *   tokens), `c4` is then the raw KV pool, and no window is added ([P1] §1,
 *   DSA: attention reads the k selected raw tokens). A query must have at
 *   least one entry (a selected entry or a window token).
 *   ws   workspace of csa_workspace_size(CSA_OP_CSA_ATTN, T, k_sel + window, H)
 *        bytes for FP8 pools, CSA_OP_CSA_ATTN_F32 for F32 pools (may be 0
 *        bytes / NULL when that size is 0).

 */
csa_status csa_sparse_attn(const void* q, csa_fmt q_fmt, int32_t T, int32_t H,
                           const int32_t* q_seq, const int32_t* q_pos,
                           const int32_t* phys_idx, int32_t k_sel, csa_kv_pool c4,
                           csa_kv_pool raw, const int32_t* raw_page_table,
                           int32_t raw_pt_stride, int32_t window, float softmax_scale,
                           void* out, csa_fmt out_fmt, void* ws, size_t ws_bytes,
                           hipStream_t stream);

/*
 * hca_dense_attn -- heavily compressed attention ([P2] HCA paragraph: ~128x
 * compression, then dense attention over the compressed blocks), plus the same
 * sliding window as CSA. As csa_sparse_attn with
 *   E = { hca entry j of sequence s : ratio*j + ratio - 1 <= p }  U  window(p).
 *   max_len HOST: an upper bound of q_pos[t] + 1 (sizes the split of the entry
 *           list); ws: csa_workspace_size(CSA_OP_HCA_ATTN, T, max_len/ratio + window, H)
 *           (CSA_OP_HCA_ATTN_F32 for F32 pools).
 */
csa_status hca_dense_attn(const void* q, csa_fmt q_fmt, int32_t T, int32_t H,
                          const int32_t* q_seq, const int32_t* q_pos, int32_t max_len,
                          int32_t ratio,
                          csa_kv_pool hca, const int32_t* hca_page_table,
                          int32_t hca_pt_stride, csa_kv_pool raw,
                          const int32_t* raw_page_table, int32_t raw_pt_stride,
                          int32_t window, float softmax_scale, void* out,
                          csa_fmt out_fmt, void* ws, size_t ws_bytes, hipStream_t stream);

/* Workspace sizes (bytes) for the calls that take `ws`.
 * op: CSA_OP_INDEXER (rows = T, heads = H_I; needed only when the query is
 *     prepared inside the call and q_used is NULL), CSA_OP_TOPK (rows = R,
 *     max_len = ld),
 *     CSA_OP_CSA_ATTN / CSA_OP_HCA_ATTN (rows = T, max_len = most entries of
 *     one query's list, heads = H; FP8 pools), CSA_OP_CSA_ATTN_F32 /
 *     CSA_OP_HCA_ATTN_F32 (the same for F32 pools), CSA_OP_INDEXER_TOPK
 *     (rows = T, max_len = max_row_len, heads = H_I), CSA_OP_TOPK_K
 *     (topk_page_select: rows = R, max_len = ld, heads = k). */
#define CSA_OP_INDEXER  0
#define CSA_OP_TOPK     1
#define CSA_OP_CSA_ATTN 2
#define CSA_OP_HCA_ATTN 3
#define CSA_OP_INDEXER_TOPK 4
#define CSA_OP_CSA_ATTN_F32 5
#define CSA_OP_HCA_ATTN_F32 6
#define CSA_OP_TOPK_K       7
size_t csa_workspace_size(int32_t op, int64_t rows, int64_t max_len, int32_t heads);

const char* csa_status_string(csa_status s);

/*
 * csa_set_debug -- debug mode on (nonzero) or off; csa_debug_enabled returns
 * the current mode. The mode starts on when the environment holds CSA_DEBUG
 * set to anything but "" or "0" when the library first needs it.
 *   In debug mode c4_compress, csa_decode_prep, indexer_score,
 *   indexer_topk512 (and _noalloc), topk_page_select / topk512_page_select,
 *   hisparse_swap_in, csa_sparse_attn and hca_dense_attn first check on the
 *   device the integers they are about to follow, within the extents the
 *   host-side arguments give: row lengths within their capacity (max_row_len,
 *   ld), non-negative positions and sequence indices, every page id of the
 *   pages a row touches in [0, num_pages) and within the page-table row
 *   (pt_stride), selected slots in [-1, num_pages * page_size), HiSparse
 *   logical entries in [-1, max_entries). The first violation is printed to
 *   stderr (entry point, kind, row, index, value) and the call returns
 *   CSA_ERR_BOUNDS without launching its kernels. The checks synchronise the
 *   stream: debug mode is for finding a caller's bad tables, not for graph
 *   capture or timing. A page-table row past the caller's last sequence
 *   cannot be known to the library and is not checked.
 *   Thread-safe to read; set it while no call is in flight.
 */
void csa_set_debug(int32_t on);
int32_t csa_debug_enabled(void);

/* Library version, e.g. "0.1.0". */
const char* csa_version(void);

#ifdef __cplusplus
}
#endif
#endif /* CSA_H_ */
