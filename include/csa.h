/*
 * csa.h -- C ABI of libcsa, the gfx950 (MI355X) kernels of the DeepSeek-V4
 * hybrid compressed attention hot path: CSA (4:1 compression, Lightning
 * Indexer, top-k, sparse MQA attention with a raw window and a sink) and HCA
 * (128:1 compression, dense MQA attention with a sink).
 *
 * Sources (cited by page and section):
 *   shareware.cn, DeepSeek V4 Hybrid Attention architecture article,
 *     sections 二-十二 (compression ratios, the three-level memory, adaptive
 *     compression, two-path overlap, Lightning Indexer, ReLU, dense HCA,
 *     causality and the window, MQA, the attention sink);
 *   trdm.cn, "从 MLA 到 CSA，聊聊大模型 Attention 的瘦身与闪送",
 *     sections 2.1 (MQA), 3.1 (online softmax), 4.2 (Lightning Indexer),
 *     4.3 (V4 hybrid attention: two streams, window concatenation, HCA);
 *   aimodeling.com news item on V4 hybrid attention (CSA: 4:1, top 1024,
 *     128-token window; HCA: 128:1, dense).
 *
 * Conventions shared by every entry point
 *   - All tensors are dense, row-major, in caller-owned DEVICE memory, 16-byte
 *     aligned.  The library never allocates, frees or synchronises: work is
 *     enqueued on `stream` (a hipStream_t; NULL = the null stream) and CSA_OK
 *     means it was enqueued.  Calls may be captured into a HIP graph.
 *   - Arguments are validated before anything is enqueued; on an error no
 *     output is touched.  Launch failures return CSA_ERR_HIP;
 *     csa_last_error() gives a thread-local detail string.
 *   - dtype selects the storage type of every bf16/fp32 tensor argument
 *     (declared `void*`).  Accumulation is fp32.  Scores, sinks, biases,
 *     head weights and lse are always fp32; indices are int32.
 *   - CSA_FP8 is the OCP 8-bit float E4M3 (1 sign, 4 exponent bits with bias
 *     7, 3 mantissa bits; exponent 0 holds subnormals m * 2^-9; codes 0x7F
 *     and 0xFF are NaN; no infinities, largest finite value 448).  The pages
 *     allow FP8 storage for the main KV and low precision for the indexer's
 *     q.k path (shareware.cn article, the low-precision item of its list of
 *     what is compressed) without naming an encoding.  Accepted by
 *     csa_compress / hca_compress (inputs and output in FP8, arithmetic in
 *     fp32, output rounded to nearest even) and by csa_index_score /
 *     csa_index_topk (q_idx and k_idx in FP8, d_I = 128, H_I in {16, 32, 64,
 *     128}), and by the attention entry points for the cached K/V only
 *     (kc, vc, kr, vr in FP8; q and out stay bf16; d = 512, H % 64 == 0):
 *     each code converts exactly to bf16 and the arithmetic is the bf16
 *     path's.  FP8 carries no scale argument: a per-tensor K scale folds into
 *     `scale`, a V scale into the caller's use of `out`.
 *   - CSA_MXFP4 is the OCP microscaling FP4 format: elements E2M1 (1 sign,
 *     2 exponent bits with bias 1, 1 mantissa bit: magnitudes 0, 0.5, 1,
 *     1.5, 2, 3, 4, 6), each block of 32 consecutive elements of a row
 *     sharing one E8M0 scale byte e (value 2^(e-127); e = 255 is NaN).  An
 *     MXFP4 tensor of N rows of d elements is one buffer: N*d/2 code bytes
 *     (row-major; element 2i in the low nibble of byte i, 2i+1 in the high
 *     nibble), then N*d/32 scale bytes (row-major; scale j of a row covers
 *     its elements 32j .. 32j+31).  The pages run the indexer's q.k in FP4
 *     (shareware.cn article, the low-precision item of its list of what is
 *     compressed); accepted by csa_index_score / csa_index_topk for q_idx (N
 *     = B*T*H_I) and k_idx (N = B*L) with d_I = 128, H_I in {16, 32, 64,
 *     128}.  As the dtype of csa_compress / hca_compress /
 *     csa_compress_append it names the output only: raw rows (and staging
 *     rings) are bf16, the entries are written as MXFP4 (out holds N =
 *     B*out_ld rows; an append's cache N = B*L rows, or num_pages*page pool
 *     rows), D a multiple of 32.  Each entry is computed in fp32 as for bf16
 *     output, then every block of 32 channels takes the scale 2^E, E =
 *     floor(log2 of the block's largest magnitude) - 2, at least -127 (an
 *     all-zero block: E = -127), and each channel the E2M1 code nearest to
 *     v / 2^E (ties to the even code, past 6 saturating to 6, sign bit of
 *     v).  Attention returns CSA_ERR_UNSUPPORTED for it.
 *   - Positions: a batch holds B sequences of n_ctx tokens (uniform length).
 *     The T queries of a sequence sit at positions t_i = n_ctx - T + i.
 *     Compressed entry s covers tokens [s*m, (s+1)*m) and is visible to the
 *     query at t iff (s+1)*m <= t (the block is complete and strictly
 *     earlier), i.e. s < floor(t/m).
 *   - Raw-window buffers kr / vr [B][R][d] hold positions n_ctx-R .. n_ctx-1;
 *     the window of query t is the raw tokens max(0, t-W+1) .. t.
 *   - Inputs and outputs must not alias.
 */
#ifndef CSA_H
#define CSA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum csa_dtype { CSA_F32 = 0, CSA_BF16 = 1, CSA_FP8 = 2, CSA_MXFP4 = 3 } csa_dtype_t;

typedef enum csa_status {
  CSA_OK = 0,
  CSA_ERR_INVALID_ARG = 1, /* null / misaligned pointer, inconsistent sizes */
  CSA_ERR_UNSUPPORTED = 2, /* shape or dtype this build has no kernel for */
  CSA_ERR_WORKSPACE = 3,   /* workspace missing or smaller than required */
  CSA_ERR_HIP = 4          /* a HIP launch failed; see csa_last_error() */
} csa_status_t;

/* ---------------------------------------------------------------------------
 * csa_layout_t -- how a serving batch is laid out, for the *_ex calls and the
 * per-token appends (trdm.cn, section 3, Paged Attention paragraph: a block
 * table maps each sequence's logical blocks to physical ones, so sequences
 * of mixed lengths share one pool).  Every field is optional:
 *   seq_len      device int64 [B]: tokens of each sequence; the n_ctx
 *                argument is then the largest.  Query i of sequence b sits
 *                at seq_len[b] - T + i.  Values outside [T, n_ctx] are
 *                clamped into it (keeping every access in bounds); NULL =
 *                every sequence has n_ctx tokens.
 *   block_table  device int32 [B][bt_stride]: the compressed caches (kc, vc,
 *                k_idx) are pools of num_pages pages of `page` entries
 *                (rows); entry s of sequence b is pool row
 *                block_table[b][s / page] * page + s % page.  page is a
 *                multiple of 16, bt_stride >= ceil(L / page), and
 *                num_pages * page < 2^31.  Page ids outside [0, num_pages)
 *                are clamped into it.  An MXFP4 key pool holds the codes of
 *                all num_pages * page keys, then their scales.  NULL = dense
 *                [B][L] caches.
 *   window_ring  1: the raw-window buffers kr / vr [B][R][d] are rings that
 *                hold position u at slot u % R (what csa_window_append
 *                writes); R >= T + W - 1 and R >= W.  0: they hold
 *                positions n_b - R .. n_b - 1 in order.
 * ------------------------------------------------------------------------- */
typedef struct csa_layout {
  const int64_t* seq_len;
  const int32_t* block_table;
  int64_t bt_stride;
  int64_t page;
  int64_t num_pages;
  int32_t window_ring;
} csa_layout_t;

/* ---------------------------------------------------------------------------
 * csa_compress -- block-weighted compression of one K/V/index-key stream.
 * shareware.cn article, section 四 (each entry is a dynamic, per-dimension
 * softmax-weighted sum of its block's raw rows) and section 五 / trdm.cn
 * section 4.3 改进二 (two-path overlap).  For entry j and channel c:
 *   candidates: stream A tokens u in [j*m, min((j+1)*m, n)) with value
 *     x_a[u][c] and logit z_a[u][c] (+ bias[m + u - j*m][c] in two-path mode,
 *     + bias[u - j*m][c] in single-path mode);
 *   two-path (x_b, z_b non-NULL) also stream B tokens u in [(j-1)*m, j*m) for
 *     j >= 1, value x_b[u][c], logit z_b[u][c] (+ bias[u - (j-1)*m][c]);
 *   out[j][c] = sum softmax(logits) * values   (one joint softmax).
 * A trailing partial block is compressed over the tokens present.
 *   x_a, z_a, x_b, z_b : [B][n_raw][D] dtype, raw positions p0 .. p0+n_raw-1
 *                        of sequences of n tokens (z = learned logits)
 *   bias               : NULL, or fp32 [m][D] (single) / [2m][D] (two-path)
 *   out                : entries e0 .. e1-1; entry j of sequence b at
 *                        out + ((b*out_ld) + (j - e0)) * D  (out_ld >= e1-e0)
 * Requires D % 8 == 0, 0 <= e0 <= e1 <= ceil(n/m), and the raw rows each
 * requested entry reads to lie in [p0, p0+n_raw).  With p0 = 0, n_raw = n,
 * e0 = 0, e1 = ceil(n/m) this is the bulk compression of whole sequences; a
 * decode step passes the last raw tokens and e0 = e1-1.
 * ------------------------------------------------------------------------- */
csa_status_t csa_compress(const void* x_a, const void* z_a, const void* x_b, const void* z_b,
                          const float* bias, void* out, int64_t B, int64_t n, int64_t D,
                          int64_t m, int64_t p0, int64_t n_raw, int64_t e0, int64_t e1,
                          int64_t out_ld, csa_dtype_t dtype, void* stream);

/* hca_compress -- the same operator with one stream and m = 128 in HCA
 * (shareware.cn article, sections 二 and 三.3; trdm.cn section 4.3, HCA
 * paragraph: no second stream).  Arguments as csa_compress single path. */
csa_status_t hca_compress(const void* x, const void* z, const float* bias, void* out, int64_t B,
                          int64_t n, int64_t D, int64_t m, int64_t p0, int64_t n_raw,
                          int64_t e0, int64_t e1, int64_t out_ld, csa_dtype_t dtype,
                          void* stream);

/* csa_compress_append -- decode-time cache maintenance of one stream: one new
 * raw token per sequence (shareware.cn article, section 十: an entry exists
 * once its block is complete, the window covers the rest; trdm.cn section 4.3
 * 改进三).  Token p = pos[b] of sequence b (x_a, z_a, and x_b, z_b in
 * two-path mode: [B][D] rows) is staged into the rings ring_xa, ring_za
 * (ring_xb, ring_zb) [B][S][D] at slot p % S; when p + 1 is a multiple of m
 * the entry p / m is compressed exactly as a bulk csa_compress launch does
 * (every candidate folded in order: the same result bit for bit; launches of
 * few entries with m >= 32 split each entry over 16 lanes instead, equal up
 * to fp32 rounding) from the staged rows of its block
 * (and of the previous block through stream B) and written to the cache:
 * row b * L + p / m of cache [B][L][D], or its pool row through
 * layout->block_table.  S >= 2m in two-path mode, >= m otherwise; bias as
 * csa_compress.  pos is device int64 [B]; a negative position stages
 * nothing, and entries at or past L are not written.  The rings must hold
 * the sequence's earlier tokens of the current (and previous) block: a
 * sequence's prefix is compressed in bulk with csa_compress and its last
 * 2m raw rows copied into the rings (slot u % S) before the first append.
 * layout: NULL, or only block_table / bt_stride / page / num_pages used. */
csa_status_t csa_compress_append(const csa_layout_t* layout, const void* x_a, const void* z_a,
                                 const void* x_b, const void* z_b, const float* bias, void* ring_xa,
                                 void* ring_za, void* ring_xb, void* ring_zb, int64_t S,
                                 const int64_t* pos, void* cache, int64_t L, int64_t B, int64_t D,
                                 int64_t m, csa_dtype_t dtype, void* stream);

/* csa_window_append -- the raw window rows (k_new, v_new [B][d]) of one new
 * token per sequence into ring windows kr, vr [B][R][d] at slot pos[b] % R
 * (shareware.cn article, section 三.1: the latest raw tokens stay
 * uncompressed).  pos: device int64 [B], non-negative. */
csa_status_t csa_window_append(const void* k_new, const void* v_new, void* kr, void* vr,
                               const int64_t* pos, int64_t B, int64_t R, int64_t d,
                               csa_dtype_t dtype, void* stream);

/* ---------------------------------------------------------------------------
 * csa_index_score -- Lightning Indexer scores (shareware.cn article,
 * sections 六-七; trdm.cn section 4.2):
 *   score[b][t][s] = sum_h w[b][t][h] * max(0, sum_c q_idx[b][t][h][c]*k_idx[b][s][c])
 * for visible s (s < floor(t/m)); -inf for the other s < L.  No scale.
 *   q_idx : [B][T][H_I][d_I] dtype      w_idx : fp32 [B][T][H_I] or NULL (= 1)
 *   k_idx : [B][L][d_I] dtype (one key per compressed entry, shared by heads)
 *   score : fp32 [B][T][L]
 * bf16 needs H_I in {16, 32, 64, 128} with d_I = 128, or H_I in {32, 64} with
 * d_I = 64; fp32 needs H_I*d_I <= 16384.
 * ------------------------------------------------------------------------- */
csa_status_t csa_index_score(const void* q_idx, const float* w_idx, const void* k_idx, int64_t B,
                             int64_t T, int64_t n_ctx, int64_t L, int64_t H_I, int64_t d_I,
                             int64_t m, float* score, csa_dtype_t dtype, void* stream);

/* csa_topk_select -- per query keep the min(k, V) highest of the V = min(L,
 * floor(t/m)) visible scores (shareware.cn article, section 六; aimodeling.com
 * CSA paragraph: 1024 per query).  Equal scores (-0 == +0) go to the lower
 * entry index.  idx int32 [B][T][k] receives the kept indices in ascending
 * order, -1 padded; out_score (NULL or fp32 [B][T][k]) their scores (-inf in
 * padded slots).  score is fp32 [B][T][L] and must hold no NaN among the
 * visible entries.  1 <= k <= 1048576.  ws: csa_topk_select_workspace(B, T, L, k)
 * bytes of device scratch for the per-part candidates. */
size_t csa_topk_select_workspace(int64_t B, int64_t T, int64_t L, int64_t k);
csa_status_t csa_topk_select(const float* score, int64_t B, int64_t T, int64_t n_ctx, int64_t L,
                             int64_t m, int64_t k, int32_t* idx, float* out_score, void* ws,
                             size_t ws_bytes, void* stream);

/* csa_index_topk -- csa_index_score followed by csa_topk_select, same
 * results bit for bit.  For bf16, d_I = 128 and decode-like shapes (the scan's
 * key ranges times k at most 16384, k <= 2048) with a full-size workspace the
 * scan keeps each key range's top-k candidates itself and no score matrix is
 * written (two kernels); decode shapes with more key ranges (one to four
 * queries at 1M entries, eight at 131,072) write the scores and each key range's exact
 * short list, merge the lists per query and run the stand-alone selection
 * only for queries whose lists do not settle them (same results); otherwise
 * the fp32 score matrix and the selection scratch are kept in the caller's
 * workspace.  When ws_bytes is below
 * csa_index_topk_workspace(B, T, L, H_I, k) the queries are processed in
 * groups that fit; ws_bytes must cover at least one query
 * (csa_index_topk_workspace(1, 1, L, H_I, k)).  Results do not depend on
 * ws_bytes.  The workspace is scratch: its contents on entry do not matter.
 * The size does not depend on H_I today; the argument keeps kernels free to
 * stage per-head data. */
size_t csa_index_topk_workspace(int64_t B, int64_t T, int64_t L, int64_t H_I, int64_t k);
csa_status_t csa_index_topk(const void* q_idx, const float* w_idx, const void* k_idx, int64_t B,
                            int64_t T, int64_t n_ctx, int64_t L, int64_t H_I, int64_t d_I,
                            int64_t m, int64_t k, int32_t* idx, float* out_score, void* ws,
                            size_t ws_bytes, csa_dtype_t dtype, void* stream);

/* csa_index_topk_ex -- csa_index_topk over a serving layout (per-sequence
 * lengths, paged index keys k_idx: a pool of layout->num_pages pages).  L is
 * the capacity in entries of the longest sequence.  NULL layout = csa_index_topk. */
csa_status_t csa_index_topk_ex(const csa_layout_t* layout, const void* q_idx, const float* w_idx,
                               const void* k_idx, int64_t B, int64_t T, int64_t n_ctx, int64_t L,
                               int64_t H_I, int64_t d_I, int64_t m, int64_t k, int32_t* idx,
                               float* out_score, void* ws, size_t ws_bytes, csa_dtype_t dtype,
                               void* stream);

/* csa_index_topk_noalloc -- csa_index_topk for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc): the same arguments without ws / ws_bytes, the same
 * kernels and the same results bit for bit.  Its scratch is a static device
 * array of csa_index_topk_noalloc_max_bytes() bytes (32 MiB) that the library
 * holds on every GPU it runs on until the process ends; the call allocates
 * and frees nothing.  The scratch must hold one query row's scores and
 * selection state (about 4 * L + 8 * 16 * k bytes, so L up to ~7.5M at
 * k = 1024); larger rows return CSA_ERR_UNSUPPORTED before anything is
 * enqueued.  Bigger batches are processed in groups of rows that fit.
 * Every call on one GPU shares that GPU's scratch: calls that overlap on one
 * GPU (different streams or threads) race; calls in order on one stream do
 * not.  The calling thread's current device must be the device of `stream`. */
size_t csa_index_topk_noalloc_max_bytes(void);
csa_status_t csa_index_topk_noalloc(const void* q_idx, const float* w_idx, const void* k_idx,
                                    int64_t B, int64_t T, int64_t n_ctx, int64_t L, int64_t H_I,
                                    int64_t d_I, int64_t m, int64_t k, int32_t* idx,
                                    float* out_score, csa_dtype_t dtype, void* stream);

/* ---------------------------------------------------------------------------
 * csa_sparse_attn -- CSA main attention (shareware.cn article, sections 三.1,
 * 十, 十一, 十二; trdm.cn section 4.3 改进三).  Per query (b, t) and head h the
 * rows are the selected compressed entries kc/vc[b][idx[b][t][j]] (slots
 * holding -1 are skipped) followed by the raw window rows; one shared K/V
 * head (MQA).  l_i = scale * q[b][t][h] . k_i, sink logit sigma_h with no
 * value:
 *   out[b][t][h] = sum_i e^{l_i} v_i / (e^{sigma_h} + sum_i e^{l_i})
 *   lse[b][t][h] = log(e^{sigma_h} + sum_i e^{l_i})        (natural log)
 *   q   : [B][T][H][d] dtype (bf16 when dtype is CSA_FP8)
 *   kc, vc : [B][L][d] dtype
 *   idx : int32 [B][T][k], entries in [0, L) or -1
 *   kr, vr : [B][R][d] raw positions n_ctx-R .. n_ctx-1 (NULL when W == 0);
 *            R >= T + W - 1 and R <= n_ctx when W > 0
 *   sink: fp32 [H] or NULL (= no sink)
 *   out : [B][T][H][d] dtype (bf16 when dtype is CSA_FP8)
 *   lse : fp32 [B][T][H] or NULL
 *   ws  : csa_sparse_attn_workspace(...) bytes (may be 0 => ws may be NULL),
 *         16-byte aligned; holds the per-split partial rows of a launch
 *         split over the row list (its contents are scratch)
 * bf16 needs H % 64 == 0, d in {128, 256, 512} and k + W <= 131072;
 * FP8 (K/V storage, bf16 q and out) needs H % 64 == 0, d = 512 and
 * k + W <= 131072; fp32 needs d <= 512.  L, R and W are at most 2^30.  Unsupported shapes
 * return CSA_ERR_UNSUPPORTED, nothing is launched.
 * ------------------------------------------------------------------------- */
size_t csa_sparse_attn_workspace(int64_t B, int64_t T, int64_t H, int64_t d, int64_t k, int64_t W,
                                 csa_dtype_t dtype);
csa_status_t csa_sparse_attn(const void* q, const void* kc, const void* vc, int64_t L,
                             const int32_t* idx, int64_t k, const void* kr, const void* vr,
                             int64_t R, int64_t W, const float* sink, float scale, int64_t B,
                             int64_t T, int64_t n_ctx, int64_t H, int64_t d, void* out,
                             float* lse, void* ws, size_t ws_bytes, csa_dtype_t dtype,
                             void* stream);

/* csa_attn_workspace -- workspace bytes that serve any attention call of the
 * given B, T, H, d whose per-query row list (csa_sparse_attn: k + W rows;
 * hca_dense_attn: min(L, floor(t/m)) + W rows) is at most n_rows long, for
 * every storage type.  It is at least csa_sparse_attn_workspace and
 * hca_dense_attn_workspace of such calls, which give the exact need. */
size_t csa_attn_workspace(int64_t B, int64_t T, int64_t H, int64_t d, int64_t n_rows);

/* hca_dense_attn -- HCA attention: every visible compressed entry s <
 * min(L, floor(t/m)) densely, no indexer (shareware.cn article, section 八;
 * aimodeling.com HCA paragraph), followed by the optional raw window (W = 0
 * for none; trdm.cn section 4.3, HCA paragraph), with the same sink softmax and
 * argument conventions as csa_sparse_attn. */
size_t hca_dense_attn_workspace(int64_t B, int64_t T, int64_t H, int64_t d, int64_t L, int64_t m,
                                int64_t n_ctx, int64_t W, csa_dtype_t dtype);
csa_status_t hca_dense_attn(const void* q, const void* kc, const void* vc, int64_t L, int64_t m,
                            const void* kr, const void* vr, int64_t R, int64_t W,
                            const float* sink, float scale, int64_t B, int64_t T, int64_t n_ctx,
                            int64_t H, int64_t d, void* out, float* lse, void* ws,
                            size_t ws_bytes, csa_dtype_t dtype, void* stream);

/* csa_sparse_attn_ex / hca_dense_attn_ex -- the attention calls over a
 * serving layout: per-sequence lengths, paged kc / vc pools, ring windows.
 * The workspace: csa_attn_workspace(B, T, H, d, rows) bytes with rows the
 * longest row list (k + W, or the most visible entries + W).  NULL layout =
 * csa_sparse_attn / hca_dense_attn. */
csa_status_t csa_sparse_attn_ex(const csa_layout_t* layout, const void* q, const void* kc,
                                const void* vc, int64_t L, const int32_t* idx, int64_t k,
                                const void* kr, const void* vr, int64_t R, int64_t W,
                                const float* sink, float scale, int64_t B, int64_t T, int64_t n_ctx,
                                int64_t H, int64_t d, void* out, float* lse, void* ws,
                                size_t ws_bytes, csa_dtype_t dtype, void* stream);
csa_status_t hca_dense_attn_ex(const csa_layout_t* layout, const void* q, const void* kc,
                               const void* vc, int64_t L, int64_t m, const void* kr, const void* vr,
                               int64_t R, int64_t W, const float* sink, float scale, int64_t B,
                               int64_t T, int64_t n_ctx, int64_t H, int64_t d, void* out,
                               float* lse, void* ws, size_t ws_bytes, csa_dtype_t dtype,
                               void* stream);

/* csa_time_next_scan -- instrumentation: the next indexer scan kernel that a
 * csa_index_score / csa_index_topk call on this host thread launches records
 * start_event (hipEvent_t) as the kernel starts and stop_event as it ends
 * (both stamped by the kernel's own dispatch, so no event command sits
 * between the call's kernels); the request then clears.  Both NULL clears a
 * pending request.  The events belong to the caller and must exist on the
 * scan's device; the call itself enqueues nothing. */
csa_status_t csa_time_next_scan(void* start_event, void* stop_event);

/* Status names and the calling thread's last error detail (never NULL). */
const char* csa_status_string(csa_status_t status);
const char* csa_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* CSA_H */
