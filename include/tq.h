/*
 * tq.h - C ABI of the TurboQuant compressed KV cache for AMD Instinct MI355X (gfx950).
 *
 * The method follows the AI Heartland news article "Apple Silicon向けSwiftLM、
 * TurboQuant KVキャッシュ圧縮とSSD Expert Streamingを実装", section 技術的な詳細:
 *   - "K-Cache圧縮: 3-bit PolarQuant + 1-bit QJL = 4.25 bits/dim", flow steps 1-5:
 *     L2 norm and normalisation, fast Walsh-Hadamard rotation, 3-bit non-linear
 *     Lloyd-Max code per coordinate, residual, 1-bit signs of a Johnson-Lindenstrauss
 *     projection of the residual (kept so that inner-product scoring stays accurate);
 *   - "V-Cache圧縮: 3-bit PolarQuant = 3.125 bits/dim" (V is not scored, so no QJL);
 *   - "TurboQuant KVキャッシュ圧縮アーキテクチャ" (Lloyd-Max codebook in a native
 *     encode path, dequantisation fused into the attention kernel).
 * The techfi24 article "SwiftLM : serveur d'inférence MLX natif pour Apple Silicon",
 * section "Contexte Technique", names the same pair: polar quantisation plus QJL
 * residual correction.
 *
 * Conventions for every entry point
 *   - Return a tq_status; negative values are errors. Argument checks run on the
 *     host before any HIP call, so a rejected call has enqueued nothing.
 *   - Device work is enqueued asynchronously on `stream` (a hipStream_t, 0 = the
 *     null stream); the call returns before the GPU finishes.
 *   - The caller owns every buffer. The library allocates no device memory, frees
 *     nothing and keeps no mutable global state; calls on different streams that
 *     touch disjoint outputs may run concurrently.
 *   - Device-side contract violations (slot, page id or sequence length out of
 *     range, NaN/Inf inputs) are undefined behaviour.
 *
 * Symbols: d = head_dim, m = d (QJL rows), P = page_size, Hkv = KV heads,
 * Hq = query heads (a multiple of Hkv; query head h reads KV head h / (Hq/Hkv)),
 * Pi = H_d / sqrt(d) (Sylvester Hadamard, natural order), c[0..7] / t[0..6] the
 * ascending codebook levels / thresholds, S the m x d QJL matrix.
 *
 * Packed page format (frozen; one section per (page, KV head), sections stored
 * [n_pages][n_kv_heads], slot = page * P + offset, little-endian words). An
 * offset is split as t = 64*b + 16*tau + 4*k + r (b: 64-token block; tau, k,
 * r = 0..3); per-token fp16 arrays are kept in side order, token t at entry
 * e(t) = 64*b + 16*k + 4*r + tau.
 *   K section, k_page_bytes = P*d/2 + 4*P:
 *     record of token t at byte t*d/2, d/2 bytes: for each coordinate group
 *     s = 0..d/32-1 four u32 words [code bit 0, code bit 1, code bit 2, QJL sign];
 *     bit e of a word belongs to coordinate 32*s + e; sign bit = [ (S r)_l >= 0 ];
 *     N (fp16, ||x||) at byte P*d/2 + 2*e(t); G (fp16, ||r||) at P*d/2 + 2*P + 2*e(t).
 *   V section, v_page_bytes = 3*d*P/8 + 2*P:
 *     code bits as u32 words: bit j of the code of coordinate i = 16*(2*kp + h) + n
 *     (h = 0..1, n = 0..15) of token t is bit 8*r + 4*h + tau of word
 *     b*6d + j*2d + (16*k + n)*(d/32) + kp. So for one block and plane the words
 *     of "lane" 16*k + n are contiguous, and a shift by 4*h plus one AND with
 *     0x01010101 << tau gathers the bits of four tokens into four bytes;
 *     N (fp16) at byte 3*d*P/8 + 2*e(t).
 *   At d = 128 that is 544 bits per K vector (4.25 bits/dim) and 400 bits per V
 *   vector (3.125 bits/dim); at d = 256, 4.125 and 3.0625 bits/dim.
 *   With kb-bit K codes (k_bits 2 or 4) a record has kb + 1 words per group
 *   (kb code planes, then the signs), (kb + 1)*d/8 bytes, and N, G follow at
 *   P*(kb + 1)*d/8; with vb-bit V codes a block holds vb planes, word
 *   b*2*vb*d + j*2d + ..., and N at vb*d*P/8.
 */
#ifndef TQ_H
#define TQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  TQ_OK = 0,
  TQ_EINVAL = -1,       /* null pointer, non-positive or inconsistent size        */
  TQ_EUNSUPPORTED = -2, /* valid request outside what the kernels implement       */
  TQ_EALIGN = -3,       /* pool not 256-byte aligned or I/O not 16-byte aligned    */
  TQ_EWORKSPACE = -4,   /* workspace smaller than *workspace_bytes (size written)  */
  TQ_EHIP = -5,         /* a HIP launch or runtime call failed                     */
  TQ_ESCRATCH = -6      /* the call needs more than TQ_STATIC_SCRATCH_BYTES         */
} tq_status;

typedef enum { TQ_F32 = 0, TQ_BF16 = 1 } tq_dtype;

#define TQ_PAGE_SIZE 256   /* the only page size the kernels implement */
#define TQ_MAX_GROUP 4096  /* max query rows per KV head per sequence (Hq/Hkv * n_q) */
#define TQ_STATIC_SCRATCH_BYTES ((size_t)64 << 20)  /* scratch of tq_append_decode_static */

/* Cache descriptor: plain data, owned by the caller, read by every call. */
typedef struct {
  int32_t head_dim;     /* d: 128 or 256                                         */
  int32_t n_kv_heads;   /* Hkv >= 1                                              */
  int32_t page_size;    /* P: must be TQ_PAGE_SIZE                               */
  int32_t n_pages;      /* pool capacity in pages                                */
  void *k_pool;         /* device, n_pages * Hkv * k_page_bytes, 256-B aligned    */
  void *v_pool;         /* device, n_pages * Hkv * v_page_bytes, 256-B aligned    */
  const float *qjl;     /* device, S as m x d float32 row-major (m = d); may be
                           NULL when k_mse_only = 1                               */
  float levels[8];      /* c[0..7], strictly ascending and odd, c[7-k] = -c[k]
                           (from tq_build_codebook); otherwise calls return
                           TQ_EINVAL                                              */
  float thresholds[7];  /* t[0..6], midpoints, thresholds[3] == 0, strictly
                           ascending (else TQ_EINVAL)                           */
  int32_t k_mse_only;   /* 0: K keeps the QJL stage ("K-Cache圧縮" steps 4-5, the
                           pages' K path). 1: keys without it, the ablation of
                           the pages' reason for QJL (inner-product scoring):
                           the encoder skips z = S r and writes a zero sign
                           plane (codes, N and G as usual; same record size),
                           the decode score keeps only <Pi q, c[code]>, and
                           tq_dequant rejects with_qjl = 1 (TQ_EINVAL). Must
                           match how the records were written. Other values:
                           TQ_EINVAL.                                           */
  int32_t v_bits;       /* V code width. 0 or 3: 3-bit V with levels and
                           thresholds above (the pages' 3.125 bits/dim). 2 or
                           4: V codes of that width with v_levels and
                           v_thresholds, the bit-width variant (2.125 or 4.125
                           bits/dim at d = 128); v_pool sections are then
                           tq_v_page_bytes_bits(d, P, v_bits). Other values:
                           TQ_EINVAL. The K code width is k_bits below.         */
  float v_levels[16];   /* with v_bits 2 or 4: the first 2^v_bits entries,
                           strictly ascending and odd (else TQ_EINVAL)          */
  float v_thresholds[15]; /* with v_bits 2 or 4: the first 2^v_bits - 1,
                           strictly ascending (else TQ_EINVAL)                  */
  int32_t k_bits;       /* K code width. 0 or 3: 3-bit K with levels and
                           thresholds above (the pages' 4.25 bits/dim). 2 or 4:
                           K codes of that width with k_levels and k_thresholds
                           (3.25 or 5.25 bits/dim at d = 128, the QJL signs
                           kept); k_pool sections are then
                           tq_k_page_bytes_bits(d, P, k_bits). Other values:
                           TQ_EINVAL.                                           */
  float k_levels[16];   /* with k_bits 2 or 4: the first 2^k_bits entries,
                           strictly ascending and odd (else TQ_EINVAL)          */
  float k_thresholds[15]; /* with k_bits 2 or 4: the first 2^k_bits - 1,
                           strictly ascending (else TQ_EINVAL)                  */
} tq_cache;

/* Bytes of one (page, KV head) section; 0 for unsupported d or P. */
size_t tq_k_page_bytes(int32_t head_dim, int32_t page_size);
size_t tq_v_page_bytes(int32_t head_dim, int32_t page_size);
/* V section for codes of `bits` bits (2, 3 or 4; 0 otherwise): bits planes of
 * d x P bits, then the fp16 norms. */
size_t tq_v_page_bytes_bits(int32_t head_dim, int32_t page_size, int32_t bits);
/* K section for codes of `bits` bits (2, 3 or 4; 0 otherwise): per token
 * (bits + 1) * d / 8 bytes (bits code planes and the sign plane per 32
 * coordinates), then the fp16 N and G arrays. */
size_t tq_k_page_bytes_bits(int32_t head_dim, int32_t page_size, int32_t bits);

/*
 * Lloyd-Max codebook and QJL matrix ("TurboQuant KVキャッシュ圧縮アーキテクチャ",
 * item 1; "K-Cache圧縮" steps 3 and 5). Host only, no GPU needed.
 *   levels[n], thresholds[n-1] (host out), n = 2^bits: the n-level MSE quantiser
 *     of N(0, 1/d), found by Lloyd iteration in float64 from the Gaussian
 *     quantiles sigma*Phi^-1((k+1/2)/n) until no level moves by 1e-14*sigma,
 *     symmetrised, thresholds at midpoints, then rounded to float32. bits = 3
 *     is the pages' codebook (K and V); 2 and 4 serve the K and V bit-width
 *     variants (tq_cache.k_bits, v_bits).
 *   qjl_host (host out, d*d floats, may be NULL): S[l][i] row-major; SplitMix64
 *     seeded with qjl_seed gives pairs (x1, x2) -> u = ((x>>11)+1)*2^-53, Box-Muller
 *     sqrt(-2 ln u1) cos(2 pi u2) then sin(...), filled in order, rounded to float32.
 *     The caller uploads it and points tq_cache.qjl at the device copy.
 * Errors: TQ_EINVAL (null levels/thresholds, head_dim < 2 or not a power of two),
 * TQ_EUNSUPPORTED (bits not 2, 3 or 4).
 */
int tq_build_codebook(int32_t head_dim, int32_t bits, uint64_t qjl_seed,
                      float *levels, float *thresholds, float *qjl_host);

/*
 * tq_build_codebook with the codebook fitted to the exact law of one coordinate
 * of a uniform unit vector in R^d, density proportional to (1 - x^2)^((d-3)/2)
 * on (-1, 1), instead of its large-d limit N(0, 1/d). The pages' "V3" line
 * ("TurboQuant KVキャッシュ圧縮アーキテクチャ") carries a Lloyd-Max codebook over the
 * rotated unit vector's coordinates without naming the density; this is the
 * density that the normalise-then-rotate steps produce for isotropic inputs.
 * Lloyd iteration in float64 from the N(0, 1/d) levels until no level moves by
 * 1e-14 of the largest, cell masses by Gauss-Legendre quadrature in u = asin x,
 * first moments in closed form; symmetrised, midpoint thresholds, rounded to
 * float32. The codebook is odd, as the kernels require. qjl_host as above.
 * Errors: TQ_EINVAL (null levels/thresholds, head_dim < 4 or not a power of
 * two), TQ_EUNSUPPORTED (bits not 2, 3 or 4).
 */
int tq_build_codebook_sphere(int32_t head_dim, int32_t bits, uint64_t qjl_seed,
                             float *levels, float *thresholds, float *qjl_host);

/*
 * K encode ("K-Cache圧縮" flow steps 1-5): for each token i and KV head h,
 * x = k[i][h][:] (float32 or bfloat16, [n_tokens][Hkv][d] row-major, 16-B aligned):
 * n = ||x||, x_hat = x/n (0 if n = 0), y = Pi x_hat, code_j = #{k: t_k <= y_j},
 * r = y - c[code], z = S r; writes the K record, N = fp16(n), G = fp16(||r||) at
 * slot slots[i] (device int32 [n_tokens]) of head h. Only the addressed records
 * change. n_tokens == 0 is a no-op. The codes have tq_cache.k_bits bits (3 by
 * default); with k_mse_only the QJL stage is skipped (see tq_cache).
 * Errors: TQ_EINVAL, TQ_EUNSUPPORTED (d, P, dtype), TQ_EALIGN, TQ_EHIP.
 */
int tq_encode_k(const tq_cache *c, const void *k, int32_t dtype,
                const int32_t *slots, int32_t n_tokens, void *stream);

/*
 * V encode ("V-Cache圧縮"): steps 1-3 of the K flow, then the V record and
 * N = fp16(n). The codes have tq_cache.v_bits bits (3 by default, with the K
 * codebook; 2 or 4 with v_levels / v_thresholds). Bits of other tokens sharing
 * the same V rows are preserved (whole aligned 64-token blocks are written
 * whole, other tokens bit by bit with atomics). Same arguments and errors as
 * tq_encode_k.
 */
int tq_encode_v(const tq_cache *c, const void *v, int32_t dtype,
                const int32_t *slots, int32_t n_tokens, void *stream);

/*
 * Query preparation (the query is rotated once per step instead of each key
 * being dequantised) for one decode call over q [batch][n_q][n_q_heads][d]
 * (float32 or bfloat16, 16-B aligned). Writes into `prep` (device, 256-B
 * aligned, *prep_bytes bytes):
 *   [rows][2][d] float32 with rows in (b, t, h) order: Pi q, then S Pi q;
 *   then, when Hq/Hkv * n_q <= TQ_MAX_GROUP, the packed scoring operand
 *   (fp6 query limbs with block scales) of each (sequence, KV head, group of
 *   4 query rows) used by the MFMA decode kernel (internal layout).
 * prep == NULL returns the size in *prep_bytes and launches nothing; a short
 * buffer returns TQ_EWORKSPACE with the size written back.
 * Errors: TQ_EINVAL, TQ_EUNSUPPORTED, TQ_EALIGN, TQ_EWORKSPACE, TQ_EHIP.
 */
int tq_query_prepare(const tq_cache *c, const void *q, int32_t dtype, int32_t batch,
                     int32_t n_q, int32_t n_q_heads, void *prep, size_t *prep_bytes,
                     void *stream);

/*
 * Decode attention over the packed cache, dequantisation fused in
 * ("TurboQuant KVキャッシュ圧縮アーキテクチャ" item 2; "K-Cache圧縮", reason for QJL).
 * For query row (b, t, h) of q [batch][n_q][Hq][d], KV head kv = h / (Hq/Hkv) and
 * visible tokens j < L_b = seq_lens[b] (causal_tail = 0) or
 * j < L_b - (n_q - 1 - t) (causal_tail = 1):
 *   score_j = scale * N_j * (<Pi q, c[code_j]> + sqrt(pi/2)/m * G_j * <S Pi q, sigma_j>)
 *   w = softmax(score),  out = Pi( sum_j w_j N^V_j c[codeV_j] )   (float32)
 * Token j of sequence b lives at slot block_table[b][j / P] * P + j % P
 * (block_table: device int32 [batch][max_pages]). The entries of the first
 * ceil(L_b / P) pages must lie in [0, n_pages) (device data, not checked);
 * later entries are never read, and tokens past max_pages * P are not seen.
 * L_b <= 0 or an empty visible range gives a zero row. Hq / Hkv * n_q must not
 * exceed TQ_MAX_GROUP, and batch * W must not exceed 65535 (TQ_EUNSUPPORTED),
 * with rows = Hq / Hkv * n_q and W the workgroups per sequence and KV head:
 * ceil(rows / 16) with 16 rows or more and 3-bit K and V codes, else
 * ceil(ceil(rows / 4) / k) with k = 2 at d = 128 when rows > 4, else 1.
 * Workspace: call with workspace == NULL to get the size in *workspace_bytes
 * (nothing is launched). It holds split partials and the prepared queries; its
 * contents need no initialisation and are scratch after the call. Calls that
 * share a workspace must not overlap. A workspace smaller than needed returns
 * TQ_EWORKSPACE with the size written back. Two kernels are enqueued after the
 * query preparation: the split-K pass and a small merge.
 * Errors: TQ_EINVAL, TQ_EUNSUPPORTED, TQ_EALIGN, TQ_EWORKSPACE, TQ_EHIP.
 */
int tq_attn_decode(const tq_cache *c, const void *q, int32_t dtype,
                   int32_t batch, int32_t n_q, int32_t n_q_heads,
                   const int32_t *block_table, int32_t max_pages,
                   const int32_t *seq_lens, int32_t causal_tail, float scale,
                   float *out, void *workspace, size_t *workspace_bytes, void *stream);

/*
 * tq_attn_decode with a window: in sequence b only tokens
 * seq_starts[b] <= j < (the tq_attn_decode bound) are visible, so a sliding-
 * window layer attends to its last W tokens with seq_starts[b] = max(0, L_b - W).
 * Pages wholly before seq_starts[b] are never read: their block-table entries
 * may name pages that were recycled for newer tokens (a ring of pages). A row
 * with no visible token is all zero. seq_starts: device int32 [batch], not null
 * (TQ_EINVAL), 4-byte aligned (TQ_EALIGN); a negative start counts as 0.
 * Everything else, including the workspace, is as tq_attn_decode.
 * Source: the agentlenshq SharpAI/SwiftLM project page (Japanese), section
 * それは何か, names sliding-window layers (a window-boundary bug) but defines no
 * mechanics; the per-sequence first visible token is this library's reading.
 */
int tq_attn_decode_window(const tq_cache *c, const void *q, int32_t dtype,
                          int32_t batch, int32_t n_q, int32_t n_q_heads,
                          const int32_t *block_table, int32_t max_pages,
                          const int32_t *seq_lens, const int32_t *seq_starts,
                          int32_t causal_tail, float scale, float *out,
                          void *workspace, size_t *workspace_bytes, void *stream);

/*
 * One decode step with an append: encode n_new new K and V vectors
 * ([n_new][Hkv][d], kv_dtype) into `slots` exactly as tq_encode_k and
 * tq_encode_v do, then run tq_attn_decode over the updated cache (seq_lens
 * must already count the new tokens). The same workspace as tq_attn_decode.
 * Short appends (n_new * Hkv < 4096) with q_dtype == kv_dtype encode and
 * prepare the query in a single launch; otherwise the separate kernels run in
 * order. n_new = 0 is a plain decode.
 * Same passages as tq_encode_k / tq_encode_v and tq_attn_decode. Errors: as
 * tq_encode_k and tq_attn_decode (TQ_EINVAL for null k_new / v_new / slots
 * with n_new > 0).
 */
int tq_append_decode(const tq_cache *c, const void *k_new, const void *v_new, int32_t kv_dtype,
                     const int32_t *slots, int32_t n_new, const void *q, int32_t q_dtype,
                     int32_t batch, int32_t n_q, int32_t n_q_heads, const int32_t *block_table,
                     int32_t max_pages, const int32_t *seq_lens, int32_t causal_tail, float scale,
                     float *out, void *workspace, size_t *workspace_bytes, void *stream);

/*
 * tq_append_decode without a workspace argument, for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation. The split partials and prepared queries
 * live in a static device buffer of TQ_STATIC_SCRATCH_BYTES (64 MiB) that the
 * library holds on every GPU it runs on until the process ends; the call itself
 * allocates and frees nothing. The first call on a device (with that device
 * current, as for every call) looks the buffer up once. A call whose workspace
 * (the size tq_append_decode reports for the same arguments) exceeds
 * TQ_STATIC_SCRATCH_BYTES returns TQ_ESCRATCH and launches nothing. The buffer
 * holds decode and verify steps with a few query rows per KV head (for example
 * 32 sequences of up to 16K tokens, or 4 sequences of 128K tokens at d = 256
 * with 16 query rows per KV head); chunked prefill with hundreds of query rows
 * per KV head needs the caller workspace of tq_append_decode.
 * The buffer needs no initialisation and is scratch after the call. Every call
 * on one GPU shares that GPU's buffer: calls that may overlap in time on one GPU
 * (unordered streams, other host threads) race on it, so the caller must order
 * them (one stream, or events). Arguments, results and other errors are those
 * of tq_append_decode.
 */
int tq_append_decode_static(const tq_cache *c, const void *k_new, const void *v_new,
                            int32_t kv_dtype, const int32_t *slots, int32_t n_new, const void *q,
                            int32_t q_dtype, int32_t batch, int32_t n_q, int32_t n_q_heads,
                            const int32_t *block_table, int32_t max_pages, const int32_t *seq_lens,
                            int32_t causal_tail, float scale, float *out, void *stream);

/*
 * The attention part of tq_attn_decode alone (one kernel launch), on queries
 * already prepared by tq_query_prepare with the same batch, n_q and n_q_heads.
 * Same semantics, workspace rules and errors; its workspace is smaller (no
 * query region).
 */
int tq_attn_decode_prepared(const tq_cache *c, const void *prep,
                            int32_t batch, int32_t n_q, int32_t n_q_heads,
                            const int32_t *block_table, int32_t max_pages,
                            const int32_t *seq_lens, int32_t causal_tail, float scale,
                            float *out, void *workspace, size_t *workspace_bytes,
                            void *stream);

/*
 * The two launches of tq_attn_decode_prepared, for callers that overlap or time
 * them separately. tq_attn_decode_split runs the split-K pass (one kernel) and
 * leaves per-split partials (running max, softmax sum, V numerator) in the
 * workspace; tq_attn_decode_merge (one small kernel) combines them by
 * log-sum-exp, applies the inverse rotation and writes `out`. Both must be called
 * with the same batch, n_q, n_q_heads and max_pages (the split plan is a
 * function of these and of the cache shape) and the same workspace, on the
 * same stream. Workspace rules and errors as for tq_attn_decode_prepared.
 */
int tq_attn_decode_split(const tq_cache *c, const void *prep,
                         int32_t batch, int32_t n_q, int32_t n_q_heads,
                         const int32_t *block_table, int32_t max_pages,
                         const int32_t *seq_lens, int32_t causal_tail, float scale,
                         void *workspace, size_t *workspace_bytes, void *stream);
int tq_attn_decode_merge(const tq_cache *c, int32_t batch, int32_t n_q, int32_t n_q_heads,
                         int32_t max_pages, float *out, const void *workspace,
                         size_t workspace_bytes, void *stream);

/*
 * Uncompressed baseline: decode attention over dense bf16 K and V
 * ([batch][Hkv][max_len][d], d = head_dim), softmax(q K^T * scale) V, with the
 * same split-K scheme and merge as tq_attn_decode. It exists to measure the
 * compressed path against; it is not part of the compressed cache.
 * q: [batch][n_q][Hq][d] fp32/bf16; every query sees seq_lens[b] tokens;
 * out: [batch][n_q][Hq][d] fp32. At most 4 query rows per KV head
 * (Hq/Hkv * n_q <= 4), else TQ_EUNSUPPORTED. Workspace as tq_attn_decode
 * (workspace == NULL: size query). Errors: TQ_EINVAL (null pointer or bad size),
 * TQ_EALIGN (k, v, q, out not 16-byte or workspace not 256-byte aligned).
 */
int tq_dense_attn_decode(const void *k, const void *v, int32_t head_dim, int32_t n_kv_heads,
                         int32_t max_len, const void *q, int32_t q_dtype, int32_t batch,
                         int32_t n_q, int32_t n_q_heads, const int32_t *seq_lens, float scale,
                         float *out, void *workspace, size_t *workspace_bytes, void *stream);

/*
 * Dequantise records back to the original domain (float32 [n_tokens][Hkv][d]):
 *   which = 0 (K): N * Pi(c[code] + sqrt(pi/2)/m * G * S^T sigma)  (with_qjl = 1)
 *                  N * Pi c[code]                                    (with_qjl = 0)
 *   which = 1 (V): N * Pi c_V[code]   (the V codebook and code width)
 * so that <q, K_tilde_j> equals the attention score estimate of token j.
 * Errors: TQ_EINVAL, TQ_EUNSUPPORTED, TQ_EALIGN, TQ_EHIP.
 */
int tq_dequant(const tq_cache *c, int32_t which, int32_t with_qjl,
               const int32_t *slots, int32_t n_tokens, float *out, void *stream);

/* Static description of a status code. */
const char *tq_status_string(int32_t status);

#ifdef __cplusplus
}
#endif

#endif /* TQ_H */
