/*
 * mla_latent.h -- C ABI of the absorbed Multi-head Latent Attention decode
 * library for MI355X (gfx950).
 *
 * Pages this interface follows:
 *  [T] "Multi-Head Latent Attention: How DeepSeek Compressed the Cache
 *      Further" (MLA tutorial page), sections "Learn a Smaller Shared
 *      Representation", "Move the Key Projection Into the Query", "Move the
 *      Value Expansion After the Weighted Sum", "Position Rotations
 *      Complicate the Absorption", "Count the Cache That Is Actually Stored".
 *  [R] "RedKnot-MLA: Multi-Head Offline-Online Reuse for DeepSeek-V4
 *      Long-Context Serving" (abstract): documents cached at canonical
 *      position zero, query-side RoPE relocation, offline and online paths
 *      merged before one shared output projection, the packed latent never
 *      split.
 *
 * One decode step of one attention layer is five calls:
 *   rope_relocate_q  -> q_rot      (per KV segment: rotary query at pos - shift)
 *   mla_absorb_q     -> q_lat      (U_K^T q_nope, once per query)
 *   mla_decode_splitkv -> partial (o_lat, lse) states per KV split / segment
 *   mla_combine_lse  -> o_lat, lse (log-sum-exp merge of the partial states)
 *   mla_out_uv       -> out        (U_V o_lat, once per query)
 *   mla_out_proj     -> layer out  (the shared output projection W_O over all heads)
 * mla_prepare_q runs the first two in one launch (all segment shifts at once);
 * mla_combine_out_uv runs the combine and U_V in one launch (few query tokens).
 *
 * Conventions shared by every call
 *  - All tensor pointers are DEVICE pointers (HIP device memory), row-major,
 *    densely packed in the shapes stated.  The caller allocates and owns every
 *    buffer; the library never allocates device memory, never creates
 *    streams and never synchronises the host.
 *  - `stream` is a hipStream_t passed as void* (NULL = the null stream).  All
 *    work is enqueued on it, asynchronously; results are ready once the
 *    stream has reached that point.
 *  - dtype arguments are MLA_BF16 (bf16 storage) or MLA_F32; arithmetic and
 *    accumulation are fp32 throughout.  The bf16-cache decode requires
 *    d_c = 512, d_rope = 64; the fp32-cache decode takes any d_c <= 512,
 *    d_rope <= 128.
 *  - Inputs and outputs must not alias.  Outputs are overwritten, never
 *    accumulated into.
 *  - Arguments are validated on the host before anything is enqueued.  On a
 *    bad argument the call returns a nonzero mla_status, enqueues nothing and
 *    records a message readable through mla_last_error() (per thread).  A
 *    launch failure returns MLA_ERR_HIP.
 *  - Numerics: log-sum-exp values are natural logarithms of
 *    sum_t exp(scaled score); a query row with no visible key has lse = -inf
 *    and output 0.  Rows a request may not see never enter any arithmetic.
 */
#ifndef MLA_LATENT_H
#define MLA_LATENT_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MLA_OK = 0,
  MLA_ERR_NULL = 1,        /* a required pointer is NULL */
  MLA_ERR_SHAPE = 2,       /* a size is out of range or sizes disagree */
  MLA_ERR_DTYPE = 3,       /* unknown dtype */
  MLA_ERR_ALIGN = 4,       /* a pointer is not 16-byte aligned */
  MLA_ERR_UNSUPPORTED = 5, /* valid request the library does not implement */
  MLA_ERR_WORKSPACE = 6,   /* reserved */
  MLA_ERR_HIP = 7          /* the HIP runtime reported an error */
} mla_status;

/* MLA_I8 and MLA_I4 are cache formats only (mla_decode_splitkv's cache_dtype).
 * MLA_I8: rows of d_c int8 latent codes followed by d_rope bf16 rotary entries
 * (d_c + 2 d_rope bytes), one fp32 scale per row in mla_segment.row_scale; see
 * mla_quantize_latent_i8.  MLA_I4: rows of d_c / 2 bytes of 4-bit latent codes
 * followed by d_rope / 2 bytes of 4-bit rotary codes, two fp32 scales per row
 * (latent, rotary) in mla_segment.row_scale; see mla_quantize_latent_i4. */
/* MLA_BF16X2 is a query format only (mla_prepare_q's lat_dtype,
 * mla_decode_splitkv's q_dtype): each fp32 value x held as two bf16 parts,
 * hi = bf16(x) and lo = bf16(x - hi) (round to nearest), the d values of a
 * row stored as a hi plane then a lo plane ([..][2][d] bf16, 4 bytes per
 * value like fp32).  The decode reads only the hi plane while streaming the
 * cache and only the lo plane at the end of each piece: half the query bytes
 * of an fp32 query each time. */
typedef enum { MLA_F32 = 0, MLA_BF16 = 1, MLA_I8 = 2, MLA_I4 = 3, MLA_BF16X2 = 4 } mla_dtype;

/*
 * rope_relocate_q -- rotary query for one KV segment.
 * [T] "Position Rotations Complicate the Absorption": the score has a separate
 * position part q^R . k^R_t computed on rotated feature pairs.  [R]: a segment
 * cached at canonical position zero is read by rotating the query by
 * (true position - shift) instead of re-rotating the cached keys.
 *
 *   q_rot[t][h][2i:2i+2] = Rot((pos[t] - shift[t]) * base^(-2i/d_rope)) q_pe[t][h][2i:2i+2]
 *   with Rot(a) = [[cos a, -sin a], [sin a, cos a]] (adjacent pairs).
 *
 * q_pe   [n_tok][n_heads][d_rope]  input, in_dtype, unrotated
 * q_rot  [n_tok][n_heads][d_rope]  output, out_dtype (fp32 keeps the rotated
 *                                  query exact to ~1e-7 for the decode call)
 * pos    [n_tok] int64             true position of each query token
 * shift  [n_tok] int64 or NULL     stored-to-true position shift of the
 *                                  segment for that token's request (NULL = 0)
 * The position difference is taken in int64 and the angle in fp64.
 * d_rope must be even, 2..128.
 */
mla_status rope_relocate_q(const void* q_pe, int in_dtype, void* q_rot, int out_dtype,
                           const int64_t* pos, const int64_t* shift, int n_tok, int n_heads,
                           int d_rope, double base, void* stream);

/*
 * mla_absorb_q -- fold the key up-projection into the query.
 * [T] "Move the Key Projection Into the Query": q^T (U_K c_t) = (U_K^T q)^T c_t,
 * so the new query is transformed once and compared with the stored latents.
 *
 *   q_lat[t][h][j] = sum_i w_uk[h][i][j] * q_nope[t][h][i]
 *
 * q_nope [n_tok][n_heads][d_nope]  input, in_dtype
 * w_uk   [n_heads][d_nope][d_c]    U_K of each head (maps d_c -> d_nope), in_dtype
 * q_lat  [n_tok][n_heads][d_c]     output, out_dtype (fp32 accumulation; an fp32
 *                                  q_lat keeps the decode scores exact to ~1e-6,
 *                                  a bf16 one costs ~1e-3 in the scores)
 */
mla_status mla_absorb_q(const void* q_nope, const void* w_uk, int in_dtype, void* q_lat,
                        int out_dtype, int n_tok, int n_heads, int d_nope, int d_c, void* stream);

/*
 * One KV segment read by mla_decode_splitkv.  Host struct holding device
 * pointers.  A cache row is [c_t | k^R_t] (d_c + d_rope numbers, [T] "Count
 * the Cache That Is Actually Stored"); rows are read whole, never split ([R]).
 */
typedef struct {
  const void* cache;          /* contiguous: [batch][max_rows][d_c+d_rope];
                                 paged: pool [n_pages][page_size][d_c+d_rope] */
  const int32_t* block_table; /* paged: [batch][max_pages] physical page ids
                                 (entries past a request's pages are ignored);
                                 NULL => contiguous layout */
  const int32_t* seq_lens;    /* [batch] valid rows T_b of each request, 0..max rows */
  const void* q_rot;          /* [n_tok][n_heads][d_rope] rotary query for THIS segment
                                 (output of rope_relocate_q with the segment's shift) */
  int64_t max_rows;           /* contiguous: rows allocated per request (>= every T_b) */
  int page_size;              /* paged: rows per page (the bf16 path takes 64) */
  int max_pages;              /* paged: entries per block-table row */
  int n_pages;                /* paged: pages in the pool (ids must be < n_pages) */
  int head_begin;             /* heads [head_begin, head_begin+head_count) read it */
  int head_count;
  int causal;                 /* 0: every row visible; 1: query s of s_q sees
                                 rows t <= T_b - s_q + s */
  int part_begin;             /* this segment writes partial slots */
  int n_split;                /* [part_begin, part_begin + n_split) of its rows */
  const float* row_rinv;      /* QK-Norm: per stored row, the inverse RMS of its content
                                 key (mla_qknorm_key_rinv), indexed like the cache rows
                                 ([batch][max_rows] or [n_pages][page_size]); the
                                 latent part of each score is multiplied by it.
                                 NULL => no QK-Norm.  Given for every segment
                                 of a call or for none (else
                                 MLA_ERR_UNSUPPORTED); needs an fp32 or split
                                 query and a 16-bit cache */
  const float* row_scale;     /* int8 cache (cache_dtype MLA_I8): per stored row the
                                 scale of its latent codes (mla_quantize_latent_i8),
                                 indexed like row_rinv; the latent is scale * code.
                                 int4 cache (MLA_I4): per stored row the pair
                                 (latent scale, rotary scale) (mla_quantize_latent_i4),
                                 8-byte aligned.  Must be NULL for 16-bit and fp32
                                 caches */
} mla_segment;

/*
 * mla_decode_splitkv -- the latent-cache attention pass.
 * [T] "Move the Key Projection Into the Query" (score against the stored
 * latent), "Position Rotations Complicate the Absorption" (content + position
 * score, scaled, masked, softmaxed), "Move the Value Expansion After the
 * Weighted Sum" (mix the latents, expand later).  [R]: separate KV segments
 * give partial states merged later by mla_combine_lse.
 *
 * For every segment g, request b, query token s, head h in g's range, and each
 * KV split j of g's rows of request b:
 *   s_t   = scale * (q_lat[t][h] . c_t + q_rot_g[t][h] . k^R_t)     (t visible rows of split j)
 *   o_part[tok][h][part_begin_g + j][:] = sum_t softmax_j(s)_t c_t   (fp32, normalised in the split)
 *   lse_part[tok][h][part_begin_g + j]  = ln sum_t exp(s_t)          (-inf if the split is empty)
 * where tok = b * s_q + s.  The library chooses the split boundaries (balanced
 * over the grid) subject to at most n_split splits per request; every slot of
 * [part_begin, part_begin + n_split) of every (tok, h in range) gets its lse
 * written, and its o_part row too when the lse is finite.  Across segments the
 * slot ranges of each head must tile [0, n_part) exactly.
 *
 * q_lat    [n_tok][n_heads][d_c]                 q_dtype, from mla_absorb_q /
 *          mla_prepare_q; each segment's q_rot has q_dtype too (fp32 for
 *          MLA_BF16X2).  MLA_BF16X2: [n_tok][n_heads][2][d_c] bf16 hi and lo
 *          planes (mla_prepare_q with lat_dtype MLA_BF16X2), for a bf16 cache
 *          (with or without QK-Norm) or a low-bit one; always the row-owning kernel; the
 *          same arithmetic as an fp32 query (which is split into exactly
 *          these parts inside the kernel).
 * caches   cache_dtype.  MLA_BF16 caches take an fp32 query or a bf16 one.
 *          An fp32 query is split into bf16 hi + lo parts: groups of up to
 *          32 query rows multiply both parts; 64-row groups multiply lo
 *          only on the rotary dims and add the latent lo part's share to
 *          the lse to first order (scale * lo . o_part; lse error second
 *          order, ~1e-5 at unit-variance inputs; with QK-Norm row factors
 *          the share is scale * rbar * lo . o_part, rbar the softmax-weighted
 *          mean factor of the piece, whose error is the weighted covariance
 *          of the factors and the lo scores, again second order).  MLA_F32 caches take an
 *          fp32 query.  MLA_I8 caches (QuantMLA abstract: a low-bit latent
 *          cache dequantized inside attention) take an fp32 or split query
 *          and every segment's row_scale: the latent score of row t is
 *          scale_t times q_lat . code_t and its softmax weight multiplies
 *          scale_t code_t, exactly the attention over the dequantized rows;
 *          not combined with QK-Norm; they run on the row-owning kernel in
 *          groups of 64 query rows, the codes unpacked inside the streaming
 *          loop.  MLA_I4 caches (the abstract's joint INT4
 *          content and rotary caches) take an fp32 or split query and every
 *          segment's (latent, rotary) scale pairs: the score of row t is
 *          scale * (sc_t q_lat . code_t + sr_t q_rot . rcode_t) and its
 *          weight multiplies sc_t code_t, the attention over the
 *          dequantized rows; they run on the row-owning kernel in groups of
 *          64 query rows, the codes unpacked inside the streaming loop.
 * o_part   [n_tok][n_heads][n_part][d_c] part_dtype  output: fp32, or bf16 (the
 *          normalised partial rounded to nearest; half the bytes to write
 *          and to merge, relative error 2^-9 per entry; fp32 caches write
 *          fp32 partials only)
 * lse_part [n_tok][n_heads][n_part]      fp32    output
 * n_tok = batch * s_q.  n_wg = workgroups per launch (0 = one per compute unit,
 * at most 65536).  With an fp32 query and a bf16 cache, segments of more than
 * 32 query rows, and every segment of a call with several, run on the
 * row-owning kernel (groups of 64 or 128 rows, 16 or 32 per wave): the
 * segments of a call share one launch (up to 8 per launch), each taking a
 * part of the n_wg workgroups proportional to row groups x batch x its row
 * capacity.  Other segments get n_wg workgroups each, one launch per segment.
 * bf16 and int8 paths: d_c = 512, d_rope = 64, page_size = 64, s_q * head_count <= 4096
 * (multi-token chunks: the rows form groups, each streaming the rows).
 */
mla_status mla_decode_splitkv(const mla_segment* segs, int n_segs, const void* q_lat, int q_dtype,
                              int cache_dtype, int batch, int s_q, int n_heads, int d_c, int d_rope,
                              float scale, void* o_part, int part_dtype, float* lse_part, int n_part, int n_wg,
                              void* stream);

/*
 * mla_combine_lse -- merge partial attention states by log-sum-exp.
 * [R]: the offline and online paths are merged before one shared output
 * projection.  For every row r (a (token, head) pair):
 *   lse[r]   = ln sum_j exp(lse_part[r][j])      (slots with -inf skipped)
 *   o_lat[r] = sum_j exp(lse_part[r][j] - lse[r]) o_part[r][j]
 * A row whose slots are all -inf gives o_lat = 0, lse = -inf.  o_part rows of
 * -inf slots are never read.
 *
 * o_part   [n_rows][n_part][d_c] part_dtype (fp32 or bf16; 16-byte aligned, d_c a
 *          multiple of 4; n_rows < 2^24)
 * lse_part [n_rows][n_part]      fp32 (n_part <= 1024)
 * o_lat    [n_rows][d_c]         out_dtype (MLA_BF16 or MLA_F32)
 * lse      [n_rows]              fp32, or NULL if not wanted
 * The sums are taken in fp32 whatever the partials' storage.
 */
mla_status mla_combine_lse(const void* o_part, int part_dtype, const float* lse_part, int n_rows, int n_part,
                           int d_c, void* o_lat, int out_dtype, float* lse, void* stream);

/*
 * mla_prepare_q -- rope_relocate_q for n_shift segment shifts and
 * mla_absorb_q, fused into one launch where the absorption runs on its MFMA
 * path (in_dtype bf16, d_nope 128, d_c 512, 16-byte aligned q_nope / w_uk / q_lat);
 * other shapes run the two kernels one after the other.  Same arithmetic and
 * layouts as those two calls ([T] "Move the Key Projection Into the Query",
 * "Position Rotations Complicate the Absorption"; [R] query-side relocation):
 *
 *   q_lat     = mla_absorb_q(q_nope, w_uk)                 (lat_dtype)
 *   q_rots[k] = rope_relocate_q(q_pe, pos, shifts[k])      (rot_dtype), k < n_shift
 *
 * q_nope, w_uk, q_lat, q_pe, pos: as in mla_absorb_q / rope_relocate_q (lat_dtype
 * may also be MLA_BF16X2 on the MFMA path: the fp32 result written as its
 * bf16 hi and lo planes, [n_tok][n_heads][2][d_c]); q_pe
 * and w_uk have in_dtype, q_nope has q_dtype: either in_dtype, or MLA_F32
 * with bf16 weights on the MFMA path (an fp32 query, e.g. the output of
 * mla_qknorm_query, enters as bf16 hi + lo parts with fp32 accumulation;
 * other shapes return MLA_ERR_UNSUPPORTED).  q_rots: host array of n_shift
 * device pointers [n_tok][n_heads][d_rope]; shifts: host array of n_shift
 * device pointers ([n_tok] int64, an entry may be NULL = no shift) or NULL for
 * all zero.  n_shift 0..8.  A small decode batch spends most of these two
 * kernels in launch latency, so one launch instead of 1 + n_shift shortens
 * the step.
 */
mla_status mla_prepare_q(const void* q_nope, int q_dtype, const void* q_pe, const void* w_uk, int in_dtype,
                         void* q_lat, int lat_dtype, void* const* q_rots, const int64_t* const* shifts, int n_shift,
                         int rot_dtype, const int64_t* pos, int n_tok, int n_heads, int d_nope, int d_rope, int d_c,
                         double base, void* stream);

/*
 * mla_prepare_q_qknorm -- mla_qknorm_query folded into mla_prepare_q's one
 * launch (QK-Norm MLA page, abstract: RMSNorm of the content query after its
 * projection; the static key weight moved into the query).  Result, layouts
 * and rotary outputs as mla_qknorm_query followed by mla_prepare_q with
 * q_dtype MLA_F32:
 *
 *   q_lat     = U_K^T (g_q g_k q_nope / rms_t),   rms_t = sqrt(mean_{h,i} q_nope[t][h][i]^2 + eps)
 *   q_rots[k] = rope_relocate_q(q_pe, pos, shifts[k])
 *
 * Every absorption workgroup sums the squares of all heads of its tokens
 * itself, so the call is meant for decode batches: n_tok * n_heads <= 512.
 * q_nope [n_tok][n_heads][128] q_dtype (MLA_BF16 or MLA_F32, 16-byte
 * aligned); g_q, g_k [n_heads][128] fp32; w_uk [n_heads][128][512] bf16
 * (16-byte aligned), in_dtype MLA_BF16 (also the dtype of q_pe); eps >= 0
 * (eps = 0 and an all-zero token: that token's q_lat is not finite).
 * The fp32 product enters the MFMA as bf16 hi + lo parts with fp32
 * accumulation.  Other arguments as mla_prepare_q.
 * Errors: MLA_ERR_NULL, MLA_ERR_DTYPE, MLA_ERR_SHAPE, MLA_ERR_UNSUPPORTED
 * (other dims, dtypes or alignment, or n_tok * n_heads > 512: use
 * mla_qknorm_query, then mla_prepare_q).
 */
mla_status mla_prepare_q_qknorm(const void* q_nope, int q_dtype, const float* g_q, const float* g_k, float eps,
                                const void* q_pe, const void* w_uk, int in_dtype, void* q_lat, int lat_dtype,
                                void* const* q_rots, const int64_t* const* shifts, int n_shift, int rot_dtype,
                                const int64_t* pos, int n_tok, int n_heads, int d_nope, int d_rope, int d_c,
                                double base, void* stream);

/*
 * mla_out_uv -- expand the mixed latent once per query.
 * [T] "Move the Value Expansion After the Weighted Sum": U_V (sum_t a_t c_t)
 * equals sum_t a_t (U_V c_t), so the value up-projection follows the sum.
 *
 *   out[t][h][i] = sum_j w_uv[h][i][j] * o_lat[t][h][j]
 *
 * o_lat [n_tok][n_heads][d_c]   o_dtype
 * w_uv  [n_heads][d_v][d_c]     U_V of each head (maps d_c -> d_v), w_dtype
 * out   [n_tok][n_heads][d_v]   out_dtype (fp32 accumulation)
 */
mla_status mla_out_uv(const void* o_lat, int o_dtype, const void* w_uv, int w_dtype, void* out,
                      int out_dtype, int n_tok, int n_heads, int d_c, int d_v, void* stream);

/*
 * mla_out_proj -- the shared output projection W_O over the heads' outputs.
 * [T] "Move the Value Expansion After the Weighted Sum" (its closing remark:
 * the value up-projection combines with each head's contribution to the
 * final output projection); [R]: the merged state of the two paths goes
 * through one shared output projection.
 *
 *   out[t][n] = sum_k x[t][k] * w_o[n][k]         (fp32 accumulation)
 *
 * x     [n_tok][k_in]     x_dtype: the heads' outputs back to back, i.e.
 *                         mla_out_uv's out viewed as [n_tok][n_heads * d_v]
 *                         (k = h * d_v + i)
 * w_o   [d_model][k_in]   w_dtype: row n = output feature n; head h owns
 *                         columns h * d_v .. h * d_v + d_v - 1
 * out   [n_tok][d_model]  out_dtype
 * The folded form takes x = o_lat viewed as [n_tok][n_heads * d_c] and, as
 * w_o, the per-head products W_O[:, head h] U_V[h] side by side
 * ([d_model][n_heads * d_c]); it reads more weight bytes than mla_out_uv
 * followed by this call whenever d_c > d_v.
 * bf16 x and w_o with k_in a multiple of 256 and both 16-byte aligned run on
 * MFMA (each W_O row is read once per 64 tokens); any other case runs a
 * plain fp32 kernel.  d_model is the layer's model width, a parameter.
 * Shapes: n_tok <= 2^20, 1 <= k_in <= 2^20, 1 <= d_model <= 2^20.
 * Errors: MLA_ERR_NULL, MLA_ERR_DTYPE, MLA_ERR_SHAPE.  The caller owns every
 * buffer; nothing is allocated.
 */
mla_status mla_out_proj(const void* x, int x_dtype, const void* w_o, int w_dtype, void* out, int out_dtype,
                        int n_tok, int k_in, int d_model, void* stream);

/*
 * mla_combine_out_uv -- mla_combine_lse followed by mla_out_uv, in one launch.
 * [R]: the merged state goes through one shared output projection; [T]
 * "Move the Value Expansion After the Weighted Sum".  For every (token t,
 * head h) row r = t * n_heads + h:
 *   lse[r]      = ln sum_j exp(lse_part[r][j])               (-inf slots skipped)
 *   o[r]        = sum_j exp(lse_part[r][j] - lse[r]) o_part[r][j]   (fp32)
 *   out[t][h][i] = sum_j w_uv[h][i][j] * o[r][j]             (fp32 accumulation)
 * A row whose slots are all -inf gives o = 0, out = 0, lse = -inf; o_part
 * rows of -inf slots are never read.  The merged row enters U_V in fp32 (the
 * two-call path rounds o_lat to out_dtype first).  Every row reads its
 * head's U_V: meant for few query tokens per head.  With few rows (<= 128)
 * each row's output columns are split over 2 or 4 workgroups, each of which
 * merges the row itself.
 *
 * o_part   [n_tok][n_heads][n_part][d_c] part_dtype (fp32 or bf16; 16-byte aligned)
 * lse_part [n_tok][n_heads][n_part]      fp32 (n_part <= 1024)
 * w_uv     [n_heads][d_v][d_c]           w_dtype
 * o_lat    [n_tok][n_heads][d_c]         out_dtype, or NULL if not wanted
 * lse      [n_tok][n_heads]              fp32, or NULL if not wanted
 * out      [n_tok][n_heads][d_v]         out_dtype
 * Shapes: d_c a multiple of 4, d_c <= 512; d_v <= 128; n_tok, n_heads <= 65535,
 * n_tok * n_heads <= 2^21.
 * Errors: MLA_ERR_NULL, MLA_ERR_DTYPE, MLA_ERR_SHAPE as for the two calls.
 */
mla_status mla_combine_out_uv(const void* o_part, int part_dtype, const float* lse_part, int n_tok, int n_heads,
                              int n_part, int d_c, const void* w_uv, int w_dtype, int d_v, void* o_lat, float* lse,
                              void* out, int out_dtype, void* stream);

/*
 * mla_quantize_latent_i8 -- write an int8 latent cache (the cache writer's
 * part; QuantMLA abstract: low-bit latent caching, here the plain per-row
 * symmetric form).  For each of the n_rows stored rows [c | k^R] (bf16,
 * d_c + d_rope entries; a cache or a page pool viewed as rows):
 *   scale = max_i |c_i| / 127                       (fp32 quotient)
 *   code_i = nearest integer to c_i / scale, ties to even, clamped to [-127, 127]
 *            (the quotient in fp32; scale 0 gives codes 0)
 *   out_rows[r] = [code_0 .. code_{d_c-1} (int8) | k^R (the d_rope bf16 entries, unchanged)]
 *   scales[r]   = scale
 * rows [n_rows][d_c + d_rope] bf16; out_rows [n_rows][d_c + 2 d_rope] bytes;
 * scales [n_rows] fp32.  n_rows <= 2^32; d_c a multiple of 8, <= 512; d_rope a
 * multiple of 4, <= 128; rows and out_rows 8-byte aligned.
 * Errors: MLA_ERR_NULL, MLA_ERR_DTYPE (rows not bf16), MLA_ERR_SHAPE, MLA_ERR_ALIGN.
 */
mla_status mla_quantize_latent_i8(const void* rows, int row_dtype, int64_t n_rows, int d_c, int d_rope,
                                  void* out_rows, float* scales, void* stream);

/*
 * mla_quantize_latent_i4 -- write an int4 cache (the cache writer's part;
 * QuantMLA abstract: joint INT4 caching of the content and rotary caches, here
 * the plain per-row symmetric form).  For each of the n_rows stored rows
 * [c | k^R] (bf16, d_c + d_rope entries), the latent c and the rotary key k^R
 * are quantized separately; for each part x:
 *   scale = max_i |x_i| / 7                         (fp32 quotient)
 *   code_i = nearest integer to x_i / scale, ties to even, clamped to [-7, 7]
 *            (the quotient in fp32; scale 0 gives codes 0)
 * Codes go two per byte, entry 2j in the low nibble of byte j and entry 2j + 1
 * in the high nibble, as 4-bit two's complement:
 *   out_rows[r] = [d_c / 2 latent code bytes | d_rope / 2 rotary code bytes]
 *   scales[r]   = (latent scale, rotary scale)
 * rows [n_rows][d_c + d_rope] bf16; out_rows [n_rows][(d_c + d_rope) / 2]
 * bytes; scales [n_rows][2] fp32.  n_rows <= 2^32; d_c a multiple of 8, <= 512;
 * d_rope a multiple of 8, <= 128; out_rows 4-byte and scales 8-byte aligned.
 * Errors: MLA_ERR_NULL, MLA_ERR_DTYPE (rows not bf16), MLA_ERR_SHAPE, MLA_ERR_ALIGN.
 */
mla_status mla_quantize_latent_i4(const void* rows, int row_dtype, int64_t n_rows, int d_c, int d_rope,
                                  void* out_rows, float* scales, void* stream);

/*
 * QK-Norm MLA (QK-Norm MLA page, abstract): RMSNorm(x) = g x / sqrt(mean(x^2)
 * + eps) of the content query and key after their projections, the statistic
 * over a token's whole projection (all heads: the heads share one latent,
 * one KV group).  The static key weight moves into the query, the key
 * statistic becomes one inverse-RMS scalar per stored row:
 *   score_t = scale * (rinv_t * (q'_lat . c_t) + q_rot . k^R_t),
 *   q'_lat = U_K^T (g_q g_k q_nope) / rms(q_nope)   (mla_qknorm_query, then mla_absorb_q),
 *   rinv_t = 1 / sqrt(mean_{h,i} (U_K[h] c_t)_i^2 + eps)
 *          = 1 / sqrt(c_t^T G c_t / (n_heads * d_nope) + eps),  G = sum_h U_K[h]^T U_K[h].
 * The rotary parts are not normalised.
 *
 * mla_qknorm_query: q_out[t][h][i] = g_q[h][i] g_k[h][i] q_nope[t][h][i] / rms_t,
 *   rms_t = sqrt(mean_{h,i} q_nope[t][h][i]^2 + eps)  (eps = 0 and an all-zero
 *   token give rms_t = 0: that token's outputs are not finite, as in the definition).
 *   q_nope [n_tok][n_heads][d_nope] in_dtype; g_q, g_k [n_heads][d_nope] fp32;
 *   q_out [n_tok][n_heads][d_nope] fp32 (then mla_prepare_q with q_dtype MLA_F32 and
 *   the bf16 w_uk, or mla_absorb_q with fp32 weights).
 * mla_qknorm_key_gram: gram[a][b] = sum_{h,i} w_uk[h][i][a] w_uk[h][i][b],
 *   w_uk [n_heads][d_nope][d_c] w_dtype, gram [d_c][d_c] fp32 (d_c <= 512).
 * mla_qknorm_key_rinv: rinv[r] = 1 / sqrt(c_r^T gram c_r / (n_heads * d_nope) + eps)
 *   for the n_rows stored rows of `rows` ([n_rows][row_width] row_dtype, the
 *   latent c_r in the first d_c entries; a cache or a page pool viewed as rows);
 *   rinv [n_rows] fp32.  The cache writer's part: once per stored row.
 * Errors: MLA_ERR_NULL, MLA_ERR_DTYPE, MLA_ERR_SHAPE (eps < 0 or non-finite).
 */
mla_status mla_qknorm_query(const void* q_nope, int in_dtype, const float* g_q, const float* g_k, int n_tok,
                            int n_heads, int d_nope, double eps, float* q_out, void* stream);
mla_status mla_qknorm_key_gram(const void* w_uk, int w_dtype, int n_heads, int d_nope, int d_c, float* gram,
                               void* stream);
mla_status mla_qknorm_key_rinv(const void* rows, int row_dtype, int64_t n_rows, int row_width, const float* gram,
                               int d_c, int n_heads, int d_nope, double eps, float* rinv, void* stream);

/* Text of a status code (static storage). */
const char* mla_status_string(int status);

/* Detail of the last failing call on this thread ("" if none). */
const char* mla_last_error(void);

/* Library ABI version (major * 100 + minor). */
int mla_version(void);

/* Compute units of the current device (0 on error): the default n_wg. */
int mla_device_cu_count(void);

/*
 * Number of row shares the bf16 decode cuts one segment into for a grid of
 * n_wg workgroups (0 = one per compute unit) when s_q * head_count query rows
 * read it.  A request of T_b rows uses at most ceil(T_b / share) + 1 split
 * slots, share = 32 * ceil(ceil(sum_b T_b / shares) / 32); a caller picks
 * n_split from it.  Returns 0 on a bad argument.
 */
int mla_decode_shares(int s_q, int head_count, int n_wg);

#ifdef __cplusplus
}
#endif

#endif /* MLA_LATENT_H */
