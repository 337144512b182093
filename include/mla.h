/*
 * mla.h — C ABI of the MI355X (gfx950) weight-absorbed MLA decode library (libmla.so).
 *
 * The method (Multi-head Latent Attention of DeepSeek-V2):
 *   - the cache keeps, per token and layer, only the latent c^KV (d_c = 512) and the
 *     rotated shared RoPE key k^R (d_R = 64): 576 elements
 *     ("論文解説: DeepSeek-V2 — MoEモデルのKVキャッシュを93.3%削減するMulti-head Latent
 *     Attention", 0h-n0.github.io, sections "MLA: 低ランクKV結合圧縮" and "Decoupled RoPE");
 *   - W^UK moves onto the query (q~_i = W^UK_i^T q^C_i) and W^UV is applied after the
 *     weighted sum of latents (same page, section "行列吸収トリック"; kasblo.com/?p=4663,
 *     sections "K側は…Qを変換する" and "V側は、小さな表現の加重和を先に求める");
 *   - scores (q~_i . c_j + q^R_i . k^R_j) / sqrt(d_h + d_h^R), softmax over the cached
 *     tokens, u = W^O [o_1; ...; o_H] (qiita.com/joule/items/57d9b3f4fc27959eaa0d,
 *     section "Attention 計算").
 *
 * Conventions for every entry point
 *   - Tensor pointers are DEVICE pointers owned by the caller; every tensor is dense,
 *     row-major, in the shape given (the _strided entry points take row strides for the
 *     inputs they name).  The library never allocates, frees or synchronises;
 *     it enqueues kernels on `stream` (a hipStream_t passed as void*; NULL = the null
 *     stream) and returns.  Structs of sizes (mla_paged_shape_t) are HOST pointers.
 *   - All arguments are validated on the host before anything is launched; on any
 *     violation the call returns an error code, launches nothing, and
 *     mla_last_error_detail() describes the problem (thread-local string).
 *   - A launch failure reported by the runtime returns MLA_ERR_LAUNCH.  Faults inside a
 *     kernel surface at the caller's next synchronisation.
 *   - Block-table entries and seq_lens are read on the device and are NOT bounds-checked
 *     there: out-of-range values are undefined behaviour.  mla_validate_indices checks
 *     them on the device beforehand.
 *   - Results are deterministic for fixed inputs and arguments, except the projections
 *     mla_linear, mla_linear_strided, mla_linear_planned and mla_out_proj with bf16
 *     weights: their long reductions are split over workgroups that add into the fp32
 *     output atomically, so the last bits of y / u / o_heads can differ between runs.
 *     mla_linear_deterministic and mla_linear_deterministic_append sum the same split in
 *     one fixed order and are bit-identical from run to run.
 *
 * Paged latent cache: kv_cache[num_pages][page_size][d_latent + d_rope]; a row is
 * [c^KV (d_latent) | RoPE(k^R) (d_rope)].  Token j (0-based) of sequence b lives at
 * page block_table[b * max_pages_per_seq + j / page_size], slot j % page_size.
 * Entries past ceil(seq_len / page_size) are never read (conventionally -1).
 *
 * RoPE: pair (x[2k], x[2k+1]) is rotated by pos * rope_base^(-2k/d_rope) with the
 * rotation [[cos, -sin], [sin, cos]]; the angle, sine and cosine are evaluated in fp64.
 */
#ifndef MLA_H_
#define MLA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MLA_OK = 0,
  MLA_ERR_NULL = 1,        /* a required pointer is NULL                               */
  MLA_ERR_SHAPE = 2,       /* a size is out of range or sizes are inconsistent         */
  MLA_ERR_UNSUPPORTED = 3, /* valid but not compiled (dims / dtype combination)        */
  MLA_ERR_WORKSPACE = 4,   /* caller workspace too small                               */
  MLA_ERR_LAUNCH = 5,      /* the HIP runtime rejected a launch                        */
  MLA_ERR_INDEX = 6        /* reserved for index errors found on the host              */
} mla_status_t;

/* MLA_FP8 names a cache format, not an element type: 656-byte rows holding the 512 latent
 * values as OCP FP8 E4M3 codes (bytes 0..511), the 64 rotated k^R values in bf16 (bytes
 * 512..639) and four fp32 power-of-two scales, one per 128-value latent block (bytes
 * 640..655); the value of a code is its E4M3 value times its block's scale.  Block b's
 * scale is the smallest 2^k with max|x| <= 448 * 2^k (1 for an all-zero block) and a code
 * the E4M3 value nearest to x / 2^k, ties to the even code.  The pages name KV-cache
 * quantisation alongside MLA but fix no format (kasblo.com/?p=4663, "GQA・量子化・
 * FlashAttentionとは何が違うのか"); this one makes dequantisation exact in bf16.  Accepted as
 * the cache dtype of mla_kv_append*, mla_quantize_cache and mla_decode_attn* (with BF16
 * queries, 128 heads, d_latent 512, d_rope 64). */
typedef enum { MLA_F32 = 0, MLA_BF16 = 1, MLA_FP8 = 2 } mla_dtype_t;

typedef struct {
  int32_t batch;             /* B: sequences                                        */
  int32_t num_heads;         /* H: query heads                                      */
  int32_t d_latent;          /* d_c: latent width (512 DeepSeek-V2, 64 tiny)        */
  int32_t d_rope;            /* d_R: shared RoPE key width (64 / 16), even          */
  int32_t page_size;         /* tokens per page, a multiple of 16                   */
  int32_t max_pages_per_seq; /* row length of block_table                           */
  int32_t num_pages;         /* pages in the pool                                   */
} mla_paged_shape_t;

/* ---------------------------------------------------------------------------------
 * Sizes and planning (pure host functions, no device access)
 * -------------------------------------------------------------------------------*/

/* Bytes of a latent cache of B sequences x T tokens x `layers` layers with
 * (d_c + d_R) elements of `elem_bytes` each (kasblo.com/?p=4663, "容量を計算する").
 * Returns 0 if any argument is negative. */
size_t mla_cache_bytes(int64_t B, int64_t T, int64_t layers, int32_t d_c, int32_t d_R,
                       int32_t elem_bytes);

/* Bytes of workspace mla_decode needs for num_splits > 1: room for fp32 split partials
 * o_part [B][H][S][d_c] followed by lse_part [B][H][S] (256-byte aligned); enough for
 * the bf16 partials mla_decode uses with bf16 caches. */
size_t mla_decode_workspace_bytes(int32_t B, int32_t H, int32_t d_c, int32_t num_splits);

/* A split count for mla_decode_attn: enough (sequence, split) work items to cover
 * `num_cus` compute units when every sequence holds `max_seq_len` tokens, and no more
 * splits than pages.  total_tokens (sum of seq_lens, or <= 0 if unknown) lets ragged
 * batches use smaller splits.  Always >= 1. */
int32_t mla_suggest_num_splits(int32_t B, int32_t max_seq_len, int64_t total_tokens,
                               int32_t page_size, int32_t num_cus);

/* ---------------------------------------------------------------------------------
 * Hot path
 * -------------------------------------------------------------------------------*/

/* Query absorption and query RoPE.
 *   q_lat[b][i][c] = sum_d w_uk[i*d_h + d][c] * q_c[b][i][d]        (q~_i = W^UK_i^T q^C_i)
 *   q_pe[b][i][:]  = RoPE(q_r[b][i][:], pos = seq_lens[b] - 1)
 * ("論文解説: DeepSeek-V2 …", "行列吸収トリック"; qiita "RoPE の扱い": q^R = RoPE(W^QR c^Q).)
 *   q_c      [B][H][d_h]       fp32
 *   w_uk     [H*d_h][d_c]      w_dtype   (nn.Linear weight of W^UK; head i = row block i)
 *   q_r      [B][H][d_R]       fp32, pre-rotation; NULL skips the RoPE part
 *   seq_lens [B]               int32, context length INCLUDING the query token (>= 1)
 *   q_lat    [B][H][d_c]       out_dtype (written)
 *   q_pe     [B][H][d_R]       out_dtype (written; may be NULL iff q_r is NULL)
 * Errors: NULL, SHAPE (non-positive sizes, odd d_R), UNSUPPORTED (dtype). */
mla_status_t mla_absorb_q(const float* q_c, const void* w_uk, const float* q_r,
                          const int32_t* seq_lens, float rope_base, void* q_lat, void* q_pe,
                          int32_t B, int32_t H, int32_t d_h, int32_t d_c, int32_t d_R,
                          mla_dtype_t w_dtype, mla_dtype_t out_dtype, void* stream);

/* mla_absorb_q on row-strided inputs: row b of q_c starts at q_c + b * ld_qc and row b of
 * q_r at q_r + b * ld_qr (elements; the heads of a row stay contiguous, d_h and d_R apart).
 * This reads q^C and q^R in place from one stacked projection y = [W^UQ; W^QR] c^Q, whose
 * rows hold q^C_b followed by q^R_b (ld_qc = ld_qr = H*(d_h + d_R), q_r = q_c + H*d_h).
 * The products and roundings are those of mla_absorb_q.  q_lat and q_pe stay dense.
 * Errors: as mla_absorb_q, and SHAPE for ld_qc < H*d_h or (q_r given) ld_qr < H*d_R. */
mla_status_t mla_absorb_q_strided(const float* q_c, int64_t ld_qc, const void* w_uk,
                                  const float* q_r, int64_t ld_qr, const int32_t* seq_lens,
                                  float rope_base, void* q_lat, void* q_pe, int32_t B, int32_t H,
                                  int32_t d_h, int32_t d_c, int32_t d_R, mla_dtype_t w_dtype,
                                  mla_dtype_t out_dtype, void* stream);

/* Packing of the query-side weights for mla_query_path, done once at load time (a
 * permutation copy).  w_pack holds H * (192 * d_cq + 128 * 512) bf16:
 *  - W^UQ and W^QR as 1 KB MFMA operand fragments.  For head i, the 192 rows
 *    [W^UQ_i; W^QR_i] form 12 tiles of 16 rows; fragment (i, c, tl, s4), for the 128-wide
 *    k chunk c, tile tl and k-step s4 < 4 of the chunk, starts at element
 *    (((c * H + i) * 12 + tl) * 4 + s4) * 512, and its element 8 l + e (l < 64,
 *    e < 8) is row 16 tl + l % 16 of [W^UQ_i; W^QR_i] at k = 32 (4 c + s4) + 8 (l / 16) + e
 *    (rows 0..127: W^UQ row i*128 + row; rows 128..191: W^QR row i*64 + row - 128).
 *  - Then W^UK: for head i and half hf (columns 256 hf .. + 255), 128 rows j of 32
 *    16-byte pieces; piece pos of row j, at element H*192*d_cq + (((2 i + hf) * 128 + j) * 32
 *    + pos) * 8, holds W^UK[i*128 + j][256 hf + 8 (pos ^ f(j)) .. + 7] with
 *    f(j) = 2 (j % 4) + 8 ((j / 8) % 2).
 *   w_uq [H*128][d_cq], w_qr [H*64][d_cq], w_uk [H*128][512] bf16 (nn.Linear weights);
 *   w_pack caller-owned, 16-byte aligned (written)
 * Errors: NULL, SHAPE (H < 1, d_cq not a positive multiple of 384), UNSUPPORTED (unaligned). */
mla_status_t mla_pack_query_weights(const void* w_uq, const void* w_qr, const void* w_uk,
                                    int32_t H, int32_t d_cq, void* w_pack, void* stream);

/* The whole query side of a decode step in one launch: up-projection, query RoPE and
 * absorption, head by head, without writing q^C or q^R to memory.
 *   q^C_i = W^UQ_i c^Q,  q^R_i = W^QR_i c^Q         (qiita.com/joule/items/57d9b3f4fc27959eaa0d,
 *                                                     "Query の圧縮", "RoPE の扱い")
 *   q_pe[b][i][:]  = RoPE(q^R_i of row b, pos = seq_lens[b] - 1)
 *   q_lat[b][i][c] = sum_d W^UK[i*d_h + d][c] * q^C_i[d]   (same page, "Absorption Trick")
 *   c_q      [B] rows of d_cq fp32, row b at c_q + b * ld_cq (ld_cq >= d_cq, % 4 == 0)
 *   w_pack   W^UQ, W^QR and W^UK as packed by mla_pack_query_weights (bf16)
 *   seq_lens [B] int32, context length INCLUDING the query token (>= 1)
 *   q_lat    [B][H][d_c] bf16, q_pe [B][H][d_R] bf16 (written)
 * Products: bf16 MFMA with fp32 accumulation, c^Q carried as two bf16 terms (about 16
 * significant bits, every product with a bf16 weight exact), q^C rounded the same way
 * before the absorption.  Every sum runs in one fixed order inside one workgroup: the
 * results are bit-identical from run to run (no atomics).  Blocks of 64 rows of the batch
 * run as separate launches, each reading the weights.  Needs d_h 128, d_R 64, d_c 512,
 * d_cq a multiple of 384 and 16-byte aligned pointers, else UNSUPPORTED (mla_linear_strided
 * followed by mla_absorb_q_strided computes the same).  The caller owns every buffer.
 * Errors: NULL, SHAPE (sizes < 1, ld_cq < d_cq, rope_base not finite), UNSUPPORTED. */
mla_status_t mla_query_path(const float* c_q, int64_t ld_cq, const void* w_pack,
                            const int32_t* seq_lens, float rope_base, void* q_lat, void* q_pe,
                            int32_t B, int32_t H, int32_t d_h, int32_t d_R, int32_t d_c,
                            int32_t d_cq, void* stream);

/* Append n_new tokens per sequence to the paged cache.
 * Token t of sequence b goes to position pos = seq_lens_before[b] + t and its row is
 * [c_kv[b][t][:] | RoPE(k_r[b][t][:], pos)] converted to cache_dtype
 * ("論文解説: DeepSeek-V2 …", "Decoupled RoPE": only c^KV and the rotated k^R are cached;
 * qiita "RoPE の扱い": k^R = RoPE(W^KR h)).
 *   c_kv [B][n_new][d_latent] fp32;  k_r [B][n_new][d_rope] fp32 (pre-rotation)
 *   seq_lens_before [B] int32;  block_table [B][max_pages_per_seq] int32
 *   kv_cache as described above (written only at the appended rows)
 * Errors: NULL, SHAPE (n_new < 1, any shape field < 1, page_size % 16, odd d_rope),
 * UNSUPPORTED (dtype). */
mla_status_t mla_kv_append(const float* c_kv, const float* k_r, int32_t n_new,
                           const int32_t* seq_lens_before, const int32_t* block_table,
                           void* kv_cache, float rope_base, const mla_paged_shape_t* shape,
                           mla_dtype_t cache_dtype, void* stream);

/* mla_kv_append on row-strided inputs: the inputs of token t of sequence b are read at
 * c_kv + (b*n_new + t) * ld_ckv and k_r + (b*n_new + t) * ld_kr (elements).  This reads
 * c^KV and k^R in place from one stacked projection y = [W^DQ; W^DKV; W^KR] h (row stride
 * d_c^Q + d_latent + d_rope).  Same rows written as mla_kv_append.
 * Errors: as mla_kv_append, and SHAPE for ld_ckv < d_latent or ld_kr < d_rope. */
mla_status_t mla_kv_append_strided(const float* c_kv, int64_t ld_ckv, const float* k_r,
                                   int64_t ld_kr, int32_t n_new, const int32_t* seq_lens_before,
                                   const int32_t* block_table, void* kv_cache, float rope_base,
                                   const mla_paged_shape_t* shape, mla_dtype_t cache_dtype,
                                   void* stream);

/* Prefill attention in the expanded form: T prompt tokens per sequence attend causally to
 * the prompt through the up-projected keys and values (for many query tokens the pages give
 * the naive order: [perforder] "極限最適化の代償：MLA特有の学習負荷と独自Tritonカーネルという
 * 障壁"; kasblo.com/?p=4663, "「キャッシュを減らせた」と「その割合だけ速い」は別の評価").
 * With k^C_{j,i} = W^UK_i c_j and v^C_{j,i} = W^UV_i c_j computed over the prompt (two
 * mla_linear products), for every sequence b, query t and head i:
 *   s_tj = softmax_scale * ([q_c; q_pe][b][t][i] . [k_c[b][j][i]; k_pe[b][j]]),  j <= t
 *   out[b][t][i][:] = sum_j softmax_j(s_tj) v_c[b][j][i][:];  lse_out[b][t][i] = ln sum_j e^s
 * (qiita.com/joule/items/57d9b3f4fc27959eaa0d, "Attention 計算": the sum runs to the query's
 * own position; "論文解説: DeepSeek-V2 …", "Decoupled RoPE": k^R is shared by the heads).
 *   q_c [B][T][H][d_h], q_pe [B][T][H][d_R] (rotated), k_c [B][T][H][d_h],
 *   k_pe [B][T][d_R] (rotated), v_c [B][T][H][d_h]: BF16, 16-byte aligned
 *   out [B][T][H][d_h] fp32 (16-byte aligned); lse_out [B][T][H] fp32 or NULL
 * Supported: d_h = 128, d_R = 64, BF16 (bf16 MFMA; the weights P are rounded to bf16 for
 * the value product and the denominators sum those rounded weights).
 * Errors: NULL, SHAPE, UNSUPPORTED. */
mla_status_t mla_prefill_attn(const void* q_c, const void* q_pe, const void* k_c,
                              const void* k_pe, const void* v_c, int32_t B, int32_t T,
                              int32_t H, int32_t d_h, int32_t d_R, float softmax_scale,
                              float* out, float* lse_out, mla_dtype_t dtype, void* stream);

/* fp8 latent rows (MLA_FP8) from rows of 576 values: dst row r = the quantised row r of
 * src (src + r * src_ld, src_dtype F32 or BF16; latent then k^R).  The latent is quantised
 * as MLA_FP8 describes; k^R is rounded to bf16 (exact for BF16 input).  rows >= 1; src_ld
 * >= 576.  The codes follow from the values alone (every step is exact in fp32).
 * Errors: NULL, SHAPE, UNSUPPORTED (src_dtype). */
mla_status_t mla_quantize_cache(const void* src, mla_dtype_t src_dtype, int64_t src_ld,
                                int64_t rows, void* dst, void* stream);

/* Decode attention over the paged latent cache, split over tokens.
 * For every sequence b, head i and split s (s = 0..num_splits-1), with
 * cps = ceil(max_pages_per_seq / num_splits) pages per split, split s covers the cached
 * tokens j in [s*cps*P, (s+1)*cps*P) with j < seq_lens[b] and computes
 *   score_j = softmax_scale * ([q_lat[b][i]; q_pe[b][i]] . row_j)     (576-wide dot)
 *   o_part[b][i][s][:] = sum_j e^{score_j} c_j / sum_j e^{score_j}   (c_j = row_j[0:d_c])
 *   lse_part[b][i][s]  = ln sum_j e^{score_j}
 * (qiita "Attention 計算" in the absorbed order; kasblo "V側は…" for the latent sum).
 * A split with no tokens writes o = 0 and lse = -inf.
 *   q_lat [B][H][d_latent], q_pe [B][H][d_rope]: `dtype` (q_pe already rotated), BF16
 *   when dtype is MLA_FP8
 *   kv_cache: `dtype` (MLA_FP8: 656-byte rows, the values dequantised exactly);
 *   block_table [B][max_pages_per_seq], seq_lens [B]: int32, device
 *   o_part [B][H][S][d_latent] in part_dtype (F32, or BF16 rounded to nearest even: half
 *   the partial traffic; the softmax sums and the PV accumulation stay fp32);
 *   lse_part [B][H][S] fp32.
 *   With num_splits == 1, o_part is the final o~ [B][H][d_latent] and lse_part may be NULL.
 * softmax_scale is normally 1/sqrt(d_h + d_R) (1/sqrt(192) at DeepSeek-V2 shape).
 * Supported: (d_latent, d_rope, dtype) = (512, 64, BF16) with H <= 128, (512, 64, FP8)
 * with H = 128 (raw rows staged in LDS and converted to bf16 there, on the kernel with 32
 * heads per wavefront when the tensors are 16-byte aligned, else the head-partitioned one),
 * or (64, 16, F32) with H <= 64; otherwise UNSUPPORTED.
 * Errors: NULL, SHAPE (sizes < 1, page_size % 16, odd d_rope, num_splits < 1,
 * seq_lens bound max_pages_per_seq*page_size does not fit int32), UNSUPPORTED. */
mla_status_t mla_decode_attn(const void* q_lat, const void* q_pe, const void* kv_cache,
                             const int32_t* block_table, const int32_t* seq_lens,
                             const mla_paged_shape_t* shape, float softmax_scale,
                             int32_t num_splits, void* o_part, mla_dtype_t part_dtype,
                             float* lse_part, mla_dtype_t dtype, void* stream);

/* Decode attention for n_q new query tokens per sequence (speculative or multi-token
 * decode), all already appended to the cache: token t (0..n_q-1) of sequence b sits at
 * position seq_lens[b] - n_q + t and attends to the cached tokens 0 .. that position, so
 * the new tokens see each other causally (qiita "Attention 計算": the sum over tokens runs
 * up to the query's own position).  Each (b, t) is a decode query as in mla_decode_attn
 * with seq_len seq_lens[b] - n_q + 1 + t; rows are numbered bq = b*n_q + t:
 *   q_lat [B][n_q][H][d_latent], q_pe [B][n_q][H][d_rope]: `dtype`
 *   o_part [B][n_q][H][S][d_latent] in part_dtype, lse_part [B][n_q][H][S] fp32
 * so mla_splitk_combine with batch B*n_q merges the splits.  A token whose position is
 * negative (seq_lens[b] < n_q - t) sees no tokens: o = 0, lse = -inf.  n_q = 1 is
 * mla_decode_attn.  The n_q workgroups of one (sequence, split) read the same cache
 * tiles at about the same time from the same XCD, so the extra tokens cost L2 reads,
 * not HBM reads.
 * Errors: as mla_decode_attn, plus SHAPE for n_q < 1 or B*n_q > 65535. */
mla_status_t mla_decode_attn_multi(const void* q_lat, const void* q_pe, const void* kv_cache,
                                   const int32_t* block_table, const int32_t* seq_lens,
                                   const mla_paged_shape_t* shape, int32_t n_q,
                                   float softmax_scale, int32_t num_splits, void* o_part,
                                   mla_dtype_t part_dtype, float* lse_part, mla_dtype_t dtype,
                                   void* stream);

/* mla_decode_attn_multi with an explicit attention kernel, for measurement and for tests
 * that cover each kernel: 0 = the library's choice (as mla_decode_attn_multi), 1 = the
 * head-partitioned MFMA kernel (16 heads per wavefront; H in {16, 32, 64, 128}), 2 = the
 * column-partitioned MFMA kernel (H = 128; each wavefront owns 64 latent columns of the
 * weighted sum), 3 = the generic VALU kernel, 4 = the MFMA kernel with 32 heads per
 * wavefront on the 32 x 32 x 16 MFMA (H = 128; four wavefronts, each fragment read from LDS
 * feeds 32 heads).  Kernels 1, 2 and 4 need d_latent 512, d_rope 64, BF16, pages of >= 32
 * tokens (a power of two), at most 1024 pages per split and 16-byte aligned q_lat, q_pe,
 * kv_cache (and o_part for 2 and 4); MLA_FP8 rows run on kernel 1 or 4.  Same results,
 * within rounding order, as mla_decode_attn_multi.
 * Errors: as mla_decode_attn_multi, plus UNSUPPORTED for a kernel the shape cannot take. */
mla_status_t mla_decode_attn_planned(const void* q_lat, const void* q_pe, const void* kv_cache,
                                     const int32_t* block_table, const int32_t* seq_lens,
                                     const mla_paged_shape_t* shape, int32_t n_q,
                                     float softmax_scale, int32_t num_splits, void* o_part,
                                     mla_dtype_t part_dtype, float* lse_part, mla_dtype_t dtype,
                                     int32_t kernel, void* stream);

/* Log-sum-exp combine of split partials (exact re-assembly of one softmax whose sum
 * over tokens was cut into disjoint ranges; qiita "Attention 計算").
 *   M = max_s lse_s; w_s = e^{lse_s - M} (0 for lse_s = -inf)
 *   out[b][i][:] = sum_s w_s o_part[b][i][s][:] / sum_s w_s;  lse_out = M + ln sum_s w_s
 * All splits empty: out = 0, lse_out = -inf.
 *   o_part [B][H][S][d_c] in part_dtype (F32 or BF16), 16-byte aligned; lse_part [B][H][S] fp32;
 *   out [B][H][d_c] fp32 (fp32 weights and sums), 16-byte aligned;  lse_out [B][H] fp32 or NULL.
 * Errors: NULL, SHAPE (sizes < 1, d_c % 4, misaligned o_part / out), UNSUPPORTED (part_dtype). */
mla_status_t mla_splitk_combine(const void* o_part, mla_dtype_t part_dtype,
                                const float* lse_part, int32_t B, int32_t H, int32_t num_splits,
                                int32_t d_c, float* out, float* lse_out, void* stream);

/* mla_splitk_combine fused with the W^UV up-projection, in one kernel (the combined latent
 * stays on the chip: it is neither written nor read back):
 *   o~[b][i][:] = combine of o_part[b][i][:][:] with lse_part[b][i][:], as mla_splitk_combine
 *   o_heads[b][i][j] = sum_c w_uv[i*d_h + j][c] * o~[b][i][c]
 * ("論文解説: DeepSeek-V2 …", "行列吸収トリック"; kasblo.com/?p=4663, "V側は、小さな表現の
 * 加重和を先に求める": the weighted sum of latents first, W^UV_i after it.)
 *   o_part [B][H][S][d_c] part_dtype (F32 or BF16);  lse_part [B][H][S] fp32;
 *   w_uv [H*d_h][d_c] bf16 (nn.Linear weight, head i = row block i);  o_heads [B][H][d_h] fp32.
 * o~ is formed in fp32 and enters the product as two bf16 terms (about 16 significant bits,
 * as mla_out_proj carries its fp32 input), fp32 accumulation.  Compiled for d_c = 512,
 * d_h = 128, num_splits <= 64, 16-byte aligned o_part and w_uv; other shapes take
 * mla_splitk_combine followed by mla_out_proj.  Deterministic (no atomics).
 * Errors: NULL, SHAPE (sizes < 1), UNSUPPORTED (dtypes, or a shape not compiled). */
mla_status_t mla_combine_out_proj(const void* o_part, mla_dtype_t part_dtype,
                                  const float* lse_part, int32_t B, int32_t H, int32_t num_splits,
                                  int32_t d_c, const void* w_uv, mla_dtype_t w_dtype, int32_t d_h,
                                  float* o_heads, void* stream);

/* Decode attention and split-K combine in one launch.  The workgroups of a query row merge
 * its splits themselves once all of them have written their partials (workgroup s combines
 * heads s, s + S, s + 2S, ... with the combine's per-row arithmetic), so no combine kernel
 * and no second launch follow.  The splits are exact pieces of one softmax whose
 * denominator is a sum over the tokens (qiita.com/joule/items/57d9b3f4fc27959eaa0d,
 * "Attention 計算"), as for mla_splitk_combine.
 * The in-launch merge needs the head-partitioned MFMA kernel (d_latent 512, d_rope 64,
 * BF16, H in {16, 32, 64, 128}) with its whole grid (B * n_q * num_splits workgroups)
 * resident on the device at once, since its workgroups wait for each other; otherwise the
 * call runs the attention and then mla_splitk_combine's kernel on the same stream.  Either
 * way out / lse_out hold the same bits as mla_decode_attn_multi + mla_splitk_combine with
 * the same num_splits and partial dtype.
 *   q_lat .. n_q, softmax_scale, num_splits, dtype: as mla_decode_attn_multi (BF16 only)
 *   o_part     [B n_q][H][S][d_latent] part_dtype, lse_part [B n_q][H][S] fp32: scratch the
 *              call overwrites (unused when num_splits == 1); 16-byte aligned
 *   counters   int32 [2 B n_q + 1], caller-owned, ZERO before the first call; every call
 *              leaves the first 2 B n_q words zero again.  The last word is an error flag:
 *              set to 1 if a merge wait ran out (only possible when other work kept part of
 *              the grid off the device for about a second); the call's out is then invalid.
 *   out        [B n_q][H][d_latent] fp32 (16-byte aligned); lse_out [B n_q][H] or NULL
 * Calls that share `counters` must not overlap (one stream, or caller-serialised).
 * Errors: as mla_decode_attn_multi, plus NULL (out, or counters with num_splits > 1),
 * SHAPE (num_splits > 64, misaligned o_part / out). */
mla_status_t mla_decode_fused(const void* q_lat, const void* q_pe, const void* kv_cache,
                              const int32_t* block_table, const int32_t* seq_lens,
                              const mla_paged_shape_t* shape, int32_t n_q, float softmax_scale,
                              int32_t num_splits, void* o_part, mla_dtype_t part_dtype,
                              float* lse_part, int32_t* counters, float* out, float* lse_out,
                              mla_dtype_t dtype, void* stream);

/* 1 if mla_decode_fused with this shape, n_q and num_splits (and 16-byte aligned BF16
 * tensors) merges its splits inside the attention launch on the current device, 0 if it
 * runs the attention and the combine kernel (or the arguments are invalid).  Host-only. */
int32_t mla_decode_fused_single_launch(const mla_paged_shape_t* shape, int32_t n_q,
                                       int32_t num_splits);

/* Bytes of workspace mla_decode_ragged needs for this paged shape (HOST pointer) on the
 * current device.  Its launch has G = max(compute units, ceil(num_pages / 1024))
 * workgroups; the workspace holds the per-sequence slot table, then (G + batch) fp32 lse
 * rows of num_heads and bf16 partials of num_heads x d_latent, each part 256-byte aligned.
 * Returns 0 for a NULL shape or a size below 1. */
size_t mla_decode_ragged_workspace_bytes(const mla_paged_shape_t* shape);

/* Decode for ragged batches (one query token per sequence, lengths free, BF16 rows with
 * H in {16, 32, 64, 128} or MLA_FP8 rows with H = 128, d_latent 512, d_rope 64): the same
 * result as mla_decode, with the
 * work cut for the device instead of per sequence.  The cached pages of the whole batch,
 * concatenated in sequence order, are divided into one equal range per compute unit, so
 * every workgroup streams the same number of pages whatever the mix of lengths; a range
 * writes one bf16 partial per sequence piece inside it, and a combine kernel merges each
 * sequence's pieces (the softmax denominator is a sum over the tokens:
 * qiita.com/joule/items/57d9b3f4fc27959eaa0d, "Attention 計算").  The plan is computed on
 * the device from seq_lens: no host synchronisation, two launches.
 *   q_lat .. dtype: as mla_decode (n_q = 1)
 *   workspace  >= mla_decode_ragged_workspace_bytes(shape) bytes, 256-byte aligned,
 *              overwritten; its int32 word 2B is set to 1 when a workgroup's range would
 *              exceed 1024 pages (more than 1024 x G cached pages in the batch, which takes
 *              pages shared between sequences, or one sequence of more than 64 x 1024
 *              pages); every output is then 0 / -inf.  Otherwise it is set to 0.
 *   out [B][H][d_latent] fp32 (16-byte aligned); lse_out [B][H] or NULL.
 * A sequence with seq_len 0 gives o = 0 and lse = -inf.
 * Errors: NULL, SHAPE, UNSUPPORTED (shape or dtype), WORKSPACE (NULL, too small, misaligned). */
mla_status_t mla_decode_ragged(const void* q_lat, const void* q_pe, const void* kv_cache,
                               const int32_t* block_table, const int32_t* seq_lens,
                               const mla_paged_shape_t* shape, float softmax_scale,
                               void* workspace, size_t workspace_bytes, float* out,
                               float* lse_out, mla_dtype_t dtype, void* stream);

/* mla_decode_attn followed by mla_splitk_combine, with the split partials in a caller
 * workspace of at least mla_decode_workspace_bytes(B, H, d_latent, num_splits) bytes
 * (unused when num_splits == 1); the partials take the cache dtype (BF16 caches: bf16
 * partials).  out [B][H][d_latent] fp32; lse_out [B][H] or NULL.
 * Errors: as the two calls, plus WORKSPACE when the workspace is NULL or too small. */
mla_status_t mla_decode(const void* q_lat, const void* q_pe, const void* kv_cache,
                        const int32_t* block_table, const int32_t* seq_lens,
                        const mla_paged_shape_t* shape, float softmax_scale,
                        int32_t num_splits, void* workspace, size_t workspace_bytes,
                        float* out, float* lse_out, mla_dtype_t dtype, void* stream);

/* mla_decode for callers that cannot allocate device memory (code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc): the split partials go to a fixed
 * device scratch array of 48 MiB that the library holds on every GPU it runs on until the
 * process ends, instead of a caller workspace.  The call itself allocates nothing: no
 * hipMalloc, no hipFree, no allocating library routine.  Same kernels, partial dtype and
 * results (bit for bit) as mla_decode with the same num_splits.  Every call on one GPU
 * shares that GPU's scratch and leaves its partials there; each call overwrites every
 * partial it reads, so nothing needs clearing, but calls that overlap on one GPU (two
 * streams, or two host threads) race and must be serialised by the caller.
 * Errors: as mla_decode, plus WORKSPACE when mla_decode_workspace_bytes(B, H, d_latent,
 * num_splits) exceeds 48 MiB (nothing is launched), LAUNCH if the scratch cannot be found. */
mla_status_t mla_decode_noalloc(const void* q_lat, const void* q_pe, const void* kv_cache,
                                const int32_t* block_table, const int32_t* seq_lens,
                                const mla_paged_shape_t* shape, float softmax_scale,
                                int32_t num_splits, float* out, float* lse_out, mla_dtype_t dtype,
                                void* stream);

/* Offline absorption of W^UK into W^UQ: the weight of q~ = W~ c^Q in one projection
 * ("論文解説: DeepSeek-V2 …", "行列吸収トリック"; qiita.com/joule/items/57d9b3f4fc27959eaa0d,
 * "Absorption Trick"):
 *   w_out[i*d_c + m][n] = sum_d w_uk[i*d_h + d][m] * w_uq[i*d_h + d][n]   (W~_i = W^UK_i^T W^UQ_i)
 *   w_uk [H*d_h][d_c], w_uq [H*d_h][d_cq] (nn.Linear weights), w_dtype; w_out [H*d_c][d_cq]
 *   out_dtype (written; bf16 rounded once from the fp32 sum).  A one-time preparation
 *   (a VALU batched GEMM), not a hot-path call.  Errors: NULL, SHAPE, UNSUPPORTED. */
mla_status_t mla_fold_uq(const void* w_uk, const void* w_uq, int32_t H, int32_t d_h,
                         int32_t d_c, int32_t d_cq, mla_dtype_t w_dtype, void* w_out,
                         mla_dtype_t out_dtype, void* stream);

/* Offline fold of W^UV into W^O: u = W_fold [o~_1; ...; o~_H] replaces o_i = W^UV_i o~_i
 * followed by u = W^O [o_1; ...; o_H] (qiita.com/joule/items/57d9b3f4fc27959eaa0d,
 * "Absorption Trick": W_UV folds into W_O):
 *   w_out[n][i*d_c + c] = sum_d w_o[n][i*d_h + d] * w_uv[i*d_h + d][c]
 *   w_o [d_model][H*d_h], w_uv [H*d_h][d_c] (nn.Linear weights), w_dtype;
 *   w_out [d_model][H*d_c] out_dtype (written).  At decode the folded weight is d_c / d_h
 *   times the size of W^O.  One-time preparation, as mla_fold_uq.
 * Errors: NULL, SHAPE, UNSUPPORTED. */
mla_status_t mla_fold_o_uv(const void* w_o, const void* w_uv, int32_t H, int32_t d_h,
                           int32_t d_c, int32_t d_model, mla_dtype_t w_dtype, void* w_out,
                           mla_dtype_t out_dtype, void* stream);

/* Value up-projection and output projection.
 *   o_heads[b][i][d] = sum_c w_uv[i*d_h + d][c] * o_lat[b][i][c]    (o_i = W^UV_i o~_i)
 *   u[b][n] = sum_k w_o[n][k] * o_heads[b][k]   (k over H*d_h; u = W^O [o_1;...;o_H])
 * (kasblo "V側は…": up-project after the weighted sum; qiita "Attention 計算" for u.)
 *   o_lat [B][H][d_c] fp32;  w_uv [H*d_h][d_c] w_dtype;  w_o [d_model][H*d_h] w_dtype or NULL
 *   o_heads [B][H][d_h] fp32 (always written);  u [B][d_model] fp32 (NULL iff w_o NULL)
 * Both products use the GEMM paths of mla_linear (bf16 MFMA for bf16 weights).
 * Errors: NULL, SHAPE, UNSUPPORTED (dtype). */
mla_status_t mla_out_proj(const float* o_lat, const void* w_uv, const void* w_o, int32_t B,
                          int32_t H, int32_t d_c, int32_t d_h, int32_t d_model,
                          mla_dtype_t w_dtype, float* o_heads, float* u, void* stream);

/* y = x w^T for an nn.Linear weight: y[m][n] = sum_k x[m][k] w[n][k], fp32 accumulate,
 * fp32 output.  Used for the projections c^Q = W^DQ h, q^C = W^UQ c^Q, q^R = W^QR c^Q,
 * c^KV = W^DKV h, k^R = W^KR h (qiita "Query の圧縮", "RoPE の扱い").
 *   x [M][K] x_dtype;  w [N][K] w_dtype;  y [M][N] fp32.
 * With bf16 w, K a multiple of 128 and 16-byte aligned x, w: bf16 MFMA (fp32 x carried as
 * two bf16 terms, about 16 significant bits; bf16 x as is), split-K partial sums added
 * atomically (y is overwritten, not accumulated into).  Which MFMA kernel runs depends on
 * the shape: for one product of 8 MB of weights or more with N >= 1024 and M <= 64, an
 * activation-stationary kernel (K <= 4096, N >= 4096) or a persistent weight-streaming
 * kernel, one workgroup per CU; otherwise a tile-grid kernel.  All give the same products
 * and roundings up to the order of the fp32 additions.  Without MFMA: an fp32 VALU GEMM.
 * Errors: NULL, SHAPE (sizes < 1), UNSUPPORTED (dtype). */
mla_status_t mla_linear(const void* x, mla_dtype_t x_dtype, const void* w,
                        mla_dtype_t w_dtype, int32_t M, int32_t N, int32_t K, float* y,
                        void* stream);

/* mla_linear with row strides and an accumulate option: x row m at x + m * ldx, y row m at
 * y + m * ldy (elements, ldx >= K, ldy >= N; only columns 0 .. N-1 of each y row are
 * touched).  accumulate = 0: y = x w^T, as mla_linear.  accumulate != 0: y += x w^T, y
 * holding its prior values (with y zeroed beforehand this is the same product; the split-k
 * kernels then launch no zero fill of their own, so a caller can clear y earlier, on
 * another stream, off the critical path).  Projections that read the same input can run as
 * one product over their stacked weights, e.g. [W^DQ; W^DKV; W^KR] h (one launch instead
 * of three, the three results side by side in each row of y), and the next product can
 * read its input columns in place, e.g. c^Q as the first d_c^Q columns of that y.  x and y
 * must not overlap.
 * Errors: as mla_linear, and SHAPE for ldx < K or ldy < N. */
mla_status_t mla_linear_strided(const void* x, mla_dtype_t x_dtype, int64_t ldx, const void* w,
                                mla_dtype_t w_dtype, int32_t M, int32_t N, int32_t K, float* y,
                                int64_t ldy, int32_t accumulate, void* stream);

/* mla_linear_strided with results that are bit-identical from run to run: the k range is
 * still split over workgroups, but each workgroup stores its partial sums of a column tile
 * in that tile's own slot of a caller workspace (plain stores, no atomics) and a second
 * launch adds the slots of every tile in one fixed order into y (after y's prior value when
 * accumulate != 0).  Same products and roundings as mla_linear up to the order of the fp32
 * additions, which is fixed here.  Used for the projections of a decode step
 * ([W^DQ; W^DKV; W^KR] h, W^O [o_1; ...; o_H]; qiita.com/joule/items/57d9b3f4fc27959eaa0d,
 * "Query の圧縮", "Attention 計算").
 *   x [M rows of ldx] x_dtype (f32 or bf16);  w [N][K] bf16;  y [M rows of ldy] fp32
 *   workspace: at least mla_linear_deterministic_workspace_bytes(M, N, K) bytes, 16-byte
 *   aligned, caller-owned, scratch (its contents on entry do not matter)
 * Needs M <= 64, N % 64 == 0, K % 128 == 0, ldx % 8 == 0, ldy % 4 == 0 and 16-byte aligned
 * x, w, y, workspace, else UNSUPPORTED.
 * Errors: NULL, SHAPE (sizes < 1, ldx < K, ldy < N), UNSUPPORTED, WORKSPACE (too small). */
size_t mla_linear_deterministic_workspace_bytes(int32_t M, int32_t N, int32_t K);
mla_status_t mla_linear_deterministic(const void* x, mla_dtype_t x_dtype, int64_t ldx,
                                      const void* w, mla_dtype_t w_dtype, int32_t M, int32_t N,
                                      int32_t K, float* y, int64_t ldy, int32_t accumulate,
                                      void* workspace, size_t workspace_bytes, void* stream);

/* mla_linear_deterministic (accumulate 0) that also appends the new token of every sequence
 * to the paged cache in its second (summing) launch: the RoPE and the append fused into the
 * down-projection ([W^DQ; W^DKV; W^KR] h gives c^KV and k^R of the new token: qiita.com/joule/
 * items/57d9b3f4fc27959eaa0d, "Query の圧縮" and "RoPE の扱い"; "論文解説: DeepSeek-V2 …",
 * "Decoupled RoPE": the cache keeps c^KV and the rotated k^R, 576 elements per token).
 * y is written exactly as mla_linear_deterministic writes it, and the cache rows exactly as
 * mla_kv_append_strided(c_kv = y + append_col, k_r = y + append_col + d_latent, n_new = 1)
 * would write them from that y: row b of y is sequence b, its row
 * [y[b][append_col .. +d_latent) | RoPE(y[b][append_col+d_latent .. +d_rope), pos)] (rounded
 * to bf16) goes to position pos = seq_lens_before[b] through the block table; no other cache
 * byte is written.  One launch fewer than the two calls, with the same bits.
 *   x, w, y, workspace: as mla_linear_deterministic, with M == shape->batch
 *   seq_lens_before [B], block_table [B][max_pages_per_seq]: int32, device
 *   kv_cache: bf16 rows of d_latent + d_rope (cache_dtype must be MLA_BF16)
 * Errors: NULL, SHAPE (as mla_linear_deterministic and check of the paged shape; M !=
 * batch; append_col + d_latent + d_rope > N), UNSUPPORTED (as mla_linear_deterministic; a
 * cache dtype other than BF16; append_col, d_latent or d_rope not a multiple of 4),
 * WORKSPACE. */
mla_status_t mla_linear_deterministic_append(
    const void* x, mla_dtype_t x_dtype, int64_t ldx, const void* w, mla_dtype_t w_dtype,
    int32_t M, int32_t N, int32_t K, float* y, int64_t ldy, void* workspace,
    size_t workspace_bytes, int32_t append_col, const int32_t* seq_lens_before,
    const int32_t* block_table, void* kv_cache, float rope_base, const mla_paged_shape_t* shape,
    mla_dtype_t cache_dtype, void* stream);

/* Device-side check of the paging indices: counts sequences whose seq_len is negative or
 * exceeds max_pages_per_seq*page_size, and referenced block-table entries outside
 * [0, num_pages).  Writes the count to *dev_count (device int32; 0 = valid).
 * Errors: NULL, SHAPE. */
mla_status_t mla_validate_indices(const int32_t* block_table, const int32_t* seq_lens,
                                  const mla_paged_shape_t* shape, int32_t* dev_count,
                                  void* stream);

/* ---------------------------------------------------------------------------------
 * Measurement aid and diagnostics
 * -------------------------------------------------------------------------------*/

/* Streams `bytes` (a multiple of 16) from src and writes one float per workgroup to
 * sink[0 .. 4095] so the reads cannot be elided: a plain read kernel giving the
 * practical HBM read ceiling next to the attention kernel.  Errors: NULL, SHAPE. */
mla_status_t mla_stream_read(const void* src, size_t bytes, float* sink, void* stream);

/* The same measurement with the copy instruction the attention kernels stage cache tiles
 * with (LDS DMA, global_load_lds_dwordx4): one workgroup of 8 wavefronts per compute unit,
 * each wavefront keeping up to 15 one-kilobyte copies in flight; nothing computes on the
 * data.  Writes one float per workgroup to sink[0 .. CUs-1] (the caller provides at least
 * as many floats as the device has compute units).  `bytes` a multiple of 1024, src
 * 16-byte aligned.  Errors: NULL, SHAPE, LAUNCH (device query). */
mla_status_t mla_stream_read_lds(const void* src, size_t bytes, float* sink, void* stream);

/* mla_linear with an explicit kernel and plan, for measurement and for tests that cover
 * each plan: kernel 0 is the tile-grid GEMM (tile = 16-column tiles per wavefront 1, 2 or
 * 4; split = workgroups along k, dividing K / 128; ring = weight k-steps in flight, 4 to 20
 * by 4, turning a whole number of times over a workgroup's chunks), kernel 1 the persistent
 * GEMM (tile as above with N a multiple of 64 tile and M <= 64; split = workgroups, at most
 * 256, dividing the unit count N / (64 tile) * K / 128; ring as above over a workgroup's
 * units); kernel 2 the activation-stationary GEMM (tile 1 or 2 = 128-column tiles of 8
 * wavefronts, M <= 64, N a multiple of 128 tile; ring = k-steps per slice, the slice
 * being 32 ring values of k: 8, 12 or 16 for fp32 x, 8, 16 or 20 for bf16 x (tile 2: 8 or
 * 16); split = workgroups, at most 256, whose runs of tiles stay inside one slice).  Same
 * product, layouts and rounding as mla_linear; bf16 weights only.
 * Errors: NULL, SHAPE, UNSUPPORTED (dtype, or a plan the kernel cannot take). */
mla_status_t mla_linear_planned(const void* x, mla_dtype_t x_dtype, const void* w,
                                mla_dtype_t w_dtype, int32_t M, int32_t N, int32_t K, float* y,
                                int32_t kernel, int32_t tile, int32_t split, int32_t ring,
                                void* stream);

/* Static string for a status code. */
const char* mla_status_string(mla_status_t status);

/* Detail of the last error returned on the calling thread ("" if none). */
const char* mla_last_error_detail(void);

#ifdef __cplusplus
}
#endif

#endif /* MLA_H_ */
