/*
 * mla.h -- C ABI of the MI355X (gfx950) MLA absorbed-decode library.
 *
 * One decode step of one Multi-head Latent Attention layer, in the
 * decoding-stage "MQA form": every head scores the same cached per-token row
 * [c_KV (d_c = 512) | rotated shared RoPE key (d_r = 64)] = 576 values, so the
 * per-head keys and values are never materialised.
 *   Su, "The Ultimate Tug-of-War Between Cache and Performance: From MHA, MQA,
 *   GQA to MLA", MLA Part 3, decoding-stage form (eq:mla-mqa);
 *   Riju, "Multi-Head Latent Attention vs GQA vs MQA", "A latent KV projection
 *   in PyTorch" (absorbed decode sketch) and "Interaction with quantisation
 *   and paging".
 *
 * A step is four calls on one stream:
 *   mla_absorb_q          q[:, :, 0:512]   = q_nope . W_UK          (query absorption)
 *   mla_rope_append_cache q[:, :, 512:576] = RoPE(q_pe, S_b - 1); cache row S_b - 1 written
 *   mla_decode_paged      o_latent = softmax(scale * q . rows^T) . rows[:, 0:512]
 *   mla_absorb_out        o = o_latent . W_UV                      (value absorption)
 *
 * Conventions for every entry point
 *   - Pointers are DEVICE pointers owned by the caller; tensors are dense and
 *     row-major (innermost dimension contiguous), strides implied by the
 *     shapes.  Every tensor pointer must be 16-byte aligned.
 *   - `stream` is a hipStream_t (NULL = the legacy default stream).  Calls only
 *     enqueue work: they never synchronise, copy to the host or allocate.
 *   - Arguments are validated on the host before anything is enqueued; on a
 *     non-zero return nothing was launched.  Values that live in device memory
 *     (seq_lens, block_table) are trusted: out-of-range page ids or lengths
 *     beyond max_seq_len are undefined behaviour.
 *   - bf16 is IEEE binary16-brain (1-8-7); every float -> bf16 conversion
 *     rounds to nearest, ties to even.
 *   - The library holds no global state; calls on different streams are
 *     independent as long as their output buffers do not overlap.
 */
#ifndef MLA_H_
#define MLA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MLA_ABI_VERSION 1

/* Longest chunk (tokens) one decode workgroup handles. */
#define MLA_MAX_SPLIT_TOKENS 131072

/* Status codes. */
enum {
  MLA_OK = 0,
  MLA_ERR_INVALID_ARGUMENT = -1,  /* null/misaligned pointer, non-positive or inconsistent size */
  MLA_ERR_UNSUPPORTED = -2,       /* a size the kernels are not built for (d_c != 512, ...) */
  MLA_ERR_WORKSPACE_TOO_SMALL = -3,
  MLA_ERR_LAUNCH = -4,            /* the HIP runtime rejected a kernel launch */
  MLA_ERR_SCRATCH_TOO_SMALL = -5  /* request exceeds the library's fixed scratch buffer */
};

/* Latent-cache storage formats. */
enum {
  /* bf16 rows of 576 values: [c_KV (512) | rotated k_R (64)], 1152 bytes. */
  MLA_KV_BF16 = 0,
  /* Packed 656-byte rows: [512 e4m3 codes | 64 bf16 rotated k_R | 4 fp32
     scales], one scale per 128-wide group of c_KV; c = code * scale.  OCP
     E4M3 (max 448, no infinity).  The pages store the latent in FP8
     ("Interaction with quantisation and paging") without fixing a layout;
     this packing is this library's. */
  MLA_KV_FP8_E4M3 = 1
};

/* Sizes the kernels are built for.  Other values return MLA_ERR_UNSUPPORTED. */
#define MLA_D_C 512        /* kv_lora_rank */
#define MLA_D_R 64         /* qk_rope_head_dim */
#define MLA_D_NOPE 128     /* qk_nope_head_dim */
#define MLA_D_V 128        /* v_head_dim */
#define MLA_D_Q 1536       /* q_lora_rank: width of the query latent */
#define MLA_BLOCK_SIZE 64  /* tokens per cache page */

/* Human-readable text for a status code (static storage). */
const char *mla_status_string(int status);

/* MLA_ABI_VERSION of the loaded library. */
int mla_abi_version(void);

/*
 * Query absorption: q[b,h,0:d_c] = bf16( sum_k q_nope[b,h,k] * W_UK[h,k,:] ).
 * The content part of every head's score is q_nope W_UK . c, so folding W_UK
 * into the query lets the cached latent c serve as the key (Su, MLA Part 1
 * identity; Riju, "Inside MLA: Absorption").  Evaluated in the sequential
 * order (q_nope first, then W_UK), never through a pre-merged W_UQ W_UK
 * (Su, MLA additional notes 1-2).  fp32 accumulation.
 *   q_nope [B, H, d_nope] bf16     W_UK [H, d_nope, d_c] bf16
 *   q      [B, H, d_c + d_r] bf16  (columns [0, d_c) written, the rest untouched)
 * Requires d_nope == 128, d_c == 512, d_r == 64; B >= 1, H >= 1.
 */
int mla_absorb_q(const void *q_nope, const void *w_uk, void *q,
                 int B, int H, int d_nope, int d_c, int d_r, void *stream);

/*
 * Decoupled RoPE and cache append for the token at position p_b = seq_lens[b]-1
 * (Su, MLA Part 2: the rotary key is shared by all heads and computed from the
 * hidden state; DL0107: it is cached already rotated).  Rotation: interleaved
 * pairs (v[2i], v[2i+1]) turned by p_b * theta^(-2i/d_r) (Riju, rope function in
 * "A latent KV projection in PyTorch"); angles in float64, rotation in float32.
 *   q_pe        [B, H, d_r] bf16, unrotated
 *   kv_new      [B, d_c + d_r] bf16: latent c_KV then the unrotated shared key
 *   seq_lens    [B] int32, counts the token being appended (0 = idle slot)
 *   block_table [B, max_blocks_per_seq] int32: page of tokens [64j, 64j+64)
 *   kv_cache    [num_blocks, block_size, row] in format kv_dtype
 *   q           [B, H, d_c + d_r] bf16: columns [d_c, d_c + d_r) receive RoPE(q_pe, p_b)
 * The row (page block_table[b][p_b / 64], slot p_b % 64) receives
 * [c_KV | RoPE(k_R, p_b)]; for MLA_KV_FP8_E4M3 the latent is quantised per
 * 128-group with scale = amax / 448 (fp32 division; 1 if amax == 0) and
 * code = round-to-nearest-even(c / scale) saturated to +-448.
 * seq_lens[b] == 0: no row is written and the query is rotated at position 0.
 */
int mla_rope_append_cache(const void *q_pe, const void *kv_new, const int32_t *seq_lens,
                          const int32_t *block_table, int max_blocks_per_seq,
                          void *kv_cache, int kv_dtype, int num_blocks, int block_size,
                          float rope_theta, void *q, int B, int H, int d_c, int d_r,
                          void *stream);

/*
 * mla_absorb_q followed by mla_rope_append_cache in a single launch (the
 * query side of one decode step): q[:, :, 0:d_c] = q_nope . W_UK,
 * q[:, :, d_c:d_c+d_r] = RoPE(q_pe, p_b) and the cache row of every sequence
 * appended, with exactly the arithmetic of the two calls (results are
 * bit-identical to them).  Arguments, layouts, requirements and errors are
 * those of the two calls, except that H <= 65527 here (MLA_ERR_UNSUPPORTED
 * above).  Reads of q_pe / kv_new and writes of q / kv_cache must not overlap.
 */
int mla_absorb_q_rope_append(const void *q_nope, const void *w_uk, const void *q_pe, const void *kv_new,
                             const int32_t *seq_lens, const int32_t *block_table, int max_blocks_per_seq,
                             void *kv_cache, int kv_dtype, int num_blocks, int block_size, float rope_theta,
                             void *q, int B, int H, int d_nope, int d_c, int d_r, void *stream);

/*
 * Bytes of the split-KV workspace for these sizes: partial outputs
 * o_part[B][n_chunks][H][512] bf16 followed (at the next 256-byte boundary)
 * by lse_part[B][n_chunks][H] fp32, n_chunks = ceil(max_seq_len / split).
 * split_tokens as passed to the decode calls (0 = library choice).
 * mla_decode_paged needs the workspace only when n_chunks > 1.
 * Returns 0 for invalid sizes or max_seq_len == 0.
 */
size_t mla_decode_workspace_bytes(int B, int H, int max_seq_len, int split_tokens);

/* Split size (tokens) mla_decode_paged uses for split_tokens == 0. */
int mla_decode_split_tokens(int B, int H, int max_seq_len);

/*
 * Checks the device-resident paging values that the other calls trust (a
 * debugging aid; not part of the decode step).  Sequence b is flagged when
 * seq_lens[b] < 0, seq_lens[b] > max_seq_len,
 * seq_lens[b] > max_blocks_per_seq * block_size, or a page it uses,
 * block_table[b][j] for j < ceil(seq_lens[b] / block_size), lies outside
 * [0, num_blocks) (the paged layout of Riju, "Interaction with quantisation
 * and paging": token t of sequence b sits in page block_table[b][t / 64],
 * slot t % 64).
 *   bad        device int32: receives the number of flagged sequences
 *   first_bad  device int32 or NULL: receives the smallest flagged b, -1 if none
 * Asynchronous like every call (read the results after synchronising the
 * stream); one small launch, no atomics, no memset.  Errors: a null seq_lens,
 * block_table or bad, B < 1, max_blocks_per_seq < 1, max_seq_len < 0 or
 * num_blocks < 1 -> MLA_ERR_INVALID_ARGUMENT; block_size != 64 ->
 * MLA_ERR_UNSUPPORTED.
 */
int mla_validate_paging(const int32_t *seq_lens, const int32_t *block_table, int max_blocks_per_seq,
                        int max_seq_len, int num_blocks, int block_size, int B, int32_t *bad,
                        int32_t *first_bad, void *stream);

/*
 * Absorbed decode attention over the paged latent cache (Su, eq:mla-mqa:
 * o^(s) = sum_i exp(q^(s) k_i) c_i / sum_i exp(q^(s) k_i) with the shared key
 * k_i = [c_i | rotated k_R,i]; Riju, absorbed decode sketch):
 *   s[b,h,t]  = softmax_scale * (q[b,h,:] . row_t)            t < seq_lens[b]
 *   o_latent  = sum_t softmax(s)_t row_t[0:d_c],   lse = log sum_t exp(s_t)
 * The row of the newest token (t = seq_lens[b]-1) is included.  Rows are
 * streamed once per head group of up to 128 heads; MFMA with the heads as the
 * matrix dimension, online softmax in fp32, P rounded to bf16 for P.V.
 *   q           [B, H, 576] bf16
 *   kv_cache    as in mla_rope_append_cache, format kv_dtype.  For
 *               MLA_KV_FP8_E4M3 each latent value is expanded in the kernel as
 *               code * scale of its 128-wide group (fp32, then rounded to
 *               bf16) before the same bf16 products; rows of a page past
 *               seq_lens[b] are never used, whatever bytes they hold.
 *   seq_lens    [B] int32, each in [0, max_seq_len]
 *   max_seq_len host-side upper bound on seq_lens (sizes the grid), >= 0,
 *               <= max_blocks_per_seq * block_size
 *   split_tokens tokens per split-KV chunk: 0 = library choice, else a
 *               positive multiple of 64, at most MLA_MAX_SPLIT_TOKENS.  With more than one chunk per
 *               sequence, partial (o, lse) pairs go to the workspace and a
 *               log-sum-exp combine kernel merges them (every choice gives
 *               the same result up to rounding).
 *   workspace   device buffer of at least mla_decode_workspace_bytes(...)
 *               bytes, needed when there is more than one chunk (may be NULL
 *               otherwise); contents on entry ignored.
 *   o_latent    [B, H, 512] bf16 output
 *   lse         [B, H] fp32 natural-log log-sum-exp output, or NULL
 * seq_lens[b] == 0 gives o_latent = 0 and lse = -inf.
 */
int mla_decode_paged(const void *q, const void *kv_cache, int kv_dtype,
                     const int32_t *block_table, int max_blocks_per_seq,
                     const int32_t *seq_lens, int max_seq_len, int num_blocks,
                     int block_size, float softmax_scale, int split_tokens,
                     void *workspace, size_t workspace_bytes,
                     void *o_latent, float *lse, int B, int H, void *stream);

/*
 * The decode query from the low-rank query latent, in one launch: the query
 * path of Su, "The Ultimate Tug-of-War Between Cache and Performance", MLA
 * Part 3 (queries through their own latent c'_i = x_i W_c'), with W_UK
 * absorbed in the sequential order of MLA additional notes 1-2 (never a
 * merged W_UQ W_UK); Riju, "Multi-Head Latent Attention vs GQA vs MQA",
 * "Query compression is separate".  For every sequence b and head h:
 *   q_h            = c_q[b] . w_uq[:, h (d_nope + d_r) : (h + 1) (d_nope + d_r)]
 *   q[b,h,0:d_c]   = q_h[0:d_nope] . w_uk[h]   (fp32 accumulation; q_h enters as the
 *                    sum of two bf16 terms, about 2^-17 relative)
 *   q[b,h,d_c:]    = RoPE(q_h[d_nope:], seq_lens[b] - 1)    (rotated in fp32)
 * and, when kv_new is not NULL, the new token's cache row exactly as
 * mla_rope_append_cache writes it.
 *   c_q         [B, d_q] bf16 query latents (d_q = 1536)
 *   w_uq        [d_q, H (d_nope + d_r)] bf16; head h's columns are
 *               [nope (d_nope) | rope (d_r)]
 *   w_uk        [H, d_nope, d_c] bf16
 *   kv_new      [B, d_c + d_r] bf16 or NULL; with NULL the block_table,
 *               kv_cache, kv_dtype, num_blocks and max_blocks_per_seq
 *               arguments are ignored (may be NULL / 0)
 *   seq_lens    [B] int32, counts the new token (seq_lens[b] = 0: position 0,
 *               no row appended)
 *   q           [B, H, d_c + d_r] bf16 output (all 576 columns written)
 * Errors: as mla_absorb_q_rope_append; d_q != 1536 -> MLA_ERR_UNSUPPORTED.
 */
int mla_query_from_latent(const void *c_q, const void *w_uq, const void *w_uk, const void *kv_new,
                          const int32_t *seq_lens, const int32_t *block_table, int max_blocks_per_seq,
                          void *kv_cache, int kv_dtype, int num_blocks, int block_size, float rope_theta,
                          void *q, int B, int H, int d_q, int d_nope, int d_c, int d_r, void *stream);

/* Bytes of the fixed device scratch buffer behind mla_decode_paged_noalloc. */
#define MLA_NOALLOC_SCRATCH_BYTES (72u << 20)

/*
 * mla_decode_paged without a caller workspace, for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc.  Same arguments, arithmetic, kernels and
 * results as mla_decode_paged; the split-KV partials go to a file-scope
 * device array of MLA_NOALLOC_SCRATCH_BYTES (72 MiB; holds the partials of
 * 128 heads x 128 chunks x 4 sequences or 8 chunks x 32 sequences) that
 * each GPU the library runs on keeps until the process ends.  The call
 * allocates nothing: no hipMalloc, hipFree or allocating library routine.
 * Every call on one GPU shares that GPU's buffer and leaves its partials
 * there; nothing in it needs to start at zero.  Calls that overlap on one
 * GPU (concurrent streams, or host threads) race on it: order them on one
 * stream.  Errors: as mla_decode_paged, plus MLA_ERR_SCRATCH_TOO_SMALL when
 * the partials, mla_decode_workspace_bytes(B, H, max_seq_len,
 * split_tokens), exceed the buffer (nothing is launched); MLA_ERR_LAUNCH if
 * the buffer's device address cannot be obtained.
 */
int mla_decode_paged_noalloc(const void *q, const void *kv_cache, int kv_dtype,
                             const int32_t *block_table, int max_blocks_per_seq,
                             const int32_t *seq_lens, int max_seq_len, int num_blocks,
                             int block_size, float softmax_scale, int split_tokens,
                             void *o_latent, float *lse, int B, int H, void *stream);

/*
 * mla_decode_paged for the fp8 cache (kv_dtype MLA_KV_FP8_E4M3) with both
 * products on fp8 matrix instructions over the stored E4M3 codes, which are
 * never expanded to bf16.  The scores and the weighted sum regroup by scale
 * group (Riju, "Interaction with quantisation and paging", the per-group
 * scales of the fp8 cache; Su, MLA Part 3, eq:mla-mqa):
 *   q . k_t = sum_g sc[t,g] (q_g . code[t,g]) + q_R . kr_t,
 *   o[g]    = sum_t (p_t sc[t,g]) code[t,g] / sum_t p_t,
 * with the query and the weights p_t sc[t,g] each carried as two E4M3 terms
 * (hi + lo, about bf16 precision), products accumulated in fp32.  Same
 * arguments, outputs, split choice, workspace and errors as
 * mla_decode_paged; results agree with it to the fp8-cache tolerance, not
 * bit for bit.  MLA_ERR_UNSUPPORTED for a bf16 cache.
 */
int mla_decode_paged_fp8_mfma(const void *q, const void *kv_cache, int kv_dtype,
                              const int32_t *block_table, int max_blocks_per_seq,
                              const int32_t *seq_lens, int max_seq_len, int num_blocks,
                              int block_size, float softmax_scale, int split_tokens,
                              void *workspace, size_t workspace_bytes, void *o_latent,
                              float *lse, int B, int H, void *stream);

/* Most new tokens per sequence that mla_decode_paged_multi takes. */
#define MLA_MAX_Q_LEN 32

/*
 * Multi-token decode: q_len new tokens per sequence (speculative decoding,
 * multi-token prediction heads) in one pass over the cache.  Such tokens use
 * the latent cache like any other decode (Riju, "Interaction with
 * quantisation and paging"); they attend causally among themselves, the rule
 * of decoder attention (Su, MHA equation with the causal mask).  The new
 * tokens are the last q_len rows of each sequence (already appended and
 * counted in seq_lens); query j sits at position seq_lens[b] - q_len + j and
 * sees the rows t <= seq_lens[b] - q_len + j:
 *   s[b,j,h,t]      = softmax_scale * (q[b,j,h,:] . row_t)
 *   o_latent[b,j,h] = sum_t softmax(s)_t row_t[0:d_c],  lse = log sum_t exp(s_t)
 *   q          [B, q_len, H, 576] bf16
 *   o_latent   [B, q_len, H, 512] bf16 output
 *   lse        [B, q_len, H] fp32 natural-log output, or NULL
 *   q_len      1 .. MLA_MAX_Q_LEN (1 gives mla_decode_paged's results)
 * Every other argument is as for mla_decode_paged, with R = q_len * H query
 * rows in place of H for the split choice and the workspace: split_tokens 0
 * means mla_decode_split_tokens(B, R, max_seq_len), and the workspace needs
 * mla_decode_workspace_bytes(B, R, max_seq_len, split_tokens) bytes.  A
 * query that sees no row (seq_lens[b] - q_len + j < 0) gives zeros and
 * lse = -inf.  The rows of a chunk are read once for up to 128 query rows;
 * above that, the workgroups of one chunk are numbered to run side by side
 * on one XCD, where their reads share the L2.  The query side of such a step
 * is the single-token calls on B * q_len virtual sequences: sequence (b, j)
 * of length seq_lens[b] - q_len + j + 1 with block-table row b.
 * Errors: MLA_ERR_INVALID_ARGUMENT for q_len < 1 and as mla_decode_paged;
 * MLA_ERR_UNSUPPORTED for q_len > MLA_MAX_Q_LEN.
 */
int mla_decode_paged_multi(const void *q, const void *kv_cache, int kv_dtype,
                           const int32_t *block_table, int max_blocks_per_seq,
                           const int32_t *seq_lens, int max_seq_len, int num_blocks,
                           int block_size, float softmax_scale, int split_tokens,
                           void *workspace, size_t workspace_bytes,
                           void *o_latent, float *lse, int B, int H, int q_len, void *stream);

/*
 * The two halves of mla_decode_paged, for callers that merge chunks
 * themselves (e.g. chunks computed on different devices, which is the same
 * log-sum-exp merge).
 *
 * mla_decode_partial: attention of every head over each chunk of split_tokens
 * tokens; writes o_part = (sum_t e^{s_t - m} row_t[0:512]) / (sum_t e^{s_t - m})
 * rounded to bf16 and lse_part = m + log sum_t e^{s_t - m} (natural log, fp32)
 * into the workspace layout above.  Chunks that start at or beyond seq_lens[b] are not written.
 * Arguments as for mla_decode_paged.
 *
 * mla_decode_combine: o_latent[b,h] = sum_c w_c o_part[b,c,h] / sum_c w_c with
 * w_c = exp(lse_part[b,c,h] - max_c lse_part), over the first
 * ceil(seq_lens[b] / split) chunks; lse = max + log sum_c w_c.  An empty
 * sequence gives zeros and lse = -inf.  split_tokens must be the value used
 * for the partial call (0 = library choice, resolved identically).
 */
int mla_decode_partial(const void *q, const void *kv_cache, int kv_dtype,
                       const int32_t *block_table, int max_blocks_per_seq,
                       const int32_t *seq_lens, int max_seq_len, int num_blocks,
                       int block_size, float softmax_scale, int split_tokens,
                       void *workspace, size_t workspace_bytes, int B, int H, void *stream);

int mla_decode_combine(const void *workspace, size_t workspace_bytes, const int32_t *seq_lens,
                       int max_seq_len, int split_tokens, void *o_latent, float *lse,
                       int B, int H, void *stream);

/*
 * Value absorption: o[b,h,:] = bf16( sum_c o_latent[b,h,c] * W_UV[h,c,:] ).
 * The per-head value up-projection applied after the latent-weighted sum
 * (Su, eq:mla-mqa first line: o_t = [o^(1) W_v^(1), ..., o^(h) W_v^(h)];
 * Riju, "Inside MLA: Absorption").  The output projection W_O is the caller's.
 *   o_latent [B, H, d_c] bf16   W_UV [H, d_c, d_v] bf16   o [B, H, d_v] bf16
 * Requires d_c == 512, d_v == 128.
 */
int mla_absorb_out(const void *o_latent, const void *w_uv, void *o,
                   int B, int H, int d_c, int d_v, void *stream);

/*
 * mla_decode_combine followed by mla_absorb_out in one launch: the chunk
 * merge of the log-sum-exp combine feeds the value up-projection directly,
 * so the merged latent output need not go through memory (Su, eq:mla-mqa
 * first line; Riju, "Inside MLA: Absorption").  Results are those of the two
 * separate calls.
 *   workspace, workspace_bytes, seq_lens, max_seq_len, split_tokens
 *            as for mla_decode_combine (split_tokens = the partial call's)
 *   w_uv     [H, 512, 128] bf16
 *   o        [B, H, 128] bf16 output
 *   o_latent [B, H, 512] bf16 merged latent output, or NULL to skip it
 *   lse      [B, H] fp32 output, or NULL
 * Requires d_c == 512, d_v == 128, H <= 65535.  An empty sequence gives
 * o = 0 (and o_latent = 0, lse = -inf).
 */
int mla_decode_combine_absorb_out(const void *workspace, size_t workspace_bytes,
                                  const int32_t *seq_lens, int max_seq_len, int split_tokens,
                                  const void *w_uv, void *o, void *o_latent, float *lse,
                                  int B, int H, int d_c, int d_v, void *stream);

/*
 * Prefill of whole prompts in the explicit (non-absorbed) form, which needs
 * (192 + 128) / (576 + 512) of the absorbed form's attention FLOPs (Su, Part
 * 3: the MHA form eq:mla-mha for prefill, the MQA form for decoding; Riju,
 * non-absorbed module).  Prompt b is tokens cu_seqlens[b] ..
 * cu_seqlens[b + 1] - 1 of the packed inputs, token t of a prompt at position
 * t; for every head h
 *   K^(h) = [c W_UK[h]^T | RoPE(k_pe)],  V^(h) = c W_UV[h]
 *   o[t,h] = sum_{i <= t} softmax_i(softmax_scale [q_nope | RoPE(q_pe)]_t . K_i^(h)) V_i^(h)
 * and row t of prompt b, [c_t | RoPE(k_pe_t, t)], is written to the paged
 * cache at position t of block-table row b (bf16, or fp8 quantised as in
 * mla_rope_append_cache), ready for the decode steps.
 *   q_nope      [T, H, 128] bf16        q_pe  [T, H, 64] bf16 (unrotated)
 *   c_kv        [T, 512] bf16 latents   k_pe  [T, 64] bf16 (unrotated)
 *   w_uk        [H, 128, 512] bf16      w_uv  [H, 512, 128] bf16
 *   cu_seqlens  [B + 1] int32 device, non-decreasing, cu_seqlens[0] = 0,
 *               cu_seqlens[B] = total_tokens (T); host bounds: max_seqlen >=
 *               every prompt length, <= max_blocks_per_seq * block_size
 *   kv_cache, kv_dtype, block_table, num_blocks, block_size as for
 *               mla_rope_append_cache
 *   o           [T, H, 128] bf16 output
 *   workspace   device buffer of mla_prefill_workspace_bytes(T, H) bytes
 *               (rotated queries and keys, per-head K and V)
 * Empty prompts write nothing.  Errors as for the decode calls.
 * Precision: the attention runs on IEEE-half operands with fp32
 * accumulation (rotated query and key, K_nope, V and the softmax weights),
 * so per-head queries, keys and values must stay below 65504 in magnitude;
 * larger values overflow to infinity.
 */
size_t mla_prefill_workspace_bytes(int total_tokens, int H);

int mla_prefill(const void *q_nope, const void *q_pe, const void *c_kv, const void *k_pe,
                const void *w_uk, const void *w_uv, const int32_t *cu_seqlens, int B,
                int total_tokens, int max_seqlen, int H, float softmax_scale, float rope_theta,
                const int32_t *block_table, int max_blocks_per_seq, void *kv_cache, int kv_dtype,
                int num_blocks, int block_size, void *o, void *workspace, size_t workspace_bytes,
                void *stream);

/*
 * A prefill chunk that continues a cached prefix (chunked prefill; the
 * prefill and the decode share one cache: Riju, "Prefill versus decode"
 * and "Interaction with quantisation and paging").  Prompt b already has
 * P_b = prefix_lens[b] rows in the paged cache (positions 0 .. P_b - 1 of
 * block-table row b, written by mla_prefill, mla_prefill_chunk or the
 * decode's appends); its chunk is tokens cu_seqlens[b] .. cu_seqlens[b+1]-1
 * of the packed inputs, token j at position P_b + j.  In the explicit form
 * of mla_prefill (Su, Part 3, eq:mla-mha, with the causal rule of the MHA
 * equation), for every head h
 *   K^(h) = [[c_prefix; c] W_UK[h]^T | [kr_prefix; RoPE(k_pe, P_b + j)]],
 *   V^(h) = [c_prefix; c] W_UV[h]
 *   o[j,h] = sum_{i <= P_b + j} softmax_i(softmax_scale [q_nope | RoPE(q_pe, P_b + j)]_j . K_i^(h)) V_i^(h)
 * where c_prefix, kr_prefix are the cached rows (fp8 rows dequantised as
 * code * group scale and carried into the up-projection as two bf16 terms,
 * within 2^-17 of the exact value), and the chunk's rows
 * [c_j | RoPE(k_pe_j, P_b + j)] are written at positions P_b + j.
 * Arguments as for mla_prefill, plus:
 *   prefix_lens  [B] int32 device: cached rows per prompt
 *   total_keys   host: sum_b (prefix_lens[b] + chunk length b), the keys the
 *                attention materialises per head (the workspace is sized for
 *                it; a wrong value gives unspecified results, while every
 *                access stays inside the workspace)
 *   max_prefix   host bound >= every prefix_lens[b], <= max_blocks_per_seq *
 *                block_size; each prompt's prefix plus chunk must fit its
 *                block-table row (prefix_lens[b] + chunk length b <=
 *                max_blocks_per_seq * block_size)
 *   workspace    mla_prefill_chunk_workspace_bytes(T, total_keys, B, H)
 *                bytes (per-head K and V of every key: 512 bytes per key
 *                and head)
 * With every prefix_lens[b] = 0 the results equal mla_prefill's.  Errors as
 * for mla_prefill.
 */
size_t mla_prefill_chunk_workspace_bytes(int total_tokens, int total_keys, int B, int H);

int mla_prefill_chunk(const void *q_nope, const void *q_pe, const void *c_kv, const void *k_pe,
                      const void *w_uk, const void *w_uv, const int32_t *cu_seqlens,
                      const int32_t *prefix_lens, int B, int total_tokens, int max_seqlen,
                      int total_keys, int max_prefix, int H, float softmax_scale, float rope_theta,
                      const int32_t *block_table, int max_blocks_per_seq, void *kv_cache,
                      int kv_dtype, int num_blocks, int block_size, void *o, void *workspace,
                      size_t workspace_bytes, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* MLA_H_ */
