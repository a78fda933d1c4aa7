/*
 * mla_absorb.h -- C ABI of the MI355X (gfx950) absorbed-MLA decode library.
 *
 * One decode step of DeepSeek Multi-head Latent Attention in "absorb" mode,
 * for one layer, split into four calls that launch hand-written HIP kernels
 * on the caller's stream:
 *
 *   mla_absorb_q        q_lat[b,h,:]  = q_nope[b,h,:] . W_UK[h]            (key absorption)
 *   mla_decode_latent   scores of every head against the shared 576-wide
 *                       latent cache (512 latent + 64 decoupled-RoPE key),
 *                       online softmax, o_lat = sum_t p_t c_t in latent space
 *   mla_combine_splits  log-sum-exp merge of split-KV partial results
 *   mla_expand_v        out[b,h,:] = W_UV[h] . o_lat[b,h,:]                 (value absorption)
 *
 * (mla_combine_expand_v runs the last two in one launch), and
 * mla_cache_append, which writes new tokens (latent row + rotated RoPE
 * key, bf16 or E4M3 with a per-token scale) into the cache that decode reads,
 * and mla_decode_step_fused, the three decode stages in one launch for short
 * contexts, and mla_naive_decode, the expand-every-step baseline.
 *
 * The method is the one described on the source pages (cited by title):
 *   [AUDIT]  "DeepSeek MLA 吸收式缓存：真实权重执行与 FlashMLA 架构边界":
 *            §2.2 moves W_UK onto the query, §2.3 applies W_UV after the
 *            latent aggregation, §2.4 keeps the 64-wide RoPE key cached
 *            separately, §6.1 describes absorbed decode as MQA with a
 *            576-wide key and a 512-wide value.
 *   [MLA80]  "80 行 PyTorch 从零写 DeepSeek 的 MLA ..." §4-§5: the absorbed
 *            decode (Q_abs = q . W_UK, content + rope scores, latent context
 *            then W_UV).
 *   [G5SPEC] "G5 MLA KV 访存建模设计规格": eq:gmkv-cache (bytes per cached
 *            token), eq:gmkv-read (bytes one decode step reads, no head
 *            term), and Appendix C (required fields, error naming the field).
 *
 * Conventions shared by every call
 * --------------------------------
 * - Pointers named "device" are HIP device pointers; the library never
 *   dereferences them on the host.  All device buffers are owned by the
 *   caller, who allocates and frees them; the library allocates and frees
 *   no device memory, keeps no state between calls and never synchronises
 *   (only the host planner mla_plan_decode_splits uses temporary host memory
 *   while it runs).
 * - `stream` is a hipStream_t passed as void* (NULL = the default stream).
 *   Every kernel is launched asynchronously on it.
 * - bf16 = IEEE bfloat16 stored as uint16; fp8 = OCP FP8 E4M3 ("FN") stored
 *   as uint8; fp32 = IEEE binary32.
 * - Every argument check runs on the host before anything is launched.  On
 *   failure the call returns a non-zero mla_status, launches nothing, and
 *   mla_last_error() returns a message naming the offending field.  The
 *   message is thread-local and stays valid until the next call on the same
 *   thread.
 * - Dimensions have no defaults: a zero or missing dimension is
 *   MLA_ERR_MISSING_DIM, never silently replaced ([G5SPEC] constraints).
 * - Supported shapes: kv_lora_rank 512, qk_rope_head_dim 64,
 *   qk_nope_head_dim 128, v_head_dim 128, num_heads in {16, 32, 64, 128}.
 *   Others return MLA_ERR_UNSUPPORTED.
 * - Device pointers to bf16/fp8/fp32 tensors must be 16-byte aligned.
 */
#ifndef MLA_ABSORB_H
#define MLA_ABSORB_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MLA_OK = 0,
  MLA_ERR_NULL = 1,          /* a required pointer is NULL                    */
  MLA_ERR_MISSING_DIM = 2,   /* a required dimension is zero / missing        */
  MLA_ERR_UNSUPPORTED = 3,   /* a shape or option this library does not build */
  MLA_ERR_BAD_LENGTH = 4,    /* max_seq_len / split / block-size arguments    */
  MLA_ERR_BUFFER = 5,        /* inconsistent buffer description               */
  MLA_ERR_ALIGN = 6,         /* pointer or stride not 16-byte aligned         */
  MLA_ERR_HIP = 7            /* the HIP runtime reported an error at launch   */
} mla_status;

typedef enum {
  MLA_DTYPE_BF16 = 0,        /* cache elements are bfloat16                   */
  MLA_DTYPE_FP8_E4M3 = 1     /* cache elements are E4M3 with a per-token fp32
                                scale: value = e4m3(code) * token_scale[slot] */
} mla_dtype;

/* Shape of one MLA attention layer.  All fields are required. */
typedef struct mla_dims {
  int32_t batch;             /* B: sequences decoded in this step            */
  int32_t num_heads;         /* H: query heads (16, 32, 64 or 128)           */
  int32_t kv_lora_rank;      /* d_c: latent width, must be 512              */
  int32_t qk_rope_head_dim;  /* d_r: decoupled RoPE key width, must be 64    */
  int32_t qk_nope_head_dim;  /* d_n: per-head no-RoPE query width, 128       */
  int32_t v_head_dim;        /* d_v: per-head value width, 128               */
  float softmax_scale;       /* multiplies q.k before the softmax; > 0       */
} mla_dims;

/*
 * Where the cached rows of the latent cache live.
 *
 * Token t of sequence b is stored in "slot"
 *     slot = b * seq_stride + t                                   (contiguous)
 *     slot = block_table[b * max_blocks_per_seq + t / block_size]
 *              * block_size + t % block_size                      (paged)
 * Its 512 latent elements start at kv + slot * kv_stride and its 64 RoPE-key
 * elements at pe + slot * pe_stride (strides in elements; multiples of 16
 * bytes: 8 bf16 or 16 E4M3 elements, else MLA_ERR_BUFFER).  A fused
 * [.., 576] row layout is kv = base, pe = base + 512, both strides 576.
 * The RoPE half holds keys that are already rotated.
 *
 * Paged mode: block_table is a device int32 array [batch, max_blocks_per_seq]
 * of physical block ids; block_size must be a positive multiple of 32.  Only
 * entries covering tokens < seq_lens[b] are read.  Contiguous mode: block_table
 * is NULL and seq_stride >= every seq_lens[b].
 */
typedef struct mla_cache {
  int32_t dtype;               /* mla_dtype                                   */
  const void *kv;              /* device: latent element 0 of slot 0          */
  const void *pe;              /* device: RoPE-key element 0 of slot 0        */
  int64_t kv_stride;           /* elements between consecutive slots (kv)     */
  int64_t pe_stride;           /* elements between consecutive slots (pe)     */
  const float *token_scale;    /* device [num_slots] fp32, fp8 only, else NULL*/
  int64_t seq_stride;          /* contiguous: slots per sequence              */
  const int32_t *block_table;  /* device, paged only; NULL = contiguous       */
  int32_t block_size;          /* paged: tokens per block                     */
  int32_t max_blocks_per_seq;  /* paged: row length of block_table            */
} mla_cache;

/* Message for the last failed call on this thread ("" after success). */
const char *mla_last_error(void);

/* Library version string. */
const char *mla_version(void);

/*
 * Bytes one cached token occupies in one layer: (d_c + d_r) * e, plus 4 for
 * the fp32 token scale of an fp8 cache ([G5SPEC] eq:gmkv-cache).  Only
 * dims->kv_lora_rank and dims->qk_rope_head_dim are read; both are required.
 * Host-only; launches nothing.
 */
mla_status mla_kv_cache_bytes(const mla_dims *dims, int32_t dtype, size_t *bytes_per_token);

/*
 * Bytes one decode step reads from the latent cache of one layer:
 * sum_b seq_lens[b] * bytes_per_token ([G5SPEC] eq:gmkv-read; no head term).
 * host_seq_lens is a HOST array of dims->batch lengths.  Host-only.
 */
mla_status mla_decode_kv_read_bytes(const mla_dims *dims, int32_t dtype, const int32_t *host_seq_lens,
                                    size_t *bytes);

/*
 * Key absorption ([AUDIT] §2.2): q_lat[b,h,c] = sum_d q_nope[b,h,d] * W_UK[h,d,c],
 * fp32 accumulation, rounded to bf16.
 *   q_nope  device bf16 [B, H, 128]
 *   w_uk    device bf16 [H, 128, 512]
 *   q_lat   device bf16 [B, H, 512] (output)
 */
mla_status mla_absorb_q(const mla_dims *dims, const void *q_nope, const void *w_uk, void *q_lat,
                        void *stream);

/*
 * Latent attention ([AUDIT] §2.2-§2.4, §6.1): for every sequence b and head h
 *   s_t     = softmax_scale * (q_lat[b,h] . c_t + q_pe[b,h] . kR_t),  t < seq_lens[b]
 *   o_lat   = sum_t softmax(s)_t * c_t          (512 wide, latent space)
 *   lse     = ln sum_t exp(s_t)
 * The decode query attends to every cached token of its sequence.
 *
 *   q_lat     device bf16 [B, H, 512]
 *   q_pe      device bf16 [B, H, 64]   (already rotated)
 *   seq_lens  device int32 [B], each in [1, max_seq_len]
 *   max_seq_len  host int: an upper bound of seq_lens, sizes the launch
 *   num_splits   P >= 1.  Split-KV: token range of split i is
 *                [i*chunk, min((i+1)*chunk, seq_lens[b])) with
 *                chunk = 32 * ceil(ceil(max_seq_len / P) / 32).
 *   P == 1: writes o_lat (device bf16 [B, H, 512]) and lse (device fp32 [B, H]);
 *           o_part / lse_part must be NULL.
 *   P  > 1: writes o_part (device bf16 [B, P, H, 512], each split normalised
 *           by its own softmax sum) and lse_part (device fp32 [B, P, H]); an
 *           empty split gets o = 0 and lse = -inf.  o_lat / lse must be NULL;
 *           merge with mla_combine_splits.
 * Precision choices (differences from a design with fp32 partials and an
 * fp8 query): the partials are bf16, since each split's o_i is a normalised
 * average with the relative rounding error of the bf16 o_lat, and there is
 * no query scale argument, since the queries stay bf16 for every cache dtype.
 * E4M3 cache (mla_cache.dtype = MLA_DTYPE_FP8_E4M3): the stored codes enter
 * the products exactly and the token scale in fp32:
 * s_t = softmax_scale * token_scale[slot] * (q . code_t).
 *   16, 32 or 64 heads: bf16 products (every E4M3 value is a bf16 value); the
 *   probability multiplying code_t in P.V is p_t * token_scale[slot], rounded
 *   to bf16 as p_t alone is for a bf16 cache.
 *   128 heads: fp8 matrix products on the codes.  q . code_t is computed with
 *   the bf16 query split into two E4M3 parts (hi + lo / 16, scaled per head),
 *   which carries the query's bf16 precision.  The P.V weights
 *   p_t * token_scale[slot] are E4M3 with a power-of-two scale per (head, 32
 *   tokens), set from a bound (the largest p_t times the largest token scale
 *   of the 32) so that the largest weight is below 256; o is normalised by
 *   the sum of the weights as stored, each over its token scale, except that
 *   a token whose scale is 0 or below 2^-6 of the largest of its 32 counts
 *   at its exact p_t; so o_lat is a convex combination of the cached rows,
 *   within the fp8 tolerance of the exact result; lse keeps the exact sum
 *   of p_t.
 * The queries stay bf16.  token_scale must then be non-NULL (4-byte aligned),
 * else MLA_ERR_NULL; a bf16 cache must pass token_scale = NULL
 * (MLA_ERR_BUFFER).
 */
mla_status mla_decode_latent(const mla_dims *dims, const mla_cache *cache, const void *q_lat,
                             const void *q_pe, const int32_t *seq_lens, int32_t max_seq_len,
                             int32_t num_splits, void *o_part, float *lse_part, void *o_lat,
                             float *lse, void *stream);

/*
 * mla_decode_latent followed by mla_combine_splits, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc): the split partials live in a device
 * array of the library (48 MiB per GPU, held until the process ends), so the
 * call allocates nothing; the caller passes inputs and outputs only.
 *   arguments as mla_decode_latent; o_lat device bf16 [B, H, 512] and lse
 *   device fp32 [B, H] are always written (num_splits == 1: directly).
 * Errors: MLA_ERR_BUFFER when batch * num_splits * num_heads partial rows
 * (1,024 + 4 bytes each) exceed the array; MLA_ERR_HIP if its device address
 * cannot be obtained.  Every call on one GPU uses that GPU's one array: calls
 * that overlap on one GPU (other streams, other threads) race; serialise them.
 * Results equal mla_decode_latent + mla_combine_splits bit for bit.
 */
mla_status mla_decode_latent_noalloc(const mla_dims *dims, const mla_cache *cache, const void *q_lat,
                                     const void *q_pe, const int32_t *seq_lens, int32_t max_seq_len,
                                     int32_t num_splits, void *o_lat, float *lse, void *stream);

/*
 * Absorbed chunked prefill ([MLA80] §2 cache test and §5: prefill, then
 * decode against the cache; [AUDIT] §2.2-§2.4: absorbed scores and latent
 * aggregation; [G5SPEC] use case 2: prefill is compute-bound): num_q query
 * tokens per sequence at positions q_start[b] + i, i < num_q, each attending
 * causally to the cached tokens 0 .. q_start[b] + i (its own row included, so
 * the chunk must be in the cache already, e.g. by mla_cache_append):
 *   s_t   = softmax_scale * (q_lat[b,i,h] . c_t + q_pe[b,i,h] . kR_t)
 *   o_lat[b,i,h] = sum_t softmax(s)_t c_t,  lse[b,i,h] = ln sum_t exp(s_t)
 *   q_lat   device bf16 [B, num_q, H, 512]  (mla_absorb_q with batch B*num_q)
 *   q_pe    device bf16 [B, num_q, H, 64]   (rotated at each query's position)
 *   q_start device int32 [B], each >= 0 (a negative start is taken as 0)
 *   max_seq_len  host bound of q_start[b] + num_q (positions past it are
 *                clamped to it); sizes the split chunks as in decode
 *   num_splits, o_part, lse_part, o_lat, lse: as mla_decode_latent with B*num_q
 *                query rows (o_lat [B, num_q, H, 512], partials
 *                [B*num_q, P, H, 512], merged by mla_combine_splits with batch
 *                B*num_q)
 * Each query runs the decode kernel's schedule over its own causal prefix:
 * with 128 heads one workgroup per query; with fewer heads, a bf16 cache
 * and one split, 128 / H consecutive queries of a sequence share a
 * workgroup (128 rows per 576-wide tile of cached rows).  The projections
 * around it are mla_absorb_q / mla_expand_v with batch B*num_q.
 */
mla_status mla_prefill_latent(const mla_dims *dims, const mla_cache *cache, const void *q_lat, const void *q_pe,
                              const int32_t *q_start, int32_t num_q, int32_t max_seq_len, int32_t num_splits,
                              void *o_part, float *lse_part, void *o_lat, float *lse, void *stream);

/*
 * Split-KV merge ([G5SPEC] Appendix B: the cache is read concurrently by
 * several workers and their attention results combined; the merge is the
 * log-sum-exp identity of softmax over a union of token ranges):
 * LSE = ln sum_i exp(lse_part[b,i,h]),
 * o_lat[b,h] = sum_i exp(lse_part[b,i,h] - LSE) * o_part[b,i,h]; splits with
 * lse = -inf carry no weight.
 *   o_part device bf16 [B, P, H, 512], lse_part device fp32 [B, P, H]
 *   (weights and sums in fp32)
 *   o_lat  device bf16 [B, H, 512] (output), lse device fp32 [B, H] (output,
 *          may be NULL)
 */
mla_status mla_combine_splits(const mla_dims *dims, const void *o_part, const float *lse_part,
                              int32_t num_splits, void *o_lat, float *lse, void *stream);

/*
 * Value absorption ([AUDIT] §2.3): out[b,h,j] = sum_c W_UV[h,j,c] * o_lat[b,h,c],
 * fp32 accumulation, rounded to bf16.
 *   o_lat device bf16 [B, H, 512]
 *   w_uv  device bf16 [H, 128, 512]
 *   out   device bf16 [B, H, 128] (output)
 */
mla_status mla_expand_v(const mla_dims *dims, const void *o_lat, const void *w_uv, void *out,
                        void *stream);

/*
 * Split-KV merge and value absorption in one launch ([AUDIT] §2.3: W_UV is
 * applied after the latent aggregation): the result of mla_combine_splits
 * followed by mla_expand_v, with the same arithmetic (the merged row is
 * rounded to bf16 before the W_UV product), so out, o_lat and lse equal the
 * two calls' bit for bit.
 *   o_part, lse_part, num_splits  as mla_combine_splits
 *   w_uv   device bf16 [H, 128, 512]
 *   out    device bf16 [B, H, 128] (output)
 *   o_lat  device bf16 [B, H, 512] (output, may be NULL)
 *   lse    device fp32 [B, H] (output, may be NULL)
 * One workgroup per (head, up to 32 sequences): W_UV[h] and the partial rows
 * are read once, and o_lat need not make a round trip through memory.
 */
mla_status mla_combine_expand_v(const mla_dims *dims, const void *o_part, const float *lse_part,
                                int32_t num_splits, const void *w_uv, void *out, void *o_lat, float *lse,
                                void *stream);

/*
 * Fused decode step for short contexts: mla_absorb_q, mla_decode_latent with
 * one split, and mla_expand_v in ONE launch ([AUDIT] §2.2-§2.4; [MLA80]
 * §4-§5), for shapes where launch latency dominates (a few sequences with
 * short contexts).
 *   q_nope  device bf16 [B, H, 128]      w_uk  device bf16 [H, 128, 512]
 *   q_pe    device bf16 [B, H, 64]       w_uv  device bf16 [H, 128, 512]
 *   seq_lens device int32 [B], max_seq_len as in mla_decode_latent
 *   out     device bf16 [B, H, 128] (output)
 *   o_lat   device bf16 [B, H, 512] (output, may be NULL)
 *   lse     device fp32 [B, H] (output, may be NULL)
 * Same result as the three calls up to rounding: q_lat and o_lat stay fp32
 * between the stages (the three-call path rounds them to bf16), and every
 * dot product is an fp32 sum.  One workgroup per (sequence, head) streams
 * that sequence's rows, so the cost grows with H * context: long contexts
 * belong to the split-KV mla_decode_latent.  The cache, sequence-length and
 * error rules are those of mla_decode_latent (no split arguments).
 */
mla_status mla_decode_step_fused(const mla_dims *dims, const mla_cache *cache, const void *q_nope, const void *q_pe,
                                 const void *w_uk, const void *w_uv, const int32_t *seq_lens, int32_t max_seq_len,
                                 void *out, void *o_lat, float *lse, void *stream);

/*
 * Naive decode, the baseline the absorbed path is compared with ([MLA80] §4
 * path A and §5: the base decode re-applies the up-projections to the whole
 * latent cache every step; [AUDIT] §2: per-head expanded keys and values).
 * Every step expands each cached token t < seq_lens[b] into
 *   k_nope[t,h] = W_UK[h] c_t,  v[t,h] = W_UV[h] c_t      (bf16, in workspace)
 * and runs multi-head attention with keys [k_nope[t,h] | kR_t] and values
 * v[t,h]: out[b,h] = sum_t softmax_t(softmax_scale * (q_nope . k_nope +
 * q_pe . kR_t)) v[t,h].  Same result as the absorbed path up to rounding.
 *   q_nope, q_pe, w_uk, w_uv, seq_lens, max_seq_len, cache: as in
 *     mla_absorb_q / mla_decode_latent / mla_expand_v
 *   workspace  device, at least mla_naive_workspace_bytes() bytes: the
 *              expanded rows [B, max_seq_len, H, 256] bf16 (k_nope | v),
 *              owned by the caller and overwritten
 *   out        device bf16 [B, H, 128] (output)
 * Two launches (an expansion GEMM on 32x32x16 bf16 MFMAs, then attention).
 * batch must be at most 65535.
 */
mla_status mla_naive_workspace_bytes(const mla_dims *dims, int32_t max_seq_len, size_t *bytes);
mla_status mla_naive_decode(const mla_dims *dims, const mla_cache *cache, const void *q_nope, const void *q_pe,
                            const void *w_uk, const void *w_uv, const int32_t *seq_lens, int32_t max_seq_len,
                            void *workspace, size_t workspace_bytes, void *out, void *stream);

/*
 * Cache append: writes num_new new tokens of every sequence into the latent
 * cache.  Each input row is the token's fused down-projection output: 512
 * latent values, then the 64-wide decoupled RoPE key BEFORE rotation ([AUDIT]
 * §2.4: the RoPE key is cached separately, rotated; [MLA80] §2 and Appendix
 * A: interleaved pairs (2i, 2i+1) turned by position * rope_base^(-2i/64)).
 * Token j of sequence b has position positions[b] + j and is stored in that
 * position's slot (addressing as in mla_cache above; contiguous:
 * b * seq_stride + position, paged: through block_table).
 *
 *   kv_in      device bf16 [B, num_new, in_stride]; elements 0..575 of a row
 *              are used; in_stride >= 576 and a multiple of 8 elements
 *   positions  device int32 [B]
 *   num_new    tokens per sequence (0 = nothing to do, no launch)
 *   rope_base  > 0, required (DeepSeek uses 10000)
 *
 * bf16 cache: the latent half is copied bit for bit; the key is rotated in
 * fp64 and rounded fp64 -> fp32 -> bf16 (nearest even at each step).
 * E4M3 cache: the token's 576 values in fp32 (latent exact, rotated key
 * rounded to fp32) share one scale = max(max|x| / 448, FLT_MIN), computed in
 * fp32 and written to token_scale[slot]; each code is the OCP E4M3 value
 * nearest to x / scale (IEEE fp32 division, clamped to +-448), ties to the
 * even code ([G5SPEC] use case 1: 576 one-byte elements plus an fp32 scale
 * per token).  Inputs must be finite.
 *
 * The call WRITES through cache->kv, cache->pe and (E4M3) cache->token_scale:
 * they must point to writable device memory that kv_in does not overlap.
 * Rows whose slot does not exist are skipped on the device without an error:
 * a negative position, position >= seq_stride (contiguous), position /
 * block_size >= max_blocks_per_seq or a negative block_table entry (paged).
 * Block ids that are >= 0 must name blocks of the pool.  Sequence lengths are
 * not updated: after the append, the caller's seq_lens[b] for decode is
 * positions[b] + num_new.  Contiguous caches need seq_stride > 0; paged
 * caches a positive block_size (any value) and max_blocks_per_seq.
 */
mla_status mla_cache_append(const mla_dims *dims, const mla_cache *cache, const void *kv_in, int64_t in_stride,
                            const int32_t *positions, int32_t num_new, float rope_base, void *stream);

/*
 * Length-aware split plan for a decode step whose sequences have different
 * lengths ("DeepSeek-V2-Lite 真实权重执行审计" §3.3 names a paged cache with
 * per-sequence lengths as a production requirement; "G5 MLA KV 访存建模设计规格"
 * Appendix B reads the cache concurrently in parts whose results are then
 * combined).  Host-only; launches nothing.
 *
 * The uniform rule of mla_decode_latent cuts every sequence at multiples of
 * ceil(max_seq_len / P), so the launch lasts as long as the longest chunk
 * while short sequences leave workgroups idle.  This plan instead cuts each
 * sequence into near-equal runs of whole 32-token tiles (no run shorter than
 * max(32, min(256, max_seq_len / 32)) tokens unless the sequence is) and
 * orders the runs longest first, the launch order of
 * mla_decode_latent_planned.  It compares tile budgets per run: the fewest
 * tiles such that every run has a resident workgroup slot (num_cus times the
 * resident workgroups per CU: 1 at 128 heads, 2 at 64, 4 at 32, 1 at 16), and
 * budgets that give about 1.1 .. 3 runs per slot, each run then starting on
 * the first slot of its XCD to free up (workgroup i runs on XCD i % 8); it
 * keeps the budget with the shortest predicted launch, counting a run as its
 * tiles plus a fixed cost of 4 tiles.  Every sequence gets at least one item
 * (an empty sequence one item with no tiles).
 *
 *   host_seq_lens  HOST int32 [batch], clamped to [0, max_seq_len]
 *   capacity       rows of `items` the caller provides; budgets whose plan
 *                  needs more rows are not considered, and batch + 12 *
 *                  num_cus rows are enough for every budget
 *   items          HOST int32 [capacity, 4], written in launch order: (sequence,
 *                  first tile, tile count, partial row) per work item; item i
 *                  covers tokens [32 * first, min(32 * (first + count),
 *                  seq_lens[seq])); the partial rows are 0 .. num_items - 1,
 *                  a sequence's items on consecutive rows in token order
 *   seq_first      HOST int32 [batch + 1], written: sequence b's partial rows
 *                  are seq_first[b] .. seq_first[b + 1] - 1 (the merge map)
 *   num_items      written: number of items
 * MLA_ERR_BUFFER if even the one-round plan needs more than `capacity` items.
 */
mla_status mla_plan_decode_splits(const mla_dims *dims, const int32_t *host_seq_lens, int32_t max_seq_len,
                                  int32_t num_cus, int32_t capacity, int32_t *items, int32_t *seq_first,
                                  int32_t *num_items);

/*
 * Latent attention (as mla_decode_latent) over the work items of a plan
 * (mla_plan_decode_splits, copied to the device by the caller): workgroup i
 * runs item i and writes its partial (o, lse) over the item's token range to
 * the item's partial row.
 *   items     device int32 [num_items, 4] (sequence, first 32-token tile,
 *             tile count, partial row); an item naming a sequence outside
 *             [0, batch), a negative or out-of-range first tile, or no tiles
 *             covers no tokens (o = 0, lse = -inf); ranges end at
 *             seq_lens[seq]; an item whose partial row is outside
 *             [0, num_items) writes nothing.  Two items with one partial row
 *             race on it (still inside the arrays).
 *   o_part    device bf16 [num_items, H, 512], lse_part device fp32
 *             [num_items, H] (outputs)
 *   other arguments as mla_decode_latent.
 */
mla_status mla_decode_latent_planned(const mla_dims *dims, const mla_cache *cache, const void *q_lat,
                                     const void *q_pe, const int32_t *seq_lens, int32_t max_seq_len,
                                     const int32_t *items, int32_t num_items, void *o_part, float *lse_part,
                                     void *stream);

/*
 * The merges of mla_combine_splits / mla_combine_expand_v over planned
 * partials: sequence b merges partial rows seq_first[b] .. seq_first[b+1]-1
 * (in that order).  seq_first: device int32 [batch + 1]; a sequence whose
 * range is empty or leaves [0, num_items) merges to o = 0, lse = -inf (and
 * out = 0).  o_part [num_items, H, 512] bf16, lse_part [num_items, H] fp32;
 * outputs as in mla_combine_splits / mla_combine_expand_v.
 */
mla_status mla_combine_splits_planned(const mla_dims *dims, const void *o_part, const float *lse_part,
                                      const int32_t *seq_first, int32_t num_items, void *o_lat, float *lse,
                                      void *stream);
mla_status mla_combine_expand_v_planned(const mla_dims *dims, const void *o_part, const float *lse_part,
                                        const int32_t *seq_first, int32_t num_items, const void *w_uv, void *out,
                                        void *o_lat, float *lse, void *stream);

/*
 * Recommended num_splits for mla_decode_latent on a device with `num_cus`
 * compute units: enough workgroups to fill the chip with the bf16 kernels'
 * resident workgroups per CU (1 at 16 heads, 4 at 32, 2 at 64, 1 at 128),
 * each split at least max_seq_len / 32 tokens, kept within [32, 256]
 * (measured on MI355X: with few sequences, shorter splits cut latency until
 * the merge and the per-split setup dominate).  Host-only.
 */
int32_t mla_recommended_splits(const mla_dims *dims, int32_t max_seq_len, int32_t num_cus);

#ifdef __cplusplus
}
#endif

#endif /* MLA_ABSORB_H */
