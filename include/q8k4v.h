/*
 * q8k4v.h -- C ABI of the int8-key / int4-value quantized-KV decode and
 * speculative-verify attention library for AMD Instinct MI355X (gfx950).
 *
 * The operations
 * --------------
 * The cache codec and the decode unit follow the engine described in the blog
 * post blog.123qwe.co.kr/?p=3927, section 5 (speculative decoding, quantized
 * KV, prefix sharing): the decode attention unit reads a "k8v4" cache whose
 * keys are 8-bit and whose values are 4-bit in groups of 32 along the head
 * dimension, each with an fp16 scale.  The same page (section 5, first table)
 * states that verifying several draft tokens should cost what one decode step
 * costs because decode is bound by memory bandwidth; attn_verify_q8k4v is that
 * pass.  Section 3 of the same page describes the first-load tuner (a 60 s
 * wall-clock budget, a weighted service cost normalised by the time of the
 * defaults, timing passes whose working set exceeds the last-level cache,
 * output-preserving candidates only); tune_select is that tuner for the two
 * attention units.  Section 4 gives the precision policy (alpha = 8) used as
 * the tuner's admission gate.
 *
 * Codec (symmetric absmax, round half to even, IEEE fp32 divisions):
 *   keys   : per (token, kv head)          s = fp16(max|x| / 127), code = clamp(rint(x / s), +-127)
 *   values : per (token, kv head, 32 dims) s = fp16(max|x| / 7),   code = clamp(rint(x / s), +-7)
 *   fp16 overflow of s saturates to 65504; s == 0 gives zero codes.
 *
 * Paged layout (page = 16 tokens; P pages, H kv heads, head dim D in {64,128}):
 *   k_codes  int8  [P][H][16][D]     two's complement, one row per token
 *   k_scales fp16  [P][H][16]        (uint16 bit patterns)
 *   v_codes  uint8 [P][H][D][8]      row d holds dimension d of the 16 tokens:
 *                                    byte j = code(slot 2j) & 0xF | (code(slot 2j+1) & 0xF) << 4
 *   v_scales fp16  [P][H][16][D/32]
 *   Token p of sequence b lives at page page_table[b * max_pages + p / 16], slot p % 16.
 *
 * Conventions
 * -----------
 * Pointers documented "device" are device memory of the current HIP device;
 * "host" pointers are read during the call only.  The caller owns every
 * buffer and the stream.  Hot-path calls (append, decode, verify) only
 * enqueue work on `stream`: they never allocate, never synchronise and keep
 * no device state between calls.  Device-resident values (lengths, page ids,
 * positions) are not validated: an out-of-range value is undefined
 * behaviour.  Every function returns Q8K4V_OK or a negative error code; the
 * message of the last error on the calling thread is q8k4v_last_error().
 */
#ifndef Q8K4V_H
#define Q8K4V_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define Q8K4V_OK            0
#define Q8K4V_EINVAL       -1   /* bad argument (null pointer, shape, range)     */
#define Q8K4V_EUNSUPPORTED -2   /* valid but not built (e.g. head_dim 96)         */
#define Q8K4V_EWORKSPACE   -3   /* workspace missing or smaller than required     */
#define Q8K4V_EHIP         -4   /* a HIP runtime call failed                      */
#define Q8K4V_ENOMEM       -5   /* the tuner's memory admission refused the work  */

#define Q8K4V_F32  0            /* float32 values                                 */
#define Q8K4V_BF16 1            /* bfloat16 bit patterns (uint16)                 */

#define Q8K4V_PAGE_SIZE 16
#define Q8K4V_MAX_DRAFT 16
#define Q8K4V_MAX_CHUNK 1024     /* new tokens per sequence in one prefill call */

/* Every workspace starts with a header of this many bytes that holds the
 * arrival counters of the in-launch split merge (fused_combine); split
 * records of every plan and entry point lie behind it. */
#define Q8K4V_WS_HEADER_BYTES 65536

#define Q8K4V_CODEC_SYMMETRIC 0   /* the codec above                            */
#define Q8K4V_CODEC_AFFINE    1   /* the affine variant below                   */

/* The paged cache: four device pools in the layout above, plus two zero-point
 * pools for the affine variant.
 *
 * Affine variant (the same page names the codec affine; unsigned codes with a
 * zero point, the block's range widened to include zero):
 *   lo = min(min x, 0), hi = max(max x, 0), s = fp16((hi - lo) / q),
 *   z = clamp(rint(-lo / s), 0, q), code = clamp(rint(x / s) + z, 0, q),
 *   value = (code - z) * s; q = 255 for keys (per token and kv head), 15 for
 *   values (per token, kv head and 32 dims); s == 0 gives code and z 0.
 *   k_codes hold code XOR 0x80 (code - 128 as int8), k_zeros z XOR 0x80;
 *   value nibbles hold the unsigned codes, v_zeros one byte (0..15) per
 *   (token, group).  Every attention entry point takes either codec. */
typedef struct q8k4v_cache {
    int32_t   num_pages;     /* P: physical pages in each pool                   */
    int32_t   num_kv_heads;  /* H                                                */
    int32_t   head_dim;      /* D: 64 or 128                                     */
    int32_t   page_size;     /* must be 16                                       */
    int8_t   *k_codes;       /* device [P][H][16][D]                             */
    uint16_t *k_scales;      /* device [P][H][16]                                */
    uint8_t  *v_codes;       /* device [P][H][D][8]                              */
    uint16_t *v_scales;      /* device [P][H][16][D/32]                          */
    int32_t   codec;         /* Q8K4V_CODEC_SYMMETRIC (0) or Q8K4V_CODEC_AFFINE  */
    int8_t   *k_zeros;       /* device [P][H][16], affine only (else NULL)       */
    uint8_t  *v_zeros;       /* device [P][H][16][D/32], affine only (else NULL) */
} q8k4v_cache;

/* Launch configuration of the attention kernels (what the tuner chooses).
 * Any field left 0 takes the library default. */
typedef struct q8k4v_config {
    int32_t wgs_per_cu;      /* split-K: target workgroups per compute unit; the split
                                length follows from it and the launch shape           */
    int32_t split_pages;     /* if > 0: pages per workgroup split (overrides wgs_per_cu) */
    int32_t tile_pages;      /* pages staged in LDS per wave per step: both kernels
                                stage 2-page tiles (0 or 2; anything else EINVAL)     */
    int32_t waves_per_wg;    /* 2, 4 or 8 waves per workgroup. Default 4, or 8 for
                                variant 5 above 16 rows per kv head                   */
    int32_t fused_combine;   /* 1: the last workgroup of a (sequence, kv head, row
                                chunk) merges the splits in the same launch (its
                                arrival counters live in the workspace header; a
                                launch with more than Q8K4V_WS_HEADER_BYTES / 4 such
                                items uses the separate kernel); 0: a separate combine
                                kernel                                                  */
    int32_t qualified;       /* out of tune_select: 1 measured and admitted, 0 default */
    int32_t variant;         /* kernel: 0 automatic (4 for 1, 2, 4, 8 or 16 query rows
                                per kv head, else 5); 4 16x16 MFMA with the rows
                                replicated across the MFMA columns (1, 2, 4, 8 or 16
                                rows); 5 16x16 MFMA row blocks, 16 or 32 rows per
                                workgroup (any row count).  Other values EINVAL      */
    int32_t stages;          /* tile buffers per wave in the HBM->LDS ring, 2 or 3
                                (prefetch depth stages - 1); 0 default               */
} q8k4v_config;

/* Last error message of the calling thread ("" if none). */
const char *q8k4v_last_error(void);

/* Library build identity, e.g. "q8k4v 1 gfx950 <hash>". */
const char *q8k4v_version(void);

/*
 * kv_quant_append -- quantize new tokens and write them into the paged cache.
 *
 * Implements the codec above (blog.123qwe.co.kr/?p=3927, section 5: 8-bit
 * keys, 4-bit values in groups of 32 with fp16 scales).  New tokens of
 * sequence b are rows cu_new[b] .. cu_new[b+1]-1 of k_new / v_new and go to
 * logical positions start_pos[b], start_pos[b]+1, ... of that sequence.
 *
 *   cache      host pointer to the cache descriptor (device pools)
 *   k_new      device [total_new][H][D], dtype `dtype` (Q8K4V_F32 or Q8K4V_BF16)
 *   v_new      device [total_new][H][D], same dtype
 *   cu_new     device int32 [n_seqs + 1], cu_new[0] = 0, nondecreasing, cu_new[n_seqs] = total_new
 *   start_pos  device int32 [n_seqs]
 *   page_table device int32 [n_seqs][max_pages]; every written slot's page must be
 *              owned by that sequence (pages shared by several sequences are read-only)
 *   total_new  host: number of new tokens (sizes the grid); 0 is a no-op
 * Codes and scales are bit-exact with the rule above (IEEE division,
 * round-half-even, no flush of fp16 subnormal scales).
 * Errors: EINVAL on null pointers, D not in {64,128}, page_size != 16,
 * n_seqs < 1, total_new < 0, bad dtype; EHIP if the launch fails.
 */
int32_t kv_quant_append(const q8k4v_cache *cache, const void *k_new, const void *v_new,
                        int32_t dtype, const int32_t *cu_new, const int32_t *start_pos,
                        const int32_t *page_table, int32_t max_pages, int32_t n_seqs,
                        int32_t total_new, hipStream_t stream);

/*
 * Workspace (bytes) that attn_decode_q8k4v / attn_verify_q8k4v need for the
 * given launch shape and configuration (cfg may be NULL for the defaults);
 * n_draft = 0 for decode, the draft count for verify, the chunk length for
 * prefill.  Returns 0 on invalid shapes, and 0 when the launch runs as one
 * split per (sequence, kv head) (it then writes the output directly and
 * needs no workspace).  Otherwise the workspace is the header of
 * Q8K4V_WS_HEADER_BYTES followed by the split-K partials.  The header holds
 * the in-launch merge's arrival counters: it must be zero before its first
 * use; every completed call of every entry point leaves it zero, and no
 * entry point writes split records into it, so a workspace zeroed once (at
 * least its header) serves any sequence of calls, plans, shapes and entry
 * points.  The partials need no initial value: records of splits past a
 * sequence's last page are masked by the merge, never read as values.
 */
size_t q8k4v_workspace_bytes(int32_t n_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                             int32_t head_dim, int32_t max_seq_len, int32_t n_draft,
                             const q8k4v_config *cfg);

/*
 * attn_decode_q8k4v -- one query token per sequence attends its whole cache.
 *
 * Exact softmax attention over the dequantized cache (the decode unit of
 * blog.123qwe.co.kr/?p=3927, section 5), computed split-K: workgroups
 * each take a range of pages of one (sequence, kv head), stage K/V pages in
 * LDS, dequantize in registers, keep an online softmax, and the splits are
 * merged by log-sum-exp.  Query head h reads kv head h / (num_q_heads / H).
 *
 *   q            device [n_seqs][num_q_heads][D], dtype q_dtype (F32 or BF16)
 *   out          device float32 [n_seqs][num_q_heads][D]
 *   seq_lens     device int32 [n_seqs]: cached tokens attended (0 gives zeros)
 *   max_seq_len  host: an upper bound of seq_lens (sizes the grid)
 *   page_table   device int32 [n_seqs][max_pages]
 *   softmax_scale  multiplies q.k (e.g. 1/sqrt(D))
 *   cfg          host, NULL = tuned table or defaults
 *   workspace    device, at least q8k4v_workspace_bytes(...) bytes
 * Supported: D in {64,128}, num_q_heads / H in {1,2,4,8}.
 * Errors: EINVAL (shapes, null pointers), EUNSUPPORTED (group size),
 * EWORKSPACE (workspace too small), EHIP.
 */
int32_t attn_decode_q8k4v(const q8k4v_cache *cache, const void *q, int32_t q_dtype,
                          float *out, int32_t n_seqs, int32_t num_q_heads,
                          const int32_t *seq_lens, int32_t max_seq_len,
                          const int32_t *page_table, int32_t max_pages, float softmax_scale,
                          const q8k4v_config *cfg, void *workspace, size_t workspace_bytes,
                          hipStream_t stream);

/*
 * attn_decode_prefix_q8k4v -- decode of sessions that share a prompt prefix
 * (blog.123qwe.co.kr/?p=3927, section 5: concurrent sessions over one cached
 * prefix).  Same result as attn_decode_q8k4v on the same arguments, computed
 * as a cascade so that the shared pages are read once for all sessions:
 *  1. prefix pass: the first n_prefix_pages logical pages, taken from row 0
 *     of page_table, against the query rows of every session at once (a
 *     dense (n_seqs * group) x D query block per kv head on the 16x16 MFMA
 *     row-block kernel), split-K partials per session row;
 *  2. suffix pass: each session's pages from n_prefix_pages on, split-K as
 *     in attn_decode_q8k4v;
 *  3. combine: per (session, q head), the log-sum-exp merge of both partial
 *     sets, normalised into out.
 *
 *   n_prefix_pages  host: leading logical pages shared by every session.
 *                   Precondition (device data, not checked): for every b,
 *                   page_table[b][i] == page_table[0][i] for i < n_prefix_pages
 *                   and seq_lens[b] >= 16 * n_prefix_pages; if violated the
 *                   output is undefined (with page ids in range no access
 *                   leaves the pools).
 *                   0 runs attn_decode_q8k4v.
 *   cfg             applies to the suffix pass (NULL: the configuration
 *                   tune_select installed for this device and head shape, else
 *                   the decode defaults with wgs_per_cu 3); the prefix pass
 *                   uses the row-block kernel's defaults
 *   workspace       at least q8k4v_prefix_workspace_bytes(...) bytes
 * Other arguments as attn_decode_q8k4v.  Errors as attn_decode_q8k4v, plus
 * EINVAL for n_prefix_pages outside 0 .. min(max_pages, max_seq_len / 16)
 * and EUNSUPPORTED for more than 4096 query rows per kv head.
 */
int32_t attn_decode_prefix_q8k4v(const q8k4v_cache *cache, const void *q, int32_t q_dtype,
                                 float *out, int32_t n_seqs, int32_t num_q_heads,
                                 const int32_t *seq_lens, int32_t max_seq_len,
                                 const int32_t *page_table, int32_t max_pages,
                                 int32_t n_prefix_pages, float softmax_scale,
                                 const q8k4v_config *cfg, void *workspace, size_t workspace_bytes,
                                 hipStream_t stream);

/* Workspace (bytes) of attn_decode_prefix_q8k4v: the header of
 * Q8K4V_WS_HEADER_BYTES (the cascade keeps no counters but writes no records
 * into it, so one workspace serves every entry point) and both passes' split
 * partials, enough for either codec.  Returns 0 on invalid shapes. */
size_t q8k4v_prefix_workspace_bytes(int32_t n_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                                    int32_t head_dim, int32_t max_seq_len, int32_t n_prefix_pages,
                                    const q8k4v_config *cfg);

/*
 * attn_verify_q8k4v -- n_draft draft queries per sequence, causal among the
 * drafts (blog.123qwe.co.kr/?p=3927, section 5: checking several drafted
 * tokens in the pass that one decode step costs).
 *
 * The drafts' keys/values must already be appended: seq_lens[b] counts them,
 * and draft j (0-based) of sequence b attends positions 0 .. seq_lens[b] -
 * n_draft + j.  Rows (draft, q head) of one kv head form a
 * (n_draft * group) x D query block.  With 1, 2, 4, 8 or 16 rows it runs on
 * the decode kernel (rows replicated across the MFMA columns); any other row
 * count on 16x16 MFMA row blocks: q.K on int8 MFMA (raw key codes against
 * the query as a 23-bit fixed-point number per row, three int8 digits,
 * int32 accumulation),
 * P.V on fp16 MFMA (exact value codes against each probability times the
 * token's value scale for that 32-dim group, rounded to fp16; fp32
 * accumulation).
 *
 *   q, out   [n_seqs][n_draft][num_q_heads][D] (q dtype q_dtype, out float32)
 *   n_draft  1 .. Q8K4V_MAX_DRAFT; every seq_lens[b] >= n_draft
 * Other arguments and errors as attn_decode_q8k4v.
 */
int32_t attn_verify_q8k4v(const q8k4v_cache *cache, const void *q, int32_t q_dtype,
                          float *out, int32_t n_seqs, int32_t num_q_heads, int32_t n_draft,
                          const int32_t *seq_lens, int32_t max_seq_len,
                          const int32_t *page_table, int32_t max_pages, float softmax_scale,
                          const q8k4v_config *cfg, void *workspace, size_t workspace_bytes,
                          hipStream_t stream);

/*
 * attn_decode_append_q8k4v -- one decode step: kv_quant_append of each
 * sequence's new token followed by attn_decode_q8k4v, in one attention
 * launch where the plan allows.  The new token of sequence b goes to
 * position seq_lens[b] - 1 (seq_lens counts it).  The cache afterwards and
 * the output are those of the two calls (same codec rule, same device
 * functions): the wave whose tile holds the token's page quantizes it,
 * puts it into its LDS copy of the page before the tile is read, and writes
 * it to the cache for later calls (blog.123qwe.co.kr/?p=3927, section 5:
 * the decode unit over the k8v4 cache).  Fused when the decode plan is the
 * replicated-row kernel with 4 waves and 2 stages, with either codec (the
 * defaults for 1, 2, 4, 8 or 16 rows per kv head); otherwise the append
 * kernel runs first, then the decode.
 *
 *   k_new, v_new  device [n_seqs][H][D], dtype new_dtype (Q8K4V_F32 or Q8K4V_BF16)
 *   seq_lens      device int32 [n_seqs], >= 1, the new token included
 * Other arguments and errors as attn_decode_q8k4v (workspace from
 * q8k4v_workspace_bytes with n_draft 0).
 */
int32_t attn_decode_append_q8k4v(const q8k4v_cache *cache, const void *k_new, const void *v_new,
                                 int32_t new_dtype, const void *q, int32_t q_dtype, float *out,
                                 int32_t n_seqs, int32_t num_q_heads, const int32_t *seq_lens,
                                 int32_t max_seq_len, const int32_t *page_table, int32_t max_pages,
                                 float softmax_scale, const q8k4v_config *cfg, void *workspace,
                                 size_t workspace_bytes, hipStream_t stream);

/*
 * attn_decode_q8k4v_noalloc -- attn_decode_q8k4v without a caller workspace,
 * for callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation).  The
 * split records and the in-launch merge's counters live in a static device
 * array of Q8K4V_NOALLOC_SCRATCH_BYTES per GPU, inside the library, held
 * until the process ends; the call allocates nothing.  The first call on a
 * device looks the array up (hipGetSymbolAddress) and clears its counter
 * header with a fill kernel enqueued on `stream` before the attention work.
 * Every call on a GPU shares that GPU's array: calls that overlap on one GPU
 * (other streams, other threads) race and give undefined output; calls
 * serialised on one stream do not.
 * Arguments, results and the other errors as attn_decode_q8k4v; EWORKSPACE
 * when the launch needs more scratch than the array holds (16 MiB: the
 * 64 KiB header plus 31,651 split records -- one per sequence, kv head,
 * split and query row -- at D = 128; the 64K decode takes 1,024).
 */
#define Q8K4V_NOALLOC_SCRATCH_BYTES (16u << 20)
int32_t attn_decode_q8k4v_noalloc(const q8k4v_cache *cache, const void *q, int32_t q_dtype,
                                  float *out, int32_t n_seqs, int32_t num_q_heads,
                                  const int32_t *seq_lens, int32_t max_seq_len,
                                  const int32_t *page_table, int32_t max_pages, float softmax_scale,
                                  const q8k4v_config *cfg, hipStream_t stream);

/*
 * attn_prefill_q8k4v -- chunked-prefill attention over the quantized cache:
 * n_new new tokens per sequence (already appended) attend the cache, causal
 * among themselves -- the computation of attn_verify_q8k4v for chunks of up
 * to Q8K4V_MAX_CHUNK tokens (blog.123qwe.co.kr/?p=3927, section 3: the
 * service cost weights 4k and 64k prompt prefill).  New token j of sequence
 * b attends positions 0 .. seq_lens[b] - n_new + j.  The (n_new * group) x D
 * query block of each kv head runs on the 16x16 MFMA row-block kernel in
 * 16- or 32-row chunks; every chunk streams the context (chunks of one
 * context range run together and share it through L2).
 *
 *   q, out   [n_seqs][n_new][num_q_heads][D] (q dtype q_dtype, out float32)
 *   n_new    1 .. Q8K4V_MAX_CHUNK; every seq_lens[b] >= n_new
 *   workspace  at least q8k4v_workspace_bytes(..., n_draft = n_new, cfg)
 * Other arguments and errors as attn_verify_q8k4v.
 */
int32_t attn_prefill_q8k4v(const q8k4v_cache *cache, const void *q, int32_t q_dtype,
                           float *out, int32_t n_seqs, int32_t num_q_heads, int32_t n_new,
                           const int32_t *seq_lens, int32_t max_seq_len,
                           const int32_t *page_table, int32_t max_pages, float softmax_scale,
                           const q8k4v_config *cfg, void *workspace, size_t workspace_bytes,
                           hipStream_t stream);

/*
 * q8k4v_hbm_probe -- streaming reference of the decode kernel's roofline
 * (the survey's memory probe; measurement only, outside the hot path).
 * Reads exactly the bytes attn_decode_q8k4v reads over the same arguments --
 * every (page, kv head) block of key codes, value codes, key scales and
 * value scales of each sequence's pages through page_table, with the decode
 * plan's split of pages over workgroups and its XCD-aware mapping, in 2-page
 * tiles copied HBM -> LDS -- and computes nothing.  Its time is what the
 * memory system gives that access pattern; blog.123qwe.co.kr/?p=3927,
 * section 5, gives the reason decode is judged by it (decode is bound by
 * memory traffic).
 *   cache, n_seqs, seq_lens, max_seq_len, page_table, max_pages: as
 *                 attn_decode_q8k4v (symmetric codec only)
 *   waves_per_wg, stages: launch shape, (4, 2..4) or (8, 2..3); stages - 1
 *                 tiles per wave in flight
 *   heads_per_wg  1: the decode kernel's mapping (one kv head per
 *                 workgroup); 2, 4 or 8 (8 with 8 waves): as many workgroups,
 *                 each streaming that many kv heads of 1/heads_per_wg of
 *                 the pages, so the heads' blocks of a page (contiguous in
 *                 every pool) are read by one compute unit together
 * Errors: EINVAL (shape, codec, launch shape), EHIP.  Writes nothing to
 * device memory.
 */
int32_t q8k4v_hbm_probe(const q8k4v_cache *cache, int32_t n_seqs, const int32_t *seq_lens,
                        int32_t max_seq_len, const int32_t *page_table, int32_t max_pages,
                        int32_t waves_per_wg, int32_t stages, int32_t heads_per_wg, hipStream_t stream);

/*
 * q8k4v_stream_probe -- the sequential reference: streams `bytes` of the
 * contiguous device buffer `buf` into LDS, one chunk per compute unit, in
 * 1 KiB wave copies with (stages - 1) x 4 KiB per wave in flight.
 *   buf       device, 16-byte aligned; bytes >= 1024 and a multiple of 16
 *   waves_per_wg 4 or 8; stages 2..4
 * Errors: EINVAL, EHIP.  Writes nothing to device memory.
 */
int32_t q8k4v_stream_probe(const void *buf, size_t bytes, int32_t waves_per_wg, int32_t stages,
                           hipStream_t stream);

/*
 * tune_select -- on-device search of the attention launch configuration
 * (blog.123qwe.co.kr/?p=3927, section 3: first-load tuner).
 *
 * For each unit (decode, verify, and with n_sessions the multi-session
 * decode) it measures candidate configurations on its two shapes -- at
 * ctx_small and ctx_large -- and keeps,
 * per unit, the admitted candidate with the least service cost
 *     cost(c) = sum over the unit's shapes p of median_time(c, p) / median_time(default, p)
 * (term weights 1, one launch per layer-step).  Every step -- allocation,
 * input synthesis, the defaults' measurement, the candidates, the gate --
 * runs inside the wall-clock budget (at most 60 s); a candidate not measured
 * before the deadline is "unknown" and never admitted.  A time is per
 * launch inside a captured graph of launches replayed on the tuner's own
 * stream (median over the timed replays); the launches rotate over distinct
 * cache copies whose total size exceeds 4 x 256 MiB (the MI355X last-level
 * cache), so no launch is served from a warm cache.  Admission
 * (section 4 of the same page, alpha = 8): on every checked output the
 * candidate's deviation from the default configuration's output must not
 * exceed alpha times the storage-resolution noise, i.e. the change of the
 * default output when every stored code is moved by one step; and, on each
 * term for which the caller supplies a reference output (the oracle gate:
 * a configuration is kept only if it reproduces the oracle), the
 * sigma-normalised deviation from it must not exceed ref_tol.  Search
 * order (section 3): after the units' defaults, each next candidate comes from the
 * unit with the earliest virtual completion time (effort + price) / (share x
 * opportunity) -- wall time spent on the unit, wall time of its last
 * measurement, its part of the default service time, the fraction of its
 * generated candidates still unmeasured; within a unit, the other kernel
 * before launch-shape refinement, and only configurations the library
 * accepts.  The JSON report lists every candidate with its verdict, the gate
 * that rejected it ("alpha" or "oracle") and why, its deviations (null where
 * not measured: unknown, never 0), its measurement order ("seq") and every
 * unit's virtual time when it was picked ("vt"); each unit's summary counts
 * the rejections per gate and lists the distinct reasons of invalid
 * candidates.
 *
 *   req         host, see q8k4v_tune_request
 *   out_table   host [2] ([3] when req->n_sessions >= 2): [0] decode,
 *               [1] verify, [2] the multi-session suffix pass; `qualified` = 1
 *               if a measured candidate was admitted, else the defaults with 0
 *   report_json host buffer for a JSON report (may be NULL), NUL-terminated
 * Returns Q8K4V_OK even when nothing could be searched (defaults,
 * unqualified); ENOMEM if memory admission refuses even the defaults;
 * EINVAL on bad shapes; EHIP.
 */
/* One reference term of the tuner's oracle gate: sequences in the caller's
 * cache with their expected attention output (e.g. from a CPU oracle). */
typedef struct q8k4v_tune_ref {
    const q8k4v_cache *cache;          /* device pools; NULL: no reference for this term  */
    const void *q;                     /* device bf16 [n][num_q_heads][D]; n = 1 for the
                                          decode terms, n_draft for the verify terms,
                                          n_seqs for the multi-session terms             */
    const int32_t *page_table;         /* device int32 [max_pages]: the sequence's pages;
                                          multi-session terms [n_seqs][max_pages]        */
    int32_t len, max_pages;            /* tokens attended (the drafts included for
                                          verify); multi-session: the longest session    */
    const float *out;                  /* host float32 [n][num_q_heads][D]                */
    const float *sigma;                /* host float32 [num_q_heads][D] or NULL (1): the
                                          deviation is |out - ref| / sigma per element    */
    const int32_t *seq_lens;           /* multi-session terms: device int32 [n_seqs]     */
    int32_t n_seqs;                    /* multi-session terms: sessions                  */
    int32_t n_prefix_pages;            /* multi-session terms: leading shared pages      */
} q8k4v_tune_ref;

typedef struct q8k4v_tune_request {
    int32_t num_q_heads, num_kv_heads, head_dim, n_draft;
    int32_t ctx_small, ctx_large;      /* e.g. 4096 and 65536 */
    int64_t budget_ms;                 /* wall clock, clamped to 60000 */
    size_t  mem_cap_bytes;             /* 0: free device memory at the call */
    uint64_t seed;                     /* synthetic cache contents */
    int32_t install;                   /* 1: qualified winners become the configuration used
                                          when cfg == NULL, on this device, for this
                                          (n_draft, num_q_heads, num_kv_heads, head_dim);
                                          the decode unit is stored under n_draft 1 */
    int32_t max_candidates;            /* 0: no limit */
    int32_t n_sessions;                /* 0: two units; 2 .. 64: also the multi-session
                                          unit -- attn_decode_prefix_q8k4v of n_sessions
                                          sessions over a shared prefix (its suffix-pass
                                          configuration is what is tuned); at ctx
                                          (ctx_small, ctx_large) the sessions share a
                                          ctx / 2 token prefix and session i owns about
                                          (i + 1) / n_sessions x ctx / 2 more tokens    */
    /* Oracle gate (optional per term; the tuner never computes references
       itself): ref[k] for term k = decode@ctx_small, decode@ctx_large,
       verify@ctx_small, verify@ctx_large, multi-session small, multi-session
       large.  A term with ref[k].cache != NULL runs every candidate on the
       caller's inputs and admits it only if
       max |out - ref[k].out| / ref[k].sigma <= ref_tol.  The default must pass
       too, else the unit keeps unqualified defaults. */
    q8k4v_tune_ref ref[6];
    float ref_tol;                     /* tolerance on the normalised deviation            */
    float softmax_scale;               /* 0: 1/sqrt(D)                                      */
    /* optional text file of stored choices (may be NULL): a call whose device
       identity (architecture, device name and CU count, HIP runtime and driver
       versions, library build) and request shape (n_draft, head counts,
       head_dim, ctx_small, ctx_large, n_sessions) match stored records uses them without
       measuring (report status "stored"); otherwise it searches and, when the
       search ran, replaces the records of that identity and shape (other
       records are kept) */
    const char *record_path;
} q8k4v_tune_request;

int32_t tune_select(const q8k4v_tune_request *req, q8k4v_config *out_table,
                    char *report_json, size_t report_cap);

#ifdef __cplusplus
}
#endif

#endif /* Q8K4V_H */
