/*
 * mla_kv.h — C ABI of the absorbed-MLA decode library for MI355X (gfx950).
 *
 * What the library computes (one transformer layer, one decode step):
 *
 *   The cache keeps, per token, the 512-d latent c_kv and the 64-d RoPE key
 *   k_pe instead of per-head keys and values ("Absorbed MLA Cache Optimization
 *   on DeepSeek-V2-Lite", section 2.1: AbsorbedMLACache.store / get; section
 *   3.1: 512 + 64 = 576 values per token). The latent is optionally quantized
 *   per 16-channel group to symmetric INT8 or asymmetric INT4, k_pe per
 *   8-channel group to INT8 (same report, section 3.2 / 4.2 tables: 32 blocks,
 *   8 blocks), each group with an fp16 scale (and an fp16 zero-point for INT4).
 *
 *   Attention for head h follows the per-head softmax(q K^T * scale) V of the
 *   tutorial "DeepSeek的MLA技术" (MLAttentionWithCache.forward_with_cache),
 *   with K_t = [W_UK[h] c_t || k_pe_t] and V_t = c_t W_UV[h] (its MLA
 *   mechanism, step 2), computed without expanding any token:
 *     q_abs   = q_nope W_UK[h]                               (512)
 *     s_t     = scale * (q_abs . c_t + q_pe . k_pe_t)
 *     o_lat   = sum_t softmax(s)_t c_t                        (512)
 *     out[h]  = o_lat W_UV[h]                                 (128)
 *
 * Conventions for every call:
 *   - Every pointer argument except `cache` and the status string is a DEVICE
 *     pointer, allocated and owned by the caller. The library allocates no
 *     memory and keeps no state between calls; calls are reentrant. The one
 *     exception is mla_decode_attn_static (below), whose workspace is a
 *     device array of the library's own, one per GPU, shared by its calls.
 *   - `hip_stream` is a hipStream_t passed as void* (NULL = the null stream).
 *     Work is enqueued asynchronously on it; no call synchronizes the host.
 *   - Arguments are checked on the host before anything is enqueued; a
 *     negative mla_status is returned and nothing is launched on error. A
 *     failed launch returns MLA_ERR_HIP.
 *   - bf16 / fp16 values are passed as their 16-bit patterns (uint16_t or an
 *     untyped pointer). All planes are dense, row-major, 16-byte aligned.
 */
#ifndef MLA_KV_H
#define MLA_KV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MLA_OK = 0,
  MLA_ERR_INVALID_ARG = -1, /* null pointer, bad size, layer out of range, misalignment */
  MLA_ERR_UNSUPPORTED = -2, /* a dimension, head count or size the library does not handle */
  MLA_ERR_WORKSPACE = -3,   /* workspace missing or smaller than required */
  MLA_ERR_CAPACITY = -4,    /* (Python binding) an append would exceed capacity */
  MLA_ERR_HIP = -5          /* a HIP launch or runtime call failed */
} mla_status;

/* Storage format of a cache row (latent c_kv and RoPE key k_pe). */
typedef enum {
  MLA_FMT_BF16 = 0,       /* c_kv and k_pe copied as bf16 */
  MLA_FMT_INT8 = 1,       /* c_kv symmetric INT8 per 16 channels, k_pe INT8 per 8 channels */
  MLA_FMT_INT4 = 2,       /* c_kv asymmetric INT4 per 16 channels (2 codes/byte), k_pe INT8 */
  MLA_FMT_INT8_KBF16 = 3, /* c_kv INT8 as MLA_FMT_INT8, k_pe copied as bf16 (the report's
                             configuration "B", section 3.2) */
  MLA_FMT_INT4_KINT4 = 4  /* c_kv INT4 as MLA_FMT_INT4, k_pe symmetric INT4 per 8 channels
                             (the report's 7.6 KB per token, section 3.2 / summary) */
} mla_format;

/*
 * The cache of all layers of one model, for a batch of sequences.
 *
 * Planes, each [num_layers][batch][capacity][row] (ckv: see below) with the
 * row sizes:
 *   ckv     BF16: 512 x bf16 (1024 B)   INT8, INT8_KBF16: 512 x int8 (512 B)
 *           INT4, INT4_KINT4: 256 x uint8 (256 B), byte k = code[2k] | code[2k+1] << 4
 *           The ckv plane is [num_layers][batch][cap16][row], cap16 = capacity
 *           rounded up to a multiple of 16, and stores each sequence's rows in
 *           blocks of 16: in the block of rows 16m..16m+15, the 16-byte chunk c
 *           of row 16m+i (its bytes 16c..16c+15) lies at byte (16c + i) * 16
 *           of the block. The rows never stored may hold anything.
 *   kpe     BF16, INT8_KBF16: 64 x bf16 (128 B)     INT8, INT4: 64 x int8 (64 B)
 *           INT4_KINT4: 32 x uint8 (32 B), byte k = (code[2k] + 8) | (code[2k+1] + 8) << 4
 *   scale   INT8, INT4, INT4_KINT4: 40 x fp16 (80 B): the 32 latent-group
 *           scales, then the 8 k_pe-group scales. INT8_KBF16: 32 x fp16 (64 B),
 *           the latent-group scales. NULL for BF16.
 *   zero    INT4, INT4_KINT4: 32 x fp16 (64 B) latent-group zero-points. NULL otherwise.
 *   seq_lens  int32 [num_layers][batch]: tokens stored per (layer, sequence).
 *
 * Quantization of one group x (the definition parity is checked against):
 *   INT8:  s = fp16_rne(max|x| / 127), q = clamp(rne(x / s), -127, 127),
 *          x_hat = q * s; s == 0 gives q = 0.
 *   INT4:  z = fp16 rounded toward -inf of min x, s = fp16_rne((max x - z) / 15)
 *          (each stored as +0 when zero), q = clamp(rne((x - z) / s), 0, 15),
 *          x_hat = q * s + z; s == 0 gives q = 0.
 *   INT4 k_pe (INT4_KINT4): s = fp16_rne(max|x| / 7), q = clamp(rne(x / s), -7, 7),
 *          x_hat = q * s; s == 0 gives q = 0.
 *   Every step is one IEEE fp32 operation; fp16 results that would overflow
 *   saturate to +-65504. Inputs must be finite.
 *
 * Domain of the decode path. It multiplies codes by scales in fp16, so every
 * product q * s of a stored row must be finite in fp16:
 *   - every format: inputs within +-65280 (bf16 planes are read as fp16;
 *     INT8 groups then have 127 * s <= 65280, INT4 k_pe groups 7 * s <= 65296);
 *   - INT4 latents (INT4, INT4_KINT4) in addition: each 16-channel group's
 *     range max - min below 65490, so that 15 * s <= 65460 (the zero-point
 *     is applied separately and never added in fp16). Inputs within +-32744
 *     satisfy both.
 * Outside this domain mla_cache_append still stores the exact codes, but the
 * decode outputs are undefined. mla_cache_get has no such limit.
 */
typedef struct mla_cache {
  int32_t format;       /* mla_format */
  int32_t num_layers;   /* >= 1 */
  int32_t batch;        /* >= 1 */
  int32_t capacity;     /* tokens per (layer, sequence), >= 1 */
  int32_t kv_lora_rank; /* latent width: must be 512 */
  int32_t rope_dim;     /* k_pe width: must be 64 */
  int32_t group_latent; /* latent channels per group: must be 16 */
  int32_t group_rope;   /* k_pe channels per group: must be 8 */
  void *ckv;
  void *kpe;
  uint16_t *scale;
  uint16_t *zero;
  int32_t *seq_lens;
  /* Paged layout (page_size > 0; "DeepSeek的MLA技术", limits and future
   * directions, item 3: MLA together with PagedAttention): each plane is a pool
   * [num_layers][num_pages][page_size][row] (the ckv pages in 16-row blocks as
   * above), and token p of sequence b lives at row p % page_size of page
   * block_table[b][p / page_size] in every layer.
   * page_size: a power of two >= 32 dividing capacity; num_pages >= 1;
   * block_table: device int32 [batch][capacity / page_size]. A page index
   * outside [0, num_pages) is never written, and the decode reads its tokens
   * as all-zero rows (they still count as tokens: score 0, value 0), so every
   * entry below a sequence's length should name a page of the pool.
   * page_size = 0 (and block_table = NULL): the contiguous planes above. */
  int32_t page_size;
  int32_t num_pages;
  const int32_t *block_table;
} mla_cache;

/*
 * Quantize-on-append ("store" of section 2.1 of the report: quantize
 * compressed_kv as it is stored, and keep k_pe beside it).
 *
 *   ckv_new  bf16 [batch][t_new][512]   latent of the new tokens
 *   kpe_new  bf16 [batch][t_new][64]    RoPE key of the new tokens (already rotated)
 *   t_new    rows per sequence in ckv_new / kpe_new, >= 0 (0 is a no-op)
 *   n_new    optional int32 [batch] (device): sequence b appends only its first
 *            n_new[b] rows, 0 <= n_new[b] <= t_new. NULL: every sequence
 *            appends t_new rows.
 *
 * Sequence b's rows go to positions seq_lens[layer][b] .. +n-1 of `layer`,
 * then seq_lens[layer][b] grows by n. Rows that would land at or past
 * `capacity` are not written and seq_lens stops at capacity: the device
 * cannot report it, so a caller must keep lengths within capacity (the Python
 * binding tracks them and raises MLA_ERR_CAPACITY first).
 */
int mla_cache_append(const mla_cache *cache, int32_t layer, const void *ckv_new,
                     const void *kpe_new, int32_t t_new, const int32_t *n_new,
                     void *hip_stream);

/*
 * Workspace bytes that mla_decode_attn needs for this cache, head count and
 * split count (0 = the split count the library would choose). Writes the size
 * to *bytes and returns MLA_OK, or returns a negative status.
 */
int mla_decode_workspace_bytes(const mla_cache *cache, int32_t heads, int32_t num_splits,
                               size_t *bytes);

/*
 * The split count mla_decode_attn uses for num_splits = 0 with this cache and
 * head count (it depends on capacity, batch and the device's CU count only,
 * never on seq_lens, which live on the device).
 */
int mla_decode_auto_splits(const mla_cache *cache, int32_t heads, int32_t *num_splits);

/*
 * Absorbed decode attention for one layer and one new query token per sequence.
 *
 *   q_nope   bf16 [batch][heads][128]  non-RoPE query part
 *   q_pe     bf16 [batch][heads][64]   RoPE query part (already rotated)
 *   w_uk     bf16 [heads][128][512]    key up-projection: K_nope[h] = W_UK[h] c
 *   w_uv     bf16 [heads][512][128]    value up-projection: V[h] = c W_UV[h]
 *   heads    16, 32, 64 or 128
 *   softmax_scale   multiplies q.k before the softmax (e.g. 1/sqrt(192))
 *   num_splits      0 = auto, else 1..4096: KV splits per sequence on
 *                   average. The batch's 32-token tiles, sequence after
 *                   sequence, are cut into W = num_splits * batch equal runs
 *                   (a run may end one sequence and start the next), so the
 *                   work is the same for every run whatever the mix of
 *                   lengths; the partial phase runs each run once per slice
 *                   of 16 heads (W * heads / 16 workgroups). Auto: about
 *                   three workgroups per CU, at least 4 tiles per run for
 *                   full sequences (up to 8 runs per sequence of 1 tile or
 *                   more where the capacity holds fewer than 32 tiles).
 *   workspace       device scratch of at least mla_decode_workspace_bytes;
 *                   its contents on entry do not matter
 *   out      fp32 [batch][heads][128]
 *
 * Sequence b attends to its first seq_lens[layer][b] cached tokens; a sequence
 * with no tokens gets an all-zero output row. Results do not depend on
 * workspace contents and are bit-identical from run to run for a fixed split
 * count; they differ between split counts only by rounding.
 */
int mla_decode_attn(const mla_cache *cache, int32_t layer, const void *q_nope,
                    const void *q_pe, const void *w_uk, const void *w_uv, int32_t heads,
                    float softmax_scale, int32_t num_splits, void *workspace,
                    size_t workspace_bytes, float *out, void *hip_stream);

/*
 * The fused decode step of one layer: store one new token per sequence, then
 * attend over every stored token, the new one included ("DeepSeek的MLA技术",
 * optimization 2: the RoPE key is cached already rotated by its position;
 * "Absorbed MLA Cache Optimization", section 2.1: store, then attend).
 *
 *   ckv_new   bf16 [batch][512]   the new token's latent
 *   kpe_new   bf16 [batch][64]    its RoPE key, NOT yet rotated
 *   q_nope, q_pe                  as for mla_decode_attn, but q_pe NOT yet rotated
 *   rope_cos, rope_sin  fp32 [rope_rows][32] angle tables, row p holding
 *                   cos / sin of p * theta_i for channel pair (2i, 2i+1);
 *                   rope_rows >= capacity + 1. Both NULL: nothing is rotated.
 *   the rest        as for mla_decode_attn
 *
 * For sequence b with length p = seq_lens[layer][b] (before the step):
 *   1. k_pe turns by table row p: y[2i] = x[2i] c - x[2i+1] s and
 *      y[2i+1] = x[2i] s + x[2i+1] c in fp32 (each product and sum rounded,
 *      no fused multiply-add), rounded to bf16 (nearest even); the token is
 *      then quantized and stored at row p exactly as mla_cache_append stores
 *      that bf16 input, and seq_lens[layer][b] becomes p + 1. A full sequence
 *      (p = capacity) stores nothing and keeps its length.
 *   2. q_pe of every head turns by the same row (fp32).
 *   3. Absorbed decode over the sequence's (now p + 1) tokens into out.
 * Three launches on hip_stream; the same workspace and split rules as
 * mla_decode_attn. Errors: as mla_cache_append and mla_decode_attn, plus
 * MLA_ERR_INVALID_ARG for one table NULL and the other not, tables not 4-byte
 * aligned, or rope_rows < capacity + 1; nothing is launched then.
 */
int mla_decode_step(const mla_cache *cache, int32_t layer, const void *ckv_new, const void *kpe_new,
                    const void *q_nope, const void *q_pe, const float *rope_cos,
                    const float *rope_sin, int32_t rope_rows, const void *w_uk, const void *w_uv,
                    int32_t heads, float softmax_scale, int32_t num_splits, void *workspace,
                    size_t workspace_bytes, float *out, void *hip_stream);

/*
 * The first launch of mla_decode_step on its own: store the new tokens (k_pe
 * turned), advance the lengths, and write the turned, absorbed queries into
 * the workspace. Calling it, then mla_decode_partial and mla_decode_combine
 * (same cache, layer, heads, num_splits and workspace, one stream) is exactly
 * mla_decode_step. Arguments and errors as there (w_uv and out are not taken).
 */
int mla_decode_step_begin(const mla_cache *cache, int32_t layer, const void *ckv_new,
                          const void *kpe_new, const void *q_nope, const void *q_pe,
                          const float *rope_cos, const float *rope_sin, int32_t rope_rows,
                          const void *w_uk, int32_t heads, float softmax_scale, int32_t num_splits,
                          void *workspace, size_t workspace_bytes, void *hip_stream);

/*
 * Several layers in one call. The configuration with independent layers
 * (one decode step of each of a model's layers over the same batch) runs as
 * one set of launches instead of one per layer: the balanced plan then cuts
 * the tiles of every (layer, sequence) pair, layer after layer, into equal
 * runs, so no launch ends on the tail of one layer's work.
 *
 *   layer0, layer_count   layers [layer0, layer0 + layer_count) of the cache,
 *                         layer_count >= 1
 *   every per-layer argument is stacked over those layers, layer-major:
 *     q_nope bf16 [layer_count][batch][heads][128], q_pe [layer_count][batch][heads][64],
 *     w_uk [layer_count][heads][128][512], w_uv [layer_count][heads][512][128],
 *     out fp32 [layer_count][batch][heads][128];
 *     for the step, ckv_new bf16 [layer_count][batch][512], kpe_new [layer_count][batch][64]
 *   num_splits      as for one layer: W = num_splits * batch runs in all,
 *                   now over every layer's tiles (0 = auto: about three
 *                   workgroups per CU)
 *   workspace       mla_decode_workspace_bytes_layers for the same
 *                   layer_count, heads and num_splits
 *
 * mla_decode_attn_layers over one layer is mla_decode_attn; mla_decode_step_layers
 * over one layer is mla_decode_step. Over several layers each layer's result
 * is what the one-layer call gives for that layer, up to the rounding that
 * depends on where the runs are cut. Errors as for the one-layer calls;
 * MLA_ERR_INVALID_ARG for a layer range outside the cache.
 */
int mla_decode_workspace_bytes_layers(const mla_cache *cache, int32_t layer_count, int32_t heads,
                                      int32_t num_splits, size_t *bytes);
int mla_decode_auto_splits_layers(const mla_cache *cache, int32_t layer_count, int32_t heads,
                                  int32_t *num_splits);
int mla_decode_attn_layers(const mla_cache *cache, int32_t layer0, int32_t layer_count, const void *q_nope,
                           const void *q_pe, const void *w_uk, const void *w_uv, int32_t heads,
                           float softmax_scale, int32_t num_splits, void *workspace, size_t workspace_bytes,
                           float *out, void *hip_stream);
int mla_decode_step_layers(const mla_cache *cache, int32_t layer0, int32_t layer_count, const void *ckv_new,
                           const void *kpe_new, const void *q_nope, const void *q_pe, const float *rope_cos,
                           const float *rope_sin, int32_t rope_rows, const void *w_uk, const void *w_uv,
                           int32_t heads, float softmax_scale, int32_t num_splits, void *workspace,
                           size_t workspace_bytes, float *out, void *hip_stream);

/* The phases of the layer-range calls, as for one layer below (layer0 only
 * where the cache is read or written). */
int mla_decode_step_begin_layers(const mla_cache *cache, int32_t layer0, int32_t layer_count,
                                 const void *ckv_new, const void *kpe_new, const void *q_nope, const void *q_pe,
                                 const float *rope_cos, const float *rope_sin, int32_t rope_rows,
                                 const void *w_uk, int32_t heads, float softmax_scale, int32_t num_splits,
                                 void *workspace, size_t workspace_bytes, void *hip_stream);
int mla_decode_absorb_layers(const mla_cache *cache, int32_t layer_count, const void *q_nope, const void *q_pe,
                             const void *w_uk, int32_t heads, float softmax_scale, int32_t num_splits,
                             void *workspace, size_t workspace_bytes, void *hip_stream);
int mla_decode_partial_layers(const mla_cache *cache, int32_t layer0, int32_t layer_count, int32_t heads,
                              int32_t num_splits, void *workspace, size_t workspace_bytes, void *hip_stream);
int mla_decode_combine_layers(const mla_cache *cache, int32_t layer_count, const void *w_uv, int32_t heads,
                              int32_t num_splits, void *workspace, size_t workspace_bytes, float *out,
                              void *hip_stream);

/*
 * The three phases of mla_decode_attn, for callers that schedule them
 * separately (for example to time or overlap them). Calling, on one stream and
 * with one workspace, mla_decode_absorb, then mla_decode_partial, then
 * mla_decode_combine with the same cache, heads and num_splits is exactly
 * mla_decode_attn: same kernels, same results. Arguments mean what they mean
 * there; each phase validates them the same way.
 *
 *   absorb    q_abs = softmax_scale * log2(e) * q_nope W_UK[h], and q_pe scaled
 *             the same way, into the workspace (fp16)
 *   partial   split-KV attention of each run of tiles (see num_splits) over
 *             the cache of `layer`: per (run, sequence) running max, sum and
 *             unnormalized latent sum
 *             into the workspace (the hot loop)
 *   combine   log-sum-exp merge of the splits, normalization, and projection
 *             through W_UV into out
 */
int mla_decode_absorb(const mla_cache *cache, const void *q_nope, const void *q_pe,
                      const void *w_uk, int32_t heads, float softmax_scale, int32_t num_splits,
                      void *workspace, size_t workspace_bytes, void *hip_stream);
int mla_decode_partial(const mla_cache *cache, int32_t layer, int32_t heads, int32_t num_splits,
                       void *workspace, size_t workspace_bytes, void *hip_stream);
int mla_decode_combine(const mla_cache *cache, const void *w_uv, int32_t heads, int32_t num_splits,
                       void *workspace, size_t workspace_bytes, float *out, void *hip_stream);

/*
 * Dequantize one layer of the cache ("get" of section 2.1 of the report):
 *   ckv_out  fp32 [batch][capacity][512], kpe_out fp32 [batch][capacity][64].
 * Rows at or past seq_lens[layer][b] are written as zeros. Either output may
 * be NULL to skip it. A test and inspection aid, not on the decode path.
 */
int mla_cache_get(const mla_cache *cache, int32_t layer, float *ckv_out, float *kpe_out,
                  void *hip_stream);

/*
 * RoPE angle tables for mla_decode_step ("DeepSeek的MLA技术", optimization 2,
 * reads the rotary embedding as first defined: channel pair (2i, 2i+1) of
 * the 64 turns by the angle p * theta_i, theta_i = base^(-2i/64)):
 *   cos_out, sin_out  fp32 [rows][32] (device, 4-byte aligned), row p holding
 *                     cos and sin of p * theta_i, each evaluated in fp64 and
 *                     rounded to fp32 (nearest even); theta_i is computed on
 *                     the host in fp64.
 *   rows >= 0 (0 is a no-op); base > 0 and finite (10000 in the rotary
 *   embedding's definition).
 * One launch on hip_stream. MLA_ERR_INVALID_ARG for a null or misaligned
 * pointer, rows < 0 or a bad base.
 */
int mla_rope_tables(float *cos_out, float *sin_out, int32_t rows, double base, void *hip_stream);

/*
 * mla_decode_attn without a workspace argument, for callers that cannot
 * allocate device memory at the call (code under HIP graph capture, tight
 * serving loops, harnesses that forbid allocation). It allocates nothing:
 * its workspace is a library-owned device array of MLA_STATIC_SCRATCH_BYTES,
 * one per GPU, held until the process ends and shared by every call on that
 * GPU. Calls that overlap on one GPU (on different streams, or from several
 * threads) race on it and give undefined results; calls in stream order are
 * fine. Its contents on entry do not matter.
 *
 * Arguments, results and errors as mla_decode_attn. MLA_ERR_WORKSPACE when
 * the workspace this cache, head count and split count need (what
 * mla_decode_workspace_bytes reports) exceeds MLA_STATIC_SCRATCH_BYTES;
 * nothing is launched then. num_splits = 0 picks the split count as
 * mla_decode_attn does.
 */
#define MLA_STATIC_SCRATCH_BYTES ((size_t)64 << 20)
int mla_decode_attn_static(const mla_cache *cache, int32_t layer, const void *q_nope, const void *q_pe,
                           const void *w_uk, const void *w_uv, int32_t heads, float softmax_scale,
                           int32_t num_splits, float *out, void *hip_stream);

/*
 * A measurement aid, not part of the decode path: reads `bytes` (a multiple of
 * 16) of device memory at `buf` (16-byte aligned) with a plain streaming
 * access pattern, as one launch of sink_words workgroups of 256 threads, and
 * writes one word per workgroup to sink (device uint32 [sink_words]), the XOR
 * of the words it read. nontemporal != 0: the loads carry the non-temporal
 * hint (the lines are not kept in the caches); 0: the default policy (the
 * lines are allocated in the caches, which evicts what they held). Timing it
 * gives the achievable HBM read rate beside the published peak.
 */
int mla_stream_read(const void *buf, size_t bytes, uint32_t *sink, int32_t sink_words, int32_t nontemporal,
                    void *hip_stream);

/*
 * A measurement aid, not part of the decode path: one launch of `workgroups`
 * workgroups of 256 threads, each wave issuing iters x 8 independent 16x16x32
 * fp16 matrix products (16384 flop each) in 8 accumulator chains; sink
 * (device float [workgroups * 256]) receives each lane's sum of its
 * accumulators. Timing it gives the achievable matrix-unit rate beside the
 * published dense fp16 peak. MLA_ERR_INVALID_ARG for a null or misaligned sink,
 * workgroups < 1 or iters < 0.
 */
int mla_mfma_rate(float *sink, int32_t workgroups, int32_t iters, void *hip_stream);

/* Static description of a status code. */
const char *mla_status_str(int status);

#ifdef __cplusplus
}
#endif

#endif /* MLA_KV_H */
