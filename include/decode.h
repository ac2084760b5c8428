/*
 * decode.h -- C ABI of libdecode.so: one LLaMA-style decoder step on an
 * MI355X (gfx950), with block-quantized weights and an f16 KV cache.
 *
 * The calls follow the inference loop of the article "llama.cpp AI LLM
 * Engine - how it works" (romankryvolapov.com): load the weights (steps 2-6),
 * create a context that owns the KV cache and every work buffer (step 7),
 * run a prompt as a batch split into ubatches (steps 10-13), run one new
 * token per step (the generation loop of step 8 and the KV-cache appendix),
 * read the logits (step 14) and take the greedy token or run the sampler
 * chain on the device (step 15).  Tokenization and text are not part of
 * this library.
 *
 * Conventions for every call:
 *  - Handles are opaque and owned by the library.
 *  - Host arrays passed in are read during the call only; the caller keeps
 *    ownership.  Pointers returned stay valid until the next prefill /
 *    decode / free on the same context.
 *  - Device work runs on one HIP stream: the one given at creation
 *    (hip_stream, a hipStream_t); a context created with NULL makes and owns
 *    a non-blocking stream of its own (decode graphs are captured on it).
 *    A prefill call of several ubatches also runs some of them on streams
 *    the context owns (DECODE_PREFILL_LANES below); those first wait for the
 *    context's stream, and before the call returns the context's stream is
 *    made to wait for them, so work queued on it afterwards sees the whole
 *    call.
 *  - Calls on one context must not overlap (no internal locking).
 *  - Errors are reported through return values (documented per call) and
 *    a message to the log callback; nothing aborts the process.
 */
#ifndef DECODE_H
#define DECODE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Element types.  Q8_0: blocks of 32 weights = f16 scale + 32 int8 codes
 * (34 bytes).  Q4_0: blocks of 32 weights = f16 scale + 16 bytes of 4-bit
 * codes offset by 8; byte k holds code k (low nibble) and code k+16 (high
 * nibble) (18 bytes).  The article names these as GGUF tensor types of
 * fixed-size blocks sharing one scale (step 2c).
 * Q4_K (named there among the k-quant types, not defined): super-blocks of
 * 256 weights in 144 bytes = f16 d, f16 dmin, 12 bytes of six-bit sub-block
 * scales sc_j and mins m_j (j = 0..7, 32 weights each), 128 bytes of 4-bit
 * codes q; a weight of sub-block j is d * sc_j * q - dmin * m_j.  For j < 4,
 * sc_j and m_j are the low six bits of bytes j and j + 4 of the 12; for j >= 4
 * they are the low / high nibble of byte j + 4 with the top two bits of bytes
 * j - 4 / j above.  Code byte 32g + l holds weight 64g + l (low nibble) and
 * 64g + 32 + l (high nibble).  This is the GGUF super-block, so files carry
 * it unchanged.  The library quantizes fp32 weights to it with a min-max
 * rule (per sub-block: the min maps to code 0 and the max to code 15, up to
 * the six-bit rounding of sc_j and m_j, rounded up; codes rounded half away
 * from zero), not with llama.cpp's scale search. */
typedef enum { DEC_F32 = 0, DEC_F16 = 1, DEC_Q8_0 = 2, DEC_Q4_0 = 3, DEC_Q4_K = 4 } dec_type;

/* Shape limits.  With quantized weights every matrix row (n_embd,
 * n_head * head_dim, n_ff) holds at most DEC_MAX_ROW elements: a decode step
 * keeps one whole input row on chip.  A context holds at most DEC_MAX_CTX
 * positions per sequence (split-K attention takes at most 1024 chunks of 64
 * positions).  Larger shapes are rejected at load / context creation. */
enum { DEC_MAX_ROW = 16384, DEC_MAX_CTX = 65536 };

/* Hyper-parameters (the article's step 4: embedding length, block count,
 * feed-forward length, head count, KV head count, RoPE frequency base).
 * wtype applies to every 2-D matrix (F32, Q8_0, Q4_0 or Q4_K); kvtype is the
 * cache element type (F32, F16, or Q8_0: the KV-cache appendix's separately
 * typed key / value cache, here one type for both; each cached head row is
 * coded in 32-element Q8_0 blocks as it is appended, from the fp32 K / V
 * values, and attention reads code * scale).  Quantized weight types need
 * n_embd, n_ff and n_head*head_dim to be multiples of 32 (of 256 for Q4_K)
 * and at most DEC_MAX_ROW; head_dim must be 64, 128 or 256, and n_head a multiple of
 * n_head_kv with at most 8 query heads per KV head. */
typedef struct {
    int32_t n_layer, n_embd, n_head, n_head_kv, head_dim, n_ff, n_vocab;
    float   rms_eps;     /* 1e-5 */
    float   rope_base;   /* 10000 */
    int32_t wtype, kvtype;
} dec_hparams;

/* fp32 source weights, row-major [out][in] (the article's step 6 tensor set
 * for the LLaMA family: tok_embd, output_norm, output, and per layer
 * attn_norm, q/k/v, wo, ffn_norm, ffn_gate, ffn_up, ffn_down).
 * Per-layer members are arrays of n_layer pointers.  Each pointer may be
 * host memory or device memory of the current HIP device; the library
 * copies / quantizes them on the device during dec_model_load and does not
 * keep them.  Shapes: tok_embd, output [n_vocab][n_embd]; wq
 * [n_head*head_dim][n_embd]; wk, wv [n_head_kv*head_dim][n_embd]; wo
 * [n_embd][n_head*head_dim]; ffn_gate, ffn_up [n_ff][n_embd]; ffn_down
 * [n_embd][n_ff]; norms [n_embd]. */
typedef struct {
    const float *tok_embd, *output_norm, *output;
    const float *const *attn_norm, *const *wq, *const *wk, *const *wv, *const *wo;
    const float *const *ffn_norm, *const *ffn_gate, *const *ffn_up, *const *ffn_down;
} dec_weights;

/* Optional device-memory provider.  alloc returns a device pointer of at
 * least `bytes` (aligned to 256) or NULL; free releases it.  NULL allocator
 * -> hipMalloc / hipFree.  The Python binding routes this to PyTorch. */
typedef struct {
    void *(*alloc)(size_t bytes, void *ud);
    void  (*free)(void *ptr, void *ud);
    void  *ud;
} dec_allocator;

typedef struct dec_model dec_model;
typedef struct dec_ctx   dec_ctx;

/* Loads (copies, and for Q8_0 / Q4_0 / Q4_K quantizes on the device) every weight.
 * Returns a model handle, or NULL on invalid hyper-parameters, a NULL
 * weight pointer, allocation failure or a device error (article step 2a:
 * the load entry returns the model or nullptr).  The allocator struct is
 * copied; hip_stream is used for the load only. */
dec_model *dec_model_load(const dec_hparams *hp, const dec_weights *w,
                          const dec_allocator *alloc, void *hip_stream);

/* Tensor ids for dec_model_tensor_blocks. */
enum { DEC_T_TOK_EMBD = 0, DEC_T_OUTPUT = 1, DEC_T_WQ = 2, DEC_T_WK = 3, DEC_T_WV = 4,
       DEC_T_WO = 5, DEC_T_FFN_GATE = 6, DEC_T_FFN_UP = 7, DEC_T_FFN_DOWN = 8 };

/* Copies one stored matrix to host memory dst in its file form: GGUF-style
 * blocks (34 or 18 bytes each, row-major, scale first) for Q8_0 / Q4_0,
 * 144-byte super-blocks for Q4_K, or fp32 rows for F32.  `layer` is ignored for tok_embd and output.  Returns
 * the byte count; when dst is NULL or cap is too small returns minus the
 * needed size (the article's size-probe convention, step 9); 0 on a bad id
 * or layer.  Synchronizes the load stream. */
int64_t dec_model_tensor_blocks(const dec_model *m, int32_t tensor_id, int32_t layer,
                                void *dst, size_t cap);

/* Frees the model (the caller owns what the load entry returned, article
 * step 2a, where a half-built model is freed before nullptr is returned).
 * When contexts created from it are still alive, the weights are released
 * together with the last of them. */
void dec_model_free(dec_model *m);

/* ---- GGUF v3 model files (article steps 2b-2c and its GGUF reference
 * section; tensor names of step 6, hyper-parameter keys of step 4) ---------
 * Layout: magic "GGUF", version 3, tensor count, key/value count; the
 * key/value pairs; one record per tensor (name, dimensions with the row
 * length first, element type, data offset); the data section at the next
 * multiple of general.alignment (32 when absent).  Matrices are Q4_0 (18-byte
 * blocks, file type 2), Q8_0 (34-byte blocks, type 8), Q4_K (144-byte
 * super-blocks, type 12) or F32, all of one type; norm vectors F32.
 * Keys read: general.architecture ("llama"), llama.embedding_length,
 * llama.block_count, llama.feed_forward_length, llama.attention.head_count
 * (required); llama.attention.head_count_kv (default head_count),
 * llama.attention.key_length or llama.rope.dimension_count (default
 * embedding_length / head_count), llama.attention.layer_norm_rms_epsilon
 * (1e-5), llama.rope.freq_base (10000).  Unknown keys and extra tensors are
 * ignored; output.weight may be absent (tied to token_embd.weight). */

/* Validates a file without loading it and fills *hp (kvtype = DEC_F16).
 * Returns the tensor count, or: -1 cannot open / bad arguments, -4 not GGUF,
 * -5 a version other than 3, -6 malformed or truncated records, -7 a
 * duplicated tensor name, -8 tensor data outside the file, -9 a missing key
 * or tensor, or one of the wrong shape or type mix, -10 an element type not
 * handled.  Touches no device. */
int32_t dec_gguf_inspect(const char *path, dec_hparams *hp);

/* Loads a file that dec_gguf_inspect accepts.  The file is memory-mapped;
 * each tensor's bytes are copied from the mapping straight to the device,
 * where its blocks are split into codes and scales and placed in the fused
 * matrices.  kvtype: the cache type (DEC_F16, DEC_F32 or DEC_Q8_0).  NULL on any error
 * (the reason is logged). */
dec_model *dec_model_load_gguf(const char *path, int32_t kvtype, const dec_allocator *alloc, void *hip_stream);

/* Writes the model as a GGUF v3 file in the layout above (its stored type,
 * the exact blocks of dec_model_tensor_blocks).  0, -1 bad arguments, -3 an
 * I/O or device error. */
int32_t dec_model_save_gguf(const dec_model *m, const char *path);

/* Context parameters (article step 7).  n_ctx: positions per sequence,
 * rounded up to a multiple of 256 (0 -> 4096), at most DEC_MAX_CTX.  n_batch: most tokens one
 * prefill call may take (0 -> n_ctx, clamped to n_ctx).  n_ubatch: most
 * tokens run through the layers at once (0 -> 512, clamped to n_batch).
 * n_seq_max: independent sequences, each with its own n_ctx cells
 * (0 -> 1).  kv_unified must be 0 (one cache stream per sequence).
 * abort_cb (optional) is polled between ubatches; a nonzero return stops
 * the call with status 2. */
typedef struct {
    uint32_t n_ctx, n_batch, n_ubatch, n_seq_max;
    int32_t  kv_unified;
    void    *hip_stream;
    int    (*abort_cb)(void *ud);
    void    *abort_ud;
} dec_ctx_params;

/* Creates a context and allocates, for the worst case, the KV cache
 * (n_layer x n_seq_max x n_ctx positions), the activation buffers for
 * n_ubatch tokens, and the logits buffer (n_batch rows).  Nothing is
 * allocated afterwards (the article's worst-case reservation, step 7 / 13b).
 * Returns NULL on invalid parameters or allocation failure.
 *
 * Environment switches, read here and applied to every context of the
 * process from then on (tuning and measurement aids; the defaults are the
 * paths the library is validated on):
 *   DECODE_GEMM_F16=1     ubatches of more than 64 tokens take f16 GEMM
 *                         operands (weights f16(d*q), activations f16): about
 *                         1.65x faster prefill, but at the 8B shape the
 *                         logits move about 3.5e-2 from the exact result
 *   DECODE_GEMM_SKINNY=0  ubatches of at most 32 tokens use the tiled GEMM
 *                         on every matrix (same exact operands)
 *   DECODE_GEMM_DW=0      ubatches of more than 64 tokens take the
 *                         256-feature direct-to-LDS GEMM instead of the
 *                         512-feature wide form (bitwise the same results;
 *                         the wide form is faster)
 *   DECODE_PREFILL_ATTN=splitk  prefill attention through the split-K
 *                         decode kernels instead of the flash kernel
 *   DECODE_PREFILL_LANES=n  buffer sets and streams the ubatches of a prefill
 *                         call go round (1..4, default 2; 1 runs them one
 *                         after another); each
 *                         extra lane holds one ubatch's activations and
 *                         GEMM workspace.  With n >= 2 the wide GEMM form
 *                         splits K at most 4 ways (8 with one lane), so rows
 *                         can differ from one lane's in rounding; they are
 *                         bitwise the same for every n >= 2
 *   DECODE_STEP_KERNEL=1  see dec_set_step_kernel */
dec_ctx *dec_ctx_new(dec_model *m, const dec_ctx_params *p);

/* Runs n prompt tokens of one sequence, continuing at seq_pos_max(seq)+1
 * (article step 10: missing positions are filled from the cache).  The
 * batch is split into ubatches of at most n_ubatch tokens, and cache cells
 * for all of them are reserved before any runs (steps 11-12).  Logits are
 * produced for the last token only, or for every token when output_all is
 * nonzero; rows are appended in batch order (step 14).
 * Returns 0 ok | 1 not enough free cells (nothing changed) | 2 aborted by
 * abort_cb (finished ubatches stay in the cache, later ones are rolled
 * back) | -1 invalid input (n <= 0, n > n_batch, token out of range, bad
 * seq_id) | -2 allocation failure | -3 device error (the article's
 * llama_decode codes, step 11). */
int32_t dec_prefill(dec_ctx *c, const int32_t *tokens, int32_t n, int32_t seq_id,
                    int32_t output_all);

/* One generation step: token i belongs to sequence seq_ids[i] and is placed
 * at that sequence's next position; K and V are appended before attending
 * (KV-cache appendix).  All n sequences must differ; n <= n_seq_max.
 * Logits are produced for every token, row i for token i.  The first step
 * with a given n runs kernel by kernel; the second is captured as a HIP
 * graph and every later one replays it (the article's graph reuse, step
 * 13b).  Return codes as dec_prefill. */
int32_t dec_decode(dec_ctx *c, const int32_t *tokens, const int32_t *seq_ids, int32_t n);

/* Logits row i of the last call: i >= 0 is the i-th output row, -1 the
 * last one (article step 14, llama_get_logits_ith).  Synchronizes the
 * stream and copies the rows to host memory on first use.  Returns n_vocab
 * floats, or NULL for an invalid index or when no call has produced
 * logits. */
const float *dec_get_logits(dec_ctx *c, int32_t i);

/* Greedy token of output row i (same indexing as dec_get_logits): the
 * index of the largest logit, lowest index on ties, computed on the device
 * (article step 15, greedy sampler; on-device sampling avoids copying the
 * logits).  Returns -1 for an invalid index. */
int32_t dec_argmax(dec_ctx *c, int32_t i);

/* Copies the greedy tokens of all n output rows of the last call into out
 * (n = the value returned); returns -1 if cap is too small. */
int32_t dec_argmax_all(dec_ctx *c, int32_t *out, int32_t cap);

/* ---- sampler chain (article step 15: the sampler list) ------------------
 * Applied in the article's order: repeat penalty on the recent history,
 * top-k, top-p, min-p, temperature, then one token drawn from the softmax of
 * the survivors.  Readings where the article gives only the idea: the
 * penalty divides a positive logit and multiplies a negative one, once per
 * distinct token of the last penalty_last_n accepted tokens; candidates are
 * ordered by logit, the lower token id first on ties; top-p keeps the
 * shortest prefix whose weight exp(l - leader) reaches top_p of the total;
 * min-p keeps weights >= min_p; the temperature divides the survivors'
 * logits; the draw takes the first candidate whose inclusive cumulative
 * weight exceeds u times the total, with u the top 24 bits of output number
 * `draws` of SplitMix64(seed) (Steele, Lea, Flood 2014), draws counting the
 * sampler's draws so far.  All weights are fp32. */
typedef struct {
    int32_t  top_k;            /* 1..1024 candidates kept by top-k */
    float    top_p;            /* (0, 1]; 1 disables */
    float    min_p;            /* [0, 1); 0 disables */
    float    temp;             /* > 0; <= 0 picks the leader (greedy) */
    float    repeat_penalty;   /* >= 1; 1 disables */
    int32_t  penalty_last_n;   /* 0..64 accepted tokens the penalty looks at */
    uint64_t seed;             /* seed of the draw stream */
} dec_sampler_params;

typedef struct dec_sampler dec_sampler;

/* A sampler with its own token history and draw count (the chain of the
 * article's llama_sampler_chain_init / _add: parameters are fixed when it is
 * built).  Allocates 260 bytes of mapped pinned host memory (the history
 * window and the drawn token pass through it, read and written by the
 * kernel directly) and a stream on the current device.  Not thread-safe: one
 * caller at a time per sampler.  NULL on parameters out of range or
 * allocation failure.  Logits must not be NaN (the drawn token is then
 * unspecified, or -3). */
dec_sampler *dec_sampler_new(const dec_sampler_params *p);

/* Appends token (>= 0) to the history, e.g. the prompt.  0, or -1. */
int32_t dec_sampler_accept(dec_sampler *s, int32_t token);

/* Samples from output row i of ctx's last call (indexing as dec_get_logits)
 * on the device, on ctx's stream; accepts the token and counts the draw.
 * Synchronizes the stream.  Returns the token, -1 for an invalid row or a
 * vocabulary over 32768 / below top_k, -3 on a device error. */
int32_t dec_sampler_sample(dec_sampler *s, dec_ctx *c, int32_t i);

/* The same chain on a logits row given by the caller (the article's chain
 * applied to an arbitrary candidate array): n_vocab floats in device memory
 * or host memory (copied to the device first), sampled on hip_stream (NULL:
 * the sampler's own stream).  Accepts the token and counts the draw.
 * Returns the token, -1 for bad arguments, -3 on a device error. */
int32_t dec_sampler_sample_row(dec_sampler *s, const float *logits, int32_t n_vocab, void *hip_stream);

/* Forgets the history and restarts the draw stream at draw 0. */
void dec_sampler_reset(dec_sampler *s);

/* Number of draws made (the index of the next one). */
int64_t dec_sampler_draws(const dec_sampler *s);

void dec_sampler_free(dec_sampler *s);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the chain
 * of dec_sampler_sample_row as one stateless call that allocates nothing.
 * p: the chain (same ranges as dec_sampler_new).  hist: the n_hist (0..64)
 * most recently accepted tokens, oldest first, host or device memory; the
 * penalty looks at the last penalty_last_n of them.  draw: the index of this
 * draw in the seed's stream (dec_sampler_draws before the equivalent
 * dec_sampler_sample_row call).  logits: n_vocab floats (top_k <= n_vocab <=
 * DEC_NOALLOC_MAX_VOCAB), device memory or host memory.  token_out: one
 * int32 in device memory or in mapped pinned host memory; the token is
 * written there by the kernel.  Enqueued on hip_stream (NULL: the null
 * stream) without synchronizing: the token is valid once the stream reaches
 * this point.  The window and a host row are staged in a fixed device buffer
 * of the library (about 128 KiB per GPU, held until the process ends), so
 * calls on one GPU must be ordered on one stream: calls that overlap on one
 * GPU race on that buffer.  Nothing is kept between calls; the caller keeps
 * the history and the draw count.  Returns 0 when enqueued, -1 for bad
 * arguments (token_out the device cannot write, ranges), -4 when n_vocab
 * exceeds DEC_NOALLOC_MAX_VOCAB (the reason is logged), -3 on a device
 * error. */
enum { DEC_NOALLOC_MAX_VOCAB = 32768 };
int32_t dec_sample_row_noalloc(const dec_sampler_params *p, const int32_t *hist, int32_t n_hist, uint64_t draw,
                               const float *logits, int32_t n_vocab, int32_t *token_out, void *hip_stream);

/* Largest cached position of a sequence, -1 when empty (the memory module's
 * seq_pos_max, KV-cache appendix). */
int32_t dec_seq_pos_max(const dec_ctx *c, int32_t seq);

/* Forgets every cached position of a sequence: the memory module's cells
 * of that sequence are free again, and its next token starts at position 0
 * (KV-cache appendix: seq_pos_max decides where a batch continues).
 * Returns 0, or -1 for a bad seq. */
int32_t dec_seq_clear(dec_ctx *c, int32_t seq);

/* Counters since creation (the article's "graphs reused" count, step 13b). */
typedef struct {
    int64_t n_prefill_calls, n_ubatches, n_decode_calls;
    int64_t n_graph_captures, n_graph_replays;
} dec_stats;
void dec_get_stats(const dec_ctx *c, dec_stats *out);

/* Kernel roles of one layer (and the final output projection) for the
 * timing probe. */
enum { DEC_K_QKV = 0, DEC_K_ATTN = 1, DEC_K_WO = 2, DEC_K_FFN_GU = 3, DEC_K_FFN_DOWN = 4,
       DEC_K_OUTPUT = 5, DEC_K_STEP = 6 };

/* Timing probe (the article's per-node evaluation callback, step 13b, in
 * measuring form): the launch(es) of kernel `role` in layer `layer` (layer
 * ignored for DEC_K_OUTPUT and DEC_K_STEP) go through hipExtLaunchKernel with a pair of HIP
 * events, which take the start time of the first kernel and the end time of
 * the last one.  Applies to prefill ubatches and to decode steps; a probed
 * decode step replays its graph in two parts around the directly launched
 * probed kernel.  DEC_K_STEP times the whole one-token decode step kernel
 * (see dec_set_step_kernel) between two events recorded around its launch;
 * any other role makes one-token decode steps take the per-layer kernels.
 * role < 0 disables.  Setting the probe resets the totals;
 * choosing a different role or layer also drops captured decode graphs.
 * Returns 0, or -1 on bad arguments. */
int32_t dec_set_probe(dec_ctx *c, int32_t role, int32_t layer);

/* Probe totals since dec_set_probe: summed kernel milliseconds (first start
 * to last end per probed unit) and the number of probed units.  Synchronizes the stream.
 * Returns 0, or -1 when no probe is set. */
int32_t dec_get_probe(dec_ctx *c, double *total_ms, int64_t *count);

/* Attainable ceilings of the current device, the measured counterparts of
 * the datasheet peaks that roofline fractions are taken against (the
 * article's point that prefill loads the compute units and decode loads
 * memory, KV-cache appendix, made quantitative).  Measurement aids: each
 * allocates, runs and frees its own buffers on hip_stream and synchronizes.
 *   dec_measure_stream_read: GB/s of a plain streaming read of `bytes`
 *     (>= 1 MiB; use several times the 256 MiB last-level cache) with 16-byte
 *     loads, averaged over `reps` passes after one untimed pass.
 *   dec_measure_mfma_f16: TFLOP/s of independent v_mfma_f32_32x32x16_f16 on
 *     register operands, 8 wavefronts per compute unit, `iters` loop
 *     iterations of 8 instructions each, over `reps` launches.
 * Return 0, -1 bad arguments, -2 allocation failure, -3 device error. */
int32_t dec_measure_stream_read(size_t bytes, int32_t reps, void *hip_stream, double *gbs);
int32_t dec_measure_mfma_f16(int32_t iters, int32_t reps, void *hip_stream, double *tflops);

/* Decode steps are captured as HIP graphs and replayed (on, the default) or
 * launched kernel by kernel (off): the article's graph reuse (step 13b,
 * can_reuse / graph_reuse_disable) as a switch.  Returns the previous
 * setting. */
int32_t dec_set_use_graphs(dec_ctx *c, int32_t on);

/* One-token decode steps (dec_decode with n = 1) as one persistent kernel:
 * every layer of the step (RMSNorm, QKV, RoPE, K/V append, attention,
 * output projection, SwiGLU FFN; then the output projection and the greedy
 * token), one block per compute unit, with grid barriers between the
 * layers' stages instead of kernel boundaries (graph reuse, step 13b, taken
 * to its limit).  Available where the context supports it: Q8_0 / Q4_0
 * weights, an f16 cache, head_dim 64 or 128, at most 8 query heads per KV
 * head, d_model and n_head * head_dim at most 4096, n_ff at most 16384, and
 * a cooperative launch of one block per compute unit.  Off by default (on
 * one MI355X the per-layer graph is faster); the environment variable
 * DECODE_STEP_KERNEL=1 turns the default on.  It is used only while
 * graphs are on and no probe role other than DEC_K_STEP is set.  Results
 * agree with the per-layer kernels within rounding (the attention merges
 * its partial sums in another order).  Every wait inside the kernel is
 * bounded.  If one times out (blocks not co-resident), the step failed: the
 * next call on the context that reads results or runs work (dec_get_logits
 * returns NULL, dec_argmax / dec_argmax_all -1, dec_sampler_sample,
 * dec_decode and dec_prefill -3) reports it once and undoes the step (the
 * sequence's position returns to what it was before, so the cache row it
 * wrote is free again, and the call's outputs are dropped); barrier state is
 * reset, and later calls work normally.
 * on: 1 use, 0 do not use, -1 query.  Returns the setting before the call
 * (0 or 1), or -1 when the context cannot use the kernel (nothing changes). */
int32_t dec_set_step_kernel(dec_ctx *c, int32_t on);

/* Frees a context: its KV cache, work buffers, captured graphs and (if it
 * made one) its stream, everything reserved at creation (article step 7).
 * Waits for the context's queued work first. */
void dec_ctx_free(dec_ctx *c);

/* Log sink: level 0 debug, 1 info, 2 warning, 3 error (the library's form
 * of the LLAMA_LOG_* messages the article's code emits, e.g. the load and
 * decode error reports of steps 2a and 11).  Process-wide.  NULL restores
 * the default (errors to stderr). */
void dec_set_log_callback(void (*cb)(int level, const char *msg, void *ud), void *ud);

/* Library build string (target, version). */
const char *dec_version(void);

#ifdef __cplusplus
}
#endif
#endif
