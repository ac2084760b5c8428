/*
 * oracle.h -- plain, slow, CPU reference of one LLaMA-style decoder step.
 *
 * TEST INFRASTRUCTURE ONLY.  Only tests/, the smoke entry point and the CPU
 * baseline leg of the benchmark may load this library.  The product path
 * (the HIP library under decode_amd/) never links, loads or calls it, and it
 * shares no code, header, table or helper with that path.
 *
 * Source of the method: the article "llama.cpp AI LLM Engine - how it works"
 * (romankryvolapov.com, Bulgarian and Russian editions).  Every function
 * below names the part of the article it follows.  Where the article is
 * silent (it names Q8_0 and "normalization" but prints no formula), the
 * plainest reading is taken; each such reading is marked READING.
 *
 * Precision: the library is built twice from the same source.
 *   liboracle_f64.so : ORC_REAL = double (the oracle of record for parity)
 *   liboracle_f32.so : ORC_REAL = float  (the fp32 decoder; used to bound
 *                                         the oracle's own rounding error)
 * Block quantizers and the f16 conversion are integer-producing and always
 * run in fp32 (both builds), the precision in which the block formats are
 * defined.  Every dot product and sum runs sequentially in index order;
 * OpenMP splits only independent outputs, so results do not depend on the
 * thread count.
 *
 * Parity pins: every function here is pinned by tests/test_oracle_*.py
 * against closed forms, brute force, library routines or hand-computed
 * fixtures (tests/golden/).  No function is "parity unpinned" except the
 * end-to-end equality with llama.cpp itself, which cannot be checked here
 * (for Q4_K also its quantizer: the article gives none, so the min-max
 * quantizer in oracle.c is a reading; the block layout and decode rule are
 * pinned by a hand-worked block).
 */
#ifndef DECODE_ORACLE_H
#define DECODE_ORACLE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#ifndef ORC_REAL
#define ORC_REAL double
#endif
typedef ORC_REAL orc_real;

/* Element types.  Values chosen by this file alone. */
enum { ORC_T_F32 = 0, ORC_T_F16 = 1, ORC_T_Q8_0 = 2, ORC_T_Q4_0 = 3, ORC_T_Q4_K = 4 };

/* sizeof(orc_real): 8 for the f64 build, 4 for the f32 build. */
int32_t orc_real_size(void);

/* ---- IEEE binary16 ------------------------------------------------------ */
uint16_t orc_f16_from_f32(float x);   /* round to nearest, ties to even */
uint16_t orc_f16_from_f64(double x);  /* round to nearest, ties to even, one rounding */
float    orc_f16_to_f32(uint16_t h);  /* exact */
void     orc_f16_from_f32_n(const float *x, int64_t n, uint16_t *h);
void     orc_f16_to_f32_n(const uint16_t *h, int64_t n, float *x);

/* ---- block codecs (32 elements per block) -------------------------------
 * Q8_0 block = 34 bytes: f16 scale d (little endian), then 32 int8 codes.
 * Q4_0 block = 18 bytes: f16 scale d, then 16 bytes; byte k holds code k in
 * its low nibble and code k+16 in its high nibble.
 * n must be a multiple of 32.  Returns bytes written (or -1 on bad n).     */
int64_t orc_q8_0_quantize(const float *x, int64_t n, uint8_t *blocks);
int64_t orc_q4_0_quantize(const float *x, int64_t n, uint8_t *blocks);
void    orc_q8_0_dequantize(const uint8_t *blocks, int64_t n, float *y);
void    orc_q4_0_dequantize(const uint8_t *blocks, int64_t n, float *y);
/* Q4_K super-block = 256 elements in 144 bytes: f16 d, f16 dmin, 12 bytes of
 * six-bit sub-block scales and mins, 128 bytes of 4-bit codes (see
 * oracle.c).  n must be a multiple of 256. */
int64_t orc_q4_k_quantize(const float *x, int64_t n, uint8_t *blocks);
void    orc_q4_k_dequantize(const uint8_t *blocks, int64_t n, float *y);
/* The eight (scale, min) six-bit pairs of one super-block, unpacked. */
void    orc_q4_k_scales(const uint8_t *block, int32_t *sc, int32_t *m);

/* ---- primitives (exposed for the pins) ---------------------------------- */
void orc_rmsnorm(const orc_real *x, const float *g, int32_t n, float eps, orc_real *y);
/* y[r] = sum_k deq(W)[r][k] * x[k]; W row-major [rows][cols] of type wtype
   (F32: float array; Q8_0/Q4_0/Q4_K: block bytes as above). */
void orc_matvec(int32_t wtype, const void *w, int32_t rows, int32_t cols,
                const orc_real *x, orc_real *y);
/* rotate n_heads consecutive head vectors of size hd in place, position pos */
void orc_rope(orc_real *v, int32_t n_heads, int32_t hd, int32_t pos, float base);
/* one query head against n cached rows: row j of K and of V starts at
   element j*ld and holds hd elements of type kvtype (F32 float / F16 uint16 /
   Q8_0 34-byte blocks of 32 elements; then ld, hd and the start of K and V
   are whole blocks).
   Row j sits at position row_pos[j] (row_pos == NULL: position j); rows whose
   position exceeds pos are masked.  Writes o[hd]; if w != NULL also the n
   softmax weights (exactly 0 for masked rows). */
void orc_attend(const orc_real *q, const void *K, const void *V, int32_t kvtype,
                int64_t ld, const int32_t *row_pos, int32_t n, int32_t hd,
                int32_t pos, orc_real *o, orc_real *w);
void orc_swiglu(const orc_real *u, const orc_real *v, int32_t n, orc_real *h);
int32_t orc_argmax(const orc_real *x, int32_t n);   /* lowest index on ties */

/* ---- the decoder --------------------------------------------------------- */
typedef struct {
    int32_t n_layer, n_embd, n_head, n_head_kv, head_dim, n_ff, n_vocab;
    float   rms_eps, rope_base;
    int32_t wtype;   /* F32, Q8_0, Q4_0 or Q4_K: every 2-D matrix            */
    int32_t kvtype;  /* F32, F16 or Q8_0 (Q8_0 needs head_dim % 32 == 0)     */
} orc_hparams;

/* fp32 source tensors, row-major [out][in]; per-layer entries are arrays of
   n_layer pointers.  Shapes: tok_embd/output [n_vocab][n_embd],
   wq [H*hd][d], wk/wv [Hkv*hd][d], wo [d][H*hd], ffn_gate/up [n_ff][d],
   ffn_down [d][n_ff], norms [d]. */
typedef struct {
    const float *tok_embd, *output_norm, *output;
    const float *const *attn_norm, *const *wq, *const *wk, *const *wv, *const *wo;
    const float *const *ffn_norm, *const *ffn_gate, *const *ffn_up, *const *ffn_down;
} orc_weights;

typedef struct orc_model orc_model;
typedef struct orc_ctx   orc_ctx;

/* Quantizes every matrix with this file's own codec.  NULL on bad input.
   The caller's arrays are only read during the call. */
orc_model *orc_model_new(const orc_hparams *hp, const orc_weights *w);
void       orc_model_free(orc_model *m);
/* Copies the encoded bytes of one tensor.  tensor id: 0 tok_embd, 1 output,
   2 wq, 3 wk, 4 wv, 5 wo, 6 ffn_gate, 7 ffn_up, 8 ffn_down (layer ignored
   for 0,1).  Returns the byte count, or -needed when cap is too small. */
int64_t    orc_model_tensor_bytes(const orc_model *m, int32_t tensor, int32_t layer,
                                  void *dst, int64_t cap);

/* n_seq independent sequences with n_ctx cached positions each. */
orc_ctx *orc_ctx_new(const orc_model *m, int32_t n_seq, int32_t n_ctx);
void     orc_ctx_free(orc_ctx *c);
int32_t  orc_seq_pos_max(const orc_ctx *c, int32_t seq);   /* -1 when empty */
void     orc_seq_clear(orc_ctx *c, int32_t seq);

/* Runs one token of sequence seq at position seq_pos_max(seq)+1: appends its
   K,V to the cache of every layer and, when logits != NULL, writes n_vocab
   logits.  Returns 0, or -1 on bad token/seq, 1 when the sequence is full. */
int32_t orc_eval(orc_ctx *c, int32_t seq, int32_t token, orc_real *logits);

/* Like orc_eval, and also returns the residual stream entering layer `tap`
   (tap == n_layer gives the stream before the final norm) into x_tap[n_embd]. */
int32_t orc_eval_tap(orc_ctx *c, int32_t seq, int32_t token, orc_real *logits,
                     int32_t tap, orc_real *x_tap);

/* Reads the cached K (which=0) or V (which=1) row of (layer, seq, pos, kv head)
   as float. Returns 0, or -1 when out of range. */
int32_t orc_kv_row(const orc_ctx *c, int32_t which, int32_t layer, int32_t seq,
                   int32_t pos, int32_t kv_head, float *out);

/* ---- sampler chain (the article's step 15 sampler list) ----------------
   Order as the article gives it: repeat penalty, top-k, top-p, min-p,
   temperature, then one token drawn from the softmax of what is left.
   Probabilities are computed in fp32, the precision the device uses for the
   same decisions. */
typedef struct {
    int32_t  top_k;            /* keep the k largest (<= 0: all) */
    float    top_p;            /* nucleus threshold in (0, 1]; 1 disables */
    float    min_p;            /* relative floor in [0, 1); 0 disables */
    float    temp;             /* > 0; <= 0 selects the leader (greedy) */
    float    repeat_penalty;   /* >= 1; 1 disables */
    int32_t  penalty_last_n;   /* history window for the penalty */
    uint64_t seed;             /* seed of the draw stream */
} orc_sampler_params;

/* Output number `index` (0-based) of SplitMix64 started at state `seed`,
   and its top 24 bits as a float in [0, 1). */
uint64_t orc_splitmix64(uint64_t seed, uint64_t index);
float    orc_uniform24(uint64_t seed, uint64_t index);

/* Runs the chain on n_vocab fp32 logits with the token history hist[n_hist]
   (oldest first) and draw number `draw`.  Returns the token, or -1 on bad
   arguments.  When ids/cum are not NULL (capacity n_vocab) they receive the
   surviving candidates in chain order and their inclusive cumulative
   weights; *n_kept, *target receive their count and the draw's target
   u * sum (both 0 for greedy). */
int32_t orc_sample(const float *logits, int32_t n_vocab, const int32_t *hist, int32_t n_hist,
                   const orc_sampler_params *p, uint64_t draw, int32_t *ids, float *cum,
                   int32_t *n_kept, float *target);

#ifdef __cplusplus
}
#endif
#endif
