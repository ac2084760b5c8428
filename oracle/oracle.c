/*
 * oracle.c -- plain CPU reference of one LLaMA-style decoder step.
 *
 * TEST INFRASTRUCTURE ONLY (see oracle.h).  Built with
 *   gcc -O2 -fopenmp -ffp-contract=off -fno-fast-math -DORC_REAL=double|float
 *
 * Article: "llama.cpp AI LLM Engine - how it works" (romankryvolapov.com).
 * The decoder below follows step 13b's per-layer graph scheme (input
 * normalization, Q/K/V, RoPE on Q and K, scores Q*K^T, causal mask, softmax,
 * weighted sum with V, output projection O, residual, normalization,
 * feed-forward of two linear layers with an activation between them,
 * residual; after the layers: keep requested rows, final normalization,
 * output matrix -> logits) and the appendix "KV-cache and the Prefill /
 * Decode stages" (K and V of the new token are appended to the cache first;
 * Q is then multiplied by every cached key, its own included).
 *
 * The cache is attended per token: each token reads the rows of its own
 * sequence at positions <= its own.  Old rows never change, so running the
 * tokens of a prompt one at a time is the plain definition of the causal
 * forward pass; ubatch splitting and graph reuse in the article are speed
 * devices and do not appear here.
 */
#include "oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>

int32_t orc_real_size(void) { return (int32_t)sizeof(orc_real); }

/* ======================================================================== */
/* IEEE binary16.  The article names F16 among the tensor element types     */
/* (step 2c, GGUF tensor info) but not the rounding; READING: IEEE 754      */
/* round-to-nearest-even, subnormals kept, overflow to infinity.            */
/* ======================================================================== */

uint16_t orc_f16_from_f64(double x)
{
    uint64_t u;
    memcpy(&u, &x, sizeof u);
    const uint16_t sign = (uint16_t)((u >> 48) & 0x8000u);
    const int ex = (int)((u >> 52) & 0x7ff);
    const uint64_t man = u & 0xFFFFFFFFFFFFFull;

    if (ex == 0x7ff)                      /* inf or NaN */
        return (uint16_t)(sign | (man ? 0x7e00u : 0x7c00u));
    if (ex == 0)                          /* zero or a double subnormal: far below 2^-25 */
        return sign;

    const uint64_t sig = man | (1ull << 52); /* value = sig * 2^(e-52) */
    const int e = ex - 1023;
    /* quantum of the target: 2^(e-10) for f16 normals, 2^-24 for subnormals */
    const int qexp = (e >= -14) ? (e - 10) : -24;
    const int shift = qexp - (e - 52);       /* >= 42 */
    if (shift >= 64)
        return sign;
    uint64_t q = sig >> shift;
    const uint64_t rem = sig & ((1ull << shift) - 1);
    const uint64_t half = 1ull << (shift - 1);
    if (rem > half || (rem == half && (q & 1)))
        q++;

    if (e >= -14) {
        int E = e + 15;
        if (q == (1u << 11)) { q >>= 1; E++; }
        if (E >= 31)
            return (uint16_t)(sign | 0x7c00u);
        return (uint16_t)(sign | ((unsigned)E << 10) | (unsigned)(q & 0x3ff));
    }
    /* subnormal; q == 1024 is the smallest normal and encodes as 0x0400 */
    return (uint16_t)(sign | (unsigned)q);
}

uint16_t orc_f16_from_f32(float x)
{
    return orc_f16_from_f64((double)x);   /* float -> double is exact */
}

float orc_f16_to_f32(uint16_t h)
{
    const uint32_t sign = (uint32_t)(h & 0x8000u) << 16;
    const int E = (h >> 10) & 0x1f;
    const uint32_t m = h & 0x3ffu;
    float v;
    if (E == 0) {
        v = ldexpf((float)m, -24);              /* zero / subnormal, exact */
        uint32_t b;
        memcpy(&b, &v, 4);
        b |= sign;
        memcpy(&v, &b, 4);
        return v;
    }
    uint32_t b;
    if (E == 31)
        b = sign | 0x7f800000u | (m << 13);
    else
        b = sign | ((uint32_t)(E - 15 + 127) << 23) | (m << 13);
    memcpy(&v, &b, 4);
    return v;
}

void orc_f16_from_f32_n(const float *x, int64_t n, uint16_t *h)
{
    for (int64_t i = 0; i < n; i++) h[i] = orc_f16_from_f32(x[i]);
}

void orc_f16_to_f32_n(const uint16_t *h, int64_t n, float *x)
{
    for (int64_t i = 0; i < n; i++) x[i] = orc_f16_to_f32(h[i]);
}

static uint16_t rd_u16(const uint8_t *p) { return (uint16_t)(p[0] | (p[1] << 8)); }
static void wr_u16(uint8_t *p, uint16_t v) { p[0] = (uint8_t)(v & 0xff); p[1] = (uint8_t)(v >> 8); }

/* ======================================================================== */
/* Block codecs.  The article (step 2c, GGUF tensor types) describes the    */
/* quantized types only as fixed-size blocks of elements sharing one scale. */
/* READING (32 elements, f16 scale, int8 codes / 4-bit codes offset 8):     */
/*  Q8_0: d = max|x| / 127, codes = x * (1/d) rounded half away from zero.  */
/*  Q4_0: m = the element of largest magnitude (sign kept, first on ties),  */
/*        d = m / -8, code = min(15, floor(x * (1/d) + 8.5)).               */
/* Both in fp32; the codes use the fp32 d, the stored scale is f16(d).      */
/* ======================================================================== */

int64_t orc_q8_0_quantize(const float *x, int64_t n, uint8_t *out)
{
    if (n < 0 || n % 32) return -1;
    const int64_t nb = n / 32;
    for (int64_t b = 0; b < nb; b++) {
        const float *xb = x + b * 32;
        uint8_t *ob = out + b * 34;
        float amax = 0.0f;
        for (int j = 0; j < 32; j++) {
            const float a = fabsf(xb[j]);
            if (a > amax) amax = a;
        }
        const float d = amax / 127.0f;
        const float id = (d != 0.0f) ? 1.0f / d : 0.0f;
        wr_u16(ob, orc_f16_from_f32(d));
        for (int j = 0; j < 32; j++) {
            const float t = xb[j] * id;
            const int qv = (int)roundf(t);      /* half away from zero */
            ob[2 + j] = (uint8_t)(int8_t)qv;
        }
    }
    return nb * 34;
}

int64_t orc_q4_0_quantize(const float *x, int64_t n, uint8_t *out)
{
    if (n < 0 || n % 32) return -1;
    const int64_t nb = n / 32;
    for (int64_t b = 0; b < nb; b++) {
        const float *xb = x + b * 32;
        uint8_t *ob = out + b * 18;
        float amax = 0.0f, m = 0.0f;
        for (int j = 0; j < 32; j++) {
            const float a = fabsf(xb[j]);
            if (a > amax) { amax = a; m = xb[j]; }
        }
        const float d = m / -8.0f;
        const float id = (d != 0.0f) ? 1.0f / d : 0.0f;
        wr_u16(ob, orc_f16_from_f32(d));
        int code[32];
        for (int j = 0; j < 32; j++) {
            const float t = xb[j] * id;
            const float s = t + 8.5f;
            int c = (int)floorf(s);
            if (c > 15) c = 15;
            if (c < 0) c = 0;
            code[j] = c;
        }
        for (int k = 0; k < 16; k++)
            ob[2 + k] = (uint8_t)(code[k] | (code[k + 16] << 4));
    }
    return nb * 18;
}

void orc_q8_0_dequantize(const uint8_t *blocks, int64_t n, float *y)
{
    for (int64_t b = 0; b < n / 32; b++) {
        const uint8_t *ib = blocks + b * 34;
        const float d = orc_f16_to_f32(rd_u16(ib));
        for (int j = 0; j < 32; j++) y[b * 32 + j] = (float)(int8_t)ib[2 + j] * d;
    }
}

void orc_q4_0_dequantize(const uint8_t *blocks, int64_t n, float *y)
{
    for (int64_t b = 0; b < n / 32; b++) {
        const uint8_t *ib = blocks + b * 18;
        const float d = orc_f16_to_f32(rd_u16(ib));
        for (int k = 0; k < 16; k++) {
            y[b * 32 + k]      = (float)((int)(ib[2 + k] & 0x0f) - 8) * d;
            y[b * 32 + k + 16] = (float)((int)(ib[2 + k] >> 4) - 8) * d;
        }
    }
}

/* ======================================================================== */
/* Q4_K.  The article names Q4_K among the GGUF tensor types (step 2c and   */
/* its GGUF reference section) without defining it.                         */
/* READING, layout (the GGUF super-block, so that blocks are interchangeable */
/* with GGUF files): 256 elements along a row in 8 sub-blocks of 32, stored */
/* in 144 bytes: d (f16), dmin (f16), 12 bytes s[] holding a six-bit scale  */
/* sc_j and a six-bit min m_j per sub-block, 128 bytes of 4-bit codes q.    */
/*   x = f32(d) * sc_j * q - f32(dmin) * m_j   (element of sub-block j)     */
/*   j < 4 : sc_j = s[j] & 63,  m_j = s[j+4] & 63                            */
/*   j >= 4: sc_j = (s[j+4] & 15) | (s[j-4] >> 6) << 4,                      */
/*           m_j  = (s[j+4] >> 4) | (s[j]   >> 6) << 4                       */
/*   code byte 32g + l (g = 0..3, l = 0..31): low nibble = element 64g + l, */
/*   high nibble = element 64g + 32 + l.                                     */
/* READING, quantizer (none is given; the plainest min-max form that keeps  */
/* every element within half a step of its code): per sub-block, lo and hi  */
/* its smallest and largest element;                                         */
/*   mn_j = max(0, -lo_j); dmin = f16(max_j mn_j / 63) (0 if that is 0);    */
/*   m_j = min(63, ceil(mn_j / dmin)); mf_j = m_j * dmin;                    */
/*   s_j = max(0, (hi_j + mf_j) / 15); d = f16(max_j s_j / 63);             */
/*   sc_j = min(63, ceil(s_j / d)); step_j = d * sc_j;                       */
/*   q = min(15, round-half-away((x + mf_j) * (1 / step_j)))  (0 if step 0). */
/* All in fp32 with d and dmin taken as their f16 values.                   */
/* ======================================================================== */

void orc_q4_k_scales(const uint8_t *ib, int32_t *sc, int32_t *m)
{
    const uint8_t *s = ib + 4;
    for (int j = 0; j < 8; j++) {
        if (j < 4) {
            sc[j] = s[j] & 63;
            m[j] = s[j + 4] & 63;
        } else {
            sc[j] = (s[j + 4] & 15) | ((s[j - 4] >> 6) << 4);
            m[j] = (s[j + 4] >> 4) | ((s[j] >> 6) << 4);
        }
    }
}

int64_t orc_q4_k_quantize(const float *x, int64_t n, uint8_t *out)
{
    if (n < 0 || n % 256) return -1;
    for (int64_t b = 0; b < n / 256; b++) {
        const float *xb = x + b * 256;
        uint8_t *ob = out + b * 144;
        float lo[8], hi[8], mn[8], sv[8], mf[8], step[8];
        int32_t sc[8], m[8];
        for (int j = 0; j < 8; j++) {
            lo[j] = hi[j] = xb[32 * j];
            for (int i = 1; i < 32; i++) {
                const float v = xb[32 * j + i];
                if (v < lo[j]) lo[j] = v;
                if (v > hi[j]) hi[j] = v;
            }
            mn[j] = lo[j] < 0.0f ? -lo[j] : 0.0f;
        }
        float mmax = 0.0f;
        for (int j = 0; j < 8; j++) if (mn[j] > mmax) mmax = mn[j];
        const uint16_t dminh = orc_f16_from_f32(mmax / 63.0f);
        const float dmin = orc_f16_to_f32(dminh);
        for (int j = 0; j < 8; j++) {
            int mj = 0;
            if (dmin > 0.0f) {
                const float r = ceilf(mn[j] / dmin);
                mj = r > 63.0f ? 63 : (int)r;
            }
            m[j] = mj;
            mf[j] = (float)mj * dmin;
            const float t = (hi[j] + mf[j]) / 15.0f;
            sv[j] = t > 0.0f ? t : 0.0f;
        }
        float smax = 0.0f;
        for (int j = 0; j < 8; j++) if (sv[j] > smax) smax = sv[j];
        const uint16_t dh = orc_f16_from_f32(smax / 63.0f);
        const float d = orc_f16_to_f32(dh);
        for (int j = 0; j < 8; j++) {
            int sj = 0;
            if (d > 0.0f) {
                const float r = ceilf(sv[j] / d);
                sj = r > 63.0f ? 63 : (int)r;
            }
            sc[j] = sj;
            step[j] = d * (float)sj;
        }
        wr_u16(ob, dh);
        wr_u16(ob + 2, dminh);
        uint8_t *s = ob + 4;
        for (int j = 0; j < 4; j++) {
            s[j] = (uint8_t)(sc[j] | ((sc[j + 4] >> 4) << 6));
            s[j + 4] = (uint8_t)(m[j] | ((m[j + 4] >> 4) << 6));
            s[j + 8] = (uint8_t)((sc[j + 4] & 15) | ((m[j + 4] & 15) << 4));
        }
        int code[256];
        for (int j = 0; j < 8; j++) {
            const float inv = step[j] > 0.0f ? 1.0f / step[j] : 0.0f;
            for (int i = 0; i < 32; i++) {
                const float t = (xb[32 * j + i] + mf[j]) * inv;
                int c = (int)roundf(t);      /* half away from zero */
                if (c > 15) c = 15;
                if (c < 0) c = 0;
                code[32 * j + i] = c;
            }
        }
        for (int g = 0; g < 4; g++)
            for (int l = 0; l < 32; l++)
                ob[16 + 32 * g + l] = (uint8_t)(code[64 * g + l] | (code[64 * g + 32 + l] << 4));
    }
    return n / 256 * 144;
}

void orc_q4_k_dequantize(const uint8_t *blocks, int64_t n, float *y)
{
    for (int64_t b = 0; b < n / 256; b++) {
        const uint8_t *ib = blocks + b * 144;
        const float d = orc_f16_to_f32(rd_u16(ib)), dmin = orc_f16_to_f32(rd_u16(ib + 2));
        int32_t sc[8], m[8];
        orc_q4_k_scales(ib, sc, m);
        for (int g = 0; g < 4; g++)
            for (int l = 0; l < 32; l++) {
                const uint8_t byte = ib[16 + 32 * g + l];
                const int e0 = 64 * g + l, e1 = 64 * g + 32 + l;
                y[b * 256 + e0] = d * (float)sc[e0 / 32] * (float)(byte & 15) - dmin * (float)m[e0 / 32];
                y[b * 256 + e1] = d * (float)sc[e1 / 32] * (float)(byte >> 4) - dmin * (float)m[e1 / 32];
            }
    }
}

/* ======================================================================== */
/* Primitives                                                               */
/* ======================================================================== */

/* Input / FFN / final normalization (step 13b names "normalization";       */
/* step 6 declares attn_norm, ffn_norm, output_norm as one vector each).    */
/* READING: RMSNorm, y_j = x_j * (1/sqrt(mean(x^2) + eps)) * g_j.           */
void orc_rmsnorm(const orc_real *x, const float *g, int32_t n, float eps, orc_real *y)
{
    orc_real ss = 0;
    for (int32_t j = 0; j < n; j++) ss += x[j] * x[j];
    const orc_real r = (orc_real)1 / (orc_real)sqrt((double)(ss / (orc_real)n + (orc_real)eps));
    for (int32_t j = 0; j < n; j++) y[j] = (x[j] * r) * (orc_real)g[j];
}

/* One row of deq(W), converted from its stored form. */
static void deq_row(int32_t wtype, const void *w, int64_t row, int32_t cols, float *dst)
{
    if (wtype == ORC_T_F32) {
        memcpy(dst, (const float *)w + row * cols, sizeof(float) * (size_t)cols);
    } else if (wtype == ORC_T_Q8_0) {
        orc_q8_0_dequantize((const uint8_t *)w + row * (cols / 32) * 34, cols, dst);
    } else if (wtype == ORC_T_Q4_K) {
        orc_q4_k_dequantize((const uint8_t *)w + row * (cols / 256) * 144, cols, dst);
    } else {
        orc_q4_0_dequantize((const uint8_t *)w + row * (cols / 32) * 18, cols, dst);
    }
}

/* Linear layers of step 13b (Q = input x W_q, ... , output matrix).        */
/* y_r = sum over k in order 0..cols-1 of deq(W)[r][k] * x_k.               */
void orc_matvec(int32_t wtype, const void *w, int32_t rows, int32_t cols,
                const orc_real *x, orc_real *y)
{
#pragma omp parallel
    {
        float *wr = (float *)malloc(sizeof(float) * (size_t)cols);
#pragma omp for schedule(static)
        for (int32_t r = 0; r < rows; r++) {
            deq_row(wtype, w, r, cols, wr);
            orc_real acc = 0;
            for (int32_t k = 0; k < cols; k++) acc += (orc_real)wr[k] * x[k];
            y[r] = acc;
        }
        free(wr);
    }
}

/* RoPE on Q and K (step 13b; positions are a separate input, not added to  */
/* the embeddings).  The rotation base is rope.freq_base (step 4, default   */
/* 10000).  READING: adjacent pairs (2i, 2i+1) rotated by                   */
/* theta = pos * base^(-2i/hd), the angle evaluated in double.              */
void orc_rope(orc_real *v, int32_t n_heads, int32_t hd, int32_t pos, float base)
{
    for (int32_t i = 0; i < hd / 2; i++) {
        const double theta = (double)pos * pow((double)base, -2.0 * (double)i / (double)hd);
        const orc_real c = (orc_real)cos(theta), s = (orc_real)sin(theta);
        for (int32_t h = 0; h < n_heads; h++) {
            orc_real *p = v + (int64_t)h * hd + 2 * i;
            const orc_real a = p[0], b = p[1];
            p[0] = a * c - b * s;
            p[1] = a * s + b * c;
        }
    }
}

/* Element idx of a cached array.  Q8_0 cache: 34-byte blocks of 32         */
/* consecutive row elements (scale, then codes), value = code * scale.      */
static orc_real kv_at(const void *base, int32_t kvtype, int64_t idx)
{
    if (kvtype == ORC_T_F16) return (orc_real)orc_f16_to_f32(((const uint16_t *)base)[idx]);
    if (kvtype == ORC_T_Q8_0) {
        const uint8_t *b = (const uint8_t *)base + (idx / 32) * 34;
        const orc_real d = (orc_real)orc_f16_to_f32(rd_u16(b));
        return (orc_real)(int8_t)b[2 + idx % 32] * d;
    }
    return (orc_real)((const float *)base)[idx];
}

/* Byte offset of element idx (a multiple of 32 for a Q8_0 cache). */
static size_t kv_bytes(int32_t kvtype, int64_t idx)
{
    if (kvtype == ORC_T_Q8_0) return (size_t)(idx / 32) * 34;
    return (size_t)idx * (kvtype == ORC_T_F16 ? 2 : 4);
}

/* Attention of step 13b: scores = Q x K^T, causal mask, softmax, weighted  */
/* sum with V.  READING: scores scaled by 1/sqrt(head_dim).                 */
void orc_attend(const orc_real *q, const void *K, const void *V, int32_t kvtype,
                int64_t ld, const int32_t *row_pos, int32_t n, int32_t hd,
                int32_t pos, orc_real *o, orc_real *w)
{
    orc_real *s = (orc_real *)malloc(sizeof(orc_real) * (size_t)(n > 0 ? n : 1));
    char *keep = (char *)malloc((size_t)(n > 0 ? n : 1));
    const orc_real scale = (orc_real)1 / (orc_real)sqrt((double)hd);
    orc_real m = 0;
    int any = 0;
    for (int32_t j = 0; j < n; j++) {
        const int32_t pj = row_pos ? row_pos[j] : j;
        keep[j] = (char)(pj <= pos);
        if (!keep[j]) { s[j] = 0; continue; }
        orc_real dot = 0;
        for (int32_t d = 0; d < hd; d++) dot += q[d] * kv_at(K, kvtype, (int64_t)j * ld + d);
        s[j] = dot * scale;
        if (!any || s[j] > m) m = s[j];
        any = 1;
    }
    orc_real sum = 0;
    for (int32_t j = 0; j < n; j++) {
        if (!keep[j]) continue;
        s[j] = (orc_real)exp((double)(s[j] - m));
        sum += s[j];
    }
    for (int32_t j = 0; j < n; j++) s[j] = keep[j] ? s[j] / sum : 0;
    for (int32_t d = 0; d < hd; d++) {
        orc_real acc = 0;
        for (int32_t j = 0; j < n; j++)
            if (keep[j]) acc += s[j] * kv_at(V, kvtype, (int64_t)j * ld + d);
        o[d] = acc;
    }
    if (w)
        for (int32_t j = 0; j < n; j++) w[j] = s[j];
    free(s);
    free(keep);
}

/* Feed-forward activation "between the two linear layers" (step 13b), with */
/* the gate / up / down matrices of step 6.  READING: SwiGLU,              */
/* h = silu(gate) * up, silu(u) = u / (1 + exp(-u)).                        */
void orc_swiglu(const orc_real *u, const orc_real *v, int32_t n, orc_real *h)
{
    for (int32_t j = 0; j < n; j++) {
        const orc_real g = u[j] / ((orc_real)1 + (orc_real)exp(-(double)u[j]));
        h[j] = g * v[j];
    }
}

/* Greedy choice of step 15: the token with the largest logit.            */
/* READING: ties go to the lowest token id.                               */
int32_t orc_argmax(const orc_real *x, int32_t n)
{
    int32_t best = 0;
    for (int32_t i = 1; i < n; i++)
        if (x[i] > x[best]) best = i;
    return n > 0 ? best : -1;
}

/* ======================================================================== */
/* Decoder                                                                  */
/* ======================================================================== */

enum { T_TOK = 0, T_OUT = 1, T_WQ, T_WK, T_WV, T_WO, T_GATE, T_UP, T_DOWN, T_COUNT };

struct orc_model {
    orc_hparams hp;
    void *tok_embd, *output;      /* encoded */
    float *output_norm;
    float **attn_norm, **ffn_norm;
    void **mat[T_COUNT];          /* per-layer encoded matrices, T_WQ..T_DOWN */
    int64_t rows[T_COUNT], cols[T_COUNT];
};

struct orc_ctx {
    const orc_model *m;
    int32_t n_seq, n_ctx;
    int32_t *pos_max;
    void **K, **V;                /* [layer*n_seq + seq] -> [n_ctx][Hkv*hd] */
};

static int64_t enc_bytes(int32_t wtype, int64_t rows, int64_t cols)
{
    if (wtype == ORC_T_F32) return rows * cols * 4;
    if (wtype == ORC_T_Q8_0) return rows * (cols / 32) * 34;
    if (wtype == ORC_T_Q4_K) return rows * (cols / 256) * 144;
    return rows * (cols / 32) * 18;
}

static void *encode(int32_t wtype, const float *src, int64_t rows, int64_t cols)
{
    const int64_t nb = enc_bytes(wtype, rows, cols);
    uint8_t *dst = (uint8_t *)malloc((size_t)nb);
    if (!dst) return NULL;
    if (wtype == ORC_T_F32) {
        memcpy(dst, src, (size_t)nb);
        return dst;
    }
    const int64_t rb = enc_bytes(wtype, 1, cols);
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; r++) {
        if (wtype == ORC_T_Q8_0)
            orc_q8_0_quantize(src + r * cols, cols, dst + r * rb);
        else if (wtype == ORC_T_Q4_K)
            orc_q4_k_quantize(src + r * cols, cols, dst + r * rb);
        else
            orc_q4_0_quantize(src + r * cols, cols, dst + r * rb);
    }
    return dst;
}

static float *copy_vec(const float *src, int64_t n)
{
    float *d = (float *)malloc(sizeof(float) * (size_t)n);
    if (d) memcpy(d, src, sizeof(float) * (size_t)n);
    return d;
}

orc_model *orc_model_new(const orc_hparams *hp, const orc_weights *w)
{
    if (!hp || !w) return NULL;
    const orc_hparams h = *hp;
    if (h.n_layer <= 0 || h.n_embd <= 0 || h.n_head <= 0 || h.n_head_kv <= 0 || h.head_dim <= 0 ||
        h.n_ff <= 0 || h.n_vocab <= 0 || h.head_dim % 2 || h.n_head % h.n_head_kv)
        return NULL;
    if (h.wtype != ORC_T_F32 && h.wtype != ORC_T_Q8_0 && h.wtype != ORC_T_Q4_0 && h.wtype != ORC_T_Q4_K) return NULL;
    if (h.kvtype != ORC_T_F32 && h.kvtype != ORC_T_F16 && h.kvtype != ORC_T_Q8_0) return NULL;
    /* a Q8_0 cache row splits into whole 32-element blocks within each head */
    if (h.kvtype == ORC_T_Q8_0 && h.head_dim % 32) return NULL;
    const int32_t qd = h.n_head * h.head_dim, kd = h.n_head_kv * h.head_dim;
    if (h.wtype != ORC_T_F32 && (h.n_embd % 32 || qd % 32 || h.n_ff % 32)) return NULL;
    /* Q4_K rows are whole 256-element super-blocks */
    if (h.wtype == ORC_T_Q4_K && (h.n_embd % 256 || qd % 256 || h.n_ff % 256)) return NULL;

    orc_model *m = (orc_model *)calloc(1, sizeof *m);
    m->hp = h;
    m->rows[T_TOK] = h.n_vocab; m->cols[T_TOK] = h.n_embd;
    m->rows[T_OUT] = h.n_vocab; m->cols[T_OUT] = h.n_embd;
    m->rows[T_WQ] = qd;         m->cols[T_WQ] = h.n_embd;
    m->rows[T_WK] = kd;         m->cols[T_WK] = h.n_embd;
    m->rows[T_WV] = kd;         m->cols[T_WV] = h.n_embd;
    m->rows[T_WO] = h.n_embd;   m->cols[T_WO] = qd;
    m->rows[T_GATE] = h.n_ff;   m->cols[T_GATE] = h.n_embd;
    m->rows[T_UP] = h.n_ff;     m->cols[T_UP] = h.n_embd;
    m->rows[T_DOWN] = h.n_embd; m->cols[T_DOWN] = h.n_ff;

    m->tok_embd = encode(h.wtype, w->tok_embd, h.n_vocab, h.n_embd);
    m->output = encode(h.wtype, w->output, h.n_vocab, h.n_embd);
    m->output_norm = copy_vec(w->output_norm, h.n_embd);
    m->attn_norm = (float **)calloc((size_t)h.n_layer, sizeof(float *));
    m->ffn_norm = (float **)calloc((size_t)h.n_layer, sizeof(float *));
    const float *const *src[T_COUNT] = {0, 0, w->wq, w->wk, w->wv, w->wo, w->ffn_gate, w->ffn_up, w->ffn_down};
    for (int t = T_WQ; t < T_COUNT; t++) m->mat[t] = (void **)calloc((size_t)h.n_layer, sizeof(void *));
    for (int32_t l = 0; l < h.n_layer; l++) {
        m->attn_norm[l] = copy_vec(w->attn_norm[l], h.n_embd);
        m->ffn_norm[l] = copy_vec(w->ffn_norm[l], h.n_embd);
        for (int t = T_WQ; t < T_COUNT; t++)
            m->mat[t][l] = encode(h.wtype, src[t][l], m->rows[t], m->cols[t]);
    }
    return m;
}

void orc_model_free(orc_model *m)
{
    if (!m) return;
    for (int32_t l = 0; l < m->hp.n_layer; l++) {
        free(m->attn_norm[l]);
        free(m->ffn_norm[l]);
        for (int t = T_WQ; t < T_COUNT; t++) free(m->mat[t][l]);
    }
    for (int t = T_WQ; t < T_COUNT; t++) free(m->mat[t]);
    free(m->attn_norm);
    free(m->ffn_norm);
    free(m->tok_embd);
    free(m->output);
    free(m->output_norm);
    free(m);
}

int64_t orc_model_tensor_bytes(const orc_model *m, int32_t tensor, int32_t layer, void *dst, int64_t cap)
{
    if (!m || tensor < 0 || tensor >= T_COUNT) return 0;
    const void *src;
    if (tensor == T_TOK) src = m->tok_embd;
    else if (tensor == T_OUT) src = m->output;
    else {
        if (layer < 0 || layer >= m->hp.n_layer) return 0;
        src = m->mat[tensor][layer];
    }
    const int64_t nb = enc_bytes(m->hp.wtype, m->rows[tensor], m->cols[tensor]);
    if (!dst || cap < nb) return -nb;
    memcpy(dst, src, (size_t)nb);
    return nb;
}

orc_ctx *orc_ctx_new(const orc_model *m, int32_t n_seq, int32_t n_ctx)
{
    if (!m || n_seq <= 0 || n_ctx <= 0) return NULL;
    orc_ctx *c = (orc_ctx *)calloc(1, sizeof *c);
    c->m = m;
    c->n_seq = n_seq;
    c->n_ctx = n_ctx;
    c->pos_max = (int32_t *)malloc(sizeof(int32_t) * (size_t)n_seq);
    for (int32_t s = 0; s < n_seq; s++) c->pos_max[s] = -1;
    const size_t n = (size_t)m->hp.n_layer * (size_t)n_seq;
    const size_t bytes = kv_bytes(m->hp.kvtype, (int64_t)n_ctx * m->hp.n_head_kv * m->hp.head_dim);
    c->K = (void **)calloc(n, sizeof(void *));
    c->V = (void **)calloc(n, sizeof(void *));
    for (size_t i = 0; i < n; i++) {
        c->K[i] = calloc(1, bytes);
        c->V[i] = calloc(1, bytes);
        if (!c->K[i] || !c->V[i]) { orc_ctx_free(c); return NULL; }
    }
    return c;
}

void orc_ctx_free(orc_ctx *c)
{
    if (!c) return;
    const size_t n = (size_t)c->m->hp.n_layer * (size_t)c->n_seq;
    for (size_t i = 0; i < n; i++) { free(c->K[i]); free(c->V[i]); }
    free(c->K);
    free(c->V);
    free(c->pos_max);
    free(c);
}

int32_t orc_seq_pos_max(const orc_ctx *c, int32_t seq)
{
    if (!c || seq < 0 || seq >= c->n_seq) return -1;
    return c->pos_max[seq];
}

void orc_seq_clear(orc_ctx *c, int32_t seq)
{
    if (c && seq >= 0 && seq < c->n_seq) c->pos_max[seq] = -1;
}

/* Store one cached row (KV appendix: one row per position holds the keys   */
/* or values of every KV head of the layer).  F16 cache: one RNE rounding.  */
/* Q8_0 cache (the -ctk / -ctv cache types of the KV-cache appendix):       */
/* READING: the row is rounded to fp32, the codec's input type, and coded   */
/* with the weights' Q8_0 codec in blocks of 32 consecutive row elements.   */
static void kv_store(void *base, int32_t kvtype, int64_t off, const orc_real *v, int32_t n)
{
    if (kvtype == ORC_T_Q8_0) {
        float *t = (float *)malloc(sizeof(float) * (size_t)n);
        for (int32_t i = 0; i < n; i++) t[i] = (float)v[i];
        orc_q8_0_quantize(t, n, (uint8_t *)base + kv_bytes(kvtype, off));
        free(t);
    } else if (kvtype == ORC_T_F16) {
        uint16_t *d = (uint16_t *)base + off;
        for (int32_t i = 0; i < n; i++) d[i] = orc_f16_from_f64((double)v[i]);
    } else {
        float *d = (float *)base + off;
        for (int32_t i = 0; i < n; i++) d[i] = (float)v[i];
    }
}

int32_t orc_eval_tap(orc_ctx *c, int32_t seq, int32_t token, orc_real *logits, int32_t tap, orc_real *x_tap)
{
    if (!c || seq < 0 || seq >= c->n_seq) return -1;
    const orc_model *m = c->m;
    const orc_hparams h = m->hp;
    if (token < 0 || token >= h.n_vocab) return -1;
    const int32_t p = c->pos_max[seq] + 1;
    if (p >= c->n_ctx) return 1;

    const int32_t d = h.n_embd, hd = h.head_dim, H = h.n_head, Hkv = h.n_head_kv;
    const int32_t qd = H * hd, kd = Hkv * hd, F = h.n_ff;
    const int32_t group = H / Hkv;
    orc_real *x = (orc_real *)malloc(sizeof(orc_real) * (size_t)d);
    orc_real *xn = (orc_real *)malloc(sizeof(orc_real) * (size_t)d);
    orc_real *q = (orc_real *)malloc(sizeof(orc_real) * (size_t)qd);
    orc_real *k = (orc_real *)malloc(sizeof(orc_real) * (size_t)kd);
    orc_real *v = (orc_real *)malloc(sizeof(orc_real) * (size_t)kd);
    orc_real *o = (orc_real *)malloc(sizeof(orc_real) * (size_t)qd);
    orc_real *y = (orc_real *)malloc(sizeof(orc_real) * (size_t)d);
    orc_real *u = (orc_real *)malloc(sizeof(orc_real) * (size_t)F);
    orc_real *g = (orc_real *)malloc(sizeof(orc_real) * (size_t)F);
    orc_real *hh = (orc_real *)malloc(sizeof(orc_real) * (size_t)F);
    float *row = (float *)malloc(sizeof(float) * (size_t)d);

    /* Token -> embedding: one row of tok_embd, dequantized to float
       ("from tokens to embeddings", ggml_get_rows). */
    deq_row(h.wtype, m->tok_embd, token, d, row);
    for (int32_t j = 0; j < d; j++) x[j] = (orc_real)row[j];

    for (int32_t l = 0; l < h.n_layer; l++) {
        if (x_tap && tap == l) memcpy(x_tap, x, sizeof(orc_real) * (size_t)d);
        orc_rmsnorm(x, m->attn_norm[l], d, h.rms_eps, xn);
        orc_matvec(h.wtype, m->mat[T_WQ][l], qd, d, xn, q);
        orc_matvec(h.wtype, m->mat[T_WK][l], kd, d, xn, k);
        orc_matvec(h.wtype, m->mat[T_WV][l], kd, d, xn, v);
        orc_rope(q, H, hd, p, h.rope_base);
        orc_rope(k, Hkv, hd, p, h.rope_base);

        /* append first, then attend over every cached row, own row included */
        void *Kc = c->K[(size_t)l * c->n_seq + seq], *Vc = c->V[(size_t)l * c->n_seq + seq];
        kv_store(Kc, h.kvtype, (int64_t)p * kd, k, kd);
        kv_store(Vc, h.kvtype, (int64_t)p * kd, v, kd);

        /* READING: consecutive query heads share one KV head (GQA), kv = h / (H/Hkv) */
#pragma omp parallel for schedule(static)
        for (int32_t hq = 0; hq < H; hq++) {
            const int32_t kvh = hq / group;
            const uint8_t *kb = (const uint8_t *)Kc + kv_bytes(h.kvtype, (int64_t)kvh * hd);
            const uint8_t *vb = (const uint8_t *)Vc + kv_bytes(h.kvtype, (int64_t)kvh * hd);
            orc_attend(q + (int64_t)hq * hd, kb, vb, h.kvtype, kd, NULL, p + 1, hd, p,
                       o + (int64_t)hq * hd, NULL);
        }
        orc_matvec(h.wtype, m->mat[T_WO][l], d, qd, o, y);
        for (int32_t j = 0; j < d; j++) x[j] = x[j] + y[j];

        orc_rmsnorm(x, m->ffn_norm[l], d, h.rms_eps, xn);
        orc_matvec(h.wtype, m->mat[T_GATE][l], F, d, xn, u);
        orc_matvec(h.wtype, m->mat[T_UP][l], F, d, xn, g);
        orc_swiglu(u, g, F, hh);
        orc_matvec(h.wtype, m->mat[T_DOWN][l], d, F, hh, y);
        for (int32_t j = 0; j < d; j++) x[j] = x[j] + y[j];
    }
    if (x_tap && tap == h.n_layer) memcpy(x_tap, x, sizeof(orc_real) * (size_t)d);

    if (logits) {
        orc_rmsnorm(x, m->output_norm, d, h.rms_eps, xn);
        orc_matvec(h.wtype, m->output, h.n_vocab, d, xn, logits);
    }
    c->pos_max[seq] = p;

    free(x); free(xn); free(q); free(k); free(v); free(o); free(y);
    free(u); free(g); free(hh); free(row);
    return 0;
}

int32_t orc_eval(orc_ctx *c, int32_t seq, int32_t token, orc_real *logits)
{
    return orc_eval_tap(c, seq, token, logits, -1, NULL);
}

int32_t orc_kv_row(const orc_ctx *c, int32_t which, int32_t layer, int32_t seq, int32_t pos,
                   int32_t kv_head, float *out)
{
    if (!c || layer < 0 || layer >= c->m->hp.n_layer || seq < 0 || seq >= c->n_seq || pos < 0 ||
        pos > c->pos_max[seq] || kv_head < 0 || kv_head >= c->m->hp.n_head_kv)
        return -1;
    const int32_t hd = c->m->hp.head_dim, kd = c->m->hp.n_head_kv * hd;
    const void *base = (which == 0 ? c->K : c->V)[(size_t)layer * c->n_seq + seq];
    for (int32_t i = 0; i < hd; i++)
        out[i] = (float)kv_at(base, c->m->hp.kvtype, (int64_t)pos * kd + (int64_t)kv_head * hd + i);
    return 0;
}

/* ======================================================================== */
/* Sampler chain (article, step 15: the sampler list and its order)         */
/* ======================================================================== */

/* SplitMix64 (Steele, Lea, Flood: "Fast splittable pseudorandom number
   generators", 2014): state advances by the golden-ratio increment, the
   output is the state passed through two xor-shift-multiply rounds. */
uint64_t orc_splitmix64(uint64_t seed, uint64_t index)
{
    uint64_t z = seed + (index + 1) * 0x9E3779B97F4A7C15ull;
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
}

float orc_uniform24(uint64_t seed, uint64_t index)
{
    return (float)(orc_splitmix64(seed, index) >> 40) * (1.0f / 16777216.0f);
}

typedef struct { float l; int32_t id; } orc_cand;

/* chain order: larger logit first, the lower token id first on equal logits */
static int cand_cmp(const void *a, const void *b)
{
    const orc_cand *x = (const orc_cand *)a, *y = (const orc_cand *)b;
    if (x->l > y->l) return -1;
    if (x->l < y->l) return 1;
    return (x->id > y->id) - (x->id < y->id);
}

int32_t orc_sample(const float *logits, int32_t n_vocab, const int32_t *hist, int32_t n_hist,
                   const orc_sampler_params *p, uint64_t draw, int32_t *ids, float *cum,
                   int32_t *n_kept, float *target)
{
    if (!logits || !p || n_vocab <= 0 || n_hist < 0 || (n_hist > 0 && !hist)) return -1;
    orc_cand *c = (orc_cand *)malloc(sizeof(orc_cand) * (size_t)n_vocab);
    if (!c) return -1;
    for (int32_t i = 0; i < n_vocab; i++) { c[i].l = logits[i]; c[i].id = i; }

    /* repeat penalty: once per distinct token of the last penalty_last_n;
       positive logits are divided by the penalty, negative ones multiplied */
    if (p->repeat_penalty != 1.0f && p->penalty_last_n > 0) {
        const int32_t w = n_hist < p->penalty_last_n ? n_hist : p->penalty_last_n;
        for (int32_t j = n_hist - w; j < n_hist; j++) {
            const int32_t t = hist[j];
            if (t < 0 || t >= n_vocab) continue;
            int seen = 0;
            for (int32_t k = n_hist - w; k < j; k++) seen |= hist[k] == t;
            if (seen) continue;
            c[t].l = c[t].l > 0.0f ? c[t].l / p->repeat_penalty : c[t].l * p->repeat_penalty;
        }
    }
    qsort(c, (size_t)n_vocab, sizeof(orc_cand), cand_cmp);

    /* top-k */
    int32_t n = (p->top_k > 0 && p->top_k < n_vocab) ? p->top_k : n_vocab;
    const float m = c[0].l;   /* the leader stays first through every cut */

    /* top-p: the shortest prefix whose weight reaches p of the total */
    if (p->top_p < 1.0f) {
        float s = 0.0f;
        for (int32_t i = 0; i < n; i++) s += expf(c[i].l - m);
        const float lim = p->top_p * s;
        float a = 0.0f;
        int32_t keep = n;
        for (int32_t i = 0; i < n; i++) {
            a += expf(c[i].l - m);
            if (a >= lim) { keep = i + 1; break; }
        }
        n = keep;
    }
    /* min-p: weight relative to the leader */
    if (p->min_p > 0.0f) {
        int32_t keep = 1;
        for (int32_t i = 1; i < n; i++)
            if (expf(c[i].l - m) >= p->min_p) keep = i + 1;
        n = keep;
    }

    int32_t tok;
    if (p->temp <= 0.0f) {
        tok = c[0].id;
        if (n_kept) *n_kept = 0;
        if (target) *target = 0.0f;
    } else {
        /* temperature, then the draw: the first candidate whose inclusive
           cumulative weight exceeds u times the total */
        float s = 0.0f;
        for (int32_t i = 0; i < n; i++) {
            s += expf(c[i].l / p->temp - m / p->temp);
            if (cum) cum[i] = s;
            if (ids) ids[i] = c[i].id;
        }
        const float t = orc_uniform24(p->seed, draw) * s;
        float a = 0.0f;
        tok = c[n - 1].id;
        for (int32_t i = 0; i < n; i++) {
            a += expf(c[i].l / p->temp - m / p->temp);
            if (a > t) { tok = c[i].id; break; }
        }
        if (n_kept) *n_kept = n;
        if (target) *target = t;
    }
    free(c);
    return tok;
}

