// misc.hip -- small kernels of the decoder step and of weight loading (gfx950).
#include "common.h"
#include "q8.h"
#include "kernels.h"

namespace {

DEV int dst_row(int mode, int r, int row_off) {
    if (mode == 1) return ((r >> 5) << 6) + (r & 31);        // gate slot of a 64-row group
    if (mode == 2) return ((r >> 5) << 6) + 32 + (r & 31);   // up slot
    return r + row_off;
}

// ---- block quantization ----------------------------------------------------
// Q8_0: d = max|x| / 127; codes = round-half-away(x * (1/d)).
// Q4_0: m = element of largest magnitude (first on ties), d = m / -8;
//       codes = min(15, floor(x * (1/d) + 8.5)).
// fp32 arithmetic with no contraction, so codes match any IEEE fp32
// implementation of the same steps bit for bit; the scale is stored as f16
// (round to nearest even).
__global__ __launch_bounds__(256) void k_quantize(const float *src, int rows, int K, QMat m,
                                                  int mode, int row_off) {
#pragma clang fp contract(off)
    const int nb = K >> 5;
    const long long idx = (long long)blockIdx.x * 256 + threadIdx.x;
    if (idx >= (long long)rows * nb) return;
    const int r = (int)(idx / nb), b = (int)(idx % nb);
    const float *x = src + (size_t)r * K + b * 32;
    float v[32];
#pragma unroll
    for (int j = 0; j < 32; j += 4) {
        const float4 t = *(const float4 *)(x + j);
        v[j] = t.x; v[j + 1] = t.y; v[j + 2] = t.z; v[j + 3] = t.w;
    }
    const int dr = dst_row(mode, r, row_off);
    if (m.wtype == T_Q8_0) {
        uint32_t packed[8];
        m.d[(size_t)dr * nb + b] = q8_block(v, packed);
        uint4 *dst = (uint4 *)((int8_t *)m.qs + (size_t)dr * K + b * 32);
        dst[0] = make_uint4(packed[0], packed[1], packed[2], packed[3]);
        dst[1] = make_uint4(packed[4], packed[5], packed[6], packed[7]);
    } else {
        float amax = 0.f, mx = 0.f;
#pragma unroll
        for (int j = 0; j < 32; j++) {
            const float a = fabsf(v[j]);
            if (a > amax) { amax = a; mx = v[j]; }
        }
        float d = mx / -8.0f;
        asm volatile("" : "+v"(d));   // see above: an all-zero block has scale -0
        const float id = d != 0.f ? 1.0f / d : 0.f;
        m.d[(size_t)dr * nb + b] = f32_to_f16_bits(d);
        int code[32];
#pragma unroll
        for (int j = 0; j < 32; j++) {
            const float t = v[j] * id;
            const float s = t + 8.5f;
            int c = (int)floorf(s);
            c = c > 15 ? 15 : (c < 0 ? 0 : c);
            code[j] = c;
        }
        uint32_t packed[4];
#pragma unroll
        for (int i = 0; i < 4; i++) {
            uint32_t w = 0;
#pragma unroll
            for (int e = 0; e < 4; e++) {
                const int k = 4 * i + e;
                w |= (uint32_t)(code[k] | (code[k + 16] << 4)) << (8 * e);
            }
            packed[i] = w;
        }
        *(uint4 *)((uint8_t *)m.qs + (size_t)dr * (K >> 1) + b * 16) =
            make_uint4(packed[0], packed[1], packed[2], packed[3]);
    }
}

// Q4_K (super-blocks of 256 = 8 sub-blocks of 32; eight consecutive threads
// take one super-block, a sub-block each): per sub-block j with smallest and
// largest element lo_j, hi_j:
//   mn_j = max(0, -lo_j); dmin = f16(max_j mn_j / 63); m_j = min(63, ceil(mn_j / dmin));
//   s_j = max(0, (hi_j + m_j dmin) / 15); d = f16(max_j s_j / 63); sc_j = min(63, ceil(s_j / d));
//   q = min(15, round-half-away((x + m_j dmin) * (1 / (d sc_j))))   (0 when d sc_j = 0)
// in fp32 without contraction (d, dmin as their f16 values).  The maxima over
// the super-block are exact whatever the order, so the eight threads meet by
// lane exchange.
__global__ __launch_bounds__(256) void k_quantize_q4k(const float *src, int rows, int K, QMat m, int mode,
                                                      int row_off) {
#pragma clang fp contract(off)
    const int nb = K >> 5;
    const long long idx = (long long)blockIdx.x * 256 + threadIdx.x;
    // rows * nb is a multiple of 8 and each super-block's threads are 8
    // aligned lanes, so a super-block is wholly in range or wholly out
    if (idx >= (long long)rows * nb) return;
    const int r = (int)(idx / nb), b = (int)(idx % nb);
    const float *x = src + (size_t)r * K + b * 32;
    float v[32];
#pragma unroll
    for (int j = 0; j < 32; j += 4) {
        const float4 t = *(const float4 *)(x + j);
        v[j] = t.x; v[j + 1] = t.y; v[j + 2] = t.z; v[j + 3] = t.w;
    }
    float lo = v[0], hi = v[0];
#pragma unroll
    for (int j = 1; j < 32; j++) {
        if (v[j] < lo) lo = v[j];
        if (v[j] > hi) hi = v[j];
    }
    const float mn = lo < 0.f ? -lo : 0.f;
    float mmax = mn;
#pragma unroll
    for (int o = 1; o < 8; o <<= 1) mmax = fmaxf(mmax, __shfl_xor(mmax, o, 64));
    const uint16_t dminh = f32_to_f16_bits(mmax / 63.0f);
    const float dmin = f16_bits_to_f32(dminh);
    int mj = 0;
    if (dmin > 0.f) {
        const float c = ceilf(mn / dmin);
        mj = c > 63.f ? 63 : (int)c;
    }
    const float mf = (float)mj * dmin;
    const float t = (hi + mf) / 15.0f;
    const float sv = t > 0.f ? t : 0.f;
    float smax = sv;
#pragma unroll
    for (int o = 1; o < 8; o <<= 1) smax = fmaxf(smax, __shfl_xor(smax, o, 64));
    const uint16_t dh = f32_to_f16_bits(smax / 63.0f);
    const float d = f16_bits_to_f32(dh);
    int sj = 0;
    if (d > 0.f) {
        const float c = ceilf(sv / d);
        sj = c > 63.f ? 63 : (int)c;
    }
    const float step = d * (float)sj;
    const float inv = step > 0.f ? 1.0f / step : 0.f;
    int code[32];
#pragma unroll
    for (int j = 0; j < 32; j++) {
        const float u = (v[j] + mf) * inv;
        int c = (int)roundf(u);
        code[j] = c > 15 ? 15 : (c < 0 ? 0 : c);
    }
    uint32_t packed[4];
#pragma unroll
    for (int i = 0; i < 4; i++) {
        uint32_t w = 0;
#pragma unroll
        for (int e = 0; e < 4; e++) {
            const int k = 4 * i + e;
            w |= (uint32_t)(code[k] | (code[k + 16] << 4)) << (8 * e);
        }
        packed[i] = w;
    }
    const int dr = dst_row(mode, r, row_off);
    *(uint4 *)((uint8_t *)m.qs + (size_t)dr * (K >> 1) + b * 16) = make_uint4(packed[0], packed[1], packed[2], packed[3]);
    m.d[(size_t)dr * nb + b] = (uint16_t)(sj | (mj << 8));
    if ((b & 7) == 0) m.dm[(size_t)dr * (K >> 8) + (b >> 3)] = (uint32_t)dh | ((uint32_t)dminh << 16);
}

__global__ __launch_bounds__(256) void k_copy_f32(const float *src, int rows, int K_src, QMat m,
                                                  int mode, int row_off) {
    const long long idx = (long long)blockIdx.x * 256 + threadIdx.x;
    if (idx >= (long long)rows * K_src) return;
    const int r = (int)(idx / K_src), k = (int)(idx % K_src);
    ((float *)m.qs)[(size_t)dst_row(mode, r, row_off) * m.K + k] = src[idx];
}

// ---- Q8_0 KV cache: staged f32 rows -> coded cells -------------------------
// One thread per 32-element block of the T new K and V rows (the same coding
// as the Q8_0 weights); block b of row (t, which) covers kv head b / (hd/32).
__global__ __launch_bounds__(256) void k_kv_quant(KVLayer kv, TokInfo tok, int T) {
    const int nbr = kv.n_kv * kv.hd >> 5;
    const long long idx = (long long)blockIdx.x * 256 + threadIdx.x;
    if (idx >= (long long)T * 2 * nbr) return;
    const int b = (int)(idx % nbr), which = (int)((idx / nbr) & 1), t = (int)(idx / (2 * nbr));
    kv_code_block(kv, t, which, b, tok.seq[t], tok.pos[t]);
}

// ---- file blocks -> stored layout ------------------------------------------
// One thread per 32-weight block of a GGUF-style tensor (f16 scale, then 16
// bytes of Q4_0 nibbles or 32 Q8_0 codes): the scale goes to m.d and the
// codes to m.qs, in row dst_row(mode, r, row_off).  Blocks are 2-byte aligned
// (18 / 34 bytes each), so they are moved 16 bits at a time.
__global__ __launch_bounds__(256) void k_put_blocks(const uint16_t *src, int rows, int K, QMat m, int mode,
                                                    int row_off) {
    const int nb = K >> 5, nbd = m.K >> 5;              // source / stored blocks per row
    const long long idx = (long long)blockIdx.x * 256 + threadIdx.x;
    if (idx >= (long long)rows * nb) return;
    const int r = (int)(idx / nb), b = (int)(idx % nb);
    const int dr = dst_row(mode, r, row_off);
    const int cw = m.wtype == T_Q8_0 ? 16 : 8;          // 16-bit words of codes per block
    const uint16_t *blk = src + (size_t)idx * (1 + cw);
    m.d[(size_t)dr * nbd + b] = blk[0];
    uint16_t *q = (uint16_t *)m.qs + ((size_t)dr * nbd + b) * cw;
    for (int j = 0; j < cw; j++) q[j] = blk[1 + j];
}

// One thread per 144-byte Q4_K super-block of a file tensor (16-byte aligned:
// the staging buffer is, and 144 = 9 x 16): header -> m.d (sc | m << 8 per
// sub-block) and m.dm; codes -> the Q4_0 nibble layout per sub-block (file
// byte 32g + l holds weight l of sub-blocks 2g (low nibble) and 2g+1 (high)).
__global__ __launch_bounds__(256) void k_put_blocks_q4k(const uint4 *src, int rows, int K, QMat m, int mode,
                                                        int row_off) {
    const int ns = K >> 8;
    const long long idx = (long long)blockIdx.x * 256 + threadIdx.x;
    if (idx >= (long long)rows * ns) return;
    const int r = (int)(idx / ns), sb = (int)(idx % ns);
    const int dr = dst_row(mode, r, row_off);
    union { uint4 v[9]; uint8_t b[144]; } blk;
#pragma unroll
    for (int i = 0; i < 9; i++) blk.v[i] = src[(size_t)idx * 9 + i];
    const uint8_t *s = blk.b + 4;
    m.dm[(size_t)dr * ns + sb] = (uint32_t)blk.b[0] | ((uint32_t)blk.b[1] << 8) | ((uint32_t)blk.b[2] << 16) |
                                 ((uint32_t)blk.b[3] << 24);
#pragma unroll
    for (int j = 0; j < 8; j++) {
        const int sc = j < 4 ? (s[j] & 63) : ((s[j + 4] & 15) | ((s[j - 4] >> 6) << 4));
        const int mn = j < 4 ? (s[j + 4] & 63) : ((s[j + 4] >> 4) | ((s[j] >> 6) << 4));
        m.d[(size_t)dr * (K >> 5) + 8 * sb + j] = (uint16_t)(sc | (mn << 8));
    }
    const uint8_t *q = blk.b + 16;
    uint8_t *dst = (uint8_t *)m.qs + (size_t)dr * (K >> 1) + (size_t)sb * 128;
#pragma unroll
    for (int g = 0; g < 4; g++)
#pragma unroll
        for (int k = 0; k < 16; k++) {
            const uint8_t a = q[32 * g + k], c = q[32 * g + 16 + k];
            dst[32 * g + k] = (uint8_t)((a & 15) | ((c & 15) << 4));         // sub-block 2g
            dst[32 * g + 16 + k] = (uint8_t)((a >> 4) | (c & 0xF0));         // sub-block 2g+1
        }
}

// ---- embedding: x[t] = dequantized row tok[t] (the article's get_rows) -----
template <int WT>
__global__ __launch_bounds__(256) void k_embed(QMat E, const int32_t *tok, float *x, int ldx, float *ss_out) {
    __shared__ float red[4];
    const int t = blockIdx.x;
    float ss = 0.f;
    const int row = tok[t];
    const int K = E.K, nb = K >> 5;
    float *xr = x + (size_t)t * ldx;
    // element j of the row, dequantized
    auto elem = [&](int j) __attribute__((always_inline)) -> float {
        if constexpr (WT == T_F32) return ((const float *)E.qs)[(size_t)row * K + j];
        const int b = j >> 5, e = j & 31;
        if constexpr (WT == T_Q4_K) {
#pragma clang fp contract(off)
            const uint32_t dd = E.dm[(size_t)row * (K >> 8) + (b >> 3)];
            const uint16_t sm = E.d[(size_t)row * nb + b];
            const uint8_t byte = ((const uint8_t *)E.qs)[(size_t)row * (K >> 1) + b * 16 + (e & 15)];
            const int c = e < 16 ? (byte & 15) : (byte >> 4);
            return f16_bits_to_f32((uint16_t)dd) * (float)(sm & 63) * (float)c -
                   f16_bits_to_f32((uint16_t)(dd >> 16)) * (float)(sm >> 8);
        }
        const float d = f16_bits_to_f32(E.d[(size_t)row * nb + b]);
        if constexpr (WT == T_Q8_0) return (float)((const int8_t *)E.qs)[(size_t)row * K + j] * d;
        const uint8_t byte = ((const uint8_t *)E.qs)[(size_t)row * (K >> 1) + b * 16 + (e & 15)];
        const int c = e < 16 ? (byte & 15) : (byte >> 4);
        return (float)(c - 8) * d;
    };
    // a thread's elements are computed 16 at a time and stored after them: a
    // store between two loads of the table would make each load wait for it
    constexpr int U = 16;
    for (int j0 = threadIdx.x; j0 < K; j0 += 256 * U) {
        float v[U];
#pragma unroll
        for (int u = 0; u < U; u++) v[u] = elem(min(j0 + 256 * u, K - 1));   // (past K: re-read, not stored)
#pragma unroll
        for (int u = 0; u < U; u++)
            if (j0 + 256 * u < K) {
                xr[j0 + 256 * u] = v[u];
                ss += v[u] * v[u];
            }
    }
    // sum of squares of the row for the first RMSNorm: slot 0, other slots 0
    if (ss_out) {
        ss = block_sum256(ss, red);
        float *so = ss_out + (size_t)t * SS_SLOTS;
        for (int j = threadIdx.x; j < SS_SLOTS; j += 256) so[j] = j == 0 ? ss : 0.f;
    }
}

// ---- RMSNorm to f16: xn = f16(x * (1/sqrt(mean(x^2) + eps)) * g) ----------
__global__ __launch_bounds__(256) void k_rmsnorm(const float *x, int ldx, const float *g, int d,
                                                 float eps, const int32_t *row_idx, uint16_t *xn,
                                                 uint16_t *xl, int ldn) {
    __shared__ float red[4];
    const int t = blockIdx.x;
    const int row = row_idx ? row_idx[t] : t;
    const float *xr = x + (size_t)row * ldx;
    float ss = 0.f;
    for (int j = threadIdx.x; j < d; j += 256) ss += xr[j] * xr[j];
    ss = block_sum256(ss, red);
    const float r = 1.0f / sqrtf(ss / (float)d + eps);
    f16 *o = (f16 *)xn + (size_t)t * ldn;
    f16 *ol = (f16 *)xl + (size_t)t * ldn;
    for (int j = threadIdx.x; j < d; j += 256) {
        const float y = xr[j] * r * g[j];
        const f16 hi = (f16)y;
        o[j] = hi;
        ol[j] = (f16)(y - (float)hi);
    }
}

// ---- greedy: index of the largest logit, lowest index on ties --------------
DEV void amax_take(float &bv, int &bi, float v, int i) {
    if (v > bv || (v == bv && i < bi)) { bv = v; bi = i; }
}

__global__ __launch_bounds__(1024) void k_argmax(const float *logits, int V, int32_t *out) {
    __shared__ float sv[16];
    __shared__ int si[16];
    const int t = blockIdx.x, tid = threadIdx.x;
    const float *l = logits + (size_t)t * V;
    float bv = -INFINITY;
    int bi = 0x7fffffff;
    int j = 0;
    if (V % 4 == 0 && ((uintptr_t)l & 15) == 0) {
        // up to 32768 values: every 16-byte load of the thread in flight at once
        constexpr int R = 8;
        float4 v[R];
#pragma unroll
        for (int r = 0; r < R; r++) {
            const int e = 4 * (tid + 1024 * r);
            v[r] = e < V ? *(const float4 *)(l + e) : make_float4(-INFINITY, -INFINITY, -INFINITY, -INFINITY);
        }
#pragma unroll
        for (int r = 0; r < R; r++) {
            const int e = 4 * (tid + 1024 * r);
            if (e < V) {
                amax_take(bv, bi, v[r].x, e);
                amax_take(bv, bi, v[r].y, e + 1);
                amax_take(bv, bi, v[r].z, e + 2);
                amax_take(bv, bi, v[r].w, e + 3);
            }
        }
        j = 4 * 1024 * R;
    }
    for (j += tid; j + 3 * 1024 < V; j += 4 * 1024) {   // four independent loads in flight
        const float v0 = l[j], v1 = l[j + 1024], v2 = l[j + 2048], v3 = l[j + 3072];
        amax_take(bv, bi, v0, j);
        amax_take(bv, bi, v1, j + 1024);
        amax_take(bv, bi, v2, j + 2048);
        amax_take(bv, bi, v3, j + 3072);
    }
    for (; j < V; j += 1024) amax_take(bv, bi, l[j], j);
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
        const float ov = __shfl_xor(bv, o, 64);
        const int oi = __shfl_xor(bi, o, 64);
        amax_take(bv, bi, ov, oi);
    }
    const int w = tid >> 6;
    if ((tid & 63) == 0) { sv[w] = bv; si[w] = bi; }
    __syncthreads();
    if (tid == 0) {
        for (int k = 1; k < 16; k++) amax_take(bv, bi, sv[k], si[k]);
        if (bi == 0x7fffffff) bi = 0;
        out[t] = bi;
    }
}

// ---- RoPE angles: theta = p * base^(-2i/hd), evaluated in double ----------
__global__ __launch_bounds__(256) void k_rope_table(float *cs, int n_ctx, int hd, float base) {
    const long long idx = (long long)blockIdx.x * 256 + threadIdx.x;
    const int half = hd >> 1;
    if (idx >= (long long)n_ctx * half) return;
    const int p = (int)(idx / half), i = (int)(idx % half);
    const double th = (double)p * pow((double)base, -2.0 * (double)i / (double)hd);
    cs[2 * idx + 0] = (float)cos(th);
    cs[2 * idx + 1] = (float)sin(th);
}

}  // namespace

void launch_quantize(const float *src, int rows, int K, QMat &m, int mode, int row_off,
                     hipStream_t s) {
    const long long n = (long long)rows * (K / 32);
    if (m.wtype == T_Q4_K)
        launch(k_quantize_q4k, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, src, rows, K, m, mode, row_off);
    else
        launch(k_quantize, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, src, rows, K, m, mode, row_off);
}

void launch_copy_f32(const float *src, int rows, int K_src, QMat &m, int mode, int row_off,
                     hipStream_t s) {
    const long long n = (long long)rows * K_src;
    launch(k_copy_f32, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, src, rows, K_src,
                       m, mode, row_off);
}

void launch_put_blocks(const void *src, int rows, int K, QMat &m, int mode, int row_off, hipStream_t s) {
    if (m.wtype == T_Q4_K) {
        const long long n = (long long)rows * (K / 256);
        launch(k_put_blocks_q4k, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, (const uint4 *)src, rows, K, m,
               mode, row_off);
        return;
    }
    const long long n = (long long)rows * (K / 32);
    launch(k_put_blocks, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, (const uint16_t *)src, rows, K, m,
           mode, row_off);
}

void launch_kv_quant(const KVLayer &kv, TokInfo tok, int T, hipStream_t s) {
    const long long n = (long long)T * 2 * (kv.n_kv * kv.hd / 32);
    launch(k_kv_quant, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, kv, tok, T);
}

void launch_embed(const QMat &E, const int32_t *tok, int T, float *x, int ldx, float *ss_out, hipStream_t s) {
    switch (E.wtype) {
    case T_F32: launch(k_embed<T_F32>, dim3(T), dim3(256), 0, s, E, tok, x, ldx, ss_out); break;
    case T_Q8_0: launch(k_embed<T_Q8_0>, dim3(T), dim3(256), 0, s, E, tok, x, ldx, ss_out); break;
    case T_Q4_K: launch(k_embed<T_Q4_K>, dim3(T), dim3(256), 0, s, E, tok, x, ldx, ss_out); break;
    default: launch(k_embed<T_Q4_0>, dim3(T), dim3(256), 0, s, E, tok, x, ldx, ss_out); break;
    }
}

void launch_rmsnorm(const float *x, int ldx, const float *g, int d, float eps,
                    const int32_t *row_idx, int T, uint16_t *xn, uint16_t *xl, int ldn, hipStream_t s) {
    launch(k_rmsnorm, dim3(T), dim3(256), 0, s, x, ldx, g, d, eps, row_idx, xn, xl, ldn);
}

void launch_argmax(const float *logits, int V, int T, int32_t *out, hipStream_t s) {
    launch(k_argmax, dim3(T), dim3(1024), 0, s, logits, V, out);
}

void launch_rope_table(float *cs, int n_ctx, int hd, float base, hipStream_t s) {
    const long long n = (long long)n_ctx * (hd / 2);
    launch(k_rope_table, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, cs, n_ctx, hd,
                       base);
}
