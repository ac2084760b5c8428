// attn.hip -- causal GQA attention over the f16 / f32 / Q8_0 KV cache (gfx950).
//
// Each query token attends to the cached rows 0..pos of its own sequence
// (the token's own K,V row was appended by the QKV epilogue before this
// kernel runs, as the article's KV-cache appendix orders it).
//
// Split-K ("flash-decoding" within one GPU): the cached positions are cut
// into chunks of CH rows.  One 256-thread block handles (chunk, KV head,
// token) for all query heads of the group that share the KV head, so each
// K/V row is read from HBM once per token and group.  Every load a block
// needs (its slice of q, its K rows, its V elements) is issued at entry;
// then
//   1. scores s[h][j] = q_h . K_j / sqrt(hd): HD/8 threads per key row, each
//      holding 16 contiguous bytes of K, summed with DPP lane exchanges;
//   2. per head: m = max_j s, e_j = exp(s_j - m), l = sum_j e_j;
//   3. acc[h][d] = sum_j e_j V_j[d]: HD/2 threads per row, 2 elements each.
// The block writes (m, l, acc) for its chunk.  A second kernel merges the
// chunks of each (token, head),
//   M = max_c m_c, L = sum_c l_c e^(m_c - M), o = sum_c acc_c e^(m_c - M) / L,
// with the chunk statistics and the partial rows all requested at entry, and
// writes o in f16 (value + remainder) for the output projection.  The grid
// covers the context's largest chunk count; blocks past a token's last chunk
// exit at once, so one captured launch serves every decode step.
//
// f16 cache, head_dim 64 / 128: the chunk partials come from matrix cores
// instead (k_attn_mfma, 64-key chunks, same partial format).  Each
// wavefront takes 32 keys and loads everything at entry:
//   S^T[key][head] = K Q^T   v_mfma_f32_32x32x16_f16, K rows straight into
//                            the A operand, Q / sqrt(hd) as f16 value +
//                            remainder (written so by the QKV epilogue) as B,
//                            so every product is exact;
//   softmax per head column over the wavefront's keys;
//   O[head][dim] = P V       A = P (value + remainder) taken from the S^T
//                            accumulators as they lie; B = V read straight
//                            from the cache, each lane gathering the 16 keys
//                            its accumulators hold for one dim (2-byte loads
//                            that 32 lanes turn into one 64-byte row segment).
// The block's two wavefronts are then combined into one chunk partial.
#include "../../include/decode.h"
#include "common.h"
#include "kernels.h"
#include "q8.h"

namespace {

constexpr int CH = 64;      // cached rows per chunk
constexpr int GMAX = 8;     // query heads per KV head handled by one block

// Element reads of cached rows: row j (of HD elements) of a chunk whose
// first row is at `base`; `sc` is that row's block scales (Q8_0 only).
template <int KVT, int HD>
struct KVRow;
template <int HD>
struct KVRow<T_F16, HD> {
    typedef uint16_t E;
    // 8 consecutive elements e0..e0+7 as float
    DEV void load8(const uint16_t *base, const uint16_t *, int j, int e0, float *o) {
        const uint4 v = *(const uint4 *)(base + (size_t)j * HD + e0);
        const h2 a = as_h2(v.x), b = as_h2(v.y), c = as_h2(v.z), d = as_h2(v.w);
        o[0] = (float)a.x; o[1] = (float)a.y; o[2] = (float)b.x; o[3] = (float)b.y;
        o[4] = (float)c.x; o[5] = (float)c.y; o[6] = (float)d.x; o[7] = (float)d.y;
    }
    DEV float2 load2(const uint16_t *base, const uint16_t *, int j, int e0) {
        const h2 a = *(const h2 *)(base + (size_t)j * HD + e0);
        return make_float2((float)a.x, (float)a.y);
    }
};
template <int HD>
struct KVRow<T_F32, HD> {
    typedef float E;
    DEV void load8(const float *base, const uint16_t *, int j, int e0, float *o) {
        const float *p = base + (size_t)j * HD + e0;
        const float4 a = *(const float4 *)p, b = *(const float4 *)(p + 4);
        o[0] = a.x; o[1] = a.y; o[2] = a.z; o[3] = a.w;
        o[4] = b.x; o[5] = b.y; o[6] = b.z; o[7] = b.w;
    }
    DEV float2 load2(const float *base, const uint16_t *, int j, int e0) {
        return *(const float2 *)(base + (size_t)j * HD + e0);
    }
};
// Q8_0 cache: value = code * block scale, exact in fp32 (an int8 code times
// an f16 scale needs at most 19 significand bits).
template <int HD>
struct KVRow<T_Q8_0, HD> {
    typedef int8_t E;
    DEV void load8(const int8_t *base, const uint16_t *sc, int j, int e0, float *o) {
        const uint2 c = *(const uint2 *)(base + (size_t)j * HD + e0);
        const float d = f16_bits_to_f32(sc[(size_t)j * (HD / 32) + (e0 >> 5)]);
#pragma unroll
        for (int k = 0; k < 4; k++) {
            o[k] = (float)(int8_t)(c.x >> (8 * k)) * d;
            o[4 + k] = (float)(int8_t)(c.y >> (8 * k)) * d;
        }
    }
    DEV float2 load2(const int8_t *base, const uint16_t *sc, int j, int e0) {
        const uint16_t c = *(const uint16_t *)(base + (size_t)j * HD + e0);
        const float d = f16_bits_to_f32(sc[(size_t)j * (HD / 32) + (e0 >> 5)]);
        return make_float2((float)(int8_t)(c & 0xff) * d, (float)(int8_t)(c >> 8) * d);
    }
};

// Sum over groups of N consecutive lanes (N = 8, 16 or 32); every lane of a
// group gets the group's total.
template <int N>
DEV float group_sum(float v) {
    v += dpp_f<0xB1>(v);
    v += dpp_f<0x4E>(v);
    if (N == 8) {
        v += dpp_f<0x141>(v);   // row_half_mirror
    } else {
        v += dpp_f<0x124>(v);
        v += dpp_f<0x128>(v);
        if (N == 32) v += __shfl_xor(v, 16, 64);
    }
    return v;
}

template <int HD, int KVT, int G>
__global__ __launch_bounds__(256) void k_attn_part(AttnArgs a) {
    static_assert(CH == 64, "softmax statistics assume one cached row per lane");
    typedef KVRow<KVT, HD> R;
    typedef typename R::E E;
    constexpr int TPK = HD / 8;          // threads per key row (scores)
    constexpr int KPP = 256 / TPK;       // key rows per pass
    constexpr int NP = CH / KPP;         // passes
    constexpr int TPR = HD / 2;          // threads per value row
    constexpr int KG = 256 / TPR;        // value-row groups
    constexpr int VPT = CH / KG;         // value rows per thread

    __shared__ float sc[G][CH];
    __shared__ float red[KG][G][2][TPR];
    __shared__ float mls[G][2];

    const int c = blockIdx.x, g = blockIdx.y, t = blockIdx.z;
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int pos = a.tok.pos[t], seq = a.tok.seq[t];
    const int c0 = c * CH;
    if (c0 > pos) return;                          // uniform per block
    const int nk = min(CH, pos + 1 - c0);
    const int n_kv = a.kv.n_kv;
    const float scale = 1.0f / sqrtf((float)HD);

    const size_t cell0 = ((size_t)seq * n_kv + g) * a.kv.n_ctx + c0;
    const E *Kb = (const E *)a.kv.k + cell0 * HD;
    const E *Vb = (const E *)a.kv.v + cell0 * HD;
    const uint16_t *Ks = KVT == T_Q8_0 ? a.kv.k_scale + cell0 * (HD / 32) : nullptr;
    const uint16_t *Vs = KVT == T_Q8_0 ? a.kv.v_scale + cell0 * (HD / 32) : nullptr;
    const int part = tid % TPK, krow = tid / TPK;
    const int dp = tid % TPR, kg = tid / TPR;

    // ---- issue every load up front ----
    float kv8[NP][8];
#pragma unroll
    for (int ps = 0; ps < NP; ps++) {
        const int j = ps * KPP + krow;
        if (j < nk)
            R::load8(Kb, Ks, j, part * 8, kv8[ps]);
        else
#pragma unroll
            for (int e = 0; e < 8; e++) kv8[ps][e] = 0.f;
    }
    float2 vv[VPT];
#pragma unroll
    for (int i = 0; i < VPT; i++) {
        const int j = kg + KG * i;
        vv[i] = j < nk ? R::load2(Vb, Vs, j, 2 * dp) : make_float2(0.f, 0.f);
    }
    float qv[G][8];
    const float *qb = a.q + ((size_t)t * a.H + g * G) * HD + part * 8;
#pragma unroll
    for (int h = 0; h < G; h++) {
        const float4 lo = *(const float4 *)(qb + h * HD), hi = *(const float4 *)(qb + h * HD + 4);
        qv[h][0] = lo.x; qv[h][1] = lo.y; qv[h][2] = lo.z; qv[h][3] = lo.w;
        qv[h][4] = hi.x; qv[h][5] = hi.y; qv[h][6] = hi.z; qv[h][7] = hi.w;
    }

    // ---- 1. scores ----
#pragma unroll
    for (int ps = 0; ps < NP; ps++) {
        const int j = ps * KPP + krow;
#pragma unroll
        for (int h = 0; h < G; h++) {
            float s = 0.f;
#pragma unroll
            for (int e = 0; e < 8; e++) s += qv[h][e] * kv8[ps][e];
            s = group_sum<TPK>(s);
            if (part == 0 && j < nk) sc[h][j] = s * scale;
        }
    }
    __syncthreads();

    // ---- 2. softmax statistics of the chunk (CH = 64: one row per lane) ----
    for (int h = w; h < G; h += 4) {
        const float sj = lane < nk ? sc[h][lane] : -INFINITY;
        float m = row16_max(sj);
        m = fmaxf(fmaxf(readlane_f(m, 0), readlane_f(m, 16)), fmaxf(readlane_f(m, 32), readlane_f(m, 48)));
        const float e = lane < nk ? __expf(sj - m) : 0.f;
        sc[h][lane] = e;
        const float l = wave_sum_dpp(e);
        if (lane == 0) {
            mls[h][0] = m;
            mls[h][1] = l;
        }
    }
    __syncthreads();

    // ---- 3. weighted sum of the value rows ----
    {
        float2 acc[G];
#pragma unroll
        for (int h = 0; h < G; h++) acc[h] = make_float2(0.f, 0.f);
#pragma unroll
        for (int i = 0; i < VPT; i++) {
            const int j = kg + KG * i;
#pragma unroll
            for (int h = 0; h < G; h++) {
                const float p = sc[h][j];          // 0 past nk
                acc[h].x += p * vv[i].x;
                acc[h].y += p * vv[i].y;
            }
        }
        for (int h = 0; h < G; h++) {
            red[kg][h][0][dp] = acc[h].x;
            red[kg][h][1][dp] = acc[h].y;
        }
    }
    __syncthreads();
    const size_t mc = (size_t)a.max_chunks;
    for (int i = tid; i < G * HD; i += 256) {
        const int h = i / HD, e = i % HD;
        float s = 0.f;
#pragma unroll
        for (int k = 0; k < KG; k++) s += red[k][h][e & 1][e >> 1];
        const size_t hh = (size_t)t * a.H + g * G + h;
        a.part[(hh * mc + c) * HD + e] = s;
        if (e == 0) {
            a.ml[(hh * mc + c) * 2 + 0] = mls[h][0];
            a.ml[(hh * mc + c) * 2 + 1] = mls[h][1];
        }
    }
}

// Sum of a value over lanes l and l ^ 16 with one v_permlane16_swap (rows 0
// and 1, and rows 2 and 3, of 16 lanes trade places; each lane gets back its
// own value and its partner's).
DEV float pair16_sum(float v) {
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
DEV float half_sum(float v);

// Merge of the chunk partials of one (head, token), 16 dims per block: one
// wavefront, so every step is a lane exchange and nothing waits at a
// barrier.  Lane l holds the statistics of chunks l and l + 64, and dims
// 4 (l % 4) .. +3 of chunks l / 4 + 16 i (i < 8): the first 128 chunks'
// loads are all requested at entry, the statistics first, so a context of
// up to 128 chunks costs one memory latency (longer ones take further rounds
// of 64 chunks).  Then
//   M = max_c m_c, w_c = e^(m_c - M), L = sum_c l_c w_c, o = sum_c acc_c w_c / L.
template <int HD>
__global__ __launch_bounds__(64) void k_attn_merge(AttnArgs a) {
    const int h = blockIdx.x, t = blockIdx.y, d0 = 16 * blockIdx.z, lane = threadIdx.x;
    const int dq = lane & 3, cg = lane >> 2;
    const int nch = a.tok.pos[t] / a.chunk + 1;
    const size_t hh = (size_t)t * a.H + h;
    const float *ml = a.ml + hh * a.max_chunks * 2;
    const float *pa = a.part + hh * a.max_chunks * HD + d0 + 4 * dq;
    // chunks past nch re-read the last one; their weights are 0
    const float2 s0 = *(const float2 *)(ml + 2 * min(lane, nch - 1));
    const float2 s1 = *(const float2 *)(ml + 2 * min(lane + 64, nch - 1));
    f4 v[8];
#pragma unroll
    for (int i = 0; i < 8; i++) v[i] = *(const f4 *)(pa + (size_t)min(cg + 16 * i, nch - 1) * HD);
    float mloc = fmaxf(lane < nch ? s0.x : -INFINITY, lane + 64 < nch ? s1.x : -INFINITY);
    for (int c = lane + 128; c < nch; c += 64) mloc = fmaxf(mloc, ml[2 * c]);
    mloc = row16_max(mloc);
    const float M = fmaxf(fmaxf(readlane_f(mloc, 0), readlane_f(mloc, 16)), fmaxf(readlane_f(mloc, 32), readlane_f(mloc, 48)));
    const float w0 = lane < nch && s0.x != -INFINITY ? __expf(s0.x - M) : 0.f;
    const float w1 = lane + 64 < nch && s1.x != -INFINITY ? __expf(s1.x - M) : 0.f;
    // (l of a chunk is finite: a weight of 0 zeroes it)
    float lloc = s0.y * w0 + s1.y * w1;
    for (int c = lane + 128; c < nch; c += 64) {
        const float2 sc = *(const float2 *)(ml + 2 * c);
        lloc += sc.x == -INFINITY ? 0.f : sc.y * __expf(sc.x - M);
    }
    const float L = wave_sum_dpp(lloc);
    f4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < 8; i++) {
        // chunk cg + 16 i: its weight is w0 (i < 4) or w1 (i >= 4) of lane cg + 16 (i % 4)
        const float wc = __shfl(i < 4 ? w0 : w1, cg + 16 * (i & 3), 64);
        if (cg + 16 * i < nch) acc += v[i] * wc;
    }
    for (int c0 = 128; c0 < nch; c0 += 64) {
#pragma unroll
        for (int i = 0; i < 4; i++) v[i] = *(const f4 *)(pa + (size_t)min(c0 + cg + 16 * i, nch - 1) * HD);
        const float2 sc = *(const float2 *)(ml + 2 * min(c0 + lane, nch - 1));
        const float wl = c0 + lane < nch && sc.x != -INFINITY ? __expf(sc.x - M) : 0.f;
#pragma unroll
        for (int i = 0; i < 4; i++) {
            const float wc = __shfl(wl, cg + 16 * i, 64);
            if (c0 + cg + 16 * i < nch) acc += v[i] * wc;
        }
    }
    // sum over the 16 chunk groups (lane bits 2..5): lanes l + 4 j of a row
    // (rotations by 4 and 8), then the other rows (lane ^ 16, lane ^ 32)
#pragma unroll
    for (int e = 0; e < 4; e++) {
        float x = acc[e];
        x += dpp_f<0x124>(x);
        x += dpp_f<0x128>(x);
        x = pair16_sum(x);
        acc[e] = half_sum(x);
    }
    if (cg == 0) {
        h2 o[2], ol[2];
#pragma unroll
        for (int e = 0; e < 4; e++) {
            const float ov = acc[e] / L;
            const f16 oh = (f16)ov;
            o[e >> 1][e & 1] = oh;
            ol[e >> 1][e & 1] = (f16)(ov - (float)oh);
        }
        const size_t off = (size_t)t * a.H * HD + (size_t)h * HD + d0 + 4 * dq;
        *(uint2 *)((f16 *)a.o + off) = make_uint2(h2_bits(o[0]), h2_bits(o[1]));
        if (a.o_lo) *(uint2 *)((f16 *)a.o_lo + off) = make_uint2(h2_bits(ol[0]), h2_bits(ol[1]));
    }
}

// Sum and max of a value over lanes l and l ^ 32 with one v_permlane32_swap
// (each lane gets back its own value and its partner's, in lane order), in
// place of a cross-lane shuffle through LDS.
DEV float half_sum(float v) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
DEV float half_max(float v) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

constexpr int MW = 2;                // wavefronts per block of the MFMA kernel
constexpr int CHM = 32 * MW;        // cached rows per chunk of the MFMA kernel

// The block's wavefronts combined into the chunk partial (m, l, acc per head)
// of an MFMA kernel: O row (head) of accumulator r < 4 is 4 (lane/32) + r,
// column lane%32; m, l are per head lane%32.
template <int HD>
DEV void mfma_combine(const AttnArgs &a, int c, int g, int t, int G, float m, float l, const f16x *o,
                      float (*cm)[32], float (*cl)[32], float (*co)[GMAX][HD]) {
    constexpr int DT = HD / 32;
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, hf = lane >> 5, ln = lane & 31;
    if (lane < 32) {
        cm[w][ln] = m;
        cl[w][ln] = l;
    }
#pragma unroll
    for (int r = 0; r < 4; r++) {
        const int hh = 4 * hf + r;
        if (hh < G)
#pragma unroll
            for (int dt = 0; dt < DT; dt++) co[w][hh][32 * dt + ln] = o[dt][r];
    }
    __syncthreads();
    const size_t mc = (size_t)a.max_chunks;
    for (int i = tid; i < G * HD; i += MW * 64) {
        const int h = i / HD, d = i % HD;
        float M = -INFINITY;
#pragma unroll
        for (int k = 0; k < MW; k++) M = fmaxf(M, cm[k][h]);
        float acc = 0.f, L = 0.f;
#pragma unroll
        for (int k = 0; k < MW; k++) {
            const float f = cm[k][h] == -INFINITY ? 0.f : __expf(cm[k][h] - M);
            acc += co[k][h][d] * f;
            L += cl[k][h] * f;
        }
        const size_t hh = (size_t)t * a.H + g * G + h;
        a.part[(hh * mc + c) * HD + d] = acc;
        if (d == 0) {
            a.ml[(hh * mc + c) * 2 + 0] = M;
            a.ml[(hh * mc + c) * 2 + 1] = L;
        }
    }
}

// KT: K rows through an LDS tile as coalesced 16-byte pieces (for calls of a
// few tokens, where the grid is small and each load's latency is exposed);
// else straight into the operand (many blocks: the tile's LDS would cut how
// many are resident, which costs more than the wider loads save).
template <int HD, bool KT>
__global__ __launch_bounds__(MW * 64) void k_attn_mfma(AttnArgs a) {
    constexpr int KS = HD / 16;          // k-steps of S^T = K Q^T
    constexpr int DT = HD / 32;          // 32-dim tiles of O = P V
    __shared__ float cm[MW][32], cl[MW][32];
    __shared__ __attribute__((aligned(16))) float co[MW][GMAX][HD];
    __shared__ __attribute__((aligned(16))) f16 vtile[MW][32 * (HD + 8)];
    __shared__ __attribute__((aligned(16))) f16 ktile[KT ? MW : 1][KT ? 32 * (HD + 8) : 8];

    const int c = blockIdx.x, g = blockIdx.y, t = blockIdx.z;
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, hf = lane >> 5, ln = lane & 31;
    const int pos = a.tok.pos[t], seq = a.tok.seq[t];
    const int G = a.H / a.kv.n_kv;
    const int c0 = c * CHM;
    if (c0 > pos) return;                              // uniform per block
    const int k0 = c0 + 32 * w;                        // this wavefront's first key
    const size_t base = (((size_t)seq * a.kv.n_kv + g) * a.kv.n_ctx) * HD;
    const f16 *Kb = (const f16 *)a.kv.k + base;
    const f16 *Vb = (const f16 *)a.kv.v + base;

    // ---- every load at entry; rows past pos are replaced by row pos (finite
    // data whose weights are 0) ----
    // A operand of S^T: key k0 + lane%32, dims 16 ks + 8 (lane/32) .. + 7.
    // KT: the wavefront's 32 K rows are requested as 16-byte pieces, HD/8
    // lanes per row (a load instruction covers 64 / (HD/8) whole rows instead
    // of 16 bytes of 32 rows), and pass through a wavefront-private LDS tile.
    constexpr int VP = HD / 8, VR = 32 * VP / 64;      // pieces per row, rounds
    u32x4 kraw[KT ? VR : 1];
    h8 kf[KS];
    if constexpr (KT) {
#pragma unroll
        for (int u = 0; u < VR; u++) {
            const int pc = u * 64 + lane, key = min(k0 + pc / VP, pos);
            kraw[u] = *(const u32x4 *)(Kb + (size_t)key * HD + 8 * (pc % VP));
        }
    } else {
        const int kr = min(k0 + ln, pos);
#pragma unroll
        for (int ks = 0; ks < KS; ks++) kf[ks] = *(const h8 *)(Kb + (size_t)kr * HD + 16 * ks + 8 * hf);
    }
    // B operand of S^T: head lane%32 (clamped to the group; the extra columns
    // are ignored), the same dims, q / sqrt(hd) as value + remainder
    h8 qa[KS], qb[KS];
    const size_t qo = ((size_t)t * a.H + g * G + min(ln, G - 1)) * HD + 8 * hf;
#pragma unroll
    for (int ks = 0; ks < KS; ks++) {
        qa[ks] = *(const h8 *)((const f16 *)a.qh + qo + 16 * ks);
        qb[ks] = *(const h8 *)((const f16 *)a.ql + qo + 16 * ks);
    }
    // B operand of O = P V for k-step s: element e of lane l is key
    // 16 s + 8 (e/4) + 4 (l/32) + e%4 -- the keys whose probabilities the lane
    // holds in its S^T accumulators 8 s + e -- at dim 32 dt + l%32
    // The wavefront's 32 V rows are requested the same way (8 KB at hd 128)
    // and pass through their own tile, from which the transposed operand is read.
    u32x4 vraw[VR];
#pragma unroll
    for (int u = 0; u < VR; u++) {
        const int pc = u * 64 + lane, key = min(k0 + pc / VP, pos);
        vraw[u] = *(const u32x4 *)(Vb + (size_t)key * HD + 8 * (pc % VP));
    }
    // keep these requests here: left to itself the compiler issues them only
    // after the scores' softmax, a second round trip in the wavefront's chain
    __builtin_amdgcn_sched_barrier(0);

    // ---- KT: K tile through LDS (rows padded by 16 bytes) ----
    if constexpr (KT) {
        f16 *kt = &ktile[w][0];
#pragma unroll
        for (int u = 0; u < VR; u++) {
            const int pc = u * 64 + lane;
            *(u32x4 *)(kt + (pc / VP) * (HD + 8) + 8 * (pc % VP)) = kraw[u];
        }
        // (a wavefront's LDS accesses complete in order: no wait or barrier)
#pragma unroll
        for (int ks = 0; ks < KS; ks++) kf[ks] = *(const h8 *)(kt + ln * (HD + 8) + 16 * ks + 8 * hf);
    }

    // ---- S^T = K Q^T (exact products, fp32 accumulation) ----
    f16x sacc;
#pragma unroll
    for (int r = 0; r < 16; r++) sacc[r] = 0.f;
#pragma unroll
    for (int ks = 0; ks < KS; ks++) {
        sacc = __builtin_amdgcn_mfma_f32_32x32x16_f16(kf[ks], qa[ks], sacc, 0, 0, 0);
        sacc = __builtin_amdgcn_mfma_f32_32x32x16_f16(kf[ks], qb[ks], sacc, 0, 0, 0);
    }

    // ---- causal mask and this wavefront's softmax statistics per head ----
    float m = -INFINITY;
#pragma unroll
    for (int r = 0; r < 16; r++) {
        const int key = k0 + (r >> 2) * 8 + 4 * hf + (r & 3);
        if (key > pos) sacc[r] = -INFINITY;
        m = fmaxf(m, sacc[r]);
    }
    m = half_max(m);
    float l = 0.f;
    h8 ph[2], pl[2];
#pragma unroll
    for (int r = 0; r < 16; r++) {
        const float p = m == -INFINITY ? 0.f : __expf(sacc[r] - m);
        l += p;
        const f16 p16 = (f16)p;
        ph[r >> 3][r & 7] = p16;
        pl[r >> 3][r & 7] = (f16)(p - (float)p16);
    }
    l = half_sum(l);

    // ---- V tile through LDS (rows padded by 16 bytes) ----
    f16 *vt = &vtile[w][0];
#pragma unroll
    for (int u = 0; u < VR; u++) {
        const int pc = u * 64 + lane;
        *(u32x4 *)(vt + (pc / VP) * (HD + 8) + 8 * (pc % VP)) = vraw[u];
    }
    // (a wavefront's LDS accesses complete in order: no wait or barrier)
    h8 vb[DT][2];
#pragma unroll
    for (int s = 0; s < 2; s++)
#pragma unroll
        for (int e = 0; e < 8; e++) {
            const int key = 16 * s + 8 * (e >> 2) + 4 * hf + (e & 3);
#pragma unroll
            for (int dt = 0; dt < DT; dt++) vb[dt][s][e] = vt[key * (HD + 8) + 32 * dt + ln];
        }

    // ---- O = P V: A = P (value + remainder) straight from the accumulators ----
    f16x o[DT];
#pragma unroll
    for (int dt = 0; dt < DT; dt++) {
#pragma unroll
        for (int r = 0; r < 16; r++) o[dt][r] = 0.f;
#pragma unroll
        for (int s = 0; s < 2; s++) {
            o[dt] = __builtin_amdgcn_mfma_f32_32x32x16_f16(ph[s], vb[dt][s], o[dt], 0, 0, 0);
            o[dt] = __builtin_amdgcn_mfma_f32_32x32x16_f16(pl[s], vb[dt][s], o[dt], 0, 0, 0);
        }
    }

    mfma_combine<HD>(a, c, g, t, G, m, l, o, cm, cl, co);
}

// Q8_0 cache: the same chunk partials from matrix cores on exact codes.
//   S^T = K Q^T   each 32-dim block b is its own temporary tile T_b (codes as
//                 f16, exact, against q / sqrt(hd) value + remainder), then
//                 S^T[key] += d_K(key, b) T_b[key] in fp32.  The dims of
//                 block b are split by lane half (16 contiguous code bytes
//                 per lane, k-step 2b taking the first 8, 2b+1 the last 8);
//                 q is read in the same order.
//   O = P V       output tile dt (32 dims) is exactly V block dt, so its
//                 scale d_V(key, dt) varies only along the keys and folds
//                 into P: A = P d_V as f16 value + remainder, B = the codes.
// A code c becomes an f16 with byte permutes: the byte c + 128 under the
// exponent of 1024 is the f16 1152 + c, and one packed subtraction of 1152
// leaves c (all exact).  Each wavefront's 32 block scales of K and V go
// through LDS as f32, one global load per lane.
constexpr uint32_t F16_1024_BYTES = 0x64646464u;   // every byte the high byte of f16 1024
constexpr uint32_t H2_1152 = 0x64806480u;          // f16 pair (1152, 1152)

DEV h2 h2_minus_1152(uint32_t v) { return as_h2(v) - as_h2(H2_1152); }

// Four codes (one dword, code k in byte k) -> f16 pairs (c0, c1), (c2, c3).
DEV void codes4_to_h2(uint32_t w, h2 &a, h2 &b) {
    const uint32_t x = w ^ 0x80808080u;
    a = h2_minus_1152(__builtin_amdgcn_perm(F16_1024_BYTES, x, 0x04010400u));
    b = h2_minus_1152(__builtin_amdgcn_perm(F16_1024_BYTES, x, 0x04030402u));
}

DEV h8 codes8_to_h8(uint32_t lo, uint32_t hi) {
    h2 p[4];
    codes4_to_h2(lo, p[0], p[1]);
    codes4_to_h2(hi, p[2], p[3]);
    h8 r;
#pragma unroll
    for (int k = 0; k < 4; k++) {
        r[2 * k] = p[k].x;
        r[2 * k + 1] = p[k].y;
    }
    return r;
}

// Two codes held in the low bytes of separate registers -> f16 pair.
DEV h2 codes2_to_h2(uint32_t c0, uint32_t c1) {
    // bytes [c0, 0, c1, 0], then c + 128 under the exponent of 1024
    return h2_minus_1152(__builtin_amdgcn_perm(c1, c0, 0x0c040c00u) ^ H2_1152);
}

template <int NB>
struct ScaleVec;
template <>
struct ScaleVec<2> {
    typedef uint32_t T;
    DEV uint16_t get(T v, int b) { return (uint16_t)(v >> (16 * b)); }
};
template <>
struct ScaleVec<4> {
    typedef uint2 T;
    DEV uint16_t get(T v, int b) { return (uint16_t)((b < 2 ? v.x : v.y) >> (16 * (b & 1))); }
};

template <int HD>
__global__ __launch_bounds__(MW * 64) void k_attn_mfma_q8(AttnArgs a) {
    constexpr int KS = HD / 16;          // k-steps of S^T = K Q^T
    constexpr int NB = HD / 32;          // blocks per row = 32-dim tiles of O
    typedef ScaleVec<NB> SV;
    typedef typename SV::T ST;
    __shared__ float cm[MW][32], cl[MW][32];
    __shared__ __attribute__((aligned(16))) float co[MW][GMAX][HD];
    __shared__ __attribute__((aligned(16))) float sks[MW][2][32][NB];   // [wave][K, V][key][block]

    const int c = blockIdx.x, g = blockIdx.y, t = blockIdx.z;
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, hf = lane >> 5, ln = lane & 31;
    const int pos = a.tok.pos[t], seq = a.tok.seq[t];
    const int G = a.H / a.kv.n_kv;
    const int c0 = c * CHM;
    if (c0 > pos) return;                              // uniform per block
    const int k0 = c0 + 32 * w;                        // this wavefront's first key
    if (a.code_new_rows && pos < c0 + CHM) {           // uniform: the chunk holding the new row
        if (tid < 2 * NB) kv_code_block(a.kv, t, tid / NB, g * NB + tid % NB, seq, pos);
        __syncthreads();
    }
    const size_t cell0 = ((size_t)seq * a.kv.n_kv + g) * a.kv.n_ctx;
    const uint8_t *Kc = (const uint8_t *)a.kv.k + cell0 * HD;
    const uint8_t *Vc = (const uint8_t *)a.kv.v + cell0 * HD;

    // ---- every load at entry; rows past pos are replaced by row pos ----
    // K codes of key k0 + lane%32: block b, dims 32 b + 16 (lane/32) .. + 15
    uint4 kc[NB];
    const int kr = min(k0 + ln, pos);
#pragma unroll
    for (int b = 0; b < NB; b++) kc[b] = *(const uint4 *)(Kc + (size_t)kr * HD + 32 * b + 16 * hf);
    // block scales of key k0 + lane%32: K from the low half-wave, V from the high
    const ST sc = *((const ST *)((hf ? a.kv.v_scale : a.kv.k_scale) + cell0 * NB) + kr);
    // q / sqrt(hd) (value + remainder) of head lane%32 in the same dim order
    h8 qa[KS], qb[KS];
    const size_t qo = ((size_t)t * a.H + g * G + min(ln, G - 1)) * HD + 16 * hf;
#pragma unroll
    for (int ks = 0; ks < KS; ks++) {
        const int off = 32 * (ks >> 1) + 8 * (ks & 1);
        qa[ks] = *(const h8 *)((const f16 *)a.qh + qo + off);
        qb[ks] = *(const h8 *)((const f16 *)a.ql + qo + off);
    }
    // V codes, B operand of O = P V for k-step s: element e of lane l is key
    // 16 s + 8 (e/4) + 4 (l/32) + e%4 at dim 32 dt + l%32
    uint32_t vc[NB][2][8];
#pragma unroll
    for (int s = 0; s < 2; s++)
#pragma unroll
        for (int e = 0; e < 8; e++) {
            const int key = min(k0 + 16 * s + 8 * (e >> 2) + 4 * hf + (e & 3), pos);
#pragma unroll
            for (int dt = 0; dt < NB; dt++) vc[dt][s][e] = Vc[(size_t)key * HD + 32 * dt + ln];
        }
#pragma unroll
    for (int b = 0; b < NB; b++) sks[w][hf][ln][b] = f16_bits_to_f32(SV::get(sc, b));
    __syncthreads();

    // ---- S^T = K Q^T, one exact tile per block, scaled per key ----
    // accumulator register r holds key 8 (r/4) + 4 (lane/32) + r%4 of the wavefront
    f16x sacc;
#pragma unroll
    for (int r = 0; r < 16; r++) sacc[r] = 0.f;
#pragma unroll
    for (int b = 0; b < NB; b++) {
        const h8 klo = codes8_to_h8(kc[b].x, kc[b].y), khi = codes8_to_h8(kc[b].z, kc[b].w);
        f16x tb;
#pragma unroll
        for (int r = 0; r < 16; r++) tb[r] = 0.f;
        tb = __builtin_amdgcn_mfma_f32_32x32x16_f16(klo, qa[2 * b], tb, 0, 0, 0);
        tb = __builtin_amdgcn_mfma_f32_32x32x16_f16(klo, qb[2 * b], tb, 0, 0, 0);
        tb = __builtin_amdgcn_mfma_f32_32x32x16_f16(khi, qa[2 * b + 1], tb, 0, 0, 0);
        tb = __builtin_amdgcn_mfma_f32_32x32x16_f16(khi, qb[2 * b + 1], tb, 0, 0, 0);
#pragma unroll
        for (int r = 0; r < 16; r++) sacc[r] += sks[w][0][8 * (r >> 2) + 4 * hf + (r & 3)][b] * tb[r];
    }

    // ---- causal mask and this wavefront's softmax statistics per head ----
    float m = -INFINITY;
#pragma unroll
    for (int r = 0; r < 16; r++) {
        const int key = k0 + (r >> 2) * 8 + 4 * hf + (r & 3);
        if (key > pos) sacc[r] = -INFINITY;
        m = fmaxf(m, sacc[r]);
    }
    m = half_max(m);
    float l = 0.f, p[16];
#pragma unroll
    for (int r = 0; r < 16; r++) {
        p[r] = m == -INFINITY ? 0.f : __expf(sacc[r] - m);
        l += p[r];
    }
    l = half_sum(l);

    // ---- O = P V: tile dt takes A = P d_V(key, dt) (value + remainder) ----
    f16x o[NB];
#pragma unroll
    for (int dt = 0; dt < NB; dt++) {
        h8 ph[2], pl[2];
#pragma unroll
        for (int r = 0; r < 16; r++) {
            const float pv = p[r] * sks[w][1][8 * (r >> 2) + 4 * hf + (r & 3)][dt];
            const f16 p16 = (f16)pv;
            ph[r >> 3][r & 7] = p16;
            pl[r >> 3][r & 7] = (f16)(pv - (float)p16);
        }
#pragma unroll
        for (int r = 0; r < 16; r++) o[dt][r] = 0.f;
#pragma unroll
        for (int s = 0; s < 2; s++) {
            h8 vb;
#pragma unroll
            for (int k = 0; k < 4; k++) {
                const h2 v2 = codes2_to_h2(vc[dt][s][2 * k], vc[dt][s][2 * k + 1]);
                vb[2 * k] = v2.x;
                vb[2 * k + 1] = v2.y;
            }
            o[dt] = __builtin_amdgcn_mfma_f32_32x32x16_f16(ph[s], vb, o[dt], 0, 0, 0);
            o[dt] = __builtin_amdgcn_mfma_f32_32x32x16_f16(pl[s], vb, o[dt], 0, 0, 0);
        }
    }
    mfma_combine<HD>(a, c, g, t, G, m, l, o, cm, cl, co);
}

// Chunk size of the path launch_attention takes for this cache.
bool mfma_path(int kvtype, int hd) { return (kvtype == T_F16 || kvtype == T_Q8_0) && (hd == 64 || hd == 128); }
int chunk_for(int kvtype, int hd) { return mfma_path(kvtype, hd) ? CHM : CH; }

template <int HD, int KVT>
bool launch_part(const AttnArgs &a, int T, hipStream_t s) {
    const dim3 grid(a.max_chunks, a.kv.n_kv, T);
    switch (a.H / a.kv.n_kv) {
    case 1: launch((k_attn_part<HD, KVT, 1>), grid, dim3(256), 0, s, a); return true;
    case 2: launch((k_attn_part<HD, KVT, 2>), grid, dim3(256), 0, s, a); return true;
    case 4: launch((k_attn_part<HD, KVT, 4>), grid, dim3(256), 0, s, a); return true;
    case 8: launch((k_attn_part<HD, KVT, 8>), grid, dim3(256), 0, s, a); return true;
    default: return false;
    }
}

template <int HD>
bool launch_hd(const AttnArgs &a, int T, hipStream_t s) {
    bool ok;
    if (mfma_path(a.kv.kvtype, HD)) {
        if constexpr (HD <= 128) {
            if (a.H / a.kv.n_kv > GMAX || !a.qh || !a.ql) return false;
            if (a.kv.kvtype == T_Q8_0)
                launch(k_attn_mfma_q8<HD>, dim3(a.max_chunks, a.kv.n_kv, T), dim3(MW * 64), 0, s, a);
            else if (T <= 4)   // (measured: batch 1 13.5 -> 12.5 us per layer; batch 32 slower)
                launch(k_attn_mfma<HD, true>, dim3(a.max_chunks, a.kv.n_kv, T), dim3(MW * 64), 0, s, a);
            else
                launch(k_attn_mfma<HD, false>, dim3(a.max_chunks, a.kv.n_kv, T), dim3(MW * 64), 0, s, a);
            ok = true;
        } else {
            return false;
        }
    } else {
        ok = a.kv.kvtype == T_F16    ? launch_part<HD, T_F16>(a, T, s)
             : a.kv.kvtype == T_Q8_0 ? launch_part<HD, T_Q8_0>(a, T, s)
                                     : launch_part<HD, T_F32>(a, T, s);
    }
    if (!ok) return false;
    launch((k_attn_merge<HD>), dim3(a.H, T, HD / 16), dim3(64), 0, s, a);
    return true;
}

}  // namespace

bool launch_attention(const AttnArgs &a, int T, hipStream_t s) {
    if (T <= 0 || a.max_chunks > 1024 || a.chunk != chunk_for(a.kv.kvtype, a.kv.hd)) return false;
    if (a.code_new_rows && !attention_codes_rows(a.kv.kvtype, a.kv.hd)) return false;
    switch (a.kv.hd) {
    case 64: return launch_hd<64>(a, T, s);
    case 128: return launch_hd<128>(a, T, s);
    case 256: return launch_hd<256>(a, T, s);
    default: return false;
    }
}

int attention_chunk(int kvtype, int hd) { return chunk_for(kvtype, hd); }

static_assert(CH == 64 && CHM == 64 && 1024 * CH == DEC_MAX_CTX,
              "the public context limit is 1024 chunks of every attention kernel");

bool attention_codes_rows(int kvtype, int hd) { return kvtype == T_Q8_0 && mfma_path(kvtype, hd); }
