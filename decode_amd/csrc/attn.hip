// attn.hip -- causal GQA attention over the f16 / f32 KV cache (gfx950).
//
// Each query token attends to the cached rows 0..pos of its own sequence
// (the token's own K,V row was appended by the QKV epilogue before this
// kernel runs, as the article's KV-cache appendix orders it).
//
// Split-K ("flash-decoding" within one GPU): the cached positions are cut
// into chunks of CH rows.  One 256-thread block handles (chunk, KV head,
// token) for all query heads of the group that share the KV head, so each
// K/V row is read from HBM once per token and group.  Per block:
//   1. scores s[h][j] = q_h . K_j / sqrt(hd): HD/8 threads per key row, each
//      reading 16 contiguous bytes, reduced with lane shuffles;
//   2. per head: m = max_j s, e_j = exp(s_j - m), l = sum_j e_j (one
//      wavefront per head, wavefront max/sum);
//   3. acc[h][d] = sum_j e_j V_j[d]: HD/2 threads per row, 2 elements each.
// The block writes (m, l, acc) for its chunk; a second kernel merges the
// chunks of a (token, head) in chunk order:
//   M = max_c m_c, L = sum_c l_c e^(m_c - M), o = sum_c acc_c e^(m_c - M) / L,
// and writes o in f16 for the output projection.  The grid covers the
// context's largest chunk count; blocks past a token's last chunk exit, so
// one captured launch serves every decode step.
#include "common.h"
#include "kernels.h"

namespace {

constexpr int CH = 64;      // cached rows per chunk
constexpr int GMAX = 8;     // query heads per KV head handled by one block

template <int KVT>
struct KVRow;
template <>
struct KVRow<T_F16> {
    typedef uint16_t E;
    // 8 consecutive elements as float
    DEV void load8(const uint16_t *p, float *o) {
        const uint4 v = *(const uint4 *)p;
        const h2 a = as_h2(v.x), b = as_h2(v.y), c = as_h2(v.z), d = as_h2(v.w);
        o[0] = (float)a.x; o[1] = (float)a.y; o[2] = (float)b.x; o[3] = (float)b.y;
        o[4] = (float)c.x; o[5] = (float)c.y; o[6] = (float)d.x; o[7] = (float)d.y;
    }
    DEV float2 load2(const uint16_t *p) {
        const h2 a = *(const h2 *)p;
        return make_float2((float)a.x, (float)a.y);
    }
};
template <>
struct KVRow<T_F32> {
    typedef float E;
    DEV void load8(const float *p, float *o) {
        const float4 a = *(const float4 *)p, b = *(const float4 *)(p + 4);
        o[0] = a.x; o[1] = a.y; o[2] = a.z; o[3] = a.w;
        o[4] = b.x; o[5] = b.y; o[6] = b.z; o[7] = b.w;
    }
    DEV float2 load2(const float *p) { return *(const float2 *)p; }
};

template <int HD, int KVT>
__global__ __launch_bounds__(256) void k_attn_part(AttnArgs a, int G) {
    typedef typename KVRow<KVT>::E E;
    constexpr int TPK = HD / 8;          // threads per key row (scores)
    constexpr int KPP = 256 / TPK;       // key rows per pass
    constexpr int TPR = HD / 2;          // threads per value row
    constexpr int KG = 256 / TPR;        // value-row groups

    __shared__ float qs[GMAX][HD];
    __shared__ float sc[GMAX][CH];
    __shared__ float red[KG][GMAX][2][TPR];
    __shared__ float mls[GMAX][2];

    const int c = blockIdx.x, g = blockIdx.y, t = blockIdx.z;
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int pos = a.tok.pos[t], seq = a.tok.seq[t];
    const int c0 = c * CH;
    if (c0 > pos) return;                          // uniform per block
    const int nk = min(CH, pos + 1 - c0);
    const int n_kv = a.kv.n_kv;
    const float scale = 1.0f / sqrtf((float)HD);

    for (int i = tid; i < G * HD; i += 256) {
        const int h = i / HD, e = i % HD;
        qs[h][e] = a.q[((size_t)t * a.H + g * G + h) * HD + e];
    }
    __syncthreads();

    const size_t rowbase = (((size_t)seq * n_kv + g) * a.kv.n_ctx + c0) * HD;
    const E *Kb = (const E *)a.kv.k + rowbase;
    const E *Vb = (const E *)a.kv.v + rowbase;

    // 1. scores
    {
        const int part = tid % TPK;
        for (int j0 = 0; j0 < nk; j0 += KPP) {
            const int j = j0 + tid / TPK;
            float kv8[8];
            if (j < nk)
                KVRow<KVT>::load8(Kb + (size_t)j * HD + part * 8, kv8);
            else
#pragma unroll
                for (int e = 0; e < 8; e++) kv8[e] = 0.f;
            for (int h = 0; h < G; h++) {
                float s = 0.f;
#pragma unroll
                for (int e = 0; e < 8; e++) s += qs[h][part * 8 + e] * kv8[e];
#pragma unroll
                for (int o = TPK / 2; o > 0; o >>= 1) s += __shfl_xor(s, o, 64);
                if (part == 0 && j < nk) sc[h][j] = s * scale;
            }
        }
    }
    __syncthreads();

    // 2. softmax statistics of the chunk
    for (int h = w; h < G; h += 4) {
        float m = -INFINITY;
        for (int j = lane; j < nk; j += 64) m = fmaxf(m, sc[h][j]);
        m = wave_max(m);
        float l = 0.f;
        for (int j = lane; j < nk; j += 64) {
            const float e = __expf(sc[h][j] - m);
            sc[h][j] = e;
            l += e;
        }
        l = wave_sum(l);
        if (lane == 0) {
            mls[h][0] = m;
            mls[h][1] = l;
        }
    }
    __syncthreads();

    // 3. weighted sum of the value rows
    {
        const int dp = tid % TPR, kg = tid / TPR;
        float2 acc[GMAX];
#pragma unroll
        for (int h = 0; h < GMAX; h++) acc[h] = make_float2(0.f, 0.f);
        for (int j = kg; j < nk; j += KG) {
            const float2 v = KVRow<KVT>::load2(Vb + (size_t)j * HD + 2 * dp);
#pragma unroll
            for (int h = 0; h < GMAX; h++) {
                if (h < G) {
                    const float p = sc[h][j];
                    acc[h].x += p * v.x;
                    acc[h].y += p * v.y;
                }
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

template <int HD>
__global__ __launch_bounds__(HD) void k_attn_merge(AttnArgs a) {
    const int h = blockIdx.x, t = blockIdx.y, e = threadIdx.x;
    const int nch = a.tok.pos[t] / a.chunk + 1;
    const size_t hh = (size_t)t * a.H + h;
    const float *ml = a.ml + hh * a.max_chunks * 2;
    const float *pa = a.part + hh * a.max_chunks * HD;
    float M = -INFINITY;
    for (int c = 0; c < nch; c++) M = fmaxf(M, ml[2 * c]);
    float L = 0.f, acc = 0.f;
    for (int c = 0; c < nch; c++) {
        const float f = __expf(ml[2 * c] - M);
        L += ml[2 * c + 1] * f;
        acc += pa[(size_t)c * HD + e] * f;
    }
    ((f16 *)a.o)[(size_t)t * a.H * HD + (size_t)h * HD + e] = (f16)(acc / L);
}

template <int HD>
bool launch_hd(const AttnArgs &a, int T, hipStream_t s) {
    const int G = a.H / a.kv.n_kv;
    if (G > GMAX) return false;
    if (a.kv.kvtype == T_F16)
        hipLaunchKernelGGL((k_attn_part<HD, T_F16>), dim3(a.max_chunks, a.kv.n_kv, T), dim3(256), 0, s,
                           a, G);
    else
        hipLaunchKernelGGL((k_attn_part<HD, T_F32>), dim3(a.max_chunks, a.kv.n_kv, T), dim3(256), 0, s,
                           a, G);
    hipLaunchKernelGGL((k_attn_merge<HD>), dim3(a.H, T), dim3(HD), 0, s, a);
    return true;
}

}  // namespace

bool launch_attention(const AttnArgs &a, int T, hipStream_t s) {
    if (a.chunk != CH || T <= 0) return false;
    switch (a.kv.hd) {
    case 64: return launch_hd<64>(a, T, s);
    case 128: return launch_hd<128>(a, T, s);
    case 256: return launch_hd<256>(a, T, s);
    default: return false;
    }
}

int attention_chunk() { return CH; }
