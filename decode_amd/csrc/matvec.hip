// matvec.hip -- dequant-fused block-quantized mat-vec for decode (gfx950).
//
// y = W x with W in Q8_0 / Q4_0 blocks and x an activation row.  This is the
// memory-bound heart of a decode step: every weight byte is read once per
// step, so the kernel is built around streaming the code bytes with 16-byte
// coalesced loads and keeping the arithmetic per weight small.
//
// Work split: a 256-thread block holds 4 wavefronts; each wavefront owns a
// contiguous range of row pairs and computes full rows.  Lane l covers the
// 32-weight blocks b = l, l+64, l+128, ... of every row, so one wavefront
// load instruction reads 64 consecutive 16-byte chunks of a row.  The lane
// keeps the matching 32 activations of each of its blocks in registers as
// f16 pairs for all rows it visits; rows end with a wavefront butterfly sum.
//
// Dequantization never materializes a weight.  A code q sits in the low bits
// of an f16 whose exponent field is that of 1024 (bit pattern 0x6400 | q), so
// the f16 value is exactly 1024 + u, with u = q (Q4_0) or q + 128 (Q8_0,
// after flipping the sign bit).  v_dot2_f32_f16 multiplies two such values by
// two activations exactly and accumulates in fp32.  The offset is removed
// once per block: sum((1024+u) x) - C * sum(x) = sum((u + 1024 - C) x) with
// C = 1032 for Q4_0 (code - 8) and C = 1152 for Q8_0 (code as signed int8).
// The block sum of x is computed once per lane when x is loaded.
//
// Optional prologue: RMSNorm of the f32 residual row (sum of squares reduced
// over the block, then x * rstd * g rounded to f16), so the normalization of
// the article's per-layer graph costs no extra launch.
#include "common.h"
#include "epilogue.h"
#include "kernels.h"

namespace {

// Activation pairs in the order the code extraction produces them.
// Q4_0 block dword i (bytes 4i..4i+3): low nibbles = codes 4i..4i+3, high
// nibbles = codes 16+4i..16+4i+3.  Masks 0x000F000F at shifts 0, 4, 8, 12
// select code pairs (4i,4i+2), (16+4i,18+4i), (4i+1,4i+3), (17+4i,19+4i).
DEV void pairs_q4(const f16 *x, h2 *xp) {
#pragma unroll
    for (int i = 0; i < 4; i++) {
        xp[4 * i + 0] = h2{x[4 * i + 0], x[4 * i + 2]};
        xp[4 * i + 1] = h2{x[16 + 4 * i + 0], x[16 + 4 * i + 2]};
        xp[4 * i + 2] = h2{x[4 * i + 1], x[4 * i + 3]};
        xp[4 * i + 3] = h2{x[16 + 4 * i + 1], x[16 + 4 * i + 3]};
    }
}
// Q8_0 block dword i holds codes 4i..4i+3; masks 0x00FF00FF at shifts 0 and 8
// select code pairs (4i, 4i+2) and (4i+1, 4i+3).
DEV void pairs_q8(const f16 *x, h2 *xp) {
#pragma unroll
    for (int i = 0; i < 8; i++) {
        xp[2 * i + 0] = h2{x[4 * i + 0], x[4 * i + 2]};
        xp[2 * i + 1] = h2{x[4 * i + 1], x[4 * i + 3]};
    }
}

DEV float blockdot_q4(const uint4 q, const h2 *xp) {
    const uint32_t w[4] = {q.x, q.y, q.z, q.w};
    float acc = 0.f;
#pragma unroll
    for (int i = 0; i < 4; i++) {
        acc = dot2(as_h2((w[i] & 0x000F000Fu) | 0x64006400u), xp[4 * i + 0], acc);
        acc = dot2(as_h2(((w[i] >> 4) & 0x000F000Fu) | 0x64006400u), xp[4 * i + 1], acc);
        acc = dot2(as_h2(((w[i] >> 8) & 0x000F000Fu) | 0x64006400u), xp[4 * i + 2], acc);
        acc = dot2(as_h2(((w[i] >> 12) & 0x000F000Fu) | 0x64006400u), xp[4 * i + 3], acc);
    }
    return acc;
}

DEV float blockdot_q8(const uint4 q0, const uint4 q1, const h2 *xp) {
    const uint32_t w[8] = {q0.x, q0.y, q0.z, q0.w, q1.x, q1.y, q1.z, q1.w};
    float acc = 0.f;
#pragma unroll
    for (int i = 0; i < 8; i++) {
        const uint32_t u = w[i] ^ 0x80808080u;
        acc = dot2(as_h2((u & 0x00FF00FFu) | 0x64006400u), xp[2 * i + 0], acc);
        acc = dot2(as_h2(((u >> 8) & 0x00FF00FFu) | 0x64006400u), xp[2 * i + 1], acc);
    }
    return acc;
}

// Code bytes + scales of one pair of rows for this lane's blocks.
template <int WT, int KB>
struct PairLoad {
    uint4 q[2][KB][WT == T_Q4_0 ? 1 : 2];
    uint16_t d[2][KB];
};

// Blocks b0 + lane + 64*i (i < KB) below b1 of rows r0, r1.
template <int WT, int KB>
DEV void load_pair(const QMat &W, int r0, int r1, int b0, int b1, int lane, PairLoad<WT, KB> &L) {
    const int K = W.K, nb = K >> 5;
    const int rows[2] = {r0, r1};
#pragma unroll
    for (int r = 0; r < 2; r++) {
        const uint16_t *dr = W.d + (size_t)rows[r] * nb;
        const uint4 *qr = WT == T_Q4_0
                              ? (const uint4 *)((const uint8_t *)W.qs + (size_t)rows[r] * (K >> 1))
                              : (const uint4 *)((const int8_t *)W.qs + (size_t)rows[r] * K);
#pragma unroll
        for (int i = 0; i < KB; i++) {
            const int b = b0 + lane + 64 * i;
            if (b < b1) {
                if (WT == T_Q4_0) {
                    L.q[r][i][0] = load_stream16(qr + b);
                } else {
                    L.q[r][i][0] = load_stream16(qr + 2 * b);
                    L.q[r][i][WT == T_Q4_0 ? 0 : 1] = load_stream16(qr + 2 * b + 1);
                }
                L.d[r][i] = dr[b];
            } else {
#pragma unroll
                for (int j = 0; j < (WT == T_Q4_0 ? 1 : 2); j++) L.q[r][i][j] = make_uint4(0, 0, 0, 0);
                L.d[r][i] = 0;
            }
        }
    }
}

template <int WT, int KB>
DEV float dot_row(const PairLoad<WT, KB> &L, int r, const h2 (*xp)[16], const float *xsum) {
    float a = 0.f;
#pragma unroll
    for (int i = 0; i < KB; i++) {
        float bd;
        if (WT == T_Q4_0)
            bd = blockdot_q4(L.q[r][i][0], xp[i]);
        else
            bd = blockdot_q8(L.q[r][i][0], L.q[r][i][WT == T_Q4_0 ? 0 : 1], xp[i]);
        a += f16_bits_to_f32(L.d[r][i]) * (bd - xsum[i]);
    }
    return a;
}

// NW wavefronts per block (one block per CU): the activation row is staged
// once per block in LDS (normalized on the way when a norm is given).  The
// K dimension is cut into S slices of at most 128 blocks; S wavefronts share
// one row pair, each covering one slice with at most 2 blocks per lane whose
// activations it keeps in registers.  Row pairs p = g, g + G, ... are
// streamed with the next pair's loads in flight while the current pair is
// reduced (DPP within the wavefront; for S > 1 the S partial sums meet in
// double-buffered LDS and are added in slice order).
template <int WT, int KB, int S, int EPI>
__global__ __launch_bounds__(1024) void k_matvec(QMat W, InArgs in, EpiArgs ep, int pair_mode) {
    constexpr int NW = 16, NT = NW * 64, G = NW / S;
    __shared__ __attribute__((aligned(16))) f16 xs[S * KB * 64 * 32];
    __shared__ float red[NW];
    __shared__ float part[2][NW][2];
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int t = blockIdx.y;
    const int K = W.K, nb = K >> 5;
    const int xrow = in.row_idx ? in.row_idx[t] : t;

    // ---- stage the activation row in LDS as f16 ----
    if (in.norm_g) {
        const float *xr = in.x32 + (size_t)xrow * in.ldx;
        float ss = 0.f;
        for (int k = tid * 4; k < K; k += NT * 4) {
            const float4 v = *(const float4 *)(xr + k);
            ss += v.x * v.x + v.y * v.y + v.z * v.z + v.w * v.w;
        }
        ss = wave_sum_dpp(ss);
        if (lane == 0) red[w] = ss;
        __syncthreads();
        float tot = 0.f;
#pragma unroll
        for (int i = 0; i < NW; i++) tot += red[i];
        const float rstd = 1.0f / sqrtf(tot / (float)K + in.eps);
        for (int k = tid * 4; k < K; k += NT * 4) {
            const float4 v = *(const float4 *)(xr + k);
            const float4 g = *(const float4 *)(in.norm_g + k);
            h2 lo, hi;
            lo.x = (f16)(v.x * rstd * g.x);
            lo.y = (f16)(v.y * rstd * g.y);
            hi.x = (f16)(v.z * rstd * g.z);
            hi.y = (f16)(v.w * rstd * g.w);
            *(uint2 *)&xs[k] = make_uint2(h2_bits(lo), h2_bits(hi));
        }
    } else {
        const uint16_t *xr = in.x16 + (size_t)xrow * in.ldx;
        for (int k = tid * 8; k < K; k += NT * 8) *(uint4 *)&xs[k] = *(const uint4 *)(xr + k);
    }
    __syncthreads();

    // ---- this wavefront's K slice -> f16 pairs in registers ----
    const int slice = w % S, grp = w / S;
    const int nbs = (nb + S - 1) / S;
    const int b0 = slice * nbs, b1 = min(nb, b0 + nbs);
    h2 xp[KB][16];
    float xsum[KB];
#pragma unroll
    for (int i = 0; i < KB; i++) {
        const int b = b0 + lane + 64 * i;
        f16 xv[32];
        if (b < b1) {
#pragma unroll
            for (int j = 0; j < 4; j++) *(uint4 *)&xv[8 * j] = *(const uint4 *)&xs[b * 32 + 8 * j];
        } else {
#pragma unroll
            for (int j = 0; j < 32; j++) xv[j] = (f16)0.f;
        }
        float sum = 0.f;
#pragma unroll
        for (int j = 0; j < 32; j++) sum += (float)xv[j];
        xsum[i] = sum * (WT == T_Q4_0 ? 1032.f : 1152.f);
        if (WT == T_Q4_0)
            pairs_q4(xv, xp[i]);
        else
            pairs_q8(xv, xp[i]);
    }

    // ---- stream row pairs ----
    const int npairs = W.N >> 1;
    const int stride = gridDim.x * G;
    const int first = blockIdx.x * G + grp;
    const int iters = (npairs + stride - 1) / stride;    // same for every wavefront of the grid
    int p = first, r0 = 0, r1 = 1;
    PairLoad<WT, KB> cur;
    if (p < npairs) {
        pair_rows(pair_mode, p, r0, r1);
        load_pair<WT, KB>(W, r0, r1, b0, b1, lane, cur);
    }
    for (int it = 0; it < iters; it++) {
        const int pn = p + stride;
        int n0 = r0, n1 = r1;
        PairLoad<WT, KB> nxt;
        if (pn < npairs) {
            pair_rows(pair_mode, pn, n0, n1);
            load_pair<WT, KB>(W, n0, n1, b0, b1, lane, nxt);
        }
        float a0 = 0.f, a1 = 0.f;
        if (p < npairs) {
            a0 = wave_sum_dpp(dot_row<WT, KB>(cur, 0, xp, xsum));
            a1 = wave_sum_dpp(dot_row<WT, KB>(cur, 1, xp, xsum));
        }
        if (S == 1) {
            if (lane == 0 && p < npairs) epi_pair<EPI>(ep, t, p, r0, r1, a0, a1);
        } else {
            if (lane == 0) {
                part[it & 1][w][0] = a0;
                part[it & 1][w][1] = a1;
            }
            __syncthreads();
            if (slice == 0 && lane == 0 && p < npairs) {
                float s0 = 0.f, s1 = 0.f;
#pragma unroll
                for (int j = 0; j < S; j++) {
                    s0 += part[it & 1][w + j][0];
                    s1 += part[it & 1][w + j][1];
                }
                epi_pair<EPI>(ep, t, p, r0, r1, s0, s1);
            }
        }
        p = pn;
        r0 = n0;
        r1 = n1;
        cur = nxt;
    }
}

int g_num_cu = 256;

template <int WT, int KB, int S, int EPI>
bool launch_epi(const QMat &W, const InArgs &in, const EpiArgs &ep, int T, int pair_mode,
                hipStream_t s) {
    constexpr int G = 16 / S;
    const int npairs = W.N / 2;
    int blocks = (npairs + G - 1) / G;
    if (blocks > g_num_cu) blocks = g_num_cu;
    hipLaunchKernelGGL((k_matvec<WT, KB, S, EPI>), dim3(blocks, T), dim3(1024), 0, s, W, in, ep,
                       pair_mode);
    return true;
}

template <int WT, int KB, int S>
bool launch_ks(const QMat &W, const InArgs &in, const EpiArgs &ep, int T, int pair_mode,
               hipStream_t s) {
    switch (ep.epi) {
    case EPI_STORE: return launch_epi<WT, KB, S, EPI_STORE>(W, in, ep, T, pair_mode, s);
    case EPI_RESID: return launch_epi<WT, KB, S, EPI_RESID>(W, in, ep, T, pair_mode, s);
    case EPI_QKV: return launch_epi<WT, KB, S, EPI_QKV>(W, in, ep, T, pair_mode, s);
    case EPI_SWIGLU: return launch_epi<WT, KB, S, EPI_SWIGLU>(W, in, ep, T, pair_mode, s);
    default: return false;
    }
}

template <int WT>
bool launch_wt(const QMat &W, const InArgs &in, const EpiArgs &ep, int T, int pair_mode,
               hipStream_t s) {
    const int nb = W.K / 32;
    if (nb <= 64) return launch_ks<WT, 1, 1>(W, in, ep, T, pair_mode, s);
    if (nb <= 128) return launch_ks<WT, 2, 1>(W, in, ep, T, pair_mode, s);
    if (nb <= 256) return launch_ks<WT, 2, 2>(W, in, ep, T, pair_mode, s);
    if (nb <= 512) return launch_ks<WT, 2, 4>(W, in, ep, T, pair_mode, s);
    return false;
}

}  // namespace

void matvec_set_num_cu(int n) {
    if (n > 0) g_num_cu = n;
}

bool launch_matvec(const QMat &W, const InArgs &in, const EpiArgs &ep, int T, hipStream_t s) {
    if (W.K % 32 || W.N % 2 || T <= 0) return false;
    const int pair_mode = ep.epi == EPI_SWIGLU ? PAIR_GU : PAIR_ADJ;
    if (pair_mode == PAIR_GU && W.N % 64) return false;
    if (W.wtype == T_Q4_0) return launch_wt<T_Q4_0>(W, in, ep, T, pair_mode, s);
    if (W.wtype == T_Q8_0) return launch_wt<T_Q8_0>(W, in, ep, T, pair_mode, s);
    return false;
}
