// matvec.hip -- dequant-fused block-quantized mat-vec for decode (gfx950).
//
// y = W x with W in Q8_0 / Q4_0 blocks (or Q4_K sub-blocks) and x an activation row.  This is the
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
#include "../../include/decode.h"
#include "common.h"
#include "epilogue.h"
#include "kernels.h"
#include "mvcore.h"

static_assert(MV_KMAX == DEC_MAX_ROW, "the public row limit is the mat-vec's LDS image");

namespace {

// NW = 16 wavefronts per block, one block per CU.  The K dimension is cut
// into S slices of at most 64 blocks: lane l of a wavefront covers block
// b0 + l of its slice, and keeps that block's activations (value and
// remainder pairs, from the block's LDS image of the input row) in
// registers.  S wavefronts share one row pair, one slice each.  A wavefront
// keeps D row pairs of codes in flight: the first D are requested right
// after the inputs of the row's LDS image, and each computed pair's
// registers are refilled with the pair D ahead.  Row sums end with a DPP reduction; for S > 1 the
// partial sums of all pairs meet in LDS once, after the last pair, and are
// added in slice order.
constexpr int MV_MAXIT = 16;   // row pairs per wavefront when K is split

template <int WT, int S, int EPI, int D>
__global__ __launch_bounds__(1024) void k_matvec(QMat W, InArgs in, EpiArgs ep, int pair_mode) {
    constexpr int NW = 16, G = NW / S;
    constexpr bool NORM = EPI != EPI_RESID;   // every epilogue except the residual add reads a normalized row
    __shared__ __attribute__((aligned(16))) uint32_t img[(MV_KMAX / 32) * XROW];
    __shared__ float bsum[MV_KMAX / 32];
    __shared__ float xsum[WT == T_Q4_K ? MV_KMAX / 32 : 1];   // Q4_K: plain block sums of x
    __shared__ float red[NW];
    __shared__ float part[S > 1 ? G * MV_MAXIT * S * 2 : 1];
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int t = blockIdx.y;
    const int K = W.K, nb = K >> 5;
    const int xrow = in.row_idx ? in.row_idx[t] : t;

    const int slice = w % S, grp = w / S;
    const int nbs = (nb + S - 1) / S;               // <= 64
    const int b0 = slice * nbs, b1 = min(nb, b0 + nbs);
    const int npairs = W.N >> 1;
    const int stride = gridDim.x * G;
    const int first = blockIdx.x * G + grp;
    const int iters = (npairs + stride - 1) / stride;    // same for every wavefront of the grid

    // ---- code loads: D row pairs in flight per wavefront ----
    PairLoad<WT, 1> L[D];
    auto issue = [&](PairLoad<WT, 1> &dst, int it) __attribute__((always_inline)) {
        const int p = min(first + it * stride, npairs - 1);   // past the end: re-read the last pair
        int r0, r1;
        pair_rows(pair_mode, p, r0, r1);
        load_pair<WT, 1>(W, r0, r1, b0, b1, lane, dst);
    };
    // with a split K, thread i finishes item i (group, pair) after the last
    // pair: its epilogue inputs are requested now
    int fin_p = -1, fin_r0 = 0, fin_r1 = 1;
    EpiPre fin_pre;
    if (S > 1 && tid < G * iters) {
        const int g = tid / iters, it = tid % iters;
        const int p = blockIdx.x * G + g + it * stride;
        if (p < npairs) {
            fin_p = p;
            pair_rows(pair_mode, p, fin_r0, fin_r1);
            fin_pre = epi_prefetch<EPI>(ep, t, fin_r0, fin_r1);
        }
    }

    // ---- LDS image of the input row, once per block ----
    // Every input of the image is requested at once (one memory latency,
    // overlapping the first code loads): thread i builds element groups
    // i, i + 1024, ... (4 elements each); the 8 groups of a quant block sit in
    // 8 consecutive lanes.  The RMSNorm factor comes from the partial sums of
    // squares left by the kernel that wrote the row (added in slot order, the
    // same in every wavefront), else from the row itself (one barrier).
    {
        constexpr int GPT = MV_KMAX / 4 / (NW * 64);
        const int n4 = K >> 2;
        typedef _Float16 h4 __attribute__((ext_vector_type(4)));
        f4 xv[GPT], gv[GPT];
        h4 hv4[GPT], lv4[GPT];
        f4 sp = {0.f, 0.f, 0.f, 0.f};
        if (NORM && in.ss_part) sp = *(const f4 *)(in.ss_part + (size_t)xrow * SS_SLOTS + 4 * lane);
#pragma unroll
        for (int j = 0; j < GPT; j++) {
            if (j * NW * 64 >= n4) break;                 // uniform
            const int q = min(tid + j * NW * 64, n4 - 1);
            if (NORM) {
                xv[j] = *(const f4 *)(in.x32 + (size_t)xrow * in.ldx + 4 * q);
                gv[j] = *(const f4 *)(in.norm_g + 4 * q);
            } else {
                hv4[j] = *(const h4 *)(in.x16 + (size_t)xrow * in.ldx + 4 * q);
                lv4[j] = *(const h4 *)(in.x16lo + (size_t)xrow * in.ldx + 4 * q);
            }
        }
        // the first D code pairs go out after the image inputs, so that waiting
        // for the inputs (loads complete in issue order) never waits for them
#pragma unroll
        for (int k = 0; k < D; k++)
            if (k < iters) issue(L[k], k);   // (iters is the same for every wavefront)
        float rs = 0.f;
        if (NORM) {
            float ss;
            if (in.ss_part) {
                ss = wave_sum_dpp((sp[0] + sp[1]) + (sp[2] + sp[3]));
            } else {
                float loc = 0.f;
#pragma unroll
                for (int j = 0; j < GPT; j++)
                    if (tid + j * NW * 64 < n4) loc += xv[j][0] * xv[j][0] + xv[j][1] * xv[j][1] + xv[j][2] * xv[j][2] + xv[j][3] * xv[j][3];
                loc = wave_sum_dpp(loc);
                if (lane == 0) red[w] = loc;
                __syncthreads();
                ss = 0.f;
#pragma unroll
                for (int i = 0; i < NW; i++) ss += red[i];
            }
            rs = 1.0f / sqrtf(ss / (float)K + in.eps);
        }
#pragma unroll
        for (int j = 0; j < GPT; j++) {
            const int q = tid + j * NW * 64;
            if (j * NW * 64 >= n4) break;                 // uniform: no group of this round
            f16 hv[4], lv[4];
#pragma unroll
            for (int e = 0; e < 4; e++) {
                if (NORM) {
                    const float y = xv[j][e] * rs * gv[j][e];
                    hv[e] = (f16)y;
                    lv[e] = (f16)(y - (float)hv[e]);
                } else {
                    hv[e] = hv4[j][e];
                    lv[e] = lv4[j][e];
                }
            }
            float v = 0.f, pl = 0.f;
            if (q < n4) v = put_group<WT>(img, q >> 3, q & 7, hv, lv, &pl);
            v += __shfl_xor(v, 1, 64);
            v += __shfl_xor(v, 2, 64);
            v += __shfl_xor(v, 4, 64);
            if (q < n4 && (q & 7) == 0) bsum[q >> 3] = v;
            if constexpr (WT == T_Q4_K) {
                pl += __shfl_xor(pl, 1, 64);
                pl += __shfl_xor(pl, 2, 64);
                pl += __shfl_xor(pl, 4, 64);
                if (q < n4 && (q & 7) == 0) xsum[q >> 3] = pl;
            }
        }
    }
    __syncthreads();

    // ---- this lane's block of the slice -> registers ----
    const int bl = b0 + lane;
    const bool lane_ok = bl < b1;
    h2 xp[32];
    {
        const uint32_t *row = img + (size_t)(lane_ok ? bl : b0) * XROW;
#pragma unroll
        for (int j = 0; j < 8; j++) {
            u32x4 v = *(const u32x4 *)(row + 4 * j);
            if (!lane_ok) v = u32x4{0u, 0u, 0u, 0u};
            xp[4 * j] = as_h2(v.x); xp[4 * j + 1] = as_h2(v.y);
            xp[4 * j + 2] = as_h2(v.z); xp[4 * j + 3] = as_h2(v.w);
        }
    }
    const float xs = lane_ok ? bsum[bl] : 0.f;
    const float xp_sum = WT == T_Q4_K && lane_ok ? xsum[bl] : 0.f;

    // ---- stream row pairs ----
    const Masks mk = make_masks();
    float ssq = 0.f;   // RESID: sum of squares of the rows this thread finished
    auto step = [&](PairLoad<WT, 1> &cur, int it) __attribute__((always_inline)) {
        if (it >= iters) return;
        const int p = first + it * stride;
        float bd0, bd1;
        if (WT != T_Q8_0) {
            bd0 = blockdot_q4(cur.q[0][0][0], xp, mk);
            bd1 = blockdot_q4(cur.q[1][0][0], xp, mk);
        } else {
            bd0 = blockdot_q8(cur.q[0][0][0], cur.q[0][0][WT == T_Q8_0 ? 1 : 0], xp, mk);
            bd1 = blockdot_q8(cur.q[1][0][0], cur.q[1][0][WT == T_Q8_0 ? 1 : 0], xp, mk);
        }
        // (lanes past the slice hold zero activations and offset sum, and the
        // scale of a real block of the row: their products are 0)
        float a0, a1;
        if constexpr (WT == T_Q4_K) {
            // d sc (q . x) - dmin m (sum x), with q . x = bd - offsets
            const uint32_t s0 = cur.d[0][0] >> cur.dsh[0][0], s1 = cur.d[1][0] >> cur.dsh[1][0];
            const uint32_t e0 = cur.dm[0][0], e1 = cur.dm[1][0];
            a0 = f16_bits_to_f32((uint16_t)e0) * (float)(s0 & 63) * (bd0 - xs) -
                 f16_bits_to_f32((uint16_t)(e0 >> 16)) * (float)((s0 >> 8) & 63) * xp_sum;
            a1 = f16_bits_to_f32((uint16_t)e1) * (float)(s1 & 63) * (bd1 - xs) -
                 f16_bits_to_f32((uint16_t)(e1 >> 16)) * (float)((s1 >> 8) & 63) * xp_sum;
        } else {
            a0 = f16_bits_to_f32((uint16_t)(cur.d[0][0] >> cur.dsh[0][0])) * (bd0 - xs);
            a1 = f16_bits_to_f32((uint16_t)(cur.d[1][0] >> cur.dsh[1][0])) * (bd1 - xs);
        }
        // everything read from this pair's registers is consumed above the
        // refill: a use below it would wait for the refill too (loads complete
        // in issue order), which would leave one pair in flight instead of D
        __builtin_amdgcn_sched_barrier(0);
        // refill with the pair D ahead, if there is one: a load of a pair past
        // the last would re-read the grid's last pair, the same lines from
        // every wavefront
        if (it + D < iters) issue(cur, it + D);
        __builtin_amdgcn_sched_barrier(0);
        a0 = wave_sum_dpp(a0);
        a1 = wave_sum_dpp(a1);
        if (p < npairs && lane == 0) {
            if (S == 1) {
                int r0, r1;
                pair_rows(pair_mode, p, r0, r1);
                if (EPI == EPI_RESID) {
                    float *y = ep.y + (size_t)t * ep.ldy;
                    const float v0 = y[r0] + a0, v1 = y[r1] + a1;
                    y[r0] = v0;
                    y[r1] = v1;
                    ssq += v0 * v0 + v1 * v1;
                } else {
                    epi_pair<EPI>(ep, t, p, r0, r1, a0, a1);
                }
            } else {
                float *pp = part + ((grp * MV_MAXIT + it) * S + slice) * 2;
                pp[0] = a0;
                pp[1] = a1;
            }
        }
    };
    for (int it = 0; it < iters; it += D) {
#pragma unroll
        for (int k = 0; k < D; k++) step(L[k], it + k);
    }
    if (S > 1) {
        // partial sums of the S slices, added in slice order (G * iters <= the
        // block's threads: MV_MAXIT * G <= 16 * 64)
        __syncthreads();
        if (fin_p >= 0) {
            const int g = tid / iters, it = tid % iters;
            float s0 = 0.f, s1 = 0.f;
#pragma unroll
            for (int j = 0; j < S; j++) {
                s0 += part[((g * MV_MAXIT + it) * S + j) * 2];
                s1 += part[((g * MV_MAXIT + it) * S + j) * 2 + 1];
            }
            epi_pair_pre<EPI>(ep, t, fin_p, fin_r0, fin_r1, s0, s1, fin_pre);
            if (EPI == EPI_RESID) ssq += (fin_pre.y0 + s0) * (fin_pre.y0 + s0) + (fin_pre.y1 + s1) * (fin_pre.y1 + s1);
        }
    }
    if (EPI == EPI_RESID && ep.ss_out) {
        // this block's share of the new rows' sum of squares -> slot blockIdx.x
        ssq = wave_sum_dpp(ssq);           // (the residual add reads no normalized row: red[] is free)
        if (lane == 0) red[w] = ssq;
        __syncthreads();
        float *so = ep.ss_out + (size_t)t * SS_SLOTS;
        if (tid == 0) {
            float tot = 0.f;
#pragma unroll
            for (int i = 0; i < NW; i++) tot += red[i];
            so[blockIdx.x] = tot;
        }
        if (blockIdx.x == 0)
            for (int i = (int)gridDim.x + tid; i < SS_SLOTS; i += NW * 64) so[i] = 0.f;
    }
}

int g_num_cu = 256;

template <int WT, int S, int EPI>
bool launch_epi(const QMat &W, const InArgs &in, const EpiArgs &ep, int T, int pair_mode, hipStream_t s) {
    constexpr int NW = 16, G = NW / S;
    constexpr int D = WT != T_Q8_0 ? 2 : 3;   // row pairs in flight per wavefront (deeper measured slower)
    const int npairs = W.N / 2;
    int blocks = (npairs + G - 1) / G;
    if (blocks > g_num_cu) blocks = g_num_cu;
    if (blocks > SS_SLOTS) blocks = SS_SLOTS;
    if (S > 1 && (npairs + blocks * G - 1) / (blocks * G) > MV_MAXIT) return false;
    launch((k_matvec<WT, S, EPI, D>), dim3(blocks, T), dim3(NW * 64), 0, s, W, in, ep, pair_mode);
    return true;
}

template <int WT, int S>
bool launch_s(const QMat &W, const InArgs &in, const EpiArgs &ep, int T, int pair_mode, hipStream_t s) {
    switch (ep.epi) {
    case EPI_STORE: return launch_epi<WT, S, EPI_STORE>(W, in, ep, T, pair_mode, s);
    case EPI_RESID: return launch_epi<WT, S, EPI_RESID>(W, in, ep, T, pair_mode, s);
    case EPI_QKV: return launch_epi<WT, S, EPI_QKV>(W, in, ep, T, pair_mode, s);
    case EPI_SWIGLU: return launch_epi<WT, S, EPI_SWIGLU>(W, in, ep, T, pair_mode, s);
    default: return false;
    }
}

// K slices per row pair: the fewest that keep a slice within 64 blocks (one
// per lane), doubled while the grid would leave compute units idle and the
// per-wavefront pair count allows.
int slices_for(int N, int K, int num_cu) {
    const int nb = K / 32, npairs = N / 2;
    int S = 1;
    while (S * 64 < nb) S *= 2;
    while (S < 16 && (long long)npairs * S < 16LL * num_cu) S *= 2;
    return S;
}

template <int WT>
bool launch_wt(const QMat &W, const InArgs &in, const EpiArgs &ep, int T, int pair_mode, hipStream_t s) {
    if (W.K > MV_KMAX) return false;
    const int S = slices_for(W.N, W.K, g_num_cu);
    switch (S) {
    case 1: return launch_s<WT, 1>(W, in, ep, T, pair_mode, s);
    case 2: return launch_s<WT, 2>(W, in, ep, T, pair_mode, s);
    case 4: return launch_s<WT, 4>(W, in, ep, T, pair_mode, s);
    case 8: return launch_s<WT, 8>(W, in, ep, T, pair_mode, s);
    case 16: return launch_s<WT, 16>(W, in, ep, T, pair_mode, s);
    default: return false;
    }
}

}  // namespace

void matvec_set_num_cu(int n) {
    if (n > 0) g_num_cu = n;
}

int matvec_slices(int N, int K, int num_cu) { return slices_for(N, K, num_cu > 0 ? num_cu : g_num_cu); }

bool launch_matvec(const QMat &W, const InArgs &in, const EpiArgs &ep, int T, hipStream_t s) {
    if (W.K % 32 || W.N % 2 || T <= 0) return false;
    if ((in.norm_g != nullptr) != (ep.epi != EPI_RESID)) return false;
    const int pair_mode = ep.epi == EPI_SWIGLU ? PAIR_GU : PAIR_ADJ;
    if (pair_mode == PAIR_GU && W.N % 64) return false;
    if (W.wtype == T_Q4_0) return launch_wt<T_Q4_0>(W, in, ep, T, pair_mode, s);
    if (W.wtype == T_Q8_0) return launch_wt<T_Q8_0>(W, in, ep, T, pair_mode, s);
    if (W.wtype == T_Q4_K) return launch_wt<T_Q4_K>(W, in, ep, T, pair_mode, s);
    return false;
}
