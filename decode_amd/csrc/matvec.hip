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
// Q4_0 block dword i (bytes 4i..4i+3): byte k holds code 4i+k in its low
// nibble and code 16+4i+k in its high nibble.  Masking a dword with
// 0x000F000F / 0x00F000F0 and or-ing the f16 exponent of 1024 gives the f16
// pairs (1024 + q[4i], 1024 + q[4i+2]) and (1024 + 16 q[4i+16], 1024 + 16
// q[4i+18]) directly; the same masks on the dword shifted right by 8 give
// codes 4i+1, 4i+3 and 16 q[4i+17], 16 q[4i+19].  All these values are exact
// in f16.  xp[4i+0..3] hold the matching activation pairs.
DEV void pairs_q4(const f16 *x, h2 *xp) {
#pragma unroll
    for (int i = 0; i < 4; i++) {
        xp[4 * i + 0] = h2{x[4 * i + 0], x[4 * i + 2]};
        xp[4 * i + 1] = h2{x[16 + 4 * i + 0], x[16 + 4 * i + 2]};
        xp[4 * i + 2] = h2{x[4 * i + 1], x[4 * i + 3]};
        xp[4 * i + 3] = h2{x[16 + 4 * i + 1], x[16 + 4 * i + 3]};
    }
}
// Q8_0 block dword i holds codes 4i..4i+3; after flipping the sign bits,
// masks 0x00FF00FF at shifts 0 and 8 select (4i, 4i+2) and (4i+1, 4i+3).
DEV void pairs_q8(const f16 *x, h2 *xp) {
#pragma unroll
    for (int i = 0; i < 8; i++) {
        xp[2 * i + 0] = h2{x[4 * i + 0], x[4 * i + 2]};
        xp[2 * i + 1] = h2{x[4 * i + 1], x[4 * i + 3]};
    }
}

// Constants held in registers so that (w & mask) | magic issues as one
// v_and_or_b32 (these VOP3 forms cannot encode literal constants).
struct Masks {
    uint32_t lo4, hi4, lo8, flip, magic;
};
DEV Masks make_masks() {
    Masks m;
    asm volatile("s_mov_b32 %0, 0x000f000f" : "=s"(m.lo4));
    asm volatile("s_mov_b32 %0, 0x00f000f0" : "=s"(m.hi4));
    asm volatile("s_mov_b32 %0, 0x00ff00ff" : "=s"(m.lo8));
    asm volatile("s_mov_b32 %0, 0x80808080" : "=s"(m.flip));
    asm volatile("v_mov_b32 %0, 0x64006400" : "=v"(m.magic));
    return m;
}

// The activations enter as two f16 parts, x = hi + lo (lo = the f16 rounding
// of x - hi), so a product uses x to about 22 significant bits: xp[0..15] are
// the hi pairs, xp[16..31] the lo pairs.
//
// Returns sum_A (1024 + q) x + sum_B (1024 + 16 q) x / 16 over the block, where
// A are the low-nibble codes 0..15 and B the high-nibble codes 16..31.
DEV float blockdot_q4(const uint4 q, const h2 *xp, const Masks &m) {
    const uint32_t w[4] = {q.x, q.y, q.z, q.w};
    float a = 0.f, b = 0.f;
#pragma unroll
    for (int i = 0; i < 4; i++) {
        const uint32_t w8 = w[i] >> 8;
        const h2 c0 = as_h2((w[i] & m.lo4) | m.magic), c1 = as_h2((w[i] & m.hi4) | m.magic);
        const h2 c2 = as_h2((w8 & m.lo4) | m.magic), c3 = as_h2((w8 & m.hi4) | m.magic);
        a = dot2(c0, xp[4 * i + 0], a);
        b = dot2(c1, xp[4 * i + 1], b);
        a = dot2(c2, xp[4 * i + 2], a);
        b = dot2(c3, xp[4 * i + 3], b);
        a = dot2(c0, xp[16 + 4 * i + 0], a);
        b = dot2(c1, xp[16 + 4 * i + 1], b);
        a = dot2(c2, xp[16 + 4 * i + 2], a);
        b = dot2(c3, xp[16 + 4 * i + 3], b);
    }
    return a + b * 0.0625f;
}

// Returns sum (1024 + 128 + q) x over the block.
DEV float blockdot_q8(const uint4 q0, const uint4 q1, const h2 *xp, const Masks &m) {
    const uint32_t w[8] = {q0.x, q0.y, q0.z, q0.w, q1.x, q1.y, q1.z, q1.w};
    float acc = 0.f;
#pragma unroll
    for (int i = 0; i < 8; i++) {
        const uint32_t u = w[i] ^ m.flip;
        const h2 c0 = as_h2((u & m.lo8) | m.magic), c1 = as_h2(((u >> 8) & m.lo8) | m.magic);
        acc = dot2(c0, xp[2 * i + 0], acc);
        acc = dot2(c1, xp[2 * i + 1], acc);
        acc = dot2(c0, xp[16 + 2 * i + 0], acc);
        acc = dot2(c1, xp[16 + 2 * i + 1], acc);
    }
    return acc;
}

constexpr int MV_KMAX = 16384;   // longest input row (elements) staged in LDS

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
DEV float dot_row(const PairLoad<WT, KB> &L, int r, const h2 (*xp)[32], const float *xsum,
                  const Masks &m) {
    float a = 0.f;
#pragma unroll
    for (int i = 0; i < KB; i++) {
        float bd;
        if (WT == T_Q4_0)
            bd = blockdot_q4(L.q[r][i][0], xp[i], m);
        else
            bd = blockdot_q8(L.q[r][i][0], L.q[r][i][WT == T_Q4_0 ? 0 : 1], xp[i], m);
        a += f16_bits_to_f32(L.d[r][i]) * (bd - xsum[i]);
    }
    return a;
}

// NW wavefronts per block (one block per CU).  The K dimension is cut into S
// slices of at most 128 blocks; S wavefronts share one row pair, each
// covering one slice with at most 2 blocks per lane whose activations it
// keeps in registers.  An f16 input row is read straight into registers; an
// f32 residual row to be RMS-normalized is normalized once per block into LDS.  Row pairs p = g, g + G, ... are
// streamed with the next pair's loads in flight while the current pair is
// reduced (DPP within the wavefront; for S > 1 the S partial sums meet in
// double-buffered LDS and are added in slice order).
template <int WT, int KB, int S, int EPI>
__global__ __launch_bounds__(1024) void k_matvec(QMat W, InArgs in, EpiArgs ep, int pair_mode) {
    constexpr int NW = 16, G = NW / S;
    // normalized input: staged through LDS (registers would not hold the row)
    constexpr int XS = EPI == EPI_RESID ? 8 : (S * KB * 64 * 32 < MV_KMAX ? S * KB * 64 * 32 : MV_KMAX);
    __shared__ __attribute__((aligned(16))) f16 xs[XS];
    __shared__ __attribute__((aligned(16))) f16 xsl[XS];
    __shared__ float red[NW];
    __shared__ float part[2][NW][2];
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int t = blockIdx.y;
    const int K = W.K, nb = K >> 5;
    const int xrow = in.row_idx ? in.row_idx[t] : t;

    const int slice = w % S, grp = w / S;
    const int nbs = (nb + S - 1) / S;
    const int b0 = slice * nbs, b1 = min(nb, b0 + nbs);
    const int npairs = W.N >> 1;
    const int stride = gridDim.x * G;
    const int first = blockIdx.x * G + grp;
    const int iters = (npairs + stride - 1) / stride;    // same for every wavefront of the grid
    int p = first, r0 = 0, r1 = 1;

    // ---- this wavefront's K slice of the activations -> f16 pairs in registers.
    //      With a norm, the wavefront also reads the rest of the row for the sum
    //      of squares: no LDS and no block barrier on the way in. ----
    // every epilogue except the residual add reads a normalized row
    constexpr bool NORM = EPI != EPI_RESID;
    f16 xv[KB][32], xl[KB][32];
    if (NORM) {
        const float *xr = in.x32 + (size_t)xrow * in.ldx;
        const int tid = threadIdx.x;
        float ss = 0.f;
        for (int k = tid * 4; k < K; k += NW * 256) {
            const float4 v = *(const float4 *)(xr + k);
            ss += v.x * v.x + v.y * v.y + v.z * v.z + v.w * v.w;
        }
        ss = wave_sum_dpp(ss);
        if (lane == 0) red[w] = ss;
        __syncthreads();
        float tot = 0.f;
#pragma unroll
        for (int i = 0; i < NW; i++) tot += red[i];
        const float rs = 1.0f / sqrtf(tot / (float)K + in.eps);
        for (int k = tid * 4; k < K; k += NW * 256) {
            const float4 v = *(const float4 *)(xr + k);
            const float4 g = *(const float4 *)(in.norm_g + k);
            const float y[4] = {v.x * rs * g.x, v.y * rs * g.y, v.z * rs * g.z, v.w * rs * g.w};
            f16 hi[4], lo[4];
#pragma unroll
            for (int e = 0; e < 4; e++) {
                hi[e] = (f16)y[e];
                lo[e] = (f16)(y[e] - (float)hi[e]);
            }
            *(uint2 *)&xs[k] = *(const uint2 *)hi;
            *(uint2 *)&xsl[k] = *(const uint2 *)lo;
        }
        __syncthreads();
#pragma unroll
        for (int i = 0; i < KB; i++) {
            const int b = b0 + lane + 64 * i;
#pragma unroll
            for (int j = 0; j < 4; j++) {
                uint4 v = make_uint4(0, 0, 0, 0), vl = v;
                if (b < b1) {
                    v = *(const uint4 *)&xs[b * 32 + 8 * j];
                    vl = *(const uint4 *)&xsl[b * 32 + 8 * j];
                }
                *(uint4 *)&xv[i][8 * j] = v;
                *(uint4 *)&xl[i][8 * j] = vl;
            }
        }
    } else {
        const uint16_t *xr = in.x16 + (size_t)xrow * in.ldx;
        const uint16_t *xrl = in.x16lo + (size_t)xrow * in.ldx;
#pragma unroll
        for (int i = 0; i < KB; i++) {
            const int b = b0 + lane + 64 * i;
#pragma unroll
            for (int j = 0; j < 4; j++) {
                uint4 v = make_uint4(0, 0, 0, 0), vl = v;
                if (b < b1) {
                    v = *(const uint4 *)(xr + b * 32 + 8 * j);
                    vl = *(const uint4 *)(xrl + b * 32 + 8 * j);
                }
                *(uint4 *)&xv[i][8 * j] = v;
                *(uint4 *)&xl[i][8 * j] = vl;
            }
        }
    }
    h2 xp[KB][32];
    float xsum[KB];
#pragma unroll
    for (int i = 0; i < KB; i++) {
        // offsets removed once per block: Q4_0 keeps 1024 + q on codes 0..15 and
        // (1024 + 16 q) / 16 on codes 16..31, so sum (q - 8) x needs
        // 1032 * sum(x[0..15]) + 72 * sum(x[16..31]) subtracted; Q8_0 keeps
        // 1024 + 128 + q everywhere.
        float s_lo = 0.f, s_hi = 0.f;
#pragma unroll
        for (int j = 0; j < 16; j++) {
            s_lo += (float)xv[i][j] + (float)xl[i][j];
            s_hi += (float)xv[i][16 + j] + (float)xl[i][16 + j];
        }
        xsum[i] = WT == T_Q4_0 ? 1032.f * s_lo + 72.f * s_hi : 1152.f * (s_lo + s_hi);
        if (WT == T_Q4_0) {
            pairs_q4(xv[i], xp[i]);
            pairs_q4(xl[i], xp[i] + 16);
        } else {
            pairs_q8(xv[i], xp[i]);
            pairs_q8(xl[i], xp[i] + 16);
        }
    }

    // ---- stream row pairs ----
    const Masks mk = make_masks();
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
            a0 = wave_sum_dpp(dot_row<WT, KB>(cur, 0, xp, xsum, mk));
            a1 = wave_sum_dpp(dot_row<WT, KB>(cur, 1, xp, xsum, mk));
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
    constexpr int NW = 16, G = NW / S;
    const int npairs = W.N / 2;
    int blocks = (npairs + G - 1) / G;
    if (blocks > g_num_cu) blocks = g_num_cu;
    launch((k_matvec<WT, KB, S, EPI>), dim3(blocks, T), dim3(NW * 64), 0, s, W, in, ep,
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

template <int WT, int KB>
bool launch_kb(int S, const QMat &W, const InArgs &in, const EpiArgs &ep, int T, int pair_mode,
               hipStream_t s) {
    switch (S) {
    case 1: return launch_ks<WT, KB, 1>(W, in, ep, T, pair_mode, s);
    case 2: return launch_ks<WT, KB, 2>(W, in, ep, T, pair_mode, s);
    case 4: return launch_ks<WT, KB, 4>(W, in, ep, T, pair_mode, s);
    case 8: return launch_ks<WT, KB, 8>(W, in, ep, T, pair_mode, s);
    case 16: return launch_ks<WT, KB, 16>(W, in, ep, T, pair_mode, s);
    default: return false;
    }
}

// K slices per row pair: enough that a lane holds at most 2 blocks, and more
// while the grid would otherwise leave compute units idle.
template <int WT>
bool launch_wt(const QMat &W, const InArgs &in, const EpiArgs &ep, int T, int pair_mode,
               hipStream_t s) {
    const int nb = W.K / 32, npairs = W.N / 2;
    const int slice_max = WT == T_Q8_0 ? 64 : 128;   // blocks per K slice (registers)
    if (nb > 16 * slice_max) return false;
    int S = 1;
    while (S * slice_max < nb) S *= 2;
    while (S < 16 && (long long)npairs * S < 16LL * g_num_cu) S *= 2;
    if (ep.epi != EPI_RESID && W.K > MV_KMAX) return false;
    const int nbs = (nb + S - 1) / S;
    if (WT == T_Q8_0 || nbs <= 64) return launch_kb<WT, 1>(S, W, in, ep, T, pair_mode, s);
    return launch_kb<T_Q4_0, 2>(S, W, in, ep, T, pair_mode, s);
}

}  // namespace

void matvec_set_num_cu(int n) {
    if (n > 0) g_num_cu = n;
}

bool launch_matvec(const QMat &W, const InArgs &in, const EpiArgs &ep, int T, hipStream_t s) {
    if (W.K % 32 || W.N % 2 || T <= 0) return false;
    if ((in.norm_g != nullptr) != (ep.epi != EPI_RESID)) return false;
    const int pair_mode = ep.epi == EPI_SWIGLU ? PAIR_GU : PAIR_ADJ;
    if (pair_mode == PAIR_GU && W.N % 64) return false;
    if (W.wtype == T_Q4_0) return launch_wt<T_Q4_0>(W, in, ep, T, pair_mode, s);
    if (W.wtype == T_Q8_0) return launch_wt<T_Q8_0>(W, in, ep, T, pair_mode, s);
    return false;
}
