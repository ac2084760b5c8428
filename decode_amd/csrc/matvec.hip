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

template <int WT, int KB, int PU, int EPI>
__global__ __launch_bounds__(256) void k_matvec(QMat W, InArgs in, EpiArgs ep, int pair_mode,
                                                int pairs_per_wave) {
    __shared__ float red[4];
    const int lane = threadIdx.x & 63;
    const int t = blockIdx.y;
    const int K = W.K, nb = K >> 5;
    const int xrow = in.row_idx ? in.row_idx[t] : t;

    // ---- activations of this lane's blocks -> f16 pairs in registers ----
    float rstd = 1.f;
    if (in.norm_g) {
        const float *xr = in.x32 + (size_t)xrow * in.ldx;
        float ss = 0.f;
        for (int k = threadIdx.x * 4; k < K; k += 1024) {
            const float4 v = *(const float4 *)(xr + k);
            ss += v.x * v.x + v.y * v.y + v.z * v.z + v.w * v.w;
        }
        ss = block_sum256(ss, red);
        rstd = 1.0f / sqrtf(ss / (float)K + in.eps);
    }
    h2 xp[KB][16];
    float xsum[KB];
#pragma unroll
    for (int i = 0; i < KB; i++) {
        const int b = lane + 64 * i;
        f16 xv[32];
        if (b < nb) {
            if (in.norm_g) {
                const float *xr = in.x32 + (size_t)xrow * in.ldx + b * 32;
                const float *g = in.norm_g + b * 32;
#pragma unroll
                for (int j = 0; j < 32; j += 4) {
                    const float4 v = *(const float4 *)(xr + j);
                    const float4 gg = *(const float4 *)(g + j);
                    xv[j + 0] = (f16)(v.x * rstd * gg.x);
                    xv[j + 1] = (f16)(v.y * rstd * gg.y);
                    xv[j + 2] = (f16)(v.z * rstd * gg.z);
                    xv[j + 3] = (f16)(v.w * rstd * gg.w);
                }
            } else {
                const uint4 *xr = (const uint4 *)(in.x16 + (size_t)xrow * in.ldx + b * 32);
#pragma unroll
                for (int j = 0; j < 4; j++) {
                    const uint4 v = xr[j];
                    *(uint4 *)&xv[8 * j] = v;
                }
            }
        } else {
#pragma unroll
            for (int j = 0; j < 32; j++) xv[j] = (f16)0.f;
        }
        float s = 0.f;
#pragma unroll
        for (int j = 0; j < 32; j++) s += (float)xv[j];
        xsum[i] = s * (WT == T_Q4_0 ? 1032.f : 1152.f);
        if (WT == T_Q4_0)
            pairs_q4(xv, xp[i]);
        else
            pairs_q8(xv, xp[i]);
    }

    // ---- rows ----
    const int wave = blockIdx.x * 4 + (threadIdx.x >> 6);
    const int npairs = W.N >> 1;
    const int pbeg = wave * pairs_per_wave;
    const int pend = min(npairs, pbeg + pairs_per_wave);
    for (int p0 = pbeg; p0 < pend; p0 += PU) {
        int rows[2 * PU];
#pragma unroll
        for (int u = 0; u < PU; u++) {
            const int p = min(p0 + u, pend - 1);
            pair_rows(pair_mode, p, rows[2 * u], rows[2 * u + 1]);
        }
        float acc[2 * PU];
        if (WT == T_Q4_0) {
            uint4 q[2 * PU][KB];
            uint16_t dsc[2 * PU][KB];
#pragma unroll
            for (int r = 0; r < 2 * PU; r++) {
                const uint4 *qr = (const uint4 *)((const uint8_t *)W.qs + (size_t)rows[r] * (K >> 1));
                const uint16_t *dr = W.d + (size_t)rows[r] * nb;
#pragma unroll
                for (int i = 0; i < KB; i++) {
                    const int b = lane + 64 * i;
                    if (b < nb) {
                        q[r][i] = load_stream16(qr + b);
                        dsc[r][i] = dr[b];
                    } else {
                        q[r][i] = make_uint4(0, 0, 0, 0);
                        dsc[r][i] = 0;
                    }
                }
            }
#pragma unroll
            for (int r = 0; r < 2 * PU; r++) {
                float a = 0.f;
#pragma unroll
                for (int i = 0; i < KB; i++)
                    a += f16_bits_to_f32(dsc[r][i]) * (blockdot_q4(q[r][i], xp[i]) - xsum[i]);
                acc[r] = a;
            }
        } else {
            uint4 q[2 * PU][KB][2];
            uint16_t dsc[2 * PU][KB];
#pragma unroll
            for (int r = 0; r < 2 * PU; r++) {
                const uint4 *qr = (const uint4 *)((const int8_t *)W.qs + (size_t)rows[r] * K);
                const uint16_t *dr = W.d + (size_t)rows[r] * nb;
#pragma unroll
                for (int i = 0; i < KB; i++) {
                    const int b = lane + 64 * i;
                    if (b < nb) {
                        q[r][i][0] = load_stream16(qr + 2 * b);
                        q[r][i][1] = load_stream16(qr + 2 * b + 1);
                        dsc[r][i] = dr[b];
                    } else {
                        q[r][i][0] = q[r][i][1] = make_uint4(0, 0, 0, 0);
                        dsc[r][i] = 0;
                    }
                }
            }
#pragma unroll
            for (int r = 0; r < 2 * PU; r++) {
                float a = 0.f;
#pragma unroll
                for (int i = 0; i < KB; i++)
                    a += f16_bits_to_f32(dsc[r][i]) * (blockdot_q8(q[r][i][0], q[r][i][1], xp[i]) - xsum[i]);
                acc[r] = a;
            }
        }
#pragma unroll
        for (int r = 0; r < 2 * PU; r++) acc[r] = wave_sum(acc[r]);
#pragma unroll
        for (int u = 0; u < PU; u++) {
            if (lane == u && p0 + u < pend)
                epi_pair<EPI>(ep, t, p0 + u, rows[2 * u], rows[2 * u + 1], acc[2 * u], acc[2 * u + 1]);
        }
    }
}

template <int WT, int KB, int EPI>
bool launch_epi(const QMat &W, const InArgs &in, const EpiArgs &ep, int T, int pair_mode,
                hipStream_t s) {
    constexpr int PU = KB >= 5 ? 1 : 2;
    const int npairs = W.N / 2;
    // aim for about 8 wavefronts per CU on 256 CUs
    const int target_waves = 2048;
    int ppw = (npairs + target_waves - 1) / target_waves;
    ppw = ((ppw + PU - 1) / PU) * PU;
    const int waves = (npairs + ppw - 1) / ppw;
    const int blocks = (waves + 3) / 4;
    hipLaunchKernelGGL((k_matvec<WT, KB, PU, EPI>), dim3(blocks, T), dim3(256), 0, s, W, in, ep,
                       pair_mode, ppw);
    return true;
}

template <int WT, int KB>
bool launch_kb(const QMat &W, const InArgs &in, const EpiArgs &ep, int T, int pair_mode,
               hipStream_t s) {
    switch (ep.epi) {
    case EPI_STORE: return launch_epi<WT, KB, EPI_STORE>(W, in, ep, T, pair_mode, s);
    case EPI_RESID: return launch_epi<WT, KB, EPI_RESID>(W, in, ep, T, pair_mode, s);
    case EPI_QKV: return launch_epi<WT, KB, EPI_QKV>(W, in, ep, T, pair_mode, s);
    case EPI_SWIGLU: return launch_epi<WT, KB, EPI_SWIGLU>(W, in, ep, T, pair_mode, s);
    default: return false;
    }
}

template <int WT>
bool launch_wt(const QMat &W, const InArgs &in, const EpiArgs &ep, int T, int pair_mode,
               hipStream_t s) {
    const int nb = W.K / 32;
    const int kb = (nb + 63) / 64;
    switch (kb) {
    case 1: return launch_kb<WT, 1>(W, in, ep, T, pair_mode, s);
    case 2: return launch_kb<WT, 2>(W, in, ep, T, pair_mode, s);
    case 3: return launch_kb<WT, 3>(W, in, ep, T, pair_mode, s);
    case 4: return launch_kb<WT, 4>(W, in, ep, T, pair_mode, s);
    case 5: return launch_kb<WT, 5>(W, in, ep, T, pair_mode, s);
    case 6: return launch_kb<WT, 6>(W, in, ep, T, pair_mode, s);
    case 7: return launch_kb<WT, 7>(W, in, ep, T, pair_mode, s);
    case 8: return launch_kb<WT, 8>(W, in, ep, T, pair_mode, s);
    default: return false;
    }
}

}  // namespace

bool launch_matvec(const QMat &W, const InArgs &in, const EpiArgs &ep, int T, hipStream_t s) {
    if (W.K % 32 || W.N % 2 || T <= 0) return false;
    const int pair_mode = ep.epi == EPI_SWIGLU ? PAIR_GU : PAIR_ADJ;
    if (pair_mode == PAIR_GU && W.N % 64) return false;
    if (W.wtype == T_Q4_0) return launch_wt<T_Q4_0>(W, in, ep, T, pair_mode, s);
    if (W.wtype == T_Q8_0) return launch_wt<T_Q8_0>(W, in, ep, T, pair_mode, s);
    return false;
}
