// gemm.hip -- ubatch GEMM Y = X W^T for prefill and batched decode (gfx950).
//
// MFMA path (Q8_0 / Q4_0 weights).  The arithmetic is exact up to fp32
// accumulation: weights enter the matrix cores as their integer codes (q - 8
// for Q4_0, q for Q8_0; exact in f16) and the activations as two f16 parts
// x = hi + lo (lo = f16 rounding remainder of x), so every product is exact.
// For each 32-wide quant block the four v_mfma_f32_32x32x16_f16 of a tile
// (2 k-halves x hi/lo) accumulate into a temporary tile that is then scaled
// by the row's block scale and added to the fp32 result: C += d[n][kb] * T.
//
// A 256-thread block computes 128 output features x BM tokens; each
// wavefront owns a 64 x BM/2 sub-tile.  Codes, activations and scales of a
// K block are staged in LDS with two stages, so one barrier per K block
// suffices: the next block's global loads are in flight during the MFMAs and
// land in the other stage afterwards.  Blocks that share a weight tile are
// placed on the same XCD (block ids go round-robin over the 8 XCDs), so the
// tile is fetched from HBM once into that XCD's L2.
// Operand layouts (checked on the device): lane l supplies A[l%32][8(l/32)+e]
// and B[8(l/32)+e][l%32]; accumulator r of lane l is C[(r/4)*8+(l/32)*4+r%4][l%32].
// A is the code tile (rows = features), B the activations transposed
// (columns = tokens), so a lane's accumulators are four runs of 4
// consecutive features of one token -- RoPE pairs and gate/up pairs meet in
// one lane and the shared epilogue applies directly.
//
// Fallback path (fp32 weights, or shapes the MFMA tiling does not cover):
// one thread per (row pair, token), plain fp32 FMA.
#include "common.h"
#include "epilogue.h"
#include "kernels.h"

namespace {

constexpr int BN = 128;
constexpr int LDS_STRIDE = 40;   // f16 elements per LDS row (32 + 8 pad)

// 16 codes (half `hb` of a 32-weight block) as exact f16 values.
template <int WT>
DEV void codes16(uint4 raw, int hb, h2 *out) {
    const uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};
    if (WT == T_Q4_0) {
        // codes 16*hb .. 16*hb+15: low (hb=0) or high (hb=1) nibbles of bytes 0..15
        const h2 off = h2{(f16)1032.f, (f16)1032.f};
#pragma unroll
        for (int i = 0; i < 4; i++) {
            const uint32_t m = (w[i] >> (4 * hb)) & 0x0F0F0F0Fu;
            const uint32_t p0 = (m & 0x000000FFu) | ((m << 8) & 0x00FF0000u);
            const uint32_t p1 = ((m >> 16) & 0x000000FFu) | ((m >> 8) & 0x00FF0000u);
            out[2 * i + 0] = as_h2(p0 | 0x64006400u) - off;
            out[2 * i + 1] = as_h2(p1 | 0x64006400u) - off;
        }
    } else {
        // codes 16*hb .. 16*hb+15 are the bytes of raw (signed)
        const h2 off = h2{(f16)1152.f, (f16)1152.f};
#pragma unroll
        for (int i = 0; i < 4; i++) {
            const uint32_t u = w[i] ^ 0x80808080u;
            const uint32_t p0 = (u & 0x000000FFu) | ((u << 8) & 0x00FF0000u);
            const uint32_t p1 = ((u >> 16) & 0x000000FFu) | ((u >> 8) & 0x00FF0000u);
            out[2 * i + 0] = as_h2(p0 | 0x64006400u) - off;
            out[2 * i + 1] = as_h2(p1 | 0x64006400u) - off;
        }
    }
}

template <int WT, int BM, int EPI>
__global__ __launch_bounds__(256, 2) void k_gemm_mfma(QMat W, const uint16_t *Xh, const uint16_t *Xl,
                                                      int ldx, EpiArgs ep, int M, int pair_mode, int NT) {
    constexpr int MT = BM / 64;   // 32x32 m-tiles per wavefront
    __shared__ __attribute__((aligned(16))) f16 As[2][BN * LDS_STRIDE];
    __shared__ __attribute__((aligned(16))) f16 Bh[2][BM * LDS_STRIDE];
    __shared__ __attribute__((aligned(16))) f16 Bl[2][BM * LDS_STRIDE];
    __shared__ __attribute__((aligned(16))) float Sc[2][BN];

    // block -> (feature tile, token tile); tiles of one feature tile share an XCD
    const int mtiles = (M + BM - 1) / BM;
    const int L = blockIdx.x, xcd = L & 7, j = L >> 3;
    const int nt = (j / mtiles) * 8 + xcd, mtile = j % mtiles;
    if (nt >= NT) return;

    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int n0 = nt * BN, m0 = mtile * BM;
    const int K = W.K, nb = K >> 5;
    const int wn = (w & 1) * 64, wm = (w >> 1) * (BM / 2);

    // loader roles
    const int a_row = tid >> 1, a_half = tid & 1;      // one half-block of one weight row
    constexpr int XCH = BM * 4;                         // 16-byte chunks of one activation tile
    constexpr int XPT = (XCH + 255) / 256;              // chunks per thread (per part)
    const size_t qrow_bytes = WT == T_Q4_0 ? (size_t)(K >> 1) : (size_t)K;
    const uint8_t *qbase = (const uint8_t *)W.qs + (size_t)(n0 + a_row) * qrow_bytes;
    const uint16_t *dbase = W.d + (size_t)(n0 + a_row) * nb;

    uint4 araw;
    uint16_t adb;
    uint4 xh[XPT], xl[XPT];
    auto gload = [&](int kb) {
        if (WT == T_Q4_0)
            araw = *(const uint4 *)(qbase + (size_t)kb * 16);
        else
            araw = *(const uint4 *)(qbase + (size_t)kb * 32 + a_half * 16);
        adb = dbase[kb];
#pragma unroll
        for (int c = 0; c < XPT; c++) {
            const int ch = tid + c * 256;
            const int mr = ch >> 2, kc = ch & 3;
            if (ch < XCH && m0 + mr < M) {
                const size_t off = (size_t)(m0 + mr) * ldx + kb * 32 + kc * 8;
                xh[c] = *(const uint4 *)(Xh + off);
                xl[c] = *(const uint4 *)(Xl + off);
            } else {
                xh[c] = xl[c] = make_uint4(0, 0, 0, 0);
            }
        }
    };
    auto lstore = [&](int st) {
        h2 v[8];
        codes16<WT>(araw, a_half, v);
        uint4 *dst = (uint4 *)(&As[st][a_row * LDS_STRIDE + a_half * 16]);
        dst[0] = __builtin_bit_cast(uint4, *(h8 *)&v[0]);
        dst[1] = __builtin_bit_cast(uint4, *(h8 *)&v[4]);
        if (a_half == 0) Sc[st][a_row] = f16_bits_to_f32(adb);
#pragma unroll
        for (int c = 0; c < XPT; c++) {
            const int ch = tid + c * 256;
            if (ch < XCH) {
                const int mr = ch >> 2, kc = ch & 3;
                *(uint4 *)(&Bh[st][mr * LDS_STRIDE + kc * 8]) = xh[c];
                *(uint4 *)(&Bl[st][mr * LDS_STRIDE + kc * 8]) = xl[c];
            }
        }
    };

    f16x acc[2][MT];
#pragma unroll
    for (int a = 0; a < 2; a++)
#pragma unroll
        for (int b = 0; b < MT; b++)
#pragma unroll
            for (int r = 0; r < 16; r++) acc[a][b][r] = 0.f;

    gload(0);
    lstore(0);
    __syncthreads();
    for (int kb = 0; kb < nb; kb++) {
        const int st = kb & 1;
        if (kb + 1 < nb) gload(kb + 1);
        f16x tmp[2][MT];
#pragma unroll
        for (int a = 0; a < 2; a++)
#pragma unroll
            for (int b = 0; b < MT; b++)
#pragma unroll
                for (int r = 0; r < 16; r++) tmp[a][b][r] = 0.f;
#pragma unroll
        for (int kk = 0; kk < 32; kk += 16) {
            h8 af[2], bh[MT], bl[MT];
#pragma unroll
            for (int a = 0; a < 2; a++)
                af[a] = *(const h8 *)(&As[st][(wn + 32 * a + (lane & 31)) * LDS_STRIDE + kk + 8 * (lane >> 5)]);
#pragma unroll
            for (int b = 0; b < MT; b++) {
                const int off = (wm + 32 * b + (lane & 31)) * LDS_STRIDE + kk + 8 * (lane >> 5);
                bh[b] = *(const h8 *)(&Bh[st][off]);
                bl[b] = *(const h8 *)(&Bl[st][off]);
            }
#pragma unroll
            for (int a = 0; a < 2; a++)
#pragma unroll
                for (int b = 0; b < MT; b++) {
                    tmp[a][b] = __builtin_amdgcn_mfma_f32_32x32x16_f16(af[a], bh[b], tmp[a][b], 0, 0, 0);
                    tmp[a][b] = __builtin_amdgcn_mfma_f32_32x32x16_f16(af[a], bl[b], tmp[a][b], 0, 0, 0);
                }
        }
        // C += d[n][kb] * T: the lane's 16 rows of n-tile a are four runs of 4
#pragma unroll
        for (int a = 0; a < 2; a++) {
            float sc[16];
#pragma unroll
            for (int r4 = 0; r4 < 4; r4++) {
                const float4 v = *(const float4 *)(&Sc[st][wn + 32 * a + r4 * 8 + (lane >> 5) * 4]);
                sc[4 * r4 + 0] = v.x; sc[4 * r4 + 1] = v.y; sc[4 * r4 + 2] = v.z; sc[4 * r4 + 3] = v.w;
            }
#pragma unroll
            for (int b = 0; b < MT; b++)
#pragma unroll
                for (int r = 0; r < 16; r++) acc[a][b][r] += sc[r] * tmp[a][b][r];
        }
        if (kb + 1 < nb) lstore(st ^ 1);
        __syncthreads();
    }

    // ---- epilogue ----
#pragma unroll
    for (int b = 0; b < MT; b++) {
        const int m = m0 + wm + 32 * b + (lane & 31);
        if (m >= M) continue;
        if (pair_mode == PAIR_GU) {
            // wavefront covers 64 stored rows = 32 gate rows then their 32 up rows
            const int g = (n0 + wn) >> 6;
#pragma unroll
            for (int r = 0; r < 16; r++) {
                const int i = (r >> 2) * 8 + (lane >> 5) * 4 + (r & 3);
                const int r0 = ((g << 6) + i);
                epi_pair<EPI>(ep, m, (g << 5) + i, r0, r0 + 32, acc[0][b][r], acc[1][b][r]);
            }
        } else {
#pragma unroll
            for (int a = 0; a < 2; a++)
#pragma unroll
                for (int r = 0; r < 16; r += 2) {
                    const int n = n0 + wn + 32 * a + (r >> 2) * 8 + (lane >> 5) * 4 + (r & 3);
                    epi_pair<EPI>(ep, m, n >> 1, n, n + 1, acc[a][b][r], acc[a][b][r + 1]);
                }
        }
    }
}

// fp32 weights (any K), f16 activations; one thread per (row pair, token).
template <int EPI>
__global__ __launch_bounds__(256) void k_gemm_f32(QMat W, const uint16_t *X, const uint16_t *Xl,
                                                  int ldx, EpiArgs ep, int M, int pair_mode) {
    const int p = blockIdx.x * 256 + threadIdx.x;
    const int m = blockIdx.y;
    if (p >= W.N / 2 || m >= M) return;
    int r0, r1;
    pair_rows(pair_mode, p, r0, r1);
    const float *w0 = (const float *)W.qs + (size_t)r0 * W.K;
    const float *w1 = (const float *)W.qs + (size_t)r1 * W.K;
    const f16 *x = (const f16 *)X + (size_t)m * ldx;
    const f16 *xl = (const f16 *)Xl + (size_t)m * ldx;
    float a = 0.f, b = 0.f;
    for (int k = 0; k < W.K; k++) {
        const float xv = (float)x[k] + (float)xl[k];
        a += w0[k] * xv;
        b += w1[k] * xv;
    }
    epi_pair<EPI>(ep, m, p, r0, r1, a, b);
}

template <int WT, int EPI>
void launch_mfma_epi(const QMat &W, const uint16_t *Xh, const uint16_t *Xl, int ldx, const EpiArgs &ep,
                     int M, int pair_mode, hipStream_t s) {
    const int NT = W.N / BN, NT8 = (NT + 7) / 8 * 8;
    if (M > 64) {
        const int mt = (M + 127) / 128;
        hipLaunchKernelGGL((k_gemm_mfma<WT, 128, EPI>), dim3(NT8 * mt), dim3(256), 0, s, W, Xh, Xl, ldx,
                           ep, M, pair_mode, NT);
    } else {
        const int mt = (M + 63) / 64;
        hipLaunchKernelGGL((k_gemm_mfma<WT, 64, EPI>), dim3(NT8 * mt), dim3(256), 0, s, W, Xh, Xl, ldx,
                           ep, M, pair_mode, NT);
    }
}

template <int WT>
void launch_mfma(const QMat &W, const uint16_t *Xh, const uint16_t *Xl, int ldx, const EpiArgs &ep,
                 int M, int pair_mode, hipStream_t s) {
    switch (ep.epi) {
    case EPI_STORE: launch_mfma_epi<WT, EPI_STORE>(W, Xh, Xl, ldx, ep, M, pair_mode, s); break;
    case EPI_RESID: launch_mfma_epi<WT, EPI_RESID>(W, Xh, Xl, ldx, ep, M, pair_mode, s); break;
    case EPI_QKV: launch_mfma_epi<WT, EPI_QKV>(W, Xh, Xl, ldx, ep, M, pair_mode, s); break;
    case EPI_SWIGLU: launch_mfma_epi<WT, EPI_SWIGLU>(W, Xh, Xl, ldx, ep, M, pair_mode, s); break;
    }
}

template <int EPI>
void launch_f32_epi(const QMat &W, const uint16_t *Xh, const uint16_t *Xl, int ldx, const EpiArgs &ep,
                    int M, int pair_mode, hipStream_t s) {
    hipLaunchKernelGGL(k_gemm_f32<EPI>, dim3((W.N / 2 + 255) / 256, M), dim3(256), 0, s, W, Xh, Xl, ldx,
                       ep, M, pair_mode);
}

}  // namespace

bool launch_gemm(const QMat &W, const uint16_t *Xh, const uint16_t *Xl, int ldx, const EpiArgs &ep,
                 int M, hipStream_t s) {
    if (M <= 0 || W.N % 2 || !Xh || !Xl) return false;
    const int pair_mode = ep.epi == EPI_SWIGLU ? PAIR_GU : PAIR_ADJ;
    if (pair_mode == PAIR_GU && W.N % 64) return false;
    if ((W.wtype == T_Q4_0 || W.wtype == T_Q8_0) && W.N % BN == 0 && W.K % 32 == 0 && ldx % 8 == 0) {
        if (W.wtype == T_Q4_0)
            launch_mfma<T_Q4_0>(W, Xh, Xl, ldx, ep, M, pair_mode, s);
        else
            launch_mfma<T_Q8_0>(W, Xh, Xl, ldx, ep, M, pair_mode, s);
        return true;
    }
    if (W.wtype != T_F32) return false;
    switch (ep.epi) {
    case EPI_STORE: launch_f32_epi<EPI_STORE>(W, Xh, Xl, ldx, ep, M, pair_mode, s); break;
    case EPI_RESID: launch_f32_epi<EPI_RESID>(W, Xh, Xl, ldx, ep, M, pair_mode, s); break;
    case EPI_QKV: launch_f32_epi<EPI_QKV>(W, Xh, Xl, ldx, ep, M, pair_mode, s); break;
    case EPI_SWIGLU: launch_f32_epi<EPI_SWIGLU>(W, Xh, Xl, ldx, ep, M, pair_mode, s); break;
    default: return false;
    }
    return true;
}
