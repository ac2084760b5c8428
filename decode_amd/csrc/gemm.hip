// gemm.hip -- ubatch GEMM Y = X W^T for prefill and batched decode (gfx950).
//
// MFMA path (Q8_0 / Q4_0 weights): a 256-thread block computes a tile of
// 128 output features x BM tokens.  Per 32-wide K step (one quant block per
// weight row) the block dequantizes the 128 weight blocks into LDS as f16,
// copies the BM x 32 activation slice into LDS, and each wavefront issues
// v_mfma_f32_32x32x16_f16 on its 64 x BM/2 sub-tile with fp32 accumulation.
// The next K step's global loads are issued before the current step's MFMAs.
// Operand layouts (checked on the device): lane l supplies A[l%32][8(l/32)+e]
// and B[8(l/32)+e][l%32]; accumulator r of lane l is C[(r/4)*8+(l/32)*4+r%4][l%32].
// Here A is the weight tile (rows = features) and B the activation tile
// transposed (columns = tokens), so a lane's accumulators are four runs of 4
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

// Dequantizes 16 weights (half `hb` of one 32-weight block) to f16.
template <int WT>
DEV void deq16(const QMat &W, int row, int blk, int hb, uint4 raw, uint16_t dbits, h2 *out) {
    const f16 d = __builtin_bit_cast(f16, dbits);
    const h2 dd = h2{d, d};
    if (WT == T_Q4_0) {
        // codes 16*hb .. 16*hb+15: low (hb=0) or high (hb=1) nibbles of bytes 0..15
        const uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};
        const h2 off = h2{(f16)1032.f, (f16)1032.f};
#pragma unroll
        for (int i = 0; i < 4; i++) {
            const uint32_t m = (w[i] >> (4 * hb)) & 0x0F0F0F0Fu;
            const uint32_t p0 = (m & 0x000000FFu) | ((m << 8) & 0x00FF0000u);
            const uint32_t p1 = ((m >> 16) & 0x000000FFu) | ((m >> 8) & 0x00FF0000u);
            out[2 * i + 0] = (as_h2(p0 | 0x64006400u) - off) * dd;
            out[2 * i + 1] = (as_h2(p1 | 0x64006400u) - off) * dd;
        }
    } else {
        // codes 16*hb .. 16*hb+15 are the bytes of raw (signed)
        const uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};
        const h2 off = h2{(f16)1152.f, (f16)1152.f};
#pragma unroll
        for (int i = 0; i < 4; i++) {
            const uint32_t u = w[i] ^ 0x80808080u;
            const uint32_t p0 = (u & 0x000000FFu) | ((u << 8) & 0x00FF0000u);
            const uint32_t p1 = ((u >> 16) & 0x000000FFu) | ((u >> 8) & 0x00FF0000u);
            out[2 * i + 0] = (as_h2(p0 | 0x64006400u) - off) * dd;
            out[2 * i + 1] = (as_h2(p1 | 0x64006400u) - off) * dd;
        }
    }
}

template <int WT, int BM, int EPI>
__global__ __launch_bounds__(256) void k_gemm_mfma(QMat W, const uint16_t *X, int ldx,
                                                   EpiArgs ep, int M, int pair_mode) {
    constexpr int MT = BM / 64;   // 32x32 m-tiles per wavefront
    __shared__ __attribute__((aligned(16))) f16 As[BN * LDS_STRIDE];
    __shared__ __attribute__((aligned(16))) f16 Bs[BM * LDS_STRIDE];

    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int n0 = blockIdx.x * BN, m0 = blockIdx.y * BM;
    const int K = W.K, nb = K >> 5;
    const int wn = (w & 1) * 64, wm = (w >> 1) * (BM / 2);

    // loader roles
    const int a_row = tid >> 1, a_half = tid & 1;     // one half-block of one weight row
    constexpr int XCH = BM * 4;                        // 16-byte chunks of the X tile
    constexpr int XPT = (XCH + 255) / 256;             // chunks per thread

    const size_t qrow_bytes = WT == T_Q4_0 ? (size_t)(K >> 1) : (size_t)K;
    const uint8_t *qbase = (const uint8_t *)W.qs + (size_t)(n0 + a_row) * qrow_bytes;
    const uint16_t *dbase = W.d + (size_t)(n0 + a_row) * nb;

    uint4 araw;
    uint16_t adb;
    uint4 xraw[XPT];

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
            if (ch < XCH && m0 + mr < M)
                xraw[c] = *(const uint4 *)(X + (size_t)(m0 + mr) * ldx + kb * 32 + kc * 8);
            else
                xraw[c] = make_uint4(0, 0, 0, 0);
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
    for (int kb = 0; kb < nb; kb++) {
        __syncthreads();
        {
            h2 v[8];
            deq16<WT>(W, n0 + a_row, kb, a_half, araw, adb, v);
            uint4 *dst = (uint4 *)(As + a_row * LDS_STRIDE + a_half * 16);
            dst[0] = __builtin_bit_cast(uint4, *(h8 *)&v[0]);
            dst[1] = __builtin_bit_cast(uint4, *(h8 *)&v[4]);
#pragma unroll
            for (int c = 0; c < XPT; c++) {
                const int ch = tid + c * 256;
                if (ch < XCH) {
                    const int mr = ch >> 2, kc = ch & 3;
                    *(uint4 *)(Bs + mr * LDS_STRIDE + kc * 8) = xraw[c];
                }
            }
        }
        __syncthreads();
        if (kb + 1 < nb) gload(kb + 1);
#pragma unroll
        for (int kk = 0; kk < 32; kk += 16) {
            h8 af[2], bf[MT];
#pragma unroll
            for (int a = 0; a < 2; a++)
                af[a] = *(const h8 *)(As + (wn + 32 * a + (lane & 31)) * LDS_STRIDE + kk + 8 * (lane >> 5));
#pragma unroll
            for (int b = 0; b < MT; b++)
                bf[b] = *(const h8 *)(Bs + (wm + 32 * b + (lane & 31)) * LDS_STRIDE + kk + 8 * (lane >> 5));
#pragma unroll
            for (int a = 0; a < 2; a++)
#pragma unroll
                for (int b = 0; b < MT; b++)
                    acc[a][b] = __builtin_amdgcn_mfma_f32_32x32x16_f16(af[a], bf[b], acc[a][b], 0, 0, 0);
        }
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
__global__ __launch_bounds__(256) void k_gemm_f32(QMat W, const uint16_t *X, int ldx, EpiArgs ep,
                                                  int M, int pair_mode) {
    const int p = blockIdx.x * 256 + threadIdx.x;
    const int m = blockIdx.y;
    if (p >= W.N / 2 || m >= M) return;
    int r0, r1;
    pair_rows(pair_mode, p, r0, r1);
    const float *w0 = (const float *)W.qs + (size_t)r0 * W.K;
    const float *w1 = (const float *)W.qs + (size_t)r1 * W.K;
    const f16 *x = (const f16 *)X + (size_t)m * ldx;
    float a = 0.f, b = 0.f;
    for (int k = 0; k < W.K; k++) {
        const float xv = (float)x[k];
        a += w0[k] * xv;
        b += w1[k] * xv;
    }
    epi_pair<EPI>(ep, m, p, r0, r1, a, b);
}

template <int WT, int EPI>
void launch_mfma_epi(const QMat &W, const uint16_t *X, int ldx, const EpiArgs &ep, int M,
                     int pair_mode, hipStream_t s) {
    if (M > 64) {
        hipLaunchKernelGGL((k_gemm_mfma<WT, 128, EPI>), dim3(W.N / BN, (M + 127) / 128), dim3(256), 0,
                           s, W, X, ldx, ep, M, pair_mode);
    } else {
        hipLaunchKernelGGL((k_gemm_mfma<WT, 64, EPI>), dim3(W.N / BN, (M + 63) / 64), dim3(256), 0, s,
                           W, X, ldx, ep, M, pair_mode);
    }
}

template <int WT>
void launch_mfma(const QMat &W, const uint16_t *X, int ldx, const EpiArgs &ep, int M,
                 int pair_mode, hipStream_t s) {
    switch (ep.epi) {
    case EPI_STORE: launch_mfma_epi<WT, EPI_STORE>(W, X, ldx, ep, M, pair_mode, s); break;
    case EPI_RESID: launch_mfma_epi<WT, EPI_RESID>(W, X, ldx, ep, M, pair_mode, s); break;
    case EPI_QKV: launch_mfma_epi<WT, EPI_QKV>(W, X, ldx, ep, M, pair_mode, s); break;
    case EPI_SWIGLU: launch_mfma_epi<WT, EPI_SWIGLU>(W, X, ldx, ep, M, pair_mode, s); break;
    }
}

template <int EPI>
void launch_f32_epi(const QMat &W, const uint16_t *X, int ldx, const EpiArgs &ep, int M,
                    int pair_mode, hipStream_t s) {
    hipLaunchKernelGGL(k_gemm_f32<EPI>, dim3((W.N / 2 + 255) / 256, M), dim3(256), 0, s, W, X, ldx,
                       ep, M, pair_mode);
}

}  // namespace

bool launch_gemm(const QMat &W, const uint16_t *X, int ldx, const EpiArgs &ep, int M,
                 hipStream_t s) {
    if (M <= 0 || W.N % 2) return false;
    const int pair_mode = ep.epi == EPI_SWIGLU ? PAIR_GU : PAIR_ADJ;
    if (pair_mode == PAIR_GU && W.N % 64) return false;
    if ((W.wtype == T_Q4_0 || W.wtype == T_Q8_0) && W.N % BN == 0 && W.K % 32 == 0 && ldx % 8 == 0) {
        if (W.wtype == T_Q4_0)
            launch_mfma<T_Q4_0>(W, X, ldx, ep, M, pair_mode, s);
        else
            launch_mfma<T_Q8_0>(W, X, ldx, ep, M, pair_mode, s);
        return true;
    }
    if (W.wtype != T_F32) return false;
    switch (ep.epi) {
    case EPI_STORE: launch_f32_epi<EPI_STORE>(W, X, ldx, ep, M, pair_mode, s); break;
    case EPI_RESID: launch_f32_epi<EPI_RESID>(W, X, ldx, ep, M, pair_mode, s); break;
    case EPI_QKV: launch_f32_epi<EPI_QKV>(W, X, ldx, ep, M, pair_mode, s); break;
    case EPI_SWIGLU: launch_f32_epi<EPI_SWIGLU>(W, X, ldx, ep, M, pair_mode, s); break;
    default: return false;
    }
    return true;
}
