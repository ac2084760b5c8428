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
// A 256-thread block computes BN = 128 output features x BM tokens; each
// wavefront owns a 64 x BM/2 sub-tile.  Pipeline per K block (32 k):
//   * global loads of codes, scale and both activation parts go to
//     registers three K blocks ahead (three register sets, the loop unrolled
//     by six so that each set has fixed registers);
//   * a K block is converted (codes -> f16) and written to one of two LDS
//     stages while the other stage feeds the MFMAs; one barrier per K block.
// Rows of an LDS tile are 40 f16 (80 bytes) apart, so the 16-byte fragment
// reads of 8 consecutive rows hit disjoint banks.
// Blocks that share a weight tile are placed on the same XCD (block ids go
// round-robin over the 8 XCDs), so the tile is fetched from HBM once into
// that XCD's L2.  When the tile grid is too small to fill the chip (the
// d x d and d x F matrices at 512 tokens), K is split over 2 or 4 blocks
// that write fp32 partial tiles; a second kernel adds them in a fixed order
// and applies the epilogue, so results do not depend on timing.
// Operand layouts (checked on the device): lane l supplies A[l%32][8(l/32)+e]
// and B[8(l/32)+e][l%32]; accumulator r of lane l is C[(r/4)*8+(l/32)*4+r%4][l%32].
// A is the activation tile (rows = tokens) and B the code tile transposed
// (columns = features): a lane's 16 accumulators of a tile are 16 tokens of
// ONE feature, so the block scale it applies is a single value per tile.
// In the epilogue gate/up pairs (feature tiles 32 apart) meet in one lane;
// RoPE pairs (adjacent features) sit in lanes l and l^1 and are exchanged.
//
// Fallback path (fp32 weights, or shapes the MFMA tiling does not cover):
// one thread per (row pair, token), plain fp32 FMA (for quantized weights on
// the codes, block by block).  Q4_K weights take the direct-to-LDS form
// (gemm_dl.hip) or such a plain kernel.
#include <stdlib.h>
#include <string.h>

#include <algorithm>
#include <type_traits>

#include "common.h"
#include "epilogue.h"
#include "kernels.h"

namespace {

void launch_sum(int epi, const float *ws, int S, int N, int M, const EpiArgs &ep, int pair_mode, hipStream_t s);

constexpr int BN = 128;
constexpr int LDS_STRIDE = 40;   // f16 elements per LDS row (32 + 8 pad)

typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// f16 pairs {1024 + byte0, 1024 + byte1} and {1024 + byte2, 1024 + byte3}
// of a word whose bytes are all below 0x400 - 1024 (v_perm_b32).
DEV h2 magic_lo(uint32_t v) { return as_h2(__builtin_amdgcn_perm(0x64646464u, v, 0x04010400u)); }
DEV h2 magic_hi(uint32_t v) { return as_h2(__builtin_amdgcn_perm(0x64646464u, v, 0x04030402u)); }

// Q4_0: the 8 bytes at offset 8h of a block hold codes 8h..8h+7 (low
// nibbles) and 16+8h..16+8h+7 (high nibbles); out0/out1 get them as exact
// f16 values q - 8.
DEV void q4_codes(u32x2 raw, h8 &out0, h8 &out1) {
    const h2 off = h2{(f16)1032.f, (f16)1032.f};
    const uint32_t l0 = raw.x & 0x0F0F0F0Fu, l1 = raw.y & 0x0F0F0F0Fu;
    const uint32_t u0 = (raw.x >> 4) & 0x0F0F0F0Fu, u1 = (raw.y >> 4) & 0x0F0F0F0Fu;
    const h2 a0 = magic_lo(l0) - off, a1 = magic_hi(l0) - off, a2 = magic_lo(l1) - off, a3 = magic_hi(l1) - off;
    const h2 b0 = magic_lo(u0) - off, b1 = magic_hi(u0) - off, b2 = magic_lo(u1) - off, b3 = magic_hi(u1) - off;
    out0 = h8{a0.x, a0.y, a1.x, a1.y, a2.x, a2.y, a3.x, a3.y};
    out1 = h8{b0.x, b0.y, b1.x, b1.y, b2.x, b2.y, b3.x, b3.y};
}

// Q8_0: 16 signed byte codes as exact f16 values.
DEV void q8_codes(u32x4 raw, h8 &out0, h8 &out1) {
    const h2 off = h2{(f16)1152.f, (f16)1152.f};
    const uint32_t w0 = raw.x ^ 0x80808080u, w1 = raw.y ^ 0x80808080u;
    const uint32_t w2 = raw.z ^ 0x80808080u, w3 = raw.w ^ 0x80808080u;
    const h2 a0 = magic_lo(w0) - off, a1 = magic_hi(w0) - off, a2 = magic_lo(w1) - off, a3 = magic_hi(w1) - off;
    const h2 b0 = magic_lo(w2) - off, b1 = magic_hi(w2) - off, b2 = magic_lo(w3) - off, b3 = magic_hi(w3) - off;
    out0 = h8{a0.x, a0.y, a1.x, a1.y, a2.x, a2.y, a3.x, a3.y};
    out1 = h8{b0.x, b0.y, b1.x, b1.y, b2.x, b2.y, b3.x, b3.y};
}

// One K block of a block's operands, held in registers between its global
// load and its LDS store.  Thread t covers weight row t/2, half t%2 of the
// block, and XC 16-byte chunks of each activation part.
// (clang vector types: HIP's uint4 is a struct whose copies are memcpys
// that keep the stage out of registers)
template <int WT, int XC>
struct Stage {
    u32x4 a;          // Q4_0: .x,.y = 8 bytes; Q8_0: 16 bytes
    uint32_t d;       // f16 scale bits of row t/2 (even threads)
    bool live;        // false: a K block past the last one (scale taken as 0)
    u32x4 xh[XC], xl[XC];
};

// F16W (opt-in, DECODE_GEMM_F16=1, ubatches of more than 64 tokens): the
// weights enter the matrix cores as f16(d * code) (the block's dequantized
// values rounded to f16) and the activations as their f16 value part only,
// with fp32 accumulation: one MFMA per 16 k and tile and no per-block
// scaling, and from 256 tokens on a block covers 256 tokens with two register
// stages.  This is the precision of a dequantize-then-f16-GEMM path; at the
// 8B shape it leaves the prefill logits about 3.5e-2 from the fp64 result,
// over the 2e-2 acceptance bound, so it is not the default.  Otherwise
// (exact operands) as described above.
template <int WT, int BM, int EPI, bool SPLIT, bool F16W>
__global__ __launch_bounds__(256, 2) void k_gemm_mfma(QMat W, const uint16_t *Xh, const uint16_t *Xl,
                                                      int ldx, EpiArgs ep, int M, int pair_mode, int NT,
                                                      int nsplit, float *part) {
    constexpr int MT = BM / 64;                         // 32x32 token tiles per wavefront
    constexpr int XC = BM * 4 / 256 > 0 ? BM * 4 / 256 : 1;   // activation chunks per thread and part
    constexpr bool XALL = BM * 4 >= 256;                // every thread loads activations
    __shared__ __attribute__((aligned(16))) f16 As[2][BN * LDS_STRIDE];
    __shared__ __attribute__((aligned(16))) f16 Bh[2][BM * LDS_STRIDE];
    __shared__ __attribute__((aligned(16))) f16 Bl[2][F16W ? 8 : BM * LDS_STRIDE];
    __shared__ __attribute__((aligned(16))) float Sc[2][F16W ? 1 : BN];

    // block -> (feature tile, token tile, K split); the tiles of one feature
    // tile (all token tiles and splits) share an XCD
    const int mtiles = (M + BM - 1) / BM;
    const int per_nt = mtiles * nsplit;
    const int L = blockIdx.x, xcd = L & 7, j = L >> 3;
    const int nt = (j / per_nt) * 8 + xcd, rem = j % per_nt;
    const int mtile = rem % mtiles, split = rem / mtiles;
    if (nt >= NT) return;

    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int n0 = nt * BN, m0 = mtile * BM;
    const int nb_all = W.K >> 5, nb = nb_all / nsplit, kb0 = split * nb;
    const int wn = (w & 1) * 64, wm = (w >> 1) * (BM / 2);

    // loader roles
    const int a_row = tid >> 1, a_half = tid & 1;
    const size_t qrow_bytes = WT == T_Q4_0 ? (size_t)(W.K >> 1) : (size_t)W.K;
    const uint8_t *qbase = (const uint8_t *)W.qs + (size_t)(n0 + a_row) * qrow_bytes +
                           (WT == T_Q4_0 ? a_half * 8 : a_half * 16);
    const uint16_t *dbase = W.d + (size_t)(n0 + a_row) * nb_all;
    const bool x_loader = XALL || tid < BM * 4;
    const uint16_t *xh_src[XC], *xl_src[XC];
    int x_lds[XC];
#pragma unroll
    for (int c = 0; c < XC; c++) {
        const int ch = (XALL ? tid + c * 256 : tid);
        const int mr = ch >> 2, kc = ch & 3;
        const int row = min(m0 + mr, M - 1);            // rows past M load row M-1; their outputs are dropped
        xh_src[c] = Xh + (size_t)row * ldx + kc * 8;
        xl_src[c] = Xl + (size_t)row * ldx + kc * 8;
        x_lds[c] = mr * LDS_STRIDE + kc * 8;
    }

    // kb may run past the last K block: the last one is re-read with a zero
    // scale, so that block adds nothing
    auto gload = [&](Stage<WT, XC> &r, int kb_raw) __attribute__((always_inline)) {
        const int kb = min(kb_raw, nb - 1);
        const int k = kb0 + kb;
        if (WT == T_Q4_0) {
            const u32x2 v = *(const u32x2 *)(qbase + (size_t)k * 16);
            r.a = u32x4{v.x, v.y, 0u, 0u};
        } else {
            r.a = *(const u32x4 *)(qbase + (size_t)k * 32);
        }
        r.d = dbase[k];
        r.live = kb_raw < nb;   // applied at the store: a select here would wait for the load
        if (x_loader) {
#pragma unroll
            for (int c = 0; c < XC; c++) {
                r.xh[c] = *(const u32x4 *)(xh_src[c] + k * 32);
                if (!F16W) r.xl[c] = *(const u32x4 *)(xl_src[c] + k * 32);
            }
        }
    };
    auto lstore = [&](const Stage<WT, XC> &r, int st) __attribute__((always_inline)) {
        h8 c0, c1;
        f16 *arow = &As[st][a_row * LDS_STRIDE];
        if (WT == T_Q4_0)
            q4_codes(u32x2{r.a.x, r.a.y}, c0, c1);
        else
            q8_codes(r.a, c0, c1);
        const uint32_t dbits = r.live ? r.d : 0u;
        if (F16W) {
            const f16 dv = __builtin_bit_cast(f16, (uint16_t)dbits);
            const h8 dd = h8{dv, dv, dv, dv, dv, dv, dv, dv};
            c0 *= dd;
            c1 *= dd;
        }
        if (WT == T_Q4_0) {
            *(h8 *)(arow + 8 * a_half) = c0;           // codes 8h .. 8h+7
            *(h8 *)(arow + 16 + 8 * a_half) = c1;      // codes 16+8h .. 16+8h+7
        } else {
            *(h8 *)(arow + 16 * a_half) = c0;          // codes 16h .. 16h+7
            *(h8 *)(arow + 16 * a_half + 8) = c1;      // codes 16h+8 .. 16h+15
        }
        if (!F16W && a_half == 0) Sc[st][a_row] = f16_bits_to_f32((uint16_t)dbits);
        if (x_loader) {
#pragma unroll
            for (int c = 0; c < XC; c++) {
                *(u32x4 *)(&Bh[st][x_lds[c]]) = r.xh[c];
                if (!F16W) *(u32x4 *)(&Bl[st][x_lds[c]]) = r.xl[c];
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

    auto compute = [&](int st) __attribute__((always_inline)) {
        if constexpr (F16W) {
#pragma unroll
            for (int h = 0; h < 2; h++) {
                h8 cf[2], xh[MT];
#pragma unroll
                for (int a = 0; a < 2; a++)
                    cf[a] = *(const h8 *)(&As[st][(wn + 32 * a + (lane & 31)) * LDS_STRIDE + 16 * h + 8 * (lane >> 5)]);
#pragma unroll
                for (int b = 0; b < MT; b++)
                    xh[b] = *(const h8 *)(&Bh[st][(wm + 32 * b + (lane & 31)) * LDS_STRIDE + 16 * h + 8 * (lane >> 5)]);
#pragma unroll
                for (int a = 0; a < 2; a++)
#pragma unroll
                    for (int b = 0; b < MT; b++)
                        acc[a][b] = __builtin_amdgcn_mfma_f32_32x32x16_f16(xh[b], cf[a], acc[a][b], 0, 0, 0);
            }
        } else {
        f16x tmp[2][MT];
#pragma unroll
        for (int kk = 0; kk < 32; kk += 16) {
            h8 cf[2], xh[MT], xl[MT];
#pragma unroll
            for (int a = 0; a < 2; a++)
                cf[a] = *(const h8 *)(&As[st][(wn + 32 * a + (lane & 31)) * LDS_STRIDE + kk + 8 * (lane >> 5)]);
#pragma unroll
            for (int b = 0; b < MT; b++) {
                const int off = (wm + 32 * b + (lane & 31)) * LDS_STRIDE + kk + 8 * (lane >> 5);
                xh[b] = *(const h8 *)(&Bh[st][off]);
                xl[b] = *(const h8 *)(&Bl[st][off]);
            }
            // consecutive MFMAs write different tiles
#pragma unroll
            for (int a = 0; a < 2; a++)
#pragma unroll
                for (int b = 0; b < MT; b++)
                    tmp[a][b] = __builtin_amdgcn_mfma_f32_32x32x16_f16(xh[b], cf[a], kk ? tmp[a][b] : f16x{}, 0, 0, 0);
#pragma unroll
            for (int a = 0; a < 2; a++)
#pragma unroll
                for (int b = 0; b < MT; b++)
                    tmp[a][b] = __builtin_amdgcn_mfma_f32_32x32x16_f16(xl[b], cf[a], tmp[a][b], 0, 0, 0);
        }
        // C += d[n][kb] * T: one scale per lane and feature tile
#pragma unroll
        for (int a = 0; a < 2; a++) {
            const float sc = Sc[st][wn + 32 * a + (lane & 31)];
#pragma unroll
            for (int b = 0; b < MT; b++)
#pragma unroll
                for (int r = 0; r < 16; r++) acc[a][b][r] += sc * tmp[a][b][r];
        }
        }
    };

    // Loads past the last K block re-read the last one (their data is never
    // used), so no load sits behind a branch: the compiler can then wait for
    // exactly the register set a store needs and leave the others in flight.
    // Three register sets rotate over two LDS stages (period 6): a K block's
    // loads are issued three compute steps before its LDS store, which covers
    // a loaded memory latency at the MFMA rate of a step.
    if constexpr (F16W ? BM == 256 : BM == 64) {
        // two register sets (the accumulators leave no room for a third): a
        // K block's loads are issued two steps before its LDS store
        Stage<WT, XC> r0, r1;
        gload(r0, 0);
        gload(r1, 1);
        lstore(r0, 0);
        __syncthreads();
        gload(r0, 2);
        // top: LDS stage 0 holds kb; r1, r0 carry kb+1, kb+2
        int kb = 0;
        // exact operands: K blocks past the last one take zero scales, so the
        // loop runs whole periods and has no guarded tail
        const int nbl = F16W ? nb - 2 : (nb + 1) / 2 * 2;
        for (; kb < nbl; kb += 2) {
            compute(0);                                 // kb
            lstore(r1, 1);
            __syncthreads();
            gload(r1, kb + 3);
            compute(1);                                 // kb+1
            lstore(r0, 0);
            __syncthreads();
            gload(r0, kb + 4);
        }
        if constexpr (F16W) {
            compute(0);                                 // last 1 or 2 K blocks
            if (kb + 1 < nb) {
                lstore(r1, 1);
                __syncthreads();
                compute(1);
            }
        }
    } else {
    Stage<WT, XC> r0, r1, r2;
    gload(r0, 0);
    gload(r1, 1);
    gload(r2, 2);
    lstore(r0, 0);
    __syncthreads();
    gload(r0, 3);
    // top of an iteration: LDS stage 0 holds kb; r1, r2, r0 carry kb+1..kb+3
    if constexpr (F16W) {
    // Step i of a period: compute K block kb+i, store kb+i+1 to the other
    // LDS stage, load kb+i+4.  Full periods run unguarded (the compiler can
    // then count exactly which loads a store waits for); the last period's
    // steps are guarded by uniform conditions rather than early exits, so the
    // accumulators stay in the same registers on every path.
    int kb = 0;
    for (; kb + 7 <= nb; kb += 6) {
        compute(0);                                     // kb
        lstore(r1, 1);
        __syncthreads();
        gload(r1, min(kb + 4, nb - 1));
        compute(1);                                     // kb+1
        lstore(r2, 0);
        __syncthreads();
        gload(r2, min(kb + 5, nb - 1));
        compute(0);                                     // kb+2
        lstore(r0, 1);
        __syncthreads();
        gload(r0, min(kb + 6, nb - 1));
        compute(1);                                     // kb+3
        lstore(r1, 0);
        __syncthreads();
        gload(r1, min(kb + 7, nb - 1));
        compute(0);                                     // kb+4
        lstore(r2, 1);
        __syncthreads();
        gload(r2, min(kb + 8, nb - 1));
        compute(1);                                     // kb+5
        lstore(r0, 0);
        __syncthreads();
        gload(r0, min(kb + 9, nb - 1));
    }
    // last 1 .. 6 K blocks (r1 and r2 still take kb+4 and kb+5)
    compute(0);                                         // kb
    if (kb + 1 < nb) {
        lstore(r1, 1);
        __syncthreads();
        gload(r1, min(kb + 4, nb - 1));
        compute(1);
    }
    if (kb + 2 < nb) {
        lstore(r2, 0);
        __syncthreads();
        gload(r2, min(kb + 5, nb - 1));
        compute(0);
    }
    if (kb + 3 < nb) {
        lstore(r0, 1);
        __syncthreads();
        compute(1);
    }
    if (kb + 4 < nb) {
        lstore(r1, 0);
        __syncthreads();
        compute(0);
    }
    if (kb + 5 < nb) {
        lstore(r2, 1);
        __syncthreads();
        compute(1);
    }
    } else {
    // exact operands: every step guarded by a uniform condition
    for (int kb = 0; kb < nb; kb += 6) {
        compute(0);                                     // kb
        if (kb + 1 < nb) {
            lstore(r1, 1);
            __syncthreads();
            gload(r1, min(kb + 4, nb - 1));
            compute(1);                                 // kb+1
        }
        if (kb + 2 < nb) {
            lstore(r2, 0);
            __syncthreads();
            gload(r2, min(kb + 5, nb - 1));
            compute(0);                                 // kb+2
        }
        if (kb + 3 < nb) {
            lstore(r0, 1);
            __syncthreads();
            gload(r0, min(kb + 6, nb - 1));
            compute(1);                                 // kb+3
        }
        if (kb + 4 < nb) {
            lstore(r1, 0);
            __syncthreads();
            gload(r1, min(kb + 7, nb - 1));
            compute(0);                                 // kb+4
        }
        if (kb + 5 < nb) {
            lstore(r2, 1);
            __syncthreads();
            gload(r2, min(kb + 8, nb - 1));
            compute(1);                                 // kb+5
        }
        if (kb + 6 < nb) {
            lstore(r0, 0);
            __syncthreads();
            gload(r0, min(kb + 9, nb - 1));
        }
    }
    }
    }

    // ---- epilogue ----
    // lane: feature f = n0 + wn + 32a + (lane & 31); token of accumulator r:
    // m = m0 + wm + 32b + (r/4)*8 + (lane/32)*4 + r%4
    const int fl = lane & 31;
    if (SPLIT) {
        // fp32 partial tile of this split: part[split][m][n]
        const int N = W.N;
#pragma unroll
        for (int b = 0; b < MT; b++)
#pragma unroll
            for (int r = 0; r < 16; r++) {
                const int m = m0 + wm + 32 * b + (r >> 2) * 8 + (lane >> 5) * 4 + (r & 3);
                if (m >= M) continue;
                float *dst = part + ((size_t)split * M + m) * N + n0 + wn + fl;
                dst[0] = acc[0][b][r];
                dst[32] = acc[1][b][r];
            }
        return;
    }
    // one copy of the epilogue per token tile (b a constant: the tile's
    // accumulators stay in registers)
    auto epi_tile = [&](auto bc) __attribute__((always_inline)) {
        constexpr int b = decltype(bc)::value;
        const int mb = m0 + wm + 32 * b + (lane >> 5) * 4;
        if (EPI == EPI_STORE || EPI == EPI_RESID) {
#pragma unroll
            for (int r = 0; r < 16; r++) {
                const int m = mb + (r >> 2) * 8 + (r & 3);
                if (m >= M) continue;
                float *y = ep.y + (size_t)m * ep.ldy + n0 + wn + fl;
                if (EPI == EPI_STORE) {
                    y[0] = acc[0][b][r];
                    y[32] = acc[1][b][r];
                } else {
                    y[0] += acc[0][b][r];
                    y[32] += acc[1][b][r];
                }
            }
        } else if (pair_mode == PAIR_GU) {
            // gate rows n0+wn .. +31 and their up rows n0+wn+32 .. +63: feature (g*32 + fl)
            const int g = (n0 + wn) >> 6;
#pragma unroll
            for (int r = 0; r < 16; r++) {
                const int m = mb + (r >> 2) * 8 + (r & 3);
                if (m >= M) continue;
                const int rr = (g << 6) + fl;
                epi_pair<EPI>(ep, m, (g << 5) + fl, rr, rr + 32, acc[0][b][r], acc[1][b][r]);
            }
        } else {
            // adjacent features f (even lane) and f+1 (odd lane): the even lane
            // takes tokens r < 8 of the pair, the odd lane tokens r >= 8
            const bool odd = lane & 1;
#pragma unroll
            for (int a = 0; a < 2; a++)
#pragma unroll
                for (int r = 0; r < 8; r++) {
                    const float send = odd ? acc[a][b][r] : acc[a][b][r + 8];
                    const float recv = __shfl_xor(send, 1, 64);
                    const int rr = odd ? r + 8 : r;
                    const int m = mb + (rr >> 2) * 8 + (rr & 3);
                    const int f = n0 + wn + 32 * a + (fl & ~1);
                    const float va = odd ? recv : acc[a][b][r];
                    const float vb = odd ? acc[a][b][r + 8] : recv;
                    if (m < M) epi_pair<EPI>(ep, m, f >> 1, f, f + 1, va, vb);
                }
        }
    };
    epi_tile(std::integral_constant<int, 0>{});
    if constexpr (MT > 1) epi_tile(std::integral_constant<int, 1>{});
    if constexpr (MT > 2) epi_tile(std::integral_constant<int, 2>{});
    if constexpr (MT > 3) epi_tile(std::integral_constant<int, 3>{});
    static_assert(MT <= 4, "epilogue covers four token tiles");
}

// Sums the K-split partial tiles in split order and applies the epilogue;
// one thread per (row pair, token).  The epilogue's memory inputs and the
// first 8 splits' values are requested together, then added in order.
template <int EPI>
__global__ __launch_bounds__(256) void k_gemm_splitk_sum(const float *part, int nsplit, int N, int M,
                                                         EpiArgs ep, int pair_mode) {
    const int p = blockIdx.x * 256 + threadIdx.x;
    const int m = blockIdx.y;
    if (p >= N / 2 || m >= M) return;
    int r0, r1;
    pair_rows(pair_mode, p, r0, r1);
    const EpiPre pre = epi_prefetch<EPI>(ep, m, r0, r1);
    const float *pm = part + (size_t)m * N;
    const size_t ps = (size_t)M * N;                   // between splits
    float va[8], vb[8];
#pragma unroll
    for (int s = 0; s < 8; s++)
        if (s < nsplit) {
            va[s] = pm[s * ps + r0];
            vb[s] = pm[s * ps + r1];
        }
    float a = 0.f, b = 0.f;
#pragma unroll
    for (int s = 0; s < 8; s++)
        if (s < nsplit) {
            a += va[s];
            b += vb[s];
        }
    for (int s = 8; s < nsplit; s++) {
        a += pm[s * ps + r0];
        b += pm[s * ps + r1];
    }
    epi_pair_pre<EPI>(ep, m, p, r0, r1, a, b, pre);
}

// The K-split sum of a residual-adding GEMM fused with the RMSNorm of the
// rows it completes: one 1024-thread block per token row; element j of the row
// is y[j] + the sum of the S partials in split order (as k_gemm_splitk_sum adds
// them), each thread holding its elements' sums in registers for the norm.
// V = 4 (N and the row stride of y multiples of 4) moves each split's values
// of a thread in one 16-byte load.
constexpr int SRN_T = 1024, SRN_E = 16;      // threads, elements per thread at most (rows <= 16384)
template <int V>
__global__ __launch_bounds__(SRN_T) void k_splitk_resid_norm(const float *part, int nsplit, int N, int M, EpiArgs ep) {
    constexpr int U = SRN_E / V;                       // chunks of V elements per thread at most
    __shared__ float red[SRN_T / 64];
    const int m = blockIdx.x, tid = threadIdx.x;
    float *y = ep.y + (size_t)m * ep.ldy;
    const float *pm = part + (size_t)m * N;
    const size_t ps = (size_t)M * N;                   // between splits
    using vec = std::conditional_t<V == 4, float4, float>;
    auto ld = [](const float *p) __attribute__((always_inline)) { return *(const vec *)p; };
    auto el = [](const vec &x, int e) __attribute__((always_inline)) -> float {
        if constexpr (V == 4) return e == 0 ? x.x : e == 1 ? x.y : e == 2 ? x.z : x.w;
        else return x;
    };
    float v[U][V];
    float ss = 0.f;
#pragma unroll
    for (int u = 0; u < U; u++) {
        const int j = (tid + SRN_T * u) * V;
        if (SRN_T * u * V >= N) break;                 // uniform
        const int jc = min(j, N - V);
        vec pv[8];
#pragma unroll
        for (int k = 0; k < 8; k++)
            if (k < nsplit) pv[k] = ld(pm + k * ps + jc);
        const vec yv = ld(y + jc);
#pragma unroll
        for (int e = 0; e < V; e++) {
            float a = 0.f;
#pragma unroll
            for (int k = 0; k < 8; k++)
                if (k < nsplit) a += el(pv[k], e);
            for (int k = 8; k < nsplit; k++) a += pm[k * ps + jc + e];
            v[u][e] = el(yv, e) + a;
        }
        if (j < N) {
#pragma unroll
            for (int e = 0; e < V; e++) {
                y[j + e] = v[u][e];
                ss += v[u][e] * v[u][e];
            }
        }
    }
    ss = wave_sum(ss);
    if ((tid & 63) == 0) red[tid >> 6] = ss;
    __syncthreads();
    float tot = 0.f;
#pragma unroll
    for (int i = 0; i < SRN_T / 64; i++) tot += red[i];
    const float r = 1.0f / sqrtf(tot / (float)N + ep.nrm_eps);
    f16 *o = (f16 *)ep.nrm_h + (size_t)m * ep.nrm_ld;
    f16 *ol = (f16 *)ep.nrm_l + (size_t)m * ep.nrm_ld;
#pragma unroll
    for (int u = 0; u < U; u++) {
        const int j = (tid + SRN_T * u) * V;
        if (SRN_T * u * V >= N) break;
        if (j < N) {
#pragma unroll
            for (int e = 0; e < V; e++) {
                const float w = v[u][e] * r * ep.nrm_g[j + e];
                const f16 hi = (f16)w;
                o[j + e] = hi;
                ol[j + e] = (f16)(w - (float)hi);
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

// Block-quantized weights of any N (shapes the MFMA forms do not cover):
// one thread per (row pair, token); per 32-weight block d * sum(c x) with c
// the signed code (Q4_0: q - 8, Q8_0: q), or for a Q4_K sub-block
// (d sc) sum q x - (dmin m) sum x, in fp32.
template <int WT, int EPI>
__global__ __launch_bounds__(256) void k_gemm_plainq(QMat W, const uint16_t *X, const uint16_t *Xl, int ldx,
                                                     EpiArgs ep, int M, int pair_mode) {
    const int p = blockIdx.x * 256 + threadIdx.x;
    const int m = blockIdx.y;
    if (p >= W.N / 2 || m >= M) return;
    int r0, r1;
    pair_rows(pair_mode, p, r0, r1);
    const f16 *x = (const f16 *)X + (size_t)m * ldx;
    const f16 *xl = (const f16 *)Xl + (size_t)m * ldx;
    const int nb = W.K >> 5;
    float out[2];
    const int rows[2] = {r0, r1};
    for (int i = 0; i < 2; i++) {
        const int row = rows[i];
        const uint8_t *q = (const uint8_t *)W.qs + (size_t)row * (WT == T_Q8_0 ? W.K : W.K >> 1);
        float a = 0.f;
        for (int b = 0; b < nb; b++) {
            float t = 0.f, xs = 0.f;
            for (int k = 0; k < 32; k++) {
                int c;
                if (WT == T_Q8_0) {
                    c = (int)(int8_t)q[b * 32 + k];
                } else {
                    const uint8_t byte = q[b * 16 + (k & 15)];
                    c = (k < 16 ? (byte & 15) : (byte >> 4)) - (WT == T_Q4_0 ? 8 : 0);
                }
                const float xv = (float)x[b * 32 + k] + (float)xl[b * 32 + k];
                t += (float)c * xv;
                xs += xv;
            }
            if (WT == T_Q4_K) {
                const uint32_t dd = W.dm[(size_t)row * (W.K >> 8) + (b >> 3)];
                const uint16_t sm = W.d[(size_t)row * nb + b];
                a += f16_bits_to_f32((uint16_t)dd) * (float)(sm & 63) * t -
                     f16_bits_to_f32((uint16_t)(dd >> 16)) * (float)((sm >> 8) & 63) * xs;
            } else {
                a += f16_bits_to_f32(W.d[(size_t)row * nb + b]) * t;
            }
        }
        out[i] = a;
    }
    epi_pair<EPI>(ep, m, p, r0, r1, out[0], out[1]);
}

// xs[m][kb] = sum of (Xh + Xl)[m][32 kb .. 32 kb + 31], in order.
__global__ __launch_bounds__(256) void k_block_sums(const uint16_t *Xh, const uint16_t *Xl, int ldx, int M, int K,
                                                    float *xs) {
    const int nb = K >> 5;
    const long long idx = (long long)blockIdx.x * 256 + threadIdx.x;
    if (idx >= (long long)M * nb) return;
    const int m = (int)(idx / nb), kb = (int)(idx % nb);
    const h8 *h = (const h8 *)(Xh + (size_t)m * ldx + kb * 32);
    const h8 *l = (const h8 *)(Xl + (size_t)m * ldx + kb * 32);
    float s = 0.f;
#pragma unroll
    for (int c = 0; c < 4; c++) {
        const h8 hv = h[c], lv = l[c];
#pragma unroll
        for (int e = 0; e < 8; e++) s += (float)hv[e] + (float)lv[e];
    }
    const f16 sh = (f16)s, sl = (f16)(s - (float)sh);
    // octet-major [K/256][M][8]: the 8 sums of one K-block octet of a token are contiguous
    ((uint32_t *)xs)[((size_t)(kb >> 3) * M + m) * 8 + (kb & 7)] =
        (uint32_t)__builtin_bit_cast(uint16_t, sh) | ((uint32_t)__builtin_bit_cast(uint16_t, sl) << 16);
}

// mfq = -f(dmin) m of sub-block kb of row n as f16 value | remainder << 16,
// octet-major ([K/256][N][8]); sf[kb][n] = f(d) sc (exact in fp32: an 11-bit
// significand times a six-bit integer).
__global__ __launch_bounds__(256) void k_q4k_mins(QMat W) {
    const int nb = W.K >> 5;
    const long long idx = (long long)blockIdx.x * 256 + threadIdx.x;
    if (idx >= (long long)W.N * nb) return;
    const int r = (int)(idx / nb), b = (int)(idx % nb);
    const uint32_t dd = W.dm[(size_t)r * (W.K >> 8) + (b >> 3)];
    W.sf[(size_t)b * W.N + r] = f16_bits_to_f32((uint16_t)dd) * (float)(W.d[idx] & 63);
    const float v = -f16_bits_to_f32((uint16_t)(dd >> 16)) * (float)((W.d[idx] >> 8) & 63);
    const f16 vh = (f16)v, vl = (f16)(v - (float)vh);
    W.mfq[((size_t)(b >> 3) * W.N + r) * 8 + (b & 7)] = (uint32_t)__builtin_bit_cast(uint16_t, vh) | ((uint32_t)__builtin_bit_cast(uint16_t, vl) << 16);
}


// dt[kb][n] = d[n][kb]
__global__ __launch_bounds__(256) void k_scales_t(QMat W) {
    const int nb = W.K >> 5;
    const long long idx = (long long)blockIdx.x * 256 + threadIdx.x;
    if (idx >= (long long)W.N * nb) return;
    const int r = (int)(idx / nb), b = (int)(idx % nb);
    W.dt[(size_t)b * W.N + r] = W.d[idx];
}


// ---- skinny form: ubatches of at most 32 tokens (batched decode) ----------
//
// The same exact operands as above, without LDS staging or a barrier per K
// block.  A wavefront owns FT tiles of 32 features and every token (one
// 32-row tile; rows past M repeat row M-1 and are dropped), and streams its
// own weight rows straight into B operands: lane l takes feature l%32 and the
// 8 bytes of the block that hold codes 8(l/32)..+7 (low nibbles: k-half 0)
// and 16+8(l/32)..+7 (high nibbles: k-half 1) for Q4_0, or those two 8-byte
// runs for Q8_0.  The activation fragments (token l%32, k 8(l/32)..+7 of each
// k-half, value and remainder) come from global memory, shared through L2.
// The four wavefronts of a block take interleaved K blocks of the block's K
// range and meet once in LDS; blocks of different K ranges write fp32 partial
// tiles that k_gemm_splitk_sum adds in order and finishes with the epilogue.
// Each wavefront reads its activation fragments itself (4 KB per K block for
// 64 features), so the form pays in L2 traffic what it saves in barriers: it
// is taken for matrices of at most 4096 features, where the tiled grid has
// too few blocks (32 tokens, d = 4096: O 13 vs 18 µs, down 29 vs 41 µs; the
// wider gate/up and QKV matrices are faster on the tiles).
// Loads run D_W K blocks ahead for weights and D_X for activations; K blocks
// past the wavefront's last one re-read it with a zero scale, so the loop has
// one body and no guards.
template <int WT, int FT>
__global__ __launch_bounds__(256) void k_gemm_skinny(QMat W, const uint16_t *Xh, const uint16_t *Xl, int ldx,
                                                     int M, int nsplit, float *part) {
    constexpr int D_W = 4, D_X = 2;
    typedef uint32_t u32x2v __attribute__((ext_vector_type(2)));
    __shared__ __attribute__((aligned(16))) float red[3][FT][16][64];
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, c = lane >> 5, fl = lane & 31;
    const int ngroups = W.N / (32 * FT);
    const int grp = blockIdx.x % ngroups, split = blockIdx.x / ngroups;
    const int nb = W.K >> 5;
    const int kb_lo = (int)((long)nb * split / nsplit), kb_hi = (int)((long)nb * (split + 1) / nsplit);
    // this wavefront's K blocks: kb_lo + w + 4 i, i < nblk
    const int nblk = kb_hi - kb_lo > w ? (kb_hi - kb_lo - w + 3) / 4 : 0;
    const int nblkp = (nblk + D_W - 1) / D_W * D_W;
    const int n0 = grp * 32 * FT;

    const size_t rowb = WT == T_Q4_0 ? (size_t)(W.K >> 1) : (size_t)W.K;
    const uint8_t *qrow[FT];
    const uint16_t *drow[FT];
#pragma unroll
    for (int t = 0; t < FT; t++) {
        const int row = n0 + 32 * t + fl;
        qrow[t] = (const uint8_t *)W.qs + (size_t)row * rowb + 8 * c;
        drow[t] = W.d + (size_t)row * nb;
    }
    const int tok = min(fl, M - 1);
    const uint16_t *xh_row = Xh + (size_t)tok * ldx + 8 * c;
    const uint16_t *xl_row = Xl + (size_t)tok * ldx + 8 * c;

    // (clamped into the block's range: a wavefront with no K block re-reads
    // the range's last one, with a zero scale)
    auto kb_of = [&](int i) __attribute__((always_inline)) {
        return min(kb_lo + w + 4 * min(i, max(nblk - 1, 0)), kb_hi - 1);
    };
    struct WSlot { u32x2v q[FT][WT == T_Q4_0 ? 1 : 2]; uint32_t d[FT]; };
    struct XSlot { u32x4 h[2], l[2]; };
    auto wload = [&](WSlot &sl, int i) __attribute__((always_inline)) {
        const int kb = kb_of(i);
#pragma unroll
        for (int t = 0; t < FT; t++) {
            if (WT == T_Q4_0) {
                sl.q[t][0] = *(const u32x2v *)(qrow[t] + (size_t)kb * 16);
            } else {
                sl.q[t][0] = *(const u32x2v *)(qrow[t] + (size_t)kb * 32);
                sl.q[t][WT == T_Q4_0 ? 0 : 1] = *(const u32x2v *)(qrow[t] + (size_t)kb * 32 + 16);
            }
            sl.d[t] = drow[t][kb];
        }
    };
    auto xload = [&](XSlot &sl, int i) __attribute__((always_inline)) {
        const int kb = kb_of(i);
#pragma unroll
        for (int h = 0; h < 2; h++) {
            sl.h[h] = *(const u32x4 *)(xh_row + (size_t)kb * 32 + 16 * h);
            sl.l[h] = *(const u32x4 *)(xl_row + (size_t)kb * 32 + 16 * h);
        }
    };

    f16x acc[FT];
#pragma unroll
    for (int t = 0; t < FT; t++)
#pragma unroll
        for (int r = 0; r < 16; r++) acc[t][r] = 0.f;

    WSlot ws[D_W];
    XSlot xs[D_X];
#pragma unroll
    for (int j = 0; j < D_W; j++) wload(ws[j], j);
#pragma unroll
    for (int j = 0; j < D_X; j++) xload(xs[j], j);

    for (int i0 = 0; i0 < nblkp; i0 += D_W) {
#pragma unroll
        for (int j = 0; j < D_W; j++) {
            const int i = i0 + j;
            const XSlot &x = xs[j % D_X];
            const h8 xh0 = __builtin_bit_cast(h8, x.h[0]), xh1 = __builtin_bit_cast(h8, x.h[1]);
            const h8 xl0 = __builtin_bit_cast(h8, x.l[0]), xl1 = __builtin_bit_cast(h8, x.l[1]);
#pragma unroll
            for (int t = 0; t < FT; t++) {
                h8 b0, b1;
                if (WT == T_Q4_0)
                    q4_codes(ws[j].q[t][0], b0, b1);
                else
                    q8_codes(u32x4{ws[j].q[t][0].x, ws[j].q[t][0].y, ws[j].q[t][WT == T_Q4_0 ? 0 : 1].x,
                                   ws[j].q[t][WT == T_Q4_0 ? 0 : 1].y}, b0, b1);
                f16x tmp = __builtin_amdgcn_mfma_f32_32x32x16_f16(xh0, b0, f16x{}, 0, 0, 0);
                tmp = __builtin_amdgcn_mfma_f32_32x32x16_f16(xl0, b0, tmp, 0, 0, 0);
                tmp = __builtin_amdgcn_mfma_f32_32x32x16_f16(xh1, b1, tmp, 0, 0, 0);
                tmp = __builtin_amdgcn_mfma_f32_32x32x16_f16(xl1, b1, tmp, 0, 0, 0);
                // past the last block: no contribution (the select is on the
                // index, so it does not wait for the scale's load)
                const float sc = f16_bits_to_f32((uint16_t)ws[j].d[t]) * (i < nblk ? 1.f : 0.f);
#pragma unroll
                for (int r = 0; r < 16; r++) acc[t][r] += sc * tmp[r];
            }
            xload(xs[j % D_X], i + D_X);
            wload(ws[j], i + D_W);
        }
    }

    // the four wavefronts' partial tiles meet in LDS; wavefront 0 writes
    if (w > 0) {
#pragma unroll
        for (int t = 0; t < FT; t++)
#pragma unroll
            for (int r = 0; r < 16; r++) red[w - 1][t][r][lane] = acc[t][r];
    }
    __syncthreads();
    if (w != 0) return;
#pragma unroll
    for (int t = 0; t < FT; t++)
#pragma unroll
        for (int r = 0; r < 16; r++) {
            const float v = acc[t][r] + red[0][t][r][lane] + red[1][t][r][lane] + red[2][t][r][lane];
            const int m = (r >> 2) * 8 + c * 4 + (r & 3);
            if (m < M) part[((size_t)split * M + m) * W.N + n0 + 32 * t + fl] = v;
        }
}

int g_gemm_cu = 256;
int g_gemm_f16w = 0;   // f16 operands for ubatches of more than 64 tokens (opt-in)
int g_gemm_skinny = 1; // skinny form for ubatches of at most 32 tokens
int g_gemm_dl = 23;    // direct-to-LDS form variant (0: off)
int g_gemm_dls = 1;    // direct-to-LDS form with 32-token tiles for at most 32 tokens (0: skinny / tiles)
int g_gemm_dls_ns = 4; // its LDS stages
int g_gemm_dls_fill = 4; // its K split aims at this many blocks per 4 compute units
int g_gemm_ws = 2;     // weight-streaming form for Q4_0 at most 32 tokens: K blocks per stage (0: off)
int g_gemm_dw = 1;     // wide direct-to-LDS form for Q4_0 / Q8_0 / Q4_K ubatches of more than 64 tokens (0: off)

bool mfma_shape(const QMat &W, int ldx) {
    return (W.wtype == T_Q4_0 || W.wtype == T_Q8_0) && W.N % BN == 0 && W.K % 32 == 0 && ldx % 8 == 0;
}

// K splits for M tokens: only when the tile grid leaves resident block slots
// (2 per CU) empty, the largest of 2 and 4 that still fits one round of
// slots, each split keeping >= 16 K blocks.  (Splitting a grid that already
// fills the chip only adds partial-tile traffic.)
// Token tile: 256 with f16 operands from 256 tokens on, else 128 above 64 tokens, else 64.
int tile_m(int M) { return g_gemm_f16w && M >= 256 ? 256 : M > 64 ? 128 : 64; }

// Skinny form: 64 features per block; K ranges so that the grid has about
// two blocks per compute unit and each wavefront at least 4 K blocks.
constexpr int SK_FT = 2;
int skinny_splits(const QMat &W) {
    const int groups = W.N / (32 * SK_FT), nb = W.K / 32;
    int S = (2 * g_gemm_cu + groups - 1) / groups;
    S = std::min(S, std::max(1, nb / 16));
    return std::max(1, std::min(S, 64));
}

int split_for(const QMat &W, int M) {
    const int bm = tile_m(M);
    const long tiles = (long)(W.N / BN) * ((M + bm - 1) / bm);
    const long slots = 2L * g_gemm_cu;
    const int nb = W.K / 32;
    int best = 1;
    for (int S = 2; S <= 4; S *= 2)
        if (tiles * S <= slots && nb % S == 0 && nb / S >= 16) best = S;
    return best;
}

template <int WT, int EPI, int BM, bool SPLIT>
void launch_mfma_tile(const QMat &W, const uint16_t *Xh, const uint16_t *Xl, int ldx, const EpiArgs &ep,
                      int M, int pair_mode, int S, float *ws, dim3 grid, bool f16w, hipStream_t s) {
    const int NT = W.N / BN;
    float *part = SPLIT ? ws : nullptr;
    if (f16w)
        launch((k_gemm_mfma<WT, BM, EPI, SPLIT, true>), grid, dim3(256), 0, s, W, Xh, Xl, ldx, ep, M, pair_mode,
               NT, S, part);
    else if constexpr (BM <= 128)   // exact operands: tiles of up to 128 tokens
        launch((k_gemm_mfma<WT, BM, EPI, SPLIT, false>), grid, dim3(256), 0, s, W, Xh, Xl, ldx, ep, M, pair_mode,
               NT, S, part);
}

template <int WT, int EPI>
void launch_mfma_epi(const QMat &W, const uint16_t *Xh, const uint16_t *Xl, int ldx, const EpiArgs &ep,
                     int M, int pair_mode, int S, float *ws, hipStream_t s) {
    const int NT = W.N / BN, NT8 = (NT + 7) / 8 * 8;
    const int bm = tile_m(M);
    const dim3 grid(NT8 * ((M + bm - 1) / bm) * S);
    // f16 operands for ubatches of more than 64 tokens; exact operands below
    const bool f16w = g_gemm_f16w && bm >= 128;
    if (S > 1) {
        if (bm == 256)
            launch_mfma_tile<WT, EPI, 256, true>(W, Xh, Xl, ldx, ep, M, pair_mode, S, ws, grid, true, s);
        else if (bm == 128)
            launch_mfma_tile<WT, EPI, 128, true>(W, Xh, Xl, ldx, ep, M, pair_mode, S, ws, grid, f16w, s);
        else
            launch_mfma_tile<WT, EPI, 64, true>(W, Xh, Xl, ldx, ep, M, pair_mode, S, ws, grid, false, s);
        launch_sum(EPI, (const float *)ws, S, W.N, M, ep, pair_mode, s);
    } else if (bm == 256) {
        launch_mfma_tile<WT, EPI, 256, false>(W, Xh, Xl, ldx, ep, M, pair_mode, 1, ws, grid, true, s);
    } else if (bm == 128) {
        launch_mfma_tile<WT, EPI, 128, false>(W, Xh, Xl, ldx, ep, M, pair_mode, 1, ws, grid, f16w, s);
    } else {
        launch_mfma_tile<WT, EPI, 64, false>(W, Xh, Xl, ldx, ep, M, pair_mode, 1, ws, grid, false, s);
    }
}

template <int WT>
void launch_mfma(const QMat &W, const uint16_t *Xh, const uint16_t *Xl, int ldx, const EpiArgs &ep,
                 int M, int pair_mode, int S, float *ws, hipStream_t s) {
    switch (ep.epi) {
    case EPI_STORE: launch_mfma_epi<WT, EPI_STORE>(W, Xh, Xl, ldx, ep, M, pair_mode, S, ws, s); break;
    case EPI_RESID: launch_mfma_epi<WT, EPI_RESID>(W, Xh, Xl, ldx, ep, M, pair_mode, S, ws, s); break;
    case EPI_QKV: launch_mfma_epi<WT, EPI_QKV>(W, Xh, Xl, ldx, ep, M, pair_mode, S, ws, s); break;
    case EPI_SWIGLU: launch_mfma_epi<WT, EPI_SWIGLU>(W, Xh, Xl, ldx, ep, M, pair_mode, S, ws, s); break;
    }
}

template <int EPI>
void launch_f32_epi(const QMat &W, const uint16_t *Xh, const uint16_t *Xl, int ldx, const EpiArgs &ep,
                    int M, int pair_mode, hipStream_t s) {
    launch(k_gemm_f32<EPI>, dim3((W.N / 2 + 255) / 256, M), dim3(256), 0, s, W, Xh, Xl, ldx,
                       ep, M, pair_mode);
}

template <int WT>
bool launch_plainq(const QMat &W, const uint16_t *Xh, const uint16_t *Xl, int ldx, const EpiArgs &ep, int M,
                   int pair_mode, hipStream_t s) {
    const dim3 g((W.N / 2 + 255) / 256, M);
    switch (ep.epi) {
    case EPI_STORE: launch(k_gemm_plainq<WT, EPI_STORE>, g, dim3(256), 0, s, W, Xh, Xl, ldx, ep, M, pair_mode); break;
    case EPI_RESID: launch(k_gemm_plainq<WT, EPI_RESID>, g, dim3(256), 0, s, W, Xh, Xl, ldx, ep, M, pair_mode); break;
    case EPI_QKV: launch(k_gemm_plainq<WT, EPI_QKV>, g, dim3(256), 0, s, W, Xh, Xl, ldx, ep, M, pair_mode); break;
    case EPI_SWIGLU: launch(k_gemm_plainq<WT, EPI_SWIGLU>, g, dim3(256), 0, s, W, Xh, Xl, ldx, ep, M, pair_mode); break;
    default: return false;
    }
    return true;
}

// The transposed scale array the direct-to-LDS forms read (dt, Q4_K sf).
static bool has_gemm_scales(const QMat &W) { return W.wtype == T_Q4_K ? W.sf != nullptr : W.dt != nullptr; }

// Direct-to-LDS form (gemm_dl.hip): ubatches of more than 64 tokens with the
// exact operands (Q4_K: any ubatch, it has no other MFMA form), feature
// counts that are whole 256-feature tiles.
bool dl_shape(const QMat &W, int M, int ldx) {
    // the direct loads address operands by 32-bit byte offsets from a base
    const size_t row_bytes = W.wtype == T_Q8_0 ? (size_t)W.K : (size_t)W.K / 2;
    const bool k4 = W.wtype == T_Q4_K;
    return g_gemm_dl > 0 && has_gemm_scales(W) && (k4 || (!g_gemm_f16w && M > 64)) &&
           W.N % gemm_dl_tile_features() == 0 &&
           (size_t)M * ldx * 2 < ((size_t)1 << 31) && (size_t)W.N * row_bytes < ((size_t)1 << 31) &&
           (size_t)M * (W.K / 32) * 4 < ((size_t)1 << 31);
}

// The wide form (Q4_0, Q8_0, Q4_K): more than 64 tokens, whole 512-feature
// tiles, K in whole periods of code super-stages.
bool dw_shape(const QMat &W, int M, int ldx) {
    const size_t row_bytes = W.wtype == T_Q8_0 ? (size_t)W.K : (size_t)W.K / 2;
    return g_gemm_dw && g_gemm_dl > 0 && !g_gemm_f16w &&
           (W.wtype == T_Q4_0 || W.wtype == T_Q8_0 || W.wtype == T_Q4_K) && has_gemm_scales(W) && M > 64 &&
           W.N % gemm_dw_tile_features() == 0 && (W.K / 32) % gemm_dw_super_blocks() == 0 &&
           (size_t)M * ldx * 2 < ((size_t)1 << 31) && (size_t)W.N * row_bytes < ((size_t)1 << 31);
}

thread_local int g_dw_split_cap = 8;   // gemm_set_split_cap

// Its K split S (1, 2, 4 or 8, at most g_dw_split_cap): the blocks are the (feature tile, split)
// units times the token tiles, units spread evenly over the 8 XCDs, and an
// XCD's share must fit one block per compute unit; splits take whole periods
// (4 K blocks; Q4_K octets) and at least 16 K blocks.  The largest such S
// wins.  (Uneven splits that fill more compute units, e.g. 5 for the 8B QKV
// matrix, gain alone but lose once two prefill lanes share the chip: their
// extra fp32 partials then cost more than the idle units.  For the same
// reason the engine caps S at 4 while lanes run.)
int dw_split(const QMat &W, int M) {
    const int NT = W.N / gemm_dw_tile_features(), mtiles = (M + 127) / 128;
    const int nb = W.K / 32;
    const int unit = W.wtype == T_Q4_K ? 8 : gemm_dw_super_blocks();
    const int P = nb / unit;
    const int per_xcd = g_gemm_cu / 8;
    int best = 1;
    for (int S = 2; S <= g_dw_split_cap; S *= 2)
        if ((NT * S + 7) / 8 * mtiles <= per_xcd && P % S == 0 && nb / S >= 16) best = S;
    return best;
}

// The 32-token direct-to-LDS form: at most 32 tokens, whole 256-feature tiles.
bool dls_shape(const QMat &W, int M, int ldx) {
    const size_t row_bytes = W.wtype == T_Q8_0 ? (size_t)W.K : (size_t)W.K / 2;
    return (g_gemm_dls || W.wtype == T_Q4_K) && g_gemm_dl > 0 && has_gemm_scales(W) && M > 0 &&
           M <= gemm_dls_tile_tokens() &&
           W.wtype != T_F32 && W.N % gemm_dl_tile_features() == 0 && ldx % 8 == 0 &&
           (size_t)M * ldx * 2 < ((size_t)1 << 31) && (size_t)W.N * row_bytes < ((size_t)1 << 31);
}

// Its K split: doubled while the grid holds fewer than g_gemm_dls_fill blocks
// per 4 compute units and every split keeps at least 4 K blocks (splits may
// be uneven).
int dls_split(const QMat &W, int M) {
    const long tiles = (long)(W.N / gemm_dl_tile_features()) *
                       ((M + gemm_dls_tile_tokens() - 1) / gemm_dls_tile_tokens());
    const int nb = W.K / 32;
    int S = 1;
    while (S < 64 && tiles * S * 4 < (long)g_gemm_dls_fill * g_gemm_cu && nb / (2 * S) >= 4) S *= 2;
    return S;
}

// The weight-streaming form (Q4_0, at most 32 tokens, K and N whole 256s).
bool ws_shape(const QMat &W, int M, int ldx) {
    return g_gemm_ws && g_gemm_dls && W.wtype == T_Q4_0 && M > 0 && M <= 32 && W.K % 256 == 0 &&
           W.N % gemm_dl_tile_features() == 0 && ldx % 8 == 0 && (size_t)M * ldx * 2 < ((size_t)1 << 31) &&
           (size_t)W.N * (W.K / 2) < ((size_t)1 << 31);
}

// Its K split, in whole octets of K blocks with at most
// gemm_ws_max_blocks_per_split() K blocks per split: the fewest splits whose
// grid fills half the resident block slots (2 per compute unit with 2 K
// blocks per stage, 1 with 4).  More splits shorten each block's stream but
// add fp32 partial tiles (S x M x N x 4 bytes written and read back), which
// at 32 tokens weigh as much as the codes of several K blocks.
int ws_split(const QMat &W, int M) {
    const long tiles = (long)(W.N / gemm_dl_tile_features()) * ((M + 31) / 32);
    const int no = W.K / 256, per = gemm_ws_max_blocks_per_split() / 8;
    const long slots = (long)(g_gemm_ws == 2 ? 2 : 1) * g_gemm_cu;
    int S = (no + per - 1) / per;
    while (S < no && tiles * S * 2 < slots) S++;
    return S;
}

// Bytes of the Q4_K block sums at the start of the workspace.
size_t q4k_sums_bytes(const QMat &W, int M) { return ((size_t)M * (W.K / 32) * 4 + 255) / 256 * 256; }

int dl_split(const QMat &W, int M) {
    const long tiles = (long)(W.N / gemm_dl_tile_features()) *
                       ((M + gemm_dl_tile_tokens() - 1) / gemm_dl_tile_tokens());
    const long slots = (g_gemm_dl == 4 && W.wtype != T_Q4_K ? 1L : 2L) * g_gemm_cu;
    const int nb = W.K / 32;
    int best = 1;
    for (int S = 2; S <= 8; S *= 2)
        if (tiles * S <= slots && nb % S == 0 && nb / S >= 16 && (W.wtype != T_Q4_K || (nb / S) % 8 == 0)) best = S;
    return best;
}

}  // namespace

void gemm_set_split_cap(int cap) { g_dw_split_cap = cap >= 8 ? 8 : cap >= 4 ? 4 : cap >= 2 ? 2 : 1; }

void gemm_set_num_cu(int n) {
    g_gemm_cu = n > 0 ? n : 256;
    const char *e = getenv("DECODE_GEMM_F16");
    g_gemm_f16w = e && strcmp(e, "1") == 0;
    const char *k = getenv("DECODE_GEMM_SKINNY");
    g_gemm_skinny = !(k && strcmp(k, "0") == 0);
    // DECODE_GEMM_DL: 0 keeps the register-staged tiles; 3 or 4 picks the
    // direct-to-LDS form with that many stages on 32x32 tiles, 13 three stages
    // on 16x16 tiles, 23 three stages with 64-feature wavefront tiles
    // (default 23)
    const char *dl = getenv("DECODE_GEMM_DL");
    g_gemm_dl = 23;
    if (dl) {
        const int v = atoi(dl);
        g_gemm_dl = (v == 0 || v == 3 || v == 4 || v == 13 || v == 23) ? v : 23;
    }
    // DECODE_GEMM_SMALL: "tiles" keeps the skinny form / register-staged
    // tiles for ubatches of at most 32 tokens; else the 32-token direct-to-LDS
    // form with DECODE_GEMM_DLS_NS stages (4, 6 or 8; default 4) and a K
    // split for DECODE_GEMM_DLS_FILL blocks per 4 compute units (default 4)
    const char *sm = getenv("DECODE_GEMM_SMALL");
    g_gemm_dls = !(sm && strcmp(sm, "tiles") == 0);
    const char *ns = getenv("DECODE_GEMM_DLS_NS");
    g_gemm_dls_ns = 4;
    if (ns) {
        const int v = atoi(ns);
        g_gemm_dls_ns = (v == 4 || v == 6 || v == 8) ? v : 4;
    }
    const char *fl = getenv("DECODE_GEMM_DLS_FILL");
    g_gemm_dls_fill = fl && atoi(fl) > 0 ? atoi(fl) : 4;
    // DECODE_GEMM_WS: K blocks per stage of the weight-streaming form (2 or 4,
    // default 2); 0 leaves Q4_0 ubatches of at most 32 tokens to the 32-token
    // direct-to-LDS form
    // DECODE_GEMM_DW=0: Q4_0 / Q8_0 / Q4_K ubatches of more than 64 tokens take the
    // 256-feature direct-to-LDS form instead of the wide one
    const char *dwv = getenv("DECODE_GEMM_DW");
    g_gemm_dw = !(dwv && strcmp(dwv, "0") == 0);
    const char *wsv = getenv("DECODE_GEMM_WS");
    g_gemm_ws = 2;
    if (wsv) g_gemm_ws = atoi(wsv) == 0 ? 0 : atoi(wsv) == 4 ? 4 : 2;
}

void launch_gemm_scales(QMat &m, hipStream_t s) {
    const long long n = (long long)m.N * (m.K / 32);
    if (m.wtype == T_Q4_K)
        launch(k_q4k_mins, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, m);
    else if (m.dt)
        launch(k_scales_t, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, m);
}

void launch_block_sums(const uint16_t *Xh, const uint16_t *Xl, int ldx, int M, int K, float *xs, hipStream_t s) {
    const long long n = (long long)M * (K / 32);
    launch(k_block_sums, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, Xh, Xl, ldx, M, K, xs);
}

namespace {
// The plain K-split sum + epilogue.
void launch_sum(int epi, const float *ws, int S, int N, int M, const EpiArgs &ep, int pair_mode, hipStream_t s) {
    const dim3 g((N / 2 + 255) / 256, M);
    switch (epi) {
    case EPI_STORE: launch(k_gemm_splitk_sum<EPI_STORE>, g, dim3(256), 0, s, ws, S, N, M, ep, pair_mode); break;
    case EPI_RESID: launch(k_gemm_splitk_sum<EPI_RESID>, g, dim3(256), 0, s, ws, S, N, M, ep, pair_mode); break;
    case EPI_QKV: launch(k_gemm_splitk_sum<EPI_QKV>, g, dim3(256), 0, s, ws, S, N, M, ep, pair_mode); break;
    case EPI_SWIGLU: launch(k_gemm_splitk_sum<EPI_SWIGLU>, g, dim3(256), 0, s, ws, S, N, M, ep, pair_mode); break;
    }
}
}  // namespace

void launch_splitk_sum(int epi, const float *ws, int S, int N, int M, const EpiArgs &ep, int pair_mode,
                       hipStream_t s) {
    if (epi == EPI_RESID && ep.nrm_g && ep.nrm_done) {
        if (N % 4 == 0 && ep.ldy % 4 == 0)
            launch(k_splitk_resid_norm<4>, dim3(M), dim3(SRN_T), 0, s, ws, S, N, M, ep);
        else
            launch(k_splitk_resid_norm<1>, dim3(M), dim3(SRN_T), 0, s, ws, S, N, M, ep);
        *ep.nrm_done = 1;
        return;
    }
    launch_sum(epi, ws, S, N, M, ep, pair_mode, s);
}

size_t gemm_workspace_bytes(const QMat &W, int M) {
    const int ms = M < gemm_dls_tile_tokens() ? M : gemm_dls_tile_tokens();
    size_t small = 0;   // the 32-token forms, for any ubatch of at most min(M, 32) tokens
    if (M > 0 && dls_shape(W, ms, W.K)) {
        const int Ss = dls_split(W, ms);
        small = Ss > 1 ? (size_t)Ss * ms * W.N * 4 : 0;
    }
    if (M > 0 && ws_shape(W, ms, W.K)) {
        const int Sw = ws_split(W, ms);
        small = std::max(small, Sw > 1 ? (size_t)Sw * ms * W.N * 4 : (size_t)0);
    }
    if (M > 0 && W.wtype == T_Q4_K) {
        if (!dl_shape(W, M, W.K)) return 0;
        const int Sd = dl_split(W, M);
        size_t tile = Sd > 1 ? (size_t)Sd * M * W.N * 4 : (size_t)0;
        if (dw_shape(W, M, W.K)) {
            const int Sw = dw_split(W, M);
            tile = std::max(tile, Sw > 1 ? (size_t)Sw * M * W.N * 4 : (size_t)0);
        }
        return q4k_sums_bytes(W, M) + std::max(small, tile);
    }
    if (M <= 0 || !mfma_shape(W, 8)) return 0;
    const int S = split_for(W, M);
    size_t tile = S > 1 ? (size_t)S * M * W.N * 4 : 0;
    if (dl_shape(W, M, W.K)) {
        const int Sd = dl_split(W, M);
        tile = std::max(tile, Sd > 1 ? (size_t)Sd * M * W.N * 4 : (size_t)0);
    }
    if (dw_shape(W, M, W.K)) {
        const int Sw = dw_split(W, M);
        tile = std::max(tile, Sw > 1 ? (size_t)Sw * M * W.N * 4 : (size_t)0);
    }
    tile = std::max(tile, small);
    // the skinny form, for any ubatch of at most min(M, 32) tokens
    return W.N <= 4096 ? std::max(tile, (size_t)skinny_splits(W) * ms * W.N * 4) : tile;
}

bool launch_gemm(const QMat &W, const uint16_t *Xh, const uint16_t *Xl, int ldx, const EpiArgs &ep,
                 int M, float *ws, size_t ws_bytes, hipStream_t s) {
    if (M <= 0 || W.N % 2 || !Xh || !Xl) return false;
    const int pair_mode = ep.epi == EPI_SWIGLU ? PAIR_GU : PAIR_ADJ;
    if (pair_mode == PAIR_GU && W.N % 64) return false;
    if (W.wtype == T_Q4_K) {
        const size_t xsb = q4k_sums_bytes(W, M);
        if (ldx % 8 == 0 && dl_shape(W, M, ldx) && ws && ws_bytes >= xsb) {
            float *part = ws + xsb / 4;
            const bool small = dls_shape(W, M, ldx), wide = !small && dw_shape(W, M, ldx);
            int S = small ? dls_split(W, M) : wide ? dw_split(W, M) : dl_split(W, M);
            while (S > 1 && (size_t)S * M * W.N * 4 > ws_bytes - xsb) S >>= 1;
            launch_block_sums(Xh, Xl, ldx, M, W.K, ws, s);
            if (small)
                launch_gemm_dls(g_gemm_dls_ns, W, Xh, Xl, ldx, ep, M, pair_mode, S, part, ws, s);
            else if (wide)
                launch_gemm_dw(W, Xh, Xl, ldx, ep, M, pair_mode, S, part, ws, s);
            else
                launch_gemm_dl(23, W, Xh, Xl, ldx, ep, M, pair_mode, S, part, ws, s);
            return true;
        }
        return launch_plainq<T_Q4_K>(W, Xh, Xl, ldx, ep, M, pair_mode, s);
    }
    // weight-streaming form (Q4_0), else the 32-token direct-to-LDS form, for
    // at most 32 tokens
    if (ws_shape(W, M, ldx)) {
        const int S = ws_split(W, M);
        if (S == 1 || (ws && (size_t)S * M * W.N * 4 <= ws_bytes)) {
            launch_gemm_ws(g_gemm_ws, W, Xh, Xl, ldx, ep, M, pair_mode, S, ws, s);
            return true;
        }
    }
    if (mfma_shape(W, ldx) && dls_shape(W, M, ldx) && g_gemm_dls) {
        int S = dls_split(W, M);
        while (S > 1 && (!ws || (size_t)S * M * W.N * 4 > ws_bytes)) S >>= 1;
        launch_gemm_dls(g_gemm_dls_ns, W, Xh, Xl, ldx, ep, M, pair_mode, S, ws, nullptr, s);
        return true;
    }
    // skinny form for at most 32 tokens and at most 4096 features: there the
    // tiled grid is too small to spread over the chip (wider matrices stay
    // on the tiles, whose LDS-shared activations cost less L2 traffic)
    if (mfma_shape(W, ldx) && M <= 32 && W.N <= 4096 && g_gemm_skinny && W.N % (32 * SK_FT) == 0) {
        const int S = skinny_splits(W);
        if (ws && (size_t)S * M * W.N * 4 <= ws_bytes) {
            const int groups = W.N / (32 * SK_FT);
            if (W.wtype == T_Q4_0)
                launch((k_gemm_skinny<T_Q4_0, SK_FT>), dim3(groups * S), dim3(256), 0, s, W, Xh, Xl, ldx, M, S, ws);
            else
                launch((k_gemm_skinny<T_Q8_0, SK_FT>), dim3(groups * S), dim3(256), 0, s, W, Xh, Xl, ldx, M, S, ws);
            if (ep.epi != EPI_STORE && ep.epi != EPI_RESID && ep.epi != EPI_QKV && ep.epi != EPI_SWIGLU) return false;
            launch_sum(ep.epi, (const float *)ws, S, W.N, M, ep, pair_mode, s);
            return true;
        }
    }
    if (mfma_shape(W, ldx) && dw_shape(W, M, ldx)) {
        int S = dw_split(W, M);
        while (S > 1 && (!ws || (size_t)S * M * W.N * 4 > ws_bytes)) S >>= 1;
        launch_gemm_dw(W, Xh, Xl, ldx, ep, M, pair_mode, S, ws, nullptr, s);
        return true;
    }
    if (mfma_shape(W, ldx) && dl_shape(W, M, ldx)) {
        int S = dl_split(W, M);
        while (S > 1 && (!ws || (size_t)S * M * W.N * 4 > ws_bytes)) S >>= 1;
        launch_gemm_dl(g_gemm_dl, W, Xh, Xl, ldx, ep, M, pair_mode, S, ws, nullptr, s);
        return true;
    }
    if (mfma_shape(W, ldx)) {
        int S = split_for(W, M);
        while (S > 1 && (!ws || (size_t)S * M * W.N * 4 > ws_bytes)) S >>= 1;
        if (W.wtype == T_Q4_0)
            launch_mfma<T_Q4_0>(W, Xh, Xl, ldx, ep, M, pair_mode, S, ws, s);
        else
            launch_mfma<T_Q8_0>(W, Xh, Xl, ldx, ep, M, pair_mode, S, ws, s);
        return true;
    }
    if (W.wtype == T_Q4_0) return launch_plainq<T_Q4_0>(W, Xh, Xl, ldx, ep, M, pair_mode, s);
    if (W.wtype == T_Q8_0) return launch_plainq<T_Q8_0>(W, Xh, Xl, ldx, ep, M, pair_mode, s);
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
