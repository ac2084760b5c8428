// mvcore.h -- pieces of the dequant-fused block-quantized mat-vec shared by
// the per-matrix kernel (matvec.hip) and the persistent decode-step kernel
// (step.hip): code extraction into exact f16 values, block dot products,
// per-lane code loads of a row pair, and the LDS image of the input row.
#pragma once

#include "common.h"
#include "kernels.h"

namespace {

// Activation pairs in the order the code extraction produces them.
// Q4_0 block dword i (bytes 4i..4i+3): byte k holds code 4i+k in its low
// nibble and code 16+4i+k in its high nibble.  Masking a dword with
// 0x000F000F / 0x00F000F0 and or-ing the f16 exponent of 1024 gives the f16
// pairs (1024 + q[4i], 1024 + q[4i+2]) and (1024 + 16 q[4i+16], 1024 + 16
// q[4i+18]) directly; the same masks on the dword shifted right by 8 give
// codes 4i+1, 4i+3 and 16 q[4i+17], 16 q[4i+19].  All these values are exact
// in f16.  So activation pairs 4i+0..3 are (x[4i], x[4i+2]), (x[16+4i],
// x[16+4i+2]), (x[4i+1], x[4i+3]), (x[16+4i+1], x[16+4i+3]).
// Q8_0 block dword i holds codes 4i..4i+3; after flipping the sign bits,
// masks 0x00FF00FF at shifts 0 and 8 select (4i, 4i+2) and (4i+1, 4i+3):
// activation pair 2i is (x[4i], x[4i+2]), pair 2i+1 is (x[4i+1], x[4i+3]).

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
DEV float blockdot_q4(const u32x4 q, const h2 *xp, const Masks &m) {
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
DEV float blockdot_q8(const u32x4 q0, const u32x4 q1, const h2 *xp, const Masks &m) {
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

constexpr int MV_KMAX = 16384;   // longest input row (elements); its LDS image holds 512 blocks

// Code bytes + scales of one pair of rows for this lane's blocks.  Q4_K
// blocks are sub-blocks: codes as in Q4_0, `d` holds the six-bit scale and
// min (sc | m << 8), `dm` the super-block's f16 d and dmin.
template <int WT, int KB>
struct PairLoad {
    u32x4 q[2][KB][WT == T_Q8_0 ? 2 : 1];
    uint32_t d[2][KB];     // the aligned dword holding the block's f16 scale ...
    uint32_t dsh[2][KB];   // ... at this bit offset
    uint32_t dm[2][WT == T_Q4_K ? KB : 1];
};

// Blocks b0 + lane + 64*i (i < KB) of rows r0, r1; lanes past the slice end
// b1 re-read its last block (their activations are zero), so every load is
// unconditional and nothing here waits for a load: a select
// on a loaded value at issue time would make the wavefront wait for the
// loads it has just requested.
template <int WT, int KB>
DEV void load_pair(const QMat &W, int r0, int r1, int b0, int b1, int lane, PairLoad<WT, KB> &L) {
    const int K = W.K, nb = K >> 5;
    const int rows[2] = {r0, r1};
#pragma unroll
    for (int r = 0; r < 2; r++) {
        const GLB u32x4 *qr = WT != T_Q8_0
                                  ? (const GLB u32x4 *)((const GLB uint8_t *)gl(W.qs) + (size_t)rows[r] * (K >> 1))
                                  : (const GLB u32x4 *)((const GLB int8_t *)gl(W.qs) + (size_t)rows[r] * K);
#pragma unroll
        for (int i = 0; i < KB; i++) {
            const int bw = b0 + lane + 64 * i;
            const int b = bw < b1 ? bw : b1 - 1;
            // streaming loads: the weights are read once per step
            if (WT != T_Q8_0) {
                L.q[r][i][0] = __builtin_nontemporal_load(qr + b);
            } else {
                L.q[r][i][0] = __builtin_nontemporal_load(qr + 2 * b);
                L.q[r][i][WT == T_Q8_0 ? 1 : 0] = __builtin_nontemporal_load(qr + 2 * b + 1);
            }
            const size_t e = (size_t)rows[r] * nb + b;   // W.d is 256-byte aligned
            L.d[r][i] = *(const GLB uint32_t *)(gl(W.d) + (e & ~(size_t)1));
            L.dsh[r][i] = (uint32_t)(e & 1) * 16;
            if constexpr (WT == T_Q4_K) L.dm[r][i] = gl(W.dm)[(size_t)rows[r] * (K >> 8) + (b >> 3)];
        }
    }
}

constexpr int XROW = 36;   // dwords per LDS image row: 32 pairs + 4 pad (conflict-free 16-byte reads)

// LDS image of the input row, built once per block: per 32-element quant
// block, 16 value pairs then 16 remainder pairs (f16x2) in the order the code
// extraction consumes them (the pair order above), padded to XROW dwords,
// plus the block's offset sum.
DEV uint32_t pk(f16 a, f16 b) { return h2_bits(h2{a, b}); }

// Elements 4g..4g+3 of block b (value hv, remainder lv) -> their image
// pairs, and their share of the block's offset sum.  Q4_0: a group of the
// low half (g < 4) gives pairs 4g and 4g+2, of the high half (g = 4 + i)
// pairs 4i+1 and 4i+3; Q8_0: pairs 2g and 2g+1.  The offsets are removed once
// per block: Q4_0 keeps 1024 + q on codes 0..15 and (1024 + 16 q) / 16 on
// codes 16..31, so sum (q - 8) x needs 1032 * sum(x[0..15]) + 72 *
// sum(x[16..31]) subtracted; Q8_0 keeps 1024 + 128 + q everywhere.
// Q4_K sub-blocks take the Q4_0 image with offsets 1024 (low nibbles) and
// 64 (high nibbles) only, since their codes are 0..15 without a shift; their
// min term needs the plain sum of the block's x, returned in *plain.
template <int WT>
DEV float put_group(uint32_t *img, int b, int g, const f16 *hv, const f16 *lv, float *plain = nullptr) {
    uint32_t *row = img + (size_t)b * XROW;
    int p0, p1;
    if (WT != T_Q8_0) {
        p0 = g < 4 ? 4 * g : 4 * (g - 4) + 1;
        p1 = p0 + 2;
    } else {
        p0 = 2 * g;
        p1 = p0 + 1;
    }
    row[p0] = pk(hv[0], hv[2]);
    row[p1] = pk(hv[1], hv[3]);
    row[16 + p0] = pk(lv[0], lv[2]);
    row[16 + p1] = pk(lv[1], lv[3]);
    float sx = 0.f;
#pragma unroll
    for (int e = 0; e < 4; e++) sx += (float)hv[e] + (float)lv[e];
    if (plain) *plain = sx;
    if (WT == T_Q4_K) return sx * (g < 4 ? 1024.f : 64.f);
    return sx * (WT == T_Q8_0 ? 1152.f : (g < 4 ? 1032.f : 72.f));
}

}  // namespace
