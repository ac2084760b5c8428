// gemm_dl.hip -- ubatch GEMM Y = X W^T with direct-to-LDS operand loads (gfx950).
//
// The arithmetic is that of k_gemm_mfma's exact form: weights enter the
// matrix cores as their integer codes (exact in f16), activations as an f16
// value and its f16 rounding remainder, and per 32-wide quant block the four
// v_mfma_f32_32x32x16_f16 of a 32x32 tile (2 k-halves x value/remainder)
// fill a temporary tile that is scaled by the row's block scale and added to
// the fp32 result, C += d[n][kb] * T.  With the same K split the results are
// bitwise those of k_gemm_mfma.
//
// What changes is how operands reach the matrix cores.  Every byte goes from
// global memory straight into LDS (global_load_lds_dwordx4, no register
// staging, no wait at a store): per K block a stage holds the block tile's
// activation values and remainders (128 tokens x 64 bytes each), its raw
// codes (256 rows x 16 or 32 bytes) and its scales (256 x 4 bytes, the f16
// in the low half).  NS
// stages form a ring; K block kb+NS-1 is requested while kb is computed, and
// a wavefront waits only for its own loads of block kb (a constant vmcnt:
// past the last K block the last one is requested again) before the one
// barrier per K block.  Each stage is its own LDS array, so the compiler sees
// that reading one stage does not depend on the loads into another.
// The codes are converted to f16 operands when read (each wavefront converts
// the rows it uses).  Activation rows are 4 chunks of 16 bytes; chunk c of
// token m sits at slot 4m + (c ^ swz(m)), which spreads the 16-byte reads of
// 16 consecutive tokens over distinct bank groups; the direct loads write
// slots in lane order, so each lane simply fetches the chunk its slot holds.
// Code rows are read 16 bytes at a time (conflict-free, where 8-byte reads at
// a 16-byte stride conflict); a Q8_0 row's two 16-byte chunks are swapped in
// rows 8..15 of every 16, for the same reason.
//
// Block: 256 threads, 256 features x 128 tokens; wavefront w covers features
// 128 (w & 1) .. +127 (four 32-feature tiles a) and tokens 64 (w >> 1) .. +63
// (two 32-token tiles b).  Operand layouts as in k_gemm_mfma: lane l supplies
// A[l%32][8(l/32)+e] (tokens) and B[8(l/32)+e][l%32] (features); accumulator r
// of lane l is C[(r/4)*8+(l/32)*4+r%4][l%32], so a lane's 16 accumulators of a
// tile are 16 tokens of one feature and the block scale is one value per tile.
// Feature tiles of one block tile share an XCD (round-robin block placement),
// as in k_gemm_mfma; K splits write fp32 partial tiles summed in order by
// k_gemm_splitk_sum.
//
// Q4_K (256-weight super-blocks of eight 32-weight sub-blocks; weight = d sc q
// - dmin m): the K block is a sub-block.  Its codes (stored in the Q4_0
// nibble layout) enter the matrix cores as exact f16 values q = 0..15, the
// temporary tile T = sum q x is scaled by d sc (an fp32 array derived at load,
// loaded where the f16 scale goes), and the min
// term sum over K blocks of (dmin m) X, with X the token's block sum of x
// (written beforehand by a small kernel), is a product of its own over K/32,
// run on the matrix cores after the main loop straight into the accumulators.
#include <type_traits>

#include "common.h"
#include "epilogue.h"
#include "kernels.h"

namespace {

constexpr int DBN = 256;    // features per block
constexpr int DBM = 128;    // tokens per block (prefill form)
constexpr int DBM_S = 32;   // tokens per block (small-ubatch form)

#define AS1 __attribute__((address_space(1)))
#define AS3 __attribute__((address_space(3)))

typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// Q4_K loads its fp32 sub-block scale d sc (one dword per row) where the f16
// scale goes.
template <int WT, int TM>
struct Geo {
    static constexpr bool K4 = WT == T_Q4_K;
    static constexpr int CB = WT == T_Q8_0 ? 32 : 16;    // code bytes per row and K block
    static constexpr int ACT = TM * 64;                  // one activation part per K block
    static constexpr int OFF_LO = ACT;
    static constexpr int OFF_CODES = 2 * ACT;
    static constexpr int OFF_SC = 2 * ACT + DBN * CB;
    static constexpr int STAGE = OFF_SC + DBN * 4;      // a 2-byte direct load fills one dword per lane
    // direct loads per wavefront and K block: 4 activation (128 tokens) or 1
    // (32 tokens), 1 or 2 code, 1 scale
    static constexpr int LOADS = TM / 32 + DBN * CB / 4096 + 1;
};

// Slot of chunk c of token row m (see the header): the 16-byte reads of a
// quarter wavefront (16 consecutive tokens, one chunk each) then fall into 16
// distinct groups of 4 banks (checked with the bank-conflict counter: no
// conflicts, against 75% of LDS cycles without the swizzle).
DEV int swz(int m) { return (m >> 2) & 3; }

DEV h2 magic_lo(uint32_t v) { return as_h2(__builtin_amdgcn_perm(0x64646464u, v, 0x04010400u)); }
DEV h2 magic_hi(uint32_t v) { return as_h2(__builtin_amdgcn_perm(0x64646464u, v, 0x04030402u)); }

// Q4_0: 8 bytes holding codes 8c..8c+7 (low nibbles) and 16+8c..16+8c+7 (high
// nibbles) -> exact f16 values q - 8 of the two k-halves.
DEV void q4_pair(u32x2 raw, h8 &k0, h8 &k1) {
    const h2 off = h2{(f16)1032.f, (f16)1032.f};
    const uint32_t l0 = raw.x & 0x0F0F0F0Fu, l1 = raw.y & 0x0F0F0F0Fu;
    const uint32_t u0 = (raw.x >> 4) & 0x0F0F0F0Fu, u1 = (raw.y >> 4) & 0x0F0F0F0Fu;
    const h2 a0 = magic_lo(l0) - off, a1 = magic_hi(l0) - off, a2 = magic_lo(l1) - off, a3 = magic_hi(l1) - off;
    const h2 b0 = magic_lo(u0) - off, b1 = magic_hi(u0) - off, b2 = magic_lo(u1) - off, b3 = magic_hi(u1) - off;
    k0 = h8{a0.x, a0.y, a1.x, a1.y, a2.x, a2.y, a3.x, a3.y};
    k1 = h8{b0.x, b0.y, b1.x, b1.y, b2.x, b2.y, b3.x, b3.y};
}

// Q4_K: the same bytes -> exact f16 values q (codes 0..15, no shift).
DEV void q4k_pair(u32x2 raw, h8 &k0, h8 &k1) {
    const h2 off = h2{(f16)1024.f, (f16)1024.f};
    const uint32_t l0 = raw.x & 0x0F0F0F0Fu, l1 = raw.y & 0x0F0F0F0Fu;
    const uint32_t u0 = (raw.x >> 4) & 0x0F0F0F0Fu, u1 = (raw.y >> 4) & 0x0F0F0F0Fu;
    const h2 a0 = magic_lo(l0) - off, a1 = magic_hi(l0) - off, a2 = magic_lo(l1) - off, a3 = magic_hi(l1) - off;
    const h2 b0 = magic_lo(u0) - off, b1 = magic_hi(u0) - off, b2 = magic_lo(u1) - off, b3 = magic_hi(u1) - off;
    k0 = h8{a0.x, a0.y, a1.x, a1.y, a2.x, a2.y, a3.x, a3.y};
    k1 = h8{b0.x, b0.y, b1.x, b1.y, b2.x, b2.y, b3.x, b3.y};
}

// Q8_0: 8 signed byte codes -> exact f16 values.
DEV h8 q8_eight(u32x2 raw) {
    const h2 off = h2{(f16)1152.f, (f16)1152.f};
    const uint32_t w0 = raw.x ^ 0x80808080u, w1 = raw.y ^ 0x80808080u;
    const h2 a0 = magic_lo(w0) - off, a1 = magic_hi(w0) - off, a2 = magic_lo(w1) - off, a3 = magic_hi(w1) - off;
    return h8{a0.x, a0.y, a1.x, a1.y, a2.x, a2.y, a3.x, a3.y};
}

// s_waitcnt with vmcnt(N), lgkmcnt(0), expcnt untouched (gfx9 encoding),
// fenced against compiler reordering of memory accesses.
template <int N>
DEV void wait_vm_lgkm0() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x0070);
    asm volatile("" ::: "memory");
}

DEV void block_barrier() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// Direct load of 16 bytes per lane from src into LDS at lds + 16 * lane, or
// of 2 bytes into the low half of the dword at lds + 4 * lane (zero-extended;
// both placements checked on the device); lds is wave-uniform.  Written as an instruction the
// compiler does not interpret: it produces no register, and the loop's own
// vmcnt waits order the LDS reads after it (the compiler, unable to tell the
// stages apart, would otherwise wait for every load in flight before each
// LDS read).  The asm sets m0 itself; the compiler uses m0 nowhere else in
// these kernels (it is a reserved register that an asm clobber cannot name).
// Same, with the address split into a wave-uniform base (SGPRs) and a
// 32-bit per-lane byte offset, so that advancing to the next K block changes
// only the base: no per-lane address arithmetic per load.
DEV void dma16s(const void *base, uint32_t off, const void AS3 *lds) {
    const uint32_t m = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(uintptr_t)lds);
    asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(off), "s"(base), "s"(m) : "memory");
}
DEV void dma4s(const void *base, uint32_t off, const void AS3 *lds) {
    const uint32_t m = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(uintptr_t)lds);
    asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dword %0, %1" ::"v"(off), "s"(base), "s"(m) : "memory");
}
DEV void dma2s(const void *base, uint32_t off, const void AS3 *lds) {
    const uint32_t m = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(uintptr_t)lds);
    asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_ushort %0, %1" ::"v"(off), "s"(base), "s"(m) : "memory");
}
DEV void dma16(const void *src, const void AS3 *lds) {
    const uint32_t m = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(uintptr_t)lds);
    asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(src), "s"(m) : "memory");
}
DEV void dma2(const void *src, const void AS3 *lds) {
    const uint32_t m = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(uintptr_t)lds);
    asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_ushort %0, off" ::"v"(src), "s"(m) : "memory");
}

// TM = 128 tokens per block tile (prefill) or 32 (ubatches of at most 32
// tokens, batched decode: one activation load per wavefront and K block,
// each wavefront 64 features x 32 tokens, more stages in flight).
template <int WT, int EPI, bool SPLIT, int NS, int MF, int WL, int TM>
__global__ __launch_bounds__(256, (NS <= 3 || TM == 32) ? 2 : 1) void k_gemm_dl(QMat W, const uint16_t *Xh,
                                                                                const uint16_t *Xl, int ldx, EpiArgs ep,
                                                                                int M, int pair_mode, int NT,
                                                                                int nsplit, float *part,
                                                                                const float *xs) {
    using G = Geo<WT, TM>;
    constexpr bool Q4L = WT != T_Q8_0;    // 16 code bytes per row and K block
    __shared__ __attribute__((aligned(16))) uint8_t S0[G::STAGE];
    __shared__ __attribute__((aligned(16))) uint8_t S1[G::STAGE];
    __shared__ __attribute__((aligned(16))) uint8_t S2[NS > 2 ? G::STAGE : 16];
    __shared__ __attribute__((aligned(16))) uint8_t S3[NS > 3 ? G::STAGE : 16];
    __shared__ __attribute__((aligned(16))) uint8_t S4[NS > 4 ? G::STAGE : 16];
    __shared__ __attribute__((aligned(16))) uint8_t S5[NS > 5 ? G::STAGE : 16];
    __shared__ __attribute__((aligned(16))) uint8_t S6[NS > 6 ? G::STAGE : 16];
    __shared__ __attribute__((aligned(16))) uint8_t S7[NS > 7 ? G::STAGE : 16];
    static_assert(NS >= 3 && NS <= 8, "stages");
    static_assert(TM == 128 || (TM == 32 && MF == 32 && WL == 1), "token tile");

    // block -> (feature tile, token tile, K split); the tiles of one feature
    // tile share an XCD
    const int mtiles = (M + TM - 1) / TM;
    const int per_nt = mtiles * nsplit;
    const int L = blockIdx.x, xcd = L & 7, j = L >> 3;
    const int nt = (j / per_nt) * 8 + xcd, rem = j % per_nt;
    const int mtile = rem % mtiles, split = rem / mtiles;
    if (nt >= NT) return;

    // the wavefront index as a wave-uniform value: the LDS addresses of the
    // direct loads then live in scalar registers
    const int tid = threadIdx.x, lane = tid & 63, w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int n0 = nt * DBN, m0 = mtile * TM;
    // K split `split` of nsplit: K blocks [nb_all * split / nsplit, nb_all * (split + 1) / nsplit)
    const int nb_all = W.K >> 5, kb0 = (int)((long)nb_all * split / nsplit);
    const int nb = (int)((long)nb_all * (split + 1) / nsplit) - kb0;
    // WL 0: wavefront w covers features 128 (w & 1) .. +127 and tokens
    // 64 (w >> 1) .. +63; WL 1: features 64 w .. +63 and all TM tokens (each
    // code converted by one wavefront only)
    constexpr int DWN = WL ? 64 : 128, DWM = WL ? TM : 64;
    const int wn = WL ? 64 * w : (w & 1) * DWN, wm = WL ? 0 : (w >> 1) * DWM;

    // ---- per-lane byte offsets of the direct loads (from a base that moves
    // with the K block; every offset below 2^31, checked by the launcher) ----
    // activations: TM 128: instructions j = w, w + 4 of each part cover
    // slots 64j .. 64j+63; TM 32: wavefront w loads slots 64 (w & 1) .. +63 of
    // part w >> 1 (value, remainder)
    uint32_t xo[2];
#pragma unroll
    for (int i = 0; i < 2; i++) {
        const int slot = TM == 128 ? 64 * (w + 4 * i) + lane : 64 * (w & 1) + lane;
        const int m = slot >> 2, c = (slot & 3) ^ swz(slot >> 2);
        const int row = min(m0 + m, M - 1);            // rows past M repeat row M-1; their outputs are dropped
        xo[i] = (uint32_t)(((size_t)row * ldx + c * 8) * 2);
    }
    // codes: Q4_0 one row of 16 bytes per lane (rows 64w + lane); Q8_0 two
    // instructions of 32 rows x 2 halves
    const size_t row_bytes = Q4L ? (size_t)(W.K >> 1) : (size_t)W.K;
    uint32_t co[2];
#pragma unroll
    for (int i = 0; i < 2; i++) {
        if (Q4L) {
            co[i] = (uint32_t)((size_t)(64 * w + lane) * row_bytes);
        } else {
            const int slot = 64 * (w + 4 * i) + lane, r = slot >> 1, half = (slot & 1) ^ ((r >> 3) & 1);
            co[i] = (uint32_t)((size_t)r * row_bytes + half * 16);
        }
    }
    // scales: the block's 256 rows of one K block are contiguous in the
    // transposed arrays (f16 dt, Q4_K fp32 sf), 64 of them per wavefront
    const uint32_t so = (uint32_t)((64 * w + lane) * (G::K4 ? 4 : 2));
    const uint8_t *xh_base = (const uint8_t *)Xh + (size_t)kb0 * 64;
    const uint8_t *xl_base = (const uint8_t *)Xl + (size_t)kb0 * 64;
    const uint8_t *c_base = (const uint8_t *)W.qs + (size_t)n0 * row_bytes + (size_t)kb0 * (Q4L ? 16 : 32);
    const size_t s_step = (size_t)W.N * (G::K4 ? 4 : 2);   // bytes per K block
    const uint8_t *s_base = (G::K4 ? (const uint8_t *)W.sf : (const uint8_t *)W.dt) +
                            (size_t)kb0 * s_step + (size_t)n0 * (G::K4 ? 4 : 2);

    auto stage_ptr = [&](auto sc) -> uint8_t * {
        constexpr int s = decltype(sc)::value;
        if constexpr (s == 0) return S0;
        else if constexpr (s == 1) return S1;
        else if constexpr (s == 2) return S2;
        else if constexpr (s == 3) return S3;
        else if constexpr (s == 4) return S4;
        else if constexpr (s == 5) return S5;
        else if constexpr (s == 6) return S6;
        else return S7;
    };

    // requests K block kb (clamped to the range) into stage s
    auto issue = [&](auto sc, int kb) __attribute__((always_inline)) {
        uint8_t *st = stage_ptr(sc);
        const size_t k = (size_t)min(kb, nb - 1);
        if constexpr (TM == 128) {
#pragma unroll
            for (int i = 0; i < 2; i++) {
                dma16s(xh_base + k * 64, xo[i], (const void AS3 *)(st + 1024 * (w + 4 * i)));
                dma16s(xl_base + k * 64, xo[i], (const void AS3 *)(st + G::OFF_LO + 1024 * (w + 4 * i)));
            }
        } else {
            dma16s((w >> 1 ? xl_base : xh_base) + k * 64, xo[0],
                   (const void AS3 *)(st + (w >> 1 ? G::OFF_LO : 0) + 1024 * (w & 1)));
        }
        if (Q4L) {
            dma16s(c_base + k * 16, co[0], (const void AS3 *)(st + G::OFF_CODES + 1024 * w));
        } else {
#pragma unroll
            for (int i = 0; i < 2; i++)
                dma16s(c_base + k * 32, co[i], (const void AS3 *)(st + G::OFF_CODES + 1024 * (w + 4 * i)));
        }
        if constexpr (G::K4)
            dma4s(s_base + k * s_step, so, (const void AS3 *)(st + G::OFF_SC + 256 * w));
        else
            dma2s(s_base + k * s_step, so, (const void AS3 *)(st + G::OFF_SC + 256 * w));
    };

    // MF = 32: 32x32 tiles, 4 feature x 2 token tiles per wavefront;
    // MF = 16: 16x16 tiles, 8 x 4 (one v_mfma_f32_16x16x32_f16 covers a whole
    // 32-wide quant block: each tile's block is a chain of two MFMAs)
    constexpr int TA = DWN / MF, TB = DWM / MF, NR = MF == 32 ? 16 : 4;
    typedef float accv __attribute__((ext_vector_type(NR)));
    accv acc[TA][TB];
#pragma unroll
    for (int a = 0; a < TA; a++)
#pragma unroll
        for (int b = 0; b < TB; b++)
#pragma unroll
            for (int r = 0; r < NR; r++) acc[a][b][r] = 0.f;

    // (each body is dependent on the lambda's argument, so only the variant
    // this instance uses is compiled)
    auto compute16 = [&](auto sc) __attribute__((always_inline)) {
        if constexpr (MF == 16 && decltype(sc)::value >= 0) {
        typedef float f4v __attribute__((ext_vector_type(4)));
        const uint8_t *st = stage_ptr(sc);
        const int g = lane >> 4;          // k group: this lane supplies k = 8g .. 8g+7
        h8 xh[TB], xl[TB];
#pragma unroll
        for (int b = 0; b < TB; b++) {
            const int m = wm + 16 * b + (lane & 15);
            const int slot = 4 * m + (g ^ swz(m));
            xh[b] = *(const h8 *)(st + 16 * slot);
            xl[b] = *(const h8 *)(st + G::OFF_LO + 16 * slot);
        }
#pragma unroll
        for (int a = 0; a < TA; a++) {
            const int f = wn + 16 * a + (lane & 15);
            h8 cf;
            if (WT == T_Q4_0) {
                // codes 8g .. 8g+7: the low (g < 2) or high (g >= 2) nibbles of
                // bytes 8(g & 1) .. 8(g & 1)+7
                const u32x4 v = *(const u32x4 *)(st + G::OFF_CODES + 16 * f);
                const u32x2 raw = (g & 1) ? u32x2{v.z, v.w} : u32x2{v.x, v.y};
                const int sh = (g >> 1) * 4;
                const uint32_t v0 = (raw.x >> sh) & 0x0F0F0F0Fu, v1 = (raw.y >> sh) & 0x0F0F0F0Fu;
                const h2 off = h2{(f16)1032.f, (f16)1032.f};
                const h2 a0 = magic_lo(v0) - off, a1 = magic_hi(v0) - off, a2 = magic_lo(v1) - off,
                         a3 = magic_hi(v1) - off;
                cf = h8{a0.x, a0.y, a1.x, a1.y, a2.x, a2.y, a3.x, a3.y};
            } else {
                // k 8g .. 8g+7: chunk g >> 1 (stored at position (g >> 1) ^ sw), half g & 1
                const int sw = (f >> 3) & 1;
                const u32x4 v = *(const u32x4 *)(st + G::OFF_CODES + 32 * f + 16 * ((g >> 1) ^ sw));
                cf = q8_eight((g & 1) ? u32x2{v.z, v.w} : u32x2{v.x, v.y});
            }
            const float d = f16_bits_to_f32(*(const uint16_t *)(st + G::OFF_SC + 4 * f));
#pragma unroll
            for (int b = 0; b < TB; b++) {
                f4v t = __builtin_amdgcn_mfma_f32_16x16x32_f16(xh[b], cf, f4v{}, 0, 0, 0);
                t = __builtin_amdgcn_mfma_f32_16x16x32_f16(xl[b], cf, t, 0, 0, 0);
#pragma unroll
                for (int r = 0; r < 4; r++) acc[a][b][r] += d * t[r];
            }
        }
        }
    };

    auto compute32 = [&](auto sc) __attribute__((always_inline)) {
        if constexpr (MF == 32 && decltype(sc)::value >= 0) {
        const uint8_t *st = stage_ptr(sc);
        // the wavefront's feature tiles: codes of both k-halves and the scale
        // (Q4_K: d sc of the sub-block)
        h8 c0[TA], c1[TA];
        float d[TA];
#pragma unroll
        for (int a = 0; a < TA; a++) {
            const int f = wn + 32 * a + (lane & 31);
            const bool hi8 = lane >> 5;      // this lane's 8 bytes of a 16-byte chunk
            if (WT == T_Q4_0) {
                const u32x4 v = *(const u32x4 *)(st + G::OFF_CODES + 16 * f);
                q4_pair(hi8 ? u32x2{v.z, v.w} : u32x2{v.x, v.y}, c0[a], c1[a]);
            } else if (WT == T_Q4_K) {
                const u32x4 v = *(const u32x4 *)(st + G::OFF_CODES + 16 * f);
                q4k_pair(hi8 ? u32x2{v.z, v.w} : u32x2{v.x, v.y}, c0[a], c1[a]);
            } else {
                const int sw = (f >> 3) & 1;
                const u32x4 v0 = *(const u32x4 *)(st + G::OFF_CODES + 32 * f + 16 * sw);
                const u32x4 v1 = *(const u32x4 *)(st + G::OFF_CODES + 32 * f + 16 * (1 - sw));
                c0[a] = q8_eight(hi8 ? u32x2{v0.z, v0.w} : u32x2{v0.x, v0.y});
                c1[a] = q8_eight(hi8 ? u32x2{v1.z, v1.w} : u32x2{v1.x, v1.y});
            }
            if constexpr (G::K4) {
                d[a] = *(const float *)(st + G::OFF_SC + 4 * f);
            } else {
                // (converted once here and kept opaque: the 16 scaling FMAs of a
                // tile then issue as plain fp32 FMAs instead of f16-operand
                // v_fma_mix_f32; measured 1.6% faster on the gate/up GEMM)
                d[a] = f16_bits_to_f32(*(const uint16_t *)(st + G::OFF_SC + 4 * f));
                asm volatile("" : "+v"(d[a]));
            }
        }
        // (keeps the token tiles' fragment reads below: hoisted above, they
        // would hold registers the codes need)
        __builtin_amdgcn_sched_barrier(0);
        h8 xh[2], xl[2];
        auto read_x = [&](int b) __attribute__((always_inline)) {
            const int m = wm + 32 * b + (lane & 31);
#pragma unroll
            for (int h = 0; h < 2; h++) {
                const int slot = 4 * m + ((2 * h + (lane >> 5)) ^ swz(m));
                xh[h] = *(const h8 *)(st + 16 * slot);
                xl[h] = *(const h8 *)(st + G::OFF_LO + 16 * slot);
            }
        };
        auto chain = [&](int a) __attribute__((always_inline)) {
            f16x t = __builtin_amdgcn_mfma_f32_32x32x16_f16(xh[0], c0[a], f16x{}, 0, 0, 0);
            t = __builtin_amdgcn_mfma_f32_32x32x16_f16(xl[0], c0[a], t, 0, 0, 0);
            t = __builtin_amdgcn_mfma_f32_32x32x16_f16(xh[1], c1[a], t, 0, 0, 0);
            return __builtin_amdgcn_mfma_f32_32x32x16_f16(xl[1], c1[a], t, 0, 0, 0);
        };
        if constexpr (WL) {
            // Tiles i = TA b + a in order, software-pipelined: the four MFMAs
            // of tile i go into one of two temporaries while the 16 scaling
            // FMAs of tile i-1 read the other, and the issue order below puts
            // four of those FMAs after each MFMA, so the matrix cores and the
            // VALU work at the same time (with one temporary every scaling
            // waits for its chain and the next chain for the scaling).
            read_x(0);
            f16x tp = chain(0);
#pragma unroll
            for (int i = 1; i < TA * TB; i++) {
                const int a = i % TA, b = i / TA, pa = (i - 1) % TA, pb = (i - 1) / TA;
                if (a == 0) read_x(b);
                const f16x tc = chain(a);
#pragma unroll
                for (int r = 0; r < 16; r++) acc[pa][pb][r] += d[pa] * tp[r];
                tp = tc;
            }
#pragma unroll
            for (int r = 0; r < 16; r++) acc[TA - 1][TB - 1][r] += d[TA - 1] * tp[r];
            // per tile: its fragment reads (first feature tile of a token
            // tile), then each MFMA followed by four FMAs
#pragma unroll
            for (int i = 0; i < TA * TB; i++) {
                if (i % TA == 0) __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
#pragma unroll
                for (int j = 0; j < 4; j++) {
                    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                    if (i > 0) __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);
                }
            }
            __builtin_amdgcn_sched_group_barrier(0x002, 16, 0);
        } else {
            // (128-feature wavefront tiles: the pipelined order would need
            // more registers than a wavefront has)
#pragma unroll
            for (int b = 0; b < TB; b++) {
                read_x(b);
#pragma unroll
                for (int a = 0; a < TA; a++) {
                    const f16x t = chain(a);
#pragma unroll
                    for (int r = 0; r < 16; r++) acc[a][b][r] += d[a] * t[r];
                }
            }
        }
        }
    };

    // one step: K block kb is in stage S; wait for it, then refill the stage
    // computed in the previous step with K block kb + NS - 1
    auto step = [&](auto sc, int kb) __attribute__((always_inline)) {
        constexpr int s = decltype(sc)::value;
        wait_vm_lgkm0<(NS - 2) * G::LOADS>();
        block_barrier();
        issue(std::integral_constant<int, (s + NS - 1) % NS>{}, kb + NS - 1);
        if constexpr (MF == 16) compute16(sc);
        else compute32(sc);
    };

    issue(std::integral_constant<int, 0>{}, 0);
    issue(std::integral_constant<int, 1>{}, 1);
    if constexpr (NS > 3) issue(std::integral_constant<int, 2>{}, 2);
    if constexpr (NS > 4) issue(std::integral_constant<int, 3>{}, 3);
    if constexpr (NS > 5) issue(std::integral_constant<int, 4>{}, 4);
    if constexpr (NS > 6) issue(std::integral_constant<int, 5>{}, 5);
    if constexpr (NS > 7) issue(std::integral_constant<int, 6>{}, 6);
    // whole periods of NS steps; K blocks past the last are clamped re-reads
    // whose stages are never computed
    for (int kb = 0; kb < nb; kb += NS) {
        step(std::integral_constant<int, 0>{}, kb);
        if (kb + 1 < nb) step(std::integral_constant<int, 1>{}, kb + 1);
        if (kb + 2 < nb) step(std::integral_constant<int, 2>{}, kb + 2);
        if constexpr (NS > 3)
            if (kb + 3 < nb) step(std::integral_constant<int, 3>{}, kb + 3);
        if constexpr (NS > 4)
            if (kb + 4 < nb) step(std::integral_constant<int, 4>{}, kb + 4);
        if constexpr (NS > 5)
            if (kb + 5 < nb) step(std::integral_constant<int, 5>{}, kb + 5);
        if constexpr (NS > 6)
            if (kb + 6 < nb) step(std::integral_constant<int, 6>{}, kb + 6);
        if constexpr (NS > 7)
            if (kb + 7 < nb) step(std::integral_constant<int, 7>{}, kb + 7);
    }
    // drain the requests past the last K block before the block can exit
    wait_vm_lgkm0<0>();

    // Q4_K min term, on the matrix cores: acc += X (-M)^T over this split's K
    // blocks, with A = the tokens' block sums of x and B = the rows' negated
    // sub-block mins -dmin m, both as f16 value | remainder << 16 per K block
    // and stored octet-major ([K/256][rows][8]), so an octet of the block's
    // rows is one contiguous run.  16 K blocks per MFMA step (each lane half
    // takes one octet), three MFMAs per step (value x value, remainder x value,
    // value x remainder).  K blocks past the split enter as zeros.
    if constexpr (G::K4 && MF == 32) {
        const uint32_t *xq = (const uint32_t *)xs;
        const int kend = kb0 + nb, hf = lane >> 5;
        auto unpack = [](const u32x4 &p0, const u32x4 &p1, h8 &hi, h8 &lo) __attribute__((always_inline)) {
            const uint32_t v[8] = {p0.x, p0.y, p0.z, p0.w, p1.x, p1.y, p1.z, p1.w};
#pragma unroll
            for (int e = 0; e < 8; e++) {
                hi[e] = __builtin_bit_cast(f16, (uint16_t)v[e]);
                lo[e] = __builtin_bit_cast(f16, (uint16_t)(v[e] >> 16));
            }
        };
        if constexpr (TM == 128) {   // (the launcher splits K in whole octets for Q4_K)
            // whole octets, 16 K blocks per chunk: the chunk's mins (2 octets x
            // 256 rows x 32 B, contiguous per octet) go by direct loads into
            // stage 0 and its sums (2 octets x 128 tokens x 32 B) into stage 1,
            // then each lane reads its row's and token's 32 bytes from LDS
            static_assert(TM != 128 || (G::STAGE >= 16384), "stage holds a chunk of mins");
            const int oend = kend >> 3;
            block_barrier();                               // every wavefront is done with the stages
            for (int k16 = kb0; k16 < kend; k16 += 16) {
                const int ob = k16 >> 3;
#pragma unroll
                for (int i = 0; i < 4; i++) {
                    const int j = 4 * w + i, oc = min(ob + (j >> 3), oend - 1);
                    const int row = (j & 7) * 32 + (lane >> 1);
                    dma16(W.mfq + ((size_t)oc * W.N + n0 + row) * 8 + 4 * (lane & 1),
                          (const void AS3 *)(S0 + 1024 * j));
                }
#pragma unroll
                for (int i = 0; i < 2; i++) {
                    const int j = 2 * w + i, oc = min(ob + (j >> 2), oend - 1);
                    const int row = min(m0 + (j & 3) * 32 + (lane >> 1), M - 1);
                    dma16(xq + ((size_t)oc * M + row) * 8 + 4 * (lane & 1), (const void AS3 *)(S1 + 1024 * j));
                }
                wait_vm_lgkm0<0>();
                block_barrier();
                const bool live = ob + hf < oend;               // this lane half's octet lies in the split
                h8 mh[TA], ml[TA];
#pragma unroll
                for (int a = 0; a < TA; a++) {
                    const uint8_t *p = S0 + 8192 * hf + 32 * (wn + 32 * a + (lane & 31));
                    u32x4 p0 = *(const u32x4 *)p, p1 = *(const u32x4 *)(p + 16);
                    if (!live) p0 = p1 = u32x4{0u, 0u, 0u, 0u};
                    unpack(p0, p1, mh[a], ml[a]);
                }
#pragma unroll
                for (int b = 0; b < TB; b++) {
                    const uint8_t *p = S1 + 4096 * hf + 32 * (wm + 32 * b + (lane & 31));
                    u32x4 p0 = *(const u32x4 *)p, p1 = *(const u32x4 *)(p + 16);
                    if (!live) p0 = p1 = u32x4{0u, 0u, 0u, 0u};
                    h8 xh, xl;
                    unpack(p0, p1, xh, xl);
#pragma unroll
                    for (int a = 0; a < TA; a++) {
                        acc[a][b] = __builtin_amdgcn_mfma_f32_32x32x16_f16(xh, mh[a], acc[a][b], 0, 0, 0);
                        acc[a][b] = __builtin_amdgcn_mfma_f32_32x32x16_f16(xl, mh[a], acc[a][b], 0, 0, 0);
                        acc[a][b] = __builtin_amdgcn_mfma_f32_32x32x16_f16(xh, ml[a], acc[a][b], 0, 0, 0);
                    }
                }
                block_barrier();                               // before the next chunk overwrites the stages
            }
        } else {
            // the 32-token form, whose splits need not be whole octets: element loads
            for (int k16 = kb0; k16 < kend; k16 += 16) {
                const int kq = k16 + 8 * hf;
                h8 mh[TA], ml[TA];
#pragma unroll
                for (int a = 0; a < TA; a++) {
                    const size_t f = n0 + wn + 32 * a + (lane & 31);
#pragma unroll
                    for (int e = 0; e < 8; e++) {
                        const int k = kq + e;
                        const uint32_t v = k < kend ? W.mfq[((size_t)(k >> 3) * W.N + f) * 8 + (k & 7)] : 0u;
                        mh[a][e] = __builtin_bit_cast(f16, (uint16_t)v);
                        ml[a][e] = __builtin_bit_cast(f16, (uint16_t)(v >> 16));
                    }
                }
#pragma unroll
                for (int b = 0; b < TB; b++) {
                    const size_t row = min(m0 + wm + 32 * b + (lane & 31), M - 1);
                    h8 xh, xl;
#pragma unroll
                    for (int e = 0; e < 8; e++) {
                        const int k = kq + e;
                        const uint32_t v = k < kend ? xq[((size_t)(k >> 3) * M + row) * 8 + (k & 7)] : 0u;
                        xh[e] = __builtin_bit_cast(f16, (uint16_t)v);
                        xl[e] = __builtin_bit_cast(f16, (uint16_t)(v >> 16));
                    }
#pragma unroll
                    for (int a = 0; a < TA; a++) {
                        acc[a][b] = __builtin_amdgcn_mfma_f32_32x32x16_f16(xh, mh[a], acc[a][b], 0, 0, 0);
                        acc[a][b] = __builtin_amdgcn_mfma_f32_32x32x16_f16(xl, mh[a], acc[a][b], 0, 0, 0);
                        acc[a][b] = __builtin_amdgcn_mfma_f32_32x32x16_f16(xh, ml[a], acc[a][b], 0, 0, 0);
                    }
                }
            }
        }
    }

    // ---- epilogue.  MF = 32: lane holds feature n0 + wn + 32a + (lane & 31)
    // and, in accumulator r, token m0 + wm + 32b + (r/4)*8 + (lane/32)*4 + r%4.
    // MF = 16: feature n0 + wn + 16a + (lane & 15), token m0 + wm + 16b +
    // 4(lane/16) + r. ----
    const int fl = lane & (MF - 1);
    auto tok_of = [&](int b, int r) __attribute__((always_inline)) {
        return MF == 32 ? m0 + wm + 32 * b + (r >> 2) * 8 + (lane >> 5) * 4 + (r & 3)
                        : m0 + wm + 16 * b + 4 * (lane >> 4) + r;
    };
    if (SPLIT) {
        const int N = W.N;
#pragma unroll
        for (int b = 0; b < TB; b++)
#pragma unroll
            for (int r = 0; r < NR; r++) {
                const int m = tok_of(b, r);
                if (m >= M) continue;
                float *dst = part + ((size_t)split * M + m) * N + n0 + wn + fl;
#pragma unroll
                for (int a = 0; a < TA; a++) dst[MF * a] = acc[a][b][r];
            }
        return;
    }
#pragma unroll
    for (int b = 0; b < TB; b++) {
        if (EPI == EPI_STORE || EPI == EPI_RESID) {
#pragma unroll
            for (int r = 0; r < NR; r++) {
                const int m = tok_of(b, r);
                if (m >= M) continue;
                float *y = ep.y + (size_t)m * ep.ldy + n0 + wn + fl;
#pragma unroll
                for (int a = 0; a < TA; a++) {
                    if (EPI == EPI_STORE) y[MF * a] = acc[a][b][r];
                    else y[MF * a] += acc[a][b][r];
                }
            }
        } else if (pair_mode == PAIR_GU) {
            // gate rows 64g .. 64g+31 and their up rows 64g+32 .. 64g+63: in
            // feature tiles a and a + 32/MF of the same 64-row group
            constexpr int UP = 32 / MF;
#pragma unroll
            for (int a = 0; a < TA; a++) {
                if ((a / UP) % 2) continue;                      // an up tile
                const int rr = n0 + wn + MF * a + fl;            // gate row
                const int g = rr >> 6;
#pragma unroll
                for (int r = 0; r < NR; r++) {
                    const int m = tok_of(b, r);
                    if (m >= M) continue;
                    epi_pair<EPI>(ep, m, (g << 5) + (rr & 31), rr, rr + 32, acc[a][b][r], acc[a + UP][b][r]);
                }
            }
        } else {
            // adjacent features f (even lane) and f+1 (odd lane): the even lane
            // takes the first half of the pair's tokens, the odd lane the second
            const bool odd = lane & 1;
            constexpr int HR = NR / 2;
#pragma unroll
            for (int a = 0; a < TA; a++)
#pragma unroll
                for (int r = 0; r < HR; r++) {
                    const float send = odd ? acc[a][b][r] : acc[a][b][r + HR];
                    const float recv = __shfl_xor(send, 1, 64);
                    const int rr = odd ? r + HR : r;
                    const int m = tok_of(b, rr);
                    const int f = n0 + wn + MF * a + (fl & ~1);
                    const float va = odd ? recv : acc[a][b][r];
                    const float vb = odd ? acc[a][b][r + HR] : recv;
                    if (m < M) epi_pair<EPI>(ep, m, f >> 1, f, f + 1, va, vb);
                }
        }
    }
}

template <int WT, int EPI, bool SPLIT>
void launch_dl_ns(int ns, const QMat &W, const uint16_t *Xh, const uint16_t *Xl, int ldx, const EpiArgs &ep, int M,
                  int pair_mode, int S, float *part, const float *xs, hipStream_t s) {
    const int NT = W.N / DBN, NT8 = (NT + 7) / 8 * 8;
    const dim3 grid(NT8 * ((M + DBM - 1) / DBM) * S);
    if constexpr (WT == T_Q4_K) {   // one form: 3 stages, 32x32 tiles, 64-feature wavefront tiles
        launch((k_gemm_dl<WT, EPI, SPLIT, 3, 32, 1, 128>), grid, dim3(256), 0, s, W, Xh, Xl, ldx, ep, M, pair_mode, NT, S,
               part, xs);
        return;
    } else {
    // ns: 3 or 4 LDS stages on 32x32 tiles (wavefront tile 128 features x 64
    // tokens); 13: 3 stages on 16x16 tiles; 23: 3 stages, 32x32 tiles,
    // wavefront tile 64 features x 128 tokens
    switch (ns) {
    case 4: launch((k_gemm_dl<WT, EPI, SPLIT, 4, 32, 0, 128>), grid, dim3(256), 0, s, W, Xh, Xl, ldx, ep, M, pair_mode, NT, S, part, xs); break;
    case 13: launch((k_gemm_dl<WT, EPI, SPLIT, 3, 16, 0, 128>), grid, dim3(256), 0, s, W, Xh, Xl, ldx, ep, M, pair_mode, NT, S, part, xs); break;
    case 23: launch((k_gemm_dl<WT, EPI, SPLIT, 3, 32, 1, 128>), grid, dim3(256), 0, s, W, Xh, Xl, ldx, ep, M, pair_mode, NT, S, part, xs); break;
    default: launch((k_gemm_dl<WT, EPI, SPLIT, 3, 32, 0, 128>), grid, dim3(256), 0, s, W, Xh, Xl, ldx, ep, M, pair_mode, NT, S, part, xs); break;
    }
    }
}

// The 32-token form: NS stages (4, 6 or 8).
template <int WT, int EPI, bool SPLIT>
void launch_dls_ns(int ns, const QMat &W, const uint16_t *Xh, const uint16_t *Xl, int ldx, const EpiArgs &ep, int M,
                   int pair_mode, int S, float *part, const float *xs, hipStream_t s) {
    const int NT = W.N / DBN, NT8 = (NT + 7) / 8 * 8;
    const dim3 grid(NT8 * ((M + DBM_S - 1) / DBM_S) * S);
    switch (ns) {
    case 8:   // (8 stages fit two blocks per compute unit for Q4_0 only)
        if constexpr (WT == T_Q4_0) {
            launch((k_gemm_dl<WT, EPI, SPLIT, 8, 32, 1, 32>), grid, dim3(256), 0, s, W, Xh, Xl, ldx, ep, M, pair_mode, NT, S, part, xs);
            break;
        }
        [[fallthrough]];
    case 6: launch((k_gemm_dl<WT, EPI, SPLIT, 6, 32, 1, 32>), grid, dim3(256), 0, s, W, Xh, Xl, ldx, ep, M, pair_mode, NT, S, part, xs); break;
    default: launch((k_gemm_dl<WT, EPI, SPLIT, 4, 32, 1, 32>), grid, dim3(256), 0, s, W, Xh, Xl, ldx, ep, M, pair_mode, NT, S, part, xs); break;
    }
}

template <int WT, int EPI>
void launch_dls_epi(int ns, const QMat &W, const uint16_t *Xh, const uint16_t *Xl, int ldx, const EpiArgs &ep, int M,
                    int pair_mode, int S, float *ws, const float *xs, hipStream_t s) {
    if (S > 1) {
        launch_dls_ns<WT, EPI, true>(ns, W, Xh, Xl, ldx, ep, M, pair_mode, S, ws, xs, s);
        launch_splitk_sum(EPI, ws, S, W.N, M, ep, pair_mode, s);
    } else {
        launch_dls_ns<WT, EPI, false>(ns, W, Xh, Xl, ldx, ep, M, pair_mode, 1, nullptr, xs, s);
    }
}

template <int WT>
void launch_dls_wt(int ns, const QMat &W, const uint16_t *Xh, const uint16_t *Xl, int ldx, const EpiArgs &ep, int M,
                   int pair_mode, int S, float *ws, const float *xs, hipStream_t s) {
    switch (ep.epi) {
    case EPI_STORE: launch_dls_epi<WT, EPI_STORE>(ns, W, Xh, Xl, ldx, ep, M, pair_mode, S, ws, xs, s); break;
    case EPI_RESID: launch_dls_epi<WT, EPI_RESID>(ns, W, Xh, Xl, ldx, ep, M, pair_mode, S, ws, xs, s); break;
    case EPI_QKV: launch_dls_epi<WT, EPI_QKV>(ns, W, Xh, Xl, ldx, ep, M, pair_mode, S, ws, xs, s); break;
    case EPI_SWIGLU: launch_dls_epi<WT, EPI_SWIGLU>(ns, W, Xh, Xl, ldx, ep, M, pair_mode, S, ws, xs, s); break;
    }
}

template <int WT, int EPI>
void launch_dl_epi(int ns, const QMat &W, const uint16_t *Xh, const uint16_t *Xl, int ldx, const EpiArgs &ep, int M,
                   int pair_mode, int S, float *ws, const float *xs, hipStream_t s) {
    if (S > 1) {
        launch_dl_ns<WT, EPI, true>(ns, W, Xh, Xl, ldx, ep, M, pair_mode, S, ws, xs, s);
        launch_splitk_sum(EPI, ws, S, W.N, M, ep, pair_mode, s);
    } else {
        launch_dl_ns<WT, EPI, false>(ns, W, Xh, Xl, ldx, ep, M, pair_mode, 1, nullptr, xs, s);
    }
}

template <int WT>
void launch_dl_wt(int ns, const QMat &W, const uint16_t *Xh, const uint16_t *Xl, int ldx, const EpiArgs &ep, int M,
                  int pair_mode, int S, float *ws, const float *xs, hipStream_t s) {
    switch (ep.epi) {
    case EPI_STORE: launch_dl_epi<WT, EPI_STORE>(ns, W, Xh, Xl, ldx, ep, M, pair_mode, S, ws, xs, s); break;
    case EPI_RESID: launch_dl_epi<WT, EPI_RESID>(ns, W, Xh, Xl, ldx, ep, M, pair_mode, S, ws, xs, s); break;
    case EPI_QKV: launch_dl_epi<WT, EPI_QKV>(ns, W, Xh, Xl, ldx, ep, M, pair_mode, S, ws, xs, s); break;
    case EPI_SWIGLU: launch_dl_epi<WT, EPI_SWIGLU>(ns, W, Xh, Xl, ldx, ep, M, pair_mode, S, ws, xs, s); break;
    }
}


// ---- weight-streaming form: Q4_0, at most 32 tokens (batched decode) --------
//
// With 32 tokens a weight byte feeds only 64 products, so the kernel has to
// stream codes at the HBM rate.  Where the forms above request one K block per
// stage (each load instruction then touches 64 rows, 16 bytes of each, and
// each scale is a 2-byte request), here a stage is KS = 2 or 4 consecutive
// K blocks: a load instruction covers 1024 / (16 KS) rows x 16 KS contiguous
// bytes of codes, or 1024 / (64 KS) tokens x 64 KS contiguous bytes of
// activations, and the scales of the block's whole K range (at most WS_RMAX
// blocks) are loaded once at entry.
// Everything else is the direct-to-LDS scheme: a ring of WS_NS stages, a
// constant vmcnt per wavefront, one barrier per stage.  Block tile: 256
// features x 32 tokens, wavefront w owning features 64 w .. +63 (two 32x32
// tiles, the same MFMA operands and per-block scaling as k_gemm_dl).
// LDS stage (16 or 32 KB): activation values [32 tokens][4 KS chunks of 16 B]
// (chunk q = 4 j + c: K block j of the stage, 16-byte piece c), remainders
// likewise, codes [256 rows][KS K blocks of 16 B], each stored at an XOR slot
// (ws_xslot, ws_cslot) that spreads a quarter wavefront's 16-byte reads over
// distinct bank groups.  With KS = 2 a block takes 80 KB of LDS, so two fit a
// compute unit.  K splits are whole octets of K blocks.
constexpr int WS_NS = 4;                      // stages
constexpr int WS_RMAX = 32;                   // K blocks per split at most

// Stage geometry for KS K blocks per stage (KS = 2 or 4).
template <int KS>
struct WsGeo {
    static constexpr int XPART = 32 * KS * 64;            // one activation part
    static constexpr int STAGE = 2 * XPART + DBN * KS * 16;
    static constexpr int XI = XPART / 1024;               // activation instructions per part
    static constexpr int CI = DBN * KS * 16 / 1024;       // code instructions
    static constexpr int LOADS = (2 * XI + CI) / 4;       // per wavefront and stage
    static constexpr int TOKB = KS * 64;                  // bytes of one token's row in a part
};
// chunk slot of activation chunk q (of KS*4) of token m; K-block slot of code
// chunk j of row f: XOR patterns that put 16 consecutive lanes' 16-byte reads
// in distinct bank groups (KS = 4: 256-byte token rows, 64-byte code rows;
// KS = 2: 128-byte token rows, 32-byte code rows)
template <int KS>
DEV int ws_xslot(int q, int m) { return KS == 4 ? q ^ (m & 15) : q ^ ((m >> 1) & 7); }
template <int KS>
DEV int ws_cslot(int j, int f) { return KS == 4 ? j ^ ((f >> 2) & 3) : j ^ ((f >> 3) & 1); }

template <int EPI, bool SPLIT, int KS>
__global__ __launch_bounds__(256, KS == 2 ? 2 : 1) void k_gemm_ws(QMat W, const uint16_t *Xh, const uint16_t *Xl,
                                                                   int ldx, EpiArgs ep, int M, int pair_mode, int NT,
                                                                   int nsplit, float *part) {
    using G = WsGeo<KS>;
    __shared__ __attribute__((aligned(16))) uint8_t S0[G::STAGE];
    __shared__ __attribute__((aligned(16))) uint8_t S1[G::STAGE];
    __shared__ __attribute__((aligned(16))) uint8_t S2[G::STAGE];
    __shared__ __attribute__((aligned(16))) uint8_t S3[G::STAGE];
    __shared__ __attribute__((aligned(16))) uint8_t SC[DBN * WS_RMAX * 2];
    static_assert(WS_NS == 4, "four stage buffers");
    static_assert(G::LOADS * 4 == 2 * G::XI + G::CI && G::XI % 2 == 0 && G::CI % 4 == 0, "loads per wavefront");
    const int mtiles = (M + 31) / 32;
    const int per_nt = mtiles * nsplit;
    const int L = blockIdx.x, xcd = L & 7, jj = L >> 3;
    const int nt = (jj / per_nt) * 8 + xcd, rem = jj % per_nt;
    const int mtile = rem % mtiles, split = rem / mtiles;
    if (nt >= NT) return;

    const int tid = threadIdx.x, lane = tid & 63, w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int n0 = nt * DBN, m0 = mtile * 32;
    const int nb_all = W.K >> 5, no = W.K >> 8;            // K blocks, octets of K blocks
    const int kb0 = 8 * (int)((long)no * split / nsplit);
    const int nb = 8 * (int)((long)no * (split + 1) / nsplit) - kb0;   // multiple of 8, <= WS_RMAX
    const int nst = nb / KS;
    const size_t row_bytes = (size_t)(W.K >> 1);

    // activations: wavefront w fills part w >> 1, instruction i the 1 KB at
    // 1024 ib, ib = (XW w + i) mod XI (XW = XI / 2 instructions per wavefront):
    // token ib * (1024 / TOKB) + lane / (TOKB / 16), stored slot lane % (TOKB / 16)
    constexpr int XW = G::XI / 2, SPT = G::TOKB / 16;
    uint32_t xo[XW];
#pragma unroll
    for (int i = 0; i < XW; i++) {
        const int ib = (XW * w + i) % G::XI, m = ib * (1024 / G::TOKB) + lane / SPT;
        const int q = ws_xslot<KS>(lane % SPT, m);     // (the XOR pattern is its own inverse)
        const int row = min(m0 + m, M - 1);            // rows past M repeat row M-1; their outputs are dropped
        xo[i] = (uint32_t)(((size_t)row * ldx + (q >> 2) * 32 + (q & 3) * 8) * 2);
    }
    const uint8_t *xbase = (const uint8_t *)(w >> 1 ? Xl : Xh) + (size_t)kb0 * 64;
    // codes: instruction i of wavefront w fills the 1 KB at 1024 (CW w + i)
    // (CW = CI / 4): rows of KS 16-byte chunks, KS lanes per row
    constexpr int CW = G::CI / 4;
    uint32_t co[CW];
#pragma unroll
    for (int i = 0; i < CW; i++) {
        const int f = (1024 / (16 * KS)) * (CW * w + i) + lane / KS, j = ws_cslot<KS>(lane % KS, f);
        co[i] = (uint32_t)((size_t)f * row_bytes + j * 16);
    }
    const uint8_t *cbase = (const uint8_t *)W.qs + (size_t)n0 * row_bytes + (size_t)kb0 * 16;

    // the f16 scales of the block's K range: row f at SC + 2 nb f, 16 bytes
    // (8 K blocks) per lane and instruction
    {
        const int nchunk = nb >> 3;                    // 16-byte pieces per row
        for (int n = w; n < nb >> 1; n += 4) {         // nb / 2 instructions of 64 pieces
            const int g = 64 * n + lane, f = g / nchunk, c = g % nchunk;
            dma16(W.d + (size_t)(n0 + f) * nb_all + kb0 + 8 * c, (const void AS3 *)(SC + 1024 * n));
        }
    }

    auto stage_ptr = [&](auto sc) -> uint8_t * {
        constexpr int s = decltype(sc)::value;
        if constexpr (s == 0) return S0;
        else if constexpr (s == 1) return S1;
        else if constexpr (s == 2) return S2;
        else return S3;
    };
    auto issue = [&](auto sc, int sg) __attribute__((always_inline)) {
        uint8_t *st = stage_ptr(sc);
        const size_t k = (size_t)min(sg, nst - 1) * KS;
#pragma unroll
        for (int i = 0; i < XW; i++)
            dma16s(xbase + k * 64, xo[i], (const void AS3 *)(st + (w >> 1) * G::XPART + 1024 * ((XW * w + i) % G::XI)));
#pragma unroll
        for (int i = 0; i < CW; i++)
            dma16s(cbase + k * 16, co[i], (const void AS3 *)(st + 2 * G::XPART + 1024 * (CW * w + i)));
    };

    f16x acc[2];
#pragma unroll
    for (int a = 0; a < 2; a++)
#pragma unroll
        for (int r = 0; r < 16; r++) acc[a][r] = 0.f;

    auto compute = [&](auto sc, int sg) __attribute__((always_inline)) {
        const uint8_t *st = stage_ptr(sc);
        const int m = lane & 31;
        const bool hi8 = lane >> 5;
        float d[2][KS];
#pragma unroll
        for (int a = 0; a < 2; a++) {
            const int f = 64 * w + 32 * a + m;
            const uint8_t *sp = SC + 2 * ((size_t)f * nb + KS * sg);
            if constexpr (KS == 4) {
                const u32x2 sv = *(const u32x2 *)sp;
                d[a][0] = f16_bits_to_f32((uint16_t)sv.x);
                d[a][1] = f16_bits_to_f32((uint16_t)(sv.x >> 16));
                d[a][2] = f16_bits_to_f32((uint16_t)sv.y);
                d[a][3] = f16_bits_to_f32((uint16_t)(sv.y >> 16));
            } else {
                const uint32_t sv = *(const uint32_t *)sp;
                d[a][0] = f16_bits_to_f32((uint16_t)sv);
                d[a][1] = f16_bits_to_f32((uint16_t)(sv >> 16));
            }
        }
#pragma unroll
        for (int j = 0; j < KS; j++) {
            h8 xh[2], xl[2];
#pragma unroll
            for (int h = 0; h < 2; h++) {
                const int q = 4 * j + 2 * h + (lane >> 5);
                const int pos = G::TOKB * m + 16 * ws_xslot<KS>(q, m);
                xh[h] = *(const h8 *)(st + pos);
                xl[h] = *(const h8 *)(st + G::XPART + pos);
            }
#pragma unroll
            for (int a = 0; a < 2; a++) {
                const int f = 64 * w + 32 * a + m;
                const u32x4 v = *(const u32x4 *)(st + 2 * G::XPART + 16 * KS * f + 16 * ws_cslot<KS>(j, f));
                h8 c0, c1;
                q4_pair(hi8 ? u32x2{v.z, v.w} : u32x2{v.x, v.y}, c0, c1);
                f16x t = __builtin_amdgcn_mfma_f32_32x32x16_f16(xh[0], c0, f16x{}, 0, 0, 0);
                t = __builtin_amdgcn_mfma_f32_32x32x16_f16(xl[0], c0, t, 0, 0, 0);
                t = __builtin_amdgcn_mfma_f32_32x32x16_f16(xh[1], c1, t, 0, 0, 0);
                t = __builtin_amdgcn_mfma_f32_32x32x16_f16(xl[1], c1, t, 0, 0, 0);
#pragma unroll
                for (int r = 0; r < 16; r++) acc[a][r] += d[a][j] * t[r];
            }
        }
    };

    auto step = [&](auto sc, int sg) __attribute__((always_inline)) {
        constexpr int s = decltype(sc)::value;
        wait_vm_lgkm0<(WS_NS - 2) * G::LOADS>();
        block_barrier();
        issue(std::integral_constant<int, (s + WS_NS - 1) % WS_NS>{}, sg + WS_NS - 1);
        compute(sc, sg);
    };

    issue(std::integral_constant<int, 0>{}, 0);
    issue(std::integral_constant<int, 1>{}, 1);
    issue(std::integral_constant<int, 2>{}, 2);
    for (int sg = 0; sg < nst; sg += WS_NS) {
        step(std::integral_constant<int, 0>{}, sg);
        if (sg + 1 < nst) step(std::integral_constant<int, 1>{}, sg + 1);
        if (sg + 2 < nst) step(std::integral_constant<int, 2>{}, sg + 2);
        if (sg + 3 < nst) step(std::integral_constant<int, 3>{}, sg + 3);
    }
    wait_vm_lgkm0<0>();

    // ---- epilogue: lane holds feature n0 + 64w + 32a + (lane & 31) and, in
    // accumulator r, token m0 + (r/4)*8 + (lane/32)*4 + r%4 ----
    const int fl = lane & 31;
    auto tok_of = [&](int r) __attribute__((always_inline)) { return m0 + (r >> 2) * 8 + (lane >> 5) * 4 + (r & 3); };
    if (SPLIT) {
#pragma unroll
        for (int r = 0; r < 16; r++) {
            const int m = tok_of(r);
            if (m >= M) continue;
            float *dst = part + ((size_t)split * M + m) * W.N + n0 + 64 * w + fl;
            dst[0] = acc[0][r];
            dst[32] = acc[1][r];
        }
        return;
    }
    if (EPI == EPI_STORE || EPI == EPI_RESID) {
#pragma unroll
        for (int r = 0; r < 16; r++) {
            const int m = tok_of(r);
            if (m >= M) continue;
            float *y = ep.y + (size_t)m * ep.ldy + n0 + 64 * w + fl;
#pragma unroll
            for (int a = 0; a < 2; a++) {
                if (EPI == EPI_STORE) y[32 * a] = acc[a][r];
                else y[32 * a] += acc[a][r];
            }
        }
    } else if (pair_mode == PAIR_GU) {
        // gate rows 64g .. +31 (tile 0) and their up rows 64g + 32 .. (tile 1)
        const int rr = n0 + 64 * w + fl, g = rr >> 6;
#pragma unroll
        for (int r = 0; r < 16; r++) {
            const int m = tok_of(r);
            if (m < M) epi_pair<EPI>(ep, m, (g << 5) + (rr & 31), rr, rr + 32, acc[0][r], acc[1][r]);
        }
    } else {
        // adjacent features f (even lane) and f+1 (odd lane), exchanged by lane pairs
        const bool odd = lane & 1;
#pragma unroll
        for (int a = 0; a < 2; a++)
#pragma unroll
            for (int r = 0; r < 8; r++) {
                const float send = odd ? acc[a][r] : acc[a][r + 8];
                const float recv = __shfl_xor(send, 1, 64);
                const int rr = odd ? r + 8 : r;
                const int m = tok_of(rr);
                const int f = n0 + 64 * w + 32 * a + (fl & ~1);
                const float va = odd ? recv : acc[a][r];
                const float vb = odd ? acc[a][r + 8] : recv;
                if (m < M) epi_pair<EPI>(ep, m, f >> 1, f, f + 1, va, vb);
            }
    }
}

template <int EPI, int KS>
void launch_ws_ks(const QMat &W, const uint16_t *Xh, const uint16_t *Xl, int ldx, const EpiArgs &ep, int M,
                  int pair_mode, int S, float *ws, hipStream_t s) {
    const int NT = W.N / DBN, NT8 = (NT + 7) / 8 * 8;
    const dim3 grid(NT8 * ((M + 31) / 32) * S);
    if (S > 1) {
        launch((k_gemm_ws<EPI, true, KS>), grid, dim3(256), 0, s, W, Xh, Xl, ldx, ep, M, pair_mode, NT, S, ws);
        launch_splitk_sum(EPI, ws, S, W.N, M, ep, pair_mode, s);
    } else {
        launch((k_gemm_ws<EPI, false, KS>), grid, dim3(256), 0, s, W, Xh, Xl, ldx, ep, M, pair_mode, NT, 1,
               (float *)nullptr);
    }
}

template <int EPI>
void launch_ws_epi(int ks, const QMat &W, const uint16_t *Xh, const uint16_t *Xl, int ldx, const EpiArgs &ep, int M,
                   int pair_mode, int S, float *ws, hipStream_t s) {
    if (ks == 4)
        launch_ws_ks<EPI, 4>(W, Xh, Xl, ldx, ep, M, pair_mode, S, ws, s);
    else
        launch_ws_ks<EPI, 2>(W, Xh, Xl, ldx, ep, M, pair_mode, S, ws, s);
}


// ---- wide form: Q4_0 / Q8_0 / Q4_K, 512 features x 128 tokens per block ----
//
// The arithmetic and operand layouts of k_gemm_dl (exact codes, activation
// value and remainder, per-block fp32 scaling, 64-feature wavefront tiles over
// all 128 tokens), with the operand movement cut into fewer, wider memory
// requests.  Measured on the direct-to-LDS form: its time follows the number
// of requests, not the bytes (per K block of a 256 x 128 tile: 256 one-row
// 16-byte code requests, 256 64-byte activation requests; codes alone took
// 102 us of a 512-token gate/up GEMM, and 46 us when each request covered 4
// K blocks of a row).  Here:
// * codes come in super-stages of 64 contiguous bytes per row and request
//   (4 K blocks of Q4_0, 2 of Q8_0), double-buffered (super-stage s+1 is
//   requested at the first K block of s);
// * a block covers 512 features (8 wavefronts), so each activation request
//   feeds twice the features;
// * activations and scales (from the transposed dt) go through a ring of
//   DW_A = 4 single-K-block stages, three K blocks ahead.
// LDS (one array, 136 KB, one block of 8 wavefronts per compute unit, two
// per SIMD): the 4 activation stages fill the first 64 KB, so every
// activation read is a fixed register plus an immediate offset; then the
// stages' scales and the two code stages.  A wavefront requests 3 loads per
// K block (2 activation, 1 scale) and, at the first K block of a super-stage,
// 4 code loads (Q4_0 after the activation loads; Q8_0 before them, since its
// codes are needed two K blocks later); loads complete in issue order, so the
// wait before K block kb is a constant per kb within its super-stage
// (dw_wait: the loads issued after the later of its activation stage and
// its codes).  The K range of a split is whole periods of 4 K blocks (Q4_K:
// whole octets), the splits as even as that allows.  Q4_K: codes as Q4_0 (exact values 0..15), the fp32 scale
// d sc from the transposed sf, and after the main loop the min term as in
// k_gemm_dl, with the chunks of mins and block sums staged in the code
// stages.
constexpr int DW_N = 512;                       // features per block
constexpr int DW_A = 4;                         // activation stages
constexpr int DW_ACT = 128 * 64;                // one activation part of a K block
constexpr int DW_AST = 2 * DW_ACT;              // activation stage: values, remainders
constexpr int DW_SST = DW_N * 4;                // scales of a K block, one dword per row
constexpr int DW_CST = DW_N * 64;               // codes of a super-stage: [512 rows][64 B]
constexpr int DW_OFF_S = DW_A * DW_AST;         // (= 64 KB)
constexpr int DW_OFF_C = DW_OFF_S + DW_A * DW_SST;
constexpr int DW_LDS = DW_OFF_C + 2 * DW_CST;

// K blocks per super-stage.
template <int WT>
constexpr int dw_ck() { return WT == T_Q8_0 ? 2 : 4; }
// Loads a wavefront issued after those that K block kb needs, for kb at
// position p of its super-stage: Q4_0 [6, 10, 10, 10], Q8_0 [6, 10].
template <int WT>
constexpr int dw_wait(int p) { return p == 0 ? 6 : 10; }

// Position of 16-byte piece q (0..3: Q4_0 K block q, Q8_0 half q % 2 of K
// block q / 2) of a super-stage in row r: XOR-swizzled so that the 16-byte
// reads of a quarter wavefront (16 consecutive rows, one piece) fall into 16
// distinct groups of 4 banks.
DEV int dw_pos(int r, int q) { return q ^ ((r >> 2) & 3); }

template <int WT, int EPI, bool SPLIT>
__global__ __launch_bounds__(512, 1) void k_gemm_dw(QMat W, const uint16_t *Xh, const uint16_t *Xl, int ldx,
                                                   EpiArgs ep, int M, int pair_mode, int NT, int nsplit,
                                                   float *part, const float *xs) {
    constexpr bool K4 = WT == T_Q4_K;
    __shared__ __attribute__((aligned(16))) uint8_t lds[DW_LDS];

    // block -> (feature tile, K split, token tile): the units (feature tile,
    // K split) go to the 8 XCDs in turn (workgroup i runs on XCD i mod 8), and
    // the token tiles of a unit, which read the same weights, run together on
    // its XCD
    const int mtiles = (M + 127) / 128;
    const int L = blockIdx.x, xcd = L & 7, j = L >> 3;
    const int unit = (j / mtiles) * 8 + xcd, mtile = j % mtiles;
    if (unit >= NT * nsplit) return;
    const int nt = unit / nsplit, split = unit % nsplit;

    const int tid = threadIdx.x, lane = tid & 63, w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int n0 = nt * DW_N, m0 = mtile * 128, wn = 64 * w;
    // split `split` of nsplit: units [P split / nsplit, P (split + 1) / nsplit)
    // of the P units of U K blocks (periods of 4; Q4_K octets), so splits may
    // differ by one unit
    constexpr int CK = dw_ck<WT>(), U = K4 ? 8 : 4;
    const int nb_all = W.K >> 5, P = nb_all / U;
    const int kb0 = U * (int)((long)P * split / nsplit), nb = U * (int)((long)P * (split + 1) / nsplit) - kb0;
    const int nsup = nb / CK;

    // ---- per-lane byte offsets of the direct loads ----
    // activations: wavefront w loads part w >> 2 (value, remainder), slots
    // 64 j .. 64 j + 63 for j = 2 (w & 3) + i; slot 4m + (c ^ swz(m)) holds
    // chunk c of token m
    uint32_t xo[2];
#pragma unroll
    for (int i = 0; i < 2; i++) {
        const int slot = 64 * (2 * (w & 3) + i) + lane;
        const int m = slot >> 2, c = (slot & 3) ^ swz(slot >> 2);
        const int row = min(m0 + m, M - 1);            // rows past M repeat row M-1; their outputs are dropped
        xo[i] = (uint32_t)(((size_t)row * ldx + c * 8) * 2);
    }
    // codes: instruction i of wavefront w covers rows 64 w + 16 i + lane / 4,
    // one 16-byte piece each (4 lanes = a super-stage's 64 contiguous bytes of
    // a row)
    const size_t row_bytes = WT == T_Q8_0 ? (size_t)W.K : (size_t)(W.K >> 1);
    uint32_t co[4];
#pragma unroll
    for (int i = 0; i < 4; i++) {
        const int r = 64 * w + 16 * i + (lane >> 2);
        const int q = dw_pos(r, lane & 3);             // the piece that lands at position lane & 3
        co[i] = (uint32_t)((size_t)r * row_bytes + 16 * q);
    }
    // scales: f16 dt, or Q4_K fp32 sf, both [K/32][N]
    constexpr int SB = K4 ? 4 : 2;
    const uint32_t so = (uint32_t)((64 * w + lane) * SB);
    const uint8_t *xh_base = (const uint8_t *)Xh + (size_t)kb0 * 64;
    const uint8_t *xl_base = (const uint8_t *)Xl + (size_t)kb0 * 64;
    const uint8_t *xp_base = (w >> 2) ? xl_base : xh_base;
    const uint8_t *c_base = (const uint8_t *)W.qs + (size_t)n0 * row_bytes + (size_t)kb0 * (64 / CK);
    const size_t s_step = (size_t)W.N * SB;
    const uint8_t *s_base =
        (K4 ? (const uint8_t *)W.sf : (const uint8_t *)W.dt) + (size_t)kb0 * s_step + (size_t)n0 * SB;

    // code stage of super-stage sup: the first for even, the second for odd
    auto cstage = [&](int sup) -> uint8_t * { return lds + DW_OFF_C + (sup & 1) * DW_CST; };
    // K block kb (clamped) -> activation stage sc: 2 loads + 1 scale load
    auto issue_act = [&](auto sc, int kb) __attribute__((always_inline)) {
        constexpr int v = decltype(sc)::value;
        const size_t k = (size_t)min(kb, nb - 1);
#pragma unroll
        for (int i = 0; i < 2; i++)
            dma16s(xp_base + k * 64, xo[i],
                   (const void AS3 *)(lds + v * DW_AST + (w >> 2) * DW_ACT + 1024 * (2 * (w & 3) + i)));
        if constexpr (K4)
            dma4s(s_base + k * s_step, so, (const void AS3 *)(lds + DW_OFF_S + v * DW_SST + 256 * w));
        else
            dma2s(s_base + k * s_step, so, (const void AS3 *)(lds + DW_OFF_S + v * DW_SST + 256 * w));
    };
    // super-stage sup (clamped) -> code stage: 4 loads
    auto issue_codes = [&](int sup) __attribute__((always_inline)) {
        uint8_t *cs = cstage(sup);
        const size_t k = (size_t)min(sup, nsup - 1);
#pragma unroll
        for (int i = 0; i < 4; i++)
            dma16s(c_base + k * 64, co[i], (const void AS3 *)(cs + (64 * w + 16 * i) * 64));
    };

    f16x acc[2][4];
#pragma unroll
    for (int a = 0; a < 2; a++)
#pragma unroll
        for (int b = 0; b < 4; b++)
#pragma unroll
            for (int r = 0; r < 16; r++) acc[a][b][r] = 0.f;

    // K block q of the code stage cs, activations of stage st, scales ss
    auto compute = [&](const uint8_t *st, const uint8_t *ss, const uint8_t *cs, int q) __attribute__((always_inline)) {
        h8 c0[2], c1[2];
        float d[2];
#pragma unroll
        for (int a = 0; a < 2; a++) {
            const int f = wn + 32 * a + (lane & 31);
            const bool hi8 = lane >> 5;      // this lane's 8 bytes of a 16-byte piece
            if constexpr (WT == T_Q8_0) {
                const u32x4 v0 = *(const u32x4 *)(cs + f * 64 + 16 * dw_pos(f, 2 * q));
                const u32x4 v1 = *(const u32x4 *)(cs + f * 64 + 16 * dw_pos(f, 2 * q + 1));
                c0[a] = q8_eight(hi8 ? u32x2{v0.z, v0.w} : u32x2{v0.x, v0.y});
                c1[a] = q8_eight(hi8 ? u32x2{v1.z, v1.w} : u32x2{v1.x, v1.y});
            } else {
                const u32x4 v = *(const u32x4 *)(cs + f * 64 + 16 * dw_pos(f, q));
                if constexpr (K4) q4k_pair(hi8 ? u32x2{v.z, v.w} : u32x2{v.x, v.y}, c0[a], c1[a]);
                else q4_pair(hi8 ? u32x2{v.z, v.w} : u32x2{v.x, v.y}, c0[a], c1[a]);
            }
            if constexpr (K4) d[a] = *(const float *)(ss + 4 * f);
            else d[a] = f16_bits_to_f32(*(const uint16_t *)(ss + 4 * f));
            asm volatile("" : "+v"(d[a]));
        }
        __builtin_amdgcn_sched_barrier(0);
        h8 xh[2], xl[2];
        auto read_x = [&](int b) __attribute__((always_inline)) {
            const int m = 32 * b + (lane & 31);
#pragma unroll
            for (int h = 0; h < 2; h++) {
                const int slot = 4 * m + ((2 * h + (lane >> 5)) ^ swz(m));
                xh[h] = *(const h8 *)(st + 16 * slot);
                xl[h] = *(const h8 *)(st + DW_ACT + 16 * slot);
            }
        };
        auto chain = [&](int a) __attribute__((always_inline)) {
            f16x t = __builtin_amdgcn_mfma_f32_32x32x16_f16(xh[0], c0[a], f16x{}, 0, 0, 0);
            t = __builtin_amdgcn_mfma_f32_32x32x16_f16(xl[0], c0[a], t, 0, 0, 0);
            t = __builtin_amdgcn_mfma_f32_32x32x16_f16(xh[1], c1[a], t, 0, 0, 0);
            return __builtin_amdgcn_mfma_f32_32x32x16_f16(xl[1], c1[a], t, 0, 0, 0);
        };
        // tiles i = 2 b + a, each tile's MFMAs against the previous tile's
        // scaling FMAs (as in k_gemm_dl)
        read_x(0);
        f16x tp = chain(0);
#pragma unroll
        for (int i = 1; i < 8; i++) {
            const int a = i & 1, b = i >> 1, pa = (i - 1) & 1, pb = (i - 1) >> 1;
            if (a == 0) read_x(b);
            const f16x tc = chain(a);
#pragma unroll
            for (int r = 0; r < 16; r++) acc[pa][pb][r] += d[pa] * tp[r];
            tp = tc;
        }
#pragma unroll
        for (int r = 0; r < 16; r++) acc[1][3][r] += d[1] * tp[r];
#pragma unroll
        for (int i = 0; i < 8; i++) {
            if ((i & 1) == 0) __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
#pragma unroll
            for (int jj = 0; jj < 4; jj++) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                if (i > 0) __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);
            }
        }
        __builtin_amdgcn_sched_group_barrier(0x002, 16, 0);
    };

    // step kb (activation stage kb % 4, position p = kb % CK of super-stage
    // kb / CK): wait for its loads, barrier, at p = 0 request the next
    // super-stage into the other code stage, refill the activation stage
    // computed at kb - 1 with kb + 3, compute
    auto step = [&](auto pc, int kb, const uint8_t *cs) __attribute__((always_inline)) {
        constexpr int j = decltype(pc)::value;     // kb % 4
        constexpr int p = j % CK;
        wait_vm_lgkm0<dw_wait<WT>(p)>();
        block_barrier();
        if constexpr (p == 0 && WT == T_Q8_0) issue_codes(kb / CK + 1);
        issue_act(std::integral_constant<int, (j + 3) % 4>{}, kb + 3);
        if constexpr (p == 0 && WT != T_Q8_0) issue_codes(kb / CK + 1);
        compute(lds + j * DW_AST, lds + DW_OFF_S + j * DW_SST, cs, p);
    };

    issue_codes(0);
    issue_act(std::integral_constant<int, 0>{}, 0);
    issue_act(std::integral_constant<int, 1>{}, 1);
    issue_act(std::integral_constant<int, 2>{}, 2);
    // periods of four K blocks (one Q4_0 super-stage, two Q8_0 ones; a split
    // is whole periods); K blocks past the last are clamped re-reads whose
    // stages are never computed
    for (int kb = 0; kb < nb; kb += 4) {
        step(std::integral_constant<int, 0>{}, kb, cstage(kb / CK));
        step(std::integral_constant<int, 1>{}, kb + 1, cstage(kb / CK));
        step(std::integral_constant<int, 2>{}, kb + 2, cstage((kb + 2) / CK));
        step(std::integral_constant<int, 3>{}, kb + 3, cstage((kb + 2) / CK));
    }
    // drain the requests past the last K block before the block can exit
    wait_vm_lgkm0<0>();

    // Q4_K min term: acc += X (-M)^T over the split's K blocks (see k_gemm_dl),
    // 16 K blocks per chunk: the chunk's mins (2 octets x 512 rows x 32 B)
    // and block sums (2 octets x 128 tokens x 32 B) go by direct loads into
    // the code stages, then each lane reads its row's and token's 32 bytes
    if constexpr (K4) {
        const uint32_t *xq = (const uint32_t *)xs;
        const int kend = kb0 + nb, oend = kend >> 3, hf = lane >> 5;
        uint8_t *mins = lds + DW_OFF_C, *sums = lds + DW_OFF_C + 32768;
        auto unpack = [](const u32x4 &p0, const u32x4 &p1, h8 &hi, h8 &lo) __attribute__((always_inline)) {
            const uint32_t v[8] = {p0.x, p0.y, p0.z, p0.w, p1.x, p1.y, p1.z, p1.w};
#pragma unroll
            for (int e = 0; e < 8; e++) {
                hi[e] = __builtin_bit_cast(f16, (uint16_t)v[e]);
                lo[e] = __builtin_bit_cast(f16, (uint16_t)(v[e] >> 16));
            }
        };
        block_barrier();                               // every wavefront is done with the code stages
        for (int k16 = kb0; k16 < kend; k16 += 16) {
            const int ob = k16 >> 3;
#pragma unroll
            for (int i = 0; i < 4; i++) {
                const int j = 4 * w + i, oc = min(ob + (j >> 4), oend - 1);
                const int row = (j & 15) * 32 + (lane >> 1);
                dma16(W.mfq + ((size_t)oc * W.N + n0 + row) * 8 + 4 * (lane & 1), (const void AS3 *)(mins + 1024 * j));
            }
            {
                const int j = w, oc = min(ob + (j >> 2), oend - 1);
                const int row = min(m0 + (j & 3) * 32 + (lane >> 1), M - 1);
                dma16(xq + ((size_t)oc * M + row) * 8 + 4 * (lane & 1), (const void AS3 *)(sums + 1024 * j));
            }
            wait_vm_lgkm0<0>();
            block_barrier();
            const bool live = ob + hf < oend;               // this lane half's octet lies in the split
            h8 mh[2], ml[2];
#pragma unroll
            for (int a = 0; a < 2; a++) {
                const uint8_t *p = mins + 16384 * hf + 32 * (wn + 32 * a + (lane & 31));
                u32x4 p0 = *(const u32x4 *)p, p1 = *(const u32x4 *)(p + 16);
                if (!live) p0 = p1 = u32x4{0u, 0u, 0u, 0u};
                unpack(p0, p1, mh[a], ml[a]);
            }
#pragma unroll
            for (int b = 0; b < 4; b++) {
                const uint8_t *p = sums + 4096 * hf + 32 * (32 * b + (lane & 31));
                u32x4 p0 = *(const u32x4 *)p, p1 = *(const u32x4 *)(p + 16);
                if (!live) p0 = p1 = u32x4{0u, 0u, 0u, 0u};
                h8 xh, xl;
                unpack(p0, p1, xh, xl);
#pragma unroll
                for (int a = 0; a < 2; a++) {
                    acc[a][b] = __builtin_amdgcn_mfma_f32_32x32x16_f16(xh, mh[a], acc[a][b], 0, 0, 0);
                    acc[a][b] = __builtin_amdgcn_mfma_f32_32x32x16_f16(xl, mh[a], acc[a][b], 0, 0, 0);
                    acc[a][b] = __builtin_amdgcn_mfma_f32_32x32x16_f16(xh, ml[a], acc[a][b], 0, 0, 0);
                }
            }
            block_barrier();                               // before the next chunk overwrites the stages
        }
    }

    // ---- epilogue: lane holds feature n0 + wn + 32a + (lane & 31) and, in
    // accumulator r, token m0 + 32b + (r/4)*8 + (lane/32)*4 + r%4 ----
    const int fl = lane & 31;
    auto tok_of = [&](int b, int r) __attribute__((always_inline)) {
        return m0 + 32 * b + (r >> 2) * 8 + (lane >> 5) * 4 + (r & 3);
    };
    if (SPLIT) {
        const int N = W.N;
#pragma unroll
        for (int b = 0; b < 4; b++)
#pragma unroll
            for (int r = 0; r < 16; r++) {
                const int m = tok_of(b, r);
                if (m >= M) continue;
                float *dst = part + ((size_t)split * M + m) * N + n0 + wn + fl;
#pragma unroll
                for (int a = 0; a < 2; a++) dst[32 * a] = acc[a][b][r];
            }
        return;
    }
#pragma unroll
    for (int b = 0; b < 4; b++) {
        if (EPI == EPI_STORE || EPI == EPI_RESID) {
#pragma unroll
            for (int r = 0; r < 16; r++) {
                const int m = tok_of(b, r);
                if (m >= M) continue;
                float *y = ep.y + (size_t)m * ep.ldy + n0 + wn + fl;
#pragma unroll
                for (int a = 0; a < 2; a++) {
                    if (EPI == EPI_STORE) y[32 * a] = acc[a][b][r];
                    else y[32 * a] += acc[a][b][r];
                }
            }
        } else if (pair_mode == PAIR_GU) {
            // gate rows 64g .. 64g+31 (tile 0) and their up rows 64g+32 .. (tile 1)
            const int rr = n0 + wn + fl, g = rr >> 6;
#pragma unroll
            for (int r = 0; r < 16; r++) {
                const int m = tok_of(b, r);
                if (m < M) epi_pair<EPI>(ep, m, (g << 5) + (rr & 31), rr, rr + 32, acc[0][b][r], acc[1][b][r]);
            }
        } else {
            // adjacent features f (even lane) and f+1 (odd lane): the even lane
            // takes the first half of the pair's tokens, the odd lane the second
            const bool odd = lane & 1;
#pragma unroll
            for (int a = 0; a < 2; a++)
#pragma unroll
                for (int r = 0; r < 8; r++) {
                    const float send = odd ? acc[a][b][r] : acc[a][b][r + 8];
                    const float recv = __shfl_xor(send, 1, 64);
                    const int rr = odd ? r + 8 : r;
                    const int m = tok_of(b, rr);
                    const int f = n0 + wn + 32 * a + (fl & ~1);
                    const float va = odd ? recv : acc[a][b][r];
                    const float vb = odd ? acc[a][b][r + 8] : recv;
                    if (m < M) epi_pair<EPI>(ep, m, f >> 1, f, f + 1, va, vb);
                }
        }
    }
}

template <int WT, int EPI>
void launch_dw_epi(const QMat &W, const uint16_t *Xh, const uint16_t *Xl, int ldx, const EpiArgs &ep, int M,
                   int pair_mode, int S, float *ws, const float *xs, hipStream_t s) {
    const int NT = W.N / DW_N, U8 = (NT * S + 7) / 8 * 8;
    const dim3 grid(U8 * ((M + 127) / 128));
    if (S > 1) {
        launch((k_gemm_dw<WT, EPI, true>), grid, dim3(512), 0, s, W, Xh, Xl, ldx, ep, M, pair_mode, NT, S, ws, xs);
        launch_splitk_sum(EPI, ws, S, W.N, M, ep, pair_mode, s);
    } else {
        launch((k_gemm_dw<WT, EPI, false>), grid, dim3(512), 0, s, W, Xh, Xl, ldx, ep, M, pair_mode, NT, 1,
               (float *)nullptr, xs);
    }
}

template <int WT>
void launch_dw_wt(const QMat &W, const uint16_t *Xh, const uint16_t *Xl, int ldx, const EpiArgs &ep, int M,
                  int pair_mode, int S, float *ws, const float *xs, hipStream_t s) {
    switch (ep.epi) {
    case EPI_STORE: launch_dw_epi<WT, EPI_STORE>(W, Xh, Xl, ldx, ep, M, pair_mode, S, ws, xs, s); break;
    case EPI_RESID: launch_dw_epi<WT, EPI_RESID>(W, Xh, Xl, ldx, ep, M, pair_mode, S, ws, xs, s); break;
    case EPI_QKV: launch_dw_epi<WT, EPI_QKV>(W, Xh, Xl, ldx, ep, M, pair_mode, S, ws, xs, s); break;
    case EPI_SWIGLU: launch_dw_epi<WT, EPI_SWIGLU>(W, Xh, Xl, ldx, ep, M, pair_mode, S, ws, xs, s); break;
    }
}

}  // namespace

int gemm_dl_tile_features() { return DBN; }
int gemm_dl_tile_tokens() { return DBM; }
int gemm_dls_tile_tokens() { return DBM_S; }
int gemm_ws_max_blocks_per_split() { return WS_RMAX; }

void launch_gemm_ws(int ks, const QMat &W, const uint16_t *Xh, const uint16_t *Xl, int ldx, const EpiArgs &ep, int M,
                    int pair_mode, int S, float *ws, hipStream_t s) {
    switch (ep.epi) {
    case EPI_STORE: launch_ws_epi<EPI_STORE>(ks, W, Xh, Xl, ldx, ep, M, pair_mode, S, ws, s); break;
    case EPI_RESID: launch_ws_epi<EPI_RESID>(ks, W, Xh, Xl, ldx, ep, M, pair_mode, S, ws, s); break;
    case EPI_QKV: launch_ws_epi<EPI_QKV>(ks, W, Xh, Xl, ldx, ep, M, pair_mode, S, ws, s); break;
    case EPI_SWIGLU: launch_ws_epi<EPI_SWIGLU>(ks, W, Xh, Xl, ldx, ep, M, pair_mode, S, ws, s); break;
    }
}

int gemm_dw_tile_features() { return DW_N; }
// A K split must give every split whole periods of 4 K blocks (whole
// super-stages of either type).
int gemm_dw_super_blocks() { return 4; }

void launch_gemm_dw(const QMat &W, const uint16_t *Xh, const uint16_t *Xl, int ldx, const EpiArgs &ep, int M,
                    int pair_mode, int S, float *ws, const float *xs, hipStream_t s) {
    if (W.wtype == T_Q8_0)
        launch_dw_wt<T_Q8_0>(W, Xh, Xl, ldx, ep, M, pair_mode, S, ws, nullptr, s);
    else if (W.wtype == T_Q4_K)
        launch_dw_wt<T_Q4_K>(W, Xh, Xl, ldx, ep, M, pair_mode, S, ws, xs, s);
    else
        launch_dw_wt<T_Q4_0>(W, Xh, Xl, ldx, ep, M, pair_mode, S, ws, nullptr, s);
}

void launch_gemm_dls(int ns, const QMat &W, const uint16_t *Xh, const uint16_t *Xl, int ldx, const EpiArgs &ep,
                     int M, int pair_mode, int S, float *ws, const float *xs, hipStream_t s) {
    if (W.wtype == T_Q4_0)
        launch_dls_wt<T_Q4_0>(ns, W, Xh, Xl, ldx, ep, M, pair_mode, S, ws, nullptr, s);
    else if (W.wtype == T_Q4_K)
        launch_dls_wt<T_Q4_K>(ns, W, Xh, Xl, ldx, ep, M, pair_mode, S, ws, xs, s);
    else
        launch_dls_wt<T_Q8_0>(ns, W, Xh, Xl, ldx, ep, M, pair_mode, S, ws, nullptr, s);
}

void launch_gemm_dl(int ns, const QMat &W, const uint16_t *Xh, const uint16_t *Xl, int ldx, const EpiArgs &ep,
                    int M, int pair_mode, int S, float *ws, const float *xs, hipStream_t s) {
    if (W.wtype == T_Q4_0)
        launch_dl_wt<T_Q4_0>(ns, W, Xh, Xl, ldx, ep, M, pair_mode, S, ws, nullptr, s);
    else if (W.wtype == T_Q4_K)
        launch_dl_wt<T_Q4_K>(ns, W, Xh, Xl, ldx, ep, M, pair_mode, S, ws, xs, s);
    else
        launch_dl_wt<T_Q8_0>(ns, W, Xh, Xl, ldx, ep, M, pair_mode, S, ws, nullptr, s);
}
