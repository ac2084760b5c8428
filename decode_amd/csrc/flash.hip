// flash.hip -- causal attention of a prefill ubatch with MFMA (gfx950).
//
// The T tokens of a ubatch belong to one sequence and sit at consecutive
// positions p0 .. p0+T-1; their K,V rows are already in the f16 cache (the
// QKV epilogue appends them before this kernel runs).  Query row t attends to
// cached rows 0 .. p0+t.
//
// Block = 4 wavefronts sharing one KV head g.  Wavefront w takes query head
// g*G + hz*Gb + w%Gb and a tile of 32 tokens (w/Gb picks the tile when a
// group has fewer than 4 heads).  The keys a token tile reads are cut into
// NS ranges of `chunk` keys, one block each, so that the grid fills the chip
// (a ubatch has only T/32 token tiles per head); a block whose tile needs
// one range writes o itself, otherwise it leaves its unnormalized output and
// (max, sum) per query, and k_flash_merge combines the ranges in order.
// Per 64-key tile, K (row-major) and V
// (transposed, keys permuted as below) are staged in LDS once for all four
// wavefronts (the next tile's loads are in flight meanwhile), then each
// wavefront runs
//   S^T[key][q] = K Q^T     v_mfma_f32_32x32x16_f16, 2 key tiles x hd/16 steps,
//                           Q as f16 value + f16 remainder (two MFMAs a step)
//   online softmax per query column (a lane holds 16 keys of one query; the
//   other 16 are in lane l^32), base-2 with log2(e)/sqrt(hd) folded into Q
//   O^T[d][q] += V^T P^T    4 key steps x hd/32 dim tiles, P as value + remainder
// The P operand comes straight from the S^T accumulators: for key step s the
// lane's eight values r = 8s'..8s'+7 are keys 16s + 8(e>>2) + 4h + (e&3)
// (h = lane/32, e = 0..7), so V^T is stored with key k at column
// 16s + 8h + e of its 16-key group, and each lane reads 16 contiguous bytes.
// A Q8_0 cache (Q8 = true): each element is code * scale, exact in fp32, and
// the tiles hold it as f16 value + f16 remainder (converted while staging);
// S^T and O^T take one more MFMA a step for the remainder (K remainder x Q
// value, V remainder x P value; remainder x remainder, about 2^-22 of a
// product, is left out).
#include "common.h"
#include "kernels.h"

int g_flash_blocks = 512;       // blocks the key split aims for (2 per compute unit)

namespace {

constexpr int BKEY = 64;        // keys per tile
constexpr int KPAD = 8;         // f16 padding of an LDS row

// Sum and max of a value over lanes l and l ^ 32 with one v_permlane32_swap
// (which exchanges the upper half of one copy with the lower half of the
// other: each lane gets back its own value and its partner's, in lane order).
DEV uint2 swap_halves(float v) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return make_uint2(r[0], r[1]);
}
DEV float sum_halves(float v) {
    const uint2 r = swap_halves(v);
    return __uint_as_float(r.x) + __uint_as_float(r.y);
}
DEV float max_halves(float v) {
    const uint2 r = swap_halves(v);
    return fmaxf(__uint_as_float(r.x), __uint_as_float(r.y));
}

DEV int vt_col(int k) {         // permuted column of key k (0..63) in V^T
    const int s = k >> 4, rem = k & 15;
    const int h = (rem >> 2) & 1, e = ((rem >> 3) << 2) | (rem & 3);
    return (s << 4) | (h << 3) | e;
}

// Q8_0 staging in f16 pairs: four codes (code k in byte k) become exact f16
// pairs (c0, c1), (c2, c3) -- byte c + 128 under the exponent of 1024 is the
// f16 1152 + c, less 1152 -- and a pair times the block scale s splits into
// value RNE(c s) and remainder RNE(c s - value), the same numbers as
// rounding the exact fp32 product and the exact fp32 difference.
constexpr uint32_t FQ_1024_BYTES = 0x64646464u;   // every byte the high byte of f16 1024
constexpr uint32_t FQ_1152 = 0x64806480u;         // f16 pair (1152, 1152)
DEV void fq_codes4(uint32_t w, h2 &a, h2 &b) {
    const uint32_t x = w ^ 0x80808080u;
    a = as_h2(__builtin_amdgcn_perm(FQ_1024_BYTES, x, 0x04010400u)) - as_h2(FQ_1152);
    b = as_h2(__builtin_amdgcn_perm(FQ_1024_BYTES, x, 0x04030402u)) - as_h2(FQ_1152);
}
DEV void fq_split(h2 c, h2 s2, uint32_t &hi, uint32_t &lo) {
    const h2 h = c * s2;
    hi = h2_bits(h);
    lo = h2_bits(__builtin_elementwise_fma(c, s2, -h));
}

template <int HD, bool Q8>
__global__ __launch_bounds__(256, 2) void k_flash_prefill(FlashArgs a) {
    constexpr int KS = HD / 16;     // k-steps of Q K^T
    constexpr int DT = HD / 32;     // 32-row dim tiles of O^T
    constexpr int NB = HD / 32;     // Q8_0 blocks per cached row
    // f16 cache: two buffers, tile kt staged in buffer kt & 1, so one barrier
    // per tile orders both its stores before the reads and the previous reads
    // of that buffer (two tiles back) before its stores.  Q8_0 cache: one
    // tile at a time, [0] its values' f16 value parts and [1] their
    // remainders (code * scale is exact in fp32 and is exactly value +
    // remainder), with a barrier before the stores as well.
    __shared__ __attribute__((aligned(16))) f16 Ks[2][BKEY][HD + KPAD];
    __shared__ __attribute__((aligned(16))) f16 Vt[2][HD][BKEY + KPAD];

    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int G = a.H / a.kv.n_kv, Gb = G < 4 ? G : 4, Tb = 4 / Gb;
    // Workgroups go to the 8 XCDs in turn (linear id mod 8), each XCD with
    // its own L2.  The linear ids are renumbered so that an XCD's blocks form
    // one contiguous run of (KV head, head group, range) order: the blocks
    // that read one KV head's keys then share an L2 instead of each XCD
    // caching every head.
    const int X = gridDim.x, Y = gridDim.y, Z = gridDim.z;
    const int B = X * Y * Z;
    const int L = blockIdx.x + X * (blockIdx.y + Y * blockIdx.z);
    const int lin = B % 8 == 0 ? (L % 8) * (B / 8) + L / 8 : L;
    const int bx = lin % X, bz = (lin / X) % Z, g = lin / (X * Z);
    const int head = g * G + bz * Gb + (w % Gb);
    const int split = bx % a.ns;
    const int tok0 = (bx / a.ns) * 32 * Tb;                 // first token of the block
    const int tw = tok0 + (w / Gb) * 32;                    // first token of this wavefront
    const int q_t = tw + (lane & 31);                       // this lane's query column
    const int p0 = a.tok.pos[0], seq = a.tok.seq[0];
    const int T = a.T;
    const bool q_ok = q_t < T;
    const int qpos = p0 + q_t;
    const int last_tok = min(T - 1, tok0 + 32 * Tb - 1);
    const int n_keys_tile = p0 + last_tok + 1;              // keys any query of the tile reads
    const int nsplit = (n_keys_tile + a.chunk - 1) / a.chunk;
    if (split >= nsplit) return;                            // uniform: this tile needs fewer ranges
    const int kbeg = split * a.chunk;
    const int n_keys = min(n_keys_tile, kbeg + a.chunk);    // keys of this block: kbeg .. n_keys-1
    const float qscale = 1.4426950408889634f / sqrtf((float)HD);

    // Q^T operand: lane supplies Q[q][16 ks + 8 (lane/32) + e], as an f16
    // value qf and its f16 rounding remainder ql (about 22 significant bits:
    // one f16 would put an error of 2^-11 of each score into the softmax)
    h8 qf[KS], ql[KS];
    {
        const float *qr = a.q + ((size_t)(q_ok ? q_t : 0) * a.H + head) * HD + 8 * (lane >> 5);
#pragma unroll
        for (int ks = 0; ks < KS; ks++) {
            float4 lo = make_float4(0.f, 0.f, 0.f, 0.f), hi = lo;
            if (q_ok) {
                lo = *(const float4 *)(qr + 16 * ks);
                hi = *(const float4 *)(qr + 16 * ks + 4);
            }
            const float v[8] = {lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
#pragma unroll
            for (int e = 0; e < 8; e++) {
                const float y = v[e] * qscale;
                qf[ks][e] = (f16)y;
                ql[ks][e] = (f16)(y - (float)qf[ks][e]);
            }
        }
    }

    f16x acc[DT];
#pragma unroll
    for (int dt = 0; dt < DT; dt++)
#pragma unroll
        for (int r = 0; r < 16; r++) acc[dt][r] = 0.f;
    float m_run = -INFINITY, l_run = 0.f;

    const size_t base = (((size_t)seq * a.kv.n_kv + g) * a.kv.n_ctx) * HD;
    const uint16_t *Kg = (const uint16_t *)a.kv.k + base;
    const uint16_t *Vg = (const uint16_t *)a.kv.v + base;
    constexpr int CHUNKS = BKEY * HD / 8;                   // 16-byte chunks per tile
    constexpr int CPT = CHUNKS / 256;

    const int ntiles = (n_keys - kbeg + BKEY - 1) / BKEY;
    // K and V of keys k0 .. k0+63 into registers (rows past n_keys read as 0).
    // K: chunk ch = 8 dims d8 of key ch / (hd/8).  V: pair chunk pc = 8 dims
    // d8 = pc / 32 of the keys 2 (pc%32) and 2 (pc%32) + 1, whose V^T columns
    // are adjacent (vt_col keeps bit 0 of the key), so each of the 8 dims is
    // one 4-byte LDS store, and a wavefront's 64 stores hit 64 different banks.
    constexpr int PPT = CPT / 2;                            // V pair chunks per thread
    uint4 kr[CPT], vr[PPT][2];
    auto load_tile = [&](int k0) {
#pragma unroll
        for (int c = 0; c < CPT; c++) {
            const int ch = tid + c * 256, key = ch / (HD / 8), d8 = ch % (HD / 8);
            const bool ok = k0 + key < n_keys;
            kr[c] = ok ? *(const uint4 *)(Kg + (size_t)(k0 + key) * HD + d8 * 8) : make_uint4(0, 0, 0, 0);
        }
#pragma unroll
        for (int c = 0; c < PPT; c++) {
            const int pc = tid + c * 256, key = 2 * (pc & 31), d8 = pc >> 5;
#pragma unroll
            for (int j = 0; j < 2; j++) {
                const bool ok = k0 + key + j < n_keys;
                vr[c][j] = ok ? *(const uint4 *)(Vg + (size_t)(k0 + key + j) * HD + d8 * 8) : make_uint4(0, 0, 0, 0);
            }
        }
    };
    // Q8_0 cache: K piece p (thread p < BKEY * NB) = block p % NB of key
    // p / NB, 32 codes and their scale; V piece p (p < 32 * HD / 16) = 16
    // dims, half p >> 5 of the blocks, of the keys 2 (p & 31) and 2 (p & 31) + 1
    // (adjacent V^T columns, as above).  Rows past n_keys read as code 0,
    // scale 0.
    const size_t cell0 = ((size_t)seq * a.kv.n_kv + g) * a.kv.n_ctx;
    const int8_t *Kc = (const int8_t *)a.kv.k + cell0 * HD;
    const int8_t *Vc = (const int8_t *)a.kv.v + cell0 * HD;
    const uint16_t *Ksc = a.kv.k_scale + cell0 * NB;
    const uint16_t *Vsc = a.kv.v_scale + cell0 * NB;
    constexpr int KPC = BKEY * NB, VPC = 32 * (HD / 16);
    uint4 kq[2] = {}, vq[2] = {};
    uint16_t ksc = 0, vsc[2] = {};
    // (a sequence's cache rows of one KV head span n_ctx * HD < 2^31 bytes)
    auto load_q8 = [&](int k0) {
        if (tid < KPC) {
            const int key = tid / NB, blk = tid % NB;
            const bool ok = k0 + key < n_keys;
            const uint32_t e = (uint32_t)(k0 + key) * HD + 32 * blk;
            kq[0] = ok ? *(const uint4 *)(Kc + e) : make_uint4(0, 0, 0, 0);
            kq[1] = ok ? *(const uint4 *)(Kc + e + 16) : make_uint4(0, 0, 0, 0);
            ksc = ok ? Ksc[e / 32] : (uint16_t)0;
        }
        if (tid < VPC) {
            const int key = 2 * (tid & 31), hb = tid >> 5;
#pragma unroll
            for (int j = 0; j < 2; j++) {
                const bool ok = k0 + key + j < n_keys;
                const uint32_t e = (uint32_t)(k0 + key + j) * HD + 16 * hb;
                vq[j] = ok ? *(const uint4 *)(Vc + e) : make_uint4(0, 0, 0, 0);
                vsc[j] = ok ? Vsc[e / 32] : (uint16_t)0;
            }
        }
    };
    auto store_q8 = [&]() {
        if (tid < KPC) {
            const int key = tid / NB, blk = tid % NB;
            const h2 s2 = as_h2((uint32_t)ksc | ((uint32_t)ksc << 16));
            const uint32_t *cw = (const uint32_t *)kq;
#pragma unroll
            for (int i = 0; i < 4; i++) {                   // codes 8i .. 8i+7
                h2 c[4];
                fq_codes4(cw[2 * i], c[0], c[1]);
                fq_codes4(cw[2 * i + 1], c[2], c[3]);
                uint4 hv, lv;
                fq_split(c[0], s2, hv.x, lv.x);
                fq_split(c[1], s2, hv.y, lv.y);
                fq_split(c[2], s2, hv.z, lv.z);
                fq_split(c[3], s2, hv.w, lv.w);
                *(uint4 *)&Ks[0][key][32 * blk + 8 * i] = hv;
                *(uint4 *)&Ks[1][key][32 * blk + 8 * i] = lv;
            }
        }
        if (tid < VPC) {
            const int key = 2 * (tid & 31), hb = tid >> 5;
            const int col = vt_col(key);                    // even; key + 1 sits at col + 1
            uint32_t hk[2][8], lk[2][8];                    // [key][dim pair]
#pragma unroll
            for (int j = 0; j < 2; j++) {
                const h2 s2 = as_h2((uint32_t)vsc[j] | ((uint32_t)vsc[j] << 16));
                const uint32_t *cw = (const uint32_t *)&vq[j];
#pragma unroll
                for (int q = 0; q < 4; q++) {
                    h2 c0, c1;
                    fq_codes4(cw[q], c0, c1);
                    fq_split(c0, s2, hk[j][2 * q], lk[j][2 * q]);
                    fq_split(c1, s2, hk[j][2 * q + 1], lk[j][2 * q + 1]);
                }
            }
            // dim 2m takes the low halves of both keys' pair m, dim 2m+1 the high
#pragma unroll
            for (int m = 0; m < 8; m++) {
                *(uint32_t *)&Vt[0][16 * hb + 2 * m][col] = __builtin_amdgcn_perm(hk[1][m], hk[0][m], 0x05040100u);
                *(uint32_t *)&Vt[0][16 * hb + 2 * m + 1][col] = __builtin_amdgcn_perm(hk[1][m], hk[0][m], 0x07060302u);
                *(uint32_t *)&Vt[1][16 * hb + 2 * m][col] = __builtin_amdgcn_perm(lk[1][m], lk[0][m], 0x05040100u);
                *(uint32_t *)&Vt[1][16 * hb + 2 * m + 1][col] = __builtin_amdgcn_perm(lk[1][m], lk[0][m], 0x07060302u);
            }
        }
    };
    // the wavefront's first query position: key tiles wholly at or below it
    // need no causal mask (nor do full query tiles)
    const int qpos_min = p0 + tw;
    const bool tile_full = tw + 31 < T;
    if constexpr (Q8) load_q8(kbeg);
    else load_tile(kbeg);
    for (int kt = 0; kt < ntiles; kt++) {
        const int k0 = kbeg + kt * BKEY, buf = Q8 ? 0 : kt & 1;
        // ---- stage K and V^T of this tile; the next tile's loads then run
        // during this tile's arithmetic ----
        if constexpr (Q8) {
            if (kt > 0) __syncthreads();                    // every wavefront is done with the last tile
            store_q8();
        } else {
#pragma unroll
            for (int c = 0; c < CPT; c++) {
                const int ch = tid + c * 256, key = ch / (HD / 8), d8 = ch % (HD / 8);
                *(uint4 *)&Ks[buf][key][d8 * 8] = kr[c];
            }
#pragma unroll
            for (int c = 0; c < PPT; c++) {
                const int pc = tid + c * 256, key = 2 * (pc & 31), d8 = pc >> 5;
                const uint16_t *v0 = (const uint16_t *)&vr[c][0], *v1 = (const uint16_t *)&vr[c][1];
                const int col = vt_col(key);                // even; key + 1 sits at col + 1
#pragma unroll
                for (int e = 0; e < 8; e++)
                    *(uint32_t *)&Vt[buf][d8 * 8 + e][col] = (uint32_t)v0[e] | ((uint32_t)v1[e] << 16);
            }
        }
        __syncthreads();
        if (kt + 1 < ntiles) {
            if constexpr (Q8) load_q8(k0 + BKEY);
            else load_tile(k0 + BKEY);
        }

        // ---- S^T = K Q^T for two 32-key halves ----
        f16x s[2];
#pragma unroll
        for (int mt = 0; mt < 2; mt++) {
#pragma unroll
            for (int r = 0; r < 16; r++) s[mt][r] = 0.f;
#pragma unroll
            for (int ks = 0; ks < KS; ks++) {
                const h8 kf = *(const h8 *)&Ks[buf][mt * 32 + (lane & 31)][16 * ks + 8 * (lane >> 5)];
                s[mt] = __builtin_amdgcn_mfma_f32_32x32x16_f16(kf, qf[ks], s[mt], 0, 0, 0);
                s[mt] = __builtin_amdgcn_mfma_f32_32x32x16_f16(kf, ql[ks], s[mt], 0, 0, 0);
                if constexpr (Q8) {                         // K remainder x Q value (remainder x remainder dropped)
                    const h8 kl = *(const h8 *)&Ks[1][mt * 32 + (lane & 31)][16 * ks + 8 * (lane >> 5)];
                    s[mt] = __builtin_amdgcn_mfma_f32_32x32x16_f16(kl, qf[ks], s[mt], 0, 0, 0);
                }
            }
        }
        // ---- causal mask + online softmax over this query column ----
        float mt_max = -INFINITY;
        if (k0 + BKEY - 1 > qpos_min || !tile_full) {       // (uniform)
#pragma unroll
            for (int mt = 0; mt < 2; mt++)
#pragma unroll
                for (int r = 0; r < 16; r++) {
                    const int key = k0 + mt * 32 + (r >> 2) * 8 + (lane >> 5) * 4 + (r & 3);
                    if (key > qpos || !q_ok) s[mt][r] = -INFINITY;
                }
        }
#pragma unroll
        for (int mt = 0; mt < 2; mt++)
#pragma unroll
            for (int r = 0; r < 16; r++) mt_max = fmaxf(mt_max, s[mt][r]);
        mt_max = max_halves(mt_max);
        const float m_new = fmaxf(m_run, mt_max);
        // exponents are <= 0 here, so the plain hardware exp2 serves (results
        // below 2^-126 flush to zero, far under what an f16 P or the fp32 sum
        // keeps); while m_new is -inf every score is -inf and exp2(-inf) = 0
        const float alpha = m_new == -INFINITY ? 1.f : __builtin_amdgcn_exp2f(m_run - m_new);
        const float m_sub = m_new == -INFINITY ? 0.f : m_new;
        if (__ballot(alpha != 1.f))                         // (uniform: skipped while no max moved)
#pragma unroll
            for (int dt = 0; dt < DT; dt++)
#pragma unroll
                for (int r = 0; r < 16; r++) acc[dt][r] *= alpha;
        // ---- P and O^T += V^T P^T, one 32-key half at a time: the second
        // half's exp2 and conversions have no operand in the first half's
        // MFMAs, so the two overlap within the wavefront ----
        float psum = 0.f;
#pragma unroll
        for (int mt = 0; mt < 2; mt++) {
            h8 pf[2], pl[2];   // P as f16 value + remainder, like Q
#pragma unroll
            for (int r = 0; r < 16; r += 2) {
                const float p0 = __builtin_amdgcn_exp2f(s[mt][r] - m_sub);
                const float p1 = __builtin_amdgcn_exp2f(s[mt][r + 1] - m_sub);
                psum += p0;
                psum += p1;
                uint32_t pb = h2_bits(h2{(f16)p0, (f16)p1});  // one packed conversion ...
                asm volatile("" : "+v"(pb));                  // ... whose halves the remainders reuse
                const h2 ph = as_h2(pb);
                pf[r >> 3][r & 7] = ph.x;
                pf[r >> 3][(r & 7) + 1] = ph.y;
                pl[r >> 3][r & 7] = (f16)(p0 - (float)ph.x);
                pl[r >> 3][(r & 7) + 1] = (f16)(p1 - (float)ph.y);
            }
#pragma unroll
            for (int sh = 0; sh < 2; sh++) {
                const int ss = 2 * mt + sh;
#pragma unroll
                for (int dt = 0; dt < DT; dt++) {
                    const h8 vf = *(const h8 *)&Vt[buf][dt * 32 + (lane & 31)][16 * ss + 8 * (lane >> 5)];
                    acc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_f16(vf, pf[sh], acc[dt], 0, 0, 0);
                    acc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_f16(vf, pl[sh], acc[dt], 0, 0, 0);
                    if constexpr (Q8) {                     // V remainder x P value
                        const h8 vl = *(const h8 *)&Vt[1][dt * 32 + (lane & 31)][16 * ss + 8 * (lane >> 5)];
                        acc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_f16(vl, pf[sh], acc[dt], 0, 0, 0);
                    }
                }
            }
        }
        psum = sum_halves(psum);
        l_run = l_run * alpha + psum;
        m_run = m_new;
    }

    if (nsplit > 1) {
        // this range's unnormalized output and statistics (base 2), merged later
        if (q_ok) {
            const size_t hh = (size_t)q_t * a.H + head;
            float *pp = a.part + (hh * a.max_chunks + split) * HD;
#pragma unroll
            for (int dt = 0; dt < DT; dt++)
#pragma unroll
                for (int r4 = 0; r4 < 4; r4++) {
                    const int d = dt * 32 + r4 * 8 + (lane >> 5) * 4;
                    *(float4 *)(pp + d) = make_float4(acc[dt][r4 * 4], acc[dt][r4 * 4 + 1], acc[dt][r4 * 4 + 2],
                                                      acc[dt][r4 * 4 + 3]);
                }
            if (lane < 32) *(float2 *)(a.ml + (hh * a.max_chunks + split) * 2) = make_float2(m_run, l_run);
        }
        return;
    }
    // ---- O = O^T / l, f16 ----
    if (q_ok) {
        const float inv = 1.0f / l_run;
        const size_t ob = ((size_t)q_t * a.H + head) * HD;
#pragma unroll
        for (int dt = 0; dt < DT; dt++)
#pragma unroll
            for (int r4 = 0; r4 < 4; r4++) {
                const int d = dt * 32 + r4 * 8 + (lane >> 5) * 4;
                f16 hv[4], lv[4];
#pragma unroll
                for (int e = 0; e < 4; e++) {
                    const float y = acc[dt][r4 * 4 + e] * inv;
                    hv[e] = (f16)y;
                    lv[e] = (f16)(y - (float)hv[e]);
                }
                *(uint2 *)((f16 *)a.o + ob + d) = *(const uint2 *)hv;
                if (a.o_lo) *(uint2 *)((f16 *)a.o_lo + ob + d) = *(const uint2 *)lv;
            }
    }
}

// Token t (row of the ubatch), 256 (head, 4-dim) items per block: combines the
// key ranges of its tile in range order, M = max m_s, L = sum l_s 2^(m_s - M),
// o = sum acc_s 2^(m_s - M) / L.  Tiles that needed one range are skipped.
// A thread requests every range's (m, l) and partial before it adds any, so a
// token's loads are in flight together (at most FM_MAXNS ranges).
constexpr int FM_MAXNS = 8;
template <int HD>
__global__ __launch_bounds__(256) void k_flash_merge(FlashArgs a, int tile_tokens) {
    const int t = blockIdx.x, i = blockIdx.y * 256 + threadIdx.x;
    const int last_tok = min(a.T - 1, (t / tile_tokens) * tile_tokens + tile_tokens - 1);
    const int nsplit = min(a.ns, (a.tok.pos[0] + last_tok + 1 + a.chunk - 1) / a.chunk);   // a.ns <= FM_MAXNS
    if (nsplit <= 1 || i >= a.H * HD / 4) return;
    const int head = i / (HD / 4), d = (i % (HD / 4)) * 4;
    const size_t hh = (size_t)t * a.H + head;
    float2 ml[FM_MAXNS];
    float4 v[FM_MAXNS];
#pragma unroll
    for (int sp = 0; sp < FM_MAXNS; sp++)
        if (sp < nsplit) {
            ml[sp] = *(const float2 *)(a.ml + (hh * a.max_chunks + sp) * 2);
            v[sp] = *(const float4 *)(a.part + (hh * a.max_chunks + sp) * HD + d);
        }
    float M = -INFINITY;
#pragma unroll
    for (int sp = 0; sp < FM_MAXNS; sp++)
        if (sp < nsplit) M = fmaxf(M, ml[sp].x);
    float L = 0.f;
    float4 o = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
    for (int sp = 0; sp < FM_MAXNS; sp++)
        if (sp < nsplit) {
            const float f = ml[sp].x == -INFINITY ? 0.f : exp2f(ml[sp].x - M);
            L += ml[sp].y * f;
            o.x += v[sp].x * f;
            o.y += v[sp].y * f;
            o.z += v[sp].z * f;
            o.w += v[sp].w * f;
        }
    const float inv = 1.0f / L;
    const float y[4] = {o.x * inv, o.y * inv, o.z * inv, o.w * inv};
    f16 hv[4], lv[4];
#pragma unroll
    for (int e = 0; e < 4; e++) {
        hv[e] = (f16)y[e];
        lv[e] = (f16)(y[e] - (float)hv[e]);
    }
    const size_t ob = hh * HD + d;
    *(uint2 *)((f16 *)a.o + ob) = *(const uint2 *)hv;
    if (a.o_lo) *(uint2 *)((f16 *)a.o_lo + ob) = *(const uint2 *)lv;
}

}  // namespace

bool launch_flash_prefill(const FlashArgs &a_in, hipStream_t s) {
    FlashArgs a = a_in;
    if ((a.kv.kvtype != T_F16 && a.kv.kvtype != T_Q8_0) || a.T <= 0) return false;
    const bool q8 = a.kv.kvtype == T_Q8_0;
    const int G = a.H / a.kv.n_kv;
    if (G != 1 && G != 2 && G != 4 && G != 8) return false;
    const int Gb = G < 4 ? G : 4, Tb = 4 / Gb;
    const int tiles = (a.T + 32 * Tb - 1) / (32 * Tb);
    // key ranges per token tile: enough blocks for two wavefronts per SIMD
    // (512 blocks of 4 on 256 compute units), ranges of whole 64-key tiles
    const long long blocks = (long long)tiles * a.kv.n_kv * (G / Gb);
    int ns = (int)((g_flash_blocks + blocks - 1) / blocks);
    ns = ns < 1 ? 1 : ns > FM_MAXNS ? FM_MAXNS : ns;
    if (!a.part || !a.ml) ns = 1;
    if (ns > a.max_chunks) ns = a.max_chunks > 0 ? a.max_chunks : 1;
    const int max_keys = a.tok_pos0_max + a.T;            // keys of the last tile (host-side bound)
    int chunk = (max_keys + ns - 1) / ns;
    chunk = (chunk + 63) / 64 * 64;
    if (ns == 1) chunk = max_keys + 64;
    a.ns = ns;
    a.chunk = chunk;
    const dim3 grid(tiles * ns, a.kv.n_kv, G / Gb);
    switch (a.kv.hd) {
    case 64:
        if (q8) launch(k_flash_prefill<64, true>, grid, dim3(256), 0, s, a);
        else launch(k_flash_prefill<64, false>, grid, dim3(256), 0, s, a);
        if (ns > 1) launch(k_flash_merge<64>, dim3(a.T, (a.H * 16 + 255) / 256), dim3(256), 0, s, a, 32 * Tb);
        return true;
    case 128:
        if (q8) launch(k_flash_prefill<128, true>, grid, dim3(256), 0, s, a);
        else launch(k_flash_prefill<128, false>, grid, dim3(256), 0, s, a);
        if (ns > 1) launch(k_flash_merge<128>, dim3(a.T, (a.H * 32 + 255) / 256), dim3(256), 0, s, a, 32 * Tb);
        return true;
    default: return false;
    }
}
