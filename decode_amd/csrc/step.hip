// step.hip -- one decode step of one token as a single persistent kernel (gfx950).
//
// At batch 1 a decode step reads every weight byte once: the article's
// per-layer graph (RMSNorm, QKV, RoPE, KV append, attention, output
// projection, FFN) is a chain of mat-vecs and one small attention, each of
// which streams a few MB per compute unit.  Launched kernel by kernel, every
// link of that chain pays a launch, a ramp-up and a drain.  Here one grid of
// one 1024-thread block per compute unit runs the whole step:
//
//   embedding | per layer: QKV+RoPE+append | attention | O+residual |
//   gate/up+SwiGLU | down+residual | ... | output projection | argmax
//
// with a grid barrier at every "|".
//
// Coherence.  The L2 of an XCD is not coherent with the other XCDs' L2s.
// Data that one block writes and another reads within the launch (the
// residual row, its sums of squares, q, the attention partials and output,
// the SwiGLU row, the new K/V rows) is written with device-scope stores
// (write-through) and, where a stale copy could sit in the reader's L2 (a
// buffer rewritten every layer), read with device-scope loads.  A new K/V
// row is read with plain loads: its cache lines are read by exactly one
// block once per launch, after they were written, so no XCD holds an older
// copy (kernel boundaries write back and invalidate the L2s).  Each wave
// waits for its stores (vmcnt 0) before its block arrives at a barrier.
//
// Barrier.  Two levels of device-scope atomic counters: blocks arrive on
// the counter of their group (block % 8), the last of a group arrives on the
// top counter, the last of all writes the barrier number into each group's
// release word, and a group's blocks poll their own word.  Barrier numbers
// run on across launches (the host passes how many barriers came before),
// so nothing is reset between steps.  Every wait is bounded: a wait that
// times out raises the failure word, every later wait returns at once, the
// grid drains, and the step's token reads -1.
//
// Arithmetic is that of the kernel-by-kernel path: the mat-vec phases use
// the same exact-code block dots, the same K slices and slice order, so
// their outputs are bitwise those of k_matvec; the attention is the same
// MFMA tile math (S^T = K Q^T, O = P V on f16 value + remainder operands)
// with an online softmax over 32-key pieces, merged in LDS per block and
// across the blocks of a KV head by the last block to finish.
#include "common.h"
#include "epilogue.h"
#include "kernels.h"
#include "mvcore.h"

namespace {

constexpr int NW = 8;               // wavefronts per block (256 registers each)
constexpr int NT = NW * 64;
constexpr int MV_MAXIT_S = 16;      // row pairs per wavefront when K is split
constexpr int SPIN_LIMIT = 1 << 21; // polls before a wait gives up (seconds)

// ---- device-scope (cross-XCD coherent) loads and stores -------------------
DEV uint32_t ldc32(const void *p) {
    return __hip_atomic_load(gl((uint32_t *)p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
DEV uint64_t ldc64(const void *p) {
    return __hip_atomic_load(gl((uint64_t *)p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
DEV float ldcf(const float *p) { return __builtin_bit_cast(float, ldc32(p)); }
DEV f4 ldc_f4(const float *p) {
    const uint64_t a = ldc64(p), b = ldc64(p + 2);
    f4 r;
    r[0] = __builtin_bit_cast(float, (uint32_t)a);
    r[1] = __builtin_bit_cast(float, (uint32_t)(a >> 32));
    r[2] = __builtin_bit_cast(float, (uint32_t)b);
    r[3] = __builtin_bit_cast(float, (uint32_t)(b >> 32));
    return r;
}
DEV void stc32(void *p, uint32_t v) {
    __hip_atomic_store(gl((uint32_t *)p), v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
DEV void stc16(void *p, uint16_t v) {
    __hip_atomic_store(gl((uint16_t *)p), v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
DEV void stcf(float *p, float v) { stc32(p, __builtin_bit_cast(uint32_t, v)); }
DEV uint32_t atom_add(uint32_t *p) {
    return __hip_atomic_fetch_add(gl(p), 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// waits until every memory operation of this wavefront has completed
DEV void wait_vm() { __builtin_amdgcn_s_waitcnt(0 | (0x7 << 4) | (0xf << 8)); }

// ---- LDS plan (one array, phases take turns) -------------------------------
// mat-vec: image [512][XROW] u32 | bsum [512] | red [16] | part [512] | amax [2][16]
// attention: q [2][8][hd] f16 | wm [NW][8] | wl [NW][8] | wo [NW][8][hd] | mlj [8][STEP_BPG_MAX][2]
constexpr int IMG_WORDS = (MV_KMAX / 32) * XROW;
constexpr int SM_BSUM = IMG_WORDS, SM_RED = SM_BSUM + 512, SM_PART = SM_RED + 16, SM_AMAX = SM_PART + 512;
constexpr int SM_MV_END = SM_AMAX + 32;
constexpr int ATT_WORDS = (2 * 8 * 128) / 2 + 2 * NW * 8 + NW * 8 * 128 + 8 * STEP_BPG_MAX * 2;
constexpr int SMEM_WORDS = SM_MV_END > ATT_WORDS ? SM_MV_END : ATT_WORDS;

struct Shared {
    int fail, last;
};

// threadIdx.x as a value the compiler cannot trace back to the thread id: each
// phase takes its own copy, so no lane-dependent address arithmetic is hoisted
// out of the layer loop and kept live (spilled) across every phase.
DEV int phase_tid() {
    int t = (int)threadIdx.x;
    asm volatile("" : "+v"(t));
    return t;
}

// ---- grid barrier ----------------------------------------------------------
DEV void grid_barrier(uint32_t *m, uint32_t n0, uint32_t &nbar, Shared &sh) {
    ++nbar;
    __syncthreads();
    if (threadIdx.x == 0 && !sh.fail) {
        const uint32_t n = n0 + nbar;
        const int ng = (int)gridDim.x < 8 ? (int)gridDim.x : 8;
        const int grp = (int)blockIdx.x % ng;
        const uint32_t gsize = (gridDim.x - grp + ng - 1) / ng;
        const uint32_t old = atom_add(m + 64 * grp);
        if (old == n * gsize - 1u) {
            const uint32_t ot = atom_add(m + 64 * 8);
            if (ot == n * (uint32_t)ng - 1u)
                for (int k = 0; k < ng; k++) stc32(m + 64 * (9 + k), n);
        }
        int spins = 0;
        while (ldc32(m + 64 * (9 + grp)) != n) {
            if ((++spins & 255) == 0 && (ldc32(m + STEP_SYNC_FAIL) != 0u || spins > SPIN_LIMIT)) {
                stc32(m + STEP_SYNC_FAIL, 1u);
                sh.fail = 1;
                break;
            }
            __builtin_amdgcn_s_sleep(1);
        }
    }
    __syncthreads();
}

// ---- mat-vec phase ---------------------------------------------------------
// Work split as in k_matvec: S wavefronts share a row pair, one K slice
// each; the block's G = 16/S groups take pairs blockIdx*G + grp + i*stride.
struct MvGeo {
    int S, G, slice, grp, b0, b1, npairs, stride, first, iters;
};
DEV MvGeo mv_geo(const QMat &W, int S, int tid) {
    MvGeo g;
    const int w = tid >> 6;
    g.S = S;
    g.G = NW / S;
    g.slice = w % S;
    g.grp = w / S;
    const int nb = W.K >> 5, nbs = (nb + S - 1) / S;
    g.b0 = g.slice * nbs;
    g.b1 = min(nb, g.b0 + nbs);
    g.npairs = W.N >> 1;
    g.stride = (int)gridDim.x * g.G;
    g.first = (int)blockIdx.x * g.G + g.grp;
    g.iters = (g.npairs + g.stride - 1) / g.stride;
    return g;
}

template <int WT>
constexpr int depth() { return WT == T_Q4_0 ? 4 : 2; }   // row pairs in flight per wavefront

template <int WT>
struct Pre {
    PairLoad<WT, 1> L[depth<WT>()];
};

template <int WT>
DEV void mv_issue(const QMat &W, const MvGeo &g, int mode, int it, int lane, PairLoad<WT, 1> &dst) {
    const int p = min(g.first + it * g.stride, g.npairs - 1);
    int r0, r1;
    pair_rows(mode, p, r0, r1);
    load_pair<WT, 1>(W, r0, r1, g.b0, g.b1, lane, dst);
}

// The first row pairs of a phase, requested before the barrier that opens it
// (weights do not depend on the barrier).
template <int WT>
DEV void mv_prefetch(const QMat &W, int S, int mode, Pre<WT> &pf) {
    const int tid = phase_tid();
    const MvGeo g = mv_geo(W, S, tid);
#pragma unroll
    for (int k = 0; k < depth<WT>(); k++) mv_issue<WT>(W, g, mode, k, tid & 63, pf.L[k]);
}

struct MvIn {
    const float *x32 = nullptr, *g = nullptr, *ss = nullptr;   // RMSNorm prologue
    const uint16_t *xh = nullptr, *xl = nullptr;                  // f16 value + remainder row
};

// epilogue inputs read ahead (old residual values, RoPE factors)
struct EPre {
    float y0 = 0.f, y1 = 0.f;
    float2 cs = make_float2(1.f, 0.f);
};

template <int EPI>
DEV EPre epre(const StepArgs &a, int pos, int r0, int r1) {
    EPre e;
    if (EPI == EPI_RESID) {
        e.y0 = ldcf(a.x + r0);
        e.y1 = ldcf(a.x + r1);
    } else if (EPI == EPI_QKV) {
        if (r0 < a.qd + a.kd) {
            const int rr = r0 < a.qd ? r0 : r0 - a.qd;
            e.cs = *(const GLB float2 *)(gl(a.rope_cs) + ((size_t)pos * (a.hd >> 1) + ((rr % a.hd) >> 1)) * 2);
        }
    }
    return e;
}

struct Amax {
    float v = -INFINITY;
    int i = 0x7fffffff;
};
DEV void amax_take(Amax &m, float v, int i) {
    if (v > m.v || (v == m.v && i < m.i)) {
        m.v = v;
        m.i = i;
    }
}

template <int EPI>
DEV void step_epi(const StepArgs &a, const StepLayer &Ly, int pos, int seq, int p, int r0, int r1,
                  float v0, float v1, const EPre &e, float &ssq, Amax &am) {
    if (EPI == EPI_RESID) {
        const float y0 = e.y0 + v0, y1 = e.y1 + v1;
        stcf(a.x + r0, y0);
        stcf(a.x + r1, y1);
        ssq += y0 * y0 + y1 * y1;
    } else if (EPI == EPI_SWIGLU) {
        const float hv = silu(v0) * v1;
        const f16 hh = (f16)hv;
        stc16(a.h + p, __builtin_bit_cast(uint16_t, hh));
        stc16(a.h_lo + p, __builtin_bit_cast(uint16_t, (f16)(hv - (float)hh)));
    } else if (EPI == EPI_STORE) {
        gl(a.logits)[r0] = v0;
        gl(a.logits)[r1] = v1;
        amax_take(am, v0, r0);
        amax_take(am, v1, r1);
    } else if (EPI == EPI_QKV) {
        const int hd = a.hd;
        if (r0 < a.qd + a.kd) {
            const float ra = v0 * e.cs.x - v1 * e.cs.y;
            const float rb = v0 * e.cs.y + v1 * e.cs.x;
            if (r0 < a.qd) {
                const float ya = ra * a.qscale, yb = rb * a.qscale;
                h2 vh, vl;
                vh.x = (f16)ya;
                vh.y = (f16)yb;
                vl.x = (f16)(ya - (float)vh.x);
                vl.y = (f16)(yb - (float)vh.y);
                stc32(a.qh + r0, h2_bits(vh));
                stc32(a.ql + r0, h2_bits(vl));
            } else {
                const int rr = r0 - a.qd, gk = rr / hd, el = rr % hd;
                h2 kv;
                kv.x = (f16)ra;
                kv.y = (f16)rb;
                stc32(Ly.k + (((size_t)seq * a.Hkv + gk) * a.n_ctx + pos) * hd + el, h2_bits(kv));
            }
        } else {
            const int rr = r0 - a.qd - a.kd, gk = rr / hd, el = rr % hd;
            h2 kv;
            kv.x = (f16)v0;
            kv.y = (f16)v1;
            stc32(Ly.v + (((size_t)seq * a.Hkv + gk) * a.n_ctx + pos) * hd + el, h2_bits(kv));
        }
    }
}

// One mat-vec of the step: entered with the phase's first row pairs in
// flight (pf, requested before the barrier), leaves every store of the
// phase issued.  GPT: 4-element groups of the input row per thread
// (K <= 4 NT GPT).
template <int WT, int EPI, int GPT, int S>
DEV void mv_phase_s(const StepArgs &a, const StepLayer &Ly, const QMat &W, int mode, const MvIn &in,
                    Pre<WT> &pf, uint32_t *sm, int pos, int seq) {
    constexpr bool NORM = EPI != EPI_RESID;
    constexpr int D = depth<WT>();
    uint32_t *img = sm;
    float *bsum = (float *)(sm + SM_BSUM);
    float *red = (float *)(sm + SM_RED);
    float *part = (float *)(sm + SM_PART);
    const int tid = phase_tid(), lane = tid & 63, w = tid >> 6;
    const int K = W.K;
    const MvGeo g = mv_geo(W, S, tid);
    const int G = g.G, iters = g.iters;

    // with a split K, thread i finishes item i (group, pair) after the last pair
    int fin_p = -1, fin_r0 = 0, fin_r1 = 1;
    EPre fin_pre;
    if (S > 1 && tid < G * iters) {
        const int gi = tid / iters, it = tid % iters;
        const int p = (int)blockIdx.x * G + gi + it * g.stride;
        if (p < g.npairs) {
            fin_p = p;
            pair_rows(mode, p, fin_r0, fin_r1);
            fin_pre = epre<EPI>(a, pos, fin_r0, fin_r1);
        }
    }

    // ---- LDS image of the input row (device-scope loads of rows the other
    // blocks wrote) ----
    {
        const int n4 = K >> 2;
        typedef _Float16 h4 __attribute__((ext_vector_type(4)));
        f4 xv[GPT], gv[GPT];
        h4 hv4[GPT], lv4[GPT];
        float sp = 0.f;
        if (NORM) sp = (ldcf(in.ss + 4 * lane) + ldcf(in.ss + 4 * lane + 1)) +
                       (ldcf(in.ss + 4 * lane + 2) + ldcf(in.ss + 4 * lane + 3));
#pragma unroll
        for (int j = 0; j < GPT; j++) {
            if (j * NT >= n4) break;                 // uniform
            const int q = min(tid + j * NT, n4 - 1);
            if (NORM) {
                xv[j] = ldc_f4(in.x32 + 4 * q);
                gv[j] = *(const GLB f4 *)(gl(in.g) + 4 * q);
            } else {
                hv4[j] = __builtin_bit_cast(h4, ldc64(in.xh + 4 * q));
                lv4[j] = __builtin_bit_cast(h4, ldc64(in.xl + 4 * q));
            }
        }
        float rs = 0.f;
        if (NORM) {
            const float ss = wave_sum_dpp(sp);
            rs = 1.0f / sqrtf(ss / (float)K + a.eps);
        }
#pragma unroll
        for (int j = 0; j < GPT; j++) {
            const int q = tid + j * NT;
            if (j * NT >= n4) break;
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
            float v = 0.f;
            if (q < n4) v = put_group<WT>(img, q >> 3, q & 7, hv, lv);
            v += __shfl_xor(v, 1, 64);
            v += __shfl_xor(v, 2, 64);
            v += __shfl_xor(v, 4, 64);
            if (q < n4 && (q & 7) == 0) bsum[q >> 3] = v;
        }
    }
    __syncthreads();

    const int bl = g.b0 + lane;
    const bool lane_ok = bl < g.b1;
    h2 xp[32];
    {
        const uint32_t *row = img + (size_t)(lane_ok ? bl : g.b0) * XROW;
#pragma unroll
        for (int j = 0; j < 8; j++) {
            u32x4 v = *(const u32x4 *)(row + 4 * j);
            if (!lane_ok) v = u32x4{0u, 0u, 0u, 0u};
            xp[4 * j] = as_h2(v.x);
            xp[4 * j + 1] = as_h2(v.y);
            xp[4 * j + 2] = as_h2(v.z);
            xp[4 * j + 3] = as_h2(v.w);
        }
    }
    const float xs = lane_ok ? bsum[bl] : 0.f;

    const Masks mk = make_masks();
    float ssq = 0.f;
    Amax am;
    auto step = [&](PairLoad<WT, 1> &cur, int it) __attribute__((always_inline)) {
        if (it >= iters) return;
        const int p = g.first + it * g.stride;
        float bd0, bd1;
        if (WT == T_Q4_0) {
            bd0 = blockdot_q4(cur.q[0][0][0], xp, mk);
            bd1 = blockdot_q4(cur.q[1][0][0], xp, mk);
        } else {
            bd0 = blockdot_q8(cur.q[0][0][0], cur.q[0][0][WT == T_Q4_0 ? 0 : 1], xp, mk);
            bd1 = blockdot_q8(cur.q[1][0][0], cur.q[1][0][WT == T_Q4_0 ? 0 : 1], xp, mk);
        }
        float a0 = f16_bits_to_f32((uint16_t)(cur.d[0][0] >> cur.dsh[0][0])) * (bd0 - xs);
        float a1 = f16_bits_to_f32((uint16_t)(cur.d[1][0] >> cur.dsh[1][0])) * (bd1 - xs);
        // refill with the pair D ahead, unconditionally (past the end: the last
        // pair again, an L2 hit) so that every wait counts exactly D pairs
        __builtin_amdgcn_sched_barrier(0);
        mv_issue<WT>(W, g, mode, it + D, lane, cur);
        __builtin_amdgcn_sched_barrier(0);
        a0 = wave_sum_dpp(a0);
        a1 = wave_sum_dpp(a1);
        if (p < g.npairs && lane == 0) {
            if (S == 1) {
                int r0, r1;
                pair_rows(mode, p, r0, r1);
                const EPre e = epre<EPI>(a, pos, r0, r1);
                step_epi<EPI>(a, Ly, pos, seq, p, r0, r1, a0, a1, e, ssq, am);
            } else {
                float *pp = part + ((g.grp * MV_MAXIT_S + it) * S + g.slice) * 2;
                pp[0] = a0;
                pp[1] = a1;
            }
        }
    };
    for (int it = 0; it < iters; it += D) {
#pragma unroll
        for (int k = 0; k < D; k++) step(pf.L[k], it + k);
    }
    if (S > 1) {
        __syncthreads();
        if (fin_p >= 0) {
            const int gi = tid / iters, it = tid % iters;
            float s0 = 0.f, s1 = 0.f;
            for (int j = 0; j < S; j++) {
                s0 += part[((gi * MV_MAXIT_S + it) * S + j) * 2];
                s1 += part[((gi * MV_MAXIT_S + it) * S + j) * 2 + 1];
            }
            step_epi<EPI>(a, Ly, pos, seq, fin_p, fin_r0, fin_r1, s0, s1, fin_pre, ssq, am);
        }
    }
    if (EPI == EPI_RESID) {
        // this block's share of the new row's sum of squares -> slot blockIdx.x
        ssq = wave_sum_dpp(ssq);
        __syncthreads();                 // (red may still be read by an earlier use)
        if (lane == 0) red[w] = ssq;
        __syncthreads();
        if (tid == 0) {
            float tot = 0.f;
#pragma unroll
            for (int i = 0; i < NW; i++) tot += red[i];
            stcf(a.ss + blockIdx.x, tot);
        }
    }
    if (EPI == EPI_STORE) {
        float *av = (float *)(sm + SM_AMAX);
        int *ai = (int *)(sm + SM_AMAX + 16);
#pragma unroll
        for (int o = 32; o > 0; o >>= 1) {
            const float ov = __shfl_xor(am.v, o, 64);
            const int oi = __shfl_xor(am.i, o, 64);
            amax_take(am, ov, oi);
        }
        __syncthreads();
        if (lane == 0) {
            av[w] = am.v;
            ai[w] = am.i;
        }
        __syncthreads();
        if (tid == 0) {
            for (int k = 1; k < NW; k++) amax_take(am, av[k], ai[k]);
            stcf(a.bmax + blockIdx.x, am.v);
            stc32(a.bidx + blockIdx.x, (uint32_t)am.i);
        }
    }
}

template <int WT, int EPI, int GPT>
DEV void mv_phase(const StepArgs &a, const StepLayer &Ly, const QMat &W, int S, int mode, const MvIn &in,
                  Pre<WT> &pf, uint32_t *sm, int pos, int seq) {
    switch (S) {
    case 1: mv_phase_s<WT, EPI, GPT, 1>(a, Ly, W, mode, in, pf, sm, pos, seq); break;
    case 2: mv_phase_s<WT, EPI, GPT, 2>(a, Ly, W, mode, in, pf, sm, pos, seq); break;
    case 4: mv_phase_s<WT, EPI, GPT, 4>(a, Ly, W, mode, in, pf, sm, pos, seq); break;
    default: mv_phase_s<WT, EPI, GPT, 8>(a, Ly, W, mode, in, pf, sm, pos, seq); break;
    }
}

// ---- embedding ---------------------------------------------------------------
DEV void embed_phase(const StepArgs &a, int row, uint32_t *sm) {
    float *red = (float *)(sm + SM_RED);
    const QMat &E = a.tok;
    const int K = a.d, nb = K >> 5, tid = phase_tid();
    float ss = 0.f;
    for (int j = (int)blockIdx.x * NT + tid; j < K; j += (int)gridDim.x * NT) {
        const int b = j >> 5, e = j & 31;
        const float d = f16_bits_to_f32(gl(E.d)[(size_t)row * nb + b]);
        float v;
        if (E.wtype == T_Q8_0) {
            v = (float)((const GLB int8_t *)gl(E.qs))[(size_t)row * K + j] * d;
        } else {
            const uint8_t byte = ((const GLB uint8_t *)gl(E.qs))[(size_t)row * (K >> 1) + b * 16 + (e & 15)];
            const int c = e < 16 ? (byte & 15) : (byte >> 4);
            v = (float)(c - 8) * d;
        }
        stcf(a.x + j, v);
        ss += v * v;
    }
    ss = wave_sum_dpp(ss);
    if ((tid & 63) == 0) red[tid >> 6] = ss;
    __syncthreads();
    if (tid == 0) {
        float tot = 0.f;
        for (int i = 0; i < NW; i++) tot += red[i];
        stcf(a.ss + blockIdx.x, tot);
    }
    if (blockIdx.x == 0)
        for (int i = (int)gridDim.x + tid; i < SS_SLOTS; i += NT) stcf(a.ss + i, 0.f);
}

// ---- attention -----------------------------------------------------------
// Block b serves KV head g = b / bpg with the 32-key pieces
// [j np / bpg, (j+1) np / bpg) of the context (j = b % bpg, np pieces);
// wavefront w takes pieces w, w + NW, ... of that range with an online
// softmax.  The wavefronts meet in LDS, the block writes one partial (max,
// sum, unnormalized output) per query head of the group, and the last block
// of the KV head to finish merges the partials into o.
//
// Per piece (32 keys, one wavefront), as in the per-layer MFMA kernel:
//   S^T = K Q^T on v_mfma_f32_32x32x16_f16: K rows as the A operand, q /
//         sqrt(hd) (value + remainder, staged in LDS) as B, so every product
//         is exact; a lane's accumulators hold 16 keys of head lane%32;
//   O   = P V with P (value + remainder) taken from the accumulators as they
//         lie and V gathered from the cache as the B operand (element e of
//         lane l: key 16 s + 8 (e/4) + 4 (l/32) + e%4, dim 32 dt + l%32).
template <int HD>
struct Piece {
    h8 kf[HD / 16];
    h8 vb[HD / 32][2];
};

template <int HD>
DEV void piece_load(const GLB f16 *Kb, const GLB f16 *Vb, int k0, int pos, int ln, int hf, Piece<HD> &P) {
    const int kr = min(k0 + ln, pos);     // rows past pos: row pos again (finite, weight 0)
#pragma unroll
    for (int ks = 0; ks < HD / 16; ks++) P.kf[ks] = *(const GLB h8 *)(Kb + (size_t)kr * HD + 16 * ks + 8 * hf);
#pragma unroll
    for (int s = 0; s < 2; s++)
#pragma unroll
        for (int e = 0; e < 8; e++) {
            const int key = min(k0 + 16 * s + 8 * (e >> 2) + 4 * hf + (e & 3), pos);
#pragma unroll
            for (int dt = 0; dt < HD / 32; dt++) P.vb[dt][s][e] = Vb[(size_t)key * HD + 32 * dt + ln];
        }
}

template <int HD>
DEV void attn_phase(const StepArgs &a, const StepLayer &Ly, int pos, int seq, uint32_t *sm, Shared &sh) {
    constexpr int KS = HD / 16, DT = HD / 32;
    const int tid = phase_tid(), lane = tid & 63, w = tid >> 6, hf = lane >> 5, ln = lane & 31;
    const int G = a.H / a.Hkv, bpg = a.bpg;
    const int g = (int)blockIdx.x / bpg, j = (int)blockIdx.x % bpg;
    if (g >= a.Hkv) return;
    const int np = pos / 32 + 1;
    const int pb = (int)((long long)j * np / bpg), pe = (int)((long long)(j + 1) * np / bpg);
    if (pb >= pe) return;
    const int nact = min(np, bpg);
    f16 *qs = (f16 *)sm;                    // [2][8][HD]: value, remainder
    float *wm = (float *)(sm + 8 * HD);     // [NW][8]
    float *wl = wm + NW * 8;                // [NW][8]
    float *wo = wl + NW * 8;                // [NW][8][HD]
    float *mlj = wo + NW * 8 * HD;          // [8][STEP_BPG_MAX][2]

    const size_t base = (((size_t)seq * a.Hkv + g) * a.n_ctx) * HD;
    const GLB f16 *Kb = (const GLB f16 *)gl(Ly.k) + base;
    const GLB f16 *Vb = (const GLB f16 *)gl(Ly.v) + base;
    const int rounds = (pe - pb + NW - 1) / NW;
    Piece<HD> P;
    // the first piece's K and V are requested before q (they do not wait for it)
    if (pb + w < pe) piece_load<HD>(Kb, Vb, (pb + w) * 32, pos, ln, hf, P);
    for (int i = tid; i < G * HD / 2; i += NT) {
        ((uint32_t *)qs)[i] = ldc32(a.qh + (size_t)g * G * HD + 2 * i);
        ((uint32_t *)(qs + 8 * HD))[i] = ldc32(a.ql + (size_t)g * G * HD + 2 * i);
    }
    // the wavefront's running output lives in its LDS slot: rows (heads)
    // 4 hf + r, dims 32 dt + ln of this lane
    float *myo = wo + (size_t)w * 8 * HD;
#pragma unroll
    for (int r = 0; r < 4; r++)
#pragma unroll
        for (int dt = 0; dt < DT; dt++) myo[(4 * hf + r) * HD + 32 * dt + ln] = 0.f;
    __syncthreads();

    float m_run = -INFINITY, l_run = 0.f;
    const int qrow = min(ln, G - 1);       // columns past the group repeat its last head (ignored)
    for (int rd = 0; rd < rounds; rd++) {
        const int piece = pb + w + NW * rd;
        if (piece >= pe) break;             // uniform per wavefront; later rounds have none either
        if (rd > 0) piece_load<HD>(Kb, Vb, piece * 32, pos, ln, hf, P);
        const int k0 = piece * 32;
        f16x sacc;
#pragma unroll
        for (int r = 0; r < 16; r++) sacc[r] = 0.f;
#pragma unroll
        for (int ks = 0; ks < KS; ks++) {
            const h8 qa = *(const h8 *)(qs + qrow * HD + 16 * ks + 8 * hf);
            const h8 qb = *(const h8 *)(qs + 8 * HD + qrow * HD + 16 * ks + 8 * hf);
            sacc = __builtin_amdgcn_mfma_f32_32x32x16_f16(P.kf[ks], qa, sacc, 0, 0, 0);
            sacc = __builtin_amdgcn_mfma_f32_32x32x16_f16(P.kf[ks], qb, sacc, 0, 0, 0);
        }
        // causal mask; the lane holds 16 keys of head ln, lane ^ 32 the other 16
        float mp = -INFINITY;
#pragma unroll
        for (int r = 0; r < 16; r++) {
            const int key = k0 + (r >> 2) * 8 + 4 * hf + (r & 3);
            if (key > pos) sacc[r] = -INFINITY;
            mp = fmaxf(mp, sacc[r]);
        }
        mp = fmaxf(mp, __shfl_xor(mp, 32, 64));
        const float mn = fmaxf(m_run, mp);      // finite: key k0 <= pos is in every piece
        const float alpha = m_run == -INFINITY ? 0.f : __expf(m_run - mn);
        float ls = 0.f;
        h8 ph[2], pl[2];
#pragma unroll
        for (int r = 0; r < 16; r++) {
            const float p = __expf(sacc[r] - mn);
            ls += p;
            const f16 p16 = (f16)p;
            ph[r >> 3][r & 7] = p16;
            pl[r >> 3][r & 7] = (f16)(p - (float)p16);
        }
        ls += __shfl_xor(ls, 32, 64);
        l_run = l_run * alpha + ls;
        m_run = mn;
        // rescale factors of the output rows this lane holds: heads 4 hf + r
        float ar[4];
#pragma unroll
        for (int r = 0; r < 4; r++) {
            const float a0 = readlane_f(alpha, r), a1 = readlane_f(alpha, 4 + r);
            ar[r] = hf ? a1 : a0;
        }
#pragma unroll
        for (int dt = 0; dt < DT; dt++) {
            f16x t;
#pragma unroll
            for (int r = 0; r < 16; r++) t[r] = 0.f;
#pragma unroll
            for (int s = 0; s < 2; s++) {
                t = __builtin_amdgcn_mfma_f32_32x32x16_f16(ph[s], P.vb[dt][s], t, 0, 0, 0);
                t = __builtin_amdgcn_mfma_f32_32x32x16_f16(pl[s], P.vb[dt][s], t, 0, 0, 0);
            }
#pragma unroll
            for (int r = 0; r < 4; r++) {
                float *op = myo + (4 * hf + r) * HD + 32 * dt + ln;
                *op = *op * ar[r] + t[r];
            }
        }
    }
    // the wavefront's statistics -> LDS (wavefronts without a piece leave m = -inf, l = 0, o = 0)
    if (hf == 0 && ln < 8) {
        wm[w * 8 + ln] = m_run;
        wl[w * 8 + ln] = l_run;
    }
    __syncthreads();
    float *pbase = a.apart + ((size_t)g * bpg + j) * G * HD;
    float *mbase = a.aml + ((size_t)g * bpg + j) * G * 2;
    for (int i = tid; i < G * HD; i += NT) {
        const int h = i / HD, dd = i % HD;
        float M = -INFINITY;
#pragma unroll
        for (int k = 0; k < NW; k++) M = fmaxf(M, wm[k * 8 + h]);
        float acc = 0.f, L = 0.f;
#pragma unroll
        for (int k = 0; k < NW; k++) {
            const float f = wm[k * 8 + h] == -INFINITY ? 0.f : __expf(wm[k * 8 + h] - M);
            acc += wo[(k * 8 + h) * HD + dd] * f;
            L += wl[k * 8 + h] * f;
        }
        stcf(pbase + h * HD + dd, acc);
        if (dd == 0) {
            stcf(mbase + 2 * h, M);
            stcf(mbase + 2 * h + 1, L);
        }
    }
    wait_vm();
    __syncthreads();
    if (tid == 0) {
        uint32_t *cnt = a.sync + 64 * (24 + g);
        const uint32_t old = atom_add(cnt);
        sh.last = old == (uint32_t)nact - 1u;
        if (sh.last) stc32(cnt, 0u);            // next use: a later layer, after several barriers
    }
    __syncthreads();
    if (!sh.last) return;
    // ---- merge of the KV head's block partials: weights e^(M_j - M) in LDS,
    // then every partial row requested at once ----
    for (int i = tid; i < G * bpg; i += NT) {
        const int h = i / bpg, jj = i % bpg;
        const bool act = (long long)(jj + 1) * np / bpg > (long long)jj * np / bpg;
        float M = -INFINITY, L = 0.f;
        if (act) {
            const float *mb = a.aml + ((size_t)g * bpg + jj) * G * 2;
            M = ldcf(mb + 2 * h);
            L = ldcf(mb + 2 * h + 1);
        }
        mlj[(h * STEP_BPG_MAX + jj) * 2] = M;
        mlj[(h * STEP_BPG_MAX + jj) * 2 + 1] = L;
    }
    __syncthreads();
    if (tid < G) {
        const int h = tid;
        float M = -INFINITY;
        for (int jj = 0; jj < bpg; jj++) M = fmaxf(M, mlj[(h * STEP_BPG_MAX + jj) * 2]);
        float L = 0.f;
        for (int jj = 0; jj < bpg; jj++) {
            const float mj = mlj[(h * STEP_BPG_MAX + jj) * 2];
            const float f = mj == -INFINITY ? 0.f : __expf(mj - M);
            L += mlj[(h * STEP_BPG_MAX + jj) * 2 + 1] * f;
            mlj[(h * STEP_BPG_MAX + jj) * 2] = f;        // weight of partial jj
        }
        mlj[(h * STEP_BPG_MAX) * 2 + 1] = 1.0f / L;    // (slot 0's sum is no longer needed)
    }
    __syncthreads();
    for (int i = tid; i < G * HD; i += NT) {
        const int h = i / HD, dd = i % HD;
        const float *pr = a.apart + ((size_t)g * bpg * G + h) * HD + dd;   // partial jj at + jj G HD
        float acc = 0.f;
        for (int j0 = 0; j0 < bpg; j0 += 8) {
            float v[8];
#pragma unroll
            for (int u = 0; u < 8; u++) {
                const int jj = j0 + u;
                v[u] = jj < bpg && mlj[(h * STEP_BPG_MAX + jj) * 2] != 0.f ? ldcf(pr + (size_t)jj * G * HD) : 0.f;
            }
#pragma unroll
            for (int u = 0; u < 8; u++)
                if (j0 + u < bpg) acc += v[u] * mlj[(h * STEP_BPG_MAX + j0 + u) * 2];
        }
        const float ov = acc * mlj[(h * STEP_BPG_MAX) * 2 + 1];
        const f16 oh = (f16)ov;
        const size_t off = (size_t)(g * G + h) * HD + dd;
        stc16(a.o + off, __builtin_bit_cast(uint16_t, oh));
        stc16(a.o_lo + off, __builtin_bit_cast(uint16_t, (f16)(ov - (float)oh)));
    }
}

// ---- the step ------------------------------------------------------------------
// The argument block lives in device memory; each phase re-reads the fields
// it uses, so no argument stays in registers across the whole step.

template <int WT, int HD>
__global__ __launch_bounds__(NT) void k_step(const StepArgs *ap, uint32_t n0) {
    constexpr int GS = 4096 / (4 * NT), GB = MV_KMAX / (4 * NT);   // input groups per thread: rows <= 4096, longer
    __shared__ __attribute__((aligned(16))) uint32_t sm[SMEM_WORDS];
    __shared__ Shared sh;
    const int tid = threadIdx.x;
    if (tid == 0) {
        sh.fail = 0;
        sh.last = 0;
    }
    uint32_t nbar = 0;
    const int tok = ap->step[0], pos = ap->step[1], seq = ap->step[2];
    uint32_t *const sync = ap->sync;
    const int n_layer = ap->n_layer;
    Pre<WT> pf;
    embed_phase(*ap, tok, sm);
    wait_vm();
    {
        const StepArgs &a = *ap;
        mv_prefetch<WT>(a.layers[0].wqkv, a.S_qkv, PAIR_ADJ, pf);
    }
    grid_barrier(sync, n0, nbar, sh);
    for (int l = 0; l < n_layer; l++) {
        {
            const StepArgs &a = *ap;
            const StepLayer &Ly = a.layers[l];
            MvIn in;
            in.x32 = a.x;
            in.g = Ly.attn_norm;
            in.ss = a.ss;
            mv_phase<WT, EPI_QKV, GS>(a, Ly, Ly.wqkv, a.S_qkv, PAIR_ADJ, in, pf, sm, pos, seq);
        }
        wait_vm();
        grid_barrier(sync, n0, nbar, sh);
        {
            const StepArgs &a = *ap;
            attn_phase<HD>(a, a.layers[l], pos, seq, sm, sh);
        }
        wait_vm();
        {
            const StepArgs &a = *ap;
            mv_prefetch<WT>(a.layers[l].wo, a.S_o, PAIR_ADJ, pf);
        }
        grid_barrier(sync, n0, nbar, sh);
        {
            const StepArgs &a = *ap;
            const StepLayer &Ly = a.layers[l];
            MvIn io;
            io.xh = a.o;
            io.xl = a.o_lo;
            mv_phase<WT, EPI_RESID, GS>(a, Ly, Ly.wo, a.S_o, PAIR_ADJ, io, pf, sm, pos, seq);
        }
        wait_vm();
        {
            const StepArgs &a = *ap;
            mv_prefetch<WT>(a.layers[l].wgu, a.S_gu, PAIR_GU, pf);
        }
        grid_barrier(sync, n0, nbar, sh);
        {
            const StepArgs &a = *ap;
            const StepLayer &Ly = a.layers[l];
            MvIn ig;
            ig.x32 = a.x;
            ig.g = Ly.ffn_norm;
            ig.ss = a.ss;
            mv_phase<WT, EPI_SWIGLU, GS>(a, Ly, Ly.wgu, a.S_gu, PAIR_GU, ig, pf, sm, pos, seq);
        }
        wait_vm();
        {
            const StepArgs &a = *ap;
            mv_prefetch<WT>(a.layers[l].wdown, a.S_down, PAIR_ADJ, pf);
        }
        grid_barrier(sync, n0, nbar, sh);
        {
            const StepArgs &a = *ap;
            const StepLayer &Ly = a.layers[l];
            MvIn ih;
            ih.xh = a.h;
            ih.xl = a.h_lo;
            mv_phase<WT, EPI_RESID, GB>(a, Ly, Ly.wdown, a.S_down, PAIR_ADJ, ih, pf, sm, pos, seq);
        }
        wait_vm();
        {
            const StepArgs &a = *ap;
            if (l + 1 < n_layer)
                mv_prefetch<WT>(a.layers[l + 1].wqkv, a.S_qkv, PAIR_ADJ, pf);
            else
                mv_prefetch<WT>(a.out, a.S_out, PAIR_ADJ, pf);
        }
        grid_barrier(sync, n0, nbar, sh);
    }
    {
        const StepArgs &a = *ap;
        MvIn iout;
        iout.x32 = a.x;
        iout.g = a.out_norm;
        iout.ss = a.ss;
        mv_phase<WT, EPI_STORE, GS>(a, a.layers[0], a.out, a.S_out, PAIR_ADJ, iout, pf, sm, pos, seq);
    }
    wait_vm();
    grid_barrier(sync, n0, nbar, sh);
    if (blockIdx.x == 0) {
        const StepArgs &a = *ap;
        Amax am;
        for (int b = tid; b < (int)gridDim.x; b += NT) amax_take(am, ldcf(a.bmax + b), (int)ldc32(a.bidx + b));
#pragma unroll
        for (int o = 32; o > 0; o >>= 1) {
            const float ov = __shfl_xor(am.v, o, 64);
            const int oi = __shfl_xor(am.i, o, 64);
            amax_take(am, ov, oi);
        }
        float *av = (float *)(sm + SM_AMAX);
        int *ai = (int *)(sm + SM_AMAX + 16);
        if ((tid & 63) == 0) {
            av[tid >> 6] = am.v;
            ai[tid >> 6] = am.i;
        }
        __syncthreads();
        if (tid == 0) {
            for (int k = 1; k < NW; k++) amax_take(am, av[k], ai[k]);
            if (am.i == 0x7fffffff) am.i = 0;
            gl(a.amax)[0] = (sh.fail || ldc32(sync + STEP_SYNC_FAIL) != 0u) ? -1 : am.i;
        }
    }
}

}  // namespace

int step_slices(int N, int K, int grid) {
    // fewest K slices that keep a slice within 64 blocks (one per lane), more
    // while some wavefront of the grid would get no row pair or a wavefront
    // would hold more than MV_MAXIT_S of them
    const int nb = K / 32, npairs = N / 2;
    int S = 1;
    while (S * 64 < nb) S *= 2;
    auto iters = [&](int s) { return (npairs + grid * (NW / s) - 1) / (grid * (NW / s)); };
    while (S < NW && ((long long)npairs * S < (long long)NW * grid || iters(S) > MV_MAXIT_S)) S *= 2;
    return S;
}

bool step_supported(const StepArgs &a, int wtype, int kvtype, int grid, const char **why) {
    const char *r = nullptr;
    if (wtype != T_Q4_0 && wtype != T_Q8_0) r = "weights are not Q4_0 / Q8_0";
    else if (kvtype != T_F16) r = "cache is not f16";
    else if (a.hd != 64 && a.hd != 128) r = "head_dim is not 64 / 128";
    else if (a.Hkv <= 0 || a.Hkv > 64 || a.H % a.Hkv || a.H / a.Hkv > 8) r = "KV heads (at most 64, at most 8 query heads each)";
    else if (grid < 1 || grid > SS_SLOTS || grid < a.Hkv) r = "grid size";
    else if (a.d > 4096 || a.qd > 4096 || a.Fp > MV_KMAX) r = "d or H*hd above 4096, or F above 16384";
    else if (a.d % 32 || a.qd % 32 || a.Fp % 32) r = "row lengths not multiples of 32";
    else if (a.bpg < 1 || a.bpg > STEP_BPG_MAX || a.bpg * a.Hkv > grid) r = "attention blocks per KV head";
    else {
        // a split K keeps at most MV_MAXIT_S row pairs per wavefront
        const int dims[5][3] = {{a.qd + 2 * a.kd, a.d, a.S_qkv}, {a.d, a.qd, a.S_o}, {2 * a.Fp, a.d, a.S_gu},
                                {a.d, a.Fp, a.S_down}, {a.V, a.d, a.S_out}};
        for (auto &m : dims) {
            const int S = m[2], npairs = m[0] / 2, G = NW / S;
            if (S < 1 || S > NW || (S & (S - 1)) || (m[1] / 32 + S - 1) / S > 64) r = "K slices";
            else if (m[0] % 2) r = "odd row count";
            else if (S > 1 && (npairs + grid * G - 1) / (grid * G) > MV_MAXIT_S) r = "too many row pairs per wavefront";
            if (r) break;
        }
    }
    if (why) *why = r;
    return r == nullptr;
}

static const void *step_fn(int wtype, int hd) {
    if (wtype == T_Q4_0) return hd == 128 ? (const void *)k_step<T_Q4_0, 128> : (const void *)k_step<T_Q4_0, 64>;
    if (wtype == T_Q8_0) return hd == 128 ? (const void *)k_step<T_Q8_0, 128> : (const void *)k_step<T_Q8_0, 64>;
    return nullptr;
}

int step_blocks_per_cu(int wtype, int hd) {
    const void *fn = step_fn(wtype, hd);
    int n = 0;
    if (!fn || hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, fn, NT, 0) != hipSuccess) {
        (void)hipGetLastError();
        return 0;
    }
    return n;
}

bool launch_step(const StepArgs *dev_args, int wtype, int hd, uint32_t n0, int grid, hipStream_t s) {
    void *args[] = {(void *)&dev_args, (void *)&n0};
    const void *fn = step_fn(wtype, hd);
    if (!fn) return false;
    return hipLaunchCooperativeKernel(fn, dim3(grid), dim3(NT), args, 0, s) == hipSuccess;
}
