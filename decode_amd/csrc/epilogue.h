// epilogue.h -- output handling shared by the mat-vec and the GEMM kernels.
//
// Output rows are handled in pairs so that the two values a RoPE rotation
// or a SwiGLU product needs always meet in one lane:
//   PAIR_ADJ: pair p = rows (2p, 2p+1)    (RoPE rotates adjacent elements)
//   PAIR_GU : gate/up matrices are stored interleaved in groups of 32 rows
//             (32 gate rows, then the 32 matching up rows); pair p = feature p
//             = rows (64*(p/32) + p%32, same + 32).
#pragma once

#include "common.h"
#include "kernels.h"

DEV void pair_rows(int mode, int p, int &r0, int &r1) {
    if (mode == PAIR_GU) {
        r0 = ((p >> 5) << 6) + (p & 31);
        r1 = r0 + 32;
    } else {
        r0 = 2 * p;
        r1 = r0 + 1;
    }
}

// q after RoPE: f32, and when asked, q * qscale as f16 value + remainder
// (the exact operand form the decode attention's matrix cores take).
DEV void store_q_pair(const EpiArgs &e, int t, int r0, float ra, float rb) {
    *(float2 *)(e.qout + (size_t)t * e.qd + r0) = make_float2(ra, rb);
    if (e.qh) {
        const float ya = ra * e.qscale, yb = rb * e.qscale;
        h2 vh, vl;
        vh.x = (f16)ya;
        vh.y = (f16)yb;
        vl.x = (f16)(ya - (float)vh.x);
        vl.y = (f16)(yb - (float)vh.y);
        *(h2 *)(e.qh + (size_t)t * e.qd + r0) = vh;
        *(h2 *)(e.ql + (size_t)t * e.qd + r0) = vl;
    }
}

DEV void store_kv_pair(void *base, int kvtype, size_t idx, float a, float b) {
    if (kvtype == T_F16) {
        h2 v;
        v.x = (f16)a;
        v.y = (f16)b;
        *(h2 *)((uint16_t *)base + idx) = v;
    } else {
        *(float2 *)((float *)base + idx) = make_float2(a, b);
    }
}

// The pair (a, b) at row rr of the token's new K (which = 0) or V (1) row:
// into its cell of an f16 / f32 cache, or into the f32 staging rows that
// launch_kv_quant codes for a Q8_0 cache.
DEV void append_kv_pair(const EpiArgs &e, int which, int t, int seq, int pos, int rr, float a, float b) {
    if (e.kv.kvtype == T_Q8_0) {
        *(float2 *)(e.kv.stage + ((size_t)t * 2 + which) * e.kd + rr) = make_float2(a, b);
        return;
    }
    const int hd = e.kv.hd, g = rr / hd, el = rr % hd;
    const size_t idx = (((size_t)seq * e.kv.n_kv + g) * e.kv.n_ctx + pos) * hd + el;
    store_kv_pair(which ? e.kv.v : e.kv.k, e.kv.kvtype, idx, a, b);
}

// Applies epilogue EPI to the pair (r0, r1) = values (a, b) of token t.
// p is the pair index (the feature index for SWIGLU).
template <int EPI>
DEV void epi_pair(const EpiArgs &e, int t, int p, int r0, int r1, float a, float b) {
    switch (EPI) {
    case EPI_STORE: {
        float *y = e.y + (size_t)t * e.ldy;
        y[r0] = a;
        y[r1] = b;
        break;
    }
    case EPI_RESID: {
        float *y = e.y + (size_t)t * e.ldy;
        y[r0] += a;
        y[r1] += b;
        break;
    }
    case EPI_SWIGLU: {
        const float hv = silu(a) * b;
        const f16 hh = (f16)hv;
        ((f16 *)e.h)[(size_t)t * e.ldh + p] = hh;
        if (e.h_lo) ((f16 *)e.h_lo)[(size_t)t * e.ldh + p] = (f16)(hv - (float)hh);
        break;
    }
    case EPI_QKV: {
        const int hd = e.kv.hd;
        const int pos = e.tok.pos[t];
        if (r0 < e.qd + e.kd) {
            // RoPE: rotate the adjacent pair by pos * base^(-2i/hd)
            const int rr = r0 < e.qd ? r0 : r0 - e.qd;
            const int i = (rr % hd) >> 1;
            const float2 cs = *(const float2 *)(e.rope_cs + ((size_t)pos * (hd >> 1) + i) * 2);
            const float ra = a * cs.x - b * cs.y;
            const float rb = a * cs.y + b * cs.x;
            if (r0 < e.qd)
                store_q_pair(e, t, r0, ra, rb);
            else
                append_kv_pair(e, 0, t, e.tok.seq[t], pos, rr, ra, rb);
        } else {
            append_kv_pair(e, 1, t, e.tok.seq[t], pos, r0 - e.qd - e.kd, a, b);
        }
        break;
    }
    }
}

// Memory inputs of an epilogue, read ahead of the arithmetic so that a
// kernel can request them at entry: the old residual values (RESID) or the
// RoPE factors, position and sequence of the pair (QKV).
struct EpiPre {
    float y0 = 0.f, y1 = 0.f;
    float2 cs = make_float2(1.f, 0.f);
    int pos = 0, seq = 0;
};

template <int EPI>
DEV EpiPre epi_prefetch(const EpiArgs &e, int t, int r0, int r1) {
    EpiPre pre;
    if (EPI == EPI_RESID) {
        const float *y = e.y + (size_t)t * e.ldy;
        pre.y0 = y[r0];
        pre.y1 = y[r1];
    } else if (EPI == EPI_QKV) {
        const int hd = e.kv.hd;
        pre.pos = e.tok.pos[t];
        pre.seq = e.tok.seq[t];
        if (r0 < e.qd + e.kd) {
            const int rr = r0 < e.qd ? r0 : r0 - e.qd;
            pre.cs = *(const float2 *)(e.rope_cs + ((size_t)pre.pos * (hd >> 1) + ((rr % hd) >> 1)) * 2);
        }
    }
    return pre;
}

// epi_pair with the memory inputs taken from epi_prefetch (same results).
template <int EPI>
DEV void epi_pair_pre(const EpiArgs &e, int t, int p, int r0, int r1, float a, float b, const EpiPre &pre) {
    if (EPI == EPI_RESID) {
        float *y = e.y + (size_t)t * e.ldy;
        y[r0] = pre.y0 + a;
        y[r1] = pre.y1 + b;
    } else if (EPI == EPI_QKV) {
        if (r0 < e.qd + e.kd) {
            const int rr = r0 < e.qd ? r0 : r0 - e.qd;
            const float ra = a * pre.cs.x - b * pre.cs.y;
            const float rb = a * pre.cs.y + b * pre.cs.x;
            if (r0 < e.qd)
                store_q_pair(e, t, r0, ra, rb);
            else
                append_kv_pair(e, 0, t, pre.seq, pre.pos, rr, ra, rb);
        } else {
            append_kv_pair(e, 1, t, pre.seq, pre.pos, r0 - e.qd - e.kd, a, b);
        }
    } else {
        epi_pair<EPI>(e, t, p, r0, r1, a, b);
    }
}

