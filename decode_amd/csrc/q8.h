// q8.h -- the Q8_0 block coding shared by the weight quantizer and the KV
// cache writers: d = max|x| / 127 (fp32), codes = round-half-away(x * (1/d)),
// the scale stored as f16 (round to nearest even); fp32 arithmetic with no
// contraction, so the codes match any IEEE fp32 implementation of these steps.
#pragma once

#include "common.h"
#include "kernels.h"

// Q8_0 coding of 32 values: the scale's f16 bits and the 32 codes packed
// little-endian into 8 dwords.
DEV uint16_t q8_block(const float *v, uint32_t *packed) {
#pragma clang fp contract(off)
    float amax = 0.f;
#pragma unroll
    for (int j = 0; j < 32; j++) amax = fmaxf(amax, fabsf(v[j]));
    float d = amax / 127.0f;
    // keep the f16 rounding a separate step: a fused multiply-add form of
    // the conversion would turn a -0 scale into +0
    asm volatile("" : "+v"(d));
    const float id = d != 0.f ? 1.0f / d : 0.f;
#pragma unroll
    for (int i = 0; i < 8; i++) {
        uint32_t w = 0;
#pragma unroll
        for (int e = 0; e < 4; e++) {
            const int q = (int)roundf(v[4 * i + e] * id);
            w |= ((uint32_t)(q & 0xff)) << (8 * e);
        }
        packed[i] = w;
    }
    return f32_to_f16_bits(d);
}


// Q8_0 KV cache: codes block b (of n_kv*hd/32) of token t's staged K
// (which = 0) or V (1) row into the cell (seq, pos); block b belongs to KV
// head b / (hd/32).
DEV void kv_code_block(const KVLayer &kv, int t, int which, int b, int seq, int pos) {
    const int hd = kv.hd, bph = hd >> 5, kd = kv.n_kv * hd;
    const float *x = kv.stage + ((size_t)t * 2 + which) * kd + (size_t)b * 32;
    float v[32];
#pragma unroll
    for (int j = 0; j < 32; j += 4) {
        const float4 f = *(const float4 *)(x + j);
        v[j] = f.x; v[j + 1] = f.y; v[j + 2] = f.z; v[j + 3] = f.w;
    }
    uint32_t packed[8];
    const uint16_t dbits = q8_block(v, packed);
    const int g = b / bph, bl = b % bph;
    const size_t cell = ((size_t)seq * kv.n_kv + g) * kv.n_ctx + pos;
    (which ? kv.v_scale : kv.k_scale)[cell * bph + bl] = dbits;
    uint4 *dst = (uint4 *)((int8_t *)(which ? kv.v : kv.k) + cell * hd + bl * 32);
    dst[0] = make_uint4(packed[0], packed[1], packed[2], packed[3]);
    dst[1] = make_uint4(packed[4], packed[5], packed[6], packed[7]);
}
