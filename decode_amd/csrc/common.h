// common.h -- device helpers shared by the gfx950 kernels of libdecode.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

typedef _Float16 f16;
typedef _Float16 h2 __attribute__((ext_vector_type(2)));
typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef float f4 __attribute__((ext_vector_type(4)));
typedef float f16x __attribute__((ext_vector_type(16)));

#define DEV static __device__ __forceinline__

// Global address space: pointers read from memory (not kernel arguments) are
// generic to the compiler, and generic (flat) accesses need a 64-bit address
// register each; casting them makes every access a global one with a scalar base.
#ifdef __HIP_DEVICE_COMPILE__
#define GLB __attribute__((address_space(1)))
#else
#define GLB
#endif
template <class T>
DEV GLB T *gl(T *p) { return (GLB T *)p; }

// Element type codes (same values as dec_type in include/decode.h).
enum { T_F32 = 0, T_F16 = 1, T_Q8_0 = 2, T_Q4_0 = 3, T_Q4_K = 4 };

DEV h2 as_h2(uint32_t u) { return __builtin_bit_cast(h2, u); }
DEV uint32_t h2_bits(h2 v) { return __builtin_bit_cast(uint32_t, v); }
DEV float f16_bits_to_f32(uint16_t b) { return (float)__builtin_bit_cast(f16, b); }
DEV uint16_t f32_to_f16_bits(float x) { return __builtin_bit_cast(uint16_t, (f16)x); }

// a.x*b.x + a.y*b.y + c with fp32 accumulation (v_dot2_f32_f16)
DEV float dot2(h2 a, h2 b, float c) { return __builtin_amdgcn_fdot2(a, b, c, false); }

// Butterfly sum over the 64 lanes of a wavefront; every lane gets the total.
DEV float wave_sum(float v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
    return v;
}
DEV float wave_max(float v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
    return v;
}

// Sum over a 256-thread block; `red` is 4 floats of shared memory.  All
// threads get the total.  Contains __syncthreads.
DEV float block_sum256(float v, float *red) {
    v = wave_sum(v);
    const int w = threadIdx.x >> 6;
    if ((threadIdx.x & 63) == 0) red[w] = v;
    __syncthreads();
    const float t = (red[0] + red[1]) + (red[2] + red[3]);
    __syncthreads();
    return t;
}

DEV float silu(float u) { return u / (1.0f + __expf(-u)); }

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
// 16-byte streaming load (non-temporal: weights are read once per step)
DEV uint4 load_stream16(const uint4 *p) {
    const u32x4 v = __builtin_nontemporal_load((const u32x4 *)p);
    return make_uint4(v.x, v.y, v.z, v.w);
}

// DPP lane exchange (v_mov_dpp) of a float.
template <int CTRL>
DEV float dpp_f(float v) {
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xF, 0xF, false));
}
// Sum over each 16-lane row; every lane of the row gets the row's total.
// quad_perm [1,0,3,2], quad_perm [2,3,0,1], row_ror:4, row_ror:8.
DEV float row16_sum(float v) {
    v += dpp_f<0xB1>(v);
    v += dpp_f<0x4E>(v);
    v += dpp_f<0x124>(v);
    v += dpp_f<0x128>(v);
    return v;
}
DEV float row16_max(float v) {
    v = fmaxf(v, dpp_f<0xB1>(v));
    v = fmaxf(v, dpp_f<0x4E>(v));
    v = fmaxf(v, dpp_f<0x124>(v));
    v = fmaxf(v, dpp_f<0x128>(v));
    return v;
}
DEV float readlane_f(float v, int lane) {
    return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), lane));
}
// Sum over the 64 lanes without LDS traffic; the (wave-uniform) total is returned.
DEV float wave_sum_dpp(float v) {
    v = row16_sum(v);
    return (readlane_f(v, 0) + readlane_f(v, 16)) + (readlane_f(v, 32) + readlane_f(v, 48));
}
