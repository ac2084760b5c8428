// sample.hip -- the sampler chain on the device (gfx950).
//
// The article's sampler list (step 15), in its order: repeat penalty on the
// recent history, top-k, top-p, min-p, temperature, then one token drawn
// from the softmax of the survivors.  One 1024-thread block samples one
// logits row:
//   1. the row (V <= 32768 floats) is copied to LDS; the penalty changes the
//      logits of the distinct tokens of the history window there;
//   2. top-k is an exact radix select over 48-bit keys
//      (monotone logit bits << 16 | 0xFFFF - id), so the k survivors are
//      unique even when logits tie (the lower id wins); digits of 8 bits from
//      the top, stopping as soon as every element matching the prefix is in;
//   3. the k keys are sorted (bitonic, in LDS) into chain order;
//   4. the weights exp(l - leader) and exp(l / T - leader / T) are computed in
//      parallel; one thread then runs top-p, min-p and the draw sequentially
//      in fp32 -- the same expressions, in the same order, as a plain
//      sequential implementation.
// The draw is u = top 24 bits of SplitMix64(seed, draw index) (Steele et al.
// 2014), so a run is reproducible from (seed, number of draws).
#include "common.h"
#include "kernels.h"

namespace {

constexpr int SV_MAX = 32768;     // logits a block holds in LDS
constexpr int SK_MAX = 1024;      // top-k bound (the sorted candidate list)
constexpr int SH_MAX = 64;        // history window bound

DEV uint64_t splitmix64(uint64_t seed, uint64_t index) {
    uint64_t z = seed + (index + 1) * 0x9E3779B97F4A7C15ull;
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
}

// Order-preserving map of a float to an unsigned integer.
DEV uint32_t mono(float f) {
    const uint32_t u = __float_as_uint(f);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
DEV uint64_t key48(float l, int id) { return ((uint64_t)mono(l) << 16) | (uint64_t)(0xFFFF - id); }

__global__ __launch_bounds__(1024) void k_sample(const float *logits, SampleArgs a) {
    __shared__ float lg[SV_MAX];
    __shared__ uint64_t ck[SK_MAX];
    __shared__ float w1[SK_MAX], w2[SK_MAX];
    __shared__ int hist[SH_MAX];
    __shared__ unsigned bins[256];
    __shared__ unsigned cnt, sel_digit, sel_rem, sel_done;
    const int tid = threadIdx.x, V = a.n_vocab;

    for (int i = tid; i < V; i += 1024) lg[i] = logits[i];
    if (tid < a.n_hist) hist[tid] = a.hist[tid];
    __syncthreads();

    // ---- 1. repeat penalty, once per distinct token of the window ----
    if (tid < a.n_hist && a.repeat_penalty != 1.0f) {
        const int t = hist[tid];
        bool first = t >= 0 && t < V;
        for (int j = 0; j < tid; j++) first = first && hist[j] != t;
        if (first) lg[t] = lg[t] > 0.0f ? lg[t] / a.repeat_penalty : lg[t] * a.repeat_penalty;
    }
    __syncthreads();

    // ---- 2. radix select of the k-th largest 48-bit key ----
    const int k = a.top_k;
    uint64_t prefix = 0;           // digits chosen so far (high bits)
    unsigned rem = (unsigned)k;    // survivors still to take inside the prefix
    int shift = 40;
    for (; shift >= 0; shift -= 8) {
        for (int b = tid; b < 256; b += 1024) bins[b] = 0;
        __syncthreads();
        const uint64_t hi_mask = shift == 40 ? 0 : (~0ull << (shift + 8)) & 0xFFFFFFFFFFFFull;
        for (int i = tid; i < V; i += 1024) {
            const uint64_t key = key48(lg[i], i);
            if ((key & hi_mask) == prefix) atomicAdd(&bins[(key >> shift) & 255], 1u);
        }
        __syncthreads();
        if (tid == 0) {
            // from the top digit down: the digit where the remaining count is reached
            unsigned acc = 0, d = 255;
            for (;; d--) {
                if (acc + bins[d] >= rem) break;
                acc += bins[d];
                if (d == 0) break;
            }
            sel_digit = d;
            sel_rem = rem - acc;                     // survivors to take inside digit d
            sel_done = bins[d] == sel_rem;           // all of digit d survive
        }
        __syncthreads();
        prefix |= (uint64_t)sel_digit << shift;
        rem = sel_rem;
        if (sel_done) break;
    }
    // survivors: keys above the prefix at this digit level, plus the prefix itself
    const int lvl = shift < 0 ? 0 : shift;
    const uint64_t cut_mask = (~0ull << lvl) & 0xFFFFFFFFFFFFull;
    if (tid == 0) cnt = 0;
    __syncthreads();
    for (int i = tid; i < V; i += 1024) {
        const uint64_t key = key48(lg[i], i);
        if ((key & cut_mask) >= prefix) {
            const unsigned slot = atomicAdd(&cnt, 1u);
            if (slot < (unsigned)SK_MAX) ck[slot] = key;
        }
    }
    __syncthreads();
    const int n = min((int)cnt, SK_MAX);           // == k: the keys are unique
    int np2 = 1;
    while (np2 < n) np2 <<= 1;
    for (int i = n + tid; i < np2; i += 1024) ck[i] = 0;   // padding sorts last

    // ---- 3. bitonic sort, descending ----
    for (int size = 2; size <= np2; size <<= 1)
        for (int stride = size >> 1; stride > 0; stride >>= 1) {
            __syncthreads();
            for (int i = tid; i < np2; i += 1024) {
                const int j = i ^ stride;
                if (j > i) {
                    const bool desc = (i & size) == 0;
                    const uint64_t x = ck[i], y = ck[j];
                    if (desc ? x < y : x > y) {
                        ck[i] = y;
                        ck[j] = x;
                    }
                }
            }
        }
    __syncthreads();

    // ---- 4. weights in parallel, the sequential chain on one thread ----
    const float m = lg[0xFFFF - (int)(ck[0] & 0xFFFF)];
    const float temp = a.temp;
    for (int i = tid; i < n; i += 1024) {
        const float l = lg[0xFFFF - (int)(ck[i] & 0xFFFF)];
        w1[i] = expf(l - m);
        w2[i] = temp > 0.0f ? expf(l / temp - m / temp) : 0.0f;
    }
    __syncthreads();
    if (tid == 0) {
        int nk = n;
        if (a.top_p < 1.0f) {
            float s = 0.0f;
            for (int i = 0; i < nk; i++) s += w1[i];
            const float lim = a.top_p * s;
            float acc = 0.0f;
            int keep = nk;
            for (int i = 0; i < nk; i++) {
                acc += w1[i];
                if (acc >= lim) {
                    keep = i + 1;
                    break;
                }
            }
            nk = keep;
        }
        if (a.min_p > 0.0f) {
            int keep = 1;
            for (int i = 1; i < nk; i++)
                if (w1[i] >= a.min_p) keep = i + 1;
            nk = keep;
        }
        int pick = 0;
        if (temp > 0.0f) {
            float s = 0.0f;
            for (int i = 0; i < nk; i++) s += w2[i];
            const float u = (float)(splitmix64(a.seed, a.draw) >> 40) * (1.0f / 16777216.0f);
            const float t = u * s;
            float acc = 0.0f;
            pick = nk - 1;
            for (int i = 0; i < nk; i++) {
                acc += w2[i];
                if (acc > t) {
                    pick = i;
                    break;
                }
            }
        }
        a.out[0] = 0xFFFF - (int)(ck[pick] & 0xFFFF);
    }
}

}  // namespace

bool launch_sample(const float *logits, const SampleArgs &a, hipStream_t s) {
    if (a.n_vocab <= 0 || a.n_vocab > SV_MAX || a.top_k < 1 || a.top_k > SK_MAX || a.top_k > a.n_vocab ||
        a.n_hist < 0 || a.n_hist > SH_MAX)
        return false;
    launch(k_sample, dim3(1), dim3(1024), 0, s, logits, a);
    return true;
}
