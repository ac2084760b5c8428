// sample.hip -- the sampler chain on the device (gfx950).
//
// The article's sampler list (step 15), in its order: repeat penalty on the
// recent history, top-k, top-p, min-p, temperature, then one token drawn
// from the softmax of the survivors.  One 1024-thread block samples one
// logits row (V <= 32768):
//   1. each thread holds 32 logits of the row in registers (ids
//      4 * (tid + 1024 j) + c); the penalty is applied there, once per
//      distinct token of the window (an LDS bitmap marks them);
//   2. top-k candidates.  Tokens are ordered by the 48-bit key
//      (monotone logit bits << 16 | 0xFFFF - id): larger logit first, the
//      lower id first among equal logits.  Fast path: with M the row's
//      largest logit, the tokens are counted per octave of M - l (per-thread
//      packed counters, no atomics); every token of an octave nearer to M
//      ranks above every token of a farther one, so the tokens up to the
//      octave where the count reaches k hold the top k; that octave is split
//      again by the top 4 mantissa bits of M - l.  They are compacted
//      (at most 2048).  Otherwise (non-finite logits, or too many tokens in
//      that octave) an exact radix select over the keys (8-bit digits from
//      the top) leaves exactly k;
//   3. the candidates are sorted: 64-key bitonic runs inside each wavefront,
//      then each key's rank is the number of larger keys over all runs
//      (a binary search per run); the first k ranks are the chain's
//      candidates, in order;
//   4. the weights exp(l - leader) and exp(l / T - leader / T) are computed in
//      parallel; one lane forms their running sums in candidate order (the
//      fp32 additions of a plain sequential loop, in that loop's order), and
//      top-p, min-p and the draw are then decided by all threads at once from
//      those sums.
// The draw is u = top 24 bits of SplitMix64(seed, draw index) (Steele et al.
// 2014), so a run is reproducible from (seed, number of draws).
#include "../../include/decode.h"
#include "common.h"
#include "kernels.h"

#include <mutex>

namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int SV_MAX = 32768;     // logits a block holds (32 per thread)
constexpr int SK_MAX = 1024;      // top-k bound
constexpr int SC_MAX = 2048;      // candidates sorted (32 runs of 64)
constexpr int SH_MAX = 64;        // history window bound
constexpr int NG = SV_MAX / 4096; // groups of 4 logits per thread
constexpr int OCT_LO = 117;       // octave 0: M - l < 2^(OCT_LO + 1 - 127)

DEV uint64_t splitmix64(uint64_t seed, uint64_t index) {
    uint64_t z = seed + (index + 1) * 0x9E3779B97F4A7C15ull;
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
}

// Order-preserving map of a float to an unsigned integer, and its inverse.
DEV uint32_t mono(float f) {
    const uint32_t u = __float_as_uint(f);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
DEV float unmono(uint32_t m) { return __uint_as_float((m & 0x80000000u) ? (m & 0x7FFFFFFFu) : ~m); }
DEV uint64_t key48(uint32_t mo, int id) { return ((uint64_t)mo << 16) | (uint64_t)(0xFFFF - id); }
DEV float key_logit(uint64_t key) { return unmono((uint32_t)(key >> 16)); }
DEV int key_id(uint64_t key) { return 0xFFFF - (int)(key & 0xFFFF); }

// A copy of v the compiler cannot see through: each pass over the row
// recomputes M - l instead of keeping 32 differences live across passes.
DEV float opaque(float v) {
    asm volatile("" : "+v"(v));
    return v;
}

// octave of d = M - l >= 0, clamped to 0..15
DEV int octave(float d) { return min(max((int)(__float_as_uint(d) >> 23) - OCT_LO, 0), 15); }

template <int CTRL>
DEV uint32_t dpp_u(uint32_t v) {
    return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, 0xF, 0xF, false);
}
// Sum over the 64 lanes (wave-uniform result), without LDS traffic.
DEV uint32_t wave_sum_u32(uint32_t v) {
    v += dpp_u<0xB1>(v);
    v += dpp_u<0x4E>(v);
    v += dpp_u<0x124>(v);
    v += dpp_u<0x128>(v);
    return ((uint32_t)__builtin_amdgcn_readlane((int)v, 0) + (uint32_t)__builtin_amdgcn_readlane((int)v, 16)) +
           ((uint32_t)__builtin_amdgcn_readlane((int)v, 32) + (uint32_t)__builtin_amdgcn_readlane((int)v, 48));
}

DEV uint64_t shfl_xor64(uint64_t v, int m) {
    const uint32_t lo = (uint32_t)__shfl_xor((int)(uint32_t)v, m, 64);
    const uint32_t hi = (uint32_t)__shfl_xor((int)(uint32_t)(v >> 32), m, 64);
    return ((uint64_t)hi << 32) | lo;
}
// Bitonic sort of one key per lane across the wavefront, largest at lane 0.
DEV uint64_t wave_sort_desc(uint64_t x, int lane) {
#pragma unroll
    for (int size = 2; size <= 64; size <<= 1)
#pragma unroll
        for (int stride = size >> 1; stride > 0; stride >>= 1) {
            const uint64_t y = shfl_xor64(x, stride);
            const bool take_max = ((lane & size) == 0) == ((lane & stride) == 0);
            x = take_max ? (x > y ? x : y) : (x < y ? x : y);
        }
    return x;
}

__global__ __launch_bounds__(1024) void k_sample(const float *logits, SampleArgs a) {
    __shared__ uint64_t cand[SC_MAX];      // candidates (then sorted runs)
    __shared__ uint64_t cs[SK_MAX];        // the top k, in chain order
    __shared__ float w1[SK_MAX], c1[SK_MAX], c2[SK_MAX];
    __shared__ uint32_t pen[SV_MAX / 32];  // penalised tokens
    __shared__ unsigned bins[2][256];
    __shared__ uint32_t oct_w[16][8];      // per-wave octave counts, 16-bit pairs
    __shared__ float max_w[16];
    __shared__ unsigned cnt, sel_digit, sel_rem, sel_done;
    __shared__ unsigned subc[16];          // tokens per 1/16 of the cut octave
    __shared__ int keep_min_p, oct_cut, n_cand, n_below, sub_cut, bad_w;
    const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6, V = a.n_vocab;
    const bool use_pen = a.n_hist > 0 && a.repeat_penalty != 1.0f;
    const int k = a.top_k;

    // ---- 1. the row into registers (every load in flight at once) ----
    const int ht = tid < a.n_hist ? a.hist[tid] : -1;
    f32x4 x[NG];
    if ((((uintptr_t)logits) & 15) == 0 && (V & 3) == 0) {
        const int V4 = V >> 2;
        const f32x4 *src = (const f32x4 *)logits;
#pragma unroll
        for (int j = 0; j < NG; j++) x[j] = src[min(tid + j * 1024, V4 - 1)];
    } else {
#pragma unroll
        for (int j = 0; j < NG; j++)
#pragma unroll
            for (int c = 0; c < 4; c++) x[j][c] = logits[min(4 * (tid + j * 1024) + c, V - 1)];
    }
    // slots past the row hold -inf: they rank below every token of the row
    // (the lower id wins among equal logits), so the fast path needs no bounds
    // tests; the exact path tests ids explicitly
    if (V < SV_MAX) {
#pragma unroll
        for (int j = 0; j < NG; j++)
#pragma unroll
            for (int c = 0; c < 4; c++)
                if (4 * (tid + j * 1024) + c >= V) x[j][c] = -INFINITY;
    }
    pen[tid] = 0;
    bins[0][tid & 255] = 0;
    if (tid < 16) subc[tid] = 0;
    if (tid == 0) {
        keep_min_p = 1;
        cnt = 0;
        bad_w = 0;
    }
    __syncthreads();
    if (use_pen && ht >= 0 && ht < V) atomicOr(&pen[ht >> 5], 1u << (ht & 31));
    __syncthreads();
    float mx = -INFINITY;
    bool bad = false;
#pragma unroll
    for (int j = 0; j < NG; j++) {
        const int id0 = 4 * (tid + j * 1024);
        const uint32_t pw = use_pen ? pen[id0 >> 5] >> (id0 & 31) : 0u;
#pragma unroll
        for (int c = 0; c < 4; c++) {
            float l = x[j][c];
            if ((pw >> c) & 1u) l = l > 0.0f ? l / a.repeat_penalty : l * a.repeat_penalty;
            x[j][c] = l;
            mx = fmaxf(mx, l);
            bad |= !(l == l);
        }
    }

    // ---- 2. top-k candidates ----
    // the row maximum (and whether any logit is NaN)
    mx = row16_max(mx);
    mx = fmaxf(fmaxf(readlane_f(mx, 0), readlane_f(mx, 16)), fmaxf(readlane_f(mx, 32), readlane_f(mx, 48)));
    if (__ballot(bad)) bad_w = 1;
    if (lane == 0) max_w[wid] = mx;
    __syncthreads();
    float M = max_w[0];
#pragma unroll
    for (int w = 1; w < 16; w++) M = fmaxf(M, max_w[w]);
    const bool fast_ok = !bad_w && M > -INFINITY && M < INFINITY;

    if (fast_ok) {
        // tokens per octave of M - l: 8-bit counters packed in two u64
        const float M1 = opaque(M);
        uint64_t lo = 0, hi = 0;
#pragma unroll
        for (int j = 0; j < NG; j++)
#pragma unroll
            for (int c = 0; c < 4; c++) {
                const int o = octave(M1 - x[j][c]);
                const uint64_t inc = 1ull << ((o & 7) * 8);
                if (o < 8) lo += inc;
                else hi += inc;
            }
        // 16 counts as 16-bit fields of 8 words, summed over the wavefront
#pragma unroll
        for (int q = 0; q < 8; q++) {
            const uint64_t src = q < 4 ? lo : hi;
            const int sh = (q & 3) * 16;
            const uint32_t v = (uint32_t)((src >> sh) & 0xFF) | ((uint32_t)((src >> (sh + 8)) & 0xFF) << 16);
            const uint32_t t = wave_sum_u32(v);
            if (lane == 0) oct_w[wid][q] = t;
        }
        __syncthreads();
        if (tid < 64) {
            // lane o < 16 totals octave o, then the first octave where the
            // running count reaches k
            uint32_t tot = 0;
            if (lane < 16)
                for (int w = 0; w < 16; w++) tot += (oct_w[w][lane >> 1] >> ((lane & 1) * 16)) & 0xFFFF;
            uint32_t incl = tot;
#pragma unroll
            for (int o = 1; o < 16; o <<= 1) {
                const uint32_t u = __shfl_up(incl, o, 64);
                if (lane >= o) incl += u;
            }
            const uint64_t reach = __ballot(lane < 16 && incl >= (uint32_t)k);
            const int cut = __ffsll((unsigned long long)reach) - 1;
            const uint32_t nc = (uint32_t)__builtin_amdgcn_readlane((int)incl, cut);
            const uint32_t below = (uint32_t)__builtin_amdgcn_readlane((int)(incl - tot), cut);
            if (lane == 0) {
                oct_cut = cut;
                n_cand = (int)nc;
                n_below = (int)below;
                sub_cut = 15;
            }
        }
        __syncthreads();
        // Within one exponent the top 4 mantissa bits of M - l order the tokens
        // too: refine an unclamped cut octave into 16 parts.
        const int cut = oct_cut;
        if (cut > 0 && cut < 15) {
            const float M2 = opaque(M);
#pragma unroll
            for (int j = 0; j < NG; j++)
#pragma unroll
                for (int c = 0; c < 4; c++) {
                    const float d = M2 - x[j][c];
                    if (octave(d) == cut)
                        atomicAdd(&subc[(__float_as_uint(d) >> 19) & 15], 1u);
                }
            __syncthreads();
            if (tid < 64) {
                const uint32_t tot = lane < 16 ? subc[lane] : 0u;
                uint32_t incl = tot;
#pragma unroll
                for (int o = 1; o < 16; o <<= 1) {
                    const uint32_t u = __shfl_up(incl, o, 64);
                    if (lane >= o) incl += u;
                }
                const uint32_t need = (uint32_t)(k - n_below);
                const uint64_t reach = __ballot(lane < 16 && incl >= need);
                const int sc = __ffsll((unsigned long long)reach) - 1;
                if (lane == 0) {
                    sub_cut = sc;
                    n_cand = n_below + (int)__builtin_amdgcn_readlane((int)incl, sc);
                }
            }
            __syncthreads();
        }
    }
    const bool fast = fast_ok && n_cand <= SC_MAX;
    int nc;
    if (fast) {
        // compact the tokens of octaves below the cut and of the cut octave's
        // parts up to sub_cut
        const int cut = oct_cut, scut = sub_cut;
        const float M3 = opaque(M);
#pragma unroll
        for (int j = 0; j < NG; j++)
#pragma unroll
            for (int c = 0; c < 4; c++) {
                const int id = 4 * (tid + j * 1024) + c;
                const float d = M3 - x[j][c];
                const int o = octave(d);
                const bool in = o < cut || (o == cut && (int)((__float_as_uint(d) >> 19) & 15) <= scut);
                const uint64_t m = __ballot(in);
                if (m) {
                    const int leader = __ffsll((unsigned long long)m) - 1;
                    unsigned off = 0;
                    if (lane == leader) off = atomicAdd(&cnt, (unsigned)__popcll(m));
                    off = __builtin_amdgcn_readlane(off, leader);
                    const unsigned slot = off + (unsigned)__popcll(m & ((1ull << lane) - 1));
                    if (in && slot < (unsigned)SC_MAX) cand[slot] = key48(mono(x[j][c]), id);
                }
            }
        nc = n_cand;
    } else {
        // exact radix select of the k-th largest key: each level counts, among
        // the keys matching the digits chosen so far, the keys per 8-bit digit
        // at bit `shift`; wave 0 picks the digit holding the rem-th largest.
        // bins alternate so that clearing the next level's needs no barrier.
        uint64_t prefix = 0;
        unsigned rem = (unsigned)k;
        int shift = 40, lvl = 0;
        for (;; lvl ^= 1) {
            unsigned *b = bins[lvl];
            const uint64_t hi_mask = shift == 40 ? 0 : (~0ull << (shift + 8)) & 0xFFFFFFFFFFFFull;
#pragma unroll
            for (int j = 0; j < NG; j++)
#pragma unroll
                for (int c = 0; c < 4; c++) {
                    const int id = 4 * (tid + j * 1024) + c;
                    const uint64_t key = key48(mono(x[j][c]), id);
                    if (id < V && (key & hi_mask) == prefix) atomicAdd(&b[(key >> shift) & 255], 1u);
                }
            bins[lvl ^ 1][tid & 255] = 0;
            __syncthreads();
            if (tid < 64) {
                // lane l holds digits 255-4l .. 252-4l; inclusive count from the top
                unsigned v[4], tot = 0;
#pragma unroll
                for (int j = 0; j < 4; j++) {
                    v[j] = b[255 - 4 * lane - j];
                    tot += v[j];
                }
                unsigned incl = tot;
#pragma unroll
                for (int o = 1; o < 64; o <<= 1) {
                    const unsigned u = __shfl_up(incl, o, 64);
                    if (lane >= o) incl += u;
                }
                unsigned acc = incl - tot;
                if (acc < rem && rem <= incl) {
#pragma unroll
                    for (int j = 0; j < 4; j++) {
                        if (acc + v[j] >= rem) {
                            sel_digit = 255 - 4 * lane - j;
                            sel_rem = rem - acc;
                            sel_done = v[j] == rem - acc;
                            break;
                        }
                        acc += v[j];
                    }
                }
            }
            __syncthreads();
            prefix |= (uint64_t)sel_digit << shift;
            rem = sel_rem;
            if (sel_done || shift == 0) break;
            shift -= 8;
        }
        // survivors: keys above the prefix at this digit level, plus the prefix itself
        const uint64_t cut_mask = (~0ull << shift) & 0xFFFFFFFFFFFFull;
#pragma unroll
        for (int j = 0; j < NG; j++)
#pragma unroll
            for (int c = 0; c < 4; c++) {
                const int id = 4 * (tid + j * 1024) + c;
                const uint64_t key = key48(mono(x[j][c]), id);
                const bool in = id < V && (key & cut_mask) >= prefix;
                const uint64_t m = __ballot(in);
                if (m) {
                    const int leader = __ffsll((unsigned long long)m) - 1;
                    unsigned off = 0;
                    if (lane == leader) off = atomicAdd(&cnt, (unsigned)__popcll(m));
                    off = __builtin_amdgcn_readlane(off, leader);
                    const unsigned slot = off + (unsigned)__popcll(m & ((1ull << lane) - 1));
                    if (in && slot < (unsigned)SC_MAX) cand[slot] = key;
                }
            }
        nc = k;                                    // the keys are unique
    }
    __syncthreads();

    // ---- 3. sort the candidates; the first k ranks are the chain's list ----
    const int runs = (nc + 63) >> 6;
    for (int r = wid; r < runs; r += 16) {
        const int i = r * 64 + lane;
        const uint64_t v = wave_sort_desc(i < nc ? cand[i] : 0ull, lane);
        cand[i] = v;                               // padding (0) sorts last
    }
    __syncthreads();
    for (int i = tid; i < nc; i += 1024) {
        // rank = the number of larger keys, summed over all runs (its own
        // run included), four independent binary searches at a time
        const uint64_t v = cand[i];
        int rank = 0;
        for (int r2 = 0; r2 < runs; r2 += 4) {
            int pos[4] = {0, 0, 0, 0};
#pragma unroll
            for (int step = 32; step > 0; step >>= 1)
#pragma unroll
                for (int u = 0; u < 4; u++)
                    if (r2 + u < runs && cand[(r2 + u) * 64 + pos[u] + step - 1] > v) pos[u] += step;
#pragma unroll
            for (int u = 0; u < 4; u++)
                if (r2 + u < runs) rank += pos[u] + (pos[u] == 63 && cand[(r2 + u) * 64 + 63] > v ? 1 : 0);
        }
        if (rank < k) cs[rank] = v;
    }
    __syncthreads();
    const int n = k;

    // ---- 4. weights, their running sums, then the cuts and the draw ----
    const float m = key_logit(cs[0]);
    const float temp = a.temp;
    {
        float x1 = 0.0f, y = 0.0f;
        if (tid < n) {
            const float l = key_logit(cs[tid]);
            x1 = expf(l - m);
            y = temp > 0.0f ? expf(l / temp - m / temp) : 0.0f;
        }
        w1[tid] = x1;
        c1[tid] = x1;
        c2[tid] = y;
    }
    __syncthreads();
    // Inclusive running sums in candidate order, one lane, 16 at a time: the
    // fp32 additions happen in the same order as a plain sequential loop.
    if (tid == 0) {
        float s1 = 0.0f, s2 = 0.0f;
        for (int i = 0; i < n; i += 16) {
            f32x4 p[4], q[4];
#pragma unroll
            for (int g = 0; g < 4; g++) {
                p[g] = *(const f32x4 *)&c1[i + 4 * g];
                q[g] = *(const f32x4 *)&c2[i + 4 * g];
            }
#pragma unroll
            for (int g = 0; g < 4; g++)
#pragma unroll
                for (int c = 0; c < 4; c++) {
                    s1 += p[g][c];
                    p[g][c] = s1;
                    s2 += q[g][c];
                    q[g][c] = s2;
                }
#pragma unroll
            for (int g = 0; g < 4; g++) {
                *(f32x4 *)&c1[i + 4 * g] = p[g];
                *(f32x4 *)&c2[i + 4 * g] = q[g];
            }
        }
    }
    __syncthreads();
    // top-p: the shortest prefix whose running sum reaches top_p of the total.
    // Running sums of non-negative terms never decrease, so the cut is one
    // plus the number of sums still below the limit.
    int nk = n;
    if (a.top_p < 1.0f) {
        const float lim = a.top_p * c1[n - 1];
        const int below = __syncthreads_count(tid < n && c1[tid] < lim);
        nk = min(n, below + 1);
    }
    // min-p: keep up to the last candidate whose weight relative to the leader
    // reaches min_p
    if (a.min_p > 0.0f) {
        if (tid >= 1 && tid < nk && w1[tid] >= a.min_p) atomicMax(&keep_min_p, tid + 1);
        __syncthreads();
        nk = keep_min_p;
    }
    int pick = 0;
    if (temp > 0.0f) {
        // the first candidate whose running sum exceeds u times the total
        const float u = (float)(splitmix64(a.seed, a.draw) >> 40) * (1.0f / 16777216.0f);
        const float t = u * c2[nk - 1];
        const int not_above = __syncthreads_count(tid < nk && c2[tid] <= t);
        pick = min(not_above, nk - 1);
    }
    if (tid == 0) a.out[0] = key_id(cs[pick]);
}

}  // namespace

bool launch_sample(const float *logits, const SampleArgs &a, hipStream_t s) {
    if (a.n_vocab <= 0 || a.n_vocab > SV_MAX || a.top_k < 1 || a.top_k > SK_MAX || a.top_k > a.n_vocab ||
        a.n_hist < 0 || a.n_hist > SH_MAX)
        return false;
    launch(k_sample, dim3(1), dim3(1024), 0, s, logits, a);
    return true;
}

// ---- the sampler chain without allocation (dec_sample_row_noalloc) -----------
// Device memory the call needs beyond its inputs and outputs -- the penalty
// window, and the device copy of a logits row given in host memory -- lives
// in one file-scope array, so the call allocates nothing.  Each GPU the
// library runs on holds its own copy until the process ends; host code reaches
// it only through the address hipGetSymbolAddress returns for the current
// device (the array's name is a host-side stand-in, not a device address).
namespace {
constexpr size_t NA_HIST_BYTES = (size_t)SH_MAX * 4;                 // window, int32
constexpr size_t NA_SCRATCH_BYTES = NA_HIST_BYTES + (size_t)SV_MAX * 4;   // + one logits row
static_assert(NA_HIST_BYTES % 256 == 0, "the row starts 256-byte aligned");
static_assert(SV_MAX == DEC_NOALLOC_MAX_VOCAB, "public limit of the no-allocation sampler");

}  // namespace

static __device__ __align__(256) uint8_t scratch[NA_SCRATCH_BYTES];

namespace {
constexpr int NA_MAX_DEV = 64;
std::mutex g_na_mu;
uint8_t *g_na_ptr[NA_MAX_DEV] = {};

// The scratch array's device address on the current device (looked up once
// per device, with that device current), or null.
uint8_t *na_scratch() {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= NA_MAX_DEV) {
        (void)hipGetLastError();
        return nullptr;
    }
    std::lock_guard<std::mutex> lk(g_na_mu);
    if (!g_na_ptr[dev]) {
        void *p = nullptr;
        const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !p) {
            (void)hipGetLastError();
            log_message(3, "dec_sample_row_noalloc: hipGetSymbolAddress failed on device %d: %s", dev,
                        hipGetErrorString(e));
            return nullptr;
        }
        g_na_ptr[dev] = (uint8_t *)p;
    }
    return g_na_ptr[dev];
}

// Device-visible address of p (device memory, or pinned host memory mapped
// into the device's address space), or null when the device cannot use it.
const void *na_device_view(const void *p, bool *is_host) {
    hipPointerAttribute_t at;
    *is_host = true;
    if (hipPointerGetAttributes(&at, p) != hipSuccess) {
        (void)hipGetLastError();
        return nullptr;
    }
    if (at.type == hipMemoryTypeDevice) {
        *is_host = false;
        return p;
    }
    return at.devicePointer;
}
}  // namespace


extern "C" int32_t dec_sample_row_noalloc(const dec_sampler_params *p, const int32_t *hist, int32_t n_hist,
                                          uint64_t draw, const float *logits, int32_t n_vocab,
                                          int32_t *token_out, void *hip_stream) {
    if (!p || p->top_k < 1 || p->top_k > SK_MAX || !(p->top_p > 0.0f && p->top_p <= 1.0f) ||
        !(p->min_p >= 0.0f && p->min_p < 1.0f) || !(p->repeat_penalty >= 1.0f) || p->penalty_last_n < 0 ||
        p->penalty_last_n > SH_MAX || p->temp != p->temp)
        return -1;
    if (!logits || !token_out || n_vocab < p->top_k || n_hist < 0 || n_hist > SH_MAX || (n_hist > 0 && !hist))
        return -1;
    if (n_vocab > SV_MAX) {
        log_message(3, "dec_sample_row_noalloc: n_vocab %d above the %d logits its static buffer holds", n_vocab,
                    SV_MAX);
        return -4;
    }
    bool out_host = false, row_host = false;
    int32_t *out = (int32_t *)na_device_view(token_out, &out_host);
    if (!out) {
        log_message(3, "dec_sample_row_noalloc: token_out is neither device memory nor mapped host memory");
        return -1;
    }
    (void)na_device_view(logits, &row_host);
    uint8_t *sc = na_scratch();
    if (!sc) return -3;
    hipStream_t st = (hipStream_t)hip_stream;
    SampleArgs a;
    const int w = n_hist < p->penalty_last_n ? n_hist : p->penalty_last_n;
    a.n_hist = p->repeat_penalty != 1.0f ? w : 0;
    a.n_vocab = n_vocab;
    a.top_k = p->top_k;
    a.top_p = p->top_p;
    a.min_p = p->min_p;
    a.temp = p->temp;
    a.repeat_penalty = p->repeat_penalty;
    a.seed = p->seed;
    a.draw = draw;
    a.hist = (const int32_t *)sc;
    a.out = out;
    if (a.n_hist > 0 && hipMemcpyAsync(sc, hist + (n_hist - a.n_hist), (size_t)a.n_hist * 4, hipMemcpyDefault,
                                       st) != hipSuccess) {
        (void)hipGetLastError();
        return -3;
    }
    const float *row = logits;
    if (row_host) {
        if (hipMemcpyAsync(sc + NA_HIST_BYTES, logits, (size_t)n_vocab * 4, hipMemcpyHostToDevice, st) != hipSuccess) {
            (void)hipGetLastError();
            return -3;
        }
        row = (const float *)(sc + NA_HIST_BYTES);
    }
    if (!launch_sample(row, a, st)) return -1;
    if (hipGetLastError() != hipSuccess) return -3;
    return 0;
}
