// kernels.h -- argument structs and host launchers of the libdecode kernels.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

// Timing of one selected launch.  While `armed`, launch() hands the events to
// hipExtLaunchKernel, which stamps them with the kernel's own start and end:
// the first launch takes e0 as its start event, every launch records e1 at
// its end, so e0..e1 spans the kernels of one probed unit (no event packets
// of their own in the interval).
struct LaunchProbe {
    hipEvent_t e0 = nullptr, e1 = nullptr;
    bool armed = false;
};
extern thread_local LaunchProbe g_launch_probe;

template <typename F, typename... Args>
inline void launch(F kernel, dim3 grid, dim3 block, uint32_t shm, hipStream_t s, Args... args) {
    LaunchProbe &p = g_launch_probe;
    if (p.armed) {
        hipExtLaunchKernelGGL(kernel, grid, block, shm, s, p.e0, p.e1, 0, args...);
        p.e0 = nullptr;
    } else {
        hipLaunchKernelGGL(kernel, grid, block, shm, s, args...);
    }
}

// One stored (possibly fused) weight matrix [N][K], row-major.
//   F32 : qs = float[N][K]
//   Q8_0: qs = int8 codes [N][K],           d = f16 scales [N][K/32]
//   Q4_0: qs = packed nibbles [N][K/2]      d = f16 scales [N][K/32]
//         (16 bytes per 32-weight block, byte k = code k | code k+16 << 4)
//   Q4_K: qs = packed nibbles [N][K/2] in the Q4_0 layout (codes 0..15 of
//         each 32-weight sub-block), d = sub-block scale | min << 8 [N][K/32]
//         (six-bit integers), dm = f16 d | f16 dmin << 16 [N][K/256]
//         (super-block factors): weight = f(d) * sc * q - f(dmin) * m;
//         mfq = -f(dmin) * m per sub-block as f16 value | remainder << 16
//         ([K/256][N][8]: the 8 sub-blocks of a super-block contiguous) and
//         sf = f(d) * sc per sub-block in fp32 (exact, [K/32][N]), derived at
//         load: the GEMM's min-term operand and block scale
//   Q4_0/Q8_0 matrices a GEMM reads also hold dt = d transposed ([K/32][N],
//   derived at load): the scales of one K block of consecutive rows are then
//   one contiguous run, which the direct-to-LDS GEMM loads with a few wide
//   requests instead of one 2-byte request per row.
struct QMat {
    int wtype = 0;
    int N = 0, K = 0;
    void *qs = nullptr;
    uint16_t *d = nullptr;
    uint16_t *dt = nullptr;
    uint32_t *dm = nullptr;
    uint32_t *mfq = nullptr;
    float *sf = nullptr;
};

// How output rows of a matrix pair up in an epilogue.
enum PairMode { PAIR_ADJ = 0, PAIR_GU = 1 };

// Epilogues shared by the mat-vec and the GEMMs.
enum Epi {
    EPI_STORE = 0,   // y[t][n] = acc                         (f32)
    EPI_RESID = 1,   // y[t][n] += acc                        (f32 residual stream)
    EPI_QKV = 2,     // RoPE on q,k; q -> qout f32; k,v -> cache (kvtype; Q8_0: -> kv.stage)
    EPI_SWIGLU = 3,  // rows interleaved 32 gate / 32 up; h[t][j] = f16(silu(g) * u)
};

// Per-token step data, device arrays indexed by the token's row in the call.
struct TokInfo {
    const int32_t *pos = nullptr;   // position of the token in its sequence
    const int32_t *seq = nullptr;   // sequence id
};

// One layer's cache, [seq][kv head][position][hd] elements of kvtype.  A
// Q8_0 cache holds int8 codes in k / v and the f16 scale of each 32-element
// block in k_scale / v_scale ([seq][kv head][position][hd/32]); the QKV
// epilogue leaves the new rows in `stage` as f32 ([token][K, V][n_kv*hd]) and
// launch_kv_quant codes them into their cells.
struct KVLayer {
    void *k = nullptr, *v = nullptr;
    uint16_t *k_scale = nullptr, *v_scale = nullptr;
    float *stage = nullptr;
    int kvtype = 0;
    int n_ctx = 0, n_kv = 0, hd = 0;
};

// Partial sums of squares of a residual row: the kernels that write x (the
// embedding, the residual-add mat-vecs) leave one per block in slots
// [row][0..SS_SLOTS) (unused slots 0), and the next RMSNorm prologue adds
// them in slot order instead of re-reading the row.
constexpr int SS_SLOTS = 256;

struct EpiArgs {
    int epi = EPI_STORE;
    float *ss_out = nullptr;   // RESID (mat-vec), optional: [T][SS_SLOTS] sums of squares of the new rows
    float *y = nullptr;        // STORE / RESID: [T][ldy]
    int ldy = 0;
    uint16_t *h = nullptr;     // SWIGLU: f16 [T][ldh]
    uint16_t *h_lo = nullptr;  // SWIGLU: optional f16 rounding remainder of h
    int ldh = 0;
    float *qout = nullptr;     // QKV: f32 [T][qd]
    uint16_t *qh = nullptr;    // QKV, optional: f16 [T][qd] of q * qscale (value) ...
    uint16_t *ql = nullptr;    // ... and its rounding remainder
    float qscale = 1.f;        // 1 / sqrt(head_dim)
    int qd = 0, kd = 0;
    KVLayer kv;
    TokInfo tok;
    const float *rope_cs = nullptr;  // [n_ctx][hd/2][2] (cos, sin)
    // RESID, optional: when the GEMM ends with a K-split sum, that kernel also
    // writes the new rows' RMSNorm (gain nrm_g, eps nrm_eps) as f16 value
    // nrm_h + remainder nrm_l [T][nrm_ld] and sets *nrm_done = 1 (host flag)
    const float *nrm_g = nullptr;
    float nrm_eps = 0.f;
    uint16_t *nrm_h = nullptr, *nrm_l = nullptr;
    int nrm_ld = 0;
    int *nrm_done = nullptr;
};

// Input of a mat-vec / GEMM: either an f32 residual row normalized on the
// fly (RMSNorm prologue) or an f16 activation row.
struct InArgs {
    const float *x32 = nullptr;      // [T][ldx] f32; used when norm_g != nullptr
    const float *norm_g = nullptr;
    float eps = 0.f;
    const float *ss_part = nullptr;  // optional: [rows][SS_SLOTS] partial sums of squares of x32 rows
    const uint16_t *x16 = nullptr;   // [T][ldx] f16 when no prologue
    const uint16_t *x16lo = nullptr; // [T][ldx] f16 remainder: the row is x16 + x16lo
    int ldx = 0;
    const int32_t *row_idx = nullptr;  // optional gather: input row of output row t
};

// ---- launchers (all asynchronous on `s`) ---------------------------------
// Block quantization of fp32 rows on the device (bit-exact with the block
// definitions).  Source rows [rows][K] f32 (device); row r goes to stored row
// dst_row(r) of `m` where mode 0: r + row_off, 1: gate slot, 2: up slot.
void launch_quantize(const float *src, int rows, int K, QMat &m, int mode, int row_off,
                     hipStream_t s);
// fp32 copy into a (possibly padded) F32 matrix: src [rows][K_src] -> m rows
// dst_row(r), columns [0, K_src); the caller zero-fills padding beforehand.
void launch_copy_f32(const float *src, int rows, int K_src, QMat &m, int mode, int row_off,
                     hipStream_t s);
// GGUF-style blocks (f16 scale + codes, 18 / 34 bytes, 2-byte aligned) of a
// rows x K Q4_0 / Q8_0 tensor, or 144-byte Q4_K super-blocks (16-byte
// aligned), -> scales and codes of rows dst_row(r) of m.
void launch_put_blocks(const void *src, int rows, int K, QMat &m, int mode, int row_off, hipStream_t s);
// Q8_0 cache: codes the T staged K and V rows (kv.stage) into the cells at
// (tok.seq[t], tok.pos[t]), with the weights' Q8_0 block definition.
void launch_kv_quant(const KVLayer &kv, TokInfo tok, int T, hipStream_t s);

// Number of compute units the mat-vec grid is sized for (default 256).
void matvec_set_num_cu(int n);
// K slices per row pair the mat-vec uses for an N x K matrix on a grid of
// num_cu blocks (num_cu <= 0: the grid matvec_set_num_cu set).
int matvec_slices(int N, int K, int num_cu);
// y = W x for T tokens (decode).  Q8_0 / Q4_0 only.  The input row is
// RMS-normalized (in.norm_g) for every epilogue but EPI_RESID, which takes
// the f16 row as is.
bool launch_matvec(const QMat &W, const InArgs &in, const EpiArgs &ep, int T, hipStream_t s);
// Y = X W^T for T tokens (prefill / batched decode), X = Xh + Xl given as two
// f16 arrays [T][ldx] (value and rounding remainder): MFMA for Q8_0 / Q4_0
// with N % 128 == 0 and Q4_K with N % 256 == 0, a plain fp32 kernel
// otherwise (on the codes for quantized weights).  `ws` (ws_bytes) holds the fp32 partial tiles of a K split (and
// for Q4_K first the tokens' block sums); with too little workspace (or none)
// the GEMM splits K less (or not at all; Q4_K then takes the plain kernel).
bool launch_gemm(const QMat &W, const uint16_t *Xh, const uint16_t *Xl, int ldx, const EpiArgs &ep,
                 int T, float *ws, size_t ws_bytes, hipStream_t s);
// Workspace launch_gemm uses for W at T tokens (0 when it does not split K).
size_t gemm_workspace_bytes(const QMat &W, int T);
// The direct-to-LDS form of the ubatch GEMM (gemm_dl.hip): a block tile of
// gemm_dl_tile_features() x gemm_dl_tile_tokens(), `ns` LDS stages (3, 4 or
// 5), K split S (fp32 partial tiles in ws, summed by launch_splitk_sum).
// Q4_K also reads xs, the tokens' block sums of x ([M][K/32], written by
// launch_block_sums).
void launch_gemm_dl(int ns, const QMat &W, const uint16_t *Xh, const uint16_t *Xl, int ldx, const EpiArgs &ep,
                    int M, int pair_mode, int S, float *ws, const float *xs, hipStream_t s);
// The sum over the 32 elements of block kb of (Xh + Xl)[m] (fp32, in order)
// as f16 value | f16 remainder << 16 (uint32) at xs[((kb / 8) M + m) 8 + kb % 8].
void launch_block_sums(const uint16_t *Xh, const uint16_t *Xl, int ldx, int M, int K, float *xs, hipStream_t s);
// Derives the GEMM's scale arrays once every row of m is stored: Q4_0/Q8_0
// m.dt from m.d; Q4_K m.mfq and m.sf from m.d and m.dm.
void launch_gemm_scales(QMat &m, hipStream_t s);
// The wide direct-to-LDS form (Q4_0 / Q8_0 / Q4_K, ubatches of more than 64
// tokens): gemm_dw_tile_features() x 128 block tiles, codes loaded 64 bytes
// of a row at a time; K split S into equal ranges of whole periods of
// gemm_dw_super_blocks() K blocks (Q4_K: whole octets; it also reads xs, the
// tokens' block sums written by launch_block_sums).
void launch_gemm_dw(const QMat &W, const uint16_t *Xh, const uint16_t *Xl, int ldx, const EpiArgs &ep, int M,
                    int pair_mode, int S, float *ws, const float *xs, hipStream_t s);
int gemm_dw_tile_features();
int gemm_dw_super_blocks();
int gemm_dl_tile_features();
int gemm_dl_tile_tokens();
// The same form with 32-token block tiles for ubatches of at most 32 tokens
// (batched decode): `ns` stages (4, 6 or 8), K split S (uneven splits allowed).
void launch_gemm_dls(int ns, const QMat &W, const uint16_t *Xh, const uint16_t *Xl, int ldx, const EpiArgs &ep,
                     int M, int pair_mode, int S, float *ws, const float *xs, hipStream_t s);
int gemm_dls_tile_tokens();
// Weight-streaming form for Q4_0 at most 32 tokens (K % 256 == 0, N % 256 ==
// 0): K split S in whole octets of K blocks, at most
// gemm_ws_max_blocks_per_split() K blocks per split.
void launch_gemm_ws(int ks, const QMat &W, const uint16_t *Xh, const uint16_t *Xl, int ldx, const EpiArgs &ep, int M,
                    int pair_mode, int S, float *ws, hipStream_t s);
int gemm_ws_max_blocks_per_split();
// Sums S fp32 partial tiles [S][M][N] in split order and applies epilogue epi.
void launch_splitk_sum(int epi, const float *ws, int S, int N, int M, const EpiArgs &ep, int pair_mode,
                       hipStream_t s);
// Number of compute units the GEMM grid is sized for (default 256).
void gemm_set_num_cu(int n);
// Largest K split of the wide GEMM form for launches from the calling thread
// (1, 2, 4 or 8; default 8).  While two prefill ubatches share the chip the
// other's blocks fill the compute units a smaller split leaves idle, and the
// fewer fp32 partials cost less.
void gemm_set_split_cap(int cap);

// x[t] = dequantized row tok[t] of the embedding table (f32).
void launch_embed(const QMat &E, const int32_t *tok, int T, float *x, int ldx, float *ss_out, hipStream_t s);
// y = rmsnorm(x[row_idx ? row_idx[t] : t]) * g as f16 value xn[t] and f16
// rounding remainder xl[t] (y = xn + xl to about 22 bits)
void launch_rmsnorm(const float *x, int ldx, const float *g, int d, float eps,
                    const int32_t *row_idx, int T, uint16_t *xn, uint16_t *xl, int ldn, hipStream_t s);
// out[t] = argmax of logits row t (lowest index on ties)
void launch_argmax(const float *logits, int V, int T, int32_t *out, hipStream_t s);
// cos/sin table [n_ctx][hd/2][2] with theta = p * base^(-2i/hd) in double
void launch_rope_table(float *cs, int n_ctx, int hd, float base, hipStream_t s);

// Causal attention of T tokens against their sequences' cached rows
// (positions 0..pos[t]), split over key chunks of `chunk` rows, then merged.
struct AttnArgs {
    const float *q = nullptr;     // [T][H*hd] f32 (after RoPE)
    const uint16_t *qh = nullptr; // [T][H*hd] f16 q / sqrt(hd): value (f16 cache, hd 64/128) ...
    const uint16_t *ql = nullptr; // ... and remainder
    KVLayer kv;
    TokInfo tok;
    int H = 0;
    float *part = nullptr;        // [T][H][max_chunks][hd] partial outputs
    float *ml = nullptr;          // [T][H][max_chunks][2] running max / sum
    int max_chunks = 0, chunk = 0;
    // Q8_0 cache, every token of its own sequence (decode): the block whose
    // chunk holds a token's position first codes the token's staged K / V
    // rows of its KV head into the cache (no launch_kv_quant needed)
    int code_new_rows = 0;
    uint16_t *o = nullptr;        // [T][H*hd] f16 output
    uint16_t *o_lo = nullptr;     // [T][H*hd] f16 rounding remainder of the output
};
bool launch_attention(const AttnArgs &a, int T, hipStream_t s);
// Whether launch_attention can take code_new_rows for this cache.
bool attention_codes_rows(int kvtype, int hd);

// Causal attention of a prefill ubatch: T tokens of sequence tok.seq[0] at
// positions tok.pos[0] + t, f16 cache, MFMA flash attention.  Returns false
// (nothing launched) when the shape is not covered.
struct FlashArgs {
    const float *q = nullptr;     // [T][H*hd] f32 (after RoPE)
    const uint16_t *qh = nullptr; // [T][H*hd] f16 q / sqrt(hd): value (f16 cache, hd 64/128) ...
    const uint16_t *ql = nullptr; // ... and remainder
    KVLayer kv;
    TokInfo tok;
    int H = 0, T = 0;
    uint16_t *o = nullptr;        // [T][H*hd] f16 output
    uint16_t *o_lo = nullptr;     // [T][H*hd] f16 rounding remainder of the output
    // key split: per-range unnormalized outputs [T][H][max_chunks][hd] and
    // (max, sum) [T][H][max_chunks][2]; null: no split
    float *part = nullptr, *ml = nullptr;
    int max_chunks = 0;
    int tok_pos0_max = 0;         // host-side upper bound of tok.pos[0] (sizes the key ranges)
    int ns = 1, chunk = 0;        // set by the launcher
};
bool launch_flash_prefill(const FlashArgs &a, hipStream_t s);

// f16 -> (rows of) GGUF-style export helpers are host code in engine.cpp.

// The sampler chain on one logits row (device): repeat penalty over the
// distinct tokens of hist[0..n_hist), top-k (1..1024), top-p, min-p,
// temperature (<= 0: the leader), then the draw with u from SplitMix64(seed,
// draw).  Writes the token to out[0].  Returns false (nothing launched) when
// the sizes are not covered (n_vocab <= 32768, n_hist <= 64).
struct SampleArgs {
    const int32_t *hist = nullptr;
    int n_hist = 0, n_vocab = 0, top_k = 0;
    float top_p = 1.f, min_p = 0.f, temp = 1.f, repeat_penalty = 1.f;
    uint64_t seed = 0, draw = 0;
    int32_t *out = nullptr;
};
bool launch_sample(const float *logits, const SampleArgs &a, hipStream_t s);

// The library's log sink (level 0 debug .. 3 error; see dec_set_log_callback).
void log_message(int level, const char *fmt, ...) __attribute__((format(printf, 2, 3)));


// ---- one decode step of one token as a single persistent kernel ----------
// One layer's weights and f16 cache as the step kernel reads them (a device
// array of n_layer entries, built once per context).
struct StepLayer {
    QMat wqkv, wo, wgu, wdown;
    const float *attn_norm = nullptr, *ffn_norm = nullptr;
    uint16_t *k = nullptr, *v = nullptr;   // [seq][n_kv][n_ctx][hd] f16
};

// Barrier and merge-counter memory of the step kernel (uint32 words, zeroed
// once; the kernel keeps it consistent from launch to launch).
constexpr int STEP_SYNC_WORDS = 64 * 96;
// Word index of the failure flag (a bounded wait timed out) in that memory.
constexpr int STEP_SYNC_FAIL = 64 * 17;
// Most blocks that share one KV head's attention (their partials meet in one merge).
constexpr int STEP_BPG_MAX = 64;

struct StepArgs {
    const StepLayer *layers = nullptr;
    int n_layer = 0;
    QMat tok, out;
    const float *out_norm = nullptr;
    int d = 0, qd = 0, kd = 0, Fp = 0, H = 0, Hkv = 0, hd = 0, V = 0, n_ctx = 0;
    float eps = 0.f, qscale = 1.f;
    const int32_t *step = nullptr;    // the token: id, position, sequence
    const float *rope_cs = nullptr;   // [n_ctx][hd/2][2]
    float *x = nullptr;               // [d] residual row
    float *ss = nullptr;              // [SS_SLOTS] partial sums of squares of x
    uint16_t *qh = nullptr, *ql = nullptr;   // [qd] q / sqrt(hd), f16 value + remainder
    uint16_t *o = nullptr, *o_lo = nullptr;  // [qd] attention output
    uint16_t *h = nullptr, *h_lo = nullptr;  // [Fp] SwiGLU output
    float *apart = nullptr;           // [Hkv][bpg][G][hd] attention partials of the blocks
    float *aml = nullptr;             // [Hkv][bpg][G][2] their running max / sum
    int bpg = 0;                      // blocks per KV head in the attention phase
    float *logits = nullptr;          // [V]
    int32_t *amax = nullptr;          // greedy token, -1 when a wait timed out
    float *bmax = nullptr;            // [grid] per-block argmax candidates
    int32_t *bidx = nullptr;
    uint32_t *sync = nullptr;         // STEP_SYNC_WORDS
    int S_qkv = 1, S_o = 1, S_gu = 1, S_down = 1, S_out = 1;   // K slices per phase
};
// Grid barriers one launch performs.
inline uint32_t step_barriers(int n_layer) { return 2u + 5u * (uint32_t)n_layer; }
// Whether the step kernel covers this shape; `why` names the first reason it does not.
bool step_supported(const StepArgs &a, int wtype, int kvtype, int grid, const char **why);
// K slices per row pair the step kernel uses for an N x K matrix on `grid` blocks.
int step_slices(int N, int K, int grid);
// Blocks of the step kernel one compute unit holds (0: not launchable).
int step_blocks_per_cu(int wtype, int hd);
// Launches the step (cooperative launch of `grid` blocks of 512 threads) with
// the argument block at dev_args (device memory, as checked by step_supported)
// after n0 grid barriers of earlier launches on the same sync memory.
bool launch_step(const StepArgs *dev_args, int wtype, int hd, uint32_t n0, int grid, hipStream_t s);
