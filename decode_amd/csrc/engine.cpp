// engine.cpp -- host side of libdecode: the C ABI of include/decode.h.
//
// Model load, context creation (all memory reserved for the worst case up
// front), batch validation, ubatch splitting with up-front cell reservation,
// the per-layer launch sequence, HIP-graph capture and replay of decode
// steps, and on-demand logits / greedy-token readback.  Every arithmetic
// step of the decoder runs in the kernels of this directory; this file only
// moves bytes and launches work.
#include "../../include/decode.h"
#include "gguf.h"

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <map>
#include <new>
#include <string>
#include <vector>

#include "kernels.h"

int attention_chunk(int kvtype, int hd);

// --------------------------------------------------------------- logging
static void (*g_log_cb)(int, const char *, void *) = nullptr;
static void *g_log_ud = nullptr;

void log_message(int level, const char *fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    if (g_log_cb)
        g_log_cb(level, buf, g_log_ud);
    else if (level >= 3)
        fprintf(stderr, "libdecode: %s\n", buf);
}
#define LOGE(...) log_message(3, __VA_ARGS__)
#define LOGW(...) log_message(2, __VA_ARGS__)
#define LOGI(...) log_message(1, __VA_ARGS__)

#define HIP_OK(expr, onfail)                                                          \
    do {                                                                              \
        hipError_t e_ = (expr);                                                       \
        if (e_ != hipSuccess) {                                                       \
            LOGE("%s failed: %s (%s:%d)", #expr, hipGetErrorString(e_), __FILE__, __LINE__); \
            onfail;                                                                   \
        }                                                                             \
    } while (0)

// --------------------------------------------------------------- memory
struct Mem {
    dec_allocator a{};
    bool custom = false;
    std::vector<void *> owned;

    void *get(size_t bytes) {
        bytes = (bytes + 255) & ~(size_t)255;
        if (bytes == 0) bytes = 256;
        void *p = nullptr;
        if (custom) {
            p = a.alloc(bytes, a.ud);
            if (p && ((uintptr_t)p & 255)) {   // the kernels rely on the 256-byte alignment the contract states
                LOGE("allocator returned memory not aligned to 256 bytes");
                a.free(p, a.ud);
                p = nullptr;
            }
        } else if (hipMalloc(&p, bytes) != hipSuccess) {
            (void)hipGetLastError();
            p = nullptr;
        }
        if (p) owned.push_back(p);
        else LOGE("device allocation of %zu bytes failed", bytes);
        return p;
    }
    // Returns one allocation of this owner before the others.
    void drop(void *p) {
        if (!p) return;
        for (size_t i = 0; i < owned.size(); i++)
            if (owned[i] == p) {
                if (custom) a.free(p, a.ud);
                else (void)hipFree(p);
                owned.erase(owned.begin() + (long)i);
                return;
            }
    }
    void release() {
        for (void *p : owned) {
            if (custom) a.free(p, a.ud);
            else (void)hipFree(p);
        }
        owned.clear();
    }
};

static bool is_device_ptr(const void *p) {
    hipPointerAttribute_t at;
    if (hipPointerGetAttributes(&at, p) != hipSuccess) {
        (void)hipGetLastError();
        return false;
    }
    return at.type == hipMemoryTypeDevice;
}

// --------------------------------------------------------------- model
struct Layer {
    QMat wqkv, wo, wgu, wdown;
    float *attn_norm = nullptr, *ffn_norm = nullptr;
};

struct dec_model {
    dec_hparams hp{};
    int qd = 0, kd = 0, F = 0, Fp = 0;
    QMat tok, out;
    float *out_norm = nullptr;
    std::vector<Layer> layers;
    Mem mem;
    hipStream_t stream = nullptr;
    int n_ctx_refs = 0;        // live contexts; the model's memory outlives them
    bool free_requested = false;
};

static void model_release(dec_model *m) {
    (void)hipStreamSynchronize(m->stream);
    m->mem.release();
    delete m;
}

// gemm: the matrix is a GEMM operand (every matrix but the token embedding),
// which also holds the GEMM's derived scale arrays.
static bool alloc_qmat(Mem &mem, QMat &m, int wtype, int N, int K, bool gemm = true) {
    m.wtype = wtype;
    m.N = N;
    m.K = K;
    size_t qbytes;
    if (wtype == DEC_F32) qbytes = (size_t)N * K * 4;
    else if (wtype == DEC_Q8_0) qbytes = (size_t)N * K;
    else qbytes = (size_t)N * K / 2;
    m.qs = mem.get(qbytes);
    if (!m.qs) return false;
    if (wtype != DEC_F32) {
        m.d = (uint16_t *)mem.get((size_t)N * (K / 32) * 2);
        if (!m.d) return false;
    } else if (hipMemset(m.qs, 0, qbytes) != hipSuccess) {   // padding must read as zero
        return false;
    }
    if (wtype == DEC_Q4_K) {
        m.dm = (uint32_t *)mem.get((size_t)N * (K / 256) * 4);
        if (!m.dm) return false;
        if (gemm) {
            m.mfq = (uint32_t *)mem.get((size_t)N * (K / 32) * 4);
            m.sf = (float *)mem.get((size_t)N * (K / 32) * 4);
            if (!m.mfq || !m.sf) return false;
        }
    } else if (gemm && (wtype == DEC_Q8_0 || wtype == DEC_Q4_0)) {
        m.dt = (uint16_t *)mem.get((size_t)N * (K / 32) * 2);
        if (!m.dt) return false;
    }
    return true;
}

// Stages one fp32 source tensor on the device (if it is host memory) and
// stores it into rows of m.
struct Loader {
    Mem &mem;
    hipStream_t s;
    float *stage = nullptr;
    size_t stage_elems = 0;

    bool put(const float *src, int rows, int K_src, QMat &m, int mode, int row_off) {
        if (!src) {
            LOGE("missing weight tensor");
            return false;
        }
        const size_t n = (size_t)rows * K_src;
        const float *dsrc = src;
        if (!is_device_ptr(src)) {
            if (n > stage_elems) {
                LOGE("staging buffer too small");
                return false;
            }
            HIP_OK(hipMemcpyAsync(stage, src, n * 4, hipMemcpyHostToDevice, s), return false);
            dsrc = stage;
        }
        if (m.wtype == DEC_F32)
            launch_copy_f32(dsrc, rows, K_src, m, mode, row_off, s);
        else
            launch_quantize(dsrc, rows, K_src, m, mode, row_off, s);
        HIP_OK(hipGetLastError(), return false);
        if (dsrc == stage) HIP_OK(hipStreamSynchronize(s), return false);   // stage reused next
        return true;
    }
    bool vec(const float *src, int n, float **dst) {
        if (!src) {
            LOGE("missing norm vector");
            return false;
        }
        *dst = (float *)mem.get((size_t)n * 4);
        if (!*dst) return false;
        HIP_OK(hipMemcpyAsync(*dst, src, (size_t)n * 4, hipMemcpyDefault, s), return false);
        return true;
    }
};

// Q4_K: the GEMM's min-term operand of every matrix, once all rows are stored.
// The GEMM operands' derived scale arrays, once every matrix is stored.
static void finish_gemm_scales(dec_model *m, hipStream_t s) {
    if (m->hp.wtype == DEC_F32) return;
    launch_gemm_scales(m->out, s);
    for (Layer &L : m->layers)
        for (QMat *q : {&L.wqkv, &L.wo, &L.wgu, &L.wdown}) launch_gemm_scales(*q, s);
}

static bool valid_hparams(const dec_hparams &h) {
    if (h.n_layer <= 0 || h.n_embd <= 0 || h.n_head <= 0 || h.n_head_kv <= 0 || h.head_dim <= 0 ||
        h.n_ff <= 0 || h.n_vocab <= 0)
        return false;
    if (h.head_dim != 64 && h.head_dim != 128 && h.head_dim != 256) return false;
    if (h.n_head % h.n_head_kv || h.n_head / h.n_head_kv > 8) return false;
    if (h.wtype != DEC_F32 && h.wtype != DEC_Q8_0 && h.wtype != DEC_Q4_0 && h.wtype != DEC_Q4_K) return false;
    if (h.kvtype != DEC_F32 && h.kvtype != DEC_F16 && h.kvtype != DEC_Q8_0) return false;
    if (h.n_embd % 32 || (h.n_head * h.head_dim) % 32) return false;
    if (h.wtype != DEC_F32 && h.n_ff % 32) return false;
    // Q4_K rows are whole 256-weight super-blocks
    if (h.wtype == DEC_Q4_K && (h.n_embd % 256 || (h.n_head * h.head_dim) % 256 || h.n_ff % 256)) return false;
    // the decode mat-vec holds a whole input row in LDS: every K of a
    // quantized matrix (d, H*hd, n_ff) is at most MV_KMAX elements
    if (h.wtype != DEC_F32 &&
        (h.n_embd > DEC_MAX_ROW || h.n_head * h.head_dim > DEC_MAX_ROW || h.n_ff > DEC_MAX_ROW))
        return false;
    if (!(h.rms_eps >= 0.f) || !(h.rope_base > 0.f)) return false;
    return true;
}

extern "C" dec_model *dec_model_load(const dec_hparams *hp, const dec_weights *w,
                                     const dec_allocator *alloc, void *hip_stream) {
    if (!hp || !w || !valid_hparams(*hp)) {
        LOGE("dec_model_load: invalid hyper-parameters");
        return nullptr;
    }
    if (alloc && (!alloc->alloc || !alloc->free)) {
        LOGE("dec_model_load: allocator needs both callbacks");
        return nullptr;
    }
    dec_model *m = new dec_model();
    m->hp = *hp;
    if (alloc) {
        m->mem.a = *alloc;
        m->mem.custom = true;
    }
    m->stream = (hipStream_t)hip_stream;
    const dec_hparams &h = m->hp;
    m->qd = h.n_head * h.head_dim;
    m->kd = h.n_head_kv * h.head_dim;
    m->F = h.n_ff;
    m->Fp = (h.n_ff + 31) / 32 * 32;
    const int d = h.n_embd, V = h.n_vocab, qd = m->qd, kd = m->kd, F = m->F, Fp = m->Fp;

    bool ok = alloc_qmat(m->mem, m->tok, h.wtype, V, d, false) && alloc_qmat(m->mem, m->out, h.wtype, V, d);
    m->layers.resize(h.n_layer);
    for (int l = 0; ok && l < h.n_layer; l++) {
        Layer &L = m->layers[l];
        ok = alloc_qmat(m->mem, L.wqkv, h.wtype, qd + 2 * kd, d) && alloc_qmat(m->mem, L.wo, h.wtype, d, qd) &&
             alloc_qmat(m->mem, L.wgu, h.wtype, 2 * Fp, d) && alloc_qmat(m->mem, L.wdown, h.wtype, d, Fp);
    }
    size_t stage = 0;
    auto need = [&](const float *p, size_t n) {
        if (p && !is_device_ptr(p) && n > stage) stage = n;
    };
    need(w->tok_embd, (size_t)V * d);
    need(w->output, (size_t)V * d);
    for (int l = 0; l < h.n_layer; l++) {
        if (!w->wq || !w->wk || !w->wv || !w->wo || !w->ffn_gate || !w->ffn_up || !w->ffn_down ||
            !w->attn_norm || !w->ffn_norm) {
            ok = false;
            break;
        }
        need(w->wq[l], (size_t)qd * d);
        need(w->wk[l], (size_t)kd * d);
        need(w->wv[l], (size_t)kd * d);
        need(w->wo[l], (size_t)d * qd);
        need(w->ffn_gate[l], (size_t)F * d);
        need(w->ffn_up[l], (size_t)F * d);
        need(w->ffn_down[l], (size_t)d * F);
    }
    Loader ld{m->mem, m->stream};
    if (ok && stage) {
        ld.stage = (float *)m->mem.get(stage * 4);
        ld.stage_elems = stage;
        ok = ld.stage != nullptr;
    }
    ok = ok && ld.put(w->tok_embd, V, d, m->tok, 0, 0) && ld.put(w->output, V, d, m->out, 0, 0) &&
         ld.vec(w->output_norm, d, &m->out_norm);
    for (int l = 0; ok && l < h.n_layer; l++) {
        Layer &L = m->layers[l];
        ok = ld.put(w->wq[l], qd, d, L.wqkv, 0, 0) && ld.put(w->wk[l], kd, d, L.wqkv, 0, qd) &&
             ld.put(w->wv[l], kd, d, L.wqkv, 0, qd + kd) && ld.put(w->wo[l], d, qd, L.wo, 0, 0) &&
             ld.put(w->ffn_gate[l], F, d, L.wgu, 1, 0) && ld.put(w->ffn_up[l], F, d, L.wgu, 2, 0) &&
             ld.put(w->ffn_down[l], d, F, L.wdown, 0, 0) && ld.vec(w->attn_norm[l], d, &L.attn_norm) &&
             ld.vec(w->ffn_norm[l], d, &L.ffn_norm);
    }
    if (ok) finish_gemm_scales(m, m->stream);
    if (ok) HIP_OK(hipStreamSynchronize(m->stream), ok = false);
    m->mem.drop(ld.stage);   // host weights are staged during the load only
    if (!ok) {
        LOGE("dec_model_load failed");
        m->mem.release();
        delete m;
        return nullptr;
    }
    LOGI("model loaded: %d layers, d=%d, wtype=%d", h.n_layer, d, h.wtype);
    return m;
}

extern "C" void dec_model_free(dec_model *m) {
    if (!m) return;
    if (m->n_ctx_refs) {
        // contexts still read the weights: release with the last of them
        LOGW("dec_model_free: %d contexts still alive, freeing with the last one", m->n_ctx_refs);
        m->free_requested = true;
        return;
    }
    model_release(m);
}

// Export of one stored matrix in its file form (GGUF-style blocks).
extern "C" int64_t dec_model_tensor_blocks(const dec_model *m, int32_t id, int32_t layer, void *dst,
                                           size_t cap) {
    if (!m || id < 0 || id > 8) return 0;
    const dec_hparams &h = m->hp;
    if (id >= 2 && (layer < 0 || layer >= h.n_layer)) return 0;
    const QMat *src = nullptr;
    int rows = 0, cols = 0, mode = 0, row_off = 0;
    const int d = h.n_embd;
    switch (id) {
    case DEC_T_TOK_EMBD: src = &m->tok; rows = h.n_vocab; cols = d; break;
    case DEC_T_OUTPUT: src = &m->out; rows = h.n_vocab; cols = d; break;
    case DEC_T_WQ: src = &m->layers[layer].wqkv; rows = m->qd; cols = d; break;
    case DEC_T_WK: src = &m->layers[layer].wqkv; rows = m->kd; cols = d; row_off = m->qd; break;
    case DEC_T_WV: src = &m->layers[layer].wqkv; rows = m->kd; cols = d; row_off = m->qd + m->kd; break;
    case DEC_T_WO: src = &m->layers[layer].wo; rows = d; cols = m->qd; break;
    case DEC_T_FFN_GATE: src = &m->layers[layer].wgu; rows = m->F; cols = d; mode = 1; break;
    case DEC_T_FFN_UP: src = &m->layers[layer].wgu; rows = m->F; cols = d; mode = 2; break;
    case DEC_T_FFN_DOWN: src = &m->layers[layer].wdown; rows = d; cols = m->F; break;
    }
    const int wt = src->wtype;
    const int nb = cols / 32;
    const size_t row_bytes = wt == DEC_F32    ? (size_t)cols * 4
                             : wt == DEC_Q4_K ? (size_t)(cols / 256) * 144
                                              : (size_t)nb * (wt == DEC_Q8_0 ? 34 : 18);
    const size_t total = row_bytes * rows;
    if (!dst || cap < total) return -(int64_t)total;
    if (hipStreamSynchronize(m->stream) != hipSuccess) return 0;

    // copy the whole stored matrix once, then pick rows / interleave blocks
    const size_t srow_q = wt == DEC_F32 ? (size_t)src->K * 4 : (wt == DEC_Q8_0 ? (size_t)src->K : (size_t)src->K / 2);
    std::vector<uint8_t> q((size_t)src->N * srow_q);
    std::vector<uint16_t> sc(wt == DEC_F32 ? 0 : (size_t)src->N * (src->K / 32));
    if (hipMemcpy(q.data(), src->qs, q.size(), hipMemcpyDeviceToHost) != hipSuccess) return 0;
    if (!sc.empty() && hipMemcpy(sc.data(), src->d, sc.size() * 2, hipMemcpyDeviceToHost) != hipSuccess)
        return 0;
    std::vector<uint32_t> dmv(wt == DEC_Q4_K ? (size_t)src->N * (src->K / 256) : 0);
    if (!dmv.empty() && hipMemcpy(dmv.data(), src->dm, dmv.size() * 4, hipMemcpyDeviceToHost) != hipSuccess)
        return 0;
    uint8_t *o = (uint8_t *)dst;
    for (int r = 0; r < rows; r++) {
        int sr = r + row_off;
        if (mode == 1) sr = ((r >> 5) << 6) + (r & 31);
        if (mode == 2) sr = ((r >> 5) << 6) + 32 + (r & 31);
        const uint8_t *qr = q.data() + (size_t)sr * srow_q;
        if (wt == DEC_F32) {
            memcpy(o, qr, (size_t)cols * 4);
            o += (size_t)cols * 4;
            continue;
        }
        if (wt == DEC_Q4_K) {
            // stored (Q4_0-layout codes, sc | m << 8 per sub-block, d | dmin << 16)
            // -> the 144-byte super-block of the public layout
            const uint16_t *sm = sc.data() + (size_t)sr * (src->K / 32);
            for (int sb = 0; sb < cols / 256; sb++) {
                const uint32_t dd = dmv[(size_t)sr * (src->K / 256) + sb];
                memcpy(o, &dd, 4);
                int scj[8], mj[8];
                for (int j = 0; j < 8; j++) {
                    scj[j] = sm[8 * sb + j] & 63;
                    mj[j] = (sm[8 * sb + j] >> 8) & 63;
                }
                for (int j = 0; j < 4; j++) {
                    o[4 + j] = (uint8_t)(scj[j] | ((scj[j + 4] >> 4) << 6));
                    o[8 + j] = (uint8_t)(mj[j] | ((mj[j + 4] >> 4) << 6));
                    o[12 + j] = (uint8_t)((scj[j + 4] & 15) | ((mj[j + 4] & 15) << 4));
                }
                // sub-block pair (2g, 2g+1): stored byte k of sub-block j holds its
                // weights k (low) and k+16 (high); file byte 32g + l holds weight
                // l of sub-block 2g (low) and of sub-block 2g+1 (high)
                const uint8_t *q = qr + (size_t)sb * 128;
                for (int g = 0; g < 4; g++)
                    for (int l = 0; l < 32; l++) {
                        const uint8_t a = q[32 * g + (l & 15)], b = q[32 * g + 16 + (l & 15)];
                        const int lo = l < 16 ? (a & 15) : (a >> 4), hi = l < 16 ? (b & 15) : (b >> 4);
                        o[16 + 32 * g + l] = (uint8_t)(lo | (hi << 4));
                    }
                o += 144;
            }
            continue;
        }
        const int qb = wt == DEC_Q8_0 ? 32 : 16;
        const uint16_t *sr_d = sc.data() + (size_t)sr * (src->K / 32);
        for (int b = 0; b < nb; b++) {
            o[0] = (uint8_t)(sr_d[b] & 0xff);
            o[1] = (uint8_t)(sr_d[b] >> 8);
            memcpy(o + 2, qr + (size_t)b * qb, qb);
            o += 2 + qb;
        }
    }
    return (int64_t)total;
}

// --------------------------------------------------------------- GGUF files
// The llama tensor names of the article's weight set (step 6) and the
// llama.* hyper-parameter keys of step 4.
static std::string layer_name(int l, const char *what) { return "blk." + std::to_string(l) + "." + what + ".weight"; }

static int file_type_of(int wtype) {
    return wtype == DEC_Q4_0   ? gguf::T_Q4_0
           : wtype == DEC_Q8_0 ? gguf::T_Q8_0
           : wtype == DEC_Q4_K ? gguf::T_Q4_K
                               : gguf::T_F32;
}

// Hyper-parameters and tensor checks of a parsed file; returns a gguf status.
static int gguf_model_params(const gguf::File &f, int32_t kvtype, dec_hparams &h) {
    const gguf::Value *arch = f.find("general.architecture");
    if (!arch || arch->type != gguf::V_STR || arch->s != "llama") return gguf::E_SHAPE;
    auto get_u = [&](const char *key, uint64_t &v, bool required, uint64_t dflt) {
        const gguf::Value *x = f.find(key);
        if (!x) {
            v = dflt;
            return !required;
        }
        return x->as_u64(v) && v > 0 && v < (1u << 30);
    };
    auto get_f = [&](const char *key, double &v, double dflt) {
        const gguf::Value *x = f.find(key);
        if (!x) {
            v = dflt;
            return true;
        }
        return x->as_f64(v);
    };
    uint64_t d, nl, ff, nh, nkv, hd;
    double eps, base;
    if (!get_u("llama.embedding_length", d, true, 0) || !get_u("llama.block_count", nl, true, 0) ||
        !get_u("llama.feed_forward_length", ff, true, 0) || !get_u("llama.attention.head_count", nh, true, 0) ||
        !get_u("llama.attention.head_count_kv", nkv, false, nh))
        return gguf::E_SHAPE;
    uint64_t rope_dims;
    if (!get_u("llama.rope.dimension_count", rope_dims, false, d / nh) ||
        !get_u("llama.attention.key_length", hd, false, rope_dims) ||
        !get_f("llama.attention.layer_norm_rms_epsilon", eps, 1e-5) || !get_f("llama.rope.freq_base", base, 10000.0))
        return gguf::E_SHAPE;
    const gguf::Tensor *emb = f.tensor("token_embd.weight");
    if (!emb || emb->n_dims != 2 || emb->dims[0] != d) return gguf::E_SHAPE;
    const uint32_t wt = emb->type;
    if (wt != gguf::T_F32 && wt != gguf::T_Q4_0 && wt != gguf::T_Q8_0 && wt != gguf::T_Q4_K) return gguf::E_TYPE;
    h = dec_hparams{};
    h.n_layer = (int32_t)nl;
    h.n_embd = (int32_t)d;
    h.n_head = (int32_t)nh;
    h.n_head_kv = (int32_t)nkv;
    h.head_dim = (int32_t)hd;
    h.n_ff = (int32_t)ff;
    h.n_vocab = (int32_t)emb->dims[1];
    h.rms_eps = (float)eps;
    h.rope_base = (float)base;
    h.wtype = wt == gguf::T_Q4_0 ? DEC_Q4_0 : wt == gguf::T_Q8_0 ? DEC_Q8_0 : wt == gguf::T_Q4_K ? DEC_Q4_K : DEC_F32;
    h.kvtype = kvtype;
    if (!valid_hparams(h)) return gguf::E_SHAPE;
    const uint64_t qd = nh * hd, kd = nkv * hd, V = (uint64_t)h.n_vocab;
    auto mat = [&](const std::string &name, uint64_t in, uint64_t out) {
        const gguf::Tensor *t = f.tensor(name);
        return t && t->n_dims == 2 && t->dims[0] == in && t->dims[1] == out && t->type == wt;
    };
    auto vec = [&](const std::string &name) {
        const gguf::Tensor *t = f.tensor(name);
        return t && t->n_dims == 1 && t->dims[0] == d && t->type == gguf::T_F32;
    };
    // the output matrix may be absent (tied to the embedding, step 6)
    if ((f.tensor("output.weight") && !mat("output.weight", d, V)) || !vec("output_norm.weight")) return gguf::E_SHAPE;
    for (int l = 0; l < h.n_layer; l++)
        if (!vec(layer_name(l, "attn_norm")) || !mat(layer_name(l, "attn_q"), d, qd) ||
            !mat(layer_name(l, "attn_k"), d, kd) || !mat(layer_name(l, "attn_v"), d, kd) ||
            !mat(layer_name(l, "attn_output"), qd, d) || !vec(layer_name(l, "ffn_norm")) ||
            !mat(layer_name(l, "ffn_gate"), d, ff) || !mat(layer_name(l, "ffn_up"), d, ff) ||
            !mat(layer_name(l, "ffn_down"), ff, d))
            return gguf::E_SHAPE;
    return gguf::OK;
}

extern "C" int32_t dec_gguf_inspect(const char *path, dec_hparams *hp) {
    if (!path || !hp) return -1;
    gguf::File f;
    int st = f.open(path);
    if (st == gguf::OK) st = gguf_model_params(f, DEC_F16, *hp);
    return st == gguf::OK ? (int32_t)f.tensors.size() : st;
}

extern "C" dec_model *dec_model_load_gguf(const char *path, int32_t kvtype, const dec_allocator *alloc,
                                          void *hip_stream) {
    if (alloc && (!alloc->alloc || !alloc->free)) {
        LOGE("dec_model_load_gguf: allocator needs both callbacks");
        return nullptr;
    }
    gguf::File f;
    dec_hparams h{};
    int st = f.open(path);
    if (st == gguf::OK) st = gguf_model_params(f, kvtype, h);
    if (st != gguf::OK) {
        LOGE("dec_model_load_gguf: %s rejected (status %d)", path ? path : "(null)", st);
        return nullptr;
    }
    dec_model *m = new dec_model();
    m->hp = h;
    if (alloc) {
        m->mem.a = *alloc;
        m->mem.custom = true;
    }
    m->stream = (hipStream_t)hip_stream;
    m->qd = h.n_head * h.head_dim;
    m->kd = h.n_head_kv * h.head_dim;
    m->F = h.n_ff;
    m->Fp = (h.n_ff + 31) / 32 * 32;
    const int d = h.n_embd, V = h.n_vocab, qd = m->qd, kd = m->kd, F = m->F, Fp = m->Fp;
    bool ok = alloc_qmat(m->mem, m->tok, h.wtype, V, d, false) && alloc_qmat(m->mem, m->out, h.wtype, V, d);
    m->layers.resize(h.n_layer);
    for (int l = 0; ok && l < h.n_layer; l++) {
        Layer &L = m->layers[l];
        ok = alloc_qmat(m->mem, L.wqkv, h.wtype, qd + 2 * kd, d) && alloc_qmat(m->mem, L.wo, h.wtype, d, qd) &&
             alloc_qmat(m->mem, L.wgu, h.wtype, 2 * Fp, d) && alloc_qmat(m->mem, L.wdown, h.wtype, d, Fp);
    }
    // one device staging buffer for the largest tensor; each tensor's bytes go
    // there straight from the file mapping, then split into codes and scales
    uint64_t largest = 0;
    for (const gguf::Tensor &t : f.tensors) largest = std::max(largest, t.nbytes);
    void *stage = ok ? m->mem.get((size_t)largest) : nullptr;
    ok = ok && stage;
    hipStream_t s = m->stream;
    auto put = [&](const std::string &name, int rows, int K_src, QMat &q, int mode, int row_off) {
        const gguf::Tensor *t = f.tensor(name);
        HIP_OK(hipMemcpyAsync(stage, t->data, (size_t)t->nbytes, hipMemcpyHostToDevice, s), return false);
        if (q.wtype == DEC_F32)
            launch_copy_f32((const float *)stage, rows, K_src, q, mode, row_off, s);
        else
            launch_put_blocks(stage, rows, K_src, q, mode, row_off, s);
        HIP_OK(hipGetLastError(), return false);
        HIP_OK(hipStreamSynchronize(s), return false);   // the staging buffer is reused next
        return true;
    };
    auto vec = [&](const std::string &name, float **dst) {
        *dst = (float *)m->mem.get((size_t)d * 4);
        if (!*dst) return false;
        HIP_OK(hipMemcpyAsync(*dst, f.tensor(name)->data, (size_t)d * 4, hipMemcpyHostToDevice, s), return false);
        return true;
    };
    const bool tied = f.tensor("output.weight") == nullptr;
    ok = ok && put("token_embd.weight", V, d, m->tok, 0, 0) &&
         put(tied ? "token_embd.weight" : "output.weight", V, d, m->out, 0, 0) && vec("output_norm.weight", &m->out_norm);
    for (int l = 0; ok && l < h.n_layer; l++) {
        Layer &L = m->layers[l];
        ok = put(layer_name(l, "attn_q"), qd, d, L.wqkv, 0, 0) && put(layer_name(l, "attn_k"), kd, d, L.wqkv, 0, qd) &&
             put(layer_name(l, "attn_v"), kd, d, L.wqkv, 0, qd + kd) && put(layer_name(l, "attn_output"), d, qd, L.wo, 0, 0) &&
             put(layer_name(l, "ffn_gate"), F, d, L.wgu, 1, 0) && put(layer_name(l, "ffn_up"), F, d, L.wgu, 2, 0) &&
             put(layer_name(l, "ffn_down"), d, F, L.wdown, 0, 0) && vec(layer_name(l, "attn_norm"), &L.attn_norm) &&
             vec(layer_name(l, "ffn_norm"), &L.ffn_norm);
    }
    if (ok) finish_gemm_scales(m, s);
    if (ok) HIP_OK(hipStreamSynchronize(s), ok = false);
    m->mem.drop(stage);   // the file's tensors pass through it during the load only
    if (!ok) {
        LOGE("dec_model_load_gguf failed");
        m->mem.release();
        delete m;
        return nullptr;
    }
    LOGI("model loaded from %s: %d layers, d=%d, wtype=%d", path, h.n_layer, d, h.wtype);
    return m;
}

extern "C" int32_t dec_model_save_gguf(const dec_model *m, const char *path) {
    if (!m || !path) return -1;
    const dec_hparams &h = m->hp;
    std::vector<std::pair<std::string, gguf::Value>> kv = {
        {"general.architecture", gguf::str_value("llama")},
        {"general.alignment", gguf::u32_value(32)},
        {"llama.embedding_length", gguf::u32_value((uint32_t)h.n_embd)},
        {"llama.block_count", gguf::u32_value((uint32_t)h.n_layer)},
        {"llama.feed_forward_length", gguf::u32_value((uint32_t)h.n_ff)},
        {"llama.attention.head_count", gguf::u32_value((uint32_t)h.n_head)},
        {"llama.attention.head_count_kv", gguf::u32_value((uint32_t)h.n_head_kv)},
        {"llama.attention.key_length", gguf::u32_value((uint32_t)h.head_dim)},
        {"llama.attention.value_length", gguf::u32_value((uint32_t)h.head_dim)},
        {"llama.rope.dimension_count", gguf::u32_value((uint32_t)h.head_dim)},
        {"llama.rope.freq_base", gguf::f32_value(h.rope_base)},
        {"llama.attention.layer_norm_rms_epsilon", gguf::f32_value(h.rms_eps)},
        {"llama.vocab_size", gguf::u32_value((uint32_t)h.n_vocab)},
    };
    const uint32_t wt = (uint32_t)file_type_of(h.wtype);
    const uint64_t d = (uint64_t)h.n_embd, V = (uint64_t)h.n_vocab, qd = (uint64_t)m->qd, kd = (uint64_t)m->kd,
                   ff = (uint64_t)h.n_ff;
    std::vector<gguf::OutTensor> ts;
    auto mat = [&](const std::string &name, int id, int layer, uint64_t in, uint64_t out) {
        ts.push_back({name, wt, {in, out}, [m, id, layer](std::vector<uint8_t> &b) {
                          const int64_t need = -dec_model_tensor_blocks(m, id, layer, nullptr, 0);
                          if (need <= 0) return false;
                          b.resize((size_t)need);
                          return dec_model_tensor_blocks(m, id, layer, b.data(), b.size()) == need;
                      }});
    };
    auto vec = [&](const std::string &name, const float *src) {
        ts.push_back({name, gguf::T_F32, {d}, [src, d](std::vector<uint8_t> &b) {
                          b.resize((size_t)d * 4);
                          return hipMemcpy(b.data(), src, b.size(), hipMemcpyDeviceToHost) == hipSuccess;
                      }});
    };
    mat("token_embd.weight", DEC_T_TOK_EMBD, 0, d, V);
    vec("output_norm.weight", m->out_norm);
    mat("output.weight", DEC_T_OUTPUT, 0, d, V);
    for (int l = 0; l < h.n_layer; l++) {
        const Layer &L = m->layers[l];
        vec(layer_name(l, "attn_norm"), L.attn_norm);
        mat(layer_name(l, "attn_q"), DEC_T_WQ, l, d, qd);
        mat(layer_name(l, "attn_k"), DEC_T_WK, l, d, kd);
        mat(layer_name(l, "attn_v"), DEC_T_WV, l, d, kd);
        mat(layer_name(l, "attn_output"), DEC_T_WO, l, qd, d);
        vec(layer_name(l, "ffn_norm"), L.ffn_norm);
        mat(layer_name(l, "ffn_gate"), DEC_T_FFN_GATE, l, d, ff);
        mat(layer_name(l, "ffn_up"), DEC_T_FFN_UP, l, d, ff);
        mat(layer_name(l, "ffn_down"), DEC_T_FFN_DOWN, l, ff, d);
    }
    if (hipStreamSynchronize(m->stream) != hipSuccess) return -3;
    const int st = gguf::write(path, kv, ts, 32);
    if (st != gguf::OK) {
        LOGE("dec_model_save_gguf: writing %s failed (status %d)", path, st);
        return -3;
    }
    return 0;
}

// --------------------------------------------------------------- context
struct dec_ctx {
    dec_model *m = nullptr;
    dec_ctx_params p{};
    hipStream_t s = nullptr;
    bool own_stream = false;
    int n_ctx = 0, n_batch = 0, n_ubatch = 0, n_seq = 0, Tmax = 0, step_cap = 0, n_out_cap = 0;
    int step_stride = 0;       // n of the staged call: ids at [0,n), positions [n,2n), sequences [2n,3n)
    Mem mem;
    std::vector<KVLayer> kv;
    float *rope_cs = nullptr;
    float *x = nullptr, *q = nullptr, *part = nullptr, *ml = nullptr, *logits = nullptr;
    float *ssp = nullptr;   // [Tmax][SS_SLOTS] partial sums of squares of the rows of x
    float *gws = nullptr;      // K-split partial tiles of the ubatch GEMMs
    size_t gws_bytes = 0;
    uint16_t *qh = nullptr, *ql = nullptr;   // q / sqrt(hd) as f16 value + remainder
    uint16_t *xn = nullptr, *xn_lo = nullptr, *o = nullptr, *h = nullptr, *o_lo = nullptr,
             *h_lo = nullptr;
    int32_t *amax = nullptr, *dev_step = nullptr, *host_step = nullptr;
    int chunk = 0, max_chunks = 0;
    hipEvent_t staged = nullptr;
    bool staged_pending = false;
    std::vector<int> pos_max;
    int n_out = 0;
    std::vector<float> host_logits;
    bool logits_fetched = false;
    std::vector<int32_t> host_amax;
    bool amax_fetched = false;
    std::map<int, hipGraphExec_t> graphs;
    std::map<int, int> seen;   // decode steps run per token count (capture from the second on)
    bool use_graphs = true;
    bool prefill_mode = false; // run_tokens is running one sequence's consecutive positions
    int prefill_p0 = 0;        // ... starting at this position
    bool flash_prefill = true; // DECODE_PREFILL_ATTN=splitk selects the split-K kernel instead
    // Prefill lanes: consecutive ubatches of a prefill call go round
    // n_lanes sets of activation buffers, each with its own stream, so that
    // one ubatch's kernels fill the compute units another's leave idle.  Lane
    // 0 is the context's own buffers and stream (the fields above while no
    // prefill runs); ubatch u+1 attends to ubatch u's keys, so its attention
    // at layer l waits for u's K/V of layer l (kv_ev of u's lane).
    struct Lane {
        hipStream_t s = nullptr;
        float *x = nullptr, *q = nullptr, *part = nullptr, *ml = nullptr, *ssp = nullptr, *gws = nullptr;
        float *kv_stage = nullptr;       // Q8_0 cache: f32 rows of the ubatch's new K / V, coded after QKV
        uint16_t *qh = nullptr, *ql = nullptr, *xn = nullptr, *xn_lo = nullptr, *o = nullptr, *o_lo = nullptr,
                 *h = nullptr, *h_lo = nullptr;
        std::vector<hipEvent_t> kv_ev;   // per layer: this lane's K/V of the layer are in the cache
        hipEvent_t done = nullptr;       // recorded when a lane hands over to the other
    };
    static constexpr int MAX_LANES = 4;
    Lane lanes[MAX_LANES];
    int n_lanes = 1;           // lanes allocated (more than 1: multi-ubatch prefill on an f16 / f32 cache)
    int lane_cur = 0;          // lane whose buffers the fields above hold
    float *kv_stage = nullptr; // the current lane's Q8_0 staging rows (null: f16 / f32 cache)
    int lane_wait = -1;        // lane whose K/V events the running ubatch's attention waits for
                               // (-1: lanes unused; -2: the call's first ubatch, which only records)
    bool registered = false;   // counted in m->n_ctx_refs
    dec_stats st{};
    // timing probe: a pool of event pairs, each stamped by the kernels of one
    // probed unit launched directly on the stream (hipExtLaunchKernel)
    static constexpr int NPROBE = 64;
    int pr_role = -1, pr_layer = -1;
    hipEvent_t pr_e0[NPROBE] = {}, pr_e1[NPROBE] = {};
    int pr_used = 0;
    double pr_ms = 0.0;
    int64_t pr_n = 0;
    // A probed decode step runs as graph(before the probed kernel), the probed
    // kernel launched directly with its timing events, graph(after): HIP
    // cannot time events that were captured into a graph.  seg_req selects which
    // launches run_tokens emits; seg_cur tracks where the sequence is.
    int seg_req = 0, seg_cur = 1;
    std::map<int, hipGraphExec_t> graphs_post;
    // one-token decode steps as one persistent kernel (dec_set_step_kernel)
    bool step_ok = false, step_on = false;
    int step_grid = 0;
    StepArgs *step_args = nullptr;     // argument block (device memory)
    uint32_t *step_sync = nullptr;     // its barrier memory
    uint32_t step_n0 = 0;              // grid barriers of earlier launches
    bool step_ran = false;             // the last decode call ran the step kernel
    bool step_unchecked = false;       // ... and its failure word has not been read yet
    int step_seq = -1;                 // the sequence that step advanced
};

thread_local LaunchProbe g_launch_probe;

static int step_settle(dec_ctx *c);

// Points the context's buffer fields and stream at lane k.
static void use_lane(dec_ctx *c, int k) {
    const dec_ctx::Lane &L = c->lanes[k];
    c->s = L.s;
    c->x = L.x;
    c->q = L.q;
    c->part = L.part;
    c->ml = L.ml;
    c->ssp = L.ssp;
    c->gws = L.gws;
    c->qh = L.qh;
    c->ql = L.ql;
    c->xn = L.xn;
    c->xn_lo = L.xn_lo;
    c->o = L.o;
    c->o_lo = L.o_lo;
    c->h = L.h;
    c->h_lo = L.h_lo;
    c->kv_stage = L.kv_stage;
    c->lane_cur = k;
}

// The lane's view of the fields (lane 0 taken from the context at creation).
static void save_lane(dec_ctx *c, int k) {
    dec_ctx::Lane &L = c->lanes[k];
    L.s = c->s;
    L.x = c->x;
    L.q = c->q;
    L.part = c->part;
    L.ml = c->ml;
    L.ssp = c->ssp;
    L.gws = c->gws;
    L.qh = c->qh;
    L.ql = c->ql;
    L.xn = c->xn;
    L.xn_lo = c->xn_lo;
    L.o = c->o;
    L.o_lo = c->o_lo;
    L.h = c->h;
    L.h_lo = c->h_lo;
    L.kv_stage = c->kv_stage;
}

enum { SEG_ALL = 0, SEG_PRE = 1, SEG_MID = 2, SEG_POST = 3 };
static bool emit(const dec_ctx *c) { return c->seg_req == SEG_ALL || c->seg_req == c->seg_cur; }

static void drop_graphs(dec_ctx *c) {
    for (auto &g : c->graphs) (void)hipGraphExecDestroy(g.second);
    for (auto &g : c->graphs_post) (void)hipGraphExecDestroy(g.second);
    c->graphs.clear();
    c->graphs_post.clear();
}

static void probe_add(dec_ctx *c, hipEvent_t a, hipEvent_t b) {
    if (hipEventSynchronize(b) != hipSuccess) {
        (void)hipGetLastError();
        return;
    }
    float ms = 0.f;
    if (hipEventElapsedTime(&ms, a, b) == hipSuccess) {
        c->pr_ms += ms;
        c->pr_n++;
    } else {
        (void)hipGetLastError();
    }
}

// Adds every recorded interval to the totals (waits for their end events).
static void probe_collect(dec_ctx *c) {
    for (int i = 0; i < c->pr_used; i++) probe_add(c, c->pr_e0[i], c->pr_e1[i]);
    c->pr_used = 0;
}

static bool probe_hit(const dec_ctx *c, int role, int layer) {
    return c->pr_role == role && (role == DEC_K_OUTPUT || c->pr_layer == layer);
}

static void probe_begin(dec_ctx *c, int role, int layer) {
    if (!probe_hit(c, role, layer)) return;
    c->seg_cur = SEG_MID;
    if (!emit(c)) return;
    if (c->pr_used == dec_ctx::NPROBE) probe_collect(c);
    g_launch_probe.e0 = c->pr_e0[c->pr_used];
    g_launch_probe.e1 = c->pr_e1[c->pr_used];
    g_launch_probe.armed = true;
}

static void probe_end(dec_ctx *c, int role, int layer) {
    if (!probe_hit(c, role, layer)) return;
    if (emit(c)) {
        g_launch_probe = LaunchProbe{};
        c->pr_used++;
    }
    c->seg_cur = SEG_POST;
}

// Prepares the one-token step kernel when the shapes allow it: the layer
// table and argument block in device memory, the barrier memory zeroed.
static void step_setup(dec_ctx *c) {
    const dec_model *m = c->m;
    const dec_hparams &h = m->hp;
    int dev = 0, ncu = 0, coop = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        hipDeviceGetAttribute(&coop, hipDeviceAttributeCooperativeLaunch, dev) != hipSuccess) {
        (void)hipGetLastError();
        return;
    }
    const int grid = ncu;
    StepArgs a;
    a.n_layer = h.n_layer;
    a.tok = m->tok;
    a.out = m->out;
    a.out_norm = m->out_norm;
    a.d = h.n_embd;
    a.qd = m->qd;
    a.kd = m->kd;
    a.Fp = m->Fp;
    a.H = h.n_head;
    a.Hkv = h.n_head_kv;
    a.hd = h.head_dim;
    a.V = h.n_vocab;
    a.n_ctx = c->n_ctx;
    a.eps = h.rms_eps;
    a.qscale = 1.0f / sqrtf((float)h.head_dim);
    a.bpg = a.Hkv > 0 ? std::min(grid / a.Hkv, STEP_BPG_MAX) : 0;
    a.S_qkv = step_slices(a.qd + 2 * a.kd, a.d, grid);
    a.S_o = step_slices(a.d, a.qd, grid);
    a.S_gu = step_slices(2 * a.Fp, a.d, grid);
    a.S_down = step_slices(a.d, a.Fp, grid);
    a.S_out = step_slices(a.V, a.d, grid);
    const char *why = nullptr;
    if (!coop) why = "no cooperative launch";
    else if (!step_supported(a, h.wtype, h.kvtype, grid, &why)) {
    } else if (step_blocks_per_cu(h.wtype, h.head_dim) < 1) why = "kernel does not fit a compute unit";
    if (why) {
        LOGI("one-token step kernel not used: %s", why);
        return;
    }
    std::vector<StepLayer> layers(h.n_layer);
    for (int l = 0; l < h.n_layer; l++) {
        const Layer &L = m->layers[l];
        StepLayer &S = layers[l];
        S.wqkv = L.wqkv;
        S.wo = L.wo;
        S.wgu = L.wgu;
        S.wdown = L.wdown;
        S.attn_norm = L.attn_norm;
        S.ffn_norm = L.ffn_norm;
        S.k = (uint16_t *)c->kv[l].k;
        S.v = (uint16_t *)c->kv[l].v;
    }
    StepLayer *dl = (StepLayer *)c->mem.get(layers.size() * sizeof(StepLayer));
    c->step_args = (StepArgs *)c->mem.get(sizeof(StepArgs));
    c->step_sync = (uint32_t *)c->mem.get(STEP_SYNC_WORDS * 4);
    a.apart = (float *)c->mem.get((size_t)a.H * a.bpg * a.hd * 4);
    a.aml = (float *)c->mem.get((size_t)a.H * a.bpg * 2 * 4);
    a.bmax = (float *)c->mem.get((size_t)grid * 4);
    a.bidx = (int32_t *)c->mem.get((size_t)grid * 4);
    if (!dl || !c->step_args || !c->step_sync || !a.apart || !a.aml || !a.bmax || !a.bidx) return;
    a.layers = dl;
    a.step = c->dev_step;
    a.rope_cs = c->rope_cs;
    a.x = c->x;
    a.ss = c->ssp;
    a.qh = c->qh;
    a.ql = c->ql;
    a.o = c->o;
    a.o_lo = c->o_lo;
    a.h = c->h;
    a.h_lo = c->h_lo;
    a.logits = c->logits;
    a.amax = c->amax;
    a.sync = c->step_sync;
    if (hipMemcpy(dl, layers.data(), layers.size() * sizeof(StepLayer), hipMemcpyHostToDevice) != hipSuccess ||
        hipMemcpy(c->step_args, &a, sizeof(StepArgs), hipMemcpyHostToDevice) != hipSuccess ||
        hipMemset(c->step_sync, 0, STEP_SYNC_WORDS * 4) != hipSuccess) {
        (void)hipGetLastError();
        return;
    }
    c->step_grid = grid;
    c->step_n0 = 0;
    c->step_ok = true;
    // off unless asked for: on one MI355X the per-layer graph is faster (the
    // step's 5 grid barriers per layer cost more than the kernel boundaries)
    const char *e = getenv("DECODE_STEP_KERNEL");
    c->step_on = e && strcmp(e, "1") == 0;
}

extern "C" dec_ctx *dec_ctx_new(dec_model *m, const dec_ctx_params *pp) {
    if (!m || !pp) return nullptr;
    dec_ctx_params p = *pp;
    if (p.kv_unified) {
        LOGE("dec_ctx_new: only one cache stream per sequence is supported (kv_unified = 0)");
        return nullptr;
    }
    dec_ctx *c = new dec_ctx();
    c->m = m;
    c->p = p;
    c->mem.a = m->mem.a;
    c->mem.custom = m->mem.custom;
    const dec_hparams &h = m->hp;
    uint32_t n_ctx = p.n_ctx ? p.n_ctx : 4096;
    n_ctx = (n_ctx + 255) / 256 * 256;
    uint32_t n_batch = p.n_batch ? p.n_batch : n_ctx;
    if (n_batch > n_ctx) n_batch = n_ctx;
    uint32_t n_ubatch = p.n_ubatch ? p.n_ubatch : 512;
    if (n_ubatch > n_batch) n_ubatch = n_batch;
    const uint32_t n_seq = p.n_seq_max ? p.n_seq_max : 1;
    if (n_seq > 256) {
        delete c;
        return nullptr;
    }
    // split-K attention keeps at most 1024 chunks of a row's positions
    if (n_ctx > (uint32_t)DEC_MAX_CTX) {
        LOGE("dec_ctx_new: n_ctx %u above the supported %d positions", n_ctx, DEC_MAX_CTX);
        delete c;
        return nullptr;
    }
    c->n_ctx = (int)n_ctx;
    c->n_batch = (int)n_batch;
    c->n_ubatch = (int)n_ubatch;
    c->n_seq = (int)n_seq;
    c->Tmax = (int)(n_ubatch > n_seq ? n_ubatch : n_seq);
    c->step_cap = (int)(n_batch > n_seq ? n_batch : n_seq);
    c->n_out_cap = c->step_cap;
    c->pos_max.assign(n_seq, -1);
    if (const char *e = getenv("DECODE_PREFILL_ATTN")) c->flash_prefill = strcmp(e, "splitk") != 0;
    {
        int dev = 0, ncu = 0;
        if (hipGetDevice(&dev) == hipSuccess &&
            hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess) {
            matvec_set_num_cu(ncu);
            gemm_set_num_cu(ncu);
        }
    }
    if (p.hip_stream) {
        c->s = (hipStream_t)p.hip_stream;
    } else {
        HIP_OK(hipStreamCreateWithFlags(&c->s, hipStreamNonBlocking), delete c; return nullptr);
        c->own_stream = true;
    }
    const int d = h.n_embd, qd = m->qd, Fp = m->Fp, V = h.n_vocab, hd = h.head_dim;
    // Q8_0: one int8 code per element plus one f16 scale per 32 elements, and
    // f32 staging rows for the new K / V of a ubatch (shared by the layers)
    const bool q8 = h.kvtype == DEC_Q8_0;
    const size_t esz = h.kvtype == DEC_F32 ? 4 : q8 ? 1 : 2;
    const size_t kv_elems = (size_t)n_seq * h.n_head_kv * n_ctx * hd;
    float *kv_stage = q8 ? (float *)c->mem.get((size_t)c->Tmax * 2 * m->kd * 4) : nullptr;
    bool ok = !q8 || kv_stage;
    c->kv_stage = kv_stage;
    c->kv.resize(h.n_layer);
    for (int l = 0; ok && l < h.n_layer; l++) {
        KVLayer &L = c->kv[l];
        L.kvtype = h.kvtype;
        L.n_ctx = (int)n_ctx;
        L.n_kv = h.n_head_kv;
        L.hd = hd;
        L.k = c->mem.get(kv_elems * esz);
        L.v = c->mem.get(kv_elems * esz);
        ok = L.k && L.v;
        if (ok && q8) {
            L.k_scale = (uint16_t *)c->mem.get(kv_elems / 32 * 2);
            L.v_scale = (uint16_t *)c->mem.get(kv_elems / 32 * 2);
            L.stage = kv_stage;
            ok = L.k_scale && L.v_scale;
        }
    }
    c->chunk = attention_chunk(h.kvtype, hd);
    c->max_chunks = (int)((n_ctx + c->chunk - 1) / c->chunk);
    const size_t T = (size_t)c->Tmax;
    if (ok) {
        c->rope_cs = (float *)c->mem.get((size_t)n_ctx * hd * 4);
        c->x = (float *)c->mem.get(T * d * 4);
        c->xn = (uint16_t *)c->mem.get(T * d * 2);
        c->xn_lo = (uint16_t *)c->mem.get(T * d * 2);
        c->ssp = (float *)c->mem.get(T * SS_SLOTS * 4);
        c->q = (float *)c->mem.get(T * qd * 4);
        c->qh = (uint16_t *)c->mem.get(T * qd * 2);
        c->ql = (uint16_t *)c->mem.get(T * qd * 2);
        c->o = (uint16_t *)c->mem.get(T * qd * 2);
        c->h = (uint16_t *)c->mem.get(T * Fp * 2);
        c->o_lo = (uint16_t *)c->mem.get(T * qd * 2);
        c->h_lo = (uint16_t *)c->mem.get(T * Fp * 2);
        c->part = (float *)c->mem.get(T * h.n_head * c->max_chunks * hd * 4);
        c->ml = (float *)c->mem.get(T * h.n_head * c->max_chunks * 2 * 4);
        // K-split partial tiles of the ubatch GEMMs (the largest any matrix uses)
        size_t ws = 0;
        for (const Layer &L : m->layers)
            for (const QMat *w : {&L.wqkv, &L.wo, &L.wgu, &L.wdown}) ws = std::max(ws, gemm_workspace_bytes(*w, (int)T));
        ws = std::max(ws, gemm_workspace_bytes(m->out, (int)T));
        c->gws_bytes = ws;
        c->gws = ws ? (float *)c->mem.get(ws) : nullptr;
        c->logits = (float *)c->mem.get((size_t)c->n_out_cap * V * 4);
        c->amax = (int32_t *)c->mem.get((size_t)c->n_out_cap * 4);
        c->dev_step = (int32_t *)c->mem.get((size_t)c->step_cap * 3 * 4);
        ok = c->rope_cs && c->x && c->ssp && c->xn && c->xn_lo && c->q && c->qh && c->ql && c->o && c->h && c->o_lo && c->h_lo && c->part && c->ml && c->logits &&
             (c->gws || !c->gws_bytes) &&
             c->amax && c->dev_step;
    }
    if (ok) save_lane(c, 0);
    // lanes 1.. (prefill calls of several ubatches; a Q8_0 cache gives each
    // lane its own staging rows); DECODE_PREFILL_LANES = 1..4 lanes, default 2
    int want = 2;
    if (const char *lv = getenv("DECODE_PREFILL_LANES")) {
        const int v = atoi(lv);
        want = v < 1 ? 1 : v > dec_ctx::MAX_LANES ? dec_ctx::MAX_LANES : v;
    }
    if (ok && n_batch > n_ubatch && want > 1) {
        bool lok = true;
        int k = 1;
        for (; lok && k < want; k++) {
            dec_ctx::Lane &L = c->lanes[k];
            const size_t Tu = (size_t)n_ubatch;
            L.x = (float *)c->mem.get(Tu * d * 4);
            L.xn = (uint16_t *)c->mem.get(Tu * d * 2);
            L.xn_lo = (uint16_t *)c->mem.get(Tu * d * 2);
            L.ssp = (float *)c->mem.get(Tu * SS_SLOTS * 4);
            L.q = (float *)c->mem.get(Tu * qd * 4);
            L.qh = (uint16_t *)c->mem.get(Tu * qd * 2);
            L.ql = (uint16_t *)c->mem.get(Tu * qd * 2);
            L.o = (uint16_t *)c->mem.get(Tu * qd * 2);
            L.o_lo = (uint16_t *)c->mem.get(Tu * qd * 2);
            L.h = (uint16_t *)c->mem.get(Tu * Fp * 2);
            L.h_lo = (uint16_t *)c->mem.get(Tu * Fp * 2);
            L.part = (float *)c->mem.get(Tu * h.n_head * c->max_chunks * hd * 4);
            L.ml = (float *)c->mem.get(Tu * h.n_head * c->max_chunks * 2 * 4);
            L.gws = c->gws_bytes ? (float *)c->mem.get(c->gws_bytes) : nullptr;
            L.kv_stage = q8 ? (float *)c->mem.get(Tu * 2 * m->kd * 4) : nullptr;
            lok = L.x && L.xn && L.xn_lo && L.ssp && L.q && L.qh && L.ql && L.o && L.o_lo && L.h && L.h_lo &&
                  L.part && L.ml && (L.gws || !c->gws_bytes) && (L.kv_stage || !q8);
            if (lok) HIP_OK(hipStreamCreateWithFlags(&L.s, hipStreamNonBlocking), lok = false);
        }
        const int nl = lok ? want : k - 1;               // lanes whose buffers and stream exist
        for (int j = 0; lok && j < nl; j++) {
            dec_ctx::Lane &L = c->lanes[j];
            L.kv_ev.assign(h.n_layer, nullptr);
            for (int l = 0; lok && l < h.n_layer; l++)
                HIP_OK(hipEventCreateWithFlags(&L.kv_ev[l], hipEventDisableTiming), lok = false);
            if (lok) HIP_OK(hipEventCreateWithFlags(&L.done, hipEventDisableTiming), lok = false);
        }
        c->n_lanes = lok ? want : 1;
        if (!lok) LOGW("dec_ctx_new: no second prefill lane; ubatches run one after another");
    }
    if (ok) HIP_OK(hipHostMalloc((void **)&c->host_step, (size_t)c->step_cap * 3 * 4, 0), ok = false);
    if (ok) HIP_OK(hipEventCreateWithFlags(&c->staged, hipEventDisableTiming), ok = false);
    for (int i = 0; ok && i < dec_ctx::NPROBE; i++) {
        HIP_OK(hipEventCreate(&c->pr_e0[i]), ok = false);
        if (ok) HIP_OK(hipEventCreate(&c->pr_e1[i]), ok = false);
    }

    if (ok) step_setup(c);
    if (ok) {
        launch_rope_table(c->rope_cs, (int)n_ctx, hd, h.rope_base, c->s);
        HIP_OK(hipGetLastError(), ok = false);
    }
    if (ok) HIP_OK(hipStreamSynchronize(c->s), ok = false);
    if (!ok) {
        LOGE("dec_ctx_new failed");
        dec_ctx_free(c);
        return nullptr;
    }
    m->n_ctx_refs++;
    c->registered = true;
    LOGI("context: n_ctx=%u n_batch=%u n_ubatch=%u n_seq=%u", n_ctx, n_batch, n_ubatch, n_seq);
    return c;
}

extern "C" void dec_ctx_free(dec_ctx *c) {
    if (!c) return;
    if (c->s) (void)hipStreamSynchronize(c->s);
    drop_graphs(c);
    if (c->staged) (void)hipEventDestroy(c->staged);
    for (int i = 0; i < dec_ctx::NPROBE; i++) {
        if (c->pr_e0[i]) (void)hipEventDestroy(c->pr_e0[i]);
        if (c->pr_e1[i]) (void)hipEventDestroy(c->pr_e1[i]);
    }

    for (int k = 1; k < dec_ctx::MAX_LANES; k++)
        if (c->lanes[k].s) (void)hipStreamSynchronize(c->lanes[k].s);
    for (dec_ctx::Lane &L : c->lanes) {
        for (hipEvent_t e : L.kv_ev)
            if (e) (void)hipEventDestroy(e);
        if (L.done) (void)hipEventDestroy(L.done);
    }
    for (int k = 1; k < dec_ctx::MAX_LANES; k++)
        if (c->lanes[k].s) (void)hipStreamDestroy(c->lanes[k].s);
    if (c->host_step) (void)hipHostFree(c->host_step);
    c->mem.release();
    if (c->own_stream) (void)hipStreamDestroy(c->s);
    dec_model *m = c->registered ? c->m : nullptr;
    delete c;
    if (m && --m->n_ctx_refs == 0 && m->free_requested) model_release(m);
}

// Waits until the pinned staging buffer may be rewritten.
static bool wait_staging(dec_ctx *c) {
    if (c->staged_pending) {
        HIP_OK(hipEventSynchronize(c->staged), return false);
        c->staged_pending = false;
    }
    return true;
}

// Copies the call's token ids, positions and sequence ids ([3][n] int32,
// packed at the start of the pinned staging buffer) to the device in one copy.
static bool stage_step(dec_ctx *c, int n) {
    c->step_stride = n;
    HIP_OK(hipMemcpyAsync(c->dev_step, c->host_step, (size_t)n * 3 * 4, hipMemcpyHostToDevice, c->s),
           return false);
    HIP_OK(hipEventRecord(c->staged, c->s), return false);
    c->staged_pending = true;
    return true;
}

// Whether a call with T tokens uses the mat-vec kernels (decode-sized).
static bool use_matvec(const dec_ctx *c, int T) {
    return c->m->hp.wtype != DEC_F32 && T <= 2;
}

// One unit of work (kernel role `role` of layer `layer`, or role -1 for
// units the probe never selects): emitted only when its segment is requested.
template <typename F>
static bool stage(dec_ctx *c, int role, int layer, F &&f) {
    probe_begin(c, role, layer);
    bool ok = true;
    if (emit(c)) {
        ok = f();
        const hipError_t e = hipGetLastError();
        if (!ok || e != hipSuccess) {
            LOGE("launch of kernel role %d, layer %d failed: %s", role, layer,
                 ok ? hipGetErrorString(e) : "shape not supported");
            ok = false;
        }
    }
    probe_end(c, role, layer);
    return ok;
}

// Enqueues the layers for T tokens whose ids / positions / sequences live at
// dev_step + off (+n, +2n for the n tokens of the staged call).  Output rows: `n_rows` rows starting at
// token row `row0` produce logits at logits row `out_row0`.
static bool run_tokens(dec_ctx *c, int off, int T, int row0, int n_rows, int out_row0) {
    dec_model *m = c->m;
    const dec_hparams &h = m->hp;
    const int d = h.n_embd, qd = m->qd, Fp = m->Fp, V = h.n_vocab;
    const size_t stride = (size_t)c->step_stride;
    const int32_t *tok = c->dev_step + off;
    TokInfo ti;
    ti.pos = c->dev_step + stride + off;
    ti.seq = c->dev_step + 2 * stride + off;
    hipStream_t s = c->s;
    const bool mv = use_matvec(c, T);
    bool ok = true;
    c->seg_cur = SEG_PRE;

    ok = stage(c, -1, -1, [&] {
        launch_embed(m->tok, tok, T, c->x, d, c->ssp, s);
        return true;
    });
    // set where a K-split sum also wrote the next RMSNorm's output (the flags
    // are per emission: a unit not emitted here leaves them 0, and the norm
    // is then launched on its own)
    int attn_normed = 0;
    for (int l = 0; ok && l < h.n_layer; l++) {
        const Layer &L = m->layers[l];
        EpiArgs eq;
        eq.epi = EPI_QKV;
        eq.qout = c->q;
        eq.qh = c->qh;
        eq.ql = c->ql;
        eq.qscale = 1.0f / sqrtf((float)h.head_dim);
        eq.qd = qd;
        eq.kd = m->kd;
        eq.kv = c->kv[l];
        if (c->kv_stage) eq.kv.stage = c->kv_stage;      // this lane's staging rows
        eq.tok = ti;
        eq.rope_cs = c->rope_cs;
        ok = ok && stage(c, DEC_K_QKV, l, [&] {
            if (mv) {
                InArgs in;
                in.x32 = c->x;
                in.norm_g = L.attn_norm;
                in.ss_part = c->ssp;
                in.eps = h.rms_eps;
                in.ldx = d;
                return launch_matvec(L.wqkv, in, eq, T, s);
            }
            // (skipped where the previous down projection's K-split sum wrote it)
            if (!attn_normed) launch_rmsnorm(c->x, d, L.attn_norm, d, h.rms_eps, nullptr, T, c->xn, c->xn_lo, d, s);
            return launch_gemm(L.wqkv, c->xn, c->xn_lo, d, eq, T, c->gws, c->gws_bytes, s);
        });
        // Q8_0 cache: a decode call's tokens are of distinct sequences, so the
        // attention block holding each new row codes it; a prefill ubatch's
        // later tokens read earlier ones' rows, so they are coded first
        const bool code_in_attn = h.kvtype == DEC_Q8_0 && !c->prefill_mode &&
                                  attention_codes_rows(h.kvtype, h.head_dim);
        if (h.kvtype == DEC_Q8_0 && !code_in_attn)
            ok = ok && stage(c, -1, l, [&] {
                KVLayer kq = c->kv[l];
                kq.stage = c->kv_stage;
                launch_kv_quant(kq, ti, T, s);
                return true;
            });
        // prefill lanes: this ubatch's K/V of layer l are in the cache; the
        // previous ubatch's must be before this one attends
        if (ok && c->lane_wait >= 0) {
            HIP_OK(hipEventRecord(c->lanes[c->lane_cur].kv_ev[l], s), ok = false);
            if (ok) HIP_OK(hipStreamWaitEvent(s, c->lanes[c->lane_wait].kv_ev[l], 0), ok = false);
        } else if (ok && c->lane_wait == -2) {
            HIP_OK(hipEventRecord(c->lanes[c->lane_cur].kv_ev[l], s), ok = false);
        }
        AttnArgs at;
        at.q = c->q;
        at.qh = c->qh;
        at.ql = c->ql;
        at.kv = c->kv[l];
        if (c->kv_stage) at.kv.stage = c->kv_stage;
        at.tok = ti;
        at.H = h.n_head;
        at.part = c->part;
        at.ml = c->ml;
        at.max_chunks = c->max_chunks;
        at.chunk = c->chunk;
        at.o = c->o;
        at.o_lo = c->o_lo;
        at.code_new_rows = code_in_attn ? 1 : 0;
        ok = ok && stage(c, DEC_K_ATTN, l, [&] {
            if (c->prefill_mode && c->flash_prefill && T > 1) {
                FlashArgs fa;
                fa.q = c->q;
                fa.kv = c->kv[l];
                fa.tok = ti;
                fa.H = h.n_head;
                fa.T = T;
                fa.o = c->o;
                fa.o_lo = c->o_lo;
                fa.part = c->part;
                fa.ml = c->ml;
                fa.max_chunks = c->max_chunks;
                fa.tok_pos0_max = c->prefill_p0;
                if (launch_flash_prefill(fa, s)) return true;
            }
            return launch_attention(at, T, s);
        });

        EpiArgs er;
        er.epi = EPI_RESID;
        er.y = c->x;
        er.ldy = d;
        er.ss_out = c->ssp;
        // a K-split sum ending the O projection also writes the FFN norm's input
        int ffn_normed = 0;
        er.nrm_g = L.ffn_norm;
        er.nrm_eps = h.rms_eps;
        er.nrm_h = c->xn;
        er.nrm_l = c->xn_lo;
        er.nrm_ld = d;
        er.nrm_done = &ffn_normed;
        ok = ok && stage(c, DEC_K_WO, l, [&] {
            if (mv) {
                InArgs in;
                in.x16 = c->o;
                in.x16lo = c->o_lo;
                in.ldx = qd;
                return launch_matvec(L.wo, in, er, T, s);
            }
            return launch_gemm(L.wo, c->o, c->o_lo, qd, er, T, c->gws, c->gws_bytes, s);
        });
        EpiArgs eg;
        eg.epi = EPI_SWIGLU;
        eg.h = c->h;
        eg.h_lo = c->h_lo;
        eg.ldh = Fp;
        ok = ok && stage(c, DEC_K_FFN_GU, l, [&] {
            if (mv) {
                InArgs in;
                in.x32 = c->x;
                in.norm_g = L.ffn_norm;
                in.ss_part = c->ssp;
                in.eps = h.rms_eps;
                in.ldx = d;
                return launch_matvec(L.wgu, in, eg, T, s);
            }
            if (!ffn_normed) launch_rmsnorm(c->x, d, L.ffn_norm, d, h.rms_eps, nullptr, T, c->xn, c->xn_lo, d, s);
            return launch_gemm(L.wgu, c->xn, c->xn_lo, d, eg, T, c->gws, c->gws_bytes, s);
        });
        // and one ending the down projection, the next layer's attention norm input
        attn_normed = 0;
        if (l + 1 < h.n_layer) {
            er.nrm_g = m->layers[l + 1].attn_norm;
            er.nrm_done = &attn_normed;
        } else {
            er.nrm_g = nullptr;
            er.nrm_done = nullptr;
        }
        ok = ok && stage(c, DEC_K_FFN_DOWN, l, [&] {
            if (mv) {
                InArgs in;
                in.x16 = c->h;
                in.x16lo = c->h_lo;
                in.ldx = Fp;
                return launch_matvec(L.wdown, in, er, T, s);
            }
            return launch_gemm(L.wdown, c->h, c->h_lo, Fp, er, T, c->gws, c->gws_bytes, s);
        });
    }
    if (ok && n_rows > 0) {
        EpiArgs eo;
        eo.epi = EPI_STORE;
        eo.y = c->logits + (size_t)out_row0 * V;
        eo.ldy = V;
        ok = stage(c, DEC_K_OUTPUT, -1, [&] {
            if (use_matvec(c, n_rows)) {
                InArgs in;
                in.x32 = c->x + (size_t)row0 * d;
                in.norm_g = m->out_norm;
                // the layers' residual adds left the sums of squares only when
                // they ran as mat-vecs
                in.ss_part = mv ? c->ssp + (size_t)row0 * SS_SLOTS : nullptr;
                in.eps = h.rms_eps;
                in.ldx = d;
                return launch_matvec(m->out, in, eo, n_rows, s);
            }
            launch_rmsnorm(c->x + (size_t)row0 * d, d, m->out_norm, d, h.rms_eps, nullptr, n_rows, c->xn,
                           c->xn_lo, d, s);
            return launch_gemm(m->out, c->xn, c->xn_lo, d, eo, n_rows, c->gws, c->gws_bytes, s);
        });
        ok = ok && stage(c, -1, -1, [&] {
            launch_argmax(c->logits + (size_t)out_row0 * V, V, n_rows, c->amax + out_row0, s);
            return true;
        });
    }
    if (!ok) LOGE("kernel launch rejected a shape");
    return ok && hipGetLastError() == hipSuccess;
}

static void reset_outputs(dec_ctx *c, int n_out) {
    c->n_out = n_out;
    c->logits_fetched = false;
    c->amax_fetched = false;
}

extern "C" int32_t dec_prefill(dec_ctx *c, const int32_t *tokens, int32_t n, int32_t seq,
                               int32_t output_all) {
    if (!c || !tokens || n <= 0 || n > c->n_batch || seq < 0 || seq >= c->n_seq) return -1;
    if (step_settle(c) != 0) return -3;
    const int V = c->m->hp.n_vocab;
    for (int i = 0; i < n; i++)
        if (tokens[i] < 0 || tokens[i] >= V) {
            LOGE("dec_prefill: token %d at %d out of range", tokens[i], i);
            return -1;
        }
    const int p0 = c->pos_max[seq] + 1;
    if (p0 + n > c->n_ctx) {
        LOGW("dec_prefill: %d tokens do not fit (sequence at %d, n_ctx %d)", n, p0, c->n_ctx);
        return 1;   // cells are reserved for the whole batch up front: nothing changes
    }
    if (!wait_staging(c)) return -3;
    for (int i = 0; i < n; i++) {
        c->host_step[i] = tokens[i];
        c->host_step[n + i] = p0 + i;
        c->host_step[2 * n + i] = seq;
    }
    if (!stage_step(c, n)) return -3;
    c->st.n_prefill_calls++;
    reset_outputs(c, 0);
    // ubatches go round the lanes when there are several (and no timing
    // probe is set: a probe times kernels on the context's stream)
    const int n_ub = (n + c->n_ubatch - 1) / c->n_ubatch;
    const int nl = c->pr_role < 0 ? std::min(c->n_lanes, n_ub) : 1;
    if (nl > 1) {
        HIP_OK(hipEventRecord(c->lanes[0].done, c->lanes[0].s), return -3);
        for (int k = 1; k < nl; k++) HIP_OK(hipStreamWaitEvent(c->lanes[k].s, c->lanes[0].done, 0), return -3);
        gemm_set_split_cap(4);    // the other lane fills what a smaller K split leaves idle
    }
    // back to lane 0, whose stream then waits for the other lanes' work
    auto join = [&]() -> bool {
        if (nl == 1) return true;
        use_lane(c, 0);
        c->lane_wait = -1;
        gemm_set_split_cap(8);
        for (int k = 1; k < nl; k++) {
            HIP_OK(hipEventRecord(c->lanes[k].done, c->lanes[k].s), return false);
            HIP_OK(hipStreamWaitEvent(c->lanes[0].s, c->lanes[k].done, 0), return false);
        }
        return true;
    };
    for (int u = 0, ub = 0; u < n; u += c->n_ubatch, ub++) {
        if (u > 0 && c->p.abort_cb && c->p.abort_cb(c->p.abort_ud)) {
            LOGW("dec_prefill: aborted after %d of %d tokens", u, n);
            return join() ? 2 : -3;
        }
        const int T = n - u < c->n_ubatch ? n - u : c->n_ubatch;
        const bool last = u + T == n;
        int row0 = 0, n_rows = 0;
        if (output_all) {
            n_rows = T;
        } else if (last) {
            row0 = T - 1;
            n_rows = 1;
        }
        if (nl > 1) {
            use_lane(c, ub % nl);
            c->lane_wait = ub == 0 ? -2 : (ub - 1) % nl;   // -2: record only
        }
        c->prefill_mode = true;
        c->prefill_p0 = p0 + u;
        const bool ok = run_tokens(c, u, T, row0, n_rows, output_all ? u : 0);
        c->prefill_mode = false;
        if (!ok) {
            (void)join();
            return -3;
        }
        c->pos_max[seq] = p0 + u + T - 1;
        c->st.n_ubatches++;
        reset_outputs(c, output_all ? u + T : (last ? 1 : 0));
    }
    return join() ? 0 : -3;
}

// Captures the decode step for n tokens (segment `seg` of it) as a graph.
static hipGraphExec_t capture_step(dec_ctx *c, int n, int seg) {
    hipGraph_t g = nullptr;
    HIP_OK(hipStreamBeginCapture(c->s, hipStreamCaptureModeThreadLocal), return nullptr);
    c->seg_req = seg;
    const bool ok = run_tokens(c, 0, n, 0, n, 0);
    c->seg_req = SEG_ALL;
    const hipError_t e = hipStreamEndCapture(c->s, &g);
    if (!ok || e != hipSuccess || !g) {
        LOGE("dec_decode: graph capture failed (%s)", hipGetErrorString(e));
        if (g) (void)hipGraphDestroy(g);
        return nullptr;
    }
    hipGraphExec_t ex = nullptr;
    const hipError_t ei = hipGraphInstantiate(&ex, g, nullptr, nullptr, 0);
    (void)hipGraphDestroy(g);
    if (ei != hipSuccess) {
        LOGE("dec_decode: graph instantiate failed (%s)", hipGetErrorString(ei));
        return nullptr;
    }
    return ex;
}

// After a step-kernel launch: reads the kernel's failure word (a bounded
// grid-barrier wait gave up).  On failure the step is undone: its position
// is free again (its cache row holds no valid K / V), its outputs are
// dropped, and the barrier memory is cleared for the next launch.  Returns
// 0, or -3 once for the failed step.
static int step_settle(dec_ctx *c) {
    if (!c->step_unchecked) return 0;
    c->step_unchecked = false;
    uint32_t fail = 0;
    HIP_OK(hipMemcpyAsync(&fail, c->step_sync + STEP_SYNC_FAIL, 4, hipMemcpyDeviceToHost, c->s), return -3);
    HIP_OK(hipStreamSynchronize(c->s), return -3);
    if (!fail) return 0;
    LOGE("decode step kernel: a grid barrier timed out; the step is rolled back");
    if (c->step_seq >= 0 && c->pos_max[c->step_seq] >= 0) c->pos_max[c->step_seq]--;
    c->step_n0 = 0;
    c->step_ran = false;
    reset_outputs(c, 0);
    HIP_OK(hipMemsetAsync(c->step_sync, 0, STEP_SYNC_WORDS * 4, c->s), return -3);
    HIP_OK(hipStreamSynchronize(c->s), return -3);
    return -3;
}

extern "C" int32_t dec_decode(dec_ctx *c, const int32_t *tokens, const int32_t *seq_ids, int32_t n) {
    if (!c || !tokens || !seq_ids || n <= 0 || n > c->n_seq || n > c->Tmax) return -1;
    if (step_settle(c) != 0) return -3;
    const int V = c->m->hp.n_vocab;
    std::vector<char> seen(c->n_seq, 0);
    for (int i = 0; i < n; i++) {
        const int sq = seq_ids[i];
        if (tokens[i] < 0 || tokens[i] >= V || sq < 0 || sq >= c->n_seq || seen[sq]) return -1;
        seen[sq] = 1;
        if (c->pos_max[sq] + 1 >= c->n_ctx) return 1;
    }
    if (!wait_staging(c)) return -3;
    for (int i = 0; i < n; i++) {
        c->host_step[i] = tokens[i];
        c->host_step[n + i] = c->pos_max[seq_ids[i]] + 1;
        c->host_step[2 * n + i] = seq_ids[i];
    }
    if (!stage_step(c, n)) return -3;
    c->step_ran = false;
    if (n == 1 && c->step_on && c->use_graphs && (c->pr_role < 0 || c->pr_role == DEC_K_STEP)) {
        // the whole step as one persistent kernel
        const bool probe = c->pr_role == DEC_K_STEP;
        if (probe) {
            if (c->pr_used == dec_ctx::NPROBE) probe_collect(c);
            HIP_OK(hipEventRecord(c->pr_e0[c->pr_used], c->s), return -3);
        }
        if (!launch_step(c->step_args, c->m->hp.wtype, c->m->hp.head_dim, c->step_n0, c->step_grid, c->s)) {
            LOGE("dec_decode: step kernel launch failed (%s)", hipGetErrorString(hipGetLastError()));
            return -3;
        }
        if (probe) {
            HIP_OK(hipEventRecord(c->pr_e1[c->pr_used], c->s), return -3);
            c->pr_used++;
        }
        c->step_n0 += step_barriers(c->m->hp.n_layer);
        c->step_ran = true;
        c->step_unchecked = true;
        c->step_seq = seq_ids[0];
        c->pos_max[seq_ids[0]]++;
        c->st.n_decode_calls++;
        reset_outputs(c, 1);
        return 0;
    }
    // The first step of a shape runs kernel by kernel: every kernel it uses is
    // then loaded, so the capture of the second step only records launches
    // (graph reuse applies to repeated shapes, as in the article's step 13b).
    if (!c->use_graphs || c->seen[n]++ == 0) {
        c->seg_req = SEG_ALL;
        if (!run_tokens(c, 0, n, 0, n, 0)) return -3;
    } else {
        const bool split = c->pr_role >= 0 && c->pr_role != DEC_K_STEP;
        auto it = c->graphs.find(n);
        if (it == c->graphs.end()) {
            hipGraphExec_t pre = capture_step(c, n, split ? SEG_PRE : SEG_ALL);
            if (!pre) return -3;
            it = c->graphs.emplace(n, pre).first;
            if (split) {
                hipGraphExec_t post = capture_step(c, n, SEG_POST);
                if (!post) {
                    drop_graphs(c);
                    return -3;
                }
                c->graphs_post[n] = post;
            }
            c->st.n_graph_captures++;
        } else {
            c->st.n_graph_replays++;
        }
        HIP_OK(hipGraphLaunch(it->second, c->s), return -3);
        if (split) {
            c->seg_req = SEG_MID;                      // the probed kernel, between its events
            const bool ok = run_tokens(c, 0, n, 0, n, 0);
            c->seg_req = SEG_ALL;
            if (!ok) return -3;
            HIP_OK(hipGraphLaunch(c->graphs_post[n], c->s), return -3);
        }
    }
    for (int i = 0; i < n; i++) c->pos_max[seq_ids[i]]++;
    c->st.n_decode_calls++;
    reset_outputs(c, n);
    return 0;
}

static int resolve_row(const dec_ctx *c, int i) {
    if (c->n_out <= 0) return -1;
    if (i < 0) i += c->n_out;
    if (i < 0 || i >= c->n_out) return -1;
    return i;
}

extern "C" const float *dec_get_logits(dec_ctx *c, int32_t i) {
    if (!c || step_settle(c) != 0) return nullptr;
    const int r = resolve_row(c, i);
    if (r < 0) return nullptr;
    const size_t V = (size_t)c->m->hp.n_vocab;
    if (!c->logits_fetched) {
        if (c->host_logits.size() < (size_t)c->n_out * V) c->host_logits.resize((size_t)c->n_out * V);
        HIP_OK(hipStreamSynchronize(c->s), return nullptr);
        HIP_OK(hipMemcpy(c->host_logits.data(), c->logits, (size_t)c->n_out * V * 4, hipMemcpyDeviceToHost),
               return nullptr);
        c->logits_fetched = true;
    }
    return c->host_logits.data() + (size_t)r * V;
}

static bool fetch_amax(dec_ctx *c) {
    if (step_settle(c) != 0) return false;
    if (c->amax_fetched) return true;
    c->host_amax.resize(c->n_out);
    HIP_OK(hipMemcpyAsync(c->host_amax.data(), c->amax, (size_t)c->n_out * 4, hipMemcpyDeviceToHost, c->s),
           return false);
    HIP_OK(hipStreamSynchronize(c->s), return false);
    c->amax_fetched = true;
    return true;
}

extern "C" int32_t dec_argmax(dec_ctx *c, int32_t i) {
    if (!c || step_settle(c) != 0) return -1;
    const int r = resolve_row(c, i);
    if (r < 0 || !fetch_amax(c)) return -1;
    return c->host_amax[r];
}

extern "C" int32_t dec_argmax_all(dec_ctx *c, int32_t *out, int32_t cap) {
    if (!c || step_settle(c) != 0) return -1;
    if (c->n_out <= 0) return 0;
    if (!out || cap < c->n_out) return -1;
    if (!fetch_amax(c)) return -1;
    memcpy(out, c->host_amax.data(), (size_t)c->n_out * 4);
    return c->n_out;
}

// ---- sampler chain ---------------------------------------------------------
struct dec_sampler {
    dec_sampler_params p{};
    std::vector<int32_t> hist;     // accepted tokens, at most the window kept
    uint64_t draws = 0;
    int32_t *h_buf = nullptr;      // mapped pinned: window [64] + token [1]
    int32_t *g_buf = nullptr;      // device address of h_buf
    float *d_row = nullptr;        // device copy of a host logits row
    size_t row_cap = 0;
    hipStream_t own = nullptr;     // stream for rows given without one
};

extern "C" dec_sampler *dec_sampler_new(const dec_sampler_params *p) {
    if (!p || p->top_k < 1 || p->top_k > 1024 || !(p->top_p > 0.0f && p->top_p <= 1.0f) ||
        !(p->min_p >= 0.0f && p->min_p < 1.0f) || !(p->repeat_penalty >= 1.0f) || p->penalty_last_n < 0 ||
        p->penalty_last_n > 64 || p->temp != p->temp)
        return nullptr;
    dec_sampler *s = new (std::nothrow) dec_sampler;
    if (!s) return nullptr;
    s->p = *p;
    bool ok = true;
    HIP_OK(hipHostMalloc((void **)&s->h_buf, 65 * 4, hipHostMallocMapped), ok = false);
    if (ok) HIP_OK(hipHostGetDevicePointer((void **)&s->g_buf, s->h_buf, 0), ok = false);
    if (ok) HIP_OK(hipStreamCreateWithFlags(&s->own, hipStreamNonBlocking), ok = false);
    if (!ok) {
        dec_sampler_free(s);
        return nullptr;
    }
    return s;
}

extern "C" int32_t dec_sampler_accept(dec_sampler *s, int32_t token) {
    if (!s || token < 0) return -1;
    s->hist.push_back(token);
    if (s->hist.size() > 64) s->hist.erase(s->hist.begin(), s->hist.end() - 64);
    return 0;
}

// Runs the chain on a device logits row on stream st; accepts the token.
static int32_t sampler_run(dec_sampler *s, const float *row, int V, hipStream_t st) {
    SampleArgs a;
    const int w = (int)std::min<size_t>(s->hist.size(), (size_t)s->p.penalty_last_n);
    a.n_hist = s->p.repeat_penalty != 1.0f ? w : 0;
    a.n_vocab = V;
    a.top_k = s->p.top_k;
    a.top_p = s->p.top_p;
    a.min_p = s->p.min_p;
    a.temp = s->p.temp;
    a.repeat_penalty = s->p.repeat_penalty;
    a.seed = s->p.seed;
    a.draw = s->draws;
    // the window and the token travel through mapped pinned memory: the kernel
    // reads the one and writes the other directly, visible at the stream sync
    a.hist = s->g_buf;
    a.out = s->g_buf + 64;
    if (a.n_hist > 0)
        memcpy(s->h_buf, s->hist.data() + (s->hist.size() - a.n_hist), (size_t)a.n_hist * 4);
    s->h_buf[64] = -1;
    if (!launch_sample(row, a, st)) return -1;
    HIP_OK(hipGetLastError(), return -3);
    HIP_OK(hipStreamSynchronize(st), return -3);
    const int32_t tok = s->h_buf[64];
    if (tok < 0 || tok >= V) return -3;
    s->draws++;
    dec_sampler_accept(s, tok);
    return tok;
}

extern "C" int32_t dec_sampler_sample(dec_sampler *s, dec_ctx *c, int32_t i) {
    if (!s || !c) return -1;
    if (step_settle(c) != 0) return -3;
    const int r = resolve_row(c, i);
    if (r < 0) return -1;
    const int V = c->m->hp.n_vocab;
    return sampler_run(s, c->logits + (size_t)r * V, V, c->s);
}

extern "C" int32_t dec_sampler_sample_row(dec_sampler *s, const float *logits, int32_t n_vocab, void *hip_stream) {
    if (!s || !logits || n_vocab <= 0) return -1;
    hipStream_t st = hip_stream ? (hipStream_t)hip_stream : s->own;
    const float *row = logits;
    if (!is_device_ptr(logits)) {
        if (s->row_cap < (size_t)n_vocab) {
            if (s->d_row) (void)hipFree(s->d_row);
            s->d_row = nullptr;
            s->row_cap = 0;
            HIP_OK(hipMalloc((void **)&s->d_row, (size_t)n_vocab * 4), return -3);
            s->row_cap = (size_t)n_vocab;
        }
        HIP_OK(hipMemcpyAsync(s->d_row, logits, (size_t)n_vocab * 4, hipMemcpyHostToDevice, st), return -3);
        row = s->d_row;
    }
    return sampler_run(s, row, n_vocab, st);
}

extern "C" void dec_sampler_reset(dec_sampler *s) {
    if (!s) return;
    s->hist.clear();
    s->draws = 0;
}

extern "C" int64_t dec_sampler_draws(const dec_sampler *s) { return s ? (int64_t)s->draws : -1; }

extern "C" void dec_sampler_free(dec_sampler *s) {
    if (!s) return;
    if (s->h_buf) (void)hipHostFree(s->h_buf);
    if (s->d_row) (void)hipFree(s->d_row);
    if (s->own) (void)hipStreamDestroy(s->own);
    delete s;
}

extern "C" int32_t dec_seq_pos_max(const dec_ctx *c, int32_t seq) {
    if (!c || seq < 0 || seq >= c->n_seq) return -1;
    return c->pos_max[seq];
}

extern "C" int32_t dec_seq_clear(dec_ctx *c, int32_t seq) {
    if (!c || seq < 0 || seq >= c->n_seq) return -1;
    (void)step_settle(c);   // a failed step's rollback does not matter to a cleared sequence
    c->pos_max[seq] = -1;
    return 0;
}

extern "C" void dec_get_stats(const dec_ctx *c, dec_stats *out) {
    if (!c || !out) return;
    *out = c->st;
}

extern "C" int32_t dec_set_probe(dec_ctx *c, int32_t role, int32_t layer) {
    if (!c || role > DEC_K_STEP) return -1;
    if (role >= 0 && role < DEC_K_OUTPUT && (layer < 0 || layer >= c->m->hp.n_layer)) return -1;
    (void)hipStreamSynchronize(c->s);
    c->pr_used = 0;
    c->pr_ms = 0.0;
    c->pr_n = 0;
    const int r = role < 0 ? -1 : role;
    if (r != c->pr_role || (r >= 0 && r < DEC_K_OUTPUT && layer != c->pr_layer)) {
        c->pr_role = r;
        c->pr_layer = layer;
        drop_graphs(c);   // captured graphs hold (or lack) the probe's event nodes
    }
    return 0;
}

extern "C" int32_t dec_get_probe(dec_ctx *c, double *total_ms, int64_t *count) {
    if (!c || c->pr_role < 0) return -1;
    probe_collect(c);
    if (total_ms) *total_ms = c->pr_ms;
    if (count) *count = c->pr_n;
    return 0;
}

extern "C" int32_t dec_set_use_graphs(dec_ctx *c, int32_t on) {
    if (!c) return -1;
    const int32_t prev = c->use_graphs ? 1 : 0;
    c->use_graphs = on != 0;
    return prev;
}

extern "C" int32_t dec_set_step_kernel(dec_ctx *c, int32_t on) {
    if (!c || !c->step_ok) return -1;
    const int32_t prev = c->step_on ? 1 : 0;
    if (on >= 0) c->step_on = on != 0;
    return prev;
}

extern "C" void dec_set_log_callback(void (*cb)(int, const char *, void *), void *ud) {
    g_log_cb = cb;
    g_log_ud = ud;
}

extern "C" const char *dec_version(void) { return "libdecode 0.1 (gfx950, HIP)"; }
