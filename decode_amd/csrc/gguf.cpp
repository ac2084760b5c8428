// gguf.cpp -- GGUF v3 reader (memory-mapped, every read bounds-checked) and
// streaming writer.  Host code only.
#include "gguf.h"

#include <fcntl.h>
#include <sys/mman.h>
#include <sys/stat.h>
#include <unistd.h>

#include <algorithm>
#include <cstdio>
#include <cstring>

namespace gguf {

namespace {

constexpr uint32_t MAGIC = 0x46554747u;   // the bytes 'G' 'G' 'U' 'F'
constexpr uint64_t MAX_COUNT = 1ull << 24;
constexpr int MAX_ARRAY_DEPTH = 4;

size_t scalar_size(uint32_t t) {
    switch (t) {
    case V_U8: case V_I8: case V_BOOL: return 1;
    case V_U16: case V_I16: return 2;
    case V_U32: case V_I32: case V_F32: return 4;
    case V_U64: case V_I64: case V_F64: return 8;
    default: return 0;
    }
}

// Cursor over the mapped bytes; every read checks the remaining size.
struct Cursor {
    const uint8_t *p;
    size_t left;
    bool bytes(void *dst, size_t n) {
        if (n > left) return false;
        memcpy(dst, p, n);
        p += n;
        left -= n;
        return true;
    }
    bool skip(size_t n) {
        if (n > left) return false;
        p += n;
        left -= n;
        return true;
    }
    template <typename T>
    bool get(T &v) { return bytes(&v, sizeof(T)); }
    bool str(std::string &s) {
        uint64_t n;
        if (!get(n) || n > left) return false;
        s.assign((const char *)p, (size_t)n);
        p += n;
        left -= (size_t)n;
        return true;
    }
};

bool read_scalar(Cursor &c, uint32_t t, Value &v) {
    v.type = (ValueType)t;
    switch (t) {
    case V_U8: { uint8_t x; if (!c.get(x)) return false; v.u = x; v.i = x; v.f = x; return true; }
    case V_I8: { int8_t x; if (!c.get(x)) return false; v.i = x; v.u = (uint64_t)x; v.f = x; return true; }
    case V_U16: { uint16_t x; if (!c.get(x)) return false; v.u = x; v.i = x; v.f = x; return true; }
    case V_I16: { int16_t x; if (!c.get(x)) return false; v.i = x; v.u = (uint64_t)x; v.f = x; return true; }
    case V_U32: { uint32_t x; if (!c.get(x)) return false; v.u = x; v.i = x; v.f = x; return true; }
    case V_I32: { int32_t x; if (!c.get(x)) return false; v.i = x; v.u = (uint64_t)x; v.f = x; return true; }
    case V_U64: { uint64_t x; if (!c.get(x)) return false; v.u = x; v.i = (int64_t)x; v.f = (double)x; return true; }
    case V_I64: { int64_t x; if (!c.get(x)) return false; v.i = x; v.u = (uint64_t)x; v.f = (double)x; return true; }
    case V_F32: { float x; if (!c.get(x)) return false; v.f = x; return true; }
    case V_F64: { double x; if (!c.get(x)) return false; v.f = x; return true; }
    case V_BOOL: {
        uint8_t x;
        if (!c.get(x) || x > 1) return false;
        v.u = x;
        return true;
    }
    case V_STR: return c.str(v.s);
    default: return false;
    }
}

// A value of type t (an array recursively), consumed from the cursor.
bool read_value(Cursor &c, uint32_t t, Value &v, int depth) {
    if (t != V_ARR) return read_scalar(c, t, v);
    if (depth >= MAX_ARRAY_DEPTH) return false;
    uint32_t et;
    uint64_t n;
    if (!c.get(et) || !c.get(n)) return false;
    v.type = V_ARR;
    v.array = true;
    v.u = n;
    if (et == V_STR || et == V_ARR) {
        if (n > c.left) return false;   // every element takes at least one byte
        for (uint64_t k = 0; k < n; k++) {
            Value e;
            if (!read_value(c, et, e, depth + 1)) return false;
        }
        return true;
    }
    const size_t es = scalar_size(et);
    if (es == 0 || n > c.left / es) return false;
    return c.skip((size_t)n * es);
}

}  // namespace

bool Value::as_u64(uint64_t &out) const {
    if (array) return false;
    switch (type) {
    case V_U8: case V_U16: case V_U32: case V_U64: out = u; return true;
    case V_I8: case V_I16: case V_I32: case V_I64:
        if (i < 0) return false;
        out = (uint64_t)i;
        return true;
    default: return false;
    }
}

bool Value::as_f64(double &out) const {
    if (array) return false;
    switch (type) {
    case V_F32: case V_F64: out = f; return true;
    case V_U8: case V_U16: case V_U32: case V_U64: out = (double)u; return true;
    case V_I8: case V_I16: case V_I32: case V_I64: out = (double)i; return true;
    default: return false;
    }
}

uint64_t type_bytes(uint32_t type, uint64_t ne0, uint64_t rows) {
    switch (type) {
    case T_F32: return ne0 * rows * 4;
    case T_F16: return ne0 * rows * 2;
    case T_Q4_0: return ne0 % 32 ? 0 : ne0 / 32 * 18 * rows;
    case T_Q8_0: return ne0 % 32 ? 0 : ne0 / 32 * 34 * rows;
    case T_Q4_K: return ne0 % 256 ? 0 : ne0 / 256 * 144 * rows;
    default: return 0;
    }
}

File::~File() {
    if (map_) munmap((void *)map_, size_);
    if (fd_ >= 0) close(fd_);
}

int File::open(const char *path) {
    if (!path) return E_OPEN;
    fd_ = ::open(path, O_RDONLY);
    if (fd_ < 0) return E_OPEN;
    struct stat st;
    if (fstat(fd_, &st) != 0) return E_OPEN;
    if (st.st_size <= 0) return E_MALFORMED;
    size_ = (size_t)st.st_size;
    void *p = mmap(nullptr, size_, PROT_READ, MAP_PRIVATE, fd_, 0);
    if (p == MAP_FAILED) {
        size_ = 0;
        return E_OPEN;
    }
    map_ = (const uint8_t *)p;
    return parse();
}

int File::parse() {
    Cursor c{map_, size_};
    uint32_t magic;
    if (!c.get(magic)) return E_MALFORMED;
    if (magic != MAGIC) return E_MAGIC;
    if (!c.get(version)) return E_MALFORMED;
    if (version != 3) return E_VERSION;
    uint64_t n_tensors, n_kv;
    if (!c.get(n_tensors) || !c.get(n_kv)) return E_MALFORMED;
    if (n_tensors > MAX_COUNT || n_kv > MAX_COUNT) return E_MALFORMED;

    for (uint64_t k = 0; k < n_kv; k++) {
        std::string key;
        uint32_t t;
        Value v;
        if (!c.str(key) || !c.get(t) || !read_value(c, t, v, 0)) return E_MALFORMED;
        kv[key] = v;   // a repeated key keeps its last value
    }
    if (const Value *a = find("general.alignment")) {
        uint64_t al;
        if (!a->as_u64(al) || al == 0 || al > (1u << 20) || (al & (al - 1))) return E_MALFORMED;
        alignment = (uint32_t)al;
    }

    tensors.resize((size_t)n_tensors);
    for (uint64_t k = 0; k < n_tensors; k++) {
        Tensor &T = tensors[(size_t)k];
        if (!c.str(T.name) || !c.get(T.n_dims)) return E_MALFORMED;
        if (T.n_dims < 1 || T.n_dims > 4) return E_MALFORMED;
        for (uint32_t j = 0; j < T.n_dims; j++)
            if (!c.get(T.dims[j]) || T.dims[j] == 0 || T.dims[j] > (1ull << 40)) return E_MALFORMED;
        if (!c.get(T.type) || !c.get(T.offset)) return E_MALFORMED;
        if (by_name_.count(T.name)) return E_DUPLICATE;
        by_name_[T.name] = (size_t)k;
    }
    const size_t header = size_ - c.left;
    const uint64_t data_start = (header + alignment - 1) / alignment * alignment;
    for (Tensor &T : tensors) {
        uint64_t rows = 1;
        for (uint32_t j = 1; j < T.n_dims; j++) {
            if (rows > (1ull << 40) / T.dims[j]) return E_MALFORMED;
            rows *= T.dims[j];
        }
        if (T.dims[0] > (1ull << 42) / rows) return E_MALFORMED;   // keeps the byte counts below 2^46
        if (T.type != T_F32 && T.type != T_F16 && T.type != T_Q4_0 && T.type != T_Q8_0 && T.type != T_Q4_K)
            return E_TYPE;
        T.nbytes = type_bytes(T.type, T.dims[0], rows);
        if (T.nbytes == 0) return E_MALFORMED;
        if (T.offset % alignment) return E_MALFORMED;
        if (data_start > size_ || T.offset > size_ - data_start || T.nbytes > size_ - data_start - T.offset)
            return E_RANGE;
        T.data = map_ + data_start + T.offset;
    }
    return OK;
}

const Value *File::find(const std::string &key) const {
    auto it = kv.find(key);
    return it == kv.end() ? nullptr : &it->second;
}

const Tensor *File::tensor(const std::string &name) const {
    auto it = by_name_.find(name);
    return it == by_name_.end() ? nullptr : &tensors[it->second];
}

Value str_value(const std::string &s) {
    Value v;
    v.type = V_STR;
    v.s = s;
    return v;
}
Value u32_value(uint32_t x) {
    Value v;
    v.type = V_U32;
    v.u = x;
    return v;
}
Value f32_value(float x) {
    Value v;
    v.type = V_F32;
    v.f = x;
    return v;
}

namespace {

struct Writer {
    FILE *f;
    uint64_t pos = 0;
    bool ok = true;
    void bytes(const void *p, size_t n) {
        if (ok && n && fwrite(p, 1, n, f) != n) ok = false;
        pos += n;
    }
    template <typename T>
    void put(T v) { bytes(&v, sizeof(T)); }
    void str(const std::string &s) {
        put<uint64_t>(s.size());
        bytes(s.data(), s.size());
    }
    void pad_to(uint64_t a) {
        static const uint8_t zeros[64] = {};
        while (pos % a) bytes(zeros, (size_t)std::min<uint64_t>(a - pos % a, sizeof zeros));
    }
};

}  // namespace

int write(const char *path, const std::vector<std::pair<std::string, Value>> &kv,
          const std::vector<OutTensor> &tensors, uint32_t alignment) {
    if (!path || alignment == 0 || (alignment & (alignment - 1))) return E_MALFORMED;
    // sizes and offsets first, from the element types and dimensions
    std::vector<uint64_t> nbytes(tensors.size()), offs(tensors.size());
    uint64_t off = 0;
    for (size_t k = 0; k < tensors.size(); k++) {
        const OutTensor &t = tensors[k];
        if (t.dims.empty() || t.dims.size() > 4 || !t.fill) return E_MALFORMED;
        uint64_t rows = 1;
        for (size_t j = 1; j < t.dims.size(); j++) rows *= t.dims[j];
        nbytes[k] = type_bytes(t.type, t.dims[0], rows);
        if (!nbytes[k]) return E_MALFORMED;
        offs[k] = off;
        off = (off + nbytes[k] + alignment - 1) / alignment * alignment;
    }
    FILE *f = fopen(path, "wb");
    if (!f) return E_OPEN;
    Writer w{f};
    w.put<uint32_t>(MAGIC);
    w.put<uint32_t>(3);
    w.put<uint64_t>(tensors.size());
    w.put<uint64_t>(kv.size());
    for (const auto &p : kv) {
        w.str(p.first);
        const Value &v = p.second;
        w.put<uint32_t>(v.type);
        switch (v.type) {
        case V_STR: w.str(v.s); break;
        case V_U32: w.put<uint32_t>((uint32_t)v.u); break;
        case V_I32: w.put<int32_t>((int32_t)v.i); break;
        case V_U64: w.put<uint64_t>(v.u); break;
        case V_F32: w.put<float>((float)v.f); break;
        case V_BOOL: w.put<uint8_t>(v.u ? 1 : 0); break;
        default: fclose(f); return E_MALFORMED;
        }
    }
    for (size_t k = 0; k < tensors.size(); k++) {
        const OutTensor &t = tensors[k];
        w.str(t.name);
        w.put<uint32_t>((uint32_t)t.dims.size());
        for (uint64_t d : t.dims) w.put<uint64_t>(d);
        w.put<uint32_t>(t.type);
        w.put<uint64_t>(offs[k]);
    }
    w.pad_to(alignment);
    const uint64_t data_start = w.pos;
    std::vector<uint8_t> buf;
    for (size_t k = 0; k < tensors.size() && w.ok; k++) {
        w.pad_to(alignment);
        if (w.pos - data_start != offs[k]) {
            w.ok = false;
            break;
        }
        buf.clear();
        if (!tensors[k].fill(buf) || buf.size() != nbytes[k]) {
            fclose(f);
            return E_MALFORMED;
        }
        w.bytes(buf.data(), buf.size());
    }
    const bool closed = fclose(f) == 0;
    return w.ok && closed ? OK : E_OPEN;
}

}  // namespace gguf
