// gguf.h -- the GGUF v3 container: a validating reader over a memory-mapped
// file, and a streaming writer.
//
// Layout (the article's GGUF reference section): magic "GGUF", format
// version, tensor count, key/value count; the key/value pairs (key string,
// value type, value; an array holds its element type and count, then the
// elements); one record per tensor (name, number of dimensions and the size
// of each, element type, offset of its data from the start of the data
// section); then the data section.  Strings are a 64-bit length followed by
// the bytes; every integer is little-endian.  The data section starts at
// the next multiple of the alignment (key general.alignment, 32 when
// absent), and every tensor offset is a multiple of it.
#pragma once

#include <cstddef>
#include <cstdint>
#include <functional>
#include <map>
#include <string>
#include <vector>

namespace gguf {

enum ValueType : uint32_t {
    V_U8 = 0, V_I8 = 1, V_U16 = 2, V_I16 = 3, V_U32 = 4, V_I32 = 5, V_F32 = 6, V_BOOL = 7,
    V_STR = 8, V_ARR = 9, V_U64 = 10, V_I64 = 11, V_F64 = 12,
};

// element types this library reads and writes (ggml numbering)
enum TensorType : uint32_t { T_F32 = 0, T_F16 = 1, T_Q4_0 = 2, T_Q8_0 = 8, T_Q4_K = 12 };

// result codes (negative = rejected)
enum Status {
    OK = 0,
    E_OPEN = -1,        // cannot open / map the file
    E_MAGIC = -4,       // not a GGUF file
    E_VERSION = -5,     // a format version other than 3
    E_MALFORMED = -6,   // header, key/value or tensor records inconsistent or truncated
    E_DUPLICATE = -7,   // two tensors with one name
    E_RANGE = -8,       // tensor data outside the file
    E_SHAPE = -9,       // a required tensor or key missing, or of the wrong shape
    E_TYPE = -10,       // an element type this library does not handle
};

struct Value {
    ValueType type = V_U8;
    bool array = false;      // arrays are skipped over and only recorded
    uint64_t u = 0;          // unsigned / bool payload
    int64_t i = 0;           // signed payload
    double f = 0.0;          // floating payload
    std::string s;           // string payload
    bool as_u64(uint64_t &out) const;   // any non-negative integer type
    bool as_f64(double &out) const;     // any number
};

struct Tensor {
    std::string name;
    uint32_t n_dims = 0;
    uint64_t dims[4] = {1, 1, 1, 1};   // dims[0] is the innermost (row length)
    uint32_t type = 0;
    uint64_t offset = 0;               // from the start of the data section
    uint64_t nbytes = 0;
    const uint8_t *data = nullptr;     // into the mapping
};

// Bytes of `ne0 x rows` elements of `type`, 0 when the type is unknown or
// the row length does not split into its blocks.
uint64_t type_bytes(uint32_t type, uint64_t ne0, uint64_t rows);

class File {
  public:
    File() = default;
    File(const File &) = delete;
    File &operator=(const File &) = delete;
    ~File();
    // Maps and validates `path`; returns a Status.
    int open(const char *path);
    const Value *find(const std::string &key) const;
    const Tensor *tensor(const std::string &name) const;
    uint32_t version = 0, alignment = 32;
    std::map<std::string, Value> kv;
    std::vector<Tensor> tensors;

  private:
    int parse();
    int fd_ = -1;
    const uint8_t *map_ = nullptr;
    size_t size_ = 0;
    std::map<std::string, size_t> by_name_;
};

// One tensor of a file being written; `fill` produces exactly
// type_bytes(type, dims[0], dims[1] * ...) bytes when asked.
struct OutTensor {
    std::string name;
    uint32_t type = T_F32;
    std::vector<uint64_t> dims;
    std::function<bool(std::vector<uint8_t> &)> fill;
};

// Writes a GGUF v3 file with the given key/value pairs (scalars and strings)
// and tensors, data aligned to `alignment`.  Returns a Status (E_OPEN on an
// I/O failure, E_MALFORMED on inconsistent input).
int write(const char *path, const std::vector<std::pair<std::string, Value>> &kv,
          const std::vector<OutTensor> &tensors, uint32_t alignment);

Value str_value(const std::string &s);
Value u32_value(uint32_t v);
Value f32_value(float v);

}  // namespace gguf
