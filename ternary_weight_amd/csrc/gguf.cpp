// Host-side lookup of a tensor in a GGUF file image (the ggml model file
// format the pages' converter writes: "BitNet Embeddings GGUF Conversion
// Implementation", s5 "GGUF Conversion Process" and s6.2 "gguf-py: I2_S
// Type"), so that I2_S projection weights and float16 norm weights can be
// fed to the GPU calls straight from a model file.
//
// Container (little-endian): magic "GGUF", version (2 or 3), tensor count and
// metadata count (64-bit), the metadata key/value pairs, the tensor infos
// (name, dimension count, dimensions with the innermost first, type id, data
// offset), then the data section at the next multiple of the alignment
// (the uint32 "general.alignment" value, 32 when absent), where each tensor's
// data starts at its offset.  Every read is bounds-checked: a truncated or
// malformed image is an error, never an out-of-range access.
//
// I2_S is type 36 with quant size (4, 1): four ternary codes per byte, so a
// [N][K] weight (dims K, N) holds N*K/4 code bytes, and the float32 scale is
// appended right after them (s3 "I2_S Ternary Packing").  The code bytes and
// the scale together are exactly the buffer bitlinear_forward takes.
#include <cstdint>
#include <cstring>
#include <string>

#include "../../include/bitlinear.h"

namespace {

class Reader {
 public:
  Reader(const uint8_t* p, size_t n) : p_(p), n_(n) {}
  bool ok() const { return ok_; }
  size_t pos() const { return pos_; }
  template <typename T>
  T get() {
    T v{};
    if (!ok_ || n_ - pos_ < sizeof(T)) {
      ok_ = false;
      return v;
    }
    std::memcpy(&v, p_ + pos_, sizeof(T));
    pos_ += sizeof(T);
    return v;
  }
  void skip(uint64_t bytes) {
    if (!ok_ || bytes > n_ - pos_) {
      ok_ = false;
      return;
    }
    pos_ += static_cast<size_t>(bytes);
  }
  // A GGUF string (uint64 length, bytes); returns a view into the image.
  bool str(const char** s, uint64_t* len) {
    *len = get<uint64_t>();
    if (!ok_ || *len > n_ - pos_) {
      ok_ = false;
      return false;
    }
    *s = reinterpret_cast<const char*>(p_ + pos_);
    pos_ += static_cast<size_t>(*len);
    return true;
  }

 private:
  const uint8_t* p_;
  size_t n_;
  size_t pos_ = 0;
  bool ok_ = true;
};

// Metadata value types of the format.
enum : uint32_t {
  kU8 = 0, kI8 = 1, kU16 = 2, kI16 = 3, kU32 = 4, kI32 = 5, kF32 = 6, kBool = 7,
  kString = 8, kArray = 9, kU64 = 10, kI64 = 11, kF64 = 12
};

int scalar_size(uint32_t t) {
  switch (t) {
    case kU8: case kI8: case kBool: return 1;
    case kU16: case kI16: return 2;
    case kU32: case kI32: case kF32: return 4;
    case kU64: case kI64: case kF64: return 8;
    default: return 0;
  }
}

// Skips one metadata value of type t (arrays hold scalars or strings).
bool skip_value(Reader& r, uint32_t t) {
  if (const int sz = scalar_size(t)) {
    r.skip(static_cast<uint64_t>(sz));
    return r.ok();
  }
  if (t == kString) {
    const char* s;
    uint64_t len;
    return r.str(&s, &len);
  }
  if (t != kArray) return false;
  const uint32_t et = r.get<uint32_t>();
  const uint64_t count = r.get<uint64_t>();
  if (!r.ok()) return false;
  if (const int sz = scalar_size(et)) {
    if (count > UINT64_MAX / static_cast<uint64_t>(sz)) return false;
    r.skip(count * static_cast<uint64_t>(sz));
    return r.ok();
  }
  if (et != kString) return false;  // nested arrays do not occur in model files
  for (uint64_t i = 0; i < count; ++i) {
    const char* s;
    uint64_t len;
    if (!r.str(&s, &len)) return false;
  }
  return true;
}

constexpr uint32_t kTypeF32 = 0, kTypeF16 = 1, kTypeI2S = 36;

}  // namespace

extern "C" bl_status bl_gguf_find_tensor(const uint8_t* file, size_t file_bytes, const char* name,
                                         bl_gguf_tensor* out) {
  try {
    if (!file || !name || !out) return BL_ERR_INVALID_ARGUMENT;
    Reader r(file, file_bytes);
    const uint32_t magic = r.get<uint32_t>();
    const uint32_t version = r.get<uint32_t>();
    const uint64_t n_tensors = r.get<uint64_t>();
    const uint64_t n_kv = r.get<uint64_t>();
    if (!r.ok() || std::memcmp(file, "GGUF", 4) != 0 || magic != 0x46554747u) return BL_ERR_INVALID_ARGUMENT;
    if (version != 2 && version != 3) return BL_ERR_UNSUPPORTED;
    uint64_t alignment = 32;
    for (uint64_t i = 0; i < n_kv; ++i) {
      const char* key;
      uint64_t klen;
      if (!r.str(&key, &klen)) return BL_ERR_INVALID_ARGUMENT;
      const uint32_t t = r.get<uint32_t>();
      if (!r.ok()) return BL_ERR_INVALID_ARGUMENT;
      if (klen == 17 && std::memcmp(key, "general.alignment", 17) == 0 && t == kU32) {
        alignment = r.get<uint32_t>();
        if (!r.ok() || alignment == 0 || (alignment & (alignment - 1)) != 0) return BL_ERR_INVALID_ARGUMENT;
        continue;
      }
      if (!skip_value(r, t)) return BL_ERR_INVALID_ARGUMENT;
    }
    const size_t want = std::strlen(name);
    bool found = false;
    bl_gguf_tensor hit{};
    for (uint64_t i = 0; i < n_tensors; ++i) {
      const char* tname;
      uint64_t tlen;
      if (!r.str(&tname, &tlen)) return BL_ERR_INVALID_ARGUMENT;
      const uint32_t nd = r.get<uint32_t>();
      if (!r.ok() || nd == 0 || nd > 4) return BL_ERR_INVALID_ARGUMENT;
      bl_gguf_tensor t{};
      t.n_dims = static_cast<int32_t>(nd);
      uint64_t elems = 1;
      for (uint32_t d = 0; d < nd; ++d) {
        const uint64_t v = r.get<uint64_t>();
        if (!r.ok() || v == 0 || v > static_cast<uint64_t>(INT64_MAX) || elems > UINT64_MAX / v)
          return BL_ERR_INVALID_ARGUMENT;
        elems *= v;
        t.dims[d] = static_cast<int64_t>(v);
      }
      t.type = static_cast<int32_t>(r.get<uint32_t>());
      t.offset = r.get<uint64_t>();  // relative to the data section for now
      if (!r.ok()) return BL_ERR_INVALID_ARGUMENT;
      if (t.type == static_cast<int32_t>(kTypeF32)) t.nbytes = elems * 4;
      else if (t.type == static_cast<int32_t>(kTypeF16)) t.nbytes = elems * 2;
      else if (t.type == static_cast<int32_t>(kTypeI2S)) t.nbytes = (elems % 4 == 0) ? elems / 4 + 4 : 0;
      if (!found && tlen == want && std::memcmp(tname, name, want) == 0) {
        hit = t;
        found = true;
      }
    }
    if (!found) return BL_ERR_NOT_FOUND;
    const uint64_t data = (static_cast<uint64_t>(r.pos()) + alignment - 1) / alignment * alignment;
    if (hit.offset > UINT64_MAX - data) return BL_ERR_INVALID_ARGUMENT;
    hit.offset += data;
    if (hit.offset > file_bytes || hit.nbytes > file_bytes - hit.offset) return BL_ERR_INVALID_ARGUMENT;
    if (hit.type == static_cast<int32_t>(kTypeI2S)) {
      // a projection weight: [N][K] with K the innermost dimension, whole
      // 128-value blocks ("gguf-gemv", "Requirements")
      if (hit.n_dims != 2 || hit.dims[0] % 128 != 0 || hit.nbytes == 0) return BL_ERR_UNSUPPORTED;
    }
    *out = hit;
    return BL_OK;
  } catch (...) {
    return BL_ERR_INTERNAL;
  }
}
