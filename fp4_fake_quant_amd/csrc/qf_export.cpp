// Checkpoint containers for the packed engine layouts (host code only: files are
// written from host buffers; nothing here touches the GPU).
//
// QATFactory project page, "Method", "Export": NVFP4 and MXFP4 checkpoints go to vLLM
// in the compressed-tensors layout, Q4_K to llama.cpp as GGUF, so the engine loads the
// trained codes and scales with no extra lossy conversion.  The pages fix neither file
// format; this library writes
//   - safetensors: an 8-byte little-endian header length, a JSON header mapping each
//     tensor name to {dtype, shape, data_offsets} (plus an optional "__metadata__" map
//     of strings), padded with spaces to a multiple of 8 bytes, then the tensors' bytes
//     back to back in the order given;
//   - a GGUF-style file: magic "GGUF", version 3, tensor and key-value counts, string
//     key-value pairs, tensor infos (name, dims innermost first, type, offset), padding
//     to 32 bytes, then each tensor's bytes at a 32-byte aligned offset.
// Byte compatibility with the engines' loaders is not checked here (no engine is
// available); the safetensors container is checked against the safetensors reader.
#include <stdio.h>
#include <string.h>

#include <string>
#include <vector>

#include "../../include/qf.h"

namespace {

struct StDtype {
  const char* name;
  int size;
};
const StDtype kStDtypes[] = {{"BOOL", 1}, {"U8", 1},  {"I8", 1},  {"F8_E4M3", 1}, {"F8_E5M2", 1}, {"F8_E8M0", 1},
                             {"U16", 2},  {"I16", 2}, {"F16", 2}, {"BF16", 2},    {"U32", 4},     {"I32", 4},
                             {"F32", 4},  {"U64", 8}, {"I64", 8}, {"F64", 8}};

int st_dtype_size(const char* dt) {
  if (!dt) return 0;
  for (const StDtype& d : kStDtypes)
    if (strcmp(d.name, dt) == 0) return d.size;
  return 0;
}

// JSON string literal of s (quotes, backslash and control characters escaped).
void json_string(std::string& out, const char* s) {
  out += '"';
  for (const unsigned char* p = (const unsigned char*)s; *p; ++p) {
    const unsigned char c = *p;
    if (c == '"' || c == '\\') {
      out += '\\';
      out += (char)c;
    } else if (c < 0x20) {
      char buf[8];
      snprintf(buf, sizeof(buf), "\\u%04x", c);
      out += buf;
    } else {
      out += (char)c;
    }
  }
  out += '"';
}

bool write_all(FILE* f, const void* p, size_t n) { return n == 0 || fwrite(p, 1, n, f) == n; }

bool shape_bytes(int ndim, const int64_t* shape, int elem, uint64_t* bytes) {
  if (ndim < 0 || ndim > 8 || (ndim > 0 && !shape)) return false;
  uint64_t n = 1;
  for (int i = 0; i < ndim; ++i) {
    if (shape[i] < 0) return false;
    if (shape[i] > 0 && n > (UINT64_MAX / 16) / (uint64_t)shape[i]) return false;
    n *= (uint64_t)shape[i];
  }
  *bytes = n * (uint64_t)elem;
  return true;
}

// GGUF scalar writers (little-endian host, as x86-64 and every HIP host is).
bool put_u32(FILE* f, uint32_t v) { return write_all(f, &v, 4); }
bool put_u64(FILE* f, uint64_t v) { return write_all(f, &v, 8); }
bool put_str(FILE* f, const char* s) {
  const uint64_t n = strlen(s);
  return put_u64(f, n) && write_all(f, s, n);
}

constexpr uint32_t GGUF_MAGIC = 0x46554747u;   // the bytes "GGUF"
constexpr uint32_t GGUF_VERSION = 3;
constexpr uint32_t GGUF_TYPE_STRING = 8;
constexpr uint64_t GGUF_ALIGN = 32;

}  // namespace

extern "C" {

qf_status qf_write_safetensors(const char* path, const qf_st_tensor* t, int n, const char* const* meta_keys,
                               const char* const* meta_values, int n_meta) {
  if (!path || (n > 0 && !t) || (n_meta > 0 && (!meta_keys || !meta_values))) return QF_ERR_NULL;
  if (n < 0 || n_meta < 0) return QF_ERR_ARG;
  std::vector<uint64_t> sizes((size_t)n);
  std::string hdr = "{";
  uint64_t off = 0;
  for (int i = 0; i < n; ++i) {
    if (!t[i].name || !t[i].dtype) return QF_ERR_NULL;
    if (t[i].name[0] == 0 || strcmp(t[i].name, "__metadata__") == 0) return QF_ERR_ARG;
    for (int j = 0; j < i; ++j)
      if (strcmp(t[i].name, t[j].name) == 0) return QF_ERR_ARG;        // names must be unique
    const int es = st_dtype_size(t[i].dtype);
    if (!es) return QF_ERR_ARG;
    if (!shape_bytes(t[i].ndim, t[i].shape, es, &sizes[(size_t)i])) return QF_ERR_SHAPE;
    if (sizes[(size_t)i] > 0 && !t[i].data) return QF_ERR_NULL;
    if (i) hdr += ',';
    json_string(hdr, t[i].name);
    hdr += ":{\"dtype\":";
    json_string(hdr, t[i].dtype);
    hdr += ",\"shape\":[";
    for (int d = 0; d < t[i].ndim; ++d) {
      if (d) hdr += ',';
      hdr += std::to_string((long long)t[i].shape[d]);
    }
    hdr += "],\"data_offsets\":[" + std::to_string((unsigned long long)off) + "," +
           std::to_string((unsigned long long)(off + sizes[(size_t)i])) + "]}";
    off += sizes[(size_t)i];
  }
  if (n_meta > 0) {
    if (n > 0) hdr += ',';
    hdr += "\"__metadata__\":{";
    for (int i = 0; i < n_meta; ++i) {
      if (!meta_keys[i] || !meta_values[i]) return QF_ERR_NULL;
      if (i) hdr += ',';
      json_string(hdr, meta_keys[i]);
      hdr += ':';
      json_string(hdr, meta_values[i]);
    }
    hdr += '}';
  }
  hdr += '}';
  while (hdr.size() % 8) hdr += ' ';
  FILE* f = fopen(path, "wb");
  if (!f) return QF_ERR_IO;
  const uint64_t hlen = hdr.size();
  bool ok = write_all(f, &hlen, 8) && write_all(f, hdr.data(), hdr.size());
  for (int i = 0; ok && i < n; ++i) ok = write_all(f, t[i].data, (size_t)sizes[(size_t)i]);
  ok = (fclose(f) == 0) && ok;
  return ok ? QF_OK : QF_ERR_IO;
}

qf_status qf_write_gguf(const char* path, const qf_gguf_tensor* t, int n, const char* const* kv_keys,
                        const char* const* kv_values, int n_kv) {
  if (!path || (n > 0 && !t) || (n_kv > 0 && (!kv_keys || !kv_values))) return QF_ERR_NULL;
  if (n < 0 || n_kv < 0) return QF_ERR_ARG;
  std::vector<uint64_t> offs((size_t)n);
  uint64_t off = 0;
  for (int i = 0; i < n; ++i) {
    if (!t[i].name) return QF_ERR_NULL;
    if (t[i].name[0] == 0) return QF_ERR_ARG;
    for (int j = 0; j < i; ++j)
      if (strcmp(t[i].name, t[j].name) == 0) return QF_ERR_ARG;
    if (t[i].ndim < 1 || t[i].ndim > 4 || !t[i].dims) return QF_ERR_SHAPE;
    for (int d = 0; d < t[i].ndim; ++d)
      if (t[i].dims[d] < 0) return QF_ERR_SHAPE;
    if (t[i].nbytes > 0 && !t[i].data) return QF_ERR_NULL;
    offs[(size_t)i] = off;
    off += (t[i].nbytes + GGUF_ALIGN - 1) / GGUF_ALIGN * GGUF_ALIGN;
  }
  for (int i = 0; i < n_kv; ++i)
    if (!kv_keys[i] || !kv_values[i]) return QF_ERR_NULL;
  FILE* f = fopen(path, "wb");
  if (!f) return QF_ERR_IO;
  bool ok = put_u32(f, GGUF_MAGIC) && put_u32(f, GGUF_VERSION) && put_u64(f, (uint64_t)n) && put_u64(f, (uint64_t)n_kv);
  for (int i = 0; ok && i < n_kv; ++i)
    ok = put_str(f, kv_keys[i]) && put_u32(f, GGUF_TYPE_STRING) && put_str(f, kv_values[i]);
  for (int i = 0; ok && i < n; ++i) {
    ok = put_str(f, t[i].name) && put_u32(f, (uint32_t)t[i].ndim);
    for (int d = 0; ok && d < t[i].ndim; ++d) ok = put_u64(f, (uint64_t)t[i].dims[d]);
    ok = ok && put_u32(f, t[i].type) && put_u64(f, offs[(size_t)i]);
  }
  static const char zeros[GGUF_ALIGN] = {0};
  long pos = ok ? ftell(f) : -1;
  if (pos < 0) ok = false;
  if (ok && pos % (long)GGUF_ALIGN) ok = write_all(f, zeros, (size_t)(GGUF_ALIGN - pos % (long)GGUF_ALIGN));
  for (int i = 0; ok && i < n; ++i) {
    ok = write_all(f, t[i].data, (size_t)t[i].nbytes);
    const uint64_t pad = (GGUF_ALIGN - t[i].nbytes % GGUF_ALIGN) % GGUF_ALIGN;
    if (ok && pad) ok = write_all(f, zeros, (size_t)pad);
  }
  ok = (fclose(f) == 0) && ok;
  return ok ? QF_OK : QF_ERR_IO;
}

}  // extern "C"
