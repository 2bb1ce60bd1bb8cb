// Strict ingestion of the transformer's weights from safetensors files, and
// the sorted-key digest of a weight table.
//
// "Local component coverage and quality handoff for the zimage FastVideo
// port", Component contracts: native loading accounts for every destination
// parameter, and auxiliary parameters (quantization scales and the like) are
// not silently ignored; the transformer keeps all 521 published checkpoint
// keys, whose sorted key digest from the safetensors index is stated there.
// "Z-Image" (AI Toolkit docs), Specifics: a single .safetensors file of the
// transformer also works.
//
// A safetensors file is an 8-byte little-endian header length N, N bytes of
// JSON, then the tensor data.  The JSON object maps each tensor name to
// {"dtype", "shape", "data_offsets": [begin, end]} (offsets relative to the
// data region), with an optional "__metadata__" object of strings.  Every
// file is validated in full -- structure, dtype, shape against the engine's
// table, offsets inside the data region and consistent with the shape,
// names unique across all files, no name outside the table, no table entry
// missing -- before a single tensor is uploaded.
#include <fcntl.h>
#include <sys/mman.h>
#include <sys/stat.h>
#include <unistd.h>

#include <algorithm>
#include <cerrno>
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <map>
#include <memory>
#include <string>
#include <vector>

#include "../../include/zimg_dit.h"
#include "../../include/zimg_ops.h"
#include "engine_internal.h"

namespace {

// ---------------------------------------------------------------- JSON

struct Json {
  enum Kind { Null, Bool, Number, String, Array, Object } kind = Null;
  std::string text;  // String: the decoded string; Number: the literal
  std::vector<Json> items;
  std::vector<std::pair<std::string, Json>> members;
};

// Recursive-descent parser for RFC 8259 JSON, bounded in depth; numbers are
// kept as their literal text (offsets can exceed a double's exact range).
class JsonParser {
 public:
  JsonParser(const char* p, size_t n) : p_(p), end_(p + n) {}
  bool parse(Json& out, std::string& err) {
    ws();
    if (!value(out, 0)) {
      err = err_.empty() ? "malformed JSON" : err_;
      return false;
    }
    ws();
    if (p_ != end_) {
      err = "trailing bytes after the JSON header";
      return false;
    }
    return true;
  }

 private:
  const char* p_;
  const char* end_;
  std::string err_;

  bool fail(const char* m) {
    if (err_.empty()) err_ = m;
    return false;
  }
  void ws() {
    while (p_ < end_ && (*p_ == ' ' || *p_ == '\t' || *p_ == '\n' || *p_ == '\r')) ++p_;
  }
  bool lit(const char* w) {
    const size_t n = std::strlen(w);
    if ((size_t)(end_ - p_) < n || std::memcmp(p_, w, n) != 0) return fail("invalid literal");
    p_ += n;
    return true;
  }
  static void utf8(uint32_t c, std::string& s) {
    if (c < 0x80) {
      s += (char)c;
    } else if (c < 0x800) {
      s += (char)(0xC0 | (c >> 6));
      s += (char)(0x80 | (c & 0x3F));
    } else if (c < 0x10000) {
      s += (char)(0xE0 | (c >> 12));
      s += (char)(0x80 | ((c >> 6) & 0x3F));
      s += (char)(0x80 | (c & 0x3F));
    } else {
      s += (char)(0xF0 | (c >> 18));
      s += (char)(0x80 | ((c >> 12) & 0x3F));
      s += (char)(0x80 | ((c >> 6) & 0x3F));
      s += (char)(0x80 | (c & 0x3F));
    }
  }
  bool hex4(uint32_t& v) {
    if (end_ - p_ < 4) return fail("truncated \\u escape");
    v = 0;
    for (int i = 0; i < 4; ++i) {
      const char c = *p_++;
      v <<= 4;
      if (c >= '0' && c <= '9') v |= (uint32_t)(c - '0');
      else if (c >= 'a' && c <= 'f') v |= (uint32_t)(c - 'a' + 10);
      else if (c >= 'A' && c <= 'F') v |= (uint32_t)(c - 'A' + 10);
      else return fail("bad \\u escape");
    }
    return true;
  }
  bool string(std::string& s) {
    if (p_ >= end_ || *p_ != '"') return fail("expected a string");
    ++p_;
    while (true) {
      if (p_ >= end_) return fail("unterminated string");
      const unsigned char c = (unsigned char)*p_++;
      if (c == '"') return true;
      if (c < 0x20) return fail("control character in a string");
      if (c != '\\') {
        s += (char)c;
        continue;
      }
      if (p_ >= end_) return fail("unterminated escape");
      const char e = *p_++;
      switch (e) {
        case '"': s += '"'; break;
        case '\\': s += '\\'; break;
        case '/': s += '/'; break;
        case 'b': s += '\b'; break;
        case 'f': s += '\f'; break;
        case 'n': s += '\n'; break;
        case 'r': s += '\r'; break;
        case 't': s += '\t'; break;
        case 'u': {
          uint32_t v;
          if (!hex4(v)) return false;
          if (v >= 0xD800 && v < 0xDC00) {  // a surrogate pair
            uint32_t lo;
            if (end_ - p_ < 2 || p_[0] != '\\' || p_[1] != 'u') return fail("lone surrogate");
            p_ += 2;
            if (!hex4(lo) || lo < 0xDC00 || lo >= 0xE000) return fail("bad surrogate pair");
            v = 0x10000 + ((v - 0xD800) << 10) + (lo - 0xDC00);
          } else if (v >= 0xDC00 && v < 0xE000) {
            return fail("lone surrogate");
          }
          utf8(v, s);
          break;
        }
        default: return fail("bad escape");
      }
    }
  }
  bool number(std::string& t) {
    const char* b = p_;
    if (p_ < end_ && *p_ == '-') ++p_;
    if (p_ >= end_ || *p_ < '0' || *p_ > '9') return fail("bad number");
    if (*p_ == '0') ++p_;
    else
      while (p_ < end_ && *p_ >= '0' && *p_ <= '9') ++p_;
    if (p_ < end_ && *p_ == '.') {
      ++p_;
      if (p_ >= end_ || *p_ < '0' || *p_ > '9') return fail("bad number");
      while (p_ < end_ && *p_ >= '0' && *p_ <= '9') ++p_;
    }
    if (p_ < end_ && (*p_ == 'e' || *p_ == 'E')) {
      ++p_;
      if (p_ < end_ && (*p_ == '+' || *p_ == '-')) ++p_;
      if (p_ >= end_ || *p_ < '0' || *p_ > '9') return fail("bad number");
      while (p_ < end_ && *p_ >= '0' && *p_ <= '9') ++p_;
    }
    t.assign(b, p_);
    return true;
  }
  bool value(Json& v, int depth) {
    if (depth > 64) return fail("JSON nested too deeply");
    if (p_ >= end_) return fail("unexpected end of the JSON header");
    switch (*p_) {
      case '{': {
        v.kind = Json::Object;
        ++p_;
        ws();
        if (p_ < end_ && *p_ == '}') {
          ++p_;
          return true;
        }
        while (true) {
          ws();
          std::string k;
          if (!string(k)) return false;
          ws();
          if (p_ >= end_ || *p_ != ':') return fail("expected ':'");
          ++p_;
          ws();
          v.members.emplace_back(std::move(k), Json{});
          if (!value(v.members.back().second, depth + 1)) return false;
          ws();
          if (p_ < end_ && *p_ == ',') {
            ++p_;
            continue;
          }
          if (p_ < end_ && *p_ == '}') {
            ++p_;
            return true;
          }
          return fail("expected ',' or '}'");
        }
      }
      case '[': {
        v.kind = Json::Array;
        ++p_;
        ws();
        if (p_ < end_ && *p_ == ']') {
          ++p_;
          return true;
        }
        while (true) {
          ws();
          v.items.emplace_back();
          if (!value(v.items.back(), depth + 1)) return false;
          ws();
          if (p_ < end_ && *p_ == ',') {
            ++p_;
            continue;
          }
          if (p_ < end_ && *p_ == ']') {
            ++p_;
            return true;
          }
          return fail("expected ',' or ']'");
        }
      }
      case '"': v.kind = Json::String; return string(v.text);
      case 't': v.kind = Json::Bool; v.text = "true"; return lit("true");
      case 'f': v.kind = Json::Bool; v.text = "false"; return lit("false");
      case 'n': v.kind = Json::Null; return lit("null");
      default: v.kind = Json::Number; return number(v.text);
    }
  }
};

// a non-negative integer literal below 2^62, else -1
int64_t as_index(const Json& j) {
  if (j.kind != Json::Number || j.text.empty() || j.text.size() > 18) return -1;
  int64_t v = 0;
  for (char c : j.text) {
    if (c < '0' || c > '9') return -1;
    v = v * 10 + (c - '0');
  }
  if (j.text.size() > 1 && j.text[0] == '0') return -1;
  return v;
}

// ---------------------------------------------------------------- files

struct TensorRef {
  std::string name;
  int dtype = -1;  // ZIMG_F32 / ZIMG_BF16
  int ndim = 0;
  int64_t shape[4] = {0, 0, 0, 0};
  const unsigned char* data = nullptr;
  size_t bytes = 0;
};

struct MappedFile {
  std::string path;
  void* base = MAP_FAILED;
  size_t size = 0;
  ~MappedFile() {
    if (base != MAP_FAILED) munmap(base, size);
  }
};

int err(int code, const std::string& msg) { return zimg::set_error(code, msg); }

// Map ``path`` and list its tensors (structure, dtype and offsets checked).
int read_file(const char* path, MappedFile& f, std::vector<TensorRef>& out) {
  f.path = path ? path : "";
  if (!path) return err(ZIMG_EINVAL, "safetensors: path is NULL");
  const int fd = open(path, O_RDONLY | O_CLOEXEC);
  if (fd < 0) return err(ZIMG_EINVAL, std::string("safetensors: cannot open ") + path + ": " + std::strerror(errno));
  struct stat st;
  if (fstat(fd, &st) != 0 || !S_ISREG(st.st_mode)) {
    close(fd);
    return err(ZIMG_EINVAL, std::string("safetensors: ") + path + " is not a regular file");
  }
  f.size = (size_t)st.st_size;
  if (f.size < 8) {
    close(fd);
    return err(ZIMG_EWEIGHT, std::string("safetensors: ") + path + " is shorter than its 8-byte header length");
  }
  f.base = mmap(nullptr, f.size, PROT_READ, MAP_PRIVATE, fd, 0);
  close(fd);
  if (f.base == MAP_FAILED) return err(ZIMG_ENOMEM, std::string("safetensors: cannot map ") + path);
  const unsigned char* b = (const unsigned char*)f.base;
  uint64_t n = 0;
  for (int i = 7; i >= 0; --i) n = (n << 8) | b[i];
  if (n > (100u << 20) || n > f.size - 8)
    return err(ZIMG_EWEIGHT, std::string("safetensors: ") + path + ": header length " + std::to_string(n) +
                                 " exceeds the file or the 100 MB limit");
  Json root;
  std::string perr;
  JsonParser parser((const char*)b + 8, (size_t)n);
  if (!parser.parse(root, perr)) return err(ZIMG_EWEIGHT, std::string("safetensors: ") + path + ": " + perr);
  if (root.kind != Json::Object) return err(ZIMG_EWEIGHT, std::string("safetensors: ") + path + ": header is not an object");
  const unsigned char* data = b + 8 + n;
  const size_t data_size = f.size - 8 - (size_t)n;
  for (const auto& m : root.members) {
    const std::string where = std::string("safetensors: ") + path + ": '" + m.first + "'";
    if (m.first == "__metadata__") {
      if (m.second.kind != Json::Object) return err(ZIMG_EWEIGHT, where + " is not an object");
      for (const auto& kv : m.second.members)
        if (kv.second.kind != Json::String) return err(ZIMG_EWEIGHT, where + " holds a value that is not a string");
      continue;
    }
    if (m.second.kind != Json::Object) return err(ZIMG_EWEIGHT, where + " is not a tensor entry");
    const Json *dt = nullptr, *sh = nullptr, *off = nullptr;
    for (const auto& kv : m.second.members) {
      if (kv.first == "dtype") dt = &kv.second;
      else if (kv.first == "shape") sh = &kv.second;
      else if (kv.first == "data_offsets") off = &kv.second;
      else return err(ZIMG_EWEIGHT, where + " has an unknown field '" + kv.first + "'");
    }
    if (!dt || !sh || !off || dt->kind != Json::String || sh->kind != Json::Array || off->kind != Json::Array ||
        off->items.size() != 2)
      return err(ZIMG_EWEIGHT, where + ": dtype, shape and data_offsets [begin, end] are required");
    TensorRef t;
    t.name = m.first;
    size_t item = 0;
    if (dt->text == "F32") {
      t.dtype = ZIMG_F32;
      item = 4;
    } else if (dt->text == "BF16") {
      t.dtype = ZIMG_BF16;
      item = 2;
    } else {
      return err(ZIMG_EUNSUPPORTED, where + " has dtype " + dt->text + "; the engine reads F32 and BF16 only");
    }
    if (sh->items.size() > 4) return err(ZIMG_EWEIGHT, where + " has more than 4 dimensions");
    t.ndim = (int)sh->items.size();
    uint64_t numel = 1;
    for (int i = 0; i < t.ndim; ++i) {
      const int64_t d = as_index(sh->items[i]);
      if (d < 0 || d > (int64_t)1 << 40) return err(ZIMG_EWEIGHT, where + " has a bad dimension");
      t.shape[i] = d;
      numel *= (uint64_t)d;
      if (numel > ((uint64_t)1 << 40)) return err(ZIMG_EWEIGHT, where + " is too large");
    }
    const int64_t b0 = as_index(off->items[0]), b1 = as_index(off->items[1]);
    if (b0 < 0 || b1 < b0 || (uint64_t)b1 > data_size)
      return err(ZIMG_EWEIGHT, where + ": data_offsets outside the file's data region");
    if ((uint64_t)(b1 - b0) != numel * item)
      return err(ZIMG_EWEIGHT, where + ": data_offsets span " + std::to_string(b1 - b0) + " bytes, the shape needs " +
                                   std::to_string(numel * item));
    t.data = data + b0;
    t.bytes = (size_t)(b1 - b0);
    out.push_back(t);
  }
  return ZIMG_OK;
}

// Every tensor of the files, checked against the table of ``cfg``: each
// name known and met once, shape as in the table, and no entry missing.
int check_all(const zimg_dit_config* cfg, const char* const* paths, int32_t n_paths,
              std::vector<std::unique_ptr<MappedFile>>& files, std::vector<TensorRef>& tensors) {
  if (n_paths < 1 || !paths) return err(ZIMG_EINVAL, "safetensors: no files given");
  int rc = zimg_dit_check_config(cfg);
  if (rc) return rc;
  int32_t n_table = 0;
  if ((rc = zimg_dit_manifest_size(cfg, &n_table))) return rc;
  struct Entry {
    int ndim;
    int64_t shape[4];
    bool seen;
  };
  std::map<std::string, Entry> table;
  for (int32_t i = 0; i < n_table; ++i) {
    const char* name = nullptr;
    Entry e{};
    if ((rc = zimg_dit_manifest_entry(cfg, i, &name, &e.ndim, e.shape))) return rc;
    table[name] = e;
  }
  for (int32_t i = 0; i < n_paths; ++i) {
    files.emplace_back(new MappedFile());
    if ((rc = read_file(paths[i], *files.back(), tensors))) return rc;
  }
  for (const TensorRef& t : tensors) {
    auto it = table.find(t.name);
    if (it == table.end())
      return err(ZIMG_EWEIGHT, "safetensors: unknown tensor '" + t.name + "' (every tensor must belong to the model)");
    if (it->second.seen) return err(ZIMG_EWEIGHT, "safetensors: duplicate tensor '" + t.name + "'");
    it->second.seen = true;
    bool same = t.ndim == it->second.ndim;
    for (int d = 0; same && d < t.ndim; ++d) same = t.shape[d] == it->second.shape[d];
    if (!same) return err(ZIMG_EWEIGHT, "safetensors: tensor '" + t.name + "' has the wrong shape");
  }
  std::string missing;
  int n_missing = 0;
  for (const auto& kv : table)
    if (!kv.second.seen) {
      if (n_missing < 5) missing += (missing.empty() ? "" : ", ") + kv.first;
      ++n_missing;
    }
  if (n_missing)
    return err(ZIMG_EWEIGHT, "safetensors: " + std::to_string(n_missing) + " tensor(s) missing: " + missing +
                                 (n_missing > 5 ? ", ..." : ""));
  return ZIMG_OK;
}

// ---------------------------------------------------------------- SHA-256
// FIPS 180-4: 64 rounds over 512-bit blocks; the round constants are the
// first 32 bits of the fractional parts of the cube roots of the first 64
// primes, the initial state those of the square roots of the first 8.

uint32_t frac_bits(double x) {  // first 32 bits of the fractional part of x
  const double f = x - (double)(uint64_t)x;
  return (uint32_t)(f * 4294967296.0);
}

// the root, corrected to the exact integer part of root * 2^32 by integer
// arithmetic (the double estimate can be off in the last place)
uint32_t root_bits(uint64_t p, int k) {
  double r = k == 2 ? std::sqrt((double)p) : std::cbrt((double)p);
  uint32_t bits = frac_bits(r);
  const uint64_t ip = (uint64_t)r;
  // v = ip * 2^32 + bits must satisfy v^k <= p * 2^(32k) < (v + 1)^k
  auto pow_le = [&](unsigned __int128 v) {
    unsigned __int128 acc = 1;
    for (int i = 0; i < k; ++i) acc *= v;
    return acc;
  };
  const unsigned __int128 target = (unsigned __int128)p << (32 * k);
  unsigned __int128 v = ((unsigned __int128)ip << 32) | bits;
  while (pow_le(v) > target) --v;
  while (pow_le(v + 1) <= target) ++v;
  return (uint32_t)v;
}

struct Sha256 {
  uint32_t h[8], k[64];
  std::vector<unsigned char> buf;
  uint64_t len = 0;
  Sha256() {
    uint64_t primes[64];
    int n = 0;
    for (uint64_t c = 2; n < 64; ++c) {
      bool prime = true;
      for (uint64_t d = 2; d * d <= c; ++d)
        if (c % d == 0) prime = false;
      if (prime) primes[n++] = c;
    }
    for (int i = 0; i < 8; ++i) h[i] = root_bits(primes[i], 2);
    for (int i = 0; i < 64; ++i) k[i] = root_bits(primes[i], 3);
  }
  static uint32_t rotr(uint32_t x, int n) { return (x >> n) | (x << (32 - n)); }
  void block(const unsigned char* p) {
    uint32_t w[64];
    for (int i = 0; i < 16; ++i)
      w[i] = ((uint32_t)p[4 * i] << 24) | ((uint32_t)p[4 * i + 1] << 16) | ((uint32_t)p[4 * i + 2] << 8) | p[4 * i + 3];
    for (int i = 16; i < 64; ++i) {
      const uint32_t s0 = rotr(w[i - 15], 7) ^ rotr(w[i - 15], 18) ^ (w[i - 15] >> 3);
      const uint32_t s1 = rotr(w[i - 2], 17) ^ rotr(w[i - 2], 19) ^ (w[i - 2] >> 10);
      w[i] = w[i - 16] + s0 + w[i - 7] + s1;
    }
    uint32_t a = h[0], b = h[1], c = h[2], d = h[3], e = h[4], f = h[5], g = h[6], hh = h[7];
    for (int i = 0; i < 64; ++i) {
      const uint32_t S1 = rotr(e, 6) ^ rotr(e, 11) ^ rotr(e, 25);
      const uint32_t ch = (e & f) ^ (~e & g);
      const uint32_t t1 = hh + S1 + ch + k[i] + w[i];
      const uint32_t S0 = rotr(a, 2) ^ rotr(a, 13) ^ rotr(a, 22);
      const uint32_t maj = (a & b) ^ (a & c) ^ (b & c);
      const uint32_t t2 = S0 + maj;
      hh = g;
      g = f;
      f = e;
      e = d + t1;
      d = c;
      c = b;
      b = a;
      a = t1 + t2;
    }
    h[0] += a, h[1] += b, h[2] += c, h[3] += d, h[4] += e, h[5] += f, h[6] += g, h[7] += hh;
  }
  void update(const std::string& s) {
    for (unsigned char c : s) {
      buf.push_back(c);
      if (buf.size() == 64) {
        block(buf.data());
        buf.clear();
      }
    }
    len += s.size();
  }
  std::string hex() {
    const uint64_t bits = len * 8;
    buf.push_back(0x80);
    while (buf.size() % 64 != 56) buf.push_back(0);
    for (int i = 7; i >= 0; --i) buf.push_back((unsigned char)(bits >> (8 * i)));
    for (size_t i = 0; i < buf.size(); i += 64) block(buf.data() + i);
    char out[65];
    for (int i = 0; i < 8; ++i) std::snprintf(out + 8 * i, 9, "%08x", h[i]);
    return std::string(out, 64);
  }
};

}  // namespace

extern "C" {

int zimg_safetensors_check(const zimg_dit_config* cfg, const char* const* paths, int32_t n_paths,
                           int32_t* n_tensors) {
  std::vector<std::unique_ptr<MappedFile>> files;
  std::vector<TensorRef> tensors;
  const int rc = check_all(cfg, paths, n_paths, files, tensors);
  if (rc) return rc;
  if (n_tensors) *n_tensors = (int32_t)tensors.size();
  return ZIMG_OK;
}

int zimg_dit_load_safetensors(zimg_dit* h, const char* const* paths, int32_t n_paths) {
  const zimg_dit_config* cfg = zimg::handle_config(h);
  if (!cfg) return err(ZIMG_EINVAL, "handle is NULL");
  if (zimg::handle_finalized(h)) return err(ZIMG_ESTATE, "safetensors: the handle's weights are already final");
  std::vector<std::unique_ptr<MappedFile>> files;
  std::vector<TensorRef> tensors;
  int rc = check_all(cfg, paths, n_paths, files, tensors);
  if (rc) return rc;
  for (const TensorRef& t : tensors) {
    zimg_tensor z{};
    z.name = t.name.c_str();
    z.data = t.data;
    z.dtype = t.dtype;
    z.ndim = t.ndim;
    for (int d = 0; d < 4; ++d) z.shape[d] = t.shape[d];
    if ((rc = zimg_dit_set_weight(h, &z))) return rc;
  }
  return ZIMG_OK;
}

int zimg_dit_create_from_safetensors(const zimg_dit_config* cfg, const char* const* paths, int32_t n_paths,
                                     void* stream, zimg_dit** out) {
  if (!out) return err(ZIMG_EINVAL, "out is NULL");
  *out = nullptr;
  {  // every file is validated before any device memory is taken
    std::vector<std::unique_ptr<MappedFile>> files;
    std::vector<TensorRef> tensors;
    const int rc = check_all(cfg, paths, n_paths, files, tensors);
    if (rc) return rc;
  }
  zimg_dit* h = nullptr;
  int rc = zimg_dit_alloc(cfg, stream, &h);
  if (rc) return rc;
  rc = zimg_dit_load_safetensors(h, paths, n_paths);
  if (!rc) rc = zimg_dit_finalize(h);
  if (rc) {
    const std::string msg = zimg_last_error();
    zimg_dit_destroy(h);
    return err(rc, msg);
  }
  *out = h;
  return ZIMG_OK;
}

int zimg_dit_manifest_digest(const zimg_dit_config* cfg, char hex[65]) {
  if (!hex) return err(ZIMG_EINVAL, "output is NULL");
  int32_t n = 0;
  int rc = zimg_dit_check_config(cfg);
  if (rc) return rc;
  if ((rc = zimg_dit_manifest_size(cfg, &n))) return rc;
  std::vector<std::string> names;
  for (int32_t i = 0; i < n; ++i) {
    const char* name = nullptr;
    int32_t nd = 0;
    int64_t shape[4];
    if ((rc = zimg_dit_manifest_entry(cfg, i, &name, &nd, shape))) return rc;
    names.emplace_back(name);
  }
  std::sort(names.begin(), names.end());
  Sha256 sha;
  for (const std::string& s : names) sha.update(s + "\n");
  const std::string d = sha.hex();
  std::memcpy(hex, d.c_str(), 65);
  return ZIMG_OK;
}

}  // extern "C"
