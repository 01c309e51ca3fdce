// Header-only checkpoint inspection: the step before the projection's weights
// exist on the device.  A safetensors file starts with an 8-byte little-endian
// header length and a JSON object mapping tensor names to {dtype, shape,
// data_offsets}; everything after it is tensor bytes, which are never read
// here.  The checkpoint's quantization_config (from its config JSON) gives the
// declaration the units are validated against.
//
// ("th#1803: the consumer half of the layout gate", sections "What lands":
//  verification from safetensors headers alone, before any weight byte is read;
//  "Why the refusals matter more than the load": row-wise trees, transposed or
//  mis-blocked grids, FP8 weights without a scale and rank-1 scales are refused
//  by name; "Proof": dense trees are refused.  "Qwen checkpoints with block FP8
//  weights", layout paragraph: quant_method fp8 with weight_block_size
//  [128,128], leaves weight and weight_scale_inv; mixed BF16/F16 tensors such
//  as the output head keep their own representation.)
#include <cerrno>
#include <cstdarg>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <map>
#include <memory>
#include <string>
#include <vector>

#include "bsf8_internal.h"

namespace bsf8 {
namespace {

bsf8_status ifail(bsf8_status s, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  set_error("%s", buf);
  return s;
}

// ---------------------------------------------------------------- JSON
// A small recursive-descent reader: objects (key order kept), arrays,
// strings (escapes decoded; \u escapes to UTF-8), numbers (integers exact
// when they fit int64, others as double only), true / false / null.
struct Json {
  enum Kind { NUL, BOOL, NUM, STR, ARR, OBJ } kind = NUL;
  bool b = false;
  double num = 0.0;
  int64_t inum = 0;
  bool is_int = false;
  std::string str;
  std::vector<Json> arr;
  std::vector<std::pair<std::string, Json>> obj;

  const Json* get(const char* key) const {
    if (kind != OBJ) return nullptr;
    for (const auto& kv : obj)
      if (kv.first == key) return &kv.second;
    return nullptr;
  }
};

class Parser {
 public:
  Parser(const char* p, size_t n) : p_(p), end_(p + n) {}
  bool parse(Json& out) {
    if (!value(out, 0)) return false;
    ws();
    return p_ == end_ || fail("trailing bytes after the JSON value");
  }
  const std::string& error() const { return err_; }

 private:
  const char* p_;
  const char* end_;
  std::string err_;

  bool fail(const char* what) {
    if (err_.empty()) err_ = what;
    return false;
  }
  void ws() {
    while (p_ < end_ && (*p_ == ' ' || *p_ == '\t' || *p_ == '\n' || *p_ == '\r')) ++p_;
  }
  bool lit(const char* s) {
    const size_t n = std::strlen(s);
    if (size_t(end_ - p_) < n || std::strncmp(p_, s, n) != 0) return fail("bad literal");
    p_ += n;
    return true;
  }
  static void utf8(std::string& s, uint32_t cp) {
    if (cp < 0x80) {
      s += char(cp);
    } else if (cp < 0x800) {
      s += char(0xC0 | (cp >> 6));
      s += char(0x80 | (cp & 0x3F));
    } else if (cp < 0x10000) {
      s += char(0xE0 | (cp >> 12));
      s += char(0x80 | ((cp >> 6) & 0x3F));
      s += char(0x80 | (cp & 0x3F));
    } else {
      s += char(0xF0 | (cp >> 18));
      s += char(0x80 | ((cp >> 12) & 0x3F));
      s += char(0x80 | ((cp >> 6) & 0x3F));
      s += char(0x80 | (cp & 0x3F));
    }
  }
  bool hex4(uint32_t& v) {
    if (end_ - p_ < 4) return fail("short \\u escape");
    v = 0;
    for (int i = 0; i < 4; ++i) {
      const char c = *p_++;
      v <<= 4;
      if (c >= '0' && c <= '9') v |= uint32_t(c - '0');
      else if (c >= 'a' && c <= 'f') v |= uint32_t(c - 'a' + 10);
      else if (c >= 'A' && c <= 'F') v |= uint32_t(c - 'A' + 10);
      else return fail("bad \\u escape");
    }
    return true;
  }
  bool string(std::string& s) {
    if (p_ >= end_ || *p_ != '"') return fail("expected a string");
    ++p_;
    while (p_ < end_ && *p_ != '"') {
      const char c = *p_++;
      if (static_cast<unsigned char>(c) < 0x20) return fail("control character in a string");
      if (c != '\\') {
        s += c;
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
          uint32_t cp;
          if (!hex4(cp)) return false;
          if (cp >= 0xD800 && cp < 0xDC00) {   // surrogate pair
            uint32_t lo;
            if (end_ - p_ < 2 || p_[0] != '\\' || p_[1] != 'u') return fail("lone surrogate");
            p_ += 2;
            if (!hex4(lo) || lo < 0xDC00 || lo >= 0xE000) return fail("bad surrogate pair");
            cp = 0x10000 + ((cp - 0xD800) << 10) + (lo - 0xDC00);
          }
          utf8(s, cp);
          break;
        }
        default: return fail("bad escape");
      }
    }
    if (p_ >= end_) return fail("unterminated string");
    ++p_;
    return true;
  }
  bool number(Json& out) {
    const char* s = p_;
    if (p_ < end_ && *p_ == '-') ++p_;
    bool digits = false, frac = false;
    while (p_ < end_ && *p_ >= '0' && *p_ <= '9') ++p_, digits = true;
    if (p_ < end_ && *p_ == '.') {
      frac = true;
      ++p_;
      while (p_ < end_ && *p_ >= '0' && *p_ <= '9') ++p_;
    }
    if (p_ < end_ && (*p_ == 'e' || *p_ == 'E')) {
      frac = true;
      ++p_;
      if (p_ < end_ && (*p_ == '+' || *p_ == '-')) ++p_;
      while (p_ < end_ && *p_ >= '0' && *p_ <= '9') ++p_;
    }
    if (!digits) return fail("bad number");
    const std::string t(s, p_);
    out.kind = Json::NUM;
    out.num = std::strtod(t.c_str(), nullptr);
    if (!frac) {
      // an integer is exact only when it fits int64: strtoll reports ERANGE
      // (and clamps) for anything larger, which then stays a plain number
      errno = 0;
      const long long v = std::strtoll(t.c_str(), nullptr, 10);
      if (errno != ERANGE) {
        out.is_int = true;
        out.inum = v;
      }
    }
    return true;
  }
  bool value(Json& out, int depth) {
    if (depth > 64) return fail("nesting too deep");
    ws();
    if (p_ >= end_) return fail("unexpected end");
    const char c = *p_;
    if (c == '{') {
      ++p_;
      out.kind = Json::OBJ;
      ws();
      if (p_ < end_ && *p_ == '}') return ++p_, true;
      for (;;) {
        ws();
        std::string key;
        if (!string(key)) return false;
        ws();
        if (p_ >= end_ || *p_ != ':') return fail("expected ':'");
        ++p_;
        out.obj.emplace_back(std::move(key), Json());
        if (!value(out.obj.back().second, depth + 1)) return false;
        ws();
        if (p_ < end_ && *p_ == ',') {
          ++p_;
          continue;
        }
        if (p_ < end_ && *p_ == '}') return ++p_, true;
        return fail("expected ',' or '}'");
      }
    }
    if (c == '[') {
      ++p_;
      out.kind = Json::ARR;
      ws();
      if (p_ < end_ && *p_ == ']') return ++p_, true;
      for (;;) {
        out.arr.emplace_back();
        if (!value(out.arr.back(), depth + 1)) return false;
        ws();
        if (p_ < end_ && *p_ == ',') {
          ++p_;
          continue;
        }
        if (p_ < end_ && *p_ == ']') return ++p_, true;
        return fail("expected ',' or ']'");
      }
    }
    if (c == '"') {
      out.kind = Json::STR;
      return string(out.str);
    }
    if (c == 't') return out.kind = Json::BOOL, out.b = true, lit("true");
    if (c == 'f') return out.kind = Json::BOOL, out.b = false, lit("false");
    if (c == 'n') return out.kind = Json::NUL, lit("null");
    return number(out);
  }
};

// ---------------------------------------------------------------- tensors

int32_t dtype_of(const std::string& s) {
  if (s == "F8_E4M3") return BSF8_DT_F8_E4M3;
  if (s == "F8_E5M2") return BSF8_DT_F8_E5M2;
  if (s == "BF16") return BSF8_DT_BF16;
  if (s == "F16") return BSF8_DT_F16;
  if (s == "F32") return BSF8_DT_F32;
  if (s == "U8") return BSF8_DT_U8;
  return BSF8_DT_OTHER;
}

// Bytes per element of a safetensors dtype name, 0 when the name is unknown.
int64_t dtype_bytes(const std::string& s) {
  static const struct { const char* name; int64_t bytes; } table[] = {
      {"BOOL", 1}, {"U8", 1}, {"I8", 1}, {"F8_E4M3", 1}, {"F8_E5M2", 1}, {"I16", 2}, {"U16", 2}, {"F16", 2},
      {"BF16", 2}, {"I32", 4}, {"U32", 4}, {"F32", 4}, {"I64", 8}, {"U64", 8}, {"F64", 8}};
  for (const auto& e : table)
    if (s == e.name) return e.bytes;
  return 0;
}

// The header's own bounds: every dimension below 2^31 (the validator and the
// kernels index rows and columns with 32-bit integers).
constexpr int64_t kMaxDim = int64_t(INT32_MAX);

struct Entry {
  int32_t dtype;
  int32_t rank;
  int64_t shape[4];
  int64_t begin;  // offset of the tensor's bytes from the file start
};

bool ends_with(const std::string& s, const char* suffix, std::string* head) {
  const size_t n = std::strlen(suffix);
  if (s.size() < n || s.compare(s.size() - n, n, suffix) != 0) return false;
  if (head) *head = s.substr(0, s.size() - n);
  return true;
}

bsf8_tensor_desc desc_of(const Entry& e) {
  bsf8_tensor_desc d{};
  d.dtype = e.dtype;
  d.rank = e.rank;
  for (int i = 0; i < 4; ++i) d.shape[i] = i < e.rank ? e.shape[i] : 0;
  d.data = nullptr;
  return d;
}

}  // namespace
}  // namespace bsf8

using namespace bsf8;

static_assert(sizeof(bsf8_unit) == 432, "bsf8_unit layout is part of the ABI");

extern "C" {

bsf8_status bsf8_parse_quant_config(const char* json_text, bsf8_decl* out) {
  if (json_text == nullptr || out == nullptr) return ifail(BSF8_E_INVALID_ARG, "null argument");
  Json root;
  Parser ps(json_text, std::strlen(json_text));
  if (!ps.parse(root)) return ifail(BSF8_E_INVALID_ARG, "quantization config JSON: %s", ps.error().c_str());
  if (root.kind != Json::OBJ) return ifail(BSF8_E_INVALID_ARG, "quantization config JSON is not an object");
  const Json* q = root.get("quantization_config");
  if (q == nullptr) q = &root;   // the quantization_config object itself
  if (q->kind != Json::OBJ) return ifail(BSF8_E_INVALID_ARG, "quantization_config is not an object");
  const Json* qm = q->get("quant_method");
  if (qm == nullptr || qm->kind != Json::STR) return ifail(BSF8_E_DECL, "no quant_method string");
  out->quant_method_fp8 = qm->str == "fp8" ? 1 : 0;
  out->block_n = out->block_k = 0;
  const Json* bs = q->get("weight_block_size");
  if (bs != nullptr && bs->kind != Json::NUL) {
    if (bs->kind != Json::ARR || bs->arr.size() != 2 || !bs->arr[0].is_int || !bs->arr[1].is_int ||
        bs->arr[0].inum <= 0 || bs->arr[1].inum <= 0 || bs->arr[0].inum > INT32_MAX || bs->arr[1].inum > INT32_MAX)
      return ifail(BSF8_E_DECL, "weight_block_size is not a pair of positive integers");
    out->block_n = static_cast<int32_t>(bs->arr[0].inum);
    out->block_k = static_cast<int32_t>(bs->arr[1].inum);
  }
  return BSF8_OK;
}

bsf8_status bsf8_inspect_safetensors(const char* path, const bsf8_decl* decl, bsf8_unit* units, int32_t capacity,
                                     int32_t* n_units) {
  if (path == nullptr || decl == nullptr || n_units == nullptr || capacity < 0 || (units == nullptr && capacity > 0))
    return ifail(BSF8_E_INVALID_ARG, "null argument or negative capacity");
  *n_units = 0;
  std::unique_ptr<FILE, int (*)(FILE*)> f(std::fopen(path, "rb"), &std::fclose);
  if (!f) return ifail(BSF8_E_INVALID_ARG, "cannot open %s", path);
  unsigned char len8[8];
  if (std::fread(len8, 1, 8, f.get()) != 8) return ifail(BSF8_E_INVALID_ARG, "%s: shorter than the 8-byte header length", path);
  uint64_t hlen = 0;
  for (int i = 7; i >= 0; --i) hlen = (hlen << 8) | len8[i];
  if (hlen < 2 || hlen > BSF8_SAFETENSORS_MAX_HEADER)
    return ifail(BSF8_E_INVALID_ARG, "%s: header length %llu outside [2, %d]", path, (unsigned long long)hlen,
                BSF8_SAFETENSORS_MAX_HEADER);
  std::string text(hlen, '\0');
  if (std::fread(&text[0], 1, hlen, f.get()) != hlen) return ifail(BSF8_E_INVALID_ARG, "%s: truncated header", path);
  f.reset();   // nothing past the header is read

  Json root;
  Parser ps(text.data(), text.size());
  if (!ps.parse(root)) return ifail(BSF8_E_INVALID_ARG, "%s: header JSON: %s", path, ps.error().c_str());
  if (root.kind != Json::OBJ) return ifail(BSF8_E_INVALID_ARG, "%s: header is not a JSON object", path);

  std::map<std::string, Entry> byname;
  std::vector<std::string> order;
  for (const auto& kv : root.obj) {
    if (kv.first == "__metadata__") continue;
    const Json& t = kv.second;
    const Json* dt = t.get("dtype");
    const Json* sh = t.get("shape");
    const Json* off = t.get("data_offsets");
    if (dt == nullptr || dt->kind != Json::STR || sh == nullptr || sh->kind != Json::ARR || off == nullptr ||
        off->kind != Json::ARR || off->arr.size() != 2 || !off->arr[0].is_int || !off->arr[1].is_int)
      return ifail(BSF8_E_INVALID_ARG, "%s: tensor '%s' lacks dtype / shape / data_offsets", path, kv.first.c_str());
    Entry e{};
    e.dtype = dtype_of(dt->str);
    e.rank = static_cast<int32_t>(sh->arr.size());
    if (e.rank > 4) e.rank = 4 + 1;   // reported as rank 5: refused below like any other bad rank
    // every dimension an integer in [0, 2^31); the element count, with
    // overflow checks, for the span check below
    int64_t numel = 1;
    for (size_t i = 0; i < sh->arr.size(); ++i) {
      const Json& d = sh->arr[i];
      if (!d.is_int || d.inum < 0 || d.inum > kMaxDim)
        return ifail(BSF8_E_INVALID_ARG, "%s: tensor '%s' has a bad shape (dimension %zu not an integer in [0, 2^31))",
                     path, kv.first.c_str(), i);
      if (i < 4) e.shape[i] = d.inum;
      if (numel != 0 && d.inum > INT64_MAX / numel)
        return ifail(BSF8_E_INVALID_ARG, "%s: tensor '%s': element count overflows", path, kv.first.c_str());
      numel *= d.inum;
    }
    // data_offsets [begin, end) relative to the end of the header: 0 <= begin
    // <= end, and end - begin is the tensor's byte size when its dtype is known
    const int64_t b0 = off->arr[0].inum, b1 = off->arr[1].inum;
    if (b0 < 0 || b1 < b0 || b1 > INT64_MAX - int64_t(8 + hlen))
      return ifail(BSF8_E_INVALID_ARG, "%s: tensor '%s' has data_offsets [%lld, %lld] out of order or range", path,
                   kv.first.c_str(), (long long)b0, (long long)b1);
    const int64_t esz = dtype_bytes(dt->str);
    if (esz > 0 && (numel > INT64_MAX / esz || b1 - b0 != numel * esz))
      return ifail(BSF8_E_INVALID_ARG, "%s: tensor '%s' spans %lld bytes, its dtype and shape need %lld", path,
                   kv.first.c_str(), (long long)(b1 - b0), (long long)(numel > INT64_MAX / esz ? -1 : numel * esz));
    e.begin = int64_t(8 + hlen) + b0;
    byname[kv.first] = e;
    order.push_back(kv.first);
  }

  // A unit is a "<prefix>.weight" tensor stored as FP8, or one with a scale
  // sibling.  Other tensors (dense BF16/F16 weights such as the output head,
  // norms, biases) keep their own representation and are not units.
  int32_t count = 0;
  int dense_2d = 0;
  bsf8_status first_bad = BSF8_OK;
  char first_msg[320] = "";
  for (const std::string& name : order) {
    std::string prefix;
    if (!ends_with(name, ".weight", &prefix)) continue;
    const Entry& w = byname[name];
    const auto si = byname.find(prefix + ".weight_scale_inv");
    const auto sc = byname.find(prefix + ".weight_scale");
    const bool fp8 = w.dtype == BSF8_DT_F8_E4M3 || w.dtype == BSF8_DT_F8_E5M2;
    if (!fp8 && si == byname.end() && sc == byname.end()) {
      if (w.rank == 2) ++dense_2d;
      continue;
    }
    bsf8_member_desc m{};
    m.weight = desc_of(w);
    bsf8_tensor_desc d_si{}, d_sc{};
    if (si != byname.end()) d_si = desc_of(si->second), m.scale_inv = &d_si;
    if (sc != byname.end()) d_sc = desc_of(sc->second), m.scale = &d_sc;
    // one-member validation; its detail is kept for the first refusal
    const bsf8_status st = bsf8_validate(decl, &m, 1);
    if (st != BSF8_OK && first_bad == BSF8_OK) {
      first_bad = st;
      std::snprintf(first_msg, sizeof(first_msg), "%s: %s", prefix.c_str(), bsf8_last_error());
    }
    if (count < capacity) {
      bsf8_unit& u = units[count];
      std::memset(&u, 0, sizeof(u));
      std::snprintf(u.prefix, sizeof(u.prefix), "%s", prefix.c_str());
      u.prefix_truncated = prefix.size() >= sizeof(u.prefix) ? 1 : 0;
      u.weight = m.weight;
      u.has_scale_inv = m.scale_inv != nullptr;
      u.has_scale = m.scale != nullptr;
      if (u.has_scale_inv) u.scale_inv = d_si;
      if (u.has_scale) u.scale = d_sc;
      u.weight_offset = w.begin;
      u.scale_offset = u.has_scale_inv ? si->second.begin : u.has_scale ? sc->second.begin : -1;
      u.status = st;
    }
    ++count;
  }
  *n_units = count;
  if (first_bad != BSF8_OK) return ifail(first_bad, "%s", first_msg);
  if (count == 0 && dense_2d > 0)
    return ifail(BSF8_E_WEIGHT_DTYPE, "%s: a dense tree (no FP8 weight) under an fp8 declaration", path);
  return BSF8_OK;
}

}  // extern "C"
