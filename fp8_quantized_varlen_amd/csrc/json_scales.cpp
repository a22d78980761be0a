// Static-scale file reader: a small strict JSON parser (no dependencies).
//
// File shape (vLLM page "FP8 ViT Encoder Attention", Scale File Format): a
// JSON object mapping attention-layer names such as
// "visual.blocks.0.attn.attn" to objects {"q": .., "k": .., "v": ..}; the keys
// "q_scale", "k_scale", "v_scale" are accepted as aliases. The values already
// include the calibration margin (Calibrate-Once Reuse Workflow section).
//
// The writer closes the calibrate-once loop in the library: it stores one
// layer's calibrated values in such a file, keeping every other entry.
#include <cerrno>
#include <clocale>
#include <cmath>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <locale.h>
#include <map>
#include <memory>
#include <string>
#include <unistd.h>
#include <vector>

#include "fp8vit.h"

namespace {

locale_t c_locale() {
  static locale_t c_loc = newlocale(LC_NUMERIC_MASK, "C", (locale_t)0);
  return c_loc;
}

struct JValue {
  enum Kind { Null, Bool, Number, String, Array, Object } kind = Null;
  double num = 0.0;
  std::string raw;  // a number's text as it was read
  bool b = false;
  std::string str;
  std::vector<JValue> arr;
  std::vector<std::pair<std::string, JValue>> obj;  // insertion order; duplicates kept
};

class Parser {
 public:
  Parser(const char* p, const char* e) : p_(p), e_(e) {}
  bool parse_document(JValue& out) {
    ws();
    if (!value(out, 0)) return false;
    ws();
    return p_ == e_;
  }

 private:
  const char* p_;
  const char* e_;
  static constexpr int kMaxDepth = 64;

  void ws() {
    while (p_ < e_ && (*p_ == ' ' || *p_ == '\t' || *p_ == '\n' || *p_ == '\r')) ++p_;
  }
  bool lit(const char* s) {
    size_t n = strlen(s);
    if ((size_t)(e_ - p_) < n || memcmp(p_, s, n) != 0) return false;
    p_ += n;
    return true;
  }
  static void put_utf8(std::string& s, unsigned cp) {
    if (cp < 0x80) {
      s.push_back((char)cp);
    } else if (cp < 0x800) {
      s.push_back((char)(0xC0 | (cp >> 6)));
      s.push_back((char)(0x80 | (cp & 0x3F)));
    } else if (cp < 0x10000) {
      s.push_back((char)(0xE0 | (cp >> 12)));
      s.push_back((char)(0x80 | ((cp >> 6) & 0x3F)));
      s.push_back((char)(0x80 | (cp & 0x3F)));
    } else {
      s.push_back((char)(0xF0 | (cp >> 18)));
      s.push_back((char)(0x80 | ((cp >> 12) & 0x3F)));
      s.push_back((char)(0x80 | ((cp >> 6) & 0x3F)));
      s.push_back((char)(0x80 | (cp & 0x3F)));
    }
  }
  bool hex4(unsigned& v) {
    if (e_ - p_ < 4) return false;
    v = 0;
    for (int i = 0; i < 4; ++i) {
      char c = *p_++;
      v <<= 4;
      if (c >= '0' && c <= '9') v |= (unsigned)(c - '0');
      else if (c >= 'a' && c <= 'f') v |= (unsigned)(c - 'a' + 10);
      else if (c >= 'A' && c <= 'F') v |= (unsigned)(c - 'A' + 10);
      else return false;
    }
    return true;
  }
  bool string(std::string& s) {
    if (p_ >= e_ || *p_ != '"') return false;
    ++p_;
    while (p_ < e_) {
      unsigned char c = (unsigned char)*p_++;
      if (c == '"') return true;
      if (c < 0x20) return false;
      if (c != '\\') {
        s.push_back((char)c);
        continue;
      }
      if (p_ >= e_) return false;
      char esc = *p_++;
      switch (esc) {
        case '"': s.push_back('"'); break;
        case '\\': s.push_back('\\'); break;
        case '/': s.push_back('/'); break;
        case 'b': s.push_back('\b'); break;
        case 'f': s.push_back('\f'); break;
        case 'n': s.push_back('\n'); break;
        case 'r': s.push_back('\r'); break;
        case 't': s.push_back('\t'); break;
        case 'u': {
          unsigned cp;
          if (!hex4(cp)) return false;
          if (cp >= 0xD800 && cp <= 0xDBFF) {
            unsigned lo;
            if (e_ - p_ < 6 || p_[0] != '\\' || p_[1] != 'u') return false;
            p_ += 2;
            if (!hex4(lo) || lo < 0xDC00 || lo > 0xDFFF) return false;
            cp = 0x10000 + ((cp - 0xD800) << 10) + (lo - 0xDC00);
          } else if (cp >= 0xDC00 && cp <= 0xDFFF) {
            return false;
          }
          put_utf8(s, cp);
          break;
        }
        default: return false;
      }
    }
    return false;
  }
  bool number(double& v, std::string& raw) {
    const char* start = p_;
    if (p_ < e_ && *p_ == '-') ++p_;
    if (p_ >= e_) return false;
    if (*p_ == '0') {
      ++p_;
    } else if (*p_ >= '1' && *p_ <= '9') {
      while (p_ < e_ && *p_ >= '0' && *p_ <= '9') ++p_;
    } else {
      return false;
    }
    if (p_ < e_ && *p_ == '.') {
      ++p_;
      if (p_ >= e_ || !(*p_ >= '0' && *p_ <= '9')) return false;
      while (p_ < e_ && *p_ >= '0' && *p_ <= '9') ++p_;
    }
    if (p_ < e_ && (*p_ == 'e' || *p_ == 'E')) {
      ++p_;
      if (p_ < e_ && (*p_ == '+' || *p_ == '-')) ++p_;
      if (p_ >= e_ || !(*p_ >= '0' && *p_ <= '9')) return false;
      while (p_ < e_ && *p_ >= '0' && *p_ <= '9') ++p_;
    }
    std::string tok(start, p_);
    raw = tok;
    // strtod in the "C" locale: the grammar above already fixed the syntax.
    const locale_t c_loc = c_locale();
    char* end = nullptr;
    v = c_loc ? strtod_l(tok.c_str(), &end, c_loc) : strtod(tok.c_str(), &end);
    return end && *end == '\0';
  }
  bool value(JValue& out, int depth) {
    if (depth > kMaxDepth || p_ >= e_) return false;
    char c = *p_;
    if (c == '{') {
      ++p_;
      out.kind = JValue::Object;
      ws();
      if (p_ < e_ && *p_ == '}') { ++p_; return true; }
      while (true) {
        ws();
        std::string key;
        if (!string(key)) return false;
        ws();
        if (p_ >= e_ || *p_ != ':') return false;
        ++p_;
        ws();
        JValue v;
        if (!value(v, depth + 1)) return false;
        out.obj.emplace_back(std::move(key), std::move(v));
        ws();
        if (p_ < e_ && *p_ == ',') { ++p_; continue; }
        if (p_ < e_ && *p_ == '}') { ++p_; return true; }
        return false;
      }
    }
    if (c == '[') {
      ++p_;
      out.kind = JValue::Array;
      ws();
      if (p_ < e_ && *p_ == ']') { ++p_; return true; }
      while (true) {
        ws();
        JValue v;
        if (!value(v, depth + 1)) return false;
        out.arr.push_back(std::move(v));
        ws();
        if (p_ < e_ && *p_ == ',') { ++p_; continue; }
        if (p_ < e_ && *p_ == ']') { ++p_; return true; }
        return false;
      }
    }
    if (c == '"') { out.kind = JValue::String; return string(out.str); }
    if (c == 't') { out.kind = JValue::Bool; out.b = true; return lit("true"); }
    if (c == 'f') { out.kind = JValue::Bool; out.b = false; return lit("false"); }
    if (c == 'n') { out.kind = JValue::Null; return lit("null"); }
    out.kind = JValue::Number;
    return number(out.num, out.raw);
  }
};

const JValue* find_last(const JValue& obj, const char* key) {
  const JValue* r = nullptr;
  for (const auto& kv : obj.obj)
    if (kv.first == key) r = &kv.second;
  return r;
}

// Whole file into `buf`; false with errno kept when it cannot be opened or read.
bool read_file(const char* path, std::string& buf) {
  FILE* f = fopen(path, "rb");
  if (!f) return false;
  char tmp[65536];
  size_t n;
  while ((n = fread(tmp, 1, sizeof(tmp), f)) > 0) buf.append(tmp, n);
  const bool err = ferror(f) != 0;
  fclose(f);
  return !err;
}

const char* skip_bom(const std::string& buf) {
  const char* b = buf.data();
  if (buf.size() >= 3 && (unsigned char)b[0] == 0xEF && (unsigned char)b[1] == 0xBB && (unsigned char)b[2] == 0xBF)
    b += 3;
  return b;
}

// ---- writer ----------------------------------------------------------------

// Shortest "%.{p}g" text of a float that reads back (strtod, then rounding to
// float, as the loader reads it) to the same value; p <= 9 always suffices.
// Formatting and parsing both run in the "C" locale, whatever the caller's
// locale is.
std::string format_float(float v) {
  locale_t loc = c_locale();
  locale_t old = loc ? uselocale(loc) : (locale_t)0;
  char text[40];
  for (int p = 1; p <= 9; ++p) {
    snprintf(text, sizeof(text), "%.*g", p, (double)v);
    char* end = nullptr;
    const double back = loc ? strtod_l(text, &end, loc) : strtod(text, &end);
    if ((float)back == v) break;
  }
  if (old) uselocale(old);
  return text;
}

void write_string(std::string& o, const std::string& s) {
  o.push_back('"');
  for (unsigned char c : s) {
    if (c == '"') o += "\\\"";
    else if (c == '\\') o += "\\\\";
    else if (c < 0x20) {
      char esc[8];
      snprintf(esc, sizeof(esc), "\\u%04x", (unsigned)c);
      o += esc;
    } else {
      o.push_back((char)c);
    }
  }
  o.push_back('"');
}

// Compact serialization; object keys keep their order (duplicates included)
// and numbers their text as read.
void write_value(std::string& o, const JValue& v) {
  switch (v.kind) {
    case JValue::Null: o += "null"; break;
    case JValue::Bool: o += v.b ? "true" : "false"; break;
    case JValue::Number: o += v.raw; break;
    case JValue::String: write_string(o, v.str); break;
    case JValue::Array:
      o.push_back('[');
      for (size_t i = 0; i < v.arr.size(); ++i) {
        if (i) o += ", ";
        write_value(o, v.arr[i]);
      }
      o.push_back(']');
      break;
    case JValue::Object:
      o.push_back('{');
      for (size_t i = 0; i < v.obj.size(); ++i) {
        if (i) o += ", ";
        write_string(o, v.obj[i].first);
        o += ": ";
        write_value(o, v.obj[i].second);
      }
      o.push_back('}');
      break;
  }
}

bool only_whitespace(const char* b, const char* e) {
  for (; b < e; ++b)
    if (!(*b == ' ' || *b == '\t' || *b == '\n' || *b == '\r')) return false;
  return true;
}

}  // namespace

extern "C" fp8vit_status fp8vit_load_static_scales(const char* json_path, const char* layer_name,
                                                   float out_qkv[3]) {
  if (!json_path || !layer_name || !out_qkv) return FP8VIT_ERR_INVALID_ARGUMENT;
  std::string buf;
  if (!read_file(json_path, buf)) return FP8VIT_ERR_IO;
  const char* b = skip_bom(buf);  // UTF-8 byte order mark
  const char* e = buf.data() + buf.size();
  JValue root;
  Parser p(b, e);
  if (!p.parse_document(root) || root.kind != JValue::Object) return FP8VIT_ERR_PARSE;
  const JValue* layer = find_last(root, layer_name);
  if (!layer) return FP8VIT_ERR_NOT_FOUND;
  if (layer->kind != JValue::Object) return FP8VIT_ERR_PARSE;
  static const char* plain[3] = {"q", "k", "v"};
  static const char* alias[3] = {"q_scale", "k_scale", "v_scale"};
  float vals[3];
  for (int i = 0; i < 3; ++i) {
    const JValue* a = find_last(*layer, plain[i]);
    const JValue* c = find_last(*layer, alias[i]);
    if (a && c) return FP8VIT_ERR_INVALID_ARGUMENT;
    const JValue* v = a ? a : c;
    if (!v) return FP8VIT_ERR_NOT_FOUND;
    if (v->kind != JValue::Number) return FP8VIT_ERR_INVALID_ARGUMENT;
    const float fv = (float)v->num;
    if (!std::isfinite(v->num) || !std::isfinite(fv) || !(fv > 0.0f)) return FP8VIT_ERR_INVALID_ARGUMENT;
    vals[i] = fv;
  }
  for (int i = 0; i < 3; ++i) out_qkv[i] = vals[i];
  return FP8VIT_OK;
}

extern "C" fp8vit_status fp8vit_save_static_scales(const char* json_path, const char* layer_name,
                                                   const float values_qkv[3]) {
  if (!json_path || !layer_name || !values_qkv) return FP8VIT_ERR_INVALID_ARGUMENT;
  for (int i = 0; i < 3; ++i)
    if (!std::isfinite(values_qkv[i]) || !(values_qkv[i] > 0.0f)) return FP8VIT_ERR_INVALID_ARGUMENT;

  // Existing entries are kept; a missing file starts an empty object.
  JValue root;
  root.kind = JValue::Object;
  std::string buf;
  if (read_file(json_path, buf)) {
    const char* b = skip_bom(buf);
    const char* e = buf.data() + buf.size();
    if (!only_whitespace(b, e)) {
      Parser p(b, e);
      if (!p.parse_document(root) || root.kind != JValue::Object) return FP8VIT_ERR_PARSE;
    }
  } else if (errno != ENOENT) {
    return FP8VIT_ERR_IO;
  }

  std::string entry = "{\"q\": " + format_float(values_qkv[0]) + ", \"k\": " +
                      format_float(values_qkv[1]) + ", \"v\": " + format_float(values_qkv[2]) + "}";
  // One top-level entry per line; the layer replaces its first occurrence (and
  // drops later duplicates), or is appended.
  std::string out = "{";
  bool placed = false, first = true;
  auto line = [&](const std::string& key, const std::string& val) {
    out += first ? "\n  " : ",\n  ";
    first = false;
    write_string(out, key);
    out += ": ";
    out += val;
  };
  for (const auto& kv : root.obj) {
    if (kv.first == layer_name) {
      if (!placed) line(kv.first, entry);
      placed = true;
      continue;
    }
    std::string val;
    write_value(val, kv.second);
    line(kv.first, val);
  }
  if (!placed) line(layer_name, entry);
  out += first ? "}\n" : "\n}\n";

  // Write a sibling file, then rename it over the target: readers see the old
  // or the new file, never a partial one.
  const std::string tmp = std::string(json_path) + ".tmp." + std::to_string((long)getpid());
  FILE* f = fopen(tmp.c_str(), "wb");
  if (!f) return FP8VIT_ERR_IO;
  bool ok = fwrite(out.data(), 1, out.size(), f) == out.size();
  ok = (fflush(f) == 0) && ok;
  ok = (fclose(f) == 0) && ok;
  if (ok) ok = rename(tmp.c_str(), json_path) == 0;
  if (!ok) {
    remove(tmp.c_str());
    return FP8VIT_ERR_IO;
  }
  return FP8VIT_OK;
}
