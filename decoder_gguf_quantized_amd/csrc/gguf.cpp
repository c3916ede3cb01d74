// gguf.cpp -- model files: the GGUF container and architecture definitions.
//
// Host code only.  A GGUF file is mapped read-only; its metadata gives the
// model's shape and its tensor table the weights, which go to
// qdec_load_weights as borrowed pointers into the mapping.  Which block the
// file's tensors form is read from an architecture definition, the text format
// of Synsema's "Local inference and architectures" page, section "The format"
// (arch / kind / param header, prologue, block run per layer with {i}, and
// epilogue; `dst = op(src, ...)` or `op(dst, ...)`; `a | b` = tensor a, else b;
// `x` is the residual).  The library runs one fused block layout, so a
// definition is compiled, not interpreted: every statement is evaluated
// symbolically (each register holds the expression it computes), and the
// residual's expression at the end of the block must equal the expression of
// one of the layouts the GPU kernels implement -- llama's block with optional
// q/k/v biases (qwen2), per-head q/k norms before RoPE (qwen3), sandwich norms
// and a gelu_tanh gate (gemma3).  Statement order, register names and in-place
// versus assigned forms do not matter; what is computed does.
//
// Container layout (the public GGUF specification, versions 2 and 3,
// little-endian): u32 magic "GGUF", u32 version, u64 tensor count, u64
// metadata count; metadata = string key, u32 value type, value; tensor infos =
// string name, u32 n_dims, u64 ne[n_dims] (ne[0] contiguous), u32 ggml type,
// u64 offset; then the data from the next multiple of general.alignment (32 by
// default), offsets counted from there.  string = u64 length + bytes; array =
// u32 element type + u64 count + elements.
#include <fcntl.h>
#include <sys/mman.h>
#include <sys/stat.h>
#include <unistd.h>

#include <algorithm>
#include <cerrno>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <map>
#include <string>
#include <vector>

#include "../../include/qdec.h"

// Sets the calling thread's qdec_last_error() text (defined beside it).
__attribute__((visibility("hidden"))) void qdec_set_error_text(const std::string& s);

namespace {

struct Fail {
  std::string msg;
};

[[noreturn]] void fail(const char* fmt, ...) {
  char buf[768];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  throw Fail{buf};
}

// ------------------------------------------------------------ container
enum : uint32_t { kU8, kI8, kU16, kI16, kU32, kI32, kF32, kBool, kStr, kArr, kU64, kI64, kF64 };

int scalar_size(uint32_t t) {
  switch (t) {
    case kU8: case kI8: case kBool: return 1;
    case kU16: case kI16: return 2;
    case kU32: case kI32: case kF32: return 4;
    case kU64: case kI64: case kF64: return 8;
    default: return 0;
  }
}

struct Meta {
  uint32_t type = 0;
  uint64_t u = 0;     // unsigned integers and non-negative signed ones
  int64_t i = 0;
  bool neg = false;   // a negative signed integer
  double f = 0;
  std::string s;
};

struct TInfo {
  std::string name;
  uint32_t n_dims = 0;
  uint64_t ne[4] = {1, 1, 1, 1};
  uint32_t type = 0;
  uint64_t offset = 0;
};

class Cursor {
 public:
  Cursor(const uint8_t* p, size_t n) : p_(p), n_(n) {}
  size_t pos() const { return pos_; }
  const uint8_t* take(uint64_t k) {
    if (k > n_ - pos_) fail("GGUF: the file ends inside a field at byte %zu", pos_);
    const uint8_t* q = p_ + pos_;
    pos_ += (size_t)k;
    return q;
  }
  template <class T>
  T get() {
    T v;
    std::memcpy(&v, take(sizeof(T)), sizeof(T));
    return v;
  }
  std::string str(uint64_t max_len) {
    const size_t at = pos_;
    const uint64_t len = get<uint64_t>();
    if (len > max_len) fail("GGUF: string of %llu bytes at byte %zu", (unsigned long long)len, at);
    const uint8_t* q = take(len);
    return std::string(reinterpret_cast<const char*>(q), (size_t)len);
  }

 private:
  const uint8_t* p_;
  size_t n_;
  size_t pos_ = 0;
};

// Read one value of type t; arrays are skipped (their element type and count
// are checked against the bytes left).  out may be null.
void read_value(Cursor& c, uint32_t t, int depth, Meta* out) {
  if (out) out->type = t;
  if (const int sz = scalar_size(t)) {
    const uint8_t* q = c.take(sz);
    if (!out) return;
    switch (t) {
      case kU8: out->u = q[0]; break;
      case kI8: { int8_t v; std::memcpy(&v, q, 1); out->i = v; break; }
      case kBool: out->u = q[0] != 0; break;
      case kU16: { uint16_t v; std::memcpy(&v, q, 2); out->u = v; break; }
      case kI16: { int16_t v; std::memcpy(&v, q, 2); out->i = v; break; }
      case kU32: { uint32_t v; std::memcpy(&v, q, 4); out->u = v; break; }
      case kI32: { int32_t v; std::memcpy(&v, q, 4); out->i = v; break; }
      case kF32: { float v; std::memcpy(&v, q, 4); out->f = v; break; }
      case kU64: { uint64_t v; std::memcpy(&v, q, 8); out->u = v; break; }
      case kI64: { int64_t v; std::memcpy(&v, q, 8); out->i = v; break; }
      default: { double v; std::memcpy(&v, q, 8); out->f = v; break; }
    }
    if (t == kI8 || t == kI16 || t == kI32 || t == kI64) {
      out->neg = out->i < 0;
      if (!out->neg) out->u = (uint64_t)out->i;
    }
    return;
  }
  if (t == kStr) {
    std::string s = c.str(~0ull);
    if (out) out->s = std::move(s);
    return;
  }
  if (t == kArr) {
    if (depth > 4) fail("GGUF: arrays nested more than four deep");
    const uint32_t et = c.get<uint32_t>();
    const uint64_t n = c.get<uint64_t>();
    if (const int sz = scalar_size(et)) {
      if (n > ~0ull / (uint64_t)sz) fail("GGUF: array of %llu elements", (unsigned long long)n);
      c.take(n * (uint64_t)sz);
    } else if (et == kStr || et == kArr) {
      for (uint64_t j = 0; j < n; ++j) read_value(c, et, depth + 1, nullptr);
    } else {
      fail("GGUF: array element type %u unknown", et);
    }
    return;
  }
  fail("GGUF: metadata value type %u unknown", t);
}

// Bytes of a tensor the decoder can read (F32, Q4_0, Q8_0, Q4_K, Q6_K), -1 for others.
int64_t tensor_nbytes(const TInfo& t) {
  uint64_t n = 1;
  for (uint32_t d = 0; d < t.n_dims; ++d)
    if (__builtin_mul_overflow(n, t.ne[d], &n) || n > (1ull << 46)) fail("GGUF: tensor '%s' is too large", t.name.c_str());
  if (t.type == QDEC_T_F32) return (int64_t)(n * 4);
  if (t.type == QDEC_T_Q8_0 || t.type == QDEC_T_Q4_0) {
    if (t.ne[0] % 32) fail("GGUF: tensor '%s': row of %llu values is not whole 32-value blocks", t.name.c_str(),
                           (unsigned long long)t.ne[0]);
    return (int64_t)(n / 32 * (t.type == QDEC_T_Q8_0 ? 34 : 18));
  }
  if (t.type == QDEC_T_Q4_K || t.type == QDEC_T_Q6_K) {
    if (t.ne[0] % 256) fail("GGUF: tensor '%s': row of %llu values is not whole 256-value super-blocks",
                            t.name.c_str(), (unsigned long long)t.ne[0]);
    return (int64_t)(n / 256 * (t.type == QDEC_T_Q4_K ? 144 : 210));
  }
  return -1;
}

struct File {
  int fd = -1;
  void* base = MAP_FAILED;
  size_t size = 0;
  std::map<std::string, Meta> meta;
  std::vector<TInfo> tensors;
  std::map<std::string, size_t> by_name;
  uint64_t data = 0;  // byte offset of the data section

  File() = default;
  File(const File&) = delete;
  File& operator=(const File&) = delete;
  ~File() {
    if (base != MAP_FAILED) munmap(base, size);
    if (fd >= 0) close(fd);
  }
  const uint8_t* bytes() const { return static_cast<const uint8_t*>(base); }
};

void open_file(const char* path, File& f) {
  f.fd = open(path, O_RDONLY | O_CLOEXEC);
  if (f.fd < 0) fail("GGUF: cannot open '%s': %s", path, strerror(errno));
  struct stat st;
  if (fstat(f.fd, &st) != 0 || !S_ISREG(st.st_mode)) fail("GGUF: '%s' is not a regular file", path);
  f.size = (size_t)st.st_size;
  if (f.size < 24) fail("GGUF: '%s' is too short (%zu bytes)", path, f.size);
  f.base = mmap(nullptr, f.size, PROT_READ, MAP_PRIVATE, f.fd, 0);
  if (f.base == MAP_FAILED) fail("GGUF: cannot map '%s': %s", path, strerror(errno));

  Cursor c(f.bytes(), f.size);
  if (std::memcmp(c.take(4), "GGUF", 4) != 0) fail("GGUF: '%s' does not start with the GGUF magic", path);
  const uint32_t version = c.get<uint32_t>();
  if (version != 2 && version != 3) fail("GGUF: version %u unsupported (2, 3)", version);
  const uint64_t nt = c.get<uint64_t>(), nkv = c.get<uint64_t>();
  // every entry takes at least 12 (metadata) or 24 (tensor info) bytes
  if (nkv > f.size / 12 || nt > f.size / 24) fail("GGUF: %llu tensors and %llu metadata entries cannot fit the file",
                                                   (unsigned long long)nt, (unsigned long long)nkv);
  for (uint64_t j = 0; j < nkv; ++j) {
    std::string key = c.str(1u << 16);
    const uint32_t t = c.get<uint32_t>();
    Meta m;
    read_value(c, t, 0, &m);
    if (!f.meta.emplace(key, std::move(m)).second) fail("GGUF: metadata key '%s' appears twice", key.c_str());
  }
  uint64_t align = 32;
  if (auto it = f.meta.find("general.alignment"); it != f.meta.end()) {
    const Meta& m = it->second;
    if (m.type != kU32 || m.u == 0 || (m.u & (m.u - 1))) fail("GGUF: general.alignment must be a power-of-two u32");
    align = m.u;
  }
  f.tensors.resize((size_t)nt);
  for (uint64_t j = 0; j < nt; ++j) {
    TInfo& t = f.tensors[(size_t)j];
    t.name = c.str(1u << 16);
    t.n_dims = c.get<uint32_t>();
    if (t.n_dims < 1 || t.n_dims > 4) fail("GGUF: tensor '%s' has %u dimensions", t.name.c_str(), t.n_dims);
    for (uint32_t d = 0; d < t.n_dims; ++d) t.ne[d] = c.get<uint64_t>();
    t.type = c.get<uint32_t>();
    t.offset = c.get<uint64_t>();
    if (!f.by_name.emplace(t.name, (size_t)j).second) fail("GGUF: tensor '%s' appears twice", t.name.c_str());
  }
  f.data = (c.pos() + align - 1) / align * align;
  for (const TInfo& t : f.tensors) {
    if (t.offset % align) fail("GGUF: tensor '%s': offset %llu is not a multiple of %llu", t.name.c_str(),
                               (unsigned long long)t.offset, (unsigned long long)align);
    const int64_t nb = tensor_nbytes(t);
    if (nb >= 0 && (t.offset > f.size || f.data > f.size - t.offset || (uint64_t)nb > f.size - f.data - t.offset))
      fail("GGUF: tensor '%s': data runs past the end of the file", t.name.c_str());
  }
}

const Meta* find_meta(const File& f, const std::string& key) {
  auto it = f.meta.find(key);
  return it == f.meta.end() ? nullptr : &it->second;
}

uint64_t meta_uint(const File& f, const std::string& key, bool required, uint64_t dflt) {
  const Meta* m = find_meta(f, key);
  if (!m) {
    if (required) fail("GGUF: metadata '%s' is missing", key.c_str());
    return dflt;
  }
  const bool integer = m->type <= kI32 || m->type == kU64 || m->type == kI64;
  if (!integer || m->type == kBool || m->neg) fail("GGUF: metadata '%s' must be a non-negative integer", key.c_str());
  return m->u;
}

double meta_float(const File& f, const std::string& key, bool required, double dflt) {
  const Meta* m = find_meta(f, key);
  if (!m) {
    if (required) fail("GGUF: metadata '%s' is missing", key.c_str());
    return dflt;
  }
  if (m->type == kF32 || m->type == kF64) return m->f;
  fail("GGUF: metadata '%s' must be a float", key.c_str());
}

// ------------------------------------------------------------ definitions
struct Stmt {
  std::string dst, op;
  std::vector<std::string> args;
  int line = 0;
};

struct ArchDef {
  std::string arch, kind;
  std::map<std::string, std::string> params;
  std::vector<Stmt> sec[3];  // prologue, block, epilogue
};

std::string trim(const std::string& s) {
  size_t a = 0, b = s.size();
  while (a < b && isspace((unsigned char)s[a])) ++a;
  while (b > a && isspace((unsigned char)s[b - 1])) --b;
  return s.substr(a, b - a);
}

bool is_ident(const std::string& s) {
  if (s.empty() || !(isalpha((unsigned char)s[0]) || s[0] == '_')) return false;
  for (char ch : s)
    if (!(isalnum((unsigned char)ch) || ch == '_')) return false;
  return true;
}

// A tensor argument with its alternatives, spaces around '|' removed.
std::string tensor_arg(const std::string& a, int line) {
  std::string out, part;
  size_t start = 0;
  while (true) {
    const size_t bar = a.find('|', start);
    part = trim(a.substr(start, bar == std::string::npos ? std::string::npos : bar - start));
    bool ok = !part.empty() && part.find('.') != std::string::npos;
    for (char ch : part)
      if (!(isalnum((unsigned char)ch) || ch == '_' || ch == '.' || ch == '{' || ch == '}')) ok = false;
    if (!ok) fail("archdef line %d: '%s' is not a tensor name", line, a.c_str());
    out += part;
    if (bar == std::string::npos) break;
    out += '|';
    start = bar + 1;
  }
  return out;
}

// op -> argument kinds (r register, t tensor, n metadata name or number) and
// whether the assigned form is required
struct OpSig {
  const char* kinds;
  bool needs_dst;
};
const std::map<std::string, OpSig>& op_table() {
  static const std::map<std::string, OpSig> t = {
      {"embed", {"t", true}},      {"rms_norm", {"rt", false}}, {"matmul", {"rt", false}},
      {"add_bias", {"rt", false}}, {"norm_heads", {"rtn", false}}, {"rope", {"rn", false}},
      {"attention", {"rrr", true}}, {"silu", {"r", false}},     {"gelu", {"r", false}},
      {"gelu_tanh", {"r", false}}, {"relu", {"r", false}},      {"mul", {"rr", false}},
      {"add", {"rr", false}},      {"scale", {"rn", false}},    {"copy", {"r", true}},
      {"last", {"r", false}}};
  return t;
}

ArchDef parse_archdef(const std::string& text) {
  static const char* kSec[3] = {"prologue", "block", "epilogue"};
  ArchDef d;
  int section = -1, line = 0;
  size_t at = 0;
  while (at <= text.size()) {
    size_t nl = text.find('\n', at);
    if (nl == std::string::npos) nl = text.size();
    std::string s = text.substr(at, nl - at);
    at = nl + 1;
    ++line;
    if (size_t h = s.find('#'); h != std::string::npos) s.resize(h);
    s = trim(s);
    if (s.empty()) continue;
    int which = -1;
    for (int k = 0; k < 3; ++k)
      if (s == kSec[k]) which = k;
    if (which >= 0) {
      if (which <= section) fail("archdef line %d: section %s out of order or repeated", line, kSec[which]);
      section = which;
      continue;
    }
    if (section < 0) {
      std::vector<std::string> w;
      for (size_t p = 0; p < s.size();) {
        while (p < s.size() && isspace((unsigned char)s[p])) ++p;
        size_t q = p;
        while (q < s.size() && !isspace((unsigned char)s[q])) ++q;
        if (q > p) w.push_back(s.substr(p, q - p));
        p = q;
      }
      if (w.size() == 2 && w[0] == "arch") d.arch = w[1];
      else if (w.size() == 2 && w[0] == "kind") d.kind = w[1];
      else if (w.size() == 3 && w[0] == "param") {
        if (w[1] != "window_pattern" && w[1] != "rope_freq_base_local")
          fail("archdef line %d: unknown param '%s'", line, w[1].c_str());
        d.params[w[1]] = w[2];
      } else {
        fail("archdef line %d: expected arch, kind or param before the sections", line);
      }
      continue;
    }
    Stmt st;
    st.line = line;
    const size_t lp = s.find('('), rp = s.rfind(')');
    if (lp == std::string::npos || rp != s.size() - 1 || rp < lp) fail("archdef line %d: not a statement", line);
    std::string head = trim(s.substr(0, lp));
    if (size_t eq = head.find('='); eq != std::string::npos) {
      st.dst = trim(head.substr(0, eq));
      head = trim(head.substr(eq + 1));
      if (!is_ident(st.dst)) fail("archdef line %d: '%s' is not a register", line, st.dst.c_str());
    }
    st.op = head;
    auto it = op_table().find(st.op);
    if (it == op_table().end()) fail("archdef line %d: unknown operation '%s'", line, st.op.c_str());
    const std::string inner = s.substr(lp + 1, rp - lp - 1);
    if (!trim(inner).empty()) {
      size_t a0 = 0;
      while (true) {
        const size_t comma = inner.find(',', a0);
        st.args.push_back(trim(inner.substr(a0, comma == std::string::npos ? std::string::npos : comma - a0)));
        if (comma == std::string::npos) break;
        a0 = comma + 1;
      }
    }
    const char* kinds = it->second.kinds;
    if (st.args.size() != strlen(kinds)) fail("archdef line %d: %s takes %zu arguments", line, st.op.c_str(), strlen(kinds));
    for (size_t k = 0; k < st.args.size(); ++k) {
      if (kinds[k] == 'r' && !is_ident(st.args[k]))
        fail("archdef line %d: '%s' is not a register", line, st.args[k].c_str());
      if (kinds[k] == 't') {
        st.args[k] = tensor_arg(st.args[k], line);
        if (section != 1 && st.args[k].find("{i}") != std::string::npos)
          fail("archdef line %d: {i} names a layer only inside the block", line);
      }
    }
    if (it->second.needs_dst && st.dst.empty()) fail("archdef line %d: %s needs a destination", line, st.op.c_str());
    if (st.dst.empty()) st.dst = st.args[0];
    d.sec[section].push_back(std::move(st));
  }
  if (d.arch.empty()) fail("archdef: no arch line");
  if (d.kind != "decoder") fail("archdef: kind must be decoder");
  if (d.sec[1].empty()) fail("archdef: no block section");
  return d;
}

// Symbolic evaluation: each register maps to the expression it holds.
std::string fn(const std::string& op, const std::vector<std::string>& a) {
  std::string s = op + "(";
  for (size_t k = 0; k < a.size(); ++k) s += (k ? "," : "") + a[k];
  return s + ")";
}
std::string commutative(const std::string& op, const std::string& a, const std::string& b) {
  return a < b ? fn(op, {a, b}) : fn(op, {b, a});
}

void evaluate(const std::vector<Stmt>& sec, std::map<std::string, std::string>& reg) {
  for (const Stmt& s : sec) {
    auto R = [&](size_t k) -> const std::string& {
      auto it = reg.find(s.args[k]);
      if (it == reg.end()) fail("archdef line %d: register '%s' has no value", s.line, s.args[k].c_str());
      return it->second;
    };
    const auto& a = s.args;
    std::string v;
    if (s.op == "embed") v = fn("embed", {a[0]});
    else if (s.op == "attention") v = fn("attention", {R(0), R(1), R(2)});
    else if (s.op == "mul" || s.op == "add") v = commutative(s.op, R(0), R(1));
    else if (s.op == "copy") v = R(0);
    else if (s.op == "rms_norm" || s.op == "matmul" || s.op == "add_bias") v = fn(s.op, {R(0), a[1]});
    else if (s.op == "norm_heads") v = fn(s.op, {R(0), a[1], a[2]});
    else if (s.op == "rope" || s.op == "scale") v = fn(s.op, {R(0), a[1]});
    else v = fn(s.op, {R(0)});  // silu, gelu, gelu_tanh, relu, last
    reg[s.dst] = v;
  }
}

// The residual after one block of the fused layout.
std::string block_layout(bool bias, bool qkn, bool sandwich, const char* act) {
  auto w = [](const char* n) { return std::string("blk.{i}.") + n; };
  const std::string X = "X";
  const std::string h = fn("rms_norm", {X, w("attn_norm.weight")});
  std::string q = fn("matmul", {h, w("attn_q.weight")}), k = fn("matmul", {h, w("attn_k.weight")}),
              v = fn("matmul", {h, w("attn_v.weight")});
  if (bias) {
    q = fn("add_bias", {q, w("attn_q.bias")});
    k = fn("add_bias", {k, w("attn_k.bias")});
    v = fn("add_bias", {v, w("attn_v.bias")});
  }
  if (qkn) {
    q = fn("norm_heads", {q, w("attn_q_norm.weight"), "head_count"});
    k = fn("norm_heads", {k, w("attn_k_norm.weight"), "head_count_kv"});
  }
  q = fn("rope", {q, "head_count"});
  k = fn("rope", {k, "head_count_kv"});
  std::string o = fn("matmul", {fn("attention", {q, k, v}), w("attn_output.weight")});
  if (sandwich) o = fn("rms_norm", {o, w("post_attention_norm.weight")});
  const std::string x1 = commutative("add", X, o);
  const std::string h2 = fn("rms_norm", {x1, w("ffn_norm.weight")});
  const std::string g = fn(act, {fn("matmul", {h2, w("ffn_gate.weight")})});
  std::string d = fn("matmul", {commutative("mul", g, fn("matmul", {h2, w("ffn_up.weight")})), w("ffn_down.weight")});
  if (sandwich) d = fn("rms_norm", {d, w("post_ffw_norm.weight")});
  return commutative("add", x1, d);
}

// Every name a statement uses must resolve in the file, statements whose
// results are never used included: a tensor argument (one of its '|'
// alternatives, in every layer for the block) must be one of the file's
// tensors, a number argument a head count, a number, or a metadata key of the
// architecture.
void check_names(const ArchDef& d, const File& f, int32_t n_layer) {
  auto is_number = [](const std::string& s) {
    char* end = nullptr;
    errno = 0;
    const double v = strtod(s.c_str(), &end);
    return !s.empty() && end && !*end && errno == 0 && std::isfinite(v);
  };
  for (int sec = 0; sec < 3; ++sec)
    for (const Stmt& st : d.sec[sec]) {
      const char* kinds = op_table().at(st.op).kinds;
      for (size_t k = 0; k < st.args.size(); ++k) {
        const std::string& a = st.args[k];
        if (kinds[k] == 'n' && a != "head_count" && a != "head_count_kv" && !is_number(a) &&
            !find_meta(f, d.arch + "." + a))
          fail("archdef line %d: '%s' is neither a number nor a metadata key of the file", st.line, a.c_str());
        if (kinds[k] != 't') continue;
        const bool per_layer = a.find("{i}") != std::string::npos;
        // distinct layers give distinct names, so a missing one is met within
        // (number of tensors + 1) layers
        for (int32_t i = 0; i < (per_layer ? n_layer : 1); ++i) {
          bool present = false;
          size_t start = 0;
          while (!present) {
            const size_t bar = a.find('|', start);
            std::string name = a.substr(start, bar == std::string::npos ? std::string::npos : bar - start);
            for (size_t at; (at = name.find("{i}")) != std::string::npos;) name.replace(at, 3, std::to_string(i));
            present = f.by_name.count(name) > 0;
            if (bar == std::string::npos) break;
            start = bar + 1;
          }
          if (!present) {
            std::string shown = a;
            for (size_t at; (at = shown.find("{i}")) != std::string::npos;) shown.replace(at, 3, std::to_string(i));
            fail("archdef line %d: tensor '%s' is not in the file", st.line, shown.c_str());
          }
        }
      }
    }
}

enum Head { kHeadEither, kHeadOutput, kHeadEmbd };

struct Compiled {
  qdec_config cfg{};
  Head head = kHeadEither;
};

Compiled compile(const ArchDef& d, const File& f) {
  Compiled r;
  {
    const Meta* m = find_meta(f, "general.architecture");
    if (!m || m->type != kStr) fail("GGUF: general.architecture is missing");
    if (m->s != d.arch) fail("archdef: the file's architecture is '%s', the definition's '%s'", m->s.c_str(), d.arch.c_str());
  }
  std::map<std::string, std::string> reg;
  evaluate(d.sec[0], reg);
  if (!reg.count("x") || reg["x"] != "embed(token_embd.weight)")
    fail("archdef: the prologue must set x = embed(token_embd.weight) and nothing else on x");
  reg.clear();
  reg["x"] = "X";
  evaluate(d.sec[1], reg);
  bool found = false;
  for (int bias = 0; bias < 2 && !found; ++bias)
    for (int qkn = 0; qkn < 2 && !found; ++qkn)
      for (int sw = 0; sw < 2 && !found; ++sw)
        for (int act = 0; act < 2 && !found; ++act)
          if (reg["x"] == block_layout(bias, qkn, sw, act ? "gelu_tanh" : "silu")) {
            found = true;
            r.cfg.qkv_bias = bias;
            r.cfg.qk_norm = qkn;
            r.cfg.sandwich_norm = sw;
            r.cfg.act = act ? QDEC_ACT_GELU_TANH : QDEC_ACT_SILU;
          }
  if (!found)
    fail("archdef: the block does not compute a layout this library runs (llama's pre-norm block with silu or "
         "gelu_tanh gating, optionally with q/k/v biases, per-head q/k norms before rope, and sandwich norms)");
  reg.clear();
  reg["x"] = "X";
  evaluate(d.sec[2], reg);
  const char* heads[3] = {"output.weight|token_embd.weight", "output.weight", "token_embd.weight"};
  bool head_ok = false;
  for (int hch = 0; hch < 3 && !head_ok; ++hch)
    for (int order = 0; order < 2 && !head_ok; ++order) {
      const std::string xn = order ? fn("rms_norm", {fn("last", {"X"}), "output_norm.weight"})
                                   : fn("last", {fn("rms_norm", {"X", "output_norm.weight"})});
      if (reg.count("logits") && reg["logits"] == fn("matmul", {xn, heads[hch]})) {
        head_ok = true;
        r.head = (Head)hch;
      }
    }
  if (!head_ok)
    fail("archdef: the epilogue must compute logits = matmul(last(rms_norm(x, output_norm.weight)), "
         "output.weight | token_embd.weight) (either tensor alone is also accepted)");

  qdec_config& c = r.cfg;
  const std::string a = d.arch + ".";
  auto U = [&](const char* k, bool req, uint64_t dflt) {
    const uint64_t v = meta_uint(f, a + k, req, dflt);
    if (v > (uint64_t)INT32_MAX) fail("GGUF: metadata '%s%s' = %llu is too large", a.c_str(), k, (unsigned long long)v);
    return (int32_t)v;
  };
  c.n_layer = U("block_count", true, 0);
  c.hidden = U("embedding_length", true, 0);
  c.ffn = U("feed_forward_length", true, 0);
  c.n_head = U("attention.head_count", true, 0);
  c.n_head_kv = U("attention.head_count_kv", false, (uint64_t)c.n_head);
  if (c.n_head <= 0) fail("GGUF: %sattention.head_count must be positive", a.c_str());
  c.head_dim = U("attention.key_length", false, (uint64_t)(c.hidden / c.n_head));
  if (U("attention.value_length", false, (uint64_t)c.head_dim) != c.head_dim)
    fail("GGUF: key_length and value_length differ");
  c.rms_eps = (float)meta_float(f, a + "attention.layer_norm_rms_epsilon", true, 0);
  c.rope_theta = (float)meta_float(f, a + "rope.freq_base", false, 10000.0);
  c.window = U("attention.sliding_window", false, 0);
  c.window_period = 0;
  c.rope_theta_local = c.rope_theta;
  if (auto it = d.params.find("rope_freq_base_local"); it != d.params.end()) {
    char* end = nullptr;
    c.rope_theta_local = strtof(it->second.c_str(), &end);
    if (!end || *end || !(c.rope_theta_local > 0.f)) fail("archdef: rope_freq_base_local must be a positive number");
  }
  if (c.window > 0) {
    auto it = d.params.find("window_pattern");
    if (it == d.params.end()) fail("archdef: the file has a sliding window but the definition no window_pattern");
    char* end = nullptr;
    const long p = strtol(it->second.c_str(), &end, 10);
    if (!end || *end || p < 1 || p > 1 << 20) fail("archdef: window_pattern must be a positive integer");
    c.window_period = (int32_t)p;
  }
  auto e = f.by_name.find("token_embd.weight");
  if (e == f.by_name.end()) fail("GGUF: tensor 'token_embd.weight' is missing");
  const TInfo& te = f.tensors[e->second];
  if (te.n_dims != 2 || te.ne[1] > (uint64_t)INT32_MAX) fail("GGUF: token_embd.weight must be a matrix");
  c.vocab = (int32_t)te.ne[1];
  if (r.head == kHeadOutput && !f.by_name.count("output.weight"))
    fail("archdef: the head names output.weight, which the file lacks");
  check_names(d, f, c.n_layer);
  return r;
}

// Names of the tensors a compiled layout reads (output.weight when the head
// takes it).
std::vector<std::string> needed(const Compiled& r, const File& f) {
  const qdec_config& c = r.cfg;
  std::vector<std::string> n = {"token_embd.weight", "output_norm.weight"};
  if (r.head == kHeadOutput || (r.head == kHeadEither && f.by_name.count("output.weight"))) n.push_back("output.weight");
  for (int i = 0; i < c.n_layer; ++i) {
    const std::string p = "blk." + std::to_string(i) + ".";
    for (const char* s : {"attn_norm.weight", "attn_q.weight", "attn_k.weight", "attn_v.weight", "attn_output.weight",
                          "ffn_norm.weight", "ffn_gate.weight", "ffn_up.weight", "ffn_down.weight"})
      n.push_back(p + s);
    if (c.qkv_bias)
      for (const char* s : {"attn_q.bias", "attn_k.bias", "attn_v.bias"}) n.push_back(p + s);
    if (c.qk_norm)
      for (const char* s : {"attn_q_norm.weight", "attn_k_norm.weight"}) n.push_back(p + s);
    if (c.sandwich_norm)
      for (const char* s : {"post_attention_norm.weight", "post_ffw_norm.weight"}) n.push_back(p + s);
  }
  return n;
}

// Built-in definitions, by architecture name.
const char* kLlama = R"(arch llama
kind decoder
prologue
  x = embed(token_embd.weight)
block
  h = rms_norm(x, blk.{i}.attn_norm.weight)
  q = matmul(h, blk.{i}.attn_q.weight)
  k = matmul(h, blk.{i}.attn_k.weight)
  v = matmul(h, blk.{i}.attn_v.weight)
  rope(q, head_count)
  rope(k, head_count_kv)
  a = attention(q, k, v)
  o = matmul(a, blk.{i}.attn_output.weight)
  add(x, o)
  h = rms_norm(x, blk.{i}.ffn_norm.weight)
  g = matmul(h, blk.{i}.ffn_gate.weight)
  silu(g)
  u = matmul(h, blk.{i}.ffn_up.weight)
  mul(g, u)
  d = matmul(g, blk.{i}.ffn_down.weight)
  add(x, d)
epilogue
  x = rms_norm(x, output_norm.weight)
  x = last(x)
  logits = matmul(x, output.weight | token_embd.weight)
)";

const char* kQwen2 = R"(arch qwen2
kind decoder
prologue
  x = embed(token_embd.weight)
block
  h = rms_norm(x, blk.{i}.attn_norm.weight)
  q = matmul(h, blk.{i}.attn_q.weight)
  k = matmul(h, blk.{i}.attn_k.weight)
  v = matmul(h, blk.{i}.attn_v.weight)
  add_bias(q, blk.{i}.attn_q.bias)
  add_bias(k, blk.{i}.attn_k.bias)
  add_bias(v, blk.{i}.attn_v.bias)
  rope(q, head_count)
  rope(k, head_count_kv)
  a = attention(q, k, v)
  o = matmul(a, blk.{i}.attn_output.weight)
  add(x, o)
  h = rms_norm(x, blk.{i}.ffn_norm.weight)
  g = matmul(h, blk.{i}.ffn_gate.weight)
  silu(g)
  u = matmul(h, blk.{i}.ffn_up.weight)
  mul(g, u)
  d = matmul(g, blk.{i}.ffn_down.weight)
  add(x, d)
epilogue
  x = rms_norm(x, output_norm.weight)
  x = last(x)
  logits = matmul(x, output.weight | token_embd.weight)
)";

const char* kQwen3 = R"(arch qwen3
kind decoder
prologue
  x = embed(token_embd.weight)
block
  h = rms_norm(x, blk.{i}.attn_norm.weight)
  q = matmul(h, blk.{i}.attn_q.weight)
  k = matmul(h, blk.{i}.attn_k.weight)
  v = matmul(h, blk.{i}.attn_v.weight)
  norm_heads(q, blk.{i}.attn_q_norm.weight, head_count)
  norm_heads(k, blk.{i}.attn_k_norm.weight, head_count_kv)
  rope(q, head_count)
  rope(k, head_count_kv)
  a = attention(q, k, v)
  o = matmul(a, blk.{i}.attn_output.weight)
  add(x, o)
  h = rms_norm(x, blk.{i}.ffn_norm.weight)
  g = matmul(h, blk.{i}.ffn_gate.weight)
  silu(g)
  u = matmul(h, blk.{i}.ffn_up.weight)
  mul(g, u)
  d = matmul(g, blk.{i}.ffn_down.weight)
  add(x, d)
epilogue
  x = rms_norm(x, output_norm.weight)
  x = last(x)
  logits = matmul(x, output.weight | token_embd.weight)
)";

const char* kGemma3 = R"(arch gemma3
kind decoder
param window_pattern 6
param rope_freq_base_local 10000
prologue
  x = embed(token_embd.weight)
block
  h = rms_norm(x, blk.{i}.attn_norm.weight)
  q = matmul(h, blk.{i}.attn_q.weight)
  k = matmul(h, blk.{i}.attn_k.weight)
  v = matmul(h, blk.{i}.attn_v.weight)
  norm_heads(q, blk.{i}.attn_q_norm.weight, head_count)
  norm_heads(k, blk.{i}.attn_k_norm.weight, head_count_kv)
  rope(q, head_count)
  rope(k, head_count_kv)
  a = attention(q, k, v)
  o = matmul(a, blk.{i}.attn_output.weight)
  rms_norm(o, blk.{i}.post_attention_norm.weight)
  add(x, o)
  h = rms_norm(x, blk.{i}.ffn_norm.weight)
  g = matmul(h, blk.{i}.ffn_gate.weight)
  gelu_tanh(g)
  u = matmul(h, blk.{i}.ffn_up.weight)
  mul(g, u)
  d = matmul(g, blk.{i}.ffn_down.weight)
  rms_norm(d, blk.{i}.post_ffw_norm.weight)
  add(x, d)
epilogue
  x = rms_norm(x, output_norm.weight)
  x = last(x)
  logits = matmul(x, output.weight | token_embd.weight)
)";

const char* builtin(const std::string& arch) {
  if (arch == "llama") return kLlama;
  if (arch == "qwen2") return kQwen2;
  if (arch == "qwen3") return kQwen3;
  if (arch == "gemma3") return kGemma3;
  return nullptr;
}

Compiled compile_file(const char* path, const char* archdef, File& f) {
  if (!path) fail("path must not be NULL");
  open_file(path, f);
  std::string text;
  if (archdef) {
    text = archdef;
  } else {
    const Meta* m = find_meta(f, "general.architecture");
    if (!m || m->type != kStr) fail("GGUF: general.architecture is missing");
    const char* b = builtin(m->s);
    if (!b) fail("archdef: no built-in definition for architecture '%s'; pass one", m->s.c_str());
    text = b;
  }
  return compile(parse_archdef(text), f);
}

}  // namespace

extern "C" {

const char* qdec_archdef_builtin(const char* arch) { return arch ? builtin(arch) : nullptr; }

int qdec_gguf_config(const char* path, const char* archdef, qdec_config* out) {
  try {
    if (!out) fail("out must not be NULL");
    File f;
    *out = compile_file(path, archdef, f).cfg;
    return QDEC_OK;
  } catch (const Fail& e) {
    qdec_set_error_text(e.msg);
    return QDEC_REFUSED;
  } catch (const std::exception& e) {
    qdec_set_error_text(std::string("GGUF: ") + e.what());
    return QDEC_REFUSED;
  }
}

int qdec_load_gguf(const char* path, const char* archdef, int32_t max_seqs, int32_t max_ctx, void* stream,
                   qdec_model** out) {
  std::vector<qdec_tensor> table;
  std::vector<std::string> names;
  File f;
  Compiled r;
  try {
    if (!out) fail("out must not be NULL");
    *out = nullptr;
    r = compile_file(path, archdef, f);
    names = needed(r, f);
    table.reserve(names.size());
    for (const std::string& n : names) {
      auto it = f.by_name.find(n);
      if (it == f.by_name.end()) continue;  // qdec_load_weights names what is missing
      const TInfo& t = f.tensors[it->second];
      const int64_t nb = tensor_nbytes(t);
      if (nb < 0) fail("GGUF: tensor '%s' has type %u (this library reads F32 = 0, Q4_0 = 2, Q8_0 = 8, Q4_K = 12, Q6_K = 14)", n.c_str(), t.type);
      if (t.n_dims > 2) fail("GGUF: tensor '%s' has %u dimensions", n.c_str(), t.n_dims);
      qdec_tensor q;
      q.name = it->first.c_str();
      q.type = (int32_t)t.type;
      q.rows = t.n_dims == 2 ? (int64_t)t.ne[1] : 1;
      q.cols = (int64_t)t.ne[0];
      q.host_data = f.bytes() + f.data + t.offset;
      q.n_bytes = nb;
      table.push_back(q);
    }
  } catch (const Fail& e) {
    qdec_set_error_text(e.msg);
    return QDEC_REFUSED;
  } catch (const std::exception& e) {
    qdec_set_error_text(std::string("GGUF: ") + e.what());
    return QDEC_REFUSED;
  }
  // the mapping stays open until the weights are on the device (the call
  // synchronizes its stream before returning)
  return qdec_load_weights(&r.cfg, table.data(), (int32_t)table.size(), max_seqs, max_ctx, stream, out);
}

}  // extern "C"
