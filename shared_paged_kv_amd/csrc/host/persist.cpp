// Persistent Q4 block pool, host side: the image size and the safetensors file
// (include/kvpool_persist.h).  Q4 KV paper summary, sec. 2.1: per-agent caches
// in 256-token Q4 blocks, kept in safetensors files, one namespace per agent.
//
// safetensors layout: u64 little-endian N, N bytes of JSON
//   {"__metadata__": {str: str}, name: {"dtype": D, "shape": [..],
//    "data_offsets": [begin, end]}, ...}
// then the tensor bytes, offsets relative to the first byte after the header.
// The header is padded with spaces to a multiple of 8 bytes.  Reads and writes
// of the tensor bytes are split over a few threads (pread / pwrite).
#include <errno.h>
#include <fcntl.h>
#include <sys/stat.h>
#include <unistd.h>

#include <algorithm>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <map>
#include <new>
#include <string>
#include <thread>
#include <vector>

#include "kvpool.h"
#include "kvpool_internal.h"
#include "kvpool_persist.h"

using kvp::fail;

namespace {

struct Q4Sizes {
  int64_t codes, params, image;  // bytes of one codes tensor, one params tensor, the image
  int64_t codes_blk, params_blk;  // per block and layer
};

bool q4_sizes(const kvp_shape* s, int32_t n, Q4Sizes* z) {
  if (kvp::check_shape(s) != KVP_OK) return false;
  if (s->kv_dtype != KVP_Q4G64 || n < 0) {
    fail(KVP_EINVAL, "persistence needs a KVP_Q4G64 shape and n >= 0");
    return false;
  }
  z->codes_blk = (int64_t)s->n_kv_heads * s->block_tokens * (s->head_dim / 2);
  z->params_blk = (int64_t)s->n_kv_heads * s->block_tokens * (s->head_dim / 64) * 2 * 2;
  z->codes = z->codes_blk * n * s->n_layers;
  z->params = z->params_blk * n * s->n_layers;
  z->image = 2 * z->codes + 2 * z->params;
  return true;
}

// ---------------------------------------------------------------- file bytes

bool io_all(bool write, int fd, uint8_t* buf, int64_t size, int64_t off) {
  while (size > 0) {
    const size_t chunk = (size_t)std::min<int64_t>(size, 1 << 30);
    const ssize_t r = write ? pwrite(fd, buf, chunk, off) : pread(fd, buf, chunk, off);
    if (r < 0 && errno == EINTR) continue;  // interrupted before any byte moved
    if (r <= 0) return false;
    buf += r;
    off += r;
    size -= r;
  }
  return true;
}

// Moves size bytes between buf and the file at off, split over up to 8 threads
// (whole 8 MiB pieces each).  A piece whose thread cannot be started is moved
// by the calling thread.
bool io_parallel(bool write, int fd, uint8_t* buf, int64_t size, int64_t off) {
  const int64_t piece = 8LL << 20;
  const int nt = (int)std::min<int64_t>(8, (size + piece - 1) / piece);
  if (nt <= 1) return io_all(write, fd, buf, size, off);
  const int64_t per = ((size + nt - 1) / nt + piece - 1) / piece * piece;
  std::vector<std::thread> th;
  char ok[8] = {1, 1, 1, 1, 1, 1, 1, 1};
  try {
    th.reserve((size_t)nt);
  } catch (...) {
    return io_all(write, fd, buf, size, off);
  }
  for (int i = 0; i < nt; ++i) {
    const int64_t b = std::min(size, i * per), e = std::min(size, b + per);
    try {
      th.emplace_back([&ok, write, fd, buf, off, i, b, e] { ok[i] = io_all(write, fd, buf + b, e - b, off + b); });
    } catch (...) {
      ok[i] = io_all(write, fd, buf + b, e - b, off + b);
    }
  }
  for (auto& t : th) t.join();
  return std::all_of(ok, ok + nt, [](char c) { return c != 0; });
}

// ---------------------------------------------------------------- JSON (the subset a header uses)

struct JVal {
  enum Kind { NUL, NUM, STR, ARR, OBJ, BOOL } kind = NUL;
  int64_t num = 0;
  bool is_int = true;
  std::string str;
  std::vector<JVal> arr;
  std::vector<std::pair<std::string, JVal>> obj;
  const JVal* get(const char* k) const {
    for (auto& kv : obj)
      if (kv.first == k) return &kv.second;
    return nullptr;
  }
};

struct JParser {
  const char* p;
  const char* end;
  int depth = 0;
  void ws() {
    while (p < end && (*p == ' ' || *p == '\t' || *p == '\n' || *p == '\r')) ++p;
  }
  bool lit(const char* w) {
    const size_t n = strlen(w);
    if ((size_t)(end - p) < n || memcmp(p, w, n) != 0) return false;
    p += n;
    return true;
  }
  bool hex4(unsigned* u) {
    if (end - p < 4) return false;
    *u = 0;
    for (int i = 0; i < 4; ++i) {
      const char c = *p++;
      *u <<= 4;
      if (c >= '0' && c <= '9') *u |= (unsigned)(c - '0');
      else if (c >= 'a' && c <= 'f') *u |= (unsigned)(c - 'a' + 10);
      else if (c >= 'A' && c <= 'F') *u |= (unsigned)(c - 'A' + 10);
      else return false;
    }
    return true;
  }
  bool string(std::string* out) {
    if (p >= end || *p != '"') return false;
    ++p;
    out->clear();
    while (p < end && *p != '"') {
      if ((unsigned char)*p < 0x20) return false;
      if (*p != '\\') {
        out->push_back(*p++);
        continue;
      }
      if (++p >= end) return false;
      const char c = *p++;
      switch (c) {
        case '"': case '\\': case '/': out->push_back(c); break;
        case 'b': out->push_back('\b'); break;
        case 'f': out->push_back('\f'); break;
        case 'n': out->push_back('\n'); break;
        case 'r': out->push_back('\r'); break;
        case 't': out->push_back('\t'); break;
        case 'u': {
          unsigned u;
          if (!hex4(&u)) return false;
          if (u >= 0xD800 && u <= 0xDBFF) {  // surrogate pair
            unsigned lo;
            if (!lit("\\u") || !hex4(&lo) || lo < 0xDC00 || lo > 0xDFFF) return false;
            u = 0x10000 + ((u - 0xD800) << 10) + (lo - 0xDC00);
          }
          if (u < 0x80) {
            out->push_back((char)u);
          } else if (u < 0x800) {
            out->push_back((char)(0xC0 | (u >> 6)));
            out->push_back((char)(0x80 | (u & 0x3F)));
          } else if (u < 0x10000) {
            out->push_back((char)(0xE0 | (u >> 12)));
            out->push_back((char)(0x80 | ((u >> 6) & 0x3F)));
            out->push_back((char)(0x80 | (u & 0x3F)));
          } else {
            out->push_back((char)(0xF0 | (u >> 18)));
            out->push_back((char)(0x80 | ((u >> 12) & 0x3F)));
            out->push_back((char)(0x80 | ((u >> 6) & 0x3F)));
            out->push_back((char)(0x80 | (u & 0x3F)));
          }
          break;
        }
        default: return false;
      }
    }
    if (p >= end) return false;
    ++p;
    return true;
  }
  bool number(JVal* v) {
    const char* s = p;
    if (p < end && *p == '-') ++p;
    if (p >= end || !(*p >= '0' && *p <= '9')) return false;
    while (p < end && *p >= '0' && *p <= '9') ++p;
    bool frac = false;
    if (p < end && *p == '.') {
      frac = true;
      ++p;
      while (p < end && *p >= '0' && *p <= '9') ++p;
    }
    if (p < end && (*p == 'e' || *p == 'E')) {
      frac = true;
      ++p;
      if (p < end && (*p == '+' || *p == '-')) ++p;
      while (p < end && *p >= '0' && *p <= '9') ++p;
    }
    v->kind = JVal::NUM;
    v->is_int = !frac && (p - s) <= 18;
    v->num = v->is_int ? strtoll(std::string(s, p).c_str(), nullptr, 10) : 0;
    return true;
  }
  bool value(JVal* v) {
    if (++depth > 32) return false;
    ws();
    bool ok = false;
    if (p >= end) {
      ok = false;
    } else if (*p == '{') {
      ++p;
      v->kind = JVal::OBJ;
      ws();
      if (p < end && *p == '}') {
        ++p;
        ok = true;
      } else {
        while (true) {
          ws();
          std::pair<std::string, JVal> kv;
          if (!string(&kv.first)) break;
          ws();
          if (p >= end || *p != ':') break;
          ++p;
          if (!value(&kv.second)) break;
          v->obj.push_back(std::move(kv));
          ws();
          if (p < end && *p == ',') {
            ++p;
            continue;
          }
          if (p < end && *p == '}') {
            ++p;
            ok = true;
          }
          break;
        }
      }
    } else if (*p == '[') {
      ++p;
      v->kind = JVal::ARR;
      ws();
      if (p < end && *p == ']') {
        ++p;
        ok = true;
      } else {
        while (true) {
          JVal e;
          if (!value(&e)) break;
          v->arr.push_back(std::move(e));
          ws();
          if (p < end && *p == ',') {
            ++p;
            continue;
          }
          if (p < end && *p == ']') {
            ++p;
            ok = true;
          }
          break;
        }
      }
    } else if (*p == '"') {
      v->kind = JVal::STR;
      ok = string(&v->str);
    } else if (lit("true") || lit("false")) {
      v->kind = JVal::BOOL;
      ok = true;
    } else if (lit("null")) {
      v->kind = JVal::NUL;
      ok = true;
    } else {
      ok = number(v);
    }
    --depth;
    return ok;
  }
};

// ---------------------------------------------------------------- tensors of a Q4 image

struct TensorSpec {
  const char* name;
  const char* dtype;
  int64_t image_off, bytes;
  std::vector<int64_t> shape;
};

std::vector<TensorSpec> q4_tensors(const kvp_shape* s, int32_t n, const Q4Sizes& z) {
  const int64_t L = s->n_layers, H = s->n_kv_heads, B = s->block_tokens, d = s->head_dim;
  std::vector<int64_t> cs{L, n, H, B, d / 2}, ps{L, n, H, B, d / 64, 2};
  return {{"k_codes", "U8", 0, z.codes, cs},
          {"v_codes", "U8", z.codes, z.codes, cs},
          {"k_params", "F16", 2 * z.codes, z.params, ps},
          {"v_params", "F16", 2 * z.codes + z.params, z.params, ps}};
}

bool agent_ok(const char* a) {
  if (!a) return false;
  const size_t n = strlen(a);
  if (n > 255) return false;
  for (size_t i = 0; i < n; ++i)
    if ((unsigned char)a[i] < 0x20 || a[i] == '"' || a[i] == '\\') return false;
  return true;
}

struct Fd {
  int fd = -1;
  ~Fd() {
    if (fd >= 0) close(fd);
  }
};

}  // namespace

extern "C" {

int64_t kvpool_q4_image_bytes(const kvp_shape* shape, int32_t n) {
  Q4Sizes z;
  if (!q4_sizes(shape, n, &z)) return KVP_EINVAL;
  return z.image;
}

int kvpool_q4_save_file(const kvp_shape* shape, const char* path, const char* agent, const void* image,
                        const int32_t* ntok, int32_t n) {
  Q4Sizes z;
  if (!q4_sizes(shape, n, &z)) return KVP_EINVAL;
  if (!path || !image || !ntok || n < 1) return fail(KVP_EINVAL, "NULL pointer or n < 1");
  if (!agent_ok(agent)) return fail(KVP_EINVAL, "agent must be a string of at most 255 bytes, no quotes or controls");
  for (int32_t i = 0; i < n; ++i)
    if (ntok[i] < 0 || ntok[i] > shape->block_tokens) return fail(KVP_EINVAL, "ntok out of range");
  std::string h;
  try {
    auto tensors = q4_tensors(shape, n, z);
    char buf[512];
    snprintf(buf, sizeof buf,
             "{\"__metadata__\":{\"format\":\"kvpool-q4g64\",\"agent\":\"%s\",\"n_layers\":\"%d\","
             "\"n_kv_heads\":\"%d\",\"block_tokens\":\"%d\",\"head_dim\":\"%d\"}",
             agent, shape->n_layers, shape->n_kv_heads, shape->block_tokens, shape->head_dim);
    h = buf;
    int64_t off = 0;
    auto add = [&](const char* name, const char* dtype, const std::vector<int64_t>& sh, int64_t bytes) {
      h += ",\"";
      h += name;
      h += "\":{\"dtype\":\"";
      h += dtype;
      h += "\",\"shape\":[";
      for (size_t i = 0; i < sh.size(); ++i) h += (i ? "," : "") + std::to_string(sh[i]);
      h += "],\"data_offsets\":[" + std::to_string(off) + "," + std::to_string(off + bytes) + "]}";
      off += bytes;
    };
    for (auto& t : tensors) add(t.name, t.dtype, t.shape, t.bytes);
    add("ntok", "I32", {n}, 4LL * n);
    h += "}";
    while ((8 + h.size()) % 8) h += ' ';
  } catch (const std::bad_alloc&) {
    return fail(KVP_ENOMEM, "header");
  }
  Fd f;
  f.fd = open(path, O_WRONLY | O_CREAT | O_TRUNC, 0644);
  if (f.fd < 0) return fail(KVP_EIO, "cannot create the file");
  uint8_t len[8];
  const uint64_t hl = h.size();
  for (int i = 0; i < 8; ++i) len[i] = (uint8_t)(hl >> (8 * i));
  const int64_t data0 = 8 + (int64_t)hl;
  bool ok = io_all(true, f.fd, len, 8, 0) && io_all(true, f.fd, (uint8_t*)h.data(), (int64_t)hl, 8) &&
            io_parallel(true, f.fd, (uint8_t*)image, z.image, data0);
  // ntok as little-endian int32 (the host is little-endian)
  ok = ok && io_all(true, f.fd, (uint8_t*)ntok, 4LL * n, data0 + z.image);
  if (!ok) return fail(KVP_EIO, "write failed");
  if (close(f.fd) != 0) {
    f.fd = -1;
    return fail(KVP_EIO, "close failed");
  }
  f.fd = -1;
  return KVP_OK;
}

}  // extern "C"

namespace {

int load_file(const kvp_shape* shape, const char* path, const char* agent, void* image, int64_t image_bytes,
              int32_t* ntok, int32_t max_blocks) {
  Q4Sizes z0;
  if (!q4_sizes(shape, 0, &z0)) return KVP_EINVAL;
  if (!path || max_blocks < 0 || image_bytes < 0) return fail(KVP_EINVAL, "NULL path or negative size");
  Fd f;
  f.fd = open(path, O_RDONLY);
  if (f.fd < 0) return fail(KVP_EIO, "cannot open the file");
  struct stat st;
  if (fstat(f.fd, &st) != 0) return fail(KVP_EIO, "cannot stat the file");
  const int64_t fsize = st.st_size;
  uint8_t len[8];
  if (fsize < 8 || !io_all(false, f.fd, len, 8, 0)) return fail(KVP_EIO, "file too short");
  uint64_t hl = 0;
  for (int i = 0; i < 8; ++i) hl |= (uint64_t)len[i] << (8 * i);
  if (hl > (100u << 20) || (int64_t)hl > fsize - 8) return fail(KVP_EIO, "bad header length");
  std::string h;
  JVal root;
  try {
    h.resize(hl);
    if (!io_all(false, f.fd, (uint8_t*)&h[0], (int64_t)hl, 8)) return fail(KVP_EIO, "cannot read the header");
    JParser jp{h.data(), h.data() + h.size()};
    if (!jp.value(&root) || root.kind != JVal::OBJ) return fail(KVP_EIO, "header is not a JSON object");
    jp.ws();
    if (jp.p != jp.end) return fail(KVP_EIO, "trailing bytes after the header");
  } catch (const std::bad_alloc&) {
    return fail(KVP_ENOMEM, "header");
  }
  const int64_t data0 = 8 + (int64_t)hl, data_size = fsize - data0;
  if (agent) {
    const JVal* md = root.get("__metadata__");
    const JVal* a = md && md->kind == JVal::OBJ ? md->get("agent") : nullptr;
    if (!a || a->kind != JVal::STR || a->str != agent) return fail(KVP_EINVAL, "the file belongs to another agent");
  }
  // every tensor entry: dtype, shape, byte range inside the data section
  struct Entry {
    std::string dtype;
    std::vector<int64_t> shape;
    int64_t b, e;
  };
  std::map<std::string, Entry> ent;
  for (auto& kv : root.obj) {
    if (kv.first == "__metadata__") continue;
    const JVal& t = kv.second;
    const JVal *dt = t.get("dtype"), *sh = t.get("shape"), *of = t.get("data_offsets");
    if (t.kind != JVal::OBJ || !dt || dt->kind != JVal::STR || !sh || sh->kind != JVal::ARR || !of ||
        of->kind != JVal::ARR || of->arr.size() != 2)
      return fail(KVP_EIO, "malformed tensor entry");
    Entry e{dt->str, {}, 0, 0};
    for (auto& x : sh->arr) {
      if (x.kind != JVal::NUM || !x.is_int || x.num < 0) return fail(KVP_EIO, "malformed shape");
      e.shape.push_back(x.num);
    }
    if (of->arr[0].kind != JVal::NUM || of->arr[1].kind != JVal::NUM || !of->arr[0].is_int || !of->arr[1].is_int)
      return fail(KVP_EIO, "malformed offsets");
    e.b = of->arr[0].num;
    e.e = of->arr[1].num;
    if (e.b < 0 || e.e < e.b || e.e > data_size) return fail(KVP_EIO, "tensor bytes outside the file");
    ent[kv.first] = e;
  }
  auto nt = ent.find("ntok");
  if (nt == ent.end() || nt->second.dtype != "I32" || nt->second.shape.size() != 1)
    return fail(KVP_EINVAL, "ntok missing or not int32 [n]");
  const int64_t n64 = nt->second.shape[0];
  if (n64 < 1 || n64 > INT32_MAX || nt->second.e - nt->second.b != 4 * n64) return fail(KVP_EINVAL, "bad ntok");
  const int32_t n = (int32_t)n64;
  Q4Sizes z;
  q4_sizes(shape, n, &z);
  const auto tensors = q4_tensors(shape, n, z);
  for (auto& t : tensors) {
    auto it = ent.find(t.name);
    if (it == ent.end()) return fail(KVP_EINVAL, "a Q4 tensor is missing");
    if (it->second.dtype != t.dtype || it->second.shape != t.shape || it->second.e - it->second.b != t.bytes)
      return fail(KVP_EINVAL, "a Q4 tensor has another dtype or shape than the pool");
  }
  if (!image || image_bytes < z.image || max_blocks < n || !ntok) return n;
  std::vector<int32_t> nt_file;
  try {
    nt_file.resize((size_t)n);
  } catch (const std::bad_alloc&) {
    return fail(KVP_ENOMEM, "ntok");
  }
  if (!io_all(false, f.fd, (uint8_t*)nt_file.data(), 4LL * n, data0 + nt->second.b))
    return fail(KVP_EIO, "read failed");
  for (int32_t i = 0; i < n; ++i)
    if (nt_file[(size_t)i] < 0 || nt_file[(size_t)i] > shape->block_tokens)
      return fail(KVP_EINVAL, "ntok out of range in the file");
  // (a read error past this point may leave the image partly written)
  for (auto& t : tensors) {
    const Entry& e = ent[t.name];
    if (!io_parallel(false, f.fd, (uint8_t*)image + t.image_off, t.bytes, data0 + e.b))
      return fail(KVP_EIO, "read failed");
  }
  memcpy(ntok, nt_file.data(), 4 * (size_t)n);
  return n;
}

}  // namespace

extern "C" int kvpool_q4_load_file(const kvp_shape* shape, const char* path, const char* agent, void* image,
                                   int64_t image_bytes, int32_t* ntok, int32_t max_blocks) {
  try {
    return load_file(shape, path, agent, image, image_bytes, ntok, max_blocks);
  } catch (const std::bad_alloc&) {
    return fail(KVP_ENOMEM, "out of host memory");
  }
}
