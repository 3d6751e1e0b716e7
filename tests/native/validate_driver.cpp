// Sanitizer driver for the host-side validation of the C ABI (validate.cpp, built
// with g++ -fsanitize=address,undefined by tests/test_sanitizers.py; no HIP).
// Fixed cases check the status of well-formed and malformed requests; then seeded
// random descriptors, drawn from edge values (0, +-1, powers of two, INT_MIN,
// INT_MAX), pointers NULL / aligned / misaligned, go through every check.  Any
// undefined behaviour (integer overflow in a size test, an out-of-bounds read)
// stops the run.  Every failing status must leave a message in csa_last_error().
#include <climits>
#include <cstdio>
#include <cstring>

#include "validate.hpp"

namespace {

int g_fail = 0;
void expect(int got, int want, const char* what) {
  if (got != want) {
    std::fprintf(stderr, "FAIL %s: status %d, want %d (%s)\n", what, got, want, csa_last_error());
    g_fail = 1;
  }
  if (got != CSA_OK && std::strlen(csa_last_error()) == 0) {
    std::fprintf(stderr, "FAIL %s: no message\n", what);
    g_fail = 1;
  }
}

unsigned long long g_s = 0x2545F4914F6CDD1Dull;
unsigned next() {
  g_s ^= g_s << 13;
  g_s ^= g_s >> 7;
  g_s ^= g_s << 17;
  return (unsigned)(g_s >> 11);
}
int edge() {
  static const int v[] = {INT_MIN, -65537, -2, -1, 0, 1, 2, 3, 4, 7, 16, 31, 32, 33, 64, 96, 127, 128, 255, 256,
                          512, 2048, 4096, 4097, 8192, 65536, 65537, 1 << 24, INT_MAX - 1, INT_MAX};
  return v[next() % (sizeof(v) / sizeof(v[0]))];
}
alignas(64) unsigned char g_buf[4096];
const void* ptr() {
  switch (next() % 4) {
    case 0: return nullptr;
    case 1: return g_buf + 4;   // misaligned
    default: return g_buf;
  }
}
float fedge() {
  static const float v[] = {0.f, -1.f, 1e-6f, 0.0625f, 1.f, 1e30f, -0.f, __builtin_inff(), __builtin_nanf("")};
  return v[next() % (sizeof(v) / sizeof(v[0]))];
}
bool valid_status(int s) { return s >= CSA_OK && s <= CSA_ERR_HIP; }

csa_compress_desc good_compress() {
  csa_compress_desc d{};
  d.batch = 2; d.channels = 512; d.m = 4; d.zc = 512; d.n_rows = 64; d.tok_base = 0;
  d.entry_begin = 0; d.entry_end = 16; d.out_cap = 16; d.in_dtype = CSA_BF16; d.out_dtype = CSA_BF16;
  return d;
}
csa_index_desc good_index() {
  csa_index_desc d{};
  d.batch = 2; d.n_q = 1; d.idx_heads = 64; d.idx_dim = 128; d.m = 4; d.topk = 512; d.n_max = 1024;
  d.k_cap = 1024; d.dtype = CSA_BF16;
  return d;
}
csa_mqa_desc good_mqa() {
  csa_mqa_desc d{};
  d.batch = 2; d.n_q = 1; d.heads = 128; d.head_dim = 512; d.topk = 512; d.m = 4; d.n_max = 1024; d.window = 128;
  d.kv_cap = 1024; d.raw_cap = 128; d.dtype = CSA_BF16; d.eps = 1e-6f;
  return d;
}

void fixed_cases() {
  const void* p = g_buf;
  const float* f = reinterpret_cast<const float*>(g_buf);
  const int32_t* i32 = reinterpret_cast<const int32_t*>(g_buf);
  const uint8_t* u8 = g_buf;
  csa_compress_desc c = good_compress();
  expect(csa::check_compress(&c, p, p, f, f, g_buf), CSA_OK, "compress ok");
  expect(csa::check_compress(nullptr, p, p, f, f, g_buf), CSA_ERR_NULL, "compress null desc");
  c.zc = 3;
  expect(csa::check_compress(&c, p, p, f, f, g_buf), CSA_ERR_SHAPE, "compress zc");
  c = good_compress();
  c.tok_base = INT_MAX;   // rows [INT_MAX, INT_MAX + 64) do not cover the entries
  expect(csa::check_compress(&c, p, p, f, f, g_buf), CSA_ERR_SHAPE, "compress coverage near INT_MAX");
  c = good_compress();
  c.norm = 1; c.norm_eps = -1.f;
  expect(csa::check_compress(&c, p, p, f, f, g_buf), CSA_ERR_SHAPE, "compress norm eps");

  csa_index_desc x = good_index();
  expect(csa::check_index("t", &x, p, nullptr, f, p, nullptr, i32, i32), CSA_OK, "index ok");
  expect(csa::check_index("t", &x, p, nullptr, reinterpret_cast<const float*>(g_buf + 4), p, nullptr, i32, i32),
         CSA_ERR_ALIGN, "index w misaligned");
  x.k_cap = 1000;
  expect(csa::check_index("t", &x, p, nullptr, f, p, nullptr, i32, i32), CSA_ERR_SHAPE, "index k_cap < n_max");
  x = good_index();
  x.dtype = CSA_MXFP4;
  expect(csa::check_index("t", &x, p, nullptr, f, p, nullptr, i32, i32), CSA_ERR_NULL, "index mxfp4 scales");
  expect(csa::check_index("t", &x, p, u8, f, p, u8, i32, i32), CSA_OK, "index mxfp4 ok");
  x.n_max = 1 << 24; x.k_cap = 1 << 24;
  expect(csa::check_index("t", &x, p, u8, f, p, u8, i32, i32), CSA_OK, "index mxfp4 largest n_max");
  x.n_max = (1 << 24) + 1; x.k_cap = (1 << 24) + 1;
  expect(csa::check_index("t", &x, p, u8, f, p, u8, i32, i32), CSA_ERR_SHAPE, "index mxfp4 n_max bound");

  csa_mqa_desc a = good_mqa();
  expect(csa::check_mqa("t", &a, 0, p, p, p, p, i32, i32, g_buf), CSA_OK, "mqa ok");
  a.head_dim = 256;
  expect(csa::check_mqa("t", &a, 0, p, p, p, p, i32, i32, g_buf), CSA_ERR_UNSUPPORTED, "mqa head_dim");
  a = good_mqa();
  a.split_items = 48;
  expect(csa::check_mqa("t", &a, 0, p, p, p, p, i32, i32, g_buf), CSA_ERR_SHAPE, "mqa split_items");
  a = good_mqa();
  a.topk = INT_MAX; a.window = INT_MAX; a.split_items = 32;   // totals near overflow
  expect(csa::check_mqa("t", &a, 0, p, p, p, p, i32, i32, g_buf), CSA_ERR_SHAPE, "mqa huge topk");
  a = good_mqa();
  a.kv_dtype = CSA_FP8; a.scale = 1.f;
  expect(csa::check_mqa("t", &a, 0, p, p, p, p, i32, i32, g_buf), CSA_ERR_UNSUPPORTED, "mqa fp8 scale");

  csa_decode_args dargs{};
  expect(csa::check_decode(nullptr), CSA_ERR_NULL, "decode null");
  dargs.index = good_index();
  dargs.attn = good_mqa();
  dargs.q_idx = p; dargs.w = f; dargs.k_idx = p; dargs.n_entries = i32; dargs.q_pos = i32;
  dargs.q = p; dargs.kv = p; dargs.kv_raw = p; dargs.raw_base = i32; dargs.out = g_buf;
  dargs.out_idx = reinterpret_cast<int32_t*>(g_buf);
  expect(csa::check_decode(&dargs), CSA_OK, "decode ok");
  dargs.attn.topk = 256;
  expect(csa::check_decode(&dargs), CSA_ERR_SHAPE, "decode topk mismatch");
}

void fuzz(int rounds) {
  for (int r = 0; r < rounds; ++r) {
    csa_compress_desc c{};
    c.batch = edge(); c.channels = edge(); c.m = edge(); c.zc = (next() & 1) ? c.channels : edge();
    c.n_rows = edge(); c.tok_base = edge(); c.entry_begin = edge(); c.entry_end = edge(); c.out_cap = edge();
    c.in_dtype = edge(); c.out_dtype = edge(); c.norm = edge() & 1; c.norm_eps = fedge();
    int s = csa::check_compress((next() & 7) ? &c : nullptr, ptr(), ptr(), (const float*)ptr(), (const float*)ptr(),
                                ptr());
    if (!valid_status(s)) { std::fprintf(stderr, "FAIL compress status %d\n", s); g_fail = 1; }

    csa_index_desc x{};
    x.batch = edge(); x.n_q = edge(); x.idx_heads = edge(); x.idx_dim = (next() & 1) ? 128 : edge(); x.m = edge();
    x.topk = edge(); x.n_max = edge(); x.k_cap = edge(); x.dtype = next() % 5; x.q_quantize = edge() & 1;
    s = csa::check_index("f", (next() & 7) ? &x : nullptr, ptr(), (const uint8_t*)ptr(), (const float*)ptr(), ptr(),
                         (const uint8_t*)ptr(), (const int32_t*)ptr(), (const int32_t*)ptr());
    if (!valid_status(s)) { std::fprintf(stderr, "FAIL index status %d\n", s); g_fail = 1; }

    csa_mqa_desc a{};
    a.batch = edge(); a.n_q = edge(); a.heads = edge(); a.head_dim = (next() & 1) ? 512 : edge(); a.topk = edge();
    a.m = edge(); a.n_max = edge(); a.window = edge(); a.kv_cap = edge(); a.raw_cap = edge(); a.dtype = next() % 4;
    a.kv_dtype = (next() & 3) ? 0 : edge(); a.split_items = (next() & 1) ? 0 : edge(); a.scale = fedge();
    a.eps = fedge();
    s = csa::check_mqa("f", (next() & 7) ? &a : nullptr, (int)(next() & 1), ptr(), ptr(), ptr(), ptr(),
                       (const int32_t*)ptr(), (const int32_t*)ptr(), ptr());
    if (!valid_status(s)) { std::fprintf(stderr, "FAIL mqa status %d\n", s); g_fail = 1; }

    csa_decode_args d{};
    d.index = x; d.attn = a;
    d.q_idx = ptr(); d.w = (const float*)ptr(); d.k_idx = ptr(); d.n_entries = (const int32_t*)ptr();
    d.q_pos = (const int32_t*)ptr(); d.q = ptr(); d.kv = ptr(); d.kv_raw = ptr(); d.raw_base = (const int32_t*)ptr();
    d.out = (void*)ptr(); d.out_idx = (int32_t*)ptr();
    csa_compress_job job{};
    job.desc = c; job.a = ptr(); job.b = ptr(); job.za = (const float*)ptr(); job.zb = (const float*)ptr();
    job.out = (void*)ptr();
    if (next() & 1) d.kv_job = &job;
    if (next() & 1) d.key_job = &job;
    s = csa::check_decode(&d);
    if (!valid_status(s)) { std::fprintf(stderr, "FAIL decode status %d\n", s); g_fail = 1; }
    if (s != CSA_OK && std::strlen(csa_last_error()) == 0) { std::fprintf(stderr, "FAIL decode no message\n"); g_fail = 1; }
  }
}

}  // namespace

int main() {
  fixed_cases();
  fuzz(200000);
  if (!g_fail) std::printf("validate driver: all checks passed\n");
  return g_fail;
}
