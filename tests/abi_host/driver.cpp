// Host-only driver of the C ABI's argument validation, built with
// AddressSanitizer and UndefinedBehaviorSanitizer against stand-in launchers
// (stubs.hip). Every call checks the documented status code, and that a
// rejected call launched nothing while an accepted one launched. Extreme
// sizes (INT_MAX extents, huge caches) exercise the size arithmetic, where
// UBSan reports any signed overflow. Prints "abi validation ok" and exits 0
// on success; reports the first mismatch and exits 1 otherwise.
#include <climits>
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <limits>

#include "sepattn.h"

extern "C" int sep_stub_launches;

namespace {

int failures = 0;
// Never dereferenced: the validation only looks at pointer values.
alignas(256) unsigned char arena[1 << 16];
void* const P = arena + 256;
void* const MIS = arena + 256 + 4;      // 4-byte aligned, not 16

void expect(const char* what, int got, int want, int launches_before, bool launched) {
  const bool ok_code = got == want;
  const int delta = sep_stub_launches - launches_before;
  const bool ok_launch = launched ? delta > 0 : delta == 0;
  if (!ok_code || !ok_launch) {
    std::fprintf(stderr, "FAIL %s: status %d (want %d), launches %d (want %s)\n", what, got, want, delta,
                 launched ? ">0" : "0");
    ++failures;
  }
}

#define CHECK(call, want)                                   \
  do {                                                      \
    const int before_ = sep_stub_launches;                  \
    const int got_ = (call);                                \
    expect(#call, got_, (want), before_, (want) == SEP_OK); \
  } while (0)

sep_cache good_cache() {
  sep_cache c;
  std::memset(&c, 0, sizeof c);
  c.a = 4; c.s = 64; c.p = 64; c.w = 256;
  c.B = 2; c.Hkv = 8; c.D = 128; c.dtype = SEP_BF16;
  c.k = P; c.v = P;
  c.pos = static_cast<int32_t*>(P);
  c.tok = static_cast<int32_t*>(P);
  c.state = static_cast<int64_t*>(P);
  c.policy = 0;
  return c;
}

const int32_t* I32 = static_cast<const int32_t*>(P);
uint8_t* U8 = static_cast<uint8_t*>(P);
int32_t* O32 = static_cast<int32_t*>(P);
float* F32 = static_cast<float*>(P);

void mask_build() {
  CHECK(sep_mask_build(I32, 1, 8, I32, 1, 4, 2, U8, nullptr, 0, 0, nullptr, nullptr), SEP_OK);
  CHECK(sep_mask_build(I32, 1, 8, I32, 1, 4, 2, U8, U8, 64, 64, U8, nullptr), SEP_OK);
  CHECK(sep_mask_build(I32, 1, 8, nullptr, 0, 0, 1, U8, nullptr, 0, 0, nullptr, nullptr), SEP_OK);
  CHECK(sep_mask_build(I32, INT_MAX, INT_MAX, I32, 64, INT_MAX, INT_MAX, U8, U8, 4096, 4096, nullptr, nullptr),
        SEP_OK);
  CHECK(sep_mask_build(nullptr, 1, 8, I32, 1, 4, 2, U8, nullptr, 0, 0, nullptr, nullptr), SEP_ERR_NULL);
  CHECK(sep_mask_build(I32, 1, 8, I32, 1, 4, 2, nullptr, nullptr, 0, 0, nullptr, nullptr), SEP_ERR_NULL);
  CHECK(sep_mask_build(I32, 1, 8, nullptr, 3, 4, 2, U8, nullptr, 0, 0, nullptr, nullptr), SEP_ERR_NULL);
  CHECK(sep_mask_build(I32, 0, 8, I32, 1, 4, 2, U8, nullptr, 0, 0, nullptr, nullptr), SEP_ERR_SHAPE);
  CHECK(sep_mask_build(I32, 1, -8, I32, 1, 4, 2, U8, nullptr, 0, 0, nullptr, nullptr), SEP_ERR_SHAPE);
  CHECK(sep_mask_build(I32, 1, 8, I32, 65, 4, 2, U8, nullptr, 0, 0, nullptr, nullptr), SEP_ERR_SHAPE);
  CHECK(sep_mask_build(I32, 1, 8, I32, -1, 4, 2, U8, nullptr, 0, 0, nullptr, nullptr), SEP_ERR_SHAPE);
  CHECK(sep_mask_build(I32, 1, 8, I32, 1, -1, 2, U8, nullptr, 0, 0, nullptr, nullptr), SEP_ERR_PARAM);
  CHECK(sep_mask_build(I32, 1, 8, I32, 1, 4, 0, U8, nullptr, 0, 0, nullptr, nullptr), SEP_ERR_PARAM);
  CHECK(sep_mask_build(I32, 1, 8, I32, 1, 4, 2, U8, U8, 0, 8, nullptr, nullptr), SEP_ERR_SHAPE);
  CHECK(sep_mask_build(I32, 1, 8, I32, 1, 4, 2, U8, U8, 8, 4097, nullptr, nullptr), SEP_ERR_SHAPE);
  CHECK(sep_mask_build(I32, 1, 8193, I32, 1, 4, 2, U8, nullptr, 0, 0, U8, nullptr), SEP_ERR_SHAPE);
  CHECK(sep_mask_build(static_cast<const int32_t*>(MIS), 1, 8, I32, 1, 4, 2, U8, nullptr, 0, 0, nullptr, nullptr),
        SEP_ERR_ALIGN);
}

void compaction() {
  CHECK(sep_index_compact(U8, 3, 100, O32, O32, O32, nullptr), SEP_OK);
  CHECK(sep_index_compact(U8, INT_MAX, INT_MAX, O32, O32, nullptr, nullptr), SEP_OK);
  CHECK(sep_index_compact(nullptr, 1, 8, O32, O32, O32, nullptr), SEP_ERR_NULL);
  CHECK(sep_index_compact(U8, 1, 8, nullptr, O32, O32, nullptr), SEP_ERR_NULL);
  CHECK(sep_index_compact(U8, 1, 8, O32, nullptr, O32, nullptr), SEP_ERR_NULL);
  CHECK(sep_index_compact(U8, 0, 8, O32, O32, O32, nullptr), SEP_ERR_SHAPE);
  CHECK(sep_index_compact(U8, 1, 0, O32, O32, O32, nullptr), SEP_ERR_SHAPE);
  CHECK(sep_mask_compact(I32, 2, 77, I32, 9, U8, O32, O32, O32, nullptr), SEP_OK);
  CHECK(sep_mask_compact(I32, 2, 77, nullptr, 0, U8, O32, O32, nullptr, nullptr), SEP_OK);
  CHECK(sep_mask_compact(nullptr, 2, 77, I32, 9, U8, O32, O32, O32, nullptr), SEP_ERR_NULL);
  CHECK(sep_mask_compact(I32, 2, 77, nullptr, 9, U8, O32, O32, O32, nullptr), SEP_ERR_NULL);
  CHECK(sep_mask_compact(I32, 2, 77, I32, 65, U8, O32, O32, O32, nullptr), SEP_ERR_SHAPE);
  CHECK(sep_mask_compact(I32, -2, 77, I32, 9, U8, O32, O32, O32, nullptr), SEP_ERR_SHAPE);
  CHECK(sep_mask_compact(I32, 2, 77, I32, 9, static_cast<uint8_t*>(MIS), O32, O32, O32, nullptr), SEP_ERR_ALIGN);
  CHECK(sep_mask_compact(I32, 2, 77, I32, 9, U8, static_cast<int32_t*>(MIS), O32, O32, nullptr), SEP_ERR_ALIGN);
}

int prefill(const void* q, int dtype, int B, int Hq, int Hkv, int S, int D, int a, int n, float scale, void* out) {
  return sep_attn_prefill(q, P, P, dtype, B, Hq, Hkv, S, D, U8, I32, I32, a, n, scale, out, F32, nullptr);
}

void prefill_checks() {
  const float sc = 0.088f, inf = std::numeric_limits<float>::infinity(), nan = std::nanf("");
  CHECK(prefill(P, SEP_BF16, 1, 32, 8, 8192, 128, 4, 256, sc, P), SEP_OK);
  CHECK(prefill(P, SEP_F32, 1, 2, 2, 512, 64, 4, 64, sc, P), SEP_OK);
  CHECK(prefill(P, SEP_BF16, INT_MAX, 16, 1, INT_MAX, 128, INT_MAX, INT_MAX, sc, P), SEP_OK);
  CHECK(prefill(nullptr, SEP_BF16, 1, 32, 8, 64, 128, 4, 16, sc, P), SEP_ERR_NULL);
  CHECK(prefill(P, SEP_BF16, 1, 32, 8, 64, 128, 4, 16, sc, nullptr), SEP_ERR_NULL);
  CHECK(sep_attn_prefill(P, P, P, SEP_BF16, 1, 32, 8, 64, 128, U8, nullptr, I32, 4, 16, sc, P, F32, nullptr),
        SEP_ERR_NULL);
  CHECK(prefill(P, 7, 1, 32, 8, 64, 128, 4, 16, sc, P), SEP_ERR_DTYPE);
  CHECK(prefill(P, SEP_BF16, 1, 30, 8, 64, 128, 4, 16, sc, P), SEP_ERR_SHAPE);
  CHECK(prefill(P, SEP_BF16, 1, 8 * 17, 8, 64, 128, 4, 16, sc, P), SEP_ERR_SHAPE);
  CHECK(prefill(P, SEP_BF16, 1, 32, 8, 64, 96, 4, 16, sc, P), SEP_ERR_SHAPE);
  CHECK(prefill(P, SEP_BF16, 1, 32, 0, 64, 128, 4, 16, sc, P), SEP_ERR_SHAPE);
  CHECK(prefill(P, SEP_BF16, 1, 32, 8, 0, 128, 4, 16, sc, P), SEP_ERR_SHAPE);
  CHECK(prefill(P, SEP_BF16, 1, 32, 8, 64, 128, -1, 16, sc, P), SEP_ERR_PARAM);
  CHECK(prefill(P, SEP_BF16, 1, 32, 8, 64, 128, 4, 0, sc, P), SEP_ERR_PARAM);
  CHECK(prefill(P, SEP_BF16, 1, 32, 8, 64, 128, 4, 16, 0.0f, P), SEP_ERR_PARAM);
  CHECK(prefill(P, SEP_BF16, 1, 32, 8, 64, 128, 4, 16, -sc, P), SEP_ERR_PARAM);
  CHECK(prefill(P, SEP_BF16, 1, 32, 8, 64, 128, 4, 16, nan, P), SEP_ERR_PARAM);
  CHECK(prefill(P, SEP_BF16, 1, 32, 8, 64, 128, 4, 16, inf, P), SEP_ERR_PARAM);
  CHECK(prefill(MIS, SEP_BF16, 1, 32, 8, 64, 128, 4, 16, sc, P), SEP_ERR_ALIGN);
  CHECK(prefill(P, SEP_BF16, 1, 32, 8, 64, 128, 4, 16, sc, MIS), SEP_ERR_ALIGN);
}

int backward(int S, float* delta, float* dq, int dtype = SEP_BF16) {
  return sep_attn_prefill_backward(P, P, P, P, P, F32, dtype, 1, 32, 8, S, 128, U8, I32, I32, 4, 256, 0.088f,
                                   delta, dq, F32, F32, nullptr);
}

void backward_checks() {
  CHECK(backward(8192, F32, F32), SEP_OK);
  CHECK(backward(SEP_MAX_BACKWARD_S, F32, F32, SEP_F32), SEP_OK);
  CHECK(backward(SEP_MAX_BACKWARD_S + 1, F32, F32), SEP_ERR_SHAPE);
  CHECK(backward(8192, nullptr, F32), SEP_ERR_NULL);
  CHECK(backward(8192, F32, nullptr), SEP_ERR_NULL);
  CHECK(backward(8192, F32, F32, 3), SEP_ERR_DTYPE);
  CHECK(backward(8192, F32, reinterpret_cast<float*>(MIS)), SEP_ERR_ALIGN);
}

void cache_checks() {
  sep_cache c = good_cache();
  const int32_t* sep = I32;
  CHECK(sep_cache_reset(&c, nullptr), SEP_OK);
  CHECK(sep_cache_update(&c, P, P, I32, 1, sep, 9, nullptr), SEP_OK);
  CHECK(sep_cache_update(&c, P, P, I32, INT_MAX, nullptr, 0, nullptr), SEP_OK);
  CHECK(sep_cache_update(nullptr, P, P, I32, 1, sep, 9, nullptr), SEP_ERR_NULL);
  CHECK(sep_cache_update(&c, nullptr, P, I32, 1, sep, 9, nullptr), SEP_ERR_NULL);
  CHECK(sep_cache_update(&c, P, P, nullptr, 1, sep, 9, nullptr), SEP_ERR_NULL);
  CHECK(sep_cache_update(&c, P, P, I32, 1, nullptr, 9, nullptr), SEP_ERR_NULL);
  CHECK(sep_cache_update(&c, P, P, I32, 0, sep, 9, nullptr), SEP_ERR_SHAPE);
  CHECK(sep_cache_update(&c, P, P, I32, 1, sep, 65, nullptr), SEP_ERR_SHAPE);
  CHECK(sep_cache_update(&c, MIS, P, I32, 1, sep, 9, nullptr), SEP_ERR_ALIGN);

  // the parameter contract of the study notes' "Streaming 参数约束", c = a+s+p+w
  struct Bad {
    const char* what;
    void (*edit)(sep_cache&);
    int want;
  } bad[] = {
      {"pos NULL", [](sep_cache& x) { x.pos = nullptr; }, SEP_ERR_NULL},
      {"state NULL", [](sep_cache& x) { x.state = nullptr; }, SEP_ERR_NULL},
      {"k NULL", [](sep_cache& x) { x.k = nullptr; }, SEP_ERR_NULL},
      {"B 0", [](sep_cache& x) { x.B = 0; }, SEP_ERR_SHAPE},
      {"Hkv -1", [](sep_cache& x) { x.Hkv = -1; }, SEP_ERR_SHAPE},
      {"D 96", [](sep_cache& x) { x.D = 96; }, SEP_ERR_SHAPE},
      {"dtype 5", [](sep_cache& x) { x.dtype = 5; }, SEP_ERR_DTYPE},
      {"a -1", [](sep_cache& x) { x.a = -1; }, SEP_ERR_PARAM},
      {"w 0", [](sep_cache& x) { x.w = 0; }, SEP_ERR_PARAM},
      {"s 0 p 5", [](sep_cache& x) { x.s = 0; }, SEP_ERR_PARAM},
      {"s 5 p 0", [](sep_cache& x) { x.p = 0; }, SEP_ERR_PARAM},
      {"s above the cap", [](sep_cache& x) { x.s = 8193; }, SEP_ERR_PARAM},
      {"unknown policy bit", [](sep_cache& x) { x.policy = 4; }, SEP_ERR_PARAM},
      {"dynamic ring too long", [](sep_cache& x) { x.policy = SEP_POLICY_DYNAMIC; x.w = 32768; }, SEP_ERR_PARAM},
      {"INT_MAX window", [](sep_cache& x) { x.w = INT_MAX; x.p = INT_MAX; }, SEP_ERR_SHAPE},
      {"INT_MAX initial", [](sep_cache& x) { x.a = INT_MAX; }, SEP_ERR_SHAPE},
      {"k misaligned", [](sep_cache& x) { x.k = MIS; }, SEP_ERR_ALIGN},
  };
  for (const Bad& b : bad) {
    sep_cache x = good_cache();
    b.edit(x);
    const bool kv = std::strcmp(b.what, "k NULL") == 0 || std::strcmp(b.what, "k misaligned") == 0;
    int before = sep_stub_launches;
    int got = sep_cache_update(&x, P, P, I32, 1, sep, 9, nullptr);
    expect(b.what, got, b.want, before, false);
    before = sep_stub_launches;
    got = sep_attn_decode(P, P, P, &x, 32, 0.088f, P, F32, nullptr);
    expect(b.what, got, b.want, before, false);
    before = sep_stub_launches;
    got = sep_cache_reset(&x, nullptr);
    expect(b.what, got, kv ? SEP_OK : b.want, before, kv);   // reset touches no K/V
  }
  sep_cache stream = good_cache();
  stream.s = 0;
  stream.p = 0;
  CHECK(sep_cache_update(&stream, P, P, I32, 1, sep, 9, nullptr), SEP_OK);   // StreamingLLM mode
}

void decode_checks() {
  sep_cache c = good_cache();
  const float sc = 0.088f;
  const int slots = c.a + c.s + c.p + c.w;
  CHECK(sep_attn_decode(P, P, P, &c, 32, sc, P, F32, nullptr), SEP_OK);
  CHECK(sep_attn_decode(P, P, P, &c, 32, sc, P, nullptr, nullptr), SEP_OK);
  CHECK(sep_attn_decode(nullptr, P, P, &c, 32, sc, P, F32, nullptr), SEP_ERR_NULL);
  CHECK(sep_attn_decode(P, P, P, &c, 32, sc, nullptr, F32, nullptr), SEP_ERR_NULL);
  CHECK(sep_attn_decode(P, P, P, &c, 30, sc, P, F32, nullptr), SEP_ERR_SHAPE);
  CHECK(sep_attn_decode(P, P, P, &c, 8 * 17, sc, P, F32, nullptr), SEP_ERR_SHAPE);
  CHECK(sep_attn_decode(P, P, P, &c, 32, 0.0f, P, F32, nullptr), SEP_ERR_PARAM);
  CHECK(sep_attn_decode(P, MIS, P, &c, 32, sc, P, F32, nullptr), SEP_ERR_ALIGN);
  sep_cache f = good_cache();
  f.dtype = SEP_F32;
  CHECK(sep_attn_decode(P, P, P, &f, 32, sc, P, F32, nullptr), SEP_ERR_DTYPE);

  CHECK(sep_rope_table(500000.0, 128, slots + 1, F32, nullptr), SEP_OK);
  CHECK(sep_rope_table(500000.0, 128, 0, F32, nullptr), SEP_ERR_SHAPE);
  CHECK(sep_rope_table(500000.0, 32, 10, F32, nullptr), SEP_ERR_SHAPE);
  CHECK(sep_rope_table(1.0, 128, 10, F32, nullptr), SEP_ERR_PARAM);
  CHECK(sep_rope_table(std::nan(""), 128, 10, F32, nullptr), SEP_ERR_PARAM);
  CHECK(sep_rope_table(500000.0, 128, 10, nullptr, nullptr), SEP_ERR_NULL);
  CHECK(sep_attn_decode_rope(P, P, P, &c, 32, sc, F32, slots + 1, P, F32, nullptr), SEP_OK);
  CHECK(sep_attn_decode_rope(P, P, P, &c, 32, sc, F32, slots, P, F32, nullptr), SEP_ERR_PARAM);
  CHECK(sep_attn_decode_rope(P, P, P, &c, 32, sc, nullptr, slots + 1, P, F32, nullptr), SEP_ERR_NULL);

  CHECK(sep_decode_update(P, P, P, I32, I32, 9, &c, 32, sc, nullptr, 0, P, F32, nullptr), SEP_OK);
  CHECK(sep_decode_update(P, P, P, I32, I32, 9, &c, 32, sc, F32, slots + 1, P, nullptr, nullptr), SEP_OK);
  CHECK(sep_decode_update(P, P, P, I32, I32, 9, &c, 32, sc, F32, slots, P, F32, nullptr), SEP_ERR_PARAM);
  CHECK(sep_decode_update(P, P, P, nullptr, I32, 9, &c, 32, sc, nullptr, 0, P, F32, nullptr), SEP_ERR_NULL);
  CHECK(sep_decode_update(P, P, P, I32, nullptr, 9, &c, 32, sc, nullptr, 0, P, F32, nullptr), SEP_ERR_NULL);
  CHECK(sep_decode_update(P, P, P, I32, I32, 65, &c, 32, sc, nullptr, 0, P, F32, nullptr), SEP_ERR_SHAPE);
  CHECK(sep_decode_update(P, P, P, I32, I32, 9, &c, 32, sc, nullptr, 0, MIS, F32, nullptr), SEP_ERR_ALIGN);
}

void chunk_checks() {
  sep_cache c = good_cache();
  const float sc = 0.088f;
  const size_t need = sep_chunk_workspace_bytes(&c, 2048);
  if (need == 0) {
    std::fprintf(stderr, "FAIL workspace size of a valid cache is 0\n");
    ++failures;
  }
  if (sep_chunk_workspace_bytes(nullptr, 2048) != 0 || sep_chunk_workspace_bytes(&c, 0) != 0) {
    std::fprintf(stderr, "FAIL workspace size of an invalid call is not 0\n");
    ++failures;
  }
  CHECK(sep_attn_prefill_chunk(P, P, P, I32, 2048, I32, 9, &c, 32, 256, sc, P, need, P, F32, nullptr), SEP_OK);
  CHECK(sep_attn_prefill_chunk(P, P, P, I32, 2048, I32, 9, &c, 32, 256, sc, P, need - 1, P, F32, nullptr),
        SEP_ERR_WORKSPACE);
  CHECK(sep_attn_prefill_chunk(P, P, P, I32, 2048, I32, 9, &c, 32, 256, sc, nullptr, need, P, F32, nullptr),
        SEP_ERR_WORKSPACE);
  CHECK(sep_attn_prefill_chunk(P, P, P, I32, 2048, I32, 9, &c, 32, 256, sc, arena + 16, need, P, F32, nullptr),
        SEP_ERR_WORKSPACE);
  CHECK(sep_attn_prefill_chunk(P, P, P, I32, 0, I32, 9, &c, 32, 256, sc, P, need, P, F32, nullptr), SEP_ERR_SHAPE);
  CHECK(sep_attn_prefill_chunk(P, P, P, I32, INT_MAX, I32, 9, &c, 32, 256, sc, P, SIZE_MAX, P, F32, nullptr),
        SEP_ERR_SHAPE);
  CHECK(sep_attn_prefill_chunk(P, P, P, I32, 2048, I32, 9, &c, 32, 0, sc, P, need, P, F32, nullptr), SEP_ERR_PARAM);
  CHECK(sep_attn_prefill_chunk(P, P, P, nullptr, 2048, I32, 9, &c, 32, 256, sc, P, need, P, F32, nullptr),
        SEP_ERR_NULL);
  CHECK(sep_attn_prefill_chunk(P, P, P, I32, 2048, I32, 9, &c, 31, 256, sc, P, need, P, F32, nullptr),
        SEP_ERR_SHAPE);
}

void strings() {
  for (int code = -7; code <= 0; ++code) {
    const char* s = sep_status_string(code);
    if (s == nullptr || std::strlen(s) == 0) {
      std::fprintf(stderr, "FAIL no status string for %d\n", code);
      ++failures;
    }
  }
  if (std::strcmp(sep_status_string(INT_MIN), "unknown status") != 0) ++failures;
  if (sep_version() < 10100) ++failures;
}

}  // namespace

int main() {
  mask_build();
  compaction();
  prefill_checks();
  backward_checks();
  cache_checks();
  decode_checks();
  chunk_checks();
  strings();
  if (failures) {
    std::fprintf(stderr, "%d check(s) failed\n", failures);
    return 1;
  }
  std::printf("abi validation ok (%d launches accepted)\n", sep_stub_launches);
  return 0;
}
