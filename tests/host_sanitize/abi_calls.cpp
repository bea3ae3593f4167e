// Host-side checks of libmla's C entry points, built together with the library
// sources under AddressSanitizer and UndefinedBehaviorSanitizer (host code only;
// the device code is compiled as usual and never launched here).
//
// Every call below fails validation before anything reaches the device, so the
// program is safe with or without a GPU: it exercises the argument checks, the
// error-message buffer, the shape arithmetic of the size queries and the
// rejection paths of every entry point, over ordinary and extreme values.
#include <climits>
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <string>
#include <thread>
#include <vector>

#include "../../include/mla.h"

static int g_failures = 0;

#define EXPECT(cond, what)                                                        \
  do {                                                                            \
    if (!(cond)) {                                                                \
      std::fprintf(stderr, "FAIL %s:%d: %s (%s)\n", __FILE__, __LINE__, what, #cond); \
      ++g_failures;                                                               \
    }                                                                             \
  } while (0)

// An aligned address that is never dereferenced: every call fails first.
static void* fake(uintptr_t off = 0) { return reinterpret_cast<void*>((uintptr_t(1) << 20) + off); }
template <class T> static T* F(uintptr_t off = 0) { return static_cast<T*>(fake(off)); }

static bool msg_has(const char* needle) {
  const char* m = mla_last_error();
  const size_t n = std::strlen(m);  // the buffer is always NUL-terminated
  return n > 0 && n < 512 && std::strstr(m, needle) != nullptr;
}

struct DecodeArgs {
  const uint16_t* q_lat = F<uint16_t>();
  const uint16_t* q_lo = nullptr;
  const uint16_t* q_pe = F<uint16_t>();
  const uint16_t* kv = F<uint16_t>();
  int64_t num_pages = 10;
  const int32_t* bt = F<int32_t>();
  int max_blocks = 4;
  const int32_t* sl = F<int32_t>();
  int b = 2, s_q = 1, h = 16;
  float scale = 0.07f;
  int causal = 0;
  const int32_t* meta = F<int32_t>();
  const int32_t* ns = F<int32_t>();
  int slots = 8;
  void* ws = fake();
  size_t ws_bytes = size_t(1) << 30;
  uint16_t* o = F<uint16_t>();
  float* lse = F<float>();
  int call() const {
    return mla_decode_paged(q_lat, q_lo, q_pe, kv, num_pages, bt, max_blocks, sl, b, s_q, h, scale, causal, meta,
                            ns, slots, ws, ws_bytes, o, lse, nullptr);
  }
  int call_noalloc() const {
    return mla_decode_paged_noalloc(q_lat, q_lo, q_pe, kv, num_pages, bt, max_blocks, sl, b, s_q, h, scale, causal,
                                    meta, ns, slots, o, lse, nullptr);
  }
  int call_fp8() const {
    return mla_decode_paged_fp8(q_lat, q_lo, q_pe, reinterpret_cast<const uint8_t*>(kv), num_pages, bt, max_blocks,
                                sl, b, s_q, h, scale, causal, meta, ns, slots, ws, ws_bytes, o, lse, nullptr);
  }
};

static void decode_rejections() {
  struct Case {
    const char* name;
    void (*edit)(DecodeArgs&);
    int code;
    const char* msg;
  };
  const Case cases[] = {
      {"q_lat null", [](DecodeArgs& a) { a.q_lat = nullptr; }, MLA_ERR_INVALID_ARG, "NULL"},
      {"kv null", [](DecodeArgs& a) { a.kv = nullptr; }, MLA_ERR_INVALID_ARG, "NULL"},
      {"lse null", [](DecodeArgs& a) { a.lse = nullptr; }, MLA_ERR_INVALID_ARG, "NULL"},
      {"b = 0", [](DecodeArgs& a) { a.b = 0; }, MLA_ERR_INVALID_ARG, "b must be"},
      {"b = INT_MIN", [](DecodeArgs& a) { a.b = INT_MIN; }, MLA_ERR_INVALID_ARG, "b must be"},
      {"s_q = 9", [](DecodeArgs& a) { a.s_q = 9; }, MLA_ERR_INVALID_ARG, "s_q"},
      {"s_q = INT_MAX", [](DecodeArgs& a) { a.s_q = INT_MAX; }, MLA_ERR_INVALID_ARG, "s_q"},
      {"h = 48", [](DecodeArgs& a) { a.h = 48; }, MLA_ERR_UNSUPPORTED, "h must be"},
      {"h = INT_MIN", [](DecodeArgs& a) { a.h = INT_MIN; }, MLA_ERR_UNSUPPORTED, "h must be"},
      {"scale 0", [](DecodeArgs& a) { a.scale = 0.f; }, MLA_ERR_INVALID_ARG, "softmax_scale"},
      {"scale nan", [](DecodeArgs& a) { a.scale = NAN; }, MLA_ERR_INVALID_ARG, "softmax_scale"},
      {"scale inf", [](DecodeArgs& a) { a.scale = INFINITY; }, MLA_ERR_INVALID_ARG, "softmax_scale"},
      {"num_pages 0", [](DecodeArgs& a) { a.num_pages = 0; }, MLA_ERR_INVALID_ARG, "num_pages"},
      {"num_pages < 0", [](DecodeArgs& a) { a.num_pages = INT64_MIN; }, MLA_ERR_INVALID_ARG, "num_pages"},
      {"max_blocks 0", [](DecodeArgs& a) { a.max_blocks = 0; }, MLA_ERR_INVALID_ARG, "num_pages"},
      {"slots 0", [](DecodeArgs& a) { a.slots = 0; }, MLA_ERR_INVALID_ARG, "num_slots"},
      {"small workspace", [](DecodeArgs& a) { a.ws_bytes = 1000; }, MLA_ERR_WORKSPACE, "workspace"},
      {"workspace null", [](DecodeArgs& a) { a.ws = nullptr; }, MLA_ERR_INVALID_ARG, "NULL"},
      {"workspace misaligned", [](DecodeArgs& a) { a.ws = fake(16); }, MLA_ERR_INVALID_ARG, "aligned"},
      {"q_lat misaligned", [](DecodeArgs& a) { a.q_lat = F<uint16_t>(2); }, MLA_ERR_INVALID_ARG, "aligned"},
      {"q_lo misaligned", [](DecodeArgs& a) { a.q_lo = F<uint16_t>(8); }, MLA_ERR_INVALID_ARG, "aligned"},
  };
  for (const Case& c : cases) {
    DecodeArgs a;
    c.edit(a);
    EXPECT(a.call() == c.code, c.name);
    EXPECT(msg_has(c.msg), c.name);
    if (a.ws != nullptr && a.ws_bytes == (size_t(1) << 30) && reinterpret_cast<uintptr_t>(a.ws) % 256 == 0) {
      // the same arguments through the no-allocation entry point (no workspace there)
      EXPECT(a.call_noalloc() == c.code, c.name);
      EXPECT(msg_has(c.msg), c.name);
    }
  }
  DecodeArgs big;
  big.b = 8192;
  big.s_q = 8;
  big.h = 128;
  big.slots = 256;
  EXPECT(big.call_noalloc() == MLA_ERR_WORKSPACE, "noalloc beyond the built-in scratch");
  EXPECT(msg_has("built-in scratch"), "noalloc beyond the built-in scratch");

  DecodeArgs q;
  q.h = 64;  // 64 rows: more than the quantised-cache decode is built for
  EXPECT(q.call_fp8() == MLA_ERR_UNSUPPORTED, "fp8 decode with 64 rows");
  EXPECT(msg_has("at most 32 query rows"), "fp8 decode with 64 rows");
  q.h = 32;
  q.ws = nullptr;
  EXPECT(q.call_fp8() == MLA_ERR_INVALID_ARG, "fp8 decode without workspace");
  q.ws = fake();
  q.ws_bytes = 1000;
  EXPECT(q.call_fp8() == MLA_ERR_WORKSPACE, "fp8 decode with a small workspace");
}

static void other_rejections() {
  int32_t* I = F<int32_t>();
  uint16_t* H = F<uint16_t>();
  EXPECT(mla_get_metadata(I, 0, 8, 2, I, I, nullptr) == MLA_ERR_INVALID_ARG, "metadata b = 0");
  EXPECT(mla_get_metadata(I, MLA_MAX_BATCH + 1, 8, 2, I, I, nullptr) == MLA_ERR_INVALID_ARG, "metadata b too large");
  EXPECT(mla_get_metadata(I, INT_MAX, 8, 2, I, I, nullptr) == MLA_ERR_INVALID_ARG, "metadata b = INT_MAX");
  EXPECT(mla_get_metadata(I, 4, 0, 2, I, I, nullptr) == MLA_ERR_INVALID_ARG, "metadata slots 0");
  EXPECT(mla_get_metadata(I, 4, INT_MIN, 2, I, I, nullptr) == MLA_ERR_INVALID_ARG, "metadata slots < 0");
  EXPECT(mla_get_metadata(I, 4, 8, -1, I, I, nullptr) == MLA_ERR_INVALID_ARG, "metadata overhead < 0");
  EXPECT(mla_get_metadata(nullptr, 4, 8, 2, I, I, nullptr) == MLA_ERR_INVALID_ARG, "metadata null lengths");
  EXPECT(mla_absorb_q(H, H, H, nullptr, 2, 1, 100, nullptr) == MLA_ERR_UNSUPPORTED, "absorb h = 100");
  EXPECT(mla_absorb_q(nullptr, H, H, nullptr, 2, 1, 16, nullptr) == MLA_ERR_INVALID_ARG, "absorb null");
  EXPECT(mla_absorb_q(H, H, H, F<uint16_t>(8), 2, 1, 16, nullptr) == MLA_ERR_INVALID_ARG, "absorb misaligned lo");
  EXPECT(mla_absorb_q(H, H, H, nullptr, INT_MIN, 1, 16, nullptr) == MLA_ERR_INVALID_ARG, "absorb b < 0");
  EXPECT(mla_absorb_q_with_plan(H, H, H, nullptr, 2, 1, 16, nullptr, 8, 2, I, I, nullptr) == MLA_ERR_INVALID_ARG,
         "absorb+plan null lengths");
  EXPECT(mla_absorb_q_with_plan(H, H, H, nullptr, 9000, 1, 16, I, 8, 2, I, I, nullptr) == MLA_ERR_INVALID_ARG,
         "absorb+plan b too large");
  EXPECT(mla_absorb_q_with_plan(H, H, H, nullptr, 2, 1, 16, I, 8, -1, I, I, nullptr) == MLA_ERR_INVALID_ARG,
         "absorb+plan overhead < 0");
  EXPECT(mla_up_v(H, H, nullptr, 2, 1, 16, nullptr) == MLA_ERR_INVALID_ARG, "up_v null");
  EXPECT(mla_up_v(H, H, H, 2, 0, 16, nullptr) == MLA_ERR_INVALID_ARG, "up_v s_q 0");
  EXPECT(mla_up_v(H, H, H, 2, 1, 0, nullptr) == MLA_ERR_UNSUPPORTED, "up_v h 0");
  EXPECT(mla_gather_pages(H, 0, I, 4, I, 2, F<int64_t>(), H, nullptr) == MLA_ERR_INVALID_ARG, "gather no pages");
  EXPECT(mla_gather_pages(H, 4, I, 4, I, 2, nullptr, H, nullptr) == MLA_ERR_INVALID_ARG, "gather null offsets");
  EXPECT(mla_gather_pages(H, 4, I, 4, I, 2, F<int64_t>(), nullptr, nullptr) == MLA_ERR_INVALID_ARG, "gather null out");
  EXPECT(mla_append_kv(nullptr, H, 4, I, 4, I, 2, 1, nullptr) == MLA_ERR_INVALID_ARG, "append null rows");
  EXPECT(mla_append_kv(H, H, 4, I, 4, nullptr, 2, 1, nullptr) == MLA_ERR_INVALID_ARG, "append null lengths");
  EXPECT(mla_append_kv(H, H, 4, I, 4, I, 0, 1, nullptr) == MLA_ERR_INVALID_ARG, "append b 0");
  EXPECT(mla_append_kv(H, H, 4, I, 4, I, 2, 9, nullptr) == MLA_ERR_INVALID_ARG, "append s_q 9");
  EXPECT(mla_append_kv(H, H, 0, I, 4, I, 2, 1, nullptr) == MLA_ERR_INVALID_ARG, "append no pages");
  EXPECT(mla_append_kv(H, H, INT64_MIN, I, 4, I, 2, 1, nullptr) == MLA_ERR_INVALID_ARG, "append pages < 0");
  EXPECT(mla_append_kv(H, H, 4, I, 0, I, 2, 1, nullptr) == MLA_ERR_INVALID_ARG, "append max_blocks 0");
  EXPECT(mla_append_kv(F<uint16_t>(8), H, 4, I, 4, I, 2, 1, nullptr) == MLA_ERR_INVALID_ARG, "append misaligned");
  uint8_t* B = F<uint8_t>();
  EXPECT(mla_quantize_pages(nullptr, 4, B, nullptr) == MLA_ERR_INVALID_ARG, "quantize null");
  EXPECT(mla_quantize_pages(H, 0, B, nullptr) == MLA_ERR_INVALID_ARG, "quantize no pages");
  EXPECT(mla_quantize_pages(H, 4, F<uint8_t>(8), nullptr) == MLA_ERR_INVALID_ARG, "quantize misaligned");
  EXPECT(mla_append_kv_fp8(H, B, 4, I, 4, I, 2, 9, nullptr) == MLA_ERR_INVALID_ARG, "append fp8 s_q 9");
  EXPECT(mla_append_kv_fp8(H, nullptr, 4, I, 4, I, 2, 1, nullptr) == MLA_ERR_INVALID_ARG, "append fp8 null cache");
  EXPECT(mla_append_kv_fp8(H, F<uint8_t>(4), 4, I, 4, I, 2, 1, nullptr) == MLA_ERR_INVALID_ARG,
         "append fp8 misaligned");
  EXPECT(mla_num_slots(2, 1, 16, nullptr) == MLA_ERR_INVALID_ARG, "num_slots null out");
  int n = -7;
  EXPECT(mla_num_slots(0, 1, 16, &n) == MLA_ERR_INVALID_ARG && n == -7, "num_slots b 0");
  EXPECT(mla_num_slots(2, 1, 17, &n) == MLA_ERR_UNSUPPORTED && n == -7, "num_slots h 17");
  EXPECT(mla_take_device_error(nullptr) == MLA_ERR_INVALID_ARG, "take_device_error null");
}

static void size_queries() {
  // the formula of the header for accepted shapes, 0 for rejected ones, and no
  // arithmetic overflow anywhere in between
  const int bs[] = {INT_MIN, -1, 0, 1, 2, 127, 128, 4096, MLA_MAX_BATCH, MLA_MAX_BATCH + 1, 1 << 20, INT_MAX};
  const int sqs[] = {INT_MIN, 0, 1, 2, 8, 9, INT_MAX};
  const int hs[] = {INT_MIN, 0, 1, 16, 32, 48, 64, 128, 256, INT_MAX};
  const int slots[] = {INT_MIN, 0, 1, 256, 1 << 20, INT_MAX};
  for (int b : bs)
    for (int s_q : sqs)
      for (int h : hs)
        for (int ns : slots) {
          const size_t got = mla_workspace_bytes(b, s_q, h, ns);
          const bool ok = b >= 1 && b <= MLA_MAX_BATCH && s_q >= 1 && s_q <= 8 &&
                          (h == 16 || h == 32 || h == 64 || h == 128) && ns >= 1 && ns <= (1 << 20);
          if (!ok) {
            EXPECT(got == 0, "workspace of a rejected shape");
            continue;
          }
          const size_t M = size_t(s_q) * h, splits = size_t(b) + ns;
          auto pad = [](size_t x) { return (x + 255) / 256 * 256; };
          EXPECT(got == pad(splits * M * 1024) + 2 * pad(splits * M * 4), "workspace formula");
        }
  for (int b : bs)
    for (int s_q : sqs)
      for (int h : hs) {
        int n = -1;
        const int rc = mla_num_slots(b, s_q, h, &n);
        // without a device the query reports a HIP error; with one, a count >= 1
        EXPECT(rc == MLA_OK ? n >= 1 : n == -1, "num_slots output only on success");
        EXPECT(rc == MLA_OK || rc == MLA_ERR_INVALID_ARG || rc == MLA_ERR_UNSUPPORTED || rc == MLA_ERR_HIP,
               "num_slots status");
      }
}

static void error_buffer_per_thread() {
  // the message belongs to the calling thread and stays within its buffer
  std::vector<std::thread> ts;
  std::vector<int> ok(8, 0);
  for (int t = 0; t < 8; ++t)
    ts.emplace_back([t, &ok] {
      for (int i = 0; i < 200; ++i) {
        const int h = (t % 2) ? 48 : 16;
        const int rc = mla_up_v(F<uint16_t>(), F<uint16_t>(), F<uint16_t>(), 2, (t % 2) ? 1 : 0, h, nullptr);
        const std::string m = mla_last_error();
        const bool mine = (t % 2) ? (rc == MLA_ERR_UNSUPPORTED && m.find("h must be") != std::string::npos)
                                  : (rc == MLA_ERR_INVALID_ARG && m.find("s_q") != std::string::npos);
        if (!mine) return;
      }
      ok[t] = 1;
    });
  for (auto& th : ts) th.join();
  for (int t = 0; t < 8; ++t) EXPECT(ok[t] == 1, "per-thread error message");
}

int main() {
  decode_rejections();
  other_rejections();
  size_queries();
  error_buffer_per_thread();
  if (g_failures) {
    std::fprintf(stderr, "%d check(s) failed\n", g_failures);
    return 1;
  }
  std::printf("host checks passed\n");
  return 0;
}
