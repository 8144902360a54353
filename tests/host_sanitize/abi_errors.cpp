// Host-only driver for the C-ABI layer under AddressSanitizer and UndefinedBehaviorSanitizer.
//
// Built with g++ from gqa_kv_cache_qwen3_amd/csrc/mtd_api.cpp (the real validation code) plus the
// stand-in launchers below, it calls every entry point with arguments that each check must refuse
// (and the size queries with extreme values) and verifies the status codes and the error text.
// No GPU is needed: every check runs before any HIP call, and a stand-in launcher that is reached
// aborts the run.
#include <limits.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "mtd.h"
#include "mtd_internal.h"

namespace mtd {
[[noreturn]] static void reached(const char* what) {
  fprintf(stderr, "launcher reached in a host-only run: %s\n", what);
  abort();
}
hipError_t launch_kv_append(const KvPools&, const uint16_t*, const uint16_t*, const int32_t*, const int32_t*,
                            const int32_t*, int, int, int, hipStream_t) { reached("kv_append"); }
hipError_t launch_prefill(const KvPools&, const uint16_t*, int, int, const int32_t*, float, void*, int, float*,
                          float*, hipStream_t) { reached("prefill"); }
hipError_t launch_decode(const KvPools&, const uint16_t*, const uint16_t*, const uint16_t*, const int32_t*,
                         const int32_t*, int, int, int, float, void*, float*, float*, hipStream_t) {
  reached("decode");
}
hipError_t launch_qkv_proj(const uint16_t*, const uint16_t*, int, uint16_t*, uint16_t*, uint16_t*, hipStream_t) {
  reached("qkv_proj");
}
hipError_t launch_o_proj(const float*, const uint16_t*, int, uint16_t*, hipStream_t) { reached("o_proj"); }
hipError_t launch_attn_merge(const float*, const float*, int, int, float*, float*, hipStream_t) {
  reached("attn_merge");
}
hipError_t launch_page_read(const KvPools&, const int32_t*, int, int, uint32_t*, hipStream_t) { reached("page_read"); }
hipError_t decode_scratch(void**) { reached("decode_scratch"); }
}  // namespace mtd

static int g_failures = 0;

static void expect(int got, int want, const char* what) {
  const char* detail = mtd_last_error();
  if (got != want) {
    fprintf(stderr, "FAIL %s: status %d, want %d (%s)\n", what, got, want, detail);
    ++g_failures;
  } else if (want != MTD_OK && (detail == nullptr || detail[0] == '\0')) {
    fprintf(stderr, "FAIL %s: no error detail\n", what);
    ++g_failures;
  }
}

int main() {
  // Placeholders: 16-byte aligned, never dereferenced (every call below fails before a launch).
  void* const P = reinterpret_cast<void*>(0x1000);
  int32_t* const I = reinterpret_cast<int32_t*>(0x2000);
  float* const F = reinterpret_cast<float*>(0x3000);
  void* const odd = reinterpret_cast<void*>(0x1004);
  mtd_kv_layer_t kv{P, P, 10, 64, 8, 128};
  mtd_kv_layer_t bad = kv;

  // layer checks (through mtd_kv_append)
  expect(mtd_kv_append(nullptr, P, P, I, I, I, 4, 1, 3, nullptr), MTD_ERR_INVALID_ARG, "append: kv NULL");
  bad = kv; bad.k_pages = nullptr;
  expect(mtd_kv_append(&bad, P, P, I, I, I, 4, 1, 3, nullptr), MTD_ERR_INVALID_ARG, "append: k_pages NULL");
  bad = kv; bad.v_pages = odd;
  expect(mtd_kv_append(&bad, P, P, I, I, I, 4, 1, 3, nullptr), MTD_ERR_INVALID_ARG, "append: v_pages unaligned");
  bad = kv; bad.num_pages = 0;
  expect(mtd_kv_append(&bad, P, P, I, I, I, 4, 1, 3, nullptr), MTD_ERR_INVALID_ARG, "append: no pages");
  bad = kv; bad.page_size = 16;
  expect(mtd_kv_append(&bad, P, P, I, I, I, 4, 1, 3, nullptr), MTD_ERR_UNSUPPORTED, "append: page size");
  bad = kv; bad.num_kv_heads = 4;
  expect(mtd_kv_append(&bad, P, P, I, I, I, 4, 1, 3, nullptr), MTD_ERR_UNSUPPORTED, "append: kv heads");
  bad = kv; bad.head_dim = 64;
  expect(mtd_kv_append(&bad, P, P, I, I, I, 4, 1, 3, nullptr), MTD_ERR_UNSUPPORTED, "append: head_dim");
  expect(mtd_kv_append(&kv, P, P, I, I, I, 4, 0, 3, nullptr), MTD_ERR_INVALID_ARG, "append: n_req");
  expect(mtd_kv_append(&kv, P, P, I, I, I, 4, 1, -1, nullptr), MTD_ERR_INVALID_ARG, "append: n_new");
  expect(mtd_kv_append(&kv, P, P, I, I, I, 0, 1, 3, nullptr), MTD_ERR_INVALID_ARG, "append: bt_stride");
  expect(mtd_kv_append(&kv, nullptr, P, I, I, I, 4, 1, 3, nullptr), MTD_ERR_INVALID_ARG, "append: k_new NULL");
  expect(mtd_kv_append(&kv, odd, P, I, I, I, 4, 1, 3, nullptr), MTD_ERR_INVALID_ARG, "append: k_new unaligned");
  expect(mtd_kv_append(&kv, P, P, nullptr, I, I, 4, 1, 3, nullptr), MTD_ERR_INVALID_ARG, "append: cu_new NULL");
  expect(mtd_kv_append(&kv, P, P, I, I, I, 4, 1, 0, nullptr), MTD_OK, "append: no tokens");

  // prefill
  expect(mtd_attn_prefill_chunk(&kv, P, 100, 0, I, 2, 8, 0.088f, nullptr, 0, F, F, nullptr), MTD_ERR_UNSUPPORTED,
         "prefill: heads");
  expect(mtd_attn_prefill_chunk(&kv, P, 100, 0, I, 2, 12, 0.088f, nullptr, 0, F, F, nullptr), MTD_ERR_UNSUPPORTED,
         "prefill: heads not a multiple");
  expect(mtd_attn_prefill_chunk(&kv, P, 100, 0, I, 2, 16, -1.f, nullptr, 0, F, F, nullptr), MTD_ERR_INVALID_ARG,
         "prefill: scale");
  expect(mtd_attn_prefill_chunk(&kv, P, 100, 0, I, 2, 16, __builtin_inff(), nullptr, 0, F, F, nullptr),
         MTD_ERR_INVALID_ARG, "prefill: scale inf");
  expect(mtd_attn_prefill_chunk(&kv, nullptr, 100, 0, I, 2, 16, 0.088f, nullptr, 0, F, F, nullptr),
         MTD_ERR_INVALID_ARG, "prefill: q NULL");
  expect(mtd_attn_prefill_chunk(&kv, P, 0, 0, I, 2, 16, 0.088f, nullptr, 0, F, F, nullptr), MTD_ERR_INVALID_ARG,
         "prefill: chunk_len");
  expect(mtd_attn_prefill_chunk(&kv, P, 100, -1, I, 2, 16, 0.088f, nullptr, 0, F, F, nullptr), MTD_ERR_INVALID_ARG,
         "prefill: prefix_len");
  expect(mtd_attn_prefill_chunk(&kv, P, INT_MAX, INT_MAX, I, INT_MAX, 16, 0.088f, nullptr, 0, F, F, nullptr),
         MTD_ERR_CAPACITY, "prefill: total overflows int");
  expect(mtd_attn_prefill_chunk(&kv, P, 100, 0, I, 1, 16, 0.088f, nullptr, 0, F, F, nullptr), MTD_ERR_CAPACITY,
         "prefill: table short");
  expect(mtd_attn_prefill_chunk(&kv, P, 100, 0, I, 2, 16, 0.088f, P, 16, F, F, nullptr), MTD_ERR_WORKSPACE,
         "prefill: workspace small");
  expect(mtd_attn_prefill_chunk(&kv, P, 100, 0, I, 2, 16, 0.088f, odd, 1 << 30, F, F, nullptr), MTD_ERR_INVALID_ARG,
         "prefill: workspace unaligned");

  expect(mtd_attn_prefill_chunk_cus(&kv, P, 100, 0, I, 2, 16, 0.088f, P, 1 << 30, -1, F, F, nullptr),
         MTD_ERR_INVALID_ARG, "prefill_cus: negative budget");
  expect(mtd_attn_prefill_chunk_cus(&kv, P, 100, 0, I, 2, 16, 0.088f, nullptr, 0, 64, F, F, nullptr),
         MTD_ERR_WORKSPACE, "prefill_cus: budget without workspace");

  // decode and its allocation-free variant
  expect(mtd_attn_decode(&kv, P, I, I, 16, 2, 1000, 16, 0.088f, nullptr, 0, F, F, nullptr), MTD_ERR_WORKSPACE,
         "decode: no workspace");
  expect(mtd_attn_decode(&kv, P, I, I, 16, 0, 1000, 16, 0.088f, P, 1 << 30, F, F, nullptr), MTD_ERR_INVALID_ARG,
         "decode: batch");
  expect(mtd_attn_decode(&kv, P, I, I, 16, 2, MTD_MAX_CONTEXT + 1, 16, 0.088f, P, 1 << 30, F, F, nullptr),
         MTD_ERR_CAPACITY, "decode: max_kv_len");
  expect(mtd_attn_decode(&kv, P, I, I, 15, 2, 1000, 16, 0.088f, P, 1 << 30, F, F, nullptr), MTD_ERR_CAPACITY,
         "decode: bt_stride");
  expect(mtd_attn_decode(&kv, P, I, I, 16, 2, 1000, 16, 0.088f, P, 1 << 30, F, nullptr, nullptr),
         MTD_ERR_INVALID_ARG, "decode: lse NULL");
  expect(mtd_attn_decode_append(&kv, P, nullptr, P, I, I, 16, 2, 1000, 16, 0.088f, P, 1 << 30, F, F, nullptr),
         MTD_ERR_INVALID_ARG, "decode_append: k_new NULL");
  expect(mtd_attn_decode_append(&kv, P, P, (const char*)P + 8, I, I, 16, 2, 1000, 16, 0.088f, P, 1 << 30, F, F,
                                nullptr),
         MTD_ERR_INVALID_ARG, "decode_append: v_new misaligned");
  expect(mtd_attn_decode_append(&kv, P, P, P, I, I, 16, 2, 1000, 16, 0.088f, nullptr, 0, F, F, nullptr),
         MTD_ERR_WORKSPACE, "decode_append: no workspace");
  expect(mtd_attn_decode_append(&kv, P, P, P, I, I, 15, 2, 1000, 16, 0.088f, P, 1 << 30, F, F, nullptr),
         MTD_ERR_CAPACITY, "decode_append: bt_stride");
  expect(mtd_attn_decode_noalloc(&kv, P, I, I, 2048, INT_MAX, MTD_MAX_CONTEXT, 16, 0.088f, F, F, nullptr),
         MTD_ERR_WORKSPACE, "decode_noalloc: beyond the scratch");
  expect(mtd_attn_decode_noalloc(&kv, P, I, I, 2048, 2, 0, 16, 0.088f, F, F, nullptr), MTD_ERR_INVALID_ARG,
         "decode_noalloc: max_kv_len");

  // projections, merge, measurement aid
  expect(mtd_qkv_proj(P, P, -1, 1024, 16, 8, 128, P, P, P, nullptr), MTD_ERR_INVALID_ARG, "qkv: n_tok");
  expect(mtd_qkv_proj(P, P, 4, 512, 16, 8, 128, P, P, P, nullptr), MTD_ERR_UNSUPPORTED, "qkv: hidden");
  expect(mtd_qkv_proj(P, P, 0, 1024, 16, 8, 128, P, P, P, nullptr), MTD_OK, "qkv: no tokens");
  expect(mtd_o_proj(F, P, 4, 16, 128, 1024, odd, nullptr), MTD_ERR_INVALID_ARG, "o_proj: out unaligned");
  expect(mtd_attn_merge(F, F, 0, 10, 128, F, F, nullptr), MTD_ERR_INVALID_ARG, "merge: no parts");
  expect(mtd_attn_merge(F, F, 3, 0, 128, F, F, nullptr), MTD_OK, "merge: no rows");
  expect(mtd_measure_page_read(&kv, I, 100, 8, reinterpret_cast<uint32_t*>(P), 1, nullptr), MTD_ERR_WORKSPACE,
         "page_read: sink small");

  // size queries at the extremes (no overflow, 0 for rejected arguments)
  if (mtd_attn_prefill_workspace_bytes(MTD_MAX_CONTEXT, 16, 128) != (size_t)MTD_MAX_CONTEXT * 16 * 129 * 4 ||
      mtd_attn_prefill_workspace_bytes(INT_MAX, 16, 128) != 0 || mtd_attn_prefill_workspace_bytes(-5, 16, 128) != 0) {
    fprintf(stderr, "FAIL prefill workspace sizes\n");
    ++g_failures;
  }
  if (mtd_attn_decode_workspace_bytes(INT_MAX, 16, MTD_MAX_CONTEXT, 128) !=
          (size_t)INT_MAX * 256 * 16 * 129 * 4 ||
      mtd_attn_decode_workspace_bytes(4, 16, INT_MIN, 128) != 0) {
    fprintf(stderr, "FAIL decode workspace sizes\n");
    ++g_failures;
  }
  if (mtd_measure_page_read_sink_words(INT_MAX, 1) != (size_t)INT_MAX * 8 * 64 ||
      mtd_measure_page_read_sink_words(INT_MAX, 64) == 0) {
    fprintf(stderr, "FAIL page read sink sizes\n");
    ++g_failures;
  }
  for (int s = -7; s <= 1; ++s)
    if (mtd_status_string(s) == nullptr || mtd_status_string(s)[0] == '\0') ++g_failures;
  if (mtd_abi_version() != MTD_ABI_VERSION) ++g_failures;

  if (g_failures) {
    fprintf(stderr, "%d failures\n", g_failures);
    return 1;
  }
  printf("host abi checks: all passed\n");
  return 0;
}
