// C-ABI layer of libmtd: argument validation on the host, then kernel launches on the caller's
// stream.  Every check below runs before any HIP call, so each error path can be exercised on a
// machine without a GPU.
#include <math.h>
#include <stdarg.h>
#include <stdio.h>

#include <hip/hip_runtime.h>

#include "../../include/mtd.h"
#include "mtd_internal.h"

namespace {

static_assert(MTD_DECODE_NOALLOC_SCRATCH_BYTES == mtd::kDecodeScratchBytes, "scratch size in the header");

thread_local char g_last_error[512] = "";

int fail(int status, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_last_error, sizeof g_last_error, fmt, ap);
  va_end(ap);
  return status;
}

int ok() {
  g_last_error[0] = '\0';
  return MTD_OK;
}

int hip_status(hipError_t err, const char* what) {
  if (err == hipSuccess) return ok();
  return fail(MTD_ERR_HIP, "%s: %s", what, hipGetErrorString(err));
}

// The kernels move 16-byte vectors through every pool, token, output and workspace array.
bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Checks shared by all calls on the layer description.
int check_layer(const mtd_kv_layer_t* kv) {
  if (kv == nullptr) return fail(MTD_ERR_INVALID_ARG, "kv is NULL");
  if (kv->k_pages == nullptr || kv->v_pages == nullptr)
    return fail(MTD_ERR_INVALID_ARG, "kv->k_pages / kv->v_pages is NULL");
  if (!aligned16(kv->k_pages) || !aligned16(kv->v_pages))
    return fail(MTD_ERR_INVALID_ARG, "kv->k_pages / kv->v_pages not 16-byte aligned");
  if (kv->num_pages <= 0) return fail(MTD_ERR_INVALID_ARG, "kv->num_pages = %d", kv->num_pages);
  if (kv->page_size != mtd::kPage)
    return fail(MTD_ERR_UNSUPPORTED, "page_size %d (supported: %d)", kv->page_size, mtd::kPage);
  if (kv->num_kv_heads != mtd::kKvHeads)
    return fail(MTD_ERR_UNSUPPORTED, "num_kv_heads %d (supported: %d)", kv->num_kv_heads, mtd::kKvHeads);
  if (kv->head_dim != mtd::kHeadDim)
    return fail(MTD_ERR_UNSUPPORTED, "head_dim %d (supported: %d)", kv->head_dim, mtd::kHeadDim);
  return MTD_OK;
}

int check_heads(int32_t num_q_heads, int32_t num_kv_heads) {
  if (num_q_heads <= 0) return fail(MTD_ERR_INVALID_ARG, "num_q_heads = %d", num_q_heads);
  if (num_q_heads % num_kv_heads != 0)
    return fail(MTD_ERR_UNSUPPORTED, "num_q_heads %d is not a multiple of num_kv_heads %d",
                num_q_heads, num_kv_heads);
  if (num_q_heads != mtd::kQHeads)
    return fail(MTD_ERR_UNSUPPORTED, "num_q_heads %d (supported: %d)", num_q_heads, mtd::kQHeads);
  return MTD_OK;
}

int check_scale(float scale) {
  if (!(scale > 0.f) || !isfinite(scale)) return fail(MTD_ERR_INVALID_ARG, "scale must be finite and > 0");
  return MTD_OK;
}

// The projections' shape arguments.
int check_proj_shape(int32_t n_tok, int32_t hidden, int32_t num_q_heads, int32_t num_kv_heads,
                     int32_t head_dim) {
  if (n_tok < 0) return fail(MTD_ERR_INVALID_ARG, "n_tok = %d", n_tok);
  if (hidden <= 0 || num_q_heads <= 0 || num_kv_heads <= 0 || head_dim <= 0)
    return fail(MTD_ERR_INVALID_ARG, "hidden %d, num_q_heads %d, num_kv_heads %d, head_dim %d",
                hidden, num_q_heads, num_kv_heads, head_dim);
  if (hidden != mtd::kHidden || num_q_heads != mtd::kQHeads || num_kv_heads != mtd::kKvHeads ||
      head_dim != mtd::kHeadDim)
    return fail(MTD_ERR_UNSUPPORTED,
                "hidden %d, heads %d/%d, head_dim %d (supported: %d, %d/%d, %d)", hidden,
                num_q_heads, num_kv_heads, head_dim, mtd::kHidden, mtd::kQHeads, mtd::kKvHeads,
                mtd::kHeadDim);
  return MTD_OK;
}

mtd::KvPools pools(const mtd_kv_layer_t* kv) {
  return mtd::KvPools{static_cast<uint16_t*>(kv->k_pages), static_cast<uint16_t*>(kv->v_pages),
                      kv->num_pages};
}

// mtd_attn_decode (k_new = v_new = NULL) and mtd_attn_decode_append (both set).
int decode_call(const mtd_kv_layer_t* kv, const void* q, const void* k_new, const void* v_new,
                const int32_t* kv_lens, const int32_t* block_tables, int32_t bt_stride, int32_t batch,
                int32_t max_kv_len, int32_t num_q_heads, float scale, void* workspace, size_t workspace_bytes,
                float* out, float* lse, void* stream) {
  int st = check_layer(kv);
  if (st != MTD_OK) return st;
  if ((st = check_heads(num_q_heads, kv->num_kv_heads)) != MTD_OK) return st;
  if ((st = check_scale(scale)) != MTD_OK) return st;
  if (q == nullptr || kv_lens == nullptr || block_tables == nullptr || out == nullptr || lse == nullptr)
    return fail(MTD_ERR_INVALID_ARG, "q / kv_lens / block_tables / out / lse is NULL");
  if (!aligned16(q) || !aligned16(out) || !aligned16(workspace))
    return fail(MTD_ERR_INVALID_ARG, "q / out / workspace not 16-byte aligned");
  if (!aligned16(k_new) || !aligned16(v_new))
    return fail(MTD_ERR_INVALID_ARG, "k_new / v_new not 16-byte aligned");
  if (batch <= 0) return fail(MTD_ERR_INVALID_ARG, "batch = %d", batch);
  if (max_kv_len <= 0) return fail(MTD_ERR_INVALID_ARG, "max_kv_len = %d", max_kv_len);
  if (max_kv_len > MTD_MAX_CONTEXT)
    return fail(MTD_ERR_CAPACITY, "max_kv_len %d exceeds %d", max_kv_len, MTD_MAX_CONTEXT);
  const int64_t pages = ((int64_t)max_kv_len + mtd::kPage - 1) / mtd::kPage;
  if (bt_stride < pages)
    return fail(MTD_ERR_CAPACITY, "bt_stride %d < %lld pages for max_kv_len %d", bt_stride,
                (long long)pages, max_kv_len);
  const size_t need = mtd::decode_workspace_bytes(batch, max_kv_len);
  if (workspace == nullptr || workspace_bytes < need)
    return fail(MTD_ERR_WORKSPACE, "workspace of %zu bytes, %zu needed", workspace_bytes, need);
  return hip_status(mtd::launch_decode(pools(kv), static_cast<const uint16_t*>(q),
                                       static_cast<const uint16_t*>(k_new), static_cast<const uint16_t*>(v_new),
                                       kv_lens, block_tables, bt_stride, batch, max_kv_len, scale,
                                       workspace, out, lse, static_cast<hipStream_t>(stream)),
                    "decode launch");
}

}  // namespace

extern "C" {

int mtd_kv_append(const mtd_kv_layer_t* kv, const void* k_new, const void* v_new,
                  const int32_t* cu_new, const int32_t* start_pos, const int32_t* block_tables,
                  int32_t bt_stride, int32_t n_req, int32_t n_new, void* stream) {
  int st = check_layer(kv);
  if (st != MTD_OK) return st;
  if (n_req <= 0) return fail(MTD_ERR_INVALID_ARG, "n_req = %d", n_req);
  if (n_new < 0) return fail(MTD_ERR_INVALID_ARG, "n_new = %d", n_new);
  if (bt_stride <= 0) return fail(MTD_ERR_INVALID_ARG, "bt_stride = %d", bt_stride);
  if (n_new > 0 && (k_new == nullptr || v_new == nullptr))
    return fail(MTD_ERR_INVALID_ARG, "k_new / v_new is NULL");
  if (!aligned16(k_new) || !aligned16(v_new))
    return fail(MTD_ERR_INVALID_ARG, "k_new / v_new not 16-byte aligned");
  if (cu_new == nullptr || start_pos == nullptr || block_tables == nullptr)
    return fail(MTD_ERR_INVALID_ARG, "cu_new / start_pos / block_tables is NULL");
  if (n_new == 0) return ok();
  return hip_status(mtd::launch_kv_append(pools(kv), static_cast<const uint16_t*>(k_new),
                                          static_cast<const uint16_t*>(v_new), cu_new, start_pos,
                                          block_tables, bt_stride, n_req, n_new,
                                          static_cast<hipStream_t>(stream)),
                    "kv_append launch");
}

int mtd_attn_prefill_chunk_cus(const mtd_kv_layer_t* kv, const void* q, int32_t chunk_len,
                               int32_t prefix_len, const int32_t* block_table, int32_t block_table_len,
                               int32_t num_q_heads, float scale, void* workspace, size_t workspace_bytes,
                               int32_t cu_budget, float* out, float* lse, void* stream) {
  int st = check_layer(kv);
  if (st != MTD_OK) return st;
  if ((st = check_heads(num_q_heads, kv->num_kv_heads)) != MTD_OK) return st;
  if ((st = check_scale(scale)) != MTD_OK) return st;
  if (q == nullptr || block_table == nullptr || out == nullptr || lse == nullptr)
    return fail(MTD_ERR_INVALID_ARG, "q / block_table / out / lse is NULL");
  if (!aligned16(q) || !aligned16(out) || !aligned16(workspace))
    return fail(MTD_ERR_INVALID_ARG, "q / out / workspace not 16-byte aligned");
  if (chunk_len <= 0) return fail(MTD_ERR_INVALID_ARG, "chunk_len = %d", chunk_len);
  if (prefix_len < 0) return fail(MTD_ERR_INVALID_ARG, "prefix_len = %d", prefix_len);
  if (cu_budget < 0) return fail(MTD_ERR_INVALID_ARG, "cu_budget = %d", cu_budget);
  const int64_t total = (int64_t)prefix_len + chunk_len;
  if (total > MTD_MAX_CONTEXT)
    return fail(MTD_ERR_CAPACITY, "prefix_len + chunk_len = %lld exceeds %d", (long long)total,
                MTD_MAX_CONTEXT);
  const int64_t pages = (total + mtd::kPage - 1) / mtd::kPage;
  if (block_table_len < pages)
    return fail(MTD_ERR_CAPACITY, "block_table_len %d < %lld pages needed", block_table_len,
                (long long)pages);
  if (workspace != nullptr && workspace_bytes < mtd::prefill_workspace_bytes(chunk_len))
    return fail(MTD_ERR_WORKSPACE, "workspace of %zu bytes, %zu needed", workspace_bytes,
                mtd::prefill_workspace_bytes(chunk_len));
  if (cu_budget > 0 && workspace == nullptr)
    return fail(MTD_ERR_WORKSPACE, "a CU budget (%d) needs the workspace", cu_budget);
  return hip_status(mtd::launch_prefill(pools(kv), static_cast<const uint16_t*>(q), chunk_len,
                                        prefix_len, block_table, scale, workspace, cu_budget, out, lse,
                                        static_cast<hipStream_t>(stream)),
                    "prefill launch");
}

int mtd_attn_prefill_chunk(const mtd_kv_layer_t* kv, const void* q, int32_t chunk_len,
                           int32_t prefix_len, const int32_t* block_table, int32_t block_table_len,
                           int32_t num_q_heads, float scale, void* workspace, size_t workspace_bytes,
                           float* out, float* lse, void* stream) {
  return mtd_attn_prefill_chunk_cus(kv, q, chunk_len, prefix_len, block_table, block_table_len,
                                    num_q_heads, scale, workspace, workspace_bytes, 0, out, lse, stream);
}

size_t mtd_attn_prefill_workspace_bytes(int32_t chunk_len, int32_t num_q_heads, int32_t head_dim) {
  if (chunk_len <= 0 || chunk_len > MTD_MAX_CONTEXT || num_q_heads != mtd::kQHeads ||
      head_dim != mtd::kHeadDim)
    return 0;
  return mtd::prefill_workspace_bytes(chunk_len);
}

size_t mtd_attn_decode_workspace_bytes(int32_t batch, int32_t num_q_heads, int32_t max_kv_len,
                                       int32_t head_dim) {
  if (batch <= 0 || num_q_heads != mtd::kQHeads || head_dim != mtd::kHeadDim) return 0;
  if (max_kv_len <= 0 || max_kv_len > MTD_MAX_CONTEXT) return 0;
  return mtd::decode_workspace_bytes(batch, max_kv_len);
}

int mtd_attn_decode(const mtd_kv_layer_t* kv, const void* q, const int32_t* kv_lens,
                    const int32_t* block_tables, int32_t bt_stride, int32_t batch,
                    int32_t max_kv_len, int32_t num_q_heads, float scale, void* workspace,
                    size_t workspace_bytes, float* out, float* lse, void* stream) {
  return decode_call(kv, q, nullptr, nullptr, kv_lens, block_tables, bt_stride, batch, max_kv_len, num_q_heads,
                     scale, workspace, workspace_bytes, out, lse, stream);
}

int mtd_attn_decode_append(const mtd_kv_layer_t* kv, const void* q, const void* k_new, const void* v_new,
                           const int32_t* kv_lens, const int32_t* block_tables, int32_t bt_stride,
                           int32_t batch, int32_t max_kv_len, int32_t num_q_heads, float scale,
                           void* workspace, size_t workspace_bytes, float* out, float* lse, void* stream) {
  if (k_new == nullptr || v_new == nullptr) return fail(MTD_ERR_INVALID_ARG, "k_new / v_new is NULL");
  return decode_call(kv, q, k_new, v_new, kv_lens, block_tables, bt_stride, batch, max_kv_len, num_q_heads,
                     scale, workspace, workspace_bytes, out, lse, stream);
}

int mtd_attn_decode_noalloc(const mtd_kv_layer_t* kv, const void* q, const int32_t* kv_lens,
                            const int32_t* block_tables, int32_t bt_stride, int32_t batch,
                            int32_t max_kv_len, int32_t num_q_heads, float scale, float* out,
                            float* lse, void* stream) {
  int st = check_layer(kv);
  if (st != MTD_OK) return st;
  if ((st = check_heads(num_q_heads, kv->num_kv_heads)) != MTD_OK) return st;
  if ((st = check_scale(scale)) != MTD_OK) return st;
  if (q == nullptr || kv_lens == nullptr || block_tables == nullptr || out == nullptr || lse == nullptr)
    return fail(MTD_ERR_INVALID_ARG, "q / kv_lens / block_tables / out / lse is NULL");
  if (!aligned16(q) || !aligned16(out)) return fail(MTD_ERR_INVALID_ARG, "q / out not 16-byte aligned");
  if (batch <= 0) return fail(MTD_ERR_INVALID_ARG, "batch = %d", batch);
  if (max_kv_len <= 0) return fail(MTD_ERR_INVALID_ARG, "max_kv_len = %d", max_kv_len);
  if (max_kv_len > MTD_MAX_CONTEXT)
    return fail(MTD_ERR_CAPACITY, "max_kv_len %d exceeds %d", max_kv_len, MTD_MAX_CONTEXT);
  const int64_t pages = ((int64_t)max_kv_len + mtd::kPage - 1) / mtd::kPage;
  if (bt_stride < pages)
    return fail(MTD_ERR_CAPACITY, "bt_stride %d < %lld pages for max_kv_len %d", bt_stride,
                (long long)pages, max_kv_len);
  const size_t need = mtd::decode_workspace_bytes(batch, max_kv_len);
  if (need > mtd::kDecodeScratchBytes)
    return fail(MTD_ERR_WORKSPACE,
                "batch %d with max_kv_len %d needs %zu bytes of scratch; the static scratch holds %zu "
                "(MTD_DECODE_NOALLOC_SCRATCH_BYTES)",
                batch, max_kv_len, need, mtd::kDecodeScratchBytes);
  void* scratch = nullptr;
  if ((st = hip_status(mtd::decode_scratch(&scratch), "decode scratch lookup")) != MTD_OK) return st;
  return hip_status(mtd::launch_decode(pools(kv), static_cast<const uint16_t*>(q), nullptr, nullptr, kv_lens,
                                       block_tables, bt_stride, batch, max_kv_len, scale, scratch,
                                       out, lse, static_cast<hipStream_t>(stream)),
                    "decode launch");
}

int mtd_qkv_proj(const void* x, const void* w_qkv, int32_t n_tok, int32_t hidden,
                 int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim, void* q, void* k_new,
                 void* v_new, void* stream) {
  int st = check_proj_shape(n_tok, hidden, num_q_heads, num_kv_heads, head_dim);
  if (st != MTD_OK) return st;
  if (x == nullptr || w_qkv == nullptr || q == nullptr || k_new == nullptr || v_new == nullptr)
    return fail(MTD_ERR_INVALID_ARG, "x / w_qkv / q / k_new / v_new is NULL");
  if (!aligned16(x) || !aligned16(w_qkv) || !aligned16(q) || !aligned16(k_new) || !aligned16(v_new))
    return fail(MTD_ERR_INVALID_ARG, "x / w_qkv / q / k_new / v_new not 16-byte aligned");
  if (n_tok == 0) return ok();
  return hip_status(mtd::launch_qkv_proj(static_cast<const uint16_t*>(x),
                                         static_cast<const uint16_t*>(w_qkv), n_tok,
                                         static_cast<uint16_t*>(q), static_cast<uint16_t*>(k_new),
                                         static_cast<uint16_t*>(v_new),
                                         static_cast<hipStream_t>(stream)),
                    "qkv projection launch");
}

int mtd_o_proj(const float* attn, const void* w_o, int32_t n_tok, int32_t num_q_heads,
               int32_t head_dim, int32_t hidden, void* out, void* stream) {
  int st = check_proj_shape(n_tok, hidden, num_q_heads, mtd::kKvHeads, head_dim);
  if (st != MTD_OK) return st;
  if (attn == nullptr || w_o == nullptr || out == nullptr)
    return fail(MTD_ERR_INVALID_ARG, "attn / w_o / out is NULL");
  if (!aligned16(attn) || !aligned16(w_o) || !aligned16(out))
    return fail(MTD_ERR_INVALID_ARG, "attn / w_o / out not 16-byte aligned");
  if (n_tok == 0) return ok();
  return hip_status(mtd::launch_o_proj(attn, static_cast<const uint16_t*>(w_o), n_tok,
                                       static_cast<uint16_t*>(out), static_cast<hipStream_t>(stream)),
                    "output projection launch");
}

int mtd_attn_merge(const float* o_parts, const float* lse_parts, int32_t n_parts, int32_t n_rows,
                   int32_t head_dim, float* out, float* lse, void* stream) {
  if (n_parts <= 0 || n_parts > MTD_MAX_MERGE_PARTS)
    return fail(MTD_ERR_INVALID_ARG, "n_parts = %d (1 .. %d)", n_parts, MTD_MAX_MERGE_PARTS);
  if (n_rows < 0) return fail(MTD_ERR_INVALID_ARG, "n_rows = %d", n_rows);
  if (head_dim != mtd::kHeadDim)
    return fail(MTD_ERR_UNSUPPORTED, "head_dim %d (supported: %d)", head_dim, mtd::kHeadDim);
  if (o_parts == nullptr || lse_parts == nullptr || out == nullptr || lse == nullptr)
    return fail(MTD_ERR_INVALID_ARG, "o_parts / lse_parts / out / lse is NULL");
  if (!aligned16(o_parts) || !aligned16(out))
    return fail(MTD_ERR_INVALID_ARG, "o_parts / out not 16-byte aligned");
  if (n_rows == 0) return ok();
  return hip_status(mtd::launch_attn_merge(o_parts, lse_parts, n_parts, n_rows, out, lse,
                                           static_cast<hipStream_t>(stream)),
                    "merge launch");
}

size_t mtd_measure_page_read_sink_words(int32_t n_ids, int32_t pages_per_wave) {
  if (n_ids < 1 || pages_per_wave < 1 || pages_per_wave > 64) return 0;
  return mtd::page_read_sink_words(n_ids, pages_per_wave);
}

int mtd_measure_page_read(const mtd_kv_layer_t* kv, const int32_t* page_ids, int32_t n_ids,
                          int32_t pages_per_wave, uint32_t* sink, size_t sink_words, void* stream) {
  if (int st = check_layer(kv)) return st;
  if (n_ids < 1) return fail(MTD_ERR_INVALID_ARG, "n_ids = %d", n_ids);
  if (pages_per_wave < 1 || pages_per_wave > 64)
    return fail(MTD_ERR_INVALID_ARG, "pages_per_wave = %d (1 .. 64)", pages_per_wave);
  if (page_ids == nullptr || sink == nullptr) return fail(MTD_ERR_INVALID_ARG, "page_ids / sink is NULL");
  const size_t need = mtd::page_read_sink_words(n_ids, pages_per_wave);
  if (sink_words < need)
    return fail(MTD_ERR_WORKSPACE, "sink holds %zu words, %zu needed", sink_words, need);
  return hip_status(mtd::launch_page_read(pools(kv), page_ids, n_ids, pages_per_wave, sink,
                                          static_cast<hipStream_t>(stream)),
                    "page read launch");
}

const char* mtd_status_string(int status) {
  switch (status) {
    case MTD_OK: return "ok";
    case MTD_ERR_INVALID_ARG: return "invalid argument";
    case MTD_ERR_UNSUPPORTED: return "unsupported shape";
    case MTD_ERR_CAPACITY: return "capacity exceeded";
    case MTD_ERR_WORKSPACE: return "workspace too small";
    case MTD_ERR_HIP: return "HIP runtime error";
    default: return "unknown status";
  }
}

const char* mtd_last_error(void) { return g_last_error; }

int mtd_abi_version(void) { return MTD_ABI_VERSION; }

}  // extern "C"
