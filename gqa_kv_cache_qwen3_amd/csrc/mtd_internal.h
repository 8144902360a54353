// Internal declarations shared by the HIP kernels and the C-ABI host layer of libmtd.
// Not installed; the public interface is include/mtd.h.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mtd {

// Shape this version builds for: the Qwen3 decoder's GQA 16/8 with head_dim 128, 64-token pages.
constexpr int kQHeads = 16;
constexpr int kKvHeads = 8;
constexpr int kGroup = kQHeads / kKvHeads;  // query heads per KV head
constexpr int kHeadDim = 128;
constexpr int kPage = 64;
constexpr int kMaxContext = 131072;
constexpr int kHidden = 1024;  // decoder hidden size (input of the QKV map, output of o_proj)
// Decode split-K partition of a request of len tokens: consecutive runs of split_tokens(len)
// logical tokens (whole pages).  The run doubles from 64 tokens with each doubling of the length
// past 1024 and stops at 512: 64 up to 1024 tokens, 128 up to 2048, 256 up to 4096, 512 beyond.
// So every request of up to 8192 tokens has between 9 and 16 splits (one page each up to 1024
// tokens), and even a lone request spreads over many wavefronts, while long requests keep
// 512-token splits, where the per-split costs (query load, partial write, merge) stay under 1 % of
// the K/V bytes and a large batch streams at full rate.  The partition depends only on the
// request's own length, in logical token space, so a request's result never depends on the batch
// or on page placement.
__host__ __device__ constexpr int split_shift(int len) {
  return 6 + (len > 1024) + (len > 2048) + (len > 4096);
}
__host__ __device__ constexpr int split_tokens(int len) { return 1 << split_shift(len); }
__host__ __device__ constexpr int split_parts(int len) {
  return len <= 0 ? 0 : (len + split_tokens(len) - 1) >> split_shift(len);
}
// Most partials one request can have (131072 tokens in 512-token splits).
constexpr int kMaxParts = split_parts(kMaxContext);
// Most partials any request of at most max_len tokens can have: split_parts rises within each
// length band and drops where the split grows, so the maximum sits at a band's upper end, and
// each band below 4096 tokens ends at 16 splits.
__host__ __device__ constexpr int split_parts_bound(int max_len) {
  const int a = split_parts(max_len < 1024 ? max_len : 1024);
  const int b = split_parts(max_len);
  return a > b ? a : b;
}

struct KvPools {
  uint16_t* k;
  uint16_t* v;
  int num_pages;
};

// Sizes are host arithmetic, inline here; launchers are defined next to their kernels.  Arguments
// are validated by the caller.
hipError_t launch_kv_append(const KvPools& kv, const uint16_t* k_new, const uint16_t* v_new,
                            const int32_t* cu_new, const int32_t* start_pos,
                            const int32_t* block_tables, int bt_stride, int n_req, int n_new,
                            hipStream_t stream);

// Optional prefill workspace: partial O float32 [chunk_len][kQHeads][kHeadDim], then partial LSE
// float32 [chunk_len][kQHeads] (one part of every split item, merged after the kernel).
// workspace == nullptr: one pass per item, no split.
inline size_t prefill_workspace_bytes(int chunk_len) {
  return (size_t)chunk_len * kQHeads * (kHeadDim + 1) * sizeof(float);
}

// cu_budget: 0 = the whole device; else (with a workspace) the call's work is spread over
// cu_budget / 8 workgroups per KV head, leaving the other CUs free.
// Compute units of the calling thread's current device (queried once per device).
int device_cus();

hipError_t launch_prefill(const KvPools& kv, const uint16_t* q, int chunk_len, int prefix_len,
                          const int32_t* block_table, float scale, void* workspace, int cu_budget,
                          float* out, float* lse, hipStream_t stream);

// Workspace layout of the decode: partial O float32 [max_parts][kQHeads][kHeadDim], then partial
// LSE float32 [max_parts][kQHeads], max_parts = batch * split_parts_bound(max_kv_len); split s of
// request b uses part b * split_parts_bound(max_kv_len) + s.
inline size_t decode_workspace_bytes(int batch, int max_kv_len) {
  const size_t parts = (size_t)batch * (size_t)split_parts_bound(max_kv_len);
  return parts * kQHeads * (kHeadDim + 1) * sizeof(float);
}

// Allocation-free decode: the partials go to a static device array of kDecodeScratchBytes per
// GPU (64 MiB: batch * split_parts_bound(max_kv_len) up to 8128 partials, e.g. 64 requests of
// 64,512 tokens or 31 of 131,072).  decode_scratch gives the calling thread's current device's
// copy (looked up with hipGetSymbolAddress on first use on that device).
constexpr size_t kDecodeScratchBytes = size_t(64) << 20;
constexpr int kMaxDevices = 64;
hipError_t decode_scratch(void** ptr);

// k_new / v_new: NULL, or bf16 [batch][kKvHeads][kHeadDim] rows that the split kernel stores at
// position kv_lens[b] - 1 of each request (and attends to) in the same launch.
hipError_t launch_decode(const KvPools& kv, const uint16_t* q, const uint16_t* k_new, const uint16_t* v_new,
                         const int32_t* kv_lens, const int32_t* block_tables, int bt_stride, int batch,
                         int max_kv_len, float scale, void* workspace, float* out, float* lse,
                         hipStream_t stream);

// The projections around the attention (n_tok >= 1; pointers 16-byte aligned):
//   x bf16 [n_tok][kHidden], w_qkv bf16 [(kQHeads + 2 kKvHeads) kHeadDim][kHidden]
//     -> q bf16 [n_tok][kQHeads][kHeadDim], k, v bf16 [n_tok][kKvHeads][kHeadDim];
//   attn float32 [n_tok][kQHeads][kHeadDim], w_o bf16 [kHidden][kQHeads kHeadDim]
//     -> out bf16 [n_tok][kHidden].
hipError_t launch_qkv_proj(const uint16_t* x, const uint16_t* w_qkv, int n_tok, uint16_t* q,
                           uint16_t* k, uint16_t* v, hipStream_t stream);
hipError_t launch_o_proj(const float* attn, const uint16_t* w_o, int n_tok, uint16_t* out,
                         hipStream_t stream);

// LSE combination of attention results over disjoint key sets: o_parts float32
// [n_parts][n_rows][kHeadDim], lse_parts float32 [n_parts][n_rows] -> out [n_rows][kHeadDim],
// lse [n_rows] (n_parts >= 1, n_rows >= 1).
hipError_t launch_attn_merge(const float* o_parts, const float* lse_parts, int n_parts, int n_rows,
                             float* out, float* lse, hipStream_t stream);

// Measurement aid: read the K and V blocks (KV head g = every head) of pages_per_wave consecutive
// entries of page_ids per wavefront, with the decode's access pattern; one word per lane of every
// wave goes to sink (page_read_sink_words(n_ids, pages_per_wave) words).
inline size_t page_read_sink_words(int n_ids, int pages_per_wave) {
  return ((size_t)n_ids + pages_per_wave - 1) / pages_per_wave * kKvHeads * 64;
}
hipError_t launch_page_read(const KvPools& kv, const int32_t* page_ids, int n_ids, int pages_per_wave,
                            uint32_t* sink, hipStream_t stream);

}  // namespace mtd
