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
// Decode split-K partition: 512 logical tokens (8 pages).  Partition boundaries are fixed in
// logical token space, so a request's result never depends on the batch or on page placement.
constexpr int kSplit = 512;

struct KvPools {
  uint16_t* k;
  uint16_t* v;
  int num_pages;
};

// Launchers (defined next to their kernels).  Arguments are validated by the caller.
hipError_t launch_kv_append(const KvPools& kv, const uint16_t* k_new, const uint16_t* v_new,
                            const int32_t* cu_new, const int32_t* start_pos,
                            const int32_t* block_tables, int bt_stride, int n_req, int n_new,
                            hipStream_t stream);

hipError_t launch_prefill(const KvPools& kv, const uint16_t* q, int chunk_len, int prefix_len,
                          const int32_t* block_table, float scale, float* out, float* lse,
                          hipStream_t stream);

// Workspace layout of the decode: partial O float32 [max_parts][kQHeads][kHeadDim], then partial
// LSE float32 [max_parts][kQHeads], max_parts = batch * ceil(max_kv_len / kSplit).
size_t decode_workspace_bytes(int batch, int max_kv_len);

hipError_t launch_decode(const KvPools& kv, const uint16_t* q, const int32_t* kv_lens,
                         const int32_t* block_tables, int bt_stride, int batch, int max_kv_len,
                         float scale, void* workspace, float* out, float* lse, hipStream_t stream);

}  // namespace mtd
