// KV append: copy the K/V rows of new tokens into their cache pages.
//
// Prefill stores the prompt's keys and values in the KV cache and every decode step adds one token
// per request ("Optimizing ASR Models to Transcribe 90-Minute Multi-Speaker Audio", section ASR
// Model Primer).  The copy is a pure bit move: no rounding, no arithmetic on the values.
//
// One workgroup per new token, 128 threads: thread t moves 16 bytes of K and 16 bytes of V
// (KV head t / 16, dims 8*(t % 16) .. +7).  Source rows are contiguous 2 KiB per token; each
// destination row is 256 contiguous bytes inside its (page, head) block.
#include "mtd_internal.h"

namespace mtd {
namespace {

__global__ __launch_bounds__(128) void kv_append_kernel(
    uint16_t* __restrict__ k_pages, uint16_t* __restrict__ v_pages, int num_pages,
    const uint16_t* __restrict__ k_new, const uint16_t* __restrict__ v_new,
    const int32_t* __restrict__ cu_new, const int32_t* __restrict__ start_pos,
    const int32_t* __restrict__ block_tables, int bt_stride, int n_req) {
  const int t = blockIdx.x;
  // Owner of token t: the request r with cu_new[r] <= t < cu_new[r+1] (binary search; empty
  // requests, where cu_new[r] == cu_new[r+1], are skipped).  A token no request owns (at or past
  // cu_new[n_req], as in a batch padded to a fixed size) is not written.
  int lo = 0, hi = n_req;
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (cu_new[mid] <= t) lo = mid; else hi = mid;
  }
  if (t < cu_new[lo] || t >= cu_new[lo + 1]) return;
  const int pos = start_pos[lo] + (t - cu_new[lo]);
  if (pos < 0 || pos >= kMaxContext) return;
  const int entry = pos / kPage;
  if (entry >= bt_stride) return;
  const int page = block_tables[(size_t)lo * bt_stride + entry];
  if (page < 0 || page >= num_pages) return;
  const int slot = pos % kPage;
  const int head = threadIdx.x >> 4;
  const int chunk = threadIdx.x & 15;
  const size_t src = ((size_t)t * kKvHeads + head) * kHeadDim + chunk * 8;
  const size_t dst = (((size_t)page * kKvHeads + head) * kPage + slot) * kHeadDim + chunk * 8;
  const uint4 kv = *reinterpret_cast<const uint4*>(k_new + src);
  const uint4 vv = *reinterpret_cast<const uint4*>(v_new + src);
  *reinterpret_cast<uint4*>(k_pages + dst) = kv;
  *reinterpret_cast<uint4*>(v_pages + dst) = vv;
}

}  // namespace

hipError_t launch_kv_append(const KvPools& kv, const uint16_t* k_new, const uint16_t* v_new,
                            const int32_t* cu_new, const int32_t* start_pos,
                            const int32_t* block_tables, int bt_stride, int n_req, int n_new,
                            hipStream_t stream) {
  if (n_new == 0) return hipSuccess;
  kv_append_kernel<<<dim3(n_new), dim3(128), 0, stream>>>(kv.k, kv.v, kv.num_pages, k_new, v_new,
                                                          cu_new, start_pos, block_tables,
                                                          bt_stride, n_req);
  return hipGetLastError();
}

}  // namespace mtd
