// Practical HBM ceiling of the decode's access pattern (a measurement aid, not part of attention).
//
// Decode is HBM-bound: it reads every K/V byte of a batch once, as whole 16 KiB (page, KV head)
// blocks in random page order, one wavefront per (request, split, KV head).  The peak to compare it
// with is what that pattern can reach on the chip, not the 8 TB/s headline.  This kernel reads the
// same blocks the same way (the decode's lane layout, 16-byte non-temporal loads, K then V of one
// page in flight per wave) and does nothing with the data but fold it into one word per wave, so
// its rate is the pattern's ceiling.  One wave reads the K and V blocks of pages_per_wave
// consecutive entries of a page list for one KV head.
#include "device_util.h"
#include "mtd_internal.h"

namespace mtd {
namespace {

typedef unsigned u32x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ u32x4_t stream_load16(const uint16_t* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
}

__global__ __launch_bounds__(64) void page_read_kernel(const uint16_t* __restrict__ k_pages,
                                                       const uint16_t* __restrict__ v_pages, int num_pages,
                                                       const int32_t* __restrict__ page_ids, int n_ids,
                                                       int pages_per_wave, uint32_t* __restrict__ sink) {
  const int lane = threadIdx.x;
  const int w = blockIdx.x / kKvHeads;
  const int g = blockIdx.x % kKvHeads;
  const int sg = lane >> 3, o = lane & 7;  // the decode's layout: slots 8a + sg, chunks o and 8 + o
  u32x4_t acc = {0u, 0u, 0u, 0u};
  const int e0 = (int)min((int64_t)w * pages_per_wave, (int64_t)n_ids);
  const int e1 = (int)min((int64_t)(w + 1) * pages_per_wave, (int64_t)n_ids);
  for (int e = e0; e < e1; ++e) {
    const int page = page_ids[e];
    if (page < 0 || page >= num_pages) continue;
    const size_t blk = ((size_t)page * kKvHeads + g) * (kPage * kHeadDim);
    u32x4_t kr[8][2], vr[8][2];
#pragma unroll
    for (int a = 0; a < 8; ++a)
#pragma unroll
      for (int c = 0; c < 2; ++c) kr[a][c] = stream_load16(k_pages + blk + (8 * a + sg) * kHeadDim + (8 * c + o) * 8);
#pragma unroll
    for (int a = 0; a < 8; ++a)
#pragma unroll
      for (int c = 0; c < 2; ++c) vr[a][c] = stream_load16(v_pages + blk + (8 * a + sg) * kHeadDim + (8 * c + o) * 8);
#pragma unroll
    for (int a = 0; a < 8; ++a)
#pragma unroll
      for (int c = 0; c < 2; ++c) acc ^= kr[a][c] ^ vr[a][c];
  }
  sink[(size_t)blockIdx.x * 64 + lane] = acc.x ^ acc.y ^ acc.z ^ acc.w;
}

}  // namespace

hipError_t launch_page_read(const KvPools& kv, const int32_t* page_ids, int n_ids, int pages_per_wave,
                            uint32_t* sink, hipStream_t stream) {
  const int waves = (int)(((int64_t)n_ids + pages_per_wave - 1) / pages_per_wave);
  page_read_kernel<<<dim3(waves * kKvHeads), dim3(64), 0, stream>>>(kv.k, kv.v, kv.num_pages, page_ids, n_ids,
                                                                     pages_per_wave, sink);
  return hipGetLastError();
}

}  // namespace mtd
