// Causal attention of one prefill chunk over the paged KV cache, flash-style, on bf16 MFMA.
//
// Long prompts are prefilled in 4096-token chunks; chunk query i (absolute position P + i) attends
// to every key before the chunk and to the chunk's keys up to itself ("Optimizing ASR Models to
// Transcribe 90-Minute Multi-Speaker Audio", section Chunked Prefill for Long Audio).  A short
// prompt is one chunk at P = 0.  No score matrix is ever materialised: the scores of one 64-key
// tile live in registers and are folded into the output with an fp32 online softmax.
//
// Work split.  One workgroup (4 wavefronts) owns 64 chunk positions of one KV head and serves
// both query heads of its GQA group, so every K/V tile staged in LDS feeds 128 query rows.
// Wave w takes positions 16w .. 16w+15 of the tile for both heads: 32 query columns.  Workgroup
// id = 8 * (tile, longest first) + KV head, so the dispatcher's round-robin over the 8 XCDs keeps
// all tiles of one KV head on one XCD and its L2 serves the K/V re-reads.
//
// K/V staging.  A 64-key tile is one page of the KV head: 16 KiB of K and 16 KiB of V, each
// brought into LDS by 16-byte direct-to-LDS loads (global_load_lds_dwordx4, no registers, no
// VALU) into one of two stages, so tile kt+1 streams in while tile kt is computed; one barrier per
// tile.  Both tiles stay row-major [key][dim] in LDS with 16-byte slots XOR-swizzled per row
// (slot of row r, chunk c = 16 r + (c ^ swz(r))), which keeps the K fragment reads and the
// transposed V reads free of bank conflicts.
//
// Per tile:
//   S^T = K Q^T   v_mfma_f32_32x32x16_bf16, keys as rows: a lane holds one query column and 16
//                 of the 32 keys of each 32-key block, so the softmax over keys is mostly in-lane
//                 (one exchange with lane ^ 32).  K fragments: ds_read_b128.
//   online softmax in fp32 (exp2, scale folded into one FMA); P rounded to bf16.
//   O^T += V^T P^T  the P^T operand is exactly the S^T accumulator layout, so P never leaves the
//                 registers.  The V^T operand comes straight from the row-major V tile through
//                 ds_read_b64_tr_b16 (each 16-lane group receives the transpose of the 4 x 16
//                 block its lanes address), two reads per MFMA.
// Causal masking is applied only on tiles that reach past the wave's first position.  Keys past
// the request's last token (tail of the last page) are loaded from the page's first row instead
// of their slots, so V stays finite where their weight is exactly zero.
#include "device_util.h"
#include "mtd_internal.h"

namespace mtd {
namespace {

constexpr int kBQ = 64;   // chunk positions per workgroup
constexpr int kBK = 64;   // keys per tile (one page)
constexpr int kTileBytes = kBK * kHeadDim * 2;  // 16 KiB
constexpr float kNegInf = -__builtin_huge_valf();

typedef short short4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) short4_t lds_short4_t;
typedef __attribute__((address_space(3))) void lds_void_t;
typedef const __attribute__((address_space(1))) void global_cvoid_t;

// XOR swizzle of the 16 slots of a 256-byte row: rows within any 16 consecutive rows get distinct
// values (conflict-free 16-byte K reads), and any 4 consecutive aligned rows differ in the two
// high bits (conflict-free 8-byte transposed V reads).
__device__ __forceinline__ int swz(int r) { return ((r & 3) << 2) | ((r >> 2) & 3); }
__device__ __forceinline__ int slot_of(int r, int c) { return 16 * r + (c ^ swz(r)); }

// Direct-to-LDS load of one K or V tile, 4 instructions per wave: instruction inst fills slots
// 64 inst .. 64 inst + 63, i.e. rows 4 inst .. 4 inst + 3; lane l writes slot 64 inst + l and
// therefore fetches row 4 inst + l/16, chunk (l % 16) ^ swz(row).  Rows >= nvalid fetch row 0.
__device__ __forceinline__ void dma_tile(const uint16_t* __restrict__ blk, uint8_t* lds, int wave,
                                         int lane, int nvalid) {
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int inst = 4 * wave + j;
    const int r = 4 * inst + (lane >> 4);
    const int c = (lane & 15) ^ swz(r);
    const int rs = r < nvalid ? r : 0;
    __builtin_amdgcn_global_load_lds((global_cvoid_t*)(blk + rs * kHeadDim + c * 8),
                                     (lds_void_t*)(lds + inst * 1024), 16, 0, 0);
  }
}

__device__ __forceinline__ void wait_dma() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

struct TileArgs {
  const uint16_t* k_pages;
  const uint16_t* v_pages;
  const int32_t* block_table;
  int num_pages, g, total, wave, lane;
};

__device__ __forceinline__ void issue_tile(const TileArgs& a, int kt, uint8_t* k_lds, uint8_t* v_lds) {
  int page = a.block_table[kt];
  if (page < 0 || page >= a.num_pages) page = 0;  // out-of-pool ids: defined reads, unspecified result
  const size_t blk = ((size_t)page * kKvHeads + a.g) * (kPage * kHeadDim);
  const int nvalid = min(kBK, a.total - kt * kBK);
  dma_tile(a.k_pages + blk, k_lds, a.wave, a.lane, nvalid);
  dma_tile(a.v_pages + blk, v_lds, a.wave, a.lane, nvalid);
}

struct SoftmaxState {
  floatx16_t o_acc[4];  // O^T tiles: dims 32dt .. 32dt+31 x 32 query columns
  float m;              // running max of the column, log2 units (same in both halves)
  float l;              // running sum of exp2(x - m) over this lane's keys
};

// One 64-key tile: S^T, online softmax, O^T update.  Reads only k_lds / v_lds.
__device__ __forceinline__ void compute_tile(SoftmaxState& st_, const bf16x8_t (&qf)[8],
                                             const uint8_t* k_lds, const uint8_t* v_lds, int kt,
                                             int n, int hk, int lane, bool need_mask, int qabs,
                                             float scale_log2) {
  floatx16_t st[2];
#pragma unroll
  for (int mt = 0; mt < 2; ++mt) {
#pragma unroll
    for (int v = 0; v < 16; ++v) st[mt][v] = 0.f;
    const int r = 32 * mt + n;
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
      const bf16x8_t a = __builtin_bit_cast(
          bf16x8_t, *reinterpret_cast<const uint4*>(k_lds + 16 * slot_of(r, 2 * ks + hk)));
      st[mt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[ks], st[mt], 0, 0, 0);
    }
  }

  // Accumulator element v of block mt is key 32mt + 8(v/4) + 4hk + v%4.
  float smax = kNegInf;
#pragma unroll
  for (int mt = 0; mt < 2; ++mt) {
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      float x = st[mt][v];
      if (need_mask) {
        const int key = kt * kBK + 32 * mt + 8 * (v >> 2) + 4 * hk + (v & 3);
        x = key <= qabs ? x : kNegInf;
      }
      st[mt][v] = x;
      smax = fmaxf(smax, x);
    }
  }
  smax = fmaxf(smax, __shfl_xor(smax, 32, 64));
  const float tmax = smax * scale_log2;
  // Exact running max, so the largest weight of a column is exactly 1 before its bf16 rounding
  // (peaked softmaxes stay accurate); the output accumulators are rescaled only on the tiles
  // where some column's max actually grew (about 1/t of the tiles at depth t).
  const float m_new = fmaxf(st_.m, tmax);
  if (__any(m_new > st_.m)) {
    const float alpha = m_new == st_.m ? 1.f : fast_exp2(st_.m - m_new);
    st_.l *= alpha;
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
      for (int v = 0; v < 16; ++v) st_.o_acc[dt][v] *= alpha;
  }
  st_.m = m_new;
  const float m_use = m_new == kNegInf ? 0.f : m_new;
  float psum = 0.f;
  bf16x8_t pf[2][2];
#pragma unroll
  for (int mt = 0; mt < 2; ++mt) {
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      uint32_t w[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float p0 = fast_exp2(fmaf(st[mt][8 * t + 2 * j], scale_log2, -m_use));
        const float p1 = fast_exp2(fmaf(st[mt][8 * t + 2 * j + 1], scale_log2, -m_use));
        psum += p0 + p1;
        w[j] = pack_bf16x2(p0, p1);
      }
      pf[mt][t] = __builtin_bit_cast(bf16x8_t, make_uint4(w[0], w[1], w[2], w[3]));
    }
  }
  st_.l += psum;

  // O^T += V^T P^T.  Block mt, k-step t: this lane's 8 keys are 32mt + 16t + 4hk + {0..3} and the
  // same + 8; lane (l % 16) of 16-lane group G addresses key base + (l%16)/4, dims
  // 32dt + 16(G % 2) + 4(l % 4) .. +3, and receives the 4 keys of dim 32dt + l % 32.
  const int gi = lane & 15;
  const int half = (lane >> 4) & 1;
#pragma unroll
  for (int dt = 0; dt < 4; ++dt) {
    const int dim = 32 * dt + 16 * half + 4 * (gi & 3);
    const int chunk = dim >> 3;
    const int byte_in = (dim & 7) * 2;
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) {
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        const int key0 = 32 * mt + 16 * t + 4 * hk + (gi >> 2);
        const short4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (lds_short4_t*)(v_lds + 16 * slot_of(key0, chunk) + byte_in));
        const short4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (lds_short4_t*)(v_lds + 16 * slot_of(key0 + 8, chunk) + byte_in));
        const bf16x8_t a = __builtin_bit_cast(
            bf16x8_t, make_uint4(__builtin_bit_cast(uint2, lo).x, __builtin_bit_cast(uint2, lo).y,
                                 __builtin_bit_cast(uint2, hi).x, __builtin_bit_cast(uint2, hi).y));
        st_.o_acc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pf[mt][t], st_.o_acc[dt], 0, 0, 0);
      }
    }
  }
}

__global__ __launch_bounds__(256, 2) void prefill_kernel(
    const uint16_t* __restrict__ k_pages, const uint16_t* __restrict__ v_pages, int num_pages,
    const uint16_t* __restrict__ q, int chunk_len, int prefix_len,
    const int32_t* __restrict__ block_table, float scale_log2, float* __restrict__ out,
    float* __restrict__ lse, int n_qtiles) {
  __shared__ __attribute__((aligned(1024))) uint8_t k_lds0[kTileBytes];
  __shared__ __attribute__((aligned(1024))) uint8_t v_lds0[kTileBytes];
  __shared__ __attribute__((aligned(1024))) uint8_t k_lds1[kTileBytes];
  __shared__ __attribute__((aligned(1024))) uint8_t v_lds1[kTileBytes];

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int n = lane & 31;   // query column of this lane
  const int hk = lane >> 5;  // which half of each 32-key block this lane holds
  const int g = blockIdx.x % kKvHeads;
  const int qt = n_qtiles - 1 - (int)(blockIdx.x / kKvHeads);
  const int q0 = qt * kBQ;
  const int qpos = q0 + 16 * wave + (n & 15);
  const int head = kGroup * g + (n >> 4);
  const bool qvalid = qpos < chunk_len;
  const int qabs = prefix_len + qpos;
  const int total = prefix_len + chunk_len;

  const int kv_end = min(prefix_len + q0 + kBQ, total);
  const int n_tiles = (kv_end + kBK - 1) / kBK;
  const int wave_first = prefix_len + q0 + 16 * wave;  // smallest query position of the wave
  const TileArgs ta{k_pages, v_pages, block_table, num_pages, g, total, wave, lane};

  issue_tile(ta, 0, k_lds0, v_lds0);

  // Q^T fragments: k-step ks covers dims 16ks..16ks+15; this lane holds dims 16ks+8hk..+7.
  bf16x8_t qf[8];
  {
    const uint16_t* qrow = q + ((size_t)(qvalid ? qpos : 0) * kQHeads + head) * kHeadDim;
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
      uint4 v = make_uint4(0, 0, 0, 0);
      if (qvalid) v = *reinterpret_cast<const uint4*>(qrow + 16 * ks + 8 * hk);
      qf[ks] = __builtin_bit_cast(bf16x8_t, v);
    }
  }

  SoftmaxState sm;
#pragma unroll
  for (int dt = 0; dt < 4; ++dt)
#pragma unroll
    for (int v = 0; v < 16; ++v) sm.o_acc[dt][v] = 0.f;
  sm.m = kNegInf;
  sm.l = 0.f;

  // Two tiles per trip: stage 0 then stage 1.  At the top of each tile: own DMAs done, barrier
  // (everyone's DMAs visible, everyone done with the other stage), start the next tile's DMA into
  // the other stage, compute this one.
  for (int kt = 0; kt < n_tiles; kt += 2) {
    wait_dma();
    __syncthreads();
    if (kt + 1 < n_tiles) issue_tile(ta, kt + 1, k_lds1, v_lds1);
    compute_tile(sm, qf, k_lds0, v_lds0, kt, n, hk, lane, kt * kBK + kBK - 1 > wave_first, qabs,
                 scale_log2);
    if (kt + 1 >= n_tiles) break;
    wait_dma();
    __syncthreads();
    if (kt + 2 < n_tiles) issue_tile(ta, kt + 2, k_lds0, v_lds0);
    compute_tile(sm, qf, k_lds1, v_lds1, kt + 1, n, hk, lane,
                 (kt + 1) * kBK + kBK - 1 > wave_first, qabs, scale_log2);
  }

  const float l_tot = sm.l + __shfl_xor(sm.l, 32, 64);
  if (qvalid) {
    const float inv = 1.f / l_tot;
    float* orow = out + ((size_t)qpos * kQHeads + head) * kHeadDim;
    // Accumulator element v of tile dt is dim 32dt + 8(v/4) + 4hk + v%4.
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
      for (int a = 0; a < 4; ++a)
        *reinterpret_cast<float4*>(orow + 32 * dt + 8 * a + 4 * hk) =
            make_float4(sm.o_acc[dt][4 * a] * inv, sm.o_acc[dt][4 * a + 1] * inv,
                        sm.o_acc[dt][4 * a + 2] * inv, sm.o_acc[dt][4 * a + 3] * inv);
    if (hk == 0) lse[(size_t)qpos * kQHeads + head] = (sm.m + log2f(l_tot)) * kLn2;
  }
}

}  // namespace

hipError_t launch_prefill(const KvPools& kv, const uint16_t* q, int chunk_len, int prefix_len,
                          const int32_t* block_table, float scale, float* out, float* lse,
                          hipStream_t stream) {
  const int n_qtiles = (chunk_len + kBQ - 1) / kBQ;
  prefill_kernel<<<dim3(n_qtiles * kKvHeads), dim3(256), 0, stream>>>(
      kv.k, kv.v, kv.num_pages, q, chunk_len, prefix_len, block_table, scale * kLog2e, out, lse,
      n_qtiles);
  return hipGetLastError();
}

}  // namespace mtd
