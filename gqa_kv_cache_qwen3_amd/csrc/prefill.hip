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
// tile.  In LDS a tile is four column groups of 64 bytes (dims 32j .. 32j+31) of 64 rows each:
// 16-byte slot of (row r, chunk c) = 256 (c/4) + 4 r + ((c%4) ^ g(r)), g(r) = (r/4)%4 for K and
// 0 for V.  That layout makes both read patterns free of bank conflicts and every read address a
// per-lane base plus a compile-time offset, and each load instruction still fetches 16 rows x
// 64 contiguous bytes.
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

constexpr int kBQ = 128;  // chunk positions per workgroup (8 waves x 16 positions x 2 heads)
constexpr int kWaves = 8;
constexpr int kBK = 64;   // keys per tile (one page)
constexpr int kTileBytes = kBK * kHeadDim * 2;  // 16 KiB
constexpr float kNegInf = -__builtin_huge_valf();

typedef short short4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) short4_t lds_short4_t;
typedef __attribute__((address_space(3))) void lds_void_t;
typedef const __attribute__((address_space(1))) void global_cvoid_t;

// Direct-to-LDS load of one K or V tile, 2 instructions per wave.  Instruction inst fills slots
// 64 inst .. 64 inst + 63 = column group inst/4, rows 16 (inst%4) .. +15; lane l writes slot
// 64 inst + l and so fetches row 16 (inst%4) + l/4, chunk 4 (inst/4) + ((l%4) ^ g(row)), where
// g = (row/4)%4 for K (kSwizzle) and 0 for V.  Rows >= nvalid fetch row 0 instead.
template <bool kSwizzle>
__device__ __forceinline__ void dma_tile(const uint16_t* __restrict__ blk, uint8_t* lds, int wave,
                                         int lane, int nvalid) {
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int inst = 2 * wave + j;
    const int r = 16 * (inst & 3) + (lane >> 2);
    const int c = 4 * (inst >> 2) + ((lane & 3) ^ (kSwizzle ? ((r >> 2) & 3) : 0));
    const int rs = r < nvalid ? r : 0;
    __builtin_amdgcn_global_load_lds((global_cvoid_t*)(blk + rs * kHeadDim + c * 8),
                                     (lds_void_t*)(lds + inst * 1024), 16, 0, 0);
  }
}

// s_waitcnt immediates (gfx9 encoding: vmcnt bits 3:0 and 15:14, expcnt 6:4, lgkmcnt 11:8; the
// counters not waited on are left at their maximum).  As builtins, so the compiler's own wait
// tracking knows which DMAs they retire.
constexpr int kWaitVm0 = 0x0F70;  // vmcnt(0)
constexpr int kWaitVm4 = 0x0F74;  // vmcnt(4): all but the most recent tile's 4 DMAs per wave
__device__ __forceinline__ void wait_dma() { __builtin_amdgcn_s_waitcnt(kWaitVm0); }
__device__ __forceinline__ void wait_dma_keep_one() { __builtin_amdgcn_s_waitcnt(kWaitVm4); }
// Workgroup barrier without a memory fence: __syncthreads() would also drain the DMA still in
// flight for the next tile.  Ordering is explicit instead: each wave waits for its own DMAs of the
// tile about to be read (above), every LDS read of the previous tile has been consumed by an MFMA
// before its wave arrives, and the empty asm statements keep the compiler from moving memory
// operations across the barrier.
__device__ __forceinline__ void tile_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

struct TileArgs {
  const uint16_t* k_pages;
  const uint16_t* v_pages;
  const int32_t* block_table;
  int num_pages, g, total, wave, lane, n_tiles;
};

// Page id of tile kt (loaded one tile ahead of its DMA so the scalar load is never waited on).
__device__ __forceinline__ int tile_page(const TileArgs& a, int kt) {
  return kt < a.n_tiles ? a.block_table[kt] : 0;
}

__device__ __forceinline__ void issue_tile(const TileArgs& a, int kt, int page, uint8_t* k_lds,
                                           uint8_t* v_lds) {
  if (page < 0 || page >= a.num_pages) page = 0;  // out-of-pool ids: defined reads, unspecified result
  const size_t blk = ((size_t)page * kKvHeads + a.g) * (kPage * kHeadDim);
  const int nvalid = min(kBK, a.total - kt * kBK);
  dma_tile<true>(a.k_pages + blk, k_lds, a.wave, a.lane, nvalid);
  dma_tile<false>(a.v_pages + blk, v_lds, a.wave, a.lane, nvalid);
}

struct SoftmaxState {
  floatx16_t o_acc[4];  // O^T tiles: dims 32dt .. 32dt+31 x 32 query columns
  float m;              // running max of the column, log2 units (same in both halves)
  float l;              // running sum of exp2(x - m) over this lane's keys
};

// Per-lane LDS byte bases; every read adds a compile-time offset to one of them.
//   kbase[ks%2]: K fragment of row n, chunk 2ks + hk  -> + 4096 (ks/2) + 2048 mt
//   vbase:       transposed V read of keys 4hk + (l%16)/4, dims 16((l/16)%2) + 4(l%4) .. +3
//                -> + 4096 dt + 64 (32 mt + 16 t + 8 sec)
struct LdsOffsets {
  int kbase[2];
  int vbase;
};

__device__ __forceinline__ LdsOffsets make_offsets(int lane) {
  LdsOffsets o;
  const int n = lane & 31, hk = lane >> 5, gi = lane & 15, half = (lane >> 4) & 1;
#pragma unroll
  for (int e = 0; e < 2; ++e) o.kbase[e] = 64 * n + 16 * ((2 * e + hk) ^ ((n >> 2) & 3));
  o.vbase = 64 * (4 * hk + (gi >> 2)) + 16 * (2 * half + ((gi & 3) >> 1)) + 8 * (gi & 1);
  return o;
}

// S^T block mt (keys 32mt .. 32mt+31 of the tile) for this wave's 32 query columns.
__device__ __forceinline__ floatx16_t scores(const bf16x8_t (&qf)[8], const uint8_t* k_lds,
                                             const LdsOffsets& off, int mt) {
  floatx16_t st;
#pragma unroll
  for (int v = 0; v < 16; ++v) st[v] = 0.f;
#pragma unroll
  for (int ks = 0; ks < 8; ++ks) {
    const bf16x8_t a = __builtin_bit_cast(
        bf16x8_t, *reinterpret_cast<const uint4*>(k_lds + off.kbase[ks & 1] + 4096 * (ks >> 1) + 2048 * mt));
    st = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[ks], st, 0, 0, 0);
  }
  return st;
}

// Online-softmax update with one 32-key block and its P^T operands (two 16-key k-steps).
template <bool kMask>
__device__ __forceinline__ void softmax_block(SoftmaxState& sm, floatx16_t& st, bf16x8_t (&pf)[2],
                                              int key0, int hk, int qabs, float scale_log2) {
  // Accumulator element v is key key0 + 8(v/4) + 4hk + v%4.
  float smax = kNegInf;
#pragma unroll
  for (int v = 0; v < 16; ++v) {
    float x = st[v];
    if (kMask) {
      const int key = key0 + 8 * (v >> 2) + 4 * hk + (v & 3);
      x = key <= qabs ? x : kNegInf;
      st[v] = x;
    }
    smax = fmaxf(smax, x);
  }
  smax = max_xor32(smax);
  // Exact running max, so the largest weight of a column is exactly 1 before its bf16 rounding
  // (peaked softmaxes stay accurate); the output accumulators are rescaled only on the blocks
  // where some column's max actually grew.
  const float m_new = fmaxf(sm.m, smax * scale_log2);
  if (__any(m_new > sm.m)) {
    const float alpha = m_new == sm.m ? 1.f : fast_exp2(sm.m - m_new);
    sm.l *= alpha;
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
      for (int v = 0; v < 16; ++v) sm.o_acc[dt][v] *= alpha;
  }
  sm.m = m_new;
  const float m_use = m_new == kNegInf ? 0.f : m_new;
  float psum = 0.f;
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    uint32_t w[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float p0 = fast_exp2(fmaf(st[8 * t + 2 * j], scale_log2, -m_use));
      const float p1 = fast_exp2(fmaf(st[8 * t + 2 * j + 1], scale_log2, -m_use));
      psum += p0 + p1;
      w[j] = pack_bf16x2(p0, p1);
    }
    pf[t] = __builtin_bit_cast(bf16x8_t, make_uint4(w[0], w[1], w[2], w[3]));
  }
  sm.l += psum;
}

// O^T += V^T P^T for 32-key block mt.  k-step t: this lane's 8 keys are 32mt + 16t + 4hk + {0..3}
// and the same + 8, read transposed from the row-major V tile (two 8-byte reads per MFMA).
__device__ __forceinline__ void accumulate_block(SoftmaxState& sm, const bf16x8_t (&pf)[2],
                                                 const uint8_t* v_lds, const LdsOffsets& off,
                                                 int mt) {
#pragma unroll
  for (int dt = 0; dt < 4; ++dt) {
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const int base = off.vbase + 4096 * dt + 64 * (32 * mt + 16 * t);
      const short4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_short4_t*)(v_lds + base));
      const short4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_short4_t*)(v_lds + base + 64 * 8));
      const bf16x8_t a = __builtin_bit_cast(bf16x8_t, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
      sm.o_acc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pf[t], sm.o_acc[dt], 0, 0, 0);
    }
  }
}

// One 64-key tile as two 32-key blocks (S^T, softmax, O^T update each); the two waves sharing a
// SIMD interleave their MFMA and VALU phases.
template <bool kMask>
__device__ __forceinline__ void compute_tile(SoftmaxState& sm, const bf16x8_t (&qf)[8],
                                             const uint8_t* k_lds, const uint8_t* v_lds,
                                             const LdsOffsets& off, int kt, int hk, int qabs,
                                             float scale_log2) {
  bf16x8_t p0[2], p1[2];
  floatx16_t s0 = scores(qf, k_lds, off, 0);
  softmax_block<kMask>(sm, s0, p0, kt * kBK, hk, qabs, scale_log2);
  accumulate_block(sm, p0, v_lds, off, 0);
  floatx16_t s1 = scores(qf, k_lds, off, 1);
  softmax_block<kMask>(sm, s1, p1, kt * kBK + 32, hk, qabs, scale_log2);
  accumulate_block(sm, p1, v_lds, off, 1);
}

__global__ __launch_bounds__(512, 1) void prefill_kernel(
    const uint16_t* __restrict__ k_pages, const uint16_t* __restrict__ v_pages, int num_pages,
    const uint16_t* __restrict__ q, int chunk_len, int prefix_len,
    const int32_t* __restrict__ block_table, float scale_log2, float* __restrict__ out,
    float* __restrict__ lse, int n_qtiles) {
  // Two stages of (K, V) tiles, 64 KiB.  Separate arrays, so the compiler can see that the DMA
  // into one stage never aliases the reads of the other and adds no wait of its own between them.
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
  // Tiles whose keys all precede the workgroup's first query need no causal mask.
  const int n_plain = min((prefix_len + q0 + 1) / kBK, n_tiles);
  const TileArgs ta{k_pages, v_pages, block_table, num_pages, g, total, wave, lane, n_tiles};

  // Tiles 0 and 1 in flight before anything else.
  issue_tile(ta, 0, tile_page(ta, 0), k_lds0, v_lds0);
  int next_page = tile_page(ta, 1);

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
  const LdsOffsets off = make_offsets(lane);

  SoftmaxState sm;
#pragma unroll
  for (int dt = 0; dt < 4; ++dt)
#pragma unroll
    for (int v = 0; v < 16; ++v) sm.o_acc[dt][v] = 0.f;
  sm.m = kNegInf;
  sm.l = 0.f;

  // Tile kt lives in stage kt % 2.  At the top of tile kt: wait for this wave's DMAs of tile kt,
  // barrier (everyone's DMAs of tile kt visible, everyone done with tile kt-1), start tile kt+1's
  // DMA into the stage tile kt-1 used, compute tile kt.  Main loop: two tiles per trip with
  // compile-time stages, none of them reaching the workgroup's first query (no causal mask).
  // Tail: the rest, masked.
#define MTD_PREFILL_STEP(KT, CUR_K, CUR_V, NXT_K, NXT_V, MASK)                          \
  {                                                                                     \
    wait_dma();                                                                         \
    tile_barrier();                                                                     \
    if ((KT) + 1 < n_tiles) issue_tile(ta, (KT) + 1, next_page, NXT_K, NXT_V);          \
    next_page = tile_page(ta, (KT) + 2);                                                \
    compute_tile<MASK>(sm, qf, CUR_K, CUR_V, off, (KT), hk, qabs, scale_log2);          \
  }
  int kt = 0;
  for (; kt + 1 < n_plain; kt += 2) {
    MTD_PREFILL_STEP(kt, k_lds0, v_lds0, k_lds1, v_lds1, false)
    MTD_PREFILL_STEP(kt + 1, k_lds1, v_lds1, k_lds0, v_lds0, false)
  }
  for (; kt < n_tiles; ++kt) {
    const bool odd = kt & 1;
    MTD_PREFILL_STEP(kt, odd ? k_lds1 : k_lds0, odd ? v_lds1 : v_lds0, odd ? k_lds0 : k_lds1,
                     odd ? v_lds0 : v_lds1, true)
  }
#undef MTD_PREFILL_STEP

  const float l_tot = sum_xor32(sm.l);
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
  prefill_kernel<<<dim3(n_qtiles * kKvHeads), dim3(64 * kWaves), 0, stream>>>(
      kv.k, kv.v, kv.num_pages, q, chunk_len, prefix_len, block_table, scale * kLog2e, out, lse,
      n_qtiles);
  return hipGetLastError();
}

}  // namespace mtd
