// Causal attention of one prefill chunk over the paged KV cache, flash-style, on bf16 MFMA.
//
// Long prompts are prefilled in 4096-token chunks; chunk query i (absolute position P + i) attends
// to every key before the chunk and to the chunk's keys up to itself ("Optimizing ASR Models to
// Transcribe 90-Minute Multi-Speaker Audio", section Chunked Prefill for Long Audio).  A short
// prompt is one chunk at P = 0.  No score matrix is ever materialised: the scores of one 64-key
// tile live in registers and are folded into the output with an fp32 online softmax.
//
// Work split.  One workgroup (8 wavefronts, two per SIMD) owns 128 chunk positions of one KV
// head and serves both query heads of its GQA group, so every K/V tile staged in LDS feeds 256
// query rows.  Wave w takes positions 16w .. 16w+15 for both heads: 32 query columns.  Workgroup
// id = 8 * (position tile, longest first) + KV head, so the dispatcher's round-robin over the 8
// XCDs keeps all tiles of one KV head on one XCD and its L2 serves the K/V re-reads.  With a
// workspace, items are rebalanced instead (see launch_prefill): tiles t and T-1-t of a chunk
// together always hold the same number of key tiles, so each such pair runs as two workgroups of
// equal work, or, in short chunks, every item runs as two halves.  Split items are merged
// afterwards by prefill_merge_kernel.
//
// K/V staging.  A 64-key tile is one page of the KV head: 16 KiB of K and 16 KiB of V, each
// brought into LDS by 16-byte direct-to-LDS buffer loads (buffer_load_dwordx4 ... lds: the page's
// address in a scalar resource descriptor, a 32-bit offset per lane, no registers, no VALU) into
// one of three stages: the tile being computed, the next one in flight, and the one
// the DMA after that will overwrite.  In LDS a tile is four column groups of 64 bytes (dims
// 32j .. 32j+31) of 64 rows each: 16-byte slot of (row r, chunk c) = 256 (c/4) + 4 r +
// ((c%4) ^ g(r)), g(r) = (r/4)%4 for K and 0 for V.  That layout makes both read patterns free
// of bank conflicts and every read address a per-lane base plus a compile-time offset, and each
// load instruction still fetches 16 rows x 64 contiguous bytes.
//
// Per 32-key block:
//   S^T = K Q^T   v_mfma_f32_32x32x16_bf16, keys as rows: a lane holds one query column and 16
//                 of the 32 keys of the block, so the softmax over keys is mostly in-lane (one
//                 exchange with lane ^ 32).  K fragments: ds_read_b128.
//   online softmax in fp32 (exp2, scale folded into one FMA); P rounded to bf16.
//   O^T += V^T P^T  the P^T operand is exactly the S^T accumulator layout, so P never leaves the
//                 registers.  The V^T operand comes straight from the row-major V tile through
//                 ds_read_b64_tr_b16 (each 16-lane group receives the transpose of the 4 x 16
//                 block its lanes address), two reads per MFMA.
// Software pipeline: the softmax of block b (VALU) is issued between the MFMAs of block b+1's
// scores and of block b-1's output update, so one wave keeps the matrix pipe and the vector ALU
// busy at once; block b's V^T fragments are read one step before their MFMAs.  One barrier per
// tile, between its two blocks.
// Causal masking is applied only on tiles that reach past the workgroup's first position.  Keys
// past the request's last token (tail of the last page) are loaded from the page's first row
// instead of their slots, so V stays finite where their weight is exactly zero.
// No score is ever NaN, so this file is compiled with -fno-honor-nans: the maxima then compile to
// bare v_max3_f32 trees without NaN-quieting copies of their operands.
#include <atomic>

#include "device_util.h"
#include "mtd_internal.h"

namespace mtd {
namespace {

constexpr int kBQ = 128;  // chunk positions per workgroup (8 waves x 16 positions x 2 heads)
constexpr int kWaves = 8;
constexpr int kBK = 64;   // keys per tile (one page)
constexpr int kTileBytes = kBK * kHeadDim * 2;  // 16 KiB
constexpr float kNegInf = -__builtin_huge_valf();
constexpr float kMaxFloor = -1e30f;  // initial running max: below any real scaled score

typedef short short4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) short4_t lds_short4_t;
typedef __attribute__((address_space(3))) void lds_void_t;
// Word 3 of a raw buffer resource descriptor on gfx9-family parts (32-bit data format, no
// swizzle, no index stride).
constexpr int kBufferWord3 = 0x00020000;

// Direct-to-LDS load of one K or V tile, 2 instructions per wave.  Instruction inst fills slots
// 64 inst .. 64 inst + 63 = column group inst/4, rows 16 (inst%4) .. +15; lane l writes slot
// 64 inst + l and so fetches row 16 (inst%4) + l/4, chunk 4 (inst/4) + ((l%4) ^ g(row)), where
// g = (row/4)%4 for K (kSwizzle) and 0 for V.  Rows >= nvalid fetch row 0 instead.
// The loads are buffer loads: the page's base address goes into a resource descriptor built by
// the scalar unit, and each lane supplies a 32-bit byte offset within the 16 KiB block, so a
// full tile costs no vector ALU work at all.
__device__ __forceinline__ uint32_t dma_offset(int wave, int j, int lane, bool swizzle, int nvalid) {
  const int inst = 2 * wave + j;
  const int r = 16 * (inst & 3) + (lane >> 2);
  const int c = 4 * (inst >> 2) + ((lane & 3) ^ (swizzle ? ((r >> 2) & 3) : 0));
  const int rs = r < nvalid ? r : 0;
  return (uint32_t)(rs * kHeadDim + c * 8) * 2u;
}

__device__ __forceinline__ void dma_tile(const uint16_t* blk, uint8_t* lds, int wave,
                                         const uint32_t (&off)[2]) {
  const __amdgpu_buffer_rsrc_t rsrc =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(blk), (short)0, kTileBytes, kBufferWord3);
#pragma unroll
  for (int j = 0; j < 2; ++j)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (lds_void_t*)(lds + (2 * wave + j) * 1024), 16, off[j], 0,
                                             0, 0);
}

// s_waitcnt vmcnt(0) (gfx9 encoding: vmcnt bits 3:0 and 15:14, expcnt 6:4, lgkmcnt 11:8; the
// counters not waited on are left at their maximum).  As a builtin, so the compiler's own wait
// tracking knows which DMAs it retires.
constexpr int kWaitVm0 = 0x0F70;
__device__ __forceinline__ void wait_dma() { __builtin_amdgcn_s_waitcnt(kWaitVm0); }
// Workgroup barrier without a memory fence: __syncthreads() would also drain the DMA still in
// flight for the next tile.  Ordering is explicit instead: each wave waits for its own DMAs of the
// tile about to be read (above), every LDS read of the stage about to be refilled has been
// consumed by an MFMA before its wave arrives, and the empty asm statements keep the compiler from
// moving memory operations across the barrier.
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
  uint32_t k_off[2], v_off[2];  // this lane's byte offsets in a full K / V block
};

// Page id of tile kt (loaded one tile ahead of its DMA so the scalar load is never waited on).
__device__ __forceinline__ int tile_page(const TileArgs& a, int kt) {
  return kt < a.n_tiles ? a.block_table[kt] : 0;
}

__device__ __forceinline__ void issue_tile(const TileArgs& a, int kt, int page, uint8_t* k_lds,
                                           uint8_t* v_lds) {
  if (page < 0 || page >= a.num_pages) page = 0;  // out-of-pool id: a defined read; the tile gets no weight
  const size_t blk = ((size_t)page * kKvHeads + a.g) * (kPage * kHeadDim);
  const int nvalid = a.total - kt * kBK;
  if (nvalid >= kBK) {
    dma_tile(a.k_pages + blk, k_lds, a.wave, a.k_off);
    dma_tile(a.v_pages + blk, v_lds, a.wave, a.v_off);
  } else {  // the request's last, partly filled page
    const uint32_t k_off[2] = {dma_offset(a.wave, 0, a.lane, true, nvalid),
                               dma_offset(a.wave, 1, a.lane, true, nvalid)};
    const uint32_t v_off[2] = {dma_offset(a.wave, 0, a.lane, false, nvalid),
                               dma_offset(a.wave, 1, a.lane, false, nvalid)};
    dma_tile(a.k_pages + blk, k_lds, a.wave, k_off);
    dma_tile(a.v_pages + blk, v_lds, a.wave, v_off);
  }
}

// Causal bound of this lane's query row for key tile kt: keys past it get no weight.  A segment
// whose table holds an out-of-pool page id runs every tile through the masked steps, and such a
// tile's bound is -1, so none of its keys gets weight (the same keys decode skips).
__device__ __forceinline__ int tile_bound(const TileArgs& a, bool any_bad, int kt, int qabs) {
  if (any_bad) {
    const int page = a.block_table[kt];
    if (page < 0 || page >= a.num_pages) return -1;
  }
  return qabs;
}

struct SoftmaxState {
  floatx16_t o_acc[4];  // O^T tiles: dims 32dt .. 32dt+31 x 32 query columns
  float m;              // running max of the column, log2 units (same in both halves); starts
                        // at a finite floor so that no step needs a special case for -inf
  float l;              // running sum of exp2(x - m) over this lane's keys
  float alpha;          // rescale of o_acc still owed for the last block's max (1 = none)
};

// Per-lane LDS byte bases; every read adds a compile-time offset to one of them.
//   kbase[ks%2]: K fragment of row n, chunk 2ks + hk  -> + 4096 (ks/2) + 2048 mt
//   vbase:       transposed V read of keys 4hk + (l%16)/4, dims 16((l/16)%2) + 4(l%4) .. +3
//                -> + 4096 dt + 64 (32 mt + 16 t + 8 sec)
struct LdsOffsets {
  int kbase[2];
  int kbase_hi[2];  // kbase + 64 KiB, for stages beyond the 16-bit immediate offset range
  int vbase;
};

__device__ __forceinline__ LdsOffsets make_offsets(int lane) {
  LdsOffsets o;
  const int n = lane & 31, hk = lane >> 5, gi = lane & 15, half = (lane >> 4) & 1;
#pragma unroll
  for (int e = 0; e < 2; ++e) {
    o.kbase[e] = 64 * n + 16 * ((2 * e + hk) ^ ((n >> 2) & 3));
    o.kbase_hi[e] = o.kbase[e] + 65536;
    asm volatile("" : "+v"(o.kbase_hi[e]));  // keep it in a register
  }
  o.vbase = 64 * (4 * hk + (gi >> 2)) + 16 * (2 * half + ((gi & 3) >> 1)) + 8 * (gi & 1);
  return o;
}

// K fragments of 32-key block mt (keys 32mt .. 32mt+31 of the tile), one per k-step.  hi: the stage
// lies past 64 KiB, so the address is formed from kbase_hi (the same byte address) to keep the
// immediate offset within 16 bits.
__device__ __forceinline__ void load_k(bf16x8_t (&kf)[8], const uint8_t* k_lds, bool hi, const LdsOffsets& off,
                                       int mt) {
#pragma unroll
  for (int ks = 0; ks < 8; ++ks) {
    const uint8_t* p = hi ? k_lds - 65536 + off.kbase_hi[ks & 1] : k_lds + off.kbase[ks & 1];
    kf[ks] = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const uint4*>(p + 4096 * (ks >> 1) + 2048 * mt));
  }
}

// V^T fragments of block mt: k-step t of dim tile dt holds this lane's 8 keys 32mt + 16t + 4hk +
// {0..3} and the same + 8, read transposed from the row-major V tile (two 8-byte reads each).
__device__ __forceinline__ void load_v(bf16x8_t (&vf)[8], const uint8_t* v_lds, const LdsOffsets& off,
                                       int mt) {
#pragma unroll
  for (int dt = 0; dt < 4; ++dt)
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const int base = off.vbase + 4096 * dt + 64 * (32 * mt + 16 * t);
      const short4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_short4_t*)(v_lds + base));
      const short4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_short4_t*)(v_lds + base + 64 * 8));
      vf[2 * dt + t] = __builtin_bit_cast(bf16x8_t, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
    }
}

// S^T block = K Q^T for this wave's 32 query columns.
__device__ __forceinline__ floatx16_t mma_scores(const bf16x8_t (&kf)[8], const bf16x8_t (&qf)[8]) {
  floatx16_t st;
#pragma unroll
  for (int v = 0; v < 16; ++v) st[v] = 0.f;
#pragma unroll
  for (int ks = 0; ks < 8; ++ks) st = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[ks], qf[ks], st, 0, 0, 0);
  return st;
}

// O^T += V^T P^T for one 32-key block.
__device__ __forceinline__ void mma_pv(floatx16_t (&o)[4], const bf16x8_t (&vf)[8], const bf16x8_t (&pf)[2]) {
#pragma unroll
  for (int dt = 0; dt < 4; ++dt)
#pragma unroll
    for (int t = 0; t < 2; ++t) o[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf[2 * dt + t], pf[t], o[dt], 0, 0, 0);
}

// New running max (log2 units) of the column after one block.  Accumulator element v is key
// key0 + 8(v/4) + 4hk + v%4; with kMask, keys after the column's position become -inf.
template <bool kMask>
__device__ __forceinline__ float block_max(floatx16_t& st, float m, int key0, int hk, int qabs,
                                           float scale_log2) {
  if (kMask) {
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int key = key0 + 8 * (v >> 2) + 4 * hk + (v & 3);
      st[v] = key <= qabs ? st[v] : kNegInf;
    }
  }
  // Balanced tree (depth 3 of 3-input maxima) instead of a 16-long chain.
  const float a0 = fmaxf(fmaxf(st[0], st[1]), st[2]), a1 = fmaxf(fmaxf(st[3], st[4]), st[5]);
  const float a2 = fmaxf(fmaxf(st[6], st[7]), st[8]), a3 = fmaxf(fmaxf(st[9], st[10]), st[11]);
  const float a4 = fmaxf(fmaxf(st[12], st[13]), st[14]);
  float smax = fmaxf(fmaxf(fmaxf(a0, a1), a2), fmaxf(fmaxf(a3, a4), st[15]));
  float other = smax;
  swap_halves(smax, other);
  return fmaxf(m, fmaxf(smax, other) * scale_log2);
}

// P^T operands of one block (exp2 of the scaled scores minus the running max, rounded to bf16)
// and the fp32 sum of the unrounded weights over this lane's keys.
__device__ __forceinline__ float block_exp(const floatx16_t& st, float m_use, float scale_log2,
                                           bf16x8_t (&pf)[2]) {
  float part[4];  // four independent partial sums instead of one 16-long chain
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    uint32_t w[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float p0 = fast_exp2(fmaf(st[8 * t + 2 * j], scale_log2, -m_use));
      const float p1 = fast_exp2(fmaf(st[8 * t + 2 * j + 1], scale_log2, -m_use));
      part[j] = t == 0 ? p0 + p1 : part[j] + (p0 + p1);
      w[j] = pack_bf16x2(p0, p1);
    }
    pf[t] = __builtin_bit_cast(bf16x8_t, make_uint4(w[0], w[1], w[2], w[3]));
  }
  return (part[0] + part[1]) + (part[2] + part[3]);
}

// One software-pipelined step: the online softmax of block b (scores s_cur, already computed)
// runs while the MFMA pipe works on the scores of block b+1 (s_next, from k_lds block mt_next;
// skipped when kScore is false) and on O^T += V^T P^T of block b-1 (p_prev, with its V^T
// fragments v_prev read one step earlier); meanwhile block b's V^T fragments (v_lds block mt_cur)
// are read for the next step.  The running max stays exact; the output accumulators take block
// b's rescale at the start of the next step, after block b-1's product has landed and before
// block b's, and only when some column's max grew.  On return p_prev and v_prev hold block b.
template <bool kMask, bool kScore>
__device__ __forceinline__ void pipe_step(SoftmaxState& sm, floatx16_t& s_cur, floatx16_t& s_next,
                                          bf16x8_t (&p_prev)[2], bf16x8_t (&v_prev)[8],
                                          const bf16x8_t (&qf)[8], const uint8_t* k_lds, bool k_hi, int mt_next,
                                          const uint8_t* v_lds, int mt_cur, const LdsOffsets& off,
                                          int key0, int hk, int qabs, float scale_log2) {
  if (__any(sm.alpha != 1.f)) {
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
      for (int v = 0; v < 16; ++v) sm.o_acc[dt][v] *= sm.alpha;
  }
  bf16x8_t kf[8], vf[8];
  if (kScore) load_k(kf, k_lds, k_hi, off, mt_next);
  const float m_new = block_max<kMask>(s_cur, sm.m, key0, hk, qabs, scale_log2);
  if (kScore) s_next = mma_scores(kf, qf);
  mma_pv(sm.o_acc, v_prev, p_prev);
  load_v(vf, v_lds, off, mt_cur);
  const float psum = block_exp(s_cur, m_new, scale_log2, p_prev);
  sm.alpha = fast_exp2(sm.m - m_new);  // exactly 1 when the max did not move
  sm.l = fmaf(sm.l, sm.alpha, psum);
  sm.m = m_new;
#pragma unroll
  for (int i = 0; i < 8; ++i) v_prev[i] = vf[i];
  // Keep block b's softmax in this step, beside the MFMAs it is meant to overlap.
  asm volatile("" ::"v"(p_prev[0]), "v"(p_prev[1]), "v"(sm.l), "v"(sm.alpha));
  __builtin_amdgcn_sched_barrier(0);
}

// How a chunk's (position tile, KV head) items are spread over workgroups.
enum PrefillMode : int {
  kOnePass = 0,  // one workgroup per item, longest first
  kHalves = 1,   // two workgroups per item, one per half of its key tiles
  kPairs = 2,    // items t and T-1-t share two workgroups with equal key-tile counts
  kSpread = 3,   // each KV head's items, longest first, laid end to end and cut into P equal ranges
};

// Key tiles of position tile qt: every key up to the tile's last position.
__host__ __device__ __forceinline__ int item_tiles(int qt, int chunk_len, int prefix_len) {
  const int kv_end = min(prefix_len + (qt + 1) * kBQ, prefix_len + chunk_len);
  return (kv_end + kBK - 1) / kBK;
}

// kSpread: a KV head's items in the order T-1, T-2, .., 0 (longest first) laid end to end; item t
// starts at key tile item_start(t) of that sequence (item_start(-1) is the total).  Every item but
// the last has ceil(P / 64) + 2 (t + 1) key tiles (P the prefix), so the sum has a closed form.
__host__ __device__ __forceinline__ long long item_start(int t, int n_qtiles, int chunk_len, int prefix_len) {
  if (t >= n_qtiles - 1) return 0;
  const long long m = n_qtiles - 2 - t;  // items strictly between t and the last one
  const long long a = (prefix_len + kBK - 1) / kBK;
  return item_tiles(n_qtiles - 1, chunk_len, prefix_len) + m * a + (long long)(n_qtiles + t + 1) * m;
}

// Workgroup (of the P per KV head) whose range [j W / P, (j+1) W / P) holds key tile x.
__host__ __device__ __forceinline__ int spread_owner(long long x, int spread, long long total) {
  return (int)(((x + 1) * spread - 1) / total);
}

// kPairs: pair p joins the long tile T-1-p (L key tiles) and the short tile p (S tiles; none when
// T is odd and p is the middle tile).  Their combined L + S tiles are the same for every pair, so
// cutting that sequence at w = (L + S) / 2 gives two workgroups equal work: the first takes the
// long tile's tiles [0, w), the second its tiles [w, L) and then the whole short tile.  The long
// tile is split when 0 < w < L; its first part goes to the workspace and is merged afterwards.
struct PairPlan {
  int t_long, t_short, n_long, n_short, cut;
};

__device__ __forceinline__ PairPlan pair_plan(int p, int n_qtiles, int chunk_len, int prefix_len) {
  PairPlan pp;
  pp.t_long = n_qtiles - 1 - p;
  pp.t_short = p < pp.t_long ? p : -1;
  pp.n_long = item_tiles(pp.t_long, chunk_len, prefix_len);
  pp.n_short = pp.t_short >= 0 ? item_tiles(pp.t_short, chunk_len, prefix_len) : 0;
  pp.cut = (pp.n_long + pp.n_short) / 2;
  return pp;
}

// One stretch of work for a workgroup: key tiles [t0, t1) of position tile qt, written to the
// workspace (partial, merged later) or to out / lse.
struct Segment {
  int qt, t0, t1, to_ws;
};

__global__ __launch_bounds__(512, 1) void prefill_kernel(
    const uint16_t* __restrict__ k_pages, const uint16_t* __restrict__ v_pages, int num_pages,
    const uint16_t* __restrict__ q, int chunk_len, int prefix_len,
    const int32_t* __restrict__ block_table, float scale_log2, float* __restrict__ out,
    float* __restrict__ lse, float* __restrict__ part_o, float* __restrict__ part_lse, int n_qtiles,
    int mode, int spread) {
  // Three stages of (K, V) tiles, 96 KiB: the tile being read, the next tile (in flight, then
  // read from the middle of the current step on) and the stage the following DMA refills.
  // Separate arrays, so the compiler can see that the DMA into one stage never aliases the reads
  // of another and adds no wait of its own between them.  The compiler places LDS variables of
  // equal size and alignment in name order, so the V stages take bytes 0 .. 48 KiB and every V^T
  // read (16 per block) is a base register plus a 16-bit immediate offset; the K stages follow,
  // and those past 64 KiB are read through kbase_hi.
  __shared__ __attribute__((aligned(1024))) uint8_t zk_lds0[kTileBytes];
  __shared__ __attribute__((aligned(1024))) uint8_t v_lds0[kTileBytes];
  __shared__ __attribute__((aligned(1024))) uint8_t zk_lds1[kTileBytes];
  __shared__ __attribute__((aligned(1024))) uint8_t v_lds1[kTileBytes];
  __shared__ __attribute__((aligned(1024))) uint8_t zk_lds2[kTileBytes];
  __shared__ __attribute__((aligned(1024))) uint8_t v_lds2[kTileBytes];

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: LDS bases in scalar registers
  const int lane = tid & 63;
  const int n = lane & 31;   // query column of this lane
  const int hk = lane >> 5;  // which half of each 32-key block this lane holds
  const int g = blockIdx.x % kKvHeads;
  const int rank = (int)(blockIdx.x / kKvHeads);
  const int total = prefix_len + chunk_len;

  // This workgroup's segments, run one after the other: at most two, or with kSpread every item
  // that meets the workgroup's range of the head's key tiles.
  Segment seg0{0, 0, 0, 0}, seg1{0, 0, 0, 0};
  int n_seg = 0;
  int sp_t = 0;                  // kSpread: next item (position tile) and key tile of the sequence
  long long sp_cur = 0, sp_hi = 0;
  if (mode == kSpread) {
    const long long w = item_start(-1, n_qtiles, chunk_len, prefix_len);
    sp_cur = (long long)rank * w / spread;
    sp_hi = (long long)(rank + 1) * w / spread;
    // first item: the smallest t with item_start(t) <= sp_cur (item_start falls as t grows)
    int lo_t = 0, hi_t = n_qtiles - 1;
    while (lo_t < hi_t) {
      const int mid = (lo_t + hi_t) >> 1;
      if (item_start(mid, n_qtiles, chunk_len, prefix_len) <= sp_cur) hi_t = mid; else lo_t = mid + 1;
    }
    sp_t = lo_t;
  } else if (mode == kPairs) {
    const PairPlan pp = pair_plan(rank >> 1, n_qtiles, chunk_len, prefix_len);
    const bool split_long = pp.cut > 0 && pp.cut < pp.n_long;
    if ((rank & 1) == 0) {
      if (pp.cut > 0) {
        seg0 = Segment{pp.t_long, 0, min(pp.cut, pp.n_long), split_long ? 1 : 0};
        n_seg = 1;
      }
    } else {
      const Segment short_seg{pp.t_short, 0, pp.n_short, 0};
      if (pp.cut < pp.n_long) {
        seg0 = Segment{pp.t_long, pp.cut, pp.n_long, 0};
        seg1 = short_seg;
        n_seg = pp.t_short >= 0 ? 2 : 1;
      } else if (pp.t_short >= 0) {
        seg0 = short_seg;
        n_seg = 1;
      }
    }
  } else {
    // Work item: position tile qt of KV head g, longest first.  kHalves: each item is two
    // workgroups, one per half of its key tiles (the dispatcher then pairs long and short halves
    // on the CUs), and the second half's partial result goes to the workspace.
    const int split = mode == kHalves;
    const int qt = n_qtiles - 1 - (split ? rank >> 1 : rank);
    const int half = split ? rank & 1 : 0;
    const int n_item = item_tiles(qt, chunk_len, prefix_len);
    const bool cut = split && n_item >= 2;
    seg0 = Segment{qt, cut && half ? n_item / 2 : 0, cut && !half ? n_item / 2 : n_item, half};
    n_seg = half && !cut ? 0 : 1;  // the second half of an item too short to split has nothing to do
  }

  const LdsOffsets off = make_offsets(lane);
  for (int si = 0;; ++si) {
    Segment seg;
    if (mode == kSpread) {
      // Item sp_t from key tile sp_cur on, up to the end of the item or of the range.  An item
      // cut by a range boundary has two parts (no item is longer than a range): the part holding
      // its first tile goes to the workspace, the other to out.
      if (sp_cur >= sp_hi || sp_t < 0) break;
      const long long f = item_start(sp_t, n_qtiles, chunk_len, prefix_len);
      const int n_item = item_tiles(sp_t, chunk_len, prefix_len);
      const int a = (int)(sp_cur - f);
      const int b = (int)min(sp_hi - f, (long long)n_item);
      seg = Segment{sp_t, a, b, a == 0 && b < n_item ? 1 : 0};
      sp_cur = f + b;
      --sp_t;
    } else {
      if (si >= n_seg) break;
      seg = si == 0 ? seg0 : seg1;
    }
    if (si > 0) __syncthreads();  // every wave is done with the previous segment's LDS stages
    // Uniform across the workgroup: keep the segment in scalar registers.
    const int qt = __builtin_amdgcn_readfirstlane(seg.qt);
    const int t0 = __builtin_amdgcn_readfirstlane(seg.t0);
    const int t1 = __builtin_amdgcn_readfirstlane(seg.t1);
    const int half = __builtin_amdgcn_readfirstlane(seg.to_ws);
    const int q0 = qt * kBQ;
    const int qpos = q0 + 16 * wave + (n & 15);
    const int head = kGroup * g + (n >> 4);
    const bool qvalid = qpos < chunk_len;
    const int qabs = prefix_len + qpos;
    // A page id outside the pool sends the whole segment through the masked steps (tile_bound).
    bool bad = false;
    for (int kt = t0 + tid; kt < t1; kt += 64 * kWaves) {
      const int page = block_table[kt];
      bad |= page < 0 || page >= num_pages;
    }
    const bool any_bad = __syncthreads_or(bad) != 0;
    // Tiles whose keys all precede the workgroup's first query need no causal mask.
    const int n_plain = any_bad ? t0 : min((prefix_len + q0 + 1) / kBK, t1);
    const TileArgs ta{k_pages,
                      v_pages,
                      block_table,
                      num_pages,
                      g,
                      total,
                      wave,
                      lane,
                      t1,
                      {dma_offset(wave, 0, lane, true, kBK), dma_offset(wave, 1, lane, true, kBK)},
                      {dma_offset(wave, 0, lane, false, kBK), dma_offset(wave, 1, lane, false, kBK)}};

    issue_tile(ta, t0, tile_page(ta, t0), zk_lds0, v_lds0);
    int next_page = tile_page(ta, t0 + 1);
    // Stage 2's V starts as zeros: the first step multiplies it by an all-zero P^T in place of a
    // previous block.
    *reinterpret_cast<uint4*>(v_lds2 + 32 * tid) = make_uint4(0, 0, 0, 0);
    *reinterpret_cast<uint4*>(v_lds2 + 32 * tid + 16) = make_uint4(0, 0, 0, 0);

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
    sm.m = kMaxFloor;
    sm.l = 0.f;
    sm.alpha = 1.f;

    wait_dma();
    __syncthreads();
    if (t0 + 1 < t1) issue_tile(ta, t0 + 1, next_page, zk_lds1, v_lds1);
    next_page = tile_page(ta, t0 + 2);
    floatx16_t s_a, s_b;
    bf16x8_t p_prev[2], v_prev[8];
    load_v(v_prev, v_lds2, off, 1);  // zeros: stands in for the V^T of block -1
    {
      bf16x8_t kf[8];
      load_k(kf, zk_lds0, false, off, 0);
      s_a = mma_scores(kf, qf);
      const bf16x8_t zero = __builtin_bit_cast(bf16x8_t, make_uint4(0, 0, 0, 0));
      p_prev[0] = zero;
      p_prev[1] = zero;
    }

    // Tile kt lives in stage (kt - t0) % 3.  Step kt: first half = softmax of block 2kt beside the scores
    // of block 2kt+1 and the O update of block 2kt-1, reading block 2kt's V^T; then wait for tile
    // kt+1's DMA and barrier (everyone is done with tile kt-1's stage), start tile kt+2's DMA into
    // that stage; second half = softmax of block 2kt+1 beside the scores of block 2kt+2 (next
    // stage) and the O update of block 2kt, reading block 2kt+1's V^T.  Main loop: three steps per
    // trip with compile-time stages, no causal mask, never the last tile.  Then the remaining
    // steps with run-time stages (masked) and the last tile, then block 2n-1's O update.
#define MTD_PREFILL_STEP(KT, CUR_K, CUR_V, PRV_V, NXT_K, PRV_K, MASK, QB)   \
    {                                                                       \
      pipe_step<MASK, true>(sm, s_a, s_b, p_prev, v_prev, qf,               \
                            CUR_K, +(CUR_K) != +zk_lds0, 1, CUR_V, 0, off,  \
                            (KT) * kBK, hk, QB, scale_log2);                \
      wait_dma();                                                           \
      tile_barrier();                                                       \
      if ((KT) + 2 < t1) issue_tile(ta, (KT) + 2, next_page, PRV_K, PRV_V); \
      next_page = tile_page(ta, (KT) + 3);                                  \
      pipe_step<MASK, true>(sm, s_b, s_a, p_prev, v_prev, qf,               \
                            NXT_K, +(NXT_K) != +zk_lds0, 0, CUR_V, 1, off,  \
                            (KT) * kBK + 32, hk, QB, scale_log2);           \
    }
    const int n_main = min(n_plain, t1 - 1);
    int kt = t0;
    for (; kt + 3 <= n_main; kt += 3) {
      MTD_PREFILL_STEP(kt, zk_lds0, v_lds0, v_lds2, zk_lds1, zk_lds2, false, qabs)
      MTD_PREFILL_STEP(kt + 1, zk_lds1, v_lds1, v_lds0, zk_lds2, zk_lds0, false, qabs)
      MTD_PREFILL_STEP(kt + 2, zk_lds2, v_lds2, v_lds1, zk_lds0, zk_lds1, false, qabs)
    }
    for (; kt < t1 - 1; ++kt) {
      const int sc = (kt - t0) % 3;
      uint8_t* ck = sc == 0 ? zk_lds0 : sc == 1 ? zk_lds1 : zk_lds2;
      uint8_t* cv = sc == 0 ? v_lds0 : sc == 1 ? v_lds1 : v_lds2;
      uint8_t* nk = sc == 0 ? zk_lds1 : sc == 1 ? zk_lds2 : zk_lds0;
      uint8_t* pk = sc == 0 ? zk_lds2 : sc == 1 ? zk_lds0 : zk_lds1;
      uint8_t* pv = sc == 0 ? v_lds2 : sc == 1 ? v_lds0 : v_lds1;
      const int qb = tile_bound(ta, any_bad, kt, qabs);
      MTD_PREFILL_STEP(kt, ck, cv, pv, nk, pk, true, qb)
    }
#undef MTD_PREFILL_STEP
    {
      const int sc = (kt - t0) % 3;
      const uint8_t* ck = sc == 0 ? zk_lds0 : sc == 1 ? zk_lds1 : zk_lds2;
      const uint8_t* cv = sc == 0 ? v_lds0 : sc == 1 ? v_lds1 : v_lds2;
      const int qb = tile_bound(ta, any_bad, kt, qabs);
      pipe_step<true, true>(sm, s_a, s_b, p_prev, v_prev, qf, ck, ck != zk_lds0, 1, cv, 0, off, kt * kBK, hk, qb,
                            scale_log2);
      pipe_step<true, false>(sm, s_b, s_a, p_prev, v_prev, qf, ck, ck != zk_lds0, 0, cv, 1, off, kt * kBK + 32, hk,
                             qb, scale_log2);
      if (__any(sm.alpha != 1.f)) {
#pragma unroll
        for (int dt = 0; dt < 4; ++dt)
#pragma unroll
          for (int v = 0; v < 16; ++v) sm.o_acc[dt][v] *= sm.alpha;
      }
      mma_pv(sm.o_acc, v_prev, p_prev);
    }

    // A second half can hold no key a row may see (early rows of a short item): its partial is then
    // O = 0 with LSE = -inf, which the merge weighs by exactly zero.
    const float l_tot = sum_xor32(sm.l);
    if (qvalid) {
      const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
      float* const o_dst = half ? part_o : out;
      float* const l_dst = half ? part_lse : lse;
      float* orow = o_dst + ((size_t)qpos * kQHeads + head) * kHeadDim;
      // Accumulator element v of tile dt is dim 32dt + 8(v/4) + 4hk + v%4.
#pragma unroll
      for (int dt = 0; dt < 4; ++dt)
#pragma unroll
        for (int a = 0; a < 4; ++a)
          *reinterpret_cast<float4*>(orow + 32 * dt + 8 * a + 4 * hk) =
              make_float4(sm.o_acc[dt][4 * a] * inv, sm.o_acc[dt][4 * a + 1] * inv,
                          sm.o_acc[dt][4 * a + 2] * inv, sm.o_acc[dt][4 * a + 3] * inv);
      if (hk == 0) l_dst[(size_t)qpos * kQHeads + head] = l_tot > 0.f ? (sm.m + log2f(l_tot)) * kLn2 : kNegInf;
    }
  }  // segments
}

// Combines the two parts of every split item: out/lse hold one part's normalised partial,
// part_o/part_lse the other's.  Rows (position, head) from row0 on; each half-wavefront takes one
// row, 4 dims per lane.  Both LSEs are read before the row's first lane overwrites lse, in program
// order within the wave.
__global__ __launch_bounds__(256) void prefill_merge_kernel(float* __restrict__ out, float* __restrict__ lse,
                                                            const float* __restrict__ part_o,
                                                            const float* __restrict__ part_lse,
                                                            int chunk_len, int prefix_len, int n_qtiles,
                                                            int mode, int spread, int row0) {
  const int row = row0 + (int)blockIdx.x * 8 + (int)(threadIdx.x >> 5);  // (position, head)
  const int lane = threadIdx.x & 31;
  if (row >= chunk_len * kQHeads) return;
  const int qt = row / kQHeads / kBQ;
  if (mode == kPairs) {
    const int p = n_qtiles - 1 - qt;  // the pair in which qt is the long tile
    if (p > qt) return;               // qt is a short tile: never split
    const PairPlan pp = pair_plan(p, n_qtiles, chunk_len, prefix_len);
    if (pp.cut <= 0 || pp.cut >= pp.n_long) return;  // not split: out/lse are final
  } else if (mode == kSpread) {
    const long long w = item_start(-1, n_qtiles, chunk_len, prefix_len);
    const long long f = item_start(qt, n_qtiles, chunk_len, prefix_len);
    const int n_item = item_tiles(qt, chunk_len, prefix_len);
    if (spread_owner(f, spread, w) == spread_owner(f + n_item - 1, spread, w)) return;  // one part
  } else if (item_tiles(qt, chunk_len, prefix_len) < 2) {
    return;  // item was not split: out/lse are final
  }
  const float l0 = lse[row], l1 = part_lse[row];
  const float mx = fmaxf(l0, l1);
  float4* o = reinterpret_cast<float4*>(out + (size_t)row * kHeadDim) + lane;
  if (mx == kNegInf) {  // neither part holds a key the row may see (out-of-pool pages): empty result
    *o = make_float4(0.f, 0.f, 0.f, 0.f);
    if (lane == 0) lse[row] = kNegInf;
    return;
  }
  const float w0 = __expf(l0 - mx), w1 = __expf(l1 - mx);
  const float inv = 1.f / (w0 + w1);
  const float4 a = *o;
  const float4 b = reinterpret_cast<const float4*>(part_o + (size_t)row * kHeadDim)[lane];
  *o = make_float4((w0 * a.x + w1 * b.x) * inv, (w0 * a.y + w1 * b.y) * inv, (w0 * a.z + w1 * b.z) * inv,
                   (w0 * a.w + w1 * b.w) * inv);
  if (lane == 0) lse[row] = mx + __logf(w0 + w1);
}

}  // namespace

// Compute units of the calling thread's current device, queried once per device.
int device_cus() {
  static std::atomic<int> cus[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  int n = cus[dev].load(std::memory_order_relaxed);
  if (n == 0) {
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
      n = 256;
    cus[dev].store(n, std::memory_order_relaxed);
  }
  return n;
}

hipError_t launch_prefill(const KvPools& kv, const uint16_t* q, int chunk_len, int prefix_len,
                          const int32_t* block_table, float scale, void* workspace, int cu_budget,
                          float* out, float* lse, hipStream_t stream) {
  const int n_qtiles = (chunk_len + kBQ - 1) / kBQ;
  // Causal work is uneven over a chunk's position tiles (the last sees prefix + chunk keys, the
  // first only prefix), and with one workgroup per CU the time is set by the longest.  With a
  // workspace the library rebalances:
  //   - a CU budget below the device's CUs: each KV head's work is cut into budget / 8 equal
  //     ranges, one workgroup each, so the call occupies only that many CUs (the rest stay free for
  //     concurrent work); the number of ranges is lowered until no item is longer than a range;
  //   - else, at least as many items as CUs: pair tile t with tile T-1-t and cut their combined key
  //     tiles into two equal workgroups (the long tile's two parts merged afterwards);
  //   - else (short chunks): split every item's keys in two halves, which also doubles the
  //     workgroups.
  // All cost the merge pass over the split rows.  Without a workspace, one pass per item.
  const int cus = device_cus();
  int mode = kOnePass, spread = 0;
  if (workspace != nullptr) {
    if (cu_budget > 0 && cu_budget < cus) {
      mode = kSpread;
      const long long w = item_start(-1, n_qtiles, chunk_len, prefix_len);
      const long long longest = item_tiles(n_qtiles - 1, chunk_len, prefix_len);
      spread = max(1, cu_budget / kKvHeads);
      spread = (int)min((long long)spread, w / longest);  // every item fits in one range
      spread = max(spread, 1);
    } else {
      mode = n_qtiles * kKvHeads >= cus ? kPairs : kHalves;
    }
  }
  const int n_wg = mode == kSpread ? spread
                   : mode == kPairs ? 2 * ((n_qtiles + 1) / 2)
                   : mode == kHalves ? 2 * n_qtiles
                                     : n_qtiles;
  float* part_o = static_cast<float*>(workspace);
  float* part_lse = mode != kOnePass ? part_o + (size_t)chunk_len * kQHeads * kHeadDim : nullptr;
  prefill_kernel<<<dim3(n_wg * kKvHeads), dim3(64 * kWaves), 0, stream>>>(
      kv.k, kv.v, kv.num_pages, q, chunk_len, prefix_len, block_table, scale * kLog2e, out, lse,
      part_o, part_lse, n_qtiles, mode, spread);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess || mode == kOnePass) return err;
  // Only long tiles are split on the pair schedule: they start at tile T/2.
  const int rows = chunk_len * kQHeads;
  const int row0 = mode == kPairs ? (n_qtiles / 2) * kBQ * kQHeads : 0;
  prefill_merge_kernel<<<dim3((rows - row0 + 7) / 8), dim3(256), 0, stream>>>(
      out, lse, part_o, part_lse, chunk_len, prefix_len, n_qtiles, mode, spread, row0);
  return hipGetLastError();
}

}  // namespace mtd
