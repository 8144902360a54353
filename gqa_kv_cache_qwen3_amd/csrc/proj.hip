// The linear maps on either side of the attention, as one bf16 MFMA GEMM with fused epilogues.
//
// The decoder around the attention is Qwen3 with hidden size 1024 and 16 query / 8 KV heads of
// dim 128 ("Optimizing ASR Models to Transcribe 90-Minute Multi-Speaker Audio", section ASR Model
// Primer, component table; "MOSS-Transcribe-Diarize" cookbook, section Model Architecture).  Each
// layer maps the hidden states of its new tokens to q, k and v (1024 -> 2048 + 1024 + 1024), and
// the attention output back (2048 -> 1024).  Both are C[T][N] = A[T][K] W[N][K]^T with W in the
// [out][in] layout:
//   QKV projection  A = hidden states, bf16 [T][1024]; W_qkv = [Wq; Wk; Wv] bf16 [4096][1024].
//                   The epilogue writes columns 0..2047 to q [T][16][128], 2048..3071 to
//                   k [T][8][128] and 3072..4095 to v [T][8][128], each rounded to bf16, in the
//                   layouts the attention calls and the KV append take.
//   output proj.    A = the attention's float32 O [T][16][128], rounded to bf16 (the model's
//                   activation type) as it is staged into LDS; W_o bf16 [1024][2048]; C rounded
//                   to bf16 [T][1024].
//
// Kernels.  Calls with more than 64 tokens run tiled kernels: proj_wide_kernel for the QKV map
// (256 x 128 tiles) and proj_ksplit_kernel for the output map (128 x 128 tiles with K split
// between two sets of waves); see their comments.  Calls of at most 64 tokens run
// proj_skinny_kernel, which spreads K over the waves, and a tiled launch computes a last partial
// tile of at most 64 rows the same way in its first workgroups (tail_block).  All three add the products in one order (fixed K slices and groups of them,
// see kKSlice), so a token's result is the same whatever the token count and whichever kernel
// runs.  The MFMA is v_mfma_f32_32x32x16_bf16 with fp32 accumulators throughout.
//
// Staging.  Operands reach LDS by 16-byte direct-to-LDS buffer loads (no registers, no VALU),
// each instruction fetching whole 128-byte rows where it can (strided half-row fetches measured
// at about 60 % of the rate).  MFMA operands are ds_read_b128 of one row's 16-byte chunk, the
// chunks of each row permuted so that every read is free of bank conflicts.  The tiled kernels'
// K loops are unrolled at compile time, so every step is straight-line code, and a slice's MFMAs
// and the addition of its sums to the running total always share a basic block: with a branch
// between an MFMA and the read of its accumulator the compiler has been seen to leave too few
// wait states, and the read then returned a stale value.
//
// Placement.  Workgroup i runs on XCD i % 8, and each XCD has its own L2.  The QKV map splits both
// ways when its tile rows come in fours: XCD x owns the tile rows = x / 2 (mod 4) and half x % 2
// of the tile columns, so A is read by 2 XCDs and W by 4.  Otherwise each XCD owns every eighth
// tile row (every XCD then reads W whole and an eighth of A) or an eighth of the tile columns (an
// eighth of W, all of A), whichever replicates the smaller operand; the output map's float32 A is
// the larger, so its XCDs own rows.  Within an XCD the owned row index varies fastest, so the
// workgroups in flight together touch few tiles of the replicated operand and each is brought
// into the XCD's L2 once rather than once per owned row.
#include <type_traits>
#include <utility>

#include "device_util.h"
#include "mtd_internal.h"

namespace mtd {
namespace {

// Summation order, the same in all the kernels: K is cut into slices of kKSlice; each slice's
// products are accumulated by one chain of MFMAs starting from zero, and the slice sums are then
// added in slice order to a running total that starts from zero.  So a token's outputs never
// depend on how many tokens share the call or which kernel serves it.
constexpr int kKSlice = 128;
// Groups of kSliceGroup consecutive slices (1024 inputs) are summed first, each in slice order
// from zero, and the group totals are then added in order to a total that starts from zero.  The
// QKV map (K = 1024) is one group; the output map (K = 2048) is two, which proj_ksplit_kernel
// gives to two sets of waves.
constexpr int kSliceGroup = 8;
constexpr int kSkinnyRows = 64;  // calls with at most this many tokens use proj_skinny_kernel

typedef __attribute__((address_space(3))) void lds_void_t;
typedef const __attribute__((address_space(1))) void global_cvoid_t;

// Where the columns of C go: columns [lo_r, lo_{r+1}) of region r land in dst[r] (bf16, leading
// dimension ld[r]) at column n - lo_r.  One region for the output projection, three for QKV.
struct OutMap {
  uint16_t* dst[3];
  int ld[3];
  int lo[3];
};

// The map for the rows from `rows` on.
__host__ __device__ __forceinline__ OutMap shift_rows(OutMap om, int rows) {
  for (int r = 0; r < 3; ++r) om.dst[r] += (size_t)rows * om.ld[r];
  return om;
}

constexpr int kSplit2D = 2;  // tile placement: rows and columns both split over the XCDs

// Tile (tm, tn) of workgroup id for tiles of tm_rows rows; see Placement.  tm == n_tm: no tile.
__device__ __forceinline__ void tile_of(int id, int rows, int tm_rows, int n_tm, int n_tn, int rows_major,
                                        int& tm, int& tn) {
  const int x = id % 8, local = id / 8;
  if (rows_major == kSplit2D) {
    // XCD x owns the tile rows = x / 2 (mod 4) and half x % 2 of the tile columns: each operand is
    // read by fewer XCDs (A by 2, W by 4) than with either one-sided split (A by 1, W by 8).
    const int per_col = n_tn / 2;
    tm = x / 2 + 4 * (local % (n_tm / 4));
    tn = (x % 2) * per_col + local / (n_tm / 4);
    return;
  }
  if (rows_major) {
    const int n_full = rows / tm_rows;
    const int m_per = (n_full + 7) / 8;
    if (local < m_per * n_tn) {
      tm = x + 8 * (local % m_per);
      tn = local / m_per;
      if (tm >= n_full) tm = n_tm;
    } else {
      tm = n_full;
      tn = x + 8 * (local - m_per * n_tn);
    }
  } else if (n_tn % 8 == 0) {
    tn = x * (n_tn / 8) + local % (n_tn / 8);
    tm = local / (n_tn / 8);
  } else {
    tm = id / n_tn;
    tn = id % n_tn;
  }
}

// The last partial tile of a tiled launch (at most 64 rows, few beside the tiles' rows): as with
// few tokens, the grid is spread over K.  Workgroup (column block x, row block y) = 32 columns of
// W against 32 tokens, 8 waves, in LDS the tiled kernel already holds; wave w takes the K slices w * q .. w * q + q - 1 (q = k_dim / kKSlice / 8: 1 for QKV,
// 2 for o_proj).  For each slice the wave stages its 32 x 128 pieces of A and W in its own 16 KiB
// of LDS with coalesced loads (each direct-to-LDS instruction fetches 8 rows x 128 contiguous
// bytes; the float32 A comes through registers, 512 contiguous bytes per row, and is rounded to
// bf16 on the way), then runs the slice's MFMA chain from ds_read_b128 fragments.  The slice sums
// meet in LDS and are added in slice order.
//
// Per-wave staging of a 32-row x 128-column bf16 piece: two column groups of 128 bytes (8 chunks of
// 16 bytes); the slot of (row r, chunk c) is 256 (c/8) + 8 r + ((c%8) ^ ((r/2)%4)), which keeps
// the 8 lanes of each ds_read_b128 phase on distinct banks.
constexpr int kSkinnyWaves = 8;
constexpr int kSkinnyStage = 16384;  // per wave: the A piece, then the W piece

__device__ __forceinline__ int slot32_bytes(int r, int c) {
  return 16 * (256 * (c >> 3) + 8 * r + ((c & 7) ^ ((r >> 1) & 3)));
}

// Direct-to-LDS copy of rows row0 .. row0+31 (at or past rows_valid: the last valid row), columns
// k0 .. k0+127 of a bf16 matrix: instruction i fills slots 64 i .. 64 i + 63 = column group i / 4,
// rows 8 (i % 4) + lane / 8.
__device__ __forceinline__ void dma_piece32(const uint16_t* __restrict__ m, int ld, int row0,
                                            int rows_valid, int k0, uint8_t* lds, int lane) {
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int r = 8 * (i & 3) + (lane >> 3);
    const int c = 8 * (i >> 2) + ((lane & 7) ^ ((r >> 1) & 3));
    const int rs = r < rows_valid ? r : rows_valid - 1;
    __builtin_amdgcn_global_load_lds((global_cvoid_t*)(m + (size_t)(row0 + rs) * ld + k0 + 8 * c),
                                     (lds_void_t*)(lds + i * 1024), 16, 0, 0);
  }
}

// The float32 piece through registers: load j covers row 2j + lane/32, floats 4 (lane%32) .. +3.
__device__ __forceinline__ void stage_f32_piece32(const float* __restrict__ a, int ld, int row0,
                                                  int rows_valid, int k0, uint8_t* lds, int lane) {
  float4 v[16];
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    const int r = 2 * j + (lane >> 5);
    const int rs = r < rows_valid ? r : rows_valid - 1;
    v[j] = *reinterpret_cast<const float4*>(a + (size_t)(row0 + rs) * ld + k0 + 4 * (lane & 31));
  }
  const int f = lane & 31;
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    const int r = 2 * j + (lane >> 5);
    *reinterpret_cast<uint2*>(lds + slot32_bytes(r, f >> 1) + 8 * (f & 1)) =
        make_uint2(pack_bf16x2(v[j].x, v[j].y), pack_bf16x2(v[j].z, v[j].w));
  }
}

// One 32-column x 32-row block of C (column block cb, row block rb) by 8 waves: wave w stages its
// K slices in its own 16 KiB of LDS (wave_lds), and the slice sums meet in part(slice) (4 KiB per
// slice, 8 consecutive slices contiguous), which may overlap the waves' stages.
template <bool kAF32, class WaveLds, class Part>
__device__ __forceinline__ void skinny_block(const void* __restrict__ a_ptr, int lda, int rows,
                                             const uint16_t* __restrict__ w, int k_dim, const OutMap& out,
                                             int cb, int rb, WaveLds wave_lds, Part part) {
  constexpr int kMaxPerWave = 2;
  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int n_slices = k_dim / kKSlice;
  const int per_wave = n_slices / kSkinnyWaves;
  const int n = lane & 31, hk = lane >> 5;
  const int col0 = 32 * cb;
  const int row0 = 32 * rb;
  const int rows_valid = min(32, rows - row0);
  uint8_t* a_lds = wave_lds(wave);
  uint8_t* w_lds = a_lds + kSkinnyStage / 2;

  floatx16_t acc[kMaxPerWave];
#pragma unroll
  for (int t = 0; t < kMaxPerWave; ++t) {
#pragma unroll
    for (int v = 0; v < 16; ++v) acc[t][v] = 0.f;
    if (t >= per_wave) continue;
    const int k0 = (wave * per_wave + t) * kKSlice;
    dma_piece32(w, k_dim, col0, 32, k0, w_lds, lane);
    if constexpr (kAF32)
      stage_f32_piece32(static_cast<const float*>(a_ptr), lda, row0, rows_valid, k0, a_lds, lane);
    else
      dma_piece32(static_cast<const uint16_t*>(a_ptr), lda, row0, rows_valid, k0, a_lds, lane);
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): this wave's pieces are in its LDS
#pragma unroll
    for (int ks = 0; ks < kKSlice / 16; ++ks) {
      const int off = slot32_bytes(n, 2 * ks + hk);
      const bf16x8_t af = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const uint4*>(a_lds + off));
      const bf16x8_t wf = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const uint4*>(w_lds + off));
      acc[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af, wf, acc[t], 0, 0, 0);
    }
  }
  __syncthreads();  // every wave is done with its pieces; the LDS now holds the slice sums
#pragma unroll
  for (int t = 0; t < kMaxPerWave; ++t) {
    if (t >= per_wave) continue;
    float* s_part = part(wave * per_wave + t);  // [accumulator element][lane]
#pragma unroll
    for (int v = 0; v < 16; ++v) s_part[v * 64 + lane] = acc[t][v];
  }
  __syncthreads();

  // Element e = (accumulator element v, lane l): C[row0 + 8(v/4) + 4(l/32) + v%4][col0 + l%32].
  const int reg = (col0 >= out.lo[2]) ? 2 : (col0 >= out.lo[1]) ? 1 : 0;
  uint16_t* dst = out.dst[reg];
  const int ld = out.ld[reg];
  for (int e = tid; e < 16 * 64; e += blockDim.x) {
    const int v = e >> 6, l = e & 63;
    const int rr = 8 * (v >> 2) + 4 * (l >> 5) + (v & 3);
    if (rr >= rows_valid) continue;
    float total = 0.f;
    for (int g0 = 0; g0 < n_slices; g0 += kSliceGroup) {
      float group = 0.f;
      for (int sl = g0; sl < g0 + kSliceGroup; ++sl) group += part(sl)[v * 64 + l];
      total += group;
    }
    dst[(size_t)(row0 + rr) * ld + col0 - out.lo[reg] + (l & 31)] = (uint16_t)pack_bf16x2(total, 0.f);
  }
}

// Workgroups tail_base .. tail_base + tail_blocks - 1 of a tiled launch compute the rows past its
// tiles (at most 64, see split_rows) with the few-token algorithm, block b of them being column
// block b % (n_cols / 32), row block b / (n_cols / 32).  They borrow LDS from the tiled kernel's
// stage arrays: wave w stages in a0 / a1 / a2 (two waves each) or w0 / w1, and the slice sums of the
// first and second 1024-input groups go to a0 and a1.  When the tiles take more than one round of
// the grid the tail comes first and runs beside the first round; when they fit one round it comes
// last, so that no tile waits for a CU the tail holds (a tile started late re-reads W into L2).
template <bool kAF32>
__device__ __forceinline__ void tail_block(const void* a_ptr, int lda, int rows, int tail_rows,
                                           const uint16_t* w, int k_dim, int n_cols, const OutMap& out, int b,
                                           uint8_t* a0, uint8_t* a1, uint8_t* a2, uint8_t* w0, uint8_t* w1) {
  const int ncb = n_cols / 32;
  const void* a_tail = kAF32 ? (const void*)(static_cast<const float*>(a_ptr) + (size_t)rows * lda)
                             : (const void*)(static_cast<const uint16_t*>(a_ptr) + (size_t)rows * lda);
  skinny_block<kAF32>(
      a_tail, lda, tail_rows, w, k_dim, shift_rows(out, rows), b % ncb, b / ncb,
      [&](int wave) -> uint8_t* {
        switch (wave) {
          case 0: return a0;
          case 1: return a0 + kSkinnyStage;
          case 2: return a1;
          case 3: return a1 + kSkinnyStage;
          case 4: return a2;
          case 5: return a2 + kSkinnyStage;
          case 6: return w0;
          default: return w1;
        }
      },
      [&](int slice) { return reinterpret_cast<float*>(slice < kSliceGroup ? a0 : a1) + (slice % kSliceGroup) * 16 * 64; });
}

// Many tokens, bf16 A (the QKV map): a 256 x 128 tile per workgroup of 8 waves, two per SIMD,
// each computing a 64 x 64 block (wave w: rows 64 (w / 2), columns 64 (w % 2)) as 2 x 2 MFMA
// blocks.  K advances 64 at a time through a ring of three 48 KiB LDS stages with the DMA two
// stages ahead of the MFMAs.  Each direct-to-LDS instruction fetches 8 rows x 128 bytes, whole
// cache lines (16 rows x 64 bytes, half lines, measured at half the rate).  A wave waits for its
// own loads of the stage about to be read and the barrier publishes everyone's.  The whole K loop
// is unrolled at compile time, so every step is straight-line code with its stage, wait count and
// fold known.  At the end of each K slice a wave adds its slice sums to its total while the other
// wave on its SIMD keeps the matrix pipe busy.
constexpr int kWM = 256;       // tile rows (tokens)
constexpr int kWN = 128;       // tile columns
constexpr int kWK = 64;        // K per stage
constexpr int kWStages = 3;
constexpr int kWWaves = 8;
constexpr int kWThreads = 64 * kWWaves;
constexpr int kWStageA = kWM * kWK * 2;
constexpr int kWStageW = kWN * kWK * 2;
constexpr int kWLoads = (kWM + kWN) / 8 / kWWaves;  // DMA instructions per wave and stage

// Byte offset in a stage of the 16-byte chunk c (k 8c .. 8c+7) of row r: rows of 128 bytes, the
// chunks of a row permuted by (r/2) % 8, so that one chunk of 16 consecutive rows (one
// ds_read_b128 phase) covers every bank once.
__device__ __forceinline__ int slot128(int r, int c) { return 16 * (8 * r + (c ^ ((r >> 1) & 7))); }

// Direct-to-LDS copies of an R-row block of a bf16 matrix with leading dimension ld, 64 columns
// at a time.  Instruction i (R/8 in all, spread over the waves) fills bytes 1024 i .. 1024 i + 1023
// of a stage = rows 8 i .. 8 i + 7; lane l takes the chunk of row 8 i + l / 8 stored in slot l % 8.
// They are buffer loads: the block's base address sits in a resource descriptor in scalar
// registers, the column offset of the step in a scalar offset, and each lane keeps one 32-bit byte
// offset per instruction for the whole K loop.  Rows at or past rows_valid re-read the last valid
// row.
constexpr int kBufferWord3 = 0x00020000;  // raw buffer descriptor word 3 on gfx9-family parts

template <int R>
struct RowDma {
  static constexpr int kPerWave = R / 8 / kWWaves;
  static_assert(kPerWave * 8 * kWWaves == R, "whole instructions per wave");
  __amdgpu_buffer_rsrc_t rsrc;
  uint32_t off[kPerWave];
  __device__ __forceinline__ RowDma(const uint16_t* block, int ld, int rows_valid, int wave, int lane) {
    rsrc = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(block), (short)0, rows_valid * ld * 2,
                                             kBufferWord3);
#pragma unroll
    for (int j = 0; j < kPerWave; ++j) {
      const int i = kPerWave * wave + j;
      const int r = 8 * i + (lane >> 3);
      const int c = (lane & 7) ^ ((r >> 1) & 7);
      const int rs = r < rows_valid ? r : rows_valid - 1;
      off[j] = (uint32_t)(rs * ld + 8 * c) * 2u;
    }
  }
  __device__ __forceinline__ void issue(int k0, uint8_t* lds, int wave) const {
#pragma unroll
    for (int j = 0; j < kPerWave; ++j)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (lds_void_t*)(lds + (kPerWave * wave + j) * 1024), 16, off[j],
                                               k0 * 2, 0, 0);
  }
};

// Scheduling groups for one k-step: after each of the M MFMAs, one of the V direct-to-LDS loads
// or, once those are out, up to two of the D LDS reads.
template <int M, int V, int D>
__device__ __forceinline__ void interleave() {
  if constexpr (M > 0) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
    if constexpr (V > 0) {
      __builtin_amdgcn_sched_group_barrier(0x010, 1, 0);  // VMEM
      interleave<M - 1, V - 1, D>();
    } else if constexpr (D > 0) {
      constexpr int d = D < 2 ? D : 2;
      __builtin_amdgcn_sched_group_barrier(0x100, d, 0);  // LDS read
      interleave<M - 1, 0, D - d>();
    } else {
      interleave<M - 1, 0, 0>();
    }
  } else {
    if constexpr (V > 0) __builtin_amdgcn_sched_group_barrier(0x010, V, 0);
    if constexpr (D > 0) __builtin_amdgcn_sched_group_barrier(0x100, D, 0);
  }
}

// f(integral_constant<int, I>) for I = 0 .. N-1, in order, at compile time.
template <class F, int... I>
__device__ __forceinline__ void for_each_index(F&& f, std::integer_sequence<int, I...>) {
  (f(std::integral_constant<int, I>{}), ...);
}

// s_waitcnt immediate: vmcnt(n) and lgkmcnt(0), expcnt left at its maximum.
constexpr int wait_vm_lgkm0(int n) { return (n & 15) | (7 << 4) | ((n >> 4) << 14); }

template <int kK>
__global__ __launch_bounds__(kWThreads, 1) void proj_wide_kernel(const uint16_t* __restrict__ a, int lda, int rows,
                                                                const uint16_t* __restrict__ w, int n_tm,
                                                                int n_tn, int rows_major, OutMap out,
                                                                int tail_base, int tail_blocks, int tail_rows) {
  // One array per stage, so that the compiler can see which stage each load and read touches.
  __shared__ __attribute__((aligned(1024))) uint8_t s_a0[kWStageA];
  __shared__ __attribute__((aligned(1024))) uint8_t s_a1[kWStageA];
  __shared__ __attribute__((aligned(1024))) uint8_t s_a2[kWStageA];
  __shared__ __attribute__((aligned(1024))) uint8_t s_w0[kWStageW];
  __shared__ __attribute__((aligned(1024))) uint8_t s_w1[kWStageW];
  __shared__ __attribute__((aligned(1024))) uint8_t s_w2[kWStageW];
  constexpr int nk = kK / kWK;
  constexpr int kStepsPerSlice = kKSlice / kWK;
  static_assert(kKSlice % kWK == 0 && nk % kStepsPerSlice == 0 && nk >= kWStages, "whole slices of whole steps");
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;

  static_assert(kWStageA >= 2 * kSkinnyStage && kWStageW >= kSkinnyStage && kWThreads == 64 * kSkinnyWaves &&
                    kWStageA >= kSliceGroup * 16 * 64 * 4,
                "the tail blocks fit the stage arrays");
  const int bid = blockIdx.x;
  if (bid >= tail_base && bid < tail_base + tail_blocks) {
    tail_block<false>(a, lda, rows, tail_rows, w, kK, n_tn * kWN, out, bid - tail_base, s_a0, s_a1, s_a2, s_w0,
                       s_w1);
    return;
  }
  int tm, tn;
  tile_of(bid < tail_base ? bid : bid - tail_blocks, rows, kWM, n_tm, n_tn, rows_major, tm, tn);
  if (tm >= n_tm || tn >= n_tn) return;  // whole workgroup, before any barrier
  const int row0 = tm * kWM;
  const int col0 = tn * kWN;
  const int rows_valid = min(kWM, rows - row0);

  const int wm = wave >> 1, wn = wave & 1;
  const int n = lane & 31, hk = lane >> 5;
  // ds_read_b128 bases of k-step ks: row 64 wm + n (A) or 64 wn + n (W), chunk 2 ks + hk.
  int abase[4], wbase[4];
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) {
    abase[ks] = slot128(64 * wm + n, 2 * ks + hk);
    wbase[ks] = slot128(64 * wn + n, 2 * ks + hk);
  }

  floatx16_t acc[2][2], sum[2][2];  // the current K slice; the slices before it
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = sum[i][j][v] = 0.f;

  uint8_t* const sa[kWStages] = {s_a0, s_a1, s_a2};
  uint8_t* const sw[kWStages] = {s_w0, s_w1, s_w2};
  const RowDma<kWN> dma_w(w + (size_t)col0 * kK, kK, kWN, wave, lane);
  const RowDma<kWM> dma_a(a + (size_t)row0 * lda, lda, rows_valid, wave, lane);
  auto issue = [&](int kt) __attribute__((always_inline)) {
    dma_w.issue(kt * kWK, sw[kt % kWStages], wave);
    dma_a.issue(kt * kWK, sa[kt % kWStages], wave);
  };
  // Step KT on stage KT % 3: wait for this wave's DMA of it (the loads of step KT + 1 may stay in
  // flight) and for its reads of the stage before; the barrier publishes the stage and frees the
  // one step KT - 1 read, which the DMA of step KT + 2 then refills.  Within the step the operands
  // of k-step ks + 1 are read while the MFMAs of k-step ks run.  kLive: the wave's first kLive
  // 32-row blocks hold tokens (2 but in a partly filled tile), the others get no MFMAs.
  auto run = [&](auto live) __attribute__((always_inline)) {
    constexpr int kLive = decltype(live)::value;
    for_each_index(
        [&](auto kt_) __attribute__((always_inline)) {
          constexpr int KT = decltype(kt_)::value;
          constexpr bool kIssue = KT + 2 < nk;
          __builtin_amdgcn_sched_barrier(0);
          __builtin_amdgcn_s_waitcnt(wait_vm_lgkm0(KT + 1 < nk ? kWLoads : 0));
          asm volatile("" ::: "memory");
          __builtin_amdgcn_s_barrier();
          asm volatile("" ::: "memory");
          if constexpr (kIssue) issue(KT + 2);
          const uint8_t* cur_a = sa[KT % kWStages];
          const uint8_t* cur_w = sw[KT % kWStages];
          bf16x8_t af[2][2], wf[2][2];
          auto read = [&](int ks, bf16x8_t(&a_f)[2], bf16x8_t(&w_f)[2]) __attribute__((always_inline)) {
#pragma unroll
            for (int i = 0; i < kLive; ++i)
              a_f[i] = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const uint4*>(cur_a + abase[ks] + 4096 * i));
#pragma unroll
            for (int j = 0; j < 2; ++j)
              w_f[j] = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const uint4*>(cur_w + wbase[ks] + 4096 * j));
          };
          if constexpr (kLive > 0) read(0, af[0], wf[0]);
          __builtin_amdgcn_sched_barrier(0);
#pragma unroll
          for (int ks = 0; ks < 4; ++ks) {
            if constexpr (kLive > 0)
              if (ks < 3) read(ks + 1, af[(ks + 1) & 1], wf[(ks + 1) & 1]);
#pragma unroll
            for (int i = 0; i < kLive; ++i)
#pragma unroll
              for (int j = 0; j < 2; ++j)
                acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[ks & 1][i], wf[ks & 1][j], acc[i][j], 0, 0, 0);
            // the first k-step also carries the DMA instructions
            if (ks == 0)
              interleave<2 * kLive, (kIssue ? kWLoads : 0), (kLive > 0 ? kLive + 2 : 0)>();
            else if (ks < 3)
              interleave<2 * kLive, 0, kLive + 2>();
            else
              interleave<2 * kLive, 0, 0>();
          }
          if constexpr ((KT + 1) % kStepsPerSlice == 0) {
#pragma unroll
            for (int i = 0; i < kLive; ++i)
#pragma unroll
              for (int j = 0; j < 2; ++j)
#pragma unroll
                for (int v = 0; v < 16; ++v) {
                  sum[i][j][v] += acc[i][j][v];
                  acc[i][j][v] = 0.f;
                }
          }
        },
        std::make_integer_sequence<int, nk>{});
  };

  issue(0);
  issue(1);
  const int live_blocks = min(2, max(0, (rows_valid - 64 * wm + 31) / 32));  // uniform per wave
  switch (live_blocks) {
    case 2: run(std::integral_constant<int, 2>{}); break;
    case 1: run(std::integral_constant<int, 1>{}); break;
    default: run(std::integral_constant<int, 0>{}); break;
  }

  // Epilogue: accumulator element v of block (i, j) is C[row0 + 64wm + 32i + 8(v/4) + 4hk + v%4]
  // [col0 + 64wn + 32j + n]; the tile lies in one region of the output map.
  const int reg = (col0 >= out.lo[2]) ? 2 : (col0 >= out.lo[1]) ? 1 : 0;
  uint16_t* dst = out.dst[reg];
  const int ld = out.ld[reg];
  const int cbase = col0 - out.lo[reg] + 64 * wn + n;
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int r = 64 * wm + 32 * i + 8 * (v >> 2) + 4 * hk + (v & 3);
      if (r < rows_valid) {
        uint16_t* drow = dst + (size_t)(row0 + r) * ld + cbase;
#pragma unroll
        for (int j = 0; j < 2; ++j) drow[32 * j] = (uint16_t)pack_bf16x2(sum[i][j][v], 0.f);
      }
    }
}

// Many tokens, float32 A (the output map): a 128 x 128 tile per workgroup of 8 waves, two per
// SIMD, with K split between them: waves 0-3 take the first 1024 inputs and waves 4-7 the last
// 1024, each wave a 64 x 64 block (wave w: rows 64 ((w % 4) / 2), columns 64 (w % 2)) as 2 x 2 MFMA
// blocks.  The two halves' totals meet in LDS at the end.  Against a whole-K tile of 4 waves this
// doubles the waves per CU (the 264 tiles of a 4127-token call give one workgroup per CU) without
// more staged bytes per flop.  K advances 32 per half at a time through a ring of three 48 KiB
// stages, the DMA two stages ahead: per half, the float32 A block (128 rows of 128 bytes, whole
// cache lines) and the W block (128 rows of 64 bytes).  A stays float32 in LDS; each MFMA operand
// is read as two 16-byte chunks and rounded to bf16 in registers.
constexpr int kOM = 128;       // tile rows (tokens)
constexpr int kON = 128;       // tile columns
constexpr int kOK = 32;        // K per stage and half
constexpr int kOStages = 3;
constexpr int kOWaves = 8;
constexpr int kOThreads = 64 * kOWaves;
constexpr int kOHalf = kOM * kOK * 4;        // float32 A block of one half and stage: 16 KiB
constexpr int kOHalfW = kON * kOK * 2;       // W block of one half and stage: 8 KiB
constexpr int kOLoadsA = 2 * kOM / 8 / kOWaves;   // A: 8 rows per instruction, both halves
constexpr int kOLoadsW = 2 * kON / 16 / kOWaves;  // W: 16 rows per instruction, both halves
constexpr int kOLoads = kOLoadsA + kOLoadsW;

// Byte offset of 16-byte chunk c of row r in a block with 64-byte rows: chunks permuted by
// (r/4) % 4, so that one chunk of 16 consecutive rows covers every bank once.
__device__ __forceinline__ int slot64(int r, int c) { return 16 * (4 * r + (c ^ ((r >> 2) & 3))); }

template <int kK>
__global__ __launch_bounds__(kOThreads, 1) void proj_ksplit_kernel(const float* __restrict__ a, int lda, int rows,
                                                                  const uint16_t* __restrict__ w, int n_tm,
                                                                  int n_tn, int rows_major, OutMap out,
                                                                  int tail_base, int tail_blocks, int tail_rows) {
  __shared__ __attribute__((aligned(1024))) uint8_t s_a0[2 * kOHalf];
  __shared__ __attribute__((aligned(1024))) uint8_t s_a1[2 * kOHalf];
  __shared__ __attribute__((aligned(1024))) uint8_t s_a2[2 * kOHalf];
  __shared__ __attribute__((aligned(1024))) uint8_t s_w0[2 * kOHalfW];
  __shared__ __attribute__((aligned(1024))) uint8_t s_w1[2 * kOHalfW];
  __shared__ __attribute__((aligned(1024))) uint8_t s_w2[2 * kOHalfW];
  constexpr int kHalfK = kK / 2;
  constexpr int nk = kHalfK / kOK;
  constexpr int kStepsPerSlice = kKSlice / kOK;
  static_assert(kHalfK == kSliceGroup * kKSlice, "each half is one group of K slices");
  static_assert(nk % kStepsPerSlice == 0 && nk >= kOStages, "whole slices of whole steps");
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;

  static_assert(2 * kOHalf >= 2 * kSkinnyStage && 2 * kOHalfW >= kSkinnyStage && kOThreads == 64 * kSkinnyWaves &&
                    2 * kOHalf >= kSliceGroup * 16 * 64 * 4,
                "the tail blocks fit the stage arrays");
  const int bid = blockIdx.x;
  if (bid >= tail_base && bid < tail_base + tail_blocks) {
    tail_block<true>(a, lda, rows, tail_rows, w, kK, n_tn * kON, out, bid - tail_base, s_a0, s_a1, s_a2, s_w0,
                       s_w1);
    return;
  }
  int tm, tn;
  tile_of(bid < tail_base ? bid : bid - tail_blocks, rows, kOM, n_tm, n_tn, rows_major, tm, tn);
  if (tm >= n_tm || tn >= n_tn) return;  // whole workgroup, before any barrier
  const int row0 = tm * kOM;
  const int col0 = tn * kON;
  const int rows_valid = min(kOM, rows - row0);

  const int half = wave >> 2;
  const int wm = (wave >> 1) & 1, wn = wave & 1;
  const int n = lane & 31, hk = lane >> 5;
  // LDS bases of k-step ks: A row 64 wm + n, float chunks 4 ks + 2 hk and + 1 (4 floats each);
  // W row 64 wn + n, chunk 2 ks + hk; each within this half's block.
  int abase[2][2], wbase[2];
#pragma unroll
  for (int ks = 0; ks < 2; ++ks) {
#pragma unroll
    for (int e = 0; e < 2; ++e) abase[ks][e] = half * kOHalf + slot128(64 * wm + n, 4 * ks + 2 * hk + e);
    wbase[ks] = half * kOHalfW + slot64(64 * wn + n, 2 * ks + hk);
  }

  floatx16_t acc[2][2], sum[2][2];  // the current K slice; the slices before it (this half)
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = sum[i][j][v] = 0.f;

  // DMA of one stage: buffer loads with per-lane byte offsets fixed for the whole K loop and the
  // step's column in the scalar offset.  A instruction i: half i / 16, rows 8 (i % 16) + lane / 8;
  // W instruction i: half i / 8, rows 16 (i % 8) + lane / 4.  Rows past rows_valid re-read the
  // last valid row.
  const __amdgpu_buffer_rsrc_t rsrc_a = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<float*>(a + (size_t)row0 * lda), (short)0, rows_valid * lda * 4, kBufferWord3);
  const __amdgpu_buffer_rsrc_t rsrc_w = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t*>(w + (size_t)col0 * kK), (short)0, kON * kK * 2, kBufferWord3);
  uint32_t off_a[kOLoadsA], off_w[kOLoadsW];
#pragma unroll
  for (int j = 0; j < kOLoadsA; ++j) {
    const int i = kOLoadsA * wave + j;
    const int r = 8 * (i % 16) + (lane >> 3);
    const int c = (lane & 7) ^ ((r >> 1) & 7);
    const int rs = r < rows_valid ? r : rows_valid - 1;
    off_a[j] = (uint32_t)(rs * lda + (i / 16) * kHalfK + 4 * c) * 4u;
  }
#pragma unroll
  for (int j = 0; j < kOLoadsW; ++j) {
    const int i = kOLoadsW * wave + j;
    const int r = 16 * (i % 8) + (lane >> 2);
    const int c = (lane & 3) ^ ((r >> 2) & 3);
    off_w[j] = (uint32_t)(r * kK + (i / 8) * kHalfK + 8 * c) * 2u;
  }
  uint8_t* const sa[kOStages] = {s_a0, s_a1, s_a2};
  uint8_t* const sw[kOStages] = {s_w0, s_w1, s_w2};
  auto issue = [&](int kt) __attribute__((always_inline)) {
#pragma unroll
    for (int j = 0; j < kOLoadsA; ++j)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc_a, (lds_void_t*)(sa[kt % kOStages] + (kOLoadsA * wave + j) * 1024),
                                               16, off_a[j], kt * kOK * 4, 0, 0);
#pragma unroll
    for (int j = 0; j < kOLoadsW; ++j)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc_w, (lds_void_t*)(sw[kt % kOStages] + (kOLoadsW * wave + j) * 1024),
                                               16, off_w[j], kt * kOK * 2, 0, 0);
  };
  // Step KT on stage KT % 3, as in proj_wide_kernel; kLive: the wave's first kLive 32-row blocks
  // hold tokens (2 but in a partly filled tile).
  auto run = [&](auto live) __attribute__((always_inline)) {
    constexpr int kLive = decltype(live)::value;
    for_each_index(
        [&](auto kt_) __attribute__((always_inline)) {
          constexpr int KT = decltype(kt_)::value;
          constexpr bool kIssue = KT + 2 < nk;
          __builtin_amdgcn_sched_barrier(0);
          __builtin_amdgcn_s_waitcnt(wait_vm_lgkm0(KT + 1 < nk ? kOLoads : 0));
          asm volatile("" ::: "memory");
          __builtin_amdgcn_s_barrier();
          asm volatile("" ::: "memory");
          if constexpr (kIssue) issue(KT + 2);
          const uint8_t* cur_a = sa[KT % kOStages];
          const uint8_t* cur_w = sw[KT % kOStages];
          bf16x8_t af[2][2], wf[2][2];
          auto read = [&](int ks, bf16x8_t(&a_f)[2], bf16x8_t(&w_f)[2]) __attribute__((always_inline)) {
#pragma unroll
            for (int i = 0; i < kLive; ++i) {
              const float4 lo = *reinterpret_cast<const float4*>(cur_a + abase[ks][0] + 4096 * i);
              const float4 hi = *reinterpret_cast<const float4*>(cur_a + abase[ks][1] + 4096 * i);
              a_f[i] = __builtin_bit_cast(bf16x8_t, make_uint4(pack_bf16x2(lo.x, lo.y), pack_bf16x2(lo.z, lo.w),
                                                               pack_bf16x2(hi.x, hi.y), pack_bf16x2(hi.z, hi.w)));
            }
#pragma unroll
            for (int j = 0; j < 2; ++j)
              w_f[j] = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const uint4*>(cur_w + wbase[ks] + 2048 * j));
          };
          if constexpr (kLive > 0) read(0, af[0], wf[0]);
          __builtin_amdgcn_sched_barrier(0);
#pragma unroll
          for (int ks = 0; ks < 2; ++ks) {
            if constexpr (kLive > 0)
              if (ks < 1) read(ks + 1, af[1], wf[1]);
#pragma unroll
            for (int i = 0; i < kLive; ++i)
#pragma unroll
              for (int j = 0; j < 2; ++j)
                acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[ks][i], wf[ks][j], acc[i][j], 0, 0, 0);
            if (ks == 0)
              interleave<2 * kLive, (kIssue ? kOLoads : 0), (kLive > 0 ? 2 * kLive + 2 : 0)>();
            else
              interleave<2 * kLive, 0, 0>();
          }
          if constexpr ((KT + 1) % kStepsPerSlice == 0) {
#pragma unroll
            for (int i = 0; i < kLive; ++i)
#pragma unroll
              for (int j = 0; j < 2; ++j)
#pragma unroll
                for (int v = 0; v < 16; ++v) {
                  sum[i][j][v] += acc[i][j][v];
                  acc[i][j][v] = 0.f;
                }
          }
        },
        std::make_integer_sequence<int, nk>{});
  };

  issue(0);
  issue(1);
  const int live_blocks = min(2, max(0, (rows_valid - 64 * wm + 31) / 32));  // uniform per wave
  switch (live_blocks) {
    case 2: run(std::integral_constant<int, 2>{}); break;
    case 1: run(std::integral_constant<int, 1>{}); break;
    default: run(std::integral_constant<int, 0>{}); break;
  }

  // The second half's totals go through LDS to the waves of the first half, which add them to
  // their own: (0 + first) + second, the order proj_skinny_kernel uses.
  __syncthreads();  // every wave is done with the stages
  // Row block i of the second half's totals goes to stage i's A array (32 KiB each):
  // [wave of the half][column block][accumulator element][lane].
  float* const s_sum[2] = {reinterpret_cast<float*>(s_a0), reinterpret_cast<float*>(s_a1)};
  const int wq = wave & 3;
  if (half == 1) {
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int v = 0; v < 16; ++v) s_sum[i][((wq * 2 + j) * 16 + v) * 64 + lane] = sum[i][j][v];
  }
  __syncthreads();
  if (half == 1) return;
  uint16_t* dst = out.dst[0];
  const int ld = out.ld[0];
  const int cbase = col0 + 64 * wn + n;
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int r = 64 * wm + 32 * i + 8 * (v >> 2) + 4 * hk + (v & 3);
      if (r < rows_valid) {
        uint16_t* drow = dst + (size_t)(row0 + r) * ld + cbase;
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          const float total = (0.f + sum[i][j][v]) + s_sum[i][((wq * 2 + j) * 16 + v) * 64 + lane];
          drow[32 * j] = (uint16_t)pack_bf16x2(total, 0.f);
        }
      }
    }
}

// Calls of at most 64 tokens.  Workgroup (column block x, row block y) = 32 columns of W against
// kRB tokens (32 for QKV, 8 for the output map), with one wave per K slice (8 for QKV, 16 for the
// output map), so that all of the block's weights are in flight at once: a call of one token has
// only 128 (QKV) or 32 (output map) workgroups, and its time is each CU's fetch of its share of W.
// Wave w copies its 32 x 128 piece of W into its own 8 KiB of LDS with the direct-to-LDS
// instructions of dma_piece32 (whole 128-byte lines per instruction: loading the MFMA fragments
// straight into registers touches 32 partial lines per instruction and measured slower), while the
// workgroup stages its valid rows of A once, as bf16, for all of K (the output map's float32 rows
// go through registers and are rounded on the way).  Row r's 16-byte chunks are permuted within
// groups of 16 (chunk c at (c & ~15) | ((c ^ r) & 15)), so that 16 lanes reading one chunk of 16
// different rows hit distinct banks; fragment rows past the call's end read its last row.  LDS:
// 64 KiB of W and 64 KiB of A for QKV; 128 KiB and 32 KiB for the output map.  The MFMA chain of
// each slice and the order in which the slice sums are added are those of skinny_block, so the
// bits are those of the tiled kernels.
template <int kK>
__device__ __forceinline__ int a_slot_bytes(int r, int c) {
  return 16 * (r * (kK / 8) + ((c & ~15) | ((c ^ r) & 15)));
}

template <bool kAF32, int kK, int kRB>
__global__ __launch_bounds__(64 * (kK / kKSlice)) void proj_skinny_kernel(
    const void* __restrict__ a_ptr, int lda, int rows, const uint16_t* __restrict__ w, OutMap out) {
  constexpr int kWaves = kK / kKSlice;
  constexpr int kChunks = kK / 8;  // 16-byte bf16 chunks per staged row of A
  constexpr int kSteps = kKSlice / 16;
  constexpr int kWBytes = kWaves * 8192;
  static_assert(kK % (kSliceGroup * kKSlice) == 0, "whole groups of slices");
  static_assert(kRB <= 32 && (kRB * kChunks) % 64 == 0, "A's stage is whole 1 KiB direct-to-LDS blocks");
  // W pieces (later the slice sums: 4 KiB per slice), then A
  __shared__ __attribute__((aligned(1024))) uint8_t s_mem[kWBytes + kRB * kK * 2];
  uint8_t* const s_a = s_mem + kWBytes;
  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int n = lane & 31, hk = lane >> 5;
  const int col0 = 32 * blockIdx.x, row0 = kRB * blockIdx.y;
  const int rows_valid = min(kRB, rows - row0);
  const int k0 = wave * kKSlice;
  uint8_t* const w_lds = s_mem + wave * 8192;
  dma_piece32(w, kK, col0, 32, k0, w_lds, lane);

  if constexpr (kAF32) {
    for (int i = tid; i < rows_valid * kChunks; i += 64 * kWaves) {
      const int r = i / kChunks, c = i % kChunks;
      const float4* src = reinterpret_cast<const float4*>(static_cast<const float*>(a_ptr) +
                                                          (size_t)(row0 + r) * lda + 8 * c);
      const float4 lo = src[0], hi = src[1];
      *reinterpret_cast<uint4*>(s_a + a_slot_bytes<kK>(r, c)) =
          make_uint4(pack_bf16x2(lo.x, lo.y), pack_bf16x2(lo.z, lo.w), pack_bf16x2(hi.x, hi.y),
                     pack_bf16x2(hi.z, hi.w));
    }
  } else {
    // Instruction i fills the 64 slots 64 i .. 64 i + 63 of the permuted layout; slot p holds row
    // p / kChunks, chunk (cp & ~15) | ((cp ^ r) & 15) with cp = p % kChunks (the permutation is its
    // own inverse).  Slots of rows past the call's end take its last row and are never read.
    const int n_instr = (rows_valid * kChunks + 63) / 64;
    for (int i = wave; i < n_instr; i += kWaves) {
      const int p = 64 * i + lane;
      const int r = p / kChunks, cp = p % kChunks;
      const int c = (cp & ~15) | ((cp ^ r) & 15);
      const int rs = r < rows_valid ? r : rows_valid - 1;
      __builtin_amdgcn_global_load_lds(
          (global_cvoid_t*)(static_cast<const uint16_t*>(a_ptr) + (size_t)(row0 + rs) * lda + 8 * c),
          (lds_void_t*)(s_a + 1024 * i), 16, 0, 0);
    }
  }
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): this wave's direct-to-LDS copies have landed
  __syncthreads();

  floatx16_t acc;
#pragma unroll
  for (int v = 0; v < 16; ++v) acc[v] = 0.f;
  const int ra = min(n, rows_valid - 1);
#pragma unroll
  for (int s = 0; s < kSteps; ++s) {
    const bf16x8_t af = __builtin_bit_cast(
        bf16x8_t, *reinterpret_cast<const uint4*>(s_a + a_slot_bytes<kK>(ra, (k0 >> 3) + 2 * s + hk)));
    const bf16x8_t wf =
        __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const uint4*>(w_lds + slot32_bytes(n, 2 * s + hk)));
    acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af, wf, acc, 0, 0, 0);
  }
  __syncthreads();  // every wave is done with its piece of W; that LDS now takes the slice sums
  float* const s_part = reinterpret_cast<float*>(s_mem);  // slice w at [w][accumulator element][lane]
#pragma unroll
  for (int v = 0; v < 16; ++v) s_part[(wave * 16 + v) * 64 + lane] = acc[v];
  __syncthreads();

  // Element e = (accumulator element v, lane l): C[row0 + 8(v/4) + 4(l/32) + v%4][col0 + l%32].
  const int reg = (col0 >= out.lo[2]) ? 2 : (col0 >= out.lo[1]) ? 1 : 0;
  uint16_t* dst = out.dst[reg];
  const int ld = out.ld[reg];
  for (int e = tid; e < 16 * 64; e += 64 * kWaves) {
    const int v = e >> 6, l = e & 63;
    const int rr = 8 * (v >> 2) + 4 * (l >> 5) + (v & 3);
    if (rr >= rows_valid) continue;
    float total = 0.f;
#pragma unroll
    for (int g0 = 0; g0 < kWaves; g0 += kSliceGroup) {
      float group = 0.f;
#pragma unroll
      for (int sl = g0; sl < g0 + kSliceGroup; ++sl) group += s_part[(sl * 16 + v) * 64 + l];
      total += group;
    }
    dst[(size_t)(row0 + rr) * ld + col0 - out.lo[reg] + (l & 31)] = (uint16_t)pack_bf16x2(total, 0.f);
  }
}

constexpr int kQkvSkinnyRows = 32;  // tokens per few-token QKV workgroup
constexpr int kOSkinnyRows = 8;     // tokens per few-token output-map workgroup (LDS: 128 + 32 KiB)

// Workgroups launched for the tiles of `rows` rows x n_tn tile columns.  Rows owned by XCD: whole
// tile rows padded to groups of 8, plus a partly filled last row dealt out over the XCDs by column.
int grid_tiles(int rows, int n_tn, int rows_major, int tm_rows) {
  const int n_tm = (rows + tm_rows - 1) / tm_rows;
  if (!rows_major || rows_major == kSplit2D) return n_tm * n_tn;
  const int n_full = rows / tm_rows;
  const int tail = n_tm > n_full ? (n_tn + 7) / 8 : 0;
  return 8 * (((n_full + 7) / 8) * n_tn + tail);
}

// The operand split (see Placement) that reads fewer bytes.
int rows_major_split(int rows, size_t a_row_bytes, size_t w_bytes) {
  return (size_t)rows * a_row_bytes >= w_bytes;
}

}  // namespace

// A call's rows: whole tiles go to the tiled kernel; a last partial tile of at most kSkinnyRows
// rows goes to workgroups of the tiled launch that run the few-token algorithm (both give a token
// the same bits), since as a tile of its own it would take a whole extra round of the grid for a
// few rows.
struct RowSplit {
  int tiled, tail;
};
RowSplit split_rows(int n_tok, int tile_rows) {
  const int rem = n_tok % tile_rows;
  if (n_tok > tile_rows && rem > 0 && rem <= kSkinnyRows) return {n_tok - rem, rem};
  return {n_tok, 0};
}


hipError_t launch_qkv_proj(const uint16_t* x, const uint16_t* w_qkv, int n_tok, uint16_t* q,
                           uint16_t* k, uint16_t* v, hipStream_t stream) {
  constexpr int kN = (kQHeads + 2 * kKvHeads) * kHeadDim;
  OutMap om;
  om.dst[0] = q;
  om.dst[1] = k;
  om.dst[2] = v;
  om.ld[0] = kQHeads * kHeadDim;
  om.ld[1] = om.ld[2] = kKvHeads * kHeadDim;
  om.lo[0] = 0;
  om.lo[1] = kQHeads * kHeadDim;
  om.lo[2] = (kQHeads + kKvHeads) * kHeadDim;
  const RowSplit rs = n_tok <= kSkinnyRows ? RowSplit{0, n_tok} : split_rows(n_tok, kWM);
  if (rs.tiled > 0) {
    const int n_wm = (rs.tiled + kWM - 1) / kWM;
    const int n_wn = kN / kWN;
    const int rows_major = n_wm % 4 == 0 && n_wn % 2 == 0
                               ? kSplit2D
                               : rows_major_split(rs.tiled, kHidden * 2, (size_t)kN * kHidden * 2);
    const int tail_blocks = (kN / 32) * ((rs.tail + 31) / 32);
    const int tiles = grid_tiles(rs.tiled, n_wn, rows_major, kWM);
    proj_wide_kernel<kHidden><<<dim3(tail_blocks + tiles), dim3(kWThreads), 0, stream>>>(
        x, kHidden, rs.tiled, w_qkv, n_wm, n_wn, rows_major, om, tiles > device_cus() ? 0 : tiles, tail_blocks,
        rs.tail);
  } else {
    proj_skinny_kernel<false, kHidden, kQkvSkinnyRows>
        <<<dim3(kN / 32, (rs.tail + kQkvSkinnyRows - 1) / kQkvSkinnyRows), dim3(64 * (kHidden / kKSlice)), 0,
           stream>>>(x, kHidden, rs.tail, w_qkv, om);
  }
  return hipGetLastError();
}

hipError_t launch_o_proj(const float* attn, const uint16_t* w_o, int n_tok, uint16_t* out,
                         hipStream_t stream) {
  constexpr int kK = kQHeads * kHeadDim;
  OutMap om;
  for (int r = 0; r < 3; ++r) {
    om.dst[r] = out;
    om.ld[r] = kHidden;
    om.lo[r] = 0;
  }
  const RowSplit rs = n_tok <= kSkinnyRows ? RowSplit{0, n_tok} : split_rows(n_tok, kOM);
  if (rs.tiled > 0) {
    const int n_tm = (rs.tiled + kOM - 1) / kOM;
    const int n_tn = kHidden / kON;
    const int rows_major = rows_major_split(rs.tiled, kK * 4, (size_t)kHidden * kK * 2);
    const int tail_blocks = (kHidden / 32) * ((rs.tail + 31) / 32);
    const int tiles = grid_tiles(rs.tiled, n_tn, rows_major, kOM);
    proj_ksplit_kernel<kK><<<dim3(tail_blocks + tiles), dim3(kOThreads), 0, stream>>>(
        attn, kK, rs.tiled, w_o, n_tm, n_tn, rows_major, om, tiles > device_cus() ? 0 : tiles, tail_blocks,
        rs.tail);
  } else {
    proj_skinny_kernel<true, kK, kOSkinnyRows>
        <<<dim3(kHidden / 32, (rs.tail + kOSkinnyRows - 1) / kOSkinnyRows), dim3(64 * (kK / kKSlice)), 0, stream>>>(
            attn, kK, rs.tail, w_o, om);
  }
  return hipGetLastError();
}

}  // namespace mtd
