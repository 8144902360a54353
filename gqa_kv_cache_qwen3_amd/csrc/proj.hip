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
// Work split.  One workgroup (4 wavefronts) owns a 128 x 128 tile of C; wave w computes the 64 x
// 64 quarter (w / 2, w % 2) as 2 x 2 blocks of v_mfma_f32_32x32x16_bf16 with fp32 accumulators.
// K advances 64 at a time through two LDS stages: right after the barrier that publishes stage
// s, the loads of the next 64-wide slice into stage s^1 are issued, so they travel while stage s
// is multiplied.  Two workgroups fit per CU (64 KiB of LDS each), so the matrix pipe of a SIMD
// always has a second wave to switch to at a barrier.
//
// Staging.  A 128 x 64 bf16 slice is two column groups of 64 bytes (k 32j .. 32j+31) of 128 rows;
// the 16-byte slot of (row r, chunk c) is 512 (c/4) + 4 r + ((c%4) ^ ((r/4)%4)).  bf16 slices
// arrive by 16-byte direct-to-LDS loads (global_load_lds_dwordx4: no registers, no VALU), each
// instruction fetching 16 rows x 64 contiguous bytes; the float32 O slice comes through registers
// (16 lanes per 256-byte row, coalesced), is rounded to bf16 and written with ds_write_b64 into
// the same layout.  MFMA operands are ds_read_b128 of one row's 16-byte chunk: A rows for the A
// operand and W rows for the B operand, both free of bank conflicts under the XOR swizzle.
//
// Placement.  Workgroup i runs on XCD i % 8.  The tiles are numbered so that each XCD takes one
// contiguous eighth of them, either whole rows of tiles (every XCD then reads W whole and an
// eighth of A) or whole columns (an eighth of W, all of A); the host picks the split that reads
// fewer bytes, so the replicated operand is the smaller one and stays in the XCD's L2.
#include "device_util.h"
#include "mtd_internal.h"

namespace mtd {
namespace {

constexpr int kTM = 128;    // tile rows (tokens)
constexpr int kTN = 128;    // tile columns (output features)
constexpr int kTK = 64;     // K per stage
constexpr int kThreads = 256;
constexpr int kSliceBytes = kTM * kTK * 2;  // 16 KiB per operand per stage

typedef __attribute__((address_space(3))) void lds_void_t;
typedef const __attribute__((address_space(1))) void global_cvoid_t;

// Byte offset in a staged slice of the 16-byte slot (row r, chunk c).
__device__ __forceinline__ int slot_bytes(int r, int c) {
  return 16 * (512 * (c >> 2) + 4 * r + ((c & 3) ^ ((r >> 2) & 3)));
}

// Direct-to-LDS copy of rows row0 .. row0+127, columns k0 .. k0+63 of a bf16 matrix with leading
// dimension ld.  Instruction i (4 per wave) fills slots 64 i .. 64 i + 63: column group i / 8,
// rows 16 (i % 8) + lane / 4.  Rows at or past rows_valid re-read the last valid row.
__device__ __forceinline__ void dma_slice(const uint16_t* __restrict__ m, int ld, int row0,
                                          int rows_valid, int k0, uint8_t* lds, int wave, int lane) {
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int i = 4 * wave + j;
    const int r = 16 * (i & 7) + (lane >> 2);
    const int c = 4 * (i >> 3) + ((lane & 3) ^ ((r >> 2) & 3));
    const int rs = r < rows_valid ? r : rows_valid - 1;
    __builtin_amdgcn_global_load_lds((global_cvoid_t*)(m + (size_t)(row0 + rs) * ld + k0 + 8 * c),
                                     (lds_void_t*)(lds + i * 1024), 16, 0, 0);
  }
}

// float32 A slice through registers: wave w, load j covers rows 32w + 4j + lane/16, floats
// 4 (lane%16) .. +3 of the 64.
struct F32Slice {
  float4 v[8];
};

__device__ __forceinline__ void load_f32_slice(F32Slice& s, const float* __restrict__ a, int ld,
                                               int row0, int rows_valid, int k0, int wave, int lane) {
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int r = 32 * wave + 4 * j + (lane >> 4);
    const int rs = r < rows_valid ? r : rows_valid - 1;
    s.v[j] = *reinterpret_cast<const float4*>(a + (size_t)(row0 + rs) * ld + k0 + 4 * (lane & 15));
  }
}

__device__ __forceinline__ void store_f32_slice(const F32Slice& s, uint8_t* lds, int wave, int lane) {
  const int f = lane & 15;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int r = 32 * wave + 4 * j + (lane >> 4);
    const uint2 packed = make_uint2(pack_bf16x2(s.v[j].x, s.v[j].y), pack_bf16x2(s.v[j].z, s.v[j].w));
    *reinterpret_cast<uint2*>(lds + slot_bytes(r, f >> 1) + 8 * (f & 1)) = packed;
  }
}

// Where the columns of C go: columns [lo_r, lo_{r+1}) of region r land in dst[r] (bf16, leading
// dimension ld[r]) at column n - lo_r.  One region for the output projection, three for QKV.
struct OutMap {
  uint16_t* dst[3];
  int ld[3];
  int lo[3];
};

template <bool kAF32>
__global__ __launch_bounds__(kThreads, 2) void proj_gemm_kernel(const void* __restrict__ a_ptr, int lda,
                                                                int rows, const uint16_t* __restrict__ w,
                                                                int k_dim, int n_tm, int n_tn,
                                                                int rows_major, OutMap out) {
  __shared__ __attribute__((aligned(1024))) uint8_t s_a[2][kSliceBytes];
  __shared__ __attribute__((aligned(1024))) uint8_t s_w[2][kSliceBytes];
  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;

  // Tile of this workgroup: XCD blockIdx.x % 8 takes a contiguous eighth of the tile list.
  const int total = n_tm * n_tn;
  const int id = blockIdx.x;
  const int t = (total % 8 == 0) ? (id % 8) * (total / 8) + id / 8 : id;
  const int tm = rows_major ? t / n_tn : t % n_tm;
  const int tn = rows_major ? t % n_tn : t / n_tm;
  const int row0 = tm * kTM;
  const int col0 = tn * kTN;
  const int rows_valid = min(kTM, rows - row0);

  const int wm = wave >> 1, wn = wave & 1;
  const int n = lane & 31, hk = lane >> 5;
  // ds_read_b128 bases: row 64 wm + n (A) or 64 wn + n (W), chunk 2 ks + hk, for ks even / odd.
  int abase[2], wbase[2];
#pragma unroll
  for (int e = 0; e < 2; ++e) {
    const int sw = ((2 * e + hk) ^ ((n >> 2) & 3)) * 16;
    abase[e] = 64 * (64 * wm + n) + sw;
    wbase[e] = 64 * (64 * wn + n) + sw;
  }

  floatx16_t acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;

  const int nk = k_dim / kTK;
  F32Slice fa;
  auto issue = [&](int kt, int st) {
    dma_slice(w, k_dim, col0, kTN, kt * kTK, s_w[st], wave, lane);
    if constexpr (kAF32)
      load_f32_slice(fa, static_cast<const float*>(a_ptr), lda, row0, rows_valid, kt * kTK, wave, lane);
    else
      dma_slice(static_cast<const uint16_t*>(a_ptr), lda, row0, rows_valid, kt * kTK, s_a[st], wave, lane);
  };

  issue(0, 0);
  if constexpr (kAF32) store_f32_slice(fa, s_a[0], wave, lane);
  for (int kt = 0; kt < nk; ++kt) {
    const int st = kt & 1;
    __syncthreads();  // stage st complete for every wave; stage st^1 no longer read
    if (kt + 1 < nk) issue(kt + 1, st ^ 1);
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      bf16x8_t af[2], wf[2];
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        af[i] = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const uint4*>(
                                                 s_a[st] + abase[ks & 1] + 8192 * (ks >> 1) + 2048 * i));
        wf[i] = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const uint4*>(
                                                 s_w[st] + wbase[ks & 1] + 8192 * (ks >> 1) + 2048 * i));
      }
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], wf[j], acc[i][j], 0, 0, 0);
    }
    if constexpr (kAF32)
      if (kt + 1 < nk) store_f32_slice(fa, s_a[st ^ 1], wave, lane);
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
        for (int j = 0; j < 2; ++j) drow[32 * j] = (uint16_t)pack_bf16x2(acc[i][j][v], 0.f);
      }
    }
}

// The operand split (see Placement) that reads fewer bytes.
int rows_major_split(int rows, size_t a_row_bytes, size_t w_bytes) {
  return (size_t)rows * a_row_bytes >= w_bytes;
}

}  // namespace

hipError_t launch_qkv_proj(const uint16_t* x, const uint16_t* w_qkv, int n_tok, uint16_t* q,
                           uint16_t* k, uint16_t* v, hipStream_t stream) {
  if (n_tok == 0) return hipSuccess;
  constexpr int kN = (kQHeads + 2 * kKvHeads) * kHeadDim;
  const int n_tm = (n_tok + kTM - 1) / kTM;
  const int n_tn = kN / kTN;
  OutMap om;
  om.dst[0] = q;
  om.dst[1] = k;
  om.dst[2] = v;
  om.ld[0] = kQHeads * kHeadDim;
  om.ld[1] = om.ld[2] = kKvHeads * kHeadDim;
  om.lo[0] = 0;
  om.lo[1] = kQHeads * kHeadDim;
  om.lo[2] = (kQHeads + kKvHeads) * kHeadDim;
  const int rows_major = rows_major_split(n_tok, kHidden * 2, (size_t)kN * kHidden * 2);
  proj_gemm_kernel<false><<<dim3(n_tm * n_tn), dim3(kThreads), 0, stream>>>(
      x, kHidden, n_tok, w_qkv, kHidden, n_tm, n_tn, rows_major, om);
  return hipGetLastError();
}

hipError_t launch_o_proj(const float* attn, const uint16_t* w_o, int n_tok, uint16_t* out,
                         hipStream_t stream) {
  if (n_tok == 0) return hipSuccess;
  constexpr int kK = kQHeads * kHeadDim;
  const int n_tm = (n_tok + kTM - 1) / kTM;
  const int n_tn = kHidden / kTN;
  OutMap om;
  for (int r = 0; r < 3; ++r) {
    om.dst[r] = out;
    om.ld[r] = kHidden;
    om.lo[r] = 0;
  }
  const int rows_major = rows_major_split(n_tok, kK * 4, (size_t)kHidden * kK * 2);
  proj_gemm_kernel<true><<<dim3(n_tm * n_tn), dim3(kThreads), 0, stream>>>(
      attn, kK, n_tok, w_o, kK, n_tm, n_tn, rows_major, om);
  return hipGetLastError();
}

}  // namespace mtd
