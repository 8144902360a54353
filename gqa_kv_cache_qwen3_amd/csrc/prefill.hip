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
// Per 64-key tile (one page of the KV head):
//   S^T = K Q^T   v_mfma_f32_32x32x16_bf16, keys as rows: a lane holds one query column and 16
//                 of the 32 keys of each 32-key block, so the softmax over keys is mostly in-lane
//                 (one exchange with lane ^ 32).
//   online softmax in fp32 (exp2 with the scale folded into log2 units); P rounded to bf16.
//   O^T += V^T P^T  the P^T operand is exactly the S^T accumulator layout, so P never leaves the
//                 registers; V^T comes from an LDS copy of the tile transposed on the way in.
// Causal masking is applied only on tiles that reach past the wave's first position.  Keys past
// the request's last token (tail of the last page) are zeroed in V and masked in S.
#include "device_util.h"
#include "mtd_internal.h"

namespace mtd {
namespace {

constexpr int kBQ = 64;        // chunk positions per workgroup
constexpr int kBK = 64;        // keys per tile (one page)
constexpr int kKStride = 136;  // K tile row stride in LDS, bf16 elements (256 B + 16 B pad)
constexpr int kVtStride = 68;  // V^T tile row stride in LDS, bf16 elements (128 B + 8 B pad)
constexpr float kNegInf = -__builtin_huge_valf();

__global__ __launch_bounds__(256) void prefill_kernel(
    const uint16_t* __restrict__ k_pages, const uint16_t* __restrict__ v_pages, int num_pages,
    const uint16_t* __restrict__ q, int chunk_len, int prefix_len,
    const int32_t* __restrict__ block_table, float scale_log2, float* __restrict__ out,
    float* __restrict__ lse, int n_qtiles) {
  __shared__ __attribute__((aligned(16))) uint16_t k_lds[kBK * kKStride];
  __shared__ __attribute__((aligned(16))) uint16_t vt_lds[kHeadDim * kVtStride];

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

  floatx16_t o_acc[4];
#pragma unroll
  for (int dt = 0; dt < 4; ++dt)
#pragma unroll
    for (int v = 0; v < 16; ++v) o_acc[dt][v] = 0.f;
  float m = kNegInf;  // running max of the column, log2 units (same in both halves)
  float l = 0.f;      // running sum over this lane's keys

  const int kv_end = min(prefix_len + q0 + kBQ, total);
  const int n_tiles = (kv_end + kBK - 1) / kBK;
  const int wave_first = prefix_len + q0 + 16 * wave;  // smallest query position of the wave

  const int ld_row = tid >> 4;    // 0..15
  const int ld_chunk = tid & 15;  // 16-byte chunk of a 256-byte row

  for (int kt = 0; kt < n_tiles; ++kt) {
    const int page = block_table[kt];
    const int nvalid = min(kBK, total - kt * kBK);
    if (page >= 0 && page < num_pages) {
      const size_t blk = ((size_t)page * kKvHeads + g) * (kPage * kHeadDim);
      uint4 kr[4], vr[4];
#pragma unroll
      for (int i = 0; i < 4; ++i)
        kr[i] = *reinterpret_cast<const uint4*>(k_pages + blk + (ld_row + 16 * i) * kHeadDim + ld_chunk * 8);
#pragma unroll
      for (int i = 0; i < 4; ++i)
        vr[i] = *reinterpret_cast<const uint4*>(v_pages + blk + (4 * ld_row + i) * kHeadDim + ld_chunk * 8);
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (4 * ld_row + i >= nvalid) vr[i] = make_uint4(0, 0, 0, 0);
#pragma unroll
      for (int i = 0; i < 4; ++i)
        *reinterpret_cast<uint4*>(k_lds + (ld_row + 16 * i) * kKStride + ld_chunk * 8) = kr[i];
      // V^T: row = dim 8*ld_chunk + e, columns = keys 4*ld_row .. 4*ld_row+3
      const uint32_t r0[4] = {vr[0].x, vr[0].y, vr[0].z, vr[0].w};
      const uint32_t r1[4] = {vr[1].x, vr[1].y, vr[1].z, vr[1].w};
      const uint32_t r2[4] = {vr[2].x, vr[2].y, vr[2].z, vr[2].w};
      const uint32_t r3[4] = {vr[3].x, vr[3].y, vr[3].z, vr[3].w};
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const int d = 8 * ld_chunk + 2 * w;
        *reinterpret_cast<uint2*>(vt_lds + d * kVtStride + 4 * ld_row) =
            make_uint2(pack_lo16(r0[w], r1[w]), pack_lo16(r2[w], r3[w]));
        *reinterpret_cast<uint2*>(vt_lds + (d + 1) * kVtStride + 4 * ld_row) =
            make_uint2(pack_hi16(r0[w], r1[w]), pack_hi16(r2[w], r3[w]));
      }
    }
    __syncthreads();

    // S^T for keys 32mt .. 32mt+31 of the tile.
    floatx16_t st[2];
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) {
#pragma unroll
      for (int v = 0; v < 16; ++v) st[mt][v] = 0.f;
      const uint16_t* krow = k_lds + (32 * mt + n) * kKStride + 8 * hk;
#pragma unroll
      for (int ks = 0; ks < 8; ++ks) {
        const bf16x8_t a = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const uint4*>(krow + 16 * ks));
        st[mt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[ks], st[mt], 0, 0, 0);
      }
    }

    // Online softmax.  Accumulator element v of block mt is key 32mt + 8(v/4) + 4hk + v%4.
    const bool need_mask = kt * kBK + kBK - 1 > wave_first;
    float mx = kNegInf;
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) {
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        float x = st[mt][v] * scale_log2;
        if (need_mask) {
          const int key = kt * kBK + 32 * mt + 8 * (v >> 2) + 4 * hk + (v & 3);
          x = key <= qabs ? x : kNegInf;
        }
        st[mt][v] = x;
        mx = fmaxf(mx, x);
      }
    }
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
    const float m_new = fmaxf(m, mx);
    const float m_use = m_new == kNegInf ? 0.f : m_new;
    const float alpha = fast_exp2(m - m_use);
    m = m_new;
    float psum = 0.f;
    bf16x8_t pf[2][2];
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) {
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        uint32_t w[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const float p0 = fast_exp2(st[mt][8 * t + 2 * j] - m_use);
          const float p1 = fast_exp2(st[mt][8 * t + 2 * j + 1] - m_use);
          psum += p0 + p1;
          w[j] = pack_bf16x2(p0, p1);
        }
        pf[mt][t] = __builtin_bit_cast(bf16x8_t, make_uint4(w[0], w[1], w[2], w[3]));
      }
    }
    l = l * alpha + psum;
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
      for (int v = 0; v < 16; ++v) o_acc[dt][v] *= alpha;

    // O^T += V^T P^T.  For block mt, k-step t, this lane's 8 keys are
    // 32mt + 16t + 4hk + {0,1,2,3} and the same + 8.
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) {
      const uint16_t* vrow = vt_lds + (32 * dt + n) * kVtStride;
#pragma unroll
      for (int mt = 0; mt < 2; ++mt) {
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          const int col = 32 * mt + 16 * t + 4 * hk;
          const uint2 lo = *reinterpret_cast<const uint2*>(vrow + col);
          const uint2 hi = *reinterpret_cast<const uint2*>(vrow + col + 8);
          const bf16x8_t a = __builtin_bit_cast(bf16x8_t, make_uint4(lo.x, lo.y, hi.x, hi.y));
          o_acc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pf[mt][t], o_acc[dt], 0, 0, 0);
        }
      }
    }
    __syncthreads();
  }

  const float l_tot = l + __shfl_xor(l, 32, 64);
  if (qvalid) {
    const float inv = 1.f / l_tot;
    float* orow = out + ((size_t)qpos * kQHeads + head) * kHeadDim;
    // Accumulator element v of tile dt is dim 32dt + 8(v/4) + 4hk + v%4.
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
      for (int a = 0; a < 4; ++a)
        *reinterpret_cast<float4*>(orow + 32 * dt + 8 * a + 4 * hk) =
            make_float4(o_acc[dt][4 * a] * inv, o_acc[dt][4 * a + 1] * inv,
                        o_acc[dt][4 * a + 2] * inv, o_acc[dt][4 * a + 3] * inv);
    if (hk == 0) lse[(size_t)qpos * kQHeads + head] = (m + log2f(l_tot)) * kLn2;
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
