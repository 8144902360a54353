// Batched single-token decode attention over the paged KV cache: split-K flash-decoding.
//
// Decode emits one token per request per step over the request's whole cache, with concurrent
// requests packed into one batch ("Optimizing ASR Models to Transcribe 90-Minute Multi-Speaker
// Audio", sections ASR Model Primer and Batched Inference).  With one query token per head the
// work is two flops per KV byte, far below the MI355X ridge point, so the kernels are built to
// stream K/V from HBM once, with coalesced 16-byte non-temporal loads, and keep every other cost
// off the memory critical path.
//
// decode_split: one wavefront per work item = (request b, split s, KV head g), where split s is
//   the logical tokens [T s, min(T s + T, L_b)) with T = split_tokens(L_b) (64 to 512 tokens, by
//   length).  Every request owns S = split_parts_bound(max_kv_len) slots: item (b, s, g) is wave
//   8 (S b + s) + g, and its partial goes to slot S b + s of the workspace.  So a wave knows its
//   request and split from its index alone and loads the length and the table entry of page s in
//   one round (a dense numbering would need the lengths of the requests before it first); the
//   waves of slots past a request's split count exit there, and the others load the query rows
//   beside their first page.
//   Both query heads of the GQA group (2g, 2g+1) are served from the same K/V loads.  The wave
//   writes the split's normalised partial output and its log-sum-exp.
// decode_merge: one workgroup per (request, query head) combines that request's partials with
//   weights exp(lse_s - LSE), reducing over wavefronts and LDS.  It loads the slots' LSEs and the
//   first partial rows of each lane group together with the length, so a request of at most 16
//   splits (64 when the batch has at most 64 slots per request) costs one round of loads.
// With kAppend, decode_split also stores this step's token: the request's new K/V row goes to its
//   slot at position kv_lens[b] - 1.  Only the last split of a request covers that position, so the
//   wave of that split for KV head g writes head g's row (8 lanes, 32 bytes each) before it reads
//   its pages, and the lanes that read those bytes are the lanes that wrote them; no other wave
//   reads the slot, so nothing has to wait for the store.
//
// Lane layout inside decode_split for one 64-token page: lane = 8*sg + o.  The lane handles the
// 8 slots {8a + sg : a = 0..7} and, of each slot row (128 dims = 256 bytes), the two 16-byte
// chunks o and 8 + o (dims 8o..8o+7 and 64+8o..64+8o+7).  One load instruction therefore reads 8
// whole 128-byte lines.  A slot's score is the sum over its 8 lanes (three DPP steps); values are
// accumulated with packed bf16 dot products pairing two slots per instruction.
#include <atomic>

#include "device_util.h"
#include "mtd_internal.h"

namespace mtd {
namespace {

constexpr float kNegInf = -__builtin_huge_valf();

// 16-byte load marked non-temporal: every K/V byte of a decode call is read exactly once, so the
// loads should stream through the caches instead of displacing other data.
typedef unsigned u32x4_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 stream_load16(const uint16_t* p) {
  const u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}

template <bool kAppend>
__global__ __launch_bounds__(64) void decode_split_kernel(
    uint16_t* __restrict__ k_pages, uint16_t* __restrict__ v_pages, int num_pages,
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k_new, const uint16_t* __restrict__ v_new,
    const int32_t* __restrict__ kv_lens, const int32_t* __restrict__ block_tables, int bt_stride,
    int max_kv_len, float scale_log2, float* __restrict__ part_o, float* __restrict__ part_lse) {
  const int lane = threadIdx.x;
  const int f = blockIdx.x / kKvHeads;
  const int g = blockIdx.x % kKvHeads;
  const int n_slots = split_parts_bound(max_kv_len);
  const int b = f / n_slots, s = f % n_slots;
  const int32_t* bt_row = block_tables + (size_t)b * bt_stride;

  const int sg = lane >> 3;  // slot group: slots 8a + sg
  const int o = lane & 7;    // chunks o and 8 + o of each row

  // The length and the table entry of page s go out together (s < n_slots <= bt_stride); the
  // query rows follow once the wave knows it has work, beside its first page's loads.
  int len = kv_lens[b];
  const int page_s = bt_row[s];
  asm volatile("" ::"v"(len), "v"(page_s));
  const int len_raw = len;
  len = min(max(len, 0), max_kv_len);
  if (s >= split_parts(len)) return;
  // This lane's 16 dims of the query rows of heads 2g and 2g+1 (as packed bf16 pairs).
  uint4 qv[2][2];
#pragma unroll
  for (int hh = 0; hh < 2; ++hh) {
    const uint16_t* qrow = q + ((size_t)b * kQHeads + kGroup * g + hh) * kHeadDim;
    qv[hh][0] = *reinterpret_cast<const uint4*>(qrow + 8 * o);
    qv[hh][1] = *reinterpret_cast<const uint4*>(qrow + 64 + 8 * o);
  }

  float m[2] = {kNegInf, kNegInf};  // running max (log2 units) over this lane's slots
  float l[2] = {0.f, 0.f};          // running sum of exp2(x - m)
  float acc[2][2][8];               // [head][chunk][dim] unnormalised output
#pragma unroll
  for (int hh = 0; hh < 2; ++hh)
#pragma unroll
    for (int c = 0; c < 2; ++c)
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[hh][c][e] = 0.f;

  const int tok0 = s * split_tokens(len);
  const int tok1 = min(tok0 + split_tokens(len), len);
  // kAppend: the new token sits at position len - 1 when the request's length is in [1, max_kv_len]
  // (len is clamped to that range; a length outside it appends nothing).  Before reading any page,
  // the wave of the last split stores head g's new row: the lanes of slot group (len - 1) % 8, 32
  // bytes of K and 32 of V each.  The page loop below then loads exactly those bytes in the same
  // lanes, so each lane reads back what it wrote itself (program order within a thread).
  if (kAppend && tok1 == len && len >= 1 && len_raw == len) {
    const int page = (len - 1) / kPage == s ? page_s : bt_row[(len - 1) / kPage];
    if (page >= 0 && page < num_pages) {  // an out-of-pool page is neither stored nor read
      const uint16_t* kn = k_new + ((size_t)b * kKvHeads + g) * kHeadDim;
      const uint16_t* vn = v_new + ((size_t)b * kKvHeads + g) * kHeadDim;
      const int ns = (len - 1) % kPage;
      if ((ns & 7) == sg) {
        const size_t row = (((size_t)page * kKvHeads + g) * kPage + ns) * kHeadDim;
#pragma unroll
        for (int c = 0; c < 2; ++c) {
          *reinterpret_cast<uint4*>(k_pages + row + (8 * c + o) * 8) =
              *reinterpret_cast<const uint4*>(kn + (8 * c + o) * 8);
          *reinterpret_cast<uint4*>(v_pages + row + (8 * c + o) * 8) =
              *reinterpret_cast<const uint4*>(vn + (8 * c + o) * 8);
        }
      }
    }
  }

  for (int e0 = tok0 / kPage; e0 * kPage < tok1; ++e0) {
    const int page = e0 == s ? page_s : bt_row[e0];
    if (page < 0 || page >= num_pages) continue;
    const int nvalid = min(kPage, tok1 - e0 * kPage);
    const size_t blk = ((size_t)page * kKvHeads + g) * (kPage * kHeadDim);
    const uint16_t* kb = k_pages + blk;
    const uint16_t* vb = v_pages + blk;

    uint4 kr[8][2], vr[8][2];
#pragma unroll
    for (int a = 0; a < 8; ++a)
#pragma unroll
      for (int c = 0; c < 2; ++c)
        kr[a][c] = stream_load16(kb + (8 * a + sg) * kHeadDim + (8 * c + o) * 8);
#pragma unroll
    for (int a = 0; a < 8; ++a)
#pragma unroll
      for (int c = 0; c < 2; ++c)
        vr[a][c] = stream_load16(vb + (8 * a + sg) * kHeadDim + (8 * c + o) * 8);

    // Scores of slots 8a + sg for both heads, in log2 units.
    float x[2][8];
#pragma unroll
    for (int a = 0; a < 8; ++a) {
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        float d = 0.f;
#pragma unroll
        for (int c = 0; c < 2; ++c) {
          d = dot2_bf16(kr[a][c].x, c == 0 ? qv[hh][0].x : qv[hh][1].x, d);
          d = dot2_bf16(kr[a][c].y, c == 0 ? qv[hh][0].y : qv[hh][1].y, d);
          d = dot2_bf16(kr[a][c].z, c == 0 ? qv[hh][0].z : qv[hh][1].z, d);
          d = dot2_bf16(kr[a][c].w, c == 0 ? qv[hh][0].w : qv[hh][1].w, d);
        }
        x[hh][a] = sum8(d) * scale_log2;
      }
    }
    if (nvalid < kPage) {  // partial last page: slots >= nvalid hold no token of this request
#pragma unroll
      for (int a = 0; a < 8; ++a) {
        const bool ok = 8 * a + sg < nvalid;
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) x[hh][a] = ok ? x[hh][a] : kNegInf;
#pragma unroll
        for (int c = 0; c < 2; ++c) {
          vr[a][c].x = ok ? vr[a][c].x : 0u;
          vr[a][c].y = ok ? vr[a][c].y : 0u;
          vr[a][c].z = ok ? vr[a][c].z : 0u;
          vr[a][c].w = ok ? vr[a][c].w : 0u;
        }
      }
    }

    uint32_t pp[2][4];  // probabilities as bf16 pairs (slots 2k, 2k+1)
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
      float mx = x[hh][0];
#pragma unroll
      for (int a = 1; a < 8; ++a) mx = fmaxf(mx, x[hh][a]);
      const float m_new = fmaxf(m[hh], mx);
      const float m_use = m_new == kNegInf ? 0.f : m_new;
      const float alpha = fast_exp2(m[hh] - m_use);
      m[hh] = m_new;
      float p[8];
      float psum = 0.f;
#pragma unroll
      for (int a = 0; a < 8; ++a) {
        p[a] = fast_exp2(x[hh][a] - m_use);
        psum += p[a];
      }
      l[hh] = l[hh] * alpha + psum;
#pragma unroll
      for (int c = 0; c < 2; ++c)
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[hh][c][e] *= alpha;
#pragma unroll
      for (int k = 0; k < 4; ++k) pp[hh][k] = pack_bf16x2(p[2 * k], p[2 * k + 1]);
    }

    // acc[h][c][d] += p[2k] * v[slot 2k][d] + p[2k+1] * v[slot 2k+1][d]
#pragma unroll
    for (int k = 0; k < 4; ++k) {
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        const uint32_t xw[4] = {vr[2 * k][c].x, vr[2 * k][c].y, vr[2 * k][c].z, vr[2 * k][c].w};
        const uint32_t yw[4] = {vr[2 * k + 1][c].x, vr[2 * k + 1][c].y, vr[2 * k + 1][c].z,
                                vr[2 * k + 1][c].w};
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          const uint32_t lo = pack_lo16(xw[w], yw[w]);
          const uint32_t hi = pack_hi16(xw[w], yw[w]);
#pragma unroll
          for (int hh = 0; hh < 2; ++hh) {
            acc[hh][c][2 * w] = dot2_bf16(lo, pp[hh][k], acc[hh][c][2 * w]);
            acc[hh][c][2 * w + 1] = dot2_bf16(hi, pp[hh][k], acc[hh][c][2 * w + 1]);
          }
        }
      }
    }
  }

  // Combine the 8 slot groups (lanes xor 8, 16, 32) and write the split's partial.
#pragma unroll
  for (int hh = 0; hh < 2; ++hh) {
    float mm = m[hh];
    mm = fmaxf(mm, __shfl_xor(mm, 8, 64));
    mm = fmaxf(mm, __shfl_xor(mm, 16, 64));
    mm = fmaxf(mm, __shfl_xor(mm, 32, 64));
    const float w = m[hh] == kNegInf ? 0.f : fast_exp2(m[hh] - mm);
    float ll = l[hh] * w;
    ll += __shfl_xor(ll, 8, 64);
    ll += __shfl_xor(ll, 16, 64);
    ll += __shfl_xor(ll, 32, 64);
    const float inv = ll > 0.f ? 1.f / ll : 0.f;  // a split with no key (its pages out of the pool): O = 0
    float* orow = part_o + ((size_t)f * kQHeads + kGroup * g + hh) * kHeadDim;
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      float r[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        float v = acc[hh][c][e] * w;
        v += __shfl_xor(v, 8, 64);
        v += __shfl_xor(v, 16, 64);
        v += __shfl_xor(v, 32, 64);
        r[e] = v * inv;
      }
      if (sg == 0) {
        float4* dst = reinterpret_cast<float4*>(orow + 64 * c + 8 * o);
        dst[0] = make_float4(r[0], r[1], r[2], r[3]);
        dst[1] = make_float4(r[4], r[5], r[6], r[7]);
      }
    }
    if (lane == 0) part_lse[(size_t)f * kQHeads + kGroup * g + hh] = (mm + log2f(ll)) * kLn2;
  }
}

// One workgroup (4 wavefronts) per (request b, query head h).  The split weights
// w_s = exp(lse_s - LSE) go to LDS; then 16 lane groups of 16 lanes each take every 16th partial
// (a lane covers 8 dims with two 16-byte loads), so all partial rows of the request are in flight
// at once instead of one after another; the 16 group sums are added in LDS.
template <int kPre>
__global__ __launch_bounds__(256) void decode_merge_kernel(
    const int32_t* __restrict__ kv_lens, int max_kv_len,
    const float* __restrict__ part_o, const float* __restrict__ part_lse, float* __restrict__ out,
    float* __restrict__ lse_out) {
  __shared__ float s_w[kMaxParts];
  __shared__ float s_red[16][kHeadDim];
  __shared__ float s_wave[4];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int h = blockIdx.x % kQHeads;
  const int b = blockIdx.x / kQHeads;

  // Request b's partials sit at b * n_slots ..; its length, the LSE of each slot and the first kPre
  // partial rows of each lane group (parts grp + 16 k, k < kPre; see below) are loaded together,
  // and slots past the request's split count are ignored.  The launcher takes kPre = 4 for 17 to
  // 64 slots, so that a request of up to 64 splits has all its partials in flight in one round,
  // and kPre = 1 otherwise: with at most 16 slots one row per group covers them, and with more
  // than 64 the rows past a request's split count would cost more than the round they save.
  const int n_slots = split_parts_bound(max_kv_len);  // at most kMaxParts = blockDim.x
  const int first = b * n_slots;
  const int grp = tid >> 4;       // parts grp, grp + 16, ...
  const int c = tid & 15;         // dims 8c .. 8c+7
  float lse_t = kNegInf;
  if (tid < n_slots) lse_t = part_lse[(size_t)(first + tid) * kQHeads + h];
  // Unconditional loads (a row past the request's slots is clamped into them), so that no branch
  // joins force a wait between them.
  float4 pre[kPre][2];
#pragma unroll
  for (int k = 0; k < kPre; ++k) {
    const int p = min(grp + 16 * k, n_slots - 1);
    const float4* src = reinterpret_cast<const float4*>(part_o + ((size_t)(first + p) * kQHeads + h) * kHeadDim + 8 * c);
    pre[k][0] = src[0];
    pre[k][1] = src[1];
  }
  int len = kv_lens[b];
  // all loads out before the first wait
  static_assert(kPre == 1 || kPre == 4, "prefetch depths the launcher uses");
  if constexpr (kPre == 1)
    asm volatile("" ::"v"(len), "v"(lse_t), "v"(pre[0][0].x), "v"(pre[0][1].x));
  else
    asm volatile("" ::"v"(len), "v"(lse_t), "v"(pre[0][0].x), "v"(pre[0][1].x), "v"(pre[1][0].x),
                 "v"(pre[1][1].x), "v"(pre[2][0].x), "v"(pre[2][1].x), "v"(pre[3][0].x), "v"(pre[3][1].x));
  len = min(max(len, 0), max_kv_len);
  const int n_parts = split_parts(len);
  float* orow = out + ((size_t)b * kQHeads + h) * kHeadDim;
  if (n_parts == 0) {  // no keys: zero output, LSE = -inf
    if (tid < kHeadDim) orow[tid] = 0.f;
    if (tid == 0) lse_out[(size_t)b * kQHeads + h] = kNegInf;
    return;
  }

  // LSE of every part -> LDS, block max
  float mx = kNegInf;
  if (tid < n_parts) {
    s_w[tid] = lse_t;
    mx = lse_t;
  }
  mx = wave_max(mx);
  if (lane == 0) s_wave[wave] = mx;
  __syncthreads();
  mx = fmaxf(fmaxf(s_wave[0], s_wave[1]), fmaxf(s_wave[2], s_wave[3]));
  if (mx == kNegInf) {  // no part holds a key (every page out of the pool): as for no keys at all
    if (tid < kHeadDim) orow[tid] = 0.f;
    if (tid == 0) lse_out[(size_t)b * kQHeads + h] = kNegInf;
    return;
  }
  __syncthreads();
  // weights and their sum
  float ws = 0.f;
  for (int p = tid; p < n_parts; p += 256) {
    const float w = fast_exp2((s_w[p] - mx) * kLog2e);
    s_w[p] = w;
    ws += w;
  }
  ws = wave_sum(ws);
  if (lane == 0) s_wave[wave] = ws;
  __syncthreads();
  ws = s_wave[0] + s_wave[1] + s_wave[2] + s_wave[3];

  // weighted sum of the partial outputs
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int k = 0; k < kPre; ++k) {
    const int p = grp + 16 * k;
    if (p < n_parts) {
      const float w = s_w[p];
      const float4 v0 = pre[k][0], v1 = pre[k][1];
      acc[0] += w * v0.x; acc[1] += w * v0.y; acc[2] += w * v0.z; acc[3] += w * v0.w;
      acc[4] += w * v1.x; acc[5] += w * v1.y; acc[6] += w * v1.z; acc[7] += w * v1.w;
    }
  }
#pragma unroll 4
  for (int p = grp + 16 * kPre; p < n_parts; p += 16) {
    const float w = s_w[p];
    const float4* src = reinterpret_cast<const float4*>(part_o + ((size_t)(first + p) * kQHeads + h) * kHeadDim + 8 * c);
    const float4 v0 = src[0];
    const float4 v1 = src[1];
    acc[0] += w * v0.x; acc[1] += w * v0.y; acc[2] += w * v0.z; acc[3] += w * v0.w;
    acc[4] += w * v1.x; acc[5] += w * v1.y; acc[6] += w * v1.z; acc[7] += w * v1.w;
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) s_red[grp][8 * c + e] = acc[e];
  __syncthreads();
  if (tid < kHeadDim) {
    float sum = 0.f;
#pragma unroll
    for (int g2 = 0; g2 < 16; ++g2) sum += s_red[g2][tid];
    orow[tid] = sum / ws;
  }
  if (tid == 0) lse_out[(size_t)b * kQHeads + h] = mx + logf(ws);
}

}  // namespace

// Scratch of mtd_attn_decode_noalloc: the split partials live in this file-scope device array
// instead of a caller workspace.  Every GPU the library runs on holds its own copy until the
// process ends.  In host code the name `scratch` is only a host-side stand-in; its device address
// comes from hipGetSymbolAddress, once per device, and only that address is ever used.
__device__ __align__(256) unsigned char scratch[kDecodeScratchBytes];

namespace {
std::atomic<void*> g_scratch[kMaxDevices];
}  // namespace

hipError_t decode_scratch(void** ptr) {
  int dev = 0;
  hipError_t err = hipGetDevice(&dev);
  if (err != hipSuccess) return err;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  void* p = g_scratch[dev].load(std::memory_order_acquire);
  if (p == nullptr) {
    err = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (err != hipSuccess) return err;
    if (p == nullptr) return hipErrorInvalidSymbol;
    g_scratch[dev].store(p, std::memory_order_release);  // the same address if two threads race here
  }
  *ptr = p;
  return hipSuccess;
}

hipError_t launch_decode(const KvPools& kv, const uint16_t* q, const uint16_t* k_new, const uint16_t* v_new,
                         const int32_t* kv_lens, const int32_t* block_tables, int bt_stride, int batch,
                         int max_kv_len, float scale, void* workspace, float* out, float* lse,
                         hipStream_t stream) {
  const size_t parts = (size_t)batch * (size_t)split_parts_bound(max_kv_len);
  float* part_o = static_cast<float*>(workspace);
  float* part_lse = part_o + parts * kQHeads * kHeadDim;
  const unsigned n_waves = (unsigned)(parts * kKvHeads);
  if (k_new != nullptr)
    decode_split_kernel<true><<<dim3(n_waves), dim3(64), 0, stream>>>(
        kv.k, kv.v, kv.num_pages, q, k_new, v_new, kv_lens, block_tables, bt_stride, max_kv_len,
        scale * kLog2e, part_o, part_lse);
  else
    decode_split_kernel<false><<<dim3(n_waves), dim3(64), 0, stream>>>(
        kv.k, kv.v, kv.num_pages, q, nullptr, nullptr, kv_lens, block_tables, bt_stride,
        max_kv_len, scale * kLog2e, part_o, part_lse);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  const int n_slots = split_parts_bound(max_kv_len);
  if (n_slots > 16 && n_slots <= 64)
    decode_merge_kernel<4><<<dim3(batch * kQHeads), dim3(256), 0, stream>>>(
        kv_lens, max_kv_len, part_o, part_lse, out, lse);
  else
    decode_merge_kernel<1><<<dim3(batch * kQHeads), dim3(256), 0, stream>>>(
        kv_lens, max_kv_len, part_o, part_lse, out, lse);
  return hipGetLastError();
}

}  // namespace mtd
