// Combining attention results over disjoint key sets by log-sum-exp.
//
// The pages list multi-GPU support as ongoing work, for audio so long that its KV cache outgrows
// one GPU ("Optimizing ASR Models to Transcribe 90-Minute Multi-Speaker Audio", section What's
// Next).  One way is to split a request's KV by sequence: each GPU holds a range of the request's
// pages and runs decode attention over its range only, which yields that range's output and
// log-sum-exp.  After the partials are gathered, one combination step gives the exact result over
// all keys:
//     LSE = log sum_k exp(lse_k),    O = sum_k exp(lse_k - LSE) o_k.
// A part with no keys (lse_k = -inf) carries zero weight; a row whose parts all have no keys gets
// O = 0 and LSE = -inf.  This kernel is that step on one GPU.
//
// One wavefront per row (token x head): lane l owns dims 2l and 2l+1, so each part's row is one
// coalesced 512-byte read.  The max over the parts is taken first, then one pass accumulates the
// weights and the weighted rows in part order.
#include "device_util.h"
#include "mtd_internal.h"

namespace mtd {
namespace {

constexpr float kNegInf = -__builtin_huge_valf();
constexpr int kRowsPerBlock = 4;

__global__ __launch_bounds__(64 * kRowsPerBlock) void attn_merge_kernel(
    const float* __restrict__ o_parts, const float* __restrict__ lse_parts, int n_parts, int n_rows,
    float* __restrict__ out, float* __restrict__ lse) {
  const int row = blockIdx.x * kRowsPerBlock + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (row >= n_rows) return;
  float mx = kNegInf;
  for (int k = 0; k < n_parts; ++k) mx = fmaxf(mx, lse_parts[(size_t)k * n_rows + row]);
  float2* orow = reinterpret_cast<float2*>(out + (size_t)row * kHeadDim) + lane;
  if (mx == kNegInf) {  // no keys in any part
    *orow = make_float2(0.f, 0.f);
    if (lane == 0) lse[row] = kNegInf;
    return;
  }
  float ws = 0.f, a0 = 0.f, a1 = 0.f;
  for (int k = 0; k < n_parts; ++k) {
    const float lk = lse_parts[(size_t)k * n_rows + row];
    const float w = lk == kNegInf ? 0.f : fast_exp2((lk - mx) * kLog2e);
    const float2 v = reinterpret_cast<const float2*>(o_parts + ((size_t)k * n_rows + row) * kHeadDim)[lane];
    ws += w;
    a0 = fmaf(w, v.x, a0);
    a1 = fmaf(w, v.y, a1);
  }
  const float inv = 1.f / ws;
  *orow = make_float2(a0 * inv, a1 * inv);
  if (lane == 0) lse[row] = mx + logf(ws);
}

}  // namespace

hipError_t launch_attn_merge(const float* o_parts, const float* lse_parts, int n_parts, int n_rows,
                             float* out, float* lse, hipStream_t stream) {
  attn_merge_kernel<<<dim3((n_rows + kRowsPerBlock - 1) / kRowsPerBlock), dim3(64 * kRowsPerBlock), 0,
                      stream>>>(o_parts, lse_parts, n_parts, n_rows, out, lse);
  return hipGetLastError();
}

}  // namespace mtd
