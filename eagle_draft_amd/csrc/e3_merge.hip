// Online-softmax merge of one attention block into a running (out, lse), float32,
// in the sigmoid form of the ring_attention page (`_update_out_and_lse`) and the
// zigzag_ring_attention page (`update_out_and_lse`):
//   out' = out - sigmoid(b_lse - lse) * (out - b_out)
//   lse' = lse - logsigmoid(lse - b_lse)
// An empty block row (b_lse = -inf) is left alone; an empty state row
// (lse = -inf) takes the block row.
#include "e3_common.h"

namespace e3 {

// 16 lanes per (b, t, h) row, 4 floats per lane per step; the row's lse is read by
// every lane of its group before lane 0 of the group writes it (one wave).
__global__ __launch_bounds__(256) void lse_merge_kernel(float* out, float* lse, const float* bo,
                                                        const float* bl, int B, int T, int H, int D,
                                                        int blayout) {
  const long long r = (long long)blockIdx.x * 16 + threadIdx.x / 16;
  const int c = threadIdx.x % 16;
  if (r >= (long long)B * T * H) return;
  const long long h = r % H, bt = r / H, t = bt % T, b = bt / T;
  const long long li = (b * H + h) * T + t;
  const long long bli = blayout == 0 ? li : (b * T + t) * H + h;
  const float L = lse[li], BL = bl[bli];
  if (BL == kNegInf) return;
  float w = 1.f, nl = BL;
  if (L != kNegInf) {
    const float x = BL - L;                       // sigmoid(x), stable on both sides
    const float ex = __expf(-fabsf(x));
    w = x >= 0.f ? 1.f / (1.f + ex) : ex / (1.f + ex);
    const float y = L - BL;                       // logsigmoid(y) = min(y,0) - log1p(exp(-|y|))
    nl = L - (fminf(y, 0.f) - log1pf(__expf(-fabsf(y))));
  }
  float* o = out + r * D;
  const float* x = bo + r * D;
  for (int d = 4 * c; d < D; d += 64) {
    f32x4 ov = *reinterpret_cast<const f32x4*>(o + d);
    const f32x4 xv = *reinterpret_cast<const f32x4*>(x + d);
#pragma unroll
    for (int e = 0; e < 4; ++e) ov[e] = L == kNegInf ? xv[e] : ov[e] - w * (ov[e] - xv[e]);
    *reinterpret_cast<f32x4*>(o + d) = ov;
  }
  if (c == 0) lse[li] = nl;
}

hipError_t launch_lse_merge(float* out, float* lse, const float* bo, const float* bl, int B, int T,
                            int H, int D, int blayout, hipStream_t st) {
  const long long rows = (long long)B * T * H;
  if (rows == 0) return hipSuccess;
  const long long nb = (rows + 15) / 16;
  hipLaunchKernelGGL(lse_merge_kernel, dim3((unsigned)nb), dim3(256), 0, st, out, lse, bo, bl, B, T,
                     H, D, blayout);
  return hipGetLastError();
}

}  // namespace e3
