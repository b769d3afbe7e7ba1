// Transposed copies of K/V/Q/dO for the MFMA operands that reduce over the
// sequence: Xt[b][h][d][p] holds X[b][row][h][d]. The rows of each run (a range
// of consecutive rows that the kernels tile together) start at a 64-aligned
// position p, padding is zero, and within each group of 16 rows the order is
// {0-3, 8-11, 4-7, 12-15}: the order in which a 32x32 MFMA accumulator holds its
// rows, so an operand of 8 consecutive positions at offset 8g of a group pairs
// with an accumulator slice directly, as one 16-byte LDS read.
#include "e3_common.h"

namespace e3 {

// Row order inside a 16-row group: position -> source row.
__device__ __forceinline__ int perm16_src(int q) {
  const int a = q >> 2;                 // 0,1,2,3 -> rows 0-3, 8-11, 4-7, 12-15
  return ((a == 1) ? 8 : (a == 2) ? 4 : 4 * a) + (q & 3);
}

// One workgroup = a 64-row x D tile of one (batch row, head).
template <typename T, int D>
__global__ __launch_bounds__(256) void xpose_kernel(const T* __restrict__ x, long long x_bs,
                                                    T* __restrict__ xt, XRuns runs, int H) {
  constexpr int R = 64;
  constexpr int STR = D + 16 / (int)sizeof(T);
  __shared__ __attribute__((aligned(16))) T tile[R * STR];
  const int tid = threadIdx.x;
  const int bh = blockIdx.y, b = bh / H, h = bh % H;
  // Which run and tile.
  int t = blockIdx.x, run = 0;
  for (; run < runs.n; ++run) {
    const int nt = (runs.len[run] + R - 1) / R;
    if (t < nt) break;
    t -= nt;
  }
  const int r0 = t * R;
  const int nv = runs.len[run] - r0;    // valid rows in this tile
  const long long rs = (long long)H * D;
  const T* src = x + (long long)b * x_bs + (long long)(runs.src[run] + r0) * rs + (long long)h * D;
  TileLoad<T, R, D, 256> ld;
  if (nv >= R) ld.load_full(src, rs, tid);
  else ld.load(src, rs, nv, tid);
  ld.store(tile, STR, tid);
  __syncthreads();
  // Write D rows of R positions: thread -> (d, 8 positions).
  T* dst = xt + ((long long)b * H + h) * (long long)D * runs.pitch + runs.dst[run] + r0;
  for (int c = tid; c < D * (R / 8); c += 256) {
    const int d = c / (R / 8), p0 = (c % (R / 8)) * 8;
    typename V8<T>::type v;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int q = p0 + i;
      const int src_row = (q & ~15) + perm16_src(q & 15);
      v[i] = tile[src_row * STR + d];
    }
    *reinterpret_cast<typename V8<T>::type*>(dst + (long long)d * runs.pitch + p0) = v;
  }
}

template <typename T, int D>
static hipError_t launch_xpose_t(const void* x, long long x_bs, void* xt, const XRuns& runs, int B,
                                 int H, hipStream_t st) {
  int tiles = 0;
  for (int i = 0; i < runs.n; ++i) tiles += (runs.len[i] + 63) / 64;
  if (tiles == 0) return hipSuccess;
  hipLaunchKernelGGL((xpose_kernel<T, D>), dim3(tiles, B * H), dim3(256), 0, st,
                     reinterpret_cast<const T*>(x), x_bs, reinterpret_cast<T*>(xt), runs, H);
  return hipGetLastError();
}

hipError_t launch_xpose(const void* x, long long x_bs, void* xt, const XRuns& runs, int B, int H,
                        int dtype, int D, hipStream_t st) {
  if (dtype == 0)
    return D == 128 ? launch_xpose_t<bf16, 128>(x, x_bs, xt, runs, B, H, st)
                    : launch_xpose_t<bf16, 64>(x, x_bs, xt, runs, B, H, st);
  return D == 128 ? launch_xpose_t<float, 128>(x, x_bs, xt, runs, B, H, st)
                  : launch_xpose_t<float, 64>(x, x_bs, xt, runs, B, H, st);
}

}  // namespace e3
