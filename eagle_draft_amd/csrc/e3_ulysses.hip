// Ulysses sequence <-> head re-sharding, the local halves around the all-to-all
// (ulysses_attention page: `_gather_seq_scatter_heads`, `_scatter_seq_gather_heads`,
// `_gather_lse`, `_scatter_lse`; `_all_to_all_single` exchanges equal splits along
// dim 0, so a send buffer is [uly][...] with part i going to rank i and a receive
// buffer is [uly][...] with part i coming from rank i).
//
// Every transform is a copy of contiguous segments of L elements between two
// strided layouts, indexed by (i0, i1, i2):
//   src + i0*s0 + i1*s1 + i2*s2  ->  dst + i0*d0 + i1*d1 + i2*d2.
// One kernel does all of them, HBM-bound: a workgroup covers a run of segments,
// each lane moves 16-byte vectors when every offset is 16-byte aligned (else
// 4-byte words), reads and writes coalesced along the segment.
#include <type_traits>

#include "e3_common.h"

namespace e3 {

// VB = bytes per lane access (16 or 4). Each workgroup walks a contiguous range
// of (segment, chunk) items; a segment of `seg` bytes is `seg / VB` items.
template <int VB>
__global__ __launch_bounds__(256) void seg_copy_kernel(const SegCopy c) {
  typedef typename std::conditional<VB == 16, uint4, unsigned>::type V;
  const long long per = c.seg / VB;
  const long long total = c.n0 * c.n1 * c.n2 * per;
  for (long long it = (long long)blockIdx.x * 256 + threadIdx.x; it < total;
       it += (long long)gridDim.x * 256) {
    const long long k = it % per;
    long long r = it / per;
    const long long i2 = r % c.n2;
    r /= c.n2;
    const long long i1 = r % c.n1;
    const long long i0 = r / c.n1;
    const V v = *reinterpret_cast<const V*>(c.src + i0 * c.s0 + i1 * c.s1 + i2 * c.s2 + k * VB);
    *reinterpret_cast<V*>(c.dst + i0 * c.d0 + i1 * c.d1 + i2 * c.d2 + k * VB) = v;
  }
}

hipError_t launch_seg_copy(const SegCopy& c, hipStream_t st) {
  const long long nseg = c.n0 * c.n1 * c.n2;
  if (nseg == 0 || c.seg == 0) return hipSuccess;
  const bool v16 = ((c.seg | c.s0 | c.s1 | c.s2 | c.d0 | c.d1 | c.d2) % 16 == 0) &&
                   ((reinterpret_cast<uintptr_t>(c.src) | reinterpret_cast<uintptr_t>(c.dst)) % 16 == 0);
  const long long items = nseg * (c.seg / (v16 ? 16 : 4));
  long long grid = (items + 255) / 256;
  if (grid > 8192) grid = 8192;   // a grid-stride loop covers the rest
  if (v16)
    hipLaunchKernelGGL((seg_copy_kernel<16>), dim3((unsigned)grid), dim3(256), 0, st, c);
  else
    hipLaunchKernelGGL((seg_copy_kernel<4>), dim3((unsigned)grid), dim3(256), 0, st, c);
  return hipGetLastError();
}

}  // namespace e3
