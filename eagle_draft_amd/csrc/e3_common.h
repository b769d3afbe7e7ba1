// Shared definitions of the EAGLE-3 mixed-attention HIP kernels (gfx950):
// vector types, MFMA steps, DPP row reductions, and the share geometry (query
// rows -> global positions, block-0 K/V segments in ring order) used by both the
// kernels and the host driver.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace e3 {

typedef __bf16 bf16;
typedef bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kNegInf = -__builtin_huge_valf();

enum { LAYOUT_FULL = 0, LAYOUT_CONTIGUOUS = 1, LAYOUT_ZIGZAG = 2, LAYOUT_HEADSHARD = 3 };

// Kernel arguments (passed by value). Strides are in elements.
struct Args {
  const void* q;
  const void* k0;
  const void* v0;
  const void* kd;
  const void* vd;
  const void* dout;
  const void* o_in;     // merged out (backward input)
  const float* lse_in;  // merged lse (backward input)
  void* out;
  float* lse;
  float* delta;         // rowsum(dO * O), [B, H, q_pitch] (rows at Geo::prow)
  float* lse2;          // lse * log2(e), same layout as delta (delta = lse2 + B*H*q_pitch)
  const float* dqd;     // float32 partial of dq from the dQ kernel, [B, T, H, D] (workspace)
  void* dq;
  void* dk0;
  void* dv0;
  void* dkd;
  void* dvd;
  int q_pitch;          // positions per (b, h) row of lse2 / delta
  const int32_t* cu;    // device cu_seqlens (global document boundaries)
  const int32_t* cu_host;   // host copy of the same (host-side geometry of a launch)
  int ndocs;            // <= 1: one document
  int B, T, Tkv, H, N;
  long long k0_bs, kd_bs, kd_blk;
  float scale;
  float c2;             // scale * log2(e): scores are kept in the base-2 domain
  int layout, cp, rank;
  // Element strides of q / out (batch, head, row) and of k0 / v0 (head, row; the
  // batch stride is k0_bs): token-major [B, T, H, D] by default, head-major
  // [B, H, T, D] in the frozen-target forward. Only the forward reads them.
  long long q_bs, q_hs, q_rs, kv_hs, kv_rs;
  // Ring-step mode (the single-GPU half of the ring protocol): only the block-0
  // keys of ring steps [step_lo, step_hi) are visited, and
  int step_lo, step_hi;
  int out_f32;          //   the forward writes a float32 (out, lse) of those keys
  int dq_accum;         //   the dQ kernel adds scale * dQ into a float32 dq (dqd)
  int kv_accum;         //   dK/dV adds into float32 dk0/dv0 for the steps' keys only
  // No-allocation backward: the block-0 dq goes through dq itself (q's dtype) instead
  // of a float32 workspace partial, and every kernel runs on the caller's stream.
  int dq_in_out;
};



// A copy of contiguous segments of `seg` bytes between two strided layouts,
// indexed by (i0, i1, i2) < (n0, n1, n2) (the Ulysses re-sharding transforms):
//   src + i0*s0 + i1*s1 + i2*s2  ->  dst + i0*d0 + i1*d1 + i2*d2 (strides in bytes).
struct SegCopy {
  const char* src;
  char* dst;
  long long n0, n1, n2;
  long long s0, s1, s2;
  long long d0, d1, d2;
  long long seg;
};

// Measurement hook (host): records the next caller-provided timing event, if any,
// on the stream. Called before the first kernel of an entry point and after each.
void timing_mark(hipStream_t st);

// A side stream (per host thread and device, created on first use and kept,
// default priority) for work that overlaps the caller's stream.
// side_begin(main, k, side): the side stream waits for all work queued on
// `main` so far; side_end(main, k): `main` waits for all work queued on the side
// stream so far. k (0 or 1) selects the event pair, so two fork/join pairs can
// be in flight in one call.
hipError_t side_begin(hipStream_t main, int k, hipStream_t& side);
hipError_t side_end(hipStream_t main, int k);
constexpr int kDiagGrid = 256;   // persistent grid of the diagonal-gradient kernel

// ---------------------------------------------------------------------------
// Share geometry (host and device)
// ---------------------------------------------------------------------------

// Document bounds from cu_seqlens (non-decreasing, cu[0] = 0, cu[nd] = S).
__host__ __device__ inline int doc_lo_of(const int32_t* cu, int nd, int pos) {
  if (nd <= 1) return 0;
  int lo = 0, hi = nd;
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (cu[mid] <= pos) lo = mid; else hi = mid;
  }
  return cu[lo];
}
__host__ __device__ inline int doc_hi_of(const int32_t* cu, int nd, int pos, int S) {
  if (nd <= 1) return S;
  int lo = 0, hi = nd;
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (cu[mid] <= pos) lo = mid; else hi = mid;
  }
  return cu[hi];
}

// Query rows of a share come in runs of contiguous global positions:
//   full / head shard: one run, positions 0..T-1
//   contiguous rank r: one run, positions r*T .. r*T+T-1
//   zig-zag rank r: every document [dlo, dhi) (one document = the whole sequence)
//     is cut into 2cp chunks of c = (dhi - dlo) / 2cp; the share holds, document by
//     document, chunk r (early) then chunk 2cp-1-r (late) (zigzag_ring_attention
//     page: module text, and `get_half_index`, which picks the front and back half
//     of each varlen document), so document d's runs are 2d and 2d+1 and start at
//     local row dlo / cp.
// Block-0 K/V segments are visited in ring order: ring step j holds rank
// (r - j) mod cp's K/V, i.e. chunk src (contiguous) or, of the query's document,
// chunks {src, 2cp-1-src} (zig-zag).
struct Geo {
  int layout, cp, rank, T, Tkv;
  const int32_t* cu;   // global document boundaries (host or device copy), or null
  int nd;              // documents; <= 1: one document spanning the sequence

  __host__ __device__ bool multidoc() const { return nd > 1 && cu != nullptr; }
  __host__ __device__ int ndoc() const { return multidoc() ? nd : 1; }
  __host__ __device__ void doc(int d, int& dlo, int& dhi) const {
    if (multidoc()) {
      dlo = cu[d];
      dhi = cu[d + 1];
    } else {
      dlo = 0;
      dhi = Tkv;
    }
  }

  __host__ __device__ int nruns() const { return layout == LAYOUT_ZIGZAG ? 2 * ndoc() : 1; }

  __host__ __device__ void run(int i, int& lstart, int& len, int& gbase) const {
    if (layout == LAYOUT_ZIGZAG) {
      int dlo, dhi;
      doc(i >> 1, dlo, dhi);
      const int c = (dhi - dlo) / (2 * cp);
      const int late = i & 1;
      lstart = dlo / cp + late * c;
      len = c;
      gbase = dlo + (late ? 2 * cp - 1 - rank : rank) * c;
    } else {
      lstart = 0;
      len = T;
      gbase = (layout == LAYOUT_CONTIGUOUS) ? rank * T : 0;
    }
  }

  // Run holding local row `row` (zig-zag: the row's document, then its half).
  __host__ __device__ int run_of(int row) const {
    if (layout != LAYOUT_ZIGZAG) return 0;
    int d = 0;
    if (multidoc()) {
      int lo = 0, hi = nd;          // last document whose local start is <= row
      while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (cu[mid] / cp <= row) lo = mid; else hi = mid;
      }
      d = lo;
    }
    int dlo, dhi;
    doc(d, dlo, dhi);
    const int c = (dhi - dlo) / (2 * cp);
    return 2 * d + (row - dlo / cp >= c ? 1 : 0);
  }

  __host__ __device__ int nsteps() const {
    return (layout == LAYOUT_CONTIGUOUS || layout == LAYOUT_ZIGZAG) ? cp : 1;
  }

  // Whether block-0 key s is held at ring step `step` (rank (rank - step) mod cp's
  // K/V: its contiguous shard, or chunks {src, 2cp-1-src} of every document).
  __host__ __device__ bool in_step(int s, int step) const {
    if (layout == LAYOUT_CONTIGUOUS) {
      const int src = ((rank - step) % cp + cp) % cp;
      return s >= src * T && s < src * T + T;
    }
    if (layout == LAYOUT_ZIGZAG) {
      const int src = ((rank - step) % cp + cp) % cp;
      const int dlo = multidoc() ? doc_lo_of(cu, nd, s) : 0;
      const int dhi = multidoc() ? doc_hi_of(cu, nd, s, Tkv) : Tkv;
      const int c = (dhi - dlo) / (2 * cp);
      if (c == 0) return false;
      const int ch = (s - dlo) / c;
      return ch == src || ch == 2 * cp - 1 - src;
    }
    return step == 0;
  }
  __host__ __device__ int nparts() const { return layout == LAYOUT_ZIGZAG ? 2 : 1; }

  // Keys [a, b) of part `part` of ring step `step`; for the zig-zag layout, of the
  // document [dlo, dlo + dlen) the query lies in.
  __host__ __device__ void seg(int step, int part, int dlo, int dlen, int& a, int& b) const {
    if (layout == LAYOUT_CONTIGUOUS) {
      const int src = ((rank - step) % cp + cp) % cp;
      a = src * T;
      b = a + T;
    } else if (layout == LAYOUT_ZIGZAG) {
      const int c = dlen / (2 * cp);
      const int src = ((rank - step) % cp + cp) % cp;
      const int id = part == 0 ? src : 2 * cp - 1 - src;
      a = dlo + id * c;
      b = a + c;
    } else {
      a = 0;
      b = Tkv;
    }
  }

  // Padded per-(b, h) row layout of lse*log2(e) and delta: run i occupies
  // [P_i, P_i + roundup64(len_i)) with P_i = roundup4(lstart_i) + 68 i, so every
  // 64-row query tile of a run starts on a 16-byte boundary and tiles never
  // reach into the next run (P_{i+1} - P_i >= len_i + 65). One run: P_0 = 0.
  __host__ __device__ int run_pad_start(int i) const {
    int ls, len, gb;
    run(i, ls, len, gb);
    return (ls + 3) / 4 * 4 + 68 * i;
  }
  __host__ __device__ int prow(int row) const {
    if (layout != LAYOUT_ZIGZAG) return row;
    const int i = run_of(row);
    int ls, len, gb;
    run(i, ls, len, gb);
    return run_pad_start(i) + (row - ls);
  }
  // Positions per (b, h) of that layout (a multiple of 64).
  __host__ __device__ int pitch() const {
    const int n = nruns();
    int ls, len, gb;
    run(n - 1, ls, len, gb);
    const int p = run_pad_start(n - 1) + (len + 63) / 64 * 64;
    return (p + 63) / 64 * 64;
  }

  // Number of query tiles of height BM over all runs.
  __host__ __device__ int ntiles(int BM) const {
    int n = 0;
    for (int r = 0; r < nruns(); ++r) {
      int ls, len, gb;
      run(r, ls, len, gb);
      n += (len + BM - 1) / BM;
    }
    return n;
  }

  // Query tile in launch order: the latest global positions (the most block-0
  // keys) first. Returns the local first row, the row count and the global
  // position of the first row.
  __host__ __device__ void qtile(int order, int BM, int& row0, int& nrows, int& gpos0) const {
    int trank = order;
    for (int r = nruns() - 1; r >= 0; --r) {
      int ls, len, gb;
      run(r, ls, len, gb);
      const int nt = (len + BM - 1) / BM;
      if (trank < nt) {
        const int t = nt - 1 - trank;
        row0 = ls + t * BM;
        nrows = (len - t * BM) < BM ? (len - t * BM) : BM;
        gpos0 = gb + t * BM;
        return;
      }
      trank -= nt;
    }
    row0 = 0;
    nrows = 0;
    gpos0 = 0;
  }
};

// Walks the block-0 key tiles of width BN that a query tile can see: segment by
// segment in ring order, each segment clipped to the key window [wlo, whi).
// Tile starts are multiples of BN (one tile grid per head, so the tiles are shared in L2); keys
// of a tile outside [a, b) or outside a row's visible range are masked by the
// kernel. The window lies inside one document for the zig-zag layout (a query
// tile lies inside one chunk of one document), whose chunks give the segments.
struct SegIter {
  int step, part, a, b, s0, end, wlo, whi, dlo, dlen, shi;
  bool valid;

  __host__ __device__ void seek(const Geo& g, int BN) {
    while (true) {
      if (step >= shi) {
        valid = false;
        return;
      }
      g.seg(step, part, dlo, dlen, a, b);
      const int lo = a > wlo ? a : wlo;
      const int hi = b < whi ? b : whi;
      if (lo < hi) {
        s0 = (lo / BN) * BN;
        end = hi;
        valid = true;
        return;
      }
      if (++part >= g.nparts()) {
        part = 0;
        ++step;
      }
    }
  }
  // Ring steps [slo, shi) (clipped to the layout's steps).
  __host__ __device__ void begin(const Geo& g, int wlo_, int whi_, int BN, int slo = 0,
                                 int shi_ = 1 << 30) {
    wlo = wlo_;
    whi = whi_;
    step = slo;
    shi = shi_ < g.nsteps() ? shi_ : g.nsteps();
    part = 0;
    dlo = 0;
    dlen = g.Tkv;
    if (g.layout == LAYOUT_ZIGZAG && g.multidoc()) {
      dlo = doc_lo_of(g.cu, g.nd, wlo_);
      dlen = doc_hi_of(g.cu, g.nd, wlo_, g.Tkv) - dlo;
    }
    seek(g, BN);
  }
  __host__ __device__ void next(const Geo& g, int BN) {
    s0 += BN;
    if (s0 < end) return;
    if (++part >= g.nparts()) {
      part = 0;
      ++step;
    }
    seek(g, BN);
  }
};

// ---------------------------------------------------------------------------
// Device helpers
// ---------------------------------------------------------------------------
template <typename T> struct V8;
template <> struct V8<bf16> { typedef bf16x8 type; };
template <> struct V8<float> { typedef f32x8 type; };

// One k = 16 slice of a 32x32 output block. bf16: one v_mfma_f32_32x32x16_bf16.
// f32: eight v_mfma_f32_32x32x2_f32 over the same per-lane data (lane group g
// holds k = 8g + i in its i-th element; step i pairs element i of both groups).
__device__ __forceinline__ void mfma16(const bf16x8& a, const bf16x8& b, f32x16& c) {
  c = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ void mfma16(const f32x8& a, const f32x8& b, f32x16& c) {
#pragma unroll
  for (int i = 0; i < 8; ++i) c = __builtin_amdgcn_mfma_f32_32x32x2f32(a[i], b[i], c, 0, 0, 0);
}

// Waits for every outstanding memory operation of the wave. Placed before a
// main loop so the loop header starts with nothing pending from the prologue;
// otherwise the wait-count pass may merge the prologue's register loads into the
// loop and wait for the next tile's prefetch at the top of every iteration.
__device__ __forceinline__ void wait_all() { __builtin_amdgcn_s_waitcnt(0); }

// <a, b> + acc over 8 elements: four packed bf16 dot products (v_dot2_f32_bf16)
// or eight fp32 FMAs.
__device__ __forceinline__ float dot8(const bf16x8& a, const bf16x8& b, float acc) {
  typedef bf16 bf16x2 __attribute__((ext_vector_type(2)));
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(a, a, 0, 1), __builtin_shufflevector(b, b, 0, 1), acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(a, a, 2, 3), __builtin_shufflevector(b, b, 2, 3), acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(a, a, 4, 5), __builtin_shufflevector(b, b, 4, 5), acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(a, a, 6, 7), __builtin_shufflevector(b, b, 6, 7), acc, false);
  return acc;
}
__device__ __forceinline__ float dot8(const f32x8& a, const f32x8& b, float acc) {
#pragma unroll
  for (int e = 0; e < 8; ++e) acc = fmaf(a[e], b[e], acc);
  return acc;
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }

#define E3_DPP(x, ctrl) \
  __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, (x)), (ctrl), 0xF, 0xF, true))

// Sum over aligned groups of `W` lanes (W = 8 or 16); every lane gets the sum.
template <int W>
__device__ __forceinline__ float group_sum(float x) {
  x += E3_DPP(x, 0xB1);   // quad_perm [1,0,3,2]
  x += E3_DPP(x, 0x4E);   // quad_perm [2,3,0,1]
  x += E3_DPP(x, 0x141);  // row_half_mirror: the other quad of 8
  if constexpr (W == 16) x += E3_DPP(x, 0x140);  // row_mirror: the other half of 16
  return x;
}

__device__ __forceinline__ float xor32(float x) {
  return __shfl_xor(x, 32);
}

// An empty asm that takes and returns `x` in registers: the value has to be
// computed before this point and stays ordered with the other volatile asm and
// scheduling fences around it (it cannot be sunk into later blocks).
template <typename V>
__device__ __forceinline__ void pin(V& x) {
  asm volatile("" : "+v"(x));
}

// max / sum of the values of lanes l and l^32, in every lane: one
// v_permlane32_swap (VALU; no LDS round trip) and one combining op. The two
// halves add in the same order, so both get bit-identical sums.
__device__ __forceinline__ void swap32(float x, float& lo, float& hi) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  const unsigned a = r[0], b = r[1];     // copy out: bit-casting a vector element misreads it
  lo = __uint_as_float(a);               // value of lane l & 31
  hi = __uint_as_float(b);               // value of lane (l & 31) + 32
}
__device__ __forceinline__ float swap32_max(float x) {
  float lo, hi;
  swap32(x, lo, hi);
  return fmaxf(lo, hi);
}
__device__ __forceinline__ float swap32_sum(float x) {
  float lo, hi;
  swap32(x, lo, hi);
  return lo + hi;
}

// Convert 8 accumulator values (fp32) to an MFMA operand of element type T.
__device__ __forceinline__ bf16x8 to_op(const f32x16& v, int off, bf16) {
  bf16x8 r;
#pragma unroll
  for (int i = 0; i < 8; ++i) r[i] = (bf16)v[off + i];
  return r;
}
__device__ __forceinline__ f32x8 to_op(const f32x16& v, int off, float) {
  f32x8 r;
#pragma unroll
  for (int i = 0; i < 8; ++i) r[i] = v[off + i];
  return r;
}

template <typename T>
__device__ __forceinline__ typename V8<T>::type load8(const T* p) {
  return *reinterpret_cast<const typename V8<T>::type*>(p);
}
template <typename T>
__device__ __forceinline__ typename V8<T>::type zero8() {
  typename V8<T>::type r;
#pragma unroll
  for (int i = 0; i < 8; ++i) r[i] = (T)0.f;
  return r;
}
template <typename T>
__device__ __forceinline__ typename V8<T>::type ones8() {
  typename V8<T>::type r;
#pragma unroll
  for (int i = 0; i < 8; ++i) r[i] = (T)1.f;
  return r;
}
template <typename T>
__device__ __forceinline__ f32x8 load8f(const T* p) {
  const typename V8<T>::type v = load8(p);
  f32x8 r;
#pragma unroll
  for (int i = 0; i < 8; ++i) r[i] = (float)v[i];
  return r;
}
template <typename T>
__device__ __forceinline__ void store8f(T* p, const f32x8& v) {
  typename V8<T>::type r;
#pragma unroll
  for (int i = 0; i < 8; ++i) r[i] = (T)v[i];
  *reinterpret_cast<typename V8<T>::type*>(p) = r;
}
// Streaming (non-temporal) variants, for data touched once, so that it does
// not evict the working set of kernels running alongside.
template <typename T>
__device__ __forceinline__ typename V8<T>::type load8_nt(const T* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const typename V8<T>::type*>(p));
}
template <typename T>
__device__ __forceinline__ void store8f_nt(T* p, const f32x8& v) {
  typename V8<T>::type r;
#pragma unroll
  for (int i = 0; i < 8; ++i) r[i] = (T)v[i];
  __builtin_nontemporal_store(r, reinterpret_cast<typename V8<T>::type*>(p));
}

// ---------------------------------------------------------------------------
// Global -> LDS tile staging. A tile is R rows x D columns of T kept in LDS in
// its natural [row][col] layout (row stride chosen per tile to spread banks);
// thread t holds 4 consecutive rows x E columns in registers between the global
// load and the LDS store.
// ---------------------------------------------------------------------------
template <typename T, int E>
struct VecE {
  typedef T type __attribute__((ext_vector_type(E)));
};

template <typename T, int R, int D, int NT>
struct TileLoad {
  static constexpr int E = R * D / (NT * 4);
  static_assert(E >= 1 && (E & (E - 1)) == 0, "tile does not split evenly");
  static constexpr int CPR = D / E;       // column chunks per row
  typedef typename VecE<T, E>::type vec;
  vec r[4];

  // rows [row0, row0+R) of a [rows, H*D] tensor (row stride rs); rows at or past
  // `rows_valid` (relative to row0) read as zero.
  __device__ __forceinline__ void load(const T* base, long long rs, int rows_valid, int tid) {
    const int cc = tid % CPR, rg = tid / CPR;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int rr = rg * 4 + i;
      if (rr < rows_valid) {
        r[i] = *reinterpret_cast<const vec*>(base + (long long)rr * rs + cc * E);
      } else {
#pragma unroll
        for (int e = 0; e < E; ++e) r[i][e] = (T)0.f;
      }
    }
  }
  // Unguarded: all R rows exist.
  __device__ __forceinline__ void load_full(const T* base, long long rs, int tid) {
    const int cc = tid % CPR, rg = tid / CPR;
#pragma unroll
    for (int i = 0; i < 4; ++i)
      r[i] = *reinterpret_cast<const vec*>(base + (long long)(rg * 4 + i) * rs + cc * E);
  }
  __device__ __forceinline__ void store(T* lds, int stride, int tid) const {
    const int cc = tid % CPR, rg = tid / CPR;
#pragma unroll
    for (int i = 0; i < 4; ++i)
      *reinterpret_cast<vec*>(lds + (rg * 4 + i) * stride + cc * E) = r[i];
  }
};

// ---- swizzled LDS tiles filled by direct global->LDS loads -----------------
// A tile of rows of RB bytes is stored unpadded; the 16-byte chunk c of row r
// sits in chunk slot c ^ sw(r). sw is a multiple of U (16-byte chunks per MFMA
// operand: 1 for bf16, 2 for fp32), so an operand's chunks stay adjacent. Tiles
// are read two ways, and the masks serve both without bank conflicts (64 banks
// of 4 bytes):
//  - along a row (lds_sw8): 32 consecutive rows, one 16-byte chunk each. Any 16
//    consecutive rows must land in 16 distinct 16-byte bank groups;
//  - down the rows (ColRead, ds_read_b64_tr_b16): 8 rows r0 + {0..3, 4..7}
//    (r0 = 0 mod 8), the same 4 aligned chunks each. Each group of 4 rows must
//    cover all 16 bank groups once.
// 256-byte rows: sw = 4 (r mod 4) + (r / 4) mod 4 (measured on gfx950, 8 waves
// per CU: 214 B/clk for row reads, 160 for transposing reads, against 222 and
// 62 with sw = r mod 16). 128-byte rows (two rows per 256 bytes): sw =
// 4 ((r / 2) mod 2) + (r / 4) mod 4. 64-byte rows (row reads only): (r / 4) mod 4.
template <int RB, int U>
__device__ __forceinline__ int sw_mask(int r) {
  constexpr int CPR = RB / 16;
  if constexpr (CPR >= 16) return ((((r & 3) << 2) | ((r >> 2) & 3)) * U) & (CPR - 1);
  else if constexpr (CPR == 8) return (((((r >> 1) & 1) << 2) | ((r >> 2) & 3)) * U) & 7;
  else return (((r >> 2) & 3) * U) & (CPR - 1);
}

// LDS byte address of a pointer into __shared__ memory.
__device__ __forceinline__ unsigned lds_addr(const void* p) {
  typedef __attribute__((address_space(3))) const char lds_char;
  return (unsigned)(unsigned long)(lds_char*)p;
}

// A wave-uniform 64-bit value moved to scalar registers.
__device__ __forceinline__ unsigned long long uniform64(unsigned long long x) {
  const unsigned lo = __builtin_amdgcn_readfirstlane((unsigned)x);
  const unsigned hi = __builtin_amdgcn_readfirstlane((unsigned)(x >> 32));
  return ((unsigned long long)hi << 32) | lo;
}

// One global_load_lds_dwordx4: 16 bytes from `base` + `voff` (per lane) to LDS
// byte `lds` + 16 * lane (lds uniform). It has no register outputs; its
// completion is waited for with vmcnt. Written as asm because the compiler
// otherwise drops to lgkmcnt(0) for every LDS read issued while such a copy is
// in flight; the copies here are waited for with s_waitcnt 0 before the
// barrier that publishes them. Writing M0 needs one wait state before the load.
// `base` and `lds` must be the same in every lane (they are read from lane 0).
__device__ __forceinline__ void lds_dma16(const char* base, unsigned voff, unsigned lds) {
  const unsigned long long b = (unsigned long long)base;
  const unsigned blo = __builtin_amdgcn_readfirstlane((unsigned)b);
  const unsigned bhi = __builtin_amdgcn_readfirstlane((unsigned)(b >> 32));
  const char* const sbase = (const char*)(((unsigned long long)bhi << 32) | blo);
  const unsigned slds = __builtin_amdgcn_readfirstlane(lds);
  asm volatile(
      "s_mov_b32 m0, %2\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %0, %1"
      :
      : "v"(voff), "s"(sbase), "s"(slds)
      : "memory");
}

// Copy R rows of a tile to LDS byte address `lds` with global_load_lds_dwordx4 (no VGPR
// staging): each wave instruction writes 1 KB of LDS, lane i at byte 16 i, so
// lane i fetches the chunk that belongs in that slot. Row r of the tile is read
// at `base` + r * `stride` bytes (base uniform, the per-lane part 32-bit); rows
// at or past `nvalid` re-read row nvalid - 1. The copies complete
// asynchronously (vmcnt). The NW waves of the workgroup split the
// instructions; `w` (the wave index) should be wave-uniform in a scalar register.
template <int R, int RB, int NW = 4>
struct DmaShape {
  static constexpr int CPR = RB / 16;     // chunks per row
  static constexpr int RPI = 64 / CPR;    // rows per wave instruction
  static constexpr int NI = R / RPI / NW; // instructions per wave
  static_assert(NI >= 1 && NI * RPI * NW == R, "tile does not split over the waves");
};

// Instruction i (0 <= i < NI) of this wave's share of the copy (NW waves).
template <int R, int RB, int U, int NW = 4>
__device__ __forceinline__ void dma_tile_part(unsigned lds, const char* base, unsigned stride,
                                              int nvalid, int w, int lane, int i) {
  using S = DmaShape<R, RB, NW>;
  const int r0 = (w * S::NI + i) * S::RPI;
  const int rl = lane / S::CPR;
  if (nvalid >= R) {
    // Full tile: the row base is scalar, the lane part depends on r0 mod 16 only.
    const unsigned off =
        (unsigned)rl * stride + 16u * (unsigned)((lane % S::CPR) ^ sw_mask<RB, U>((r0 & 15) + rl));
    lds_dma16(base + (long long)r0 * stride, off, lds + (unsigned)(r0 * RB));
  } else {
    const int r = r0 + rl;
    const int rr = r < nvalid ? r : nvalid - 1;
    const unsigned off = (unsigned)rr * stride + 16u * (unsigned)((lane % S::CPR) ^ sw_mask<RB, U>(r));
    lds_dma16(base, off, lds + (unsigned)(r0 * RB));
  }
}

// Per-lane source offset of instruction i of this wave's share of a full-tile
// copy (all R rows valid), relative to the tile's first row: the same for every
// tile of a given stride, so a loop computes it once and then issues each copy
// from a scalar tile base (no per-copy address arithmetic).
template <int R, int RB, int U, int NW = 4>
__device__ __forceinline__ unsigned dma_full_off(unsigned stride, int w, int lane, int i) {
  using S = DmaShape<R, RB, NW>;
  const int r0 = (w * S::NI + i) * S::RPI;
  const int rl = lane / S::CPR;
  return (unsigned)(r0 + rl) * stride + 16u * (unsigned)((lane % S::CPR) ^ sw_mask<RB, U>((r0 & 15) + rl));
}

// LDS byte offset, within the tile, of instruction i of this wave's share.
template <int R, int RB, int NW = 4>
__device__ __forceinline__ unsigned dma_full_lds(int w, int i) {
  using S = DmaShape<R, RB, NW>;
  return (unsigned)((w * S::NI + i) * S::RPI * RB);
}

template <int R, int RB, int U, int NW = 4>
__device__ __forceinline__ void dma_tile(unsigned lds, const char* base, unsigned stride, int nvalid,
                                         int w, int lane) {
#pragma unroll
  for (int i = 0; i < DmaShape<R, RB, NW>::NI; ++i)
    dma_tile_part<R, RB, U, NW>(lds, base, stride, nvalid, w, lane, i);
}

// A wave's share of the copies of R-row tiles of one row stride. Full tiles are
// copied from a scalar tile base with per-lane offsets computed once here (no
// address arithmetic per copy); a partial tile takes dma_tile's clamped path.
template <int R, int RB, int U, int NW = 4>
struct TileDma {
  static constexpr int NI = DmaShape<R, RB, NW>::NI;
  unsigned off[NI];
  unsigned stride;
  int w, lane;
  __device__ __forceinline__ TileDma(unsigned stride_, int w_, int lane_) : stride(stride_), w(w_), lane(lane_) {
#pragma unroll
    for (int i = 0; i < NI; ++i) off[i] = dma_full_off<R, RB, U, NW>(stride, w, lane, i);
  }
  // Copy instruction i of a full tile whose first row is at `tile` (wave-uniform,
  // in scalar registers) to the tile at LDS byte address `lds`.
  __device__ __forceinline__ void part(unsigned lds, const char* tile, int i) const {
    lds_dma16(tile, off[i], lds + dma_full_lds<R, RB, NW>(w, i));
  }
  // The whole share of the copy of the tile at `base`; rows at or past `nvalid`
  // re-read row nvalid - 1.
  __device__ __forceinline__ void operator()(unsigned lds, const char* base, int nvalid) const {
    if (nvalid >= R) {
      const char* const tile = (const char*)uniform64((unsigned long long)base);
#pragma unroll
      for (int i = 0; i < NI; ++i) part(lds, tile, i);
    } else {
      dma_tile<R, RB, U, NW>(lds, base, stride, nvalid, w, lane);
    }
  }
};

// Runs the n MFMAs of a phase with their LDS operands read A steps ahead into a
// ring, one fence per step so the compiler keeps the reads ahead:
// `read(i)` returns operand i, `mma(i, op)` issues MFMA i.
template <int N, int A, typename Read, typename Mma>
__device__ __forceinline__ void mfma_ring(Read read, Mma mma) {
  using Op = decltype(read(0));
  Op ring[A + 1];
#pragma unroll
  for (int i = 0; i < A && i < N; ++i) ring[i] = read(i);
#pragma unroll
  for (int i = 0; i < N; ++i) {
    if (i + A < N) ring[(i + A) % (A + 1)] = read(i + A);
    mma(i, ring[i % (A + 1)]);
    __builtin_amdgcn_sched_barrier(0);
  }
}

// MFMA operand of 8 consecutive elements (columns col..col+7) of row `row` of a
// swizzled tile.
template <typename T, int RB>
__device__ __forceinline__ typename V8<T>::type lds_sw8(const char* tile, int row, int col) {
  constexpr int U = 8 * (int)sizeof(T) / 16;
  const int c = col * (int)sizeof(T) / 16;
  return *reinterpret_cast<const typename V8<T>::type*>(tile + row * RB +
                                                       16 * (c ^ sw_mask<RB, U>(row)));
}

// MFMA operand taken down the rows of a swizzled tile X[k][m] (rows of RB bytes):
// lane (m = l%32, g = l/32) gets X[k0 + o][c0 + m] for o = 4g..4g+3, 8+4g..8+4g+3,
// the row order in which a 32x32 accumulator holds its rows, so that an
// accumulator slice converted to T is the other operand. k0 is a multiple of 16
// and c0 of 32.
// bf16: two ds_read_b64_tr_b16. In each 16-lane group (j = l%16, h = (l/16)%2),
// source lane j reads the 4 elements c0 + 16h + 4(j%4) .. +3 of row k0 + 4g + j/4
// (then of that row + 8), and lane j receives element c0 + 16h + j of the 4 rows.
// The per-lane byte offsets are fixed for k0 = c0 = 0: since sw depends on r mod
// 16 only, rows k0 + o add k0 * RB, and since the lane's chunk (c0/8 + 2h +
// (j/2)%2) has c0/8 in bits the lane part leaves free, columns c0 + ... XOR the
// chunk slot with c0/8.
template <typename T, int RB>
struct ColRead;

template <int RB>
struct ColRead<bf16, RB> {
  unsigned o0, o1;
  __device__ __forceinline__ explicit ColRead(int lane) {
    const int g = lane >> 5, j = lane & 15, h = (lane >> 4) & 1;
    const int r = 4 * g + (j >> 2), c = 2 * h + ((j >> 1) & 1), byte = 8 * (j & 1);
    o0 = (unsigned)(r * RB + 16 * (c ^ sw_mask<RB, 1>(r)) + byte);
    o1 = (unsigned)((r + 8) * RB + 16 * (c ^ sw_mask<RB, 1>(r + 8)) + byte);
  }
  // `tile` must start at a multiple of 256 bytes of LDS: then the column XOR
  // (below 256) commutes with adding the tile address, and the row offset k0 * RB
  // (a multiple of 256) is an immediate offset of the read.
  __device__ __forceinline__ bf16x8 operator()(const char* tile, int k0, int c0) const {
    typedef short v4s __attribute__((ext_vector_type(4)));
    typedef __attribute__((address_space(3))) v4s lv4s;
    typedef __attribute__((address_space(3))) char lchar;
    const unsigned x = 2u * (unsigned)c0;          // 16 * (c0 / 8)
    lchar* const t = (lchar*)tile;
    const unsigned ta = (unsigned)(unsigned long)t;
    lchar* const pa = t + (((ta + o0) ^ x) - ta) + k0 * RB;
    lchar* const pb = t + (((ta + o1) ^ x) - ta) + k0 * RB;
    const v4s va = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lv4s*)pa);
    const v4s vb = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lv4s*)pb);
    // Whole-register concatenation (element-wise inserts cost a VALU op each).
    typedef short v8s __attribute__((ext_vector_type(8)));
    const v8s r = __builtin_shufflevector(va, vb, 0, 1, 2, 3, 4, 5, 6, 7);
    return __builtin_bit_cast(bf16x8, r);
  }
};

// fp32: eight scalar LDS reads (there is no transposing read of 32-bit
// elements), at per-lane offsets fixed for k0 = c0 = 0; c0 (a multiple of 32)
// XORs the chunk slot with c0/4 as in the bf16 case.
template <int RB>
struct ColRead<float, RB> {
  unsigned o[8];
  __device__ __forceinline__ explicit ColRead(int lane) {
    const int g = lane >> 5, m = lane & 31;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int r = (i < 4 ? 4 * g + i : 8 + 4 * g + i - 4);
      o[i] = (unsigned)(r * RB + 16 * ((m >> 2) ^ sw_mask<RB, 2>(r)) + 4 * (m & 3));
    }
  }
  __device__ __forceinline__ f32x8 operator()(const char* tile, int k0, int c0) const {
    const unsigned x = 4u * (unsigned)c0;          // 16 * (c0 / 4)
    const char* const base = tile + k0 * RB;
    f32x8 r;
#pragma unroll
    for (int i = 0; i < 8; ++i) r[i] = *reinterpret_cast<const float*>(base + (o[i] ^ x));
    return r;
  }
};

}  // namespace e3
