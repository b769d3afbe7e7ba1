// EAGLE-3 mixed attention, forward (gfx950).
//
// One workgroup = 4 waves = a tile of 128 query rows of one (batch row, head);
// each wave owns 32 rows. Block 0 (ring_attention page, `_CachedRingAttention`;
// ulysses_attention page, `_block0_forward`): the wave computes S^T = K Q^T on
// MFMA 32x32x16 so that every lane holds ONE query row (row max and row sum are
// lane-local plus one exchange with lane^32), keeps (m, l, O^T) in registers and
// walks the K/V tiles the share can see in ring order, skipping masked tiles and
// masking only boundary tiles. K/V tiles are double-buffered in LDS in their
// natural layout; V^T operands come from transposing LDS reads. The running max
// is only moved (and O, l rescaled) when a row's max grows by more than 2^8, which
// leaves the result exact and skips most rescales. The diagonal TTT blocks
// (ring_attention page, `_merge_diag`) are merged in the epilogue: O is staged
// through LDS into a row-major mapping (16 lanes per row, 8 columns each) so kd/vd
// rows are read with coalesced 16-byte loads, each diagonal score is one dot
// product, and out = O/l and lse = m + log l are written once.
#include "e3_common.h"

namespace e3 {

template <typename T, int D>
struct FwdCfg {
  static constexpr int NT = 256;
  static constexpr int BM = 128;
  static constexpr int BN = 64;
  static constexpr int KSTR = Stride<T, D>::nat;
  static constexpr int VSTR = Stride<T, D>::col;
  static constexpr int OSTR = D + 4;       // fp32 staging rows of the epilogue
  static constexpr int KS = D / 16;        // MFMA k-steps over D
  static constexpr int DB = D / 32;        // 32-row blocks of O^T
  static constexpr int STAGE = (BN * KSTR + BN * VSTR) * (int)sizeof(T);
  static constexpr int LDS_KV = 2 * STAGE;
  static constexpr int LDS_EPI = 4 * 32 * OSTR * 4 + 2 * BM * 4;
  static constexpr int LDS = LDS_KV > LDS_EPI ? LDS_KV : LDS_EPI;
  static constexpr int NB = sizeof(T) == 2 ? 8 : 4;   // diagonal blocks per epilogue group
};

constexpr float kRescaleSlack = 8.0f;      // log2 of the largest un-rescaled growth

template <typename T, int D>
__global__ __launch_bounds__(256, 2) void fwd_kernel(const Args a) {
  using C = FwdCfg<T, D>;
  using Op = typename V8<T>::type;
  constexpr int BM = C::BM, BN = C::BN, KS = C::KS, DB = C::DB;
  __shared__ __attribute__((aligned(16))) char smem[C::LDS];

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, g = lane >> 5, l32 = lane & 31;
  const int BH = a.B * a.H;
  const int trank = blockIdx.x / BH, bh = blockIdx.x % BH, b = bh / a.H, h = bh % a.H;
  const Geo geo{a.layout, a.cp, a.rank, a.T, a.Tkv};
  int row0, nrows, gpos0;
  geo.qtile(trank, BM, row0, nrows, gpos0);

  const long long rs = (long long)a.H * D;
  const T* qb = reinterpret_cast<const T*>(a.q) + (long long)b * a.T * rs + (long long)h * D;
  const T* k0b = reinterpret_cast<const T*>(a.k0) + (long long)b * a.k0_bs + (long long)h * D;
  const T* v0b = reinterpret_cast<const T*>(a.v0) + (long long)b * a.k0_bs + (long long)h * D;

  // This lane's query row.
  const int qr = w * 32 + l32;
  const bool qvalid = qr < nrows;
  const int gq = gpos0 + qr;
  const int loq = doc_lo_of(a.cu, a.ndocs, qvalid ? gq : gpos0);
  // Key window of the tile and the bounds used to recognise unmasked tiles.
  const int g_min = gpos0, g_max = gpos0 + nrows - 1;
  const int lo_min = doc_lo_of(a.cu, a.ndocs, g_min);
  const int lo_max = doc_lo_of(a.cu, a.ndocs, g_max);

  Op qreg[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks)
    qreg[ks] = qvalid ? load8(qb + (long long)(row0 + qr) * rs + 16 * ks + 8 * g) : zero8<T>();

  f32x16 acc[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int j = 0; j < 16; ++j) acc[db][j] = 0.f;
  float m_i = kNegInf, l_i = 0.f;
  const float c2 = a.c2;

  auto kbuf = [&](int s) { return reinterpret_cast<T*>(smem + s * C::STAGE); };
  auto vbuf = [&](int s) { return reinterpret_cast<T*>(smem + s * C::STAGE) + BN * C::KSTR; };

  SegIter it;
  it.begin(geo, lo_min, g_max + 1, BN);
  TileLoad<T, BN, D, 256> kt, vt;
  auto fetch = [&](int s0) {
    const int nv = a.Tkv - s0;
    if (nv >= BN) {
      kt.load_full(k0b + (long long)s0 * rs, rs, tid);
      vt.load_full(v0b + (long long)s0 * rs, rs, tid);
    } else {
      kt.load(k0b + (long long)s0 * rs, rs, nv, tid);
      vt.load(v0b + (long long)s0 * rs, rs, nv, tid);
    }
  };
  // Prologue: tile 0 into stage 0, tile 1 into registers.
  int stage = 0;
  if (it.valid) {
    fetch(it.s0);
    kt.store(kbuf(0), C::KSTR, tid);
    vt.store(vbuf(0), C::VSTR, tid);
  }
  SegIter nx = it;
  if (nx.valid) nx.next(geo, BN);
  if (nx.valid) fetch(nx.s0);
  __syncthreads();

  while (it.valid) {
    const int s0 = it.s0, sa = it.a, sb = it.b;
    const T* Ks = kbuf(stage);
    const T* Vs = vbuf(stage);

    // S^T for keys [s0, s0+64): two 32-key blocks, lane = query, 16 keys per block.
    f32x16 st[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
      for (int j = 0; j < 16; ++j) st[kb][j] = 0.f;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
        mfma16(lds_row8(Ks, C::KSTR, 32 * kb + l32, 16 * ks + 8 * g), qreg[ks], st[kb]);
    }
    const bool interior = s0 >= sa && s0 + BN <= sb && s0 >= lo_max && s0 + BN - 1 <= g_min;
    float mx = kNegInf;
    if (interior) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int j = 0; j < 16; ++j) mx = fmaxf(mx, st[kb][j]);
    } else {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int j = 0; j < 16; ++j) {
          const int s = s0 + 32 * kb + 8 * (j >> 2) + 4 * g + (j & 3);
          const bool vis = s >= sa && s < sb && s >= loq && s <= gq;
          st[kb][j] = vis ? st[kb][j] : kNegInf;
          mx = fmaxf(mx, st[kb][j]);
        }
    }
    mx = fmaxf(mx, xor32(mx)) * c2;     // this tile's row max, base-2 scaled
    if (__any(mx > m_i + kRescaleSlack)) {
      const float m_new = fmaxf(m_i, mx);
      const float alpha = m_new == kNegInf ? 1.f : fast_exp2(m_i - m_new);
      l_i *= alpha;
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int j = 0; j < 16; ++j) acc[db][j] *= alpha;
      m_i = m_new;
    }
    const float nb = m_i == kNegInf ? 0.f : -m_i;
    float rsum = 0.f;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const float p = fast_exp2(fmaf(st[kb][j], c2, nb));
        st[kb][j] = p;
        rsum += p;
      }
    l_i += rsum;
    // O^T += V^T P^T over the 64 keys (4 k-steps of 16).
#pragma unroll
    for (int ks = 0; ks < BN / 16; ++ks) {
      const Op pv = to_op(st[ks >> 1], 8 * (ks & 1), T());
#pragma unroll
      for (int db = 0; db < DB; ++db)
        mfma16(lds_col8(Vs, C::VSTR, 16 * ks, 32 * db, lane), pv, acc[db]);
    }

    // Next tile: registers -> the other stage; fetch the one after.
    it = nx;
    if (it.valid) {
      kt.store(kbuf(stage ^ 1), C::KSTR, tid);
      vt.store(vbuf(stage ^ 1), C::VSTR, tid);
      nx.next(geo, BN);
      if (nx.valid) fetch(nx.s0);
    }
    stage ^= 1;
    __syncthreads();
  }
  l_i += xor32(l_i);

  // ---- epilogue: stage O^T (unnormalised), m, l through LDS ----------------
  float* Ow = reinterpret_cast<float*>(smem) + w * 32 * C::OSTR;
  float* Ms = reinterpret_cast<float*>(smem) + 4 * 32 * C::OSTR;
  float* Ls = Ms + BM;
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      f32x4 v;
      v[0] = acc[db][4 * jj + 0];
      v[1] = acc[db][4 * jj + 1];
      v[2] = acc[db][4 * jj + 2];
      v[3] = acc[db][4 * jj + 3];
      *reinterpret_cast<f32x4*>(Ow + l32 * C::OSTR + 32 * db + 8 * jj + 4 * g) = v;
    }
  if (g == 0) {
    Ms[qr] = m_i;
    Ls[qr] = l_i;
  }
  __syncthreads();

  // ---- diagonal blocks, row-major: LPR lanes per row, 8 columns per lane ----
  // All kd/vd loads of a group of NB blocks are issued before any is used.
  constexpr int LPR = D / 8;
  constexpr int RPP = 64 / LPR;
  constexpr int NB = C::NB;
  const int lr = lane / LPR, cc = (lane % LPR) * 8;
  const T* kdb = reinterpret_cast<const T*>(a.kd) + (long long)b * a.kd_bs + (long long)h * D + cc;
  const T* vdb = reinterpret_cast<const T*>(a.vd) + (long long)b * a.kd_bs + (long long)h * D + cc;
  T* ob = reinterpret_cast<T*>(a.out) + (long long)b * a.T * rs + (long long)h * D + cc;
  float* lseb = a.lse + ((long long)b * a.H + h) * a.T;
  for (int pass = 0; pass < 32 / RPP; ++pass) {
    const int rr = pass * RPP + lr;
    const int tr = w * 32 + rr;
    const bool ok = tr < nrows;                // whole row groups agree
    const long long row = row0 + (ok ? tr : 0);
    float m = Ms[tr], l = Ls[tr];
    f32x8 o = *reinterpret_cast<const f32x8*>(Ow + rr * C::OSTR + cc);
    const f32x8 qv = load8f(qb + row * rs + cc);
    for (int i0 = 0; i0 < a.N; i0 += NB) {
      const int n = (a.N - i0) < NB ? (a.N - i0) : NB;
      typename V8<T>::type kv[NB], vv[NB];
#pragma unroll
      for (int i = 0; i < NB; ++i)
        if (i < n) {
          const long long off = (long long)(i0 + i) * a.kd_blk + row * rs;
          kv[i] = load8(kdb + off);
          vv[i] = load8(vdb + off);
        }
      float y[NB];
      float mg = m;
#pragma unroll
      for (int i = 0; i < NB; ++i)
        if (i < n) {
          float d = 0.f;
#pragma unroll
          for (int e = 0; e < 8; ++e) d += qv[e] * (float)kv[i][e];
          y[i] = group_sum<LPR>(d) * c2;
          mg = fmaxf(mg, y[i]);
        }
      const float al = fast_exp2(m - mg);
      l *= al;
#pragma unroll
      for (int e = 0; e < 8; ++e) o[e] *= al;
#pragma unroll
      for (int i = 0; i < NB; ++i)
        if (i < n) {
          const float p = fast_exp2(y[i] - mg);
          l += p;
#pragma unroll
          for (int e = 0; e < 8; ++e) o[e] += p * (float)vv[i][e];
        }
      m = mg;
    }
    if (ok) {
      const float inv = 1.f / l;
#pragma unroll
      for (int e = 0; e < 8; ++e) o[e] *= inv;
      store8f(ob + row * rs, o);
      if ((lane % LPR) == 0) lseb[row] = (m + fast_log2(l)) * kLn2;
    }
  }
}

template <typename T, int D>
static hipError_t launch_fwd_t(const Args& a, hipStream_t st) {
  const Geo geo{a.layout, a.cp, a.rank, a.T, a.Tkv};
  const long long nt = (long long)geo.ntiles(FwdCfg<T, D>::BM) * a.B * a.H;
  if (nt == 0) return hipSuccess;
  timing_mark(st);
  hipLaunchKernelGGL((fwd_kernel<T, D>), dim3((unsigned)nt), dim3(256), 0, st, a);
  timing_mark(st);
  return hipGetLastError();
}

hipError_t launch_fwd(const Args& a, int dtype, int D, hipStream_t st) {
  if (dtype == 0) return D == 128 ? launch_fwd_t<bf16, 128>(a, st) : launch_fwd_t<bf16, 64>(a, st);
  return D == 128 ? launch_fwd_t<float, 128>(a, st) : launch_fwd_t<float, 64>(a, st);
}

int fwd_tile_rows() { return 128; }
int fwd_tile_keys() { return 64; }

}  // namespace e3
