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
  static constexpr int KSTR = Stride<T, D>::nat;        // K tile [BN keys][D]
  static constexpr int VSTR = Stride<T, BN>::nat;       // V^T tile [D][BN keys]
  static constexpr int OSTR = D + 4;       // fp32 staging rows of the epilogue
  static constexpr int KS = D / 16;        // MFMA k-steps over D
  static constexpr int DB = D / 32;        // 32-row blocks of O^T
  static constexpr int STAGE = (BN * KSTR + D * VSTR) * (int)sizeof(T);
  static constexpr int LDS_KV = 2 * STAGE;
  static constexpr int LDS_EPI = 4 * 32 * OSTR * 4 + 2 * BM * 4;
  static constexpr int LDS = LDS_KV > LDS_EPI ? LDS_KV : LDS_EPI;
  static constexpr int NB = sizeof(T) == 2 ? 8 : 2;   // diagonal blocks per epilogue group
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
  const T* vtb = reinterpret_cast<const T*>(a.vt) + ((long long)b * a.H + h) * D * a.kv_pitch;

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
  auto vbuf = [&](int s) { return reinterpret_cast<T*>(smem + s * C::STAGE) + BN * C::KSTR; };  // V^T

  SegIter it;
  it.begin(geo, lo_min, g_max + 1, BN);
  TileLoad<T, BN, D, 256> kt;
  TileLoad<T, D, BN, 256> vt;   // V^T: D rows of BN key positions (zero padded)
  auto fetch = [&](int s0) {
    const int nv = a.Tkv - s0;
    if (nv >= BN) kt.load_full(k0b + (long long)s0 * rs, rs, tid);
    else kt.load(k0b + (long long)s0 * rs, rs, nv, tid);
    vt.load_full(vtb + s0, a.kv_pitch, tid);
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
  wait_all();
  __syncthreads();

  while (it.valid) {
    const int s0 = it.s0, sa = it.a, sb = it.b;
    const T* Ks = kbuf(stage);
    const T* Vs = vbuf(stage);

    // S^T for keys [s0, s0+64): two 32-key blocks, lane = query, 16 keys per block.
    // The two accumulator chains alternate and operands are read a step ahead.
    f32x16 st[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int j = 0; j < 16; ++j) st[kb][j] = 0.f;
    {
      Op a0 = lds_row8(Ks, C::KSTR, l32, 8 * g);
      Op a1 = lds_row8(Ks, C::KSTR, 32 + l32, 8 * g);
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        Op n0 = a0, n1 = a1;
        if (ks + 1 < KS) {
          n0 = lds_row8(Ks, C::KSTR, l32, 16 * (ks + 1) + 8 * g);
          n1 = lds_row8(Ks, C::KSTR, 32 + l32, 16 * (ks + 1) + 8 * g);
        }
        mfma16(a0, qreg[ks], st[0]);
        mfma16(a1, qreg[ks], st[1]);
        a0 = n0;
        a1 = n1;
      }
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
    {
      Op pv[BN / 16];
#pragma unroll
      for (int ks = 0; ks < BN / 16; ++ks) pv[ks] = to_op(st[ks >> 1], 8 * (ks & 1), T());
      Op va[DB];
#pragma unroll
      for (int db = 0; db < DB; ++db) va[db] = lds_row8(Vs, C::VSTR, 32 * db + l32, 8 * g);
#pragma unroll
      for (int ks = 0; ks < BN / 16; ++ks) {
#pragma unroll
        for (int db = 0; db < DB; ++db) {
          const Op cur = va[db];
          if (ks + 1 < BN / 16) va[db] = lds_row8(Vs, C::VSTR, 32 * db + l32, 16 * (ks + 1) + 8 * g);
          mfma16(cur, pv[ks], acc[db]);
        }
      }
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
  // Two row passes at a time, and all kd/vd loads of a group of NB blocks for
  // both issued before any is used (the epilogue is bound by memory latency).
  constexpr int LPR = D / 8;
  constexpr int RPP = 64 / LPR;
  constexpr int NB = C::NB;
  using V = typename V8<T>::type;
  const int lr = lane / LPR, cc = (lane % LPR) * 8;
  const T* kdb = reinterpret_cast<const T*>(a.kd) + (long long)b * a.kd_bs + (long long)h * D + cc;
  const T* vdb = reinterpret_cast<const T*>(a.vd) + (long long)b * a.kd_bs + (long long)h * D + cc;
  T* ob = reinterpret_cast<T*>(a.out) + (long long)b * a.T * rs + (long long)h * D + cc;
  float* lseb = a.lse + ((long long)b * a.H + h) * a.T;
  for (int pass = 0; pass < 32 / RPP; pass += 2) {
    bool ok[2];
    long long row[2];
    float m[2], l[2];
    f32x8 o[2];
    V qv[2];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int rr = (pass + u) * RPP + lr;
      const int tr = w * 32 + rr;
      ok[u] = tr < nrows;                      // whole row groups agree
      row[u] = row0 + (ok[u] ? tr : 0);
      m[u] = Ms[tr];
      l[u] = Ls[tr];
      o[u] = *reinterpret_cast<const f32x8*>(Ow + rr * C::OSTR + cc);
      qv[u] = load8(qb + row[u] * rs + cc);
    }
    for (int i0 = 0; i0 < a.N; i0 += NB) {
      const int n = (a.N - i0) < NB ? (a.N - i0) : NB;
      // Unconditional loads (block index clamped): conditional ones would be
      // waited for one at a time.
      V kv[2][NB], vv[2][NB];
#pragma unroll
      for (int i = 0; i < NB; ++i)
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          const long long off = (long long)(i0 + (i < n ? i : n - 1)) * a.kd_blk + row[u] * rs;
          kv[u][i] = load8(kdb + off);
          vv[u][i] = load8(vdb + off);
        }
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        float y[NB];
        float mg = m[u];
#pragma unroll
        for (int i = 0; i < NB; ++i) {
          const float d = group_sum<LPR>(dot8(qv[u], kv[u][i], 0.f));
          y[i] = i < n ? d * c2 : kNegInf;
          mg = fmaxf(mg, y[i]);
        }
        const float al = fast_exp2(m[u] - mg);
        l[u] *= al;
#pragma unroll
        for (int e = 0; e < 8; ++e) o[u][e] *= al;
#pragma unroll
        for (int i = 0; i < NB; ++i) {
          const float p = fast_exp2(y[i] - mg);
          l[u] += p;
#pragma unroll
          for (int e = 0; e < 8; ++e) o[u][e] = fmaf(p, (float)vv[u][i][e], o[u][e]);
        }
        m[u] = mg;
      }
    }
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      if (!ok[u]) continue;
      const float inv = 1.f / l[u];
#pragma unroll
      for (int e = 0; e < 8; ++e) o[u][e] *= inv;
      store8f(ob + row[u] * rs, o[u]);
      if ((lane % LPR) == 0) lseb[row[u]] = (m[u] + fast_log2(l[u])) * kLn2;
    }
  }
}

template <typename T, int D>
static hipError_t launch_fwd_t(const Args& a, hipStream_t st) {
  const Geo geo{a.layout, a.cp, a.rank, a.T, a.Tkv};
  const long long nt = (long long)geo.ntiles(FwdCfg<T, D>::BM) * a.B * a.H;
  if (nt == 0) return hipSuccess;
  timing_mark(st);
  hipError_t e = launch_xpose(a.v0, a.k0_bs, const_cast<void*>(a.vt), geo.kvruns(), a.B, a.H,
                              sizeof(T) == 2 ? 0 : 1, D, st);
  if (e != hipSuccess) return e;
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
