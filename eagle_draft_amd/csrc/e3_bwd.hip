// EAGLE-3 mixed attention, backward (gfx950).
//
// The backward runs against the MERGED joint-softmax out/lse (ring_attention page,
// `_CachedRingAttention`; ulysses_attention page, `_block0_backward`;
// zigzag_ring_attention page, `zigzag_ring_flash_attn_varlen_backward`), so block-0
// probabilities are P = exp(scale*q.k - lse) with the lse that includes the diagonal
// blocks, and the diagonal gradients follow in closed form.
//
// Three kernels, no atomics (every output element has one writer):
//   delta_kernel  delta[b,h,t] = <dO_t, O_t> (O = the stored merged out)
//   dkdv_kernel   one workgroup per 128 block-0 keys (32 per wave, lane = key);
//                 loops over the query tiles that see them:
//                   S = Q K^T, P, dP = dO V^T, dS = P (dP - delta),
//                   dV += P^T dO, dK += scale dS^T Q
//                 Q and dO tiles are staged in LDS both as-is and transposed.
//   dq_kernel     one workgroup per 128 query rows (lane = query, as in the
//                 forward); loops over the visible key tiles in ring order:
//                   dQ += dS K; then the epilogue adds the diagonal terms
//                   pi = exp(y - lse), dpi = <dO, vd>, ds = pi (dpi - delta),
//                   dq += scale ds kd, dkd = scale ds q, dvd = pi dO.
#include "e3_common.h"

namespace e3 {

// ---------------------------------------------------------------------------
// delta = rowsum(dO * O)
// ---------------------------------------------------------------------------
template <typename T, int D>
__global__ __launch_bounds__(256) void delta_kernel(const Args a) {
  constexpr int LPR = D / 8;
  constexpr int RPB = 256 / LPR;   // rows (b, t, h) per block
  const int lane = threadIdx.x;
  const long long r = (long long)blockIdx.x * RPB + lane / LPR;   // row over B*T*H
  const long long nrow = (long long)a.B * a.T * a.H;
  const bool valid = r < nrow;
  const long long rr = valid ? r : 0;
  const int cc = (lane % LPR) * 8;
  const f32x8 x = load8f(reinterpret_cast<const T*>(a.dout) + rr * D + cc);
  const f32x8 y = load8f(reinterpret_cast<const T*>(a.o_in) + rr * D + cc);
  float d = 0.f;
#pragma unroll
  for (int e = 0; e < 8; ++e) d += x[e] * y[e];
  d = group_sum<LPR>(d);
  if (valid && (lane % LPR) == 0) {
    const long long h = rr % a.H, bt = rr / a.H, t = bt % a.T, b = bt / a.T;
    a.delta[(b * a.H + h) * a.T + t] = d;
  }
}

// ---------------------------------------------------------------------------
// dK0 / dV0
// ---------------------------------------------------------------------------
template <typename T, int D>
struct DkdvCfg {
  static constexpr int BNK = 128;            // keys per workgroup (32 per wave)
  static constexpr int BMQ = 64;             // query rows per iteration
  static constexpr int STR = Stride<T, D>::both;   // Q and dO tiles are read both ways
  static constexpr int KS = D / 16;
  static constexpr int DB = D / 32;
  static constexpr int STAGE = 2 * BMQ * STR * (int)sizeof(T) + 2 * BMQ * 4;
  static constexpr int LDS = 2 * STAGE;
};

// Query tiles (rows of the share) that can see keys [k_lo, k_hi) with document
// end doc_end(k_hi - 1): per run, rows whose global position lies in
// [k_lo, dend). Tile starts are aligned to BMQ relative to the run start.
struct QIter {
  int run, ls, len, gb, t0, tend;
  int qlo, qhi;
  bool valid;
  __device__ void seek(const Geo& g, int BMQ) {
    while (run < g.nruns()) {
      g.run(run, ls, len, gb);
      const int lo = qlo > gb ? qlo : gb;
      const int hi = qhi < gb + len ? qhi : gb + len;
      if (lo < hi) {
        t0 = ((lo - gb) / BMQ) * BMQ;   // offset within the run
        tend = hi - gb;
        valid = true;
        return;
      }
      ++run;
    }
    valid = false;
  }
  __device__ void begin(const Geo& g, int qlo_, int qhi_, int BMQ) {
    qlo = qlo_;
    qhi = qhi_;
    run = 0;
    seek(g, BMQ);
  }
  __device__ void next(const Geo& g, int BMQ) {
    t0 += BMQ;
    if (t0 < tend) return;
    ++run;
    seek(g, BMQ);
  }
  __device__ int row0() const { return ls + t0; }
  __device__ int nrows(int BMQ) const { return (len - t0) < BMQ ? (len - t0) : BMQ; }
  __device__ int gpos0() const { return gb + t0; }
};

template <typename T, int D>
__global__ __launch_bounds__(256, 1) void dkdv_kernel(const Args a) {
  using C = DkdvCfg<T, D>;
  using Op = typename V8<T>::type;
  constexpr int BNK = C::BNK, BMQ = C::BMQ, KS = C::KS, DB = C::DB, STR = C::STR;
  __shared__ __attribute__((aligned(16))) char smem[C::LDS];
  auto qbuf = [&](int s) { return reinterpret_cast<T*>(smem + s * C::STAGE); };
  auto obuf = [&](int s) { return reinterpret_cast<T*>(smem + s * C::STAGE) + BMQ * STR; };
  auto lbuf = [&](int s) { return reinterpret_cast<float*>(smem + s * C::STAGE + 2 * BMQ * STR * (int)sizeof(T)); };

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, g = lane >> 5, l32 = lane & 31;
  const int BH = a.B * a.H;
  const int kt = tile_order(blockIdx.x / BH, (a.Tkv + BNK - 1) / BNK), bh = blockIdx.x % BH,
            b = bh / a.H, h = bh % a.H;
  const Geo geo{a.layout, a.cp, a.rank, a.T, a.Tkv};
  const int kt0 = kt * BNK;
  const int kt1 = (kt0 + BNK) < a.Tkv ? (kt0 + BNK) : a.Tkv;

  const long long rs = (long long)a.H * D;
  const T* k0b = reinterpret_cast<const T*>(a.k0) + (long long)b * a.k0_bs + (long long)h * D;
  const T* v0b = reinterpret_cast<const T*>(a.v0) + (long long)b * a.k0_bs + (long long)h * D;
  const T* qb = reinterpret_cast<const T*>(a.q) + (long long)b * a.T * rs + (long long)h * D;
  const T* dob = reinterpret_cast<const T*>(a.dout) + (long long)b * a.T * rs + (long long)h * D;
  const float* lseb = a.lse_in + ((long long)b * a.H + h) * a.T;
  const float* delb = a.delta + ((long long)b * a.H + h) * a.T;

  // This lane's key; a query at global position gm sees it iff s <= gm < s_hi.
  const int s = kt0 + w * 32 + l32;
  const bool svalid = s < a.Tkv;
  const int s_hi = svalid ? doc_hi_of(a.cu, a.ndocs, s, a.Tkv) : 0;
  Op kreg[KS], vreg[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    kreg[ks] = svalid ? load8(k0b + (long long)s * rs + 16 * ks + 8 * g) : zero8<T>();
    vreg[ks] = svalid ? load8(v0b + (long long)s * rs + 16 * ks + 8 * g) : zero8<T>();
  }
  const int hi_min = doc_hi_of(a.cu, a.ndocs, kt0, a.Tkv);   // smallest document end of the tile
  const int q_hi = doc_hi_of(a.cu, a.ndocs, kt1 - 1, a.Tkv);  // queries past this see no key

  f32x16 dk[DB], dv[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      dk[db][j] = 0.f;
      dv[db][j] = 0.f;
    }
  const float c2 = a.c2;

  QIter it;
  it.begin(geo, kt0, q_hi, BMQ);
  TileLoad<T, BMQ, D, 256> qt, ot;
  float lv = 0.f, dl = 0.f;
  auto fetch = [&](const QIter& q) {
    const int r0 = q.row0(), nr = q.nrows(BMQ);
    if (nr == BMQ) {
      qt.load_full(qb + (long long)r0 * rs, rs, tid);
      ot.load_full(dob + (long long)r0 * rs, rs, tid);
    } else {
      qt.load(qb + (long long)r0 * rs, rs, nr, tid);
      ot.load(dob + (long long)r0 * rs, rs, nr, tid);
    }
    if (tid < BMQ) {
      lv = tid < nr ? lseb[r0 + tid] * kLog2e : 0.f;
      dl = tid < nr ? delb[r0 + tid] : 0.f;
    }
  };
  auto put = [&](int st) {
    qt.store(qbuf(st), STR, tid);
    ot.store(obuf(st), STR, tid);
    if (tid < BMQ) {
      lbuf(st)[tid] = lv;
      lbuf(st)[BMQ + tid] = dl;
    }
  };
  int stage = 0;
  if (it.valid) {
    fetch(it);
    put(0);
  }
  QIter nx = it;
  if (nx.valid) nx.next(geo, BMQ);
  if (nx.valid) fetch(nx);
  wait_all();
  __syncthreads();

  while (it.valid) {
    const int nr = it.nrows(BMQ), gq0 = it.gpos0();
    const T* Qs = qbuf(stage);
    const T* Os = obuf(stage);
    const float* L2s = lbuf(stage);
    const float* Ds = L2s + BMQ;

    // S = Q K^T and dP = dO V^T: two 32-query blocks, lane = key, 16 queries each.
    f32x16 sp[2], dp[2];
#pragma unroll
    for (int mb = 0; mb < 2; ++mb) {
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        sp[mb][j] = 0.f;
        dp[mb][j] = 0.f;
      }
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        mfma16(lds_row8(Qs, STR, 32 * mb + l32, 16 * ks + 8 * g), kreg[ks], sp[mb]);
        mfma16(lds_row8(Os, STR, 32 * mb + l32, 16 * ks + 8 * g), vreg[ks], dp[mb]);
      }
    }
    const bool interior = nr == BMQ && kt0 + BNK <= a.Tkv && gq0 >= kt0 + BNK - 1 &&
                          gq0 + BMQ - 1 < hi_min;
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const int m0 = 32 * mb + 8 * jj + 4 * g;
        const f32x4 l4 = *reinterpret_cast<const f32x4*>(L2s + m0);
        const f32x4 d4 = *reinterpret_cast<const f32x4*>(Ds + m0);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int j = 4 * jj + i;
          float p = fast_exp2(fmaf(sp[mb][j], c2, -l4[i]));
          if (!interior) {
            const int m = m0 + i, gm = gq0 + m;
            const bool vis = svalid && m < nr && gm >= s && gm < s_hi;
            p = vis ? p : 0.f;
          }
          sp[mb][j] = p;
          dp[mb][j] = p * (dp[mb][j] - d4[i]);
        }
      }
    // dV^T += dO^T P, dK^T += Q^T dS over the 64 queries (4 k-steps of 16).
#pragma unroll
    for (int ks = 0; ks < BMQ / 16; ++ks) {
      const Op pb = to_op(sp[ks >> 1], 8 * (ks & 1), T());
      const Op sb = to_op(dp[ks >> 1], 8 * (ks & 1), T());
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        mfma16(lds_col8(Os, STR, 16 * ks, 32 * db, lane), pb, dv[db]);
        mfma16(lds_col8(Qs, STR, 16 * ks, 32 * db, lane), sb, dk[db]);
      }
    }

    it = nx;
    if (it.valid) {
      put(stage ^ 1);
      nx.next(geo, BMQ);
      if (nx.valid) fetch(nx);
    }
    stage ^= 1;
    __syncthreads();
  }

  // Write dK0 = scale * dK, dV0 (rows of keys no query sees are zeros).
  if (svalid) {
    T* dkb = reinterpret_cast<T*>(a.dk0) + (long long)b * a.k0_bs + (long long)h * D + (long long)s * rs;
    T* dvb = reinterpret_cast<T*>(a.dv0) + (long long)b * a.k0_bs + (long long)h * D + (long long)s * rs;
    typedef typename VecE<T, 4>::type v4;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        v4 x, y;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          x[i] = (T)(dk[db][4 * jj + i] * a.scale);
          y[i] = (T)dv[db][4 * jj + i];
        }
        const int d0 = 32 * db + 8 * jj + 4 * g;
        *reinterpret_cast<v4*>(dkb + d0) = x;
        *reinterpret_cast<v4*>(dvb + d0) = y;
      }
  }
}

// ---------------------------------------------------------------------------
// dQ (block 0) + closed-form diagonal gradients
// ---------------------------------------------------------------------------
template <typename T, int D>
struct DqCfg {
  static constexpr int BM = 128;
  static constexpr int BN = 64;
  static constexpr int KSTR = Stride<T, D>::both;  // K is read both ways
  static constexpr int VSTR = Stride<T, D>::nat;
  static constexpr int OSTR = D + 4;
  static constexpr int KS = D / 16;
  static constexpr int DB = D / 32;
  static constexpr int STAGE = (BN * KSTR + BN * VSTR) * (int)sizeof(T);
  static constexpr int LDS_KV = 2 * STAGE;
  static constexpr int LDS_EPI = 4 * 32 * OSTR * 4;
  static constexpr int LDS = LDS_KV > LDS_EPI ? LDS_KV : LDS_EPI;
  static constexpr int NB = sizeof(T) == 2 ? 8 : 2;   // diagonal blocks per epilogue group
};

#ifndef E3_DQ_OCC
#define E3_DQ_OCC 2
#endif

template <typename T, int D>
__global__ __launch_bounds__(256, E3_DQ_OCC) void dq_kernel(const Args a) {
  using C = DqCfg<T, D>;
  using Op = typename V8<T>::type;
  constexpr int BM = C::BM, BN = C::BN, KS = C::KS, DB = C::DB;
  __shared__ __attribute__((aligned(16))) char smem[C::LDS];
  auto kbuf = [&](int s) { return reinterpret_cast<T*>(smem + s * C::STAGE); };
  auto vbuf = [&](int s) { return reinterpret_cast<T*>(smem + s * C::STAGE) + BN * C::KSTR; };

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, g = lane >> 5, l32 = lane & 31;
  const int BH = a.B * a.H;
  const int trank = blockIdx.x / BH, bh = blockIdx.x % BH, b = bh / a.H, h = bh % a.H;
  const Geo geo{a.layout, a.cp, a.rank, a.T, a.Tkv};
  int row0, nrows, gpos0;
  geo.qtile(trank, BM, row0, nrows, gpos0);

  const long long rs = (long long)a.H * D;
  const T* qb = reinterpret_cast<const T*>(a.q) + (long long)b * a.T * rs + (long long)h * D;
  const T* dob = reinterpret_cast<const T*>(a.dout) + (long long)b * a.T * rs + (long long)h * D;
  const T* k0b = reinterpret_cast<const T*>(a.k0) + (long long)b * a.k0_bs + (long long)h * D;
  const T* v0b = reinterpret_cast<const T*>(a.v0) + (long long)b * a.k0_bs + (long long)h * D;
  const float* lseb = a.lse_in + ((long long)b * a.H + h) * a.T;
  const float* delb = a.delta + ((long long)b * a.H + h) * a.T;

  const int qr = w * 32 + l32;
  const bool qvalid = qr < nrows;
  const int gq = gpos0 + qr;
  const int loq = doc_lo_of(a.cu, a.ndocs, qvalid ? gq : gpos0);
  const int g_min = gpos0, g_max = gpos0 + nrows - 1;
  const int lo_min = doc_lo_of(a.cu, a.ndocs, g_min);
  const int lo_max = doc_lo_of(a.cu, a.ndocs, g_max);
  const float lq = qvalid ? lseb[row0 + qr] * kLog2e : 0.f;
  const float dq_delta = qvalid ? delb[row0 + qr] : 0.f;

  Op qreg[KS], oreg[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    const long long off = (long long)(row0 + qr) * rs + 16 * ks + 8 * g;
    qreg[ks] = qvalid ? load8(qb + off) : zero8<T>();
    oreg[ks] = qvalid ? load8(dob + off) : zero8<T>();
  }
  f32x16 acc[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int j = 0; j < 16; ++j) acc[db][j] = 0.f;
  const float c2 = a.c2;

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

    // One 32-key block at a time: S^T, dP^T, then dS^T as two MFMA operands.
    const bool interior = s0 >= sa && s0 + BN <= sb && s0 >= lo_max && s0 + BN - 1 <= g_min;
    Op dsop[BN / 16];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      f32x16 st, dpt;
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        st[j] = 0.f;
        dpt[j] = 0.f;
      }
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        mfma16(lds_row8(Ks, C::KSTR, 32 * kb + l32, 16 * ks + 8 * g), qreg[ks], st);
        mfma16(lds_row8(Vs, C::VSTR, 32 * kb + l32, 16 * ks + 8 * g), oreg[ks], dpt);
      }
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        float p = fast_exp2(fmaf(st[j], c2, -lq));
        if (!interior) {
          const int s = s0 + 32 * kb + 8 * (j >> 2) + 4 * g + (j & 3);
          const bool vis = s >= sa && s < sb && s >= loq && s <= gq;
          p = vis ? p : 0.f;
        }
        dpt[j] = p * (dpt[j] - dq_delta);
      }
      dsop[2 * kb] = to_op(dpt, 0, T());
      dsop[2 * kb + 1] = to_op(dpt, 8, T());
    }
    // dQ^T += K^T dS^T over the 64 keys (4 k-steps of 16).
#pragma unroll
    for (int ks = 0; ks < BN / 16; ++ks)
#pragma unroll
      for (int db = 0; db < DB; ++db)
        mfma16(lds_col8(Ks, C::KSTR, 16 * ks, 32 * db, lane), dsop[ks], acc[db]);

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

  // ---- epilogue: stage dQ^T through LDS, then the diagonal terms row-major ----
  float* Qw = reinterpret_cast<float*>(smem) + w * 32 * C::OSTR;
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      f32x4 v;
      v[0] = acc[db][4 * jj + 0];
      v[1] = acc[db][4 * jj + 1];
      v[2] = acc[db][4 * jj + 2];
      v[3] = acc[db][4 * jj + 3];
      *reinterpret_cast<f32x4*>(Qw + l32 * C::OSTR + 32 * db + 8 * jj + 4 * g) = v;
    }
  __syncthreads();

  // All kd/vd loads of a group of NB blocks are issued before any is used.
  constexpr int LPR = D / 8;
  constexpr int RPP = 64 / LPR;
  constexpr int NB = C::NB;
  using V = typename V8<T>::type;
  const int lr = lane / LPR, cc = (lane % LPR) * 8;
  const T* kdb = reinterpret_cast<const T*>(a.kd) + (long long)b * a.kd_bs + (long long)h * D + cc;
  const T* vdb = reinterpret_cast<const T*>(a.vd) + (long long)b * a.kd_bs + (long long)h * D + cc;
  T* dkdb = reinterpret_cast<T*>(a.dkd) + (long long)b * a.kd_bs + (long long)h * D + cc;
  T* dvdb = reinterpret_cast<T*>(a.dvd) + (long long)b * a.kd_bs + (long long)h * D + cc;
  T* dqb = reinterpret_cast<T*>(a.dq) + (long long)b * a.T * rs + (long long)h * D + cc;
  const float scale = a.scale;
  for (int pass = 0; pass < 32 / RPP; ++pass) {
    const int rr = pass * RPP + lr;
    const int tr = w * 32 + rr;
    const bool ok = tr < nrows;              // whole row groups agree
    const long long row = row0 + (ok ? tr : 0);
    f32x8 dqv = *reinterpret_cast<const f32x8*>(Qw + rr * C::OSTR + cc);
    const V qv = load8(qb + row * rs + cc);
    const V ov = load8(dob + row * rs + cc);
    const float l2 = lseb[row] * kLog2e;
    const float dl = delb[row];
    for (int i0 = 0; i0 < a.N; i0 += NB) {
      const int n = (a.N - i0) < NB ? (a.N - i0) : NB;
      // Unconditional loads (block index clamped): conditional ones would be
      // waited for one at a time.
      V kv[NB], vv[NB];
#pragma unroll
      for (int i = 0; i < NB; ++i) {
        const long long off = (long long)(i0 + (i < n ? i : n - 1)) * a.kd_blk + row * rs;
        kv[i] = load8(kdb + off);
        vv[i] = load8(vdb + off);
      }
#pragma unroll
      for (int i = 0; i < NB; ++i) {
        const float y = group_sum<LPR>(dot8(qv, kv[i], 0.f));
        const float dpi = group_sum<LPR>(dot8(ov, vv[i], 0.f));
        const float pi = i < n ? fast_exp2(y * c2 - l2) : 0.f;
        const float ds = pi * (dpi - dl);
        const float sds = scale * ds;
        f32x8 gk, gv;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          dqv[e] = fmaf(ds, (float)kv[i][e], dqv[e]);
          gk[e] = sds * (float)qv[e];
          gv[e] = pi * (float)ov[e];
        }
        if (ok && i < n) {
          const long long off = (long long)(i0 + i) * a.kd_blk + row * rs;
          store8f(dkdb + off, gk);
          store8f(dvdb + off, gv);
        }
      }
    }
    if (ok) {
#pragma unroll
      for (int e = 0; e < 8; ++e) dqv[e] *= scale;
      store8f(dqb + row * rs, dqv);
    }
  }
}

template <typename T, int D>
static hipError_t launch_bwd_t(const Args& a, hipStream_t st) {
  const long long nrow = (long long)a.B * a.T * a.H;
  timing_mark(st);
  if (nrow > 0) {
    const long long nb = (nrow + (256 / (D / 8)) - 1) / (256 / (D / 8));
    hipLaunchKernelGGL((delta_kernel<T, D>), dim3((unsigned)nb), dim3(256), 0, st, a);
    timing_mark(st);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  const long long nk = (long long)((a.Tkv + DkdvCfg<T, D>::BNK - 1) / DkdvCfg<T, D>::BNK) * a.B * a.H;
  if (nk > 0) {
    hipLaunchKernelGGL((dkdv_kernel<T, D>), dim3((unsigned)nk), dim3(256), 0, st, a);
    timing_mark(st);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  const Geo geo{a.layout, a.cp, a.rank, a.T, a.Tkv};
  const long long nq = (long long)geo.ntiles(DqCfg<T, D>::BM) * a.B * a.H;
  if (nq > 0) {
    hipLaunchKernelGGL((dq_kernel<T, D>), dim3((unsigned)nq), dim3(256), 0, st, a);
    timing_mark(st);
    return hipGetLastError();
  }
  return hipSuccess;
}

hipError_t launch_bwd(const Args& a, int dtype, int D, hipStream_t st) {
  if (dtype == 0) return D == 128 ? launch_bwd_t<bf16, 128>(a, st) : launch_bwd_t<bf16, 64>(a, st);
  return D == 128 ? launch_bwd_t<float, 128>(a, st) : launch_bwd_t<float, 64>(a, st);
}

}  // namespace e3
