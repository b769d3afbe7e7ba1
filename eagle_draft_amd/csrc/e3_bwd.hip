// EAGLE-3 mixed attention, backward (gfx950).
//
// The backward runs against the MERGED joint-softmax out/lse (ring_attention page,
// `_CachedRingAttention`; ulysses_attention page, `_block0_backward`;
// zigzag_ring_attention page, `zigzag_ring_flash_attn_varlen_backward`), so block-0
// probabilities are P = exp(scale*q.k - lse) with the lse that includes the diagonal
// blocks, and the diagonal gradients follow in closed form.
//
// Kernels, no atomics (every output element has one writer):
//   delta_kernel  delta[b,h,t] = <dO_t, O_t> (O = the stored merged out) and
//                 lse2 = lse * log2(e), in the 64-aligned per-run row layout
//   xpose (x2)    Q^T and dO^T copies (e3_xpose.hip) for the dK/dV operands
//   dkdv_kernel   one workgroup per 128 block-0 keys (32 per wave, lane = key);
//                 loops over the query tiles that see them:
//                   S = Q K^T, P, dP = dO V^T, dS = P (dP - delta),
//                   dV += P^T dO, dK += scale dS^T Q
//                 Q / dO tiles and their transposes stream through swizzled
//                 LDS stages filled by direct global->LDS copies; the S / dP
//                 MFMAs of tile j+1 overlap the P / dS arithmetic of tile j.
//   dq_kernel     one workgroup per 128 query rows (lane = query, as in the
//                 forward); loops over the visible key tiles in ring order:
//                   dQ += dS K; then the epilogue adds the diagonal terms
//                   pi = exp(y - lse), dpi = <dO, vd>, ds = pi (dpi - delta),
//                   dq += scale ds kd, dkd = scale ds q, dvd = pi dO.
#include "e3_common.h"

namespace e3 {

// ---------------------------------------------------------------------------
// delta = rowsum(dO * O), lse2 = lse * log2(e); one row per LPR lanes, rows in
// the padded layout [b][h][p] (padding positions get 0)
// ---------------------------------------------------------------------------
template <typename T, int D>
__global__ __launch_bounds__(256) void delta_kernel(const Args a) {
  constexpr int LPR = D / 8;
  constexpr int RPB = 256 / LPR;   // rows per block
  const Geo geo{a.layout, a.cp, a.rank, a.T, a.Tkv};
  const int lane = threadIdx.x;
  const int qp = a.q_pitch;
  const long long r = (long long)blockIdx.x * RPB + lane / LPR;   // over B*H*qp
  const long long nrow = (long long)a.B * a.H * qp;
  const bool valid = r < nrow;
  const long long rr = valid ? r : 0;
  const int bh = (int)(rr / qp), p = (int)(rr % qp), b = bh / a.H, h = bh % a.H;
  const int t = geo.trow(p);
  const int cc = (lane % LPR) * 8;
  float d = 0.f;
  if (t >= 0) {
    const long long off = (((long long)b * a.T + t) * a.H + h) * D + cc;
    const f32x8 x = load8f(reinterpret_cast<const T*>(a.dout) + off);
    const f32x8 y = load8f(reinterpret_cast<const T*>(a.o_in) + off);
#pragma unroll
    for (int e = 0; e < 8; ++e) d += x[e] * y[e];
  }
  d = group_sum<LPR>(d);
  if (valid && (lane % LPR) == 0) {
    a.delta[rr] = d;
    a.lse2[rr] = t >= 0 ? a.lse_in[(long long)bh * a.T + t] * kLog2e : 0.f;
  }
}

// ---------------------------------------------------------------------------
// dK0 / dV0
// ---------------------------------------------------------------------------
template <typename T, int D>
struct DkdvCfg {
  static constexpr int BNK = 128;            // keys per workgroup (32 per wave)
  static constexpr int BMQ = 32;            // queries per step
  static constexpr int MB = BMQ / 32;        // 32-query blocks per step
  static constexpr int KS = D / 16;
  static constexpr int DB = D / 32;
  static constexpr int U = 8 * (int)sizeof(T) / 16;     // 16-byte chunks per operand
  static constexpr int RRB = D * (int)sizeof(T);        // row tiles Q, dO [BMQ][D]: row bytes
  static constexpr int CRB = BMQ * (int)sizeof(T);      // column tiles Q^T, dO^T [D][BMQ]
  static constexpr int RT = BMQ * RRB, CT = D * CRB;     // bytes per tile
  static constexpr int RSTAGE = 2 * RT;                 // Q, dO
  static constexpr int CSTAGE = 2 * CT;                 // Q^T, dO^T
  static constexpr int LSTAGE = 2 * BMQ * 4;            // lse2, delta
  // The tile stages come first so that every operand read addresses them with
  // one lane register and an immediate offset (below 64 KB).
  static constexpr int LDS = 2 * RSTAGE + 2 * CSTAGE + 2 * LSTAGE;
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
  constexpr int BNK = C::BNK, BMQ = C::BMQ, MB = C::MB, KS = C::KS, DB = C::DB;
  constexpr int sz = (int)sizeof(T);
  __shared__ __attribute__((aligned(16))) char smem[C::LDS];
  // Row stages hold Q at 0 and dO at RT; column stages hold Q^T at 0 and dO^T
  // at CT; each column stage has an lse2 / delta stage (BMQ floats each).
  char* const rb0 = smem;
  char* const rb1 = rb0 + C::RSTAGE;
  char* const cb0 = rb1 + C::RSTAGE;
  char* const cb1 = cb0 + C::CSTAGE;
  char* const lb0 = cb1 + C::CSTAGE;
  auto lstage = [&](const char* cb) { return lb0 + (cb == cb0 ? 0 : C::LSTAGE); };
  const unsigned sbase = lds_addr(smem);
  auto la = [&](const char* p) { return sbase + (unsigned)(p - smem); };

  const int tid = threadIdx.x, lane = tid & 63, g = lane >> 5, l32 = lane & 31;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int BH = a.B * a.H;
  const int kt = tile_order(blockIdx.x / BH, (a.Tkv + BNK - 1) / BNK), bh = blockIdx.x % BH,
            b = bh / a.H, h = bh % a.H;
  const Geo geo{a.layout, a.cp, a.rank, a.T, a.Tkv};
  const int kt0 = kt * BNK;
  const int kt1 = (kt0 + BNK) < a.Tkv ? (kt0 + BNK) : a.Tkv;

  const long long rs = (long long)a.H * D;
  const T* k0b = reinterpret_cast<const T*>(a.k0) + (long long)b * a.k0_bs + (long long)h * D;
  const T* v0b = reinterpret_cast<const T*>(a.v0) + (long long)b * a.k0_bs + (long long)h * D;
  const char* const qbytes =
      reinterpret_cast<const char*>(reinterpret_cast<const T*>(a.q) + (long long)b * a.T * rs + (long long)h * D);
  const char* const obytes =
      reinterpret_cast<const char*>(reinterpret_cast<const T*>(a.dout) + (long long)b * a.T * rs + (long long)h * D);
  const long long cbase = (long long)bh * D * a.q_pitch;
  const char* const qtbytes = reinterpret_cast<const char*>(reinterpret_cast<const T*>(a.qt) + cbase);
  const char* const otbytes = reinterpret_cast<const char*>(reinterpret_cast<const T*>(a.dot) + cbase);
  const char* const lbytes = reinterpret_cast<const char*>(a.lse2 + (long long)bh * a.q_pitch);
  const unsigned ldoff = (unsigned)((long long)BH * a.q_pitch * 4);   // lse2 -> delta
  const unsigned rrow = (unsigned)(rs * sz), crow = (unsigned)((long long)a.q_pitch * sz);

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

  auto dma_rows = [&](char* dst, const QIter& q) {
    const int r0 = q.row0(), nr = q.nrows(BMQ);
    dma_tile<BMQ, C::RRB, C::U>(la(dst), qbytes + (long long)r0 * rrow, rrow, nr, w, lane);
    dma_tile<BMQ, C::RRB, C::U>(la(dst) + C::RT, obytes + (long long)r0 * rrow, rrow, nr, w, lane);
  };
  auto dma_cols = [&](char* dst, const QIter& q) {
    const int p0 = geo.prow(q.row0());
    dma_tile<D, C::CRB, C::U>(la(dst), qtbytes + (long long)p0 * sz, crow, D, w, lane);
    dma_tile<D, C::CRB, C::U>(la(dst) + C::CT, otbytes + (long long)p0 * sz, crow, D, w, lane);
    if (w == 0 && lane < BMQ / 2) {
      const unsigned voff = lane < BMQ / 4 ? 16u * lane : ldoff + 16u * (lane - BMQ / 4);
      lds_dma16(lbytes + (long long)p0 * 4, voff, la(lstage(dst)));
    }
  };
  // S^T-like scores and dP for a row stage: lane = key, 16 queries per block.
  auto sdp = [&](const char* R, f32x16 (&sp)[MB], f32x16 (&dp)[MB]) {
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        sp[mb][j] = 0.f;
        dp[mb][j] = 0.f;
      }
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) {
        mfma16(lds_sw8<T, C::RRB>(R, 32 * mb + l32, 16 * ks + 8 * g), kreg[ks], sp[mb]);
        mfma16(lds_sw8<T, C::RRB>(R + C::RT, 32 * mb + l32, 16 * ks + 8 * g), vreg[ks], dp[mb]);
      }
  };
  auto interior = [&](const QIter& q) {
    const int gq0 = q.gpos0();
    return q.nrows(BMQ) == BMQ && kt0 + BNK <= a.Tkv && gq0 >= kt0 + BNK - 1 &&
           gq0 + BMQ - 1 < hi_min;
  };
  // Query m of the tile (m = 4g + o, o = 32mb + 8(j/4) + j%4 a constant per
  // element) sees this lane's key when mlo <= m <= mhi.
  auto mask = [&](f32x16 (&sp)[MB], const QIter& q) {
    const int gq0 = q.gpos0(), nr = q.nrows(BMQ);
    const int lo = s - gq0 - 4 * g;
    const int hi = (svalid ? ((nr < s_hi - gq0 ? nr : s_hi - gq0) - 1) : -1) - 4 * g;
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const int o = 32 * mb + 8 * (j >> 2) + (j & 3);
        sp[mb][j] = (o >= lo && o <= hi) ? sp[mb][j] : kNegInf;
      }
  };

  QIter it, i1, i2;
  it.begin(geo, kt0, q_hi, BMQ);
  i1 = it;
  if (i1.valid) i1.next(geo, BMQ);
  i2 = i1;
  if (i2.valid) i2.next(geo, BMQ);
  if (it.valid) {
    dma_rows(rb0, it);
    dma_cols(cb0, it);
  }
  if (i1.valid) dma_rows(rb1, i1);
  wait_all();
  __syncthreads();
  f32x16 sa[MB], da[MB], sb[MB], dbb[MB];
  if (it.valid) sdp(rb0, sa, da);
  __syncthreads();   // the first step overwrites row stage 0

  // Step j: S(j), dP(j) in registers; rows of tile j+1 and columns of tile j in
  // LDS. Starts the copies of rows(j+2) and columns(j+1) into the stages step
  // j-1 finished with. Phase A: S, dP of tile j+1 on MFMA while P(j), dS(j) are
  // formed on VALU; phase B: dV += dO^T P, dK += Q^T dS for tile j.
  auto step = [&](f32x16 (&sc)[MB], f32x16 (&dc)[MB], f32x16 (&sn)[MB], f32x16 (&dn)[MB],
                  const char* Rn, const char* Cc, char* Rw, char* Cw) {
    // Copies of rows(j+2) and columns(j+1), one instruction at a time between
    // the phase A MFMAs (a missing tile re-copies the current one into the free
    // stage, so the sequence has no branches).
    constexpr int NR = DmaShape<BMQ, C::RRB>::NI, NC = DmaShape<D, C::CRB>::NI;
    constexpr int NDMA = 2 * NR + 2 * NC + 1;
    const int dr0 = (i2.valid ? i2 : it).row0(), dnr = (i2.valid ? i2 : it).nrows(BMQ);
    const int dp0 = geo.prow((i1.valid ? i1 : it).row0());
    const unsigned lrw = la(Rw), lcw = la(Cw);
    auto dma_part = [&](int k) {
      if (k < NR) {
        dma_tile_part<BMQ, C::RRB, C::U>(lrw, qbytes + (long long)dr0 * rrow, rrow, dnr, w, lane, k);
      } else if (k < 2 * NR) {
        dma_tile_part<BMQ, C::RRB, C::U>(lrw + C::RT, obytes + (long long)dr0 * rrow, rrow, dnr, w, lane, k - NR);
      } else if (k < 2 * NR + NC) {
        dma_tile_part<D, C::CRB, C::U>(lcw, qtbytes + (long long)dp0 * sz, crow, D, w, lane, k - 2 * NR);
      } else if (k < 2 * NR + 2 * NC) {
        dma_tile_part<D, C::CRB, C::U>(lcw + C::CT, otbytes + (long long)dp0 * sz, crow, D, w, lane,
                                       k - 2 * NR - NC);
      } else if (w == 0 && lane < BMQ / 2) {
        const unsigned voff = lane < BMQ / 4 ? 16u * lane : ldoff + 16u * (lane - BMQ / 4);
        lds_dma16(lbytes + (long long)dp0 * 4, voff, la(lstage(Cw)));
      }
    };
    if (!interior(it)) mask(sc, it);
    const float* L2s = reinterpret_cast<const float*>(lstage(Cc));
    const float* Ds = L2s + BMQ;
    // lse2 / delta of the tile's queries, 4 at a time (group e/4 of the lane's
    // elements), read one group ahead.
    auto ld4 = [&](int grp, f32x4& l, f32x4& d) {
      const int off = 32 * (grp >> 2) + 8 * (grp & 3) + 4 * g;
      l = *reinterpret_cast<const f32x4*>(L2s + off);
      d = *reinterpret_cast<const f32x4*>(Ds + off);
    };
    // Phase A. MFMA i: ks = i / (2 MB), block mb, S (even) or dP (odd); its
    // A operand is read two MFMAs ahead. E elements of P / dS per lane spread
    // over the NQ steps.
    Op pb[BMQ / 16], sbo[BMQ / 16];
    {
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int j = 0; j < 16; ++j) {
          sn[mb][j] = 0.f;
          dn[mb][j] = 0.f;
        }
      constexpr int NQ = 2 * MB * KS, E = 16 * MB;
      auto opnd = [&](int i) {
        const int ks = i / (2 * MB), mb = (i / 2) % MB;
        return lds_sw8<T, C::RRB>(Rn + (i & 1) * C::RT, 32 * mb + l32, 16 * ks + 8 * g);
      };
      Op ka[3];
      ka[0] = opnd(0);
      ka[1] = opnd(1);
      f32x4 lg[2], dg[2];
      ld4(0, lg[0], dg[0]);
#pragma unroll
      for (int i = 0; i < NQ; ++i) {
        if (i + 2 < NQ) ka[(i + 2) % 3] = opnd(i + 2);
        {
          const int ks = i / (2 * MB), mb = (i / 2) % MB;
          if (i & 1) mfma16(ka[i % 3], vreg[ks], dn[mb]);
          else mfma16(ka[i % 3], kreg[ks], sn[mb]);
        }
#pragma unroll
        for (int k = (NDMA * i + NQ - 1) / NQ; k < (NDMA * (i + 1) + NQ - 1) / NQ; ++k) dma_part(k);
#pragma unroll
        for (int e = (E * i) / NQ; e < (E * (i + 1)) / NQ; ++e) {
          const int mb = e >> 4, j = e & 15, grp = e >> 2;
          if ((e & 3) == 0 && grp + 1 < E / 4) ld4(grp + 1, lg[(grp + 1) & 1], dg[(grp + 1) & 1]);
          const float p = fast_exp2(fmaf(sc[mb][j], c2, -lg[grp & 1][j & 3]));
          sc[mb][j] = p;
          dc[mb][j] = p * (dc[mb][j] - dg[grp & 1][j & 3]);
        }
#pragma unroll
        for (int q = 0; q < BMQ / 16; ++q)
          if ((E * (i + 1)) / NQ >= 8 * (q + 1) && (E * i) / NQ < 8 * (q + 1)) {
            pb[q] = to_op(sc[q >> 1], 8 * (q & 1), T());
            sbo[q] = to_op(dc[q >> 1], 8 * (q & 1), T());
            pin(pb[q]);
            pin(sbo[q]);
          }
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    // Phase B: dV^T += dO^T P^T and dK^T += Q^T dS^T over the BMQ queries.
    // Step k = (ks, db) issues the two MFMAs of one 32-row block of D; its
    // operands are read two steps ahead.
    {
      constexpr int NK = (BMQ / 16) * DB;
      auto vop = [&](int k) {
        return lds_sw8<T, C::CRB>(Cc + C::CT, 32 * (k % DB) + l32, 16 * (k / DB) + 8 * g);
      };
      auto qop = [&](int k) {
        return lds_sw8<T, C::CRB>(Cc, 32 * (k % DB) + l32, 16 * (k / DB) + 8 * g);
      };
      Op va[3], qa[3];
      va[0] = vop(0);
      qa[0] = qop(0);
      va[1] = vop(1);
      qa[1] = qop(1);
#pragma unroll
      for (int k = 0; k < NK; ++k) {
        if (k + 2 < NK) {
          va[(k + 2) % 3] = vop(k + 2);
          qa[(k + 2) % 3] = qop(k + 2);
        }
        mfma16(va[k % 3], pb[k / DB], dv[k % DB]);
        mfma16(qa[k % 3], sbo[k / DB], dk[k % DB]);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    // The next tile's S / dP become the current ones (accumulator -> VALU registers).
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
      sc[mb] = sn[mb];
      dc[mb] = dn[mb];
    }
    it = i1;
    i1 = i2;
    if (i2.valid) i2.next(geo, BMQ);
    wait_all();
    __syncthreads();
  };
  // One step per iteration; the stages alternate with the step parity.
  for (int par = 0; it.valid; par ^= 1) {
    const int odd = __builtin_amdgcn_readfirstlane(par);
    step(sa, da, sb, dbb, odd ? rb0 : rb1, odd ? cb1 : cb0, odd ? rb1 : rb0, odd ? cb0 : cb1);
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
  // lse2 / delta rows in the padded layout; the tile lies inside one run.
  const float* lseb = a.lse2 + (long long)bh * a.q_pitch + (geo.prow(row0) - row0);
  const float* delb = a.delta + (long long)bh * a.q_pitch + (geo.prow(row0) - row0);

  const int qr = w * 32 + l32;
  const bool qvalid = qr < nrows;
  const int gq = gpos0 + qr;
  const int loq = doc_lo_of(a.cu, a.ndocs, qvalid ? gq : gpos0);
  const int g_min = gpos0, g_max = gpos0 + nrows - 1;
  const int lo_min = doc_lo_of(a.cu, a.ndocs, g_min);
  const int lo_max = doc_lo_of(a.cu, a.ndocs, g_max);
  const float lq = qvalid ? lseb[row0 + qr] : 0.f;
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
    const float l2 = lseb[row];
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
  const Geo geo{a.layout, a.cp, a.rank, a.T, a.Tkv};
  const long long nrow = (long long)a.B * a.H * a.q_pitch;
  if (nrow == 0) return hipSuccess;
  timing_mark(st);
  {
    const long long nb = (nrow + (256 / (D / 8)) - 1) / (256 / (D / 8));
    hipLaunchKernelGGL((delta_kernel<T, D>), dim3((unsigned)nb), dim3(256), 0, st, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  timing_mark(st);
  {
    const long long qbs = (long long)a.T * a.H * D;
    hipError_t e = launch_xpose(a.q, qbs, const_cast<void*>(a.qt), geo.qruns(), a.B, a.H,
                                sizeof(T) == 2 ? 0 : 1, D, st);
    if (e == hipSuccess)
      e = launch_xpose(a.dout, qbs, const_cast<void*>(a.dot), geo.qruns(), a.B, a.H,
                       sizeof(T) == 2 ? 0 : 1, D, st);
    if (e != hipSuccess) return e;
  }
  timing_mark(st);
  const long long nk = (long long)((a.Tkv + DkdvCfg<T, D>::BNK - 1) / DkdvCfg<T, D>::BNK) * a.B * a.H;
  if (nk > 0) {
    hipLaunchKernelGGL((dkdv_kernel<T, D>), dim3((unsigned)nk), dim3(256), 0, st, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  timing_mark(st);
  const long long nq = (long long)geo.ntiles(DqCfg<T, D>::BM) * a.B * a.H;
  if (nq > 0) {
    hipLaunchKernelGGL((dq_kernel<T, D>), dim3((unsigned)nq), dim3(256), 0, st, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  timing_mark(st);
  return hipSuccess;
}

hipError_t launch_bwd(const Args& a, int dtype, int D, hipStream_t st) {
  if (dtype == 0) return D == 128 ? launch_bwd_t<bf16, 128>(a, st) : launch_bwd_t<bf16, 64>(a, st);
  return D == 128 ? launch_bwd_t<float, 128>(a, st) : launch_bwd_t<float, 64>(a, st);
}

}  // namespace e3
