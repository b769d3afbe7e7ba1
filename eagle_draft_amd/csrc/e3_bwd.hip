// EAGLE-3 mixed attention, backward (gfx950).
//
// The backward takes the out/lse of the WHOLE joint softmax (ring_attention page,
// `_CachedRingAttention`; ulysses_attention page, `_block0_backward`;
// zigzag_ring_attention page, `zigzag_ring_flash_attn_varlen_backward`), so block-0
// probabilities are P = exp(scale*q.k - lse) with the lse that includes the diagonal
// blocks, and the diagonal gradients follow in closed form.
//
// Kernels, no atomics (every output element has one writer):
//   dkdv_kernel   one workgroup per 128 block-0 keys (lane = key); loops over
//                 the query tiles that see them:
//                   S = Q K^T, P, dP = dO V^T, dS = P (dP - delta),
//                   dV += P^T dO, dK += scale dS^T Q
//                 Q / dO tiles stream through swizzled LDS stages filled by
//                 direct global->LDS copies and are read both along their rows
//                 and, with transposing reads, down them; one wave of each pair
//                 forms P and dV, the other dP, dS and dK, so the two waves
//                 sharing a SIMD overlap their MFMA and VALU phases.
//   diag_bwd_kernel  (side stream, after dQ, overlapping dK/dV) the closed-form
//                 diagonal terms pi = exp(y - lse), dpi = <dO, vd>,
//                 ds = pi (dpi - delta): dkd = scale ds q, dvd = pi dO, and
//                 dq = (float32 partial from dQ) + scale sum_i ds_i kd_i
//   dq_kernel     one workgroup per 128 query rows (lane = query, as in the
//                 forward); first writes delta[b,h,t] = <dO_t, O_t> (O = the
//                 stored merged out) and lse2 = lse * log2(e) of its rows in the
//                 64-aligned per-run row layout; then loops over the visible
//                 64-key tiles (32 for float32) in ring order
//                 (K and V staged in swizzled LDS by direct copies; K^T read
//                 down the K tile): dQ += dS K (float32 partial when there are
//                 diagonals).
#include "e3_common.h"


namespace e3 {

// ---------------------------------------------------------------------------
// dK0 / dV0
// ---------------------------------------------------------------------------
template <typename T, int D>
struct DkdvCfg {
  static constexpr int NT = 512;             // 8 waves: 4 that form P, 4 that form dS
  static constexpr int NW = NT / 64;
  static constexpr int BNK = 128;            // keys per workgroup (32 per wave of each kind)
  static constexpr int BMQ = sizeof(T) == 2 ? 64 : 32;   // queries per step
  static constexpr int MB = BMQ / 32;        // 32-query blocks per step
  static constexpr int KS = D / 16;
  static constexpr int DB = D / 32;
  static constexpr int U = 8 * (int)sizeof(T) / 16;     // 16-byte chunks per operand
  static constexpr int RRB = D * (int)sizeof(T);        // tiles Q, dO [BMQ][D]: row bytes
  static constexpr int RT = BMQ * RRB;                  // bytes per tile
  static constexpr int STAGE = 2 * RT;                  // Q, dO
  static constexpr int LSTAGE = 2 * BMQ * 4;            // lse2, delta
  static constexpr int PW = 64 * 16 * MB * (int)sizeof(T);   // P of one wave (per lane: 16 MB values)
  static constexpr int NS = 3;                          // Q / dO stages
  static constexpr int LDS = NS * STAGE + NS * LSTAGE + 2 * 4 * PW;   // + two P buffers
};

// Query tiles (rows of the share) that can see keys [k_lo, k_hi) with document
// end doc_end(k_hi - 1): per run, rows whose global position lies in
// [k_lo, dend). Tile starts are aligned to BMQ relative to the run start.
struct QIter {
  int run, ls, len, gb, t0, tend, pst;
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
        pst = (ls + 3) / 4 * 4 + 68 * run;   // = Geo::run_pad_start(run)
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
  __device__ int prow0() const { return pst + t0; }   // = Geo::prow(row0())
};

// Waves 0-3 ("P" waves) hold K for their 32 keys and form S = Q K^T, P and
// dV += dO^T P; waves 4-7 ("dS" waves) hold V for the same keys and form
// dP = dO V^T, dS = P (dP - delta) and dK += Q^T dS, taking P from the P wave of
// their keys through LDS. Wave w and w + 4 share a SIMD, so the exponentials of
// one overlap the MFMAs of the other. Both kinds run the same MFMA code on
// different tiles (read along the rows of Q or dO, then down the rows of dO or
// Q) and share registers.
// KVACC: ring-step mode (only the keys of the launch's ring step, added into
// float32 accumulators). ZZD: a zig-zag share of several documents (query runs
// per document). Separate instantiations keep the common one within the
// registers that let the diagonal-gradient kernel share its SIMDs.
template <typename T, int D, bool KVACC, bool ZZD>
__global__ __launch_bounds__(512, 1) void dkdv_kernel(const Args a) {
  using C = DkdvCfg<T, D>;
  using Op = typename V8<T>::type;
  constexpr int BNK = C::BNK, BMQ = C::BMQ, MB = C::MB, KS = C::KS, DB = C::DB, NW = C::NW;
  constexpr int sz = (int)sizeof(T);
  __shared__ __attribute__((aligned(16))) char smem[C::LDS];
  // Stage p: Q at 0, dO at RT. Then the three lse2 / delta stages and the two
  // sets of P exchange buffers.
  char* const lb0 = smem + C::NS * C::STAGE;
  char* const pbuf = lb0 + C::NS * C::LSTAGE;
  const unsigned sbase = lds_addr(smem);

  const int tid = threadIdx.x, lane = tid & 63, g = lane >> 5, l32 = lane & 31;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int role = w >> 2;   // 0: S, P, dV   1: dP, dS, dK
  const int kw = w & 3;      // 32-key block
  // Issue priority: the P wave of a SIMD ahead of its dS wave (its exponentials
  // gate the dS wave), both ahead of the diagonal-gradient waves that share the
  // SIMDs (memory-bound; they fill the issue gaps).
  if (role == 0) __builtin_amdgcn_s_setprio(2);
  else __builtin_amdgcn_s_setprio(1);
  const int BH = a.B * a.H;
  const int kt = blockIdx.x / BH, bh = blockIdx.x % BH,
            b = bh / a.H, h = bh % a.H;
  // (the document table matters for the query runs only in a multi-document zig-zag share)
  const Geo geo{a.layout, a.cp, a.rank, a.T, a.Tkv, ZZD ? a.cu : nullptr, ZZD ? a.ndocs : 1};
  const int kt0 = kt * BNK;
  const int kt1 = (kt0 + BNK) < a.Tkv ? (kt0 + BNK) : a.Tkv;

  const long long rs = (long long)a.H * D;
  const T* kvb = reinterpret_cast<const T*>(role ? a.v0 : a.k0) + (long long)b * a.k0_bs + (long long)h * D;
  const char* const qbytes = (const char*)uniform64(
      (unsigned long long)(reinterpret_cast<const T*>(a.q) + (long long)b * a.T * rs + (long long)h * D));
  const char* const obytes = (const char*)uniform64(
      (unsigned long long)(reinterpret_cast<const T*>(a.dout) + (long long)b * a.T * rs + (long long)h * D));
  const char* const lbytes = reinterpret_cast<const char*>(a.lse2 + (long long)bh * a.q_pitch);
  const unsigned ldoff = (unsigned)((long long)BH * a.q_pitch * 4);   // lse2 -> delta
  const unsigned rrow = (unsigned)(rs * sz);

  // This lane's key; a query at global position gm sees it iff s <= gm < s_hi.
  // In ring-step mode only the keys held at the launch's ring step count.
  const int s = kt0 + kw * 32 + l32;
  const bool svalid = s < a.Tkv && (!KVACC || geo.in_step(s, a.step_lo));
  if (KVACC && !__syncthreads_or(svalid)) return;   // no key of the step in this tile
  const int s_hi = svalid ? doc_hi_of(a.cu, a.ndocs, s, a.Tkv) : 0;
  Op kv[KS];   // K (P waves) or V (dS waves) of this lane's key
#pragma unroll
  for (int ks = 0; ks < KS; ++ks)
    kv[ks] = svalid ? load8(kvb + (long long)s * rs + 16 * ks + 8 * g) : zero8<T>();
  const int hi_min = doc_hi_of(a.cu, a.ndocs, kt0, a.Tkv);   // smallest document end of the tile
  const int q_hi = doc_hi_of(a.cu, a.ndocs, kt1 - 1, a.Tkv);  // queries past this see no key

  f32x16 acc[DB];   // dV^T (P waves) or dK^T (dS waves)
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int j = 0; j < 16; ++j) acc[db][j] = 0.f;
  const float c2 = a.c2;

  // Copy one query tile (Q and dO rows, lse2 / delta) into stage p; the 8
  // waves share the instructions.
  const TileDma<BMQ, C::RRB, C::U, NW> tdma(rrow, w, lane);
  auto dma_stage = [&](int p, const QIter& q) {
    const unsigned st = sbase + (unsigned)(p * C::STAGE);
    const int r0 = q.row0(), nr = q.nrows(BMQ), p0 = q.prow0();
    tdma(st, qbytes + (long long)r0 * rrow, nr);
    tdma(st + C::RT, obytes + (long long)r0 * rrow, nr);
    if (w == 0 && lane < BMQ / 2) {
      const unsigned voff = lane < BMQ / 4 ? 16u * lane : ldoff + 16u * (lane - BMQ / 4);
      lds_dma16(lbytes + (long long)p0 * 4, voff, sbase + (unsigned)(lb0 - smem) + p * C::LSTAGE);
    }
  };
  auto interior = [&](const QIter& q) {
    const int gq0 = q.gpos0();
    return q.nrows(BMQ) == BMQ && kt0 + BNK <= a.Tkv && gq0 >= kt0 + BNK - 1 &&
           gq0 + BMQ - 1 < hi_min;
  };
  // Query m of the tile (m = 4g + o, o = 32mb + 8(j/4) + j%4 a constant per
  // element) sees this lane's key when lo <= m - 4g <= hi.
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

  // Three stages and one barrier per step: the barrier of step j publishes P(j)
  // and the copy of tile j+1, and by then every wave has finished step j-1, so
  // tile j+2 is copied into the stage of tile j-1 right after it. Without an
  // end-of-step barrier the P wave runs on into S(j+1) and its exponentials
  // while the dS wave forms dS(j) and dK(j). P alternates between two buffers.
  QIter it, i1, i2;
  it.begin(geo, kt0, q_hi, BMQ);
  i1 = it;
  if (i1.valid) i1.next(geo, BMQ);
  i2 = i1;
  if (i2.valid) i2.next(geo, BMQ);
  if (it.valid) dma_stage(0, it);
  if (i1.valid) dma_stage(1, i1);
  wait_all();
  __syncthreads();

  const ColRead<T, C::RRB> rcol(lane);
  int cur = 0;                          // stage of tile j (j mod 3)
  for (int par = 0; it.valid; par ^= 1) {
    const char* const st = smem + cur * C::STAGE;
    const float* const L2s = reinterpret_cast<const float*>(lb0 + cur * C::LSTAGE);
    const float* const Ds = L2s + BMQ;
    char* const pw = pbuf + (par * 4 + kw) * C::PW;   // P(j) of this key block, lane-major
    // S^T (P waves, rows Q) or dP^T (dS waves, rows dO): lane = key.
    f32x16 sp[MB];
    {
      const char* const R = st + role * C::RT;
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int j = 0; j < 16; ++j) sp[mb][j] = 0.f;
      // MFMA i = ks * MB + mb, operands read three ahead.
      mfma_ring<KS * MB, 3>(
          [&](int i) { return lds_sw8<T, C::RRB>(R, 32 * (i % MB) + l32, 16 * (i / MB) + 8 * g); },
          [&](int i, const Op& op) { mfma16(op, kv[i / MB], sp[i % MB]); });
    }
    Op ops[BMQ / 16];
    if (role == 0) {
      if (KVACC || !interior(it)) mask(sp, it);   // ring-step mode: keys outside the step are masked
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
          const f32x4 l4 = *reinterpret_cast<const f32x4*>(L2s + 32 * mb + 8 * jj + 4 * g);
#pragma unroll
          for (int i = 0; i < 4; ++i) sp[mb][4 * jj + i] = fast_exp2(fmaf(sp[mb][4 * jj + i], c2, -l4[i]));
        }
#pragma unroll
      for (int q = 0; q < BMQ / 16; ++q) {
        ops[q] = to_op(sp[q >> 1], 8 * (q & 1), T());
        *reinterpret_cast<Op*>(pw + (q * 64 + lane) * (int)sizeof(Op)) = ops[q];
      }
    }
    wait_all();
    __syncthreads();   // P(j) and tile j+1 are in LDS; tile j-1's stage is free
    if (i2.valid) dma_stage(cur == 0 ? 2 : cur - 1, i2);
    if (role == 1) {
#pragma unroll
      for (int q = 0; q < BMQ / 16; ++q) {
        const Op pq = *reinterpret_cast<const Op*>(pw + (q * 64 + lane) * (int)sizeof(Op));
        const int mb = q >> 1, j0 = 8 * (q & 1);
        const f32x4 d0 = *reinterpret_cast<const f32x4*>(Ds + 32 * mb + 8 * (j0 >> 2) + 4 * g);
        const f32x4 d1 = *reinterpret_cast<const f32x4*>(Ds + 32 * mb + 8 * ((j0 >> 2) + 1) + 4 * g);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float dl = e < 4 ? d0[e] : d1[e - 4];
          sp[mb][j0 + e] = (float)pq[e] * (sp[mb][j0 + e] - dl);
        }
        ops[q] = to_op(sp[mb], j0, T());
      }
    }
    // dV^T += dO^T P^T (P waves) or dK^T += Q^T dS^T (dS waves), the first
    // operand read down the rows of the dO or Q tile.
    {
      const char* const Cc = st + (1 - role) * C::RT;
#pragma unroll
      for (int ks = 0; ks < BMQ / 16; ++ks)
#pragma unroll
        for (int db = 0; db < DB; ++db) mfma16(rcol(Cc, 16 * ks, 32 * db), ops[ks], acc[db]);
    }
    it = i1;
    i1 = i2;
    if (i2.valid) i2.next(geo, BMQ);
    cur = cur == 2 ? 0 : cur + 1;
  }

  // dV0 (P waves) or dK0 = scale * dK (dS waves); keys no query sees get zeros.
  // Ring-step mode adds into the float32 accumulators of the step's keys.
  if (KVACC && svalid) {
    const float f = role ? a.scale : 1.f;
    float* ob = reinterpret_cast<float*>(role ? a.dk0 : a.dv0) + (long long)b * a.k0_bs + (long long)h * D +
                (long long)s * rs;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        f32x4 x = *reinterpret_cast<const f32x4*>(ob + 32 * db + 8 * jj + 4 * g);
#pragma unroll
        for (int i = 0; i < 4; ++i) x[i] += acc[db][4 * jj + i] * f;
        *reinterpret_cast<f32x4*>(ob + 32 * db + 8 * jj + 4 * g) = x;
      }
  } else if (!KVACC && svalid) {
    const float f = role ? a.scale : 1.f;
    T* ob = reinterpret_cast<T*>(role ? a.dk0 : a.dv0) + (long long)b * a.k0_bs + (long long)h * D +
            (long long)s * rs;
    typedef typename VecE<T, 4>::type v4;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        v4 x;
#pragma unroll
        for (int i = 0; i < 4; ++i) x[i] = (T)(acc[db][4 * jj + i] * f);
        *reinterpret_cast<v4*>(ob + 32 * db + 8 * jj + 4 * g) = x;
      }
  }
}

// ---------------------------------------------------------------------------
// dQ (block 0) + closed-form diagonal gradients
// ---------------------------------------------------------------------------
template <typename T, int D>
struct DqCfg {
  static constexpr int BM = 128;        // query rows per workgroup (32 per wave)
  static constexpr int BN = sizeof(T) == 2 ? 64 : 32;   // keys per step
  static constexpr int KB = BN / 32;    // 32-key blocks per step
  static constexpr int KS = D / 16;
  static constexpr int DB = D / 32;
  static constexpr int U = 8 * (int)sizeof(T) / 16;    // 16-byte chunks per operand
  static constexpr int KRB = D * (int)sizeof(T);       // K, V rows [BN][D]: row bytes
  static constexpr int KT = BN * KRB;                  // bytes per tile
  static constexpr int STAGE = 2 * KT;                 // K, V
  static constexpr int OSTR = D + 4;
  static constexpr int LDS_KV = 2 * STAGE;
  static constexpr int LDS_EPI = 4 * 32 * OSTR * 4;
  static constexpr int LDS = LDS_KV > LDS_EPI ? LDS_KV : LDS_EPI;
  static constexpr int NB = sizeof(T) == 2 ? 8 : 2;   // diagonal blocks per epilogue group
};

template <typename T, int D>
__global__ __launch_bounds__(256, sizeof(T) == 2 ? 2 : 1) void dq_kernel(const Args a) {
  using C = DqCfg<T, D>;
  using Op = typename V8<T>::type;
  constexpr int BM = C::BM, BN = C::BN, KB = C::KB, KS = C::KS, DB = C::DB;
  constexpr int sz = (int)sizeof(T);
  __shared__ __attribute__((aligned(16))) char smem[C::LDS];
  const unsigned sbase = lds_addr(smem);

  const int tid = threadIdx.x, lane = tid & 63, g = lane >> 5, l32 = lane & 31;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int BH = a.B * a.H;
  const int trank = blockIdx.x / BH, bh = blockIdx.x % BH, b = bh / a.H, h = bh % a.H;
  const Geo geo{a.layout, a.cp, a.rank, a.T, a.Tkv, a.cu, a.ndocs};
  int row0, nrows, gpos0;
  geo.qtile(trank, BM, row0, nrows, gpos0);

  const long long rs = (long long)a.H * D;
  const T* qb = reinterpret_cast<const T*>(a.q) + (long long)b * a.T * rs + (long long)h * D;
  const T* dob = reinterpret_cast<const T*>(a.dout) + (long long)b * a.T * rs + (long long)h * D;
  const char* const kbytes =
      reinterpret_cast<const char*>(reinterpret_cast<const T*>(a.k0) + (long long)b * a.k0_bs + (long long)h * D);
  const char* const vbytes =
      reinterpret_cast<const char*>(reinterpret_cast<const T*>(a.v0) + (long long)b * a.k0_bs + (long long)h * D);
  const unsigned krow = (unsigned)(rs * sz);
  // lse2 / delta of the tile's rows in the padded layout (the tile lies inside
  // one run, which starts at a multiple of 64 positions).
  const long long prow0 = (long long)bh * a.q_pitch + geo.prow(row0);

  const int qr = w * 32 + l32;
  const bool qvalid = qr < nrows;
  const int gq = gpos0 + qr;
  const int loq = doc_lo_of(a.cu, a.ndocs, qvalid ? gq : gpos0);
  const int g_min = gpos0, g_max = gpos0 + nrows - 1;
  const int lo_min = doc_lo_of(a.cu, a.ndocs, g_min);
  const int lo_max = doc_lo_of(a.cu, a.ndocs, g_max);

  // This lane's half of its query row (columns 16 ks + 8 g .. + 7) of q and dO;
  // delta = <dO, O> with O the merged forward output (each lane sums its half,
  // one exchange with lane ^ 32 adds the other), lse2 = lse * log2(e). Both are
  // written to the workspace for the dK/dV and diagonal-gradient kernels; the
  // positions of the padded layout past the run's end get 0.
  Op qreg[KS], oreg[KS];
  float dpart = 0.f;
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    const long long off = (long long)(row0 + qr) * rs + 16 * ks + 8 * g;
    qreg[ks] = qvalid ? load8(qb + off) : zero8<T>();
    oreg[ks] = qvalid ? load8(dob + off) : zero8<T>();
    const Op ov = qvalid ? load8(reinterpret_cast<const T*>(a.o_in) + (long long)b * a.T * rs + (long long)h * D + off)
                         : zero8<T>();
    dpart = dot8(oreg[ks], ov, dpart);
  }
  const float dq_delta = swap32_sum(dpart);
  const float lq = qvalid ? a.lse_in[(long long)bh * a.T + row0 + qr] * kLog2e : 0.f;
  if (g == 0 && qr < ((nrows + 63) & ~63)) {
    a.lse2[prow0 + qr] = lq;
    a.delta[prow0 + qr] = dq_delta;
  }
  f32x16 acc[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int j = 0; j < 16; ++j) acc[db][j] = 0.f;
  const float c2 = a.c2;

  // Stage p: K rows at 0, V rows at KT (swizzled, direct copies). K / V rows
  // past the end re-read the last row: those keys are masked.
  auto dma_stage = [&](int p, int s0) {
    const unsigned st = sbase + (unsigned)(p * C::STAGE);
    const int nv = a.Tkv - s0 < BN ? a.Tkv - s0 : BN;
    dma_tile<BN, C::KRB, C::U>(st, kbytes + (long long)s0 * krow, krow, nv, w, lane);
    dma_tile<BN, C::KRB, C::U>(st + C::KT, vbytes + (long long)s0 * krow, krow, nv, w, lane);
  };
  const ColRead<T, C::KRB> kcol(lane);
  auto interior = [&](const SegIter& t) {
    return t.s0 >= t.a && t.s0 + BN <= t.b && t.s0 >= lo_max && t.s0 + BN - 1 <= g_min;
  };
  // Key s = t.s0 + 4g + o (o = 32 kb + 8(j/4) + j%4) is visible when lo <= o <= hi.
  auto mask = [&](f32x16 (&st)[KB], const SegIter& t) {
    const int base = t.s0 + 4 * g;
    const int lo = (t.a > loq ? t.a : loq) - base;
    const int hi = ((t.b - 1) < gq ? (t.b - 1) : gq) - base;
#pragma unroll
    for (int kb = 0; kb < KB; ++kb)
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const int o = 32 * kb + 8 * (j >> 2) + (j & 3);
        st[kb][j] = (o >= lo && o <= hi) ? st[kb][j] : kNegInf;
      }
  };

  SegIter it, i1;
  it.begin(geo, lo_min, g_max + 1, BN, a.step_lo, a.step_hi);
  i1 = it;
  if (i1.valid) i1.next(geo, BN);
  if (it.valid) dma_stage(0, it.s0);
  wait_all();
  __syncthreads();

  for (int par = 0; it.valid; par ^= 1) {
    const int cur = __builtin_amdgcn_readfirstlane(par);
    const char* const Ks = smem + cur * C::STAGE;
    const char* const Vs = Ks + C::KT;
    // Alternate the issue priority every step: the two workgroups on a CU then
    // share each SIMD's MFMA pipe evenly instead of the older one running ahead.
    if (cur) __builtin_amdgcn_s_setprio(1);
    else __builtin_amdgcn_s_setprio(0);
    if (i1.valid) dma_stage(cur ^ 1, i1.s0);
    // S^T and dP^T for the BN keys: lane = query.
    f32x16 st[KB], dpt[KB];
#pragma unroll
    for (int kb = 0; kb < KB; ++kb)
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        st[kb][j] = 0.f;
        dpt[kb][j] = 0.f;
      }
    // MFMA i: k-step i / (2 KB), 32-key block (i / 2) mod KB, S (even i, rows of
    // K) or dP (odd i, rows of V).
    mfma_ring<2 * KS * KB, 3>(
        [&](int i) {
          return lds_sw8<T, C::KRB>((i & 1) ? Vs : Ks, 32 * ((i >> 1) % KB) + l32, 16 * (i / (2 * KB)) + 8 * g);
        },
        [&](int i, const Op& op) {
          if (i & 1) mfma16(op, oreg[i / (2 * KB)], dpt[(i >> 1) % KB]);
          else mfma16(op, qreg[i / (2 * KB)], st[(i >> 1) % KB]);
        });
    if (!interior(it)) mask(st, it);
#pragma unroll
    for (int kb = 0; kb < KB; ++kb)
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const float p = fast_exp2(fmaf(st[kb][j], c2, -lq));
        dpt[kb][j] = p * (dpt[kb][j] - dq_delta);
      }
    Op ds[2 * KB];   // k-step k: keys 16 k .. 16 k + 15
#pragma unroll
    for (int k = 0; k < 2 * KB; ++k) ds[k] = to_op(dpt[k >> 1], 8 * (k & 1), T());
    // dQ^T += K^T dS^T over the BN keys (2 KB k-steps of 16); K^T is read down
    // the rows of the K tile. MFMA i: 32-row block i mod DB of D, k-step i / DB.
    mfma_ring<2 * KB * DB, (sizeof(T) == 2 ? 3 : 1)>(
        [&](int i) { return kcol(Ks, 16 * (i / DB), 32 * (i % DB)); },
        [&](int i, const Op& op) { mfma16(op, ds[i / DB], acc[i % DB]); });
    it = i1;
    if (i1.valid) i1.next(geo, BN);
    wait_all();
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

  // scale * dQ(block 0): the final dq when there are no diagonal blocks, else a
  // float32 partial that diag_bwd_kernel completes.
  constexpr int LPR = D / 8;
  constexpr int RPP = 64 / LPR;
  const int lr = lane / LPR, cc = (lane % LPR) * 8;
  T* dqb = reinterpret_cast<T*>(a.dq) + (long long)b * a.T * rs + (long long)h * D + cc;
  float* dqdb = const_cast<float*>(a.dqd) + (long long)b * a.T * rs + (long long)h * D + cc;
  for (int pass = 0; pass < 32 / RPP; ++pass) {
    const int rr = pass * RPP + lr;
    const int tr = w * 32 + rr;
    if (tr >= nrows) continue;               // whole row groups agree
    const long long row = row0 + tr;
    f32x8 dqv = *reinterpret_cast<const f32x8*>(Qw + rr * C::OSTR + cc);
#pragma unroll
    for (int e = 0; e < 8; ++e) dqv[e] *= a.scale;
    if (a.dq_accum) {
      // ring-step mode: this launch's ring steps add into the caller's float32 dq
      f32x8 acc = *reinterpret_cast<const f32x8*>(dqdb + row * rs);
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[e] += dqv[e];
      *reinterpret_cast<f32x8*>(dqdb + row * rs) = acc;
    } else if (a.N > 0 && !a.dq_in_out) {
      *reinterpret_cast<f32x8*>(dqdb + row * rs) = dqv;
    } else {
      store8f(dqb + row * rs, dqv);   // final dq, or (dq_in_out) the block-0 part
    }
  }
}

// ---------------------------------------------------------------------------
// Closed-form diagonal gradients (ring_attention page, `_merge_diag`: each
// position's TTT blocks are one score each), against the merged lse:
//   pi = exp(y - lse), dpi = <dO, vd>, ds = pi (dpi - delta),
//   dkd = scale ds q, dvd = pi dO, dq_diag = scale sum_i ds_i kd_i (float32).
// LPR lanes per (b, t, h) row, 8 columns each; a persistent grid strides over
// the rows. It only reads q, dO, lse2, delta, kd, vd, so it runs on a side
// stream next to the dK/dV kernel, whose CUs it shares (few registers, no LDS).
// ---------------------------------------------------------------------------
// MODE: 0 = the float32 block-0 dq partial from the workspace; 1 = ring-step mode
// (delta and lse*log2(e) formed here from the merged out/lse; the partial is the
// caller's float32 accumulator); 2 = no-allocation backward (the block-0 dq read
// back from dq itself, in q's dtype). Separate instantiations keep the default
// one's registers low enough to share the SIMDs with the dK/dV kernel.
template <typename T, int D, int MODE>
__global__ __launch_bounds__(256, 4) void diag_bwd_kernel(const Args a) {
  constexpr int LPR = D / 8;
  constexpr int GPB = 256 / LPR;           // row groups per workgroup
  // blocks per load group: 4 keeps the kernel within 120 VGPRs, so one of its
  // waves fits on each SIMD beside the two dK/dV waves (2 x 192 + 120 = 504)
  constexpr int NB = sizeof(T) == 2 ? 4 : 2;
  using V = typename V8<T>::type;
  const Geo geo{a.layout, a.cp, a.rank, a.T, a.Tkv, a.cu, a.ndocs};
  const int tid = threadIdx.x, cc = (tid % LPR) * 8;
  const long long nrow = (long long)a.B * a.T * a.H;
  const long long rs = (long long)a.H * D;
  const float c2 = a.c2, scale = a.scale;
  for (long long r = (long long)blockIdx.x * GPB + tid / LPR; r < nrow; r += (long long)gridDim.x * GPB) {
    const int h = (int)(r % a.H);
    const long long bt = r / a.H;
    const int t = (int)(bt % a.T), b = (int)(bt / a.T);
    const long long qoff = r * D + cc;                         // [B,T,H,D] row
    const long long doff = (long long)b * a.kd_bs + ((long long)t * a.H + h) * D + cc;
    const long long loff = ((long long)b * a.H + h) * a.q_pitch + geo.prow(t);
    const V qv = load8(reinterpret_cast<const T*>(a.q) + qoff);
    const V ov = load8(reinterpret_cast<const T*>(a.dout) + qoff);
    float l2, dl;
    if constexpr (MODE == 1) {
      // ring-step mode: delta = <dO, O> and lse*log2(e) formed here from the merged out/lse
      const V oo = load8(reinterpret_cast<const T*>(a.o_in) + qoff);
      dl = group_sum<LPR>(dot8(ov, oo, 0.f));
      l2 = a.lse_in[((long long)b * a.H + h) * a.T + t] * kLog2e;
    } else {
      l2 = a.lse2[loff];
      dl = a.delta[loff];
    }
    // scale * dQ(block 0): the float32 partial, or (MODE 2) dq itself in q's dtype
    f32x8 dq;
    if constexpr (MODE == 2) dq = load8f(reinterpret_cast<const T*>(a.dq) + qoff);
    else dq = *reinterpret_cast<const f32x8*>(a.dqd + qoff);
    for (int i0 = 0; i0 < a.N; i0 += NB) {
      const int n = (a.N - i0) < NB ? (a.N - i0) : NB;
      // Unconditional loads (block index clamped), all issued before any use.
      V kv[NB], vv[NB];
#pragma unroll
      for (int i = 0; i < NB; ++i) {
        const long long off = (long long)(i0 + (i < n ? i : n - 1)) * a.kd_blk + doff;
        kv[i] = load8_nt(reinterpret_cast<const T*>(a.kd) + off);
        vv[i] = load8_nt(reinterpret_cast<const T*>(a.vd) + off);
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
          dq[e] = fmaf(sds, (float)kv[i][e], dq[e]);
          gk[e] = sds * (float)qv[e];
          gv[e] = pi * (float)ov[e];
        }
        if (i < n) {
          const long long off = (long long)(i0 + i) * a.kd_blk + doff;
          store8f_nt(reinterpret_cast<T*>(a.dkd) + off, gk);
          store8f_nt(reinterpret_cast<T*>(a.dvd) + off, gv);
        }
      }
    }
    store8f(reinterpret_cast<T*>(a.dq) + qoff, dq);
  }
}

// Order, with the timing hook's marks m0..m5:
//   main:  m0 dQ (also writes delta and lse*log2(e)) m1 | dK/dV m4 | join m5
//   side:                    (forked at m1) m2 diagonal gradients m3
// The diagonal gradients (memory-bound) overlap the dK/dV kernel (MFMA-bound).
template <typename T, int D>
static hipError_t launch_bwd_t(const Args& a, hipStream_t st) {
  const Geo geo{a.layout, a.cp, a.rank, a.T, a.Tkv, a.cu_host, a.ndocs};
  const long long nrow = (long long)a.B * a.H * a.q_pitch;
  if (nrow == 0) return hipSuccess;
  hipError_t e;
  timing_mark(st);
  const long long nq = (long long)geo.ntiles(DqCfg<T, D>::BM) * a.B * a.H;
  if (nq > 0) {
    hipLaunchKernelGGL((dq_kernel<T, D>), dim3((unsigned)nq), dim3(256), 0, st, a);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  timing_mark(st);
  if (a.N > 0 && !a.dq_in_out) {
    hipStream_t side = nullptr;
    if ((e = side_begin(st, 0, side)) != hipSuccess) return e;
    timing_mark(side);
    hipLaunchKernelGGL((diag_bwd_kernel<T, D, 0>), dim3(kDiagGrid), dim3(256), 0, side, a);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    timing_mark(side);
  } else {
    timing_mark(st);   // no side-stream work: its two marks are an empty stage
    timing_mark(st);
  }
  const long long nk = (long long)((a.Tkv + DkdvCfg<T, D>::BNK - 1) / DkdvCfg<T, D>::BNK) * a.B * a.H;
  if (nk > 0) {
    const bool zzd = a.layout == LAYOUT_ZIGZAG && a.ndocs > 1;
    if (a.kv_accum)
      hipLaunchKernelGGL((dkdv_kernel<T, D, true, true>), dim3((unsigned)nk), dim3(DkdvCfg<T, D>::NT), 0, st, a);
    else if (zzd)
      hipLaunchKernelGGL((dkdv_kernel<T, D, false, true>), dim3((unsigned)nk), dim3(DkdvCfg<T, D>::NT), 0, st, a);
    else
      hipLaunchKernelGGL((dkdv_kernel<T, D, false, false>), dim3((unsigned)nk), dim3(DkdvCfg<T, D>::NT), 0, st, a);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  timing_mark(st);
  if (a.N > 0 && a.dq_in_out) {
    // no-allocation backward: the diagonal gradients after dK/dV on the same stream
    // (they read the block-0 dq the dQ kernel left in dq)
    hipLaunchKernelGGL((diag_bwd_kernel<T, D, 2>), dim3(kDiagGrid), dim3(256), 0, st, a);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  } else if (a.N > 0 && (e = side_end(st, 0)) != hipSuccess) {
    return e;
  }
  timing_mark(st);
  return hipSuccess;
}

// Ring-step mode: the closed-form diagonal gradients alone, on the caller's
// stream, with delta and lse*log2(e) formed in the kernel (mode 1).
template <typename T, int D>
static hipError_t launch_diag_bwd_t(const Args& a, hipStream_t st) {
  if ((long long)a.B * a.T * a.H == 0) return hipSuccess;
  hipLaunchKernelGGL((diag_bwd_kernel<T, D, 1>), dim3(kDiagGrid), dim3(256), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_diag_bwd(const Args& a, int dtype, int D, hipStream_t st) {
  if (dtype == 0) return D == 128 ? launch_diag_bwd_t<bf16, 128>(a, st) : launch_diag_bwd_t<bf16, 64>(a, st);
  return D == 128 ? launch_diag_bwd_t<float, 128>(a, st) : launch_diag_bwd_t<float, 64>(a, st);
}

hipError_t launch_bwd(const Args& a, int dtype, int D, hipStream_t st) {
  if (dtype == 0) return D == 128 ? launch_bwd_t<bf16, 128>(a, st) : launch_bwd_t<bf16, 64>(a, st);
  return D == 128 ? launch_bwd_t<float, 128>(a, st) : launch_bwd_t<float, 64>(a, st);
}

}  // namespace e3
