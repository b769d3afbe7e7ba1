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
  static constexpr int NW = 4;             // waves
  static constexpr int NT = 64 * NW;
  static constexpr int BM = 32 * NW;       // query rows per workgroup (32 per wave)
  static constexpr int BN = 64;
  static constexpr int KRB = D * (int)sizeof(T);        // K tile [BN keys][D], row bytes
  static constexpr int U = 8 * (int)sizeof(T) / 16;     // 16-byte chunks per operand
  static constexpr int OSTR = D + 4;       // fp32 staging rows of the epilogue
  static constexpr int KS = D / 16;        // MFMA k-steps over D
  static constexpr int DB = D / 32;        // 32-row blocks of O^T
  static constexpr int KBYTES = BN * KRB, VBYTES = BN * KRB;   // K, V tiles [BN keys][D]
  static constexpr int LDS_KV = 2 * (KBYTES + VBYTES);
  static constexpr int LDS_EPI = NW * 32 * OSTR * 4 + 2 * BM * 4;
  static constexpr int LDS = LDS_KV > LDS_EPI ? LDS_KV : LDS_EPI;
  static constexpr int NB = sizeof(T) == 2 ? 8 : 2;   // diagonal blocks per epilogue group
};

constexpr float kRescaleSlack = 8.0f;      // log2 of the largest un-rescaled growth

// TO: element type of out (T; float for the float32 partials of ring-step mode,
// where a row that sees no key of the visited steps gets out = 0, lse = -inf).
template <typename T, int D, typename TO>
__global__ __launch_bounds__(256, 2) void fwd_kernel(const Args a) {
  using C = FwdCfg<T, D>;
  constexpr int NW = C::NW;
  using Op = typename V8<T>::type;
  constexpr int BM = C::BM, BN = C::BN, KS = C::KS, DB = C::DB;
  __shared__ __attribute__((aligned(16))) char smem[C::LDS];

  const int tid = threadIdx.x, lane = tid & 63, g = lane >> 5, l32 = lane & 31;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int BH = a.B * a.H;
  const int trank = blockIdx.x / BH, bh = blockIdx.x % BH, b = bh / a.H, h = bh % a.H;
  const Geo geo{a.layout, a.cp, a.rank, a.T, a.Tkv, a.cu, a.ndocs};
  int row0, nrows, gpos0;
  geo.qtile(trank, BM, row0, nrows, gpos0);

  // Row (position) strides: rs for the [B, N, T, H, D] diagonal blocks; q / out and
  // k0 / v0 take theirs from the arguments (token-major [B, T, H, D] by default,
  // head-major [B, H, T, D] for the frozen-target forward).
  const long long rs = (long long)a.H * D;
  const long long qrs = a.q_rs;
  const T* qb = reinterpret_cast<const T*>(a.q) + (long long)b * a.q_bs + (long long)h * a.q_hs;
  const T* k0b = reinterpret_cast<const T*>(a.k0) + (long long)b * a.k0_bs + (long long)h * a.kv_hs;
  const T* vb = reinterpret_cast<const T*>(a.v0) + (long long)b * a.k0_bs + (long long)h * a.kv_hs;

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
    qreg[ks] = qvalid ? load8(qb + (long long)(row0 + qr) * qrs + 16 * ks + 8 * g) : zero8<T>();

  f32x16 acc[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int j = 0; j < 16; ++j) acc[db][j] = 0.f;
  float m_i = kNegInf, l_i = 0.f;
  const float c2 = a.c2;

  // LDS: two K stages, then two V stages, swizzled, filled by direct loads.
  // (pointers for the reads, LDS byte addresses for the copies)
  char* const kb0 = smem;
  char* const kb1 = kb0 + C::KBYTES;
  char* const vb0 = kb1 + C::KBYTES;
  char* const vb1 = vb0 + C::VBYTES;
  const unsigned sbase = lds_addr(smem);
  auto la = [&](const char* p) { return sbase + (unsigned)(p - smem); };
  // Scalar K / V bases and the per-lane offsets of this wave's full-tile copies
  // (the same for K and V), so a step issues each copy with no address math.
  const char* const kbase = (const char*)uniform64((unsigned long long)k0b);
  const char* const vbase = (const char*)uniform64((unsigned long long)vb);
  const unsigned krow = (unsigned)(a.kv_rs * (long long)sizeof(T));
  const TileDma<BN, C::KRB, C::U, NW> tdma(krow, w, lane);
  // K / V rows past the end re-read the last row: those keys are masked.
  auto dma_k = [&](char* dst, int s0) {
    const int nv = a.Tkv - s0 < BN ? a.Tkv - s0 : BN;
    tdma(la(dst), kbase + (long long)s0 * krow, nv);
  };
  auto dma_v = [&](char* dst, int s0) {
    const int nv = a.Tkv - s0 < BN ? a.Tkv - s0 : BN;
    tdma(la(dst), vbase + (long long)s0 * krow, nv);
  };
  // V^T operands are read down the rows of the V tile.
  const ColRead<T, C::KRB> vcol(lane);

  // S^T = K Q^T for 64 keys: two 32-key accumulator chains, lane = query.
  auto qk = [&](const char* Ks, f32x16 (&st)[2]) {
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int j = 0; j < 16; ++j) st[kb][j] = 0.f;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
        mfma16(lds_sw8<T, C::KRB>(Ks, 32 * kb + l32, 16 * ks + 8 * g), qreg[ks], st[kb]);
  };
  auto interior = [&](const SegIter& t) {
    return t.s0 >= t.a && t.s0 + BN <= t.b && t.s0 >= lo_max && t.s0 + BN - 1 <= g_min;
  };
  // Key s = t.s0 + 4g + o with o = 32kb + 8(j/4) + j%4 a constant per element;
  // it is visible to this lane's query when lo <= o <= hi.
  auto mask = [&](f32x16 (&st)[2], const SegIter& t) {
    const int base = t.s0 + 4 * g;
    const int lo = (t.a > loq ? t.a : loq) - base;
    const int hi = ((t.b - 1) < gq ? (t.b - 1) : gq) - base;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const int o = 32 * kb + 8 * (j >> 2) + (j & 3);
        st[kb][j] = (o >= lo && o <= hi) ? st[kb][j] : kNegInf;
      }
  };
  // Row max over the tile (two independent chains), base-2 scaled.
  auto rowmax = [&](const f32x16 (&st)[2]) {
    float m0 = kNegInf, m1 = kNegInf;
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      m0 = fmaxf(m0, st[0][j]);
      m1 = fmaxf(m1, st[1][j]);
    }
    return swap32_max(fmaxf(m0, m1)) * c2;
  };
  // Move the running max when a row's max grew by more than 2^kRescaleSlack.
  auto rescale = [&](float mx) {
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
  };

  // Step j: S^T(j) is in registers, K(j+1) and V(j) are in LDS. Phase A
  // overlaps the MFMAs of S^T(j+1) with the exponentials of tile j; phase B
  // the MFMAs of O^T += V^T P^T for tile j with the mask and row max of tile
  // j+1. Tiles j, j+1, j+2 of the walk are it, i1, i2.
  SegIter it, i1, i2;
  it.begin(geo, lo_min, g_max + 1, BN, a.step_lo, a.step_hi);
  i1 = it;
  if (i1.valid) i1.next(geo, BN);
  i2 = i1;
  if (i2.valid) i2.next(geo, BN);
  if (it.valid) {
    dma_k(kb0, it.s0);
    dma_v(vb0, it.s0);
  }
  if (i1.valid) dma_k(kb1, i1.s0);
  wait_all();
  __syncthreads();

  f32x16 sa[2], sb[2];
  if (it.valid) {
    qk(kb0, sa);
    if (!interior(it)) mask(sa, it);
    rescale(rowmax(sa));
  }
  __syncthreads();   // K(0) is read; K(2) may be copied into its stage
  const Op ones = ones8<T>();

  // This wave's share of the copy of tile t's K or V rows into a stage
  // (nothing when the walk has no tile t).
  auto copy_k = [&](const SegIter& t, char* dst) {
    if (t.valid) dma_k(dst, t.s0);
  };
  auto copy_v = [&](const SegIter& t, char* dst) {
    if (t.valid) dma_v(dst, t.s0);
  };
  Op pv[BN / 16];   // P(j) as MFMA operands, from phase A to phase B
  // Phase A: S^T(j+1) on MFMA (stale LDS when there is no tile j+1: the
  // result is then never used); P(j) and its row sum on VALU. The order is
  // fixed by scheduling fences: in step i the K operand of MFMA i+2 is read,
  // MFMA i issues, and 2 of the 32 exponentials of this lane are computed.
  auto phase_a = [&](f32x16 (&sc)[2], f32x16 (&sn)[2], const char* Kn) {
    const float nb = m_i == kNegInf ? 0.f : -m_i;
    float rsum = 0.f;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int j = 0; j < 16; ++j) sn[kb][j] = 0.f;
    constexpr int NQ = 2 * KS;                 // MFMAs: i = 2 ks + kb
    Op ka[3];
    ka[0] = lds_sw8<T, C::KRB>(Kn, l32, 8 * g);
    ka[1] = lds_sw8<T, C::KRB>(Kn, 32 + l32, 8 * g);
#pragma unroll
    for (int i = 0; i < NQ; ++i) {
      if (i + 2 < NQ)
        ka[(i + 2) % 3] = lds_sw8<T, C::KRB>(Kn, 32 * ((i + 2) & 1) + l32, 16 * ((i + 2) >> 1) + 8 * g);
      mfma16(ka[i % 3], qreg[i >> 1], sn[i & 1]);
      // Exponentials: 32 per lane over the NQ steps.
#pragma unroll
      for (int e = (32 * i) / NQ; e < (32 * (i + 1)) / NQ; ++e)
        sc[e >> 4][e & 15] = fast_exp2(fmaf(sc[e >> 4][e & 15], c2, nb));
      // Every 8 exponentials: one bf16 operand and its part of the row sum.
      // (pinned here: otherwise they sink past the mask branch below, away
      // from the MFMAs they overlap).
#pragma unroll
      for (int q = 0; q < BN / 16; ++q)
        if ((32 * (i + 1)) / NQ >= 8 * (q + 1) && (32 * i) / NQ < 8 * (q + 1)) {
          pv[q] = to_op(sc[q >> 1], 8 * (q & 1), T());
          rsum = dot8(pv[q], ones, rsum);
          pin(pv[q]);
          pin(rsum);
        }
      __builtin_amdgcn_sched_barrier(0);
    }
    l_i += rsum;
    if (i1.valid && !interior(i1)) mask(sn, i1);
  };
  // Phase B: O^T += V^T(j) P^T(j) on MFMA, operands read one k-step ahead;
  // the row max of tile j+1 on VALU, a quarter per k-step.
  auto phase_b = [&](const f32x16 (&sn)[2], const char* Vc) {
    float mx0 = kNegInf, mx1 = kNegInf;
    Op va[2][DB];
#pragma unroll
    for (int db = 0; db < DB; ++db) va[0][db] = vcol(Vc, 0, 32 * db);
#pragma unroll
    for (int ks = 0; ks < BN / 16; ++ks) {
      if (ks + 1 < BN / 16) {
#pragma unroll
        for (int db = 0; db < DB; ++db)
          va[(ks + 1) & 1][db] = vcol(Vc, 16 * (ks + 1), 32 * db);
      }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int db = 0; db < DB; ++db) mfma16(va[ks & 1][db], pv[ks], acc[db]);
#pragma unroll
      for (int j = 4 * ks; j < 4 * ks + 4; ++j) {
        mx0 = fmaxf(mx0, sn[0][j]);
        mx1 = fmaxf(mx1, sn[1][j]);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    const float mx = swap32_max(fmaxf(mx0, mx1)) * c2;
    if (i1.valid) rescale(mx);
  };
  auto advance = [&]() {
    it = i1;
    i1 = i2;
    if (i2.valid) i2.next(geo, BN);
  };
  auto sync = [&]() {
    wait_all();
    __syncthreads();
  };

  // Two workgroups share a CU, one wave of each on every SIMD. At equal
  // priority the SIMD issues for the older wave first, which then runs far
  // ahead of its partner and leaves lone-wave tails at the end of the grid;
  // alternating the issue priority every key tile shares the MFMA pipe.
  // Each step first starts the copies of K(j+2) and V(j+1) into the stages
  // step j-1 finished with (spreading them between the phase A MFMAs
  // measured ~8% slower).
  int hi_prio = 0;
  auto step = [&](f32x16 (&sc)[2], f32x16 (&sn)[2], const char* Kn, const char* Vc, char* Kw,
                  char* Vw) {
    copy_k(i2, Kw);
    copy_v(i1, Vw);
    if (hi_prio) __builtin_amdgcn_s_setprio(1);
    else __builtin_amdgcn_s_setprio(0);
    hi_prio ^= 1;
    phase_a(sc, sn, Kn);
    phase_b(sn, Vc);
    advance();
    sync();
  };
  while (it.valid) {
    step(sa, sb, kb1, vb0, kb0, vb1);
    if (!it.valid) break;
    step(sb, sa, kb0, vb1, kb1, vb0);
  }
  l_i = swap32_sum(l_i);

  // ---- epilogue: stage O^T (unnormalised), m, l through LDS ----------------
  float* Ow = reinterpret_cast<float*>(smem) + w * 32 * C::OSTR;
  float* Ms = reinterpret_cast<float*>(smem) + NW * 32 * C::OSTR;
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
  TO* ob = reinterpret_cast<TO*>(a.out) + (long long)b * a.q_bs + (long long)h * a.q_hs + cc;
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
      qv[u] = load8(qb + row[u] * qrs + cc);
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
          kv[u][i] = load8_nt(kdb + off);
          vv[u][i] = load8_nt(vdb + off);
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
      const float inv = l[u] > 0.f ? 1.f / l[u] : 0.f;   // l = 0: the row saw no key
#pragma unroll
      for (int e = 0; e < 8; ++e) o[u][e] *= inv;
      store8f(ob + row[u] * qrs, o[u]);
      if ((lane % LPR) == 0 && a.lse) lseb[row[u]] = (m[u] + fast_log2(l[u])) * kLn2;   // lse may be omitted (frozen-target forward)
    }
  }
}

template <typename T, int D>
static hipError_t launch_fwd_t(const Args& a, hipStream_t st) {
  using C = FwdCfg<T, D>;
  const Geo geo{a.layout, a.cp, a.rank, a.T, a.Tkv, a.cu_host, a.ndocs};
  const long long nt = (long long)geo.ntiles(C::BM) * a.B * a.H;
  if (nt == 0) return hipSuccess;
  timing_mark(st);
  if (a.out_f32)
    hipLaunchKernelGGL((fwd_kernel<T, D, float>), dim3((unsigned)nt), dim3(C::NT), 0, st, a);
  else
    hipLaunchKernelGGL((fwd_kernel<T, D, T>), dim3((unsigned)nt), dim3(C::NT), 0, st, a);
  timing_mark(st);
  return hipGetLastError();
}

// Ring-step mode: merges the N diagonal blocks into the float32 running state
// (out_acc, lse_acc) that the chained block-0 ring steps produced (ring_attention
// page, `_merge_diag`, once per block i = 1..N) and writes the final out in q's
// dtype and lse. LPR lanes per (b, t, h) row, 8 columns each; an online merge
// over the blocks in base 2.
template <typename T, int D>
__global__ __launch_bounds__(256) void diag_merge_fwd_kernel(const Args a, const float* out_acc,
                                                             const float* lse_acc) {
  constexpr int LPR = D / 8;
  constexpr int GPB = 256 / LPR;
  using V = typename V8<T>::type;
  const int tid = threadIdx.x, cc = (tid % LPR) * 8;
  const long long nrow = (long long)a.B * a.T * a.H;
  for (long long r = (long long)blockIdx.x * GPB + tid / LPR; r < nrow; r += (long long)gridDim.x * GPB) {
    const int h = (int)(r % a.H);
    const long long bt = r / a.H;
    const int t = (int)(bt % a.T), b = (int)(bt / a.T);
    const long long qoff = r * D + cc;
    const long long doff = (long long)b * a.kd_bs + ((long long)t * a.H + h) * D + cc;
    const long long loff = ((long long)b * a.H + h) * a.T + t;
    const V qv = load8(reinterpret_cast<const T*>(a.q) + qoff);
    f32x8 o = *reinterpret_cast<const f32x8*>(out_acc + qoff);
    float m = lse_acc[loff] * kLog2e;          // state: (m, l = 1, o) or empty
    float l = m == kNegInf ? 0.f : 1.f;
    for (int i = 0; i < a.N; ++i) {
      const long long off = (long long)i * a.kd_blk + doff;
      const V kv = load8(reinterpret_cast<const T*>(a.kd) + off);
      const V vv = load8(reinterpret_cast<const T*>(a.vd) + off);
      const float y = group_sum<LPR>(dot8(qv, kv, 0.f)) * a.c2;
      const float mn = fmaxf(m, y);
      const float al = fast_exp2(m - mn), p = fast_exp2(y - mn);
      l = l * al + p;
#pragma unroll
      for (int e = 0; e < 8; ++e) o[e] = fmaf(p, (float)vv[e], o[e] * al);
      m = mn;
    }
    const float inv = l > 0.f ? 1.f / l : 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) o[e] *= inv;
    store8f(reinterpret_cast<T*>(a.out) + qoff, o);
    if ((tid % LPR) == 0) a.lse[loff] = (m + fast_log2(l)) * kLn2;
  }
}

template <typename T, int D>
static hipError_t launch_diag_merge_t(const Args& a, const float* out_acc, const float* lse_acc,
                                      hipStream_t st) {
  const long long nrow = (long long)a.B * a.T * a.H;
  if (nrow == 0) return hipSuccess;
  constexpr int GPB = 256 / (D / 8);
  const long long g = (nrow + GPB - 1) / GPB;
  hipLaunchKernelGGL((diag_merge_fwd_kernel<T, D>), dim3((unsigned)(g < 4096 ? g : 4096)), dim3(256), 0,
                     st, a, out_acc, lse_acc);
  return hipGetLastError();
}

hipError_t launch_diag_merge(const Args& a, const float* out_acc, const float* lse_acc, int dtype, int D,
                             hipStream_t st) {
  if (dtype == 0)
    return D == 128 ? launch_diag_merge_t<bf16, 128>(a, out_acc, lse_acc, st)
                    : launch_diag_merge_t<bf16, 64>(a, out_acc, lse_acc, st);
  return D == 128 ? launch_diag_merge_t<float, 128>(a, out_acc, lse_acc, st)
                  : launch_diag_merge_t<float, 64>(a, out_acc, lse_acc, st);
}

hipError_t launch_fwd(const Args& a, int dtype, int D, hipStream_t st) {
  if (dtype == 0) return D == 128 ? launch_fwd_t<bf16, 128>(a, st) : launch_fwd_t<bf16, 64>(a, st);
  return D == 128 ? launch_fwd_t<float, 128>(a, st) : launch_fwd_t<float, 64>(a, st);
}

int fwd_tile_rows() { return FwdCfg<bf16, 128>::BM; }
int fwd_tile_keys() { return 64; }

}  // namespace e3
