// C ABI of libeagle3_attn.so: argument validation, share geometry (the shard
// driver) and kernel launches. Declarations and the contract are in
// include/eagle3_attn.h.
#include "eagle3_attn.h"

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdint>
#include <cstdio>
#include <map>
#include <mutex>
#include <string>

#include "e3_common.h"

namespace e3 {
hipError_t launch_fwd(const Args& a, int dtype, int D, hipStream_t st);
hipError_t launch_bwd(const Args& a, int dtype, int D, hipStream_t st);
hipError_t launch_lse_merge(float* out, float* lse, const float* bo, const float* bl, int B, int T,
                            int H, int D, int blayout, hipStream_t st);
hipError_t launch_diag_merge(const Args& a, const float* out_acc, const float* lse_acc, int dtype, int D,
                             hipStream_t st);
hipError_t launch_diag_bwd(const Args& a, int dtype, int D, hipStream_t st);
int fwd_tile_rows();
int fwd_tile_keys();
hipError_t launch_seg_copy(const SegCopy& c, hipStream_t st);
}  // namespace e3

namespace {

thread_local std::string g_err;
thread_local hipEvent_t* g_events = nullptr;
thread_local int g_events_cap = 0;
thread_local int g_events_n = 0;

void timing_reset() { g_events_n = 0; }

int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return code;
}

int ok() {
  g_err.clear();
  return E3_OK;
}

struct Resolved {
  int N;
  long long k0_bs, kd_bs, kd_blk;
  int ndocs;
};

bool misaligned(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) != 0; }

// Validates a problem; fills the resolved strides. `whole` restricts the layout to
// the full-sequence entry points (FULL or HEADSHARD).
int validate(const e3_problem* p, Resolved& r, bool whole, bool need_dev = true) {
  if (!p) return fail(E3_EINVAL, "problem is NULL");
  if (p->dtype != E3_BF16 && p->dtype != E3_F32) return fail(E3_EINVAL, "dtype %d is not E3_BF16 or E3_F32", p->dtype);
  if (p->D != 64 && p->D != 128) return fail(E3_EUNSUPPORTED, "head dim D=%d (supported: 64, 128)", p->D);
  if (p->B < 1) return fail(E3_EINVAL, "B=%d must be >= 1", p->B);
  if (p->H < 1) return fail(E3_EINVAL, "H=%d must be >= 1", p->H);
  if (p->T < 0 || p->T_kv < 0) return fail(E3_EINVAL, "T=%d, T_kv=%d must be >= 0", p->T, p->T_kv);
  if (p->num_blocks < 1 || p->num_blocks > 16)
    return fail(E3_EINVAL, "num_blocks=%d must be in [1, 16]", p->num_blocks);
  if (!(std::isfinite(p->scale) && p->scale > 0.f)) return fail(E3_EINVAL, "scale must be finite and > 0");
  const long long T = p->T, Tkv = p->T_kv;
  switch (p->layout) {
    case E3_LAYOUT_FULL:
      if (p->cp != 1 || p->rank != 0) return fail(E3_EINVAL, "FULL layout needs cp=1, rank=0");
      if (Tkv != T) return fail(E3_EINVAL, "FULL layout needs T_kv == T (%lld vs %lld)", Tkv, T);
      break;
    case E3_LAYOUT_HEADSHARD:
      if (p->cp < 1 || p->rank < 0 || p->rank >= p->cp) return fail(E3_EINVAL, "bad cp=%d / rank=%d", p->cp, p->rank);
      if (Tkv != T) return fail(E3_EINVAL, "HEADSHARD layout needs T_kv == T (%lld vs %lld)", Tkv, T);
      if (T % p->cp != 0)
        return fail(E3_EINVAL, "HEADSHARD: sequence length %lld must divide by the Ulysses degree %d", T, p->cp);
      break;
    case E3_LAYOUT_CONTIGUOUS:
      if (p->cp < 1 || p->rank < 0 || p->rank >= p->cp) return fail(E3_EINVAL, "bad cp=%d / rank=%d", p->cp, p->rank);
      if (Tkv != (long long)p->cp * T) return fail(E3_EINVAL, "CONTIGUOUS layout needs T_kv == cp*T");
      break;
    case E3_LAYOUT_ZIGZAG:
      if (p->cp < 1 || p->rank < 0 || p->rank >= p->cp) return fail(E3_EINVAL, "bad cp=%d / rank=%d", p->cp, p->rank);
      if (T % 2 != 0) return fail(E3_EINVAL, "ZIGZAG layout needs an even local length (two chunks), T=%lld", T);
      if (Tkv != (long long)p->cp * T) return fail(E3_EINVAL, "ZIGZAG layout needs T_kv == cp*T");
      if (p->B != 1) return fail(E3_EINVAL, "ZIGZAG layout is varlen and unbatched: B must be 1");
      break;
    default:
      return fail(E3_EINVAL, "unknown layout %d", p->layout);
  }
  if (whole && p->layout != E3_LAYOUT_FULL && p->layout != E3_LAYOUT_HEADSHARD)
    return fail(E3_EINVAL, "eagle3_attn_fwd/bwd take the FULL or HEADSHARD layout; use eagle3_shard_fwd/bwd");
  if (Tkv > 0x3fffffffLL) return fail(E3_EUNSUPPORTED, "sequence length %lld too large", Tkv);
  if (p->num_docs < 0) return fail(E3_EINVAL, "num_docs=%d must be >= 0", p->num_docs);
  r.ndocs = p->num_docs;
  if (p->num_docs >= 1) {
    const int32_t* cu = p->cu_seqlens_host;
    if (!cu) return fail(E3_EINVAL, "cu_seqlens_host is NULL with num_docs=%d", p->num_docs);
    if (cu[0] != 0) return fail(E3_EINVAL, "cu_seqlens[0]=%d must be 0", cu[0]);
    for (int i = 0; i < p->num_docs; ++i)
      if (cu[i + 1] < cu[i]) return fail(E3_EINVAL, "cu_seqlens must be non-decreasing (index %d)", i + 1);
    if (cu[p->num_docs] != Tkv)
      return fail(E3_EINVAL, "cu_seqlens ends at %d, the sequence length is %lld", cu[p->num_docs], Tkv);
    if (p->num_docs > 1) {
      if (p->B != 1) return fail(E3_EINVAL, "several documents (varlen) need B == 1");
      if (p->layout == E3_LAYOUT_ZIGZAG) {
        // every document is cut into 2cp chunks (zigzag_ring_attention page, `get_half_index`)
        for (int i = 0; i < p->num_docs; ++i)
          if ((cu[i + 1] - cu[i]) % (2 * p->cp) != 0)
            return fail(E3_EINVAL, "ZIGZAG: document %d has length %d, not a multiple of 2*cp = %d", i,
                        cu[i + 1] - cu[i], 2 * p->cp);
      }
      if (need_dev && !p->cu_seqlens_dev)
        return fail(E3_EINVAL, "cu_seqlens_dev is NULL with num_docs=%d", p->num_docs);
    }
  }
  r.N = p->num_blocks - 1;
  const long long HD = (long long)p->H * p->D;
  r.k0_bs = p->k0_batch_stride ? p->k0_batch_stride : Tkv * HD;
  r.kd_blk = p->kd_block_stride ? p->kd_block_stride : T * HD;
  r.kd_bs = p->kd_batch_stride ? p->kd_batch_stride : (long long)r.N * T * HD;
  if (r.k0_bs < 0 || r.kd_blk < 0 || r.kd_bs < 0 || (r.k0_bs % 8) || (r.kd_blk % 8) || (r.kd_bs % 8))
    return fail(E3_EINVAL, "strides must be non-negative multiples of 8 elements");
  // Rows of different batch rows or blocks must not overlap: the gradients are
  // written through the same strides, and overlapping rows would race.
  if (p->B > 1 && r.k0_bs < Tkv * HD)
    return fail(E3_EINVAL, "k0_batch_stride %lld < T_kv*H*D = %lld (batch rows would overlap)", r.k0_bs, Tkv * HD);
  if (r.N > 1 && r.kd_blk < T * HD)
    return fail(E3_EINVAL, "kd_block_stride %lld < T*H*D = %lld (blocks would overlap)", r.kd_blk, T * HD);
  if (p->B > 1 && r.N > 0 && r.kd_bs < (long long)(r.N - 1) * r.kd_blk + T * HD)
    return fail(E3_EINVAL, "kd_batch_stride %lld < (N-1)*kd_block_stride + T*H*D = %lld (batch rows would overlap)",
                r.kd_bs, (long long)(r.N - 1) * r.kd_blk + T * HD);
  return E3_OK;
}

e3::Geo geo_of(const e3_problem* p) {
  return e3::Geo{p->layout, p->cp, p->rank, p->T, p->T_kv, p->num_docs > 1 ? p->cu_seqlens_host : nullptr,
                 p->num_docs > 1 ? p->num_docs : 1};
}

e3::Args make_args(const e3_problem* p, const Resolved& r) {
  e3::Args a{};
  a.cu = p->num_docs > 1 ? p->cu_seqlens_dev : nullptr;
  a.cu_host = p->num_docs > 1 ? p->cu_seqlens_host : nullptr;
  a.ndocs = p->num_docs > 1 ? p->num_docs : 1;
  a.B = p->B;
  a.T = p->T;
  a.Tkv = p->T_kv;
  a.H = p->H;
  a.N = r.N;
  a.k0_bs = r.k0_bs;
  a.kd_bs = r.kd_bs;
  a.kd_blk = r.kd_blk;
  a.scale = p->scale;
  a.c2 = p->scale * 1.4426950408889634f;
  a.layout = p->layout;
  a.cp = p->cp;
  a.rank = p->rank;
  a.step_lo = 0;
  a.step_hi = 1 << 30;
  const long long HD = (long long)p->H * p->D;
  a.q_bs = (long long)p->T * HD;
  a.q_hs = p->D;
  a.q_rs = HD;
  a.kv_hs = p->D;
  a.kv_rs = HD;
  return a;
}

int check_ptrs(const char* const* names, const void* const* ptrs, int n) {
  for (int i = 0; i < n; ++i) {
    if (!ptrs[i]) return fail(E3_EINVAL, "%s is NULL", names[i]);
    if (misaligned(ptrs[i])) return fail(E3_EINVAL, "%s is not 16-byte aligned", names[i]);
  }
  return E3_OK;
}

int fwd_impl(const e3_problem* p, const void* q, const void* k0, const void* v0, const void* kd,
             const void* vd, void* out, float* lse, hipStream_t st, bool whole) {
  Resolved r;
  int rc = validate(p, r, whole);
  if (rc) return rc;
  if (p->T == 0) return ok();
  {
    const char* names[] = {"q", "k0", "v0", "out", "lse"};
    const void* ptrs[] = {q, k0, v0, out, lse};
    if ((rc = check_ptrs(names, ptrs, 5))) return rc;
  }
  if (r.N > 0) {
    const char* names[] = {"kd", "vd"};
    const void* ptrs[] = {kd, vd};
    if ((rc = check_ptrs(names, ptrs, 2))) return rc;
  }
  timing_reset();
  e3::Args a = make_args(p, r);
  a.q = q;
  a.k0 = k0;
  a.v0 = v0;
  a.kd = kd;
  a.vd = vd;
  a.out = out;
  a.lse = lse;
  hipError_t e = e3::launch_fwd(a, p->dtype, p->D, st);
  if (e != hipSuccess) return fail(E3_EHIP, "forward launch failed: %s", hipGetErrorString(e));
  return ok();
}

// Backward workspace: lse2 and delta (float [B,H,P], P = the 64-aligned per-run
// row layout of the local queries), then the block-0 part of dq (float
// [B,T,H,D], when there are diagonal blocks).
struct BwdWs {
  int pitch;
  size_t delta, dqd, total;
};

BwdWs bwd_ws_layout(const e3_problem* p) {
  BwdWs l;
  l.pitch = geo_of(p).pitch();
  const size_t rows = (size_t)p->B * p->H * l.pitch;       // multiple of 64
  l.delta = rows * sizeof(float);
  l.dqd = 2 * rows * sizeof(float);
  const int N = p->num_blocks - 1;
  l.total = l.dqd + (N > 0 ? (size_t)p->B * p->T * p->H * p->D * sizeof(float) : 0);
  return l;
}

int bwd_impl(const e3_problem* p, const void* dout, const void* q, const void* k0, const void* v0,
             const void* kd, const void* vd, const void* out, const float* lse, void* ws, void* dq,
             void* dk0, void* dv0, void* dkd, void* dvd, hipStream_t st, bool whole) {
  Resolved r;
  int rc = validate(p, r, whole);
  if (rc) return rc;
  if (p->T == 0) return ok();
  {
    const char* names[] = {"dout", "q", "k0", "v0", "out", "lse", "workspace", "dq", "dk0", "dv0"};
    const void* ptrs[] = {dout, q, k0, v0, out, lse, ws, dq, dk0, dv0};
    if ((rc = check_ptrs(names, ptrs, 10))) return rc;
  }
  if (r.N > 0) {
    const char* names[] = {"kd", "vd", "dkd", "dvd"};
    const void* ptrs[] = {kd, vd, dkd, dvd};
    if ((rc = check_ptrs(names, ptrs, 4))) return rc;
  }
  timing_reset();
  e3::Args a = make_args(p, r);
  a.q = q;
  a.k0 = k0;
  a.v0 = v0;
  a.kd = kd;
  a.vd = vd;
  a.dout = dout;
  a.o_in = out;
  a.lse_in = lse;
  {
    const BwdWs l = bwd_ws_layout(p);
    if (l.delta > 0xffffffffull)   // the kernels address delta from lse*log2(e) with a 32-bit offset
      return fail(E3_EUNSUPPORTED, "B*H*P = %zu rows of delta do not fit a 32-bit byte offset", l.delta / 4);
    char* w = static_cast<char*>(ws);
    a.q_pitch = l.pitch;
    a.lse2 = reinterpret_cast<float*>(w);
    a.delta = reinterpret_cast<float*>(w + l.delta);
    a.dqd = reinterpret_cast<float*>(w + l.dqd);
  }
  a.dq = dq;
  a.dk0 = dk0;
  a.dv0 = dv0;
  a.dkd = dkd;
  a.dvd = dvd;
  hipError_t e = e3::launch_bwd(a, p->dtype, p->D, st);
  if (e != hipSuccess) return fail(E3_EHIP, "backward launch failed: %s", hipGetErrorString(e));
  return ok();
}

int doc_lo_host(const e3_problem* p, int pos) {
  return e3::doc_lo_of(p->cu_seqlens_host, p->num_docs > 1 ? p->num_docs : 1, pos);
}

}  // namespace

// ---- no-allocation backward: a static device scratch array -----------------------
// Holds lse*log2(e) and delta (float32, 2 x B*H*P) for eagle3_bwd_noalloc. In host
// code `scratch` names a host-side stand-in, never the device memory: kernels get
// the address hipGetSymbolAddress returns, looked up once per device.
namespace {
constexpr size_t kScratchBytes = size_t(16) << 20;
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_dev[kMaxDevices] = {};
}  // namespace
static __device__ __align__(256) char scratch[kScratchBytes];

namespace {
hipError_t scratch_ptr(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (!g_scratch_dev[dev]) {
    void* p = nullptr;
    if ((e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch))) != hipSuccess) return e;
    g_scratch_dev[dev] = p;
  }
  *out = g_scratch_dev[dev];
  return hipSuccess;
}

struct SideRes {
  hipStream_t s = nullptr;
  hipEvent_t fork[2] = {nullptr, nullptr}, join[2] = {nullptr, nullptr};
};
thread_local std::map<int, SideRes> t_side;

hipError_t side_res(SideRes*& out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  SideRes& r = t_side[dev];
  if (!r.s) {
    if ((e = hipStreamCreateWithFlags(&r.s, hipStreamNonBlocking)) != hipSuccess) return e;
    for (int k = 0; k < 2; ++k) {
      if ((e = hipEventCreateWithFlags(&r.fork[k], hipEventDisableTiming)) != hipSuccess) return e;
      if ((e = hipEventCreateWithFlags(&r.join[k], hipEventDisableTiming)) != hipSuccess) return e;
    }
  }
  out = &r;
  return hipSuccess;
}
}  // namespace

hipError_t e3::side_begin(hipStream_t main, int k, hipStream_t& side) {
  SideRes* r = nullptr;
  hipError_t e = side_res(r);
  if (e != hipSuccess) return e;
  if ((e = hipEventRecord(r->fork[k], main)) != hipSuccess) return e;
  if ((e = hipStreamWaitEvent(r->s, r->fork[k], 0)) != hipSuccess) return e;
  side = r->s;
  return hipSuccess;
}

hipError_t e3::side_end(hipStream_t main, int k) {
  SideRes* r = nullptr;
  hipError_t e = side_res(r);
  if (e != hipSuccess) return e;
  if ((e = hipEventRecord(r->join[k], r->s)) != hipSuccess) return e;
  return hipStreamWaitEvent(main, r->join[k], 0);
}

void e3::timing_mark(hipStream_t st) {
  if (g_events && g_events_n < g_events_cap) (void)hipEventRecord(g_events[g_events_n++], st);
}

extern "C" {

int eagle3_set_timing_events(hipEvent_t* events, int capacity) {
  g_events = capacity > 0 ? events : nullptr;
  g_events_cap = events ? capacity : 0;
  g_events_n = 0;
  return E3_OK;
}

int eagle3_timing_events_recorded(void) { return g_events_n; }

int eagle3_abi_version(void) { return EAGLE3_ABI_VERSION; }

const char* eagle3_last_error(void) { return g_err.c_str(); }

size_t eagle3_bwd_workspace_bytes(const e3_problem* p) {
  Resolved r;
  if (validate(p, r, false, false)) return 0;
  g_err.clear();
  if (p->T == 0) return 0;
  return bwd_ws_layout(p).total;
}



int eagle3_attn_fwd(const e3_problem* p, const void* q, const void* k0, const void* v0, const void* kd,
                    const void* vd, void* out, float* lse, hipStream_t stream) {
  return fwd_impl(p, q, k0, v0, kd, vd, out, lse, stream, true);
}

int eagle3_shard_fwd(const e3_problem* p, const void* q, const void* k0, const void* v0,
                     const void* kd, const void* vd, void* out, float* lse, hipStream_t stream) {
  return fwd_impl(p, q, k0, v0, kd, vd, out, lse, stream, false);
}

int eagle3_attn_bwd(const e3_problem* p, const void* dout, const void* q, const void* k0,
                    const void* v0, const void* kd, const void* vd, const void* out, const float* lse,
                    void* workspace, void* dq, void* dk0, void* dv0, void* dkd, void* dvd,
                    hipStream_t stream) {
  return bwd_impl(p, dout, q, k0, v0, kd, vd, out, lse, workspace, dq, dk0, dv0, dkd, dvd, stream, true);
}

int eagle3_shard_bwd(const e3_problem* p, const void* dout, const void* q, const void* k0,
                     const void* v0, const void* kd, const void* vd, const void* out, const float* lse,
                     void* workspace, void* dq, void* dk0, void* dv0, void* dkd, void* dvd,
                     hipStream_t stream) {
  return bwd_impl(p, dout, q, k0, v0, kd, vd, out, lse, workspace, dq, dk0, dv0, dkd, dvd, stream, false);
}

int eagle3_bwd_noalloc(const e3_problem* p, const void* dout, const void* q, const void* k0, const void* v0,
                       const void* kd, const void* vd, const void* out, const float* lse, void* dq, void* dk0,
                       void* dv0, void* dkd, void* dvd, hipStream_t stream) {
  Resolved r;
  int rc = validate(p, r, false);
  if (rc) return rc;
  if (p->T == 0) return ok();
  {
    const char* names[] = {"dout", "q", "k0", "v0", "out", "lse", "dq", "dk0", "dv0"};
    const void* ptrs[] = {dout, q, k0, v0, out, lse, dq, dk0, dv0};
    if ((rc = check_ptrs(names, ptrs, 9))) return rc;
  }
  if (r.N > 0) {
    const char* names[] = {"kd", "vd", "dkd", "dvd"};
    const void* ptrs[] = {kd, vd, dkd, dvd};
    if ((rc = check_ptrs(names, ptrs, 4))) return rc;
  }
  const BwdWs l = bwd_ws_layout(p);
  if (l.dqd > kScratchBytes)
    return fail(E3_EINVAL, "eagle3_bwd_noalloc: needs %zu bytes of scratch (2 x B*H*P floats), the static "
                "scratch holds %zu; use eagle3_shard_bwd with a workspace", l.dqd, kScratchBytes);
  void* sp = nullptr;
  hipError_t e = scratch_ptr(&sp);
  if (e != hipSuccess) return fail(E3_EHIP, "eagle3_bwd_noalloc: scratch address: %s", hipGetErrorString(e));
  timing_reset();
  e3::Args a = make_args(p, r);
  a.dq_in_out = 1;
  a.q = q;
  a.k0 = k0;
  a.v0 = v0;
  a.kd = kd;
  a.vd = vd;
  a.dout = dout;
  a.o_in = out;
  a.lse_in = lse;
  a.q_pitch = l.pitch;
  a.lse2 = reinterpret_cast<float*>(sp);
  a.delta = reinterpret_cast<float*>(static_cast<char*>(sp) + l.delta);
  a.dqd = nullptr;
  a.dq = dq;
  a.dk0 = dk0;
  a.dv0 = dv0;
  a.dkd = dkd;
  a.dvd = dvd;
  e = e3::launch_bwd(a, p->dtype, p->D, stream);
  if (e != hipSuccess) return fail(E3_EHIP, "backward launch failed: %s", hipGetErrorString(e));
  return ok();
}

size_t eagle3_bwd_noalloc_max_scratch_bytes(void) { return kScratchBytes; }

int lse_merge(float* out, float* lse, const float* block_out, const float* block_lse, int B, int T,
              int H, int D, int block_lse_layout, hipStream_t stream) {
  if (B < 1 || T < 0 || H < 1 || D < 4 || D % 4 != 0)
    return fail(E3_EINVAL, "lse_merge: bad shape B=%d T=%d H=%d D=%d (D must be a multiple of 4)", B, T, H, D);
  if (block_lse_layout != 0 && block_lse_layout != 1)
    return fail(E3_EINVAL, "lse_merge: block_lse_layout must be 0 ([B,H,T]) or 1 ([B,T,H])");
  if (T == 0) return ok();
  const char* names[] = {"out", "lse", "block_out", "block_lse"};
  const void* ptrs[] = {out, lse, block_out, block_lse};
  for (int i = 0; i < 4; ++i) {
    if (!ptrs[i]) return fail(E3_EINVAL, "lse_merge: %s is NULL", names[i]);
    if (reinterpret_cast<uintptr_t>(ptrs[i]) & 3u) return fail(E3_EINVAL, "lse_merge: %s misaligned", names[i]);
  }
  if ((reinterpret_cast<uintptr_t>(out) | reinterpret_cast<uintptr_t>(block_out)) & 15u)
    return fail(E3_EINVAL, "lse_merge: out and block_out must be 16-byte aligned");
  hipError_t e = e3::launch_lse_merge(out, lse, block_out, block_lse, B, T, H, D, block_lse_layout, stream);
  if (e != hipSuccess) return fail(E3_EHIP, "lse_merge launch failed: %s", hipGetErrorString(e));
  return ok();
}

int eagle3_target_cp_fwd(const e3_problem* p, const void* q, const void* k, const void* v, void* out,
                         float* lse, hipStream_t stream) {
  Resolved r;
  int rc = validate(p, r, false);
  if (rc) return rc;
  if (p->layout != E3_LAYOUT_FULL && p->layout != E3_LAYOUT_CONTIGUOUS)
    return fail(E3_EINVAL, "the frozen-target forward takes the FULL or CONTIGUOUS layout");
  if (p->num_blocks != 1) return fail(E3_EINVAL, "the frozen-target forward has no diagonal blocks: num_blocks must be 1");
  if (p->k0_batch_stride || p->kd_batch_stride || p->kd_block_stride)
    return fail(E3_EINVAL, "the frozen-target forward takes dense head-major tensors (strides must be 0)");
  if (p->T == 0) return ok();
  {
    const char* names[] = {"q", "k", "v", "out"};
    const void* ptrs[] = {q, k, v, out};
    if ((rc = check_ptrs(names, ptrs, 4))) return rc;
  }
  if (lse && misaligned(lse)) return fail(E3_EINVAL, "lse is not 16-byte aligned");
  timing_reset();
  e3::Args a = make_args(p, r);
  const long long D = p->D, T = p->T, Tkv = p->T_kv;
  a.q_bs = (long long)p->H * T * D;    // head-major [B, H, T, D]
  a.q_hs = T * D;
  a.q_rs = D;
  a.k0_bs = (long long)p->H * Tkv * D; // head-major [B, H, T_kv, D]
  a.kv_hs = Tkv * D;
  a.kv_rs = D;
  a.q = q;
  a.k0 = k;
  a.v0 = v;
  a.out = out;
  a.lse = lse;
  hipError_t e = e3::launch_fwd(a, p->dtype, p->D, stream);
  if (e != hipSuccess) return fail(E3_EHIP, "frozen-target forward launch failed: %s", hipGetErrorString(e));
  return ok();
}

int eagle3_ring_fwd_step(const e3_problem* p, int step, const void* q, const void* k0, const void* v0,
                         float* out_step, float* lse_step, hipStream_t stream) {
  Resolved r;
  int rc = validate(p, r, false);
  if (rc) return rc;
  const int nsteps = geo_of(p).nsteps();
  if (step < 0 || step >= nsteps) return fail(E3_EINVAL, "ring step %d out of range [0, %d)", step, nsteps);
  if (p->T == 0) return ok();
  {
    const char* names[] = {"q", "k0", "v0", "out_step", "lse_step"};
    const void* ptrs[] = {q, k0, v0, out_step, lse_step};
    if ((rc = check_ptrs(names, ptrs, 5))) return rc;
  }
  timing_reset();
  e3::Args a = make_args(p, r);
  a.N = 0;                 // block 0 only; the diagonals are merged by eagle3_diag_merge_fwd
  a.step_lo = step;
  a.step_hi = step + 1;
  a.out_f32 = 1;
  a.q = q;
  a.k0 = k0;
  a.v0 = v0;
  a.out = out_step;
  a.lse = lse_step;
  hipError_t e = e3::launch_fwd(a, p->dtype, p->D, stream);
  if (e != hipSuccess) return fail(E3_EHIP, "ring-step forward launch failed: %s", hipGetErrorString(e));
  return ok();
}

int eagle3_diag_merge_fwd(const e3_problem* p, const void* q, const void* kd, const void* vd,
                          const float* out_acc, const float* lse_acc, void* out, float* lse,
                          hipStream_t stream) {
  Resolved r;
  int rc = validate(p, r, false);
  if (rc) return rc;
  if (p->T == 0) return ok();
  {
    const char* names[] = {"q", "out_acc", "lse_acc", "out", "lse"};
    const void* ptrs[] = {q, out_acc, lse_acc, out, lse};
    if ((rc = check_ptrs(names, ptrs, 5))) return rc;
  }
  if (r.N > 0) {
    const char* names[] = {"kd", "vd"};
    const void* ptrs[] = {kd, vd};
    if ((rc = check_ptrs(names, ptrs, 2))) return rc;
  }
  timing_reset();
  e3::Args a = make_args(p, r);
  a.q = q;
  a.kd = kd;
  a.vd = vd;
  a.out = out;
  a.lse = lse;
  hipError_t e = e3::launch_diag_merge(a, out_acc, lse_acc, p->dtype, p->D, stream);
  if (e != hipSuccess) return fail(E3_EHIP, "diagonal merge launch failed: %s", hipGetErrorString(e));
  return ok();
}

int eagle3_ring_bwd_step(const e3_problem* p, int step, const void* dout, const void* q, const void* k0,
                         const void* v0, const void* out, const float* lse, void* workspace, float* dq_acc,
                         float* dk0_acc, float* dv0_acc, hipStream_t stream) {
  Resolved r;
  int rc = validate(p, r, false);
  if (rc) return rc;
  const int nsteps = geo_of(p).nsteps();
  if (step < 0 || step >= nsteps) return fail(E3_EINVAL, "ring step %d out of range [0, %d)", step, nsteps);
  if (p->T == 0) return ok();
  {
    const char* names[] = {"dout", "q", "k0", "v0", "out", "lse", "workspace", "dq_acc", "dk0_acc", "dv0_acc"};
    const void* ptrs[] = {dout, q, k0, v0, out, lse, workspace, dq_acc, dk0_acc, dv0_acc};
    if ((rc = check_ptrs(names, ptrs, 10))) return rc;
  }
  timing_reset();
  e3::Args a = make_args(p, r);
  a.N = 0;                 // block 0 only; the diagonals are eagle3_diag_bwd's
  a.step_lo = step;
  a.step_hi = step + 1;
  a.dq_accum = 1;
  a.kv_accum = 1;
  a.q = q;
  a.k0 = k0;
  a.v0 = v0;
  a.dout = dout;
  a.o_in = out;
  a.lse_in = lse;
  {
    const BwdWs l = bwd_ws_layout(p);
    if (l.delta > 0xffffffffull)   // the kernels address delta from lse*log2(e) with a 32-bit offset
      return fail(E3_EUNSUPPORTED, "B*H*P = %zu rows of delta do not fit a 32-bit byte offset", l.delta / 4);
    char* w = static_cast<char*>(workspace);
    a.q_pitch = l.pitch;
    a.lse2 = reinterpret_cast<float*>(w);
    a.delta = reinterpret_cast<float*>(w + l.delta);
  }
  a.dqd = dq_acc;
  a.dk0 = dk0_acc;
  a.dv0 = dv0_acc;
  hipError_t e = e3::launch_bwd(a, p->dtype, p->D, stream);
  if (e != hipSuccess) return fail(E3_EHIP, "ring-step backward launch failed: %s", hipGetErrorString(e));
  return ok();
}

int eagle3_diag_bwd(const e3_problem* p, const void* dout, const void* q, const void* kd, const void* vd,
                    const void* out, const float* lse, const float* dq_acc, void* dq, void* dkd, void* dvd,
                    hipStream_t stream) {
  Resolved r;
  int rc = validate(p, r, false);
  if (rc) return rc;
  if (p->T == 0) return ok();
  {
    const char* names[] = {"dout", "q", "out", "lse", "dq_acc", "dq"};
    const void* ptrs[] = {dout, q, out, lse, dq_acc, dq};
    if ((rc = check_ptrs(names, ptrs, 6))) return rc;
  }
  if (r.N > 0) {
    const char* names[] = {"kd", "vd", "dkd", "dvd"};
    const void* ptrs[] = {kd, vd, dkd, dvd};
    if ((rc = check_ptrs(names, ptrs, 4))) return rc;
  }
  timing_reset();
  e3::Args a = make_args(p, r);
  a.q = q;
  a.kd = kd;
  a.vd = vd;
  a.dout = dout;
  a.o_in = out;
  a.lse_in = lse;
  a.dqd = dq_acc;
  a.dq = dq;
  a.dkd = dkd;
  a.dvd = dvd;
  hipError_t e = e3::launch_diag_bwd(a, p->dtype, p->D, stream);
  if (e != hipSuccess) return fail(E3_EHIP, "diagonal backward launch failed: %s", hipGetErrorString(e));
  return ok();
}

// Ulysses re-sharding: arguments shared by the four transforms.
static int ulysses_check(const char* what, int stage, int esz, int B, int S_local, int H, int D, int uly,
                         const void* src, const void* dst) {
  if (stage != 0 && stage != 1) return fail(E3_EINVAL, "%s: stage must be 0 (pack) or 1 (unpack)", what);
  if (esz == 0) return fail(E3_EINVAL, "%s: dtype must be E3_BF16 or E3_F32", what);
  if (B < 1 || S_local < 0 || H < 1 || D < 1 || uly < 1)
    return fail(E3_EINVAL, "%s: bad shape B=%d S_local=%d H=%d D=%d uly=%d", what, B, S_local, H, D, uly);
  if (H % uly != 0)   // ulysses_attention page, `_gather_seq_scatter_heads`
    return fail(E3_EINVAL, "%s: H=%d must divide by the Ulysses degree %d", what, H, uly);
  if ((long long)uly * S_local > 0x3fffffffLL) return fail(E3_EUNSUPPORTED, "%s: sequence too long", what);
  if (S_local == 0) return E3_OK;
  if (!src || !dst) return fail(E3_EINVAL, "%s: src / dst is NULL", what);
  if ((reinterpret_cast<uintptr_t>(src) | reinterpret_cast<uintptr_t>(dst)) & 3u)
    return fail(E3_EINVAL, "%s: src / dst must be 4-byte aligned", what);
  if (src == dst) return fail(E3_EINVAL, "%s: src and dst must not be the same buffer", what);
  return E3_OK;
}

static int seg_copy(const char* what, const e3::SegCopy& c, hipStream_t st) {
  hipError_t e = e3::launch_seg_copy(c, st);
  if (e != hipSuccess) return fail(E3_EHIP, "%s launch failed: %s", what, hipGetErrorString(e));
  return ok();
}

static int esize(int dtype) { return dtype == E3_BF16 ? 2 : dtype == E3_F32 ? 4 : 0; }

int eagle3_ulysses_seq_to_head(int stage, int dtype, int B, int S_local, int H, int D, int uly,
                               const void* src, void* dst, hipStream_t stream) {
  const char* what = "eagle3_ulysses_seq_to_head";
  const int es = esize(dtype);
  int rc = ulysses_check(what, stage, es, B, S_local, H, D, uly, src, dst);
  if (rc) return rc;
  if (((long long)(H / uly) * D * es) % 4 != 0)   // segments are moved in 4-byte words
    return fail(E3_EUNSUPPORTED, "%s: a segment of H/uly*D = %lld elements is not a multiple of 4 bytes", what,
                (long long)(H / uly) * D);
  if (S_local == 0) return ok();
  const long long Hl = H / uly, HD = (long long)H * D, RL = Hl * D, Sl = S_local, Sf = (long long)uly * Sl;
  e3::SegCopy c{static_cast<const char*>(src), static_cast<char*>(dst), 0, 0, 0, 0, 0, 0, 0, 0, 0, 0};
  if (stage == 0) {
    // x [B, S_local, H, D] -> send [uly][B][S_local][H/uly][D]: head group g goes to rank g
    c.n0 = uly; c.n1 = B; c.n2 = Sl;
    c.s0 = RL; c.s1 = Sl * HD; c.s2 = HD;
    c.d0 = (long long)B * Sl * RL; c.d1 = Sl * RL; c.d2 = RL;
    c.seg = RL;
  } else {
    // recv [uly][B][S_local][H/uly][D] (part j = sequence chunk j) -> y [B, uly*S_local, H/uly, D]
    c.n0 = uly; c.n1 = B; c.n2 = 1;
    c.s0 = (long long)B * Sl * RL; c.s1 = Sl * RL; c.s2 = 0;
    c.d0 = Sl * RL; c.d1 = Sf * RL; c.d2 = 0;
    c.seg = Sl * RL;
  }
  c.s0 *= es; c.s1 *= es; c.s2 *= es; c.d0 *= es; c.d1 *= es; c.d2 *= es; c.seg *= es;
  return seg_copy(what, c, stream);
}

int eagle3_ulysses_head_to_seq(int stage, int dtype, int B, int S_local, int H, int D, int uly,
                               const void* src, void* dst, hipStream_t stream) {
  const char* what = "eagle3_ulysses_head_to_seq";
  const int es = esize(dtype);
  int rc = ulysses_check(what, stage, es, B, S_local, H, D, uly, src, dst);
  if (rc) return rc;
  if (((long long)(H / uly) * D * es) % 4 != 0)   // segments are moved in 4-byte words
    return fail(E3_EUNSUPPORTED, "%s: a segment of H/uly*D = %lld elements is not a multiple of 4 bytes", what,
                (long long)(H / uly) * D);
  if (S_local == 0) return ok();
  const long long Hl = H / uly, HD = (long long)H * D, RL = Hl * D, Sl = S_local, Sf = (long long)uly * Sl;
  e3::SegCopy c{static_cast<const char*>(src), static_cast<char*>(dst), 0, 0, 0, 0, 0, 0, 0, 0, 0, 0};
  if (stage == 0) {
    // y [B, uly*S_local, H/uly, D] -> send [uly][B][S_local][H/uly][D]: sequence chunk j goes to rank j
    c.n0 = uly; c.n1 = B; c.n2 = 1;
    c.s0 = Sl * RL; c.s1 = Sf * RL; c.s2 = 0;
    c.d0 = (long long)B * Sl * RL; c.d1 = Sl * RL; c.d2 = 0;
    c.seg = Sl * RL;
  } else {
    // recv [uly][B][S_local][H/uly][D] (part g = head group g) -> x [B, S_local, H, D]
    c.n0 = uly; c.n1 = B; c.n2 = Sl;
    c.s0 = (long long)B * Sl * RL; c.s1 = Sl * RL; c.s2 = RL;
    c.d0 = RL; c.d1 = Sl * HD; c.d2 = HD;
    c.seg = RL;
  }
  c.s0 *= es; c.s1 *= es; c.s2 *= es; c.d0 *= es; c.d1 *= es; c.d2 *= es; c.seg *= es;
  return seg_copy(what, c, stream);
}

int eagle3_ulysses_lse_gather(int stage, int B, int S_local, int H, int uly, const float* src, float* dst,
                              hipStream_t stream) {
  const char* what = "eagle3_ulysses_lse_gather";
  int rc = ulysses_check(what, stage, 4, B, S_local, H, 1, uly, src, dst);
  if (rc) return rc;
  if (S_local == 0) return ok();
  const long long Hl = H / uly, Sl = S_local, Sf = (long long)uly * Sl;
  e3::SegCopy c{reinterpret_cast<const char*>(src), reinterpret_cast<char*>(dst), 0, 0, 0, 0, 0, 0, 0, 0, 0, 0};
  if (stage == 0) {
    // lse [B, H, S_local] -> send [uly][B][H/uly][S_local]: head group g goes to rank g
    c.n0 = uly; c.n1 = B; c.n2 = 1;
    c.s0 = Hl * Sl; c.s1 = (long long)H * Sl; c.s2 = 0;
    c.d0 = (long long)B * Hl * Sl; c.d1 = Hl * Sl; c.d2 = 0;
    c.seg = Hl * Sl;
  } else {
    // recv [uly][B][H/uly][S_local] (part j = sequence chunk j) -> [B, H/uly, uly*S_local], contiguous
    c.n0 = uly; c.n1 = B; c.n2 = Hl;
    c.s0 = (long long)B * Hl * Sl; c.s1 = Hl * Sl; c.s2 = Sl;
    c.d0 = Sl; c.d1 = Hl * Sf; c.d2 = Sf;
    c.seg = Sl;
  }
  c.s0 *= 4; c.s1 *= 4; c.s2 *= 4; c.d0 *= 4; c.d1 *= 4; c.d2 *= 4; c.seg *= 4;
  return seg_copy(what, c, stream);
}

int eagle3_ulysses_lse_scatter(int stage, int B, int S_local, int H, int uly, const float* src, float* dst,
                               hipStream_t stream) {
  const char* what = "eagle3_ulysses_lse_scatter";
  int rc = ulysses_check(what, stage, 4, B, S_local, H, 1, uly, src, dst);
  if (rc) return rc;
  if (S_local == 0) return ok();
  const long long Hl = H / uly, Sl = S_local, Sf = (long long)uly * Sl;
  e3::SegCopy c{reinterpret_cast<const char*>(src), reinterpret_cast<char*>(dst), 0, 0, 0, 0, 0, 0, 0, 0, 0, 0};
  if (stage == 0) {
    // [B, H/uly, uly*S_local] -> send [uly][B][H/uly][S_local]: sequence chunk j goes to rank j
    c.n0 = uly; c.n1 = B; c.n2 = Hl;
    c.s0 = Sl; c.s1 = Hl * Sf; c.s2 = Sf;
    c.d0 = (long long)B * Hl * Sl; c.d1 = Hl * Sl; c.d2 = Sl;
    c.seg = Sl;
  } else {
    // recv [uly][B][H/uly][S_local] (part g = head group g) -> lse [B, H, S_local]
    c.n0 = uly; c.n1 = B; c.n2 = 1;
    c.s0 = (long long)B * Hl * Sl; c.s1 = Hl * Sl; c.s2 = 0;
    c.d0 = Hl * Sl; c.d1 = (long long)H * Sl; c.d2 = 0;
    c.seg = Hl * Sl;
  }
  c.s0 *= 4; c.s1 *= 4; c.s2 *= 4; c.d0 *= 4; c.d1 *= 4; c.d2 *= 4; c.seg *= 4;
  return seg_copy(what, c, stream);
}

int eagle3_query_positions(const e3_problem* p, int64_t* pos) {
  Resolved r;
  int rc = validate(p, r, false, false);
  if (rc) return rc;
  if (!pos && p->T) return fail(E3_EINVAL, "pos_host is NULL");
  const e3::Geo g = geo_of(p);
  for (int ri = 0; ri < g.nruns(); ++ri) {
    int ls, len, gb;
    g.run(ri, ls, len, gb);
    for (int i = 0; i < len; ++i) pos[ls + i] = gb + i;
  }
  return ok();
}

int64_t eagle3_pair_count(const e3_problem* p) {
  Resolved r;
  int rc = validate(p, r, false, false);
  if (rc) return rc;
  const e3::Geo g = geo_of(p);
  int64_t n = 0;
  for (int ri = 0; ri < g.nruns(); ++ri) {
    int ls, len, gb;
    g.run(ri, ls, len, gb);
    for (int i = 0; i < len; ++i) n += (gb + i) - doc_lo_host(p, gb + i) + 1;
  }
  g_err.clear();
  return n;
}

int eagle3_fwd_tiles(const e3_problem* p, int32_t* tile_rows) {
  Resolved r;
  int rc = validate(p, r, false, false);
  if (rc) return rc;
  if (tile_rows) *tile_rows = e3::fwd_tile_rows();
  g_err.clear();
  return geo_of(p).ntiles(e3::fwd_tile_rows());
}

int eagle3_fwd_tile_segments(const e3_problem* p, int tile, int32_t* rows, int32_t* seg, int max_segments) {
  Resolved r;
  int rc = validate(p, r, false, false);
  if (rc) return rc;
  const e3::Geo g = geo_of(p);
  const int BM = e3::fwd_tile_rows(), BN = e3::fwd_tile_keys();
  if (tile < 0 || tile >= g.ntiles(BM)) return fail(E3_EINVAL, "tile %d out of range", tile);
  int row0, nrows, gpos0;
  g.qtile(tile, BM, row0, nrows, gpos0);
  if (rows) {
    rows[0] = row0;
    rows[1] = row0 + nrows;
  }
  const int g_min = gpos0, g_max = gpos0 + nrows - 1;
  const int lo_min = doc_lo_host(p, g_min), lo_max = doc_lo_host(p, g_max);
  e3::SegIter it;
  it.begin(g, lo_min, g_max + 1, BN);
  int n = 0;
  while (it.valid) {
    if (seg && n < max_segments) {
      const int s0 = it.s0, e = (s0 + BN) < it.b ? (s0 + BN) : it.b;
      const bool interior = s0 >= it.a && s0 + BN <= it.b && s0 >= lo_max && s0 + BN - 1 <= g_min;
      seg[3 * n + 0] = s0 > it.a ? s0 : it.a;
      seg[3 * n + 1] = e;
      seg[3 * n + 2] = interior ? 0 : 1;
    }
    ++n;
    it.next(g, BN);
  }
  g_err.clear();
  return n;
}

}  // extern "C"
