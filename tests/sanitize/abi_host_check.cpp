// Host-side check of the C ABI library's validation and shard driver, built with
// AddressSanitizer and UndefinedBehaviorSanitizer (host code only) by
// tests/test_sanitize_host.py. It links the library's host source with stub
// launchers (no GPU, no kernel): every compute entry point it calls either fails
// validation or reaches a stub that reports a launch failure.
//
// Seeded random problems of every layout (valid and invalid) are passed to
// eagle3_bwd_workspace_bytes, eagle3_pair_count, eagle3_query_positions,
// eagle3_fwd_tiles and eagle3_fwd_tile_segments; for valid ones the positions
// are checked to be distinct and in range, the pair count against a plain count
// from the positions and documents, and the key tiles of every query tile to
// count each visible key exactly once.
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <random>
#include <set>
#include <vector>

#include "eagle3_attn.h"
#include "e3_common.h"

namespace e3 {
// Stub launchers: the sanitizer build has no device code.
hipError_t launch_fwd(const Args&, int, int, hipStream_t) { return hipErrorNotSupported; }
hipError_t launch_bwd(const Args&, int, int, hipStream_t) { return hipErrorNotSupported; }
hipError_t launch_lse_merge(float*, float*, const float*, const float*, int, int, int, int, int, hipStream_t) {
  return hipErrorNotSupported;
}
hipError_t launch_diag_merge(const Args&, const float*, const float*, int, int, hipStream_t) {
  return hipErrorNotSupported;
}
hipError_t launch_diag_bwd(const Args&, int, int, hipStream_t) { return hipErrorNotSupported; }
hipError_t launch_seg_copy(const SegCopy&, hipStream_t) { return hipErrorNotSupported; }
int fwd_tile_rows() { return 128; }
int fwd_tile_keys() { return 64; }
}  // namespace e3

static int failures = 0;
#define CHECK(c)                                                              \
  do {                                                                        \
    if (!(c)) {                                                               \
      std::fprintf(stderr, "check failed at line %d: %s\n", __LINE__, #c);   \
      if (++failures > 20) std::exit(1);                                      \
    }                                                                         \
  } while (0)

int main(int argc, char** argv) {
  const int cases = argc > 1 ? std::atoi(argv[1]) : 400;
  std::mt19937 rng(12345);
  auto uni = [&](int lo, int hi) { return std::uniform_int_distribution<int>(lo, hi)(rng); };
  int valid = 0;
  for (int c = 0; c < cases; ++c) {
    e3_problem p{};
    p.dtype = uni(0, 2) == 2 ? 7 : uni(0, 1);           // sometimes an invalid dtype
    p.D = uni(0, 9) == 0 ? 96 : (uni(0, 1) ? 64 : 128);
    p.H = uni(0, 20) == 0 ? 0 : uni(1, 4);
    p.num_blocks = uni(0, 18);
    p.scale = uni(0, 15) == 0 ? -1.f : 0.125f;
    p.layout = uni(0, 4);                               // 4 is invalid
    p.cp = uni(1, 5);
    p.rank = uni(0, 20) == 0 ? p.cp : uni(0, p.cp - 1);
    const int unit = p.layout == 2 ? 2 * p.cp : (p.layout == 1 ? p.cp : 1);
    int S = unit * uni(0, 160 / unit + 1) + (uni(0, 12) == 0 ? 1 : 0);
    p.B = (p.layout == 2 || uni(0, 1)) ? 1 : uni(1, 3);
    if (p.layout == 1 || p.layout == 2) {
      p.T = S / p.cp;
      p.T_kv = uni(0, 15) == 0 ? S + 1 : S;
    } else {
      if (p.layout == 0) p.cp = 1, p.rank = 0;
      p.T = S;
      p.T_kv = S;
    }
    // documents (several need B == 1; zig-zag needs lengths divisible by 2cp)
    std::vector<int32_t> cu;
    if (uni(0, 2) > 0) {
      cu.push_back(0);
      while (cu.back() < p.T_kv) {
        int len = p.layout == 2 ? 2 * p.cp * uni(0, 6) : uni(0, 40);
        if (uni(0, 30) == 0) len = 1;
        cu.push_back(std::min(p.T_kv, cu.back() + len));
      }
      if (cu.size() == 1) cu.push_back(p.T_kv);
      p.num_docs = (int)cu.size() - 1;
      p.cu_seqlens_host = cu.data();
      p.cu_seqlens_dev = reinterpret_cast<const int32_t*>(0x1000);   // never dereferenced on the host
    }
    const size_t ws = eagle3_bwd_workspace_bytes(&p);
    const int64_t pairs = eagle3_pair_count(&p);
    if (pairs < 0) {                                    // invalid: every entry point agrees
      CHECK(ws == 0);
      CHECK(eagle3_attn_fwd(&p, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr) != E3_OK ||
            p.T == 0);
      continue;
    }
    ++valid;
    std::vector<int64_t> pos(p.T > 0 ? p.T : 1, -1);
    CHECK(eagle3_query_positions(&p, pos.data()) == E3_OK);
    std::set<int64_t> seen;
    for (int i = 0; i < p.T; ++i) {
      CHECK(pos[i] >= 0 && pos[i] < p.T_kv);
      seen.insert(pos[i]);
    }
    CHECK((int)seen.size() == p.T);
    auto doc_lo = [&](int64_t g) -> int64_t {
      if (p.num_docs <= 1) return 0;
      int64_t lo = 0;
      for (int d = 0; d < p.num_docs; ++d)
        if (cu[d] <= g && g < cu[d + 1]) lo = cu[d];
      return lo;
    };
    int64_t want = 0;
    for (int i = 0; i < p.T; ++i) want += pos[i] - doc_lo(pos[i]) + 1;
    CHECK(pairs == want);
    int32_t rows = 0;
    const int nt = eagle3_fwd_tiles(&p, &rows);
    CHECK(nt >= 0 && rows == 128);
    std::vector<int> cover(p.T > 0 ? p.T : 1, 0);
    for (int t = 0; t < nt; ++t) {
      int32_t rr[2];
      const int n = eagle3_fwd_tile_segments(&p, t, rr, nullptr, 0);
      CHECK(n >= 0);
      std::vector<int32_t> seg(3 * (n > 0 ? n : 1));
      CHECK(eagle3_fwd_tile_segments(&p, t, rr, seg.data(), n) == n);
      CHECK(0 <= rr[0] && rr[0] < rr[1] && rr[1] <= p.T && rr[1] - rr[0] <= 128);
      for (int r = rr[0]; r < rr[1]; ++r) {
        ++cover[r];
        const int64_t g = pos[r], lo = doc_lo(g);
        int64_t counted = 0;
        for (int k = 0; k < n; ++k)
          for (int64_t s = seg[3 * k]; s < seg[3 * k + 1]; ++s) counted += (s >= lo && s <= g);
        CHECK(counted == g - lo + 1);
      }
    }
    for (int r = 0; r < p.T; ++r) CHECK(cover[r] == 1);
    // compute entry points: null pointers are refused before any launch
    CHECK(eagle3_shard_fwd(&p, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr) ==
          (p.T == 0 ? E3_OK : E3_EINVAL));
    if (p.T > 0 && p.num_blocks == 1 && (p.layout == 0 || p.layout == 1) && p.dtype != 7) {
      void* a = reinterpret_cast<void*>(0x1000);
      // valid arguments reach the stub launcher: a launch failure, never a crash
      CHECK(eagle3_target_cp_fwd(&p, a, a, a, a, nullptr, nullptr) == E3_EHIP);
    }
  }
  // Ulysses transforms: argument checks and the stub launcher
  void* a = reinterpret_cast<void*>(0x1000);
  void* b = reinterpret_cast<void*>(0x2000);
  CHECK(eagle3_ulysses_seq_to_head(0, E3_BF16, 1, 16, 6, 128, 4, a, b, nullptr) == E3_EINVAL);   // 6 % 4
  CHECK(eagle3_ulysses_seq_to_head(2, E3_BF16, 1, 16, 8, 128, 4, a, b, nullptr) == E3_EINVAL);
  CHECK(eagle3_ulysses_seq_to_head(0, E3_BF16, 1, 16, 8, 128, 4, a, a, nullptr) == E3_EINVAL);
  CHECK(eagle3_ulysses_lse_gather(1, 1, 16, 8, 4, (float*)a, (float*)b, nullptr) == E3_EHIP);
  CHECK(lse_merge(nullptr, nullptr, nullptr, nullptr, 1, 4, 2, 6, 0, nullptr) == E3_EINVAL);
  std::printf("abi host check: %d cases, %d valid, %d failures\n", cases, valid, failures);
  return failures ? 1 : 0;
}
