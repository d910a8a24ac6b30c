// Drives the host side of the C ABI (argument validation, workspace sizing and
// the segment planners in la_api.hip) for a build with AddressSanitizer and
// UndefinedBehaviorSanitizer on the host code.  Every call here either returns a
// size or fails validation before any HIP call, so it runs without a GPU; the
// kernel launchers are replaced by stubs that abort if ever reached.  Shapes
// sweep batch, length, heads and chunk, including sizes near the planners'
// limits, and variable-length tables with empty, single-token and long
// sequences.  Exit status 0 = clean.
#include <stdio.h>
#include <stdlib.h>

#include <vector>

#include "la_internal.hpp"
#include "lightning_la.h"

[[noreturn]] static void reached(const char* what) {
  fprintf(stderr, "a kernel launcher was reached: %s\n", what);
  abort();
}

namespace la {
hipError_t launch_linear(const LinearParams&, hipStream_t) { reached("launch_linear"); }
hipError_t launch_prefill(const PrefillParams&, const PrefillPlan&, hipStream_t, hipEvent_t const*) { reached("launch_prefill"); }
hipError_t launch_decode(const DecodeParams&, hipStream_t) { reached("launch_decode"); }
hipError_t launch_segment_states(const BackwardParams&, const PrefillPlan&, bool, hipStream_t) { reached("launch_segment_states"); }
hipError_t launch_backward_chunks(const BackwardParams&, const PrefillPlan&, hipStream_t) { reached("launch_backward_chunks"); }
hipError_t launch_sparse_means(const SparseParams&, int, int, hipStream_t) { reached("launch_sparse_means"); }
hipError_t launch_sparse_prefill(const SparseParams&, int32_t*, hipStream_t) { reached("launch_sparse_prefill"); }
hipError_t launch_sparse_decode(const SparseParams&, hipStream_t) { reached("launch_sparse_decode"); }
}  // namespace la

#define CHECK(c) do { if (!(c)) { fprintf(stderr, "check failed: %s (line %d)\n", #c, __LINE__); return 1; } } while (0)

static uint64_t rng = 88172645463325252ull;
static uint64_t next() { rng ^= rng << 13; rng ^= rng >> 7; rng ^= rng << 17; return rng; }

int main() {
  typedef la_bf16 bf;
  // fake device addresses: never dereferenced, validation fails first
  bf* A = reinterpret_cast<bf*>((uintptr_t)1 << 40);
  auto at = [&](size_t mb) { return reinterpret_cast<bf*>(reinterpret_cast<uint8_t*>(A) + (mb << 20)); };
  float* Sf = reinterpret_cast<float*>(at(4096));
  // every value the enum's range holds (other integers, which callers in other
  // languages may pass, are covered through ctypes in the ABI tests)
  for (int s = 0; s <= 15; ++s) CHECK(la_status_string(static_cast<la_status>(s)) != nullptr);
  CHECK(la_version() > 0);

  // workspace sizes over many shapes, chunk sizes and extreme sizes
  const int Bs[] = {1, 2, 3, 8, 64, 1000, 65535, 1 << 20, 1 << 30};
  const int Ts[] = {1, 2, 63, 64, 65, 300, 4096, 32768, 262144, 1 << 20, 1 << 30, 2147483647};
  const int Hs[] = {1, 2, 32, 300, 1100, 65536, 1 << 24};
  const int Cs[] = {0, 64, 96, 128, 256, 512, -1};
  size_t nonzero = 0;
  for (int B : Bs)
    for (int T : Ts)
      for (int H : Hs)
        for (int C : Cs) {
          nonzero += la_prefill_workspace_bytes(B, T, H, 128, C) > 0;
          nonzero += la_layer_workspace_bytes(B, T, H, 128, C) > 0;
          nonzero += la_backward_workspace_bytes(B, T, H, 128, C) > 0;
          nonzero += la_sparse_prefill_workspace_bytes(B, T, H, 128, 0, 16) > 0;
        }
  CHECK(nonzero > 0);
  CHECK(la_prefill_workspace_bytes(0, 10, 1, 128, 0) == 0 && la_prefill_workspace_bytes(1, 10, 1, 64, 0) == 0);

  // validation failures of every entry point (no launch is reached)
  CHECK(la_prefill(nullptr, A, A, A, nullptr, Sf, at(64), 1, 64, 2, 128, 0, 0, 1e4f, 1e-6f, nullptr, nullptr, at(200),
                   1 << 20, nullptr) == LA_ERR_NULL_PTR);
  CHECK(la_prefill(A, at(8), at(16), at(24), nullptr, Sf, at(32), 1, 64, 2, 96, 0, 0, 1e4f, 1e-6f, nullptr, nullptr,
                   at(200), 1 << 20, nullptr) == LA_ERR_UNSUPPORTED);
  CHECK(la_prefill(A, at(8), at(16), at(24), nullptr, Sf, A, 1, 64, 2, 128, 0, 0, 1e4f, 1e-6f, nullptr, nullptr,
                   at(200), 1 << 20, nullptr) == LA_ERR_ALIASING);
  CHECK(la_prefill(A, at(8 << 10), at(16 << 10), at(24 << 10), nullptr, reinterpret_cast<float*>(at(40 << 10)),
                   at(32 << 10), 1, 65536, 300, 128, 0, 0, 1e4f, 1e-6f, nullptr, nullptr, at(48 << 10), 16,
                   nullptr) == LA_ERR_WORKSPACE);
  CHECK(la_prefill_noalloc(A, at(8), at(16), at(24), nullptr, Sf, A, 1, 64, 2, 128, 0, 0, 1e4f, 1e-6f, nullptr,
                           nullptr, nullptr) == LA_ERR_ALIASING);
  CHECK(la_decode_step(A, at(8), at(16), at(24), Sf, at(32) + 1, 4, 2, 128, 0, 1e4f, 1e-6f, nullptr, nullptr,
                       nullptr) == LA_ERR_ALIGNMENT);
  CHECK(la_linear(A, at(8), at(16), 100, 200, 64, nullptr) == LA_ERR_UNSUPPORTED);
  CHECK(la_layer_forward(A, at(8), at(16), nullptr, Sf, A, 1, 64, 512, 4, 128, 0, 0, 1e4f, 1e-6f, nullptr, nullptr,
                         at(300), 1 << 30, nullptr) == LA_ERR_ALIASING);
  CHECK(la_backward(A, at(8), at(16), at(24), nullptr, at(32), nullptr, at(40), at(48), at(56), at(64), Sf, nullptr,
                    nullptr, 1, 64, 2, 128, 0, 128, 1e4f, 1e-6f, nullptr, nullptr, at(300), 1 << 30,
                    nullptr) == LA_ERR_UNSUPPORTED);
  // the forward's workspace: smaller than la_prefill's for the shape, then overlapping an output
  // (activations of 10 MiB at this shape, 16 MiB apart)
  CHECK(la_backward_saved(A, at(16), at(32), at(48), nullptr, at(64), nullptr, at(80), at(96), at(112), at(128), Sf,
                          nullptr, nullptr, 1, 20000, 2, 128, 0, 0, 1e4f, 1e-6f, nullptr, nullptr, at(300), 1 << 30,
                          at(2048), 4096, nullptr) == LA_ERR_WORKSPACE);
  CHECK(la_backward_saved(A, at(16), at(32), at(48), nullptr, at(64), nullptr, at(80), at(96), at(112), at(128), Sf,
                          nullptr, nullptr, 1, 20000, 2, 128, 0, 0, 1e4f, 1e-6f, nullptr, nullptr, at(300), 1 << 30,
                          at(90), 1 << 26, nullptr) == LA_ERR_ALIASING);   // overlaps dq and dk
  CHECK(la_sparse_prefill(A, at(8), at(16), at(24), at(32), nullptr, 1, 100, 2, 128, 0, 0, at(300), 1 << 30,
                          nullptr) == LA_ERR_UNSUPPORTED);
  CHECK(la_sparse_block_means(A, Sf, 1, 1024, 2, 128, 0, 10, 7, nullptr) == LA_ERR_BAD_SHAPE);
  CHECK(la_sparse_decode(A, at(8), at(16), Sf, at(24), reinterpret_cast<int32_t*>(at(32)), at(40), nullptr, 1, 1024,
                         2, 128, 0, 65, nullptr) == LA_ERR_UNSUPPORTED);

  // variable-length planning: random tables with empty, single-token and long sequences
  for (int trial = 0; trial < 300; ++trial) {
    const int nseq = 1 + (int)(next() % 200);
    std::vector<int32_t> cu(nseq + 1, 0);
    std::vector<int64_t> pos(nseq);
    for (int b = 0; b < nseq; ++b) {
      const uint64_t r = next() % 10;
      const int32_t len = r < 2 ? 0 : r < 5 ? 1 : (int32_t)(next() % (r < 8 ? 300 : 70000));
      cu[b + 1] = cu[b] + len;
      pos[b] = (int64_t)(next() % 2000000);
    }
    const int H = 1 + (int)(next() % 40);
    for (int C : {0, 64, 128, 256}) {
      const size_t ws = la_prefill_varlen_workspace_bytes(nseq, cu.data(), H, 128, C);
      CHECK(ws > 0);
      // fails on the workspace size, after the planner ran on the table
      // buffers 16 TiB apart: no two can overlap whatever the table's size
      auto far = [](int i) { return reinterpret_cast<bf*>((uintptr_t)i << 44); };
      CHECK(la_prefill_varlen(far(1), far(2), far(3), far(4), cu.data(), pos.data(), nullptr,
                              reinterpret_cast<float*>(far(5)), far(6), nseq, cu[nseq], H, 128, C, 1e4f, 1e-6f,
                              nullptr, nullptr, far(7), ws - 1, nullptr) == LA_ERR_WORKSPACE);
    }
    // a malformed table: decreasing offsets
    if (nseq > 1) {
      std::vector<int32_t> bad(cu);
      bad[1] = bad[2] + 1;
      CHECK(la_prefill_varlen_workspace_bytes(nseq, bad.data(), H, 128, 0) == 0);
    }
  }
  printf("host driver: clean\n");
  return 0;
}
