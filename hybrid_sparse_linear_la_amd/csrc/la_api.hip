// C ABI of the linear-attention library: argument validation, work planning and
// kernel launch.  Validation finishes before anything is enqueued, so every
// error status leaves the outputs untouched.
#include <math.h>
#include <stdint.h>
#include <string.h>

#include <algorithm>
#include <atomic>
#include <mutex>
#include <utility>
#include <vector>

#include "la_internal.hpp"
#include "lightning_la.h"

namespace la {

namespace {

constexpr int kDefaultChunk = 64;
// Segment planning. The chunk-walking kernels run one workgroup per compute unit,
// and each workgroup pays a pipeline fill and a state hand-off per segment. One
// round of 256 workgroups is used while its segments stay within
// kLongSegmentChunks 64-token chunks; longer inputs are cut into segments of that
// length, up to kTargetWorkgroups workgroups (whole rounds), beyond which the
// segments grow instead. Measured on the 32-head layer: 32K and 64K tokens run
// about 9% faster in one round than in four, 128K-1M are as fast as or faster
// than with any other round count tried.
constexpr int64_t kComputeUnits = 256;
constexpr int64_t kLongSegmentChunks = 128;
constexpr int64_t kTargetWorkgroups = 1024;
// Launch-size limits (grid.x * block.x must stay below 2^32 work-items).
constexpr int64_t kMaxWorkgroups = (int64_t)1 << 23;
constexpr int64_t kMaxHeads = (int64_t)1 << 20;  // sequences x heads of one call

struct Range {
  uintptr_t lo, hi;
};

Range range_of(const void* p, uint64_t bytes) {
  const uintptr_t a = reinterpret_cast<uintptr_t>(p);
  return Range{a, a + (uintptr_t)bytes};
}

bool overlaps(const void* a, uint64_t na, const void* b, uint64_t nb) {
  if (!a || !b || na == 0 || nb == 0) return false;
  const Range x = range_of(a, na), y = range_of(b, nb);
  return x.lo < y.hi && y.lo < x.hi;
}

bool aligned16(const void* p) { return p == nullptr || (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

void rope_freqs(float base, RopeFreqs* f) {
  const double two_pi = 6.283185307179586476925287;
  for (int i = 0; i < kFreqs; ++i)
    f->rev[i] = pow((double)base, -2.0 * (double)i / (double)kHeadDim) / two_pi;
}

bool finite_positive(float x) { return isfinite(x) && x > 0.0f; }

}  // namespace

// 64-token chunks per segment for `work` (sequence, head, chunk) items, a multiple of sub.
static int64_t segment_chunks(int64_t work, int64_t sub) {
  const int64_t one_round = (work + kComputeUnits - 1) / kComputeUnits;
  const int64_t at_target = (work + kTargetWorkgroups - 1) / kTargetWorkgroups;
  const int64_t cps = std::max(at_target, std::min(one_round, kLongSegmentChunks));
  return std::max<int64_t>(sub, (cps + sub - 1) / sub * sub);
}

// Whether one workgroup per (b, h), walking the whole sequence, keeps the compute
// units busy: at least one full round, and the last round at least a quarter
// full of the rounds' capacity (bh >= 3/4 of the rounds' slots).  Then the
// segmented form's second read of k and v (in the state pass) buys nothing.
static bool heads_fill_device(int64_t bh) {
  const int64_t rounds = (bh + kComputeUnits - 1) / kComputeUnits;
  return bh >= kComputeUnits && 4 * bh >= 3 * kComputeUnits * rounds;
}

// Workspace of a direct plan: no segment states are kept; a minimum size keeps
// 0 meaning "invalid shape".
constexpr size_t kDirectWorkspaceBytes = 256;

static void set_direct(PrefillPlan* plan, int B) {
  const int64_t sub = plan->C / 64;
  plan->cps = (int)((plan->nchunks + sub - 1) / sub * sub);
  plan->nseg = 1;
  plan->nwork = B;
  plan->direct = true;
  plan->ws_bytes = kDirectWorkspaceBytes;
}

bool plan_prefill(int B, int T, int H, int chunk, PrefillPlan* plan, bool direct_ok) {
  if (B < 1 || T < 1 || H < 1) return false;
  const int C = chunk == 0 ? kDefaultChunk : chunk;
  if (C != 64 && C != 128 && C != 256) return false;
  // Work is counted in 64-token sub-chunks; a segment holds whole C-chunks.
  const int64_t sub = C / 64;
  const int64_t bh = (int64_t)B * H;
  if (bh > kMaxHeads) return false;  // before any product with it can overflow
  const int64_t nchunks = ((int64_t)T + 63) / 64;
  int64_t cps = segment_chunks(bh * nchunks, sub);
  if (cps > (nchunks + sub - 1) / sub * sub) cps = (nchunks + sub - 1) / sub * sub;
  const int64_t nseg = (nchunks + cps - 1) / cps;
  if (bh * nseg > kMaxWorkgroups) return false;
  plan->C = C;
  plan->nchunks = (int)nchunks;
  plan->cps = (int)cps;
  plan->nseg = (int)nseg;
  plan->nwork = (int64_t)B * nseg;
  plan->direct = false;
  plan->ws_bytes = (size_t)(bh * nseg) * kHeadDim * kHeadDim * sizeof(float);
  if (direct_ok && (nseg == 1 || heads_fill_device(bh))) set_direct(plan, B);
  return true;
}

// A plan whose workspace fits max_bytes: the planner's, or fewer and longer
// segments, or (when not even one segment state per (b, h) fits) the direct
// form, which keeps no states.
void cap_plan(int B, int H, size_t max_bytes, PrefillPlan* plan) {
  if (plan->ws_bytes <= max_bytes) return;
  const int64_t bh = (int64_t)B * H;
  const int64_t sub = plan->C / 64;
  const int64_t state = (int64_t)kHeadDim * kHeadDim * sizeof(float);
  const int64_t max_seg = (int64_t)(max_bytes / state) / bh;
  if (max_seg < 2) {
    set_direct(plan, B);
    return;
  }
  int64_t cps = (plan->nchunks + max_seg - 1) / max_seg;
  cps = (cps + sub - 1) / sub * sub;
  plan->cps = (int)cps;
  plan->nseg = (int)((plan->nchunks + cps - 1) / cps);
  plan->nwork = (int64_t)B * plan->nseg;
  plan->ws_bytes = (size_t)(bh * plan->nseg) * state;
  if (plan->nseg == 1) set_direct(plan, B);
}

// Host plan of a variable-length batch: the segment, sequence and single-token
// tables and where they and the segment states sit in the workspace.
struct VarlenPlan {
  PrefillPlan plan;
  std::vector<SegDesc> segs;
  std::vector<SeqDesc> seqs;
  std::vector<DecDesc> decs;
  size_t seq_off = 0, dec_off = 0, table_bytes = 0, state_off = 0;
};

static size_t round_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

la_status plan_varlen(int nseq, const int32_t* cu, const int64_t* pos0, int H, int chunk, VarlenPlan* vp) {
  if (nseq < 1 || H < 1 || cu == nullptr) return cu == nullptr ? LA_ERR_NULL_PTR : LA_ERR_BAD_SHAPE;
  if (nseq > (1 << 24) || (int64_t)nseq * H > kMaxHeads) return LA_ERR_BAD_SHAPE;
  const int C = chunk == 0 ? kDefaultChunk : chunk;
  if (C != 64 && C != 128 && C != 256) return LA_ERR_UNSUPPORTED;
  if (cu[0] != 0) return LA_ERR_BAD_SHAPE;
  int64_t sub_chunks = 0;
  for (int b = 0; b < nseq; ++b) {
    const int64_t len = (int64_t)cu[b + 1] - cu[b];
    if (len < 0) return LA_ERR_BAD_SHAPE;
    if (len >= 2) sub_chunks += (len + 63) / 64;
  }
  const int64_t sub = C / 64;
  const int64_t cps = segment_chunks((int64_t)H * sub_chunks, sub);
  vp->segs.clear();
  vp->seqs.assign(nseq, SeqDesc{0, 0, 0, 0});
  vp->decs.clear();
  bool scan = false;
  for (int b = 0; b < nseq; ++b) {
    const int32_t t0 = cu[b], t1 = cu[b + 1];
    const int64_t p0 = pos0 ? pos0[b] : 0;
    if (t1 - t0 == 1) {
      vp->seqs[b].decode = 1;
      vp->decs.push_back(DecDesc{b, t0, p0});
      continue;
    }
    scan = true;
    vp->seqs[b].first_seg = (int32_t)vp->segs.size();
    for (int64_t t = t0, s = 0; t < t1; t += cps * 64, ++s) {
      vp->segs.push_back(SegDesc{b, (int32_t)t, (int32_t)std::min<int64_t>(t1, t + cps * 64), (int32_t)s, p0 - t0});
      vp->seqs[b].nseg += 1;
    }
  }
  const int64_t nsegs = (int64_t)vp->segs.size();
  if (nsegs * H > kMaxWorkgroups || (int64_t)vp->decs.size() * H > ((int64_t)1 << 30)) return LA_ERR_BAD_SHAPE;
  vp->plan = PrefillPlan{};
  vp->plan.C = C;
  vp->plan.cps = (int)cps;
  vp->plan.nwork = nsegs;
  vp->plan.scan = scan;
  vp->seq_off = round_up(nsegs * sizeof(SegDesc), 16);
  vp->dec_off = round_up(vp->seq_off + nseq * sizeof(SeqDesc), 16);
  vp->table_bytes = vp->dec_off + vp->decs.size() * sizeof(DecDesc);
  vp->state_off = round_up(vp->table_bytes, 256);
  vp->plan.ws_bytes = vp->state_off + (size_t)nsegs * H * kHeadDim * kHeadDim * sizeof(float);
  return LA_OK;
}

}  // namespace la

// ---------------------------------------------------------------------------
// Scratch of la_prefill_noalloc: a static device array holding up to
// kScratchStates fp32 D x D segment states.  Every GPU the library runs on holds
// its own copy at its own address, for the life of the process.  In host code
// `scratch` names a host-side stand-in, never the device memory: the device
// address comes from hipGetSymbolAddress, taken once per device with that device
// current, and only that address is passed to kernels.
namespace la {
namespace {
constexpr int64_t kScratchStates = 1024;
constexpr size_t kScratchBytes = (size_t)kScratchStates * kHeadDim * kHeadDim * sizeof(float);  // 64 MiB
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
std::atomic<void*> g_scratch_ptr[kMaxDevices];
}  // namespace
}  // namespace la

static __device__ __align__(256) uint8_t scratch[la::kScratchBytes];

namespace la {
namespace {
// The device address of this device's scratch, for the device `stream` belongs
// to (the current device for the null stream).
la_status scratch_address(hipStream_t stream, void** out) {
  int dev = -1;
  if (stream != nullptr) {
    if (hipStreamGetDevice(stream, &dev) != hipSuccess) return LA_ERR_HIP;
  } else if (hipGetDevice(&dev) != hipSuccess) {
    return LA_ERR_HIP;
  }
  if (dev < 0 || dev >= kMaxDevices) return LA_ERR_HIP;
  void* p = g_scratch_ptr[dev].load(std::memory_order_acquire);
  if (p == nullptr) {
    std::lock_guard<std::mutex> lock(g_scratch_mutex);
    p = g_scratch_ptr[dev].load(std::memory_order_relaxed);
    if (p == nullptr) {
      int cur = -1;
      if (hipGetDevice(&cur) != hipSuccess) return LA_ERR_HIP;
      if (cur != dev && hipSetDevice(dev) != hipSuccess) return LA_ERR_HIP;
      const hipError_t err = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
      if (cur != dev && hipSetDevice(cur) != hipSuccess) return LA_ERR_HIP;
      if (err != hipSuccess || p == nullptr) return LA_ERR_HIP;
      g_scratch_ptr[dev].store(p, std::memory_order_release);
    }
  }
  *out = p;
  return LA_OK;
}
}  // namespace
}  // namespace la

using namespace la;

extern "C" {

int la_version(void) { return 200; }

const char* la_status_string(la_status s) {
  // Callers in other languages pass any integer; read it as one (an enum
  // variable holding a value outside its enumerators would be undefined in C++).
  int code;
  memcpy(&code, &s, sizeof code);
  switch (code) {
    case LA_OK: return "LA_OK";
    case LA_ERR_NULL_PTR: return "LA_ERR_NULL_PTR: a required pointer is NULL";
    case LA_ERR_BAD_SHAPE: return "LA_ERR_BAD_SHAPE: B, T and H must be >= 1 and the launch must fit";
    case LA_ERR_UNSUPPORTED: return "LA_ERR_UNSUPPORTED: need D == 128, chunk in {0, 64, 128, 256}, rope_base > 0 and finite, rms_eps >= 0 and finite";
    case LA_ERR_ALIGNMENT: return "LA_ERR_ALIGNMENT: pointers must be 16-byte aligned";
    case LA_ERR_ALIASING: return "LA_ERR_ALIASING: an output overlaps another argument";
    case LA_ERR_WORKSPACE: return "LA_ERR_WORKSPACE: workspace missing or too small";
    case LA_ERR_HIP: return "LA_ERR_HIP: kernel launch failed";
    case LA_ERR_CAPTURING: return "LA_ERR_CAPTURING: the stream is capturing a graph and this call copies host data";
  }
  return "unknown la_status";
}

size_t la_prefill_workspace_bytes(int B, int T, int H, int D, int chunk) {
  PrefillPlan plan;
  if (D != kHeadDim || !plan_prefill(B, T, H, chunk, &plan, true)) return 0;
  return plan.ws_bytes;
}

static la_status prefill_impl(const la_bf16* q, const la_bf16* k, const la_bf16* v,
                              const la_bf16* gate_logits, const float* S_in, float* S_out,
                              la_bf16* o, int B, int T, int H, int D, int64_t pos0, int chunk,
                              float rope_base, float rms_eps, const float* q_norm_w,
                              const float* k_norm_w, void* workspace, size_t workspace_bytes,
                              void* stream, hipEvent_t const* events,
                              const PrefillPlan* given_plan = nullptr, bool use_scratch = false) {
  // use_scratch: the segment states go to the library's static scratch, whose
  // address is taken only once the call has passed every check
  if (!q || !k || !v || !gate_logits || !S_out || !o || (!workspace && !use_scratch)) return LA_ERR_NULL_PTR;
  if (B < 1 || T < 1 || H < 1) return LA_ERR_BAD_SHAPE;
  if (D != kHeadDim || (chunk != 0 && chunk != 64 && chunk != 128 && chunk != 256)) return LA_ERR_UNSUPPORTED;
  if (!finite_positive(rope_base) || !isfinite(rms_eps) || rms_eps < 0.0f) return LA_ERR_UNSUPPORTED;
  PrefillPlan plan;
  if (given_plan != nullptr)
    plan = *given_plan;
  else if (!plan_prefill(B, T, H, chunk, &plan, true))
    return LA_ERR_BAD_SHAPE;
  const void* ptrs[] = {q, k, v, gate_logits, S_in, S_out, o, workspace, q_norm_w, k_norm_w};
  for (const void* ptr : ptrs)
    if (!aligned16(ptr)) return LA_ERR_ALIGNMENT;

  const uint64_t act = (uint64_t)B * T * H * D * sizeof(la_bf16);
  const uint64_t st = (uint64_t)B * H * D * D * sizeof(float);
  const void* ins[] = {q, k, v, gate_logits};
  for (const void* in : ins) {
    if (overlaps(o, act, in, act) || overlaps(S_out, st, in, act)) return LA_ERR_ALIASING;
  }
  if (overlaps(o, act, S_out, st) || overlaps(o, act, S_in, st)) return LA_ERR_ALIASING;
  if (S_in && S_in != S_out && overlaps(S_in, st, S_out, st)) return LA_ERR_ALIASING;
  const void* all[] = {q, k, v, gate_logits, S_in, S_out, o};
  for (const void* x : all)
    if (overlaps(workspace, plan.ws_bytes, x, x == S_in || x == S_out ? st : act)) return LA_ERR_ALIASING;
  if (workspace_bytes < plan.ws_bytes) return LA_ERR_WORKSPACE;
  if (use_scratch) {
    const la_status got = scratch_address(static_cast<hipStream_t>(stream), &workspace);
    if (got != LA_OK) return got;
  }

  PrefillParams p{};
  p.q = q;
  p.k = k;
  p.v = v;
  p.g = gate_logits;
  p.o = o;
  p.ws = static_cast<float*>(workspace);
  p.segs = nullptr;
  p.seqs = nullptr;
  p.S_in = S_in;
  p.S_out = S_out;
  p.qw = q_norm_w;
  p.kw = k_norm_w;
  p.B = B;
  p.T = T;
  p.H = H;
  p.nseg = plan.nseg;
  p.cps = plan.cps;
  p.pos0 = pos0;
  p.eps = rms_eps;
  rope_freqs(rope_base, &p.freqs);
  return launch_prefill(p, plan, static_cast<hipStream_t>(stream), events) == hipSuccess ? LA_OK
                                                                                     : LA_ERR_HIP;
}

la_status la_prefill(const la_bf16* q, const la_bf16* k, const la_bf16* v,
                     const la_bf16* gate_logits, const float* S_in, float* S_out, la_bf16* o,
                     int B, int T, int H, int D, int64_t pos0, int chunk, float rope_base,
                     float rms_eps, const float* q_norm_w, const float* k_norm_w,
                     void* workspace, size_t workspace_bytes, void* stream) {
  return prefill_impl(q, k, v, gate_logits, S_in, S_out, o, B, T, H, D, pos0, chunk, rope_base,
                      rms_eps, q_norm_w, k_norm_w, workspace, workspace_bytes, stream, nullptr);
}

la_status la_prefill_profiled(const la_bf16* q, const la_bf16* k, const la_bf16* v,
                              const la_bf16* gate_logits, const float* S_in, float* S_out,
                              la_bf16* o, int B, int T, int H, int D, int64_t pos0, int chunk,
                              float rope_base, float rms_eps, const float* q_norm_w,
                              const float* k_norm_w, void* workspace, size_t workspace_bytes,
                              void* stream, void* const* events, int n_events) {
  if (!events || n_events != 4) return LA_ERR_NULL_PTR;
  for (int i = 0; i < 4; ++i)
    if (!events[i]) return LA_ERR_NULL_PTR;
  return prefill_impl(q, k, v, gate_logits, S_in, S_out, o, B, T, H, D, pos0, chunk, rope_base,
                      rms_eps, q_norm_w, k_norm_w, workspace, workspace_bytes, stream,
                      reinterpret_cast<hipEvent_t const*>(events));
}

la_status la_prefill_noalloc(const la_bf16* q, const la_bf16* k, const la_bf16* v,
                             const la_bf16* gate_logits, const float* S_in, float* S_out, la_bf16* o,
                             int B, int T, int H, int D, int64_t pos0, int chunk, float rope_base,
                             float rms_eps, const float* q_norm_w, const float* k_norm_w, void* stream) {
  if (!q || !k || !v || !gate_logits || !S_out || !o) return LA_ERR_NULL_PTR;
  if (B < 1 || T < 1 || H < 1) return LA_ERR_BAD_SHAPE;
  if (D != kHeadDim || (chunk != 0 && chunk != 64 && chunk != 128 && chunk != 256)) return LA_ERR_UNSUPPORTED;
  PrefillPlan plan;
  if (!plan_prefill(B, T, H, chunk, &plan, true)) return LA_ERR_BAD_SHAPE;
  cap_plan(B, H, kScratchBytes, &plan);
  return prefill_impl(q, k, v, gate_logits, S_in, S_out, o, B, T, H, D, pos0, chunk, rope_base, rms_eps,
                      q_norm_w, k_norm_w, nullptr, kScratchBytes, stream, nullptr, &plan, true);
}

la_status la_decode_step(const la_bf16* q, const la_bf16* k, const la_bf16* v,
                         const la_bf16* gate_logits, float* S, la_bf16* o, int B, int H, int D,
                         int64_t pos, float rope_base, float rms_eps, const float* q_norm_w,
                         const float* k_norm_w, void* stream) {
  if (!q || !k || !v || !gate_logits || !S || !o) return LA_ERR_NULL_PTR;
  if (B < 1 || H < 1 || (int64_t)B * H > ((int64_t)1 << 30)) return LA_ERR_BAD_SHAPE;
  if (D != kHeadDim) return LA_ERR_UNSUPPORTED;
  if (!finite_positive(rope_base) || !isfinite(rms_eps) || rms_eps < 0.0f) return LA_ERR_UNSUPPORTED;
  const void* ptrs[] = {q, k, v, gate_logits, S, o, q_norm_w, k_norm_w};
  for (const void* ptr : ptrs)
    if (!aligned16(ptr)) return LA_ERR_ALIGNMENT;
  const uint64_t act = (uint64_t)B * H * D * sizeof(la_bf16);
  const uint64_t st = (uint64_t)B * H * D * D * sizeof(float);
  const void* ins[] = {q, k, v, gate_logits};
  for (const void* in : ins)
    if (overlaps(o, act, in, act) || overlaps(S, st, in, act)) return LA_ERR_ALIASING;
  if (overlaps(o, act, S, st)) return LA_ERR_ALIASING;

  DecodeParams p;
  p.q = q;
  p.k = k;
  p.v = v;
  p.g = gate_logits;
  p.o = o;
  p.S = S;
  p.S_in = nullptr;
  p.S_zero = false;
  p.rows = nullptr;
  p.qw = q_norm_w;
  p.kw = k_norm_w;
  p.B = B;
  p.H = H;
  p.pos = pos;
  p.eps = rms_eps;
  rope_freqs(rope_base, &p.freqs);
  return launch_decode(p, static_cast<hipStream_t>(stream)) == hipSuccess ? LA_OK : LA_ERR_HIP;
}

size_t la_prefill_varlen_workspace_bytes(int nseq, const int32_t* cu_seqlens, int H, int D, int chunk) {
  VarlenPlan vp;
  if (D != kHeadDim || plan_varlen(nseq, cu_seqlens, nullptr, H, chunk, &vp) != LA_OK) return 0;
  return vp.plan.ws_bytes;
}

la_status la_prefill_varlen(const la_bf16* q, const la_bf16* k, const la_bf16* v,
                            const la_bf16* gate_logits, const int32_t* cu_seqlens, const int64_t* pos0,
                            const float* S_in, float* S_out, la_bf16* o, int nseq, int total_T, int H,
                            int D, int chunk, float rope_base, float rms_eps, const float* q_norm_w,
                            const float* k_norm_w, void* workspace, size_t workspace_bytes, void* stream) {
  if (!S_out || !workspace || !cu_seqlens) return LA_ERR_NULL_PTR;
  if (total_T > 0 && (!q || !k || !v || !gate_logits || !o)) return LA_ERR_NULL_PTR;
  if (nseq < 1 || H < 1 || total_T < 0) return LA_ERR_BAD_SHAPE;
  if (D != kHeadDim || (chunk != 0 && chunk != 64 && chunk != 128 && chunk != 256)) return LA_ERR_UNSUPPORTED;
  if (!finite_positive(rope_base) || !isfinite(rms_eps) || rms_eps < 0.0f) return LA_ERR_UNSUPPORTED;
  VarlenPlan vp;
  const la_status planned = plan_varlen(nseq, cu_seqlens, pos0, H, chunk, &vp);
  if (planned != LA_OK) return planned;
  if (cu_seqlens[nseq] != total_T) return LA_ERR_BAD_SHAPE;
  const void* ptrs[] = {q, k, v, gate_logits, S_in, S_out, o, workspace, q_norm_w, k_norm_w};
  for (const void* ptr : ptrs)
    if (!aligned16(ptr)) return LA_ERR_ALIGNMENT;
  const uint64_t act = (uint64_t)total_T * H * D * sizeof(la_bf16);
  const uint64_t st = (uint64_t)nseq * H * D * D * sizeof(float);
  const void* ins[] = {q, k, v, gate_logits};
  for (const void* in : ins) {
    if (overlaps(o, act, in, act) || overlaps(S_out, st, in, act)) return LA_ERR_ALIASING;
  }
  if (overlaps(o, act, S_out, st) || overlaps(o, act, S_in, st)) return LA_ERR_ALIASING;
  if (S_in && S_in != S_out && overlaps(S_in, st, S_out, st)) return LA_ERR_ALIASING;
  const void* all[] = {q, k, v, gate_logits, S_in, S_out, o};
  for (const void* x : all)
    if (overlaps(workspace, vp.plan.ws_bytes, x, x == S_in || x == S_out ? st : act)) return LA_ERR_ALIASING;
  if (workspace_bytes < vp.plan.ws_bytes) return LA_ERR_WORKSPACE;

  // The table copy below reads host memory owned by this call; a graph captured
  // around it would replay the copy from freed memory, so a capturing stream is
  // refused before anything is enqueued.
  const hipStream_t s = static_cast<hipStream_t>(stream);
  hipStreamCaptureStatus capture = hipStreamCaptureStatusNone;
  if (hipStreamIsCapturing(s, &capture) != hipSuccess) return LA_ERR_HIP;
  if (capture != hipStreamCaptureStatusNone) return LA_ERR_CAPTURING;

  // the tables go to the front of the workspace, in stream order
  std::vector<uint8_t> tables(vp.table_bytes, 0);
  if (!vp.segs.empty()) memcpy(tables.data(), vp.segs.data(), vp.segs.size() * sizeof(SegDesc));
  memcpy(tables.data() + vp.seq_off, vp.seqs.data(), vp.seqs.size() * sizeof(SeqDesc));
  if (!vp.decs.empty()) memcpy(tables.data() + vp.dec_off, vp.decs.data(), vp.decs.size() * sizeof(DecDesc));
  uint8_t* ws = static_cast<uint8_t*>(workspace);
  if (hipMemcpyAsync(ws, tables.data(), tables.size(), hipMemcpyHostToDevice, s) != hipSuccess) return LA_ERR_HIP;

  RopeFreqs freqs;
  rope_freqs(rope_base, &freqs);
  if (vp.plan.scan || vp.plan.nwork > 0) {
    PrefillParams p{};
    p.q = q;
    p.k = k;
    p.v = v;
    p.g = gate_logits;
    p.o = o;
    p.ws = reinterpret_cast<float*>(ws + vp.state_off);
    p.segs = reinterpret_cast<const SegDesc*>(ws);
    p.seqs = reinterpret_cast<const SeqDesc*>(ws + vp.seq_off);
    p.S_in = S_in;
    p.S_out = S_out;
    p.qw = q_norm_w;
    p.kw = k_norm_w;
    p.B = nseq;
    p.T = total_T;
    p.H = H;
    p.nseg = 0;
    p.cps = vp.plan.cps;
    p.pos0 = 0;
    p.eps = rms_eps;
    p.freqs = freqs;
    if (launch_prefill(p, vp.plan, s) != hipSuccess) return LA_ERR_HIP;
  }
  if (!vp.decs.empty()) {
    DecodeParams d;
    d.q = q;
    d.k = k;
    d.v = v;
    d.g = gate_logits;
    d.o = o;
    d.S = S_out;
    d.S_in = S_in;
    d.S_zero = S_in == nullptr;
    d.rows = reinterpret_cast<const DecDesc*>(ws + vp.dec_off);
    d.qw = q_norm_w;
    d.kw = k_norm_w;
    d.B = (int)vp.decs.size();
    d.H = H;
    d.pos = 0;
    d.eps = rms_eps;
    d.freqs = freqs;
    if (launch_decode(d, s) != hipSuccess) return LA_ERR_HIP;
  }
  return LA_OK;
}

la_status la_linear(const la_bf16* x, const la_bf16* w, la_bf16* y, int64_t M, int N, int K, void* stream) {
  if (!x || !w || !y) return LA_ERR_NULL_PTR;
  if (M < 1 || N < 1 || K < 1 || M > ((int64_t)1 << 31)) return LA_ERR_BAD_SHAPE;
  if (K % 64 != 0 || N % 256 != 0) return LA_ERR_UNSUPPORTED;
  if (((M + 255) / 256) * (N / 256) >= ((int64_t)1 << 31)) return LA_ERR_BAD_SHAPE;
  const void* ptrs[] = {x, w, y};
  for (const void* ptr : ptrs)
    if (!aligned16(ptr)) return LA_ERR_ALIGNMENT;
  const uint64_t ybytes = (uint64_t)M * N * sizeof(la_bf16);
  if (overlaps(y, ybytes, x, (uint64_t)M * K * sizeof(la_bf16)) ||
      overlaps(y, ybytes, w, (uint64_t)N * K * sizeof(la_bf16)))
    return LA_ERR_ALIASING;
  LinearParams p{};
  p.x = x;
  p.w = w;
  p.y[0] = y;
  p.M = M;
  p.N = N;
  p.K = K;
  p.nsplit = 1;
  return launch_linear(p, static_cast<hipStream_t>(stream)) == hipSuccess ? LA_OK : LA_ERR_HIP;
}

size_t la_layer_workspace_bytes(int B, int T, int H, int D, int chunk) {
  PrefillPlan plan;
  if (D != kHeadDim || !plan_prefill(B, T, H, chunk, &plan, true)) return 0;
  const size_t act = (size_t)B * T * H * D * sizeof(la_bf16);
  return 5 * round_up(act, 256) + plan.ws_bytes;
}

la_status la_layer_forward(const la_bf16* x, const la_bf16* w_qkvg, const la_bf16* w_o, const float* S_in,
                           float* S_out, la_bf16* y, int B, int T, int hidden, int H, int D, int64_t pos0,
                           int chunk, float rope_base, float rms_eps, const float* q_norm_w,
                           const float* k_norm_w, void* workspace, size_t workspace_bytes, void* stream) {
  if (!x || !w_qkvg || !w_o || !S_out || !y || !workspace) return LA_ERR_NULL_PTR;
  if (B < 1 || T < 1 || H < 1 || hidden < 1) return LA_ERR_BAD_SHAPE;
  if (D != kHeadDim || (chunk != 0 && chunk != 64 && chunk != 128 && chunk != 256)) return LA_ERR_UNSUPPORTED;
  if (hidden % 256 != 0 || (H * D) % 256 != 0) return LA_ERR_UNSUPPORTED;
  if (!finite_positive(rope_base) || !isfinite(rms_eps) || rms_eps < 0.0f) return LA_ERR_UNSUPPORTED;
  PrefillPlan plan;
  if (!plan_prefill(B, T, H, chunk, &plan, true)) return LA_ERR_BAD_SHAPE;
  const void* ptrs[] = {x, w_qkvg, w_o, S_in, S_out, y, workspace, q_norm_w, k_norm_w};
  for (const void* ptr : ptrs)
    if (!aligned16(ptr)) return LA_ERR_ALIGNMENT;
  const int64_t M = (int64_t)B * T;
  const int HD = H * D;
  const uint64_t xbytes = (uint64_t)M * hidden * sizeof(la_bf16);
  const uint64_t st = (uint64_t)B * H * D * D * sizeof(float);
  const size_t act = round_up((size_t)M * HD * sizeof(la_bf16), 256);
  const size_t need = 5 * act + plan.ws_bytes;
  if (workspace_bytes < need) return LA_ERR_WORKSPACE;
  const std::pair<const void*, uint64_t> regions[] = {
      {x, xbytes}, {w_qkvg, (uint64_t)4 * HD * hidden * sizeof(la_bf16)},
      {w_o, (uint64_t)hidden * HD * sizeof(la_bf16)}, {S_in, st}, {S_out, st}, {y, xbytes}};
  for (const auto& r : regions)
    if (overlaps(workspace, need, r.first, r.second)) return LA_ERR_ALIASING;
  for (int i = 0; i < 5; ++i)  // every region but y's own (index 5), even one starting at y
    if (overlaps(y, xbytes, regions[i].first, regions[i].second)) return LA_ERR_ALIASING;
  for (const auto& r : {regions[0], regions[1], regions[2], regions[5]})
    if (overlaps(S_out, st, r.first, r.second)) return LA_ERR_ALIASING;
  if (S_in && S_in != S_out && overlaps(S_in, st, S_out, st)) return LA_ERR_ALIASING;

  uint8_t* ws = static_cast<uint8_t*>(workspace);
  la_bf16* qkvg[4];
  for (int i = 0; i < 4; ++i) qkvg[i] = reinterpret_cast<la_bf16*>(ws + i * act);
  la_bf16* o = reinterpret_cast<la_bf16*>(ws + 4 * act);
  const hipStream_t s = static_cast<hipStream_t>(stream);

  LinearParams in{};
  in.x = x;
  in.w = w_qkvg;
  for (int i = 0; i < 4; ++i) in.y[i] = qkvg[i];
  in.M = M;
  in.N = 4 * HD;
  in.K = hidden;
  in.nsplit = 4;
  if (launch_linear(in, s) != hipSuccess) return LA_ERR_HIP;
  const la_status st_pre = la_prefill(qkvg[0], qkvg[1], qkvg[2], qkvg[3], S_in, S_out, o, B, T, H, D, pos0, chunk,
                                      rope_base, rms_eps, q_norm_w, k_norm_w, ws + 5 * act, plan.ws_bytes, stream);
  if (st_pre != LA_OK) return st_pre;
  LinearParams out{};
  out.x = o;
  out.w = w_o;
  out.y[0] = y;
  out.M = M;
  out.N = hidden;
  out.K = HD;
  out.nsplit = 1;
  return launch_linear(out, s) == hipSuccess ? LA_OK : LA_ERR_HIP;
}

// Workspace of la_backward: forward and gradient segment states, the final
// forward state (unused), bf16 gradients of the rotated q and k, and the parts of
// the norm-weight gradients.
static bool backward_layout(int B, int T, int H, const PrefillPlan& plan, size_t off[6]) {
  const size_t st = (size_t)B * H * kHeadDim * kHeadDim * sizeof(float);
  const size_t rows = (size_t)B * T * H * kHeadDim * sizeof(la_bf16);
  off[0] = 0;                                   // forward segment states
  off[1] = round_up(off[0] + plan.ws_bytes, 256);  // gradient segment states
  off[2] = round_up(off[1] + plan.ws_bytes, 256);  // final forward state
  off[3] = round_up(off[2] + st, 256);             // dqh
  off[4] = round_up(off[3] + rows, 256);           // dkh
  off[5] = round_up(off[4] + rows, 256);           // weight-gradient parts
  return true;
}

size_t la_backward_workspace_bytes(int B, int T, int H, int D, int chunk) {
  PrefillPlan plan;
  if (D != kHeadDim || (chunk != 0 && chunk != 64) || !plan_prefill(B, T, H, chunk, &plan)) return 0;
  size_t off[6];
  backward_layout(B, T, H, plan, off);
  return off[5] + (size_t)2 * kPrologueBlocks * kHeadDim * sizeof(float);
}

// The backward, with the forward segment states recomputed (fwd_ws null) or read
// from the workspace of the forward call (fwd_ws, when that call kept them).
static la_status backward_impl(const la_bf16* q, const la_bf16* k, const la_bf16* v, const la_bf16* gate_logits,
                               const float* S_in, const la_bf16* d_o, const float* dS_out, la_bf16* dq,
                               la_bf16* dk, la_bf16* dv, la_bf16* dgate, float* dS_in, float* dq_norm_w,
                               float* dk_norm_w, int B, int T, int H, int D, int64_t pos0, int chunk,
                               float rope_base, float rms_eps, const float* q_norm_w, const float* k_norm_w,
                               void* workspace, size_t workspace_bytes, const void* fwd_ws, size_t fwd_ws_bytes,
                               void* stream) {
  if (!q || !k || !v || !gate_logits || !d_o || !dq || !dk || !dv || !dgate || !dS_in || !workspace)
    return LA_ERR_NULL_PTR;
  if (B < 1 || T < 1 || H < 1) return LA_ERR_BAD_SHAPE;
  if (D != kHeadDim || (chunk != 0 && chunk != 64)) return LA_ERR_UNSUPPORTED;
  if (!finite_positive(rope_base) || !isfinite(rms_eps) || rms_eps < 0.0f) return LA_ERR_UNSUPPORTED;
  PrefillPlan plan;
  if (!plan_prefill(B, T, H, chunk, &plan)) return LA_ERR_BAD_SHAPE;
  const size_t need = la_backward_workspace_bytes(B, T, H, D, chunk);
  const void* ptrs[] = {q, k, v, gate_logits, S_in, d_o, dS_out, dq, dk, dv, dgate, dS_in,
                        dq_norm_w, dk_norm_w, q_norm_w, k_norm_w, workspace, fwd_ws};
  for (const void* ptr : ptrs)
    if (!aligned16(ptr)) return LA_ERR_ALIGNMENT;
  // The forward kept its segment states when its own plan (la_prefill's) is not the
  // one-workgroup-per-(b, h) form; it is then this plan, so the layouts agree.
  const float* saved = nullptr;
  uint64_t saved_bytes = 0;
  if (fwd_ws) {
    PrefillPlan fplan;
    plan_prefill(B, T, H, chunk, &fplan, true);
    if (!fplan.direct) {
      if (fplan.nseg != plan.nseg || fplan.cps != plan.cps) return LA_ERR_UNSUPPORTED;
      if (fwd_ws_bytes < fplan.ws_bytes) return LA_ERR_WORKSPACE;
      saved = static_cast<const float*>(fwd_ws);
      saved_bytes = fplan.ws_bytes;
    }
  }
  const uint64_t act = (uint64_t)B * T * H * D * sizeof(la_bf16);
  const uint64_t st = (uint64_t)B * H * D * D * sizeof(float);
  const uint64_t wb = (uint64_t)D * sizeof(float);
  const std::pair<const void*, uint64_t> ins[] = {{q, act},      {k, act},          {v, act},
                                                  {gate_logits, act}, {d_o, act},    {S_in, st},
                                                  {dS_out, st},  {q_norm_w, wb},    {k_norm_w, wb},
                                                  {saved, saved_bytes}};
  const std::pair<const void*, uint64_t> outs[] = {{dq, act}, {dk, act}, {dv, act}, {dgate, act}, {dS_in, st},
                                                   {dq_norm_w, wb}, {dk_norm_w, wb}, {workspace, need}};
  for (size_t a = 0; a < sizeof(outs) / sizeof(outs[0]); ++a) {
    for (const auto& in : ins)
      if (overlaps(outs[a].first, outs[a].second, in.first, in.second)) return LA_ERR_ALIASING;
    for (size_t b = a + 1; b < sizeof(outs) / sizeof(outs[0]); ++b)
      if (overlaps(outs[a].first, outs[a].second, outs[b].first, outs[b].second)) return LA_ERR_ALIASING;
  }
  if (workspace_bytes < need) return LA_ERR_WORKSPACE;

  size_t off[6];
  backward_layout(B, T, H, plan, off);
  uint8_t* ws = static_cast<uint8_t*>(workspace);
  BackwardParams bp{};
  PrefillParams& p = bp.f;
  p.q = q;
  p.k = k;
  p.v = v;
  p.g = gate_logits;
  p.o = nullptr;
  // the kernels only read the forward states once they are formed
  p.ws = saved ? const_cast<float*>(saved) : reinterpret_cast<float*>(ws + off[0]);
  p.segs = nullptr;
  p.seqs = nullptr;
  p.S_in = S_in;
  p.S_out = reinterpret_cast<float*>(ws + off[2]);
  p.qw = q_norm_w;
  p.kw = k_norm_w;
  p.dout = d_o;
  p.B = B;
  p.T = T;
  p.H = H;
  p.nseg = plan.nseg;
  p.cps = plan.cps;
  p.pos0 = pos0;
  p.eps = rms_eps;
  rope_freqs(rope_base, &p.freqs);
  bp.wsg = reinterpret_cast<float*>(ws + off[1]);
  bp.dS_out = dS_out;
  bp.dS_in = dS_in;
  bp.dq = dq;
  bp.dk = dk;
  bp.dv = dv;
  bp.dg = dgate;
  bp.dqh = reinterpret_cast<la_bf16*>(ws + off[3]);
  bp.dkh = reinterpret_cast<la_bf16*>(ws + off[4]);
  bp.dq_w = dq_norm_w;
  bp.dk_w = dk_norm_w;
  bp.wpart = reinterpret_cast<float*>(ws + off[5]);
  const hipStream_t s = static_cast<hipStream_t>(stream);
  if (launch_segment_states(bp, plan, saved != nullptr, s) != hipSuccess) return LA_ERR_HIP;
  return launch_backward_chunks(bp, plan, s) == hipSuccess ? LA_OK : LA_ERR_HIP;
}

la_status la_backward(const la_bf16* q, const la_bf16* k, const la_bf16* v, const la_bf16* gate_logits,
                      const float* S_in, const la_bf16* d_o, const float* dS_out, la_bf16* dq, la_bf16* dk,
                      la_bf16* dv, la_bf16* dgate, float* dS_in, float* dq_norm_w, float* dk_norm_w, int B,
                      int T, int H, int D, int64_t pos0, int chunk, float rope_base, float rms_eps,
                      const float* q_norm_w, const float* k_norm_w, void* workspace, size_t workspace_bytes,
                      void* stream) {
  return backward_impl(q, k, v, gate_logits, S_in, d_o, dS_out, dq, dk, dv, dgate, dS_in, dq_norm_w, dk_norm_w, B,
                       T, H, D, pos0, chunk, rope_base, rms_eps, q_norm_w, k_norm_w, workspace, workspace_bytes,
                       nullptr, 0, stream);
}

la_status la_backward_saved(const la_bf16* q, const la_bf16* k, const la_bf16* v, const la_bf16* gate_logits,
                            const float* S_in, const la_bf16* d_o, const float* dS_out, la_bf16* dq, la_bf16* dk,
                            la_bf16* dv, la_bf16* dgate, float* dS_in, float* dq_norm_w, float* dk_norm_w, int B,
                            int T, int H, int D, int64_t pos0, int chunk, float rope_base, float rms_eps,
                            const float* q_norm_w, const float* k_norm_w, void* workspace, size_t workspace_bytes,
                            const void* fwd_workspace, size_t fwd_workspace_bytes, void* stream) {
  return backward_impl(q, k, v, gate_logits, S_in, d_o, dS_out, dq, dk, dv, dgate, dS_in, dq_norm_w, dk_norm_w, B,
                       T, H, D, pos0, chunk, rope_base, rms_eps, q_norm_w, k_norm_w, workspace, workspace_bytes,
                       fwd_workspace, fwd_workspace_bytes, stream);
}

static bool sparse_shape_ok(int B, int T, int H, int D, int block, int topk, la_status* st) {
  if (B < 1 || T < 1 || H < 1 || B > 65535 || H > 65535) {
    *st = LA_ERR_BAD_SHAPE;
    return false;
  }
  if (D != kHeadDim || (block != 0 && block != kSparseBlock) || topk < 1 || topk > kSparseMaxTopk ||
      T / kSparseBlock > kSparseMaxBlocks) {
    *st = LA_ERR_UNSUPPORTED;
    return false;
  }
  return true;
}

size_t la_sparse_prefill_workspace_bytes(int B, int T, int H, int D, int block, int topk) {
  la_status st;
  if (!sparse_shape_ok(B, T, H, D, block, topk, &st)) return 0;
  const size_t means = (size_t)B * H * (T / kSparseBlock) * D * sizeof(float);
  const size_t choice = (size_t)B * H * ((T + kSparseBlock - 1) / kSparseBlock) * topk * sizeof(int32_t);
  return round_up(means > 0 ? means : 1, 256) + round_up(choice, 256);
}

la_status la_sparse_prefill(const la_bf16* q, const la_bf16* k, const la_bf16* v, const la_bf16* gate_logits,
                            la_bf16* o, int32_t* sel, int B, int T, int H, int D, int block, int topk,
                            void* workspace, size_t workspace_bytes, void* stream) {
  if (!q || !k || !v || !gate_logits || !o || !workspace) return LA_ERR_NULL_PTR;
  la_status st;
  if (!sparse_shape_ok(B, T, H, D, block, topk, &st)) return st;
  const int64_t nqb = (T + kSparseBlock - 1) / kSparseBlock;
  if (nqb * H * B >= ((int64_t)1 << 31) - 8) return LA_ERR_BAD_SHAPE;  // work items, rounded up to 8 in int
  const void* ptrs[] = {q, k, v, gate_logits, o, sel, workspace};
  for (const void* ptr : ptrs)
    if (!aligned16(ptr)) return LA_ERR_ALIGNMENT;
  const size_t need = la_sparse_prefill_workspace_bytes(B, T, H, D, block, topk);
  if (workspace_bytes < need) return LA_ERR_WORKSPACE;
  const uint64_t act = (uint64_t)B * T * H * D * sizeof(la_bf16);
  const uint64_t selb = sel ? (uint64_t)B * H * nqb * topk * sizeof(int32_t) : 0;
  const void* ins[] = {q, k, v, gate_logits};
  for (const void* in : ins)
    if (overlaps(o, act, in, act) || overlaps(sel, selb, in, act) || overlaps(workspace, need, in, act))
      return LA_ERR_ALIASING;
  if (overlaps(o, act, sel, selb) || overlaps(o, act, workspace, need) || overlaps(sel, selb, workspace, need))
    return LA_ERR_ALIASING;
  SparseParams p{};
  p.q = q;
  p.k = k;
  p.v = v;
  p.g = gate_logits;
  p.o = o;
  p.kmean = static_cast<float*>(workspace);
  p.sel = nullptr;
  p.B = B;
  p.T = T;
  p.H = H;
  p.topk = topk;
  // the block choice goes to sel when given, else to the workspace after the means
  const size_t means = (size_t)B * H * (T / kSparseBlock) * D * sizeof(float);
  int32_t* choice = sel ? sel
                        : reinterpret_cast<int32_t*>(static_cast<uint8_t*>(workspace) +
                                                     round_up(means > 0 ? means : 1, 256));
  return launch_sparse_prefill(p, choice, static_cast<hipStream_t>(stream)) == hipSuccess ? LA_OK : LA_ERR_HIP;
}

la_status la_sparse_block_means(const la_bf16* k_cache, float* means, int B, int Tmax, int H, int D, int block,
                                int first_block, int nblocks, void* stream) {
  if (!k_cache || !means) return LA_ERR_NULL_PTR;
  la_status st;
  if (!sparse_shape_ok(B, Tmax, H, D, block, 1, &st)) return st;
  if (first_block < 0 || nblocks < 0 || (int64_t)first_block + nblocks > Tmax / kSparseBlock)
    return LA_ERR_BAD_SHAPE;
  if (!aligned16(k_cache) || !aligned16(means)) return LA_ERR_ALIGNMENT;
  const uint64_t cache = (uint64_t)B * Tmax * H * D * sizeof(la_bf16);
  if (overlaps(means, (uint64_t)B * H * (Tmax / kSparseBlock) * D * sizeof(float), k_cache, cache))
    return LA_ERR_ALIASING;
  SparseParams p{};
  p.k = k_cache;
  p.kmean = means;
  p.B = B;
  p.T = Tmax;
  p.H = H;
  p.topk = 1;
  return launch_sparse_means(p, first_block, nblocks, static_cast<hipStream_t>(stream)) == hipSuccess ? LA_OK
                                                                                                     : LA_ERR_HIP;
}

la_status la_sparse_decode(const la_bf16* q, const la_bf16* k_cache, const la_bf16* v_cache, const float* means,
                           const la_bf16* gate_logits, const int32_t* lens, la_bf16* o, int32_t* sel, int B,
                           int Tmax, int H, int D, int block, int topk, void* stream) {
  if (!q || !k_cache || !v_cache || !means || !gate_logits || !lens || !o) return LA_ERR_NULL_PTR;
  la_status st;
  if (!sparse_shape_ok(B, Tmax, H, D, block, topk, &st)) return st;
  if ((int64_t)B * H >= ((int64_t)1 << 31)) return LA_ERR_BAD_SHAPE;
  const void* ptrs[] = {q, k_cache, v_cache, means, gate_logits, o, sel};
  for (const void* ptr : ptrs)
    if (!aligned16(ptr)) return LA_ERR_ALIGNMENT;
  const uint64_t row = (uint64_t)B * H * D * sizeof(la_bf16);
  const uint64_t cache = (uint64_t)B * Tmax * H * D * sizeof(la_bf16);
  const uint64_t mb = (uint64_t)B * H * (Tmax / kSparseBlock) * D * sizeof(float);
  const uint64_t selb = sel ? (uint64_t)B * H * topk * sizeof(int32_t) : 0;
  const std::pair<const void*, uint64_t> ins[] = {{q, row}, {k_cache, cache}, {v_cache, cache},
                                                  {means, mb}, {gate_logits, row}, {lens, (uint64_t)B * 4}};
  for (const auto& in : ins)
    if (overlaps(o, row, in.first, in.second) || overlaps(sel, selb, in.first, in.second)) return LA_ERR_ALIASING;
  if (overlaps(o, row, sel, selb)) return LA_ERR_ALIASING;
  SparseParams p{};
  p.q = q;
  p.k = k_cache;
  p.v = v_cache;
  p.g = gate_logits;
  p.o = o;
  p.kmean = const_cast<float*>(means);
  p.sel = sel;
  p.lens = lens;
  p.B = B;
  p.T = Tmax;
  p.H = H;
  p.topk = topk;
  return launch_sparse_decode(p, static_cast<hipStream_t>(stream)) == hipSuccess ? LA_OK : LA_ERR_HIP;
}

}  // extern "C"
