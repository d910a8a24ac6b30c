// Host-side plan and launcher declarations shared by the C-ABI layer and the
// kernel translation units.  Not part of the public interface.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace la {

constexpr int kHeadDim = 128;
constexpr int kFreqs = 64;

// RoPE frequencies in revolutions per position, rev_i = base^(-2i/D) / (2 pi),
// computed on the host in double.
struct RopeFreqs {
  double rev[kFreqs];
};

// How one prefill call is cut up: T tokens -> sub-chunks of 64 tokens ->
// segments of `cps` consecutive sub-chunks (a multiple of C / 64, so a segment
// holds whole chunks of C tokens).  One workgroup walks one (b, h, segment).
struct PrefillPlan {
  int C = 0;        // chunk length: 64, 128 or 256
  int nchunks = 0;  // ceil(T / 64)
  int cps = 0;      // 64-token sub-chunks per segment
  int nseg = 0;     // segments per (b, h)
  size_t ws_bytes = 0;
};

bool plan_prefill(int B, int T, int H, int chunk, PrefillPlan* plan);

struct PrefillParams {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  const uint16_t* g;
  uint16_t* o;
  float* ws;          // [B][H][nseg][D][D] fp32 segment states
  const float* S_in;  // [B][H][D][D] or nullptr
  float* S_out;       // [B][H][D][D]
  const float* qw;    // [D] or nullptr
  const float* kw;    // [D] or nullptr
  int B, T, H, nseg, cps;
  int64_t pos0;
  float eps;
  RopeFreqs freqs;
};

struct DecodeParams {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  const uint16_t* g;
  uint16_t* o;
  float* S;
  const float* qw;
  const float* kw;
  int B, H;
  int64_t pos;
  float eps;
  RopeFreqs freqs;
};

// events: nullptr, or 4 events recorded before each of the three kernels and after the last.
hipError_t launch_prefill(const PrefillParams& p, const PrefillPlan& plan, hipStream_t stream,
                          hipEvent_t const* events = nullptr);
hipError_t launch_decode(const DecodeParams& p, hipStream_t stream);

}  // namespace la
