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
  int nseg = 0;     // segments per (b, h) (equal-length batches)
  int64_t nwork = 0;  // segment workgroups per head: B * nseg, or the table's segments
  bool scan = true;   // launch the state scan
  bool direct = false;  // one segment per (b, h): the output kernel alone, S_in -> S_out
  size_t ws_bytes = 0;
};

// direct_ok: la_prefill's plan, which may use one segment per (b, h) with no
// state pass; otherwise the segmented form (state sums, scan, output) that the
// backward also uses.
bool plan_prefill(int B, int T, int H, int chunk, PrefillPlan* plan, bool direct_ok = false);

// Variable-length batches (packed [total_T, H, D] activations).  The host cuts
// every sequence of two or more tokens into segments and sends the tables below
// to the device in the workspace; single-token sequences take the decode kernel.
struct SegDesc {      // one segment: its workgroups are blockIdx = h + H * (index)
  int32_t seq;        // sequence
  int32_t t_begin;    // packed token range [t_begin, t_end)
  int32_t t_end;
  int32_t seg_local;  // segment number within the sequence
  int64_t pos_base;   // absolute position of packed token 0 for this sequence
};
struct SeqDesc {      // one sequence, for the state scan
  int32_t first_seg;  // index of its first segment
  int32_t nseg;       // 0 for an empty sequence (S_out = S_in)
  int32_t decode;     // 1: a single-token sequence handled by the decode kernel
  int32_t pad;
};
struct DecDesc {      // one single-token sequence
  int32_t seq;
  int32_t t;          // its packed token
  int64_t pos;        // absolute position
};

struct PrefillParams {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  const uint16_t* g;
  uint16_t* o;
  float* ws;          // fp32 segment states: [B][H][nseg][D][D], or [segment][H][D][D] with segs
  const SegDesc* segs;  // nullptr: B sequences of T tokens; else one entry per segment
  const SeqDesc* seqs;  // with segs: one entry per sequence
  const float* S_in;  // [B][H][D][D] or nullptr
  float* S_out;       // [B][H][D][D]
  const float* qw;    // [D] or nullptr
  const float* kw;    // [D] or nullptr
  const uint16_t* dout;  // backward only: gradient of o, [B][T][H][D]
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
  float* S;             // state written (and read when S_in is nullptr)
  const float* S_in;    // nullptr: update S in place
  bool S_zero;          // the state before the step is zero (S_in and S are not read)
  const DecDesc* rows;  // nullptr: B rows [B][H][D]; else B entries into packed [*, H, D] rows
  const float* qw;
  const float* kw;
  int B, H;
  int64_t pos;
  float eps;
  RopeFreqs freqs;
};

// y = x W^T, bf16 in and out, fp32 accumulation; y split by columns into nsplit
// tensors [M, N / nsplit].  K % 64 == 0, (N / nsplit) % 256 == 0.
struct LinearParams {
  const uint16_t* x;  // [M, K]
  const uint16_t* w;  // [N, K]
  uint16_t* y[4];
  int64_t M;
  int N, K, nsplit;
};

hipError_t launch_linear(const LinearParams& p, hipStream_t stream);

// events: nullptr, or 4 events recorded before each of the three kernels and after the last.
hipError_t launch_prefill(const PrefillParams& p, const PrefillPlan& plan, hipStream_t stream,
                          hipEvent_t const* events = nullptr);
hipError_t launch_decode(const DecodeParams& p, hipStream_t stream);

// Backward of la_prefill (chunk 64, equal-length batches).
struct BackwardParams {
  PrefillParams f;  // forward inputs; f.ws: forward segment states, f.dout: gradient of o
  float* wsg;       // gradient segment states, same layout as f.ws
  const float* dS_out;  // [B][H][D][D] or nullptr
  float* dS_in;         // [B][H][D][D]
  uint16_t* dq;
  uint16_t* dk;
  uint16_t* dv;
  uint16_t* dg;
  uint16_t* dqh;    // [B][T][H][D] bf16 scratch: gradients of the rotated, normalized q and k
  uint16_t* dkh;
  float* dq_w;      // [D] or nullptr (norm-weight gradients)
  float* dk_w;
  float* wpart;     // [2][kPrologueBlocks][D] fp32 scratch for the weight gradients
};
constexpr int kPrologueBlocks = 2048;

// The forward segment states of la_prefill into f.ws (f.S_out receives the final
// state), then the gradient segment states into wsg and dS_in.
// forward_saved: f.ws already holds the forward segment states (only the gradient
// states are formed)
hipError_t launch_segment_states(const BackwardParams& p, const PrefillPlan& plan, bool forward_saved,
                                 hipStream_t stream);
hipError_t launch_backward_chunks(const BackwardParams& p, const PrefillPlan& plan, hipStream_t stream);

// Sparse attention layer (block-selected causal softmax attention, NoPE, output
// gate).  Blocks of kSparseBlock tokens; a key block is scored by its mean key.
constexpr int kSparseBlock = 64;
constexpr int kSparseMaxTopk = 64;
constexpr int kSparseMaxBlocks = 8192;  // key blocks per sequence (512K tokens)

struct SparseParams {
  const uint16_t* q;   // prefill [B][T][H][D]; decode [B][H][D]
  const uint16_t* k;   // prefill [B][T][H][D]; decode: cache [B][T][H][D] (T = Tmax)
  const uint16_t* v;
  const uint16_t* g;   // shaped as q
  uint16_t* o;         // shaped as q
  float* kmean;        // [B][H][T / kSparseBlock][D] fp32 block means of k
  int32_t* sel;        // decode: [B][H][topk] output, or nullptr
  const int32_t* lens; // decode: valid tokens per sequence (the query is the last)
  int B, T, H, topk;
};

// Means of key blocks [first, first + nblocks) of every (b, h) of p.k into p.kmean.
hipError_t launch_sparse_means(const SparseParams& p, int first, int nblocks, hipStream_t stream);
// Key means, the block choice of every query block into sel ([B][H][nqb][topk]),
// then the attention.
hipError_t launch_sparse_prefill(const SparseParams& p, int32_t* sel, hipStream_t stream);
hipError_t launch_sparse_decode(const SparseParams& p, hipStream_t stream);

}  // namespace la
