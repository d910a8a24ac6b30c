// Chunked prefill of the gated causal linear-attention layer on gfx950.
//
// The state update S_t = S_{t-1} + k_t v_t^T ("MiniCPM-SALA: Hybridizing Sparse
// and Linear Attention for Efficient Long-Context Modeling", 前置知识 > 线性注意力)
// with readout o_t = sigmoid(g_t) * (qh_t S_t) is evaluated chunk by chunk.  For a
// chunk of C tokens with prefix state S_pre (the state before its first token):
//     O     = ((Qh Kh^T) masked to s <= t) V  +  Qh S_pre
//     S_pre <- S_pre + Kh^T V
// which is the recurrence regrouped (sum the update over the chunk).
//
// With one segment per (b, h) ("direct": the (b, h) alone fill the compute
// units) only the output kernel runs, starting from S_in and writing S_out from
// its carried state, so k and v are read once.  Otherwise three launches on the
// caller's stream:
//   1. la_chunk_state_kernel : one workgroup per (b, h, segment of cps chunks)
//      sums Kh^T V over its segment (bf16 MFMA, fp32 accumulate) -> workspace;
//      the last segment of each sequence has no later segment to feed and is
//      skipped.
//   2. la_state_scan_kernel  : per state element, exclusive prefix over segments
//      (plus S_in) in place.
//   3. la_chunk_output_kernel: one workgroup per (b, h, segment) starts from its
//      segment's prefix state and walks the chunks; the last segment of each
//      sequence writes its carried state to S_out.  Eight producer waves apply
//      QK-RMSNorm + RoPE to q, k and the sigmoid to the gate of chunk c+1 (bf16) and
//      stage the tiles into one half of a ping-pong LDS buffer (their global
//      loads run two chunks further ahead), while four consumer waves run all
//      the MFMA work of chunk c from the other half: the masked scores
//      P = Qh Kh^T into a shared LDS tile and O^T = S^T Qh^T, then
//      O^T += V^T P^T, the gate multiply, the bf16 store of o and S += Kh^T V.
//      Two barriers per chunk.
//
// MFMA layouts (v_mfma_f32_16x16x32_bf16; lane l = 16 g + n16 supplies
// A[n16][8g + e], B[8g + e][n16] and holds D[4g + r][n16]):
//   * a consumer wave owns value columns [32w, 32w + 32) of S; S stays in
//     accumulators, and an accumulator tile pair is the A operand of S^T Qh^T
//     directly when the key dims of the contraction are taken in the order
//     pi(8g + e) = 32kk + 4g + 16(e/4) + e%4, with Qh read in that order;
//   * the score tiles P^T (lane holds 4 consecutive keys of one query) pair up
//     into the B operand of V^T P^T with the same order over keys, so P never
//     goes through LDS;
//   * the token contractions take their "transposed" operands (V^T, Kh^T)
//     straight from the row-major tiles through ds_read_b64_tr_b16, so no tile
//     is ever written transposed.
#include "la_device.hpp"
#include "la_internal.hpp"
#include "la_tiles.hpp"

namespace la {
namespace {

// One segment per (b, h) of an equal-length batch: the output kernels start from
// S_in and write S_out themselves.
__device__ __forceinline__ bool is_direct(const PrefillParams& p) { return p.segs == nullptr && p.nseg == 1; }

// --------------------------------------------------------------------------
// Kh^T V summed over each segment.  LDS is double-buffered, so one barrier per
// chunk separates staging from use.  With kGrad, the same sum for the backward:
// Qh^T dU, the "keys" being the prologue of q and the "values" du = do * sigmoid(g).
template <bool kWeights, bool kGrad>
__global__ __launch_bounds__(kThreads) void la_chunk_state_kernel(PrefillParams p) {
  __shared__ __attribute__((aligned(16))) uint8_t sK[2][kTileBytes];
  __shared__ __attribute__((aligned(16))) uint8_t sV[2][kTileBytes];
  __shared__ float2 sRot[2][kHalf];

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int n16 = lane & 15, g4 = lane >> 4;
  const int j = tid & 15, rg = tid >> 4;
  const Tile tl = decode_tile(p);
  // forward: the last segment's sum feeds no prefix (its output workgroup carries
  // the state to S_out); the backward's gradient sums feed every segment
  if (!kGrad && last_segment(p, tl)) return;
  const int64_t rs = (int64_t)p.H * kD;
  const uint16_t* const kin = kGrad ? p.q : p.k;
  const uint16_t* const vin = kGrad ? p.dout : p.v;

  float wk[8];
  load_norm_weights(kGrad ? p.qw : p.kw, j, wk);
  Rope L;
  rope_init<32>(p, tid, rg, j, L);

  f32x4 Sacc[8];
#pragma unroll
  for (int a = 0; a < 8; ++a) Sacc[a] = f32x4{0.f, 0.f, 0.f, 0.f};

  Rows<2> Kr, Vr, Gr;
  auto load = [&](int t, int nv) {
    load_rows<2, 32>(kin + tl.base + (int64_t)t * rs, rs, nv, rg, j, Kr);
    load_rows<2, 32>(vin + tl.base + (int64_t)t * rs, rs, nv, rg, j, Vr);
    if (kGrad) load_rows<2, 32>(p.g + tl.base + (int64_t)t * rs, rs, nv, rg, j, Gr);
  };
  load(tl.t_begin, min(kC, tl.t_end - tl.t_begin));
  if (tid < kHalf) sRot[0][tid] = rope_rotation(tl.pos_base + tl.t_begin, L.base_rev);
  __syncthreads();

  for (int c = 0; c < tl.nch; ++c) {
    const int t0 = tl.t_begin + c * kC;
    const int nv = min(kC, tl.t_end - t0);
    // staging and the next chunk's load issue run at raised priority, the MFMA
    // accumulation at normal: a wave that is about to issue loads goes ahead of
    // another workgroup's wave that is accumulating (3-4% on this memory-bound kernel;
    // the opposite order was slower)
    __builtin_amdgcn_s_setprio(1);
    uint8_t* bK = sK[c & 1];
    uint8_t* bV = sV[c & 1];
    norm_rope_stage<kWeights, 2, 32>(Kr, wk, p.eps, sRot[c & 1], L, rg, j, bK);
    if (kGrad)
      du_stage<2, 32>(bV, nullptr, Vr, Gr, nv, rg, j);
    else
      store_rows_masked<2, 32>(bV, Vr, nv, rg, j);
    if (c + 1 < tl.nch) {
      const int t1 = t0 + kC;
      load(t1, min(kC, tl.t_end - t1));
      if (tid < kHalf) sRot[(c + 1) & 1][tid] = rope_rotation(tl.pos_base + t1, L.base_rev);
    }
    __syncthreads();
    __builtin_amdgcn_s_setprio(0);
    bf16x8 Vop[2];
    Vop[0] = v_operand(bV, 0, 16 * w, g4, n16);
    Vop[1] = v_operand(bV, 1, 16 * w, g4, n16);
    accumulate_state(Sacc, bK, Vop, g4, n16);
  }

  float* dst = tl.state;
#pragma unroll
  for (int rtk = 0; rtk < 8; ++rtk)
#pragma unroll
    for (int r = 0; r < 4; ++r) dst[state_elem(rtk, r, w, g4, n16)] = Sacc[rtk][r];
}

// --------------------------------------------------------------------------
// Exclusive prefix of the per-segment states, in place, seeded with S_in (the last
// segment's sum is not formed: its output workgroup writes S_out).  One thread per
// 4 consecutive elements.  A variable-length batch walks each sequence's own run
// of segments and skips single-token sequences; an empty sequence has none, and
// its final state S_in is written here.  kReverse (backward): the inclusive suffix
// seeded with dS_out (in S_in), so each segment gets the state gradient at its
// first token; the total goes to S_out.
template <bool kReverse>
__global__ __launch_bounds__(256) void la_state_scan_kernel(PrefillParams p) {
  constexpr int64_t per = kD * kD / 4;
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= (int64_t)p.B * p.H * per) return;
  const int64_t bh = idx / per, e = idx - bh * per;
  int nseg = p.nseg;
  float4* ws = reinterpret_cast<float4*>(p.ws) + bh * p.nseg * per + e;
  int64_t stride = per;
  if (p.seqs != nullptr) {
    const SeqDesc d = p.seqs[bh / p.H];
    if (d.decode) return;
    nseg = d.nseg;
    ws = reinterpret_cast<float4*>(p.ws) + ((int64_t)d.first_seg * p.H + bh % p.H) * per + e;
    stride = (int64_t)p.H * per;
  }
  float4 run = p.S_in ? reinterpret_cast<const float4*>(p.S_in)[idx] : make_float4(0.f, 0.f, 0.f, 0.f);
  for (int i = 0; i < nseg; ++i) {
    const int s = kReverse ? nseg - 1 - i : i;
    if (!kReverse && i == nseg - 1) {
      ws[s * stride] = run;
      break;
    }
    const float4 d = ws[s * stride];
    if (!kReverse) ws[s * stride] = run;
    run.x += d.x;
    run.y += d.y;
    run.z += d.z;
    run.w += d.w;
    if (kReverse) ws[s * stride] = run;
  }
  if (kReverse || nseg == 0) reinterpret_cast<float4*>(p.S_out)[idx] = run;
}

// --------------------------------------------------------------------------
// Output kernel.  Threads 0..255 are the consumer waves (wave w owns value
// columns [32w, 32w + 32)); threads 256..767 are the producer waves (thread
// (rg, j) stages rows rg and rg + 32).  Both roles run their own loop with the
// same number of barriers: two before the loop and two per chunk.
constexpr int kConsumers = 256;               // 4 consumer waves
constexpr int kProducers = 512;               // 8 producer waves
constexpr int kOutThreads = kConsumers + kProducers;

template <bool kWeights>
__device__ __forceinline__ void produce(const PrefillParams& p, const Tile& tl, uint8_t (*sQ)[kTileBytes],
                                        uint8_t (*sK)[kTileBytes], uint8_t (*sV)[kTileBytes],
                                        uint8_t (*sG)[kTileBytes], uint8_t* sQl, uint8_t* sKl,
                                        float2 (*sRot)[kHalf]) {
  // Producer waves issue ahead of the consumer wave on their SIMD, so that the next
  // chunk's loads go out as early as possible: 3-4% on this memory-bound kernel
  // (priority for the consumers' MFMAs instead gave under 1%).
  __builtin_amdgcn_s_setprio(1);
  const int ptid = threadIdx.x - kConsumers;
  const int j = ptid & 15, rg = ptid >> 4;
  const int64_t rs = (int64_t)p.H * kD;
  float wq[8], wk[8];
  load_norm_weights(p.qw, j, wq);
  load_norm_weights(p.kw, j, wk);
  Rope L;
  rope_init<32>(p, ptid, rg, j, L);
  struct Chunk {
    Rows<2> q, k, v, g;
  };
  Chunk X, Y;
  // chunk c's rows into R; with real false, the same loads of one row (row stride
  // 0: one cache line per load), whose values are never used
  auto load_chunk = [&](int c, Chunk& R, bool real) {
    const int t = tl.t_begin + c * kC;
    const int nv = real ? min(kC, tl.t_end - t) : 1;
    const int64_t off = tl.base + (int64_t)t * rs, rs_c = real ? rs : 0;
    load_rows<2, 32>(p.q + off, rs_c, nv, rg, j, R.q);
    load_rows<2, 32>(p.k + off, rs_c, nv, rg, j, R.k);
    load_rows<2, 32>(p.v + off, rs_c, nv, rg, j, R.v);
    load_rows<2, 32>(p.g + off, rs_c, nv, rg, j, R.g);
  };
  auto stage = [&](int c, const Chunk& R) {
    const int b = c & 1;
    const bool exact = tl.seg == 0 && c == 0;
    const int nv = min(kC, tl.t_end - (tl.t_begin + c * kC));
    norm_rope_stage_qk<kWeights, 2, 32>(R.q, R.k, wq, wk, p.eps, sRot[b], L, rg, j, sQ[b], sK[b],
                                        exact ? sQl : nullptr, exact ? sKl : nullptr);
    store_rows_masked<2, 32>(sV[b], R.v, nv, rg, j);
    sigmoid_stage<2, 32>(sG[b], R.g, rg, j);
  };
  // One step of the pipeline while the consumers work on chunk c: stage chunk
  // c + 1 from R, then reuse R for chunk c + 3 (chunk c + 2 is in flight in the
  // other register set).  Every step issues the same loads and staging, past the
  // segment's end too (one row of the last chunk per load, staged into the tile
  // half that the consumers no longer read): a load issued on some paths only made
  // the compiler wait for both register sets' loads before staging, which left one
  // chunk in flight instead of two.
  auto step = [&](int c, Chunk& R) {
    stage(c + 1, R);
    load_chunk(min(c + 3, tl.nch - 1), R, c + 3 < tl.nch);
    if (c + 2 < tl.nch && ptid < kHalf)
      sRot[c & 1][ptid] = rope_rotation(tl.pos_base + tl.t_begin + (c + 2) * kC, L.base_rev);
    __syncthreads();
    __syncthreads();
  };

  load_chunk(0, Y, true);
  if (ptid < kHalf) {
    sRot[0][ptid] = rope_rotation(tl.pos_base + tl.t_begin, L.base_rev);
    if (tl.nch > 1) sRot[1][ptid] = rope_rotation(tl.pos_base + tl.t_begin + kC, L.base_rev);
  }
  __syncthreads();
  stage(0, Y);
  load_chunk(min(1, tl.nch - 1), X, tl.nch > 1);
  load_chunk(min(2, tl.nch - 1), Y, tl.nch > 2);
  __syncthreads();
  int c = 0;
  for (; c + 1 < tl.nch; c += 2) {
    step(c, X);
    step(c + 1, Y);
  }
  if (c < tl.nch) step(c, X);
}

// Phase A of a consumer chunk: this wave's share of the masked scores P = Qh Kh^T
// (computed as P^T tiles, lane holding 4 consecutive keys of one query) into the
// score tile, and the inter-chunk term O^T = S_pre^T Qh^T for all 64 queries.
__device__ __forceinline__ void consume_phase_a(const uint8_t* Q, const uint8_t* K, const uint8_t* sQl,
                                                const uint8_t* sKl, uint8_t* sP, const f32x4 (&Sacc)[2][8],
                                                f32x4 (&Oacc)[2][4], bool exact, int w, int g4, int n16) {
  for (int idx = w; idx < 10; idx += 4) {
    const int rt = (kTileRT >> (2 * idx)) & 3, st = (kTileST >> (2 * idx)) & 3;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < kD / 32; ++ks) {
      const int ka = tile_off(16 * st + n16, 32 * ks + 8 * g4);
      const int qa = tile_off(16 * rt + n16, 32 * ks + 8 * g4);
      const bf16x8 kf = as_bf16x8(lds_ld<uint4>(K, ka));
      const bf16x8 qf = as_bf16x8(lds_ld<uint4>(Q, qa));
      if (exact && idx == 0) {  // tile (0, 0) of a call's first chunk: hi/lo cross terms
        acc = mma(as_bf16x8(lds_ld<uint4>(sKl, ka)), qf, acc);
        acc = mma(kf, as_bf16x8(lds_ld<uint4>(sQl, qa)), acc);
      }
      acc = mma(kf, qf, acc);
    }
    if (st == rt) {
#pragma unroll
      for (int r = 0; r < 4; ++r)
        if (4 * g4 + r > n16) acc[r] = 0.f;
    }
    lds_st<uint2>(sP, score_off(16 * rt + n16, 16 * st + 4 * g4),
                  make_uint2(pack2(acc[0], acc[1]), pack2(acc[2], acc[3])));
  }
  bf16x8 SA[2][4];  // S_pre^T as A operand (bf16), key dims in order pi
#pragma unroll
  for (int dt = 0; dt < 2; ++dt)
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) SA[dt][kk] = pack8(Sacc[dt][2 * kk], Sacc[dt][2 * kk + 1]);
#pragma unroll
  for (int rt = 0; rt < 4; ++rt) {
    bf16x8 Qf[4];
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) Qf[kk] = pi_operand(Q, 16 * rt + n16, kk, g4);
#pragma unroll
    for (int dt = 0; dt < 2; ++dt) {
      Oacc[dt][rt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) Oacc[dt][rt] = mma(SA[dt][kk], Qf[kk], Oacc[dt][rt]);
    }
  }
}

// Phase B: O^T += V^T P^T (scores read from the shared tile in key order pi),
// gate and store each row block, then S_pre += Kh^T V.
__device__ __forceinline__ void consume_phase_b(const uint8_t* K, const uint8_t* V, const uint8_t* G,
                                                const uint8_t* sP, f32x4 (&Sacc)[2][8], f32x4 (&Oacc)[2][4],
                                                int nv, uint16_t* orow, int64_t rs, int w, int g4, int n16) {
  bf16x8 Vf[2][2];  // V^T (token order pi), columns 32w + 16 dt + n16
#pragma unroll
  for (int dt = 0; dt < 2; ++dt)
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) Vf[dt][kk] = v_operand(V, kk, 32 * w + 16 * dt, g4, n16);
#pragma unroll
  for (int rt = 0; rt < 4; ++rt) {
    const int t = 16 * rt + n16;
#pragma unroll
    for (int kk = 0; kk <= rt / 2; ++kk) {
      const bf16x8 pb = as_bf16x8(lds_ld<uint2>(sP, score_off(t, 32 * kk + 4 * g4)),
                                  lds_ld<uint2>(sP, score_off(t, 32 * kk + 16 + 4 * g4)));
#pragma unroll
      for (int dt = 0; dt < 2; ++dt) Oacc[dt][rt] = mma(Vf[dt][kk], pb, Oacc[dt][rt]);
    }
    // gate and store: lane holds o[16 rt + n16][32 w + 16 dt + 4 g .. + 3]
    uint16_t* dst = orow + (int64_t)(16 * rt) * rs;
#pragma unroll
    for (int dt = 0; dt < 2; ++dt) {
      const uint2 sg = lds_ld<uint2>(G, tile_off(t, 32 * w + 16 * dt + 4 * g4));
      const uint2 out = make_uint2(pack2(Oacc[dt][rt][0] * bf2f_lo(sg.x), Oacc[dt][rt][1] * bf2f_hi(sg.x)),
                                   pack2(Oacc[dt][rt][2] * bf2f_lo(sg.y), Oacc[dt][rt][3] * bf2f_hi(sg.y)));
      if (t < nv) *reinterpret_cast<uint2*>(dst + 16 * dt) = out;
    }
  }
  // state carry S_pre += Kh^T V
#pragma unroll
  for (int kk = 0; kk < kC / 32; ++kk) {
    const int tr0 = 32 * kk + 4 * g4 + (n16 >> 2);
#pragma unroll
    for (int rtk = 0; rtk < 8; ++rtk) {
      const int col = 16 * rtk + 4 * (n16 & 3);
      const bf16x8 a = as_bf16x8(lds_tr(K, tile_off(tr0, col)), lds_tr(K, tile_off(tr0 + 16, col)));
#pragma unroll
      for (int dt = 0; dt < 2; ++dt) Sacc[dt][rtk] = mma(a, Vf[dt][kk], Sacc[dt][rtk]);
    }
  }
}

__device__ __forceinline__ void consume(const PrefillParams& p, const Tile& tl, uint8_t (*sQ)[kTileBytes],
                                        uint8_t (*sK)[kTileBytes], uint8_t (*sV)[kTileBytes],
                                        uint8_t (*sG)[kTileBytes], const uint8_t* sQl,
                                        const uint8_t* sKl, uint8_t* sP) {
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int n16 = lane & 15, g4 = lane >> 4;
  const int64_t rs = (int64_t)p.H * kD;

  // prefix state of this segment: S[:, 32w + 16 dt .. + 16) in accumulator tiles
  // (direct: S_in, or zero)
  const bool direct = is_direct(p);
  const int64_t bh = (int64_t)tl.b * p.H + tl.h;
  f32x4 Sacc[2][8];
  {
    const float* src = direct ? (p.S_in ? p.S_in + bh * kD * kD : nullptr) : tl.state;
#pragma unroll
    for (int dt = 0; dt < 2; ++dt)
#pragma unroll
      for (int rtk = 0; rtk < 8; ++rtk)
#pragma unroll
        for (int r = 0; r < 4; ++r) Sacc[dt][rtk][r] = src ? src[state_elem(rtk, r, 2 * w + dt, g4, n16)] : 0.0f;
  }
  // this lane's output pointer at chunk-relative row n16, column 32 w + 4 g
  uint16_t* const obase = p.o + tl.base + (int64_t)n16 * rs + 32 * w + 4 * g4;
  // score tiles above the diagonal are never written: zero the tile once
  for (int i = tid; i < kC * kScoreRowBytes / 16; i += kConsumers)
    reinterpret_cast<uint4*>(sP)[i] = make_uint4(0u, 0u, 0u, 0u);
  __syncthreads();
  __syncthreads();

  for (int c = 0; c < tl.nch; ++c) {
    const int b = c & 1;
    const uint8_t* Q = sQ[b];
    const uint8_t* K = sK[b];
    const uint8_t* V = sV[b];
    const uint8_t* G = sG[b];
    const int t0 = tl.t_begin + c * kC;
    const int nv = min(kC, tl.t_end - t0);
    // The first chunk of a call forms the scores of its first 16 rows from a
    // hi/lo split of qh and kh: those rows sum only a few scores, so the bf16
    // rounding of qh, kh would otherwise dominate their error.
    const bool exact = tl.seg == 0 && c == 0;
    f32x4 Oacc[2][4];
    consume_phase_a(Q, K, sQl, sKl, sP, Sacc, Oacc, exact, w, g4, n16);
    __syncthreads();
    consume_phase_b(K, V, G, sP, Sacc, Oacc, nv, obase + (int64_t)t0 * rs, rs, w, g4, n16);
    __syncthreads();
  }
  if (last_segment(p, tl)) {  // the sequence's final state (direct: its only segment)
    // lane offsets formed afresh here, so that none stays live across the loop
    int t2 = threadIdx.x;
    asm volatile("" : "+v"(t2));
    float* dst = p.S_out + ((int64_t)tl.b * p.H + tl.h) * kD * kD + (int64_t)(4 * ((t2 & 63) >> 4)) * kD +
                 32 * (t2 >> 6) + (t2 & 15);
#pragma unroll
    for (int dt = 0; dt < 2; ++dt)
#pragma unroll
      for (int rtk = 0; rtk < 8; ++rtk)
#pragma unroll
        for (int r = 0; r < 4; ++r) dst[(16 * rtk + r) * kD + 16 * dt] = Sacc[dt][rtk][r];
  }
}

template <bool kWeights>
__global__ __launch_bounds__(kOutThreads) void la_chunk_output_kernel(PrefillParams p) {
  __shared__ __attribute__((aligned(16))) uint8_t sQ[2][kTileBytes];
  __shared__ __attribute__((aligned(16))) uint8_t sK[2][kTileBytes];
  __shared__ __attribute__((aligned(16))) uint8_t sV[2][kTileBytes];
  __shared__ __attribute__((aligned(16))) uint8_t sG[2][kTileBytes];  // sigmoid(gate), bf16
  __shared__ __attribute__((aligned(16))) uint8_t sQl[kExactRows * kRowBytes];
  __shared__ __attribute__((aligned(16))) uint8_t sKl[kExactRows * kRowBytes];
  __shared__ __attribute__((aligned(16))) uint8_t sP[kC * kScoreRowBytes];
  __shared__ float2 sRot[2][kHalf];

  const Tile tl = decode_tile(p);
  if (threadIdx.x >= kConsumers)
    produce<kWeights>(p, tl, sQ, sK, sV, sG, sQl, sKl, sRot);
  else
    consume(p, tl, sQ, sK, sV, sG, sQl, sKl, sP);
}


// --------------------------------------------------------------------------
// Wide-chunk output kernel, C = 64 kSub (kSub = 2 or 4), in the producer/consumer
// form of the C = 64 kernel.  The chunked form with chunk C: query sub-block i
// (64 rows) of a chunk takes its scores against key sub-blocks jj <= i (causally
// masked at jj = i) and its inter-chunk term from the state at the chunk start;
// the chunk's Kh^T V joins the state after the chunk.  A segment's work is a
// sequence of units (i, jj), kSub (kSub + 1) / 2 per chunk in the order of
// WideSchedule (a segment's last chunk stops after the rows of its sub-blocks).
// Threads 0..255 are the consumer waves (wave w owns value columns [32w, 32w + 32)
// of S and o), threads 256..511 the producer waves (thread (rg, j) stages rows
// rg + 16m, m < 4).  While the consumers work on unit u, the producers stage unit
// u + 1 into the tiles the consumers are not reading: k and v of sub-block jj into
// the tile half the schedule names, unless that half already holds them, and q and
// the gate of sub-block i (at a row's first unit) by the parity of i.  Units u + 2
// and u + 3 load into registers meanwhile.  Two barriers per unit on both sides.
// The inter-chunk term of every sub-block of a chunk uses the chunk-start state,
// kept as bf16 operands while the fp32 state already takes the chunk's sub-blocks.
constexpr int kWideConsumers = 256;
constexpr int kWideThreads = kWideConsumers + 256;

// The units of one chunk in order, and the k/v tile half each one reads.  A row
// (query sub-block i) takes its units together; a unit whose key sub-block is
// already in a tile half reuses it, and a new one goes to the half the previous
// unit does not read.  Fields, unit e of the chunk at bits 2e (i, jj) or e:
// query sub-block, key sub-block, tile half, staged here, first unit of its row.
// kSub = 2: (0,0) (1,0) (1,1); halves 0 0 1, staged 1 0 1: two k/v stagings per
// chunk.  kSub = 4: (0,0) (1,0) (1,1) (2,0) (2,1) (2,2) (3,2) (3,1) (3,0) (3,3);
// halves 0 0 1 0 1 0 0 1 0 1, staged 1 0 1 0 0 1 0 0 1 1: five per chunk.  Every
// chunk's schedule ends in half 1 and starts in half 0, and each row ends with its
// diagonal unit.
template <int kSub>
struct WideSchedule;
template <>
struct WideSchedule<2> {
  static constexpr uint32_t kI = 0x14, kJ = 0x10, kHalfBuf = 0x4, kStage = 0x5, kFirst = 0x3;
};
template <>
struct WideSchedule<4> {
  static constexpr uint32_t kI = 0xffa94, kJ = 0xc6910, kHalfBuf = 0x294, kStage = 0x325, kFirst = 0x4b;
};

// Units of a segment of n tokens (the last chunk's rows stop at its sub-blocks).
template <int kSub>
__device__ __forceinline__ int wide_units(int n) {
  if (n <= 0) return 0;
  constexpr int kU = kSub * (kSub + 1) / 2;
  const int nchunk = (n + kSub * kC - 1) / (kSub * kC);
  const int last = (n - (nchunk - 1) * kSub * kC + kC - 1) / kC;  // sub-blocks of the last chunk
  return (nchunk - 1) * kU + last * (last + 1) / 2;
}

// Unit u of a segment: its sub-blocks' first tokens and its schedule fields.
template <int kSub>
struct WideUnit {
  int i, jj, ti, tj, buf;
  bool stage, first, chunk_start;
  __device__ __forceinline__ WideUnit(const Tile& tl, int u) {
    using Sch = WideSchedule<kSub>;
    constexpr int kU = kSub * (kSub + 1) / 2;
    const int c = u / kU, e = u - c * kU;
    i = (Sch::kI >> (2 * e)) & 3;
    jj = (Sch::kJ >> (2 * e)) & 3;
    buf = (Sch::kHalfBuf >> e) & 1;
    stage = (Sch::kStage >> e) & 1;
    first = (Sch::kFirst >> e) & 1;
    chunk_start = e == 0;
    const int t0 = tl.t_begin + c * kSub * kC;
    ti = t0 + i * kC;
    tj = t0 + jj * kC;
  }
};

template <bool kWeights, int kSub>
__device__ __forceinline__ void wide_produce(const PrefillParams& p, const Tile& tl, int nunit,
                                             uint8_t (*sQ)[kTileBytes], uint8_t (*sK)[kTileBytes],
                                             uint8_t (*sV)[kTileBytes], uint8_t (*sG)[kTileBytes], uint8_t* sQl,
                                             uint8_t* sKl) {
  __builtin_amdgcn_s_setprio(1);
  const int ptid = threadIdx.x - kWideConsumers;
  const int j = ptid & 15, rg = ptid >> 4;
  const int64_t rs = (int64_t)p.H * kD;
  float wq[8], wk[8];
  load_norm_weights(p.qw, j, wq);
  load_norm_weights(p.kw, j, wk);
  Rope L;
  rope_init<16>(p, ptid, rg, j, L);
  double rev[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) rev[e] = p.freqs.rev[4 * j + e];
  struct Set {
    Rows<4> q, k, v, g;
  };
  Set X, Y;
  auto load_unit = [&](int u, Set& R) {
    const WideUnit<kSub> U(tl, u);
    if (U.stage) {
      load_rows<4, 16>(p.k + tl.base + (int64_t)U.tj * rs, rs, min(kC, tl.t_end - U.tj), rg, j, R.k);
      load_rows<4, 16>(p.v + tl.base + (int64_t)U.tj * rs, rs, min(kC, tl.t_end - U.tj), rg, j, R.v);
    }
    if (U.first) {
      load_rows<4, 16>(p.q + tl.base + (int64_t)U.ti * rs, rs, min(kC, tl.t_end - U.ti), rg, j, R.q);
      load_rows<4, 16>(p.g + tl.base + (int64_t)U.ti * rs, rs, min(kC, tl.t_end - U.ti), rg, j, R.g);
    }
  };
  auto stage = [&](int u, const Set& R) {
    const WideUnit<kSub> U(tl, u);
    const bool exact = tl.seg == 0 && u == 0;  // the hi/lo rows: a call's first unit
    float2 E[4];
    if (U.stage) {
#pragma unroll
      for (int e = 0; e < 4; ++e) E[e] = cmul(rope_rotation(tl.pos_base + U.tj, rev[e]), L.A[e]);
      norm_rope_rows<kWeights, 4, 16>(R.k, wk, p.eps, E, L, rg, j, sK[U.buf], exact ? sKl : nullptr);
      store_rows_masked<4, 16>(sV[U.buf], R.v, min(kC, tl.t_end - U.tj), rg, j);
    }
    if (U.first) {
#pragma unroll
      for (int e = 0; e < 4; ++e) E[e] = cmul(rope_rotation(tl.pos_base + U.ti, rev[e]), L.A[e]);
      norm_rope_rows<kWeights, 4, 16>(R.q, wq, p.eps, E, L, rg, j, sQ[U.i & 1], exact ? sQl : nullptr);
      sigmoid_stage<4, 16>(sG[U.i & 1], R.g, rg, j);
    }
  };
  // one step while the consumers work on unit u: stage unit u + 1 from R, then reuse
  // R for unit u + 3 (unit u + 2 is in flight in the other register set)
  auto step = [&](int u, Set& R) {
    if (u + 1 < nunit) {
      stage(u + 1, R);
      if (u + 3 < nunit) load_unit(u + 3, R);
    }
    __syncthreads();
    __syncthreads();
  };
  if (nunit > 0) load_unit(0, Y);
  __syncthreads();
  if (nunit > 0) stage(0, Y);
  if (nunit > 1) load_unit(1, X);
  if (nunit > 2) load_unit(2, Y);
  __syncthreads();
  for (int u = 0; u < nunit; u += 2) {
    step(u, X);
    if (u + 1 < nunit) step(u + 1, Y);
  }
}

template <int kSub>
__device__ __forceinline__ void wide_consume(const PrefillParams& p, const Tile& tl, int nunit,
                                             uint8_t (*sQ)[kTileBytes], uint8_t (*sK)[kTileBytes],
                                             uint8_t (*sV)[kTileBytes], uint8_t (*sG)[kTileBytes],
                                             const uint8_t* sQl, const uint8_t* sKl, uint8_t* sP) {
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int n16 = lane & 15, g4 = lane >> 4;
  const int64_t rs = (int64_t)p.H * kD;

  // prefix state of this segment: S[:, 32w + 16 dt .. + 16) in accumulator tiles
  // (direct: S_in, or zero)
  const bool direct = is_direct(p);
  f32x4 Sacc[2][8];
  {
    const float* src =
        direct ? (p.S_in ? p.S_in + ((int64_t)tl.b * p.H + tl.h) * kD * kD : nullptr) : tl.state;
#pragma unroll
    for (int dt = 0; dt < 2; ++dt)
#pragma unroll
      for (int rtk = 0; rtk < 8; ++rtk)
#pragma unroll
        for (int r = 0; r < 4; ++r) Sacc[dt][rtk][r] = src ? src[state_elem(rtk, r, 2 * w + dt, g4, n16)] : 0.0f;
  }
  uint16_t* const obase = p.o + tl.base + (int64_t)n16 * rs + 32 * w + 4 * g4;
  // score tiles above the diagonal that a diagonal unit reads stay zero (off-diagonal
  // units overwrite them, and a diagonal unit zeroes them again)
  for (int i = tid; i < kC * kScoreRowBytes / 16; i += kWideConsumers)
    reinterpret_cast<uint4*>(sP)[i] = make_uint4(0u, 0u, 0u, 0u);
  __syncthreads();
  __syncthreads();

  bf16x8 SA[2][4];  // chunk-start state S^T as A operand (bf16), key dims in order pi
  f32x4 Oacc[2][4];
  for (int u = 0; u < nunit; ++u) {
    const WideUnit<kSub> U(tl, u);
    const uint8_t* Q = sQ[U.i & 1];
    const uint8_t* K = sK[U.buf];
    const uint8_t* V = sV[U.buf];
    const uint8_t* G = sG[U.i & 1];
    const bool diag = U.jj == U.i;
    const bool exact = tl.seg == 0 && u == 0;
    if (U.chunk_start) {
#pragma unroll
      for (int dt = 0; dt < 2; ++dt)
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) SA[dt][kk] = pack8(Sacc[dt][2 * kk], Sacc[dt][2 * kk + 1]);
    }
    // ---- phase A: scores P = Qh_i Kh_jj^T (as P^T tiles: lane holds 4 consecutive
    // keys of one query), causal at jj = i; the inter-chunk term at jj = 0
    if (diag) {
      for (int idx = w; idx < 10; idx += 4) {
        const int rt = (kTileRT >> (2 * idx)) & 3, st = (kTileST >> (2 * idx)) & 3;
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < kD / 32; ++ks) {
          const int ka = tile_off(16 * st + n16, 32 * ks + 8 * g4);
          const int qa = tile_off(16 * rt + n16, 32 * ks + 8 * g4);
          const bf16x8 kf = as_bf16x8(lds_ld<uint4>(K, ka));
          const bf16x8 qf = as_bf16x8(lds_ld<uint4>(Q, qa));
          if (exact && idx == 0) {
            acc = mma(as_bf16x8(lds_ld<uint4>(sKl, ka)), qf, acc);
            acc = mma(kf, as_bf16x8(lds_ld<uint4>(sQl, qa)), acc);
          }
          acc = mma(kf, qf, acc);
        }
        if (st == rt) {
#pragma unroll
          for (int r = 0; r < 4; ++r)
            if (4 * g4 + r > n16) acc[r] = 0.f;
        }
        lds_st<uint2>(sP, score_off(16 * rt + n16, 16 * st + 4 * g4),
                      make_uint2(pack2(acc[0], acc[1]), pack2(acc[2], acc[3])));
      }
      if (U.i > 0 && w < 2) {
        // the two tiles above the diagonal that the products below read: (0, 1), (2, 3)
        const int rt = 2 * w, st = rt + 1;
        lds_st<uint2>(sP, score_off(16 * rt + n16, 16 * st + 4 * g4), make_uint2(0u, 0u));
      }
    } else {
      for (int idx = w; idx < 16; idx += 4) {
        const int rt = idx >> 2, st = idx & 3;
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < kD / 32; ++ks) {
          const bf16x8 kf = as_bf16x8(lds_ld<uint4>(K, tile_off(16 * st + n16, 32 * ks + 8 * g4)));
          const bf16x8 qf = as_bf16x8(lds_ld<uint4>(Q, tile_off(16 * rt + n16, 32 * ks + 8 * g4)));
          acc = mma(kf, qf, acc);
        }
        lds_st<uint2>(sP, score_off(16 * rt + n16, 16 * st + 4 * g4),
                      make_uint2(pack2(acc[0], acc[1]), pack2(acc[2], acc[3])));
      }
    }
    if (U.first) {
      // O^T = S_start^T Qh_i^T for all 64 queries
#pragma unroll
      for (int rt = 0; rt < 4; ++rt) {
        bf16x8 Qf[4];
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) Qf[kk] = pi_operand(Q, 16 * rt + n16, kk, g4);
#pragma unroll
        for (int dt = 0; dt < 2; ++dt) {
          Oacc[dt][rt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int kk = 0; kk < 4; ++kk) Oacc[dt][rt] = mma(SA[dt][kk], Qf[kk], Oacc[dt][rt]);
        }
      }
    }
    __syncthreads();
    // ---- phase B: O^T += V_jj^T P^T (scores read in key order pi)
    bf16x8 Vf[2][2];  // V^T (token order pi), columns 32w + 16 dt + n16
#pragma unroll
    for (int dt = 0; dt < 2; ++dt)
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) Vf[dt][kk] = v_operand(V, kk, 32 * w + 16 * dt, g4, n16);
#pragma unroll
    for (int rt = 0; rt < 4; ++rt) {
      const int t = 16 * rt + n16;
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        if (diag && kk > rt / 2) continue;
        const bf16x8 pb = as_bf16x8(lds_ld<uint2>(sP, score_off(t, 32 * kk + 4 * g4)),
                                    lds_ld<uint2>(sP, score_off(t, 32 * kk + 16 + 4 * g4)));
#pragma unroll
        for (int dt = 0; dt < 2; ++dt) Oacc[dt][rt] = mma(Vf[dt][kk], pb, Oacc[dt][rt]);
      }
    }
    if (diag) {
      // gate and store sub-block i: lane holds o[ti + 16 rt + n16][32 w + 16 dt + 4 g .. + 3]
      const int nv = min(kC, tl.t_end - U.ti);
      uint16_t* const orow = obase + (int64_t)U.ti * rs;
#pragma unroll
      for (int rt = 0; rt < 4; ++rt) {
        const int t = 16 * rt + n16;
        uint16_t* dst = orow + (int64_t)(16 * rt) * rs;
#pragma unroll
        for (int dt = 0; dt < 2; ++dt) {
          const uint2 sg = lds_ld<uint2>(G, tile_off(t, 32 * w + 16 * dt + 4 * g4));
          const uint2 out = make_uint2(pack2(Oacc[dt][rt][0] * bf2f_lo(sg.x), Oacc[dt][rt][1] * bf2f_hi(sg.x)),
                                       pack2(Oacc[dt][rt][2] * bf2f_lo(sg.y), Oacc[dt][rt][3] * bf2f_hi(sg.y)));
          if (t < nv) *reinterpret_cast<uint2*>(dst + 16 * dt) = out;
        }
      }
      // S += Kh_i^T V_i
#pragma unroll
      for (int kk = 0; kk < kC / 32; ++kk) {
        const int tr0 = 32 * kk + 4 * g4 + (n16 >> 2);
#pragma unroll
        for (int rtk = 0; rtk < 8; ++rtk) {
          const int col = 16 * rtk + 4 * (n16 & 3);
          const bf16x8 a = as_bf16x8(lds_tr(K, tile_off(tr0, col)), lds_tr(K, tile_off(tr0 + 16, col)));
#pragma unroll
          for (int dt = 0; dt < 2; ++dt) Sacc[dt][rtk] = mma(a, Vf[dt][kk], Sacc[dt][rtk]);
        }
      }
    }
    __syncthreads();
  }
  if (last_segment(p, tl)) {  // the sequence's final state (direct: its only segment)
    // lane offsets formed afresh here, so that none stays live across the loop
    int t2 = threadIdx.x;
    asm volatile("" : "+v"(t2));
    float* dst = p.S_out + ((int64_t)tl.b * p.H + tl.h) * kD * kD + (int64_t)(4 * ((t2 & 63) >> 4)) * kD +
                 32 * (t2 >> 6) + (t2 & 15);
#pragma unroll
    for (int dt = 0; dt < 2; ++dt)
#pragma unroll
      for (int rtk = 0; rtk < 8; ++rtk)
#pragma unroll
        for (int r = 0; r < 4; ++r) dst[(16 * rtk + r) * kD + 16 * dt] = Sacc[dt][rtk][r];
  }
}

template <bool kWeights, int kSub>
__global__ __launch_bounds__(kWideThreads) void la_chunk_output_wide_kernel(PrefillParams p) {
  __shared__ __attribute__((aligned(16))) uint8_t sQ[2][kTileBytes];
  __shared__ __attribute__((aligned(16))) uint8_t sK[2][kTileBytes];
  __shared__ __attribute__((aligned(16))) uint8_t sV[2][kTileBytes];
  __shared__ __attribute__((aligned(16))) uint8_t sG[2][kTileBytes];  // sigmoid(gate), bf16
  __shared__ __attribute__((aligned(16))) uint8_t sQl[kExactRows * kRowBytes];
  __shared__ __attribute__((aligned(16))) uint8_t sKl[kExactRows * kRowBytes];
  __shared__ __attribute__((aligned(16))) uint8_t sP[kC * kScoreRowBytes];

  const Tile tl = decode_tile(p);
  const int nunit = wide_units<kSub>(tl.t_end - tl.t_begin);
  if (threadIdx.x >= kWideConsumers)
    wide_produce<kWeights, kSub>(p, tl, nunit, sQ, sK, sV, sG, sQl, sKl);
  else
    wide_consume<kSub>(p, tl, nunit, sQ, sK, sV, sG, sQl, sKl, sP);
}

}  // namespace

hipError_t launch_prefill(const PrefillParams& p, const PrefillPlan& plan, hipStream_t stream,
                          hipEvent_t const* events) {
  const dim3 grid((unsigned)(plan.nwork * p.H));
  const int64_t scan_threads = (int64_t)p.B * p.H * kD * kD / 4;
  const bool weights = p.qw != nullptr || p.kw != nullptr;
  hipError_t err = hipSuccess;
  auto mark = [&](int i) {
    if (events && err == hipSuccess) err = hipEventRecord(events[i], stream);
  };
  mark(0);
  if (plan.nwork > 0 && !plan.direct) {
    if (weights)
      hipLaunchKernelGGL((la_chunk_state_kernel<true, false>), grid, dim3(kThreads), 0, stream, p);
    else
      hipLaunchKernelGGL((la_chunk_state_kernel<false, false>), grid, dim3(kThreads), 0, stream, p);
  }
  mark(1);
  if (plan.scan && !plan.direct)
    hipLaunchKernelGGL(la_state_scan_kernel<false>, dim3((unsigned)((scan_threads + 255) / 256)), dim3(256), 0,
                       stream, p);
  mark(2);
  if (plan.nwork > 0 && plan.C == kC) {
    if (weights)
      hipLaunchKernelGGL(la_chunk_output_kernel<true>, grid, dim3(kOutThreads), 0, stream, p);
    else
      hipLaunchKernelGGL(la_chunk_output_kernel<false>, grid, dim3(kOutThreads), 0, stream, p);
  } else if (plan.nwork > 0 && plan.C == 2 * kC) {
    if (weights)
      hipLaunchKernelGGL((la_chunk_output_wide_kernel<true, 2>), grid, dim3(kWideThreads), 0, stream, p);
    else
      hipLaunchKernelGGL((la_chunk_output_wide_kernel<false, 2>), grid, dim3(kWideThreads), 0, stream, p);
  } else if (plan.nwork > 0) {
    if (weights)
      hipLaunchKernelGGL((la_chunk_output_wide_kernel<true, 4>), grid, dim3(kWideThreads), 0, stream, p);
    else
      hipLaunchKernelGGL((la_chunk_output_wide_kernel<false, 4>), grid, dim3(kWideThreads), 0, stream, p);
  }
  mark(3);
  const hipError_t launch = hipGetLastError();
  return err != hipSuccess ? err : launch;
}

hipError_t launch_segment_states(const BackwardParams& bp, const PrefillPlan& plan, bool forward_saved,
                                 hipStream_t stream) {
  const dim3 grid((unsigned)(plan.nwork * bp.f.H));
  const dim3 scan_grid((unsigned)(((int64_t)bp.f.B * bp.f.H * kD * kD / 4 + 255) / 256));
  PrefillParams f = bp.f;  // forward states into f.ws, final state into f.S_out
  if (!forward_saved) {
    if (f.kw)
      hipLaunchKernelGGL((la_chunk_state_kernel<true, false>), grid, dim3(kThreads), 0, stream, f);
    else
      hipLaunchKernelGGL((la_chunk_state_kernel<false, false>), grid, dim3(kThreads), 0, stream, f);
    hipLaunchKernelGGL(la_state_scan_kernel<false>, scan_grid, dim3(256), 0, stream, f);
  }
  PrefillParams g = bp.f;  // gradient states: sums of Qh^T dU, suffix-scanned from dS_out
  g.ws = bp.wsg;
  g.S_in = bp.dS_out;
  g.S_out = bp.dS_in;
  if (g.qw)
    hipLaunchKernelGGL((la_chunk_state_kernel<true, true>), grid, dim3(kThreads), 0, stream, g);
  else
    hipLaunchKernelGGL((la_chunk_state_kernel<false, true>), grid, dim3(kThreads), 0, stream, g);
  hipLaunchKernelGGL(la_state_scan_kernel<true>, scan_grid, dim3(256), 0, stream, g);
  return hipGetLastError();
}

}  // namespace la
