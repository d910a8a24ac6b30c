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
// Three launches on the caller's stream:
//   1. la_chunk_state_kernel : one workgroup per (b, h, segment of cps chunks)
//      sums Kh^T V over its segment (bf16 MFMA, fp32 accumulate) -> workspace.
//   2. la_state_scan_kernel  : per state element, exclusive prefix over segments
//      (plus S_in) in place, and the final state -> S_out.
//   3. la_chunk_output_kernel: one workgroup per (b, h, segment) starts from its
//      segment's prefix state and walks the chunks.  Eight producer waves apply
//      QK-RMSNorm + RoPE to q, k and the sigmoid to the gate of chunk c+1 and
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

namespace la {
namespace {

constexpr int kC = 64;      // tokens per chunk
constexpr int kWaves = 8;
constexpr int kThreads = 64 * kWaves;
constexpr int kRowBytes = kD * 2 + 16;     // 128 bf16 + 16 bytes of padding
constexpr int kTileBytes = kC * kRowBytes;  // one [64][128] bf16 tile
constexpr int kExactRows = 16;              // rows whose scores use the hi/lo split

typedef short bf16x4 __attribute__((ext_vector_type(4)));

// [64][128] bf16 row tile with 272-byte rows: consecutive rows start 16 bytes
// apart in the bank space, so the 8-byte operand reads (16 rows x 4 lane
// groups), the transposed reads (4 rows x 4 groups) and the staging writes all
// spread over the banks, and every offset is linear (immediate offsets).
__device__ __forceinline__ int tile_off(int t, int d) { return t * kRowBytes + 2 * d; }

// Transposed read: within each 16-lane group, lane L supplies the address of 4
// bf16 and receives element L of each of the 4 rows formed by lanes 4r..4r+3.
// Reading rows t0 + L / 4, columns c0 + 4 (L % 4) of a row tile gives lane L the
// column c0 + L at rows t0 .. t0 + 3.
__device__ __forceinline__ uint2 lds_tr(const uint8_t* base, int off) {
  typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;
  const bf16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_bf16x4*)(base + off));
  return __builtin_bit_cast(uint2, v);
}

// Sum over the 16 lanes of a DPP row (quad swaps, then rotations by 4 and 8).
__device__ __forceinline__ float row16_sum(float x) {
  x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0xB1, 0xF, 0xF, false));
  x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x4E, 0xF, 0xF, false));
  x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x124, 0xF, 0xF, false));
  x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x128, 0xF, 0xF, false));
  return x;
}

// Staging coordinates: a thread (rg, j) holds rows rg + kStep m (m < M) of a
// chunk and dims {4j..4j+3} U {64+4j..64+4j+3}: each RoPE pair (i, i + 64) sits
// in one thread, and 16 consecutive lanes cover a row.
template <int M>
struct Rows {
  uint2 lo[M];  // dims 4j..4j+3, four bf16
  uint2 hi[M];  // dims 64+4j..64+4j+3
};

// Unmasked, branch-free loads: rows at or beyond nvalid (>= 1) re-read the last
// valid row, keeping every address inside the tensor.  Such rows of q, k and the
// gate only reach masked scores and unstored outputs; v's are zeroed when staged.
template <int M, int kStep>
__device__ __forceinline__ void load_rows(const uint16_t* __restrict__ base, int64_t rs, int nvalid,
                                          int rg, int j, Rows<M>& R) {
#pragma unroll
  for (int m = 0; m < M; ++m) {
    const uint16_t* src = base + (int64_t)min(rg + kStep * m, nvalid - 1) * rs;
    R.lo[m] = ld_stream(src + 4 * j);
    R.hi[m] = ld_stream(src + kHalf + 4 * j);
  }
}

template <int M, int kStep>
__device__ __forceinline__ void store_rows_masked(uint8_t* tile, const Rows<M>& R, int nvalid, int rg,
                                                  int j) {
#pragma unroll
  for (int m = 0; m < M; ++m) {
    const bool ok = rg + kStep * m < nvalid;
    lds_st<uint2>(tile, tile_off(rg + kStep * m, 4 * j), ok ? R.lo[m] : make_uint2(0u, 0u));
    lds_st<uint2>(tile, tile_off(rg + kStep * m, kHalf + 4 * j), ok ? R.hi[m] : make_uint2(0u, 0u));
  }
}

// sigmoid of the gate logits, staged as f16 (the value lies in (0, 1); f16 keeps
// 11 significant bits, round toward zero).
template <int M, int kStep>
__device__ __forceinline__ void sigmoid_stage(uint8_t* tile, const Rows<M>& R, int rg, int j) {
#pragma unroll
  for (int m = 0; m < M; ++m) {
    const uint2 a = R.lo[m], b = R.hi[m];
    const uint2 lo = make_uint2(pack_f16x2(sigmoidf_(bf2f_lo(a.x)), sigmoidf_(bf2f_hi(a.x))),
                                pack_f16x2(sigmoidf_(bf2f_lo(a.y)), sigmoidf_(bf2f_hi(a.y))));
    const uint2 hi = make_uint2(pack_f16x2(sigmoidf_(bf2f_lo(b.x)), sigmoidf_(bf2f_hi(b.x))),
                                pack_f16x2(sigmoidf_(bf2f_lo(b.y)), sigmoidf_(bf2f_hi(b.y))));
    lds_st<uint2>(tile, tile_off(rg + kStep * m, 4 * j), lo);
    lds_st<uint2>(tile, tile_off(rg + kStep * m, kHalf + 4 * j), hi);
  }
}

// RoPE per thread: A[e] = e^{i rg theta}, Z[e] = e^{i kStep theta} for the
// thread's frequencies 4j+e; row rg + kStep m of a chunk at position p0 is
// rotated by base(p0) * A * Z^m.  base_rev is the frequency of pair i = tid % 64,
// for the per-chunk base rotation, kept in a register so the loop loads nothing.
struct Rope {
  float2 A[4];
  float2 Z[4];
  double base_rev;
};

template <int kStep>
__device__ __forceinline__ void rope_init(const PrefillParams& p, int tid, int rg, int j, Rope& L) {
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const double rv = p.freqs.rev[4 * j + e];
    L.A[e] = rope_rotation(rg, rv);
    L.Z[e] = rope_rotation(kStep, rv);
  }
  L.base_rev = p.freqs.rev[tid & (kHalf - 1)];
}

// QK-normalization (RMSNorm over the 128 dims of row t, weights w) followed by
// rotate-half RoPE with rotations E, in fp32; the bf16 result goes to `tile`.
// With `lo` set, rows below kExactRows also store lo = bf16(y - bf16(y)) into
// `lo`, for the scores of the first rows of a call.
template <bool kWeights>
__device__ __forceinline__ void norm_rope_row(uint2 rl, uint2 rh, const float (&w)[8], float eps,
                                              const float2 (&E)[4], int t, int j, uint8_t* tile,
                                              uint8_t* lo) {
  const float ss = dot2_bf16(rh.y, rh.y, dot2_bf16(rh.x, rh.x, dot2_bf16(rl.y, rl.y, dot2_bf16(rl.x, rl.x, 0.f))));
  const float inv = rsqrt_(row16_sum(ss) * (1.0f / kD) + eps);
  const float x[8] = {bf2f_lo(rl.x), bf2f_hi(rl.x), bf2f_lo(rl.y), bf2f_hi(rl.y),
                      bf2f_lo(rh.x), bf2f_hi(rh.x), bf2f_lo(rh.y), bf2f_hi(rh.y)};
  float y[8];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const float a = kWeights ? x[e] * w[e] : x[e];
    const float b = kWeights ? x[4 + e] * w[4 + e] : x[4 + e];
    const float c = E[e].x * inv, s = E[e].y * inv;
    y[e] = fmaf(a, c, -b * s);
    y[4 + e] = fmaf(b, c, a * s);
  }
  const uint2 hlo = make_uint2(pack2(y[0], y[1]), pack2(y[2], y[3]));
  const uint2 hhi = make_uint2(pack2(y[4], y[5]), pack2(y[6], y[7]));
  lds_st<uint2>(tile, tile_off(t, 4 * j), hlo);
  lds_st<uint2>(tile, tile_off(t, kHalf + 4 * j), hhi);
  if (lo != nullptr && t < kExactRows) {
    const uint2 llo = make_uint2(pack2(y[0] - bf2f_lo(hlo.x), y[1] - bf2f_hi(hlo.x)),
                                 pack2(y[2] - bf2f_lo(hlo.y), y[3] - bf2f_hi(hlo.y)));
    const uint2 lhi = make_uint2(pack2(y[4] - bf2f_lo(hhi.x), y[5] - bf2f_hi(hhi.x)),
                                 pack2(y[6] - bf2f_lo(hhi.y), y[7] - bf2f_hi(hhi.y)));
    lds_st<uint2>(lo, tile_off(t, 4 * j), llo);
    lds_st<uint2>(lo, tile_off(t, kHalf + 4 * j), lhi);
  }
}

// Rotations of the thread's rows rg + kStep m at its frequencies 4j + e, from the
// chunk's base rotations sRot: E_0 = sRot * A, E_m = E_{m-1} * Z.
template <int kStep>
__device__ __forceinline__ void first_rotation(const float2* sRot, const Rope& L, int j, float2 (&E)[4]) {
#pragma unroll
  for (int e = 0; e < 4; ++e) E[e] = cmul(sRot[4 * j + e], L.A[e]);
}
__device__ __forceinline__ void next_rotation(const Rope& L, float2 (&E)[4]) {
#pragma unroll
  for (int e = 0; e < 4; ++e) E[e] = cmul(E[e], L.Z[e]);
}

// One tensor (k in the state kernel).
template <bool kWeights, int M, int kStep>
__device__ __forceinline__ void norm_rope_stage(const Rows<M>& R, const float (&w)[8], float eps,
                                                const float2* sRot, const Rope& L, int rg, int j,
                                                uint8_t* tile) {
  float2 E[4];
  first_rotation<kStep>(sRot, L, j, E);
#pragma unroll
  for (int m = 0; m < M; ++m) {
    if (m > 0) next_rotation(L, E);
    norm_rope_row<kWeights>(R.lo[m], R.hi[m], w, eps, E, rg + kStep * m, j, tile, nullptr);
  }
}

// One tensor, with the first row's rotations E already formed (advanced in place).
template <bool kWeights, int M, int kStep>
__device__ __forceinline__ void norm_rope_rows(const Rows<M>& R, const float (&w)[8], float eps, float2 (&E)[4],
                                               const Rope& L, int rg, int j, uint8_t* tile, uint8_t* lo) {
#pragma unroll
  for (int m = 0; m < M; ++m) {
    if (m > 0) next_rotation(L, E);
    norm_rope_row<kWeights>(R.lo[m], R.hi[m], w, eps, E, rg + kStep * m, j, tile, lo);
  }
}

// q and k of the same rows share one rotation chain.
template <bool kWeights, int M, int kStep>
__device__ __forceinline__ void norm_rope_stage_qk(const Rows<M>& Qr, const Rows<M>& Kr, const float (&wq)[8],
                                                   const float (&wk)[8], float eps, const float2* sRot,
                                                   const Rope& L, int rg, int j, uint8_t* tq, uint8_t* tk,
                                                   uint8_t* lq, uint8_t* lk) {
  float2 E[4];
  first_rotation<kStep>(sRot, L, j, E);
#pragma unroll
  for (int m = 0; m < M; ++m) {
    if (m > 0) next_rotation(L, E);
    const int t = rg + kStep * m;
    norm_rope_row<kWeights>(Qr.lo[m], Qr.hi[m], wq, eps, E, t, j, tq, lq);
    norm_rope_row<kWeights>(Kr.lo[m], Kr.hi[m], wk, eps, E, t, j, tk, lk);
  }
}

__device__ __forceinline__ void load_norm_weights(const float* w, int j, float (&out)[8]) {
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    out[e] = w ? w[4 * j + e] : 1.0f;
    out[4 + e] = w ? w[kHalf + 4 * j + e] : 1.0f;
  }
}

struct Tile {
  int b, h, seg, t_begin, t_end, nch;
  int64_t base;      // element offset of (row 0, h, d = 0) for the rows of this tile's sequence
  int64_t pos_base;  // absolute position of row 0 in those rows
  float* state;      // this (b, h, segment)'s D x D state in the workspace
};

// Workgroup -> (b, h, segment).  Equal-length batches: blockIdx = h + H (seg +
// nseg b), rows t of sequence b.  Variable-length batches: blockIdx = h + H s for
// segment s of the table, rows t of the packed activations.
__device__ __forceinline__ Tile decode_tile(const PrefillParams& p) {
  Tile tl;
  int bid = blockIdx.x;
  tl.h = bid % p.H;
  bid /= p.H;
  if (p.segs != nullptr) {
    const SegDesc d = p.segs[bid];
    tl.b = d.seq;
    tl.seg = d.seg_local;
    tl.t_begin = d.t_begin;
    tl.t_end = d.t_end;
    tl.base = (int64_t)tl.h * kD;
    tl.pos_base = d.pos_base;
    tl.state = p.ws + ((int64_t)bid * p.H + tl.h) * kD * kD;
  } else {
    tl.seg = bid % p.nseg;
    tl.b = bid / p.nseg;
    tl.t_begin = tl.seg * p.cps * kC;
    tl.t_end = min(p.T, tl.t_begin + p.cps * kC);
    tl.base = ((int64_t)tl.b * p.T * p.H + tl.h) * kD;
    tl.pos_base = p.pos0;
    tl.state = p.ws + (((int64_t)tl.b * p.H + tl.h) * p.nseg + tl.seg) * kD * kD;
  }
  tl.nch = (tl.t_end - tl.t_begin + kC - 1) / kC;
  return tl;
}

// S accumulator tile rtk of wave w: lane (g, n16) element r is
// S[16 rtk + 4 g + r][16 w + n16].
__device__ __forceinline__ int64_t state_elem(int rtk, int r, int w, int g4, int n16) {
  return (int64_t)(16 * rtk + 4 * g4 + r) * kD + 16 * w + n16;
}

// Token-contraction operand of V: lane n16 gets V[32kk + 4g + 16(e/4) + e%4][c0 + n16].
__device__ __forceinline__ bf16x8 v_operand(const uint8_t* sV, int kk, int c0, int g4, int n16) {
  const int t0 = 32 * kk + 4 * g4 + (n16 >> 2), c = c0 + 4 * (n16 & 3);
  return as_bf16x8(lds_tr(sV, tile_off(t0, c)), lds_tr(sV, tile_off(t0 + 16, c)));
}

// S[:, 16w .. 16w+16) += Kh^T V over one chunk.
__device__ __forceinline__ void accumulate_state(f32x4 (&Sacc)[8], const uint8_t* sK,
                                                 const bf16x8 (&Vop)[2], int g4, int n16) {
#pragma unroll
  for (int kk = 0; kk < kC / 32; ++kk) {
    const int t0 = 32 * kk + 4 * g4 + (n16 >> 2);
#pragma unroll
    for (int rtk = 0; rtk < 8; ++rtk) {
      const int c = 16 * rtk + 4 * (n16 & 3);
      const bf16x8 a = as_bf16x8(lds_tr(sK, tile_off(t0, c)), lds_tr(sK, tile_off(t0 + 16, c)));
      Sacc[rtk] = mma(a, Vop[kk], Sacc[rtk]);
    }
  }
}

// --------------------------------------------------------------------------
// Kh^T V summed over each segment.  LDS is double-buffered, so one barrier per
// chunk separates staging from use.
template <bool kWeights>
__global__ __launch_bounds__(kThreads) void la_chunk_state_kernel(PrefillParams p) {
  __shared__ __attribute__((aligned(16))) uint8_t sK[2][kTileBytes];
  __shared__ __attribute__((aligned(16))) uint8_t sV[2][kTileBytes];
  __shared__ float2 sRot[2][kHalf];

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int n16 = lane & 15, g4 = lane >> 4;
  const int j = tid & 15, rg = tid >> 4;
  const Tile tl = decode_tile(p);
  const int64_t rs = (int64_t)p.H * kD;

  float wk[8];
  load_norm_weights(p.kw, j, wk);
  Rope L;
  rope_init<32>(p, tid, rg, j, L);

  f32x4 Sacc[8];
#pragma unroll
  for (int a = 0; a < 8; ++a) Sacc[a] = f32x4{0.f, 0.f, 0.f, 0.f};

  Rows<2> Kr, Vr;
  {
    const int nv = min(kC, tl.t_end - tl.t_begin);
    load_rows<2, 32>(p.k + tl.base + (int64_t)tl.t_begin * rs, rs, nv, rg, j, Kr);
    load_rows<2, 32>(p.v + tl.base + (int64_t)tl.t_begin * rs, rs, nv, rg, j, Vr);
  }
  if (tid < kHalf) sRot[0][tid] = rope_rotation(tl.pos_base + tl.t_begin, L.base_rev);
  __syncthreads();

  for (int c = 0; c < tl.nch; ++c) {
    const int t0 = tl.t_begin + c * kC;
    const int nv = min(kC, tl.t_end - t0);
    uint8_t* bK = sK[c & 1];
    uint8_t* bV = sV[c & 1];
    norm_rope_stage<kWeights, 2, 32>(Kr, wk, p.eps, sRot[c & 1], L, rg, j, bK);
    store_rows_masked<2, 32>(bV, Vr, nv, rg, j);
    if (c + 1 < tl.nch) {
      const int t1 = t0 + kC;
      const int nv1 = min(kC, tl.t_end - t1);
      load_rows<2, 32>(p.k + tl.base + (int64_t)t1 * rs, rs, nv1, rg, j, Kr);
      load_rows<2, 32>(p.v + tl.base + (int64_t)t1 * rs, rs, nv1, rg, j, Vr);
      if (tid < kHalf) sRot[(c + 1) & 1][tid] = rope_rotation(tl.pos_base + t1, L.base_rev);
    }
    __syncthreads();
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
// Exclusive prefix of the per-segment states, in place, seeded with S_in; the
// inclusive total is the final state.  One thread per 4 consecutive elements.
// A variable-length batch walks each sequence's own run of segments (none for an
// empty sequence, whose final state is S_in) and skips single-token sequences.
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
  for (int s = 0; s < nseg; ++s) {
    const float4 d = ws[s * stride];
    ws[s * stride] = run;
    run.x += d.x;
    run.y += d.y;
    run.z += d.z;
    run.w += d.w;
  }
  reinterpret_cast<float4*>(p.S_out)[idx] = run;
}

// --------------------------------------------------------------------------
// Output kernel.  Threads 0..255 are the consumer waves (wave w owns value
// columns [32w, 32w + 32)); threads 256..767 are the producer waves (thread
// (rg, j) stages rows rg and rg + 32).  Both roles run their own loop with the
// same number of barriers: two before the loop and two per chunk.
constexpr int kConsumers = 256;               // 4 consumer waves
constexpr int kProducers = 512;               // 8 producer waves
constexpr int kOutThreads = kConsumers + kProducers;

// Consumer operand in key order pi: lane n16 gets X[row][32kk + 4g + 16(e/4) + e%4].
__device__ __forceinline__ bf16x8 pi_operand(const uint8_t* tile, int row, int kk, int g4) {
  return as_bf16x8(lds_ld<uint2>(tile, tile_off(row, 32 * kk + 4 * g4)),
                   lds_ld<uint2>(tile, tile_off(row, 32 * kk + 16 + 4 * g4)));
}

template <bool kWeights>
__device__ __forceinline__ void produce(const PrefillParams& p, const Tile& tl, uint8_t (*sQ)[kTileBytes],
                                        uint8_t (*sK)[kTileBytes], uint8_t (*sV)[kTileBytes],
                                        uint8_t (*sG)[kTileBytes], uint8_t* sQl, uint8_t* sKl,
                                        float2 (*sRot)[kHalf]) {
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
  auto load_chunk = [&](int c, Chunk& R) {
    const int t = tl.t_begin + c * kC;
    const int nv = min(kC, tl.t_end - t);
    const int64_t off = tl.base + (int64_t)t * rs;
    load_rows<2, 32>(p.q + off, rs, nv, rg, j, R.q);
    load_rows<2, 32>(p.k + off, rs, nv, rg, j, R.k);
    load_rows<2, 32>(p.v + off, rs, nv, rg, j, R.v);
    load_rows<2, 32>(p.g + off, rs, nv, rg, j, R.g);
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
  // other register set).
  auto step = [&](int c, Chunk& R) {
    if (c + 1 < tl.nch) {
      stage(c + 1, R);
      if (c + 3 < tl.nch) load_chunk(c + 3, R);
      if (c + 2 < tl.nch && ptid < kHalf)
        sRot[c & 1][ptid] = rope_rotation(tl.pos_base + tl.t_begin + (c + 2) * kC, L.base_rev);
    }
    __syncthreads();
    __syncthreads();
  };

  load_chunk(0, Y);
  if (ptid < kHalf) {
    sRot[0][ptid] = rope_rotation(tl.pos_base + tl.t_begin, L.base_rev);
    if (tl.nch > 1) sRot[1][ptid] = rope_rotation(tl.pos_base + tl.t_begin + kC, L.base_rev);
  }
  __syncthreads();
  stage(0, Y);
  if (tl.nch > 1) load_chunk(1, X);
  if (tl.nch > 2) load_chunk(2, Y);
  __syncthreads();
  for (int c = 0; c < tl.nch; c += 2) {
    step(c, X);
    if (c + 1 < tl.nch) step(c + 1, Y);
  }
}

// Score tiles (row block rt, key block st <= rt) of a chunk dealt to the 4 consumer
// waves (3/3/2/2): tile idx has rt = (kTileRT >> 2 idx) & 3, st = (kTileST >> 2 idx)
// & 3 for the order (0,0) (1,1) (2,2) (3,3) (1,0) (2,1) (3,2) (2,0) (3,1) (3,0).
constexpr uint32_t kTileRT = 0xfb9e4;
constexpr uint32_t kTileST = 0x124e4;
constexpr int kScoreRowBytes = kC * 2 + 16;  // [64][64] bf16 score tile, padded rows

__device__ __forceinline__ int score_off(int t, int s) { return t * kScoreRowBytes + 2 * s; }

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
      const uint2 out = make_uint2(pack2(Oacc[dt][rt][0] * f16_lo(sg.x), Oacc[dt][rt][1] * f16_hi(sg.x)),
                                   pack2(Oacc[dt][rt][2] * f16_lo(sg.y), Oacc[dt][rt][3] * f16_hi(sg.y)));
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
  f32x4 Sacc[2][8];
  {
    const float* src = tl.state;
#pragma unroll
    for (int dt = 0; dt < 2; ++dt)
#pragma unroll
      for (int rtk = 0; rtk < 8; ++rtk)
#pragma unroll
        for (int r = 0; r < 4; ++r) Sacc[dt][rtk][r] = src[state_elem(rtk, r, 2 * w + dt, g4, n16)];
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
}

template <bool kWeights>
__global__ __launch_bounds__(kOutThreads) void la_chunk_output_kernel(PrefillParams p) {
  __shared__ __attribute__((aligned(16))) uint8_t sQ[2][kTileBytes];
  __shared__ __attribute__((aligned(16))) uint8_t sK[2][kTileBytes];
  __shared__ __attribute__((aligned(16))) uint8_t sV[2][kTileBytes];
  __shared__ __attribute__((aligned(16))) uint8_t sG[2][kTileBytes];  // sigmoid(gate), f16
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
// Wide-chunk output kernel, C = 64 kSub (kSub = 2 or 4).  The chunked form with
// chunk C: query sub-block i (64 rows) of a chunk takes its scores against key
// sub-blocks jj <= i (causally masked at jj = i) and its inter-chunk term from the
// state at the chunk start; the chunk's Kh^T V joins the state after the chunk.
// Tiles are single-buffered and k, v of sub-block jj are staged again for every
// i >= jj, so a wider chunk costs more work and more reads than C = 64.  Eight
// waves; wave w owns value columns [16 w, 16 w + 16) of S and o.  Three barriers
// per (i, jj): after staging, after the scores, after the intra-chunk product.
constexpr int kWideThreads = 512;

template <bool kWeights, int kSub>
__global__ __launch_bounds__(kWideThreads, 2) void la_chunk_output_wide_kernel(PrefillParams p) {
  __shared__ __attribute__((aligned(16))) uint8_t sQ[kTileBytes];
  __shared__ __attribute__((aligned(16))) uint8_t sK[kTileBytes];
  __shared__ __attribute__((aligned(16))) uint8_t sV[kTileBytes];
  __shared__ __attribute__((aligned(16))) uint8_t sQl[kExactRows * kRowBytes];
  __shared__ __attribute__((aligned(16))) uint8_t sKl[kExactRows * kRowBytes];
  __shared__ __attribute__((aligned(16))) uint8_t sP[kC * kScoreRowBytes];

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int n16 = lane & 15, g4 = lane >> 4;
  const int j = tid & 15, rg = tid >> 4;
  const Tile tl = decode_tile(p);
  const int64_t rs = (int64_t)p.H * kD;

  float wq[8], wk[8];
  load_norm_weights(p.qw, j, wq);
  load_norm_weights(p.kw, j, wk);
  Rope L;
  rope_init<32>(p, tid, rg, j, L);
  double rev[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) rev[e] = p.freqs.rev[4 * j + e];
  // rotations of row rg of a sub-block starting at token t
  auto first_rows = [&](int t, float2 (&E)[4]) {
#pragma unroll
    for (int e = 0; e < 4; ++e) E[e] = cmul(rope_rotation(tl.pos_base + t, rev[e]), L.A[e]);
  };

  // prefix state of this segment: S[:, 16 w .. 16 w + 16)
  f32x4 Sacc[8];
  {
    const float* src = tl.state;
#pragma unroll
    for (int rtk = 0; rtk < 8; ++rtk)
#pragma unroll
      for (int r = 0; r < 4; ++r) Sacc[rtk][r] = src[state_elem(rtk, r, w, g4, n16)];
  }
  // this lane's output (and gate) columns 16 w + 4 g .. + 3 of (b, h)
  const int64_t col_off = tl.base + 16 * w + 4 * g4;

  for (int t0 = tl.t_begin; t0 < tl.t_end; t0 += kSub * kC) {
    f32x4 Dacc[8];
#pragma unroll
    for (int a = 0; a < 8; ++a) Dacc[a] = f32x4{0.f, 0.f, 0.f, 0.f};
    for (int i = 0; i < kSub; ++i) {
      const int ti = t0 + i * kC;
      if (ti >= tl.t_end) break;
      const int nvi = min(kC, tl.t_end - ti);
      // scores of the first 16 rows of a call use the hi/lo split (see the C = 64 kernel)
      const bool exact = tl.seg == 0 && t0 == tl.t_begin && i == 0;
      // gate logits of the lane's rows ti + 16 rt + n16 (clamped to the sub-block's last valid row)
      uint2 graw[4];
#pragma unroll
      for (int rt = 0; rt < 4; ++rt)
        graw[rt] = ld_stream(p.g + col_off + (int64_t)(ti + min(16 * rt + n16, nvi - 1)) * rs);
      f32x4 Oacc[4];
      for (int jj = 0; jj <= i; ++jj) {
        const int tj = t0 + jj * kC;
        const int nvj = min(kC, tl.t_end - tj);
        {
          Rows<2> Kr, Vr;
          load_rows<2, 32>(p.k + tl.base + (int64_t)tj * rs, rs, nvj, rg, j, Kr);
          load_rows<2, 32>(p.v + tl.base + (int64_t)tj * rs, rs, nvj, rg, j, Vr);
          if (jj == 0) {
            Rows<2> Qr;
            load_rows<2, 32>(p.q + tl.base + (int64_t)ti * rs, rs, nvi, rg, j, Qr);
            float2 E[4];
            first_rows(ti, E);
            norm_rope_rows<kWeights, 2, 32>(Qr, wq, p.eps, E, L, rg, j, sQ, exact ? sQl : nullptr);
          }
          float2 E[4];
          first_rows(tj, E);
          norm_rope_rows<kWeights, 2, 32>(Kr, wk, p.eps, E, L, rg, j, sK, exact && jj == 0 ? sKl : nullptr);
          store_rows_masked<2, 32>(sV, Vr, nvj, rg, j);
        }
        __syncthreads();
        if (jj == 0) {
          // inter-chunk term O^T = S^T Qh^T (key dims in order pi)
          bf16x8 SA[4];
#pragma unroll
          for (int kk = 0; kk < 4; ++kk) SA[kk] = pack8(Sacc[2 * kk], Sacc[2 * kk + 1]);
#pragma unroll
          for (int rt = 0; rt < 4; ++rt) {
            Oacc[rt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) Oacc[rt] = mma(SA[kk], pi_operand(sQ, 16 * rt + n16, kk, g4), Oacc[rt]);
          }
        }
        // scores of query sub-block i against key sub-block jj, two 16x16 tiles per wave
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          const int idx = w + 8 * u;
          const int rt = idx >> 2, st = idx & 3;
          f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int ks = 0; ks < kD / 32; ++ks) {
            const int ka = tile_off(16 * st + n16, 32 * ks + 8 * g4);
            const int qa = tile_off(16 * rt + n16, 32 * ks + 8 * g4);
            const bf16x8 kf = as_bf16x8(lds_ld<uint4>(sK, ka));
            const bf16x8 qf = as_bf16x8(lds_ld<uint4>(sQ, qa));
            if (exact && idx == 0) {
              acc = mma(as_bf16x8(lds_ld<uint4>(sKl, ka)), qf, acc);
              acc = mma(kf, as_bf16x8(lds_ld<uint4>(sQl, qa)), acc);
            }
            acc = mma(kf, qf, acc);
          }
          if (jj == i) {
#pragma unroll
            for (int r = 0; r < 4; ++r)
              if (st > rt || (st == rt && 4 * g4 + r > n16)) acc[r] = 0.f;
          }
          lds_st<uint2>(sP, score_off(16 * rt + n16, 16 * st + 4 * g4),
                        make_uint2(pack2(acc[0], acc[1]), pack2(acc[2], acc[3])));
        }
        bf16x8 Vf[2];
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) Vf[kk] = v_operand(sV, kk, 16 * w, g4, n16);
        if (jj == i) accumulate_state(Dacc, sK, Vf, g4, n16);
        __syncthreads();
        // O^T += V^T P^T
#pragma unroll
        for (int rt = 0; rt < 4; ++rt) {
          const int t = 16 * rt + n16;
#pragma unroll
          for (int kk = 0; kk < 2; ++kk) {
            const bf16x8 pb = as_bf16x8(lds_ld<uint2>(sP, score_off(t, 32 * kk + 4 * g4)),
                                        lds_ld<uint2>(sP, score_off(t, 32 * kk + 16 + 4 * g4)));
            Oacc[rt] = mma(Vf[kk], pb, Oacc[rt]);
          }
        }
        __syncthreads();
      }
      // gate and store: lane holds o[ti + 16 rt + n16][16 w + 4 g .. + 3]
#pragma unroll
      for (int rt = 0; rt < 4; ++rt) {
        if (16 * rt + n16 < nvi) {
          const uint2 gr = graw[rt];
          const uint2 out = make_uint2(pack2(Oacc[rt][0] * sigmoidf_(bf2f_lo(gr.x)), Oacc[rt][1] * sigmoidf_(bf2f_hi(gr.x))),
                                       pack2(Oacc[rt][2] * sigmoidf_(bf2f_lo(gr.y)), Oacc[rt][3] * sigmoidf_(bf2f_hi(gr.y))));
          *reinterpret_cast<uint2*>(p.o + col_off + (int64_t)(ti + 16 * rt + n16) * rs) = out;
        }
      }
    }
#pragma unroll
    for (int a = 0; a < 8; ++a) Sacc[a] += Dacc[a];
  }
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
  if (plan.nwork > 0) {
    if (weights)
      hipLaunchKernelGGL(la_chunk_state_kernel<true>, grid, dim3(kThreads), 0, stream, p);
    else
      hipLaunchKernelGGL(la_chunk_state_kernel<false>, grid, dim3(kThreads), 0, stream, p);
  }
  mark(1);
  if (plan.scan)
    hipLaunchKernelGGL(la_state_scan_kernel, dim3((unsigned)((scan_threads + 255) / 256)), dim3(256), 0,
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

}  // namespace la
