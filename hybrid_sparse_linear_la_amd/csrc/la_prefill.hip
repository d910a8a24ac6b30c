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
//      segment's prefix state (held in MFMA accumulators, fp32) and walks the
//      chunks: QK-RMSNorm + RoPE prologue into LDS, masked scores, P V + Qh S,
//      sigmoid gate, coalesced bf16 store, then S += Kh^T V.
//
// Workgroup: 256 threads = 4 waves.  Wave w owns value columns [32w, 32w + 32)
// of S and of the chunk output, so S never leaves registers: an accumulator
// tile pair converts to the B operand of Qh S directly (the key-dim order of the
// operand is permuted, and Qh is read with the same permutation).
#include "la_device.hpp"
#include "la_internal.hpp"

namespace la {
namespace {

constexpr int kThreads = 256;

// Staging coordinates: thread (rg = tid / 16, j = tid % 16) holds rows 4rg..4rg+3
// of a chunk and dims {4j..4j+3} U {64+4j..64+4j+3} (so each RoPE pair (i, i+64)
// sits in one thread).
struct RawRows {
  uint2 lo[4];  // dims 4j..4j+3 of rows 4rg+m, four bf16 each
  uint2 hi[4];  // dims 64+4j..64+4j+3
};

__device__ __forceinline__ void load_rows(const uint16_t* __restrict__ base, int64_t row_stride,
                                          int nvalid, int rg, int j, RawRows& R) {
#pragma unroll
  for (int m = 0; m < 4; ++m) {
    const int r = 4 * rg + m;
    if (r < nvalid) {
      const uint16_t* src = base + (int64_t)r * row_stride;
      R.lo[m] = *reinterpret_cast<const uint2*>(src + 4 * j);
      R.hi[m] = *reinterpret_cast<const uint2*>(src + kHalf + 4 * j);
    } else {
      R.lo[m] = make_uint2(0u, 0u);
      R.hi[m] = make_uint2(0u, 0u);
    }
  }
}

// QK-normalization (RMSNorm over the 128 dims of a row) followed by rotate-half
// RoPE, in fp32, rounded to bf16 in place.  E[m][e] is the rotation of row 4rg+m
// at frequency 4j+e.  Rows at or beyond nvalid stay zero.
__device__ __forceinline__ void norm_rope(RawRows& R, const float (&w)[8], float eps,
                                          const float2 (&E)[4][4], int nvalid, int rg) {
#pragma unroll
  for (int m = 0; m < 4; ++m) {
    float x[8] = {bf2f_lo(R.lo[m].x), bf2f_hi(R.lo[m].x), bf2f_lo(R.lo[m].y), bf2f_hi(R.lo[m].y),
                  bf2f_lo(R.hi[m].x), bf2f_hi(R.hi[m].x), bf2f_lo(R.hi[m].y), bf2f_hi(R.hi[m].y)};
    float ss = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) ss = fmaf(x[e], x[e], ss);
    ss += __shfl_xor(ss, 1);
    ss += __shfl_xor(ss, 2);
    ss += __shfl_xor(ss, 4);
    ss += __shfl_xor(ss, 8);
    const float inv = (4 * rg + m < nvalid) ? rsqrtf(ss * (1.0f / kD) + eps) : 0.f;
    float y[8];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float a = x[e] * inv * w[e];
      const float b = x[4 + e] * inv * w[4 + e];
      const float c = E[m][e].x, s = E[m][e].y;
      y[e] = a * c - b * s;
      y[4 + e] = b * c + a * s;
    }
    R.lo[m] = make_uint2(pack2(y[0], y[1]), pack2(y[2], y[3]));
    R.hi[m] = make_uint2(pack2(y[4], y[5]), pack2(y[6], y[7]));
  }
}

// As norm_rope, but also splits each normalized value y into bf16 hi = bf16(y)
// and lo = bf16(y - hi) and writes both row tiles to LDS; R keeps hi.  The score
// tile is then formed from hi*hi + hi*lo + lo*hi, which removes the bf16
// rounding of qh and kh from the scores (that rounding would otherwise dominate
// the error of early rows, whose output is a sum of only a few scores).
__device__ __forceinline__ void norm_rope_split(RawRows& R, const float (&w)[8], float eps,
                                                const float2 (&E)[4][4], int nvalid, int rg, int j,
                                                uint8_t* sHi, uint8_t* sLo) {
#pragma unroll
  for (int m = 0; m < 4; ++m) {
    float x[8] = {bf2f_lo(R.lo[m].x), bf2f_hi(R.lo[m].x), bf2f_lo(R.lo[m].y), bf2f_hi(R.lo[m].y),
                  bf2f_lo(R.hi[m].x), bf2f_hi(R.hi[m].x), bf2f_lo(R.hi[m].y), bf2f_hi(R.hi[m].y)};
    float ss = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) ss = fmaf(x[e], x[e], ss);
    ss += __shfl_xor(ss, 1);
    ss += __shfl_xor(ss, 2);
    ss += __shfl_xor(ss, 4);
    ss += __shfl_xor(ss, 8);
    const float inv = (4 * rg + m < nvalid) ? rsqrtf(ss * (1.0f / kD) + eps) : 0.f;
    float y[8], r[8];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float a = x[e] * inv * w[e];
      const float b = x[4 + e] * inv * w[4 + e];
      const float c = E[m][e].x, s = E[m][e].y;
      y[e] = a * c - b * s;
      y[4 + e] = b * c + a * s;
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) r[e] = y[e] - bf2f(f2bf(y[e]));
    R.lo[m] = make_uint2(pack2(y[0], y[1]), pack2(y[2], y[3]));
    R.hi[m] = make_uint2(pack2(y[4], y[5]), pack2(y[6], y[7]));
    const int t = 4 * rg + m;
    lds_st<uint2>(sHi, row_off(t, 4 * j), R.lo[m]);
    lds_st<uint2>(sHi, row_off(t, kHalf + 4 * j), R.hi[m]);
    lds_st<uint2>(sLo, row_off(t, 4 * j), make_uint2(pack2(r[0], r[1]), pack2(r[2], r[3])));
    lds_st<uint2>(sLo, row_off(t, kHalf + 4 * j), make_uint2(pack2(r[4], r[5]), pack2(r[6], r[7])));
  }
}

__device__ __forceinline__ uint32_t half16(uint2 u, int e) {
  const uint32_t word = (e < 2) ? u.x : u.y;
  return (e & 1) ? (word >> 16) : (word & 0xffffu);
}

// Rows 4rg..4rg+3 of the thread's 8 dims -> transposed tile [128][C]: one 8-byte
// write (4 consecutive tokens) per dim.
template <int C>
__device__ __forceinline__ void store_transposed(uint8_t* sT, const RawRows& R, int rg, int j) {
#pragma unroll
  for (int hf = 0; hf < 2; ++hf) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const uint2* src = hf ? R.hi : R.lo;
      const uint2 packed = make_uint2(half16(src[0], e) | (half16(src[1], e) << 16),
                                      half16(src[2], e) | (half16(src[3], e) << 16));
      lds_st<uint2>(sT, col_off<C>(hf * kHalf + 4 * j + e, 4 * rg), packed);
    }
  }
}

__device__ __forceinline__ void store_rows(uint8_t* sR, const RawRows& R, int rg, int j) {
#pragma unroll
  for (int m = 0; m < 4; ++m) {
    lds_st<uint2>(sR, row_off(4 * rg + m, 4 * j), R.lo[m]);
    lds_st<uint2>(sR, row_off(4 * rg + m, kHalf + 4 * j), R.hi[m]);
  }
}

// Per-thread RoPE offsets: A[e] = e^{i 4rg theta}, Z[e] = e^{i theta} for the
// thread's four frequencies 4j+e.  Row 4rg+m of a chunk starting at position p0
// is rotated by base(p0) * A * Z^m.
struct RopeLane {
  float2 A[4];
  float2 Z[4];
};

__device__ __forceinline__ void rope_lane_init(const PrefillParams& p, int rg, int j, RopeLane& L) {
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const double th = p.freqs.theta[4 * j + e];
    L.A[e] = rope_rotation(4 * rg, th);
    L.Z[e] = rope_rotation(1, th);
  }
}

__device__ __forceinline__ void chunk_rotations(const float2* sRot, const RopeLane& L, int j,
                                                float2 (&E)[4][4]) {
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    E[0][e] = cmul(sRot[4 * j + e], L.A[e]);
#pragma unroll
    for (int m = 1; m < 4; ++m) E[m][e] = cmul(E[m - 1][e], L.Z[e]);
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
  int64_t base;  // element offset of (b, t = 0, h, d = 0)
};

template <int C>
__device__ __forceinline__ Tile decode_tile(const PrefillParams& p) {
  Tile tl;
  int bid = blockIdx.x;
  tl.h = bid % p.H;
  bid /= p.H;
  tl.seg = bid % p.nseg;
  tl.b = bid / p.nseg;
  tl.t_begin = tl.seg * p.cps * C;
  tl.t_end = min(p.T, tl.t_begin + p.cps * C);
  tl.nch = (tl.t_end - tl.t_begin + C - 1) / C;
  tl.base = ((int64_t)tl.b * p.T * p.H + tl.h) * kD;
  return tl;
}

// S tile (rows 16 rtk + 4 g4 + r, columns 32 w + 16 ct + n16) <-> global fp32 [D][D].
__device__ __forceinline__ int64_t state_elem(int rtk, int ct, int r, int w, int g4, int n16) {
  return (int64_t)(16 * rtk + 4 * g4 + r) * kD + 32 * w + 16 * ct + n16;
}

// S[:, 32w .. 32w+32) += Kh^T V over one chunk (K = C tokens).
template <int C>
__device__ __forceinline__ void accumulate_state(f32x4 (&Sacc)[8][2], const uint8_t* sKT,
                                                 const uint8_t* sVT, int w, int g4, int n16) {
#pragma unroll
  for (int kk = 0; kk < C / 32; ++kk) {
    const bf16x8 b0 = as_bf16x8(lds_ld<uint4>(sVT, col_off<C>(32 * w + n16, 32 * kk + 8 * g4)));
    const bf16x8 b1 = as_bf16x8(lds_ld<uint4>(sVT, col_off<C>(32 * w + 16 + n16, 32 * kk + 8 * g4)));
#pragma unroll
    for (int rtk = 0; rtk < 8; ++rtk) {
      const bf16x8 a = as_bf16x8(lds_ld<uint4>(sKT, col_off<C>(16 * rtk + n16, 32 * kk + 8 * g4)));
      Sacc[rtk][0] = mma(a, b0, Sacc[rtk][0]);
      Sacc[rtk][1] = mma(a, b1, Sacc[rtk][1]);
    }
  }
}

// --------------------------------------------------------------------------
template <int C>
__global__ __launch_bounds__(kThreads) void la_chunk_state_kernel(PrefillParams p) {
  static_assert(C == 64, "staging layout assumes 64-token chunks");
  __shared__ __attribute__((aligned(16))) uint8_t sKT[kD * C * 2];
  __shared__ __attribute__((aligned(16))) uint8_t sVT[kD * C * 2];
  __shared__ float2 sRot[2][kHalf];

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int n16 = lane & 15, g4 = lane >> 4;
  const int j = tid & 15, rg = tid >> 4;
  const Tile tl = decode_tile<C>(p);
  const int64_t rs = (int64_t)p.H * kD;

  float wk[8];
  load_norm_weights(p.kw, j, wk);
  RopeLane L;
  rope_lane_init(p, rg, j, L);

  f32x4 Sacc[8][2];
#pragma unroll
  for (int a = 0; a < 8; ++a) Sacc[a][0] = Sacc[a][1] = f32x4{0.f, 0.f, 0.f, 0.f};

  RawRows Kr, Vr;
  {
    const int nv = min(C, tl.t_end - tl.t_begin);
    load_rows(p.k + tl.base + (int64_t)tl.t_begin * rs, rs, nv, rg, j, Kr);
    load_rows(p.v + tl.base + (int64_t)tl.t_begin * rs, rs, nv, rg, j, Vr);
  }
  if (tid < kHalf) sRot[0][tid] = rope_rotation(p.pos0 + tl.t_begin, p.freqs.theta[tid]);
  __syncthreads();

  for (int c = 0; c < tl.nch; ++c) {
    const int t0 = tl.t_begin + c * C;
    const int nv = min(C, tl.t_end - t0);
    float2 E[4][4];
    chunk_rotations(sRot[c & 1], L, j, E);
    norm_rope(Kr, wk, p.eps, E, nv, rg);
    store_transposed<C>(sKT, Kr, rg, j);
    store_transposed<C>(sVT, Vr, rg, j);
    if (c + 1 < tl.nch) {
      const int t1 = t0 + C;
      const int nv1 = min(C, tl.t_end - t1);
      load_rows(p.k + tl.base + (int64_t)t1 * rs, rs, nv1, rg, j, Kr);
      load_rows(p.v + tl.base + (int64_t)t1 * rs, rs, nv1, rg, j, Vr);
      if (tid < kHalf) sRot[(c + 1) & 1][tid] = rope_rotation(p.pos0 + t1, p.freqs.theta[tid]);
    }
    __syncthreads();
    accumulate_state<C>(Sacc, sKT, sVT, w, g4, n16);
    __syncthreads();
  }

  float* dst = p.ws + (((int64_t)tl.b * p.H + tl.h) * p.nseg + tl.seg) * kD * kD;
#pragma unroll
  for (int rtk = 0; rtk < 8; ++rtk)
#pragma unroll
    for (int ct = 0; ct < 2; ++ct)
#pragma unroll
      for (int r = 0; r < 4; ++r) dst[state_elem(rtk, ct, r, w, g4, n16)] = Sacc[rtk][ct][r];
}

// --------------------------------------------------------------------------
// Exclusive prefix of the per-segment states, in place, seeded with S_in; the
// inclusive total is the final state.  One thread per 4 consecutive elements.
__global__ __launch_bounds__(256) void la_state_scan_kernel(PrefillParams p) {
  constexpr int64_t per = kD * kD / 4;
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= (int64_t)p.B * p.H * per) return;
  const int64_t bh = idx / per, e = idx - bh * per;
  float4 run = p.S_in ? reinterpret_cast<const float4*>(p.S_in)[idx] : make_float4(0.f, 0.f, 0.f, 0.f);
  float4* ws = reinterpret_cast<float4*>(p.ws) + bh * p.nseg * per + e;
  for (int s = 0; s < p.nseg; ++s) {
    const float4 d = ws[s * per];
    ws[s * per] = run;
    run.x += d.x;
    run.y += d.y;
    run.z += d.z;
    run.w += d.w;
  }
  reinterpret_cast<float4*>(p.S_out)[idx] = run;
}

// --------------------------------------------------------------------------
// Score tiles (row block rt, column block st <= rt) of a 64-token chunk, dealt
// to the 4 waves three/three/two/two.
__constant__ const int kTileRT[10] = {0, 1, 2, 3, 1, 2, 3, 2, 3, 3};
__constant__ const int kTileST[10] = {0, 1, 2, 3, 0, 1, 2, 0, 1, 0};

template <int C>
__global__ __launch_bounds__(kThreads) void la_chunk_output_kernel(PrefillParams p) {
  static_assert(C == 64, "tile schedule assumes 64-token chunks");
  __shared__ __attribute__((aligned(16))) uint8_t sQ[C * kD * 2];
  __shared__ __attribute__((aligned(16))) uint8_t sK[C * kD * 2];  // also output staging
  __shared__ __attribute__((aligned(16))) uint8_t sQl[C * kD * 2];  // lo parts of qh, kh
  __shared__ __attribute__((aligned(16))) uint8_t sKl[C * kD * 2];
  __shared__ __attribute__((aligned(16))) uint8_t sKT[kD * C * 2];
  __shared__ __attribute__((aligned(16))) uint8_t sVT[kD * C * 2];
  __shared__ __attribute__((aligned(16))) uint8_t sP[C * C * 2];
  __shared__ __attribute__((aligned(16))) uint8_t sG[C * kD * 2];
  __shared__ float2 sRot[2][kHalf];

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int n16 = lane & 15, g4 = lane >> 4;
  const int j = tid & 15, rg = tid >> 4;
  const Tile tl = decode_tile<C>(p);
  const int64_t rs = (int64_t)p.H * kD;

  float wq[8], wk[8];
  load_norm_weights(p.qw, j, wq);
  load_norm_weights(p.kw, j, wk);
  RopeLane L;
  rope_lane_init(p, rg, j, L);

  // prefix state of this segment
  f32x4 Sacc[8][2];
  {
    const float* src = p.ws + (((int64_t)tl.b * p.H + tl.h) * p.nseg + tl.seg) * kD * kD;
#pragma unroll
    for (int rtk = 0; rtk < 8; ++rtk)
#pragma unroll
      for (int ct = 0; ct < 2; ++ct)
#pragma unroll
        for (int r = 0; r < 4; ++r) Sacc[rtk][ct][r] = src[state_elem(rtk, ct, r, w, g4, n16)];
  }
  // score tiles above the diagonal are never written: zero them once
  for (int i = tid; i < C * C * 2 / 16; i += kThreads)
    reinterpret_cast<uint4*>(sP)[i] = make_uint4(0u, 0u, 0u, 0u);

  RawRows Qr, Kr, Vr, Gr;
  {
    const int nv = min(C, tl.t_end - tl.t_begin);
    const int64_t off = tl.base + (int64_t)tl.t_begin * rs;
    load_rows(p.q + off, rs, nv, rg, j, Qr);
    load_rows(p.k + off, rs, nv, rg, j, Kr);
    load_rows(p.v + off, rs, nv, rg, j, Vr);
    load_rows(p.g + off, rs, nv, rg, j, Gr);
  }
  if (tid < kHalf) sRot[0][tid] = rope_rotation(p.pos0 + tl.t_begin, p.freqs.theta[tid]);
  __syncthreads();

  for (int c = 0; c < tl.nch; ++c) {
    const int t0 = tl.t_begin + c * C;
    const int nv = min(C, tl.t_end - t0);

    // ---- prologue: RMSNorm + RoPE of q and k, staging of all four inputs
    {
      float2 E[4][4];
      chunk_rotations(sRot[c & 1], L, j, E);
      norm_rope_split(Qr, wq, p.eps, E, nv, rg, j, sQ, sQl);
      norm_rope_split(Kr, wk, p.eps, E, nv, rg, j, sK, sKl);
    }
    store_transposed<C>(sKT, Kr, rg, j);
    store_transposed<C>(sVT, Vr, rg, j);
    store_rows(sG, Gr, rg, j);
    if (c + 1 < tl.nch) {
      const int t1 = t0 + C;
      const int nv1 = min(C, tl.t_end - t1);
      const int64_t off = tl.base + (int64_t)t1 * rs;
      load_rows(p.q + off, rs, nv1, rg, j, Qr);
      load_rows(p.k + off, rs, nv1, rg, j, Kr);
      load_rows(p.v + off, rs, nv1, rg, j, Vr);
      load_rows(p.g + off, rs, nv1, rg, j, Gr);
      if (tid < kHalf) sRot[(c + 1) & 1][tid] = rope_rotation(p.pos0 + t1, p.freqs.theta[tid]);
    }
    __syncthreads();

    // ---- masked scores, computed transposed: P^T = Kh Qh^T (lane holds 4
    // consecutive keys s of one query t) from the hi/lo split of qh and kh,
    // then stored as P[t][s] in bf16
    for (int idx = w; idx < 10; idx += 4) {
      const int rt = kTileRT[idx], st = kTileST[idx];
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < kD / 32; ++ks) {
        const int ka = row_off(16 * st + n16, 32 * ks + 8 * g4);
        const int qa = row_off(16 * rt + n16, 32 * ks + 8 * g4);
        const bf16x8 kh = as_bf16x8(lds_ld<uint4>(sK, ka));
        const bf16x8 kl = as_bf16x8(lds_ld<uint4>(sKl, ka));
        const bf16x8 qh = as_bf16x8(lds_ld<uint4>(sQ, qa));
        const bf16x8 ql = as_bf16x8(lds_ld<uint4>(sQl, qa));
        acc = mma(kl, qh, acc);
        acc = mma(kh, ql, acc);
        acc = mma(kh, qh, acc);
      }
      if (st == rt) {
#pragma unroll
        for (int r = 0; r < 4; ++r)
          if (4 * g4 + r > n16) acc[r] = 0.f;
      }
      lds_st<uint2>(sP, score_off<C>(16 * rt + n16, 16 * st + 4 * g4),
                    make_uint2(pack2(acc[0], acc[1]), pack2(acc[2], acc[3])));
    }

    // ---- inter-chunk term Qh S_pre (S_pre in bf16, key dims permuted)
    f32x4 Oacc[4][2];
#pragma unroll
    for (int rt = 0; rt < 4; ++rt) Oacc[rt][0] = Oacc[rt][1] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kk = 0; kk < kD / 32; ++kk) {
      const bf16x8 b0 = pack8(Sacc[2 * kk][0], Sacc[2 * kk + 1][0]);
      const bf16x8 b1 = pack8(Sacc[2 * kk][1], Sacc[2 * kk + 1][1]);
#pragma unroll
      for (int rt = 0; rt < 4; ++rt) {
        const int t = 16 * rt + n16;
        const bf16x8 a = as_bf16x8(lds_ld<uint2>(sQ, row_off(t, 32 * kk + 4 * g4)),
                                   lds_ld<uint2>(sQ, row_off(t, 32 * kk + 16 + 4 * g4)));
        Oacc[rt][0] = mma(a, b0, Oacc[rt][0]);
        Oacc[rt][1] = mma(a, b1, Oacc[rt][1]);
      }
    }
    __syncthreads();  // scores complete

    // ---- intra-chunk term P V
#pragma unroll
    for (int rt = 0; rt < 4; ++rt) {
#pragma unroll
      for (int kk = 0; kk <= rt / 2; ++kk) {
        const bf16x8 a = as_bf16x8(lds_ld<uint4>(sP, score_off<C>(16 * rt + n16, 32 * kk + 8 * g4)));
        const bf16x8 b0 = as_bf16x8(lds_ld<uint4>(sVT, col_off<C>(32 * w + n16, 32 * kk + 8 * g4)));
        const bf16x8 b1 = as_bf16x8(lds_ld<uint4>(sVT, col_off<C>(32 * w + 16 + n16, 32 * kk + 8 * g4)));
        Oacc[rt][0] = mma(a, b0, Oacc[rt][0]);
        Oacc[rt][1] = mma(a, b1, Oacc[rt][1]);
      }
    }

    // ---- state carry S_pre += Kh^T V
    accumulate_state<C>(Sacc, sKT, sVT, w, g4, n16);

    // ---- gate epilogue into the output staging tile (reuses sK)
#pragma unroll
    for (int rt = 0; rt < 4; ++rt)
#pragma unroll
      for (int ct = 0; ct < 2; ++ct)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int t = 16 * rt + 4 * g4 + r, d = 32 * w + 16 * ct + n16;
          const float gl = bf2f(lds_ld<uint16_t>(sG, row_off(t, d)));
          lds_st<uint16_t>(sK, row_off(t, d), (uint16_t)f2bf(Oacc[rt][ct][r] * sigmoidf_(gl)));
        }
    __syncthreads();
#pragma unroll
    for (int pass = 0; pass < C / 16; ++pass) {
      const int row = (tid >> 4) + 16 * pass, blk = tid & 15;
      if (row < nv) {
        const uint4 val = lds_ld<uint4>(sK, row_off(row, 8 * blk));
        *reinterpret_cast<uint4*>(p.o + tl.base + (int64_t)(t0 + row) * rs + 8 * blk) = val;
      }
    }
    __syncthreads();
  }
}

}  // namespace

hipError_t launch_prefill(const PrefillParams& p, const PrefillPlan& plan, hipStream_t stream,
                          hipEvent_t const* events) {
  const dim3 grid((unsigned)((int64_t)p.B * p.H * plan.nseg));
  const int64_t scan_threads = (int64_t)p.B * p.H * kD * kD / 4;
  hipError_t err = hipSuccess;
  auto mark = [&](int i) {
    if (events && err == hipSuccess) err = hipEventRecord(events[i], stream);
  };
  mark(0);
  hipLaunchKernelGGL(la_chunk_state_kernel<64>, grid, dim3(kThreads), 0, stream, p);
  mark(1);
  hipLaunchKernelGGL(la_state_scan_kernel, dim3((unsigned)((scan_threads + 255) / 256)), dim3(256), 0,
                     stream, p);
  mark(2);
  hipLaunchKernelGGL(la_chunk_output_kernel<64>, grid, dim3(kThreads), 0, stream, p);
  mark(3);
  const hipError_t launch = hipGetLastError();
  return err != hipSuccess ? err : launch;
}

}  // namespace la
