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
//      segment's prefix state and walks the chunks: QK-RMSNorm + RoPE prologue
//      into LDS, masked scores, O^T = S^T Qh^T + V^T P^T, sigmoid gate, coalesced
//      bf16 store, then S += Kh^T V.
//
// Workgroup: 512 threads = 8 waves (two per SIMD).  Wave w owns value columns
// [16w, 16w + 16) of S and of the chunk output.  S stays in MFMA accumulators:
// an accumulator tile pair is the A operand of S^T Qh^T directly, with the key
// dims of the contraction taken in the order pi(8g + e) = 32kk + 4g + 16(e/4) +
// e%4 (lane group g = lane / 16, operand element e), and Qh read in that order.
// The token contractions (Kh^T V and V^T P^T) use the same order over tokens, and
// their "transposed" operands come straight from the row-major tiles through
// ds_read_b64_tr_b16, so no tile is ever written transposed.
#include "la_device.hpp"
#include "la_internal.hpp"

namespace la {
namespace {

constexpr int kC = 64;      // tokens per chunk
constexpr int kWaves = 8;
constexpr int kThreads = 64 * kWaves;
constexpr int kTileBytes = kC * kD * 2;  // one [64][128] bf16 tile
constexpr int kExactRows = 16;           // rows whose scores use the hi/lo split

typedef short bf16x4 __attribute__((ext_vector_type(4)));

// [64][128] bf16 row tile, 256-byte rows; the 16-byte block index is XORed with
// t & 15, which spreads every access pattern below over all banks.
__device__ __forceinline__ int tile_off(int t, int d) {
  return t * (kD * 2) + ((((d >> 3) ^ (t & 15))) << 4) + ((d & 7) << 1);
}
// [64][64] bf16 score tile, 128-byte rows; block index XORed with (t >> 1) & 7.
__device__ __forceinline__ int score_off(int t, int s) {
  return t * (kC * 2) + ((((s >> 3) ^ ((t >> 1) & 7))) << 4) + ((s & 7) << 1);
}

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

// Staging coordinates: thread (rg = tid / 16, j = tid % 16) holds rows rg and
// rg + 32 of a chunk, dims {4j..4j+3} U {64+4j..64+4j+3}: each RoPE pair (i,
// i + 64) sits in one thread, and 16 lanes cover a row.
struct Rows {
  uint2 lo[2];  // dims 4j..4j+3, four bf16
  uint2 hi[2];  // dims 64+4j..64+4j+3
};

// Unmasked, branch-free loads: rows at or beyond nvalid (>= 1) re-read the last
// valid row, keeping every address inside the tensor.  Such rows of q, k and the
// gate only reach masked scores and unstored outputs; v's are zeroed when staged.
__device__ __forceinline__ void load_rows(const uint16_t* __restrict__ base, int64_t rs, int nvalid,
                                          int rg, int j, Rows& R) {
#pragma unroll
  for (int m = 0; m < 2; ++m) {
    const uint16_t* src = base + (int64_t)min(rg + 32 * m, nvalid - 1) * rs;
    R.lo[m] = *reinterpret_cast<const uint2*>(src + 4 * j);
    R.hi[m] = *reinterpret_cast<const uint2*>(src + kHalf + 4 * j);
  }
}

__device__ __forceinline__ void store_rows(uint8_t* tile, const Rows& R, int rg, int j) {
#pragma unroll
  for (int m = 0; m < 2; ++m) {
    lds_st<uint2>(tile, tile_off(rg + 32 * m, 4 * j), R.lo[m]);
    lds_st<uint2>(tile, tile_off(rg + 32 * m, kHalf + 4 * j), R.hi[m]);
  }
}

__device__ __forceinline__ void store_rows_masked(uint8_t* tile, const Rows& R, int nvalid, int rg,
                                                  int j) {
#pragma unroll
  for (int m = 0; m < 2; ++m) {
    const bool ok = rg + 32 * m < nvalid;
    lds_st<uint2>(tile, tile_off(rg + 32 * m, 4 * j), ok ? R.lo[m] : make_uint2(0u, 0u));
    lds_st<uint2>(tile, tile_off(rg + 32 * m, kHalf + 4 * j), ok ? R.hi[m] : make_uint2(0u, 0u));
  }
}

// RoPE per thread: A[e] = e^{i rg theta}, Z[e] = e^{i 32 theta} for the thread's
// frequencies 4j+e; row rg + 32m of a chunk at position p0 is rotated by
// base(p0) * A * Z^m.  base_rev is the frequency of pair tid (tid < 64), for the
// per-chunk base rotation, kept in a register so the loop loads nothing for it.
struct Rope {
  float2 A[4];
  float2 Z[4];
  double base_rev;
};

__device__ __forceinline__ void rope_init(const PrefillParams& p, int tid, int rg, int j, Rope& L) {
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const double rv = p.freqs.rev[4 * j + e];
    L.A[e] = rope_rotation(rg, rv);
    L.Z[e] = rope_rotation(32, rv);
  }
  L.base_rev = p.freqs.rev[tid & (kHalf - 1)];
}

// QK-normalization (RMSNorm over the 128 dims of a row, weights w) followed by
// rotate-half RoPE, in fp32; the bf16 result goes to `tile`.  With `lo` set, rows
// below kExactRows also store lo = bf16(y - bf16(y)) into `lo`, for the scores
// of the first rows of a call.
template <bool kWeights>
__device__ __forceinline__ void norm_rope_stage(const Rows& R, const float (&w)[8], float eps,
                                                const float2* sRot, const Rope& L, int rg, int j,
                                                uint8_t* tile, uint8_t* lo) {
  float2 E[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) E[e] = cmul(sRot[4 * j + e], L.A[e]);
#pragma unroll
  for (int m = 0; m < 2; ++m) {
    if (m == 1) {
#pragma unroll
      for (int e = 0; e < 4; ++e) E[e] = cmul(E[e], L.Z[e]);
    }
    float x[8] = {bf2f_lo(R.lo[m].x), bf2f_hi(R.lo[m].x), bf2f_lo(R.lo[m].y), bf2f_hi(R.lo[m].y),
                  bf2f_lo(R.hi[m].x), bf2f_hi(R.hi[m].x), bf2f_lo(R.hi[m].y), bf2f_hi(R.hi[m].y)};
    float ss = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) ss = fmaf(x[e], x[e], ss);
    const float inv = rsqrt_(row16_sum(ss) * (1.0f / kD) + eps);
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
    const int t = rg + 32 * m;
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

__device__ __forceinline__ Tile decode_tile(const PrefillParams& p) {
  Tile tl;
  int bid = blockIdx.x;
  tl.h = bid % p.H;
  bid /= p.H;
  tl.seg = bid % p.nseg;
  tl.b = bid / p.nseg;
  tl.t_begin = tl.seg * p.cps * kC;
  tl.t_end = min(p.T, tl.t_begin + p.cps * kC);
  tl.nch = (tl.t_end - tl.t_begin + kC - 1) / kC;
  tl.base = ((int64_t)tl.b * p.T * p.H + tl.h) * kD;
  return tl;
}

// S accumulator tile rtk of wave w: lane (g, n16) element r is
// S[16 rtk + 4 g + r][16 w + n16].
__device__ __forceinline__ int64_t state_elem(int rtk, int r, int w, int g4, int n16) {
  return (int64_t)(16 * rtk + 4 * g4 + r) * kD + 16 * w + n16;
}

// Token-contraction operand of V: lane n16 gets V[32kk + 4g + 16(e/4) + e%4][16w + n16].
__device__ __forceinline__ bf16x8 v_operand(const uint8_t* sV, int kk, int w, int g4, int n16) {
  const int t0 = 32 * kk + 4 * g4 + (n16 >> 2), c = 16 * w + 4 * (n16 & 3);
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
  rope_init(p, tid, rg, j, L);

  f32x4 Sacc[8];
#pragma unroll
  for (int a = 0; a < 8; ++a) Sacc[a] = f32x4{0.f, 0.f, 0.f, 0.f};

  Rows Kr, Vr;
  {
    const int nv = min(kC, tl.t_end - tl.t_begin);
    load_rows(p.k + tl.base + (int64_t)tl.t_begin * rs, rs, nv, rg, j, Kr);
    load_rows(p.v + tl.base + (int64_t)tl.t_begin * rs, rs, nv, rg, j, Vr);
  }
  if (tid < kHalf) sRot[0][tid] = rope_rotation(p.pos0 + tl.t_begin, L.base_rev);
  __syncthreads();

  for (int c = 0; c < tl.nch; ++c) {
    const int t0 = tl.t_begin + c * kC;
    const int nv = min(kC, tl.t_end - t0);
    uint8_t* bK = sK[c & 1];
    uint8_t* bV = sV[c & 1];
    norm_rope_stage<kWeights>(Kr, wk, p.eps, sRot[c & 1], L, rg, j, bK, nullptr);
    store_rows_masked(bV, Vr, nv, rg, j);
    if (c + 1 < tl.nch) {
      const int t1 = t0 + kC;
      const int nv1 = min(kC, tl.t_end - t1);
      load_rows(p.k + tl.base + (int64_t)t1 * rs, rs, nv1, rg, j, Kr);
      load_rows(p.v + tl.base + (int64_t)t1 * rs, rs, nv1, rg, j, Vr);
      if (tid < kHalf) sRot[(c + 1) & 1][tid] = rope_rotation(p.pos0 + t1, L.base_rev);
    }
    __syncthreads();
    bf16x8 Vop[2];
    Vop[0] = v_operand(bV, 0, w, g4, n16);
    Vop[1] = v_operand(bV, 1, w, g4, n16);
    accumulate_state(Sacc, bK, Vop, g4, n16);
  }

  float* dst = p.ws + (((int64_t)tl.b * p.H + tl.h) * p.nseg + tl.seg) * kD * kD;
#pragma unroll
  for (int rtk = 0; rtk < 8; ++rtk)
#pragma unroll
    for (int r = 0; r < 4; ++r) dst[state_elem(rtk, r, w, g4, n16)] = Sacc[rtk][r];
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
// Score tiles (row block rt, column block st <= rt) of a chunk, dealt to the 8
// waves (waves 0 and 1 take two): tile idx has rt = (kTileRT >> 2 idx) & 3 and
// st = (kTileST >> 2 idx) & 3 for the order (0,0) (1,1) (2,2) (3,3) (1,0) (2,1)
// (3,2) (2,0) (3,1) (3,0).  Packed in immediates so no table is loaded.
constexpr uint32_t kTileRT = 0xfb9e4;
constexpr uint32_t kTileST = 0x124e4;

template <bool kWeights>
__global__ __launch_bounds__(kThreads) void la_chunk_output_kernel(PrefillParams p) {
  __shared__ __attribute__((aligned(16))) uint8_t sQ[kTileBytes];
  __shared__ __attribute__((aligned(16))) uint8_t sK[kTileBytes];
  __shared__ __attribute__((aligned(16))) uint8_t sV[kTileBytes];
  __shared__ __attribute__((aligned(16))) uint8_t sG[kTileBytes];
  __shared__ __attribute__((aligned(16))) uint8_t sO[kTileBytes];
  __shared__ __attribute__((aligned(16))) uint8_t sP[kC * kC * 2];
  __shared__ __attribute__((aligned(16))) uint8_t sQl[kExactRows * kD * 2];
  __shared__ __attribute__((aligned(16))) uint8_t sKl[kExactRows * kD * 2];
  __shared__ float2 sRot[2][kHalf];

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int n16 = lane & 15, g4 = lane >> 4;
  const int j = tid & 15, rg = tid >> 4;
  const Tile tl = decode_tile(p);
  const int64_t rs = (int64_t)p.H * kD;

  float wq[8], wk[8];
  load_norm_weights(p.qw, j, wq);
  load_norm_weights(p.kw, j, wk);
  Rope L;
  rope_init(p, tid, rg, j, L);

  // prefix state of this segment
  f32x4 Sacc[8];
  {
    const float* src = p.ws + (((int64_t)tl.b * p.H + tl.h) * p.nseg + tl.seg) * kD * kD;
#pragma unroll
    for (int rtk = 0; rtk < 8; ++rtk)
#pragma unroll
      for (int r = 0; r < 4; ++r) Sacc[rtk][r] = src[state_elem(rtk, r, w, g4, n16)];
  }
  // score tiles above the diagonal are never written: zero them once
  for (int i = tid; i < kC * kC * 2 / 16; i += kThreads)
    reinterpret_cast<uint4*>(sP)[i] = make_uint4(0u, 0u, 0u, 0u);

  Rows Qr, Kr, Vr, Gr;
  {
    const int nv = min(kC, tl.t_end - tl.t_begin);
    const int64_t off = tl.base + (int64_t)tl.t_begin * rs;
    load_rows(p.q + off, rs, nv, rg, j, Qr);
    load_rows(p.k + off, rs, nv, rg, j, Kr);
    load_rows(p.v + off, rs, nv, rg, j, Vr);
    load_rows(p.g + off, rs, nv, rg, j, Gr);
  }
  if (tid < kHalf) sRot[0][tid] = rope_rotation(p.pos0 + tl.t_begin, L.base_rev);
  __syncthreads();

  for (int c = 0; c < tl.nch; ++c) {
    const int t0 = tl.t_begin + c * kC;
    const int nv = min(kC, tl.t_end - t0);
    // The first chunk of a call forms the scores of its first rows from a hi/lo
    // split of qh and kh: those rows sum only a few scores, so the bf16 rounding
    // of qh, kh would otherwise dominate their error.
    const bool exact = (tl.seg == 0 && c == 0);

    // ---- prologue: RMSNorm + RoPE of q and k, staging of all four inputs
    norm_rope_stage<kWeights>(Qr, wq, p.eps, sRot[c & 1], L, rg, j, sQ, exact ? sQl : nullptr);
    norm_rope_stage<kWeights>(Kr, wk, p.eps, sRot[c & 1], L, rg, j, sK, exact ? sKl : nullptr);
    store_rows_masked(sV, Vr, nv, rg, j);
    store_rows(sG, Gr, rg, j);
    if (c + 1 < tl.nch) {
      const int t1 = t0 + kC;
      const int nv1 = min(kC, tl.t_end - t1);
      const int64_t off = tl.base + (int64_t)t1 * rs;
      load_rows(p.q + off, rs, nv1, rg, j, Qr);
      load_rows(p.k + off, rs, nv1, rg, j, Kr);
      load_rows(p.v + off, rs, nv1, rg, j, Vr);
      load_rows(p.g + off, rs, nv1, rg, j, Gr);
      if (tid < kHalf) sRot[(c + 1) & 1][tid] = rope_rotation(p.pos0 + t1, L.base_rev);
    }
    __syncthreads();

    // ---- masked scores P^T = Kh Qh^T (lane holds 4 consecutive keys s of one
    // query t), stored as P[t][s] in bf16
    for (int idx = w; idx < 10; idx += kWaves) {
      const int rt = (kTileRT >> (2 * idx)) & 3, st = (kTileST >> (2 * idx)) & 3;
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < kD / 32; ++ks) {
        const int ka = tile_off(16 * st + n16, 32 * ks + 8 * g4);
        const int qa = tile_off(16 * rt + n16, 32 * ks + 8 * g4);
        const bf16x8 kh = as_bf16x8(lds_ld<uint4>(sK, ka));
        const bf16x8 qh = as_bf16x8(lds_ld<uint4>(sQ, qa));
        if (exact && idx == 0) {  // tile (0, 0): add the lo cross terms
          acc = mma(as_bf16x8(lds_ld<uint4>(sKl, ka)), qh, acc);
          acc = mma(kh, as_bf16x8(lds_ld<uint4>(sQl, qa)), acc);
        }
        acc = mma(kh, qh, acc);
      }
      if (st == rt) {
#pragma unroll
        for (int r = 0; r < 4; ++r)
          if (4 * g4 + r > n16) acc[r] = 0.f;
      }
      lds_st<uint2>(sP, score_off(16 * rt + n16, 16 * st + 4 * g4),
                    make_uint2(pack2(acc[0], acc[1]), pack2(acc[2], acc[3])));
    }

    // ---- inter-chunk term O^T = S_pre^T Qh^T (S_pre in bf16, key dims in order pi)
    f32x4 Oacc[4];
#pragma unroll
    for (int rt = 0; rt < 4; ++rt) Oacc[rt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kk = 0; kk < kD / 32; ++kk) {
      const bf16x8 a = pack8(Sacc[2 * kk], Sacc[2 * kk + 1]);
#pragma unroll
      for (int rt = 0; rt < 4; ++rt) {
        const int t = 16 * rt + n16;
        const bf16x8 b = as_bf16x8(lds_ld<uint2>(sQ, tile_off(t, 32 * kk + 4 * g4)),
                                   lds_ld<uint2>(sQ, tile_off(t, 32 * kk + 16 + 4 * g4)));
        Oacc[rt] = mma(a, b, Oacc[rt]);
      }
    }
    __syncthreads();  // scores complete

    // ---- intra-chunk term O^T += V^T P^T (tokens in order pi)
    bf16x8 Vop[2];
    Vop[0] = v_operand(sV, 0, w, g4, n16);
    Vop[1] = v_operand(sV, 1, w, g4, n16);
#pragma unroll
    for (int rt = 0; rt < 4; ++rt) {
      const int t = 16 * rt + n16;
#pragma unroll
      for (int kk = 0; kk <= rt / 2; ++kk) {
        const bf16x8 b = as_bf16x8(lds_ld<uint2>(sP, score_off(t, 32 * kk + 4 * g4)),
                                   lds_ld<uint2>(sP, score_off(t, 32 * kk + 16 + 4 * g4)));
        Oacc[rt] = mma(Vop[kk], b, Oacc[rt]);
      }
    }

    // ---- state carry S_pre += Kh^T V
    accumulate_state(Sacc, sK, Vop, g4, n16);

    // ---- gate epilogue: lane holds o[t = 16 rt + n16][16 w + 4 g .. + 3]
#pragma unroll
    for (int rt = 0; rt < 4; ++rt) {
      const int off = tile_off(16 * rt + n16, 16 * w + 4 * g4);
      const uint2 gl = lds_ld<uint2>(sG, off);
      const float o0 = Oacc[rt][0] * sigmoidf_(bf2f_lo(gl.x));
      const float o1 = Oacc[rt][1] * sigmoidf_(bf2f_hi(gl.x));
      const float o2 = Oacc[rt][2] * sigmoidf_(bf2f_lo(gl.y));
      const float o3 = Oacc[rt][3] * sigmoidf_(bf2f_hi(gl.y));
      lds_st<uint2>(sO, off, make_uint2(pack2(o0, o1), pack2(o2, o3)));
    }
    __syncthreads();
#pragma unroll
    for (int pass = 0; pass < 2; ++pass) {
      const int row = (tid >> 4) + 32 * pass, blk = tid & 15;
      if (row < nv) {
        const uint4 val = lds_ld<uint4>(sO, tile_off(row, 8 * blk));
        *reinterpret_cast<uint4*>(p.o + tl.base + (int64_t)(t0 + row) * rs + 8 * blk) = val;
      }
    }
  }
}

}  // namespace

hipError_t launch_prefill(const PrefillParams& p, const PrefillPlan& plan, hipStream_t stream,
                          hipEvent_t const* events) {
  const dim3 grid((unsigned)((int64_t)p.B * p.H * plan.nseg));
  const int64_t scan_threads = (int64_t)p.B * p.H * kD * kD / 4;
  const bool weights = p.qw != nullptr || p.kw != nullptr;
  hipError_t err = hipSuccess;
  auto mark = [&](int i) {
    if (events && err == hipSuccess) err = hipEventRecord(events[i], stream);
  };
  mark(0);
  if (weights)
    hipLaunchKernelGGL(la_chunk_state_kernel<true>, grid, dim3(kThreads), 0, stream, p);
  else
    hipLaunchKernelGGL(la_chunk_state_kernel<false>, grid, dim3(kThreads), 0, stream, p);
  mark(1);
  hipLaunchKernelGGL(la_state_scan_kernel, dim3((unsigned)((scan_threads + 255) / 256)), dim3(256), 0,
                     stream, p);
  mark(2);
  if (weights)
    hipLaunchKernelGGL(la_chunk_output_kernel<true>, grid, dim3(kThreads), 0, stream, p);
  else
    hipLaunchKernelGGL(la_chunk_output_kernel<false>, grid, dim3(kThreads), 0, stream, p);
  mark(3);
  const hipError_t launch = hipGetLastError();
  return err != hipSuccess ? err : launch;
}

}  // namespace la
