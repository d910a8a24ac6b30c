// Chunk tiles shared by the prefill and backward kernels: LDS tile layout, the
// staging of rows (QK-RMSNorm + RoPE prologue), the work decomposition into
// (b, h, segment) workgroups and the MFMA operand forms.
//
// MFMA layout (v_mfma_f32_16x16x32_bf16; lane l = 16 g + n16 supplies
// A[n16][8g + e], B[8g + e][n16] and holds D[4g + r][n16]).  Token contractions
// read "transposed" operands straight from row-major tiles with
// ds_read_b64_tr_b16; key-dim contractions against a state held in accumulators
// take the key dims in the order pi(8g + e) = 32kk + 4g + 16(e/4) + e%4.
#pragma once

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

// [64][128] bf16 row tile with 272-byte rows (16-byte aligned, linear offsets).
// Measured on gfx950 at this stride: staging writes (16 lanes per row) and
// transposed reads are near conflict-free (0 and 2 conflict cycles per
// instruction), 8-byte stores of an MFMA result (16 rows x 4 lane groups) cost 8,
// and 8- and 16-byte reads in that row pattern take about twice and 1.5 times
// their conflict-free time.  No stride suits every access: 16-byte row reads are
// conflict-free only at strides of 32 mod 64 bytes (288), where the 8-byte row
// accesses conflict heavily, and 280 serves the 8-byte accesses but breaks the
// 16-byte alignment.
__device__ __forceinline__ int tile_off(int t, int d) { return t * kRowBytes + 2 * d; }

// Row-tile layouts for the staging helpers.  TileNat is the tile above.  TilePi
// has 288-byte rows and stores each 32-dim block in the key order pi: dim
// 32kk + 16h + 4g + r sits at position 32kk + 8g + 4h + r, so the 8 dims a lane
// takes in order pi are 16 contiguous bytes (one ds_read_b128, which is
// conflict-free at this row stride), while any 4 consecutive dims starting at a
// multiple of 4 stay contiguous (8-byte stores and transposed reads).
struct TileNat {
  static constexpr int kRow = kRowBytes;
  __device__ static __forceinline__ int off(int t, int d) { return tile_off(t, d); }
};
struct TilePi {
  static constexpr int kRow = kD * 2 + 32;
  __device__ static __forceinline__ int pos(int d) {
    return (d & ~31) | ((d & 12) << 1) | ((d & 16) >> 2) | (d & 3);
  }
  __device__ static __forceinline__ int off(int t, int d) { return t * kRow + 2 * pos(d); }
};

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

template <int M, int kStep, class Lay = TileNat>
__device__ __forceinline__ void store_rows_masked(uint8_t* tile, const Rows<M>& R, int nvalid, int rg,
                                                  int j) {
#pragma unroll
  for (int m = 0; m < M; ++m) {
    const bool ok = rg + kStep * m < nvalid;
    lds_st<uint2>(tile, Lay::off(rg + kStep * m, 4 * j), ok ? R.lo[m] : make_uint2(0u, 0u));
    lds_st<uint2>(tile, Lay::off(rg + kStep * m, kHalf + 4 * j), ok ? R.hi[m] : make_uint2(0u, 0u));
  }
}

// sigmoid of the gate logits, staged as bf16 (round to nearest even: relative
// error at most 2^-9, and bf16 keeps fp32's exponent range, so gates down to the
// fp32 underflow of the sigmoid keep their relative precision).
template <int M, int kStep>
__device__ __forceinline__ void sigmoid_stage(uint8_t* tile, const Rows<M>& R, int rg, int j) {
#pragma unroll
  for (int m = 0; m < M; ++m) {
    const uint2 a = R.lo[m], b = R.hi[m];
    const uint2 lo = make_uint2(pack2(sigmoidf_(bf2f_lo(a.x)), sigmoidf_(bf2f_hi(a.x))),
                                pack2(sigmoidf_(bf2f_lo(a.y)), sigmoidf_(bf2f_hi(a.y))));
    const uint2 hi = make_uint2(pack2(sigmoidf_(bf2f_lo(b.x)), sigmoidf_(bf2f_hi(b.x))),
                                pack2(sigmoidf_(bf2f_lo(b.y)), sigmoidf_(bf2f_hi(b.y))));
    lds_st<uint2>(tile, tile_off(rg + kStep * m, 4 * j), lo);
    lds_st<uint2>(tile, tile_off(rg + kStep * m, kHalf + 4 * j), hi);
  }
}

// du = do * sigmoid(g) of rows rg + kStep m as bf16 into `tile` (rows at or past
// nvalid zeroed); with `lo`, also lo = bf16(du - bf16(du)) for exact chunks.
template <int M, int kStep, class Lay = TileNat>
__device__ __forceinline__ void du_stage(uint8_t* tile, uint8_t* lo, const Rows<M>& D, const Rows<M>& G,
                                         int nvalid, int rg, int j) {
#pragma unroll
  for (int m = 0; m < M; ++m) {
    const int t = rg + kStep * m;
    const bool ok = t < nvalid;
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      const uint2 d = half ? D.hi[m] : D.lo[m];
      const uint2 g = half ? G.hi[m] : G.lo[m];
      const float u[4] = {bf2f_lo(d.x) * sigmoidf_(bf2f_lo(g.x)), bf2f_hi(d.x) * sigmoidf_(bf2f_hi(g.x)),
                          bf2f_lo(d.y) * sigmoidf_(bf2f_lo(g.y)), bf2f_hi(d.y) * sigmoidf_(bf2f_hi(g.y))};
      const uint2 hiw = ok ? make_uint2(pack2(u[0], u[1]), pack2(u[2], u[3])) : make_uint2(0u, 0u);
      const int off = Lay::off(t, half * kHalf + 4 * j);
      lds_st<uint2>(tile, off, hiw);
      if (lo != nullptr) {
        const uint2 low = ok ? make_uint2(pack2(u[0] - bf2f_lo(hiw.x), u[1] - bf2f_hi(hiw.x)),
                                          pack2(u[2] - bf2f_lo(hiw.y), u[3] - bf2f_hi(hiw.y)))
                             : make_uint2(0u, 0u);
        lds_st<uint2>(lo, off, low);
      }
    }
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
template <bool kWeights, int kLoRows = kExactRows, class Lay = TileNat>
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
  lds_st<uint2>(tile, Lay::off(t, 4 * j), hlo);
  lds_st<uint2>(tile, Lay::off(t, kHalf + 4 * j), hhi);
  if (lo != nullptr && t < kLoRows) {
    const uint2 llo = make_uint2(pack2(y[0] - bf2f_lo(hlo.x), y[1] - bf2f_hi(hlo.x)),
                                 pack2(y[2] - bf2f_lo(hlo.y), y[3] - bf2f_hi(hlo.y)));
    const uint2 lhi = make_uint2(pack2(y[4] - bf2f_lo(hhi.x), y[5] - bf2f_hi(hhi.x)),
                                 pack2(y[6] - bf2f_lo(hhi.y), y[7] - bf2f_hi(hhi.y)));
    lds_st<uint2>(lo, Lay::off(t, 4 * j), llo);
    lds_st<uint2>(lo, Lay::off(t, kHalf + 4 * j), lhi);
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

// One tensor, with the first row's rotations E already formed (advanced in place);
// `lo` receives the lo parts of rows below kLoRows.
template <bool kWeights, int M, int kStep, int kLoRows = kExactRows, class Lay = TileNat>
__device__ __forceinline__ void norm_rope_rows(const Rows<M>& R, const float (&w)[8], float eps, float2 (&E)[4],
                                               const Rope& L, int rg, int j, uint8_t* tile, uint8_t* lo) {
#pragma unroll
  for (int m = 0; m < M; ++m) {
    if (m > 0) next_rotation(L, E);
    norm_rope_row<kWeights, kLoRows, Lay>(R.lo[m], R.hi[m], w, eps, E, rg + kStep * m, j, tile, lo);
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

// Whether the tile is the last segment of its sequence: its output workgroup
// carries the state to the sequence's end and writes S_out, so the state pass
// has no sum to form for it.
__device__ __forceinline__ bool last_segment(const PrefillParams& p, const Tile& tl) {
  return p.segs != nullptr ? tl.seg == p.seqs[tl.b].nseg - 1 : tl.seg == p.nseg - 1;
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

// Consumer operand in key order pi: lane n16 gets X[row][32kk + 4g + 16(e/4) + e%4].
__device__ __forceinline__ bf16x8 pi_operand(const uint8_t* tile, int row, int kk, int g4) {
  return as_bf16x8(lds_ld<uint2>(tile, tile_off(row, 32 * kk + 4 * g4)),
                   lds_ld<uint2>(tile, tile_off(row, 32 * kk + 16 + 4 * g4)));
}

// The 10 causal 16 x 16 score tiles (row block rt, key block st <= rt) of a chunk,
// dealt to waves in this order: tile idx has rt = (kTileRT >> 2 idx) & 3 and
// st = (kTileST >> 2 idx) & 3, i.e. (0,0) (1,1) (2,2) (3,3) (1,0) (2,1) (3,2)
// (2,0) (3,1) (3,0).
constexpr uint32_t kTileRT = 0xfb9e4;
constexpr uint32_t kTileST = 0x124e4;

constexpr int kScoreRowBytes = kC * 2 + 16;  // [64][64] bf16 score tile, padded rows

__device__ __forceinline__ int score_off(int t, int s) { return t * kScoreRowBytes + 2 * s; }

// ---- operands in natural token order and from TilePi tiles

// Row operand in key order pi from a TilePi tile: lane (g, n16) gets dims
// pi(8g + e) of row t, which are 16 contiguous bytes.
__device__ __forceinline__ bf16x8 pi_row(const uint8_t* tile, int t, int kk, int g4) {
  return as_bf16x8(lds_ld<uint4>(tile, t * TilePi::kRow + 2 * (32 * kk + 8 * g4)));
}

// Column operand with tokens in natural order: lane n16 gets X[32kk + 8g + e][c0 + n16]
// (two transposed reads of 4 rows each).
template <class Lay>
__device__ __forceinline__ bf16x8 col_nat(const uint8_t* tile, int kk, int c0, int g4, int n16) {
  const int t0 = 32 * kk + 8 * g4 + (n16 >> 2), c = c0 + 4 * (n16 & 3);
  return as_bf16x8(lds_tr(tile, Lay::off(t0, c)), lds_tr(tile, Lay::off(t0 + 4, c)));
}

// Score row operand, tokens in natural order: lane n16 gets P[t][32kk + 8g + e].
__device__ __forceinline__ bf16x8 score_row(const uint8_t* sP, int t, int kk, int g4) {
  return as_bf16x8(lds_ld<uint4>(sP, score_off(t, 32 * kk + 8 * g4)));
}

// ---- operands with tokens in interleaved order
//
// A contraction over the chunk's tokens may take them in any order that both of
// its operands share.  For transposed reads the interleaved order is cheaper: lane
// group g's K elements e = 0..7 are tokens 8g + 2(e % 4) + e / 4 of the 32-token
// block, so each of the two transposed reads takes rows 8g, 8g+2, 8g+4, 8g+6 (or the
// odd ones).  Rows two apart fall on different banks both in the 288-byte TilePi
// tiles (whose 4-dim pieces lie 16 bytes apart) and in the 144-byte score tiles,
// while four consecutive rows collide.  gfx950's conflict counter gives, per
// transposed read, 6 cycles (natural order) against 2 (interleaved) on a TilePi
// tile and 2 against 0 on a score tile.

// Column operand, tokens interleaved: lane n16 gets X[32kk + 8g + 2(e%4) + e/4][c0 + n16].
template <class Lay>
__device__ __forceinline__ bf16x8 col_il(const uint8_t* tile, int kk, int c0, int g4, int n16) {
  const int t0 = 32 * kk + 8 * g4 + 2 * (n16 >> 2), c = c0 + 4 * (n16 & 3);
  return as_bf16x8(lds_tr(tile, Lay::off(t0, c)), lds_tr(tile, Lay::off(t0 + 1, c)));
}

// Score column operand, tokens interleaved: lane n16 gets P[32kk + 8g + 2(e%4) + e/4][s0 + n16].
__device__ __forceinline__ bf16x8 score_col_il(const uint8_t* sP, int kk, int s0, int g4, int n16) {
  const int t0 = 32 * kk + 8 * g4 + 2 * (n16 >> 2), c = s0 + 4 * (n16 & 3);
  return as_bf16x8(lds_tr(sP, score_off(t0, c)), lds_tr(sP, score_off(t0 + 1, c)));
}

// acc[rtk] (rows 16 rtk .. + 16 of X = A^T B, this wave's 16 columns) += over one
// chunk, A a TilePi tile whose 128 columns are the rows of X, B the chunk's column
// operand with tokens interleaved (col_il).
__device__ __forceinline__ void accumulate_il(f32x4 (&acc)[8], const uint8_t* A, const bf16x8 (&Bop)[2],
                                              int g4, int n16) {
#pragma unroll
  for (int kk = 0; kk < kC / 32; ++kk) {
    const int t0 = 32 * kk + 8 * g4 + 2 * (n16 >> 2);
#pragma unroll
    for (int rtk = 0; rtk < 8; ++rtk) {
      const int c = 16 * rtk + 4 * (n16 & 3);
      const bf16x8 a = as_bf16x8(lds_tr(A, TilePi::off(t0, c)), lds_tr(A, TilePi::off(t0 + 1, c)));
      acc[rtk] = mma(a, Bop[kk], acc[rtk]);
    }
  }
}

}  // namespace
}  // namespace la
