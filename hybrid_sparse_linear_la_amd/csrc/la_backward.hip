// Backward of the chunked prefill on gfx950 (chunk 64).
//
// For a loss with gradients do (of o) and dS_out (of the final state), per (b, h),
// with du_t = do_t * sigmoid(g_t), u_t = qh_t S_t (the output before the gate),
// and G_s = dS_out + sum_{t >= s} qh_t du_t^T (the gradient of the state S_s):
//     dg  = do * u * sigmoid'(g)            dqh_t = du_t S_t^T
//     dkh_s = G_s v_s                       dv_s  = G_s^T kh_s,      dS_in = G_0,
// the reverse mode of S_t = S_{t-1} + k_t v_t^T and o_t = sigmoid(g_t) (q_t S_t)
// ("MiniCPM-SALA: Hybridizing Sparse and Linear Attention for Efficient
// Long-Context Modeling", 前置知识 > 线性注意力; output gate and QK-normalization
// from "創新Transformer！面壁基於稀疏-線性混合架構SALA訓練9B模型，端側跑通百萬上下文",
// 04 技術報告 > 02 模型架構 > (3) 線性注意力模塊).
//
// Chunked, for a chunk with state S (before it) and G (after it):
//     u   = (Qh Kh^T . M) V + Qh S
//     dQh = (dU V^T . M) Kh + dU S^T
//     dKh = (dU V^T . M)^T Qh + V G^T
//     dV  = (Qh Kh^T . M)^T dU + Kh G
// and across chunks S <- S + Kh^T V, G(before) = G(after) + Qh^T dU.
//
// la_backward_chunk_kernel: one 512-thread workgroup per (b, h, segment) walks
// its chunks forward from the segment's forward state S and gradient state G (at
// the segment's first token, from the suffix scan) and subtracts Qh^T dU from G
// chunk by chunk.  Wave w owns columns [16w, 16w + 16) of every output and of the
// S, G accumulators; S and G are also written to LDS as bf16 (transposed) so the
// S^T and G^T products can read any row.  dqh and dkh, rounded to bf16, go
// through the prologue backward (rotated back, then the RMSNorm Jacobian): inside
// this kernel for grids of up to 2048 workgroups, else in
// la_prologue_backward_kernel.  Chunks at the start and end of a sequence form their scores from a
// hi/lo split of qh, kh and du: rows there sum few scores, and the bf16 rounding
// of the operands would otherwise dominate their error.
#include "la_device.hpp"
#include "la_internal.hpp"
#include "la_tiles.hpp"

namespace la {
namespace {

constexpr int kBwdThreads = 512;

// Row loads that stay in L2: q, k, do and the gate are read again later in the
// same chunk (do and the gate by the outputs in another lane layout, q and k by the
// prologue backward), and with streaming loads those second reads went to the
// fabric (the chunk kernel moved 27.9 GB at 256K against 19.5 GB by design).  v is read
// once and keeps the streaming loads of load_rows.
template <int M, int kStep>
__device__ __forceinline__ void load_rows_cached(const uint16_t* __restrict__ base, int64_t rs, int nvalid, int rg,
                                                 int j, Rows<M>& R) {
#pragma unroll
  for (int m = 0; m < M; ++m) {
    const uint16_t* src = base + (int64_t)min(rg + kStep * m, nvalid - 1) * rs;
    R.lo[m] = *reinterpret_cast<const uint2*>(src + 4 * j);
    R.hi[m] = *reinterpret_cast<const uint2*>(src + kHalf + 4 * j);
  }
}

// The chunk's q, k, v and du tiles use the TilePi layout (288-byte rows, key
// dims stored in order pi); the S^T, G^T snapshots and the score tiles are
// row-major with natural columns.
constexpr int kPiTileBytes = kC * TilePi::kRow;

// The snapshot area ([128][128] bf16 S^T and G^T; later the chunk's dqh and dkh
// tiles) has 280-byte rows: the 8-byte stores of an MFMA result (16 rows x 4 lane
// groups) are conflict-free there, where 272-byte rows cost 8 conflict cycles per
// store (gfx950 counters).  With it the kernel's LDS is exactly 160 KiB.
constexpr int kSnapRow = kD * 2 + 24;
constexpr int kSnapBytes = kD * kSnapRow;
__device__ __forceinline__ int snap_off(int t, int d) { return t * kSnapRow + 2 * d; }

// Column operand of a snapshot in order pi over its rows: lane n16 gets
// X[32kk + 4g + 16(e/4) + e%4][c0 + n16].
__device__ __forceinline__ bf16x8 snap_col(const uint8_t* snap, int kk, int c0, int g4, int n16) {
  const int t0 = 32 * kk + 4 * g4 + (n16 >> 2), c = c0 + 4 * (n16 & 3);
  return as_bf16x8(lds_tr(snap, snap_off(t0, c)), lds_tr(snap, snap_off(t0 + 16, c)));
}

// The q and k norm weights (ones if absent) live in the 32 padding bytes of rows
// 0..31 of the q tile, which no tile access touches: weight i of tensor a at row
// (128a + i) / 8, byte 256 + 4 ((128a + i) % 8).
__device__ __forceinline__ int norm_weight_off(int a, int i) {
  const int f = kD * a + i;
  return (f >> 3) * TilePi::kRow + kD * 2 + 4 * (f & 7);
}

// Norm weights of dims 4j..4j+3 and 64+4j..64+4j+3 of tensor a (0: q, 1: k).
__device__ __forceinline__ void pad_norm_weights(const uint8_t* sQ, int a, int j, float (&out)[8]) {
  const float4 lo = lds_ld<float4>(sQ, norm_weight_off(a, 4 * j));
  const float4 hi = lds_ld<float4>(sQ, norm_weight_off(a, kHalf + 4 * j));
  out[0] = lo.x;
  out[1] = lo.y;
  out[2] = lo.z;
  out[3] = lo.w;
  out[4] = hi.x;
  out[5] = hi.y;
  out[6] = hi.z;
  out[7] = hi.w;
}

__device__ __forceinline__ bf16x8 negate(bf16x8 x) {
  uint4 u = __builtin_bit_cast(uint4, x);
  u.x ^= 0x80008000u;
  u.y ^= 0x80008000u;
  u.z ^= 0x80008000u;
  u.w ^= 0x80008000u;
  return __builtin_bit_cast(bf16x8, u);
}

__device__ __forceinline__ void store_bf16x4(uint16_t* dst, f32x4 x) {
  *reinterpret_cast<uint2*>(dst) = make_uint2(pack2(x[0], x[1]), pack2(x[2], x[3]));
}

// One row piece of the prologue backward.  x: the raw row's dims 4j..4j+3 and
// 64+4j..64+4j+3 (xl, xh), y: the gradient of the rotated normalized row at the
// same dims, w: the norm weights there, E: the row's rotations.  Rotating back
// gives dn, then through RMSNorm (n = w x / r):
//     dx_i = w_i dn_i / r - x_i (sum_j w_j x_j dn_j) / (D r^3),
// the sums over the row's 16 lanes.  Returns dx and, for the weight gradient
// (dw_i += dn_i x_i / r), dn and 1 / r.
__device__ __forceinline__ void prologue_back_row(uint2 xl, uint2 xh, uint2 yl, uint2 yh, const float (&w)[8],
                                                  const float2 (&E)[4], float eps, float (&dx)[8], float (&dn)[8],
                                                  float (&x)[8], float& inv) {
  const float xs[8] = {bf2f_lo(xl.x), bf2f_hi(xl.x), bf2f_lo(xl.y), bf2f_hi(xl.y),
                       bf2f_lo(xh.x), bf2f_hi(xh.x), bf2f_lo(xh.y), bf2f_hi(xh.y)};
  const float y[8] = {bf2f_lo(yl.x), bf2f_hi(yl.x), bf2f_lo(yl.y), bf2f_hi(yl.y),
                      bf2f_lo(yh.x), bf2f_hi(yh.x), bf2f_lo(yh.y), bf2f_hi(yh.y)};
  float ss = 0.f, dot = 0.f;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    dn[e] = y[e] * E[e].x + y[4 + e] * E[e].y;
    dn[4 + e] = y[4 + e] * E[e].x - y[e] * E[e].y;
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    x[e] = xs[e];
    ss += xs[e] * xs[e];
    dot += w[e] * xs[e] * dn[e];
  }
  ss = row16_sum(ss);
  dot = row16_sum(dot);
  inv = rsqrt_(ss * (1.0f / kD) + eps);
  const float k3 = dot * inv * inv * inv * (1.0f / kD);
#pragma unroll
  for (int e = 0; e < 8; ++e) dx[e] = w[e] * dn[e] * inv - xs[e] * k3;
}

__device__ __forceinline__ void store_row_pieces(uint16_t* dst, int j, const float (&v)[8]) {
  *reinterpret_cast<uint2*>(dst + 4 * j) = make_uint2(pack2(v[0], v[1]), pack2(v[2], v[3]));
  *reinterpret_cast<uint2*>(dst + kHalf + 4 * j) = make_uint2(pack2(v[4], v[5]), pack2(v[6], v[7]));
}

// The prologue backward of one chunk inside the chunk kernel: thread (rg, j) takes
// rows rg and rg + 32 (E: row rg's rotations); dqh, dkh come from LDS row tiles
// (the snapshot area's rows), the raw q, k rows X from memory (loaded by the caller).
// dw receives the thread's norm-weight gradient terms (its two rows summed).
template <bool kWeights>
__device__ __forceinline__ void prologue_back_rows(const PrefillParams& p, const BackwardParams& bp, int64_t base,
                                                   int nv, int64_t rs, int rg, int j, const Rope& L, float2 (&E)[4],
                                                   const uint8_t* sDq, const uint8_t* sDk, const uint8_t* sQ,
                                                   const Rows<2> (&X)[2], float (&dw)[2][8]) {
  float w[2][8];
#pragma unroll
  for (int a = 0; a < 2; ++a)
    if (kWeights) {
      pad_norm_weights(sQ, a, j, w[a]);
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) w[a][e] = 1.0f;
    }
#pragma unroll
  for (int m = 0; m < 2; ++m) {
    if (m > 0) next_rotation(L, E);
    const int t = rg + 32 * m;
#pragma unroll
    for (int a = 0; a < 2; ++a) {
      const uint8_t* Y = a ? sDk : sDq;
      float dx[8], dn[8], x[8], inv;
      prologue_back_row(X[a].lo[m], X[a].hi[m], lds_ld<uint2>(Y, snap_off(t, 4 * j)),
                        lds_ld<uint2>(Y, snap_off(t, kHalf + 4 * j)), w[a], E, p.eps, dx, dn, x, inv);
#pragma unroll
      for (int e = 0; e < 8; ++e) dw[a][e] = (m > 0 ? dw[a][e] : 0.f) + (t < nv ? dn[e] * x[e] * inv : 0.f);
      if (t < nv) store_row_pieces((a ? bp.dk : bp.dq) + base + (int64_t)t * rs, j, dx);
    }
  }
}

// Stores row blocks rt = 0..3 (row 16 rt + n16 of the chunk, columns col..col+3) of
// a bf16 output, rows at or past nv skipped.
__device__ __forceinline__ void store_rows4(uint16_t* out, const f32x4 (&acc)[4], int64_t base, int t0,
                                            int64_t rs, int col, int nv, int n16) {
#pragma unroll
  for (int rt = 0; rt < 4; ++rt)
    if (16 * rt + n16 < nv) store_bf16x4(out + base + (int64_t)(t0 + 16 * rt + n16) * rs + col, acc[rt]);
}

template <bool kWeights, bool kFuse>
__global__ __launch_bounds__(kBwdThreads) void la_backward_chunk_kernel(BackwardParams bp) {
  const PrefillParams& p = bp.f;
  __shared__ __attribute__((aligned(16))) uint8_t sQ[kPiTileBytes];
  __shared__ __attribute__((aligned(16))) uint8_t sK[kPiTileBytes];
  __shared__ __attribute__((aligned(16))) uint8_t sV[kPiTileBytes];
  __shared__ __attribute__((aligned(16))) uint8_t sU[kPiTileBytes];
  __shared__ __attribute__((aligned(16))) uint8_t sP[kC * kScoreRowBytes];
  __shared__ __attribute__((aligned(16))) uint8_t sdP[kC * kScoreRowBytes];
  // S^T and G^T snapshots; during the scores of an exact chunk the lo tiles of qh,
  // kh and du live here instead
  __shared__ __attribute__((aligned(16))) uint8_t sX[2 * kSnapBytes];
  uint8_t* const sST = sX;
  uint8_t* const sGT = sX + kSnapBytes;
  uint8_t* const sQl = sX;
  uint8_t* const sKl = sX + kPiTileBytes;
  uint8_t* const sUl = sX + 2 * kPiTileBytes;
  static_assert(3 * kPiTileBytes <= 2 * kSnapBytes, "lo tiles must fit the snapshot area");

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int n16 = lane & 15, g4 = lane >> 4;
  const int j = tid & 15, rg = tid >> 4;
  const Tile tl = decode_tile(p);
  const int64_t rs = (int64_t)p.H * kD;

  Rope L;
  rope_init<32>(p, tid, rg, j, L);
  double rev[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) rev[e] = p.freqs.rev[4 * j + e];

  // S (forward) and G (gradient) states at the segment's first token: columns [16w, 16w + 16)
  f32x4 Sacc[8], Gacc[8];
  {
    const float* gst = bp.wsg + (tl.state - p.ws);
#pragma unroll
    for (int rtk = 0; rtk < 8; ++rtk)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        Sacc[rtk][r] = tl.state[state_elem(rtk, r, w, g4, n16)];
        Gacc[rtk][r] = gst[state_elem(rtk, r, w, g4, n16)];
      }
  }
  if (tid < 2 * kD) {
    const float* nw = tid < kD ? p.qw : p.kw;
    lds_st<float>(sQ, norm_weight_off(tid / kD, tid % kD), nw ? nw[tid % kD] : 1.0f);
  }
  const bool wgrad = kFuse && (bp.dq_w != nullptr || bp.dk_w != nullptr);
  float dw_acc = 0.f;  // with wgrad: thread tid < 256 sums dw[tid / 128][tid % 128] over the chunks
  // score tiles above the diagonal are never written
  for (int i = tid; i < kC * kScoreRowBytes / 16; i += kBwdThreads) {
    reinterpret_cast<uint4*>(sP)[i] = make_uint4(0u, 0u, 0u, 0u);
    reinterpret_cast<uint4*>(sdP)[i] = make_uint4(0u, 0u, 0u, 0u);
  }
  __syncthreads();  // the norm weights in LDS before the first staging

  for (int c = 0; c < tl.nch; ++c) {
    const int t0 = tl.t_begin + c * kC;
    const int nv = min(kC, tl.t_end - t0);
    const bool exact = (tl.seg == 0 && c == 0) || t0 + 2 * kC > p.T;
    // ---- staging: qh, kh (prologue), v, du = do * sigmoid(g)
    {
      Rows<2> Qr, Kr, Vr, Dr, Gr;
      const int64_t off = tl.base + (int64_t)t0 * rs;
      load_rows_cached<2, 32>(p.q + off, rs, nv, rg, j, Qr);
      load_rows_cached<2, 32>(p.k + off, rs, nv, rg, j, Kr);
      load_rows<2, 32>(p.v + off, rs, nv, rg, j, Vr);
      load_rows_cached<2, 32>(p.dout + off, rs, nv, rg, j, Dr);
      load_rows_cached<2, 32>(p.g + off, rs, nv, rg, j, Gr);
      float2 E[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) E[e] = cmul(rope_rotation(tl.pos_base + t0, rev[e]), L.A[e]);
      float2 E2[4] = {E[0], E[1], E[2], E[3]};
      // norm weights are re-read each chunk (from LDS) rather than held in registers
      float wq[8], wk[8];
      if (kWeights) {
        pad_norm_weights(sQ, 0, j, wq);
        pad_norm_weights(sQ, 1, j, wk);
      }
      norm_rope_rows<kWeights, 2, 32, kC, TilePi>(Qr, wq, p.eps, E, L, rg, j, sQ, exact ? sQl : nullptr);
      norm_rope_rows<kWeights, 2, 32, kC, TilePi>(Kr, wk, p.eps, E2, L, rg, j, sK, exact ? sKl : nullptr);
      store_rows_masked<2, 32, TilePi>(sV, Vr, nv, rg, j);
      du_stage<2, 32, TilePi>(sU, exact ? sUl : nullptr, Dr, Gr, nv, rg, j);
    }
    __syncthreads();
    // do and g of this lane's output rows in the outputs' layout (rows past the chunk
    // clamped to its last row), loaded here so that their latency passes under the
    // scores (L2 hits: the staging loaded the same rows)
    uint2 dor[4], gr[4];
    {
      const int col = 16 * w + 4 * g4;
#pragma unroll
      for (int rt = 0; rt < 4; ++rt) {
        const int64_t crow = tl.base + (int64_t)(t0 + min(16 * rt + n16, nv - 1)) * rs + col;
        dor[rt] = *reinterpret_cast<const uint2*>(p.dout + crow);
        gr[rt] = *reinterpret_cast<const uint2*>(p.g + crow);
      }
    }
    // ---- scores P = Qh Kh^T and dP = dU V^T (masked to s <= t), 20 tiles over 8 waves
    for (int idx = w; idx < 20; idx += 8) {
      const bool grad = idx >= 10;
      const int ti = grad ? idx - 10 : idx;
      const int rt = (kTileRT >> (2 * ti)) & 3, st = (kTileST >> (2 * ti)) & 3;
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < kD / 32; ++ks) {
        // any order of the 128 dims serves the dot products: both operands read the
        // same 16 stored bytes
        const int ka = (16 * st + n16) * TilePi::kRow + 2 * (32 * ks + 8 * g4);
        const int qa = (16 * rt + n16) * TilePi::kRow + 2 * (32 * ks + 8 * g4);
        if (!grad) {
          const bf16x8 kf = as_bf16x8(lds_ld<uint4>(sK, ka));
          const bf16x8 qf = as_bf16x8(lds_ld<uint4>(sQ, qa));
          if (exact) {
            acc = mma(as_bf16x8(lds_ld<uint4>(sKl, ka)), qf, acc);
            acc = mma(kf, as_bf16x8(lds_ld<uint4>(sQl, qa)), acc);
          }
          acc = mma(kf, qf, acc);
        } else {
          const bf16x8 vf = as_bf16x8(lds_ld<uint4>(sV, ka));
          const bf16x8 uf = as_bf16x8(lds_ld<uint4>(sU, qa));
          if (exact) acc = mma(vf, as_bf16x8(lds_ld<uint4>(sUl, qa)), acc);
          acc = mma(vf, uf, acc);
        }
      }
      if (st == rt) {
#pragma unroll
        for (int r = 0; r < 4; ++r)
          if (4 * g4 + r > n16) acc[r] = 0.f;
      }
      lds_st<uint2>(grad ? sdP : sP, score_off(16 * rt + n16, 16 * st + 4 * g4),
                    make_uint2(pack2(acc[0], acc[1]), pack2(acc[2], acc[3])));
    }
    // ---- G after the chunk: G -= Qh^T dU (this wave's columns)
    {
      bf16x8 nU[2];
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) nU[kk] = negate(col_il<TilePi>(sU, kk, 16 * w, g4, n16));
      accumulate_il(Gacc, sQ, nU, g4, n16);
    }
    // the snapshot area holds an exact chunk's lo tiles until every wave's scores are done
    if (exact) __syncthreads();
    // ---- snapshots S^T[j][i] (S before the chunk) and G^T[j][i] (G after it), bf16
#pragma unroll
    for (int rtk = 0; rtk < 8; ++rtk) {
      const int off = snap_off(16 * w + n16, 16 * rtk + 4 * g4);
      lds_st<uint2>(sST, off, make_uint2(pack2(Sacc[rtk][0], Sacc[rtk][1]), pack2(Sacc[rtk][2], Sacc[rtk][3])));
      lds_st<uint2>(sGT, off, make_uint2(pack2(Gacc[rtk][0], Gacc[rtk][1]), pack2(Gacc[rtk][2], Gacc[rtk][3])));
    }
    __syncthreads();
    // ---- outputs of this wave's 16 columns.  Each output is formed for the four row
    // blocks at once: every A operand (S, G, S^T, G^T, or a column of V, Kh, dU, Qh)
    // is read once and feeds four independent accumulation chains.
    uint2 dqp[4], dkp[4];  // fused: this lane's bf16 dqh, dkh (rows 16 rt + n16, 4 columns)
    {
      const int col = 16 * w + 4 * g4;
      f32x4 acc[4];
      // u = Qh S + (P V)  ->  dg = do * u * sigmoid'(g)
#pragma unroll
      for (int rt = 0; rt < 4; ++rt) acc[rt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        const bf16x8 a = pack8(Sacc[2 * kk], Sacc[2 * kk + 1]);
#pragma unroll
        for (int rt = 0; rt < 4; ++rt) acc[rt] = mma(a, pi_row(sQ, 16 * rt + n16, kk, g4), acc[rt]);
      }
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        const bf16x8 a = col_nat<TilePi>(sV, kk, 16 * w, g4, n16);
#pragma unroll
        for (int rt = 2 * kk; rt < 4; ++rt) acc[rt] = mma(a, score_row(sP, 16 * rt + n16, kk, g4), acc[rt]);
      }
#pragma unroll
      for (int rt = 0; rt < 4; ++rt) {
        const float d[4] = {bf2f_lo(dor[rt].x), bf2f_hi(dor[rt].x), bf2f_lo(dor[rt].y), bf2f_hi(dor[rt].y)};
        const float gg[4] = {bf2f_lo(gr[rt].x), bf2f_hi(gr[rt].x), bf2f_lo(gr[rt].y), bf2f_hi(gr[rt].y)};
        float dg[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float sg = sigmoidf_(gg[r]);
          dg[r] = d[r] * acc[rt][r] * sg * (1.0f - sg);
        }
        if (16 * rt + n16 < nv)
          *reinterpret_cast<uint2*>(bp.dg + tl.base + (int64_t)(t0 + 16 * rt + n16) * rs + col) =
              make_uint2(pack2(dg[0], dg[1]), pack2(dg[2], dg[3]));
      }
      // dV = Kh G + (P^T dU)   (the row is the key token s here)
#pragma unroll
      for (int rt = 0; rt < 4; ++rt) acc[rt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        const bf16x8 a = pack8(Gacc[2 * kk], Gacc[2 * kk + 1]);
#pragma unroll
        for (int rt = 0; rt < 4; ++rt) acc[rt] = mma(a, pi_row(sK, 16 * rt + n16, kk, g4), acc[rt]);
      }
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        const bf16x8 a = col_il<TilePi>(sU, kk, 16 * w, g4, n16);
#pragma unroll
        for (int rt = 0; rt < 2 * kk + 2; ++rt) acc[rt] = mma(a, score_col_il(sP, kk, 16 * rt, g4, n16), acc[rt]);
      }
      store_rows4(bp.dv, acc, tl.base, t0, rs, col, nv, n16);
      // S before the next chunk: S += Kh^T V (dQh below reads S before the chunk from its snapshot)
      bf16x8 Vf[2];
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) Vf[kk] = col_il<TilePi>(sV, kk, 16 * w, g4, n16);
      accumulate_il(Sacc, sK, Vf, g4, n16);
      // dKh = V G^T + (dP^T Qh)
#pragma unroll
      for (int rt = 0; rt < 4; ++rt) acc[rt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        const bf16x8 a = snap_col(sGT, kk, 16 * w, g4, n16);
#pragma unroll
        for (int rt = 0; rt < 4; ++rt) acc[rt] = mma(a, pi_row(sV, 16 * rt + n16, kk, g4), acc[rt]);
      }
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        const bf16x8 a = col_il<TilePi>(sQ, kk, 16 * w, g4, n16);
#pragma unroll
        for (int rt = 0; rt < 2 * kk + 2; ++rt) acc[rt] = mma(a, score_col_il(sdP, kk, 16 * rt, g4, n16), acc[rt]);
      }
      if (kFuse) {
#pragma unroll
        for (int rt = 0; rt < 4; ++rt) dkp[rt] = make_uint2(pack2(acc[rt][0], acc[rt][1]), pack2(acc[rt][2], acc[rt][3]));
      } else {
        store_rows4(bp.dkh, acc, tl.base, t0, rs, col, nv, n16);
      }
      // dQh = dU S^T + (dP Kh)
#pragma unroll
      for (int rt = 0; rt < 4; ++rt) acc[rt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        const bf16x8 a = snap_col(sST, kk, 16 * w, g4, n16);
#pragma unroll
        for (int rt = 0; rt < 4; ++rt) acc[rt] = mma(a, pi_row(sU, 16 * rt + n16, kk, g4), acc[rt]);
      }
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        const bf16x8 a = col_nat<TilePi>(sK, kk, 16 * w, g4, n16);
#pragma unroll
        for (int rt = 2 * kk; rt < 4; ++rt) acc[rt] = mma(a, score_row(sdP, 16 * rt + n16, kk, g4), acc[rt]);
      }
      if (kFuse) {
#pragma unroll
        for (int rt = 0; rt < 4; ++rt) dqp[rt] = make_uint2(pack2(acc[rt][0], acc[rt][1]), pack2(acc[rt][2], acc[rt][3]));
      } else {
        store_rows4(bp.dqh, acc, tl.base, t0, rs, col, nv, n16);
      }
    }
    // the prologue backward's raw q, k rows (L2 hits: the staging loaded them), issued
    // here so that their latency passes under the two barriers and the tile stores
    Rows<2> PX[2];
    if (kFuse) {
      load_rows_cached<2, 32>(p.q + tl.base + (int64_t)t0 * rs, rs, nv, rg, j, PX[0]);
      load_rows_cached<2, 32>(p.k + tl.base + (int64_t)t0 * rs, rs, nv, rg, j, PX[1]);
    }
    __syncthreads();
    if (kFuse) {
      // dqh, dkh of this chunk through LDS (the snapshot area is free now) into the
      // staging layout, then rotated back and through the RMSNorm Jacobian
      const int col = 16 * w + 4 * g4;
#pragma unroll
      for (int rt = 0; rt < 4; ++rt) {
        lds_st<uint2>(sX, snap_off(16 * rt + n16, col), dqp[rt]);
        lds_st<uint2>(sX + kSnapBytes, snap_off(16 * rt + n16, col), dkp[rt]);
      }
      __syncthreads();
      float2 E[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) E[e] = cmul(rope_rotation(tl.pos_base + t0, rev[e]), L.A[e]);
      float dw[2][8];
      prologue_back_rows<kWeights>(p, bp, tl.base + (int64_t)t0 * rs, nv, rs, rg, j, L, E, sX, sX + kSnapBytes, sQ, PX,
                                   dw);
      if (wgrad) {
        // the wave's four row groups (lanes 16 apart) summed, then the 8 waves' parts in
        // the unused middle of the area, summed in a fixed order into dw_acc
#pragma unroll
        for (int a = 0; a < 2; ++a)
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            float x = dw[a][e];
            x += __shfl_xor(x, 16);
            x += __shfl_xor(x, 32);
            dw[a][e] = x;
          }
        // [8 waves][2][128] between the dqh tile (the first 64 rows) and the dkh tile
        float* part = reinterpret_cast<float*>(sX + kC * kSnapRow);
        static_assert(kC * kSnapRow + kWaves * 2 * kD * 4 <= kSnapBytes, "weight parts overlap the dkh tile");
        if (lane < 16)
#pragma unroll
          for (int a = 0; a < 2; ++a)
#pragma unroll
            for (int e = 0; e < 8; ++e) part[(w * 2 + a) * kD + (e < 4 ? 4 * j + e : kHalf + 4 * j + e - 4)] = dw[a][e];
        __syncthreads();
        if (tid < 2 * kD) {
          float sum = 0.f;
#pragma unroll
          for (int ww = 0; ww < kWaves; ++ww) sum += part[(ww * 2 + tid / kD) * kD + tid % kD];
          dw_acc += sum;
        }
      }
      // the next chunk's hi/lo tiles overwrite the area
      const int t1 = t0 + kC;
      if (c + 1 < tl.nch && t1 + 2 * kC > p.T) __syncthreads();
    }
  }
  if (kFuse && wgrad && tid < 2 * kD)
    bp.wpart[((int64_t)(tid / kD) * kPrologueBlocks + blockIdx.x) * kD + tid % kD] = dw_acc;
}

// dq, dk from the gradients of the rotated, normalized rows (dqh, dkh): rotating
// back by the same angle gives dn, then through RMSNorm (n = w x / r):
//     dx_i = w_i dn_i / r - x_i (sum_j w_j x_j dn_j) / (D r^3),   dw_i += dn_i x_i / r.
// A workgroup of 512 threads takes 64-token chunks of one head in turn, staged like
// the forward: thread (rg, j) holds rows rg and rg + 32 and dims 4j..4j+3 with
// their RoPE partners 64+4j..; the rotations come from the chunk's base rotation.
// Each workgroup leaves its part of dw in wpart[which][blockIdx].
constexpr int kProThreads = 512;

template <bool kWeights>
__global__ __launch_bounds__(kProThreads) void la_prologue_backward_kernel(BackwardParams bp) {
  const PrefillParams& p = bp.f;
  __shared__ float2 sRot[kHalf];
  __shared__ float sW[2][32][kD / 8][8];  // weight-gradient parts of each row group, per tensor

  const int tid = threadIdx.x, j = tid & 15, rg = tid >> 4;
  const int64_t rs = (int64_t)p.H * kD;
  float w[2][8];
  load_norm_weights(p.qw, j, w[0]);
  load_norm_weights(p.kw, j, w[1]);
  Rope L;
  rope_init<32>(p, tid, rg, j, L);
  float dw[2][8];
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int e = 0; e < 8; ++e) dw[a][e] = 0.f;

  const int nch = (p.T + kC - 1) / kC;
  const int64_t items = (int64_t)p.B * p.H * nch;
  for (int64_t item = blockIdx.x; item < items; item += gridDim.x) {
    const int c = (int)(item % nch);
    const int64_t bh = item / nch;
    const int64_t base = ((bh / p.H) * p.T * p.H + bh % p.H) * kD;
    const int t0 = c * kC, nv = min(kC, p.T - t0);
    if (tid < kHalf) sRot[tid] = rope_rotation(p.pos0 + t0, L.base_rev);
    Rows<2> X[2], Y[2];
    load_rows<2, 32>(p.q + base + (int64_t)t0 * rs, rs, nv, rg, j, X[0]);
    load_rows<2, 32>(p.k + base + (int64_t)t0 * rs, rs, nv, rg, j, X[1]);
    load_rows<2, 32>(bp.dqh + base + (int64_t)t0 * rs, rs, nv, rg, j, Y[0]);
    load_rows<2, 32>(bp.dkh + base + (int64_t)t0 * rs, rs, nv, rg, j, Y[1]);
    __syncthreads();
    float2 E[4];
    first_rotation<32>(sRot, L, j, E);
#pragma unroll
    for (int m = 0; m < 2; ++m) {
      if (m > 0) next_rotation(L, E);
      const int t = rg + 32 * m;
#pragma unroll
      for (int a = 0; a < 2; ++a) {
        float dx[8], dn[8], x[8], inv;
        prologue_back_row(X[a].lo[m], X[a].hi[m], Y[a].lo[m], Y[a].hi[m], w[a], E, p.eps, dx, dn, x, inv);
        if (kWeights && t < nv)
#pragma unroll
          for (int e = 0; e < 8; ++e) dw[a][e] += dn[e] * x[e] * inv;
        if (t < nv) store_row_pieces((a ? bp.dk : bp.dq) + base + (int64_t)(t0 + t) * rs, j, dx);
      }
    }
    __syncthreads();  // sRot is rewritten for the next chunk
  }
  if (kWeights) {
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
      for (int e = 0; e < 8; ++e) sW[a][rg][j][e] = dw[a][e];
    __syncthreads();
    if (tid < 2 * kD) {
      const int a = tid / kD, i = tid % kD;
      // dim i is held by thread j = (i % 64) / 4 as element e = i % 4 (+ 4 for the upper half)
      const int jj = (i % kHalf) / 4, e = (i % 4) + (i >= kHalf ? 4 : 0);
      float s = 0.f;
      for (int r = 0; r < 32; ++r) s += sW[a][r][jj][e];
      bp.wpart[((int64_t)a * kPrologueBlocks + blockIdx.x) * kD + i] = s;
    }
  }
}

// dw[i] = sum of the workgroup parts (fixed order).
__global__ __launch_bounds__(256) void la_weight_grad_kernel(BackwardParams bp, int nblocks) {
  const int i = threadIdx.x & (kD - 1), which = threadIdx.x >> 7;
  float* const out = which ? bp.dk_w : bp.dq_w;
  if (out == nullptr) return;
  float s = 0.f;
  for (int b = 0; b < nblocks; ++b) s += bp.wpart[((int64_t)which * kPrologueBlocks + b) * kD + i];
  out[i] = s;
}

}  // namespace

hipError_t launch_backward_chunks(const BackwardParams& bp, const PrefillPlan& plan, hipStream_t stream) {
  const PrefillParams& p = bp.f;
  // weight gradients without weights are taken at weights of one
  const bool weights = p.qw != nullptr || p.kw != nullptr || bp.dq_w != nullptr || bp.dk_w != nullptr;
  const dim3 grid((unsigned)(plan.nwork * p.H));
  // the prologue backward runs inside the chunk kernel (its norm-weight gradient parts,
  // one per workgroup, summed after) unless there are more workgroups than parts
  if (grid.x <= (unsigned)kPrologueBlocks) {
    if (weights)
      hipLaunchKernelGGL(HIP_KERNEL_NAME(la_backward_chunk_kernel<true, true>), grid, dim3(kBwdThreads), 0, stream, bp);
    else
      hipLaunchKernelGGL(HIP_KERNEL_NAME(la_backward_chunk_kernel<false, true>), grid, dim3(kBwdThreads), 0, stream,
                         bp);
    if (bp.dq_w != nullptr || bp.dk_w != nullptr)
      hipLaunchKernelGGL(la_weight_grad_kernel, dim3(1), dim3(256), 0, stream, bp, (int)grid.x);
    return hipGetLastError();
  }
  if (weights)
    hipLaunchKernelGGL(HIP_KERNEL_NAME(la_backward_chunk_kernel<true, false>), grid, dim3(kBwdThreads), 0, stream, bp);
  else
    hipLaunchKernelGGL(HIP_KERNEL_NAME(la_backward_chunk_kernel<false, false>), grid, dim3(kBwdThreads), 0, stream,
                       bp);
  const int64_t items = (int64_t)p.B * p.H * ((p.T + kC - 1) / kC);
  const int nblocks = (int)std::min<int64_t>(kPrologueBlocks, items);
  if (weights)
    hipLaunchKernelGGL(la_prologue_backward_kernel<true>, dim3(nblocks), dim3(kProThreads), 0, stream, bp);
  else
    hipLaunchKernelGGL(la_prologue_backward_kernel<false>, dim3(nblocks), dim3(kProThreads), 0, stream, bp);
  if (weights) hipLaunchKernelGGL(la_weight_grad_kernel, dim3(1), dim3(256), 0, stream, bp, nblocks);
  return hipGetLastError();
}

}  // namespace la
