// The sparse attention layers of the hybrid on gfx950: causal softmax attention
// in which every query reaches only a few key/value blocks chosen by a block score
// (InfLLM-v2 block selection), with no position encoding and an output gate
// ("創新Transformer！面壁基於稀疏-線性混合架構SALA訓練9B模型，端側跑通百萬上下文",
// 04 技術報告 > 02 模型架構 > (2) 稀疏注意力模塊 and (4) 混合位置編碼).
//
// What is computed (the pages give the mechanism in one line; the rest is the
// plainest reading): tokens form blocks of 64; key block j is scored by its mean
// key kbar_j; query block i (64 queries; one token in decode) by its mean query,
// s_ij = qbar_i . kbar_j, over the complete blocks j < i; the topk best blocks
// (ties to the lower index) plus the query's own block up to the query itself are
// attended with softmax(q k / sqrt(D)), and o = sigmoid(g) * (attention output).
// With no more than topk earlier blocks this is dense causal attention.
//
// la_sparse_means_kernel: block means of k (fp32), one workgroup per (block, h, b).
// la_sparse_prefill_kernel: one 256-thread workgroup per (query block, h, b).
//   1. selection: the query-block mean, its scores against the key means (16 lanes
//      per key block), top-k (a threshold from the maxima of 64 residue classes,
//      then exact ranks among the candidates above it), sorted by block index;
//   2. attention, flash style over the own block (first: every query sees at least
//      itself, so the running max is finite from the start) and then the selected
//      blocks, K and V tiles double-buffered in LDS with the next block's global
//      loads in flight.  Wave w owns queries 16w .. 16w + 15.  Per key block:
//      S^T = K Q^T on v_mfma_f32_16x16x32_bf16 (lane holds 4 keys of one query),
//      running max over the block's keys (two lane swaps across the 4 lane groups),
//      P^T rounded to bf16 straight from the accumulators is the B operand of
//      O^T += V^T P^T in the key order pi (V^T read transposed from LDS), so P never
//      goes through LDS.
// la_sparse_decode_kernel: one workgroup per (b, h): scores, top-k, then the
//   attention of the single query over the chosen tokens (16 lanes per key row).
#include <limits.h>

#include "la_device.hpp"
#include "la_internal.hpp"
#include "la_tiles.hpp"

namespace la {
namespace {

constexpr int kSB = kSparseBlock;
constexpr int kSparseThreads = 256;
constexpr int kKRow = kD * 2 + 32;       // 288-byte K rows: the 16-byte row reads meet no bank conflicts
constexpr int kKTile = kSB * kKRow;
constexpr int kVTile = kSB * kRowBytes;  // 272-byte V rows, read transposed
constexpr int kKVStage = kKTile + kVTile;
constexpr float kLog2e = 1.4426950408889634f;

__device__ __forceinline__ void add_bf16x8(float (&acc)[8], uint4 u) {
  acc[0] += bf2f_lo(u.x);
  acc[1] += bf2f_hi(u.x);
  acc[2] += bf2f_lo(u.y);
  acc[3] += bf2f_hi(u.y);
  acc[4] += bf2f_lo(u.z);
  acc[5] += bf2f_hi(u.z);
  acc[6] += bf2f_lo(u.w);
  acc[7] += bf2f_hi(u.w);
}

__device__ __forceinline__ float dot_bf16x8(uint4 u, const float (&x)[8]) {
  float s = bf2f_lo(u.x) * x[0];
  s = fmaf(bf2f_hi(u.x), x[1], s);
  s = fmaf(bf2f_lo(u.y), x[2], s);
  s = fmaf(bf2f_hi(u.y), x[3], s);
  s = fmaf(bf2f_lo(u.z), x[4], s);
  s = fmaf(bf2f_hi(u.z), x[5], s);
  s = fmaf(bf2f_lo(u.w), x[6], s);
  s = fmaf(bf2f_hi(u.w), x[7], s);
  return s;
}

// ---- block means of k: thread (rp, c) sums rows rp + 16 m (m < 4) of the block at
// dims 8c .. 8c + 7; the 16 partial sums meet in LDS.
__global__ __launch_bounds__(kSparseThreads) void la_sparse_means_kernel(SparseParams p, int first) {
  __shared__ float part[16][kD];
  const int tid = threadIdx.x, rp = tid >> 4, c = tid & 15;
  const int j = first + blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int64_t rs = (int64_t)p.H * kD;
  const uint16_t* src = p.k + ((int64_t)b * p.T + (int64_t)j * kSB) * rs + (int64_t)h * kD + 8 * c;
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int m = 0; m < 4; ++m) add_bf16x8(acc, *reinterpret_cast<const uint4*>(src + (int64_t)(rp + 16 * m) * rs));
#pragma unroll
  for (int e = 0; e < 8; ++e) part[rp][8 * c + e] = acc[e];
  __syncthreads();
  if (tid < kD) {
    float s = 0.f;
#pragma unroll
    for (int r = 0; r < 16; ++r) s += part[r][tid];
    p.kmean[(((int64_t)b * p.H + h) * (p.T / kSB) + j) * kD + tid] = s * (1.0f / kSB);
  }
}

// Scores sc[j] = qm . kmean[j] for j < n: 16 lanes per key block (8 dims each),
// kInFlight key blocks per lane group in flight.  qm is in LDS; every thread of the
// workgroup calls it.
template <int kInFlight>
__device__ __forceinline__ void block_scores(const float* qm, const float* kmean, int n, float* sc) {
  const int tid = threadIdx.x, grp = tid >> 4, c = tid & 15;
  constexpr int kGroups = kSparseThreads / 16;
  float q8[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) q8[e] = qm[8 * c + e];
  for (int j0 = grp; j0 < n; j0 += kInFlight * kGroups) {
    float4 a[kInFlight], b[kInFlight];
#pragma unroll
    for (int u = 0; u < kInFlight; ++u) {
      const int j = min(j0 + u * kGroups, n - 1);  // past n: a valid row, result unused
      a[u] = *reinterpret_cast<const float4*>(kmean + (int64_t)j * kD + 8 * c);
      b[u] = *reinterpret_cast<const float4*>(kmean + (int64_t)j * kD + 8 * c + 4);
    }
#pragma unroll
    for (int u = 0; u < kInFlight; ++u) {
      float s = a[u].x * q8[0];
      s = fmaf(a[u].y, q8[1], s);
      s = fmaf(a[u].z, q8[2], s);
      s = fmaf(a[u].w, q8[3], s);
      s = fmaf(b[u].x, q8[4], s);
      s = fmaf(b[u].y, q8[5], s);
      s = fmaf(b[u].z, q8[6], s);
      s = fmaf(b[u].w, q8[7], s);
      s = row16_sum(s);  // the 16 lanes of a DPP row share j0, so all of them are active here
      const int j = j0 + u * kGroups;
      if (c == 0 && j < n) sc[j] = s;
    }
  }
}

__device__ __forceinline__ bool better(float v, int i, float bv, int bi) { return v > bv || (v == bv && i < bi); }

// Scratch of select_topk in LDS.
struct SelectScratch {
  float gmax[kSparseThreads];  // per-thread best (score, index)
  int gidx[kSparseThreads];
  int count;                   // survivors
  float thresh;                // the threshold candidate (score, index)
  int thresh_idx;
};

__device__ __forceinline__ bool above(float v, int i, float bv, int bi) { return v > bv || (v == bv && i < bi); }

__device__ __forceinline__ float lane_f(float x, int l) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), l));
}

// The min(topk, n) best of sc[0..n) (higher score first, ties to the lower index)
// into list, sorted by index; returns their number.  For n > topk:
//   1. the best candidate of each of the 64 residue classes j mod 64 (each class
//      non-empty since n > topk and topk <= 64); the topk-th best of these,
//      (M, jM), is reached by topk distinct candidates, so every chosen candidate
//      ranks at or above it (wave 0 ranks the 64 class bests by reading one lane
//      per step);
//   2. the candidates at or above (M, jM) survive into surv as (score, index)
//      pairs (order immaterial): with random scores a few dozen, with all scores
//      equal exactly topk;
//   3. with at most 64 survivors wave 0 holds one per lane and counts, reading one
//      lane per step, each survivor's rank and, for the chosen ones, its place in
//      index order; more survivors (a few classes holding most of the best scores)
//      are ranked from LDS by all threads and then sorted.
// surv holds 2 cap ints (cap pairs) and at least n ints.  Every thread calls it;
// it ends on a barrier.
__device__ int select_topk(const float* sc, int n, int topk, int* list, int* surv, int cap, SelectScratch* ss) {
  const int tid = threadIdx.x, lane = tid & 63;
  if (n <= topk) {
    for (int x = tid; x < n; x += kSparseThreads) list[x] = x;
    __syncthreads();
    return n;
  }
  float gm = -INFINITY;
  int gi = INT_MAX;
  for (int j = tid; j < n; j += kSparseThreads)
    if (above(sc[j], j, gm, gi)) {
      gm = sc[j];
      gi = j;
    }
  ss->gmax[tid] = gm;
  ss->gidx[tid] = gi;
  if (tid == 0) ss->count = 0;
  if (tid < topk) list[tid] = -1;  // slots left empty (non-finite scores) are skipped by the callers
  __syncthreads();
  if (tid < 64) {
    float c = ss->gmax[tid];
    int ci = ss->gidx[tid];
#pragma unroll
    for (int q = 1; q < 4; ++q)
      if (above(ss->gmax[tid + 64 * q], ss->gidx[tid + 64 * q], c, ci)) {
        c = ss->gmax[tid + 64 * q];
        ci = ss->gidx[tid + 64 * q];
      }
    int rank = 0;
    for (int y = 0; y < 64; ++y) rank += above(lane_f(c, y), __builtin_amdgcn_readlane(ci, y), c, ci);
    if (lane == 0) {
      ss->thresh = -INFINITY;  // kept only if no class best ranks topk - 1 (non-finite scores)
      ss->thresh_idx = INT_MAX;
    }
    __builtin_amdgcn_wave_barrier();
    if (rank == topk - 1) {
      ss->thresh = c;
      ss->thresh_idx = ci;
    }
  }
  __syncthreads();
  const float M = ss->thresh;
  const int jM = ss->thresh_idx;
  for (int j = tid; j < n; j += kSparseThreads) {
    const float v = sc[j];
    if (v > M || (v == M && j <= jM)) {
      const int x = atomicAdd(&ss->count, 1);
      if (x < cap) {
        surv[2 * x] = __float_as_int(v);
        surv[2 * x + 1] = j;
      }
    }
  }
  __syncthreads();
  const int S = ss->count;
  if (S <= 64) {
    if (tid < 64) {
      const bool mine = lane < S;
      const float vx = mine ? __int_as_float(surv[2 * lane]) : -INFINITY;
      const int jx = mine ? surv[2 * lane + 1] : INT_MAX;
      int r = 0;
      for (int y = 0; y < S; ++y) r += above(lane_f(vx, y), __builtin_amdgcn_readlane(jx, y), vx, jx);
      const bool chosen = mine && r < topk;
      int pos = 0;  // place among the chosen in index order
      for (int y = 0; y < S; ++y) {
        const int jy = __builtin_amdgcn_readlane(jx, y);
        const int ry = __builtin_amdgcn_readlane(r, y);
        pos += (ry < topk) && (jy < jx);
      }
      if (chosen) list[pos] = jx;
    }
    __syncthreads();
    return topk;
  }
  if (S <= cap) {
    for (int x = tid; x < S; x += kSparseThreads) {
      const float vx = __int_as_float(surv[2 * x]);
      const int jx = surv[2 * x + 1];
      int r = 0;
#pragma unroll 8
      for (int y = 0; y < S; ++y) {
        const int2 e = reinterpret_cast<const int2*>(surv)[y];
        r += above(__int_as_float(e.x), e.y, vx, jx);
      }
      if (r < topk) list[r] = jx;
    }
  } else {
    // more survivors than pairs fit: indices only, scores read back
    if (tid == 0) ss->count = 0;
    __syncthreads();
    for (int j = tid; j < n; j += kSparseThreads)
      if (sc[j] > M || (sc[j] == M && j <= jM)) surv[atomicAdd(&ss->count, 1)] = j;
    __syncthreads();
    for (int x = tid; x < S; x += kSparseThreads) {
      const int jx = surv[x];
      const float vx = sc[jx];
      int r = 0;
      for (int y = 0; y < S; ++y) r += above(sc[surv[y]], surv[y], vx, jx);
      if (r < topk) list[r] = jx;
    }
  }
  __syncthreads();
  if (tid == 0)  // insertion sort by block index
    for (int a = 1; a < topk; ++a) {
      const int x = list[a];
      int y = a - 1;
      while (y >= 0 && list[y] > x) {
        list[y + 1] = list[y];
        --y;
      }
      list[y + 1] = x;
    }
  __syncthreads();
  return topk;
}

__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) x = fmaxf(x, __shfl_xor(x, off));
  return x;
}
__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) x += __shfl_xor(x, off);
  return x;
}

__global__ __launch_bounds__(kSparseThreads) void la_sparse_prefill_kernel(SparseParams p) {
  // K/V tile stages; during the selection the first stage holds the scores and the
  // second the partial sums of the query mean
  __shared__ __attribute__((aligned(16))) uint8_t sKV[2][kKVStage];
  __shared__ float sQm[kD];
  __shared__ int sList[kSparseMaxTopk];
  __shared__ SelectScratch ss;
  static_assert(kSparseMaxBlocks * 4 <= kKVStage, "scores and survivor indices must each fit one tile stage");
  static_assert(16 * kD * 4 <= kKVStage, "partial sums must fit one tile stage");

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int n16 = lane & 15, g4 = lane >> 4;
  const int nqb = (p.T + kSB - 1) / kSB, nkb = p.T / kSB;
  const int i = blockIdx.x % nqb;
  const int bh = blockIdx.x / nqb, h = bh % p.H, b = bh / p.H;
  const int64_t rs = (int64_t)p.H * kD;
  const int64_t base = (int64_t)b * p.T * rs + (int64_t)h * kD;
  const int r0 = i * kSB, nv = min(kSB, p.T - r0);
  const int ncand = min(i, nkb);

  // ---- selection
  int nlist;
  if (ncand <= p.topk) {
    nlist = select_topk(nullptr, ncand, p.topk, sList, nullptr, 0, &ss);
  } else {
    float* part = reinterpret_cast<float*>(sKV[1]);
    {
      const int rp = tid >> 4, c = tid & 15;
      float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        const int r = rp + 16 * m;
        if (r < nv) add_bf16x8(acc, *reinterpret_cast<const uint4*>(p.q + base + (int64_t)(r0 + r) * rs + 8 * c));
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) part[rp * kD + 8 * c + e] = acc[e];
    }
    __syncthreads();
    if (tid < kD) {
      float s = 0.f;
#pragma unroll
      for (int r = 0; r < 16; ++r) s += part[r * kD + tid];
      sQm[tid] = s / (float)nv;
    }
    __syncthreads();
    float* sc = reinterpret_cast<float*>(sKV[0]);
    block_scores<4>(sQm, p.kmean + ((int64_t)b * p.H + h) * nkb * kD, ncand, sc);
    __syncthreads();
    nlist = select_topk(sc, ncand, p.topk, sList, reinterpret_cast<int*>(sKV[1]), kKVStage / 8, &ss);
  }
  if (p.sel != nullptr)
    for (int x = tid; x < p.topk; x += kSparseThreads) {
      // the chosen blocks in increasing order, then -1
      int cnt = 0, val = -1;
      for (int y = 0; y < nlist; ++y)
        if (sList[y] >= 0) {
          if (cnt == x) val = sList[y];
          ++cnt;
        }
      p.sel[((int64_t)bh * nqb + i) * p.topk + x] = val;
    }

  // ---- attention: own block first, then the chosen blocks
  const int nblk = 1 + nlist;
  auto block_row0 = [&](int n) { return n == 0 ? r0 : sList[n - 1] * kSB; };
  const int lr = tid >> 2, lq = tid & 3;  // loader: row lr, bytes 64 lq .. 64 lq + 63 of K and of V
  uint4 rk[4], rv[4];
  auto load_block = [&](int n) {
    const int64_t row = min(block_row0(n) + lr, p.T - 1);
    const uint16_t* ks = p.k + base + row * rs + 32 * lq;
    const uint16_t* vs = p.v + base + row * rs + 32 * lq;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      rk[u] = *reinterpret_cast<const uint4*>(ks + 8 * u);
      rv[u] = *reinterpret_cast<const uint4*>(vs + 8 * u);
    }
  };
  auto store_block = [&](int buf) {
    uint8_t* K = sKV[buf];
    uint8_t* V = sKV[buf] + kKTile;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      lds_st<uint4>(K, lr * kKRow + 64 * lq + 16 * u, rk[u]);
      lds_st<uint4>(V, lr * kRowBytes + 64 * lq + 16 * u, rv[u]);
    }
  };
  // skip empty slots (only possible with non-finite scores)
  auto next_valid = [&](int n) {
    while (n < nblk && n > 0 && sList[n - 1] < 0) ++n;
    return n;
  };

  const int qr = 16 * w + n16;  // this lane's query row in the block
  bf16x8 Qf[4];
  {
    const int64_t row = min(r0 + qr, p.T - 1);
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
      Qf[ks] = as_bf16x8(*reinterpret_cast<const uint4*>(p.q + base + row * rs + 32 * ks + 8 * g4));
  }
  f32x4 O[8];
#pragma unroll
  for (int dt = 0; dt < 8; ++dt) O[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, l_run = 0.f;
  const float cs = kLog2e * rsqrtf((float)kD);

  int cur = 0;                       // block being computed
  int nxt = next_valid(1);           // block staged next
  load_block(cur);
  store_block(0);
  if (nxt < nblk) load_block(nxt);
  __syncthreads();
  for (int step = 0; cur < nblk; ++step) {
    const uint8_t* K = sKV[step & 1];
    const uint8_t* V = K + kKTile;
    f32x4 S[4];
#pragma unroll
    for (int kt = 0; kt < 4; ++kt) {
      S[kt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < 4; ++ks)
        S[kt] = mma(as_bf16x8(lds_ld<uint4>(K, (16 * kt + n16) * kKRow + 64 * ks + 16 * g4)), Qf[ks], S[kt]);
    }
    // lane holds S^T[key 16 kt + 4 g + r][query qr]
    float mx = -INFINITY;
#pragma unroll
    for (int kt = 0; kt < 4; ++kt)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        float x = S[kt][r] * cs;
        if (cur == 0 && 16 * kt + 4 * g4 + r > qr) x = -INFINITY;
        S[kt][r] = x;
        mx = fmaxf(mx, x);
      }
    mx = fmaxf(mx, __shfl_xor(mx, 16));
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float m_new = fmaxf(m_run, mx);
    const float alpha = exp2f(m_run - m_new);
    m_run = m_new;
    float ls = 0.f;
#pragma unroll
    for (int kt = 0; kt < 4; ++kt)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        S[kt][r] = exp2f(S[kt][r] - m_new);
        ls += S[kt][r];
      }
    l_run = fmaf(l_run, alpha, ls);
    const bf16x8 P0 = pack8(S[0], S[1]), P1 = pack8(S[2], S[3]);  // keys in order pi
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) {
      O[dt] *= alpha;
      O[dt] = mma(v_operand(V, 0, 16 * dt, g4, n16), P0, O[dt]);
      O[dt] = mma(v_operand(V, 1, 16 * dt, g4, n16), P1, O[dt]);
    }
    cur = nxt;
    if (cur < nblk) {
      store_block((step + 1) & 1);
      nxt = next_valid(cur + 1);
      if (nxt < nblk) load_block(nxt);
    }
    __syncthreads();
  }
  // lane holds O^T[16 dt + 4 g + r][query qr]: normalize, gate, store 4 consecutive values
  float lt = l_run + __shfl_xor(l_run, 16);
  lt += __shfl_xor(lt, 32);
  const float inv = 1.0f / lt;
  if (qr < nv) {
    const int64_t orow = base + (int64_t)(r0 + qr) * rs;
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) {
      const int d = 16 * dt + 4 * g4;
      const uint2 gg = *reinterpret_cast<const uint2*>(p.g + orow + d);
      const float o0 = O[dt][0] * inv * sigmoidf_(bf2f_lo(gg.x));
      const float o1 = O[dt][1] * inv * sigmoidf_(bf2f_hi(gg.x));
      const float o2 = O[dt][2] * inv * sigmoidf_(bf2f_lo(gg.y));
      const float o3 = O[dt][3] * inv * sigmoidf_(bf2f_hi(gg.y));
      *reinterpret_cast<uint2*>(p.o + orow + d) = make_uint2(pack2(o0, o1), pack2(o2, o3));
    }
  }
}

// ---- decode: one query per (b, h) against its cache
__global__ __launch_bounds__(kSparseThreads) void la_sparse_decode_kernel(SparseParams p) {
  __shared__ float sc[kSparseMaxBlocks];  // block scores, then the attention weights
  __shared__ float sQ[kD];
  __shared__ float part[16][kD];
  __shared__ int surv[2 * kSparseMaxBlocks];
  __shared__ int sList[kSparseMaxTopk];
  __shared__ SelectScratch ss;
  __shared__ float red_v[4];
  static_assert((kSparseMaxTopk + 1) * kSB <= kSparseMaxBlocks, "weights must fit the score array");

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int bh = blockIdx.x, h = bh % p.H, b = bh / p.H;
  const int len = min(max(p.lens[b], 1), p.T);
  const int t = len - 1, own = t / kSB, ncand = own;
  const int64_t rs = (int64_t)p.H * kD;
  const int64_t cbase = (int64_t)b * p.T * rs + (int64_t)h * kD;
  const int64_t qoff = (int64_t)bh * kD;
  if (tid < kD) sQ[tid] = bf2f(p.q[qoff + tid]);
  __syncthreads();
  int nlist;
  if (ncand <= p.topk) {
    nlist = select_topk(nullptr, ncand, p.topk, sList, nullptr, 0, &ss);
  } else {
    block_scores<8>(sQ, p.kmean + (int64_t)bh * (p.T / kSB) * kD, ncand, sc);
    __syncthreads();
    nlist = select_topk(sc, ncand, p.topk, sList, surv, kSparseMaxBlocks, &ss);
  }
  if (p.sel != nullptr)
    for (int x = tid; x < p.topk; x += kSparseThreads) {
      int cnt = 0, val = -1;
      for (int y = 0; y < nlist; ++y)
        if (sList[y] >= 0) {
          if (cnt == x) val = sList[y];
          ++cnt;
        }
      p.sel[(int64_t)bh * p.topk + x] = val;
    }
  // keys: the chosen blocks' 64 tokens each (empty slots contribute none), then own block up to t
  const int nk = nlist * kSB + (t - own * kSB + 1);
  auto key_row = [&](int n) -> int {
    if (n < nlist * kSB) {
      const int blk = sList[n / kSB];
      return blk < 0 ? -1 : blk * kSB + n % kSB;
    }
    return own * kSB + (n - nlist * kSB);
  };
  const float cs = kLog2e * rsqrtf((float)kD);
  {
    const int grp = tid >> 4, c = tid & 15;
    float q8[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) q8[e] = sQ[8 * c + e];
    constexpr int kGroups = kSparseThreads / 16;
    for (int n0 = grp; n0 < nk; n0 += 4 * kGroups) {  // four key rows per lane group in flight
      uint4 u[4];
      int row[4];
#pragma unroll
      for (int x = 0; x < 4; ++x) {
        const int n = n0 + x * kGroups;
        row[x] = n < nk ? key_row(n) : -1;
        u[x] = *reinterpret_cast<const uint4*>(p.k + cbase + (int64_t)max(row[x], 0) * rs + 8 * c);
      }
#pragma unroll
      for (int x = 0; x < 4; ++x) {
        const int n = n0 + x * kGroups;
        const float s = row16_sum(dot_bf16x8(u[x], q8));
        if (c == 0 && n < nk) sc[n] = row[x] >= 0 ? s * cs : -INFINITY;
      }
    }
  }
  __syncthreads();
  float mx = -INFINITY;
  for (int n = tid; n < nk; n += kSparseThreads) mx = fmaxf(mx, sc[n]);
  mx = wave_max(mx);
  if (lane == 0) red_v[w] = mx;
  __syncthreads();
  mx = fmaxf(fmaxf(red_v[0], red_v[1]), fmaxf(red_v[2], red_v[3]));
  float den = 0.f;
  for (int n = tid; n < nk; n += kSparseThreads) {
    const float e = exp2f(sc[n] - mx);
    sc[n] = e;
    den += e;
  }
  den = wave_sum(den);
  __syncthreads();  // every thread has read red_v (max) before it is reused
  if (lane == 0) red_v[w] = den;
  __syncthreads();
  den = red_v[0] + red_v[1] + red_v[2] + red_v[3];
  {
    const int kg = tid >> 4, c = tid & 15;
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    constexpr int kGroups = kSparseThreads / 16;
    for (int n0 = kg; n0 < nk; n0 += 4 * kGroups) {  // four value rows per lane group in flight
      uint4 u[4];
      float pn[4];
#pragma unroll
      for (int x = 0; x < 4; ++x) {
        const int n = n0 + x * kGroups;
        const int row = n < nk ? key_row(n) : -1;
        u[x] = *reinterpret_cast<const uint4*>(p.v + cbase + (int64_t)max(row, 0) * rs + 8 * c);
        pn[x] = row >= 0 ? sc[n] : 0.f;  // empty slots and rows past the list weigh nothing
      }
#pragma unroll
      for (int x = 0; x < 4; ++x) {
        acc[0] = fmaf(pn[x], bf2f_lo(u[x].x), acc[0]);
        acc[1] = fmaf(pn[x], bf2f_hi(u[x].x), acc[1]);
        acc[2] = fmaf(pn[x], bf2f_lo(u[x].y), acc[2]);
        acc[3] = fmaf(pn[x], bf2f_hi(u[x].y), acc[3]);
        acc[4] = fmaf(pn[x], bf2f_lo(u[x].z), acc[4]);
        acc[5] = fmaf(pn[x], bf2f_hi(u[x].z), acc[5]);
        acc[6] = fmaf(pn[x], bf2f_lo(u[x].w), acc[6]);
        acc[7] = fmaf(pn[x], bf2f_hi(u[x].w), acc[7]);
      }
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) part[kg][8 * c + e] = acc[e];
  }
  __syncthreads();
  if (tid < kD) {
    float s = 0.f;
#pragma unroll
    for (int r = 0; r < 16; ++r) s += part[r][tid];
    const float o = s / den * sigmoidf_(bf2f(p.g[qoff + tid]));
    p.o[qoff + tid] = (uint16_t)f2bf(o);
  }
}

}  // namespace

hipError_t launch_sparse_means(const SparseParams& p, int first, int nblocks, hipStream_t stream) {
  if (nblocks <= 0) return hipSuccess;
  hipLaunchKernelGGL(la_sparse_means_kernel, dim3((unsigned)nblocks, (unsigned)p.H, (unsigned)p.B),
                     dim3(kSparseThreads), 0, stream, p, first);
  return hipGetLastError();
}

hipError_t launch_sparse_prefill(const SparseParams& p, hipStream_t stream) {
  hipError_t e = launch_sparse_means(p, 0, p.T / kSB, stream);
  if (e != hipSuccess) return e;
  const int64_t nqb = (p.T + kSB - 1) / kSB;
  hipLaunchKernelGGL(la_sparse_prefill_kernel, dim3((unsigned)(nqb * p.H * p.B)), dim3(kSparseThreads), 0, stream,
                     p);
  return hipGetLastError();
}

hipError_t launch_sparse_decode(const SparseParams& p, hipStream_t stream) {
  hipLaunchKernelGGL(la_sparse_decode_kernel, dim3((unsigned)(p.B * p.H)), dim3(kSparseThreads), 0, stream, p);
  return hipGetLastError();
}

}  // namespace la
