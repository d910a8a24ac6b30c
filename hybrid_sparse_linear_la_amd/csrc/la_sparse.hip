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
// la_sparse_select_kernel: one wave per (query block, h, b): the query-block mean,
//   its scores against the key means (16 lanes per key block), top-k (a threshold
//   from the maxima of 64 residue classes, then exact ranks among the candidates
//   above it), written in increasing block order.
// la_sparse_attn_kernel: one wave per (query block, h, b), all 64 queries, flash
//   style over the own block and the chosen blocks: S^T = K Q^T on
//   v_mfma_f32_16x16x32_bf16 with K and Q in operand registers, P^T rounded to bf16
//   straight from the accumulators as the B operand of O^T += V^T P^T (V^T read
//   transposed from LDS), softmax against a per-query reference without rescaling.
// la_sparse_decode_kernel: one 1024-thread workgroup per (b, h): scores, top-k, then the
//   attention of the single query over the chosen tokens (16 lanes per key row).
#include <limits.h>

#include "la_device.hpp"
#include "la_internal.hpp"
#include "la_tiles.hpp"

namespace la {
namespace {

constexpr int kSB = kSparseBlock;
constexpr int kSparseThreads = 256;  // block means
constexpr int kDecodeThreads = 1024;  // decode: 16 waves keep enough of each sequence's reads in flight
constexpr int kVTile = kSB * kRowBytes;  // 272-byte V rows, read transposed
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
template <int kInFlight, int kT>
__device__ __forceinline__ void block_scores(const float* qm, const float* kmean, int n, float* sc) {
  const int tid = threadIdx.x, grp = tid >> 4, c = tid & 15;
  constexpr int kGroups = kT / 16;
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
template <int kT>
struct SelectScratch {
  float gmax[kT];  // per-thread best (score, index)
  int gidx[kT];
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
template <int kT>
__device__ int select_topk(const float* sc, int n, int topk, int* list, int* surv, int cap, SelectScratch<kT>* ss) {
  const int tid = threadIdx.x, lane = tid & 63;
  if (n <= topk) {
    for (int x = tid; x < n; x += kT) list[x] = x;
    __syncthreads();
    return n;
  }
  float gm = -INFINITY;
  int gi = INT_MAX;
  for (int j = tid; j < n; j += kT)
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
    for (int q = 1; q < kT / 64; ++q)
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
  for (int j = tid; j < n; j += kT) {
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
    for (int x = tid; x < S; x += kT) {
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
    for (int j = tid; j < n; j += kT)
      if (sc[j] > M || (sc[j] == M && j <= jM)) surv[atomicAdd(&ss->count, 1)] = j;
    __syncthreads();
    for (int x = tid; x < S; x += kT) {
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

// Work item of a workgroup when a launch hands its workgroups to the 8 XCDs in
// turn (workgroup w to XCD w mod 8): XCD x takes the contiguous items
// [x c, x c + c), c = ceil(n / 8), in order, so the workgroups sharing an XCD (and
// its L2) work on the same head and reuse its most chosen key blocks.  The grid
// has 8 c workgroups; items from n on do nothing.
__device__ __forceinline__ int xcd_item(int n) {
  const int c = (n + 7) / 8;
  return (int)(blockIdx.x % 8) * c + (int)(blockIdx.x / 8);
}

// ---- prefill, selection: one wave per (query block, h, b).  The query-block mean
// (16 lanes x 8 dims per row, 4 rows per step), its scores against the key means
// (16 lanes per key block, kSelInFlight blocks per lane group in flight) into LDS,
// then the top-k in one wave: the best of each of the 64 residue classes j mod 64,
// the topk-th best of those as a threshold (reached by topk distinct candidates,
// so every chosen block ranks at or above it), the candidates at or above it as
// survivors, and exact ranks among them.  Writes the chosen blocks in increasing
// order, then -1, to sel.  Dynamic LDS: scores (4 B) and survivor indices (2 B)
// per key block.
constexpr int kSelInFlight = 8;

__global__ __launch_bounds__(64) void la_sparse_select_kernel(SparseParams p, int32_t* sel) {
  extern __shared__ __attribute__((aligned(16))) float sel_lds[];
  __shared__ int sTop[kSparseMaxTopk];
  const int lane = threadIdx.x;
  const int nqb = (p.T + kSB - 1) / kSB, nkb = p.T / kSB;
  const int item = xcd_item(nqb * p.H * p.B);
  if (item >= nqb * p.H * p.B) return;
  const int i = item % nqb;
  const int bh = item / nqb, h = bh % p.H, b = bh / p.H;
  const int n = min(i, nkb);
  const int topk = p.topk;
  int32_t* out = sel + ((int64_t)bh * nqb + i) * topk;
  if (n <= topk) {
    if (lane < topk) out[lane] = lane < n ? lane : -1;
    return;
  }
  const int64_t rs = (int64_t)p.H * kD;
  const int64_t base = (int64_t)b * p.T * rs + (int64_t)h * kD;
  const int r0 = i * kSB, nv = min(kSB, p.T - r0);
  const int c = lane & 15, rg = lane >> 4;

  float qm[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  {
    uint4 x[16];
    // every row is loaded (rows past the block's end: its last row again) and the
    // extra ones zeroed afterwards, so no load sits under a branch of its own and all
    // sixteen are in flight together
#pragma unroll
    for (int m = 0; m < 16; ++m) {
      const int r = rg + 4 * m;
      x[m] = *reinterpret_cast<const uint4*>(p.q + base + (int64_t)(r0 + min(r, nv - 1)) * rs + 8 * c);
    }
#pragma unroll
    for (int m = 0; m < 16; ++m) {
      const uint32_t keep = rg + 4 * m < nv ? 0xffffffffu : 0u;
      x[m] = make_uint4(x[m].x & keep, x[m].y & keep, x[m].z & keep, x[m].w & keep);
    }
#pragma unroll
    for (int m = 0; m < 16; ++m) add_bf16x8(qm, x[m]);
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    qm[e] += __shfl_xor(qm[e], 16);
    qm[e] += __shfl_xor(qm[e], 32);
    qm[e] /= (float)nv;
  }

  float* sc = sel_lds;
  uint16_t* surv = reinterpret_cast<uint16_t*>(sel_lds + nkb);
  const float* km = p.kmean + (int64_t)bh * nkb * kD + 8 * c;
  for (int j0 = rg; j0 < n; j0 += 4 * kSelInFlight) {
    float4 a[kSelInFlight], a2[kSelInFlight];
#pragma unroll
    for (int u = 0; u < kSelInFlight; ++u) {
      const int j = min(j0 + 4 * u, n - 1);  // past n: a valid row, result unused
      a[u] = *reinterpret_cast<const float4*>(km + (int64_t)j * kD);
      a2[u] = *reinterpret_cast<const float4*>(km + (int64_t)j * kD + 4);
    }
#pragma unroll
    for (int u = 0; u < kSelInFlight; ++u) {
      float s = a[u].x * qm[0];
      s = fmaf(a[u].y, qm[1], s);
      s = fmaf(a[u].z, qm[2], s);
      s = fmaf(a[u].w, qm[3], s);
      s = fmaf(a2[u].x, qm[4], s);
      s = fmaf(a2[u].y, qm[5], s);
      s = fmaf(a2[u].z, qm[6], s);
      s = fmaf(a2[u].w, qm[7], s);
      s = row16_sum(s);  // the 16 lanes of a DPP row share j0, so all of them are active here
      const int j = j0 + 4 * u;
      if (c == 0 && j < n) sc[j] = s;
    }
  }
  __syncthreads();

  // threshold: the class best of rank topk - 1 (kept at -inf if none has it: non-finite scores)
  float gm = -INFINITY;
  int gi = INT_MAX;
  for (int j = lane; j < n; j += 64) {
    const float v = sc[j];
    if (above(v, j, gm, gi)) {
      gm = v;
      gi = j;
    }
  }
  int rank = 0;
  for (int y = 0; y < 64; ++y) rank += above(lane_f(gm, y), __builtin_amdgcn_readlane(gi, y), gm, gi);
  const uint64_t at = __ballot(rank == topk - 1);
  float M = -INFINITY;
  int jM = INT_MAX;
  if (at != 0) {
    const int l = __builtin_amdgcn_readfirstlane(__ffsll((unsigned long long)at) - 1);
    M = lane_f(gm, l);
    jM = __builtin_amdgcn_readlane(gi, l);
  }
  // survivors, packed by a prefix sum of the per-lane counts
  int cnt = 0;
  for (int j = lane; j < n; j += 64) {
    const float v = sc[j];
    cnt += (v > M || (v == M && j <= jM)) ? 1 : 0;
  }
  int incl = cnt;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int t = __shfl_up(incl, off);
    if (lane >= off) incl += t;
  }
  const int S = __shfl(incl, 63);
  int pos = incl - cnt;
  for (int j = lane; j < n; j += 64) {
    const float v = sc[j];
    if (v > M || (v == M && j <= jM)) surv[pos++] = (uint16_t)j;
  }
  __syncthreads();

  bool chosen;
  int jx, ord = 0;
  if (S <= 64) {
    // one survivor per lane; ranks and index-order places by reading one lane per step
    const bool mine = lane < S;
    const int jl = min((int)surv[min(lane, max(S - 1, 0))], n - 1);  // in bounds even with no survivor
    jx = mine ? jl : INT_MAX;
    const float vx = mine ? sc[jl] : -INFINITY;
    int r = 0;
    for (int y = 0; y < S; ++y) r += above(lane_f(vx, y), __builtin_amdgcn_readlane(jx, y), vx, jx);
    chosen = mine && r < topk;
    for (int y = 0; y < S; ++y) {
      const int jy = __builtin_amdgcn_readlane(jx, y);
      const int ry = __builtin_amdgcn_readlane(r, y);
      ord += (ry < topk && jy < jx) ? 1 : 0;
    }
  } else {
    // many survivors (a few classes hold most of the best scores): ranks from LDS
    sTop[lane] = -1;
    __syncthreads();
    for (int x = lane; x < S; x += 64) {
      const int jv = surv[x];
      const float vv = sc[jv];
      int r = 0;
      for (int y = 0; y < S; ++y) {
        const int jy = surv[y];
        r += above(sc[jy], jy, vv, jv) ? 1 : 0;
      }
      if (r < topk) sTop[r] = jv;
    }
    __syncthreads();
    jx = lane < topk ? sTop[lane] : -1;
    chosen = jx >= 0;
    for (int y = 0; y < topk; ++y) {
      const int jy = __builtin_amdgcn_readlane(jx, y);
      ord += (jy >= 0 && jy < jx) ? 1 : 0;
    }
  }
  if (chosen) out[ord] = jx;
  const int nch = __popcll(__ballot(chosen));
  if (lane >= nch && lane < topk) out[lane] = -1;
}

// ---- prefill, attention: one wave per (query block, h, b), all 64 queries, over
// the own block (first: every query sees at least itself, so the running maximum is
// finite from the start) and the chosen blocks.  Per key block:
//   S^T = K Q^T on v_mfma_f32_16x16x32_bf16 (K and Q straight from global memory in
//   the A and B operand layouts, Q loaded once): lane holds 4 keys of one query per
//   (key tile, query tile);
//   softmax in base 2 against a fixed reference per query, the own block's maximum;
//   when a later block drives a lane's 16 numerators past 2^kRestart, the query
//   block starts over from the own block with the reference raised by log2 of that
//   sum (at least kRestart, so passes are few and, with ordinary logits, one; at
//   most kMaxPasses).  So P stays within 2^kRestart, no block maximum is taken after
//   the own block and the accumulators are never rescaled;
//   O^T += V^T P^T with V^T read transposed from LDS (272-byte rows) and P^T rounded
//   to bf16 straight from the accumulators in the key order pi; each V^T operand
//   read feeds the four query tiles.
// The next block's K and V loads are in flight while the current block computes;
// V goes through one LDS tile (the wave's LDS operations run in order).
// Direct global -> LDS load of 16 bytes per lane from a per-lane address (lane i's
// bytes land at LDS byte address lds + 16 i).  Issued from assembly: it writes no
// register, and the kernel waits for it explicitly before reading the LDS it fills.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void dma16_lane(const void* addr, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(addr), "s"(lds)
               : "memory", "m0");
}
#pragma clang diagnostic pop

// The gate tile: 64 rows of 256 bytes, row r's 16-byte piece p at position
// p ^ (r % 16), so that 16 rows' pieces at one column fall in 16 different bank
// groups.
constexpr int kGateRow = kD * 2;
__device__ __forceinline__ int gate_off(int row, int byte) {
  return row * kGateRow + 16 * ((byte >> 4) ^ (row & 15)) + (byte & 15);
}

constexpr float kRestart = 64.0f;  // base-2 units: P, l and O stay far inside the fp32 range
constexpr float kRestartSum = 18446744073709551616.0f;  // 2^kRestart
constexpr int kMaxPasses = 8;  // bounds the passes for non-finite logits

__global__ __launch_bounds__(64) void la_sparse_attn_kernel(SparseParams p, const int32_t* sel) {
  __shared__ __attribute__((aligned(16))) uint8_t sV[kVTile];
  __shared__ __attribute__((aligned(256))) uint8_t sG[kSB * kGateRow];  // gate rows, then the output rows
  const int lane = threadIdx.x, n16 = lane & 15, g4 = lane >> 4;
  const int nqb = (p.T + kSB - 1) / kSB;
  const int item = xcd_item(nqb * p.H * p.B);
  if (item >= nqb * p.H * p.B) return;
  const int i = item % nqb;
  const int bh = item / nqb, h = bh % p.H, b = bh / p.H;
  const int64_t rs = (int64_t)p.H * kD;
  const int64_t base = (int64_t)b * p.T * rs + (int64_t)h * kD;
  const int r0 = i * kSB, nv = min(kSB, p.T - r0);
  const uint32_t rsb = (uint32_t)rs * 2;  // bytes between rows (at most 64 rows are addressed from a block start)

  // lane x < topk holds chosen block x (the chosen ones first, in increasing order);
  // loaded first, so that the q and own-block loads below go out before its wait
  const int myblk = lane < p.topk ? sel[((int64_t)bh * nqb + i) * p.topk + lane] : -1;
  auto block_row0 = [&](int n) -> int { return n == 0 ? r0 : kSB * __builtin_amdgcn_readlane(myblk, n - 1); };
  // rows of block n that exist: the own block may end at T, and then its missing rows
  // repeat its last row (finite values that the causal mask and the unstored query
  // rows leave without effect)
  auto block_rows = [&](int n) -> int { return n == 0 ? nv : kSB; };

  auto row_ptr = [&](const uint16_t* x, int row0) {
    return reinterpret_cast<const uint8_t*>(x + base + (int64_t)row0 * rs);
  };

  // Every block's K and V loads take the same form (rows clamped to the block's
  // last row, which only the own block can need), so that the compiler counts the
  // loads in flight alike on every path and waits for exactly the ones it needs.
  // The clamp is taken on the byte offset within the block (uniform block base plus
  // a 32-bit lane offset): one add and one min per load, no multiply or 64-bit add.
  uint4 Vr[16];  // rows 4 u + g4, bytes 16 n16 .. 16 n16 + 15
  const uint32_t v_lane = (uint32_t)g4 * rsb + 16u * n16;
  auto load_rows = [&](const uint16_t* x, int row0, int rows) {
    const uint8_t* src = row_ptr(x, row0);
    const uint32_t last = (uint32_t)(rows - 1) * rsb + 16u * n16;
#pragma unroll
    for (int u = 0; u < 16; ++u)
      Vr[u] = *reinterpret_cast<const uint4*>(src + min(4u * u * rsb + v_lane, last));
  };
  // B operand Q[16 qt + n16][32 ks + 8 g4 + e], held in registers (rows past the
  // block's end repeat its last row; their outputs are not stored)
  bf16x8 Qf[4][4];
#pragma unroll
  for (int qt = 0; qt < 4; ++qt) {
    const uint32_t r = (uint32_t)min(16 * qt + n16, nv - 1);
    const uint8_t* src = row_ptr(p.q, r0) + r * rsb + 16u * g4;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) Qf[qt][ks] = as_bf16x8(*reinterpret_cast<const uint4*>(src + 64 * ks));
  }
  auto q_operand = [&](int qt, int ks) { return Qf[qt][ks]; };
  bf16x8 Kf[4][4];  // [key tile][k-step]: A operand, K[16 kt + n16][32 ks + 8 g4 + e]
  const uint32_t k_lane = (uint32_t)n16 * rsb + 16u * g4;
  auto load_k = [&](int n) {
    const uint8_t* src = row_ptr(p.k, block_row0(n));
    const uint32_t last = (uint32_t)(block_rows(n) - 1) * rsb + 16u * g4;
#pragma unroll
    for (int kt = 0; kt < 4; ++kt) {
      const uint8_t* row = src + min(16u * kt * rsb + k_lane, last);
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) Kf[kt][ks] = as_bf16x8(*reinterpret_cast<const uint4*>(row + 64 * ks));
    }
  };
  auto load_v = [&](int n) { load_rows(p.v, block_row0(n), block_rows(n)); };
  auto store_v = [&]() {
#pragma unroll
    for (int u = 0; u < 16; ++u) lds_st<uint4>(sV, (4 * u + g4) * kRowBytes + 16 * n16, Vr[u]);
  };

  load_v(0);  // the own block of the first pass: its rows do not depend on the choice
  load_k(0);
  // the gate rows go straight to LDS now, so the epilogue finds them there: load
  // m brings rows 4 m .. 4 m + 3, lane i the row's piece at position i % 16
  {
    const int lr = lane >> 4, pos = lane & 15;
    const uint32_t lds_g = __builtin_amdgcn_readfirstlane(
        (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) uint8_t*)sG);
#pragma unroll
    for (int m = 0; m < 16; ++m) {
      const int row = 4 * m + lr;
      const uint16_t* src = p.g + base + (int64_t)(r0 + min(row, nv - 1)) * rs + 8 * (pos ^ (row & 15));
      dma16_lane(src, lds_g + 1024u * m);
    }
  }
  const int nblk = 1 + __popcll(__ballot(myblk >= 0));

  f32x4 O[8][4];  // O^T[16 dt + 4 g4 + r][query 16 qt + n16]
  float m_ref[4], l_run[4];
#pragma unroll
  for (int qt = 0; qt < 4; ++qt) m_ref[qt] = -INFINITY;
  const float cs = kLog2e * rsqrtf((float)kD);

  for (int pass = 0, again = 1; again; ++pass) {
    // one pass over the blocks; a block far above the reference starts a new pass
    again = 0;
#pragma unroll
    for (int qt = 0; qt < 4; ++qt) {
      l_run[qt] = 0.f;
#pragma unroll
      for (int dt = 0; dt < 8; ++dt) O[dt][qt] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
    if (pass > 0) {
      load_v(0);  // V before K, as in the loop
      load_k(0);
    }
    for (int n = 0; n < nblk; ++n) {
      store_v();
      // the next block's loads, issued on every block (after the last block they
      // fetch it again): a load issued on some paths only made the compiler wait for
      // all loads in flight, the next block's V included, before the first products
      const int nn = min(n + 1, nblk - 1);
      load_v(nn);
      // per query tile: S^T = K Q^T, then its softmax numerators (the next tile's
      // products can run meanwhile)
      bf16x8 P[4][2];  // B operand of O^T += V^T P^T, keys in order pi
      float ls[4];
#pragma unroll
      for (int qt = 0; qt < 4; ++qt) {
        f32x4 S[4];  // S^T[16 kt + 4 g4 + r][16 qt + n16]
#pragma unroll
        for (int kt = 0; kt < 4; ++kt) S[kt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
          const bf16x8 qo = q_operand(qt, ks);
#pragma unroll
          for (int kt = 0; kt < 4; ++kt) S[kt] = mma(Kf[kt][ks], qo, S[kt]);
        }
        if (n == 0) {
          // the own block: keys after the query are masked, and on the first pass its
          // maximum becomes the query's reference
#pragma unroll
          for (int kt = 0; kt < 4; ++kt)
#pragma unroll
            for (int r = 0; r < 4; ++r)
              if (16 * kt + 4 * g4 + r > 16 * qt + n16) S[kt][r] = -INFINITY;
          if (pass == 0) {
            float m = fmaxf(fmaxf(fmaxf(S[0][0], S[0][1]), fmaxf(S[0][2], S[0][3])),
                            fmaxf(fmaxf(S[1][0], S[1][1]), fmaxf(S[1][2], S[1][3])));
            m = fmaxf(m, fmaxf(fmaxf(fmaxf(S[2][0], S[2][1]), fmaxf(S[2][2], S[2][3])),
                               fmaxf(fmaxf(S[3][0], S[3][1]), fmaxf(S[3][2], S[3][3]))));
            m = fmaxf(m, __shfl_xor(m, 16));
            m = fmaxf(m, __shfl_xor(m, 32));
            m_ref[qt] = m * cs;
          }
        }
        const float nm = -m_ref[qt];
        float l = 0.f;
#pragma unroll
        for (int kt = 0; kt < 4; ++kt)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const float e = __builtin_amdgcn_exp2f(fmaf(S[kt][r], cs, nm));
            S[kt][r] = e;
            l += e;
          }
        ls[qt] = l;
        P[qt][0] = pack8(S[0], S[1]);
        P[qt][1] = pack8(S[2], S[3]);
      }
      load_k(nn);
      // a lane's 16 numerators summing past 2^kRestart: a key far above the reference
      bool need = false;
#pragma unroll
      for (int qt = 0; qt < 4; ++qt) need |= !(ls[qt] <= kRestartSum);
      if (__ballot(need) != 0 && pass < kMaxPasses - 1) {
        // raise the reference of the queries concerned past their largest numerator
        // (log2 of a lane's sum bounds it; non-finite sums raise it by the most a pass
        // can) and start a new pass
#pragma unroll
        for (int qt = 0; qt < 4; ++qt) {
          float up = ls[qt] <= kRestartSum ? 0.f : fminf(__builtin_amdgcn_logf(ls[qt]), 2.f * kRestart);
          up = isnan(up) ? 2.f * kRestart : up;
          up = fmaxf(up, __shfl_xor(up, 16));
          up = fmaxf(up, __shfl_xor(up, 32));
          m_ref[qt] += up;
        }
        again = 1;
        break;
      }
#pragma unroll
      for (int qt = 0; qt < 4; ++qt) l_run[qt] += ls[qt];
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // this block's V tile written
#pragma unroll
      for (int dt = 0; dt < 8; ++dt) {
        const bf16x8 a0 = v_operand(sV, 0, 16 * dt, g4, n16);
        const bf16x8 a1 = v_operand(sV, 1, 16 * dt, g4, n16);
#pragma unroll
        for (int qt = 0; qt < 4; ++qt) {
          O[dt][qt] = mma(a0, P[qt][0], O[dt][qt]);
          O[dt][qt] = mma(a1, P[qt][1], O[dt][qt]);
        }
      }
    }
  }
  // normalize, gate, store, with every global access in whole rows: the gate rows
  // came into LDS 16 bytes per lane (4 rows of 256 bytes per load) at the start;
  // each lane reads back its accumulator positions, writes the bf16 outputs over
  // them, and the rows go out 16 bytes per lane.  Accesses in the accumulator
  // layout (16 rows x 8 bytes per instruction) ran 4 times the L2 transactions,
  // about a fifth of the kernel at this size.
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // the gate tile's loads landed
  const int lr = lane >> 4, lc = 16 * (lane & 15);  // rows 4 m + lr, bytes lc .. lc + 15
#pragma unroll
  for (int qt = 0; qt < 4; ++qt) {
    float lt = l_run[qt] + __shfl_xor(l_run[qt], 16);
    lt += __shfl_xor(lt, 32);
    const float inv = 1.0f / lt;
    const int qr = 16 * qt + n16;
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) {
      const int off = gate_off(qr, 2 * (16 * dt + 4 * g4));
      const uint2 g2 = lds_ld<uint2>(sG, off);
      const float o0 = O[dt][qt][0] * inv * sigmoidf_(bf2f_lo(g2.x));
      const float o1 = O[dt][qt][1] * inv * sigmoidf_(bf2f_hi(g2.x));
      const float o2 = O[dt][qt][2] * inv * sigmoidf_(bf2f_lo(g2.y));
      const float o3 = O[dt][qt][3] * inv * sigmoidf_(bf2f_hi(g2.y));
      lds_st<uint2>(sG, off, make_uint2(pack2(o0, o1), pack2(o2, o3)));
    }
  }
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // the output tile written
#pragma unroll
  for (int m = 0; m < 16; ++m) {
    const int row = 4 * m + lr;
    const uint4 ov = lds_ld<uint4>(sG, gate_off(row, lc));
    if (row < nv) *reinterpret_cast<uint4*>(p.o + base + (int64_t)(r0 + row) * rs + lc / 2) = ov;
  }
}

// ---- decode: one query per (b, h) against its cache
__global__ __launch_bounds__(kDecodeThreads) void la_sparse_decode_kernel(SparseParams p) {
  constexpr int kT = kDecodeThreads, kWaves = kT / 64, kGroups = kT / 16, kRowsInFlight = 8;
  __shared__ float sc[kSparseMaxBlocks];  // block scores, then the attention weights
  __shared__ float sQ[kD];
  __shared__ float part[kGroups][kD];
  __shared__ int surv[2 * kSparseMaxBlocks];
  __shared__ int sList[kSparseMaxTopk];
  __shared__ SelectScratch<kT> ss;
  __shared__ float red_v[kWaves];
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
    block_scores<8, kT>(sQ, p.kmean + (int64_t)bh * (p.T / kSB) * kD, ncand, sc);
    __syncthreads();
    nlist = select_topk(sc, ncand, p.topk, sList, surv, kSparseMaxBlocks, &ss);
  }
  if (p.sel != nullptr)
    for (int x = tid; x < p.topk; x += kT) {
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
    for (int n0 = grp; n0 < nk; n0 += kRowsInFlight * kGroups) {  // rows per lane group in flight
      uint4 u[kRowsInFlight];
      int row[kRowsInFlight];
#pragma unroll
      for (int x = 0; x < kRowsInFlight; ++x) {
        const int n = n0 + x * kGroups;
        row[x] = n < nk ? key_row(n) : -1;
        u[x] = *reinterpret_cast<const uint4*>(p.k + cbase + (int64_t)max(row[x], 0) * rs + 8 * c);
      }
#pragma unroll
      for (int x = 0; x < kRowsInFlight; ++x) {
        const int n = n0 + x * kGroups;
        const float s = row16_sum(dot_bf16x8(u[x], q8));
        if (c == 0 && n < nk) sc[n] = row[x] >= 0 ? s * cs : -INFINITY;
      }
    }
  }
  __syncthreads();
  float mx = -INFINITY;
  for (int n = tid; n < nk; n += kT) mx = fmaxf(mx, sc[n]);
  mx = wave_max(mx);
  if (lane == 0) red_v[w] = mx;
  __syncthreads();
  mx = red_v[0];
#pragma unroll
  for (int x = 1; x < kWaves; ++x) mx = fmaxf(mx, red_v[x]);
  float den = 0.f;
  for (int n = tid; n < nk; n += kT) {
    const float e = exp2f(sc[n] - mx);
    sc[n] = e;
    den += e;
  }
  den = wave_sum(den);
  __syncthreads();  // every thread has read red_v (max) before it is reused
  if (lane == 0) red_v[w] = den;
  __syncthreads();
  den = 0.f;
#pragma unroll
  for (int x = 0; x < kWaves; ++x) den += red_v[x];
  {
    const int kg = tid >> 4, c = tid & 15;
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    for (int n0 = kg; n0 < nk; n0 += kRowsInFlight * kGroups) {  // rows per lane group in flight
      uint4 u[kRowsInFlight];
      float pn[kRowsInFlight];
#pragma unroll
      for (int x = 0; x < kRowsInFlight; ++x) {
        const int n = n0 + x * kGroups;
        const int row = n < nk ? key_row(n) : -1;
        u[x] = *reinterpret_cast<const uint4*>(p.v + cbase + (int64_t)max(row, 0) * rs + 8 * c);
        pn[x] = row >= 0 ? sc[n] : 0.f;  // empty slots and rows past the list weigh nothing
      }
#pragma unroll
      for (int x = 0; x < kRowsInFlight; ++x) {
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
    for (int r = 0; r < kGroups; ++r) s += part[r][tid];
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

hipError_t launch_sparse_prefill(const SparseParams& p, int32_t* sel, hipStream_t stream) {
  hipError_t e = launch_sparse_means(p, 0, p.T / kSB, stream);
  if (e != hipSuccess) return e;
  const int64_t nqb = (p.T + kSB - 1) / kSB;
  const unsigned grid = (unsigned)((nqb * p.H * p.B + 7) / 8 * 8);  // see xcd_item
  const size_t sel_lds = (size_t)(p.T / kSB) * (sizeof(float) + sizeof(uint16_t)) + 16;
  hipLaunchKernelGGL(la_sparse_select_kernel, dim3(grid), dim3(64), sel_lds, stream, p, sel);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(la_sparse_attn_kernel, dim3(grid), dim3(64), 0, stream, p, sel);
  return hipGetLastError();
}

hipError_t launch_sparse_decode(const SparseParams& p, hipStream_t stream) {
  hipLaunchKernelGGL(la_sparse_decode_kernel, dim3((unsigned)(p.B * p.H)), dim3(kDecodeThreads), 0, stream, p);
  return hipGetLastError();
}

}  // namespace la
