// Dense projection y = x W^T on gfx950 (bf16 inputs, fp32 accumulation, bf16
// output): the q/k/v/gate projections in front of the linear-attention layer and
// the output projection after its gate.  The layer's structure (hidden size 4096,
// 32 heads of 128, GQA turned into MHA, output gate) is the one the report gives
// for its linear-attention modules ("創新Transformer！面壁基於稀疏-線性混合架構SALA
// 訓練9B模型，端側跑通百萬上下文", 04 技術報告 > 02 模型架構 > (3) 線性注意力模塊).
//
// x: [M, K] row-major, W: [N, K] row-major (the nn.Linear weight layout), y:
// [M, N] row-major, optionally split by columns into `nsplit` separate [M, N /
// nsplit] tensors (the fused q/k/v/gate projection writes q, k, v, g directly).
// Requires K % 64 == 0 and (N / nsplit) % 256 == 0; M is arbitrary.
//
// Workgroup tile 256 x 256, eight waves: wave (wm, wn) computes rows
// [64 wm, 64 wm + 64) x columns [128 wn, 128 wn + 128) of the tile as 4 x 8
// accumulator tiles of v_mfma_f32_16x16x32_bf16.  Both operands are
// K-contiguous, so every MFMA operand is one 16-byte LDS read per lane.  The
// tile is formed transposed (W rows as the A operand), so each lane ends up
// holding 4 consecutive output columns of one row and stores them as 8 bytes.
//
// Two kernels share that tiling:
//   * la_linear_ring_kernel (K % 128 == 0, the projection shapes): K steps of
//     64 double-buffered in LDS, filled by direct global-to-LDS loads (16 bytes
//     per lane, no register staging and no LDS store instructions, whole 128-byte
//     lines per request); 128-byte rows with an XOR swizzle of the 16-byte pieces
//     keep the operand reads conflict-free.  The two waves of each SIMD take turns
//     between workgroup barriers: one issues a 32-deep step's MFMAs while the other
//     reads the next step's operands from LDS.  One workgroup per compute unit walks
//     the tiles blockIdx.x, blockIdx.x + gridDim.x, ...; a tile's first two stages
//     are loaded while the previous tile's outputs are stored.
//   * la_linear_kernel (any K % 64 == 0): K steps of 64 double-buffered in LDS
//     through registers.
// Both sum each output in the same order (32-deep MFMA steps in K order), so
// they give identical results.
#include "la_device.hpp"
#include "la_internal.hpp"

namespace la {
namespace {

constexpr int kBM = 256, kBN = 256, kBK = 64;
constexpr int kGemmThreads = 512;
// 160-byte LDS rows: the operand reads (16 rows x 4 lane groups, 16 bytes each) are
// conflict-free there, while 144-byte rows cost 4 conflict cycles per read (gfx950
// counters); the 16-byte staging stores cost the same at both strides.
constexpr int kLdsRow = kBK * 2 + 32;
constexpr int kLdsTile = kBM * kLdsRow;        // one 256 x 64 bf16 tile
constexpr int kChunksPerThread = kBM * kBK / 8 / kGemmThreads;  // 16-byte pieces of a tile per thread (4)

__global__ __launch_bounds__(kGemmThreads) void la_linear_kernel(LinearParams p) {
  __shared__ __attribute__((aligned(16))) uint8_t sA[2][kLdsTile];  // x rows
  __shared__ __attribute__((aligned(16))) uint8_t sB[2][kLdsTile];  // W rows

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int n16 = lane & 15, g4 = lane >> 4;
  const int wm = w & 3, wn = w >> 2;
  const int tiles_n = p.N / kBN;
  const int tm = blockIdx.x / tiles_n, tn = blockIdx.x - tm * tiles_n;
  const int64_t m0 = (int64_t)tm * kBM;
  const int n0 = tn * kBN;

  // staging: piece i = tid + 512 u covers row i / 8, bytes 16 (i % 8) .. of the K step
  const uint16_t* a_src[kChunksPerThread];
  const uint16_t* b_src[kChunksPerThread];
  int lds_off[kChunksPerThread];
#pragma unroll
  for (int u = 0; u < kChunksPerThread; ++u) {
    const int i = tid + kGemmThreads * u, r = i >> 3, c = i & 7;
    const int64_t row = m0 + r < p.M ? m0 + r : p.M - 1;  // rows past M re-read the last row
    a_src[u] = p.x + row * p.K + 8 * c;
    b_src[u] = p.w + (int64_t)(n0 + r) * p.K + 8 * c;
    lds_off[u] = r * kLdsRow + 16 * c;
  }
  uint4 ra[kChunksPerThread], rb[kChunksPerThread];
  auto load = [&](int kt) {
#pragma unroll
    for (int u = 0; u < kChunksPerThread; ++u) {
      ra[u] = *reinterpret_cast<const uint4*>(a_src[u] + kt * kBK);
      rb[u] = *reinterpret_cast<const uint4*>(b_src[u] + kt * kBK);
    }
  };
  auto stage = [&](int buf) {
#pragma unroll
    for (int u = 0; u < kChunksPerThread; ++u) {
      lds_st<uint4>(sA[buf], lds_off[u], ra[u]);
      lds_st<uint4>(sB[buf], lds_off[u], rb[u]);
    }
  };

  f32x4 acc[4][8];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int nk = p.K / kBK;
  load(0);
  stage(0);
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    const int buf = kt & 1;
    if (kt + 1 < nk) load(kt + 1);
#pragma unroll
    for (int kk = 0; kk < kBK / 32; ++kk) {
      bf16x8 xa[4], wb[8];
#pragma unroll
      for (int i = 0; i < 4; ++i)
        xa[i] = as_bf16x8(lds_ld<uint4>(sA[buf], (64 * wm + 16 * i + n16) * kLdsRow + 64 * kk + 16 * g4));
#pragma unroll
      for (int j = 0; j < 8; ++j)
        wb[j] = as_bf16x8(lds_ld<uint4>(sB[buf], (128 * wn + 16 * j + n16) * kLdsRow + 64 * kk + 16 * g4));
      // D[4 g + r][n16] = sum_k W[col 4 g + r][k] x[row n16][k] = y[row n16][col 4 g + r]
      // The wave issuing its MFMA block takes issue priority over the SIMD's other wave
      // (then busy with LDS reads, loads or stores): 5-6% on the projection shapes.
      __builtin_amdgcn_s_setprio(1);
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 8; ++j) acc[i][j] = mma(wb[j], xa[i], acc[i][j]);
      __builtin_amdgcn_s_setprio(0);
    }
    if (kt + 1 < nk) stage(buf ^ 1);
    __syncthreads();
  }

  // epilogue: lane holds y[m0 + 64 wm + 16 i + n16][n0 + 128 wn + 16 j + 4 g .. + 3]
  const int split_cols = p.N / p.nsplit;
  const int part = n0 / split_cols;
  uint16_t* const out = p.y[part];
  const int col0 = n0 - part * split_cols + 128 * wn + 4 * g4;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int64_t row = m0 + 64 * wm + 16 * i + n16;
    if (row < p.M) {
      uint16_t* dst = out + row * split_cols + col0;
#pragma unroll
      for (int j = 0; j < 8; ++j)
        *reinterpret_cast<uint2*>(dst + 16 * j) =
            make_uint2(pack2(acc[i][j][0], acc[i][j][1]), pack2(acc[i][j][2], acc[i][j][3]));
    }
  }
}

// ---------------------------------------------------------------------------
// Ring kernel.  Stage kt (K columns [64 kt, 64 kt + 64)) of both operands sits in
// slot kt % 2: a 256-row x 128-byte tile per operand, each row's eight 16-byte
// pieces stored at piece position c ^ ((row / 2) % 8).  A wave loads 8 rows per
// direct load (lane i: row i / 8, position i % 8), so it fetches the global piece
// that belongs there, and every 8 lanes read one 128-byte row: each direct load
// asks L2 for whole 128-byte lines.  (With 32-deep stages a row gave 64 bytes, and
// the kernel sent twice the requests for the same bytes: 3.6-3.8 ms against
// 3.5 ms for the q/k/v/gate projection of a 32K layer.)  The MFMA reads of 16 rows
// at one piece column hit 16 different 16-byte bank groups.
constexpr int kRingBK = 64, kRingSlots = 2;
constexpr int kRingTile = kBM * kRingBK * 2;  // 32 KiB per operand per stage

__device__ __forceinline__ int ring_pos(int row, int piece) { return piece ^ ((row >> 1) & 7); }

// Direct global -> LDS load of 16 bytes per lane from base + off (lane i's bytes
// land at LDS byte address lds + 16 i).  Issued from assembly so that the
// compiler, which cannot tell the ring slots apart across loop iterations, adds
// no waits of its own (it would wait for every load before each LDS read); every
// wait on these loads is explicit in the kernel.  No register is written.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void dma16(const void* base, uint32_t off, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(off), "s"(base), "s"(lds)
               : "memory", "m0");
}
#pragma clang diagnostic pop

__device__ __forceinline__ uint32_t lds_addr(const uint8_t* ptr) {
  return __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(const __attribute__((address_space(3))) uint8_t*)ptr);
}

__global__ __launch_bounds__(kGemmThreads) void la_linear_ring_kernel(LinearParams p) {
  __shared__ __attribute__((aligned(1024))) uint8_t sA0[kRingTile], sA1[kRingTile];
  __shared__ __attribute__((aligned(1024))) uint8_t sB0[kRingTile], sB1[kRingTile];

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int n16 = lane & 15, g4 = lane >> 4;
  const int wm = w & 3, wn = w >> 2;
  const int tiles_n = p.N / kBN;
  const int64_t ntiles = (p.M + kBM - 1) / kBM * (int64_t)tiles_n;
  const int K = p.K;
  const int nk = K / kRingBK;
  const uint32_t la[2] = {lds_addr(sA0), lds_addr(sA1)};
  const uint32_t lb[2] = {lds_addr(sB0), lds_addr(sB1)};

  // per tile: this wave loads rows 32 w .. 32 w + 31 of both operand tiles, 8 per load
  const uint8_t* xbase;
  const uint8_t* wbase;
  uint32_t aoff[4], boff[4];
  auto setup = [&](int64_t t) {
    const int tm = (int)(t / tiles_n), tn = (int)(t - (int64_t)tm * tiles_n);
    const int64_t m0 = (int64_t)tm * kBM;
    xbase = reinterpret_cast<const uint8_t*>(p.x + m0 * K);
    wbase = reinterpret_cast<const uint8_t*>(p.w + (int64_t)tn * kBN * K);
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int row = 32 * w + 8 * u + (lane >> 3);
      const int piece = ring_pos(row, lane & 7);  // the position is its own inverse
      const int arow = m0 + row < p.M ? row : (int)(p.M - 1 - m0);  // rows past M re-read the last row
      aoff[u] = (uint32_t)(arow * K + 8 * piece) * 2u;
      boff[u] = (uint32_t)(row * K + 8 * piece) * 2u;
    }
  };
  auto issue = [&](int kt, int slot) {
    const uint8_t* xa = xbase + (int64_t)kt * kRingBK * 2;
    const uint8_t* wa = wbase + (int64_t)kt * kRingBK * 2;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const uint32_t rows = __builtin_amdgcn_readfirstlane((32 * w + 8 * u) * 128);
      dma16(xa, aoff[u], la[slot] + rows);
      dma16(wa, boff[u], lb[slot] + rows);
    }
  };

  const int group = __builtin_amdgcn_readfirstlane(w >> 2);
  f32x4 acc[4][8];
  bf16x8 xa[2][4], wb[2][8];
  auto read = [&](int buf, const uint8_t* A, const uint8_t* B, int ks) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = 64 * wm + 16 * i + n16;
      xa[buf][i] = as_bf16x8(lds_ld<uint4>(A, row * 128 + 16 * ring_pos(row, g4 + 4 * ks)));
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int row = 128 * wn + 16 * j + n16;
      wb[buf][j] = as_bf16x8(lds_ld<uint4>(B, row * 128 + 16 * ring_pos(row, g4 + 4 * ks)));
    }
    if (ks == 1) asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  };
  auto mfma = [&](int buf) {
    __builtin_amdgcn_s_setprio(1);
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 8; ++j) acc[i][j] = mma(wb[buf][j], xa[buf][i], acc[i][j]);
    __builtin_amdgcn_s_setprio(0);
  };
  auto bar = [&]() {
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
    asm volatile("" ::: "memory");
  };
  // tiles blockIdx.x + k gridDim.x; with gridDim.x a multiple of 8, tile t stays on
  // XCD t % 8, as with one workgroup per tile
  int64_t t = blockIdx.x;
  setup(t);
  issue(0, 0);
  issue(1, 1);  // nk >= 2
  for (;;) {
    const int tm = (int)(t / tiles_n), tn = (int)(t - (int64_t)tm * tiles_n);
    const int64_t m0 = (int64_t)tm * kBM;
    const int n0 = tn * kBN;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 8; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
    asm volatile("s_waitcnt vmcnt(8)" ::: "memory");  // stage 1's 8 loads may still be out
    bar();
    read(0, sA0, sB0, 0);
    if (group == 1) bar();
    for (int u = 0; u < nk; ++u) {
      const int slot = u & 1;
      const uint8_t* const Ac = slot ? sA1 : sA0;
      const uint8_t* const Bc = slot ? sB1 : sB0;
      const uint8_t* const An = slot ? sA0 : sA1;
      const uint8_t* const Bn = slot ? sB0 : sB1;
      read(1, Ac, Bc, 1);
      if (group == 1) asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      bar();
      mfma(0);
      if (group == 0) asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      bar();
      if (u + 2 < nk) issue(u + 2, slot);
      if (u + 1 < nk) read(0, An, Bn, 0);
      bar();
      mfma(1);
      bar();
    }
    if (group == 0) bar();
    // every wave has read this tile's last stage: the next tile's first two stages
    // go out before this tile's outputs
    const int64_t tnext = t + gridDim.x;
    if (tnext < ntiles) {
      setup(tnext);
      issue(0, 0);
      issue(1, 1);
    }
    const int split_cols = p.N / p.nsplit;
    const int part = n0 / split_cols;
    uint16_t* const out = p.y[part];
    const int col0 = n0 - part * split_cols + 128 * wn + 4 * g4;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int64_t row = m0 + 64 * wm + 16 * i + n16;
      if (row < p.M) {
        uint16_t* dst = out + row * split_cols + col0;
#pragma unroll
        for (int j = 0; j < 8; ++j)
          *reinterpret_cast<uint2*>(dst + 16 * j) =
              make_uint2(pack2(acc[i][j][0], acc[i][j][1]), pack2(acc[i][j][2], acc[i][j][3]));
      }
    }
    if (tnext >= ntiles) break;
    t = tnext;
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // no load may still write LDS when the workgroup ends
}

}  // namespace

hipError_t launch_linear(const LinearParams& p, hipStream_t stream) {
  const int64_t tiles = ((p.M + kBM - 1) / kBM) * (int64_t)(p.N / kBN);
  // the ring kernel forms per-lane byte offsets within a 256-row tile in 32 bits
  const bool ring = p.K % (kRingSlots * kRingBK) == 0 && (int64_t)kBM * p.K * 2 < ((int64_t)1 << 32);
  // the ring kernel holds 128 KiB of LDS, so one workgroup per compute unit (256 on
  // gfx950); it walks the tiles, and any grid size gives the same results
  constexpr int64_t kRingGrid = 256;
  if (ring)
    hipLaunchKernelGGL(la_linear_ring_kernel, dim3((unsigned)(tiles < kRingGrid ? tiles : kRingGrid)), dim3(kGemmThreads),
                       0, stream, p);
  else
    hipLaunchKernelGGL(la_linear_kernel, dim3((unsigned)tiles), dim3(kGemmThreads), 0, stream, p);
  return hipGetLastError();
}

}  // namespace la
