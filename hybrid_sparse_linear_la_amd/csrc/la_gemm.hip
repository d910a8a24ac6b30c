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
// Workgroup tile 256 x 256, K step 64, LDS double-buffered (160 KiB).  Eight
// waves, wave (wm, wn) computes rows [64 wm, 64 wm + 64) x columns
// [128 wn, 128 wn + 128) of the tile as 4 x 8 accumulator tiles of
// v_mfma_f32_16x16x32_bf16.  Both operands are K-contiguous, so every MFMA
// operand is one 16-byte LDS read per lane.  The tile is formed transposed
// (W rows as the A operand), so each lane ends up holding 4 consecutive output
// columns of one row and stores them as 8 bytes.
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

}  // namespace

hipError_t launch_linear(const LinearParams& p, hipStream_t stream) {
  const int64_t tiles = ((p.M + kBM - 1) / kBM) * (int64_t)(p.N / kBN);
  hipLaunchKernelGGL(la_linear_kernel, dim3((unsigned)tiles), dim3(kGemmThreads), 0, stream, p);
  return hipGetLastError();
}

}  // namespace la
