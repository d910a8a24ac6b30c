// Single-token decode of the gated causal linear-attention layer on gfx950.
//
// Per (b, h): qh = RoPE(RMSNorm(q)), kh = RoPE(RMSNorm(k)) at position pos;
// S <- S + kh v^T in place; o = sigmoid(g) * (qh S).  The state update is the
// recurrence of "MiniCPM-SALA: Hybridizing Sparse and Linear Attention for
// Efficient Long-Context Modeling" (前置知识 > 线性注意力): constant work and
// memory per token, i.e. one read and one write of the D x D fp32 state.
//
// The step is bound by HBM: per (b, h) it moves 128 KiB of state and 1.25 KiB
// of token data for 64 Ki flops.  One 256-thread workgroup per (b, h): every
// thread owns 4 consecutive value columns (one float4) of 16 key rows, issues
// all 16 row loads before using any (64 KiB in flight per workgroup, fully
// coalesced: a wave covers two full 512-byte rows per load), updates and writes
// back, and reduces qh . S over its rows; the 8 row groups meet in LDS.
//
// Batches whose states exceed kStreamStateBytes write them back with non-temporal
// stores.  Measured per step (32 heads): at 128 and 192 MiB of state plain stores
// are 2-3% faster (the states stay in the 256 MB memory-side cache from step to
// step); at 256, 320, 384 and 512 MiB non-temporal stores are 8%, 12%, 22% and 25%
// faster; at 768 MiB both run at the same 5.1-5.2 TB/s.
#include "la_device.hpp"
#include "la_internal.hpp"

namespace la {
namespace {

constexpr int kThreads = 256;
constexpr int64_t kStreamStateBytes = (int64_t)192 << 20;

typedef float f32x4v __attribute__((ext_vector_type(4)));
__device__ __forceinline__ void store_state(float4* dst, float4 s, bool stream) {
  if (stream) {
    const f32x4v v = {s.x, s.y, s.z, s.w};
    __builtin_nontemporal_store(v, reinterpret_cast<f32x4v*>(dst));
  } else {
    *dst = s;
  }
}
constexpr int kRowGroups = kThreads / (kD / 4);  // 8
constexpr int kRowsPerThread = kD / kRowGroups;  // 16

template <bool kStreamState>
__global__ __launch_bounds__(kThreads) void la_decode_kernel(DecodeParams p) {
  __shared__ float sq[kD], sk[kD], sv[kD], sgate[kD];
  __shared__ float4 spart[kRowGroups][kD / 4];

  const int tid = threadIdx.x;
  const int64_t bh = blockIdx.x;  // b * H + h
  // token row and state of this (b, h): row b of [B, H, D] inputs and state b, or
  // for a packed batch the row and sequence of single-token sequence b
  int64_t tok = bh * kD, sbh = bh, pos = p.pos;
  if (p.rows != nullptr) {
    const DecDesc d = p.rows[bh / p.H];
    const int64_t h = bh % p.H;
    tok = ((int64_t)d.t * p.H + h) * kD;
    sbh = (int64_t)d.seq * p.H + h;
    pos = d.pos;
  }

  const int cg = tid & 31;  // value columns 4cg .. 4cg + 3
  const int rgp = tid >> 5; // key rows rgp + 8 m
  float4* Sbh = reinterpret_cast<float4*>(p.S + sbh * kD * kD);
  const float4* Sin = reinterpret_cast<const float4*>((p.S_in ? p.S_in : p.S) + sbh * kD * kD);

  // Issue the state loads first; the prologue overlaps their latency.
  float4 sreg[kRowsPerThread];
#pragma unroll
  for (int m = 0; m < kRowsPerThread; ++m)
    sreg[m] = p.S_zero ? make_float4(0.f, 0.f, 0.f, 0.f) : Sin[(rgp + kRowGroups * m) * (kD / 4) + cg];

  if (tid < 64) {
    // wave 0: RMSNorm + RoPE of q and k; lane i holds the rotate-half pair (i, i + 64)
    const int i = tid;
    float q0 = bf2f(p.q[tok + i]), q1 = bf2f(p.q[tok + i + kHalf]);
    float k0 = bf2f(p.k[tok + i]), k1 = bf2f(p.k[tok + i + kHalf]);
    float ssq = q0 * q0 + q1 * q1, ssk = k0 * k0 + k1 * k1;
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
      ssq += __shfl_xor(ssq, off);
      ssk += __shfl_xor(ssk, off);
    }
    const float iq = rsqrt_(ssq * (1.0f / kD) + p.eps), ik = rsqrt_(ssk * (1.0f / kD) + p.eps);
    q0 *= iq * (p.qw ? p.qw[i] : 1.f);
    q1 *= iq * (p.qw ? p.qw[i + kHalf] : 1.f);
    k0 *= ik * (p.kw ? p.kw[i] : 1.f);
    k1 *= ik * (p.kw ? p.kw[i + kHalf] : 1.f);
    const float2 rot = rope_rotation(pos, p.freqs.rev[i]);
    sq[i] = q0 * rot.x - q1 * rot.y;
    sq[i + kHalf] = q1 * rot.x + q0 * rot.y;
    sk[i] = k0 * rot.x - k1 * rot.y;
    sk[i + kHalf] = k1 * rot.x + k0 * rot.y;
  } else if (tid < 64 + kD) {
    const int d = tid - 64;
    sv[d] = bf2f(p.v[tok + d]);
    sgate[d] = sigmoidf_(bf2f(p.g[tok + d]));
  }
  __syncthreads();

  const float4 vv = reinterpret_cast<const float4*>(sv)[cg];
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
  for (int m = 0; m < kRowsPerThread; ++m) {
    const int i = rgp + kRowGroups * m;
    const float kk = sk[i], qq = sq[i];
    float4 s = sreg[m];
    s.x = fmaf(kk, vv.x, s.x);
    s.y = fmaf(kk, vv.y, s.y);
    s.z = fmaf(kk, vv.z, s.z);
    s.w = fmaf(kk, vv.w, s.w);
    store_state(Sbh + i * (kD / 4) + cg, s, kStreamState);
    acc.x = fmaf(qq, s.x, acc.x);
    acc.y = fmaf(qq, s.y, acc.y);
    acc.z = fmaf(qq, s.z, acc.z);
    acc.w = fmaf(qq, s.w, acc.w);
  }
  spart[rgp][cg] = acc;
  __syncthreads();

  if (tid < kD / 4) {
    float4 u = spart[0][tid];
#pragma unroll
    for (int r = 1; r < kRowGroups; ++r) {
      const float4 x = spart[r][tid];
      u.x += x.x;
      u.y += x.y;
      u.z += x.z;
      u.w += x.w;
    }
    const float4 gg = reinterpret_cast<const float4*>(sgate)[tid];
    const uint2 packed = make_uint2(pack2(u.x * gg.x, u.y * gg.y), pack2(u.z * gg.z, u.w * gg.w));
    *reinterpret_cast<uint2*>(p.o + tok + 4 * tid) = packed;
  }
}

}  // namespace

hipError_t launch_decode(const DecodeParams& p, hipStream_t stream) {
  const dim3 grid((unsigned)((int64_t)p.B * p.H));
  if ((int64_t)p.B * p.H * kD * kD * (int64_t)sizeof(float) > kStreamStateBytes)
    hipLaunchKernelGGL(la_decode_kernel<true>, grid, dim3(kThreads), 0, stream, p);
  else
    hipLaunchKernelGGL(la_decode_kernel<false>, grid, dim3(kThreads), 0, stream, p);
  return hipGetLastError();
}

}  // namespace la
