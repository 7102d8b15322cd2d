// router.hip - the router projection before the path:
//   logits[t][e] = sum_c x[t][c] * Wr[e][c]
// x bf16 [T][H], Wr fp32 [E][H], logits fp32 [T][E], fp32 accumulation
// (the router picks each token's experts from these logits: page
// "hn.213312.xyz/article/49090233", section on how it works; the pages do
// not give the router's form, so the weights are a synthetic fp32 matrix).
//
// Few tokens (decode, T <= 4): the projection streams Wr once (25.7 MB at
// 896 x 7168), so it is a GEMV, one block per expert row.
// More tokens: a tiled fp32 GEMM, 32 tokens x 64 experts per block of 256
// threads, K tiles of 32 in LDS (x converted to fp32 as it is staged), each
// thread 2 tokens x 4 experts; every output is one thread's sum over K in
// ascending order.
#include "moe_internal.h"

namespace {

constexpr int kGemvTokens = 4;
constexpr int kThreads = 256;
constexpr int kWaves = kThreads / MOE_WAVE;

__device__ __forceinline__ float bf16_lo(uint32_t v) { return __uint_as_float(v << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t v) { return __uint_as_float(v & 0xFFFF0000u); }

// One block per expert row: wave w streams the w-th quarter of the row (at
// H = 7168 seven float4 per lane, all in flight at once) against the tokens'
// x read straight from global memory (a few KB, cache-resident), and the
// four waves' butterfly sums meet in LDS in wave order.
template <int TT>
__global__ __launch_bounds__(kThreads) void router_gemv_kernel(const uint16_t* __restrict__ x, int H,
                                                               const float* __restrict__ wr, int E,
                                                               float* __restrict__ logits, int T) {
  __shared__ float s_part[kWaves][TT];
  const int lane = threadIdx.x & (MOE_WAVE - 1), wave = threadIdx.x / MOE_WAVE;
  const int e = blockIdx.x;
  const int n4 = H >> 2, q4 = n4 / kWaves;  // float4 per row, per wave (H % 32 == 0: q4 even)
  const int c_beg = wave * q4, c_end = c_beg + q4;
  const float4* row = (const float4*)(wr + (int64_t)e * H);
  float acc[TT];
#pragma unroll
  for (int t = 0; t < TT; ++t) acc[t] = 0.0f;
  constexpr int kBatch = 7;
  for (int c0 = c_beg + lane; c0 < c_end; c0 += MOE_WAVE * kBatch) {
    float4 wv[kBatch];
    uint2 xv[kBatch][TT];
#pragma unroll
    for (int b = 0; b < kBatch; ++b) {
      const int c = c0 + MOE_WAVE * b;
      const bool ok = c < c_end;
      wv[b] = ok ? row[c] : make_float4(0.0f, 0.0f, 0.0f, 0.0f);
#pragma unroll
      for (int t = 0; t < TT; ++t)
        xv[b][t] = ok && t < T ? ((const uint2*)(x + (int64_t)t * H))[c] : make_uint2(0u, 0u);
    }
#pragma unroll
    for (int b = 0; b < kBatch; ++b) {
#pragma unroll
      for (int t = 0; t < TT; ++t) {
        acc[t] += bf16_lo(xv[b][t].x) * wv[b].x;
        acc[t] += bf16_hi(xv[b][t].x) * wv[b].y;
        acc[t] += bf16_lo(xv[b][t].y) * wv[b].z;
        acc[t] += bf16_hi(xv[b][t].y) * wv[b].w;
      }
    }
  }
#pragma unroll
  for (int t = 0; t < TT; ++t) {
    const float v = wave_sum(acc[t]);
    if (lane == 0) s_part[wave][t] = v;
  }
  __syncthreads();
  if (threadIdx.x < T) {
    const int t = threadIdx.x;
    float v = s_part[0][t];
#pragma unroll
    for (int w = 1; w < kWaves; ++w) v += s_part[w][t];
    logits[(int64_t)t * E + e] = v;
  }
}

constexpr int kTileT = 32, kTileE = 64, kTileK = 32;

__global__ __launch_bounds__(kThreads) void router_gemm_kernel(const uint16_t* __restrict__ x, int H,
                                                               const float* __restrict__ wr, int E,
                                                               float* __restrict__ logits, int T) {
  __shared__ float s_x[kTileK][kTileT];  // k-major
  __shared__ float s_w[kTileK][kTileE];
  const int tid = threadIdx.x, tx = tid & 15, ty = tid >> 4;
  const int t0 = blockIdx.y * kTileT, e0 = blockIdx.x * kTileE;
  float acc[2][4] = {};
  // staging: the x tile (32 tokens x 32 k) as one uint2 of 4 bf16 per thread
  // (token tid/8, k 4*(tid%8)); the w tile (64 experts x 32 k) as two float4
  // per thread; both stored k-major
  for (int k0 = 0; k0 < H; k0 += kTileK) {
    {
      const int t = tid >> 3, kk = 4 * (tid & 7);
      float4 v = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
      if (t0 + t < T) {
        const uint2 b = *(const uint2*)(x + (int64_t)(t0 + t) * H + k0 + kk);
        v = make_float4(bf16_lo(b.x), bf16_hi(b.x), bf16_lo(b.y), bf16_hi(b.y));
      }
      s_x[kk + 0][t] = v.x;
      s_x[kk + 1][t] = v.y;
      s_x[kk + 2][t] = v.z;
      s_x[kk + 3][t] = v.w;
    }
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int i = tid + kThreads * h;  // 512 float4 = 64 experts x 8 float4
      const int ee = i >> 3, kk = 4 * (i & 7);
      float4 v = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
      if (e0 + ee < E) v = *(const float4*)(wr + (int64_t)(e0 + ee) * H + k0 + kk);
      s_w[kk + 0][ee] = v.x;
      s_w[kk + 1][ee] = v.y;
      s_w[kk + 2][ee] = v.z;
      s_w[kk + 3][ee] = v.w;
    }
    __syncthreads();
#pragma unroll 8
    for (int kk = 0; kk < kTileK; ++kk) {
      const float2 xv = *(const float2*)&s_x[kk][2 * ty];
      const float4 wv = *(const float4*)&s_w[kk][4 * tx];
      acc[0][0] += xv.x * wv.x;
      acc[0][1] += xv.x * wv.y;
      acc[0][2] += xv.x * wv.z;
      acc[0][3] += xv.x * wv.w;
      acc[1][0] += xv.y * wv.x;
      acc[1][1] += xv.y * wv.y;
      acc[1][2] += xv.y * wv.z;
      acc[1][3] += xv.y * wv.w;
    }
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int t = t0 + 2 * ty + i;
    if (t >= T) continue;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int e = e0 + 4 * tx + j;
      if (e < E) logits[(int64_t)t * E + e] = acc[i][j];
    }
  }
}

}  // namespace

namespace moe {

hipError_t launch_router_logits(const uint16_t* x, int T, int H, const float* wr, int E, float* logits,
                                hipStream_t s) {
  if (T == 0) return hipSuccess;
  if (T <= kGemvTokens) {
    const dim3 g(E), b(kThreads);
    if (T == 1)
      hipLaunchKernelGGL(router_gemv_kernel<1>, g, b, 0, s, x, H, wr, E, logits, T);
    else
      hipLaunchKernelGGL(router_gemv_kernel<kGemvTokens>, g, b, 0, s, x, H, wr, E, logits, T);
  } else {
    const dim3 g((E + kTileE - 1) / kTileE, (T + kTileT - 1) / kTileT), b(kThreads);
    hipLaunchKernelGGL(router_gemm_kernel, g, b, 0, s, x, H, wr, E, logits, T);
  }
  return hipGetLastError();
}

}  // namespace moe
