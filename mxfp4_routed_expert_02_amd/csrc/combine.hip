// combine.hip - weighted combine of the routed rows back to tokens, and the
// RMS rescale that joins stacked layers (gfx950).
//
// combine: out[t][n] = sum_j w[t][j] * y_rows[row_pos[t*k+j]][n], j ascending.
// nck blocks per token (blockIdx.x = t * nck + chunk), 4 consecutive outputs per thread
// with 16-byte loads; the k (weight, position) pairs are wave-uniform.
#include "moe_internal.h"

namespace {

constexpr int kThreads = 256;
constexpr int kCombineThreads = 64;

// a thread's loads are issued before its sums, 16 rows at a time (k <= 32),
// so the usual k = 16 takes one round trip; they carry the non-temporal
// hint (prefill4096's combine streams 1.9 GB of y rows it reads once)
__global__ __launch_bounds__(kCombineThreads) void combine_vec4_kernel(const float* __restrict__ y_rows,
                                                                       const float* __restrict__ w,
                                                                       const int32_t* __restrict__ row_pos, int k,
                                                                       int H, int nck, float* __restrict__ out) {
  const int t = blockIdx.x / nck;
  const int i = (blockIdx.x - t * nck) * kCombineThreads + threadIdx.x;  // float4 index
  if (4 * i >= H) return;
  const float* wt = w + (int64_t)t * k;
  const int32_t* rp = row_pos + (int64_t)t * k;
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int j0 = 0; j0 < k; j0 += 16) {
    float4 y[16];
#pragma unroll
    for (int u = 0; u < 16; ++u)
      if (j0 + u < k) {  // each y row is read once: non-temporal loads
        const f32x4_t v = __builtin_nontemporal_load((const f32x4_t*)(y_rows + (int64_t)rp[j0 + u] * H) + i);
        y[u] = make_float4(v.x, v.y, v.z, v.w);
      }
#pragma unroll
    for (int u = 0; u < 16; ++u) {
      if (j0 + u < k) {
        const float c = wt[j0 + u];
        acc.x += c * y[u].x;
        acc.y += c * y[u].y;
        acc.z += c * y[u].z;
        acc.w += c * y[u].w;
      }
    }
  }
  ((float4*)(out + (int64_t)t * H))[i] = acc;
}

__global__ __launch_bounds__(kThreads) void combine_scalar_kernel(const float* __restrict__ y_rows,
                                                                  const float* __restrict__ w,
                                                                  const int32_t* __restrict__ row_pos, int k,
                                                                  int H, int nck, float* __restrict__ out) {
  const int t = blockIdx.x / nck;
  const int n = (blockIdx.x - t * nck) * kThreads + threadIdx.x;
  if (n >= H) return;
  float acc = 0.0f;
  for (int j = 0; j < k; ++j)
    acc += w[(int64_t)t * k + j] * y_rows[(int64_t)row_pos[(int64_t)t * k + j] * H + n];
  out[(int64_t)t * H + n] = acc;
}

// one block per token: sum of squares -> 1/sqrt(mean + eps) -> bf16 RNE
// One block of 1024 threads per token: each thread keeps up to 4 float4 of
// y in registers (H <= 16384), so y is read once; the sum of squares meets
// in a wave butterfly and then across the 16 waves in LDS.

__global__ __launch_bounds__(kRmsThreads) void rms_rescale_kernel(const float* __restrict__ y, int H, float eps,
                                                                  uint16_t* __restrict__ x_next) {
  __shared__ float s_part[kRmsThreads / MOE_WAVE];
  const int t = blockIdx.x;
  const int n4 = H >> 2;
  const float4* yr = (const float4*)(y + (int64_t)t * H);
  float4 v[kRmsVec];
  float ss = 0.0f;
#pragma unroll
  for (int i = 0; i < kRmsVec; ++i) {
    const int c = threadIdx.x + kRmsThreads * i;
    v[i] = c < n4 ? yr[c] : make_float4(0.0f, 0.0f, 0.0f, 0.0f);
  }
#pragma unroll
  for (int i = 0; i < kRmsVec; ++i) ss += sumsq4(v[i]);
  ss = wave_sum(ss);
  if ((threadIdx.x & (MOE_WAVE - 1)) == 0) s_part[threadIdx.x / MOE_WAVE] = ss;
  __syncthreads();
  float tot = 0.0f;
#pragma unroll
  for (int i = 0; i < kRmsThreads / MOE_WAVE; ++i) tot += s_part[i];
  const float r = rms_factor(tot, H, eps);
  uint2* xo = (uint2*)(x_next + (int64_t)t * H);
#pragma unroll
  for (int i = 0; i < kRmsVec; ++i) {
    const int c = threadIdx.x + kRmsThreads * i;
    if (c < n4) {
      const uint32_t lo = f32_to_bf16_rne_dev(v[i].x * r) | ((uint32_t)f32_to_bf16_rne_dev(v[i].y * r) << 16);
      const uint32_t hi = f32_to_bf16_rne_dev(v[i].z * r) | ((uint32_t)f32_to_bf16_rne_dev(v[i].w * r) << 16);
      xo[c] = make_uint2(lo, hi);
    }
  }
}

// combine then RMS rescale, one block of 1024 threads per token: thread c
// of the rescale's layout forms its float4 of out with the combine's
// arithmetic (j ascending), stores it, and goes on as rms_rescale_kernel
// with those values in registers, so out and x_next equal the two separate
// launches' bit for bit.
__global__ __launch_bounds__(kRmsThreads) void combine_rms_kernel(const float* __restrict__ y_rows,
                                                                  const float* __restrict__ w,
                                                                  const int32_t* __restrict__ row_pos, int k, int H,
                                                                  float eps, float* __restrict__ out,
                                                                  uint16_t* __restrict__ x_next) {
  __shared__ float s_part[kRmsThreads / MOE_WAVE];
  const int t = blockIdx.x;
  const int n4 = H >> 2;
  const float* wt = w + (int64_t)t * k;
  const int32_t* rp = row_pos + (int64_t)t * k;
  float4 v[kRmsVec];
#pragma unroll
  for (int i = 0; i < kRmsVec; ++i) v[i] = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
  for (int j0 = 0; j0 < k; j0 += 8) {
#pragma unroll
    for (int i = 0; i < kRmsVec; ++i) {
      const int c = threadIdx.x + kRmsThreads * i;
      if (c >= n4) continue;
      float4 y[8];
#pragma unroll
      for (int u = 0; u < 8; ++u)
        if (j0 + u < k) y[u] = ((const float4*)(y_rows + (int64_t)rp[j0 + u] * H))[c];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        if (j0 + u < k) {
          const float cw = wt[j0 + u];
          v[i].x += cw * y[u].x;
          v[i].y += cw * y[u].y;
          v[i].z += cw * y[u].z;
          v[i].w += cw * y[u].w;
        }
      }
    }
  }
  float4* orow = (float4*)(out + (int64_t)t * H);
  float ss = 0.0f;
#pragma unroll
  for (int i = 0; i < kRmsVec; ++i) {
    const int c = threadIdx.x + kRmsThreads * i;
    if (c < n4) orow[c] = v[i];
  }
#pragma unroll
  for (int i = 0; i < kRmsVec; ++i) ss += sumsq4(v[i]);
  ss = wave_sum(ss);
  if ((threadIdx.x & (MOE_WAVE - 1)) == 0) s_part[threadIdx.x / MOE_WAVE] = ss;
  __syncthreads();
  float tot = 0.0f;
#pragma unroll
  for (int i = 0; i < kRmsThreads / MOE_WAVE; ++i) tot += s_part[i];
  const float r = rms_factor(tot, H, eps);
  uint2* xo = (uint2*)(x_next + (int64_t)t * H);
#pragma unroll
  for (int i = 0; i < kRmsVec; ++i) {
    const int c = threadIdx.x + kRmsThreads * i;
    if (c < n4) {
      const uint32_t lo = f32_to_bf16_rne_dev(v[i].x * r) | ((uint32_t)f32_to_bf16_rne_dev(v[i].y * r) << 16);
      const uint32_t hi = f32_to_bf16_rne_dev(v[i].z * r) | ((uint32_t)f32_to_bf16_rne_dev(v[i].w * r) << 16);
      xo[c] = make_uint2(lo, hi);
    }
  }
}

}  // namespace

namespace moe {

hipError_t launch_combine_rms(const float* y_rows, const float* w, const int32_t* row_pos, int T, int k, int H,
                              float eps, float* out, uint16_t* x_next, hipStream_t s) {
  if (T == 0) return hipSuccess;
  static_assert(MOE_MAX_DIM <= 4 * kRmsVec * kRmsThreads, "one register tile per token");
  hipLaunchKernelGGL(combine_rms_kernel, dim3(T), dim3(kRmsThreads), 0, s, y_rows, w, row_pos, k, H, eps, out,
                     x_next);
  return hipGetLastError();
}

hipError_t launch_combine(const float* y_rows, const float* w, const int32_t* row_pos, int T, int k, int H,
                          float* out, hipStream_t s) {
  if (T == 0) return hipSuccess;
  if (H % 4 == 0) {
    const int nck = (H / 4 + kCombineThreads - 1) / kCombineThreads;
    hipLaunchKernelGGL(combine_vec4_kernel, dim3((unsigned)T * nck), dim3(kCombineThreads), 0, s, y_rows, w, row_pos,
                       k, H, nck, out);
  } else {
    const int nck = (H + kThreads - 1) / kThreads;
    hipLaunchKernelGGL(combine_scalar_kernel, dim3((unsigned)T * nck), dim3(kThreads), 0, s, y_rows, w, row_pos,
                       k, H, nck, out);
  }
  return hipGetLastError();
}

hipError_t launch_rms_rescale(const float* y, int T, int H, float eps, uint16_t* x_next, hipStream_t s) {
  if (T == 0) return hipSuccess;
  // H is a multiple of 32 and at most MOE_MAX_DIM = 16384 = 4 * 4 * 1024
  static_assert(MOE_MAX_DIM <= 4 * kRmsVec * kRmsThreads, "one register tile per token");
  hipLaunchKernelGGL(rms_rescale_kernel, dim3(T), dim3(kRmsThreads), 0, s, y, H, eps, x_next);
  return hipGetLastError();
}

}  // namespace moe
