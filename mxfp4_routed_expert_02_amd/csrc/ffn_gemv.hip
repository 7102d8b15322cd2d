// ffn_gemv.hip - MXFP4 dequant-GEMV kernels of the expert FFN (gfx950).
//
// Work unit: one active expert (blockIdx.y = slot in the active list, read
// on the device) x a tile of weight rows (blockIdx.x).  The expert's routed
// rows are taken MT at a time; their activations are staged in LDS and
// every 16-byte weight chunk (32 E2M1 codes = one MX block, one scale byte)
// is loaded once, dequantized in registers and applied to all MT rows.
// Each wave owns one weight row at a time, its lanes stride over the row's
// 32-value blocks, and a butterfly over the wavefront finishes the dot.
//
// gate/up: the block's gate row n and up row n are read together, so the
//          SiLU(g)*u epilogue stays in registers.  E2M1 -> bf16 (exact) and
//          v_dot2_f32_bf16 against the bf16 activations (exact products,
//          fp32 sums); the E8M0 scale multiplies each block's partial sum.
// down:    E2M1 -> fp32 (exact) and fp32 FMA against the fp32 h rows.
#include "moe_internal.h"

namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / MOE_WAVE;
constexpr int kRowsPerBlock = 16;

// 16 bytes = 32 E2M1 codes -> 16 bf16 pairs; pair j holds elements 2j, 2j+1.
__device__ __forceinline__ void dequant_bf16(const uint4 q, bf16x2_t (&v)[16]) {
  const uint32_t d[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    v[4 * i + 0] = fp4x2_to_bf16x2<0>(d[i]);
    v[4 * i + 1] = fp4x2_to_bf16x2<1>(d[i]);
    v[4 * i + 2] = fp4x2_to_bf16x2<2>(d[i]);
    v[4 * i + 3] = fp4x2_to_bf16x2<3>(d[i]);
  }
}

__device__ __forceinline__ void dequant_f32(const uint4 q, f32x2_t (&v)[16]) {
  const uint32_t d[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    v[4 * i + 0] = fp4x2_to_f32x2<0>(d[i]);
    v[4 * i + 1] = fp4x2_to_f32x2<1>(d[i]);
    v[4 * i + 2] = fp4x2_to_f32x2<2>(d[i]);
    v[4 * i + 3] = fp4x2_to_f32x2<3>(d[i]);
  }
}

// dot of a dequantized chunk with 32 bf16 activations (16 dwords in LDS)
__device__ __forceinline__ float chunk_dot_bf16(const bf16x2_t (&wv)[16], const uint32_t* xs) {
  const uint4* x4 = (const uint4*)xs;
  float acc = 0.0f;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint4 xx = x4[i];
    acc = dot2_bf16(wv[4 * i + 0], as_bf16x2(xx.x), acc);
    acc = dot2_bf16(wv[4 * i + 1], as_bf16x2(xx.y), acc);
    acc = dot2_bf16(wv[4 * i + 2], as_bf16x2(xx.z), acc);
    acc = dot2_bf16(wv[4 * i + 3], as_bf16x2(xx.w), acc);
  }
  return acc;
}

__device__ __forceinline__ float chunk_dot_f32(const f32x2_t (&wv)[16], const float* hs) {
  const float4* h4 = (const float4*)hs;
  float acc = 0.0f;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const float4 hh = h4[i];
    acc += wv[2 * i].x * hh.x;
    acc += wv[2 * i].y * hh.y;
    acc += wv[2 * i + 1].x * hh.z;
    acc += wv[2 * i + 1].y * hh.w;
  }
  return acc;
}

template <int MT>
__global__ __launch_bounds__(kThreads) void gateup_gemv_kernel(const uint16_t* __restrict__ x, int k,
                                                               moe_mxfp4_weights w,
                                                               const int32_t* __restrict__ offsets,
                                                               const int32_t* __restrict__ sorted_rows,
                                                               const int32_t* __restrict__ active,
                                                               float* __restrict__ h) {
  extern __shared__ uint32_t s_x[];  // [MT][H/2] bf16 pairs
  const int slot = blockIdx.y;
  if (slot >= active[0]) return;
  const int H = w.hidden, I = w.inter;
  const int e = active[1 + slot];
  const int p0 = offsets[e];
  const int cnt = offsets[e + 1] - p0;
  const int n0 = blockIdx.x * kRowsPerBlock;
  const int lane = threadIdx.x & (MOE_WAVE - 1), wave = threadIdx.x / MOE_WAVE;
  const int nb = H >> 5;
  const int64_t qrow = H >> 1;
  const uint8_t* gq = w.gate_q + (int64_t)e * w.expert_stride;
  const uint8_t* gs = w.gate_s + (int64_t)e * w.expert_stride;
  const uint8_t* uq = w.up_q + (int64_t)e * w.expert_stride;
  const uint8_t* us = w.up_s + (int64_t)e * w.expert_stride;
  const int xv = H >> 3;  // uint4 per activation row

  for (int m0 = 0; m0 < cnt; m0 += MT) {
    const int mt = min(MT, cnt - m0);
    __syncthreads();
    for (int i = threadIdx.x; i < mt * xv; i += kThreads) {
      const int m = i / xv, c = i - m * xv;
      const int64_t t = sorted_rows[p0 + m0 + m] / k;
      ((uint4*)(s_x + m * (H >> 1)))[c] = ((const uint4*)(x + t * H))[c];
    }
    __syncthreads();
    for (int r = wave; r < kRowsPerBlock; r += kWaves) {
      const int n = n0 + r;
      if (n >= I) break;
      float ag[MT], au[MT];
#pragma unroll
      for (int m = 0; m < MT; ++m) ag[m] = au[m] = 0.0f;
      const uint8_t* gqr = gq + (int64_t)n * qrow;
      const uint8_t* uqr = uq + (int64_t)n * qrow;
      const uint8_t* gsr = gs + (int64_t)n * nb;
      const uint8_t* usr = us + (int64_t)n * nb;
      for (int b = lane; b < nb; b += MOE_WAVE) {
        const uint4 qg = *(const uint4*)(gqr + 16 * b);
        const uint4 qu = *(const uint4*)(uqr + 16 * b);
        const float sg = e8m0_to_f32(gsr[b]);
        const float su = e8m0_to_f32(usr[b]);
        bf16x2_t wg[16], wu[16];
        dequant_bf16(qg, wg);
        dequant_bf16(qu, wu);
#pragma unroll
        for (int m = 0; m < MT; ++m) {
          if (m < mt) {
            const uint32_t* xs = s_x + m * (H >> 1) + 16 * b;
            ag[m] += chunk_dot_bf16(wg, xs) * sg;
            au[m] += chunk_dot_bf16(wu, xs) * su;
          }
        }
      }
#pragma unroll
      for (int m = 0; m < MT; ++m) {
        if (m < mt) {
          const float g = wave_sum(ag[m]);
          const float u = wave_sum(au[m]);
          if (lane == 0) h[(int64_t)(p0 + m0 + m) * I + n] = silu_mul(g, u);
        }
      }
    }
  }
}

template <int MT>
__global__ __launch_bounds__(kThreads) void down_gemv_kernel(const float* __restrict__ h, moe_mxfp4_weights w,
                                                             const int32_t* __restrict__ offsets,
                                                             const int32_t* __restrict__ active,
                                                             float* __restrict__ y_rows) {
  extern __shared__ float s_h[];  // [MT][I]
  const int slot = blockIdx.y;
  if (slot >= active[0]) return;
  const int H = w.hidden, I = w.inter;
  const int e = active[1 + slot];
  const int p0 = offsets[e];
  const int cnt = offsets[e + 1] - p0;
  const int n0 = blockIdx.x * kRowsPerBlock;
  const int lane = threadIdx.x & (MOE_WAVE - 1), wave = threadIdx.x / MOE_WAVE;
  const int nb = I >> 5;
  const int64_t qrow = I >> 1;
  const uint8_t* dq = w.down_q + (int64_t)e * w.expert_stride;
  const uint8_t* ds = w.down_s + (int64_t)e * w.expert_stride;
  const int hv = I >> 2;  // float4 per h row

  for (int m0 = 0; m0 < cnt; m0 += MT) {
    const int mt = min(MT, cnt - m0);
    __syncthreads();
    for (int i = threadIdx.x; i < mt * hv; i += kThreads) {
      const int m = i / hv, c = i - m * hv;
      ((float4*)(s_h + m * I))[c] = ((const float4*)(h + (int64_t)(p0 + m0 + m) * I))[c];
    }
    __syncthreads();
    for (int r = wave; r < kRowsPerBlock; r += kWaves) {
      const int n = n0 + r;
      if (n >= H) break;
      float acc[MT];
#pragma unroll
      for (int m = 0; m < MT; ++m) acc[m] = 0.0f;
      const uint8_t* dqr = dq + (int64_t)n * qrow;
      const uint8_t* dsr = ds + (int64_t)n * nb;
      for (int b = lane; b < nb; b += MOE_WAVE) {
        const uint4 q = *(const uint4*)(dqr + 16 * b);
        const float sc = e8m0_to_f32(dsr[b]);
        f32x2_t wv[16];
        dequant_f32(q, wv);
#pragma unroll
        for (int m = 0; m < MT; ++m)
          if (m < mt) acc[m] += chunk_dot_f32(wv, s_h + m * I + 32 * b) * sc;
      }
#pragma unroll
      for (int m = 0; m < MT; ++m) {
        if (m < mt) {
          const float y = wave_sum(acc[m]);
          if (lane == 0) y_rows[(int64_t)(p0 + m0 + m) * H + n] = y;
        }
      }
    }
  }
}

constexpr size_t kMaxLds = 65536;

int pick_mt(size_t bytes_per_row) {
  if (4 * bytes_per_row <= kMaxLds) return 4;
  if (2 * bytes_per_row <= kMaxLds) return 2;
  return 1;
}

size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

}  // namespace

namespace moe {

size_t expert_ffn_workspace(int T, int k, int E, int H, int I) {
  (void)E;
  (void)H;
  return align_up((size_t)T * k * I * sizeof(float), 256);  // h[R][I]
}

hipError_t launch_expert_ffn(const uint16_t* x, int T, int k, const moe_mxfp4_weights& w, const int32_t* offsets,
                             const int32_t* sorted_rows, const int32_t* active, float* y_rows, void* ws,
                             hipStream_t s) {
  if (T == 0) return hipSuccess;
  const int R = T * k, E = w.num_experts, H = w.hidden, I = w.inter;
  const int max_active = R < E ? R : E;
  float* hbuf = (float*)ws;

  const int mt_g = pick_mt((size_t)H * 2);
  dim3 grid_g((I + kRowsPerBlock - 1) / kRowsPerBlock, max_active);
  const size_t lds_g = (size_t)mt_g * H * 2;
  if (mt_g == 4)
    hipLaunchKernelGGL(gateup_gemv_kernel<4>, grid_g, dim3(kThreads), lds_g, s, x, k, w, offsets, sorted_rows,
                       active, hbuf);
  else if (mt_g == 2)
    hipLaunchKernelGGL(gateup_gemv_kernel<2>, grid_g, dim3(kThreads), lds_g, s, x, k, w, offsets, sorted_rows,
                       active, hbuf);
  else
    hipLaunchKernelGGL(gateup_gemv_kernel<1>, grid_g, dim3(kThreads), lds_g, s, x, k, w, offsets, sorted_rows,
                       active, hbuf);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;

  const int mt_d = pick_mt((size_t)I * 4);
  dim3 grid_d((H + kRowsPerBlock - 1) / kRowsPerBlock, max_active);
  const size_t lds_d = (size_t)mt_d * I * 4;
  if (mt_d == 4)
    hipLaunchKernelGGL(down_gemv_kernel<4>, grid_d, dim3(kThreads), lds_d, s, hbuf, w, offsets, active, y_rows);
  else if (mt_d == 2)
    hipLaunchKernelGGL(down_gemv_kernel<2>, grid_d, dim3(kThreads), lds_d, s, hbuf, w, offsets, active, y_rows);
  else
    hipLaunchKernelGGL(down_gemv_kernel<1>, grid_d, dim3(kThreads), lds_d, s, hbuf, w, offsets, active, y_rows);
  return hipGetLastError();
}

}  // namespace moe
