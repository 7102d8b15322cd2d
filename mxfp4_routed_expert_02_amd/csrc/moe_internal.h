// moe_internal.h - device helpers and launcher declarations shared by the
// HIP sources of libmoe_mxfp4 (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/moe_mxfp4.h"

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

#define MOE_WAVE 64

// Up to kInvariantTokens tokens every expert runs on the register GEMV
// kernels (rows in passes of kRegRows, each row with the arithmetic a single
// row gets), so a token's rows come out bitwise the same alone or in such a
// batch.  In larger batches experts with more than reg_rows_max(T) routed
// rows take the grouped GEMM (MFMA) path: only one-row experts stay on the
// GEMV, since applying a weight chunk to 2..4 rows makes the GEMV
// compute-bound while the GEMM stays memory-bound.
constexpr int kRegRows = 4;
constexpr int kInvariantTokens = 16;
inline int reg_rows_max(int T) { return T > kInvariantTokens ? 1 : kRegRows; }

// ------------------------------------------------------------------ device --
// E8M0 scale byte -> 2^(s-127) as fp32 (s = 0 is the subnormal 2^-127).
__device__ __forceinline__ float e8m0_to_f32(uint32_t s) {
  return s == 0 ? __uint_as_float(0x00400000u) : __uint_as_float(s << 23);
}

// Two E2M1 codes (byte `sel` of `v`, low nibble first) -> two bf16, unscaled.
// v_cvt_scalef32_pk_bf16_fp4 with scale 1.0: every E2M1 value is exact in bf16.
template <int SEL>
__device__ __forceinline__ bf16x2_t fp4x2_to_bf16x2(uint32_t v) {
  return __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(v, 1.0f, SEL);
}

// Two E2M1 codes -> two fp32, unscaled (exact).
template <int SEL>
__device__ __forceinline__ f32x2_t fp4x2_to_f32x2(uint32_t v) {
  return __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(v, 1.0f, SEL);
}

__device__ __forceinline__ bf16x2_t as_bf16x2(uint32_t u) { return __builtin_bit_cast(bf16x2_t, u); }

// a.lo*b.lo + a.hi*b.hi + c in fp32 (v_dot2_f32_bf16); bf16 products are exact.
__device__ __forceinline__ float dot2_bf16(bf16x2_t a, bf16x2_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(a, b, c, false);
}

// Butterfly sum over the 64 lanes; every lane ends with the same bits.
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, MOE_WAVE);
  return v;
}

// DPP lane moves (GFX9 encodings): row_shr:n = 0x110 + n, row_bcast:15 =
// 0x142, row_bcast:31 = 0x143.  Lanes without a source read 0.
template <int CTRL, int ROW_MASK = 0xF>
__device__ __forceinline__ float dpp_f32(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, ROW_MASK, 0xF, false));
}
template <int CTRL, int ROW_MASK = 0xF>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, ROW_MASK, 0xF, false);
}

// Sum over each aligned group of G lanes (G a power of two, 1..64, uniform);
// the total lands in the last lane of the group (other lanes hold partials).
__device__ __forceinline__ float group_sum_last(float v, int G) {
  if (G >= 2) v += dpp_f32<0x111>(v);
  if (G >= 4) v += dpp_f32<0x112>(v);
  if (G >= 8) v += dpp_f32<0x114>(v);
  if (G >= 16) v += dpp_f32<0x118>(v);
  if (G >= 32) v += dpp_f32<0x142, 0xA>(v);
  if (G >= 64) v += dpp_f32<0x143, 0xC>(v);
  return v;
}

// Maximum over the wave (unsigned), valid in lane 63.
__device__ __forceinline__ uint32_t wave_max_u32_last(uint32_t v) {
  v = max(v, dpp_u32<0x111>(v));
  v = max(v, dpp_u32<0x112>(v));
  v = max(v, dpp_u32<0x114>(v));
  v = max(v, dpp_u32<0x118>(v));
  v = max(v, dpp_u32<0x142, 0xA>(v));
  v = max(v, dpp_u32<0x143, 0xC>(v));
  return v;
}

__device__ __forceinline__ float silu_mul(float g, float u) { return g / (1.0f + __expf(-g)) * u; }

// The weightless RMS rescale's arithmetic, shared by every kernel that forms
// it so that all give the same bits.  Layout: kRmsThreads threads, thread c
// owning float4 c + kRmsThreads*i of the row; a thread's squares summed
// float4 by float4 (sumsq4), then a wave butterfly (wave_sum), then the
// kRmsThreads/64 wave sums in wave order; factor 1/sqrt(mean + eps).
// Slots of the experts with exactly one routed row (l1, when lo4 > 1) and
// with lo4 .. reg_max rows (l4), in slot order: l[0] = count, l[1..] =
// slots.  Run by one block of kThreadsT threads; s_part is LDS for
// 2 * kThreadsT / MOE_WAVE ints.
template <int kThreadsT>
__device__ __forceinline__ void build_small_lists(const int32_t* __restrict__ offsets,
                                                  const int32_t* __restrict__ active, int32_t* __restrict__ l1,
                                                  int32_t* __restrict__ l4, int lo4, int reg_max, int* s_part) {
  constexpr int kW = kThreadsT / MOE_WAVE;
  const int na = active[0];
  const int lane = threadIdx.x & (MOE_WAVE - 1), wave = threadIdx.x / MOE_WAVE;
  int base1 = 0, base4 = 0;
  for (int a0 = 0; a0 < na; a0 += kThreadsT) {
    const int a = a0 + threadIdx.x;
    int f1 = 0, f4 = 0;
    if (a < na) {
      const int e = active[1 + a];
      const int cnt = offsets[e + 1] - offsets[e];
      f1 = cnt == 1 && lo4 > 1;
      f4 = cnt >= lo4 && cnt <= reg_max;
    }
    int v1 = f1, v4 = f4;
#pragma unroll
    for (int o = 1; o < MOE_WAVE; o <<= 1) {
      const int u1 = __shfl_up(v1, o, MOE_WAVE), u4 = __shfl_up(v4, o, MOE_WAVE);
      if (lane >= o) {
        v1 += u1;
        v4 += u4;
      }
    }
    if (lane == MOE_WAVE - 1) {
      s_part[wave] = v1;
      s_part[kW + wave] = v4;
    }
    __syncthreads();
    int b1 = base1 + v1 - f1, b4 = base4 + v4 - f4, t1 = 0, t4 = 0;
    for (int w2 = 0; w2 < kW; ++w2) {
      if (w2 < wave) {
        b1 += s_part[w2];
        b4 += s_part[kW + w2];
      }
      t1 += s_part[w2];
      t4 += s_part[kW + w2];
    }
    if (f1) l1[1 + b1] = a;
    if (f4) l4[1 + b4] = a;
    base1 += t1;
    base4 += t4;
    __syncthreads();
  }
  if (threadIdx.x == 0) {
    l1[0] = base1;
    l4[0] = base4;
  }
}

constexpr int kRmsThreads = 1024;
constexpr int kRmsVec = 4;  // float4 per thread (H <= 16384)
__device__ __forceinline__ float sumsq4(const float4& v) { return v.x * v.x + v.y * v.y + v.z * v.z + v.w * v.w; }
__device__ __forceinline__ float rms_factor(float tot, int H, float eps) { return 1.0f / sqrtf(tot / (float)H + eps); }

__device__ __forceinline__ uint16_t f32_to_bf16_rne_dev(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7F800000u) == 0x7F800000u) return (uint16_t)((u >> 16) | ((u & 0xFFFFu) ? 0x40u : 0u));
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// ---------------------------------------------------------------- launchers --
// Each returns hipSuccess or the launch error; all arguments were validated.
namespace moe {

hipError_t launch_route_topk(const float* logits, int T, int E, int k, int32_t* ids, float* w, hipStream_t s);

hipError_t launch_group_rows(const int32_t* ids, int T, int k, int E, int32_t* offsets, int32_t* sorted_rows,
                             int32_t* row_pos, int32_t* active, void* ws, hipStream_t s);
size_t group_rows_workspace(int T, int k, int E);

hipError_t launch_expert_ffn(const uint16_t* x, int T, int k, const moe_mxfp4_weights& w, const int32_t* offsets,
                             const int32_t* sorted_rows, const int32_t* active, float* y_rows, void* ws,
                             hipStream_t s);
size_t expert_ffn_workspace(int T, int k, int E, int H, int I);
bool route_ffn_combine_one_ok(int E, int k, const moe_mxfp4_weights& w);
// x from y_prev's RMS rescale (written to x_next) when y_prev is not null
hipError_t launch_route_ffn_combine_one(const float* logits, int k, const uint16_t* x, const float* y_prev,
                                        float eps, uint16_t* x_next, const moe_mxfp4_weights& w, int32_t* ids,
                                        float* topk_w, int32_t* offsets, int32_t* sorted_rows, int32_t* row_pos,
                                        int32_t* active, float* y_rows, float* out, void* ws, hipStream_t s);
hipError_t launch_expert_ffn_combine(const uint16_t* x, int T, int k, const moe_mxfp4_weights& w,
                                     const int32_t* offsets, const int32_t* sorted_rows, const int32_t* active,
                                     const float* topk_w, const int32_t* row_pos, float* y_rows, float* out,
                                     void* ws, hipStream_t s);

// MFMA grouped-GEMM path (experts with more than 4 routed rows)
bool mfma_shape_ok(int H, int I);
size_t mfma_workspace(int T, int k, int E, int H, int I);
hipError_t launch_mfma_prep(const uint16_t* x, int T, int k, const moe_mxfp4_weights& w, const int32_t* offsets,
                            const int32_t* active, uint8_t* ws, int32_t* l1, int32_t* l4, int lo4, int reg_max,
                            hipStream_t s);
hipError_t launch_mfma_gateup(int T, int k, const moe_mxfp4_weights& w, const int32_t* sorted_rows, uint8_t* ws,
                              hipStream_t s);
hipError_t launch_mfma_down(int T, int k, const moe_mxfp4_weights& w, const int32_t* sorted_rows, float* y_rows,
                            uint8_t* ws, hipStream_t s);

hipError_t launch_combine(const float* y_rows, const float* w, const int32_t* row_pos, int T, int k, int H,
                          float* out, hipStream_t s);

hipError_t launch_rms_rescale(const float* y, int T, int H, float eps, uint16_t* x_next, hipStream_t s);
hipError_t launch_route_group_one(const float* logits, int E, int k, int32_t* ids, float* w, int32_t* offsets,
                                  int32_t* sorted_rows, int32_t* row_pos, int32_t* active, hipStream_t s);
hipError_t launch_combine_rms(const float* y_rows, const float* w, const int32_t* row_pos, int T, int k, int H,
                              float eps, float* out, uint16_t* x_next, hipStream_t s);

hipError_t launch_router_logits(const uint16_t* x, int T, int H, const float* wr, int E, float* logits,
                                hipStream_t s);

}  // namespace moe
