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
#include <climits>

#include "moe_internal.h"
#include "topk_device.h"

namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / MOE_WAVE;
constexpr int kRowsPerBlock = 16;
// row-group unroll of the kernels specialized for 224-block (H = 7168) and
// 48-block (I = 1536) rows; the host grid uses the same constants
constexpr int kGateU224 = 1;
constexpr int kDownU48 = 2;
constexpr int kDownOneU48 = 1;  // the one-token down kernel (measured faster at 4 waves per SIMD)

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
__global__ __launch_bounds__(kThreads) void gateup_gemv_lds_kernel(const uint16_t* __restrict__ x, int k,
                                                                   moe_mxfp4_weights w,
                                                                   const int32_t* __restrict__ offsets,
                                                                   const int32_t* __restrict__ sorted_rows,
                                                                   const int32_t* __restrict__ active,
                                                                   float* __restrict__ h, int skip_upto) {
  extern __shared__ uint32_t s_x[];  // [MT][H/2] bf16 pairs
  const int slot = blockIdx.y;
  if (slot >= active[0]) return;
  const int H = w.hidden, I = w.inter;
  const int e = active[1 + slot];
  const int p0 = offsets[e];
  const int cnt = offsets[e + 1] - p0;
  if (cnt <= skip_upto) return;
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
__global__ __launch_bounds__(kThreads) void down_gemv_lds_kernel(const float* __restrict__ h, moe_mxfp4_weights w,
                                                                 const int32_t* __restrict__ offsets,
                                                                 const int32_t* __restrict__ active,
                                                                 float* __restrict__ y_rows, int skip_upto) {
  extern __shared__ float s_h[];  // [MT][I]
  const int slot = blockIdx.y;
  if (slot >= active[0]) return;
  const int H = w.hidden, I = w.inter;
  const int e = active[1 + slot];
  const int p0 = offsets[e];
  const int cnt = offsets[e + 1] - p0;
  if (cnt <= skip_upto) return;
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

// ---------------------------------------------------------------------------
// Register-resident GEMV (the decode path).  A wave owns P consecutive weight
// rows per iteration, P*nb = 64*J chunks (nb = 32-value blocks per row): lane
// l takes chunks c = 64j + l, i.e. row c / nb and block c % nb.  That block
// index is the same in every iteration, so the lane keeps the J activation
// blocks it needs in registers for the whole kernel and only weight bytes
// stream from HBM; all of an iteration's loads are issued before any math.
// Each row's partial sums are gathered by a wavefront butterfly.

// 32 bf16 activations (4 x 16 B) against a dequantized chunk
__device__ __forceinline__ float chunk_dot_bf16_reg(const bf16x2_t (&wv)[16], const uint4 (&xr)[4]) {
  float acc = 0.0f;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    acc = dot2_bf16(wv[4 * i + 0], as_bf16x2(xr[i].x), acc);
    acc = dot2_bf16(wv[4 * i + 1], as_bf16x2(xr[i].y), acc);
    acc = dot2_bf16(wv[4 * i + 2], as_bf16x2(xr[i].z), acc);
    acc = dot2_bf16(wv[4 * i + 3], as_bf16x2(xr[i].w), acc);
  }
  return acc;
}

__device__ __forceinline__ float chunk_dot_f32_reg(const f32x2_t (&wv)[16], const float4 (&hr)[8]) {
  float acc = 0.0f;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    acc += wv[2 * i].x * hr[i].x;
    acc += wv[2 * i].y * hr[i].y;
    acc += wv[2 * i + 1].x * hr[i].z;
    acc += wv[2 * i + 1].y * hr[i].w;
  }
  return acc;
}

// Buffer resource over one expert matrix: loads past `bytes` return zero,
// which masks the rows beyond the last one of a partial iteration.
// log2 of the largest power of two (at most 64) dividing n
__host__ __device__ constexpr int ctz_const(int n) {
  return (n % 64 == 0) ? 6 : (n % 32 == 0) ? 5 : (n % 16 == 0) ? 4 : (n % 8 == 0) ? 3 : (n % 4 == 0) ? 2 : (n % 2 == 0) ? 1 : 0;
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* p, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, (int)bytes, 0x00020000);
}

// Weight loads of the GEMVs: every weight byte is read once per call, so
// they carry the non-temporal cache policy (nt): the stream does not push
// the activations, h and y out of the caches (measured: the decode FFN
// call 5-7% faster than with the default policy).
constexpr int kStreamPolicy = 2;  // cache-policy operand of the buffer loads: nt

__device__ __forceinline__ uint4 load16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, kStreamPolicy));
}

__device__ __forceinline__ uint32_t load1(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return (uint32_t)__builtin_amdgcn_raw_buffer_load_b8(r, (int)off, 0, kStreamPolicy);
}

__device__ __forceinline__ uint32_t load4(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b32(r, (int)off, 0, kStreamPolicy);
}

// Scale bytes of the one-token gate/up GEMVs (G lanes per row, lane li of
// row group gi takes blocks li + G*j, j < J).  A lane's J bytes lie G bytes
// apart, so instead of J byte loads per matrix each lane loads dwords
// li + G*r (r < (J+3)/4) of its row's scales, and the byte of block li + G*j
// (dword li/4 + (G/4)*j) comes from register j/4 of lane gi*G + li/4 +
// (G/4)*(j%4) by ds_bpermute (measured: the decode FFN call 0.75 us faster).
template <int J>
constexpr int scale_dwords() { return (J + 3) / 4; }

template <int U, int J, int G>
__device__ __forceinline__ void load_scale_dwords(__amdgpu_buffer_rsrc_t rs, uint32_t row_off, uint32_t u_step, int li,
                                                  uint32_t (&d)[U][scale_dwords<J>()]) {
  static_assert(G >= 4 && G % 4 == 0 && scale_dwords<J>() <= 2, "scale dwords of the register GEMV layout");
#pragma unroll
  for (int u = 0; u < U; ++u)
#pragma unroll
    for (int r = 0; r < scale_dwords<J>(); ++r) d[u][r] = load4(rs, row_off + u * u_step + 4u * (uint32_t)(li + G * r));
}

template <int U, int J, int G>
__device__ __forceinline__ void spread_scale_bytes(const uint32_t (&d)[U][scale_dwords<J>()], int gi, int li,
                                                   uint32_t (&sc)[U][J]) {
  const uint32_t sh = 8u * (uint32_t)(li & 3);
#pragma unroll
  for (int u = 0; u < U; ++u)
#pragma unroll
    for (int j = 0; j < J; ++j) {
      const int src = 4 * (gi * G + (li >> 2) + (G / 4) * (j & 3));
      sc[u][j] = ((uint32_t)__builtin_amdgcn_ds_bpermute(src, (int)d[u][j >> 2]) >> sh) & 0xFFu;
    }
}

// Lane layout: G = 2^lg lanes share one weight row (G divides nb, the row's
// count of 32-value blocks) and lane l takes blocks (l % G) + G*j, j < J = nb/G,
// of row l / G; a wave instruction covers 64/G rows and an iteration U such
// row groups.  A row's partial sums then meet in log2(G) DPP steps, in the
// group's last lane.
// The activation row sits in LDS as planes of 16-byte sub-chunks (sub-chunk q
// of block b at [q][b]), so consecutive lanes read consecutive 16 bytes, and
// every block read from LDS serves all U rows of the iteration.
//
// Work items are (expert slot, block b of the expert); wave w of item b runs
// row-iterations [(4b + w) * ipw, (4b + w + 1) * ipw).  One token: one block
// per item, slot = blockIdx / blocks_per_expert over the active list.
// Several tokens: `list` holds the slots of this kernel's row-count class,
// and a grid sized to the machine strides over list[0] * blocks_per_expert
// items, so the work spreads over the experts that exist, not the upper
// bound of them.

// Added to a buffer offset, puts it past every matrix these kernels address
// (all are far below 2 GiB), so the load returns 0 without a memory access.
constexpr uint32_t kPastEnd = 0x80000000u;

// The register GEMVs' class lists (build_small_lists), one block.
__global__ __launch_bounds__(kThreads) void small_lists_kernel(const int32_t* __restrict__ offsets,
                                                              const int32_t* __restrict__ active,
                                                              int32_t* __restrict__ l1, int32_t* __restrict__ l4,
                                                              int lo4, int reg_max) {
  __shared__ int s_part[2 * kWaves];
  build_small_lists<kThreads>(offsets, active, l1, l4, lo4, reg_max, s_part);
}

template <int J, int U, int MT, int NB>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2))) void gateup_gemv_reg_kernel(
    const uint16_t* __restrict__ x, int k, moe_mxfp4_weights w, const int32_t* __restrict__ offsets,
    const int32_t* __restrict__ sorted_rows, const int32_t* __restrict__ active, const int32_t* __restrict__ list,
    float* __restrict__ h, int lg_rt, int blocks_per_expert, int cnt_lo, int cnt_hi) {
  extern __shared__ uint4 s_x4[];  // [MT][4][nb]
  const int n_items = list ? list[0] * blocks_per_expert : (int)gridDim.x;
  for (int item = blockIdx.x; item < n_items; item += gridDim.x) {
  const int slot = list ? list[1 + item / blocks_per_expert] : item / blocks_per_expert;
  if (slot >= active[0]) return;
  const int e = active[1 + slot];
  const int p0 = offsets[e];
  const int cnt = offsets[e + 1] - p0;
  if (cnt < cnt_lo || cnt > cnt_hi) continue;
  // NB > 0: the row's block count is a compile-time constant (so are the LDS
  // and buffer offsets); NB == 0: taken from the weights at run time
  const int I = w.inter, nb = NB > 0 ? NB : (w.hidden >> 5), H = 32 * nb;
  const int lg = NB > 0 ? ctz_const(NB) : lg_rt;
  const int lane = threadIdx.x & (MOE_WAVE - 1), wave = threadIdx.x / MOE_WAVE;
  const int G = 1 << lg, rpi = MOE_WAVE >> lg, rows_it = rpi * U;
  const int li = lane & (G - 1), gi = lane >> lg;
  const int total_iters = (I + rows_it - 1) / rows_it;
  const int it0 = (item % blocks_per_expert) * kWaves + wave;
  const int istep = blocks_per_expert * kWaves;
  const int it1 = total_iters;
  const uint32_t qrow = (uint32_t)H >> 1;
  const int64_t eo = (int64_t)e * w.expert_stride;
  const __amdgpu_buffer_rsrc_t rgq = make_rsrc(w.gate_q + eo, (uint32_t)I * qrow);
  const __amdgpu_buffer_rsrc_t ruq = make_rsrc(w.up_q + eo, (uint32_t)I * qrow);
  const __amdgpu_buffer_rsrc_t rgs = make_rsrc(w.gate_s + eo, (uint32_t)(I * nb));
  const __amdgpu_buffer_rsrc_t rus = make_rsrc(w.up_s + eo, (uint32_t)(I * nb));
  const uint32_t vq0 = (uint32_t)gi * qrow + 16u * li, vs0 = (uint32_t)(gi * nb + li);
  const int plane = 4 * nb;  // uint4 per staged row
  uint4 qg[U][J], qu[U][J];
  uint32_t sg[U][J], su[U][J];
  // chunk j of row group u of iteration it (off = kPastEnd: no memory
  // access); with a compile-time row the scale bytes come separately, as
  // dwords per iteration (load_sc)
  auto load_chunk = [&](int it, int u, int j, uint32_t off) {
    const int n = it * rows_it + u * rpi;
    const uint32_t bq = (uint32_t)n * qrow + off, bs = (uint32_t)(n * nb) + off;
    qg[u][j] = load16(rgq, vq0 + bq + 16u * G * j);
    qu[u][j] = load16(ruq, vq0 + bq + 16u * G * j);
    if constexpr (NB == 0) {
      sg[u][j] = load1(rgs, vs0 + bs + G * j);
      su[u][j] = load1(rus, vs0 + bs + G * j);
    }
  };
  constexpr int Gc = NB > 0 ? 1 << ctz_const(NB) : 4;  // G when the row is a compile-time shape
  uint32_t dg[U][scale_dwords<J>()], du[U][scale_dwords<J>()];  // the scale dwords of an iteration
  auto load_sc = [&](int it, uint32_t off) {
    const uint32_t row_off = (uint32_t)((it * rows_it + gi) * nb) + off;
    load_scale_dwords<U, J, Gc>(rgs, row_off, (uint32_t)(rpi * nb), li, dg);
    load_scale_dwords<U, J, Gc>(rus, row_off, (uint32_t)(rpi * nb), li, du);
  };
  for (int m0 = 0; m0 < cnt; m0 += MT) {
    const int mt = min(MT, cnt - m0);
    if constexpr (NB > 0) {
#pragma unroll
      for (int j = 0; j < J; ++j)
#pragma unroll
        for (int u = 0; u < U; ++u) load_chunk(it0, u, j, it0 < it1 ? 0u : kPastEnd);
      load_sc(it0, it0 < it1 ? 0u : kPastEnd);
    }
    __syncthreads();
    for (int i = threadIdx.x; i < mt * plane; i += kThreads) {
      const int m = i / plane, c = i - m * plane;
      const int64_t t = sorted_rows[p0 + m0 + m] / k;
      s_x4[m * plane + (c & 3) * nb + (c >> 2)] = ((const uint4*)(x + t * H))[c];
    }
    __syncthreads();
    for (int it = it0; it < it1; it += istep) {
      const uint32_t next_off = it + istep < it1 ? 0u : kPastEnd;
      const int n0 = it * rows_it;
      if constexpr (NB == 0) {
#pragma unroll
        for (int j = 0; j < J; ++j)
#pragma unroll
          for (int u = 0; u < U; ++u) load_chunk(it, u, j, 0u);
      } else {
        spread_scale_bytes<U, J, Gc>(dg, gi, li, sg);
        spread_scale_bytes<U, J, Gc>(du, gi, li, su);
        load_sc(it + istep, next_off);
      }
      float ag[U][MT], au[U][MT];
#pragma unroll
      for (int u = 0; u < U; ++u)
#pragma unroll
        for (int m = 0; m < MT; ++m) ag[u][m] = au[u][m] = 0.0f;
#pragma unroll
      for (int j = 0; j < J; ++j) {
        if (MT == 1) {
          // one row: one activation block read, gate and up chunks in turn
          uint4 xr[4];
#pragma unroll
          for (int q = 0; q < 4; ++q) xr[q] = s_x4[q * nb + li + G * j];
#pragma unroll
          for (int u = 0; u < U; ++u) {
            bf16x2_t wv[16];
            dequant_bf16(qg[u][j], wv);
            ag[u][0] += chunk_dot_bf16_reg(wv, xr) * e8m0_to_f32(sg[u][j]);
            dequant_bf16(qu[u][j], wv);
            au[u][0] += chunk_dot_bf16_reg(wv, xr) * e8m0_to_f32(su[u][j]);
            if constexpr (NB > 0) load_chunk(it + istep, u, j, next_off);
          }
        } else {
          // several rows: each chunk is dequantized once and serves every row
#pragma unroll
          for (int u = 0; u < U; ++u) {
            bf16x2_t wg[16], wu[16];
            dequant_bf16(qg[u][j], wg);
            dequant_bf16(qu[u][j], wu);
            const float fg = e8m0_to_f32(sg[u][j]), fu = e8m0_to_f32(su[u][j]);
            if constexpr (NB > 0) load_chunk(it + istep, u, j, next_off);
#pragma unroll
            for (int m = 0; m < MT; ++m) {
              if (m < mt) {
                uint4 xr[4];
#pragma unroll
                for (int q = 0; q < 4; ++q) xr[q] = s_x4[m * plane + q * nb + li + G * j];
                ag[u][m] += chunk_dot_bf16_reg(wg, xr) * fg;
                au[u][m] += chunk_dot_bf16_reg(wu, xr) * fu;
              }
            }
          }
        }
        // keeps the scheduler from hoisting every LDS read (and its registers)
        __builtin_amdgcn_sched_barrier(0);
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int n = n0 + u * rpi + gi;
#pragma unroll
        for (int m = 0; m < MT; ++m) {
          if (m < mt) {
            const float g = group_sum_last(ag[u][m], G);
            const float uu = group_sum_last(au[u][m], G);
            if (li == G - 1 && n < I) h[(int64_t)(p0 + m0 + m) * I + n] = silu_mul(g, uu);
          }
        }
      }
    }
  }
  }
}

template <int J, int U, int MT, int NB>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2))) void down_gemv_reg_kernel(
    const float* __restrict__ h, moe_mxfp4_weights w, const int32_t* __restrict__ offsets,
    const int32_t* __restrict__ active, const int32_t* __restrict__ list, float* __restrict__ y_rows, int lg_rt,
    int blocks_per_expert, int cnt_lo, int cnt_hi) {
  extern __shared__ float4 s_h4[];  // [MT][8][nb]
  const int n_items = list ? list[0] * blocks_per_expert : (int)gridDim.x;
  for (int item = blockIdx.x; item < n_items; item += gridDim.x) {
  const int slot = list ? list[1 + item / blocks_per_expert] : item / blocks_per_expert;
  if (slot >= active[0]) return;
  const int e = active[1 + slot];
  const int p0 = offsets[e];
  const int cnt = offsets[e + 1] - p0;
  if (cnt < cnt_lo || cnt > cnt_hi) continue;
  const int H = w.hidden, nb = NB > 0 ? NB : (w.inter >> 5), I = 32 * nb;
  const int lg = NB > 0 ? ctz_const(NB) : lg_rt;
  const int lane = threadIdx.x & (MOE_WAVE - 1), wave = threadIdx.x / MOE_WAVE;
  const int G = 1 << lg, rpi = MOE_WAVE >> lg, rows_it = rpi * U;
  const int li = lane & (G - 1), gi = lane >> lg;
  const int total_iters = (H + rows_it - 1) / rows_it;
  const int it0 = (item % blocks_per_expert) * kWaves + wave;
  const int istep = blocks_per_expert * kWaves;
  const int it1 = total_iters;
  const uint32_t qrow = (uint32_t)I >> 1;
  const int64_t eo = (int64_t)e * w.expert_stride;
  const __amdgpu_buffer_rsrc_t rq = make_rsrc(w.down_q + eo, (uint32_t)H * qrow);
  const __amdgpu_buffer_rsrc_t rs = make_rsrc(w.down_s + eo, (uint32_t)(H * nb));
  const uint32_t vq0 = (uint32_t)gi * qrow + 16u * li, vs0 = (uint32_t)(gi * nb + li);
  const int plane = 8 * nb;  // float4 per staged row
  uint4 q[U][J];
  uint32_t sc[U][J];
  auto load_chunk = [&](int it, int u, int j, uint32_t off) {
    const int n = it * rows_it + u * rpi;
    q[u][j] = load16(rq, vq0 + (uint32_t)n * qrow + off + 16u * G * j);
    sc[u][j] = load1(rs, vs0 + (uint32_t)(n * nb) + off + G * j);
  };
  for (int m0 = 0; m0 < cnt; m0 += MT) {
    const int mt = min(MT, cnt - m0);
    if constexpr (NB > 0) {
#pragma unroll
      for (int j = 0; j < J; ++j)
#pragma unroll
        for (int u = 0; u < U; ++u) load_chunk(it0, u, j, it0 < it1 ? 0u : kPastEnd);
    }
    __syncthreads();
    for (int i = threadIdx.x; i < mt * plane; i += kThreads) {
      const int m = i / plane, c = i - m * plane;
      s_h4[m * plane + (c & 7) * nb + (c >> 3)] = ((const float4*)(h + (int64_t)(p0 + m0 + m) * I))[c];
    }
    __syncthreads();
    for (int it = it0; it < it1; it += istep) {
      const uint32_t next_off = it + istep < it1 ? 0u : kPastEnd;
      const int n0 = it * rows_it;
      if constexpr (NB == 0) {
#pragma unroll
        for (int j = 0; j < J; ++j)
#pragma unroll
          for (int u = 0; u < U; ++u) load_chunk(it, u, j, 0u);
      }
      float acc[U][MT];
#pragma unroll
      for (int u = 0; u < U; ++u)
#pragma unroll
        for (int m = 0; m < MT; ++m) acc[u][m] = 0.0f;
#pragma unroll
      for (int j = 0; j < J; ++j) {
        if (MT == 1) {
          // one row: each h block read from LDS serves all U weight rows
          float4 hr[8];
#pragma unroll
          for (int i = 0; i < 8; ++i) hr[i] = s_h4[i * nb + li + G * j];
#pragma unroll
          for (int u = 0; u < U; ++u) {
            f32x2_t wv[16];
            dequant_f32(q[u][j], wv);
            acc[u][0] += chunk_dot_f32_reg(wv, hr) * e8m0_to_f32(sc[u][j]);
            if constexpr (NB > 0) load_chunk(it + istep, u, j, next_off);
            __builtin_amdgcn_sched_barrier(0);  // one dequantized chunk live at a time
          }
        } else {
          // several rows: each chunk is dequantized once and serves every row
#pragma unroll
          for (int u = 0; u < U; ++u) {
            f32x2_t wv[16];
            dequant_f32(q[u][j], wv);
            const float f = e8m0_to_f32(sc[u][j]);
            if constexpr (NB > 0) load_chunk(it + istep, u, j, next_off);
#pragma unroll
            for (int m = 0; m < MT; ++m) {
              if (m < mt) {
                float4 hr[8];
#pragma unroll
                for (int i = 0; i < 8; ++i) hr[i] = s_h4[m * plane + i * nb + li + G * j];
                acc[u][m] += chunk_dot_f32_reg(wv, hr) * f;
              }
            }
          }
        }
        __builtin_amdgcn_sched_barrier(0);
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int n = n0 + u * rpi + gi;
#pragma unroll
        for (int m = 0; m < MT; ++m) {
          if (m < mt) {
            const float v = group_sum_last(acc[u][m], G);
            if (li == G - 1 && n < H) y_rows[(int64_t)(p0 + m0 + m) * H + n] = v;
          }
        }
      }
    }
  }
  }
}

// One token, rows of a compile-time NB blocks (the decode shape): the lane
// layout and arithmetic of the MT = 1 kernels above, one work item per
// block, with three changes to keep HBM busy:
//  * every routed row belongs to token 0, so nothing the first weight loads
//    need waits on the routing beyond the expert id (gate/up issues its
//    activation loads before any routing read); the offsets are read while
//    the first loads are in flight;
//  * rolling prefetch: as soon as chunk j of an iteration has been used, the
//    same registers are refilled with chunk j of the wave's next iteration,
//    so a wave's loads stay in flight through its math instead of stopping
//    at every iteration boundary, at no extra register cost;
//  * the waves of an expert take its row-iterations round robin (wave i of
//    the expert takes i, i + istep, ...), so at any moment they read one
//    contiguous front of each matrix rather than one stretch per wave.
// An expert the token picked more than once gets the same h (and y) in each
// of its rows.
template <int J, int U, int NB>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2))) void gateup_gemv_one_kernel(
    const uint16_t* __restrict__ x, moe_mxfp4_weights w, const int32_t* __restrict__ offsets,
    const int32_t* __restrict__ active, float* __restrict__ h, int blocks_per_expert) {
  extern __shared__ uint4 s_x4[];  // [4][NB]
  // x's 4*NB uint4 in four named registers per thread (an array here went to scratch)
  static_assert(4 * NB > 3 * kThreads && 4 * NB <= 4 * kThreads, "x staging assumes 3..4 uint4 per thread");
  const uint4* x4 = (const uint4*)x;
  const int tx = threadIdx.x;
  const uint4 xs0 = x4[tx], xs1 = x4[tx + kThreads], xs2 = x4[tx + 2 * kThreads];
  uint4 xs3 = make_uint4(0u, 0u, 0u, 0u);
  if (tx + 3 * kThreads < 4 * NB) xs3 = x4[tx + 3 * kThreads];
  const int slot = blockIdx.x / blocks_per_expert;
  if (slot >= active[0]) return;
  const int e = active[1 + slot];
  constexpr int nb = NB, H = 32 * NB, lg = ctz_const(NB), G = 1 << lg, rpi = MOE_WAVE >> lg, rows_it = rpi * U;
  const int I = w.inter;
  const int lane = threadIdx.x & (MOE_WAVE - 1), wave = threadIdx.x / MOE_WAVE;
  const int li = lane & (G - 1), gi = lane >> lg;
  const int total_iters = (I + rows_it - 1) / rows_it;
  const int it0 = (blockIdx.x % blocks_per_expert) * kWaves + wave;
  const int istep = blocks_per_expert * kWaves;
  const int it1 = total_iters;
  constexpr uint32_t qrow = (uint32_t)H >> 1;
  const int64_t eo = (int64_t)e * w.expert_stride;
  const __amdgpu_buffer_rsrc_t rgq = make_rsrc(w.gate_q + eo, (uint32_t)I * qrow);
  const __amdgpu_buffer_rsrc_t ruq = make_rsrc(w.up_q + eo, (uint32_t)I * qrow);
  const __amdgpu_buffer_rsrc_t rgs = make_rsrc(w.gate_s + eo, (uint32_t)(I * nb));
  const __amdgpu_buffer_rsrc_t rus = make_rsrc(w.up_s + eo, (uint32_t)(I * nb));
  const uint32_t vq0 = (uint32_t)gi * qrow + 16u * li;
  uint4 qg[U][J], qu[U][J];
  uint32_t sg[U][J], su[U][J];
  // chunk j of row group u of iteration it; `off` = kPastEnd turns the loads
  // into out-of-range buffer reads, which return 0 and touch no memory
  auto load_chunk = [&](int it, int u, int j, uint32_t off) {
    const int n = it * rows_it + u * rpi;
    const uint32_t bq = (uint32_t)n * qrow + off;
    qg[u][j] = load16(rgq, vq0 + bq + 16u * G * j);
    qu[u][j] = load16(ruq, vq0 + bq + 16u * G * j);
  };
  uint32_t dg[U][scale_dwords<J>()], du[U][scale_dwords<J>()];  // the scale dwords of an iteration
  auto load_sc = [&](int it, uint32_t off) {
    const uint32_t row_off = (uint32_t)((it * rows_it + gi) * nb) + off;
    load_scale_dwords<U, J, G>(rgs, row_off, (uint32_t)(rpi * nb), li, dg);
    load_scale_dwords<U, J, G>(rus, row_off, (uint32_t)(rpi * nb), li, du);
  };
#pragma unroll
  for (int j = 0; j < J; ++j)
#pragma unroll
    for (int u = 0; u < U; ++u) load_chunk(it0, u, j, it0 < it1 ? 0u : kPastEnd);
  load_sc(it0, it0 < it1 ? 0u : kPastEnd);
  const int p0 = offsets[e];
  const int cnt = offsets[e + 1] - p0;
  auto stage = [&](int c, const uint4& v) { s_x4[(c & 3) * nb + (c >> 2)] = v; };
  stage(tx, xs0);
  stage(tx + kThreads, xs1);
  stage(tx + 2 * kThreads, xs2);
  if (tx + 3 * kThreads < 4 * NB) stage(tx + 3 * kThreads, xs3);
  __syncthreads();
  for (int it = it0; it < it1; it += istep) {
    const uint32_t next_off = it + istep < it1 ? 0u : kPastEnd;
    const int n0 = it * rows_it;
    spread_scale_bytes<U, J, G>(dg, gi, li, sg);
    spread_scale_bytes<U, J, G>(du, gi, li, su);
    load_sc(it + istep, next_off);
    float ag[U], au[U];
#pragma unroll
    for (int u = 0; u < U; ++u) ag[u] = au[u] = 0.0f;
#pragma unroll
    for (int j = 0; j < J; ++j) {
      uint4 xr[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) xr[q] = s_x4[q * nb + li + G * j];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        bf16x2_t wv[16];
        dequant_bf16(qg[u][j], wv);
        ag[u] += chunk_dot_bf16_reg(wv, xr) * e8m0_to_f32(sg[u][j]);
        dequant_bf16(qu[u][j], wv);
        au[u] += chunk_dot_bf16_reg(wv, xr) * e8m0_to_f32(su[u][j]);
        load_chunk(it + istep, u, j, next_off);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int n = n0 + u * rpi + gi;
      const float g = group_sum_last(ag[u], G);
      const float uu = group_sum_last(au[u], G);
      if (li == G - 1 && n < I) {
        const float v = silu_mul(g, uu);
        for (int r = 0; r < cnt; ++r) h[(int64_t)(p0 + r) * I + n] = v;
      }
    }
  }
}

template <int J, int U, int NB>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2))) void down_gemv_one_kernel(
    const float* __restrict__ h, moe_mxfp4_weights w, const int32_t* __restrict__ offsets,
    const int32_t* __restrict__ active, float* __restrict__ y_rows, int blocks_per_expert) {
  extern __shared__ float4 s_h4[];  // [8][NB]
  static_assert(8 * NB > kThreads && 8 * NB <= 2 * kThreads, "h staging assumes 1..2 float4 per thread");
  const int slot = blockIdx.x / blocks_per_expert;
  if (slot >= active[0]) return;
  const int e = active[1 + slot];
  constexpr int nb = NB, I = 32 * NB, lg = ctz_const(NB), G = 1 << lg, rpi = MOE_WAVE >> lg, rows_it = rpi * U;
  const int H = w.hidden;
  const int lane = threadIdx.x & (MOE_WAVE - 1), wave = threadIdx.x / MOE_WAVE;
  const int li = lane & (G - 1), gi = lane >> lg;
  const int total_iters = (H + rows_it - 1) / rows_it;
  const int it0 = (blockIdx.x % blocks_per_expert) * kWaves + wave;
  const int istep = blocks_per_expert * kWaves;
  const int it1 = total_iters;
  constexpr uint32_t qrow = (uint32_t)I >> 1;
  const int64_t eo = (int64_t)e * w.expert_stride;
  const __amdgpu_buffer_rsrc_t rq = make_rsrc(w.down_q + eo, (uint32_t)H * qrow);
  const __amdgpu_buffer_rsrc_t rs = make_rsrc(w.down_s + eo, (uint32_t)(H * nb));
  const uint32_t vq0 = (uint32_t)gi * qrow + 16u * li, vs0 = (uint32_t)(gi * nb + li);
  uint4 q[U][J];
  uint32_t sc[U][J];
  auto load_chunk = [&](int it, int u, int j, uint32_t off) {
    const int n = it * rows_it + u * rpi;
    q[u][j] = load16(rq, vq0 + (uint32_t)n * qrow + off + 16u * G * j);
    sc[u][j] = load1(rs, vs0 + (uint32_t)(n * nb) + off + G * j);
  };
  const int p0 = offsets[e];
  const int cnt = offsets[e + 1] - p0;
  const float4* h4 = (const float4*)(h + (int64_t)p0 * I);
  const int tx = threadIdx.x;
  const float4 hs0 = h4[tx];
  float4 hs1 = make_float4(0.f, 0.f, 0.f, 0.f);
  if (tx + kThreads < 8 * NB) hs1 = h4[tx + kThreads];
#pragma unroll
  for (int j = 0; j < J; ++j)
#pragma unroll
    for (int u = 0; u < U; ++u) load_chunk(it0, u, j, it0 < it1 ? 0u : kPastEnd);
  s_h4[(tx & 7) * nb + (tx >> 3)] = hs0;
  if (tx + kThreads < 8 * NB) s_h4[((tx + kThreads) & 7) * nb + ((tx + kThreads) >> 3)] = hs1;
  __syncthreads();
  for (int it = it0; it < it1; it += istep) {
    const uint32_t next_off = it + istep < it1 ? 0u : kPastEnd;
    const int n0 = it * rows_it;
    float acc[U];
#pragma unroll
    for (int u = 0; u < U; ++u) acc[u] = 0.0f;
#pragma unroll
    for (int j = 0; j < J; ++j) {
      float4 hr[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) hr[i] = s_h4[i * nb + li + G * j];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        f32x2_t wv[16];
        dequant_f32(q[u][j], wv);
        acc[u] += chunk_dot_f32_reg(wv, hr) * e8m0_to_f32(sc[u][j]);
        load_chunk(it + istep, u, j, next_off);
        __builtin_amdgcn_sched_barrier(0);  // one dequantized chunk live at a time
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int n = n0 + u * rpi + gi;
      const float v = group_sum_last(acc[u], G);
      if (li == G - 1 && n < H)
        for (int r = 0; r < cnt; ++r) y_rows[(int64_t)(p0 + r) * H + n] = v;
    }
  }
}

// One token, I = 32*NB, k <= kFMaxK: the down projection of every routed
// expert and the weighted combine in one launch (the step after gate/up at
// decode).  Block b owns output rows [kRows*b, kRows*b + kRows) of every
// active expert.  Each wave serves one slot (16 / na waves per slot, na the
// number of active experts, rounded down): it stages that slot's h row in
// its own LDS planes and starts on its rows as soon as they are in, with no
// block barrier before the first dot, so a wave whose h arrives early is not
// held by the rest of the block's h rows.  Every row's y (the arithmetic of
// the down GEMVs: G lanes per row, per-block scaled partial sums, DPP
// reduction, rolling prefetch of the wave's next row iteration) goes to
// y_rows and to an LDS tile indexed by sorted row.  After one barrier, kRows
// threads form out[n] = sum_j w[j] * y[row_pos[j]][n] with j ascending, the
// combine kernel's arithmetic, so both outputs equal the separate down and
// combine launches bit for bit.
constexpr int kFThreads = 1024;
constexpr int kFWaves = kFThreads / MOE_WAVE;
constexpr int kFIters = 7;  // 4-row iterations per block and expert
constexpr int kFMaxK = 16;

template <int NB>
__global__ __launch_bounds__(kFThreads) void down_combine_one_kernel(
    const float* __restrict__ h, moe_mxfp4_weights w, const int32_t* __restrict__ offsets,
    const int32_t* __restrict__ active, const float* __restrict__ topk_w, const int32_t* __restrict__ row_pos,
    int k, float* __restrict__ y_rows, float* __restrict__ out) {
  constexpr int nb = NB, I = 32 * NB, lg = ctz_const(NB), G = 1 << lg, J = NB / G, rpi = MOE_WAVE >> lg;
  constexpr int kRows = kFIters * rpi;  // output rows per block
  constexpr int kH4 = 8 * NB;           // float4 of an h row
  static_assert(J * G == NB && J <= 8, "register lane layout");
  static_assert(kH4 % MOE_WAVE == 0, "h row in whole wave loads");
  constexpr uint32_t qrow = (uint32_t)I >> 1;
  __shared__ float4 s_h4[kFWaves][kH4];  // h of each wave's slot, planes [8][NB]
  __shared__ float s_y[kFMaxK][kRows];   // y of this block's rows, by sorted row
  const int H = w.hidden;
  const int na = active[0];
  const int lane = threadIdx.x & (MOE_WAVE - 1);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / MOE_WAVE);
  const int li = lane & (G - 1), gi = lane >> lg;
  const int n_base = blockIdx.x * kRows;
  // the waves split evenly over the slots: wave w takes slot w / wps and
  // that slot's row iterations w % wps, w % wps + wps, ...
  const int wps = kFWaves / na;
  const int slot = wave / wps;
  int itr = wave - slot * wps;  // the wave's first row iteration
  if (slot < na && itr < kFIters) {
    const int e = active[1 + slot];
    const int p0 = offsets[e], cnt = offsets[e + 1] - p0;
    const int64_t eo = (int64_t)e * w.expert_stride;
    const __amdgpu_buffer_rsrc_t rq = make_rsrc(w.down_q + eo, (uint32_t)H * qrow);
    const __amdgpu_buffer_rsrc_t rs = make_rsrc(w.down_s + eo, (uint32_t)(H * nb));
    const uint32_t vq0 = 16u * li, vs0 = (uint32_t)li;
    uint4 q[J];
    uint32_t sc[J];
    // chunk j of row iteration itr (past the last: no memory access)
    auto load_chunk = [&](int itr, int j) {
      const int n = n_base + itr * rpi + gi;
      const uint32_t off = itr < kFIters ? 0u : kPastEnd;
      q[j] = load16(rq, vq0 + (uint32_t)n * qrow + off + 16u * G * j);
      sc[j] = load1(rs, vs0 + (uint32_t)(n * nb) + off + G * j);
    };
#pragma unroll
    for (int j = 0; j < J; ++j) load_chunk(itr, j);
    const float4* h4 = (const float4*)(h + (int64_t)p0 * I);
    float4 hv[kH4 / MOE_WAVE];
#pragma unroll
    for (int i = 0; i < kH4 / MOE_WAVE; ++i) hv[i] = h4[lane + MOE_WAVE * i];
    float4* sh = s_h4[wave];
#pragma unroll
    for (int i = 0; i < kH4 / MOE_WAVE; ++i) {
      const int c = lane + MOE_WAVE * i;
      sh[(c & 7) * nb + (c >> 3)] = hv[i];
    }
    // the wave reads only what its own lanes wrote: LDS keeps a wave's
    // accesses in order, so only the compiler's order needs the fence
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    for (; itr < kFIters; itr += wps) {
      const int n = n_base + itr * rpi + gi;
      float acc = 0.0f;
#pragma unroll
      for (int j = 0; j < J; ++j) {
        float4 hr[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) hr[i] = sh[i * nb + li + G * j];
        f32x2_t wv[16];
        dequant_f32(q[j], wv);
        acc += chunk_dot_f32_reg(wv, hr) * e8m0_to_f32(sc[j]);
        load_chunk(itr + wps, j);  // chunk j of the wave's next iteration
        __builtin_amdgcn_sched_barrier(0);
      }
      const float v = group_sum_last(acc, G);
      if (li == G - 1 && n < H) {
        for (int r = 0; r < cnt; ++r) {
          y_rows[(int64_t)(p0 + r) * H + n] = v;
          s_y[p0 + r][n - n_base] = v;
        }
      }
    }
  }
  __syncthreads();
  if (threadIdx.x < kRows) {
    const int n = n_base + threadIdx.x;
    if (n < H) {
      float acc = 0.0f;
      for (int j = 0; j < k; ++j) acc += topk_w[j] * s_y[row_pos[j]][threadIdx.x];
      out[n] = acc;
    }
  }
}

// One token routed inside the gate/up launch, in blocks of 16 waves (one
// block per CU at 4 waves per SIMD): the block first runs the token's top-k
// (topk_block_wide: its first four waves hold the logits; the picks equal
// the routing kernels' bit for bit, the top k being unique; one top-k per
// CU rather than one per 4-wave block), then every wave takes the expert of
// the block's slot, the slot-th smallest picked id (the active list the
// grouping writes; the picks are distinct, so that expert's one row sits at
// sorted position `slot`).  The blocks also write the routing weights and
// the grouping, equal to what the fused route + group kernel writes.  The
// rest is gateup_gemv_one_kernel's lane layout and arithmetic: the
// activation loads go out before the top-k, the first weight loads as soon
// as the expert is known, rolling prefetch, round-robin row iterations.
//
// RMS: the input is the previous layer's fp32 output y_prev; every block
// forms x = bf16_rne(y_prev * rms factor) itself with the RMS rescale's
// arithmetic and thread layout (its 1024 threads are the rescale's), and
// block 0 also writes that x to x_next.
constexpr int kRGThreads = 1024;
constexpr int kRGWaves = kRGThreads / MOE_WAVE;

template <int J, int U, int NB, int C, bool RMS>
__global__ __launch_bounds__(kRGThreads) void route_gateup_one_kernel(
    const float* __restrict__ logits, int E, int k, const uint16_t* __restrict__ x, const float* __restrict__ y_prev,
    float eps, uint16_t* __restrict__ x_next, moe_mxfp4_weights w, float* __restrict__ h, int32_t* __restrict__ ids,
    float* __restrict__ topk_w, int32_t* __restrict__ offsets, int32_t* __restrict__ sorted_rows,
    int32_t* __restrict__ row_pos, int32_t* __restrict__ active, int blocks_per_expert) {
  static_assert(kRGThreads == kRmsThreads, "the block is the rescale's layout");
  extern __shared__ uint4 s_x4[];  // [4][NB]
  __shared__ TopkWideLds<C> s;
  constexpr int kN4 = 8 * NB;  // float4 (and half-uint4) of a row
  static_assert(4 * NB <= kRGThreads && kN4 <= kRmsVec * kRmsThreads, "x staging layout");
  constexpr int kIV = (kN4 + kRmsThreads - 1) / kRmsThreads;  // float4 per thread in the rescale's layout
  const int tx = threadIdx.x;
  uint4 xs = make_uint4(0u, 0u, 0u, 0u);
  float4 yv[kIV];
  if constexpr (RMS) {
    const float4* y4 = (const float4*)y_prev;
#pragma unroll
    for (int i = 0; i < kIV; ++i) {
      const int c = tx + kRmsThreads * i;
      yv[i] = c < kN4 ? y4[c] : make_float4(0.0f, 0.0f, 0.0f, 0.0f);
    }
  } else {
    if (tx < 4 * NB) xs = ((const uint4*)x)[tx];
  }
  // x (non-RMS) or the RMS partial sums go into LDS while the logits loads
  // are in flight, before the top-k's first barrier
  __shared__ float s_part[kRmsThreads / MOE_WAVE];
  const int lane = tx & (MOE_WAVE - 1), wave = tx / MOE_WAVE;
  auto pre = [&]() {
    if constexpr (RMS) {
      float ss = 0.0f;
#pragma unroll
      for (int i = 0; i < kIV; ++i) ss += sumsq4(yv[i]);  // the layout's later float4 are all zero
      ss = wave_sum(ss);
      if (lane == 0) s_part[wave] = ss;
    } else {
      if (tx < 4 * NB) s_x4[(tx & 3) * NB + (tx >> 2)] = xs;
    }
  };
  topk_block_wide<C>(logits, E, k, s, pre);
  // the k <= 16 pick ids (padded with INT_MAX) in registers: 4 LDS reads
  static_assert(kFMaxK == 16, "four int4 of pick ids");
  int4 pv[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) pv[i] = ((const int4*)s.pick_id)[i];
  // routing and grouping outputs (the picks are distinct: expert e's offset
  // is the number of picks below e, a pick's sorted place the number of picks
  // below its id); block 0 writes the per-pick ones, and the E+1 offsets are
  // spread over the blocks so that no block's weight stream starts late
  if (blockIdx.x == 0) {
    if (tx < MOE_WAVE) {
      int id;
      float wv;
      if (topk_softmax(s, k, tx, id, wv)) {
        ids[tx] = id;
        topk_w[tx] = wv;
      }
    } else if (tx < MOE_WAVE + k) {
      const int t = tx - MOE_WAVE, pid = s.pick_id[t];
      const int r = picks_below<4>(pv, pid);
      sorted_rows[r] = t;
      row_pos[t] = r;
      active[1 + r] = pid;
      if (t == 0) active[0] = k;
    }
  }
  for (int e = blockIdx.x + (int)gridDim.x * tx; e <= E; e += (int)gridDim.x * kRGThreads)
    offsets[e] = picks_below<4>(pv, e);
  const int slot = blockIdx.x / blocks_per_expert;
  if (slot >= k) return;
  // lane j < k: pick j's id and its rank among the picks by id
  int pid = INT_MAX, prank = -1;
  if (lane < k) {
    pid = s.pick_id[lane];
    prank = picks_below<4>(pv, pid);
  }
  const int src = __ffsll((unsigned long long)__ballot(prank == slot)) - 1;
  const int e = __builtin_amdgcn_readlane(pid, src);
  const int p0 = slot;  // offsets[e]: the picks below e
  constexpr int nb = NB, H = 32 * NB, lg = ctz_const(NB), G = 1 << lg, rpi = MOE_WAVE >> lg, rows_it = rpi * U;
  const int I = w.inter;
  const int li = lane & (G - 1), gi = lane >> lg;
  const int total_iters = (I + rows_it - 1) / rows_it;
  const int it0 = (blockIdx.x % blocks_per_expert) * kRGWaves + wave;
  const int istep = blocks_per_expert * kRGWaves;
  const int it1 = total_iters;
  constexpr uint32_t qrow = (uint32_t)H >> 1;
  const int64_t eo = (int64_t)e * w.expert_stride;
  const __amdgpu_buffer_rsrc_t rgq = make_rsrc(w.gate_q + eo, (uint32_t)I * qrow);
  const __amdgpu_buffer_rsrc_t ruq = make_rsrc(w.up_q + eo, (uint32_t)I * qrow);
  const __amdgpu_buffer_rsrc_t rgs = make_rsrc(w.gate_s + eo, (uint32_t)(I * nb));
  const __amdgpu_buffer_rsrc_t rus = make_rsrc(w.up_s + eo, (uint32_t)(I * nb));
  const uint32_t vq0 = (uint32_t)gi * qrow + 16u * li;
  uint4 qg[U][J], qu[U][J];
  uint32_t sg[U][J], su[U][J];
  auto load_chunk = [&](int it, int u, int j, uint32_t off) {
    const int n = it * rows_it + u * rpi;
    const uint32_t bq = (uint32_t)n * qrow + off;
    qg[u][j] = load16(rgq, vq0 + bq + 16u * G * j);
    qu[u][j] = load16(ruq, vq0 + bq + 16u * G * j);
  };
  uint32_t dg[U][scale_dwords<J>()], du[U][scale_dwords<J>()];  // the scale dwords of an iteration
  auto load_sc = [&](int it, uint32_t off) {
    const uint32_t row_off = (uint32_t)((it * rows_it + gi) * nb) + off;
    load_scale_dwords<U, J, G>(rgs, row_off, (uint32_t)(rpi * nb), li, dg);
    load_scale_dwords<U, J, G>(rus, row_off, (uint32_t)(rpi * nb), li, du);
  };
#pragma unroll
  for (int j = 0; j < J; ++j)
#pragma unroll
    for (int u = 0; u < U; ++u) load_chunk(it0, u, j, it0 < it1 ? 0u : kPastEnd);
  load_sc(it0, it0 < it1 ? 0u : kPastEnd);
  if constexpr (RMS) {  // x = bf16(y_prev * factor) into LDS while the first weight loads are in flight
    float tot = 0.0f;
#pragma unroll
    for (int i = 0; i < kRmsThreads / MOE_WAVE; ++i) tot += s_part[i];
    const float r = rms_factor(tot, H, eps);
    uint2* sx2 = (uint2*)s_x4;
#pragma unroll
    for (int i = 0; i < kIV; ++i) {
      const int c = tx + kRmsThreads * i;  // float4 index = elements 4c .. 4c+3
      if (c < kN4) {
        const float4 v = yv[i];
        const uint32_t lo = f32_to_bf16_rne_dev(v.x * r) | ((uint32_t)f32_to_bf16_rne_dev(v.y * r) << 16);
        const uint32_t hi = f32_to_bf16_rne_dev(v.z * r) | ((uint32_t)f32_to_bf16_rne_dev(v.w * r) << 16);
        const int c8 = c >> 1;  // staged 16-byte piece
        sx2[2 * ((c8 & 3) * nb + (c8 >> 2)) + (c & 1)] = make_uint2(lo, hi);
        if (blockIdx.x == 0) ((uint2*)x_next)[c] = make_uint2(lo, hi);
      }
    }
    __syncthreads();
  }
  for (int it = it0; it < it1; it += istep) {
    const uint32_t next_off = it + istep < it1 ? 0u : kPastEnd;
    const int n0 = it * rows_it;
    spread_scale_bytes<U, J, G>(dg, gi, li, sg);
    spread_scale_bytes<U, J, G>(du, gi, li, su);
    load_sc(it + istep, next_off);
    float ag[U], au[U];
#pragma unroll
    for (int u = 0; u < U; ++u) ag[u] = au[u] = 0.0f;
#pragma unroll
    for (int j = 0; j < J; ++j) {
      uint4 xr[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) xr[q] = s_x4[q * nb + li + G * j];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        bf16x2_t wv[16];
        dequant_bf16(qg[u][j], wv);
        ag[u] += chunk_dot_bf16_reg(wv, xr) * e8m0_to_f32(sg[u][j]);
        dequant_bf16(qu[u][j], wv);
        au[u] += chunk_dot_bf16_reg(wv, xr) * e8m0_to_f32(su[u][j]);
        load_chunk(it + istep, u, j, next_off);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int n = n0 + u * rpi + gi;
      const float g = group_sum_last(ag[u], G);
      const float uu = group_sum_last(au[u], G);
      if (li == G - 1 && n < I) h[(int64_t)p0 * I + n] = silu_mul(g, uu);
    }
  }
}

constexpr size_t kMaxLds = 65536;

int pick_mt(size_t bytes_per_row) {
  if (4 * bytes_per_row <= kMaxLds) return 4;
  if (2 * bytes_per_row <= kMaxLds) return 2;
  return 1;
}

// Lane layout of the register GEMV for rows of nb blocks: G = 2^lg lanes per
// row with G the largest power of two (at most 64) dividing nb, J = nb / G
// blocks per lane, U row groups per iteration (loads in flight per lane =
// U * J for down, 2 * U * J for gate/up).  J above 8 takes the LDS path.
struct GemvShape {
  bool ok;
  int lg, J, U;
};

GemvShape gemv_shape(int nb, bool gateup) {
  int lg = 0;
  while (lg < 6 && (nb % (2 << lg)) == 0) ++lg;
  const int J = nb >> lg;
  if (J > 8) return {false, 0, 0, 0};
  if (gateup && nb == 224) return {true, lg, J, kGateU224};
  if (!gateup && nb == 48) return {true, lg, J, kDownU48};
  int U;
  if (gateup)
    U = J == 1 ? 4 : (J <= 3 ? 2 : 1);
  else
    U = J == 1 ? 8 : (J == 2 ? 4 : (J == 3 ? 4 : (J == 4 ? 2 : 1)));
  return {true, lg, J, U};
}

struct GemvGrid {
  int ipw;                // row-iterations per wave
  int blocks_per_expert;  // blocks of 4 waves per active-expert slot
};

// One round of resident waves (waves_per_simd on each of the 1024 SIMDs) for
// the upper bound of active experts, and at least 8 blocks per expert so that
// a few busy experts still spread.
GemvGrid gemv_grid(int iters_per_expert, int max_active, int waves_per_simd) {
  const long total = (long)iters_per_expert * max_active;
  const long slots = 1024L * waves_per_simd;
  int ipw = (int)((total + slots - 1) / slots);
  const int cap = (iters_per_expert + 31) / 32;
  if (ipw > cap) ipw = cap;
  if (ipw < 1) ipw = 1;
  const int bpe = (iters_per_expert + kWaves * ipw - 1) / (kWaves * ipw);
  return {ipw, bpe};
}

// Several tokens: about 32 blocks (128 waves) per expert, so a few dozen
// small experts already fill the machine; the grid strides over the items.
GemvGrid multi_grid(int iters_per_expert) {
  const int ipw = max(1, (iters_per_expert + 127) / 128);
  return {ipw, (iters_per_expert + kWaves * ipw - 1) / (kWaves * ipw)};
}
constexpr int kMultiGridCap = 2048;  // blocks of a grid-stride GEMV launch

size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

struct GemvArgs {
  const uint16_t* x;
  int k;
  const moe_mxfp4_weights* w;
  const int32_t *offsets, *sorted_rows, *active;
  float *h, *y_rows;
  hipStream_t s;
};

// Register gate/up GEMV for experts with lo..hi rows, MT rows per weight pass.
template <int MT>
void gateup_reg(const GemvArgs& a, const GemvShape& sh, const GemvGrid& gg, dim3 grid, const int32_t* list, int lo,
                int hi) {
  const int H = a.w->hidden;
  const size_t lds = (size_t)MT * H * 2;
#define GU(JJ, UU, NB)                                                                                          \
  hipLaunchKernelGGL((gateup_gemv_reg_kernel<JJ, UU, MT, NB>), grid, dim3(kThreads), lds, a.s, a.x, a.k, *a.w, \
                     a.offsets, a.sorted_rows, a.active, list, a.h, sh.lg, gg.blocks_per_expert, lo, hi)
  if (H == 7168) {
    GU(7, kGateU224, 224);
    return;
  }
  switch (sh.J) {
    case 1: GU(1, 4, 0); break;
    case 2: GU(2, 2, 0); break;
    case 3: GU(3, 2, 0); break;
    case 4: GU(4, 1, 0); break;
    case 5: GU(5, 1, 0); break;
    case 6: GU(6, 1, 0); break;
    case 7: GU(7, 1, 0); break;
    default: GU(8, 1, 0); break;
  }
#undef GU
}

// Register down GEMV for experts with lo..hi rows, MT rows per weight pass.
template <int MT>
void down_reg(const GemvArgs& a, const GemvShape& sh, const GemvGrid& gg, dim3 grid, const int32_t* list, int lo,
              int hi) {
  const int I = a.w->inter;
  const size_t lds = (size_t)MT * I * 4;
#define DN(JJ, UU, NB)                                                                                              \
  hipLaunchKernelGGL((down_gemv_reg_kernel<JJ, UU, MT, NB>), grid, dim3(kThreads), lds, a.s, a.h, *a.w, a.offsets, \
                     a.active, list, a.y_rows, sh.lg, gg.blocks_per_expert, lo, hi)
  if (I == 1536) {
    DN(3, kDownU48, 48);
    return;
  }
  switch (sh.J) {
    case 1: DN(1, 8, 0); break;
    case 2: DN(2, 4, 0); break;
    case 3: DN(3, 4, 0); break;
    case 4: DN(4, 2, 0); break;
    case 5: DN(5, 1, 0); break;
    case 6: DN(6, 1, 0); break;
    case 7: DN(7, 1, 0); break;
    default: DN(8, 1, 0); break;
  }
#undef DN
}

// Class lists of the register GEMVs (several tokens): 2 x (1 + max_active).
size_t lists_bytes(int T, int k, int E) {
  const size_t R = (size_t)T * k, mx = R < (size_t)E ? R : (size_t)E;
  return align_up(2 * (1 + mx) * sizeof(int32_t), 256);
}

}  // namespace

namespace moe {

size_t expert_ffn_workspace(int T, int k, int E, int H, int I) {
  size_t b = align_up((size_t)T * k * I * sizeof(float), 256);  // h[R][I]
  if (T > 1) b += lists_bytes(T, k, E);
  if (T > 1 && mfma_shape_ok(H, I)) b += mfma_workspace(T, k, E, H, I);
  return b;
}

namespace {

// The expert FFN; with gateup_only (one token, register gate/up shape) it
// stops after h, for the fused down + combine launch.
hipError_t expert_ffn_impl(const uint16_t* x, int T, int k, const moe_mxfp4_weights& w, const int32_t* offsets,
                           const int32_t* sorted_rows, const int32_t* active, float* y_rows, void* ws,
                           hipStream_t s, bool gateup_only) {
  if (T == 0) return hipSuccess;
  const int R = T * k, E = w.num_experts, H = w.hidden, I = w.inter;
  const int max_active = R < E ? R : E;
  float* hbuf = (float*)ws;
  // Register GEMVs: experts with one row (MT = 1) and with 2..reg_max rows
  // (MT = kRegRows, same per-row arithmetic); a single token sends every
  // expert through MT = 1 (its row loop covers an id repeated in the token).
  // Experts with more rows take the grouped GEMM (MFMA) when the shape
  // allows it, else the LDS GEMV.  Shapes the register layout cannot take
  // (more than 8 blocks per lane) run on the LDS GEMV throughout.
  const GemvShape sg = gemv_shape(H >> 5, true), sd = gemv_shape(I >> 5, false);
  const bool reg_g = sg.ok, reg_d = sd.ok;
  // up to kInvariantTokens tokens every expert stays on the register GEMVs
  // (rows in passes of kRegRows), so no grouped-GEMM launch is made at all
  const bool all_reg = T <= kInvariantTokens && reg_g && reg_d;
  const bool use_mfma = !all_reg && T > 1 && reg_g && reg_d && mfma_shape_ok(H, I);
  const int reg_max = all_reg ? INT32_MAX : use_mfma ? reg_rows_max(T) : kRegRows;
  // fewest rows of the multi-row class: with every expert on the GEMVs one
  // launch per projection takes them all (one-row experts get a single pass)
  const int lo4 = all_reg ? 1 : 2;

  hipError_t err = hipSuccess;
  const GemvArgs ga{x, k, &w, offsets, sorted_rows, active, hbuf, y_rows, s};
  // several tokens: class lists of the register GEMVs (after h in the workspace)
  size_t off = align_up((size_t)R * I * sizeof(float), 256);
  int32_t *l1 = nullptr, *l4 = nullptr;
  if (T > 1) {
    l1 = (int32_t*)((uint8_t*)ws + off);
    l4 = l1 + 1 + max_active;
    off += lists_bytes(T, k, E);
    if (use_mfma) {  // the grouped GEMM's prep launch also writes the class lists
      if ((err = launch_mfma_prep(x, T, k, w, offsets, active, (uint8_t*)ws + off, l1, l4, lo4, reg_max, s)) !=
          hipSuccess)
        return err;
    } else if ((reg_g || reg_d) && !all_reg) {  // with every expert on the GEMVs the active list is the class list
      hipLaunchKernelGGL(small_lists_kernel, dim3(1), dim3(kThreads), 0, s, offsets, active, l1, l4, lo4, reg_max);
      if ((err = hipGetLastError()) != hipSuccess) return err;
    }
  }
  // grids of the class launches: n_max experts of the class at most
  auto multi = [&](int n_max, const GemvGrid& gg) {
    const long b = (long)n_max * gg.blocks_per_expert;
    return dim3((unsigned)(b < kMultiGridCap ? b : kMultiGridCap));
  };
  const int n1_max = lo4 > 1 ? max_active : 0, n4_max = lo4 > 1 && R / 2 < max_active ? R / 2 : max_active;
  if (reg_g) {
    const int rows_it = (64 >> sg.lg) * sg.U, iters = (I + rows_it - 1) / rows_it;
    if (T == 1) {
      const GemvGrid gg = gemv_grid(iters, max_active, H == 7168 ? 4 : 2);
      if (H == 7168)
        hipLaunchKernelGGL((gateup_gemv_one_kernel<7, kGateU224, 224>), dim3(max_active * gg.blocks_per_expert),
                           dim3(kThreads), (size_t)H * 2, s, x, w, offsets, active, hbuf, gg.blocks_per_expert);
      else
        gateup_reg<1>(ga, sg, gg, dim3(max_active * gg.blocks_per_expert), nullptr, 1, INT32_MAX);
    } else {
      const GemvGrid gg = multi_grid(iters);
      if (n1_max > 0) gateup_reg<1>(ga, sg, gg, multi(n1_max, gg), l1, 1, 1);
      if ((err = hipGetLastError()) != hipSuccess) return err;
      if (all_reg)  // one block per (active slot, block of the expert), no list
        gateup_reg<kRegRows>(ga, sg, gg, dim3(max_active * gg.blocks_per_expert), nullptr, 1, reg_max);
      else if (reg_max > 1)
        gateup_reg<kRegRows>(ga, sg, gg, multi(n4_max, gg), l4, lo4, reg_max);
    }
    if ((err = hipGetLastError()) != hipSuccess) return err;
  }
  if (gateup_only) return hipSuccess;
  uint8_t* mfma_ws = (uint8_t*)ws + off;
  if (use_mfma) {
    if ((err = launch_mfma_gateup(T, k, w, sorted_rows, mfma_ws, s)) != hipSuccess)
      return err;
  } else if (!reg_g || (T > 1 && !all_reg)) {
    const int mt_g = pick_mt((size_t)H * 2);
    dim3 grid_g((I + kRowsPerBlock - 1) / kRowsPerBlock, max_active);
    const size_t lds_g = (size_t)mt_g * H * 2;
    const int skip = reg_g ? kRegRows : 0;
    if (mt_g == 4)
      hipLaunchKernelGGL(gateup_gemv_lds_kernel<4>, grid_g, dim3(kThreads), lds_g, s, x, k, w, offsets, sorted_rows,
                         active, hbuf, skip);
    else if (mt_g == 2)
      hipLaunchKernelGGL(gateup_gemv_lds_kernel<2>, grid_g, dim3(kThreads), lds_g, s, x, k, w, offsets, sorted_rows,
                         active, hbuf, skip);
    else
      hipLaunchKernelGGL(gateup_gemv_lds_kernel<1>, grid_g, dim3(kThreads), lds_g, s, x, k, w, offsets, sorted_rows,
                         active, hbuf, skip);
    if ((err = hipGetLastError()) != hipSuccess) return err;
  }

  if (reg_d) {
    const int rows_it = (64 >> sd.lg) * sd.U, iters = (H + rows_it - 1) / rows_it;
    if (T == 1 && I == 1536) {
      // the one-token down kernel: one row group per iteration (94 VGPRs),
      // a grid for 4 waves per SIMD
      const int rows_one = (64 >> sd.lg) * kDownOneU48, iters_one = (H + rows_one - 1) / rows_one;
      const GemvGrid gd = gemv_grid(iters_one, max_active, 4);
      hipLaunchKernelGGL((down_gemv_one_kernel<3, kDownOneU48, 48>), dim3(max_active * gd.blocks_per_expert),
                         dim3(kThreads), (size_t)I * 4, s, hbuf, w, offsets, active, y_rows, gd.blocks_per_expert);
    } else if (T == 1) {
      const GemvGrid gd = gemv_grid(iters, max_active, 2);
      down_reg<1>(ga, sd, gd, dim3(max_active * gd.blocks_per_expert), nullptr, 1, INT32_MAX);
    } else {
      const GemvGrid gd = multi_grid(iters);
      if (n1_max > 0) down_reg<1>(ga, sd, gd, multi(n1_max, gd), l1, 1, 1);
      if ((err = hipGetLastError()) != hipSuccess) return err;
      if (all_reg)
        down_reg<kRegRows>(ga, sd, gd, dim3(max_active * gd.blocks_per_expert), nullptr, 1, reg_max);
      else if (reg_max > 1)
        down_reg<kRegRows>(ga, sd, gd, multi(n4_max, gd), l4, lo4, reg_max);
    }
    if ((err = hipGetLastError()) != hipSuccess) return err;
  }
  if (use_mfma) {
    if ((err = launch_mfma_down(T, k, w, sorted_rows, y_rows, mfma_ws, s)) != hipSuccess)
      return err;
  } else if (!reg_d || (T > 1 && !all_reg)) {
    const int mt_d = pick_mt((size_t)I * 4);
    dim3 grid_d((H + kRowsPerBlock - 1) / kRowsPerBlock, max_active);
    const size_t lds_d = (size_t)mt_d * I * 4;
    const int skip = reg_d ? kRegRows : 0;
    if (mt_d == 4)
      hipLaunchKernelGGL(down_gemv_lds_kernel<4>, grid_d, dim3(kThreads), lds_d, s, hbuf, w, offsets, active, y_rows,
                         skip);
    else if (mt_d == 2)
      hipLaunchKernelGGL(down_gemv_lds_kernel<2>, grid_d, dim3(kThreads), lds_d, s, hbuf, w, offsets, active, y_rows,
                         skip);
    else
      hipLaunchKernelGGL(down_gemv_lds_kernel<1>, grid_d, dim3(kThreads), lds_d, s, hbuf, w, offsets, active, y_rows,
                         skip);
    if ((err = hipGetLastError()) != hipSuccess) return err;
  }
  return hipSuccess;
}

}  // namespace

hipError_t launch_expert_ffn(const uint16_t* x, int T, int k, const moe_mxfp4_weights& w, const int32_t* offsets,
                             const int32_t* sorted_rows, const int32_t* active, float* y_rows, void* ws,
                             hipStream_t s) {
  return expert_ffn_impl(x, T, k, w, offsets, sorted_rows, active, y_rows, ws, s, false);
}

hipError_t launch_expert_ffn_combine(const uint16_t* x, int T, int k, const moe_mxfp4_weights& w,
                                     const int32_t* offsets, const int32_t* sorted_rows, const int32_t* active,
                                     const float* topk_w, const int32_t* row_pos, float* y_rows, float* out,
                                     void* ws, hipStream_t s) {
  if (T == 0) return hipSuccess;
  const bool fused = T == 1 && k <= kFMaxK && w.inter == 1536 && gemv_shape(w.hidden >> 5, true).ok;
  if (!fused) {
    hipError_t err = expert_ffn_impl(x, T, k, w, offsets, sorted_rows, active, y_rows, ws, s, false);
    if (err != hipSuccess) return err;
    return launch_combine(y_rows, topk_w, row_pos, T, k, w.hidden, out, s);
  }
  hipError_t err = expert_ffn_impl(x, T, k, w, offsets, sorted_rows, active, y_rows, ws, s, true);
  if (err != hipSuccess) return err;
  constexpr int kRows = kFIters * 4;  // NB = 48: 16 lanes per row, 4 rows per iteration
  hipLaunchKernelGGL(down_combine_one_kernel<48>, dim3((w.hidden + kRows - 1) / kRows), dim3(kFThreads), 0, s,
                     (const float*)ws, w, offsets, active, topk_w, row_pos, k, y_rows, out);
  return hipGetLastError();
}

bool route_ffn_combine_one_ok(int E, int k, const moe_mxfp4_weights& w) {
  return w.hidden == 7168 && w.inter == 1536 && k >= 1 && k <= kFMaxK && k <= E && E <= kRegExperts;
}

hipError_t launch_route_ffn_combine_one(const float* logits, int k, const uint16_t* x, const float* y_prev,
                                        float eps, uint16_t* x_next, const moe_mxfp4_weights& w, int32_t* ids,
                                        float* topk_w, int32_t* offsets, int32_t* sorted_rows, int32_t* row_pos,
                                        int32_t* active, float* y_rows, float* out, void* ws, hipStream_t s) {
  const int E = w.num_experts, H = w.hidden, I = w.inter;
  const GemvShape sg = gemv_shape(H >> 5, true);
  const int rows_it = (64 >> sg.lg) * sg.U, iters = (I + rows_it - 1) / rows_it;
  // the one-token gate/up grid (4 waves per SIMD) in blocks of 16 waves
  const GemvGrid gg = gemv_grid(iters, k, 4);
  const int bpe = (iters + kRGWaves * gg.ipw - 1) / (kRGWaves * gg.ipw);
  const dim3 grid(k * bpe);
  float* hbuf = (float*)ws;
  const size_t lds = (size_t)H * 2;
#define RG(C, RMS)                                                                                             \
  hipLaunchKernelGGL((route_gateup_one_kernel<7, kGateU224, 224, C, RMS>), grid, dim3(kRGThreads), lds, s,      \
                     logits, E, k, x, y_prev, eps, x_next, w, hbuf, ids, topk_w, offsets, sorted_rows, row_pos,     \
                     active, bpe)
  const bool rms = y_prev != nullptr;
  static_assert(kWideThreads * 8 >= kRegExperts, "C <= 8 covers every fused E");
  if (E <= kWideThreads) {
    if (rms) RG(1, true); else RG(1, false);
  } else if (E <= 2 * kWideThreads) {
    if (rms) RG(2, true); else RG(2, false);
  } else if (E <= 4 * kWideThreads) {
    if (rms) RG(4, true); else RG(4, false);
  } else {
    if (rms) RG(8, true); else RG(8, false);
  }
#undef RG
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  constexpr int kRows = kFIters * 4;
  hipLaunchKernelGGL(down_combine_one_kernel<48>, dim3((H + kRows - 1) / kRows), dim3(kFThreads), 0, s,
                     (const float*)ws, w, offsets, active, topk_w, row_pos, k, y_rows, out);
  return hipGetLastError();
}

}  // namespace moe
