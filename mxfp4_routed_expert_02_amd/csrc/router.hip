// router.hip - the router projection before the path:
//   logits[t][e] = sum_c x[t][c] * Wr[e][c]
// x bf16 [T][H], Wr fp32 [E][H], logits fp32 [T][E], fp32 accumulation
// (the router picks each token's experts from these logits: page
// "hn.213312.xyz/article/49090233", section on how it works; the pages do
// not give the router's form, so the weights are a synthetic fp32 matrix).
//
// Few tokens (decode, T <= 4): the projection streams Wr once (25.7 MB at
// 896 x 7168), so it is a GEMV, one block per expert row.
// More tokens: a GEMM on the bf16 MFMA with the weights split exactly in
// three bf16 terms (below).
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

// More tokens: a GEMM on the bf16 MFMA (v_mfma_f32_32x32x16_bf16).  x is
// bf16 already; each fp32 weight w splits exactly into three bf16 terms
// (w1 = w with its low 16 bits cleared, w2 the same of w - w1, w3 = the
// remainder, at most 8 significant bits), so every product x * w_i is exact
// in fp32 and the MFMA accumulates sum_c x[c] * (w1 + w2 + w3)[c] in fp32,
// three bf16 MFMAs per 16-deep step (a third of the bf16 rate, five times
// the fp32 MFMA's).  Tile: 32 experts x 64 tokens per block of 8 waves (at
// 512 tokens and 896 experts, 224 blocks for the 256 CUs): waves 0-3 take
// the first half of K and waves 4-7 the second; within a half, wave w takes
// token block w % 2 and the 16-deep steps 2 (w / 2), 2 (w / 2) + 1 of every
// 64-value stage, so each output element has four partial sums, which meet
// in LDS at the end in a fixed order (first half's two, then the second
// half's two).  K stages of 64 values sit in LDS as three weight planes
// [32][64] and one x plane [64][64] of bf16, double-buffered, the 16-byte
// piece p of row r at r*128 + 16*(p ^ ((r >> 1) & 7)) so that the fragment
// reads of 16 consecutive rows hit distinct bank groups.  Global loads run
// two stages ahead through two register sets.  Blocks of one expert tile
// run on one XCD, which then reads that tile of Wr once.
constexpr int kRe = 32, kRtok = 64;  // experts and tokens per block
constexpr int kRk = 64;              // K values per stage
constexpr int kRthreads = 512;  // two halves of 4 waves
constexpr int kWPlane = kRe * kRk * 2, kXPlane = kRtok * kRk * 2;  // bytes
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float v16f_t __attribute__((ext_vector_type(16)));

__device__ __forceinline__ int swz(int r, int p) { return r * 128 + 16 * (p ^ ((r >> 1) & 7)); }

struct RouterStage {
  float4 w[2];  // 8 weights of one expert row
  uint4 x[2];   // 16 bf16 of one token row
};

// high halves of two fp32 bit patterns packed as two bf16 (a low, b high)
__device__ __forceinline__ uint32_t hi_pair(float a, float b) {
  return __builtin_amdgcn_perm(__float_as_uint(b), __float_as_uint(a), 0x07060302u);
}
__device__ __forceinline__ float lo_rest(float v) {  // v minus v with its low 16 bits cleared (exact)
  return v - __uint_as_float(__float_as_uint(v) & 0xFFFF0000u);
}

__global__ __launch_bounds__(kRthreads) void router_mfma_kernel(const uint16_t* __restrict__ x, int H,
                                                                const float* __restrict__ wr, int E,
                                                                float* __restrict__ logits, int T, int n_t) {
  // [K half][buffer]: w1, w2, w3 planes then the x plane
  __shared__ __attribute__((aligned(16))) uint8_t s_all[2][2][3 * kWPlane + kXPlane];
  const int khalf = threadIdx.x >> 8;
  uint8_t(&s_buf)[2][3 * kWPlane + kXPlane] = s_all[khalf];
  const int tid = threadIdx.x & 255, lane = tid & 63, wave = tid >> 6;
  // XCD x = blockIdx % 8 takes expert tiles x, x + 8, ...; within one, all token tiles
  const int bx = blockIdx.x, slot = bx >> 3;
  const int et = (bx & 7) + 8 * (slot / n_t), ttile = slot - (slot / n_t) * n_t;
  const int e0 = et * kRe, t0 = ttile * kRtok;
  if (e0 >= E) return;

  // staging: thread t takes expert row t/8, K values 8 (t%8) .. +7 of the
  // stage, and token row t/4, K values 16 (t%4) .. +15
  const int wrow = tid >> 3, wk = 8 * (tid & 7), xrow = tid >> 2, xk = 16 * (tid & 3);
  // rows past E or T read row 0 (their outputs are never stored); K past H
  // reads in range and is zeroed, so every load is unconditional
  // this half's stages: nst of 64 K values from kbase (both halves run the
  // same number, so their barriers pair up; the second half's last may lie
  // past H and loads zeros)
  const int nst = ((H + kRk - 1) / kRk + 1) / 2;
  const int kbase = khalf * nst * kRk;
  const float* wsrc = wr + (int64_t)(e0 + wrow < E ? e0 + wrow : 0) * H;
  const uint16_t* xsrc = x + (int64_t)(t0 + xrow < T ? t0 + xrow : 0) * H;
  auto load = [&](int k0, RouterStage& r) {
    // H % 32 == 0: an 8- or 16-value segment is all in or all out
    const bool win = kbase + k0 + wk < H, xin = kbase + k0 + xk < H;
    const int kw = win ? kbase + k0 + wk : 0, kx = xin ? kbase + k0 + xk : 0;
    const uint32_t mw = win ? ~0u : 0u, mx = xin ? ~0u : 0u;  // bit masks, not branches
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const uint4 v = *(const uint4*)(wsrc + kw + 4 * i);
      r.w[i] = make_float4(__uint_as_float(v.x & mw), __uint_as_float(v.y & mw), __uint_as_float(v.z & mw),
                           __uint_as_float(v.w & mw));
    }
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const uint4 v = *(const uint4*)(xsrc + kx + 8 * i);
      r.x[i] = make_uint4(v.x & mx, v.y & mx, v.z & mx, v.w & mx);
    }
  };
  auto store = [&](int b, const RouterStage& r) {
    const float f[8] = {r.w[0].x, r.w[0].y, r.w[0].z, r.w[0].w, r.w[1].x, r.w[1].y, r.w[1].z, r.w[1].w};
    uint32_t t1[4], t2[4], t3[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float a = f[2 * i], c = f[2 * i + 1];
      const float ra = lo_rest(a), rc = lo_rest(c);    // w - w1
      const float qa = lo_rest(ra), qc = lo_rest(rc);  // w - w1 - w2 = w3
      t1[i] = hi_pair(a, c);
      t2[i] = hi_pair(ra, rc);
      t3[i] = hi_pair(qa, qc);
    }
    const int o = swz(wrow, wk >> 3);  // 8 weights = one 16-byte piece per plane
    *(uint4*)&s_buf[b][o] = make_uint4(t1[0], t1[1], t1[2], t1[3]);
    *(uint4*)&s_buf[b][kWPlane + o] = make_uint4(t2[0], t2[1], t2[2], t2[3]);
    *(uint4*)&s_buf[b][2 * kWPlane + o] = make_uint4(t3[0], t3[1], t3[2], t3[3]);
#pragma unroll
    for (int h = 0; h < 2; ++h) *(uint4*)&s_buf[b][3 * kWPlane + swz(xrow, (xk >> 3) + h)] = r.x[h];
  };

  // wave's output block: all 32 experts x tokens 32 (wave & 1) ..; its
  // 16-deep steps 2 (wave >> 1) and 2 (wave >> 1) + 1 of every stage
  const int n = lane & 31, kh = lane >> 5;
  const int tb = wave & 1, kg = wave >> 1;
  const int arow = n, brow = 32 * tb + n;
  v16f_t acc;
#pragma unroll
  for (int r = 0; r < 16; ++r) acc[r] = 0.0f;
  auto compute = [&](int b) {
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2) {
      const int p = 2 * (2 * kg + s2) + kh;  // lane's 8 K values: 16 s + 8 kh
      const bf16x8_t xb = *(const bf16x8_t*)&s_buf[b][3 * kWPlane + swz(brow, p)];
#pragma unroll
      for (int term = 0; term < 3; ++term) {
        const bf16x8_t wa = *(const bf16x8_t*)&s_buf[b][term * kWPlane + swz(arow, p)];
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wa, xb, acc, 0, 0, 0);
      }
    }
  };

  // stage st of the half in LDS buffer st % 2; its global loads were issued
  // two stages earlier into register set st % 2.  The main loop (a stage
  // three ahead still to load) has no conditions, so its body schedules as
  // one block; the last (at most three) stages follow.
  RouterStage r0, r1;
  load(0, r0);
  if (nst > 1) load(kRk, r1);
  store(0, r0);
  __syncthreads();
  int st = 0;
  for (; st + 3 < nst; st += 2) {
    load((st + 2) * kRk, r0);
    compute(0);
    store(1, r1);
    __syncthreads();
    load((st + 3) * kRk, r1);
    compute(1);
    store(0, r0);
    __syncthreads();
  }
  // buffer 0 holds stage st, r1 stage st + 1 (if they exist)
  if (st + 2 < nst) load((st + 2) * kRk, r0);
  compute(0);
  if (st + 1 < nst) {
    store(1, r1);
    __syncthreads();
    compute(1);
    if (st + 2 < nst) {
      store(0, r0);
      __syncthreads();
      compute(0);
    }
  }
  // the four partial sums of each output element meet in LDS (over the
  // stage buffers, now free): every wave but the first half's kg = 0 pair
  // writes its sums to slot (half, kg) of its token block; those two waves
  // add them in the order (half 0, kg 1), (half 1, kg 0), (half 1, kg 1).
  // D lane l, register r: token l % 32 of the block, expert 8 (r/4) + 4 (l/32) + r%4
  float* s_red = (float*)&s_all[0][0][0];
  __syncthreads();  // every wave is done reading its stages
  const int part = 2 * khalf + kg;  // 0 .. 3
  if (part > 0) {
#pragma unroll
    for (int r = 0; r < 16; ++r) s_red[(((part - 1) * 2 + tb) * 16 + r) * 64 + lane] = acc[r];
  }
  __syncthreads();
  if (part > 0) return;
  const int t = t0 + 32 * tb + n;
  if (t >= T) return;
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int e = e0 + 8 * (r >> 2) + 4 * kh + (r & 3);
    float v = acc[r];
#pragma unroll
    for (int q = 0; q < 3; ++q) v += s_red[((q * 2 + tb) * 16 + r) * 64 + lane];
    if (e < E) logits[(int64_t)t * E + e] = v;
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
    const int n_e = (E + kRe - 1) / kRe, n_t = (T + kRtok - 1) / kRtok;
    const dim3 g((unsigned)(8 * ((n_e + 7) / 8) * n_t)), b(kRthreads);
    hipLaunchKernelGGL(router_mfma_kernel, g, b, 0, s, x, H, wr, E, logits, T, n_t);
  }
  return hipGetLastError();
}

}  // namespace moe
