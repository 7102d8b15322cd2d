// route_group.hip - router top-k and expert-major row grouping (gfx950).
//
// Top-k: one wavefront per token.  The token's logits sit in LDS; each of
// the k rounds is a wavefront arg-max over the experts not yet taken (lane
// scan, then a butterfly of (value, id) pairs: larger value wins, equal
// values go to the lower id), so the ids come out in rank order.  The
// softmax over the k picked logits runs in one lane in rank order.
//
// Grouping: a stable counting sort of the flat rows r = t*k + j by expert.
// Counts and OR-ed bitmaps are the only LDS atomics (both order-free), so
// the permutation does not depend on scheduling.  Within a chunk of rows a
// row's rank among the rows of its expert is the popcount of that expert's
// bitmap below the row.
#include "moe_internal.h"

namespace {

constexpr int kRouteThreads = 64;  // one wave per token

__global__ __launch_bounds__(kRouteThreads) void route_topk_kernel(const float* __restrict__ logits, int E, int k,
                                                                   int32_t* __restrict__ ids,
                                                                   float* __restrict__ weights) {
  extern __shared__ float s_logit[];               // [E]
  uint32_t* s_taken = (uint32_t*)(s_logit + E);   // [ceil(E/32)] bitmap
  __shared__ float s_val[MOE_MAX_TOPK];
  const int t = blockIdx.x;
  const int lane = threadIdx.x;
  const float* row = logits + (int64_t)t * E;
  for (int e = lane; e < E; e += kRouteThreads) s_logit[e] = row[e];
  for (int i = lane; i < (E + 31) / 32; i += kRouteThreads) s_taken[i] = 0u;
  __syncthreads();

  for (int j = 0; j < k; ++j) {
    float bv = 0.0f;
    int bi = -1;
    for (int e = lane; e < E; e += kRouteThreads) {
      if (s_taken[e >> 5] & (1u << (e & 31))) continue;
      const float v = s_logit[e];
      if (bi < 0 || v > bv) {  // ascending e per lane: a tie keeps the lower id
        bv = v;
        bi = e;
      }
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
      const float ov = __shfl_xor(bv, o, kRouteThreads);
      const int oi = __shfl_xor(bi, o, kRouteThreads);
      if (oi >= 0 && (bi < 0 || ov > bv || (ov == bv && oi < bi))) {
        bv = ov;
        bi = oi;
      }
    }
    if (lane == 0) {
      s_taken[bi >> 5] |= 1u << (bi & 31);
      s_val[j] = bv;
      ids[(int64_t)t * k + j] = bi;
    }
    __syncthreads();
  }

  if (lane == 0) {
    const float m = s_val[0];
    float S = 0.0f;
    for (int j = 0; j < k; ++j) {
      const float ex = expf(s_val[j] - m);
      s_val[j] = ex;
      S += ex;
    }
    for (int j = 0; j < k; ++j) weights[(int64_t)t * k + j] = s_val[j] / S;
  }
}

// ------------------------------------------------------------------ group --
constexpr int kGroupThreads = 1024;
constexpr int kGroupLds = 61440;  // bytes of dynamic LDS the grouping kernel may use

// words of bitmap per expert per chunk (chunk = 32 * W rows)
__host__ __device__ inline int group_words(int E) {
  int words = (kGroupLds - 8 * E) / 4 / E;
  return words > 32 ? 32 : (words < 1 ? 1 : words);
}

// In-place exclusive scan of a[0..n) in LDS by the whole block; returns total.
__device__ int block_exclusive_scan(int* a, int n, int* s_wave) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int per = (n + kGroupThreads - 1) / kGroupThreads;
  const int beg = min(n, tid * per), end = min(n, beg + per);
  int local = 0;
  for (int i = beg; i < end; ++i) local += a[i];
  // inclusive scan of `local` within the wave
  int v = local;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int u = __shfl_up(v, o, 64);
    if (lane >= o) v += u;
  }
  if (lane == 63) s_wave[wave] = v;
  __syncthreads();
  if (tid == 0) {
    int acc = 0;
    for (int w = 0; w < kGroupThreads / 64; ++w) {
      const int c = s_wave[w];
      s_wave[w] = acc;
      acc += c;
    }
    s_wave[kGroupThreads / 64] = acc;
  }
  __syncthreads();
  int run = s_wave[wave] + v - local;
  for (int i = beg; i < end; ++i) {
    const int c = a[i];
    a[i] = run;
    run += c;
  }
  const int total = s_wave[kGroupThreads / 64];
  __syncthreads();
  return total;
}

__global__ __launch_bounds__(kGroupThreads) void group_rows_kernel(const int32_t* __restrict__ ids, int R, int E,
                                                                   int32_t* __restrict__ offsets,
                                                                   int32_t* __restrict__ sorted_rows,
                                                                   int32_t* __restrict__ row_pos,
                                                                   int32_t* __restrict__ active) {
  extern __shared__ int s_mem[];
  int* s_count = s_mem;             // [E] counts, then running positions
  int* s_flag = s_mem + E;          // [E] active flags, then their scan
  uint32_t* s_bits = (uint32_t*)(s_mem + 2 * E);
  __shared__ int s_wave[kGroupThreads / 64 + 1];
  const int tid = threadIdx.x;
  const int W = group_words(E);
  const int CH = 32 * W;

  for (int e = tid; e < E; e += kGroupThreads) s_count[e] = 0;
  __syncthreads();
  // ids outside [0, E) break the documented precondition; they are skipped so
  // that no LDS access leaves the arrays
  for (int r = tid; r < R; r += kGroupThreads) {
    const int e = ids[r];
    if ((unsigned)e < (unsigned)E) atomicAdd(&s_count[e], 1);
  }
  __syncthreads();
  for (int e = tid; e < E; e += kGroupThreads) s_flag[e] = s_count[e] > 0 ? 1 : 0;
  __syncthreads();
  const int total = block_exclusive_scan(s_count, E, s_wave);  // s_count = offsets
  for (int e = tid; e < E; e += kGroupThreads) offsets[e] = s_count[e];
  if (tid == 0) offsets[E] = total;
  // active list: experts whose offset range is non-empty, ascending
  for (int e = tid; e < E; e += kGroupThreads) {
    const int next = (e + 1 < E) ? s_count[e + 1] : total;
    s_flag[e] = next > s_count[e] ? 1 : 0;
  }
  __syncthreads();
  {
    // keep flags to know which slots to write: scan a copy held per thread
    const int per = (E + kGroupThreads - 1) / kGroupThreads;
    const int beg = min(E, tid * per), end = min(E, beg + per);
    int mine[MOE_MAX_EXPERTS / kGroupThreads];
    for (int i = beg; i < end; ++i) mine[i - beg] = s_flag[i];
    __syncthreads();
    const int na = block_exclusive_scan(s_flag, E, s_wave);
    for (int i = beg; i < end; ++i)
      if (mine[i - beg]) active[1 + s_flag[i]] = i;
    if (tid == 0) active[0] = na;
  }

  // stable placement, one chunk of CH rows at a time (s_count = running position)
  for (int c0 = 0; c0 < R; c0 += CH) {
    const int n = min(CH, R - c0);
    for (int i = tid; i < E * W; i += kGroupThreads) s_bits[i] = 0u;
    __syncthreads();
    for (int p = tid; p < n; p += kGroupThreads) {
      const int e = ids[c0 + p];
      if ((unsigned)e < (unsigned)E) atomicOr(&s_bits[e * W + (p >> 5)], 1u << (p & 31));
    }
    __syncthreads();
    for (int p = tid; p < n; p += kGroupThreads) {
      const int e = ids[c0 + p];
      if ((unsigned)e >= (unsigned)E) continue;
      const uint32_t* b = s_bits + e * W;
      int rank = __popc(b[p >> 5] & ((1u << (p & 31)) - 1u));
      for (int w = 0; w < (p >> 5); ++w) rank += __popc(b[w]);
      const int pos = s_count[e] + rank;
      sorted_rows[pos] = c0 + p;
      row_pos[c0 + p] = pos;
    }
    __syncthreads();
    for (int e = tid; e < E; e += kGroupThreads) {
      int c = 0;
      for (int w = 0; w < W; ++w) c += __popc(s_bits[e * W + w]);
      s_count[e] += c;
    }
    __syncthreads();
  }
}

}  // namespace

namespace moe {

hipError_t launch_route_topk(const float* logits, int T, int E, int k, int32_t* ids, float* w, hipStream_t s) {
  if (T == 0) return hipSuccess;
  const size_t lds = (size_t)E * sizeof(float) + (size_t)((E + 31) / 32) * sizeof(uint32_t);
  hipLaunchKernelGGL(route_topk_kernel, dim3(T), dim3(kRouteThreads), lds, s, logits, E, k, ids, w);
  return hipGetLastError();
}

size_t group_rows_workspace(int T, int k, int E) {
  (void)T;
  (void)k;
  (void)E;
  return 0;
}

hipError_t launch_group_rows(const int32_t* ids, int T, int k, int E, int32_t* offsets, int32_t* sorted_rows,
                             int32_t* row_pos, int32_t* active, void* ws, hipStream_t s) {
  (void)ws;
  const int R = T * k;
  const size_t lds = (size_t)8 * E + (size_t)4 * E * group_words(E);
  hipLaunchKernelGGL(group_rows_kernel, dim3(1), dim3(kGroupThreads), lds, s, ids, R, E, offsets, sorted_rows,
                     row_pos, active);
  return hipGetLastError();
}

}  // namespace moe
