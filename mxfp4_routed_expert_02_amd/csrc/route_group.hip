// route_group.hip - router top-k and expert-major row grouping (gfx950).
//
// Top-k: one wavefront per token; each of the k rounds is a wavefront
// arg-max over the experts not yet taken (larger value wins, equal values go
// to the lower id), so the ids come out in rank order.  Up to 2048 experts
// the logits stay in registers (ordered keys, wave max + ballot); beyond
// that they sit in LDS.  The softmax over the k picked logits runs in one
// lane in rank order.
//
// Grouping: a stable counting sort of the flat rows r = t*k + j by expert.
// Counts and OR-ed bitmaps are the only LDS atomics (both order-free), so
// the permutation does not depend on scheduling.  Within a chunk of rows a
// row's rank among the rows of its expert is the popcount of that expert's
// bitmap below the row.
#include <climits>

#include "moe_internal.h"
#include "topk_device.h"

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

template <int C>
__global__ __launch_bounds__(kRoute4Threads) void route_topk_4w_kernel(const float* __restrict__ logits, int E,
                                                                      int k, int32_t* __restrict__ ids,
                                                                      float* __restrict__ weights) {
  __shared__ TopkLds s;
  const int t = blockIdx.x;
  topk_block<C, false>(logits + (int64_t)t * E, E, k, s);
  if (threadIdx.x >= MOE_WAVE) return;
  int id;
  float wv;
  if (topk_softmax(s, k, threadIdx.x, id, wv)) {
    ids[(int64_t)t * k + threadIdx.x] = id;
    weights[(int64_t)t * k + threadIdx.x] = wv;
  }
}

// One token: the top-k as above, then its grouping in the same block.  The
// outputs equal group_rows_small_kernel's on the same ids.
template <int C>
__global__ __launch_bounds__(kRoute4Threads) void route_group_one_kernel(const float* __restrict__ logits, int E,
                                                                        int k, int32_t* __restrict__ ids,
                                                                        float* __restrict__ weights,
                                                                        int32_t* __restrict__ offsets,
                                                                        int32_t* __restrict__ sorted_rows,
                                                                        int32_t* __restrict__ row_pos,
                                                                        int32_t* __restrict__ active) {
  __shared__ TopkLds s;
  topk_block<C, true>(logits, E, k, s);
  if (threadIdx.x < MOE_WAVE) {
    int id;
    float wv;
    if (topk_softmax(s, k, threadIdx.x, id, wv)) {
      ids[threadIdx.x] = id;
      weights[threadIdx.x] = wv;
    }
  } else if (k <= 16) {
    group_one<4>(s, E, k, offsets, sorted_rows, row_pos, active);
  } else {
    group_one<8>(s, E, k, offsets, sorted_rows, row_pos, active);
  }
}

// ------------------------------------------------------------------ group --
// In-place exclusive scan of a[0..n) in LDS by the whole block (NT threads,
// s_wave holding NT/64 + 1 ints); returns the total.
template <int NT>
__device__ int block_exclusive_scan(int* a, int n, int* s_wave) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int per = (n + NT - 1) / NT;
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
    for (int w = 0; w < NT / 64; ++w) {
      const int c = s_wave[w];
      s_wave[w] = acc;
      acc += c;
    }
    s_wave[NT / 64] = acc;
  }
  __syncthreads();
  int run = s_wave[wave] + v - local;
  for (int i = beg; i < end; ++i) {
    const int c = a[i];
    a[i] = run;
    run += c;
  }
  const int total = s_wave[NT / 64];
  __syncthreads();
  return total;
}

// Grouping for many rows: three kernels over chunks of kChunkRows rows.
//   count:   per chunk, each expert's row count and each row's rank among
//            the chunk's earlier rows of the same expert (many blocks)
//   scan:    per expert, the chunks' counts become exclusive positions
//            within the expert, and the expert's total is written (many
//            blocks: 32 lanes per expert, each over a run of chunks, the
//            runs joined by a scan across the 32 lanes)
//   scatter: every block scans the E totals into expert offsets in LDS;
//            block 0 also writes expert_offsets and the active list; each
//            row goes to expert offset + chunk position + rank (many blocks)
// Positions follow (chunk, rank in chunk) = ascending row index within each
// expert, the same stable order as a counting sort.  Workspace: cnt
// [chunks][E], rank [R], then the totals [E] (int32).
constexpr int kChunkRows = 256;

__global__ __launch_bounds__(kChunkRows) void group_count_kernel(const int32_t* __restrict__ ids, int R, int E,
                                                                int32_t* __restrict__ cnt,
                                                                int32_t* __restrict__ rank) {
  extern __shared__ int s_cnt[];  // [E]
  __shared__ int s_ids[kChunkRows];
  const int c = blockIdx.x, tid = threadIdx.x, r = c * kChunkRows + tid;
  for (int e = tid; e < E; e += kChunkRows) s_cnt[e] = 0;
  const int e = r < R ? ids[r] : -1;
  s_ids[tid] = e;
  __syncthreads();
  // ids outside [0, E) break the documented precondition; they are skipped so
  // that no LDS access leaves the array
  if ((unsigned)e < (unsigned)E) {
    atomicAdd(&s_cnt[e], 1);
    int k = 0;
    for (int j = 0; j < tid; ++j) k += s_ids[j] == e;
    rank[r] = k;
  }
  __syncthreads();
  for (int x = tid; x < E; x += kChunkRows) cnt[(int64_t)c * E + x] = s_cnt[x];
}

constexpr int kScanExperts = 8;  // experts per scan block (2 per wave of 64 lanes)
__global__ __launch_bounds__(kChunkRows) void group_scan_kernel(int nch, int E, int32_t* __restrict__ cnt,
                                                                int32_t* __restrict__ tot) {
  static_assert(kChunkRows == 32 * kScanExperts, "32 lanes per expert");
  const int e = blockIdx.x * kScanExperts + (threadIdx.x >> 5), cl = threadIdx.x & 31;
  const int per = (nch + 31) / 32;
  const int c0 = min(nch, cl * per), c1 = min(nch, c0 + per);
  int local = 0;
  if (e < E) {
    // all of this lane's counts are loaded before any is rewritten
    for (int c = c0; c < c1; c += 8) {
      int v[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) v[i] = c + i < c1 ? cnt[(int64_t)(c + i) * E + e] : 0;
#pragma unroll
      for (int i = 0; i < 8; ++i) local += v[i];
    }
  }
  // inclusive scan across the expert's 32 lanes (chunk runs in order)
  int incl = local;
#pragma unroll
  for (int o = 1; o < 32; o <<= 1) {
    const int u = __shfl_up(incl, o, 32);
    if (cl >= o) incl += u;
  }
  if (e >= E) return;
  int run = incl - local;
  for (int c = c0; c < c1; ++c) {
    const int v = cnt[(int64_t)c * E + e];
    cnt[(int64_t)c * E + e] = run;
    run += v;
  }
  if (cl == 31) tot[e] = incl;
}

__global__ __launch_bounds__(kChunkRows) void group_scatter_kernel(const int32_t* __restrict__ ids, int R, int E,
                                                                  const int32_t* __restrict__ tot,
                                                                  const int32_t* __restrict__ cnt,
                                                                  const int32_t* __restrict__ rank,
                                                                  int32_t* __restrict__ offsets,
                                                                  int32_t* __restrict__ active,
                                                                  int32_t* __restrict__ sorted_rows,
                                                                  int32_t* __restrict__ row_pos) {
  extern __shared__ int s_off[];  // [E] offsets, then [E] active flags (block 0)
  __shared__ int s_wave[kChunkRows / 64 + 1];
  const int tid = threadIdx.x;
  for (int x = tid; x < E; x += kChunkRows) s_off[x] = tot[x];
  __syncthreads();
  const int total = block_exclusive_scan<kChunkRows>(s_off, E, s_wave);
  if (blockIdx.x == 0) {
    int* s_flag = s_off + E;
    for (int x = tid; x < E; x += kChunkRows) {
      offsets[x] = s_off[x];
      const int next = x + 1 < E ? s_off[x + 1] : total;
      s_flag[x] = next > s_off[x] ? 1 : 0;
    }
    if (tid == 0) offsets[E] = total;
    __syncthreads();
    // the flags' scan gives each active expert its place in the list
    const int per = (E + kChunkRows - 1) / kChunkRows;
    const int beg = min(E, tid * per), end = min(E, beg + per);
    int mine[MOE_MAX_EXPERTS / kChunkRows];
    for (int i = beg; i < end; ++i) mine[i - beg] = s_flag[i];
    __syncthreads();
    const int na = block_exclusive_scan<kChunkRows>(s_flag, E, s_wave);
    for (int i = beg; i < end; ++i)
      if (mine[i - beg]) active[1 + s_flag[i]] = i;
    if (tid == 0) active[0] = na;
  }
  const int c = blockIdx.x, r = c * kChunkRows + tid;
  if (r >= R) return;
  const int e = ids[r];
  if ((unsigned)e >= (unsigned)E) return;
  const int pos = s_off[e] + cnt[(int64_t)c * E + e] + rank[r];
  sorted_rows[pos] = r;
  row_pos[r] = pos;
}

// Grouping for few rows (R <= kSmallRows): one block; counts by LDS
// histogram, one scan of (flag << 32 | count) pairs, and each row's rank
// among the earlier rows of its expert by direct comparison.
constexpr int kSmallRows = 512;
constexpr int kSmallThreads = 512;

__global__ __launch_bounds__(kSmallThreads) void group_rows_small_kernel(const int32_t* __restrict__ ids, int R,
                                                                         int E, int32_t* __restrict__ offsets,
                                                                         int32_t* __restrict__ sorted_rows,
                                                                         int32_t* __restrict__ row_pos,
                                                                         int32_t* __restrict__ active) {
  extern __shared__ uint64_t s_pair[];  // [E] (flag << 32) | count, then their exclusive scan
  __shared__ int s_ids[kSmallRows];
  __shared__ uint64_t s_wave[kSmallThreads / 64 + 1];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  for (int e = tid; e < E; e += kSmallThreads) s_pair[e] = 0ull;
  int my = -1;
  if (tid < R) {
    my = ids[tid];
    s_ids[tid] = my;
  }
  __syncthreads();
  if ((unsigned)my < (unsigned)E) atomicAdd((unsigned long long*)&s_pair[my], 1ull);
  __syncthreads();
  const int per = (E + kSmallThreads - 1) / kSmallThreads;
  const int beg = min(E, tid * per), end = min(E, beg + per);
  uint64_t local = 0;
  for (int i = beg; i < end; ++i) {
    const uint64_t c = s_pair[i];
    local += (c ? (1ull << 32) : 0ull) + c;
  }
  uint64_t v = local;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const uint64_t u = __shfl_up(v, o, 64);
    if (lane >= o) v += u;
  }
  if (lane == 63) s_wave[wave] = v;
  __syncthreads();
  if (tid == 0) {
    uint64_t acc = 0;
    for (int w = 0; w < kSmallThreads / 64; ++w) {
      const uint64_t c = s_wave[w];
      s_wave[w] = acc;
      acc += c;
    }
    s_wave[kSmallThreads / 64] = acc;
  }
  __syncthreads();
  uint64_t run = s_wave[wave] + v - local;
  for (int i = beg; i < end; ++i) {
    const uint64_t c = s_pair[i];
    offsets[i] = (int32_t)(run & 0xFFFFFFFFull);
    if (c) active[1 + (int)(run >> 32)] = i;
    s_pair[i] = run;
    run += (c ? (1ull << 32) : 0ull) + c;
  }
  if (tid == 0) {
    const uint64_t tot = s_wave[kSmallThreads / 64];
    offsets[E] = (int32_t)(tot & 0xFFFFFFFFull);
    active[0] = (int32_t)(tot >> 32);
  }
  __syncthreads();
  if ((unsigned)my < (unsigned)E) {
    int rank = 0;
    for (int r = 0; r < tid; ++r) rank += (s_ids[r] == my);
    const int pos = (int)(s_pair[my] & 0xFFFFFFFFull) + rank;
    sorted_rows[pos] = tid;
    row_pos[tid] = pos;
  }
}

}  // namespace

namespace moe {

hipError_t launch_route_topk(const float* logits, int T, int E, int k, int32_t* ids, float* w, hipStream_t s) {
  if (T == 0) return hipSuccess;
  const dim3 g(T), b(kRouteThreads), b4(kRoute4Threads);
  if (E <= 4 * 64 * 1)
    hipLaunchKernelGGL(route_topk_4w_kernel<1>, g, b4, 0, s, logits, E, k, ids, w);
  else if (E <= 4 * 64 * 2)
    hipLaunchKernelGGL(route_topk_4w_kernel<2>, g, b4, 0, s, logits, E, k, ids, w);
  else if (E <= 4 * 64 * 4)
    hipLaunchKernelGGL(route_topk_4w_kernel<4>, g, b4, 0, s, logits, E, k, ids, w);
  else if (E <= 4 * 64 * 8)
    hipLaunchKernelGGL(route_topk_4w_kernel<8>, g, b4, 0, s, logits, E, k, ids, w);
  else {
    const size_t lds = (size_t)E * sizeof(float) + (size_t)((E + 31) / 32) * sizeof(uint32_t);
    hipLaunchKernelGGL(route_topk_kernel, g, b, lds, s, logits, E, k, ids, w);
  }
  return hipGetLastError();
}

// One token's top-k and grouping in one launch (E <= 2048; the caller falls
// back to the two launches above that).
hipError_t launch_route_group_one(const float* logits, int E, int k, int32_t* ids, float* w, int32_t* offsets,
                                  int32_t* sorted_rows, int32_t* row_pos, int32_t* active, hipStream_t s) {
  const dim3 g(1), b4(kRoute4Threads);
  if (E <= 4 * 64 * 1)
    hipLaunchKernelGGL(route_group_one_kernel<1>, g, b4, 0, s, logits, E, k, ids, w, offsets, sorted_rows, row_pos,
                       active);
  else if (E <= 4 * 64 * 2)
    hipLaunchKernelGGL(route_group_one_kernel<2>, g, b4, 0, s, logits, E, k, ids, w, offsets, sorted_rows, row_pos,
                       active);
  else if (E <= 4 * 64 * 4)
    hipLaunchKernelGGL(route_group_one_kernel<4>, g, b4, 0, s, logits, E, k, ids, w, offsets, sorted_rows, row_pos,
                       active);
  else
    hipLaunchKernelGGL(route_group_one_kernel<8>, g, b4, 0, s, logits, E, k, ids, w, offsets, sorted_rows, row_pos,
                       active);
  return hipGetLastError();
}

size_t group_rows_workspace(int T, int k, int E) {
  const size_t R = (size_t)T * k;
  if (R <= (size_t)kSmallRows) return 0;
  const size_t nch = (R + kChunkRows - 1) / kChunkRows;
  return (nch * (size_t)E + R + (size_t)E) * sizeof(int32_t);
}

hipError_t launch_group_rows(const int32_t* ids, int T, int k, int E, int32_t* offsets, int32_t* sorted_rows,
                             int32_t* row_pos, int32_t* active, void* ws, hipStream_t s) {
  const int R = T * k;
  if (R <= kSmallRows) {
    hipLaunchKernelGGL(group_rows_small_kernel, dim3(1), dim3(kSmallThreads), (size_t)8 * E, s, ids, R, E, offsets,
                       sorted_rows, row_pos, active);
    return hipGetLastError();
  }
  const int nch = (R + kChunkRows - 1) / kChunkRows;
  int32_t* cnt = (int32_t*)ws;
  int32_t* rank = cnt + (size_t)nch * E;
  int32_t* tot = rank + R;
  hipLaunchKernelGGL(group_count_kernel, dim3(nch), dim3(kChunkRows), (size_t)4 * E, s, ids, R, E, cnt, rank);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  hipLaunchKernelGGL(group_scan_kernel, dim3((E + kScanExperts - 1) / kScanExperts), dim3(kChunkRows), 0, s, nch, E,
                     cnt, tot);
  if ((err = hipGetLastError()) != hipSuccess) return err;
  hipLaunchKernelGGL(group_scatter_kernel, dim3(nch), dim3(kChunkRows), (size_t)8 * E, s, ids, R, E, tot, cnt, rank,
                     offsets, active, sorted_rows, row_pos);
  return hipGetLastError();
}

}  // namespace moe
