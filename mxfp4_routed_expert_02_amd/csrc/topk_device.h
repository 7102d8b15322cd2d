// topk_device.h - the top-k of one token's router logits (a four-wave form
// for the routing kernels, a wide form for the one-token kernel that routes
// inside the expert-FFN launch) and the grouping of its k distinct picks, as
// device functions (gfx950).  Included by HIP sources only, after
// moe_internal.h.
#pragma once

#include <climits>

#include "moe_internal.h"

namespace {

// Order-preserving unsigned key of a logit (0 is below every finite value
// and marks taken or absent slots).
__device__ __forceinline__ uint32_t order_key(float v) {
  uint32_t u = __float_as_uint(v);
  if (u == 0x80000000u) u = 0u;  // -0 ranks equal to +0
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Four-wave top-k: wave w holds the keys of experts [w*Qw, w*Qw + Qw),
// Qw = ceil(E/4) (an even split keeps the waves' thresholds alike, so few
// rounds follow the first ones), lane l those of experts w*Qw + l*C + i.
//   1. Each lane sorts its C experts by (key descending, id ascending).
//   2. Each wave takes picks in rounds; a round only looks at the lane
//      heads: the wave maximum of the head keys, the lowest lane holding it
//      (lanes are in id order, so that is the lowest id among equal keys),
//      and that lane drops its head.  The n non-empty waves first take
//      R = ceil(k/n) picks each; the smallest of their R-th keys, tau, has
//      at least k keys at or above it, so no expert below tau can be among
//      the top k, and each wave then goes on only while its maximum is at
//      least tau (at most k picks in all).
//   3. The global top-k lies among the 4 lists; a candidate's global rank
//      is its place in its own list plus, for every other list, the entries
//      that beat it (a list of a lower wave beats it on an equal key, since
//      all its ids are lower).  Ranks below k are those of the true top k,
//      so each pick lands in its slot without a further selection round.
// Keys of absent experts are 0, below every finite logit, and never picked.
constexpr int kRoute4Threads = 256;
constexpr int kList = MOE_MAX_TOPK;  // LDS stride of one wave's list
constexpr int kRegExperts = 4 * MOE_WAVE * 8;  // widest register top-k (four waves of C = 8; eight of C = 4)

// (key, id) in one word: a larger word is a larger key, then a lower id.
__device__ __forceinline__ uint64_t pick_word(uint32_t key, int id) {
  return ((uint64_t)key << 32) | (uint32_t)~id;
}

// Odd-even transposition sort, descending (C passes of compare-exchange).
template <int C>
__device__ __forceinline__ void sort_desc(uint64_t (&v)[C]) {
#pragma unroll
  for (int p = 0; p < C; ++p)
#pragma unroll
    for (int i = p & 1; i + 1 < C; i += 2) {
      const uint64_t a = v[i], b = v[i + 1];
      const bool sw = b > a;
      v[i] = sw ? b : a;
      v[i + 1] = sw ? a : b;
    }
}

// The lane's sorted experts: keys kh[] and ids ki[], head first.
template <int C>
struct LaneList {
  uint32_t kh[C];
  int32_t ki[C];
};

// One round: the wave maximum of the heads (returned) goes to list slot j
// unless it is below tau, in which case nothing changes.
template <int C>
__device__ __forceinline__ uint32_t wave_round(LaneList<C>& L, int lane, int j, uint32_t tau, uint32_t* list_key,
                                               int32_t* list_id) {
  const uint32_t m = (uint32_t)__builtin_amdgcn_readlane((int)wave_max_u32_last(L.kh[0]), 63);
  if (m < tau) return m;
  const int win = __ffsll((unsigned long long)__ballot(L.kh[0] == m)) - 1;
  const bool w = lane == win;
  if (w) {
    list_key[j] = m;
    list_id[j] = L.ki[0];
  }
  const uint32_t wm = w ? ~0u : 0u;  // mask arithmetic keeps the arrays in registers
#pragma unroll
  for (int i = 0; i + 1 < C; ++i) {
    L.kh[i] ^= (L.kh[i] ^ L.kh[i + 1]) & wm;
    L.ki[i] ^= (L.ki[i] ^ L.ki[i + 1]) & (int32_t)wm;
  }
  L.kh[C - 1] &= ~wm;
  return m;
}

struct TopkLds {
  uint32_t key[4 * kList];  // per-wave lists, 0 past the wave's last pick
  int32_t id[4 * kList];
  uint32_t pick_key[kList];            // global picks in rank order
  alignas(16) int32_t pick_id[kList];  // padded with INT_MAX
  uint32_t bits[(kRegExperts + 32) / 32];  // picked experts (grouping only)
};

// Entries of a 0-padded list above thr (the first 4*KQ entries).
template <int KQ>
__device__ __forceinline__ int count_above(const uint32_t* list, uint32_t thr) {
  const uint4* q = (const uint4*)list;
  uint4 u[KQ];
#pragma unroll
  for (int i = 0; i < KQ; ++i) u[i] = q[i];
  int n = 0;
#pragma unroll
  for (int i = 0; i < KQ; ++i) n += (u[i].x > thr) + (u[i].y > thr) + (u[i].z > thr) + (u[i].w > thr);
  return n;
}

// Candidate (list `wave`, slot `lane`, key ck >= 1)'s rank: its slot plus
// the entries of the other lists that beat it, ">= ck" in a lower wave's
// list and "> ck" in a higher one's.
template <int KQ>
__device__ __forceinline__ int merge_rank(const TopkLds& s, int wave, int lane, uint32_t ck) {
  const int o0 = wave == 0 ? 1 : 0, o1 = wave <= 1 ? 2 : 1, o2 = wave <= 2 ? 3 : 2;
  return lane + count_above<KQ>(s.key + o0 * kList, ck - (o0 < wave ? 1u : 0u)) +
         count_above<KQ>(s.key + o1 * kList, ck - (o1 < wave ? 1u : 0u)) +
         count_above<KQ>(s.key + o2 * kList, ck - (o2 < wave ? 1u : 0u));
}

// Top-k of one token's logits row by the first 4 waves of a block (waves
// past the fourth hold no expert and only meet the barriers).  Every thread
// must call it (it holds three block barriers); on return s.pick_key/pick_id
// [0..k) hold the picks in rank order (pick_id padded with INT_MAX up to
// kList) and, with BITS, s.bits marks the picked experts.
template <int C, bool BITS>
__device__ __forceinline__ void topk_block(const float* __restrict__ row, int E, int k, TopkLds& s) {
  const int Qw = (E + 3) / 4;  // experts per wave (at most 64*C), contiguous ranges
  const int lane = threadIdx.x & (MOE_WAVE - 1);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / MOE_WAVE);  // uniform: wave branches
  const int base = wave * Qw + lane * C;
  // every load unconditional (slots past E re-read the last logit and are
  // masked below), so the lane's C loads are in flight together instead of
  // one round trip each
  float lv[C];
#pragma unroll
  for (int i = 0; i < C; ++i) lv[i] = row[min(base + i, E - 1)];
  uint64_t v[C];
#pragma unroll
  for (int i = 0; i < C; ++i) {
    const int e = base + i;
    v[i] = pick_word(lane * C + i < Qw && e < E ? order_key(lv[i]) : 0u, e);
  }
  if (wave == 0 && lane >= k && lane < kList) s.pick_id[lane] = INT_MAX;
  if (BITS)
    for (int i = threadIdx.x; i < (int)(sizeof(s.bits) / 4); i += kRoute4Threads) s.bits[i] = 0u;
  sort_desc<C>(v);
  LaneList<C> L;
#pragma unroll
  for (int i = 0; i < C; ++i) {
    L.kh[i] = (uint32_t)(v[i] >> 32);
    L.ki[i] = (int32_t)~(uint32_t)v[i];
  }
  const int n_waves = min(4, (E + Qw - 1) / Qw);  // waves holding an expert
  const int R = min(k, (k + n_waves - 1) / n_waves);
  uint32_t* list_key = s.key + wave * kList;
  int32_t* list_id = s.id + wave * kList;
  int j = 0;
  if (wave < n_waves)
    for (; j < R; ++j) wave_round<C>(L, lane, j, 0u, list_key, list_id);
  __syncthreads();
  uint32_t tau = ~0u;
  for (int w = 0; w < n_waves; ++w) tau = min(tau, s.key[w * kList + R - 1]);
  tau = (uint32_t)__builtin_amdgcn_readfirstlane((int)tau);  // uniform: the early stop is a wave branch
  if (wave < n_waves)
    for (; j < k; ++j)
      if (wave_round<C>(L, lane, j, tau, list_key, list_id) < tau) break;
  if (wave < 4 && lane >= j && lane < kList) list_key[lane] = 0u;
  __syncthreads();
  if (wave < 4 && lane < k) {
    const uint32_t ck = list_key[lane];
    if (ck != 0u) {
      const int rank = k <= 16 ? merge_rank<4>(s, wave, lane, ck) : merge_rank<8>(s, wave, lane, ck);
      if (rank < k) {
        const int id = list_id[lane];
        s.pick_key[rank] = ck;
        s.pick_id[rank] = id;
        if (BITS) atomicOr(&s.bits[id >> 5], 1u << (id & 31));
      }
    }
  }
  __syncthreads();
}

// One token's top-k for the one-token kernels, where the selection's
// latency is on every block's critical path.  The first four waves (one per
// SIMD, so no SIMD interleaves two selections) hold the experts, 16-lane row
// r (thread t = 16r + j) experts r + 16j + 256i, i < C, so that from E = 16
// on every row holds one:
//   1. each 16-lane row's largest key; tau, the smallest of the 16 row
//      maxima, has at least 16 keys at or above it (one per row; with fewer
//      than k rows holding an expert, tau = 1 and every expert qualifies),
//      so for k <= 16 every top-k expert is among the keys >= tau;
//   2. each wave compacts its experts with key >= tau (absent experts have
//      key 0 and never qualify) into its own LDS region of (key, ~id)
//      words, by ballots;
//   3. a candidate's rank is the number of candidate words above its own
//      (larger key first, then the lower id): its wave gives it 4 lanes,
//      lane p counting in wave p's region, so ranks 0..k-1 are the top k in
//      order and each pick lands in its slot.
// The picks are those of topk_block bit for bit: the top k under this order
// is unique.  The candidate count is a few times k for spread-out logits and
// at most E (many equal logits); step 3 costs its square in word compares.
// pre() runs in every thread once the logits loads are in flight and before
// the first block barrier (the caller's own staging, overlapping their
// latency); three block barriers in all.
constexpr int kWideThreads = 4 * MOE_WAVE;  // threads holding experts

template <int C>
struct TopkWideLds {
  static constexpr int kRegion = MOE_WAVE * C + 2;  // a wave's candidates, a zero pad and a spare word
  static_assert(kRegion >= 16, "the ranking reads 16 words of every region at once");
  alignas(16) uint32_t rmax[16];  // largest key of each 16-lane row (0: the row holds none)
  alignas(16) uint32_t cnt[4];    // candidates per wave
  alignas(16) uint2 cand[4 * kRegion];  // (~id, key): the word's low and high halves
  uint32_t pick_key[kList];            // picks in rank order
  alignas(16) int32_t pick_id[kList];  // padded with INT_MAX
};

template <int C, class Pre>
__device__ __forceinline__ void topk_block_wide(const float* __restrict__ row, int E, int k, TopkWideLds<C>& s,
                                                Pre pre) {
  constexpr int kRegion = TopkWideLds<C>::kRegion;
  const int tid = threadIdx.x;
  const int lane = tid & (MOE_WAVE - 1);
  const int wave = __builtin_amdgcn_readfirstlane(tid / MOE_WAVE);  // uniform: wave branches
  const bool holder = wave < 4;
  const int eb = 16 * (tid & 15) + (tid >> 4);  // this thread's first expert
  float lv[C];
  if (holder) {
#pragma unroll
    for (int i = 0; i < C; ++i) lv[i] = row[min(eb + kWideThreads * i, E - 1)];
  }
  pre();
  uint64_t v[C];
  if (holder) {
    uint32_t m = 0u;
#pragma unroll
    for (int i = 0; i < C; ++i) {
      const int e = eb + kWideThreads * i;
      v[i] = pick_word(e < E ? order_key(lv[i]) : 0u, e);
      m = max(m, (uint32_t)(v[i] >> 32));
    }
    m = max(m, dpp_u32<0x111>(m));  // row maxima land in each row's last lane
    m = max(m, dpp_u32<0x112>(m));
    m = max(m, dpp_u32<0x114>(m));
    m = max(m, dpp_u32<0x118>(m));
    if ((lane & 15) == 15) s.rmax[4 * wave + (lane >> 4)] = m;
    if (wave == 0 && lane >= k && lane < kList) s.pick_id[lane] = INT_MAX;
  }
  __syncthreads();
  if (holder) {
    uint32_t tau = ~0u;
    int rows = 0;  // rows holding an expert
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const uint4 r4 = ((const uint4*)s.rmax)[q];
      const uint32_t r[4] = {r4.x, r4.y, r4.z, r4.w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        tau = r[i] != 0u ? min(tau, r[i]) : tau;
        rows += r[i] != 0u;
      }
    }
    if (rows < k) tau = 1u;
    int pos = 0, total = 0;  // candidates of the lanes below this one, of the whole wave
#pragma unroll
    for (int i = 0; i < C; ++i) {
      const uint64_t bal = __ballot((uint32_t)(v[i] >> 32) >= tau);
      pos += (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(bal >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)bal, 0u));
      total += __popcll(bal);
    }
    uint2* reg = s.cand + wave * kRegion;
    // the lane's candidates follow those of the lanes below, in i order; a
    // non-candidate goes to the region's spare last word, which nothing reads
#pragma unroll
    for (int i = 0; i < C; ++i) {
      const bool c = (uint32_t)(v[i] >> 32) >= tau;
      reg[c ? pos : kRegion - 1] = make_uint2((uint32_t)v[i], (uint32_t)(v[i] >> 32));
      pos += c;
    }
    if (lane == 0) {
      reg[total] = make_uint2(0u, 0u);  // pads the region's last pair: below every word
      s.cnt[wave] = (uint32_t)total;
    }
  }
  __syncthreads();
  if (holder) {
    const int q = lane >> 2, p = lane & 3;
    const int nc = (int)s.cnt[wave];  // this wave's candidates, sixteen at a time
    const int np = (int)s.cnt[p];     // entries of the region lane p counts in
    const uint2* mine = s.cand + wave * kRegion;
    const uint4* other = (const uint4*)(s.cand + p * kRegion);
    for (int i = q; i - q < nc; i += 16) {  // the same trip count in the whole wave
      const uint2 w2 = mine[min(i, nc)];
      const uint64_t W = (uint64_t)w2.y << 32 | w2.x;
      // the region's first 16 entries in one batch of independent reads (the
      // region holds at least 66 words, so they stay inside it; words past
      // np are not counted), then any further ones pair by pair
      uint4 o8[8];
#pragma unroll
      for (int b = 0; b < 8; ++b) o8[b] = other[b];
      int r = 0;
#pragma unroll
      for (int b = 0; b < 8; ++b) {
        r += (2 * b < np && ((uint64_t)o8[b].y << 32 | o8[b].x) > W) +
             (2 * b + 1 < np && ((uint64_t)o8[b].w << 32 | o8[b].z) > W);
      }
      for (int e = 16; e < np; e += 2) {
        const uint4 o = other[e >> 1];
        r += (((uint64_t)o.y << 32 | o.x) > W) + (((uint64_t)o.w << 32 | o.z) > W);
      }
      r += (int)dpp_u32<0x111>((uint32_t)r);  // quad sums land in each quad's last lane
      r += (int)dpp_u32<0x112>((uint32_t)r);
      if (p == 3 && i < nc && r < k) {
        s.pick_key[r] = w2.y;
        s.pick_id[r] = (int32_t)~w2.x;
      }
    }
  }
  __syncthreads();
}

// Softmax over the k picks in wave 0: lanes j < k get pick j's id and
// weight; exponentials in parallel, the sum in rank order.
template <class Lds>
__device__ __forceinline__ bool topk_softmax(const Lds& s, int k, int lane, int& out_id, float& out_w) {
  float my_val = 0.0f;
  int my_id = 0;
  if (lane < k) {
    const uint32_t mk = s.pick_key[lane];
    my_id = s.pick_id[lane];
    my_val = __uint_as_float((mk & 0x80000000u) ? (mk & 0x7FFFFFFFu) : ~mk);  // key -> value
  }
  const float mx = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(my_val), 0));
  const float ex = lane < k ? expf(my_val - mx) : 0.0f;
  float S = 0.0f;
  for (int j = 0; j < k; ++j) S += __int_as_float(__builtin_amdgcn_readlane(__float_as_int(ex), j));
  out_id = my_id;
  out_w = ex / S;
  return lane < k;
}

// Number of the picks below e, from the padded pick ids held in registers.
template <int KQ>
__device__ __forceinline__ int picks_below(const int4 (&p)[KQ], int e) {
  int n = 0;
#pragma unroll
  for (int i = 0; i < KQ; ++i) n += (p[i].x < e) + (p[i].y < e) + (p[i].z < e) + (p[i].w < e);
  return n;
}

// Grouping of one token's k distinct picks by waves 1..3: expert e's offset
// is the number of picks below e (a count for the first of every 4 experts,
// then the pick bitmap), and pick j's place in expert-major order is the
// number of picks below its id.
template <int KQ>
__device__ __forceinline__ void group_one(const TopkLds& s, int E, int k, int32_t* __restrict__ offsets,
                                          int32_t* __restrict__ sorted_rows, int32_t* __restrict__ row_pos,
                                          int32_t* __restrict__ active) {
  int4 p[KQ];
  const int4* q = (const int4*)s.pick_id;
#pragma unroll
  for (int i = 0; i < KQ; ++i) p[i] = q[i];
  const int t = threadIdx.x - MOE_WAVE;  // 0 .. 3*64-1
  for (int e0 = 4 * t; e0 <= E; e0 += 4 * (kRoute4Threads - MOE_WAVE)) {
    const int r0 = picks_below<KQ>(p, e0);
    const uint32_t b = s.bits[e0 >> 5] >> (e0 & 31);  // e0 % 4 == 0: its 4 bits share a word
#pragma unroll
    for (int i = 0; i < 4; ++i)
      if (e0 + i <= E) offsets[e0 + i] = r0 + __popc(b & ((1u << i) - 1u));
  }
  if (t < k) {
    const int pid = s.pick_id[t];
    const int r = picks_below<KQ>(p, pid);
    sorted_rows[r] = t;
    row_pos[t] = r;
    active[1 + r] = pid;
  }
  if (t == 0) active[0] = k;
}

}  // namespace
