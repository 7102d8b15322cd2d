// ffn_mfma.hip - expert-major grouped GEMM of the expert FFN on the CDNA4
// scaled MFMA (v_mfma_scale_f32_32x32x64_f8f6f4), for experts whose routed
// rows make the product a dense contraction (more than kRegRows rows).
//
// A operand = the expert's MXFP4 weights exactly as stored (E2M1 codes with
// their own E8M0 scale per 32 values); B operand = the activations split in
// two E4M3 terms, each with an E8M0 scale per 32 values:
//     a = q1 * 2^e1 + q2 * 2^e2,   q1 = rne_e4m3(a / 2^e1), q2 = rne_e4m3((a - q1 2^e1) / 2^e2)
// with e = ceil(log2(amax / 448)) per block and term.  A bf16 value has 8
// significant bits and each E4M3 term carries 4, so for x the two terms are
// exact; for the fp32 h they carry the leading ~8 bits.  D accumulates both
// terms in fp32.
//
// Operand layout of one 32x32x64 step (64 K values; lane-group h = lane / 32
// of the FP4 operand holds K values 32h .. 32h+31 and lane l gives the E8M0
// scale of 32-block l / 32 of its operand):
//   A lane (m, h): weight row m, the 16 bytes (32 E2M1 codes) of block h of
//                  the step, exactly as stored; that block's scale byte.
//   B lane (n, h): token n, 32 E4M3 bytes holding K values 16h .. 16h+15 and
//                  32 + 16h .. 32 + 16h + 15 (the FP8 operand's lane-groups
//                  split K in 16-value halves); the scale byte of K values
//                  32h .. 32h+31.  The quantizer stores the terms with the
//                  middle two 16-value quarters of every 64 values swapped, so
//                  that these 32 bytes are contiguous.
//   D lane l, register r: token l % 32, weight row 8*(r/4) + 4*(l/32) + r%4.
//
// Tiles: 256 weight rows x 128 tokens per block of 4 waves, one block per
// CU (32 tokens per wave, 8 row blocks of 32 each, accumulators in AGPRs).
// For gate/up the 256 rows are gate rows i0..i0+127 followed by the same up
// rows, so SiLU(g)*u is formed in registers.  The A tile of each 256-value K
// stage is staged in LDS (double-buffered, rows padded against bank
// conflicts) and shared by the 4 waves; each wave streams its own B into
// registers one stage ahead.  256 rows per tile halve the B bytes per MFMA
// against 128, which keeps the vector-memory path under the MFMA time.
// A tile's 128 token slots form 4 groups of 32; a tile whose expert rows
// fill only 1 or 2 groups runs with the 4 waves splitting the row blocks
// instead (2 or 4 blocks each, gate blocks kept with their up blocks), so
// MFMA work follows the routed rows rather than the padded tile.  The plan
// orders (expert, token tile) pairs heaviest first and deals them to the 8
// XCDs in turn; each XCD runs its pairs' weight tiles consecutively, so
// tiles sharing a token tile share that XCD's L2.
#include <climits>
#include <type_traits>

#include "moe_internal.h"

namespace {

constexpr int kThreads = 256;
constexpr int kTileRows = 256;    // weight rows per block
constexpr int kTileTok = 128;     // tokens per block
constexpr int kStageK = 256;      // K values per LDS stage
constexpr int kStageBytes = 128;  // FP4 bytes per row per stage

typedef int v8i_t __attribute__((ext_vector_type(8)));
typedef float v16f_t __attribute__((ext_vector_type(16)));

// ------------------------------------------------------------ E4M3 terms --
// Round |a| <= 448 to E4M3 (ties to even); returns the code and the rounded
// value (in the same units as a).
__device__ __forceinline__ uint32_t e4m3_rne(float a, float& qv) {
  const float x = fabsf(a);
  uint32_t code;
  if (x < 0.015625f) {  // below 2^-6: the subnormal grid m * 2^-9 (m = 8 is 2^-6)
    const float m = rintf(x * 512.0f);
    code = (uint32_t)m;
    qv = m * (1.0f / 512.0f);
  } else {
    uint32_t b = __float_as_uint(x);
    b += 0x7FFFFu + ((b >> 20) & 1u);  // keep 3 mantissa bits
    b &= 0xFFF00000u;
    code = (b >> 20) - (120u << 3);    // exponent bias 127 -> 7
    if (code > 0x7Eu) {
      code = 0x7Eu;
      b = 0x43E00000u;  // 448
    }
    qv = __uint_as_float(b);
  }
  if (a < 0.0f) {
    code |= 0x80u;
    qv = -qv;
  }
  return code;
}

// E8M0 exponent e with amax / 2^e <= 448, e = ceil(log2(amax / 448)); 0 for amax = 0
__device__ __forceinline__ int e4m3_block_exp(float amax) {
  if (!(amax > 0.0f)) return 0;
  const uint32_t b = __float_as_uint(amax);
  const int E = (int)((b >> 23) & 0xFF) - 127;
  int e = ((b & 0x7FFFFFu) <= 0x600000u) ? E - 8 : E - 7;  // 448 = 1.75 * 2^8
  return e < -126 ? -126 : (e > 126 ? 126 : e);  // 2^e and 2^-e stay normal floats
}

// Quantizes rows of a [rows][K] matrix (bf16 bits or fp32) into two E4M3
// terms: q[row][2][K] bytes (quarters of each 64 values in the order
// 0,2,1,3), s[row][2][K/256][2][4] scale bytes where the scale of 32-block
// j = 8*stage + 2*step + half sits at [stage][half][step].
// One thread per (row, 32-block).
template <bool BF16_IN>
__device__ __forceinline__ void quantize_block(const void* src, int row, int blk, int K, uint8_t* __restrict__ q,
                                               uint8_t* __restrict__ s) {
  float v[32];
  if (BF16_IN) {
    const uint4* p = (const uint4*)((const uint16_t*)src + (int64_t)row * K + 32 * blk);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint4 w = p[i];
      const uint32_t d[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        v[8 * i + 2 * j] = __uint_as_float(d[j] << 16);
        v[8 * i + 2 * j + 1] = __uint_as_float(d[j] & 0xFFFF0000u);
      }
    }
  } else {
    const float4* p = (const float4*)((const float*)src + (int64_t)row * K + 32 * blk);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float4 w = p[i];
      v[4 * i] = w.x;
      v[4 * i + 1] = w.y;
      v[4 * i + 2] = w.z;
      v[4 * i + 3] = w.w;
    }
  }
  const int sidx = (blk >> 3) * 8 + (blk & 1) * 4 + ((blk >> 1) & 3);
#pragma unroll
  for (int term = 0; term < 2; ++term) {
    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < 32; ++i) amax = fmaxf(amax, fabsf(v[i]));
    const int e = e4m3_block_exp(amax);
    const float inv = __uint_as_float((uint32_t)(127 - e) << 23);  // 2^-e
    const float scl = __uint_as_float((uint32_t)(127 + e) << 23);  // 2^e
    uint32_t packed[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) packed[i] = 0u;
#pragma unroll
    for (int i = 0; i < 32; ++i) {
      float qv;
      const uint32_t c = e4m3_rne(v[i] * inv, qv);
      packed[i >> 2] |= c << (8 * (i & 3));
      v[i] -= qv * scl;  // residual for the next term (exact)
    }
    // quarters 0,1,2,3 of each 64 values are stored in the order 0,2,1,3
    uint8_t* g64 = q + ((int64_t)row * 2 + term) * K + 64 * (blk >> 1);
    *(uint4*)(g64 + 16 * (blk & 1)) = make_uint4(packed[0], packed[1], packed[2], packed[3]);
    *(uint4*)(g64 + 32 + 16 * (blk & 1)) = make_uint4(packed[4], packed[5], packed[6], packed[7]);
    s[((int64_t)row * 2 + term) * (K / 32) + sidx] = (uint8_t)(e + 127);
  }
}

// x [T][H] bf16 -> two E4M3 terms; block 0 also writes the tile plan: one
// (slot, token tile) pair per token tile of every active expert with more
// than kRegRows rows, in active-list order, and the pair count in plan[0].
__global__ __launch_bounds__(kThreads) void mfma_prep_kernel(const uint16_t* __restrict__ x, int T, int H,
                                                            const int32_t* __restrict__ offsets,
                                                            const int32_t* __restrict__ active,
                                                            uint8_t* __restrict__ xq, uint8_t* __restrict__ xs,
                                                            int32_t* __restrict__ plan) {
  if (blockIdx.x == 0) {
    // Tile plan: the (slot, token tile) pairs of experts with more than
    // kRegRows rows, heaviest first: tiles with 4 token groups (65..128
    // rows), then 2 (33..64), then 1 (5..32).  The GEMM deals pair g to XCD
    // g % 8, so every XCD gets a near-equal share of each class and starts
    // with its heaviest tiles.  Within a class pairs keep slot order, so
    // the plan is deterministic.
    __shared__ int s_part[3][kThreads / 64];
    const int na = active[0];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    // pairs of slot a by class: c[0] (4 groups), c[1] (2 groups), c[2] (1 group)
    auto classes = [&](int a, int (&c)[3]) {
      c[0] = c[1] = c[2] = 0;
      if (a >= na) return;
      const int e = active[1 + a];
      const int cnt = offsets[e + 1] - offsets[e];
      if (cnt <= kRegRows) return;
      const int nt = (cnt + kTileTok - 1) / kTileTok;
      const int last = cnt - (nt - 1) * kTileTok;
      c[0] = nt - 1 + (last > 64);
      c[1] = (last > 32 && last <= 64);
      c[2] = (last <= 32);
    };
    // block-wide exclusive scan of three counters; returns the block totals
    auto scan3 = [&](int (&c)[3], int (&before)[3], int (&total)[3]) {
#pragma unroll
      for (int q = 0; q < 3; ++q) {
        int v = c[q];
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
          const int u = __shfl_up(v, o, 64);
          if (lane >= o) v += u;
        }
        if (lane == 63) s_part[q][wave] = v;
        before[q] = v - c[q];
      }
      __syncthreads();
#pragma unroll
      for (int q = 0; q < 3; ++q) {
        total[q] = 0;
        for (int w2 = 0; w2 < kThreads / 64; ++w2) {
          if (w2 < wave) before[q] += s_part[q][w2];
          total[q] += s_part[q][w2];
        }
      }
      __syncthreads();
    };
    // pass 1: class totals
    int tot[3] = {0, 0, 0};
    for (int a0 = 0; a0 < na; a0 += kThreads) {
      int c[3], bf[3], t[3];
      classes(a0 + threadIdx.x, c);
      scan3(c, bf, t);
      for (int q = 0; q < 3; ++q) tot[q] += t[q];
    }
    // pass 2: positions
    int base[3] = {0, tot[0], tot[0] + tot[1]};
    for (int a0 = 0; a0 < na; a0 += kThreads) {
      const int a = a0 + threadIdx.x;
      int c[3], bf[3], t[3];
      classes(a, c);
      scan3(c, bf, t);
      if (c[0] + c[1] + c[2] > 0) {
        const int e = active[1 + a];
        const int cnt = offsets[e + 1] - offsets[e];
        const int nt = (cnt + kTileTok - 1) / kTileTok;
        for (int j = 0; j < nt; ++j) {
          const int r = min(cnt - j * kTileTok, kTileTok);
          const int q = r > 64 ? 0 : r > 32 ? 1 : 2;
          const int g = base[q] + bf[q]++;
          plan[1 + 2 * g] = a;
          plan[2 + 2 * g] = j;
        }
      }
      for (int q = 0; q < 3; ++q) base[q] += t[q];
    }
    if (threadIdx.x == 0) plan[0] = tot[0] + tot[1] + tot[2];
    return;
  }
  const int nblk = H >> 5;
  const int64_t i = (int64_t)(blockIdx.x - 1) * kThreads + threadIdx.x;
  if (i >= (int64_t)T * nblk) return;
  quantize_block<true>(x, (int)(i / nblk), (int)(i % nblk), H, xq, xs);
}

// h [R][I] fp32 -> two E4M3 terms, for every row
__global__ __launch_bounds__(kThreads) void quantize_h_kernel(const float* __restrict__ h, int R, int I,
                                                             uint8_t* __restrict__ hq, uint8_t* __restrict__ hs) {
  const int nblk = I >> 5;
  const int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  if (i >= (int64_t)R * nblk) return;
  quantize_block<false>(h, (int)(i / nblk), (int)(i % nblk), I, hq, hs);
}

// ------------------------------------------------------------------ GEMM --

// 8 scale bytes of a row (natural order j = 2*step + half) -> [half][step]
__device__ __forceinline__ uint2 scales_by_half(uint2 v) {
  // bytes b0..b7 -> (b0, b2, b4, b6), (b1, b3, b5, b7)
  const uint32_t lo = __builtin_amdgcn_perm(v.y, v.x, 0x06040200u);
  const uint32_t hi = __builtin_amdgcn_perm(v.y, v.x, 0x07050301u);
  return make_uint2(lo, hi);
}

// One 64-deep K step of a 32x32 block: FP4 weights (format 4) times the
// two E4M3 activation terms (format 0); OPSEL picks byte OPSEL of each
// packed scale word (the step's block scale).
template <int OPSEL>
__device__ __forceinline__ v16f_t mfma_step(const v8i_t& A, const v8i_t& B0, const v8i_t& B1, v16f_t acc,
                                            uint32_t sa, uint32_t sb0, uint32_t sb1) {
  acc = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(A, B0, acc, 4, 0, OPSEL, sa, OPSEL, sb0);
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(A, B1, acc, 4, 0, OPSEL, sa, OPSEL, sb1);
}

template <bool GATEUP>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(1, 1))) void mfma_ffn_kernel(
    moe_mxfp4_weights w, int k, const int32_t* __restrict__ offsets, const int32_t* __restrict__ sorted_rows,
    const int32_t* __restrict__ active, const int32_t* __restrict__ plan,
    const uint8_t* __restrict__ bq,  // B terms [rows][2][K]
    const uint8_t* __restrict__ bs,  // B scales [rows][2][K/32]
    float* __restrict__ out, int m_tiles) {
  // A stage: kTileRows rows of 128 bytes, rows padded to 144 bytes so that
  // 16 consecutive rows read at the same column fall in distinct LDS banks
  constexpr int kRowPitch = kStageBytes + 16;
  constexpr int kRB = kTileRows / 32;  // 32-row blocks per wave
  static_assert(kTileRows == kThreads, "one scale row per thread");
  __shared__ __attribute__((aligned(16))) uint8_t s_a[2][kTileRows * kRowPitch];
  __shared__ __attribute__((aligned(16))) uint32_t s_sc[2][kTileRows * 2];  // [row][half] words by step

  const int H = w.hidden, I = w.inter;
  const int K = GATEUP ? H : I;               // reduction length
  const int out_cols = GATEUP ? I : H;        // columns of the output rows
  const uint32_t qrow = (uint32_t)K >> 1;     // FP4 bytes per weight row
  const int nsb = K >> 5;                     // scale bytes per weight row

  // tile: XCD x = blockIdx % 8 runs pairs g = x, x + 8, ... of the plan
  // (heaviest first), each as m_tiles consecutive weight tiles
  const int bx = blockIdx.x;
  const int q8 = (bx >> 3) / m_tiles, mt = (bx >> 3) - q8 * m_tiles;
  const int pair = (bx & 7) + 8 * q8;
  if (pair >= plan[0]) return;
  const int slot = plan[1 + 2 * pair], ntile = plan[2 + 2 * pair];
  const int e = active[1 + slot];
  const int p0 = offsets[e], cnt = offsets[e + 1] - p0;
  const int tok0 = ntile * kTileTok;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t eo = (int64_t)e * w.expert_stride;
  // tile rows: gate/up = gate rows row0 .. row0+127 then the same up rows;
  // down = rows row0 .. row0+255
  const int row0 = GATEUP ? mt * (kTileRows / 2) : mt * kTileRows;

  // A staging: thread t copies the 16-byte pieces (row (t/8) + 32 i, piece
  // t%8), i = 0..7, and the 8 scale bytes of row t.  The pieces travel
  // through named registers (no array, so they stay in VGPRs).
  const int64_t rstride = (int64_t)32 * qrow;  // 32 rows
  const uint8_t* a_lo;                         // pieces 0..3
  const uint8_t* a_hi;                         // pieces 4..7
  const uint8_t* s_row;
  if (GATEUP) {
    a_lo = w.gate_q + eo + (int64_t)(row0 + (tid >> 3)) * qrow + 16 * (tid & 7);
    a_hi = w.up_q + eo + (int64_t)(row0 + (tid >> 3)) * qrow + 16 * (tid & 7);
    s_row = tid < kTileRows / 2 ? w.gate_s + eo + (int64_t)(row0 + tid) * nsb
                                : w.up_s + eo + (int64_t)(row0 + tid - kTileRows / 2) * nsb;
  } else {
    a_lo = w.down_q + eo + (int64_t)(row0 + (tid >> 3)) * qrow + 16 * (tid & 7);
    a_hi = a_lo + 4 * rstride;
    s_row = w.down_s + eo + (int64_t)(row0 + tid) * nsb;
  }
  uint4 aq0, aq1, aq2, aq3, aq4, aq5, aq6, aq7;
  uint2 as2;
#define MFMA_LOAD_A(ST)                                                  \
  do {                                                                   \
    const int so_ = (ST) * kStageBytes;                                  \
    aq0 = *(const uint4*)(a_lo + so_);                                   \
    aq1 = *(const uint4*)(a_lo + rstride + so_);                         \
    aq2 = *(const uint4*)(a_lo + 2 * rstride + so_);                     \
    aq3 = *(const uint4*)(a_lo + 3 * rstride + so_);                     \
    aq4 = *(const uint4*)(a_hi + so_);                                   \
    aq5 = *(const uint4*)(a_hi + rstride + so_);                         \
    aq6 = *(const uint4*)(a_hi + 2 * rstride + so_);                     \
    aq7 = *(const uint4*)(a_hi + 3 * rstride + so_);                     \
    as2 = *(const uint2*)(s_row + (ST) * 8);                             \
  } while (0)
#define MFMA_STORE_A(BUF)                                                          \
  do {                                                                             \
    uint8_t* d_ = &s_a[BUF][(tid >> 3) * kRowPitch + 16 * (tid & 7)];              \
    *(uint4*)(d_) = aq0;                                                           \
    *(uint4*)(d_ + 32 * kRowPitch) = aq1;                                          \
    *(uint4*)(d_ + 64 * kRowPitch) = aq2;                                          \
    *(uint4*)(d_ + 96 * kRowPitch) = aq3;                                          \
    *(uint4*)(d_ + 128 * kRowPitch) = aq4;                                         \
    *(uint4*)(d_ + 160 * kRowPitch) = aq5;                                         \
    *(uint4*)(d_ + 192 * kRowPitch) = aq6;                                         \
    *(uint4*)(d_ + 224 * kRowPitch) = aq7;                                         \
    *(uint2*)(&s_sc[BUF][2 * tid]) = scales_by_half(as2);                          \
  } while (0)

  // Token groups of 32 that hold routed rows: 1, 2 or 4 (3 runs as 4).
  // With tg groups, wave w takes token group w % tg and 2*tg of the 8 row
  // blocks: gate/up keeps each gate block with its up block (b and b+4).
  const int rows_in_tile = min(cnt - tok0, kTileTok);
  const int tg = rows_in_tile <= 32 ? 1 : rows_in_tile <= 64 ? 2 : 4;

  auto body = [&](auto rbw_c) {
    constexpr int RBW = decltype(rbw_c)::value;  // row blocks of this wave
    constexpr int TG = RBW / 2;                  // token groups of the tile
    // row block of slot j is rb_base + rel(j); rel(j) is a compile-time
    // offset so LDS addresses fold to immediates (rb_base = 0 with 8 blocks)
    const int rb_base = RBW == kRB ? 0 : (wave / TG) * (RBW / 2);
    auto rel = [](int j) { return j < RBW / 2 ? j : kRB / 2 + (j - RBW / 2); };
    auto rb_of = [&](int j) { return rb_base + rel(j); };

    // this lane's B row (token); rows past the expert's count re-read its last row
    const int n = lane & 31, half = lane >> 5;
    const int tok = tok0 + (wave % TG) * 32 + n;
    const bool tok_ok = tok < cnt;
    const int p = p0 + (tok_ok ? tok : cnt - 1);
    const int64_t brow = GATEUP ? (int64_t)(sorted_rows[p] / k) : (int64_t)p;
    const uint8_t* b0 = bq + (brow * 2 + 0) * K + 32 * half;
    const uint8_t* b1 = bq + (brow * 2 + 1) * K + 32 * half;
    const uint32_t* bs0 = (const uint32_t*)(bs + (brow * 2 + 0) * nsb) + half;
    const uint32_t* bs1 = (const uint32_t*)(bs + (brow * 2 + 1) * nsb) + half;

    // B of one stage in two register sets used in turn: [step][piece]
    // (pieces 0,1 = term 1, pieces 2,3 = term 2) and the two scale words
    uint4 bp[16], bq2[16];
    uint32_t sp0, sp1, sq0, sq1;
    auto load_b = [&](int st, uint4 (&bb)[16], uint32_t& s0, uint32_t& s1) {
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const int koff = st * kStageK + 64 * s;
        bb[4 * s + 0] = *(const uint4*)(b0 + koff);
        bb[4 * s + 1] = *(const uint4*)(b0 + koff + 16);
        bb[4 * s + 2] = *(const uint4*)(b1 + koff);
        bb[4 * s + 3] = *(const uint4*)(b1 + koff + 16);
      }
      s0 = bs0[2 * st];
      s1 = bs1[2 * st];
    };

    v16f_t acc[RBW];
#pragma unroll
    for (int j = 0; j < RBW; ++j)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[j][i] = 0.0f;

    // the MFMAs of one stage: 4 steps x RBW row blocks x 2 terms.  Each A
    // fragment (16 bytes per lane from LDS) feeds two MFMAs (128 cycles),
    // less than the LDS latency under load, so the reads run kAhead
    // fragments ahead of their use in a rotating set of registers.
    constexpr int kAhead = 3;
    constexpr int kFrags = 4 * RBW;  // (step, row block), step-major
    auto compute = [&](int buf, const uint4 (&bb)[16], uint32_t s0, uint32_t s1) {
      const uint8_t* a_base = &s_a[buf][(32 * rb_base + n) * kRowPitch + 16 * half];
      const uint32_t* sc_base = &s_sc[buf][2 * (32 * rb_base + n) + half];
      uint32_t sa[RBW];
#pragma unroll
      for (int j = 0; j < RBW; ++j) sa[j] = sc_base[64 * rel(j)];
      // fragment f = (s, j): row 32 rb_of(j) + n, 16-byte piece 2 s + half
      // (block 2s+half of the stage row)
      auto frag = [&](int f) {
        return *(const uint4*)(a_base + (32 * rel(f % RBW)) * kRowPitch + 32 * (f / RBW));
      };
      uint4 fr[kAhead + 1];
#pragma unroll
      for (int f = 0; f < kAhead; ++f) fr[f] = frag(f);
#pragma unroll
      for (int f = 0; f < kFrags; ++f) {
        if (f + kAhead < kFrags) fr[(f + kAhead) % (kAhead + 1)] = frag(f + kAhead);
        const int s = f / RBW, j = f % RBW;
        v8i_t B0, B1;
        B0[0] = bb[4 * s].x; B0[1] = bb[4 * s].y; B0[2] = bb[4 * s].z; B0[3] = bb[4 * s].w;
        B0[4] = bb[4 * s + 1].x; B0[5] = bb[4 * s + 1].y; B0[6] = bb[4 * s + 1].z; B0[7] = bb[4 * s + 1].w;
        B1[0] = bb[4 * s + 2].x; B1[1] = bb[4 * s + 2].y; B1[2] = bb[4 * s + 2].z; B1[3] = bb[4 * s + 2].w;
        B1[4] = bb[4 * s + 3].x; B1[5] = bb[4 * s + 3].y; B1[6] = bb[4 * s + 3].z; B1[7] = bb[4 * s + 3].w;
        const uint4 wa = fr[f % (kAhead + 1)];
        v8i_t A;
        A[0] = wa.x; A[1] = wa.y; A[2] = wa.z; A[3] = wa.w;
        A[4] = 0; A[5] = 0; A[6] = 0; A[7] = 0;
        if (s == 0) acc[j] = mfma_step<0>(A, B0, B1, acc[j], sa[j], s0, s1);
        else if (s == 1) acc[j] = mfma_step<1>(A, B0, B1, acc[j], sa[j], s0, s1);
        else if (s == 2) acc[j] = mfma_step<2>(A, B0, B1, acc[j], sa[j], s0, s1);
        else acc[j] = mfma_step<3>(A, B0, B1, acc[j], sa[j], s0, s1);
      }
    };

    // Issue order of one stage (masks: 0x100 LDS read, 0x008 MFMA, 0x020
    // global read, 0x200 LDS write): the scale reads and the first kAhead
    // fragments, then two MFMAs, one fragment read and the next share of
    // the next stage's global loads at a time, and the A stores last.
    // Spreading the 27 global loads over the MFMAs keeps the wave from
    // stalling on the address path with its MFMAs queued behind them.
    constexpr int kLoads = 9 + 18;  // A pieces + scales, B pieces + scale words
    constexpr int kSlots = kFrags - kAhead;
    constexpr int kPer = (kLoads + kSlots - 1) / kSlots;
    auto stage_schedule = [&]() {
      __builtin_amdgcn_sched_group_barrier(0x100, (RBW + 1) / 2 + kAhead, 0);
#pragma unroll
      for (int f = 0; f < kSlots; ++f) {
        __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        if (f * kPer < kLoads) __builtin_amdgcn_sched_group_barrier(0x020, kPer, 0);
      }
      __builtin_amdgcn_sched_group_barrier(0x008, 2 * kAhead, 0);
      __builtin_amdgcn_sched_group_barrier(0x200, 9, 0);
    };

    // Pipeline: while the MFMAs of stage st run on LDS buffer st&1 and B
    // register set st&1, the A pieces of stage st+1 (registers, stored to
    // the other buffer after the MFMAs) and its B (the other register set)
    // are in flight.  Both halves of a loop iteration are single basic
    // blocks whose prefetches are used unconditionally (the odd half of the
    // last pair re-loads the last stage), so the stage schedule applies to
    // each.
    const int nst = K / kStageK;
    load_b(0, bp, sp0, sp1);
    MFMA_LOAD_A(0);
    MFMA_STORE_A(0);
    __syncthreads();
    int st = 0;
    for (; st + 1 < nst; st += 2) {
      // even stage: LDS buffer 0, register set bp; stage st+1 -> buffer 1 / bq2
      MFMA_LOAD_A(st + 1);
      load_b(st + 1, bq2, sq0, sq1);
      compute(0, bp, sp0, sp1);
      MFMA_STORE_A(1);
      stage_schedule();
      __syncthreads();
      // odd stage: LDS buffer 1, register set bq2; stage st+2 -> buffer 0 / bp
      const int nx = min(st + 2, nst - 1);
      MFMA_LOAD_A(nx);
      load_b(nx, bp, sp0, sp1);
      compute(1, bq2, sq0, sq1);
      MFMA_STORE_A(0);
      stage_schedule();
      __syncthreads();
    }
    if (st < nst) compute(0, bp, sp0, sp1);  // odd stage count: the last stage

    if (!tok_ok) return;
    float* orow = out + (int64_t)(p0 + tok) * out_cols;
    if (GATEUP) {
      // j < RBW/2: gate block rb_of(j); j + RBW/2: the matching up block
#pragma unroll
      for (int j = 0; j < RBW / 2; ++j)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int m = row0 + 32 * rb_of(j) + 8 * g + 4 * half;
          float4 v;
          v.x = silu_mul(acc[j][4 * g + 0], acc[j + RBW / 2][4 * g + 0]);
          v.y = silu_mul(acc[j][4 * g + 1], acc[j + RBW / 2][4 * g + 1]);
          v.z = silu_mul(acc[j][4 * g + 2], acc[j + RBW / 2][4 * g + 2]);
          v.w = silu_mul(acc[j][4 * g + 3], acc[j + RBW / 2][4 * g + 3]);
          *(float4*)(orow + m) = v;
        }
    } else {
#pragma unroll
      for (int j = 0; j < RBW; ++j) {
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int m = row0 + 32 * rb_of(j) + 8 * g + 4 * half;
          *(float4*)(orow + m) =
              make_float4(acc[j][4 * g + 0], acc[j][4 * g + 1], acc[j][4 * g + 2], acc[j][4 * g + 3]);
        }
      }
    }
  };
  if (tg == 1) body(std::integral_constant<int, 2>());
  else if (tg == 2) body(std::integral_constant<int, 4>());
  else body(std::integral_constant<int, 8>());
#undef MFMA_LOAD_A
#undef MFMA_STORE_A
}

size_t align256(size_t v) { return (v + 255) / 256 * 256; }

}  // namespace

namespace moe {

// K of both products in whole stages, whole row tiles (gate/up: I/128 tiles
// of 128 gate + 128 up rows; down: H/256 tiles)
bool mfma_shape_ok(int H, int I) {
  return H % kStageK == 0 && I % kStageK == 0 && I % (kTileRows / 2) == 0 && H % kTileRows == 0;
}

// Workspace of the MFMA path after the h buffer: x terms, x scales, h terms,
// h scales, tile plan.
size_t mfma_workspace(int T, int k, int E, int H, int I) {
  const size_t R = (size_t)T * k;
  const size_t mx = (size_t)(R < (size_t)E ? R : E);
  const size_t pairs = R / kTileTok + (mx < R / (kRegRows + 1) ? mx : R / (kRegRows + 1)) + 1;
  return align256((size_t)T * 2 * H) + align256((size_t)T * 2 * (H / 32)) + align256(R * 2 * I) +
         align256(R * 2 * (I / 32)) + align256((1 + 2 * pairs) * sizeof(int32_t));
}

size_t mfma_max_pairs(int T, int k, int E) {
  const size_t R = (size_t)T * k;
  const size_t mx = (size_t)(R < (size_t)E ? R : E);
  return R / kTileTok + (mx < R / (kRegRows + 1) ? mx : R / (kRegRows + 1)) + 1;
}

// Launches prep, gate/up GEMM (h for experts with more than kRegRows rows).
hipError_t launch_mfma_gateup(const uint16_t* x, int T, int k, const moe_mxfp4_weights& w, const int32_t* offsets,
                              const int32_t* sorted_rows, const int32_t* active, float* h, uint8_t* ws,
                              hipStream_t s) {
  const int H = w.hidden, I = w.inter;
  const size_t R = (size_t)T * k;
  uint8_t* xq = ws;
  uint8_t* xs = xq + align256((size_t)T * 2 * H);
  uint8_t* hq = xs + align256((size_t)T * 2 * (H / 32));
  uint8_t* hs = hq + align256(R * 2 * I);
  int32_t* plan = (int32_t*)(hs + align256(R * 2 * (I / 32)));
  (void)hq;
  (void)hs;
  const int64_t nq = (int64_t)T * (H / 32);
  hipLaunchKernelGGL(mfma_prep_kernel, dim3(1 + (unsigned)((nq + kThreads - 1) / kThreads)), dim3(kThreads), 0, s,
                     x, T, H, offsets, active, xq, xs, plan);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  const int m_tiles = I / (kTileRows / 2);
  const unsigned grid = (unsigned)(8 * ((mfma_max_pairs(T, k, w.num_experts) + 7) / 8) * m_tiles);
  hipLaunchKernelGGL((mfma_ffn_kernel<true>), dim3(grid), dim3(kThreads), 0, s, w, k, offsets, sorted_rows, active,
                     plan, xq, xs, h, m_tiles);
  return hipGetLastError();
}

// Launches h quantization and the down GEMM (y_rows for the same experts).
hipError_t launch_mfma_down(int T, int k, const moe_mxfp4_weights& w, const int32_t* offsets,
                            const int32_t* sorted_rows, const int32_t* active, const float* h, float* y_rows,
                            uint8_t* ws, hipStream_t s) {
  const int H = w.hidden, I = w.inter;
  const size_t R = (size_t)T * k;
  uint8_t* xq = ws;
  uint8_t* xs = xq + align256((size_t)T * 2 * H);
  uint8_t* hq = xs + align256((size_t)T * 2 * (H / 32));
  uint8_t* hs = hq + align256(R * 2 * I);
  int32_t* plan = (int32_t*)(hs + align256(R * 2 * (I / 32)));
  const int64_t nq = (int64_t)R * (I / 32);
  hipLaunchKernelGGL(quantize_h_kernel, dim3((unsigned)((nq + kThreads - 1) / kThreads)), dim3(kThreads), 0, s, h,
                     (int)R, I, hq, hs);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  const int m_tiles = H / kTileRows;
  const unsigned grid = (unsigned)(8 * ((mfma_max_pairs(T, k, w.num_experts) + 7) / 8) * m_tiles);
  hipLaunchKernelGGL((mfma_ffn_kernel<false>), dim3(grid), dim3(kThreads), 0, s, w, k, offsets, sorted_rows, active,
                     plan, hq, hs, y_rows, m_tiles);
  return hipGetLastError();
}

}  // namespace moe
