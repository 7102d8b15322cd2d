// ffn_mfma.hip - expert-major grouped GEMM of the expert FFN on the CDNA4
// scaled MFMA (v_mfma_scale_f32_32x32x64_f8f6f4), for experts whose routed
// rows make the product a dense contraction (more than reg_rows_max(T) rows).
//
// A operand = the expert's MXFP4 weights exactly as stored (E2M1 codes with
// their own E8M0 scale per 32 values); B operand = the activations split in
// two terms, each with an E8M0 scale per 32 values:
//     a = q1 * 2^e1 + q2 * 2^e2,   q1 = rne(a / 2^e1), q2 = rne((a - q1 2^e1) / 2^e2)
// gate/up: x in two E2M3 (FP6) terms, e = ceil(log2(amax / 7.5)) per block
// and term, so the MFMA runs at the FP4/FP6 rate; the two terms carry the
// leading ~8 bits of each value (not always all of a bf16 x).  down: the
// fp32 h in two E4M3 terms, e = ceil(log2(amax / 448)), the leading ~8 bits.
// D accumulates both terms in fp32.
//
// Operand layout of one 32x32x64 step (64 K values; lane-group h = lane / 32
// of the FP4 operand holds K values 32h .. 32h+31 and lane l gives the E8M0
// scale of 32-block l / 32 of its operand):
//   A lane (m, h): weight row m, the 16 bytes (32 E2M1 codes) of block h of
//                  the step, exactly as stored; that block's scale byte.
//   B lane (n, h), down (E4M3): token n, 32 bytes holding K values
//                  16h .. 16h+15 and 32 + 16h .. 32 + 16h + 15 (the FP8
//                  operand's lane-groups split K in 16-value halves); the
//                  scale byte of K values 32h .. 32h+31.  The quantizer stores
//                  the terms with the middle two 16-value quarters of every 64
//                  values swapped, so that these 32 bytes are contiguous.
//   B lane (n, h), gate/up (E2M3): token n, 24 bytes holding K values
//                  32h .. 32h+31 as 6-bit codes packed densely (value i in
//                  bits 6i .. 6i+5); the scale byte of those 32 values.  A
//                  term's 128 values of a stage form one 128-byte record per
//                  token: per 64-value step s, bytes 48s + 16h hold half h's
//                  first 16 bytes and bytes 48s + 32 + 8h its last 8; the
//                  scale bytes sit at 96 + 4h + 2s.
//   D lane l, register r: token l % 32, weight row 8*(r/4) + 4*(l/32) + r%4.
//
// Tiles: 256 weight rows x 128 tokens per block of 4 waves, one block per
// CU (32 tokens per wave, 8 row blocks of 32 each, accumulators in AGPRs).
// For gate/up the 256 rows are gate rows i0..i0+127 followed by the same up
// rows, so SiLU(g)*u is formed in registers.  Every operand of a K stage
// (weight codes and scales, activation terms and scales) travels from
// global memory into an LDS ring slot by LDS DMA loads, with no trip
// through registers; the ring keeps two or three stages in flight per CU
// while one is read, so tiles with few tokens stream their weights at
// memory speed and full tiles keep the MFMA pipe fed.  The waits on those
// loads are explicit counts of each wave's own loads, which complete in
// issue order.
// A tile's 128 token slots form 4 groups of 32; a tile whose expert rows
// fill only 1 or 2 groups runs with the 4 waves splitting the row blocks
// instead (2 or 4 blocks each, gate blocks kept with their up blocks) and a
// ring shaped for them (two groups: a deeper ring of smaller 128-value
// stages; one group: 256-value stages whose weight loads take whole cache
// lines), so MFMA work follows the routed rows rather than the padded tile.
// The plan orders (expert, token tile) pairs heaviest first, an expert's
// full token tiles next to each other, and deals them to the 8 XCDs in runs
// of four; each XCD steps through the weight tiles of its run with all four
// token tiles at each, so the token tiles of one expert read each weight
// tile into that XCD's L2 together.
#include <climits>
#include <type_traits>

#include "moe_internal.h"

namespace {

constexpr int kThreads = 256;
constexpr int kTileRows = 256;    // weight rows per block
constexpr int kTileTok = 128;     // tokens per block
constexpr int kStageK = 128;      // K values per LDS stage
constexpr int kBand = 4;          // consecutive plan pairs per XCD

typedef int v8i_t __attribute__((ext_vector_type(8)));
typedef float v16f_t __attribute__((ext_vector_type(16)));
typedef float v32f_t __attribute__((ext_vector_type(32)));
typedef unsigned v6u_t __attribute__((ext_vector_type(6)));

// ------------------------------------------------------------ E4M3 terms --
// Rounding to E4M3 (the OCP format: bias 7, largest finite 448, subnormals
// m * 2^-9) is the hardware conversion v_cvt_pk_fp8_f32, round to nearest
// even in the default mode, and v_cvt_f32_fp8 gives the rounded value back
// exactly.  Every input here has |a| <= 448 by the choice of the block
// exponent, so no saturation or NaN case arises.

// E8M0 exponent e with amax / 2^e <= 448, e = ceil(log2(amax / 448)); 0 for amax = 0
__device__ __forceinline__ int e4m3_block_exp(float amax) {
  if (!(amax > 0.0f)) return 0;
  const uint32_t b = __float_as_uint(amax);
  const int E = (int)((b >> 23) & 0xFF) - 127;
  int e = ((b & 0x7FFFFFu) <= 0x600000u) ? E - 8 : E - 7;  // 448 = 1.75 * 2^8
  return e < -126 ? -126 : (e > 126 ? 126 : e);  // 2^e and 2^-e stay normal floats
}

// E8M0 exponent e with amax / 2^e <= 7.5, e = ceil(log2(amax / 7.5)); 0 for amax = 0
__device__ __forceinline__ int e2m3_block_exp(float amax) {
  if (!(amax > 0.0f)) return 0;
  const uint32_t b = __float_as_uint(amax);
  const int E = (int)((b >> 23) & 0xFF) - 127;
  int e = ((b & 0x7FFFFFu) <= 0x700000u) ? E - 2 : E - 1;  // 7.5 = 1.875 * 2^2
  return e < -126 ? -126 : (e > 126 ? 126 : e);  // 2^e and 2^-e stay normal floats
}

// Quantizes rows of a [rows][K] bf16 matrix into two E2M3 (FP6) terms,
//     a = q1 * 2^e1 + q2 * 2^e2,  q1 = rne_e2m3(a / 2^e1),  q2 = rne_e2m3((a - q1 2^e1) / 2^e2),
// e = ceil(log2(amax / 7.5)) per 32-value block and term.  Stored stage-major
// as records of 128 bytes per (128-value K stage, row, term):
//   bytes 48 s .. 48 s + 47 (MFMA step s = 0, 1 of the stage): the 16 low
//     bytes of block 2s, the 16 low bytes of block 2s+1, the 8 high bytes of
//     block 2s, the 8 high bytes of block 2s+1 (a block = 32 codes packed 6
//     bits each, code i at bits 6i .. 6i+5 of its 24 bytes)
//   bytes 96 + 4h + 2s: the E8M0 scale of block 2s + h
// so that MFMA lane-half h reads 16 + 8 aligned bytes and one scale word
// whose bytes 0 and 2 serve steps 0 and 1.  One thread per (row, 32-block).
__device__ __forceinline__ void quantize_block_fp6(const uint16_t* __restrict__ src, int row, int rows, int blk,
                                                   int K, uint8_t* __restrict__ q) {
  float v[32];
  const uint4* p = (const uint4*)(src + (int64_t)row * K + 32 * blk);
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
  const int st = blk >> 2, s = (blk >> 1) & 1, h = blk & 1;
  uint8_t* rec = q + ((int64_t)st * rows + row) * 256;
#pragma unroll
  for (int term = 0; term < 2; ++term) {
    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < 32; ++i) amax = fmaxf(amax, fabsf(v[i]));
    const int e = e2m3_block_exp(amax);
    const float scl = __uint_as_float((uint32_t)(127 + e) << 23);  // 2^e
    // v_cvt_scalef32_2xpk16_fp6_f32 rounds a[j] / 2^e and b[j] / 2^e to E2M3
    // (nearest, ties to even) into codes 2j and 2j+1, 6 bits each, code i at
    // bits 6i .. 6i+5; v_cvt_scalef32_pk32_f32_fp6 gives the 32 rounded
    // values times 2^e back.  (Checked against a software rounding over every
    // E2M3 value, the midpoints between neighbours and points just off them at
    // several scales, 20,000 random blocks and 2,000 blocks of fp32
    // subnormals: equal codes and values, but for the sign of a zero code
    // from an input of -0.)
    v16f_t a, b;
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      a[j] = v[2 * j];
      b[j] = v[2 * j + 1];
    }
    const v6u_t pk = __builtin_amdgcn_cvt_scalef32_2xpk16_fp6_f32(a, b, scl);
    const v32f_t qv = __builtin_amdgcn_cvt_scalef32_pk32_f32_fp6(pk, scl);
#pragma unroll
    for (int i = 0; i < 32; ++i) v[i] -= qv[i];  // residual for the next term (exact)
    uint8_t* r = rec + term * 128;
    *(uint4*)(r + 48 * s + 16 * h) = make_uint4(pk[0], pk[1], pk[2], pk[3]);
    *(uint2*)(r + 48 * s + 32 + 8 * h) = make_uint2(pk[4], pk[5]);
    r[96 + 4 * h + 2 * s] = (uint8_t)(e + 127);
  }
}

// Two E4M3 terms of one 32-value block v (row `row` of `rows`, block blk
// along K), a = q1 * 2^e1 + q2 * 2^e2 with e = ceil(log2(amax / 448)) per
// term, stored stage-major so that one 128-value K stage of every row is one
// contiguous block (whatever rows a GEMM tile gathers, its loads of a stage
// stay within a few pages):
//   q[K/128][rows][2][128]  bytes (quarters of each 64 values in the order
//                           0,2,1,3)
//   s[K/128][rows][2][4]    E8M0 scale bytes of the stage's four 32-blocks
__device__ __forceinline__ void e4m3_two_terms(float (&v)[32], int row, int rows, int blk, uint8_t* __restrict__ q,
                                               uint8_t* __restrict__ s) {
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
    for (int i = 0; i < 8; ++i) {
      // codes of values 4i .. 4i+3 in bytes 0 .. 3
      int w = __builtin_amdgcn_cvt_pk_fp8_f32(v[4 * i] * inv, v[4 * i + 1] * inv, 0, false);
      w = __builtin_amdgcn_cvt_pk_fp8_f32(v[4 * i + 2] * inv, v[4 * i + 3] * inv, w, true);
      packed[i] = (uint32_t)w;
      // residual for the next term (exact)
      v[4 * i] -= __builtin_amdgcn_cvt_f32_fp8(w, 0) * scl;
      v[4 * i + 1] -= __builtin_amdgcn_cvt_f32_fp8(w, 1) * scl;
      v[4 * i + 2] -= __builtin_amdgcn_cvt_f32_fp8(w, 2) * scl;
      v[4 * i + 3] -= __builtin_amdgcn_cvt_f32_fp8(w, 3) * scl;
    }
    const int64_t st = blk >> 2;
    uint8_t* g64 = q + (st * rows + row) * 256 + term * 128 + 64 * ((blk >> 1) & 1);
    *(uint4*)(g64 + 16 * (blk & 1)) = make_uint4(packed[0], packed[1], packed[2], packed[3]);
    *(uint4*)(g64 + 32 + 16 * (blk & 1)) = make_uint4(packed[4], packed[5], packed[6], packed[7]);
    s[(st * rows + row) * 8 + term * 4 + (blk & 3)] = (uint8_t)(e + 127);
  }
}

// x [T][H] bf16 -> two E2M3 terms (blocks 2 ..).  Block 0 writes the tile
// plan: the pair count in plan[0], and from int4 1 on one record per token tile of
// every active expert with more than reg_max rows: (expert, its first
// sorted row, its row count, the tile's first token), so a GEMM block finds
// its work with one load after the count.  Block 1 writes the register
// GEMVs' class lists l1 / l4, so they need no launch of their own.
__global__ __launch_bounds__(kThreads) void mfma_prep_kernel(const uint16_t* __restrict__ x, int T, int H,
                                                            const int32_t* __restrict__ offsets,
                                                            const int32_t* __restrict__ active,
                                                            uint8_t* __restrict__ xq, int32_t* __restrict__ plan,
                                                            int reg_max, int32_t* __restrict__ l1,
                                                            int32_t* __restrict__ l4, int lo4) {
  if (blockIdx.x == 1) {  // the register GEMVs' class lists, beside the plan
    __shared__ int s_lists[2 * kThreads / MOE_WAVE];
    build_small_lists<kThreads>(offsets, active, l1, l4, lo4, reg_max, s_lists);
    return;
  }
  if (blockIdx.x == 0) {
    // Tile plan: the (expert, token tile) pairs of experts with more than
    // reg_max rows, heaviest first: tiles with 4 token groups (65..128
    // rows), then 2 (33..64), then 1 (up to 32).  The GEMM deals the pairs to
    // the XCDs in bands of eight runs of kBand neighbours, serpentine (the
    // rest one by one), so every XCD gets a near-equal share of each class
    // and starts with its heaviest tiles.  Within a class pairs keep slot order, so
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
      if (cnt <= reg_max) return;
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
          ((int4*)plan)[1 + g] = make_int4(e, offsets[e], cnt, j * kTileTok);
        }
      }
      for (int q = 0; q < 3; ++q) base[q] += t[q];
    }
    if (threadIdx.x == 0) plan[0] = tot[0] + tot[1] + tot[2];
    return;
  }
  const int nblk = H >> 5;
  const int64_t i = (int64_t)(blockIdx.x - 2) * kThreads + threadIdx.x;
  if (i >= (int64_t)T * nblk) return;
  quantize_block_fp6(x, (int)(i / nblk), T, (int)(i % nblk), H, xq);
}

// ------------------------------------------------------------------ GEMM --

// LDS ring.  A slot holds one 128-value K stage of the tile's weight codes
// and activations, written straight from global memory by LDS DMA loads (a
// wave's load puts lane l's 16 or 4 bytes at the slot offset + size * l):
//   A   [256 rows][64 B]    weight codes; 16-byte piece p of row r at
//                           r*64 + 16*(p ^ ((r >> 2) & 3))
//   B   [2][32*TG][128 B]   activation terms; piece p of (term u, token t) at
//                           (u*32*TG + t)*128 + 16*(p ^ ((t >> 1) & 7))
//   BS  [2][32*TG][4 B]     their four scale bytes of the stage
// The XOR swizzles give the 16 lanes that read one K offset of 16
// consecutive rows or tokens 16 distinct 16-byte bank groups.  A tile with
// TG = 2 or 4 token groups of 32 has slots of 32.5 or 49 KB and a ring of 4
// or 3 of them, so 3 or 2 stages are in flight per CU while one is read.
// The weight scales travel in blocks of four stages (16 bytes per row, one
// memory request per row instead of four) through kScaleBufs buffers of
// [256 rows][16 B] after the ring; each stage's loads carry a quarter of
// the next block.
constexpr int kLdsBytes = 160 * 1024;
constexpr int kScaleBuf = kTileRows * 16;

template <int TG, bool FP6>
struct Ring {
  static_assert(TG == 2 || TG == 4, "one-group tiles use Ring1");
  static constexpr int kTok = 32 * TG;
  static constexpr int kA = kTileRows * 64;
  static constexpr int kB = 2 * kTok * 128;
  static constexpr int kBS = FP6 ? 0 : 2 * kTok * 4;  // FP6 records carry their scales
  static constexpr int kStage = kA + kB + kBS;
  static constexpr int kSlots = TG == 2 ? 4 : 3;
  // a scale block is refilled only after the barrier that follows its last
  // reader: 4 * kScaleBufs >= kSlots + 7
  static constexpr int kScaleBufs = (kSlots + 7 + 3) / 4;
  static constexpr int kScaleBase = kSlots * kStage;
  static constexpr int kBytes = kScaleBase + kScaleBufs * kScaleBuf;
  static constexpr int kOps = 4 + 1 + 2 * TG + (FP6 ? 0 : 1);  // DMA loads per wave per stage
  static constexpr int kX = 5;  // of them the weight codes and scales (loads 0 .. 4), issued first
  static_assert(kStage % 16 == 0, "16-byte aligned slots");
  static_assert(kBytes <= kLdsBytes, "ring fits in LDS");
};
constexpr int cmax(int a, int b) { return a > b ? a : b; }
// One-group tiles (1..32 routed rows) are bound by their weight stream.
// They run 256-value stages, so that every weight DMA load covers 8 rows x
// 128 bytes (whole cache lines) and can carry the non-temporal policy.  A
// slot holds
//   A   [256 rows][128 B]              piece p of row r at r*128 + 16*(p ^ ((r >> 1) & 7))
//   B   [2 terms][2 records][32][128 B] the stage's two 128-value records of
//                                      each (term, token t), piece p at
//                                      16*(p ^ ((t >> 1) & 7))
//   BS  [2 terms][2 records][32][4 B]  (E4M3 terms only) their scale words
// in a ring of 3 slots; the weight scales travel in blocks of two stages
// (16 bytes per row) through 3 buffers after the ring.
template <bool FP6>
struct Ring1 {
  static constexpr int kA = kTileRows * 128;
  static constexpr int kB = 2 * 2 * 32 * 128;
  static constexpr int kBS = FP6 ? 0 : 2 * 2 * 32 * 4;
  static constexpr int kStage = kA + kB + kBS;
  static constexpr int kSlots = 3;
  // a scale block is refilled only after the barrier that follows its last
  // reader: 2 * kScaleBufs >= kSlots + 3
  static constexpr int kScaleBufs = (kSlots + 3 + 1) / 2;
  static constexpr int kScaleBase = kSlots * kStage;
  static constexpr int kBytes = kScaleBase + kScaleBufs * kScaleBuf;
  static constexpr int kX = 8 + 2;                       // weight loads per wave and stage: codes, 2 scale quarters
  static constexpr int kOps = kX + 4 + (FP6 ? 0 : 1);    // and activation loads (terms, E4M3 scale words)
  static_assert(kBytes <= kLdsBytes, "ring fits in LDS");
};
constexpr int kRingBytes = cmax(cmax(cmax(Ring<2, false>::kBytes, Ring<4, false>::kBytes), Ring1<false>::kBytes),
                                Ring1<true>::kBytes);

// LDS DMA loads of 16 and 4 bytes per lane to the wave-uniform LDS address
// `lds` (lane l at lds + size*l).  Issued from asm, so the compiler neither
// counts them nor waits for them: the ring's waits below are explicit.
// From a wave-uniform base (scalar registers) plus this lane's 32-bit
// offset: a stage's loads advance only the bases, with scalar adds.  The
// asm sets m0 (the LDS address) itself and declares it clobbered; the
// compiler's note that a reserved register may not be preserved is moot,
// since no code here reads m0 after these loads.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void lds_dma16(const void* base, uint32_t off, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(off), "s"(base), "s"(lds) : "memory", "m0");
}
__device__ __forceinline__ void lds_dma4(const void* base, uint32_t off, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dword %0, %1" ::"v"(off), "s"(base), "s"(lds) : "memory", "m0");
}

__device__ __forceinline__ void lds_dma16_nt(const void* base, uint32_t off, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %1 nt" ::"v"(off), "s"(base), "s"(lds) : "memory", "m0");
}
#pragma clang diagnostic pop

// s_waitcnt vmcnt(N) (N clamped to the counter's 63) with the other counters free
template <int N>
__device__ __forceinline__ void wait_vm() {
  constexpr int M = N > 63 ? 63 : N;
  __builtin_amdgcn_s_waitcnt((M & 15) | ((M >> 4) << 14) | (7 << 4) | (15 << 8));
}

// Wait until at most n stages of this wave's DMA loads (OPS each) are
// outstanding.  Vector-memory loads complete in issue order, so this waits
// for every stage issued before the n most recent ones.
template <int OPS>
__device__ __forceinline__ void wait_stages(int n) {
  switch (n) {
    case 0: wait_vm<0>(); break;
    case 1: wait_vm<OPS>(); break;
    case 2: wait_vm<2 * OPS>(); break;
    case 3: wait_vm<3 * OPS>(); break;
    case 4: wait_vm<4 * OPS>(); break;
    default: wait_vm<5 * OPS>(); break;
  }
}

__device__ __forceinline__ v8i_t pack_b(const uint4& lo, const uint4& hi) {
  v8i_t v;
  v[0] = lo.x; v[1] = lo.y; v[2] = lo.z; v[3] = lo.w;
  v[4] = hi.x; v[5] = hi.y; v[6] = hi.z; v[7] = hi.w;
  return v;
}

// f(integral_constant<int, I>) for I = B .. E-1, in order
template <int B, int E, class F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (B < E) {
    f(std::integral_constant<int, B>());
    static_for<B + 1, E>(f);
  }
}

template <bool GATEUP>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(1, 1))) void mfma_ffn_kernel(
    moe_mxfp4_weights w, int k, const int32_t* __restrict__ sorted_rows, const int32_t* __restrict__ plan,
    const uint8_t* __restrict__ bq,  // B terms [K/128][brows][2][128]
    const uint8_t* __restrict__ bs,  // B scales [K/128][brows][2][4]
    int brows, float* __restrict__ out, int m_tiles,
    uint8_t* __restrict__ hq,  // gate/up: h terms written for the down GEMM ([I/128][hrows][2][128])
    uint8_t* __restrict__ hs,  // and their scales ([I/128][hrows][2][4])
    int hrows) {
  __shared__ __attribute__((aligned(1024))) uint8_t s_ring[kRingBytes];
  constexpr int kRB = kTileRows / 32;  // 32-row blocks of the tile

  const int H = w.hidden, I = w.inter;
  const int K = GATEUP ? H : I;         // reduction length
  const int out_cols = GATEUP ? I : H;  // columns of the output rows
  const int64_t qrow = K >> 1;          // FP4 bytes per weight row
  const int nsb = K >> 5;               // scale bytes per weight row
  const int nst = K / kStageK;

  // tile: block b runs on XCD b % 8.  The plan's pairs (heaviest first) go
  // in bands of 8 * kBand, one run of kBand neighbours per XCD, weight tile
  // major, so the token tiles of one expert that land on an XCD read each
  // weight tile into its L2 together.  The runs are dealt serpentine (even
  // bands XCD 0 first, odd bands XCD 7 first), so no XCD takes the heaviest
  // run of every band; pairs past the last whole band go one by one in the
  // next band's direction, one weight tile after another.
  const int bx = blockIdx.x, xcd = bx & 7, q = bx >> 3;
  const int npairs = plan[0];
  const int bands = npairs / (8 * kBand);
  const int q_bands = bands * kBand * m_tiles;  // blocks per XCD in whole bands
  int pair, mt;
  if (q < q_bands) {
    const int b = q / (kBand * m_tiles), qi = q - b * (kBand * m_tiles);
    mt = qi / kBand;
    pair = b * 8 * kBand + ((b & 1) ? 7 - xcd : xcd) * kBand + (qi - mt * kBand);
  } else {
    const int r = (q - q_bands) / m_tiles;
    mt = (q - q_bands) - r * m_tiles;
    pair = bands * 8 * kBand + ((bands & 1) ? 7 - xcd : xcd) + 8 * r;
  }
  if (pair >= npairs) return;
  const int4 rec = ((const int4*)plan)[1 + pair];  // (expert, first sorted row, row count, first token)
  const int e = rec.x, p0 = rec.y, cnt = rec.z, tok0 = rec.w;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n = lane & 31, half = lane >> 5;
  const uint32_t lds0 = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) uint8_t*)s_ring;
  const int64_t eo = (int64_t)e * w.expert_stride;
  // tile rows: gate/up = gate rows row0 .. row0+127 then the same up rows;
  // down = rows row0 .. row0+255
  const int row0 = GATEUP ? mt * (kTileRows / 2) : mt * kTileRows;

  auto a_row = [&](int r) -> const uint8_t* {  // codes of tile row r
    if (GATEUP)
      return r < kTileRows / 2 ? w.gate_q + eo + (int64_t)(row0 + r) * qrow
                               : w.up_q + eo + (int64_t)(row0 + r - kTileRows / 2) * qrow;
    return w.down_q + eo + (int64_t)(row0 + r) * qrow;
  };
  auto a_srow = [&](int r) -> const uint8_t* {  // scales of tile row r
    if (GATEUP)
      return r < kTileRows / 2 ? w.gate_s + eo + (int64_t)(row0 + r) * nsb
                               : w.up_s + eo + (int64_t)(row0 + r - kTileRows / 2) * nsb;
    return w.down_s + eo + (int64_t)(row0 + r) * nsb;
  };
  // B row of tile token t; tokens past the expert's count re-read its last row
  auto b_row = [&](int t) -> int64_t {
    const int tok = tok0 + t;
    const int p = p0 + (tok < cnt ? tok : cnt - 1);
    return GATEUP ? (int64_t)(sorted_rows[p] / k) : (int64_t)p;
  };

  // Token groups of 32 that hold routed rows: 1, 2 or 4 (3 runs as 4).
  // With TG groups, wave w takes token group w % TG and 2*TG of the 8 row
  // blocks: gate/up keeps each gate block with its up block (b and b+4).
  const int rows_in_tile = min(cnt - tok0, kTileTok);
  const int tg = rows_in_tile <= 32 ? 1 : rows_in_tile <= 64 ? 2 : 4;

  // Epilogue of a tile (acc: RBW row blocks of 32 rows x 32 tokens, row
  // block j at rows 32 rb_of(j); this lane's token tt).
  auto store_tile = [&](auto tok_c, auto rbw_c, const auto& acc, auto rb_of, int tt) {
    constexpr int kTok = decltype(tok_c)::value;
    constexpr int RBW = decltype(rbw_c)::value;
    // Epilogue: the tile's outputs pass through LDS (the ring is free once
    // every wave is past its last fragment reads), so that each store
    // instruction writes whole output rows (1 KB contiguous) instead of 64
    // scattered 16-byte pieces of 32 token rows.  LDS rows are padded by 4
    // floats: a 16-lane group's float4 writes then hit 64 distinct banks.
    constexpr int kCols = GATEUP ? kTileRows / 2 : kTileRows;  // output columns of the tile
    constexpr int kPitch = kCols + 4;                           // floats per LDS row
    static_assert(kTok * kPitch * 4 <= kRingBytes, "the output tile fits in the ring's LDS");
    float* so = (float*)s_ring;
    wait_vm<0>();  // no LDS DMA of this wave still in flight (the last scale prefetch)
    __syncthreads();
    float* srow = so + tt * kPitch;  // this lane's token
    if (GATEUP) {
      // j < RBW/2: gate block rb_of(j); j + RBW/2: the matching up block
#pragma unroll
      for (int j = 0; j < RBW / 2; ++j)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int c = 32 * rb_of(j) + 8 * g + 4 * half;
          float4 v;
          v.x = silu_mul(acc[j][4 * g + 0], acc[j + RBW / 2][4 * g + 0]);
          v.y = silu_mul(acc[j][4 * g + 1], acc[j + RBW / 2][4 * g + 1]);
          v.z = silu_mul(acc[j][4 * g + 2], acc[j + RBW / 2][4 * g + 2]);
          v.w = silu_mul(acc[j][4 * g + 3], acc[j + RBW / 2][4 * g + 3]);
          *(float4*)(srow + c) = v;
        }
    } else {
#pragma unroll
      for (int j = 0; j < RBW; ++j) {
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int c = 32 * rb_of(j) + 8 * g + 4 * half;
          *(float4*)(srow + c) = make_float4(acc[j][4 * g + 0], acc[j][4 * g + 1], acc[j][4 * g + 2], acc[j][4 * g + 3]);
        }
      }
    }
    __syncthreads();
    const int nrow = min(kTok, cnt - tok0);  // tokens of the tile with routed rows
    if (GATEUP) {
      // h never goes to memory in fp32: each thread takes (token, 32-block)
      // items of the tile's 128 columns (one 128-value K stage of the down
      // GEMM) and writes their two E4M3 terms, the down GEMM's B operand
      for (int it = tid; it < 4 * nrow; it += kThreads) {
        const int t = it >> 2, b = it & 3;
        const float4* src = (const float4*)(so + t * kPitch + 32 * b);
        float v[32];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const float4 f = src[i];
          v[4 * i] = f.x;
          v[4 * i + 1] = f.y;
          v[4 * i + 2] = f.z;
          v[4 * i + 3] = f.w;
        }
        e4m3_two_terms(v, p0 + tok0 + t, hrows, row0 / 32 + b, hq, hs);
      }
    } else {
      constexpr int kLanesPerRow = kCols / 4;              // float4 of an output row
      constexpr int kRowsPerOp = MOE_WAVE / kLanesPerRow;  // output rows per store instruction
      const int c4 = lane % kLanesPerRow;
      for (int t = wave * kRowsPerOp + lane / kLanesPerRow; t < nrow; t += 4 * kRowsPerOp)
        *(float4*)(out + (int64_t)(p0 + tok0 + t) * out_cols + row0 + 4 * c4) = *(const float4*)(so + t * kPitch + 4 * c4);
    }
  };

  auto body = [&](auto tg_c) {
    constexpr int TG = decltype(tg_c)::value;
    constexpr bool FP6 = GATEUP;  // gate/up: x in two E2M3 terms; down: h in two E4M3 terms
    using G = Ring<TG, FP6>;
    constexpr int R = G::kSlots;
    constexpr int RBW = 2 * TG;  // row blocks of this wave
    const int tgi = wave % TG;
    const int rb_base = RBW == kRB ? 0 : (wave / TG) * (RBW / 2);
    auto rel = [](int j) { return j < RBW / 2 ? j : kRB / 2 + (j - RBW / 2); };
    auto rb_of = [&](int j) { return rb_base + rel(j); };

    // DMA sources of this lane (stage 0).  A: load i of wave w fills 1 KB
    // chunk c = 4i + w, rows 16c + lane/4, slot lane%4 of the row taking
    // piece (lane%4) ^ ((lane >> 4) & 3).  AS: rows 64w + lane.  B: load j
    // fills chunk c = w + 4j: term c / (4TG), tokens 8 (c % 4TG) + lane/8,
    // slot lane%8 taking piece (lane%8) ^ ((token >> 1) & 7).  BS: entry
    // 64 (w % TG) + lane = term * 32TG + token (waves past TG repeat it).
    // Each DMA source is a wave-uniform base (tile rows 0 and 128: the gate
    // and up matrices of gate/up, or two halves of down) plus this lane's
    // 32-bit offset, the same for every stage.
    const int apiece = (lane & 3) ^ ((lane >> 4) & 3);
    const uint8_t* const a_base[2] = {a_row(0), a_row(kTileRows / 2)};
    const uint8_t* const as_base[2] = {a_srow(0), a_srow(kTileRows / 2)};
    uint32_t a_off_s[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
      a_off_s[i] = (uint32_t)((16 * (4 * i + wave) + (lane >> 2) - (i >= 2 ? kTileRows / 2 : 0)) * qrow + 16 * apiece);
    // AS: quarter q of a scale block = rows 64q + 16w + lane/4, word lane%4:
    // base q / 2 advanced by 64 rows for odd q (scalar), this lane's offset
    const uint32_t as_off_s = (uint32_t)((16 * wave + (lane >> 2)) * nsb + 4 * (lane & 3));
    const int nblk = nst >> 2;  // scale blocks per row
    uint32_t b_off_s[2 * TG];
#pragma unroll
    for (int j = 0; j < 2 * TG; ++j) {
      const int c = wave + 4 * j, u = c / (4 * TG);
      const int t = 8 * (c % (4 * TG)) + (lane >> 3);
      b_off_s[j] = (uint32_t)((b_row(t) * 2 + u) * 128 + 16 * ((lane & 7) ^ ((t >> 1) & 7)));
    }
    const int be = 64 * tgi + lane;
    const uint32_t bs_off_s = (uint32_t)((b_row(be % G::kTok) * 2 + be / G::kTok) * 4);
    const int64_t bq_stage = (int64_t)brows * 256, bs_stage = (int64_t)brows * 8;

    // quarter q of weight-scale block b (clamped to the last block) into its buffer
    auto issue_scales = [&](int b, int q) {
      const uint32_t dst = lds0 + (uint32_t)(G::kScaleBase + (b % G::kScaleBufs) * kScaleBuf + (64 * q + 16 * wave) * 16);
      lds_dma4(as_base[q >= 2 ? 1 : 0] + (q & 1) * 64 * nsb + 16 * min(b, nblk - 1), as_off_s, dst);
    };
    // load o (0 .. kOps-1) of this wave's share of stage st into slot sl;
    // load 4 is quarter st % 4 of the scale block after st's
    auto issue_op = [&](int st, int sl, auto o_c) {
      constexpr int o = decltype(o_c)::value;
      const uint32_t sb = lds0 + (uint32_t)(sl * G::kStage);
      if constexpr (o < 4) lds_dma16(a_base[o >= 2 ? 1 : 0] + st * 64, a_off_s[o], sb + (4 * o + wave) * 1024);
      else if constexpr (o == 4) issue_scales((st >> 2) + 1, st & 3);
      else if constexpr (o < 5 + 2 * TG)
        lds_dma16(bq + st * bq_stage, b_off_s[o - 5], sb + G::kA + (wave + 4 * (o - 5)) * 1024);
      else if constexpr (!FP6) lds_dma4(bs + st * bs_stage, bs_off_s, sb + G::kA + G::kB + tgi * 256);
    };
    // a stage's weight loads (X: codes, scale quarter) and activation loads (Y)
    auto issue_x = [&](int st, int sl) { static_for<0, G::kX>([&](auto o) { issue_op(st, sl, o); }); };
    auto issue_y = [&](int st, int sl) { static_for<G::kX, G::kOps>([&](auto o) { issue_op(st, sl, o); }); };

    // fragment offsets of this lane within a slot: A row 32 rb + n, piece
    // 2 s + half; B token 32 tgi + n, pieces 4 s + 2 half + i (i = 0, 1)
    const int tt = 32 * tgi + n;
    const uint32_t a_off[2] = {(uint32_t)((32 * rb_base + n) * 64 + 16 * ((0 + half) ^ ((n >> 2) & 3))),
                               (uint32_t)((32 * rb_base + n) * 64 + 16 * ((2 + half) ^ ((n >> 2) & 3)))};
    const uint32_t as_off = (uint32_t)((32 * rb_base + n) * 16);  // within a scale buffer
    // E4M3: two 16-byte pieces 4s + 2 half + i; E2M3: the 16 bytes of piece
    // 3s + half and the 8 bytes at 8 half in piece 3s + 2; its scale word at
    // 4 half in piece 6 of the same record (bytes 0 and 2 for steps 0 and 1)
    const int bsw = (n >> 1) & 7;
    uint32_t b_off[2][2];
#pragma unroll
    for (int s = 0; s < 2; ++s)
#pragma unroll
      for (int i = 0; i < 2; ++i)
        b_off[s][i] = FP6 ? (uint32_t)(G::kA + tt * 128 + (i == 0 ? 16 * ((3 * s + half) ^ bsw)
                                                                     : 16 * ((3 * s + 2) ^ bsw) + 8 * half))
                          : (uint32_t)(G::kA + tt * 128 + 16 * ((4 * s + 2 * half + i) ^ bsw));
    const uint32_t bs_off = FP6 ? (uint32_t)(G::kA + tt * 128 + 16 * (6 ^ bsw) + 4 * half)
                                : (uint32_t)(G::kA + G::kB + tt * 4);
    constexpr int kBSTerm = FP6 ? G::kTok * 128 : G::kTok * 4;  // scale words of term 1 after term 0's
    constexpr int kBSShift = FP6 ? 0 : 1;  // E4M3 scale words need byte 2s + half moved to 2s
    // one B fragment: E4M3 32 bytes, E2M3 24 (the high half's last 8 bytes zero)
    auto ld_b = [&](const uint8_t* p, int i) -> uint4 {
      if (FP6 && i == 1) {
        const uint2 v = *(const uint2*)p;
        return make_uint4(v.x, v.y, 0u, 0u);
      }
      return *(const uint4*)p;
    };

    auto read_a = [&](int sl, int s, uint4 (&a)[RBW]) {
      const uint8_t* base = s_ring + sl * G::kStage + a_off[s];
#pragma unroll
      for (int j = 0; j < RBW; ++j) a[j] = *(const uint4*)(base + 32 * rel(j) * 64);
    };
    auto read_b = [&](int sl, int s, uint4 (&b)[2][2]) {
#pragma unroll
      for (int u = 0; u < 2; ++u)
#pragma unroll
        for (int i = 0; i < 2; ++i) b[u][i] = ld_b(s_ring + sl * G::kStage + b_off[s][i] + u * G::kTok * 128, i);
    };
    // weight-scale words of stage st in LDS
    auto sa_base = [&](int st) -> const uint8_t* {
      return s_ring + G::kScaleBase + ((st >> 2) % G::kScaleBufs) * kScaleBuf + as_off + 4 * (st & 3);
    };
    // stage st's scale words (in slot sl), as stored
    auto read_sc = [&](int st, int sl, uint32_t (&sa)[RBW], uint32_t (&sb)[2]) {
      const uint8_t* ab = sa_base(st);
#pragma unroll
      for (int j = 0; j < RBW; ++j) sa[j] = *(const uint32_t*)(ab + 32 * rel(j) * 16);
#pragma unroll
      for (int u = 0; u < 2; ++u) sb[u] = *(const uint32_t*)(s_ring + sl * G::kStage + bs_off + u * kBSTerm);
    };
    // The words arrive as stored (this lane's byte of step s at 2s + half);
    // moving it to byte 2s, the MFMA's select, happens in the stage that
    // uses them (a draining stage at its start, a steady stage just before
    // each word's first MFMA), so no scale read waits for its data mid-stage.
    auto place_sc = [&](uint32_t (&sa)[RBW], uint32_t (&sb)[2]) {
#pragma unroll
      for (int j = 0; j < RBW; ++j) sa[j] >>= 8 * half;
#pragma unroll
      for (int u = 0; u < 2; ++u) sb[u] >>= 8 * half * kBSShift;
    };

    v16f_t acc[RBW];
#pragma unroll
    for (int j = 0; j < RBW; ++j)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[j][i] = 0.0f;

    // One 64-deep step: FP4 weights (format 4) times the two activation
    // terms (E2M3 format 2 or E4M3 format 0), byte 2s of the scale words.
    constexpr int kBFmt = FP6 ? 2 : 0;
    auto mma = [&](auto s_c, const uint4 (&a)[RBW], const uint4 (&b)[2][2], const uint32_t (&sa)[RBW],
                   const uint32_t (&sb)[2]) {
      constexpr int OP = 2 * decltype(s_c)::value;
      const v8i_t B0 = pack_b(b[0][0], b[0][1]), B1 = pack_b(b[1][0], b[1][1]);
#pragma unroll
      for (int u = 0; u < 2; ++u)
#pragma unroll
        for (int j = 0; j < RBW; ++j) {
          v8i_t A;
          A[0] = a[j].x; A[1] = a[j].y; A[2] = a[j].z; A[3] = a[j].w;
          A[4] = 0; A[5] = 0; A[6] = 0; A[7] = 0;
          acc[j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(A, u == 0 ? B0 : B1, acc[j], 4, kBFmt, OP, sa[j],
                                                                   OP, sb[u]);
        }
    };

    // Pipeline over stages st (slot st % R).  The ring is filled R stages
    // ahead.  Within stage st: read its step-1 fragments, run step 0, wait
    // for this wave's loads of stage st+1 and meet the other waves (after
    // which stage st+1 is in LDS and nobody reads slot st % R any more),
    // refill that slot with stage st+R's weights, read stage st+1's step-0
    // fragments and scales, run step 1; stage st+R's activation loads follow
    // in step 0 of stage st+1, so each step carries a share of the DMA
    // issues.  Loads still go out stage after stage, so the wait counts are
    // those of whole stages.  The steady-state loop (a stage R ahead left to
    // load) is one basic block of two stages, so the step-0 MFMAs stay ahead
    // of the wait and keep the pipe busy through it; the last R stages drain.
    // Scale block 0, then stages 0 .. R-1 (each with a quarter of block 1,
    // 2, ...); stage R-1's activation loads go out in stage 0.
#pragma unroll
    for (int q = 0; q < 4; ++q) issue_scales(0, q);
#pragma unroll
    for (int j = 0; j < R; ++j)
      if (j < nst) {
        issue_x(j, j);
        if (j < R - 1) issue_y(j, j);
      }
    if (nst >= R)
      wait_vm<(R - 2) * G::kOps + G::kX>();
    else
      wait_stages<G::kOps>(nst - 1);
    __syncthreads();
    uint4 a0[RBW], b0[2][2];
    // scale words: two sets, the current stage's and the next one's, which
    // trade roles every stage (no copies between them in the loop)
    uint32_t sa[2][RBW], sb[2][2];
    read_sc(0, 0, sa[0], sb[0]);
    read_a(0, 0, a0);
    read_b(0, 0, b0);
    // all of them in before the loop: the loop's own waits then follow the
    // order of its reads, not the order these were issued in
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
    int st = 0, sl = 0;
    // one MFMA of row block j at step s with activation term u
    auto mma_ju = [&](auto s_c, auto j_c, auto u_c, const uint4& a, const v8i_t& Bu, uint32_t sa_j, uint32_t sb_u) {
      constexpr int OP = 2 * decltype(s_c)::value;
      constexpr int j = decltype(j_c)::value;
      v8i_t A;
      A[0] = a.x; A[1] = a.y; A[2] = a.z; A[3] = a.w;
      A[4] = 0; A[5] = 0; A[6] = 0; A[7] = 0;
      acc[j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(A, Bu, acc[j], 4, kBFmt, OP, sa_j, OP, sb_u);
    };
    // Steady stage (a stage R ahead left to load), scale set P current.  A step's MFMAs run term
    // major (term 0 of every row block, then term 1), so the two MFMAs that
    // accumulate into one row block are RBW issues apart.  Issue order, fixed
    // by scheduling fences between MFMAs: step 0's MFMAs each followed by a
    // share of the step-1 fragment reads; the wait and the barrier; step 1's
    // MFMAs each followed by a share of the refill loads and of the next
    // stage's step-0 and scale reads.  Vector-memory issues spread over the
    // MFMAs this way never back up the address path far enough to hold up
    // the next MFMA.
    auto steady_stage = [&](auto p_c) {
      constexpr int P = decltype(p_c)::value, Q = 1 - P;
      constexpr int kM = 2 * RBW;             // MFMAs per step
      constexpr int kReads1 = RBW + 4;        // step-1 fragments: RBW of A, 4 of B
      constexpr int kReadsN = RBW + 4 + RBW + 2;  // next stage: A, B fragments and scale words
      constexpr int kY = G::kOps - G::kX;      // activation loads of stage st+R-1
      uint4 a1[RBW], b1[2][2];
      const v8i_t B0 = pack_b(b0[0][0], b0[0][1]), B1 = pack_b(b0[1][0], b0[1][1]);
      const uint8_t* a1_base = s_ring + sl * G::kStage + a_off[1];
      const int psl = sl == 0 ? R - 1 : sl - 1;  // slot of stage st+R-1
      static_for<0, kM>([&](auto i_c) {
        constexpr int i = decltype(i_c)::value;
        constexpr int u = i / RBW;
        // each scale word moves to the MFMA's byte select just before its
        // first use, so the first MFMAs wait only for the first reads
        if constexpr (i < RBW) sa[P][i] >>= 8 * half;
        if constexpr (i % RBW == 0) sb[P][u] >>= 8 * half * kBSShift;
        mma_ju(std::integral_constant<int, 0>(), std::integral_constant<int, i % RBW>(),
               std::integral_constant<int, u>(), a0[i % RBW], u == 0 ? B0 : B1, sa[P][i % RBW], sb[P][u]);
        static_for<G::kX + i * kY / kM, G::kX + (i + 1) * kY / kM>([&](auto o_c) { issue_op(st + R - 1, psl, o_c); });
        static_for<i * kReads1 / kM, (i + 1) * kReads1 / kM>([&](auto r_c) {
          constexpr int r = decltype(r_c)::value;
          if constexpr (r < RBW) a1[r] = *(const uint4*)(a1_base + 32 * rel(r) * 64);
          else b1[(r - RBW) / 2][(r - RBW) % 2] =
                   ld_b(s_ring + sl * G::kStage + b_off[1][(r - RBW) % 2] + ((r - RBW) / 2) * G::kTok * 128, (r - RBW) % 2);
        });
        __builtin_amdgcn_sched_barrier(0);
      });
      const int nsl = sl + 1 == R ? 0 : sl + 1;
      wait_vm<(R - 2) * G::kOps>();
      __syncthreads();
      const v8i_t C0 = pack_b(b1[0][0], b1[0][1]), C1 = pack_b(b1[1][0], b1[1][1]);
      const uint8_t* an_base = s_ring + nsl * G::kStage + a_off[0];
      const uint8_t* sn_base = s_ring + nsl * G::kStage;
      const uint8_t* san_base = sa_base(st + 1);
      static_for<0, kM>([&](auto i_c) {
        constexpr int i = decltype(i_c)::value;
        constexpr int u = i / RBW;
        mma_ju(std::integral_constant<int, 1>(), std::integral_constant<int, i % RBW>(),
               std::integral_constant<int, u>(), a1[i % RBW], u == 0 ? C0 : C1, sa[P][i % RBW], sb[P][u]);
        static_for<i * G::kX / kM, (i + 1) * G::kX / kM>([&](auto o_c) { issue_op(st + R, sl, o_c); });
        // next stage's reads in the order its step 0 uses them: term 0's
        // scale word and fragment, then per row block its scale word and
        // weight fragment, then term 1's scale word and fragment
        static_for<i * kReadsN / kM, (i + 1) * kReadsN / kM>([&](auto r_c) {
          constexpr int r = decltype(r_c)::value;
          constexpr int rt = r < 3 ? r : r - 3 - 2 * RBW;  // 0 .. 2 within a term group
          constexpr int ut = r < 3 ? 0 : 1;
          if constexpr (r < 3 || r >= 3 + 2 * RBW) {
            if constexpr (rt == 0)
              sb[Q][ut] = *(const uint32_t*)(sn_base + bs_off + ut * kBSTerm);
            else
              b0[ut][rt - 1] = ld_b(sn_base + b_off[0][rt - 1] + ut * G::kTok * 128, rt - 1);
          } else if constexpr ((r - 3) % 2 == 0) {
            sa[Q][(r - 3) / 2] = *(const uint32_t*)(san_base + 32 * rel((r - 3) / 2) * 16);
          } else {
            a0[(r - 3) / 2] = *(const uint4*)(an_base + 32 * rel((r - 3) / 2) * 64);
          }
        });
        __builtin_amdgcn_sched_barrier(0);
      });
      sl = nsl;
    };
    // Draining stage: nothing left to load; scale set 0 current.
    auto drain_stage = [&]() {
      uint4 a1[RBW], b1[2][2];
      if (st + R - 1 < nst) issue_y(st + R - 1, sl == 0 ? R - 1 : sl - 1);  // the last stage's activations
      place_sc(sa[0], sb[0]);
      read_a(sl, 1, a1);
      read_b(sl, 1, b1);
      mma(std::integral_constant<int, 0>(), a0, b0, sa[0], sb[0]);
      const int nsl = sl + 1 == R ? 0 : sl + 1;
      if (st + 1 < nst) {
        wait_stages<G::kOps>(nst - 2 - st);
        __syncthreads();
        read_sc(st + 1, nsl, sa[1], sb[1]);
        read_a(nsl, 0, a0);
        read_b(nsl, 0, b0);
      }
      mma(std::integral_constant<int, 1>(), a1, b1, sa[0], sb[0]);
#pragma unroll
      for (int j = 0; j < RBW; ++j) sa[0][j] = sa[1][j];
      sb[0][0] = sb[1][0];
      sb[0][1] = sb[1][1];
      sl = nsl;
    };
    // the steady loop two stages per trip, so the scale sets keep their registers
    constexpr std::integral_constant<int, 0> kSet0;
    constexpr std::integral_constant<int, 1> kSet1;
    for (; st + R + 1 < nst; ++st) {
      steady_stage(kSet0);
      ++st;
      steady_stage(kSet1);
    }
    if (st + R < nst) {
      steady_stage(kSet0);
      ++st;
#pragma unroll
      for (int j = 0; j < RBW; ++j) sa[0][j] = sa[1][j];
      sb[0][0] = sb[1][0];
      sb[0][1] = sb[1][1];
    }
    for (; st < nst; ++st) drain_stage();

    store_tile(std::integral_constant<int, G::kTok>(), std::integral_constant<int, RBW>(), acc, rb_of, tt);
  };
  // One-group tiles: 256-value stages of four 64-deep steps (Ring1).  Wave
  // w takes row blocks w and w + 4 (gate/up: a gate block and its up block)
  // for the tile's 32 token slots.  Per stage and wave: 8 weight-code loads
  // (chunk c = 4i + w: rows 8c .. 8c+7, 128 bytes each, non-temporal), 2
  // quarters of a weight-scale block, 4 activation-term loads (chunk c = w +
  // 4j: units v = 8c + lane/8 = (term, record, token)), for E4M3 terms one
  // scale-word load.  The pipeline is the generic one's with four steps: the
  // barrier follows the reads of the stage's last step, the freed slot's
  // weight loads and the next stage's reads go with step 3, and the
  // activation loads of a stage follow in step 0 of the stage after.
  auto body1 = [&]() {
    constexpr bool FP6 = GATEUP;
    using G = Ring1<FP6>;
    constexpr int R = G::kSlots;
    constexpr int RBW = 2;
    constexpr int S = 4;
    const int nst1 = K / 256;
    const int nblk = nst1 >> 1;  // scale blocks (two stages) per row
    auto rel = [](int j) { return j == 0 ? 0 : kRB / 2; };
    auto rb_of = [&](int j) { return wave + rel(j); };

    // DMA sources: wave-uniform bases, per-lane 32-bit offsets
    const int apiece = (lane & 7) ^ ((4 * (wave & 1) + (lane >> 4)) & 7);
    const uint8_t* const a_base[2] = {a_row(0), a_row(kTileRows / 2)};
    const uint8_t* const as_base[2] = {a_srow(0), a_srow(kTileRows / 2)};
    uint32_t a_off_s[8];
#pragma unroll
    for (int i = 0; i < 8; ++i)
      a_off_s[i] = (uint32_t)((8 * (4 * i + wave) + (lane >> 3) - (i >= 4 ? kTileRows / 2 : 0)) * qrow + 16 * apiece);
    const uint32_t as_off_s = (uint32_t)((16 * wave + (lane >> 2)) * nsb + 4 * (lane & 3));
    uint32_t b_off_s[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int v = 8 * (wave + 4 * j) + (lane >> 3);
      const int u = v >> 6, r = (v >> 5) & 1, t = v & 31;
      b_off_s[j] = (uint32_t)(((r * (int64_t)brows + b_row(t)) * 2 + u) * 128 + 16 * ((lane & 7) ^ ((t >> 1) & 7)));
    }
    const int bsd = 64 * (wave & 1) + lane;  // E4M3 scale word: (term, record, token) = (bsd >> 6, (bsd >> 5) & 1, bsd & 31)
    const uint32_t bs_off_s =
        (uint32_t)((((bsd >> 5) & 1) * (int64_t)brows + b_row(bsd & 31)) * 8 + 4 * (bsd >> 6));
    const int64_t bq_stage = (int64_t)brows * 512, bs_stage = (int64_t)brows * 16;

    auto issue_scales = [&](int b, int q) {
      const uint32_t dst = lds0 + (uint32_t)(G::kScaleBase + (b % G::kScaleBufs) * kScaleBuf + (64 * q + 16 * wave) * 16);
      lds_dma4(as_base[q >= 2 ? 1 : 0] + (q & 1) * 64 * nsb + 16 * min(b, nblk - 1), as_off_s, dst);
    };
    // load o of this wave's share of stage st into slot sl; loads 8 and 9
    // are quarters 2 (st % 2) and 2 (st % 2) + 1 of the scale block after st's
    auto issue_op = [&](int st, int sl, auto o_c) {
      constexpr int o = decltype(o_c)::value;
      const uint32_t sb = lds0 + (uint32_t)(sl * G::kStage);
      if constexpr (o < 8) lds_dma16_nt(a_base[o >= 4 ? 1 : 0] + st * 128, a_off_s[o], sb + (4 * o + wave) * 1024);
      else if constexpr (o < G::kX) issue_scales((st >> 1) + 1, 2 * (st & 1) + (o - 8));
      else if constexpr (o < G::kX + 4)
        lds_dma16(bq + st * bq_stage, b_off_s[o - G::kX], sb + G::kA + (wave + 4 * (o - G::kX)) * 1024);
      else lds_dma4(bs + st * bs_stage, bs_off_s, sb + G::kA + G::kB + (wave & 1) * 256);
    };
    auto issue_x = [&](int st, int sl) { static_for<0, G::kX>([&](auto o) { issue_op(st, sl, o); }); };
    auto issue_y = [&](int st, int sl) { static_for<G::kX, G::kOps>([&](auto o) { issue_op(st, sl, o); }); };

    // fragment offsets within a slot: A row 32 rb + n, piece 2s + half; B
    // record (term u, record s/2, token n): E2M3 the 16 bytes of piece
    // 3(s%2) + half and the 8 bytes at 8 half in piece 3(s%2) + 2, its scale
    // word at 4 half in piece 6; E4M3 pieces 4(s%2) + 2 half + i
    const int bsw = (n >> 1) & 7;
    uint32_t a_off[S];
#pragma unroll
    for (int s = 0; s < S; ++s) a_off[s] = (uint32_t)((32 * wave + n) * 128 + 16 * ((2 * s + half) ^ bsw));
    constexpr int kRecB = 32 * 128;  // bytes between records of one term
    uint32_t b_off[S][2];
#pragma unroll
    for (int s = 0; s < S; ++s)
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int sp = s & 1;
        const uint32_t rec = (uint32_t)(G::kA + (s >> 1) * kRecB + n * 128);
        b_off[s][i] = FP6 ? rec + (i == 0 ? 16 * ((3 * sp + half) ^ bsw) : 16 * ((3 * sp + 2) ^ bsw) + 8 * half)
                          : rec + 16 * ((4 * sp + 2 * half + i) ^ bsw);
      }
    // scale words of record r (steps 2r, 2r+1): E2M3 in the record, E4M3 in BS
    auto sb_off = [&](int u, int r) -> uint32_t {
      return FP6 ? (uint32_t)(G::kA + (2 * u + r) * kRecB + n * 128 + 16 * (6 ^ bsw) + 4 * half)
                 : (uint32_t)(G::kA + G::kB + ((2 * u + r) * 32 + n) * 4);
    };
    constexpr int kTermB = 2 * kRecB;  // bytes between the terms' records
    constexpr int kBSShift = FP6 ? 0 : 1;
    const uint32_t as_off = (uint32_t)((32 * wave + n) * 16);  // within a scale buffer
    auto ld_b = [&](const uint8_t* p, int i) -> uint4 {
      if (FP6 && i == 1) {
        const uint2 v = *(const uint2*)p;
        return make_uint4(v.x, v.y, 0u, 0u);
      }
      return *(const uint4*)p;
    };
    // fragments of step s of the stage in slot sl
    auto read_a = [&](int sl, int s, uint4 (&a)[RBW]) {
      const uint8_t* base = s_ring + sl * G::kStage + a_off[s];
#pragma unroll
      for (int j = 0; j < RBW; ++j) a[j] = *(const uint4*)(base + 32 * rel(j) * 128);
    };
    auto read_b = [&](int sl, int s, uint4 (&b)[2][2]) {
#pragma unroll
      for (int u = 0; u < 2; ++u)
#pragma unroll
        for (int i = 0; i < 2; ++i) b[u][i] = ld_b(s_ring + sl * G::kStage + b_off[s][i] + u * kTermB, i);
    };
    // scale words of stage st (slot sl) as stored: sa[j][r], sb[u][r] serve steps 2r, 2r+1
    auto read_sc = [&](int st, int sl, uint32_t (&sa)[RBW][2], uint32_t (&sb)[2][2]) {
      const uint8_t* ab = s_ring + G::kScaleBase + ((st >> 1) % G::kScaleBufs) * kScaleBuf + as_off + 8 * (st & 1);
#pragma unroll
      for (int j = 0; j < RBW; ++j)
#pragma unroll
        for (int r = 0; r < 2; ++r) sa[j][r] = *(const uint32_t*)(ab + 32 * rel(j) * 16 + 4 * r);
#pragma unroll
      for (int u = 0; u < 2; ++u)
#pragma unroll
        for (int r = 0; r < 2; ++r) sb[u][r] = *(const uint32_t*)(s_ring + sl * G::kStage + sb_off(u, r));
    };

    v16f_t acc[RBW];
#pragma unroll
    for (int j = 0; j < RBW; ++j)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[j][i] = 0.0f;
    constexpr int kBFmt = FP6 ? 2 : 0;
    // the MFMAs of step s, term major; scale words shifted to the MFMA's byte
    // select on their first use (step 2r for record r)
    auto mma_step = [&](auto s_c, const uint4 (&a)[RBW], const uint4 (&b)[2][2], uint32_t (&sa)[RBW][2],
                        uint32_t (&sb)[2][2]) {
      constexpr int s = decltype(s_c)::value;
      constexpr int r = s >> 1, OP = 2 * (s & 1);
      if constexpr ((s & 1) == 0) {
#pragma unroll
        for (int j = 0; j < RBW; ++j) sa[j][r] >>= 8 * half;
#pragma unroll
        for (int u = 0; u < 2; ++u) sb[u][r] >>= 8 * half * kBSShift;
      }
      const v8i_t B0 = pack_b(b[0][0], b[0][1]), B1 = pack_b(b[1][0], b[1][1]);
#pragma unroll
      for (int u = 0; u < 2; ++u)
#pragma unroll
        for (int j = 0; j < RBW; ++j) {
          v8i_t A;
          A[0] = a[j].x; A[1] = a[j].y; A[2] = a[j].z; A[3] = a[j].w;
          A[4] = 0; A[5] = 0; A[6] = 0; A[7] = 0;
          acc[j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(A, u == 0 ? B0 : B1, acc[j], 4, kBFmt, OP,
                                                                   sa[j][r], OP, sb[u][r]);
        }
    };

    // prologue: scale block 0, then stages 0 .. R-1 (stage R-1's activation
    // loads go out in stage 0)
#pragma unroll
    for (int q = 0; q < 4; ++q) issue_scales(0, q);
#pragma unroll
    for (int j = 0; j < R; ++j)
      if (j < nst1) {
        issue_x(j, j);
        if (j < R - 1) issue_y(j, j);
      }
    if (nst1 >= R)
      wait_vm<(R - 2) * G::kOps + G::kX>();
    else
      wait_stages<G::kOps>(nst1 - 1);
    __syncthreads();
    uint4 fa[2][RBW], fb[2][2][2];  // fragments of the current and the next step
    uint32_t sa[2][RBW][2], sb[2][2][2];
    read_sc(0, 0, sa[0], sb[0]);
    read_a(0, 0, fa[0]);
    read_b(0, 0, fb[0]);
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): the loop's waits then follow its own reads
    int st = 0, sl = 0;

    // Steady stage (a stage R ahead left to load), scale set P current
    auto steady_stage = [&](auto p_c) {
      constexpr int P = decltype(p_c)::value, Q = 1 - P;
      const int psl = sl == 0 ? R - 1 : sl - 1;  // slot of stage st+R-1
      const int nsl = sl + 1 == R ? 0 : sl + 1;
      // step 0: its MFMAs, the activation loads of stage st+R-1, step 1's fragments
      read_a(sl, 1, fa[1]);
      read_b(sl, 1, fb[1]);
      mma_step(std::integral_constant<int, 0>(), fa[0], fb[0], sa[P], sb[P]);
      issue_y(st + R - 1, psl);
      __builtin_amdgcn_sched_barrier(0);
      // step 1, step 2's fragments
      read_a(sl, 2, fa[0]);
      read_b(sl, 2, fb[0]);
      mma_step(std::integral_constant<int, 1>(), fa[1], fb[1], sa[P], sb[P]);
      __builtin_amdgcn_sched_barrier(0);
      // step 2, step 3's fragments (the last reads of this slot)
      read_a(sl, 3, fa[1]);
      read_b(sl, 3, fb[1]);
      mma_step(std::integral_constant<int, 2>(), fa[0], fb[0], sa[P], sb[P]);
      __builtin_amdgcn_sched_barrier(0);
      // stage st+1 in LDS, nobody reads slot sl any more
      wait_vm<(R - 2) * G::kOps>();
      __syncthreads();
      // step 3, the freed slot's weight loads, the next stage's step-0 fragments and scale words
      issue_x(st + R, sl);
      read_sc(st + 1, nsl, sa[Q], sb[Q]);
      read_a(nsl, 0, fa[0]);
      read_b(nsl, 0, fb[0]);
      mma_step(std::integral_constant<int, 3>(), fa[1], fb[1], sa[P], sb[P]);
      __builtin_amdgcn_sched_barrier(0);
      sl = nsl;
    };
    // Draining stage: nothing left to load; scale set 0 current
    auto drain_stage = [&]() {
      if (st + R - 1 < nst1) issue_y(st + R - 1, sl == 0 ? R - 1 : sl - 1);  // the last stage's activations
      const int nsl = sl + 1 == R ? 0 : sl + 1;
      read_a(sl, 1, fa[1]);
      read_b(sl, 1, fb[1]);
      mma_step(std::integral_constant<int, 0>(), fa[0], fb[0], sa[0], sb[0]);
      read_a(sl, 2, fa[0]);
      read_b(sl, 2, fb[0]);
      mma_step(std::integral_constant<int, 1>(), fa[1], fb[1], sa[0], sb[0]);
      read_a(sl, 3, fa[1]);
      read_b(sl, 3, fb[1]);
      mma_step(std::integral_constant<int, 2>(), fa[0], fb[0], sa[0], sb[0]);
      if (st + 1 < nst1) {
        wait_stages<G::kOps>(nst1 - 2 - st);
        __syncthreads();
        read_sc(st + 1, nsl, sa[1], sb[1]);
        read_a(nsl, 0, fa[0]);
        read_b(nsl, 0, fb[0]);
      }
      mma_step(std::integral_constant<int, 3>(), fa[1], fb[1], sa[0], sb[0]);
#pragma unroll
      for (int j = 0; j < RBW; ++j) {
        sa[0][j][0] = sa[1][j][0];
        sa[0][j][1] = sa[1][j][1];
      }
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        sb[0][u][0] = sb[1][u][0];
        sb[0][u][1] = sb[1][u][1];
      }
      sl = nsl;
    };
    constexpr std::integral_constant<int, 0> kSet0;
    constexpr std::integral_constant<int, 1> kSet1;
    for (; st + R + 1 < nst1; ++st) {
      steady_stage(kSet0);
      ++st;
      steady_stage(kSet1);
    }
    if (st + R < nst1) {
      steady_stage(kSet0);
      ++st;
#pragma unroll
      for (int j = 0; j < RBW; ++j) {
        sa[0][j][0] = sa[1][j][0];
        sa[0][j][1] = sa[1][j][1];
      }
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        sb[0][u][0] = sb[1][u][0];
        sb[0][u][1] = sb[1][u][1];
      }
    }
    for (; st < nst1; ++st) drain_stage();
    store_tile(std::integral_constant<int, 32>(), std::integral_constant<int, RBW>(), acc, rb_of, n);
  };
  if (tg == 1) body1();
  else if (tg == 2) body(std::integral_constant<int, 2>());
  else body(std::integral_constant<int, 4>());
}

size_t align256(size_t v) { return (v + 255) / 256 * 256; }

}  // namespace

namespace moe {

// Whole row tiles (gate/up: I/128 tiles of 128 gate + 128 up rows; down:
// H/256 tiles) and K of both products a whole number of weight-scale blocks
// (four 128-value stages)
bool mfma_shape_ok(int H, int I) {
  return H % kTileRows == 0 && I % (kTileRows / 2) == 0 && H % 512 == 0 && I % 512 == 0;
}

// Workspace of the MFMA path after the h buffer: x terms, x scales, h terms,
// h scales, tile plan.
size_t mfma_workspace(int T, int k, int E, int H, int I) {
  const size_t R = (size_t)T * k;
  const size_t mx = (size_t)(R < (size_t)E ? R : E);
  const size_t per = (size_t)reg_rows_max(T) + 1;  // fewest rows of a GEMM expert
  const size_t pairs = R / kTileTok + (mx < R / per ? mx : R / per) + 1;
  return align256((size_t)T * 2 * H) + align256((size_t)T * 2 * (H / 32)) + align256(R * 2 * I) +
         align256(R * 2 * (I / 32)) + align256((1 + pairs) * 4 * sizeof(int32_t));
}

size_t mfma_max_pairs(int T, int k, int E) {
  const size_t R = (size_t)T * k;
  const size_t mx = (size_t)(R < (size_t)E ? R : E);
  const size_t per = (size_t)reg_rows_max(T) + 1;
  return R / kTileTok + (mx < R / per ? mx : R / per) + 1;
}

// Launches prep: the x terms, the tile plan of the experts with more than
// reg_rows_max(T) rows, and the register GEMVs' class lists l1 / l4.
hipError_t launch_mfma_prep(const uint16_t* x, int T, int k, const moe_mxfp4_weights& w, const int32_t* offsets,
                            const int32_t* active, uint8_t* ws, int32_t* l1, int32_t* l4, int lo4, int reg_max,
                            hipStream_t s) {
  const int H = w.hidden, I = w.inter;
  const size_t R = (size_t)T * k;
  uint8_t* xq = ws;
  uint8_t* xs = xq + align256((size_t)T * 2 * H);
  uint8_t* hq = xs + align256((size_t)T * 2 * (H / 32));
  uint8_t* hs = hq + align256(R * 2 * I);
  int32_t* plan = (int32_t*)(hs + align256(R * 2 * (I / 32)));
  const int64_t nq = (int64_t)T * (H / 32);
  hipLaunchKernelGGL(mfma_prep_kernel, dim3(2 + (unsigned)((nq + kThreads - 1) / kThreads)), dim3(kThreads), 0, s,
                     x, T, H, offsets, active, xq, plan, reg_max, l1, l4, lo4);
  return hipGetLastError();
}

// Launches the gate/up GEMM, which writes h of the experts with more than
// reg_rows_max(T) rows as the down GEMM's two E4M3 terms.
hipError_t launch_mfma_gateup(int T, int k, const moe_mxfp4_weights& w, const int32_t* sorted_rows, uint8_t* ws,
                              hipStream_t s) {
  const int H = w.hidden, I = w.inter;
  const size_t R = (size_t)T * k;
  uint8_t* xq = ws;
  uint8_t* xs = xq + align256((size_t)T * 2 * H);
  uint8_t* hq = xs + align256((size_t)T * 2 * (H / 32));
  uint8_t* hs = hq + align256(R * 2 * I);
  int32_t* plan = (int32_t*)(hs + align256(R * 2 * (I / 32)));
  const int m_tiles = I / (kTileRows / 2);
  const unsigned grid = (unsigned)(8 * ((mfma_max_pairs(T, k, w.num_experts) + 7) / 8) * m_tiles);
  hipLaunchKernelGGL((mfma_ffn_kernel<true>), dim3(grid), dim3(kThreads), 0, s, w, k, sorted_rows, plan, xq, xs, T,
                     (float*)nullptr, m_tiles, hq, hs, (int)R);
  return hipGetLastError();
}

// Launches the down GEMM (y_rows for the same experts) on the h terms the
// gate/up GEMM wrote.
hipError_t launch_mfma_down(int T, int k, const moe_mxfp4_weights& w, const int32_t* sorted_rows, float* y_rows,
                            uint8_t* ws, hipStream_t s) {
  const int H = w.hidden, I = w.inter;
  const size_t R = (size_t)T * k;
  uint8_t* xq = ws;
  uint8_t* xs = xq + align256((size_t)T * 2 * H);
  uint8_t* hq = xs + align256((size_t)T * 2 * (H / 32));
  uint8_t* hs = hq + align256(R * 2 * I);
  int32_t* plan = (int32_t*)(hs + align256(R * 2 * (I / 32)));
  const int m_tiles = H / kTileRows;
  const unsigned grid = (unsigned)(8 * ((mfma_max_pairs(T, k, w.num_experts) + 7) / 8) * m_tiles);
  hipLaunchKernelGGL((mfma_ffn_kernel<false>), dim3(grid), dim3(kThreads), 0, s, w, k, sorted_rows, plan, hq, hs,
                     (int)R, y_rows, m_tiles, (uint8_t*)nullptr, (uint8_t*)nullptr, 0);
  return hipGetLastError();
}

}  // namespace moe
