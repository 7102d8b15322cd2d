// synth_gpu.hip - device-side twin of the expert-slab generator in
// moe_synth.c: the same counter-mode SplitMix64 streams, written straight
// into device memory, so pools of tens to hundreds of GB (the 92-layer
// stack) are filled at memory speed instead of through the host.
//
// Like moe_synth.c it draws inputs only and holds none of the layer's
// arithmetic.  Byte for byte it must equal synth_expert_slabs() of
// moe_synth.c; a GPU test compares the two.  It also holds a plain
// streaming-read probe that the benchmark times as the box's achievable
// read bandwidth.
//
//   key(seed, tag) = mix(mix(seed + GAMMA) ^ tag)
//   tag(array, sub, layer, expert) = array<<56 | sub<<40 | layer<<24 | expert
//   word w of a stream = mix(key + (w + 1) * GAMMA), bytes little-endian
//   nibble arrays: the bytes of the words; scale arrays: 121 + (byte & 3)
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

constexpr uint64_t kGamma = 0x9e3779b97f4a7c15ULL;

__device__ __forceinline__ uint64_t mix64(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xbf58476d1ce4e5b9ULL;
  z = (z ^ (z >> 27)) * 0x94d049bb133111ebULL;
  return z ^ (z >> 31);
}

__device__ __forceinline__ uint64_t stream_key(uint64_t seed, uint64_t array, uint64_t sub, uint64_t layer,
                                               uint64_t expert) {
  const uint64_t tag = (array << 56) | ((sub & 0xFFFF) << 40) | ((layer & 0xFFFF) << 24) | (expert & 0xFFFFFF);
  return mix64(mix64(seed + kGamma) ^ tag);
}

// Slab of one expert: gate_q | gate_s | up_q | up_s | down_q | down_s with
// q arrays of qb bytes and s arrays of sb bytes (arrays 1..6); every array
// is a whole number of 8-byte words when H and I are multiples of 32.
__global__ void slab_kernel(uint64_t seed, int pool, int layer, int e0, uint64_t qw, uint64_t sw,
                            uint64_t* __restrict__ dst, uint64_t stride_words) {
  const uint64_t w = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const uint64_t slab_words = 3 * (qw + sw);
  if (w >= slab_words) return;
  const int e = e0 + (int)blockIdx.y;
  const uint64_t pair = w / (qw + sw), r = w - pair * (qw + sw);
  const bool is_scale = r >= qw;
  const uint64_t array = 1 + 2 * pair + (is_scale ? 1 : 0);
  const uint64_t idx = is_scale ? r - qw : r;
  uint64_t z = mix64(stream_key(seed, array, (uint64_t)pool, (uint64_t)layer, (uint64_t)e) + (idx + 1) * kGamma);
  if (is_scale) z = (z & 0x0303030303030303ULL) + 0x7979797979797979ULL;  // 121 + (byte & 3), no carries
  dst[(uint64_t)blockIdx.y * stride_words + w] = z;
}

// Streaming-read probe, measurement context for the bandwidth-bound kernels:
// every 16-byte word of the buffer is read once by grid-stride loads (four
// per thread in flight) with the non-temporal cache policy (the fastest
// plain stream on this GPU), each thread writing the XOR of what it read so
// the loads are live.  It draws and computes nothing of the layer.
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
__global__ __launch_bounds__(256) void stream_read_kernel(const u32x4_t* __restrict__ src, uint64_t n16,
                                                          uint32_t* __restrict__ out) {
  const uint64_t step = (uint64_t)gridDim.x * 256 * 4;
  uint32_t acc = 0u;
  for (uint64_t i = (uint64_t)blockIdx.x * 256 * 4 + threadIdx.x; i < n16; i += step) {
    u32x4_t v[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      v[u] = u32x4_t{0u, 0u, 0u, 0u};
      if (i + 256u * u < n16) v[u] = __builtin_nontemporal_load(src + i + 256u * u);
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) acc ^= v[u][0] ^ v[u][1] ^ v[u][2] ^ v[u][3];
  }
  out[(uint64_t)blockIdx.x * 256 + threadIdx.x] = acc;
}

}  // namespace

extern "C" {

// Reads `bytes` (a multiple of 16) from 16-byte aligned device memory `src`
// with `blocks` blocks of 256 threads; `out` holds blocks * 256 words.
// Returns 0, -1 for arguments it cannot take, or the HIP error code.
__attribute__((visibility("default"))) int synth_stream_read(const void* src, uint64_t bytes, void* out, int blocks,
                                                             void* stream) {
  if (!src || !out || blocks < 1 || (bytes & 15) || ((uintptr_t)src & 15)) return -1;
  hipLaunchKernelGGL(stream_read_kernel, dim3(blocks), dim3(256), 0, (hipStream_t)stream, (const u32x4_t*)src,
                     bytes / 16, (uint32_t*)out);
  const hipError_t err = hipGetLastError();
  return err == hipSuccess ? 0 : (int)err;
}

// Fills experts e0 .. e0+n-1 of (pool, layer) into device memory, slab i at
// dst + i*stride bytes (stride and dst 8-byte aligned), on `stream`.
// Returns 0, or -1 for arguments it cannot take, or the HIP error code.
__attribute__((visibility("default"))) int synth_expert_slabs_gpu(uint64_t seed, int pool, int layer, int e0, int n,
                                                                  int H, int I, void* dst, uint64_t stride,
                                                                  void* stream) {
  if (n <= 0) return 0;
  if (H <= 0 || I <= 0 || H % 32 || I % 32 || n > 65535 || ((uintptr_t)dst & 7) || (stride & 7)) return -1;
  const uint64_t qw = (uint64_t)I * H / 2 / 8, sw = (uint64_t)I * H / 32 / 8;
  const uint64_t words = 3 * (qw + sw);
  const dim3 grid((unsigned)((words + 255) / 256), (unsigned)n);
  hipLaunchKernelGGL(slab_kernel, grid, dim3(256), 0, (hipStream_t)stream, seed, pool, layer, e0, qw, sw,
                     (uint64_t*)dst, stride / 8);
  const hipError_t err = hipGetLastError();
  return err == hipSuccess ? 0 : (int)err;
}
}
