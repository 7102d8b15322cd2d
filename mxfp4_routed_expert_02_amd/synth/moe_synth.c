/*
 * moe_synth.c - seeded, counter-based generator of synthetic inputs for the
 * routed-expert MXFP4 layer (expert weight slabs, activations, router logits).
 *
 * This module holds no arithmetic of the layer itself: it only draws the
 * random inputs that both the HIP path and the CPU oracle consume.  It is
 * built by gcc on the host and called through ctypes.
 *
 * Generator: SplitMix64 (Steele, Lea & Flood, "Fast splittable pseudorandom
 * number generators", OOPSLA 2014) used in counter mode.  A stream is named
 * by a 64-bit key; draw i of the stream is mix(key + (i + 1) * GAMMA), so any
 * slice of any array can be regenerated on its own.
 *
 *   key(seed, tag) = mix(mix(seed + GAMMA) ^ tag)
 *   tag(array, sub, layer, expert) = array<<56 | sub<<40 | layer<<24 | expert
 *
 * Arrays (bytes are little-endian slices of the 64-bit draws):
 *   nibble bytes   byte i = byte (i % 8) of draw(i / 8): two uniform E2M1 codes
 *   scale bytes    byte i = lo + ((draw(i / 8) >> 8*(i % 8)) & mask)
 *   normals        value i = Box-Muller(draw(i)) in double, rounded to float:
 *                  u1 = ((z >> 40) + 1) * 2^-24 in (0, 1],
 *                  u2 = ((z >> 16) & 0xFFFFFF) * 2^-24 in [0, 1),
 *                  n  = sqrt(-2 ln u1) * cos(2 pi u2)
 *   bf16 normals   round-to-nearest-even of the float normal
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <string.h>

#define GAMMA 0x9e3779b97f4a7c15ULL

static inline uint64_t mix64(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xbf58476d1ce4e5b9ULL;
  z = (z ^ (z >> 27)) * 0x94d049bb133111ebULL;
  return z ^ (z >> 31);
}

static inline uint64_t draw(uint64_t key, uint64_t i) { return mix64(key + (i + 1) * GAMMA); }

uint64_t synth_tag(uint64_t array, uint64_t sub, uint64_t layer, uint64_t expert) {
  return (array << 56) | ((sub & 0xFFFF) << 40) | ((layer & 0xFFFF) << 24) | (expert & 0xFFFFFF);
}

uint64_t synth_key(uint64_t seed, uint64_t tag) { return mix64(mix64(seed + GAMMA) ^ tag); }

uint64_t synth_draw(uint64_t key, uint64_t i) { return draw(key, i); }

/* bytes [start, start + n) of the uniform byte stream */
void synth_bytes(uint64_t key, uint64_t start, uint64_t n, uint8_t* out) {
  uint64_t i = 0;
  while (i < n) {
    uint64_t idx = start + i;
    uint64_t z = draw(key, idx >> 3);
    unsigned b = (unsigned)(idx & 7);
    if (b == 0 && n - i >= 8) {
      memcpy(out + i, &z, 8); /* little-endian host */
      i += 8;
      continue;
    }
    out[i] = (uint8_t)(z >> (8 * b));
    ++i;
  }
}

/* byte i = lo + ((byte i of the uniform stream) & mask) */
void synth_small_bytes(uint64_t key, uint64_t start, uint64_t n, uint8_t lo, uint8_t mask, uint8_t* out) {
  synth_bytes(key, start, n, out);
  for (uint64_t i = 0; i < n; ++i) out[i] = (uint8_t)(lo + (out[i] & mask));
}

static inline double box_muller(uint64_t z) {
  double u1 = (double)((z >> 40) + 1) * (1.0 / 16777216.0);
  double u2 = (double)((z >> 16) & 0xFFFFFFULL) * (1.0 / 16777216.0);
  return sqrt(-2.0 * log(u1)) * cos(6.283185307179586476925 * u2);
}

void synth_normal_f32(uint64_t key, uint64_t start, uint64_t n, float stddev, float* out) {
  for (uint64_t i = 0; i < n; ++i) out[i] = (float)(stddev * box_muller(draw(key, start + i)));
}

static inline uint16_t f32_to_bf16_rne(float f) {
  uint32_t u;
  memcpy(&u, &f, 4);
  if ((u & 0x7F800000u) == 0x7F800000u) return (uint16_t)((u >> 16) | ((u & 0xFFFFu) ? 0x40u : 0u));
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

void synth_normal_bf16(uint64_t key, uint64_t start, uint64_t n, uint16_t* out) {
  for (uint64_t i = 0; i < n; ++i) out[i] = f32_to_bf16_rne((float)box_muller(draw(key, start + i)));
}

/* ---- expert slabs --------------------------------------------------------
 * Slab of one (layer, expert): gate_q | gate_s | up_q | up_s | down_q | down_s
 *   gate_q, up_q : [I][H/2] bytes   gate_s, up_s : [I][H/32] bytes
 *   down_q       : [H][I/2] bytes   down_s       : [H][I/32] bytes
 * Arrays 1..6 are drawn from their own streams (tag sub field = pool id).  Scale bytes are
 * 121 + (2 uniform bits): an exponent uniform over {-6, -5, -4, -3}. */
enum { ARR_GATE_Q = 1, ARR_GATE_S = 2, ARR_UP_Q = 3, ARR_UP_S = 4, ARR_DOWN_Q = 5, ARR_DOWN_S = 6 };

uint64_t synth_slab_bytes(int64_t H, int64_t I) { return (uint64_t)(3 * (I * H / 2 + I * H / 32)); }

static void fill_slab(uint64_t seed, int pool, int layer, int expert, int64_t H, int64_t I, uint8_t* slab) {
  uint64_t qb = (uint64_t)(I * H / 2), sb = (uint64_t)(I * H / 32);
  uint8_t* p = slab;
  synth_bytes(synth_key(seed, synth_tag(ARR_GATE_Q, pool, layer, expert)), 0, qb, p); p += qb;
  synth_small_bytes(synth_key(seed, synth_tag(ARR_GATE_S, pool, layer, expert)), 0, sb, 121, 3, p); p += sb;
  synth_bytes(synth_key(seed, synth_tag(ARR_UP_Q, pool, layer, expert)), 0, qb, p); p += qb;
  synth_small_bytes(synth_key(seed, synth_tag(ARR_UP_S, pool, layer, expert)), 0, sb, 121, 3, p); p += sb;
  synth_bytes(synth_key(seed, synth_tag(ARR_DOWN_Q, pool, layer, expert)), 0, qb, p); p += qb;
  synth_small_bytes(synth_key(seed, synth_tag(ARR_DOWN_S, pool, layer, expert)), 0, sb, 121, 3, p);
}

typedef struct {
  uint64_t seed;
  int pool, layer, e0, n, H, I, step, first;
  uint64_t stride;
  uint8_t* dst;
} slab_job;

static void* slab_worker(void* arg) {
  slab_job* j = (slab_job*)arg;
  for (int e = j->first; e < j->n; e += j->step)
    fill_slab(j->seed, j->pool, j->layer, j->e0 + e, j->H, j->I, j->dst + (uint64_t)e * j->stride);
  return 0;
}

/* Fills n consecutive expert slabs (experts e0 .. e0+n-1 of `layer` in weight
 * pool `pool`) into dst, slab e at dst + e*stride, using up to nthreads host
 * threads.  The bytes do not depend on nthreads. */
int synth_expert_slabs(uint64_t seed, int pool, int layer, int e0, int n, int H, int I, uint8_t* dst,
                       uint64_t stride, int nthreads) {
  if (nthreads < 1) nthreads = 1;
  if (nthreads > 64) nthreads = 64;
  if (nthreads > n) nthreads = n > 0 ? n : 1;
  pthread_t th[64];
  slab_job jobs[64];
  for (int t = 0; t < nthreads; ++t) {
    jobs[t] = (slab_job){seed, pool, layer, e0, n, H, I, nthreads, t, stride, dst};
    if (t > 0 && pthread_create(&th[t], 0, slab_worker, &jobs[t]) != 0) return -1;
  }
  slab_worker(&jobs[0]);
  for (int t = 1; t < nthreads; ++t) pthread_join(th[t], 0);
  return 0;
}
