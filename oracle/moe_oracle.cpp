// moe_oracle.cpp - plain CPU oracle of the routed-expert MXFP4 layer.
//
// TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the bench's
// CPU-baseline leg load this library; the product path never does.  It shares
// no code with the HIP library (no headers, tables or helpers).
//
// What it computes (the layer the pages describe: the Kimi K3 routed experts,
// 16 picked per layer per token by the router, page "hn.213312.xyz/article/
// 49090233", section on how it works; weights used at their published MXFP4
// precision, page "agentlenshq.com ... Deltafin", section on what Deltafin
// does; a fused MXFP4 dequant + matmul computes them, page 1, technical
// highlights; experts processed expert-major, every expert read once per
// layer, page 2, section on what the author still needs help with):
//
//   route    ids[t] = the k largest logits of token t, larger value first,
//            equal values ordered by lower expert id; w[t] = softmax over the
//            k selected logits (fp32 expf, sum in rank order)
//   group    counting sort of the flat rows r = t*k + j by expert id; rows of
//            one expert in ascending r; row_pos = inverse permutation;
//            active = experts with rows, ascending
//   dequant  W[n][c] = E2M1[nibble] * 2^(scale - 127); nibble 2m in the low
//            half of byte m; one E8M0 scale byte per 32 values along K
//   gate/up  g_i = sum_c x_c Wg[i][c], u_i likewise (fp32, c ascending);
//            h_i = g_i / (1 + exp(-g_i)) * u_i
//   down     y_n = sum_i h_i Wd[n][i] (fp32, i ascending)
//   combine  out[t] = sum_j w[t][j] y(t, j) (fp32, j ascending)
//   rescale  x_next = bf16_rne(y / sqrt(mean(y^2) + eps)) between stacked layers
//   router   logits[t][e] = sum_c x[t][c] Wr[e][c] (fp32 weights, fp32, c
//            ascending): the projection before the path that feeds route
//            (page 1, section on how it works: the router picks the experts)
//
// Accumulation is fp32 in the stated order; the build uses -ffp-contract=off
// so no product is fused into an add.  A double-accumulation variant of the
// per-token layer serves the error-budget measurement.
#include <algorithm>
#include <cmath>
#include <cstdint>
#include <cstring>
#include <thread>
#include <vector>

namespace {

// OCP MX v1.0 E2M1 element values, codes 0..15 (sign bit = bit 3).
const float kE2M1[16] = {0.0f,  0.5f,  1.0f,  1.5f,  2.0f,  3.0f,  4.0f,  6.0f,
                         -0.0f, -0.5f, -1.0f, -1.5f, -2.0f, -3.0f, -4.0f, -6.0f};

struct Weights {  // one layer's expert pool, host memory
  const uint8_t *gate_q, *gate_s, *up_q, *up_s, *down_q, *down_s;
  int64_t expert_stride;  // bytes between consecutive experts in every array
  int32_t num_experts, hidden, inter;
};

inline float bf16_to_f32(uint16_t b) {
  uint32_t u = (uint32_t)b << 16;
  float f;
  std::memcpy(&f, &u, 4);
  return f;
}

inline uint16_t f32_to_bf16_rne(float f) {
  uint32_t u;
  std::memcpy(&u, &f, 4);
  if ((u & 0x7F800000u) == 0x7F800000u) return (uint16_t)((u >> 16) | ((u & 0xFFFFu) ? 0x40u : 0u));
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// One element of an MXFP4 matrix stored as q[N][K/2], s[N][K/32].
inline float dequant(const uint8_t* q, const uint8_t* s, int64_t K, int64_t n, int64_t c) {
  uint8_t byte = q[n * (K / 2) + c / 2];
  int nib = (c % 2 == 0) ? (byte & 0xF) : (byte >> 4);
  int sc = s[n * (K / 32) + c / 32];
  return kE2M1[nib] * std::ldexp(1.0f, sc - 127);
}

template <class Acc>
void expert_ffn_row(const Weights& w, int e, const float* x /*[H]*/, float* h /*[I] scratch*/, float* y /*[H]*/) {
  const int64_t H = w.hidden, I = w.inter;
  const uint8_t* gq = w.gate_q + e * w.expert_stride;
  const uint8_t* gs = w.gate_s + e * w.expert_stride;
  const uint8_t* uq = w.up_q + e * w.expert_stride;
  const uint8_t* us = w.up_s + e * w.expert_stride;
  const uint8_t* dq = w.down_q + e * w.expert_stride;
  const uint8_t* ds = w.down_s + e * w.expert_stride;
  for (int64_t i = 0; i < I; ++i) {
    Acc g = 0, u = 0;
    for (int64_t c = 0; c < H; ++c) {
      g += (Acc)x[c] * (Acc)dequant(gq, gs, H, i, c);
      u += (Acc)x[c] * (Acc)dequant(uq, us, H, i, c);
    }
    h[i] = (float)(g / ((Acc)1 + std::exp(-g)) * u);
  }
  for (int64_t n = 0; n < H; ++n) {
    Acc acc = 0;
    for (int64_t i = 0; i < I; ++i) acc += (Acc)h[i] * (Acc)dequant(dq, ds, I, n, i);
    y[n] = (float)acc;
  }
}

template <class F>
void parallel_for(int64_t n, int nthreads, F f) {
  if (nthreads <= 1 || n <= 1) {
    for (int64_t i = 0; i < n; ++i) f(i);
    return;
  }
  if (nthreads > n) nthreads = (int)n;
  std::vector<std::thread> th;
  for (int t = 0; t < nthreads; ++t)
    th.emplace_back([=] {
      for (int64_t i = t; i < n; i += nthreads) f(i);
    });
  for (auto& x : th) x.join();
}

bool better(float a, int ia, float b, int ib) { return a > b || (a == b && ia < ib); }

}  // namespace

extern "C" {

typedef Weights oracle_weights;

float oracle_e2m1_value(int code) { return kE2M1[code & 0xF]; }

float oracle_dequant(const uint8_t* q, const uint8_t* s, int64_t K, int64_t n, int64_t c) {
  return dequant(q, s, K, n, c);
}

// Top-k by k passes of an explicit arg-max over the experts not yet taken.
int oracle_route_topk(const float* logits, int32_t T, int32_t E, int32_t k, int32_t* ids, float* w) {
  if (T < 0 || E < 1 || k < 1 || k > E) return 1;
  std::vector<char> taken(E);
  std::vector<float> v(k);
  for (int t = 0; t < T; ++t) {
    const float* l = logits + (int64_t)t * E;
    std::fill(taken.begin(), taken.end(), 0);
    for (int j = 0; j < k; ++j) {
      int best = -1;
      for (int e = 0; e < E; ++e) {
        if (!std::isfinite(l[e])) return 2;
        if (taken[e]) continue;
        if (best < 0 || better(l[e], e, l[best], best)) best = e;
      }
      taken[best] = 1;
      ids[(int64_t)t * k + j] = best;
      v[j] = l[best];
    }
    const float m = v[0];
    float S = 0.0f;
    std::vector<float> ex(k);
    for (int j = 0; j < k; ++j) {
      ex[j] = std::exp(v[j] - m);
      S += ex[j];
    }
    for (int j = 0; j < k; ++j) w[(int64_t)t * k + j] = ex[j] / S;
  }
  return 0;
}

// Counting sort of flat rows by expert id (stable in the flat index).
int oracle_group_rows(const int32_t* ids, int32_t T, int32_t k, int32_t E, int32_t* expert_offsets,
                      int32_t* sorted_rows, int32_t* row_pos, int32_t* active) {
  const int64_t R = (int64_t)T * k;
  std::vector<int32_t> count(E, 0);
  for (int64_t r = 0; r < R; ++r) {
    if (ids[r] < 0 || ids[r] >= E) return 1;
    count[ids[r]]++;
  }
  expert_offsets[0] = 0;
  for (int e = 0; e < E; ++e) expert_offsets[e + 1] = expert_offsets[e] + count[e];
  std::vector<int32_t> fill(expert_offsets, expert_offsets + E);
  for (int64_t r = 0; r < R; ++r) {
    int32_t p = fill[ids[r]]++;
    sorted_rows[p] = (int32_t)r;
    row_pos[r] = p;
  }
  int na = 0;
  for (int e = 0; e < E; ++e)
    if (count[e] > 0) active[1 + na++] = e;
  active[0] = na;
  return 0;
}

// Gate/up + SiLU*mul for every routed row, in expert-major (sorted) order:
// h[p][i] for p = position in sorted_rows.
int oracle_gateup(const uint16_t* x, int32_t T, int32_t k, const oracle_weights* w, const int32_t* expert_offsets,
                  const int32_t* sorted_rows, const int32_t* active, float* h, int32_t nthreads) {
  const int64_t H = w->hidden, I = w->inter;
  (void)T;
  std::vector<int64_t> work;  // (position) list over active experts
  for (int a = 0; a < active[0]; ++a) {
    int e = active[1 + a];
    for (int32_t p = expert_offsets[e]; p < expert_offsets[e + 1]; ++p) work.push_back(p);
  }
  std::vector<int32_t> expert_of(work.size());
  for (size_t i = 0; i < work.size(); ++i) {
    int32_t p = (int32_t)work[i];
    int e = 0;
    while (expert_offsets[e + 1] <= p) ++e;
    expert_of[i] = e;
  }
  parallel_for((int64_t)work.size(), nthreads, [&](int64_t wi) {
    const int64_t p = work[wi];
    const int e = expert_of[wi];
    const int64_t t = sorted_rows[p] / k;
    std::vector<float> xf(H);
    for (int64_t c = 0; c < H; ++c) xf[c] = bf16_to_f32(x[t * H + c]);
    const uint8_t* gq = w->gate_q + e * w->expert_stride;
    const uint8_t* gs = w->gate_s + e * w->expert_stride;
    const uint8_t* uq = w->up_q + e * w->expert_stride;
    const uint8_t* us = w->up_s + e * w->expert_stride;
    for (int64_t i = 0; i < I; ++i) {
      float g = 0.0f, u = 0.0f;
      for (int64_t c = 0; c < H; ++c) {
        g += xf[c] * dequant(gq, gs, H, i, c);
        u += xf[c] * dequant(uq, us, H, i, c);
      }
      h[p * I + i] = g / (1.0f + std::exp(-g)) * u;
    }
  });
  return 0;
}

// Down projection for every routed row: y_rows[p][n] = sum_i h[p][i] Wd[n][i].
int oracle_down(const float* h, const oracle_weights* w, const int32_t* expert_offsets, const int32_t* active,
                float* y_rows, int32_t nthreads) {
  const int64_t H = w->hidden, I = w->inter;
  std::vector<std::pair<int32_t, int32_t>> work;  // (position, expert)
  for (int a = 0; a < active[0]; ++a) {
    int e = active[1 + a];
    for (int32_t p = expert_offsets[e]; p < expert_offsets[e + 1]; ++p) work.push_back({p, e});
  }
  parallel_for((int64_t)work.size(), nthreads, [&](int64_t wi) {
    const int64_t p = work[wi].first;
    const int e = work[wi].second;
    const uint8_t* dq = w->down_q + e * w->expert_stride;
    const uint8_t* ds = w->down_s + e * w->expert_stride;
    for (int64_t n = 0; n < H; ++n) {
      float acc = 0.0f;
      for (int64_t i = 0; i < I; ++i) acc += h[p * I + i] * dequant(dq, ds, I, n, i);
      y_rows[p * H + n] = acc;
    }
  });
  return 0;
}

int oracle_combine(const float* y_rows, const float* w, const int32_t* row_pos, int32_t T, int32_t k, int32_t H,
                   float* out) {
  for (int64_t t = 0; t < T; ++t)
    for (int64_t n = 0; n < H; ++n) {
      float acc = 0.0f;
      for (int j = 0; j < k; ++j) acc += w[t * k + j] * y_rows[(int64_t)row_pos[t * k + j] * H + n];
      out[t * H + n] = acc;
    }
  return 0;
}

// x_next = bf16_rne(y * (1 / sqrt(mean(y^2) + eps))), per token; sum of squares
// in fp32, n ascending.
int oracle_rms_rescale_bf16(const float* y, int32_t T, int32_t H, float eps, uint16_t* x_next) {
  for (int64_t t = 0; t < T; ++t) {
    float ss = 0.0f;
    for (int64_t n = 0; n < H; ++n) ss += y[t * H + n] * y[t * H + n];
    const float r = 1.0f / std::sqrt(ss / (float)H + eps);
    for (int64_t n = 0; n < H; ++n) x_next[t * H + n] = f32_to_bf16_rne(y[t * H + n] * r);
  }
  return 0;
}

// One token's layer output straight from its routed experts (no grouping):
// out = sum_j w[j] * FFN_{ids[j]}(x), j ascending.  Same per-element order
// as the grouped path, so the two agree bit for bit.
int oracle_token_layer(const uint16_t* x_t, const int32_t* ids_t, const float* w_t, int32_t k,
                       const oracle_weights* w, float* out_t) {
  const int64_t H = w->hidden, I = w->inter;
  std::vector<float> xf(H), h(I), y((size_t)k * H);
  for (int64_t c = 0; c < H; ++c) xf[c] = bf16_to_f32(x_t[c]);
  for (int j = 0; j < k; ++j) expert_ffn_row<float>(*w, ids_t[j], xf.data(), h.data(), y.data() + (int64_t)j * H);
  for (int64_t n = 0; n < H; ++n) {
    float acc = 0.0f;
    for (int j = 0; j < k; ++j) acc += w_t[j] * y[(int64_t)j * H + n];
    out_t[n] = acc;
  }
  return 0;
}

// Same as oracle_token_layer but every dot product and the combine are
// accumulated in double (the error-budget reference).
int oracle_token_layer_f64(const uint16_t* x_t, const int32_t* ids_t, const float* w_t, int32_t k,
                           const oracle_weights* w, double* out_t) {
  const int64_t H = w->hidden, I = w->inter;
  std::vector<float> xf(H), h(I), y((size_t)k * H);
  for (int64_t c = 0; c < H; ++c) xf[c] = bf16_to_f32(x_t[c]);
  for (int j = 0; j < k; ++j)
    expert_ffn_row<double>(*w, ids_t[j], xf.data(), h.data(), y.data() + (int64_t)j * H);
  for (int64_t n = 0; n < H; ++n) {
    double acc = 0.0;
    for (int j = 0; j < k; ++j) acc += (double)w_t[j] * (double)y[(int64_t)j * H + n];
    out_t[n] = acc;
  }
  return 0;
}

// Brute force for one token: evaluate every expert of the pool densely, pick
// the top k by a full stable sort on (value desc, id asc), weight by the
// softmax of the picked logits and sum in rank order.
int oracle_dense_token(const uint16_t* x_t, const float* logits_t, int32_t E, int32_t k, const oracle_weights* w,
                       float* out_t) {
  const int64_t H = w->hidden, I = w->inter;
  std::vector<float> xf(H), h(I), yall((size_t)E * H);
  for (int64_t c = 0; c < H; ++c) xf[c] = bf16_to_f32(x_t[c]);
  for (int e = 0; e < E; ++e) expert_ffn_row<float>(*w, e, xf.data(), h.data(), yall.data() + (int64_t)e * H);
  std::vector<int> order(E);
  for (int e = 0; e < E; ++e) order[e] = e;
  std::stable_sort(order.begin(), order.end(), [&](int a, int b) { return logits_t[a] > logits_t[b]; });
  std::vector<float> ex(k);
  float S = 0.0f;
  for (int j = 0; j < k; ++j) {
    ex[j] = std::exp(logits_t[order[j]] - logits_t[order[0]]);
    S += ex[j];
  }
  for (int64_t n = 0; n < H; ++n) {
    float acc = 0.0f;
    for (int j = 0; j < k; ++j) acc += (ex[j] / S) * yall[(int64_t)order[j] * H + n];
    out_t[n] = acc;
  }
  return 0;
}

// Router projection: logits[t][e] = sum_{c=0}^{H-1} x[t][c] * wr[e][c], x bf16
// (exact in fp32), wr fp32 [E][H], fp32 accumulation with c ascending.
// Tokens are spread over nthreads host threads (each logit is one thread's
// fixed-order sum, so the result does not depend on nthreads).
int oracle_router_logits(const uint16_t* x, int32_t T, int32_t H, const float* wr, int32_t E, float* logits,
                         int32_t nthreads) {
  parallel_for(T, nthreads, [&](int64_t t) {
    std::vector<float> xf(H);
    for (int64_t c = 0; c < H; ++c) xf[c] = bf16_to_f32(x[t * H + c]);
    for (int64_t e = 0; e < E; ++e) {
      float acc = 0.0f;
      for (int64_t c = 0; c < H; ++c) acc += xf[c] * wr[e * H + c];
      logits[t * E + e] = acc;
    }
  });
  return 0;
}

}  // extern "C"
