/*
 * moe_mxfp4.h - C ABI of the MI355X (gfx950) routed-expert MXFP4 layer.
 *
 * The layer is the routed-expert half of one Kimi K3 MoE layer as the pages
 * describe it: for every token the router picks 16 of the layer's experts
 * (page "hn.213312.xyz/article/49090233", section on how it works), the
 * experts keep their published MXFP4 weights (page "agentlenshq.com ...
 * Deltafin", section on what Deltafin does) and a fused MXFP4 dequant +
 * matmul evaluates them (page 1, technical highlights).  Rows are processed
 * expert-major so that each expert's weights are read once per layer (page 2,
 * section on what the author still needs help with).
 *
 * One layer is four calls on one stream:
 *   moe_route_topk -> moe_group_rows -> moe_expert_ffn_mxfp4 -> moe_combine
 *
 * Conventions shared by every call
 *   - Pointers are DEVICE pointers unless a comment says "host".  The caller
 *     owns every buffer; the library never allocates, frees or synchronizes.
 *   - Every call only enqueues work on `stream` (NULL = the device's default
 *     stream) and returns at once.  Outputs are valid once the stream reaches
 *     that point.  There is no device-to-host copy anywhere in the layer.
 *   - Arguments are validated before anything is enqueued.  A call that
 *     returns anything but MOE_OK has enqueued nothing and written nothing.
 *   - T = 0 is a valid empty batch; arrays whose size is a multiple of T may
 *     then be NULL (moe_group_rows still writes expert_offsets and active).
 *   - The current HIP device must be a gfx950 GPU (MOE_ERR_UNSUPPORTED_DEVICE
 *     otherwise).  The library keeps no other state (apart from the static
 *     scratch of moe_decode_layer_mxfp4_noalloc) and is re-entrant.
 *   - Preconditions not checked on the device: logits are finite, the ids
 *     handed to moe_group_rows lie in [0, E), and every dequantized weight
 *     E2M1 * 2^(s-127) is a finite fp32 value (always so for scale bytes
 *     up to 252; at 253 and 254 codes of magnitude 2 or more exceed the
 *     fp32 range, and 0xFF is NaN in E8M0).
 *   - Results are deterministic: the same inputs give the same bits on every
 *     run (no atomics decide any order or any sum).
 *
 * MXFP4 weights (OCP MX v1.0): a matrix W[N][K] (K = reduction dimension) is
 *   q[N][K/2] bytes: element 2m of a row in the low nibble of byte m, element
 *                    2m+1 in the high nibble; nibble = E2M1 code
 *                    {0,.5,1,1.5,2,3,4,6} with bit 3 the sign
 *   s[N][K/32] bytes: E8M0 scale of each 32 consecutive values along K,
 *                    value 2^(s-127)
 * An expert holds Wg[I][H] and Wu[I][H] (gate, up; K = H) and Wd[H][I]
 * (down; K = I).  The synthetic pools keep one expert per contiguous slab
 * gate_q | gate_s | up_q | up_s | down_q | down_s (17,547,264 bytes at
 * H = 7168, I = 1536: one "file" per (layer, expert) as the pages put it).
 */
#ifndef MOE_MXFP4_H
#define MOE_MXFP4_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#if defined(__GNUC__) || defined(__clang__)
#define MOE_API __attribute__((visibility("default")))
#else
#define MOE_API
#endif

/* Same type as hipStream_t. */
typedef struct ihipStream_t* moe_stream_t;

typedef enum {
  MOE_OK = 0,
  MOE_ERR_INVALID_ARG = 1,         /* a null/misaligned pointer or a size out of range */
  MOE_ERR_UNSUPPORTED_DEVICE = 2,  /* the current device is not gfx950 */
  MOE_ERR_WORKSPACE_TOO_SMALL = 3, /* workspace_bytes < moe_workspace_bytes(...) */
  MOE_ERR_HIP = 4,                 /* the HIP runtime refused a launch */
  MOE_ERR_SCRATCH_TOO_SMALL = 5    /* moe_decode_layer_mxfp4_noalloc: the shape needs more than
                                      MOE_NOALLOC_SCRATCH_BYTES of scratch */
} moe_status;

#define MOE_MAX_EXPERTS 4096 /* E */
#define MOE_MAX_TOPK 32      /* k */
#define MOE_MAX_DIM 16384    /* H and I */

/* One layer's resident expert pool.  Each base pointer addresses expert 0's
 * array; expert e's array starts expert_stride bytes after expert e-1's.
 * The struct itself is host memory read during the call; the arrays are
 * device memory.  gate_q/up_q/down_q and expert_stride must be multiples of
 * 16 bytes, gate_s/up_s/down_s multiples of 4; hidden and inter multiples
 * of 32. */
typedef struct {
  const uint8_t* gate_q; /* [E][I][H/2] */
  const uint8_t* gate_s; /* [E][I][H/32] */
  const uint8_t* up_q;   /* [E][I][H/2] */
  const uint8_t* up_s;   /* [E][I][H/32] */
  const uint8_t* down_q; /* [E][H][I/2] */
  const uint8_t* down_s; /* [E][H][I/32] */
  int64_t expert_stride; /* bytes between consecutive experts */
  int32_t num_experts;   /* E */
  int32_t hidden;        /* H */
  int32_t inter;         /* I */
} moe_mxfp4_weights;

/*
 * moe_route_topk - the router's pick of k experts per token (page
 * "hn.213312.xyz/article/49090233", section on how it works: 16 routed
 * experts per layer per token; all 16 are kept, page "uuaihub.com ...", the
 * performance section).
 *   logits        [T][E] fp32 router logits (row-major)
 *   topk_ids      [T][k] int32 out: the k largest logits of each token in
 *                 rank order: larger value first, equal values (+0 == -0)
 *                 ordered by lower expert id
 *   topk_weights  [T][k] fp32 out: softmax over the k selected logits,
 *                 w_j = exp(l_j - l_0) / sum_i exp(l_i - l_0)
 * T >= 0 (T = 0 does nothing), 1 <= E <= MOE_MAX_EXPERTS,
 * 1 <= k <= min(E, MOE_MAX_TOPK).
 */
MOE_API moe_status moe_route_topk(const float* logits, int32_t T, int32_t E, int32_t k, int32_t* topk_ids,
                          float* topk_weights, moe_stream_t stream);

/*
 * moe_group_rows - expert-major grouping of the routed rows (page
 * "agentlenshq.com ... Deltafin", section on what the author still needs
 * help with: read each expert once per layer and process all its routed rows
 * in one pass).  Row r = t*k + j is token t's j-th pick.
 *   topk_ids        [T*k] int32, each in [0, E)
 *   expert_offsets  [E+1] int32 out: exclusive prefix sum of rows per expert
 *   sorted_rows     [T*k] int32 out: rows grouped by expert, each group in
 *                   ascending r (expert e owns positions
 *                   expert_offsets[e] .. expert_offsets[e+1]-1)
 *   row_pos         [T*k] int32 out: inverse, sorted_rows[row_pos[r]] == r
 *   active          [E+1] int32 out: active[0] = number of experts with at
 *                   least one row, active[1..] = those experts ascending
 *                   (entries past the count are left unchanged)
 *   workspace       device scratch of at least
 *                   moe_workspace_bytes(T, k, E, H, I) bytes (any H, I),
 *                   16-byte aligned (more than 512 rows use it; fewer may
 *                   pass NULL)
 * Same ranges as moe_route_topk (k may exceed E here; ids may repeat).
 */
MOE_API moe_status moe_group_rows(const int32_t* topk_ids, int32_t T, int32_t k, int32_t E, int32_t* expert_offsets,
                          int32_t* sorted_rows, int32_t* row_pos, int32_t* active, void* workspace,
                          size_t workspace_bytes, moe_stream_t stream);

/*
 * moe_expert_ffn_mxfp4 - fused MXFP4 dequant + SwiGLU expert FFN for every
 * routed row (page "hn.213312.xyz/article/49090233", technical highlights:
 * fused MXFP4 dequant and matmul; page "uuaihub.com ...", section on how it
 * is done: expert math at native MXFP4 precision).  For the row at sorted
 * position p, owned by expert e, with token t = sorted_rows[p] / k:
 *   g = Wg_e x_t,  u = Wu_e x_t,  h = g * sigmoid(g) * u   (h kept fp32)
 *   y_rows[p] = Wd_e h
 *   x              [T][H] bf16 activations (raw bits), 16-byte aligned
 *   w              host struct describing the device expert pool
 *   expert_offsets, sorted_rows, active: as written by moe_group_rows
 *   y_rows         [T*k][H] fp32 out, expert-major (sorted) order,
 *                  16-byte aligned
 *   workspace      device scratch, moe_workspace_bytes(T, k, E, H, I) bytes
 * Accumulation is fp32; the result agrees with the exact dequantized
 * product to well within rel-L2 2e-3.  In batches of up to 16 tokens every
 * token's rows are bitwise the same as when the token runs alone (a
 * speculative-verify batch reproduces the decode results).  In larger
 * batches experts with more than one row take the grouped MFMA GEMM, whose
 * activations travel as block-scaled terms per 32-value block (x in two
 * E2M3 terms, h in two E4M3 terms: same bar, different rounding).
 */
MOE_API moe_status moe_expert_ffn_mxfp4(const uint16_t* x, int32_t T, int32_t k, const moe_mxfp4_weights* w,
                                const int32_t* expert_offsets, const int32_t* sorted_rows, const int32_t* active,
                                float* y_rows, void* workspace, size_t workspace_bytes, moe_stream_t stream);

/*
 * moe_combine - weighted combine of each token's k expert outputs back to
 * the token (the MoE output):
 *   out[t][n] = sum_{j=0}^{k-1} topk_weights[t][j] * y_rows[row_pos[t*k+j]][n]
 * with j ascending, fp32.
 *   y_rows [T*k][H] fp32, topk_weights [T][k] fp32, row_pos [T*k] int32,
 *   out [T][H] fp32 out.  y_rows and out 16-byte aligned.
 */
MOE_API moe_status moe_combine(const float* y_rows, const float* topk_weights, const int32_t* row_pos, int32_t T,
                       int32_t k, int32_t H, float* out, moe_stream_t stream);

/* Bytes of device workspace that moe_group_rows and moe_expert_ffn_mxfp4
 * need for this shape (one buffer of this size serves both calls and can be
 * reused for every layer; its contents between calls mean nothing).
 * Returns 0 for shapes outside the supported ranges. Host function. */
MOE_API size_t moe_workspace_bytes(int32_t T, int32_t k, int32_t E, int32_t H, int32_t I);

/* Static, human-readable name of a status.  Host function. */
MOE_API const char* moe_status_string(moe_status s);

/*
 * moe_router_logits - the router projection that feeds moe_route_topk (the
 * step before the path; the router picks each token's experts from these
 * logits: page "hn.213312.xyz/article/49090233", section on how it works;
 * the pages give no router form, so this takes the plain linear one):
 *   logits[t][e] = sum_{c=0}^{H-1} x[t][c] * w_router[e][c]
 * with fp32 products and sums (the order of the sums is the library's; the
 * result lies within the fp32 summation bound of the exact value).
 *   x_bf16    [T][H] bf16 bits, 16-byte aligned
 *   w_router  [E][H] fp32, 16-byte aligned
 *   logits    [T][E] fp32 out
 * E in 1..MOE_MAX_EXPERTS, H a multiple of 32 in 32..MOE_MAX_DIM,
 * T*E <= INT32_MAX (MOE_ERR_INVALID_ARG otherwise).
 */
MOE_API moe_status moe_router_logits(const uint16_t* x_bf16, int32_t T, int32_t H, const float* w_router,
                                     int32_t E, float* logits, moe_stream_t stream);

/*
 * moe_rms_rescale_bf16 - glue between stacked layers (not one of the four
 * calls of a layer): x_next[t] = bf16_rne(y[t] / sqrt(mean(y[t]^2) + eps)),
 * the weightless RMS rescaling that feeds layer l's output to layer l+1.
 *   y [T][H] fp32, x_next [T][H] bf16 out (raw bits); H a multiple of 32 in
 *   32..MOE_MAX_DIM, eps >= 0; y 16-byte and x_next 8-byte aligned
 *   (MOE_ERR_INVALID_ARG otherwise).
 */
MOE_API moe_status moe_rms_rescale_bf16(const float* y, int32_t T, int32_t H, float eps, uint16_t* x_next,
                                moe_stream_t stream);

/*
 * Fused calls for callers that step one token, or one layer of a stack, at
 * a time (batch-1 decode through the layer stack: page
 * "hn.213312.xyz/article/49090233", technical highlights, double-buffered
 * layer loading; each of the calls below replaces two calls).  Their
 * outputs equal those of the calls they replace bit for bit.
 *
 * moe_route_group_one - moe_route_topk followed by moe_group_rows for a
 * single token (T = 1): logits [E] fp32 in; topk_ids [k], topk_weights [k],
 * expert_offsets [E+1], sorted_rows [k], row_pos [k], active [E+1] out, as
 * those two calls define them.  E in 1..MOE_MAX_EXPERTS, 1 <= k <=
 * min(E, MOE_MAX_TOPK); all pointers non-null (MOE_ERR_INVALID_ARG
 * otherwise).  Needs no workspace.
 */
MOE_API moe_status moe_route_group_one(const float* logits, int32_t E, int32_t k, int32_t* topk_ids,
                                       float* topk_weights, int32_t* expert_offsets, int32_t* sorted_rows,
                                       int32_t* row_pos, int32_t* active, moe_stream_t stream);

/*
 * moe_combine_rms_bf16 - moe_combine followed by moe_rms_rescale_bf16 of its
 * output: out [T][H] fp32 as moe_combine writes it and x_next [T][H] bf16 as
 * moe_rms_rescale_bf16(out) writes it, in one launch (one block per token).
 * Arguments as those two calls take them: H a multiple of 32 in
 * 32..MOE_MAX_DIM, eps >= 0, y_rows and out 16-byte and x_next 8-byte
 * aligned (MOE_ERR_INVALID_ARG otherwise).
 */
MOE_API moe_status moe_combine_rms_bf16(const float* y_rows, const float* topk_weights, const int32_t* row_pos,
                                        int32_t T, int32_t k, int32_t H, float eps, float* out, uint16_t* x_next,
                                        moe_stream_t stream);

/*
 * moe_expert_ffn_combine_mxfp4 - moe_expert_ffn_mxfp4 followed by
 * moe_combine of its y_rows: y_rows [T*k][H] fp32 and out [T][H] fp32 as
 * those two calls write them, bit for bit.  For a single token (T = 1) with
 * I = 1536, k <= 16 and a hidden size the register gate/up takes, the down
 * projection and the weighted combine run in one launch (block b owns
 * output rows of every routed expert, so the combine needs no second pass
 * over y_rows); other shapes run the two calls.  Arguments as
 * moe_expert_ffn_mxfp4 and moe_combine take them (same workspace size;
 * MOE_ERR_INVALID_ARG / MOE_ERR_WORKSPACE_TOO_SMALL as those calls).
 */
MOE_API moe_status moe_expert_ffn_combine_mxfp4(const uint16_t* x, int32_t T, int32_t k,
                                                const moe_mxfp4_weights* w, const int32_t* expert_offsets,
                                                const int32_t* sorted_rows, const int32_t* active,
                                                const float* topk_weights, const int32_t* row_pos, float* y_rows,
                                                float* out, void* workspace, size_t workspace_bytes,
                                                moe_stream_t stream);

/*
 * moe_decode_layer_mxfp4 - one token through the whole layer: what
 * moe_route_group_one followed by moe_expert_ffn_combine_mxfp4 (T = 1)
 * write, bit for bit, for batch-1 decode (the pages' runtime steps one
 * token through every layer: page "hn.213312.xyz/article/49090233", how it
 * works).  At H = 7168, I = 1536, k <= 16 and E <= 2048 it takes two
 * launches: the top-k runs inside every block of the gate/up launch (each
 * block picks the expert of its slot itself, block 0 writes the routing and
 * grouping outputs), then the down projection with the combine; other
 * shapes run the two calls.
 *   logits [E] fp32 (E = w->num_experts), x [H] bf16 bits (16-byte aligned)
 *   topk_ids [k], topk_weights [k], expert_offsets [E+1], sorted_rows [k],
 *   row_pos [k], active [E+1]: out, as moe_route_group_one writes them
 *   y_rows [k][H] fp32 and out [H] fp32 (16-byte aligned): out
 *   workspace: moe_workspace_bytes(1, k, E, H, I) bytes, 16-byte aligned
 * 1 <= k <= min(E, MOE_MAX_TOPK); every pointer non-null
 * (MOE_ERR_INVALID_ARG otherwise; MOE_ERR_WORKSPACE_TOO_SMALL).
 */
MOE_API moe_status moe_decode_layer_mxfp4(const float* logits, const uint16_t* x, int32_t k,
                                          const moe_mxfp4_weights* w, int32_t* topk_ids, float* topk_weights,
                                          int32_t* expert_offsets, int32_t* sorted_rows, int32_t* row_pos,
                                          int32_t* active, float* y_rows, float* out, void* workspace,
                                          size_t workspace_bytes, moe_stream_t stream);

/*
 * moe_decode_layer_rms_mxfp4 - the next layer of a batch-1 stack straight
 * from the previous layer's output: x_next = moe_rms_rescale_bf16(y_prev)
 * (T = 1), then moe_decode_layer_mxfp4(logits, x_next, ...); every output
 * bit for bit as those two calls write it.  At the decode shape the rescale
 * runs inside the gate/up launch (each block forms x itself with the
 * rescale's arithmetic; block 0 writes x_next), so a stacked layer takes
 * two launches.
 *   y_prev [H] fp32 and x_next [H] bf16 out, both 16-byte aligned; eps >= 0;
 *   out may be y_prev's own buffer; the other arguments as moe_decode_layer_mxfp4 takes
 *   them (MOE_ERR_INVALID_ARG / MOE_ERR_WORKSPACE_TOO_SMALL likewise).
 */
MOE_API moe_status moe_decode_layer_rms_mxfp4(const float* logits, const float* y_prev, float eps,
                                              uint16_t* x_next, int32_t k, const moe_mxfp4_weights* w,
                                              int32_t* topk_ids, float* topk_weights, int32_t* expert_offsets,
                                              int32_t* sorted_rows, int32_t* row_pos, int32_t* active,
                                              float* y_rows, float* out, void* workspace, size_t workspace_bytes,
                                              moe_stream_t stream);

/*
 * moe_decode_layer_mxfp4_noalloc - moe_decode_layer_mxfp4 for callers that
 * cannot allocate or hand over device memory: code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc.  Same arguments and
 * the same outputs bit for bit, without the workspace: its scratch (h, the
 * k x I fp32 gate/up results) lives in a static device array of
 * MOE_NOALLOC_SCRATCH_BYTES in the library, one per GPU, held until the
 * process ends.  The call allocates nothing (no hipMalloc, hipFree or
 * allocating library routine); the first call on a device looks up that
 * device's array address once.
 *   k * I * 4 bytes (rounded up to 256) must fit in the scratch, i.e.
 *   k * I <= 262144 (the decode shape k = 16, I = 1536 takes 96 KiB);
 *   larger shapes return MOE_ERR_SCRATCH_TOO_SMALL before anything is
 *   enqueued.  Other errors as moe_decode_layer_mxfp4.
 * Every call on one GPU shares that GPU's scratch: calls that may overlap on
 * one device (on different streams without ordering between them, or from
 * several threads) race and must be serialized by the caller.  Nothing in
 * the scratch needs to start at zero; its contents between calls mean
 * nothing.
 */
#define MOE_NOALLOC_SCRATCH_BYTES (1u << 20)
MOE_API moe_status moe_decode_layer_mxfp4_noalloc(const float* logits, const uint16_t* x, int32_t k,
                                                  const moe_mxfp4_weights* w, int32_t* topk_ids,
                                                  float* topk_weights, int32_t* expert_offsets, int32_t* sorted_rows,
                                                  int32_t* row_pos, int32_t* active, float* y_rows, float* out,
                                                  moe_stream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* MOE_MXFP4_H */
