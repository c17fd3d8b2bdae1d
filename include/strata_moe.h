/*
 * strata_moe.h - C ABI of the MI355X (gfx950) routed mixture-of-experts FFN
 * layer over low-bit block-quantised experts.
 *
 * The operation (blog.5616760.com/0039.html, section 五 "MoE 的本质": the
 * router scores every expert of the layer, the top-k are selected and their
 * outputs merged with softmax weights; ai-coding.wiselychen.com "Strata two
 * weeks", section 成功思路一: the GPU computes the selected experts and sums
 * their results; lcz.me/topic/2153, section 一: 256 routed experts plus one
 * always-on shared expert in the DeepSeek-shaped layer), per token t:
 *
 *   l[t,e]  = sum_h x[t,h] Wr[e,h] + b[e]                  router logits
 *   S_t     = the k largest l[t,.]                          top-k
 *   w[t,j]  = softmax of l[t,.] over S_t                    renormalised weights
 *   y_e(x)  = Wd_e (silu(Wg_e x) * (Wu_e x))                SwiGLU expert
 *   out[t]  = sum_{e in S_t} w[t,e] y_e(x_t) [+ y_shared(x_t)] [+ x_t | + out_t]
 *
 * Expert weights are 32-weight blocks: b-bit codes q then an fp16 scale d,
 * w = d (q - c): Q2 (8 code bytes, c = 1.5), Q3 (12 bytes, c = 3.5),
 * Q4 (16 bytes, c = 8).  Code j of a block occupies bits [b*j, b*j+b) of
 * the code bytes read as one little-endian bit string.  MXFP4 (OCP
 * Microscaling Formats v1.0, a format the pages name for their DeepSeek
 * suites): 16 bytes of FP4 E2M1 codes in the same bit order, then one E8M0
 * scale byte e, w = 2^(e - 127) E2M1(q).
 * Block scales the 16-bit weight operands cannot carry are refused at
 * create (STRATA_E_UNSUPPORTED): an fp16 d that is NaN, infinite or above
 * 2^15 (Q2), 2^14 (Q3) or 2^12 (Q4); an MXFP4 byte e above 140 (2^13), 255
 * (NaN) included.
 *
 * Canonical expert record (the input of strata_moe_create): gate
 * [I rows][H/32 blocks], up [I][H/32], down [H rows][I/32 blocks], each
 * block = code bytes followed by the little-endian fp16 scale (MXFP4: the
 * scale byte), no padding.
 * Routed experts are stored back to back in expert-id order.
 *
 * Conventions
 *  - Every pointer named "device" is HIP device memory owned by the caller.
 *    The library never allocates or frees device memory and never
 *    synchronises inside route/forward.
 *  - Streams are hipStream_t passed as void* (NULL = the null stream).
 *  - Every function returning int returns STRATA_OK or a negative status;
 *    argument checks run on the host before anything is enqueued, and the
 *    reason is available from strata_moe_last_error() (thread-local).
 *    Nothing aborts and no C++ exception crosses the ABI.
 *  - One handle's workspace serves one call at a time: calls on one handle
 *    must be ordered on one stream.  Distinct handles (with distinct
 *    workspaces) are independent.
 */
#ifndef STRATA_MOE_H
#define STRATA_MOE_H

#include <stddef.h>
#include <stdint.h>

#if defined(__GNUC__) || defined(__clang__)
#define STRATA_API __attribute__((visibility("default")))
#else
#define STRATA_API
#endif

#ifdef __cplusplus
extern "C" {
#endif

enum {
    STRATA_OK = 0,
    STRATA_E_INVALID = -1,      /* bad argument (shape, pointer, size, flag) */
    STRATA_E_UNSUPPORTED = -2,  /* valid but outside what the kernels cover  */
    STRATA_E_HIP = -3           /* a HIP runtime call or launch failed       */
};

enum { STRATA_Q2 = 2, STRATA_Q3 = 3, STRATA_Q4 = 4,        /* expert block format */
       STRATA_MXFP4 = 5 };
enum { STRATA_BF16 = 0, STRATA_FP32 = 1 };                 /* activation dtype    */

/* forward flags */
enum {
    STRATA_ACCUMULATE = 1u,     /* out[t] += moe(x)[t]                          */
    STRATA_ADD_INPUT = 2u,      /* out[t]  = x[t] + moe(x)[t] (residual)        */
    STRATA_FORCE_DECODE = 4u,   /* use the GEMV path (T <= STRATA_DECODE_MAX_T) */
    STRATA_FORCE_PREFILL = 8u,  /* use the grouped-GEMM path at any T           */
    /* grouped path only (calls on the decode path ignore them): route in one
     * launch (router, top-k, permutation; T <= 64, E <= 512, k <= 64, else
     * STRATA_E_UNSUPPORTED), or in the multi-launch sequence.  Without
     * either the library picks the faster for the call. */
    STRATA_FUSED_ROUTE = 16u,
    STRATA_SPLIT_ROUTE = 32u
};

/* Calls with T <= STRATA_DECODE_MAX_T take the decode (GEMV) path unless
 * STRATA_FORCE_PREFILL is given or its down kernel's LDS cannot hold the
 * call's routing table (thousands of active experts); larger T take the
 * grouped-GEMM path. */
#define STRATA_DECODE_MAX_T 16
/* Grouped-path calls of at most this many tokens (and E <= 512, k <= 64)
 * route in one launch unless STRATA_SPLIT_ROUTE is given. */
#define STRATA_FUSED_ROUTE_DEFAULT_T 0

typedef struct {
    int32_t hidden;      /* H: multiple of 32 (whole blocks), <= 65536        */
    int32_t inter;       /* I: expert intermediate width, multiple of 32,     */
                         /*    <= 65536 (widths that are not whole 256-weight */
                         /*    superblocks are zero-padded inside the packed  */
                         /*    layout; one packed expert must stay < 2 GiB)   */
    int32_t n_experts;   /* E: routed experts, 1..4096                        */
    int32_t top_k;       /* k: 1..E                                           */
    int32_t n_shared;    /* 0 or 1 always-on shared expert (weight 1)         */
    int32_t qfmt;        /* STRATA_Q2 / STRATA_Q3 / STRATA_Q4 / STRATA_MXFP4  */
    int32_t max_tokens;  /* largest T any call on the handle will pass, >= 1; */
                         /* max_tokens * top_k <= 2^28 and                   */
                         /* max_tokens * hidden * 2 < 4 GiB (else            */
                         /* STRATA_E_UNSUPPORTED)                            */
} strata_moe_config;

typedef struct strata_moe strata_moe;   /* opaque; one per MoE layer */

/* Bytes of one canonical expert record, 3 * I * (H/32) * (code bytes +
 * scale bytes: 2, or 1 for MXFP4).  Returns 0 for an invalid config. */
STRATA_API size_t strata_moe_expert_bytes(const strata_moe_config* cfg);

/* Bytes of the device buffer `packed` that strata_moe_create fills: the
 * experts (routed, then shared) repacked into the kernels' layout (the same
 * byte count as the canonical records when H and I are multiples of 256,
 * else with the padding rows and blocks; for MXFP4 one byte more per block,
 * the scale taking a 16-bit slot) plus a bf16 hi/lo split of the router
 * rows.  Returns 0 for an invalid config. */
STRATA_API size_t strata_moe_packed_bytes(const strata_moe_config* cfg);

/* Bytes of the device buffer `workspace` (router logits, top-k, counts,
 * offsets, permutation, per-pair activations and outputs), sized for
 * cfg->max_tokens.  Returns 0 for an invalid config. */
STRATA_API size_t strata_moe_workspace_bytes(const strata_moe_config* cfg);

/*
 * Build a layer handle: one MoE layer's router and experts, repacked once
 * into the kernels' layout (the one-time re-layout of the expert set into a
 * compute-friendly copy: devotd.net "Strata memory tiers", section
 * 小模型包不等于合适的模型; one contiguous record per expert: lcz.me/topic/2153,
 * section 三 item 4).  Every expert stays resident in `packed`.
 *   router_w       device, fp32 [E][H] row-major; borrowed for the handle's life
 *   router_bias    device, fp32 [E], or NULL for no bias; borrowed
 *   experts_canon  device, E canonical records back to back; read during the
 *                  call only (may be freed once it returns)
 *   shared_canon   device, one canonical record if n_shared = 1, else NULL;
 *                  read during the call only
 *   packed         device, strata_moe_packed_bytes(cfg) bytes, 256-B aligned;
 *                  filled here and borrowed for the handle's life
 *   workspace      device, strata_moe_workspace_bytes(cfg) bytes, 256-B aligned;
 *                  borrowed for the handle's life (its counters are zeroed here)
 *   stream         the repack runs on it; the call synchronises it before
 *                  returning
 *   out            receives the handle (host memory, freed by _destroy)
 */
STRATA_API int strata_moe_create(const strata_moe_config* cfg, const float* router_w,
                      const float* router_bias, const void* experts_canon,
                      const void* shared_canon, void* packed, void* workspace,
                      void* stream, strata_moe** out);

/*
 * Routing only (router logits, top-k, renormalised weights, stable
 * token->expert permutation): the router scores of every expert, the top-k
 * selection and the softmax merge weights of blog.5616760.com/0039.html,
 * section 五 "MoE 的本质", and the grouping of tokens by expert that lets one
 * read of an expert's weights serve all its tokens (same page, section 十二;
 * devotd.net "Strata memory tiers", section 读取提示与写出回答时).  Ties
 * between equal logits go to the lower expert id; a NaN logit ranks below
 * every number.  All outputs are device buffers:
 *   x          device, [T][H] of x_dtype (STRATA_BF16 or STRATA_FP32)
 *   topk_idx   int32 [T][k], expert ids of S_t in ascending order
 *   topk_w     fp32  [T][k], weights matching topk_idx
 *   perm       int32 [T*k], sorted slot -> pair p = t*k + j, pairs ordered
 *              by (expert, p)
 *   offsets    int32 [E+1], first slot of each expert; offsets[E] = T*k
 * T must be in [1, max_tokens].  Uses the same kernels as strata_moe_forward
 * for the same T and flags (STRATA_FORCE_DECODE / STRATA_FORCE_PREFILL).
 */
STRATA_API int strata_moe_route(strata_moe* h, const void* x, int32_t x_dtype, int32_t T,
                     int32_t* topk_idx, float* topk_w, int32_t* perm,
                     int32_t* offsets, uint32_t flags, void* stream);

/*
 * The full layer (blog.5616760.com/0039.html, section 五: router scores,
 * top-k, softmax-weighted merge of the selected experts' outputs;
 * ai-coding.wiselychen.com "Strata two weeks", section 成功思路一: each
 * selected expert computed and the results summed; lcz.me/topic/2153,
 * section 一: the always-on shared expert): out[T][H] fp32 (device) = moe(x), or with
 * STRATA_ACCUMULATE out += moe(x), or with STRATA_ADD_INPUT out = x + moe(x).
 * x and out must not overlap.  Stream-ordered and asynchronous.
 * Precision: the decode kernels (T <= 16) multiply exact weight values by the
 * activations carried as two fp16 parts (22 significant bits) with fp32
 * accumulation.  The prefill expert GEMMs round weights and activations to
 * fp16 with fp32 accumulation (weights below 2^-24 in magnitude round to
 * zero there); the prefill router stays fp32-accurate.
 * Range: the 16-bit token operands of both paths hold x_t 2^-e_t, with e_t
 * chosen per token from its largest magnitude m_t (0 while 2^-4 <= m_t < 16,
 * else the power that brings m_t into [8, 16), |e_t| <= 60; 0 for an
 * all-zero token), the SwiGLU activations are kept as silu(g) u 2^-2e_t and
 * the expert outputs are scaled back by 2^2e_t: every step is a power of
 * two, so a token's results do not depend on e_t, and tokens from about
 * 2^-64 to 2^64 in magnitude keep their precision.  The activations still
 * have to fit the 16-bit range at that scale (|silu(g) u| 2^-2e_t below
 * 65504: weights of ordinary magnitude keep them far inside it).
 */
STRATA_API int strata_moe_forward(strata_moe* h, const void* x, int32_t x_dtype, int32_t T,
                       float* out, uint32_t flags, void* stream);

/*
 * For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the same
 * layer as strata_moe_forward, same arguments, kernels and results, but the
 * per-call regions (logits, top-k, permutation, activation and per-pair rows)
 * live in a fixed array inside the library, STRATA_STATIC_SCRATCH_BYTES per
 * device, instead of the handle's workspace.  It allocates nothing (no
 * hipMalloc/hipFree, no allocating library call).  The array is resolved for
 * the device current at strata_moe_create and kept until the process ends.
 * Calls whose regions exceed the array (more tokens than fit; a 2560-wide,
 * 512-expert, top-10 layer fits up to about 256 tokens, every decode call of
 * 16 tokens or fewer of it fits) return STRATA_E_UNSUPPORTED before anything is
 * enqueued.  Every handle on a device shares that device's one array:
 * static calls that overlap in time on one device (different streams, or
 * different threads) race and give wrong results; order them on one stream.
 */
#define STRATA_STATIC_SCRATCH_BYTES (16u << 20)
STRATA_API int strata_moe_forward_static(strata_moe* h, const void* x, int32_t x_dtype, int32_t T,
                              float* out, uint32_t flags, void* stream);

/*
 * A stack of MoE layers with residual adds (48 layers x 512 experts is the
 * Qwen3.8-Flash-Next expert set of the pages: ai-coding.wiselychen.com
 * "Strata two weeks", Table 1):  h_0 = x,  h_{l+1} = h_l + moe_l(h_l),
 * computed in fp32.  The final h is written to `out` (device fp32 [T][H]);
 * `tmp` (device fp32 [T][H]) is scratch for the ping-pong.  Layers must share
 * H and run their calls on this stream; x must not overlap out or tmp.
 */
STRATA_API int strata_moe_stack_forward(strata_moe* const* layers, int32_t n_layers,
                             const void* x, int32_t x_dtype, int32_t T,
                             float* out, float* tmp, void* stream);

/*
 * Per-kernel timing of the next route/forward/stack call on this handle
 * (one-shot).  events are hipEvent_t created by the caller (void*), taken in
 * pairs: kernel i of the call is launched with events[2i] and events[2i+1]
 * bound to its own dispatch (hipExtLaunchKernelGGL), so the elapsed time of
 * the pair is that kernel's execution, without launch gaps.  Kernels beyond
 * n_events / 2 are not traced.  Kernel order: decode forward = router GEMV,
 * top-k + permutation, gate/up + SwiGLU, down + weighted combine; prefill
 * forward = router GEMM, top-k, column scan, scan, scatter, gate/up GEMM,
 * down GEMM, combine, where for T <= 32 the top-k kernel also does the
 * column scan, the scan and the scatter (5 kernels); route-only calls stop
 * after the routing kernels.  A layer whose H is not a multiple of 256 runs
 * one more kernel first in the grouped path (the tokens widened with zero
 * columns); a top-k above 64 runs its selection as one more kernel before
 * the top-k / histogram kernel (grouped path) or in place of the top-k
 * kernel (decode path).  A stack call
 * traces the handle's layer only.  n_events even, in
 * [0, STRATA_MAX_TRACE_EVENTS]; 0 disarms.  The events must outlive the
 * call's completion on its stream.
 */
#define STRATA_MAX_TRACE_EVENTS 16
STRATA_API int strata_moe_trace_next_call(strata_moe* h, void* const* events, int32_t n_events);

/* Free the host-side handle.  NULL-safe.  Device buffers stay the caller's. */
STRATA_API void strata_moe_destroy(strata_moe* h);

/* Message for the last failing call on this thread ("" if none). */
STRATA_API const char* strata_moe_last_error(void);

#ifdef __cplusplus
}
#endif
#endif /* STRATA_MOE_H */
