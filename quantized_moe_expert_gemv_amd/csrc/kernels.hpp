// Kernel argument blocks and launchers shared between the host code and the
// kernel translation units.  Internal to the library.
#pragma once
#include <hip/hip_runtime.h>
#include <hip/hip_ext.h>
#include <stdint.h>
#include <stddef.h>

#include "strata_moe.h"

namespace strata {

// Workspace regions (device pointers), sized for max_tokens by the host.
struct Work {
  float* logits;      // [Tmax][E]
  int* topk_idx;      // [Tmax][k]
  float* topk_w;      // [Tmax][k]
  int* counts;        // [E]
  int* offsets;       // [E+1]
  int* perm;          // [Tmax*k]   sorted slot -> pair
  int* inv;           // [Tmax*k]   pair -> sorted slot
  int* slot_tok;      // [Tmax*k]   prefill: sorted slot -> token
  int* udesc;         // [E+1][2]   decode: per active expert {expert id, token mask}
  float* wtab;        // [E+1][8 or 16] decode: routing weight per (active expert, token), 0 if not routed
  int* meta;          // [16]       meta[0] active experts (decode), meta[1] GEMM tiles (prefill),
                      //            meta[2] prefill: some token of the call is scaled (e != 0),
                      //            meta[3] decode: some token has a nonzero second fp16 part,
                      //            meta[4] create: block scales the operands cannot carry,
                      //            meta[8] decode: the prefetch's discarded word
  int* chunk_base;    // [nchunks][E] prefill: per-chunk counts, then bases
  int* pair_rank;     // [Tmax*k]   prefill: rank of a pair inside its chunk
  int* texp;          // [Tmax]     the exponent e of each token's operand scale 2^-e
  uint32_t* tmax;     // [32][Tmax] prefill: each token's largest |x| (float bits) per router K split
  int4* tiles;        // [max_tiles] prefill: {expert, first slot, rows, 0}, in XCD segments,
                      //             each sorted by row class (see k_scan)
  float* act;         // prefill: fp16 SwiGLU rows [slots][I] (same region as actp)
  _Float16* actp;     // decode: SwiGLU rows as two fp16 parts [active expert][2][T][I]
  _Float16* xparts;   // decode: token rows as two fp16 parts [2][T][H]
  uint16_t* ybf;      // [slots][H]  prefill: per-pair expert outputs, bf16; before the
                      //             expert GEMMs it holds the router's split-K partials
  size_t ybf_bytes;
  void* xpad;         // [Tmax][H]   prefill: the tokens with zero columns past Ho (only
                      //             when Ho < H), in the call's activation type
  int nchunks;
  int max_tiles;
};

// Kernel geometry.  H and I are the hidden and intermediate widths rounded up
// to whole 256-weight superblocks; Ho and Io are the layer's own widths (the
// canonical records, x, out and the router rows).  The padded rows and
// columns of every packed matrix hold zero codes with zero scales, so they
// contribute exactly zero (a padded gate/up row gives silu(0) * 0 = 0).
struct Layer {
  int H, I, E, k, n_shared, fmt;
  int Ho, Io;
  const float* router_w;        // [E][H] fp32
  const float* router_b;        // [E] or null
  const uint8_t* packed;        // experts (routed then shared) in the packed layout
  size_t expert_stride;         // bytes per expert
  const uint16_t* router_hi;    // bf16 high part of router_w, MFMA operand order (k_router_split)
  const uint16_t* router_lo;    // bf16 remainder, same order
  int* route_done;              // one-launch routing: completion counter (0 between calls)
};

struct Call {
  const void* x;
  int x_f32;
  int T;
  float* out;
  uint32_t flags;
  // decode gate/up prefetch of what a later kernel reads (a hint: no result
  // depends on it): the router rows of the next layer of a stack (null: none)
  const float* next_router = nullptr;
  int next_E = 0, next_Ho = 0;
};

// Optional per-kernel timing: with a tracer armed, each kernel is launched
// with the next two caller events bound to its own dispatch, so the pair
// brackets that kernel's execution (start and end of the dispatch), not the
// gaps between kernels.
struct Tracer {
  hipEvent_t* ev = nullptr;
  int n = 0, i = 0;
};

template <typename K, typename... Args>
inline void launch(Tracer* tr, K kernel, dim3 grid, dim3 block, size_t lds, hipStream_t s, Args... args) {
  if (tr && tr->i + 2 <= tr->n) {
    hipExtLaunchKernelGGL(kernel, grid, block, (uint32_t)lds, s, tr->ev[tr->i], tr->ev[tr->i + 1], 0u,
                          args...);
    tr->i += 2;
  } else {
    hipLaunchKernelGGL(kernel, grid, block, lds, s, args...);
  }
}

// create-time repack (canonical -> packed) and router split
hipError_t launch_repack(const Layer& L, const uint8_t* canon, int n_experts_in, int first_expert,
                         hipStream_t s);
hipError_t launch_router_split(const Layer& L, hipStream_t s);
// count (into *bad, device) the canonical blocks whose scale the kernels
// cannot carry (see k_check_scales)
hipError_t launch_check_scales(const Layer& L, const uint8_t* canon, int n_records, int* bad, hipStream_t s);

// decode path: router GEMV, top-k (+ the permutation when asked for), then
// gate/up and down + combine; prepare_decode_kernels raises the gate/up
// kernels' dynamic-LDS ceiling (once per process is enough)
hipError_t prepare_decode_kernels();
// LDS ceiling of the decode kernels, and whether the decode path covers T
// tokens of a layer with top-k k over E experts (+ n_shared): its down kernel
// keeps the routing table and the staged activation rows in LDS
constexpr size_t DECODE_LDS_MAX = 160 * 1024;
bool decode_fits(int T, int k, int E, int n_shared, int I);
hipError_t launch_decode_route(const Layer& L, const Work& W, const Call& c, hipStream_t s, Tracer* tr,
                               bool permutation);
hipError_t launch_decode_experts(const Layer& L, const Work& W, const Call& c, hipStream_t s, Tracer* tr);
// bytes of the router rows one decode router workgroup reads for a call of T
// tokens (the unit the gate/up kernel prefetches them in)
uint32_t decode_route_chunk_bytes(int T, int Ho);

// top-k of T logit rows (row t at rows + t * stride, + bias[e] when bias is
// not null) for any k <= E <= 4096: one workgroup per token
hipError_t launch_topk_block(const float* rows, size_t stride, const float* bias, int T, int E, int k, int* idx,
                             float* w, hipStream_t s, Tracer* tr);

// prefill path
hipError_t launch_prefill_route(const Layer& L, const Work& W, const Call& c, hipStream_t s, Tracer* tr);
hipError_t launch_prefill_experts(const Layer& L, const Work& W, const Call& c, hipStream_t s, Tracer* tr);

constexpr int PREFILL_BM = 128;     // token rows per GEMM tile
constexpr int PREFILL_CHUNK_T = 32; // most tokens per top-k/histogram chunk (32-bit token masks)
// Tokens per chunk for a call of T tokens.  A chunk is one workgroup whose
// waves select one or two tokens each, a chain of dependent memory round
// trips and a radix descent: small chunks spread a short call's selections
// over more workgroups, large ones keep the column scan of the chunk
// histograms short for long calls.
inline int prefill_chunk_t(int T) { return T <= 256 ? 8 : T <= 4096 ? 16 : PREFILL_CHUNK_T; }
inline int prefill_chunks(int T) { return (T + prefill_chunk_t(T) - 1) / prefill_chunk_t(T); }
// most chunks of any call of up to Tmax tokens (the chunk count grows with T
// inside each range of prefill_chunk_t)
inline int prefill_max_chunks(int Tmax) {
  const int a = prefill_chunks(Tmax < 256 ? Tmax : 256), b = prefill_chunks(Tmax < 4096 ? Tmax : 4096);
  const int c = prefill_chunks(Tmax);
  return a > b ? (a > c ? a : c) : (b > c ? b : c);
}

// one-launch routing of the grouped path (forward/route flag bits as in the
// public header): where it applies, and up to how many tokens it is taken
// without being asked for
constexpr uint32_t STRATA_FUSED_ROUTE_FLAG = 16u, STRATA_SPLIT_ROUTE_FLAG = 32u;
constexpr int FUSED_ROUTE_DEFAULT_T = STRATA_FUSED_ROUTE_DEFAULT_T;
inline bool fused_route_fits(int E, int k, int T) { return T <= 64 && E <= 512 && k <= 64; }

}  // namespace strata
