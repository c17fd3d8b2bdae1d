// Kernel argument blocks and launchers shared between the host code and the
// kernel translation units.  Internal to the library.
#pragma once
#include <hip/hip_runtime.h>
#include <hip/hip_ext.h>
#include <stdint.h>
#include <stddef.h>

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
  float* wtab;        // [E+1][8]   decode: routing weight per (active expert, token), 0 if not routed
  int* meta;          // [16]       meta[0] active experts (decode), meta[1] GEMM tiles (prefill)
  int* chunk_base;    // [nchunks][E] prefill: per-chunk counts, then bases
  int* pair_rank;     // [Tmax*k]   prefill: rank of a pair inside its chunk
  int4* tiles;        // [max_tiles] prefill: {expert, first slot, rows, 0}, in XCD segments,
                      //             each sorted by row class (see k_scan)
  float* act;         // prefill: fp16 SwiGLU rows [slots][I] (same region as actp)
  _Float16* actp;     // decode: SwiGLU rows as two fp16 parts [active expert][2][T][I]
  _Float16* xparts;   // decode: token rows as two fp16 parts [2][T][H]
  uint16_t* ybf;      // [slots][H]  prefill: per-pair expert outputs, bf16; before the
                      //             expert GEMMs it holds the router's split-K partials
  size_t ybf_bytes;
  int nchunks;
  int max_tiles;
};

struct Layer {
  int H, I, E, k, n_shared, fmt;
  const float* router_w;        // [E][H] fp32
  const float* router_b;        // [E] or null
  const uint8_t* packed;        // experts (routed then shared) in the packed layout
  size_t expert_stride;         // bytes per expert
  const uint16_t* router_hi;    // bf16 high part of router_w, MFMA operand order (k_router_split)
  const uint16_t* router_lo;    // bf16 remainder, same order
};

struct Call {
  const void* x;
  int x_f32;
  int T;
  float* out;
  uint32_t flags;
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

// decode path: router GEMV, top-k (+ the permutation when asked for), then
// gate/up and down + combine; prepare_decode_kernels raises the gate/up
// kernels' dynamic-LDS ceiling (once per process is enough)
hipError_t prepare_decode_kernels();
// LDS ceiling of the decode kernels, and whether the decode path covers T
// tokens of a layer with top-k k over E experts (+ n_shared): its down kernel
// keeps the routing table and the staged activation rows in LDS
constexpr size_t DECODE_LDS_MAX = 160 * 1024;
bool decode_fits(int T, int k, int E, int n_shared);
hipError_t launch_decode_route(const Layer& L, const Work& W, const Call& c, hipStream_t s, Tracer* tr,
                               bool permutation);
hipError_t launch_decode_experts(const Layer& L, const Work& W, const Call& c, hipStream_t s, Tracer* tr);

// prefill path
hipError_t launch_prefill_route(const Layer& L, const Work& W, const Call& c, hipStream_t s, Tracer* tr);
hipError_t launch_prefill_experts(const Layer& L, const Work& W, const Call& c, hipStream_t s, Tracer* tr);

constexpr int PREFILL_BM = 128;     // token rows per GEMM tile
constexpr int PREFILL_CHUNK_T = 32; // tokens per top-k/histogram chunk

}  // namespace strata
