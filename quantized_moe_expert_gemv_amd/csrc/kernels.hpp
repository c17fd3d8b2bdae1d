// Kernel argument blocks and launchers shared between the host code and the
// kernel translation units.  Internal to the library.
#pragma once
#include <hip/hip_runtime.h>
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
  int* uexp;          // [E+1]      decode: active experts (ascending, shared last)
  int* uoff;          // [E+2]      decode: first slot of each active expert
  int* meta;          // [16]       meta[0] active experts (decode), meta[1] GEMM tiles (prefill)
  int* tickets;       // [H/64 + 1] completion counters (last entry: router)
  int* chunk_base;    // [E][nchunks] prefill: per-chunk counts, then bases
  int* pair_rank;     // [Tmax*k]   prefill: rank of a pair inside its chunk
  int4* tiles;        // [max_tiles] prefill: {expert, first slot, rows, 0}
  void* act;          // [slots][I]  fp32 (decode) or bf16 (prefill)
  float* y;           // [slots][H]  per-pair expert outputs
  int nchunks;
  int max_tiles;
};

struct Layer {
  int H, I, E, k, n_shared, fmt;
  const float* router_w;        // [E][H] fp32
  const float* router_b;        // [E] or null
  const uint8_t* packed;        // experts (routed then shared) in the packed layout
  size_t expert_stride;         // bytes per expert
  const uint16_t* router_hi;    // [E][H] bf16 high part of router_w
  const uint16_t* router_lo;    // [E][H] bf16 remainder
};

struct Call {
  const void* x;
  int x_f32;
  int T;
  float* out;
  uint32_t flags;
};

// create-time repack (canonical -> packed) and router split
hipError_t launch_repack(const Layer& L, const uint8_t* canon, int n_experts_in, int first_expert,
                         hipStream_t s);
hipError_t launch_router_split(const Layer& L, hipStream_t s);

// decode path: router + top-k + permute (one launch), gate/up, down + combine
hipError_t launch_decode_route(const Layer& L, const Work& W, const Call& c, hipStream_t s);
hipError_t launch_decode_experts(const Layer& L, const Work& W, const Call& c, hipStream_t s);

// prefill path
hipError_t launch_prefill_route(const Layer& L, const Work& W, const Call& c, hipStream_t s);
hipError_t launch_prefill_experts(const Layer& L, const Work& W, const Call& c, hipStream_t s);

constexpr int PREFILL_BM = 128;     // token rows per GEMM tile
constexpr int PREFILL_CHUNK_T = 32; // tokens per top-k/histogram chunk

}  // namespace strata
