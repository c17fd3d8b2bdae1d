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
  int* udesc;         // [E+1][16]  decode: per active expert {e, first slot, n, 0, tokens[8]}
  float* wtab;        // [E+1][8]   decode: routing weight per (active expert, token), 0 if not routed
  int* meta;          // [16]       meta[0] active experts (decode), meta[1] GEMM tiles (prefill)
  int* tickets;       // [H/64 + 1] completion counters (last entry: router)
  int* chunk_base;    // [E][nchunks] prefill: per-chunk counts, then bases
  int* pair_rank;     // [Tmax*k]   prefill: rank of a pair inside its chunk
  int4* tiles;        // [max_tiles] prefill: {expert, first slot, rows, 0}
  float* act;         // prefill: bf16 SwiGLU rows [slots][I] (same region as actp)
  _Float16* actp;     // decode: SwiGLU rows as three fp16 parts [slots][3][I]
  _Float16* xparts;   // decode: token rows as three fp16 parts [8][3][H]
  float* y;           // [slots][H]  prefill: per-pair expert outputs
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

// Optional per-kernel timing: mark() records the next caller-supplied event
// on the stream; called once before a call's first kernel and after each
// kernel.
struct Tracer {
  hipEvent_t* ev = nullptr;
  int n = 0, i = 0;
  void mark(hipStream_t s) {
    if (i < n) (void)hipEventRecord(ev[i], s);
    ++i;
  }
};
inline void mark(Tracer* t, hipStream_t s) {
  if (t) t->mark(s);
}

// create-time repack (canonical -> packed) and router split
hipError_t launch_repack(const Layer& L, const uint8_t* canon, int n_experts_in, int first_expert,
                         hipStream_t s);
hipError_t launch_router_split(const Layer& L, hipStream_t s);

// decode path: router + top-k + permute (one launch), gate/up, down + combine
hipError_t launch_decode_route(const Layer& L, const Work& W, const Call& c, hipStream_t s, Tracer* tr);
hipError_t launch_decode_experts(const Layer& L, const Work& W, const Call& c, hipStream_t s, Tracer* tr);

// prefill path
hipError_t launch_prefill_route(const Layer& L, const Work& W, const Call& c, hipStream_t s, Tracer* tr);
hipError_t launch_prefill_experts(const Layer& L, const Work& W, const Call& c, hipStream_t s, Tracer* tr);

constexpr int PREFILL_BM = 128;     // token rows per GEMM tile
constexpr int PREFILL_CHUNK_T = 32; // tokens per top-k/histogram chunk

}  // namespace strata
