// Decode path (T <= 8 tokens): the per-token expert GEMV regime of the
// pages (ai-coding.wiselychen.com "Strata two weeks", section 成功思路一: per
// layer the GPU runs the router, picks 10 experts and computes them; the
// expert step is bound by the bytes of expert weights read), including the
// 1+3-token MTP verify window (devotd.net "Strata memory tiers", section
// 用草拟 token 提高生成速度的 MTP) where tokens that pick the same expert share
// one read of its weights (blog.5616760.com/0039.html, section 十二).
//
// Three launches per layer:
//   k_decode_route    router GEMV (one wave per expert row, fp32), then the
//                     last workgroup to finish (ticket) runs top-k, the
//                     renormalised softmax and the stable token->expert
//                     permutation for all T tokens;
//   k_decode_gateup   one workgroup per (active expert, 64-row tile of I);
//                     waves split the H superblocks, every lane owns one
//                     gate row and the matching up row; packed codes stream
//                     in as 16-B loads and are dequantised in registers;
//                     the SwiGLU product is written per (pair, i);
//   k_decode_down     one workgroup per (active expert, 64-row tile of H);
//                     the last workgroup of each H tile (ticket) forms the
//                     routing-weighted combine for that tile.
//
// Dequantisation uses sum_j d (q_j - c) x_j = d (sum_j q_j x_j - c sum_j x_j):
// codes convert from bytes straight to fp32, and the per-block sums of x are
// computed once per workgroup.  (q - c) * d is exact in fp32 and so is each
// product with a bf16 x; only the fp32 accumulation rounds.
#include "common.hpp"
#include "kernels.hpp"

namespace strata {
namespace {

// ------------------------------------------------------------------ helpers
__device__ inline float ld_x(const void* x, int x_f32, size_t i) {
  return x_f32 ? reinterpret_cast<const float*>(x)[i]
               : bf16_to_f32(reinterpret_cast<const uint16_t*>(x)[i]);
}

__device__ inline float4 ld_x4(const void* x, int x_f32, size_t i) {
  if (x_f32) return *reinterpret_cast<const float4*>(reinterpret_cast<const float*>(x) + i);
  const uint2 r = *reinterpret_cast<const uint2*>(reinterpret_cast<const uint16_t*>(x) + i);
  return make_float4(__uint_as_float(r.x << 16), __uint_as_float(r.x & 0xffff0000u),
                     __uint_as_float(r.y << 16), __uint_as_float(r.y & 0xffff0000u));
}

__device__ inline float ld_coherent(const float* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ inline int ld_coherent(const int* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Position of element h inside the permuted LDS copy of an activation row.
// Within each 32-weight block, the 4 codes that one extraction step puts in
// the 4 bytes of a register map to 4 consecutive floats, so one 16-B LDS
// read feeds 4 multiply-adds.
template <int FMT>
__device__ inline int perm_pos(int h) {
  constexpr int G = (FMT == 4) ? 8 : 16;   // codes per 32-bit word
  constexpr int Q = G / 4;                 // codes per byte
  const int b = h >> 5, r = h & 31;
  const int w = r / G, rr = r % G;
  const int i = rr / Q, s = rr % Q;
  return b * 32 + w * G + s * 4 + i;
}

__device__ inline float byte_f(uint32_t d, int n) { return (float)((d >> (8 * n)) & 0xffu); }

__device__ inline uint32_t comp(const uint4& v, int i) {
  return i == 0 ? v.x : (i == 1 ? v.y : (i == 2 ? v.z : v.w));
}

// 4 codes of 32-bit word W (shift step s) as 4 bytes, for block bb of the
// row-superblock held in vec[] (NCV code vectors).
template <int FMT>
__device__ inline uint32_t codes4(const uint4* vec, int bb, int w, int s) {
  if constexpr (FMT == 2) {
    const uint32_t W = comp(vec[bb >> 1], (bb & 1) * 2 + w);
    return (W >> (2 * s)) & 0x03030303u;
  } else if constexpr (FMT == 4) {
    const uint32_t W = comp(vec[bb], w);
    return (W >> (4 * s)) & 0x0F0F0F0Fu;
  } else {
    const uint32_t W = comp(vec[bb >> 1], (bb & 1) * 2 + w);
    const uint32_t Hw = comp(vec[4 + (bb >> 2)], bb & 3);
    return ((W >> (2 * s)) & 0x03030303u) | (((Hw >> (4 * w + s)) & 0x01010101u) << 2);
  }
}

template <int FMT> struct Steps {
  static constexpr int W = (FMT == 4) ? 4 : 2;   // 32-bit words per block (per plane)
  static constexpr int S = (FMT == 4) ? 2 : 4;   // extraction steps per word
  static constexpr int G = (FMT == 4) ? 8 : 16;
};

// ------------------------------------------------------------------ router
struct RouteArgs {
  const float* Wr;
  const float* bias;
  const void* x;
  int x_f32, T, H, E, k, n_shared;
  Work w;
};

// Top-k, weights and the permutation for all T tokens; one workgroup of 256.
__device__ void route_tail(const RouteArgs& a, float* rows /* [4][E] */, int* sel /* [T][k] */,
                           int* hist /* [E] */, int2* tmp) {
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int E = a.E, k = a.k, T = a.T, P = T * k;
  __shared__ int s_sel[4][64];
  for (int t = wv; t < T; t += 4) {
    float* row = rows + wv * E;
    for (int e = lane; e < E; e += 64) row[e] = ld_coherent(a.w.logits + (size_t)t * E + e);
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    wave_topk(row, E, k, sel + t * k, a.w.topk_w + (size_t)t * k, s_sel[wv]);
  }
  for (int e = threadIdx.x; e < E; e += blockDim.x) hist[e] = 0;
  __syncthreads();
  for (int p = threadIdx.x; p < P; p += blockDim.x) {
    a.w.topk_idx[p] = sel[p];
    atomicAdd(&hist[sel[p]], 1);
  }
  __syncthreads();
  // exclusive scans over experts of (count, non-empty flag), in chunks
  const int per = (E + blockDim.x - 1) / blockDim.x;
  const int e0 = threadIdx.x * per;
  int2 loc = make_int2(0, 0);
  for (int e = e0; e < min(E, e0 + per); ++e) { loc.x += hist[e]; loc.y += (hist[e] > 0); }
  int2 total;
  int2 base = block_exclusive_scan(loc, tmp, &total);
  for (int e = e0; e < min(E, e0 + per); ++e) {
    const int c = hist[e];
    a.w.counts[e] = c;
    a.w.offsets[e] = base.x;
    if (c > 0) {
      a.w.uexp[base.y] = e;
      a.w.uoff[base.y] = base.x;
    }
    base.x += c;
    base.y += (c > 0);
  }
  __syncthreads();
  // stable slot of every pair: earlier tokens that chose the same expert go first
  for (int p = threadIdx.x; p < P; p += blockDim.x) {
    const int t = p / k, e = sel[p];
    int rank = 0;
    for (int t2 = 0; t2 < t; ++t2)
      for (int j = 0; j < k; ++j) rank += (sel[t2 * k + j] == e);
    const int slot = a.w.offsets[e] + rank;
    a.w.perm[slot] = p;
    a.w.inv[p] = slot;
  }
  if (threadIdx.x == 0) {
    const int U = total.y;
    a.w.offsets[E] = P;
    if (a.n_shared) {
      a.w.uexp[U] = E;
      a.w.uoff[U] = P;
      a.w.uoff[U + 1] = P + T;
      a.w.meta[0] = U + 1;
    } else {
      a.w.uoff[U] = P;
      a.w.meta[0] = U;
    }
  }
}

__global__ __launch_bounds__(256) void k_decode_route(RouteArgs a) {
  extern __shared__ float lds_route[];
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int e = blockIdx.x * 4 + wv;
  if (e < a.E) {
    float acc[DECODE_MAX_T];
#pragma unroll
    for (int t = 0; t < DECODE_MAX_T; ++t) acc[t] = 0.f;
    const float4* wrow = reinterpret_cast<const float4*>(a.Wr + (size_t)e * a.H);
    const int H4 = a.H >> 2;
    for (int c = lane; c < H4; c += 64) {
      const float4 w = wrow[c];
#pragma unroll
      for (int t = 0; t < DECODE_MAX_T; ++t) {
        if (t < a.T) {
          const float4 xv = ld_x4(a.x, a.x_f32, (size_t)t * a.H + 4 * c);
          acc[t] = fmaf(w.x, xv.x, acc[t]);
          acc[t] = fmaf(w.y, xv.y, acc[t]);
          acc[t] = fmaf(w.z, xv.z, acc[t]);
          acc[t] = fmaf(w.w, xv.w, acc[t]);
        }
      }
    }
    const float b = a.bias ? a.bias[e] : 0.f;
#pragma unroll
    for (int t = 0; t < DECODE_MAX_T; ++t) {
      if (t < a.T) {
        const float s = wave_sum(acc[t]);
        if (lane == 0) a.w.logits[(size_t)t * a.E + e] = s + b;
      }
    }
  }
  // the last workgroup to finish routes every token
  __shared__ int s_last;
  __threadfence();
  __syncthreads();
  int* ticket = a.w.tickets + (a.H / 64);
  if (threadIdx.x == 0) s_last = (atomicAdd(ticket, 1) == (int)gridDim.x - 1);
  __syncthreads();
  if (!s_last) return;
  __threadfence();
  float* rows = lds_route;                                   // [4][E]
  int* sel = reinterpret_cast<int*>(rows + 4 * a.E);         // [T*k]
  int* hist = sel + a.T * a.k;                               // [E]
  __shared__ int2 tmp[16];
  route_tail(a, rows, sel, hist, tmp);
  if (threadIdx.x == 0) __hip_atomic_store(ticket, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// ------------------------------------------------------------------ experts
struct ExpertArgs {
  const uint8_t* packed;
  size_t stride;
  int H, I, E, k, T, P, n_shared;
  const void* x;
  int x_f32;
  uint32_t flags;
  float* out;
  Work w;
};

// Dot products of one 32-weight block of two rows (gate and up, or a single
// row when TWO is false) with NTn permuted activation rows.
template <int FMT, int NTn, bool TWO>
__device__ inline void block_dot(const uint4* gv, const uint4* uv, int bb, const float* xrow,
                                 int row_stride, float* ag, float* au) {
  using St = Steps<FMT>;
#pragma unroll
  for (int w = 0; w < St::W; ++w) {
#pragma unroll
    for (int s = 0; s < St::S; ++s) {
      const uint32_t dg = codes4<FMT>(gv, bb, w, s);
      uint32_t du = 0;
      if constexpr (TWO) du = codes4<FMT>(uv, bb, w, s);
      const float g0 = byte_f(dg, 0), g1 = byte_f(dg, 1), g2 = byte_f(dg, 2), g3 = byte_f(dg, 3);
      float u0 = 0.f, u1 = 0.f, u2 = 0.f, u3 = 0.f;
      if constexpr (TWO) { u0 = byte_f(du, 0); u1 = byte_f(du, 1); u2 = byte_f(du, 2); u3 = byte_f(du, 3); }
#pragma unroll
      for (int j = 0; j < NTn; ++j) {
        const float4 xv = *reinterpret_cast<const float4*>(xrow + j * row_stride + w * St::G + s * 4);
        ag[j] = fmaf(g0, xv.x, ag[j]);
        ag[j] = fmaf(g1, xv.y, ag[j]);
        ag[j] = fmaf(g2, xv.z, ag[j]);
        ag[j] = fmaf(g3, xv.w, ag[j]);
        if constexpr (TWO) {
          au[j] = fmaf(u0, xv.x, au[j]);
          au[j] = fmaf(u1, xv.y, au[j]);
          au[j] = fmaf(u2, xv.z, au[j]);
          au[j] = fmaf(u3, xv.w, au[j]);
        }
      }
    }
  }
}

__device__ inline float scale_of(const uint4& sv, int bb) {
  const uint32_t w = comp(sv, bb >> 1);
  return half_bits_to_f32((uint16_t)((bb & 1) ? (w >> 16) : (w & 0xffffu)));
}

// Main loop over this wave's superblocks for NTn tokens.  TWO: gate+up rows.
template <int FMT, int NTn, bool TWO>
__device__ inline void gemv_rows(const uint8_t* tile_base, size_t sb_stride, size_t mat_stride,
                                 int nsb, const float* xp, const float* xs, int len, float* res_g,
                                 float* res_u) {
  constexpr int NCV = Fmt<FMT>::ncv, NV = NCV + 1;
  constexpr float C = Fmt<FMT>::c;
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6, nw = blockDim.x >> 6;
  const int nblk = len / BLOCK_W;
  for (int sb = wv; sb < nsb; sb += nw) {
    const uint8_t* base = tile_base + sb * sb_stride + lane * 16;
    uint4 gv[NV], uv[NV];
#pragma unroll
    for (int v = 0; v < NV; ++v) gv[v] = *reinterpret_cast<const uint4*>(base + v * 1024);
    if constexpr (TWO) {
#pragma unroll
      for (int v = 0; v < NV; ++v) uv[v] = *reinterpret_cast<const uint4*>(base + mat_stride + v * 1024);
    }
#pragma unroll
    for (int bb = 0; bb < 8; ++bb) {
      float ag[NTn], au[NTn];
#pragma unroll
      for (int j = 0; j < NTn; ++j) { ag[j] = 0.f; au[j] = 0.f; }
      block_dot<FMT, NTn, TWO>(gv, uv, bb, xp + sb * SB_WEIGHTS + bb * BLOCK_W, len, ag, au);
      const float dg = scale_of(gv[NCV], bb);
      float du = 0.f;
      if constexpr (TWO) du = scale_of(uv[NCV], bb);
#pragma unroll
      for (int j = 0; j < NTn; ++j) {
        const float sx = xs[j * nblk + sb * 8 + bb];
        res_g[j] = fmaf(dg, fmaf(-C, sx, ag[j]), res_g[j]);
        if constexpr (TWO) res_u[j] = fmaf(du, fmaf(-C, sx, au[j]), res_u[j]);
      }
    }
  }
}

// token of a slot: routed slots map through the permutation, shared slots
// (slot >= P) are the tokens in order
__device__ inline int slot_token(const ExpertArgs& a, int slot) {
  return slot < a.P ? a.w.perm[slot] / a.k : slot - a.P;
}

template <int FMT, int NT>
__global__ __launch_bounds__(1024) void k_decode_gateup(ExpertArgs a) {
  extern __shared__ float lds[];
  const int u = blockIdx.y;
  if (u >= a.w.meta[0]) return;
  const int tile = blockIdx.x;
  const int e = a.w.uexp[u];
  const int s0 = a.w.uoff[u];
  const int n = a.w.uoff[u + 1] - s0;
  const int H = a.H, nblk = H / BLOCK_W, nsb = H / SB_WEIGHTS;
  float* xp = lds;                 // [NT][H] permuted activations
  float* xs = lds + NT * H;        // [NT][H/32] block sums

  for (int idx = threadIdx.x; idx < NT * H; idx += blockDim.x) {
    const int j = idx / H, h = idx - j * H;
    float v = 0.f;
    if (j < n) v = ld_x(a.x, a.x_f32, (size_t)slot_token(a, s0 + j) * H + h);
    xp[j * H + perm_pos<FMT>(h)] = v;
  }
  __syncthreads();
  for (int idx = threadIdx.x; idx < NT * nblk; idx += blockDim.x) {
    const float* p = xp + (idx / nblk) * H + (idx % nblk) * BLOCK_W;
    float s = 0.f;
#pragma unroll
    for (int i = 0; i < BLOCK_W; ++i) s += p[i];
    xs[idx] = s;
  }
  __syncthreads();

  constexpr int NV = Fmt<FMT>::ncv + 1;
  const uint8_t* tile_base = a.packed + (size_t)e * a.stride + gu_off(NV, nsb, tile, 0, 0, 0);
  const size_t sb_stride = (size_t)2 * NV * 1024, mat_stride = (size_t)NV * 1024;
  float g[NT], uu[NT];
#pragma unroll
  for (int j = 0; j < NT; ++j) { g[j] = 0.f; uu[j] = 0.f; }
  if (n <= 1) gemv_rows<FMT, 1, true>(tile_base, sb_stride, mat_stride, nsb, xp, xs, H, g, uu);
  else if constexpr (NT >= 2) {
    if (n <= 2) gemv_rows<FMT, 2, true>(tile_base, sb_stride, mat_stride, nsb, xp, xs, H, g, uu);
    else if constexpr (NT >= 4) {
      if (n <= 4) gemv_rows<FMT, 4, true>(tile_base, sb_stride, mat_stride, nsb, xp, xs, H, g, uu);
      else if constexpr (NT >= 8) gemv_rows<FMT, 8, true>(tile_base, sb_stride, mat_stride, nsb, xp, xs, H, g, uu);
    }
  }
  __syncthreads();                 // LDS activations no longer needed: reuse for the reduction
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6, nw = blockDim.x >> 6;
  float* red = lds;                // [nw][NT][2][64]
#pragma unroll
  for (int j = 0; j < NT; ++j) {
    red[((wv * NT + j) * 2 + 0) * 64 + lane] = g[j];
    red[((wv * NT + j) * 2 + 1) * 64 + lane] = uu[j];
  }
  __syncthreads();
  float* act = reinterpret_cast<float*>(a.w.act);
  for (int idx = threadIdx.x; idx < n * 64; idx += blockDim.x) {
    const int j = idx >> 6, l = idx & 63;
    float gs = 0.f, us = 0.f;
    for (int w = 0; w < nw; ++w) {
      gs += red[((w * NT + j) * 2 + 0) * 64 + l];
      us += red[((w * NT + j) * 2 + 1) * 64 + l];
    }
    act[(size_t)(s0 + j) * a.I + tile * 64 + l] = silu_f(gs) * us;
  }
}

template <int FMT, int NT>
__global__ __launch_bounds__(1024) void k_decode_down(ExpertArgs a) {
  extern __shared__ float lds[];
  const int u = blockIdx.y;
  const int U = a.w.meta[0];
  if (u >= U) return;
  const int tile = blockIdx.x;
  const int e = a.w.uexp[u];
  const int s0 = a.w.uoff[u];
  const int n = a.w.uoff[u + 1] - s0;
  const int H = a.H, I = a.I, nblk = I / BLOCK_W, nsb = I / SB_WEIGHTS;
  float* ap = lds;                 // [NT][I]
  float* as = lds + NT * I;        // [NT][I/32]
  const float* act = reinterpret_cast<const float*>(a.w.act);
  for (int idx = threadIdx.x; idx < NT * I; idx += blockDim.x) {
    const int j = idx / I, i = idx - j * I;
    ap[j * I + perm_pos<FMT>(i)] = (j < n) ? act[(size_t)(s0 + j) * I + i] : 0.f;
  }
  __syncthreads();
  for (int idx = threadIdx.x; idx < NT * nblk; idx += blockDim.x) {
    const float* p = ap + (idx / nblk) * I + (idx % nblk) * BLOCK_W;
    float s = 0.f;
#pragma unroll
    for (int i = 0; i < BLOCK_W; ++i) s += p[i];
    as[idx] = s;
  }
  __syncthreads();
  constexpr int NV = Fmt<FMT>::ncv + 1;
  const uint8_t* tile_base = a.packed + (size_t)e * a.stride + gu_bytes(FMT, H, I) +
                             dn_off(NV, nsb, tile, 0, 0);
  const size_t sb_stride = (size_t)NV * 1024;
  float r[NT], dummy[NT];
#pragma unroll
  for (int j = 0; j < NT; ++j) { r[j] = 0.f; dummy[j] = 0.f; }
  if (n <= 1) gemv_rows<FMT, 1, false>(tile_base, sb_stride, 0, nsb, ap, as, I, r, dummy);
  else if constexpr (NT >= 2) {
    if (n <= 2) gemv_rows<FMT, 2, false>(tile_base, sb_stride, 0, nsb, ap, as, I, r, dummy);
    else if constexpr (NT >= 4) {
      if (n <= 4) gemv_rows<FMT, 4, false>(tile_base, sb_stride, 0, nsb, ap, as, I, r, dummy);
      else if constexpr (NT >= 8) gemv_rows<FMT, 8, false>(tile_base, sb_stride, 0, nsb, ap, as, I, r, dummy);
    }
  }
  __syncthreads();
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6, nw = blockDim.x >> 6;
  float* red = lds;                // [nw][NT][64]
#pragma unroll
  for (int j = 0; j < NT; ++j) red[(wv * NT + j) * 64 + lane] = r[j];
  __syncthreads();
  for (int idx = threadIdx.x; idx < n * 64; idx += blockDim.x) {
    const int j = idx >> 6, l = idx & 63;
    float s = 0.f;
    for (int w = 0; w < nw; ++w) s += red[(w * NT + j) * 64 + l];
    a.w.y[(size_t)(s0 + j) * H + tile * 64 + l] = s;
  }

  // the last expert to finish this H tile combines it for every token
  __shared__ int s_last;
  __threadfence();
  __syncthreads();
  if (threadIdx.x == 0) s_last = (atomicAdd(&a.w.tickets[tile], 1) == U - 1);
  __syncthreads();
  if (!s_last) return;
  __threadfence();
  const int k = a.k;
  for (int idx = threadIdx.x; idx < a.T * 64; idx += blockDim.x) {
    const int t = idx >> 6, h = tile * 64 + (idx & 63);
    float acc = 0.f;
    for (int j = 0; j < k; ++j) {
      const int p = t * k + j;
      acc = fmaf(a.w.topk_w[p], ld_coherent(a.w.y + (size_t)ld_coherent(a.w.inv + p) * H + h), acc);
    }
    if (a.n_shared) acc += ld_coherent(a.w.y + (size_t)(a.P + t) * H + h);   // weight 1
    const size_t o = (size_t)t * H + h;
    if (a.flags & 2u) acc += ld_x(a.x, a.x_f32, o);
    if (a.flags & 1u) acc += a.out[o];
    a.out[o] = acc;
  }
  if (threadIdx.x == 0)
    __hip_atomic_store(&a.w.tickets[tile], 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

template <int FMT>
hipError_t launch_experts_fmt(const Layer& L, const Work& W, const Call& c, hipStream_t s) {
  ExpertArgs a;
  a.packed = L.packed;
  a.stride = L.expert_stride;
  a.H = L.H; a.I = L.I; a.E = L.E; a.k = L.k; a.T = c.T; a.P = c.T * L.k; a.n_shared = L.n_shared;
  a.x = c.x; a.x_f32 = c.x_f32; a.flags = c.flags; a.out = c.out; a.w = W;
  const int umax = (a.P < L.E ? a.P : L.E) + L.n_shared;
  const int nsbH = L.H / SB_WEIGHTS, nsbI = L.I / SB_WEIGHTS;
  const int nwg = nsbH < 16 ? nsbH : 16, nwd = nsbI < 16 ? nsbI : 16;
  auto lds_gu = [&](int NT) {
    size_t stage = (size_t)NT * (L.H + L.H / BLOCK_W) * 4, red = (size_t)nwg * NT * 128 * 4;
    return stage > red ? stage : red;
  };
  auto lds_dn = [&](int NT) {
    size_t stage = (size_t)NT * (L.I + L.I / BLOCK_W) * 4, red = (size_t)nwd * NT * 64 * 4;
    return stage > red ? stage : red;
  };
  dim3 ggu(L.I / 64, umax), gdn(L.H / 64, umax);
#define STRATA_LAUNCH(NT)                                                                       \
  hipLaunchKernelGGL((k_decode_gateup<FMT, NT>), ggu, dim3(64 * nwg), lds_gu(NT), s, a);       \
  hipLaunchKernelGGL((k_decode_down<FMT, NT>), gdn, dim3(64 * nwd), lds_dn(NT), s, a);
  if (c.T <= 1) { STRATA_LAUNCH(1) }
  else if (c.T <= 2) { STRATA_LAUNCH(2) }
  else if (c.T <= 4) { STRATA_LAUNCH(4) }
  else { STRATA_LAUNCH(8) }
#undef STRATA_LAUNCH
  return hipGetLastError();
}

}  // namespace

hipError_t launch_decode_route(const Layer& L, const Work& W, const Call& c, hipStream_t s) {
  RouteArgs a;
  a.Wr = L.router_w; a.bias = L.router_b; a.x = c.x; a.x_f32 = c.x_f32; a.T = c.T;
  a.H = L.H; a.E = L.E; a.k = L.k; a.n_shared = L.n_shared; a.w = W;
  const size_t lds = (size_t)4 * L.E * 4 + (size_t)c.T * L.k * 4 + (size_t)L.E * 4;
  hipLaunchKernelGGL(k_decode_route, dim3((L.E + 3) / 4), dim3(256), lds, s, a);
  return hipGetLastError();
}

// Raise a kernel's dynamic-LDS ceiling to what the device allows beside its
// static LDS.  A refusal is not fatal (the launch reports it if a call really
// needs more than the default); the runtime's error state is cleared.
static void raise_lds_limit(const void* k, int device_limit) {
  hipFuncAttributes fa;
  if (hipFuncGetAttributes(&fa, k) != hipSuccess) { (void)hipGetLastError(); return; }
  const int want = device_limit - (int)fa.sharedSizeBytes;
  if (want > 0 && hipFuncSetAttribute(k, hipFuncAttributeMaxDynamicSharedMemorySize, want) != hipSuccess)
    (void)hipGetLastError();
}

template <int FMT>
void set_lds_limits(int lim) {
  const void* ks[] = {
      reinterpret_cast<const void*>(&k_decode_gateup<FMT, 1>), reinterpret_cast<const void*>(&k_decode_gateup<FMT, 2>),
      reinterpret_cast<const void*>(&k_decode_gateup<FMT, 4>), reinterpret_cast<const void*>(&k_decode_gateup<FMT, 8>),
      reinterpret_cast<const void*>(&k_decode_down<FMT, 1>), reinterpret_cast<const void*>(&k_decode_down<FMT, 2>),
      reinterpret_cast<const void*>(&k_decode_down<FMT, 4>), reinterpret_cast<const void*>(&k_decode_down<FMT, 8>)};
  for (const void* k : ks) raise_lds_limit(k, lim);
}

// Allow the decode kernels the dynamic LDS the widest decode call needs
// (more than 64 KiB for H = 4096 with 8 tokens).
hipError_t prepare_decode_kernels(const Layer& L, int) {
  int dev = 0, lim = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e == hipSuccess) e = hipDeviceGetAttribute(&lim, hipDeviceAttributeMaxSharedMemoryPerBlock, dev);
  if (e != hipSuccess) return e;
  raise_lds_limit(reinterpret_cast<const void*>(&k_decode_route), lim);
  switch (L.fmt) {
    case 2: set_lds_limits<2>(lim); break;
    case 3: set_lds_limits<3>(lim); break;
    default: set_lds_limits<4>(lim); break;
  }
  return hipSuccess;
}

hipError_t launch_decode_experts(const Layer& L, const Work& W, const Call& c, hipStream_t s) {
  switch (L.fmt) {
    case 2: return launch_experts_fmt<2>(L, W, c, s);
    case 3: return launch_experts_fmt<3>(L, W, c, s);
    default: return launch_experts_fmt<4>(L, W, c, s);
  }
}

}  // namespace strata
