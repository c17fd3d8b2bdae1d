// Shared definitions of the strata_moe HIP library (gfx950, wave64).
//
// Packed expert layout ("packed"), written once by the create-time repack:
//
//   A matrix with R rows and reduction length K is cut into 64-row tiles and
//   256-weight superblocks (8 quantised blocks).  For one tile and one
//   superblock the bytes are NV vectors of 64 rows x 16 B: vector v, row
//   (lane) r sits at  v*1024 + r*16.  NV = NCV code vectors + 1 scale vector
//   (the 8 fp16 scales of the superblock's blocks).  A wavefront reading
//   vector v of a tile therefore issues one fully contiguous 1 KiB load,
//   every lane owning one output row.
//
//   Expert = [gate/up section][down section]:
//     gate/up: tiles of 64 intermediate rows i; per (tile, superblock) the
//              gate vectors then the up vectors (2*NV vectors), so one lane
//              owns gate row i and up row i and SwiGLU stays in-lane;
//     down:    tiles of 64 hidden rows h, K = I.
//   The byte count equals the canonical record's (codes + scales only).
//
//   Code vectors inside one row-superblock:
//     Q2: v = 0..3 holds blocks 2v, 2v+1 (8 B each, canonical bit order);
//     Q4: v = 0..7 holds block v (16 B, canonical nibble order);
//     Q3: v = 0..3 holds the low two bits of blocks 2v, 2v+1 laid out like
//         Q2; v = 4..5 holds the third bit of blocks 4(v-4)..4(v-4)+3, one
//         32-bit word per block, bit (8i + 4w + s) = bit 2 of code 16w+4i+s.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace strata {

constexpr int WAVE = 64;
constexpr int ROWS_PER_TILE = 64;
constexpr int SB_WEIGHTS = 256;        // weights per superblock (8 blocks)
constexpr int BLOCK_W = 32;            // weights per quantised block
constexpr int DECODE_MAX_T = 8;

template <int FMT> struct Fmt;
template <> struct Fmt<2> {
  static constexpr int bits = 2, code_bytes = 8, ncv = 4;
  static constexpr float c = 1.5f;
};
template <> struct Fmt<3> {
  static constexpr int bits = 3, code_bytes = 12, ncv = 6;
  static constexpr float c = 3.5f;
};
template <> struct Fmt<4> {
  static constexpr int bits = 4, code_bytes = 16, ncv = 8;
  static constexpr float c = 8.0f;
};

__host__ __device__ inline int fmt_code_bytes(int fmt) { return fmt == 2 ? 8 : (fmt == 3 ? 12 : 16); }
__host__ __device__ inline int fmt_ncv(int fmt) { return fmt == 2 ? 4 : (fmt == 3 ? 6 : 8); }
__host__ __device__ inline int fmt_nv(int fmt) { return fmt_ncv(fmt) + 1; }
__host__ __device__ inline size_t expert_bytes(int fmt, int H, int I) {
  return (size_t)3 * I * (H / BLOCK_W) * (fmt_code_bytes(fmt) + 2);
}
// bytes of the gate/up section of one expert
__host__ __device__ inline size_t gu_bytes(int fmt, int H, int I) {
  return (size_t)2 * I * (H / BLOCK_W) * (fmt_code_bytes(fmt) + 2);
}
// byte offset of (tile, superblock, matrix m in {0 gate, 1 up}, vector v) in the gate/up section
__host__ __device__ inline size_t gu_off(int nv, int nsbH, int tile, int sb, int m, int v) {
  return ((((size_t)tile * nsbH + sb) * 2 + m) * nv + v) * 1024;
}
// byte offset of (tile, superblock, vector v) in the down section (relative to its start)
__host__ __device__ inline size_t dn_off(int nv, int nsbI, int tile, int sb, int v) {
  return (((size_t)tile * nsbI + sb) * nv + v) * 1024;
}

// ------------------------------------------------------------------ device helpers
__device__ inline float bf16_to_f32(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

__device__ inline uint16_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

__device__ inline float half_bits_to_f32(uint16_t h) {
  _Float16 v;
  __builtin_memcpy(&v, &h, 2);
  return (float)v;
}

__device__ inline float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, WAVE);
  return v;
}

// argmax over the wave of (value, index); ties resolved towards the smaller index
__device__ inline void wave_argmax(float& v, int& i) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    float ov = __shfl_xor(v, o, WAVE);
    int oi = __shfl_xor(i, o, WAVE);
    if (ov > v || (ov == v && oi < i)) { v = ov; i = oi; }
  }
}

__device__ inline float silu_f(float g) { return g / (1.0f + expf(-g)); }

// Top-k of one token's logits row[0..E) (LDS or global), computed by one
// wave.  Round r selects the best entry ranked after round r-1's winner in
// the total order (value descending, id ascending), so nothing is written
// back to the row and equal values resolve to the lower id.  NaN ranks as
// -inf, so k <= E rounds always yield k distinct valid ids.  Writes the ids
// in ascending order to idx_out[0..k) and the renormalised softmax weights
// to w_out[0..k).  k <= 64.  Every lane of the wave must call it.
__device__ inline void wave_topk(const float* row, int E, int k, int* idx_out, float* w_out,
                                 int* sel_lds) {
  const int lane = threadIdx.x & (WAVE - 1);
  float my_val = 0.f, top = 0.f, pv = INFINITY;
  int my_id = 0, pi = -1;
  for (int r = 0; r < k; ++r) {
    float bv = -INFINITY;
    int bi = 0x7fffffff;
    for (int e = lane; e < E; e += WAVE) {
      float v = row[e];
      v = (v != v) ? -INFINITY : v;
      bool after = (v < pv) || (v == pv && e > pi);
      if (after && (v > bv || (v == bv && e < bi))) { bv = v; bi = e; }
    }
    wave_argmax(bv, bi);
    if (r == 0) top = bv;
    if (lane == r) { my_val = bv; my_id = bi; }
    pv = bv;
    pi = bi;
  }
  // renormalised softmax over the selected logits
  float z = (lane < k) ? expf(my_val - top) : 0.f;
  float s = wave_sum(z);
  if (lane < k) sel_lds[lane] = my_id;
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  if (lane < k) {
    int pos = 0;
    for (int j = 0; j < k; ++j) pos += (sel_lds[j] < my_id);
    idx_out[pos] = my_id;
    w_out[pos] = z / s;
  }
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
}

// Exclusive scan of an int2 over the workgroup (<= 16 waves); *total gets the sum.
__device__ inline int2 block_exclusive_scan(int2 v, int2* tmp /* >= 16 */, int2* total) {
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6, nw = blockDim.x >> 6;
  int2 inc = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    int ax = __shfl_up(inc.x, o, 64), ay = __shfl_up(inc.y, o, 64);
    if (lane >= o) { inc.x += ax; inc.y += ay; }
  }
  if (lane == 63) tmp[wv] = inc;
  __syncthreads();
  int2 pre = make_int2(0, 0), tot = make_int2(0, 0);
  for (int i = 0; i < nw; ++i) {
    if (i < wv) { pre.x += tmp[i].x; pre.y += tmp[i].y; }
    tot.x += tmp[i].x;
    tot.y += tmp[i].y;
  }
  *total = tot;
  __syncthreads();
  return make_int2(pre.x + inc.x - v.x, pre.y + inc.y - v.y);
}

}  // namespace strata
