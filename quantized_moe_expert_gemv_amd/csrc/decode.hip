// Decode path (T <= 8 tokens): the per-token expert GEMV regime of the
// pages (ai-coding.wiselychen.com "Strata two weeks", section 成功思路一: per
// layer the GPU runs the router, picks 10 experts and computes them; the
// expert step is bound by the bytes of expert weights read), including the
// 1+3-token MTP verify window (devotd.net "Strata memory tiers", section
// 用草拟 token 提高生成速度的 MTP) where tokens that pick the same expert share
// one read of its weights (blog.5616760.com/0039.html, section 十二).
//
// Four launches per layer:
//   k_route_gemv  router GEMV, one wave per expert row (fp32, the row held
//                 in registers); each workgroup also writes a slice of the
//                 tokens as three fp16 parts (x = p0 + p1 + p2 exactly);
//   k_topk        one workgroup: top-k + renormalised softmax per token, the
//                 stable token->expert permutation, one descriptor per active
//                 expert (id, first slot, token ids) and a dense table of
//                 routing weights per (active expert, token);
//   k_gateup      one workgroup per (active expert, 64 rows of I); waves split
//                 the H superblocks; gate and up rows of the same i stay in
//                 one lane; writes silu(g) * u as three fp16 parts per pair;
//   k_down        one workgroup per 32 rows of H; waves take (active expert,
//                 superblock) units, scale each expert's rows by its routing
//                 weights and the workgroup reduces them in a fixed order:
//                 the weighted combine happens here, with no cross-workgroup
//                 synchronisation.
//
// The multiply-accumulate runs on the matrix cores (16x16x32 fp16 MFMA, fp32
// accumulation) with exact operands: the code q of a weight becomes the fp16
// value q (2-bit codes through the FP4->fp16 conversion, Q3 as a 2-bit and a
// 1-bit plane) or (q - 8)/16 (Q4, magic-number construction), the
// activations enter as their three fp16 parts, and the per-block offset
// -c * sum_j x_j comes from one extra MFMA against a constant operand.  Every
// product is exact; only the fp32 accumulation rounds.  The fp16 block scale
// d multiplies each block's 16x16 result in fp32.
#include "common.hpp"
#include "kernels.hpp"

namespace strata {
namespace {

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef __attribute__((__vector_size__(8 * sizeof(_Float16)))) _Float16 f16x8;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;

constexpr int DESC = 16;   // ints per active-expert descriptor: e, first slot, n, 0, tokens[8], pad
constexpr int WTAB = 8;    // routing weights per active expert, indexed by token
constexpr int NPART = 3;   // fp16 parts of an fp32 activation

__device__ inline float4 bf16x4(uint32_t lo, uint32_t hi) {
  return make_float4(__uint_as_float(lo << 16), __uint_as_float(lo & 0xffff0000u),
                     __uint_as_float(hi << 16), __uint_as_float(hi & 0xffff0000u));
}

__device__ inline uint32_t comp(const uint4& v, int i) {
  return i == 0 ? v.x : (i == 1 ? v.y : (i == 2 ? v.z : v.w));
}

// x = p0 + p1 + p2 with fp16 parts (exact for fp32 values of fp16 range)
__device__ inline void split3(float x, _Float16* p) {
  p[0] = (_Float16)x;
  float r = x - (float)p[0];
  p[1] = (_Float16)r;
  r -= (float)p[1];
  p[2] = (_Float16)r;
}

__device__ inline f32x4 mfma(const f16x8& a, const f16x8& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

__device__ inline f16x8 as_f16x8(const uint4& v) { return __builtin_bit_cast(f16x8, v); }

__device__ inline f16x8 join(half2_t a, half2_t b, half2_t c, half2_t d) {
  f16x8 r;
  r[0] = a.x; r[1] = a.y; r[2] = b.x; r[3] = b.y;
  r[4] = c.x; r[5] = c.y; r[6] = d.x; r[7] = d.y;
  return r;
}

// ------------------------------------------------------------------ weight operands
// Codes of one lane of a slab (see common.hpp for the bit order).
template <int FMT> struct Codes;
template <> struct Codes<2> { uint4 lo; };
template <> struct Codes<3> { uint4 lo; uint2 hi; };
template <> struct Codes<4> { uint4 v0, v1; };

template <int FMT>
__device__ inline void load_codes(const uint8_t* slab, int lane, Codes<FMT>& c) {
  if constexpr (FMT == 4) {
    c.v0 = *reinterpret_cast<const uint4*>(slab + lane * 16);
    c.v1 = *reinterpret_cast<const uint4*>(slab + 1024 + lane * 16);
  } else {
    c.lo = *reinterpret_cast<const uint4*>(slab + lane * 16);
    if constexpr (FMT == 3) c.hi = *reinterpret_cast<const uint2*>(slab + 1024 + lane * 8);
  }
}

// The 8 codes of block BB (this lane's K-slice) as fp16 values q.
template <int BB>
__device__ inline f16x8 lo2_operand(const uint4& lo) {
  const uint32_t W = comp(lo, BB >> 1);
  const uint32_t E = W & 0x33333333u, O = (W >> 2) & 0x33333333u;
  constexpr int b0 = 2 * (BB & 1);
  return join(__builtin_amdgcn_cvt_scalef32_pk_f16_fp4(E, 2.0f, b0),
              __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(O, 2.0f, b0),
              __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(E, 2.0f, b0 + 1),
              __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(O, 2.0f, b0 + 1));
}

// Third bit of the Q3 codes of block BB as fp16 values 4 * bit.
template <int BB>
__device__ inline f16x8 hi3_operand(const uint2& hi) {
  const uint32_t Hd = (BB >> 2) ? hi.y : hi.x;
  const uint32_t X = (Hd >> (BB & 3)) & 0x11111111u;
  return join(__builtin_amdgcn_cvt_scalef32_pk_f16_fp4(X, 8.0f, 0),
              __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(X, 8.0f, 1),
              __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(X, 8.0f, 2),
              __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(X, 8.0f, 3));
}

// Q4 codes of block BB as fp16 values (q - 8) / 16: 1 + q/16 from the bit
// pattern 0x3C00 | q << 6, minus 1.5 (both steps exact).
template <int BB>
__device__ inline f16x8 q4_operand(const Codes<4>& c) {
  const uint32_t W = comp((BB >> 2) ? c.v1 : c.v0, BB & 3);
  const half2_t off = {(_Float16)-1.5f, (_Float16)-1.5f};
  half2_t p[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const uint32_t t = (k == 0) ? (W << 6) : (k == 1) ? (W << 2) : (k == 2) ? (W >> 2) : (W >> 6);
    const uint32_t bits = (t & 0x03C003C0u) | 0x3C003C00u;
    p[k] = __builtin_bit_cast(half2_t, bits) + off;
  }
  return join(p[0], p[1], p[2], p[3]);
}

// scale of block BB of this lane's row; Q4 folds in the factor 16
template <int FMT, int BB>
__device__ inline float block_scale(const uint4& sc) {
  const uint32_t w = comp(sc, BB >> 1);
  const float d = half_bits_to_f32((uint16_t)((BB & 1) ? (w >> 16) : (w & 0xffffu)));
  return FMT == 4 ? 16.0f * d : d;
}

// D = A * B(codes of block BB) + Doff, in fp32
template <int FMT, int BB>
__device__ inline f32x4 block_product(const f16x8& a, const Codes<FMT>& c, const f32x4& doff) {
  if constexpr (FMT == 4) {
    return mfma(a, q4_operand<BB>(c), doff);
  } else {
    f32x4 d = mfma(a, lo2_operand<BB>(c.lo), doff);
    if constexpr (FMT == 3) d = mfma(a, hi3_operand<BB>(c.hi), d);
    return d;
  }
}

// the block offset -c * sum_j x_j, for every output column
template <int FMT>
__device__ inline f32x4 block_offset(const f16x8& a) {
  const f32x4 z = {0.f, 0.f, 0.f, 0.f};
  if constexpr (FMT == 4) {
    return z;
  } else {
    f16x8 cst;
#pragma unroll
    for (int i = 0; i < 8; ++i) cst[i] = (_Float16)(-Fmt<FMT>::c);
    return mfma(a, cst, z);
  }
}

// sum over the three part rows of the 16x16 result (lane groups 0..2; group 3 holds zeros)
__device__ inline float sum_parts(float v) {
  v += __shfl_xor(v, 16, WAVE);
  v += __shfl_xor(v, 32, WAVE);
  return v;
}

// ------------------------------------------------------------------ router
struct RouteArgs {
  const float* Wr;
  const float* bias;
  const void* x;
  int x_f32, T, H, E;
  float* logits;
  _Float16* xparts;
};

// T rows of x -> fp32 LDS (natural order): batches of 16 loads per thread,
// all issued before any is used (indices clamped into the input)
__device__ inline void stage_x(const void* x, int x_f32, int T, int H, float* xs) {
  const int tid = threadIdx.x, nt = blockDim.x;
  float4* dst = reinterpret_cast<float4*>(xs);
  if (x_f32) {
    const float4* src = reinterpret_cast<const float4*>(x);
    const int n4 = T * H / 4;
    for (int b = tid; b < n4; b += 16 * nt) {
      float4 r[16];
#pragma unroll
      for (int q = 0; q < 16; ++q) r[q] = src[min(b + q * nt, n4 - 1)];
#pragma unroll
      for (int q = 0; q < 16; ++q) if (b + q * nt < n4) dst[b + q * nt] = r[q];
    }
  } else {
    const uint4* src = reinterpret_cast<const uint4*>(x);
    const int n8 = T * H / 8;
    for (int b = tid; b < n8; b += 16 * nt) {
      uint4 r[16];
#pragma unroll
      for (int q = 0; q < 16; ++q) r[q] = src[min(b + q * nt, n8 - 1)];
#pragma unroll
      for (int q = 0; q < 16; ++q) {
        const int i = b + q * nt;
        if (i < n8) {
          dst[2 * i] = bf16x4(r[q].x, r[q].y);
          dst[2 * i + 1] = bf16x4(r[q].z, r[q].w);
        }
      }
    }
  }
}

__global__ __launch_bounds__(256) void k_route_gemv(RouteArgs a) {
  extern __shared__ float xs[];                // [T][H] fp32
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int H = a.H, E = a.E, T = a.T;
  const int e = blockIdx.x * 4 + wv;
  const int nc = H >> 8;                       // float4 per lane
  const bool have_row = e < E;
  // all 16 loads issued unconditionally (indices clamped into the row), used only for c < nc
  float4 wr[16];
  {
    const float4* row = reinterpret_cast<const float4*>(a.Wr + (size_t)(have_row ? e : 0) * H);
#pragma unroll
    for (int c = 0; c < 16; ++c) wr[c] = row[lane + 64 * (c < nc ? c : nc - 1)];
  }
  const float bias = (have_row && a.bias) ? a.bias[e] : 0.f;
  stage_x(a.x, a.x_f32, T, H, xs);
  __syncthreads();
  // this workgroup's slice of the token rows as fp16 parts [t][part][H]
  const int chunk = ((H + gridDim.x - 1) / gridDim.x + 7) & ~7;
  const int h0 = blockIdx.x * chunk, len = min(H, h0 + chunk) - h0;
  for (int idx = tid; idx < T * len; idx += blockDim.x) {
    const int t = idx / len, h = h0 + idx % len;
    _Float16 p[NPART];
    split3(xs[(size_t)t * H + h], p);
#pragma unroll
    for (int q = 0; q < NPART; ++q) a.xparts[((size_t)t * NPART + q) * H + h] = p[q];
  }
  if (have_row) {
    float acc[DECODE_MAX_T];
#pragma unroll
    for (int t = 0; t < DECODE_MAX_T; ++t) acc[t] = 0.f;
#pragma unroll
    for (int c = 0; c < 16; ++c) {
      if (c < nc) {
#pragma unroll
        for (int t = 0; t < DECODE_MAX_T; ++t) {
          if (t < T) {
            const float4 xv = *reinterpret_cast<const float4*>(xs + (size_t)t * H + 4 * (lane + 64 * c));
            acc[t] = fmaf(wr[c].x, xv.x, acc[t]);
            acc[t] = fmaf(wr[c].y, xv.y, acc[t]);
            acc[t] = fmaf(wr[c].z, xv.z, acc[t]);
            acc[t] = fmaf(wr[c].w, xv.w, acc[t]);
          }
        }
      }
    }
#pragma unroll
    for (int t = 0; t < DECODE_MAX_T; ++t) {
      if (t < T) {
        const float s = wave_sum(acc[t]);
        if (lane == 0) a.logits[(size_t)t * E + e] = s + bias;
      }
    }
  }
}

// ------------------------------------------------------------------ top-k + permutation
struct TopkArgs {
  int T, E, k, n_shared;
  Work w;
};

// T tokens, one wave each (512 threads); LDS: T*k + 2E ints.
__global__ __launch_bounds__(512) void k_topk(TopkArgs a) {
  extern __shared__ int lds_i[];
  __shared__ int s_sel[8][64];
  __shared__ int2 tmp[16];
  const int tid = threadIdx.x, wv = tid >> 6, nt = blockDim.x;
  const int E = a.E, k = a.k, T = a.T, P = T * k;
  int* sel = lds_i;        // [T][k]
  int* hist = sel + P;     // [E] counts, then offsets
  int* uidx = hist + E;    // [E] active-expert index
  if (wv < T)
    wave_topk_any(a.w.logits + (size_t)wv * E, E, k, sel + wv * k, a.w.topk_w + (size_t)wv * k, s_sel[wv]);
  for (int e = tid; e < E; e += nt) hist[e] = 0;
  __syncthreads();
  for (int p = tid; p < P; p += nt) {
    a.w.topk_idx[p] = sel[p];
    atomicAdd(&hist[sel[p]], 1);
  }
  __syncthreads();
  // exclusive scans over experts of (count, non-empty), contiguous chunks per thread
  const int per = (E + nt - 1) / nt;
  const int e0 = tid * per, e1 = min(E, e0 + per);
  int2 loc = make_int2(0, 0);
  for (int e = e0; e < e1; ++e) { loc.x += hist[e]; loc.y += (hist[e] > 0); }
  int2 total;
  int2 base = block_exclusive_scan(loc, tmp, &total);
  for (int e = e0; e < e1; ++e) {
    const int c = hist[e];
    a.w.counts[e] = c;
    a.w.offsets[e] = base.x;
    hist[e] = base.x;
    if (c > 0) {
      uidx[e] = base.y;
      *reinterpret_cast<int4*>(a.w.udesc + (size_t)base.y * DESC) = make_int4(e, base.x, c, 0);
      float4* wt = reinterpret_cast<float4*>(a.w.wtab + (size_t)base.y * WTAB);
      wt[0] = make_float4(0.f, 0.f, 0.f, 0.f);
      wt[1] = make_float4(0.f, 0.f, 0.f, 0.f);
    }
    base.x += c;
    base.y += (c > 0);
  }
  __syncthreads();
  // stable slot of every pair: earlier tokens that chose the same expert go first
  for (int p = tid; p < P; p += nt) {
    const int t = p / k, e = sel[p];
    int rank = 0;
    for (int t2 = 0; t2 < t; ++t2)
      for (int j = 0; j < k; ++j) rank += (sel[t2 * k + j] == e);
    const int slot = hist[e] + rank;
    a.w.perm[slot] = p;
    a.w.inv[p] = slot;
    a.w.udesc[(size_t)uidx[e] * DESC + 4 + rank] = t;
    a.w.wtab[(size_t)uidx[e] * WTAB + t] = a.w.topk_w[p];
  }
  if (tid == 0) {
    const int U = total.y;
    a.w.offsets[E] = P;
    if (a.n_shared) {
      *reinterpret_cast<int4*>(a.w.udesc + (size_t)U * DESC) = make_int4(E, P, T, 0);
      for (int t = 0; t < DECODE_MAX_T; ++t) {
        a.w.udesc[(size_t)U * DESC + 4 + t] = t;
        a.w.wtab[(size_t)U * WTAB + t] = (t < T) ? 1.0f : 0.0f;
      }
      a.w.meta[0] = U + 1;
    } else {
      a.w.meta[0] = U;
    }
  }
}

// ------------------------------------------------------------------ experts
struct ExpertArgs {
  const uint8_t* packed;
  size_t stride;
  int H, I, E, k, T, P;
  const void* x;
  int x_f32;
  uint32_t flags;
  float* out;
  Work w;
};

__device__ inline int desc_token(const int4& d1, const int4& d2, int j) {
  const int4 v = (j < 4) ? d1 : d2;
  const int q = j & 3;
  return q == 0 ? v.x : (q == 1 ? v.y : (q == 2 ? v.z : v.w));
}

// gate/up: a workgroup covers 2 row groups (32 rows i) of one active expert;
// its waves split the H superblocks, each wave 2 gate + 2 up slabs per
// superblock; partial sums meet in LDS.
constexpr int GU_GROUPS = 2;
constexpr int GU_SLABS = 2 * GU_GROUPS;

template <int FMT, int NTG>
__global__ __launch_bounds__(640) void k_gateup(ExpertArgs a) {
  extern __shared__ float red[];               // [nw][NTG][GU_SLABS][4 tokens][16 rows]
  const int u = blockIdx.y, gp = blockIdx.x;
  const int4* dsc = reinterpret_cast<const int4*>(a.w.udesc + (size_t)u * DESC);
  const int4 d0 = dsc[0], d1 = dsc[1], d2 = dsc[2];
  if (u >= a.w.meta[0]) return;
  const int e = d0.x, s0 = d0.y, n = d0.z;
  const int H = a.H, I = a.I, nsb = H / SB_WEIGHTS;
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6, nw = blockDim.x >> 6;
  const int r = lane & 15, ks = lane >> 4;          // weight row in the group, K-slice
  const int part = (lane & 15) >> 2, jj = lane & 3;  // A-operand row of this lane: (part, token)
  const uint8_t* gate = a.packed + (size_t)e * a.stride;
  const uint8_t* up = gate + up_off(FMT, H, I);
  constexpr int SLAB = Fmt<FMT>::slab_codes + 256;

  for (int tg = 0; tg < NTG; ++tg) {                // token groups of 4
    float acc[GU_SLABS][4];
#pragma unroll
    for (int s = 0; s < GU_SLABS; ++s)
#pragma unroll
      for (int v = 0; v < 4; ++v) acc[s][v] = 0.f;
    const int j = 4 * tg + jj;
    const bool valid = part < NPART && j < n;
    const _Float16* xsrc = a.w.xparts + ((size_t)(valid ? desc_token(d1, d2, j) : 0) * NPART +
                                         (valid ? part : 0)) * H + 8 * ks;
    for (int sb = wv; sb < nsb; sb += nw) {
      Codes<FMT> cd[GU_SLABS];
      uint4 sc[GU_SLABS];
#pragma unroll
      for (int s = 0; s < GU_SLABS; ++s) {
        const uint8_t* slab = (s < GU_GROUPS ? gate : up) +
                              ((size_t)(GU_GROUPS * gp + (s % GU_GROUPS)) * nsb + sb) * SLAB;
        load_codes<FMT>(slab, lane, cd[s]);
        sc[s] = *reinterpret_cast<const uint4*>(slab + Fmt<FMT>::slab_codes + r * 16);
      }
      uint4 av[8];
#pragma unroll
      for (int bb = 0; bb < 8; ++bb)
        av[bb] = valid ? *reinterpret_cast<const uint4*>(xsrc + sb * SB_WEIGHTS + bb * BLOCK_W)
                       : make_uint4(0, 0, 0, 0);
#define STRATA_BLOCK(BB)                                                          \
      {                                                                           \
        const f16x8 af = as_f16x8(av[BB]);                                        \
        const f32x4 off = block_offset<FMT>(af);                                  \
        f32x4 d[GU_SLABS];                                                        \
        _Pragma("unroll") for (int s = 0; s < GU_SLABS; ++s)                      \
          d[s] = block_product<FMT, BB>(af, cd[s], off);                          \
        _Pragma("unroll") for (int s = 0; s < GU_SLABS; ++s) {                    \
          const float ds = block_scale<FMT, BB>(sc[s]);                           \
          _Pragma("unroll") for (int v = 0; v < 4; ++v)                           \
            acc[s][v] = fmaf(ds, d[s][v], acc[s][v]);                             \
        }                                                                         \
      }
      STRATA_BLOCK(0) STRATA_BLOCK(1) STRATA_BLOCK(2) STRATA_BLOCK(3)
      STRATA_BLOCK(4) STRATA_BLOCK(5) STRATA_BLOCK(6) STRATA_BLOCK(7)
#undef STRATA_BLOCK
    }
    // parts -> lanes 0..15 hold (row r, token v) of each slab
#pragma unroll
    for (int s = 0; s < GU_SLABS; ++s)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const float t = sum_parts(acc[s][v]);
        if (lane < 16) red[((((size_t)wv * NTG + tg) * GU_SLABS + s) * 4 + v) * 16 + lane] = t;
      }
  }
  __syncthreads();
  for (int idx = threadIdx.x; idx < NTG * 4 * GU_GROUPS * 16; idx += blockDim.x) {
    const int row = idx & 15, gi = (idx >> 4) % GU_GROUPS, v = (idx / (16 * GU_GROUPS)) & 3;
    const int tg = idx / (64 * GU_GROUPS);
    const int j = 4 * tg + v;
    if (j >= n) continue;
    float g = 0.f, uu = 0.f;
    for (int w = 0; w < nw; ++w) {
      g += red[((((size_t)w * NTG + tg) * GU_SLABS + gi) * 4 + v) * 16 + row];
      uu += red[((((size_t)w * NTG + tg) * GU_SLABS + GU_GROUPS + gi) * 4 + v) * 16 + row];
    }
    const float act = silu_f(g) * uu;
    _Float16 p[NPART];
    split3(act, p);
    const int i = (GU_GROUPS * gp + gi) * 16 + row;
#pragma unroll
    for (int q = 0; q < NPART; ++q) a.w.actp[((size_t)(s0 + j) * NPART + q) * I + i] = p[q];
  }
}

// down + weighted combine: one 16-row group of H per workgroup, every active
// expert; waves take (expert, superblock) units, the next unit's loads in
// flight while the current one computes.  Descriptors and routing weights of
// all active experts sit in LDS.
template <int FMT> struct DownUnit {
  Codes<FMT> cd;
  uint4 sc;
  uint4 av[8];
};

template <int FMT>
__device__ inline void down_load(const ExpertArgs& a, const int* ldesc, int unit, int nsb, int g,
                                 int tg, DownUnit<FMT>& du) {
  const int lane = threadIdx.x & 63, r = lane & 15, ks = lane >> 4;
  const int part = (lane & 15) >> 2, jj = lane & 3;
  const int u = unit / nsb, sb = unit % nsb;
  const int* d = ldesc + u * DESC;
  const int e = d[0], s0 = d[1], n = d[2];
  const uint8_t* slab = a.packed + (size_t)e * a.stride + down_off(FMT, a.H, a.I) +
                        ((size_t)g * nsb + sb) * (Fmt<FMT>::slab_codes + 256);
  load_codes<FMT>(slab, lane, du.cd);
  du.sc = *reinterpret_cast<const uint4*>(slab + Fmt<FMT>::slab_codes + r * 16);
  // A row (part, token t = 4tg + jj): the pair slot of (expert u, token t), if routed
  const int t = 4 * tg + jj;
  int slot = -1;
  for (int j = 0; j < n; ++j)
    if (d[4 + j] == t) slot = s0 + j;
  const bool valid = part < NPART && slot >= 0;
  const _Float16* src = a.w.actp + ((size_t)(valid ? slot : 0) * NPART + (valid ? part : 0)) * a.I +
                        sb * SB_WEIGHTS + 8 * ks;
#pragma unroll
  for (int bb = 0; bb < 8; ++bb)
    du.av[bb] = valid ? *reinterpret_cast<const uint4*>(src + bb * BLOCK_W) : make_uint4(0, 0, 0, 0);
}

template <int FMT>
__device__ inline void down_compute(const DownUnit<FMT>& du, float* acc /* [4] */) {
  f32x4 dd[2];
#define STRATA_BLOCK(BB)                                                          \
  {                                                                               \
    const f16x8 af = as_f16x8(du.av[BB]);                                         \
    dd[BB & 1] = block_product<FMT, BB>(af, du.cd, block_offset<FMT>(af));        \
    if (BB > 0) {                                                                 \
      const float ds = block_scale<FMT, (BB > 0 ? BB - 1 : 0)>(du.sc);            \
      _Pragma("unroll") for (int v = 0; v < 4; ++v)                               \
        acc[v] = fmaf(ds, dd[(BB - 1) & 1][v], acc[v]);                           \
    }                                                                             \
  }
  STRATA_BLOCK(0) STRATA_BLOCK(1) STRATA_BLOCK(2) STRATA_BLOCK(3)
  STRATA_BLOCK(4) STRATA_BLOCK(5) STRATA_BLOCK(6) STRATA_BLOCK(7)
#undef STRATA_BLOCK
  const float ds = block_scale<FMT, 7>(du.sc);
#pragma unroll
  for (int v = 0; v < 4; ++v) acc[v] = fmaf(ds, dd[1][v], acc[v]);
}

template <int FMT, int NTG>
__global__ __launch_bounds__(512) void k_down(ExpertArgs a) {
  extern __shared__ float lds_dn[];
  const int U = a.w.meta[0];
  const int H = a.H, I = a.I, nsb = I / SB_WEIGHTS, T = a.T;
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6, nw = blockDim.x >> 6;
  const int g = blockIdx.x;
  int* ldesc = reinterpret_cast<int*>(lds_dn);                  // [U][DESC]
  float* lwt = reinterpret_cast<float*>(ldesc + U * DESC);      // [U][WTAB]
  float* red = lwt + U * WTAB;                                  // [nw][NTG][4][16]
  for (int i = threadIdx.x; i < U * DESC; i += blockDim.x) ldesc[i] = a.w.udesc[i];
  for (int i = threadIdx.x; i < U * WTAB; i += blockDim.x) lwt[i] = a.w.wtab[i];
  __syncthreads();

  const int units = U * nsb;
  for (int tg = 0; tg < NTG; ++tg) {
    float out[4] = {0.f, 0.f, 0.f, 0.f};
    DownUnit<FMT> cur, nxt;
    if (wv < units) down_load<FMT>(a, ldesc, wv, nsb, g, tg, cur);
    for (int unit = wv; unit < units; unit += nw) {
      if (unit + nw < units) down_load<FMT>(a, ldesc, unit + nw, nsb, g, tg, nxt);
      float acc[4] = {0.f, 0.f, 0.f, 0.f};
      down_compute<FMT>(cur, acc);
      // routing weight of token 4tg + v for this unit's expert (0 when not routed)
      const float* wt = lwt + (unit / nsb) * WTAB + 4 * tg;
#pragma unroll
      for (int v = 0; v < 4; ++v) out[v] = fmaf(wt[v], acc[v], out[v]);
      cur = nxt;
    }
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const float t = sum_parts(out[v]);
      if (lane < 16) red[(((size_t)wv * NTG + tg) * 4 + v) * 16 + lane] = t;
    }
  }
  __syncthreads();
  for (int idx = threadIdx.x; idx < NTG * 4 * 16; idx += blockDim.x) {
    const int row = idx & 15, v = (idx >> 4) & 3, tg = idx >> 6;
    const int t = 4 * tg + v;
    if (t >= T) continue;
    float s = 0.f;
    for (int w = 0; w < nw; ++w) s += red[(((size_t)w * NTG + tg) * 4 + v) * 16 + row];
    const int h = g * 16 + row;
    const size_t o = (size_t)t * H + h;
    if (a.flags & 2u) {
      s += a.x_f32 ? reinterpret_cast<const float*>(a.x)[o]
                   : bf16_to_f32(reinterpret_cast<const uint16_t*>(a.x)[o]);
    }
    if (a.flags & 1u) s += a.out[o];
    a.out[o] = s;
  }
}

template <int FMT, int NTG>
hipError_t launch_experts_t(const Layer& L, const Work& W, const Call& c, hipStream_t s, Tracer* tr) {
  ExpertArgs a;
  a.packed = L.packed;
  a.stride = L.expert_stride;
  a.H = L.H; a.I = L.I; a.E = L.E; a.k = L.k; a.T = c.T; a.P = c.T * L.k;
  a.x = c.x; a.x_f32 = c.x_f32; a.flags = c.flags; a.out = c.out; a.w = W;
  const int umax = (a.P < L.E ? a.P : L.E) + L.n_shared;
  // gate/up waves: the largest divisor of the superblock count that is <= 10,
  // so every wave takes the same number of superblocks
  const int nsbH = L.H / SB_WEIGHTS;
  int nwg = 1;
  for (int d = 1; d <= 10; ++d)
    if (nsbH % d == 0) nwg = d;
  const int nwd = 8;
  const size_t lds_gu = (size_t)nwg * NTG * GU_SLABS * 4 * 16 * 4;
  const size_t lds_dn = (size_t)umax * (DESC + WTAB) * 4 + (size_t)nwd * NTG * 4 * 16 * 4;
  hipLaunchKernelGGL((k_gateup<FMT, NTG>), dim3(L.I / (16 * GU_GROUPS), umax), dim3(64 * nwg), lds_gu, s, a);
  mark(tr, s);
  hipLaunchKernelGGL((k_down<FMT, NTG>), dim3(L.H / 16), dim3(64 * nwd), lds_dn, s, a);
  mark(tr, s);
  return hipGetLastError();
}

template <int FMT>
hipError_t launch_experts_fmt(const Layer& L, const Work& W, const Call& c, hipStream_t s, Tracer* tr) {
  return c.T <= 4 ? launch_experts_t<FMT, 1>(L, W, c, s, tr) : launch_experts_t<FMT, 2>(L, W, c, s, tr);
}

// Raise a kernel's dynamic-LDS ceiling to what the device allows beside its
// static LDS.  A refusal is not fatal (the launch reports it if a call really
// needs more than the default); the runtime's error state is cleared.
void raise_lds_limit(const void* k, int device_limit) {
  hipFuncAttributes fa;
  if (hipFuncGetAttributes(&fa, k) != hipSuccess) { (void)hipGetLastError(); return; }
  const int want = device_limit - (int)fa.sharedSizeBytes;
  if (want > 0 && hipFuncSetAttribute(k, hipFuncAttributeMaxDynamicSharedMemorySize, want) != hipSuccess)
    (void)hipGetLastError();
}

}  // namespace

// Allow the decode kernels the dynamic LDS the widest decode call needs
// (the router stages up to 8 x 4096 fp32 activations: 128 KiB).
hipError_t prepare_decode_kernels(const Layer& L, int) {
  int dev = 0, lim = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e == hipSuccess) e = hipDeviceGetAttribute(&lim, hipDeviceAttributeMaxSharedMemoryPerBlock, dev);
  if (e != hipSuccess) return e;
  raise_lds_limit(reinterpret_cast<const void*>(&k_route_gemv), lim);
  raise_lds_limit(reinterpret_cast<const void*>(&k_topk), lim);
  return hipSuccess;
}

hipError_t launch_decode_route(const Layer& L, const Work& W, const Call& c, hipStream_t s, Tracer* tr) {
  RouteArgs a;
  a.Wr = L.router_w; a.bias = L.router_b; a.x = c.x; a.x_f32 = c.x_f32; a.T = c.T;
  a.H = L.H; a.E = L.E; a.logits = W.logits; a.xparts = W.xparts;
  mark(tr, s);
  hipLaunchKernelGGL(k_route_gemv, dim3((L.E + 3) / 4), dim3(256), (size_t)c.T * L.H * 4, s, a);
  mark(tr, s);
  TopkArgs t;
  t.T = c.T; t.E = L.E; t.k = L.k; t.n_shared = L.n_shared; t.w = W;
  hipLaunchKernelGGL(k_topk, dim3(1), dim3(512), ((size_t)c.T * L.k + 2 * (size_t)L.E) * 4, s, t);
  mark(tr, s);
  return hipGetLastError();
}

hipError_t launch_decode_experts(const Layer& L, const Work& W, const Call& c, hipStream_t s, Tracer* tr) {
  switch (L.fmt) {
    case 2: return launch_experts_fmt<2>(L, W, c, s, tr);
    case 3: return launch_experts_fmt<3>(L, W, c, s, tr);
    default: return launch_experts_fmt<4>(L, W, c, s, tr);
  }
}

}  // namespace strata
