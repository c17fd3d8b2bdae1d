// Decode path (T <= 16 tokens): the per-token expert GEMV regime of the
// pages (ai-coding.wiselychen.com "Strata two weeks", section 成功思路一: per
// layer the GPU runs the router, picks 10 experts and computes them; the
// expert step is bound by the bytes of expert weights read), including the
// 1+3-token MTP verify window (devotd.net "Strata memory tiers", section
// 用草拟 token 提高生成速度的 MTP) where tokens that pick the same expert share
// one read of its weights (blog.5616760.com/0039.html, section 十二).
//
// Four launches per forward call, each with many short waves (the time of a
// kernel this small is the longest chain of dependent memory round trips and
// instructions of one wave, not the bytes):
//   k_route_gemv  router GEMV, one workgroup per 1 or 2 expert rows split over
//                 its waves; each workgroup reads the whole token rows, so it
//                 also finds each token's operand scale 2^-e (up to 4
//                 tokens) and writes a slice of the tokens as two fp16 parts
//                 of x 2^-e (x 2^-e = p0 + p1 to 22 significant bits);
//   k_topk        one workgroup per token: two-level radix selection of the k
//                 largest logits and the renormalised softmax weights (more
//                 than 4 tokens: also the operand scale, rescaling the parts
//                 of a token that needs one);
//   k_gateup      one workgroup per (active expert, 32 rows of I): it finds
//                 its expert from the top-k ids (experts chosen by any token,
//                 ascending, then the shared one), its waves split the H
//                 superblocks; writes silu(g) * u as two fp16 parts per
//                 (active expert, token);
//   k_down        one workgroup per 16 rows of H; waves take (active expert,
//                 superblock) units with the next units' loads in flight,
//                 scale each expert's rows by its routing weights and the
//                 workgroup reduces them in a fixed order: the weighted
//                 combine happens here, with no cross-workgroup
//                 synchronisation (k_down16 from 9 tokens: the token rows of
//                 each unit's routed tokens only).
// A route() call runs k_route_gemv, k_topk and k_permute (the stable
// token->expert permutation that the expert kernels do not need).
//
// The multiply-accumulate runs on the matrix cores (16x16x32 fp16 MFMA, fp32
// accumulation): the code q of a weight becomes the fp16 value q (2-bit codes
// through the FP4->fp16 conversion, Q3 as a 2-bit and a 1-bit plane, Q4
// through the E4M3->fp16 conversion), exactly; the activations enter
// as two fp16 parts (16 A-operand rows: 2 parts x up to 8 tokens; from 9 to
// 16 tokens the rows are the tokens and each part is its own MFMA into the
// same result, so every decode call is one pass over the weights), which
// carry 22 significant bits
// (bf16 inputs exactly); the per-block offset -c * sum_j x_j comes from one
// extra MFMA against a constant operand.  Every product is exact; the fp32
// accumulation and the 2^-22 activation split are the only roundings.  The
// fp16 block scale d multiplies each block's 16x16 result in fp32.
#include <algorithm>
#include <type_traits>

#include "common.hpp"
#include "kernels.hpp"

namespace strata {
namespace {

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef __attribute__((__vector_size__(8 * sizeof(_Float16)))) _Float16 f16x8;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;

constexpr int DESC = 2;    // ints per active expert for the down kernel: expert id, token mask
constexpr int WTAB = 8;    // routing weights per active expert, indexed by token (T <= 8)
constexpr int WTAB16 = 16; // the same for 9..16 tokens
constexpr int NPART = 2;   // fp16 parts of an fp32 activation
constexpr uint32_t OOB = 0x80000000u;   // buffer offset past every record: the load returns 0

__device__ inline float4 bf16x4(uint32_t lo, uint32_t hi) {
  return make_float4(__uint_as_float(lo << 16), __uint_as_float(lo & 0xffff0000u),
                     __uint_as_float(hi << 16), __uint_as_float(hi & 0xffff0000u));
}

__device__ inline uint32_t comp(const uint4& v, int i) {
  return i == 0 ? v.x : (i == 1 ? v.y : (i == 2 ? v.z : v.w));
}

// x = p0 + p1 + p2 with fp16 parts (exact for fp32 values of fp16 range)
// x as two fp16 parts: p0 = fp16(x), p1 = fp16(x - p0) (the difference is
// exact), so |x - p0 - p1| <= 2^-22 |x| while x - p0 is an fp16 normal
__device__ inline void split2(float x, _Float16* p) {
  p[0] = (_Float16)x;
  p[1] = (_Float16)(x - (float)p[0]);
}

// The A operand of the 16x16x32 MFMAs: row r = lane % 16 holds part r / 8 of
// token r % 8 (every token of a call, T <= 8)
__device__ inline int arow_token(int lane) { return lane & 7; }
__device__ inline int arow_part(int lane) { return (lane & 15) >> 3; }
// D element v of a lane: row 4 (lane / 16) + v, i.e. part lane / 32 of token
// 4 ((lane / 16) % 2) + v; column lane % 16
__device__ inline int drow_token(int lane, int v) { return 4 * ((lane >> 4) & 1) + v; }

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
template <> struct Codes<5> { uint4 v0, v1; };

// Codes of one lane of the slab at byte soff of an expert record.
template <int FMT>
__device__ inline void bload_codes(rsrc_t r, uint32_t soff, int lane, Codes<FMT>& c) {
  if constexpr (FMT == 4 || FMT == FMT_MXFP4) {
    c.v0 = bload4(r, lane * 16, soff);
    c.v1 = bload4(r, 1024 + lane * 16, soff);
  } else {
    c.lo = bload4(r, lane * 16, soff);
    if constexpr (FMT == 3) c.hi = bload2(r, 1024 + lane * 8, soff);
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

// Q4 codes of block BB as fp16 values q: each byte 0000qqqq of the masked
// word is the E4M3 value q 2^-9, converted at scale 2^9 (exact)
template <int BB>
__device__ inline f16x8 q4_operand(const Codes<4>& c) {
  const uint32_t W = comp((BB >> 2) ? c.v1 : c.v0, BB & 3);
  const uint32_t E = W & 0x0F0F0F0Fu, O = (W >> 4) & 0x0F0F0F0Fu;
  return join(__builtin_amdgcn_cvt_scalef32_pk_f16_fp8(E, 512.0f, false),
              __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(E, 512.0f, true),
              __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(O, 512.0f, false),
              __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(O, 512.0f, true));
}

// MXFP4 codes of block BB as their E2M1 values (exact in fp16): byte j of
// the block's word holds elements 2j (low nibble) and 2j + 1
template <int BB>
__device__ inline f16x8 mx_operand(const Codes<5>& c) {
  const uint32_t W = comp((BB >> 2) ? c.v1 : c.v0, BB & 3);
  return join(__builtin_amdgcn_cvt_scalef32_pk_f16_fp4(W, 1.0f, 0),
              __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(W, 1.0f, 1),
              __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(W, 1.0f, 2),
              __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(W, 1.0f, 3));
}

// scale of block BB of this lane's row; MXFP4's 16-bit slot holds the E8M0 byte e: 2^(e - 127) (e = 0: 2^-127, a
// subnormal, e <= 140 checked at create)
template <int FMT, int BB>
__device__ inline float block_scale(const uint4& sc) {
  const uint32_t w = comp(sc, BB >> 1);
  const uint32_t h = (BB & 1) ? (w >> 16) : (w & 0xffffu);
  if constexpr (FMT == FMT_MXFP4) return __uint_as_float(h ? h << 23 : 0x00400000u);
  const float d = half_bits_to_f32((uint16_t)h);
  return d;
}

// D = A * B(codes of block BB) + Doff, in fp32
template <int FMT, int BB>
__device__ inline f32x4 block_product(const f16x8& a, const Codes<FMT>& c, const f32x4& doff) {
  if constexpr (FMT == 4) {
    return mfma(a, q4_operand<BB>(c), doff);
  } else if constexpr (FMT == FMT_MXFP4) {
    return mfma(a, mx_operand<BB>(c), doff);
  } else {
    f32x4 d = mfma(a, lo2_operand<BB>(c.lo), doff);
    if constexpr (FMT == 3) d = mfma(a, hi3_operand<BB>(c.hi), d);
    return d;
  }
}

// the block offset -c * sum_j x_j, for every output column, added to acc
template <int FMT>
__device__ inline f32x4 block_offset_acc(const f16x8& a, const f32x4& acc) {
  if constexpr (FMT == FMT_MXFP4) {               // no offset term
    return acc;
  } else {
    f16x8 cst;
#pragma unroll
    for (int i = 0; i < 8; ++i) cst[i] = (_Float16)(-Fmt<FMT>::c);
    return mfma(a, cst, acc);
  }
}
template <int FMT>
__device__ inline f32x4 block_offset(const f16x8& a) {
  const f32x4 z = {0.f, 0.f, 0.f, 0.f};
  return block_offset_acc<FMT>(a, z);
}


// ------------------------------------------------------------------ router
struct RouteArgs {
  const float* Wr;           // [E][Ho]
  const float* bias;
  const void* x;             // [T][Ho]
  int x_f32, T, H, E;        // H: the token-part rows' width (whole superblocks)
  int Ho;                    // the layer's hidden width
  float* logits;
  _Float16* xparts;          // [2][T][H], zero past Ho, of x 2^-e (e: the token's operand scale)
  int* part1;                // set to 1 when some token has a nonzero second part
  int* texp;                 // [T] the exponent e of each token's operand scale 2^-e
};

constexpr int ROUTE_WAVES = 4;
// up to this many tokens the router kernel finds the tokens' operand scales
constexpr int TOKEN_SCALE_IN_ROUTE_T = 4;
constexpr int ROUTE_BATCH = 4;   // float4 columns per lane issued together

// token t, columns 4q..4q+3 of x as loaded (fp32 or bf16), and as fp32
template <bool XF32> struct XQuad;
template <> struct XQuad<true> { float4 v; };
template <> struct XQuad<false> { uint2 v; };
template <bool XF32>
__device__ inline XQuad<XF32> x_quad_load(const void* x, int H, int t, int q) {
  if constexpr (XF32) return {reinterpret_cast<const float4*>(x)[((size_t)t * H >> 2) + q]};
  else return {reinterpret_cast<const uint2*>(x)[((size_t)t * H >> 2) + q]};
}
template <bool XF32>
__device__ inline float4 x_quad_f32(const XQuad<XF32>& r) {
  if constexpr (XF32) return r.v;
  else return bf16x4(r.v.x, r.v.y);
}

// Expert rows per router workgroup: every wave reads its columns of the
// tokens once for all of them (fewer register batches for more tokens)
constexpr int route_rows(int T) { return T <= 4 ? 2 : 1; }
// float4 columns per lane in flight together: every load of a batch is
// issued before the first is used, so a batch costs one memory round trip;
// 3 columns of 16 tokens cover a 3072-wide row in one batch
constexpr int route_batch(int T) { return T <= 8 ? ROUTE_BATCH : 3; }

// route_rows(T) expert rows per workgroup; its waves split the rows into
// float4 columns (strided, so every load instruction of a wave reads 1 KiB
// contiguously) and meet in LDS.  Each workgroup reads every token's whole
// row, so up to 4 tokens (SCALE) each also finds the tokens' operand scales
// 2^-e (e from the largest magnitude: token_scale_exp) and writes its slice
// of the tokens as fp16 parts of x 2^-e; workgroup 0 writes the exponents.
// For more tokens the per-column maxima lengthen this kernel by more than
// the top-k kernel's pass over the tokens costs (measured at 6 and 16
// tokens): the parts are written unscaled and the top-k kernel rescales
// (decode_token_scale).  TT and the input type are template constants so
// that every load is unconditional (clamped into bounds) and all of a batch
// are in flight together: TT = T up to 8, TT = 16 for 9..16 tokens (tokens
// past T repeat the last one: loaded and computed, not stored).
template <int TT, bool XF32>
__global__ __launch_bounds__(64 * ROUTE_WAVES) void k_route_gemv(RouteArgs a) {
  constexpr int RR = route_rows(TT);
  constexpr int RB = route_batch(TT);
  constexpr bool SCALE = TT <= TOKEN_SCALE_IN_ROUTE_T;
  __shared__ float part[ROUTE_WAVES][RR][TT];
  __shared__ uint32_t s_max[ROUTE_WAVES][TT];         // per wave: each token's largest |x| (bits)
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int H = a.Ho, E = a.E, e0 = blockIdx.x * RR, T = a.T;
  uint32_t mx[TT];                                    // each token's largest |x| seen (bits)
#pragma unroll
  for (int t = 0; t < TT; ++t) mx[t] = 0u;
  const int nq = H >> 2;
  const float4* rows[RR];
#pragma unroll
  for (int r = 0; r < RR; ++r)      // rows past E repeat the last one (computed, not stored)
    rows[r] = reinterpret_cast<const float4*>(a.Wr + (size_t)min(e0 + r, E - 1) * H);
  float acc[RR][TT];
#pragma unroll
  for (int r = 0; r < RR; ++r)
#pragma unroll
    for (int t = 0; t < TT; ++t) acc[r][t] = 0.f;
  for (int q0 = tid; q0 < nq; q0 += RB * 64 * ROUTE_WAVES) {
    float4 w[RB][RR];
    XQuad<XF32> xr[RB][TT];
#pragma unroll
    for (int j = 0; j < RB; ++j) {
      const int q = min(q0 + j * 64 * ROUTE_WAVES, nq - 1);
#pragma unroll
      for (int r = 0; r < RR; ++r) w[j][r] = rows[r][q];
#pragma unroll
      for (int t = 0; t < TT; ++t) xr[j][t] = x_quad_load<XF32>(a.x, H, TT <= DECODE_NARROW_T ? t : min(t, T - 1), q);
    }
    // (without this the scheduler interleaves the loads with their uses and
    // pays several round trips per batch at 4 and 16 tokens)
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int j = 0; j < RB; ++j) {
      const float m = (q0 + j * 64 * ROUTE_WAVES < nq) ? 1.f : 0.f;   // clamped duplicates count 0
#pragma unroll
      for (int t = 0; t < TT; ++t) {
        const float4 xv = x_quad_f32<XF32>(xr[j][t]);
        if constexpr (SCALE)       // (clamped duplicate columns do not change a maximum)
          mx[t] = max(mx[t], max(max(__float_as_uint(xv.x) & 0x7fffffffu, __float_as_uint(xv.y) & 0x7fffffffu),
                                 max(__float_as_uint(xv.z) & 0x7fffffffu, __float_as_uint(xv.w) & 0x7fffffffu)));
#pragma unroll
        for (int r = 0; r < RR; ++r) {
          float d = w[j][r].x * xv.x;
          d = fmaf(w[j][r].y, xv.y, d);
          d = fmaf(w[j][r].z, xv.z, d);
          d = fmaf(w[j][r].w, xv.w, d);
          acc[r][t] = fmaf(m, d, acc[r][t]);
        }
      }
    }
  }
#pragma unroll
  for (int r = 0; r < RR; ++r)
#pragma unroll
    for (int t = 0; t < TT; ++t) {
      const float s = wave_sum(acc[r][t]);
      if (lane == 0) part[wv][r][t] = s;
    }
  if constexpr (SCALE) {
#pragma unroll
    for (int t = 0; t < TT; ++t) {
      const uint32_t m = wave_max_u32(mx[t]);
      if (lane == 0) s_max[wv][t] = m;
    }
  }
  __syncthreads();
  // token t's operand scale exponent
  auto texp_of = [&](int t) __attribute__((always_inline)) {
    uint32_t m = 0u;
#pragma unroll
    for (int w = 0; w < ROUTE_WAVES; ++w) m = max(m, s_max[w][t]);
    return token_scale_exp(__uint_as_float(m));
  };
  if (SCALE && blockIdx.x == 0 && tid < T) a.texp[tid] = texp_of(tid);
  // this workgroup's slice of the token rows as fp16 parts of x 2^-e (SCALE;
  // else of x), [part][t][a.H] (columns past the layer's width are zero)
  const int Hp = a.H, n = T * Hp, chunk = (n + gridDim.x - 1) / gridDim.x, b = blockIdx.x;
  bool nz = false;
  for (int i = b * chunk + tid; i < min(n, (b + 1) * chunk); i += blockDim.x) {
    const int t = i / Hp, h = i - t * Hp;
    const int src = t * H + min(h, H - 1);
    float v = XF32 ? reinterpret_cast<const float*>(a.x)[src]
                   : bf16_to_f32(reinterpret_cast<const uint16_t*>(a.x)[src]);
    v = h < H ? (SCALE ? v * pow2i(-texp_of(t)) : v) : 0.f;
    _Float16 p[NPART];
    split2(v, p);
#pragma unroll
    for (int q = 0; q < NPART; ++q) a.xparts[(size_t)q * n + i] = p[q];
    nz |= p[1] != (_Float16)0.0f;
  }
  if (__ballot(nz) && lane == 0) *a.part1 = 1;
  if (tid < RR * TT) {
    const int r = tid / TT, t = tid - r * TT, e = e0 + r;
    float s = 0.f;
#pragma unroll
    for (int w = 0; w < ROUTE_WAVES; ++w) s += part[w][r][t];
    if (e < E && t < T) a.logits[(size_t)t * E + e] = s + (a.bias ? a.bias[e] : 0.f);
  }
}

// ------------------------------------------------------------------ top-k
// Radix selection over the keys u[i] of entries lane + 64 i (i < V): marks
// the k largest (equal keys: lower entry first) and gives each marked entry
// its rank in entry order.  Needs at least k entries (padding keys 0 count).
template <int V>
__device__ inline void wave_select(const uint32_t (&u)[V], int k, bool (&sel)[V], int (&pos)[V]) {
  uint32_t tau = 0;
  for (int b = 31; b >= 0; --b) {
    const uint32_t cand = tau | (1u << b);
    int cnt = 0;
#pragma unroll
    for (int i = 0; i < V; ++i) cnt += __popcll(__ballot(u[i] >= cand));
    if (cnt >= k) {
      tau = cand;
      if (cnt == k) break;                 // {u >= tau} is the selection
    }
  }
  int gt = 0;
#pragma unroll
  for (int i = 0; i < V; ++i) gt += __popcll(__ballot(u[i] > tau));
  const int need = k - gt;
  int ties_before = 0, sel_before = 0;
#pragma unroll
  for (int i = 0; i < V; ++i) {
    const bool tie = u[i] == tau;
    const uint64_t tm = __ballot(tie);
    const int trank = ties_before + (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(tm >> 32),
                                          __builtin_amdgcn_mbcnt_lo((uint32_t)tm, 0u));
    ties_before += __popcll(tm);
    sel[i] = (u[i] > tau) || (tie && trank < need);
    const uint64_t sm = __ballot(sel[i]);
    pos[i] = sel_before + (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(sm >> 32),
                                     __builtin_amdgcn_mbcnt_lo((uint32_t)sm, 0u));
    sel_before += __popcll(sm);
  }
}

struct TopkArgs {
  int T, E, k, n_shared;
  const void* x;             // [T][Ho] the tokens (bf16, or fp32 when x_f32)
  int x_f32, H, Ho;          // H: the token-part rows' width
  Work w;
};

// The operand scale of token t for calls of more than 4 tokens (one
// workgroup, any number of waves; up to 4 tokens the router kernel finds it):
// e from the token's largest magnitude (token_scale_exp) into texp[t]; a
// token with e != 0 has its fp16 parts (written unscaled by the router
// kernel) rewritten as parts of x 2^-e.  s_m: one LDS word per wave.  Ends
// with a barrier.
__device__ inline void decode_token_scale(const TopkArgs& a, int t, uint32_t* s_m) {
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6, nw = blockDim.x >> 6;
  const int per = a.x_f32 ? 4 : 8;                 // elements per 16-byte load
  const int nch = a.Ho / per;
  const char* row = reinterpret_cast<const char*>(a.x) + (size_t)t * a.Ho * (a.x_f32 ? 4 : 2);
  uint32_t m = 0;                                  // largest |x| as bits (non-negative: bit order)
  for (int c = threadIdx.x; c < nch; c += blockDim.x) {
    const uint4 v = *reinterpret_cast<const uint4*>(row + 16 * (size_t)c);
    const uint32_t q[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int i = 0; i < 4; ++i)
      m = a.x_f32 ? max(m, q[i] & 0x7fffffffu) : max(m, max((q[i] & 0x7fffu) << 16, q[i] & 0x7fff0000u));
  }
  m = wave_max_u32(m);
  if (lane == 0) s_m[wv] = m;
  __syncthreads();
  for (int w = 0; w < nw; ++w) m = max(m, s_m[w]);
  const int e = token_scale_exp(__uint_as_float(m));
  if (threadIdx.x == 0) a.w.texp[t] = e;
  if (e == 0) return;
  bool nz = false;
  const size_t n = (size_t)a.T * a.H;
  const float sc = pow2i(-e);
  for (int h = threadIdx.x; h < a.Ho; h += blockDim.x) {
    const size_t src = (size_t)t * a.Ho + h;
    const float v = (a.x_f32 ? reinterpret_cast<const float*>(a.x)[src]
                             : bf16_to_f32(reinterpret_cast<const uint16_t*>(a.x)[src])) * sc;
    _Float16 p[NPART];
    split2(v, p);
#pragma unroll
    for (int q = 0; q < NPART; ++q) a.w.xparts[q * n + (size_t)t * a.H + h] = p[q];
    nz |= p[1] != (_Float16)0.0f;
  }
  if (__ballot(nz) && (threadIdx.x & 63) == 0) a.w.meta[3] = 1;
}

constexpr int TOPK_WAVES = 8;

// One workgroup per token.  Each wave keeps the k best of its own contiguous
// id range; the candidates land in LDS in id order and wave 0 keeps the k
// best of those (the global k best are among them: same order everywhere).
// Writes the ids in ascending order and the renormalised softmax weights
// (max-shifted exp over the k selected, divided by their sum).
template <int V1, int V2>
__global__ __launch_bounds__(64 * TOPK_WAVES) void k_topk(TopkArgs a) {
  __shared__ uint32_t c_key[TOPK_WAVES * 64];
  __shared__ float c_val[TOPK_WAVES * 64];
  __shared__ int c_id[TOPK_WAVES * 64];
  __shared__ uint32_t s_m[TOPK_WAVES];
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int E = a.E, k = a.k, t = blockIdx.x;
  const float* row = a.w.logits + (size_t)t * E;
  const int e0 = wv * 64 * V1;
  // the logits are requested first, so that they and the token row of the
  // operand scale (more than 4 tokens) are in flight together
  float val[V1];
#pragma unroll
  for (int i = 0; i < V1; ++i) val[i] = row[min(e0 + lane + 64 * i, E - 1)];
  if (a.T > TOKEN_SCALE_IN_ROUTE_T) decode_token_scale(a, t, s_m);
  uint32_t u[V1];
#pragma unroll
  for (int i = 0; i < V1; ++i) u[i] = e0 + lane + 64 * i < E ? sortable_bits(val[i]) : 0u;
  bool sel[V1];
  int pos[V1];
  wave_select<V1>(u, k, sel, pos);
#pragma unroll
  for (int i = 0; i < V1; ++i) {
    if (sel[i]) {
      const int c = wv * k + pos[i];
      c_key[c] = u[i];
      c_val[c] = val[i];
      c_id[c] = e0 + lane + 64 * i;
    }
  }
  __syncthreads();
  if (wv != 0) return;
  const int nc = TOPK_WAVES * k;
  uint32_t u2[V2];
  float v2[V2];
  int id2[V2];
#pragma unroll
  for (int i = 0; i < V2; ++i) {
    const int c = lane + 64 * i;
    u2[i] = c < nc ? c_key[c] : 0u;
    v2[i] = c < nc ? c_val[c] : 0.f;
    id2[i] = c < nc ? c_id[c] : 0;
  }
  bool sel2[V2];
  int pos2[V2];
  wave_select<V2>(u2, k, sel2, pos2);
  uint32_t umax = 0;
#pragma unroll
  for (int i = 0; i < V2; ++i) umax = (sel2[i] && u2[i] > umax) ? u2[i] : umax;
  const float top = unsortable_bits((uint32_t)wave_max_u64(umax));
  float z[V2], zs = 0.f;
#pragma unroll
  for (int i = 0; i < V2; ++i) {
    z[i] = sel2[i] ? expf(v2[i] - top) : 0.f;
    zs += z[i];
  }
  const float s = wave_sum(zs);
#pragma unroll
  for (int i = 0; i < V2; ++i) {
    if (sel2[i]) {
      a.w.topk_idx[(size_t)t * k + pos2[i]] = id2[i];
      a.w.topk_w[(size_t)t * k + pos2[i]] = z[i] / s;
    }
  }
}

// Top-k for any k (used when k > 64, past the candidate slots of k_topk):
// one 1024-thread workgroup per token over its logit row (+ bias).
__global__ __launch_bounds__(1024) void k_topk_block(const float* rows, size_t stride, const float* bias, int E,
                                                     int k, int* idx, float* w) {
  const size_t t = blockIdx.x;
  block_topk(rows + t * stride, bias, E, k, idx + t * k, w + t * k);
}

// the decode path's selection past 64 (as above), and its token scale for
// more than 4 tokens
__global__ __launch_bounds__(1024) void k_topk_block_decode(TopkArgs a) {
  __shared__ uint32_t s_m[16];
  const int t = blockIdx.x;
  if (a.T > TOKEN_SCALE_IN_ROUTE_T) decode_token_scale(a, t, s_m);
  block_topk(a.w.logits + (size_t)t * a.E, nullptr, a.E, a.k, a.w.topk_idx + (size_t)t * a.k,
             a.w.topk_w + (size_t)t * a.k);
}

// The stable token->expert permutation of the routing (route() only): counts,
// offsets (exclusive scan over experts), and for every pair p = t * k + j its
// slot, earlier tokens of the same expert first: its rank is the number of
// earlier tokens in the expert's token bitmask (T <= 16).  One workgroup.
__global__ __launch_bounds__(512) void k_permute(TopkArgs a) {
  extern __shared__ int lds_i[];
  __shared__ int2 tmp[16];
  const int tid = threadIdx.x, nt = blockDim.x;
  const int E = a.E, k = a.k, T = a.T, P = T * k;
  int* hist = lds_i;                                           // [E] counts, then offsets
  uint32_t* tmask = reinterpret_cast<uint32_t*>(hist + E);     // [E] tokens of each expert
  for (int e = tid; e < E; e += nt) { hist[e] = 0; tmask[e] = 0u; }
  __syncthreads();
  for (int p = tid; p < P; p += nt) {
    const int e = a.w.topk_idx[p];
    atomicAdd(&hist[e], 1);
    atomicOr(&tmask[e], 1u << (p / k));
  }
  __syncthreads();
  const int per = (E + nt - 1) / nt;
  const int e0 = tid * per, e1 = min(E, e0 + per);
  int2 loc = make_int2(0, 0);
  for (int e = e0; e < e1; ++e) loc.x += hist[e];
  int2 total;
  int2 base = block_exclusive_scan(loc, tmp, &total);
  for (int e = e0; e < e1; ++e) {
    const int c = hist[e];
    a.w.counts[e] = c;
    a.w.offsets[e] = base.x;
    hist[e] = base.x;
    base.x += c;
  }
  __syncthreads();
  for (int p = tid; p < P; p += nt) {
    const int t = p / k, e = a.w.topk_idx[p];
    const int slot = hist[e] + __popc(tmask[e] & ((1u << t) - 1u));
    a.w.perm[slot] = p;
    a.w.inv[p] = slot;
  }
  if (tid == 0) a.w.offsets[E] = P;
}

// ------------------------------------------------------------------ experts
struct ExpertArgs {
  const uint8_t* packed;
  size_t stride;
  int H, I, E, k, T, P, n_shared;   // H, I: whole superblocks (the packed geometry)
  int Ho;                            // the layer's hidden width (x, out)
  uint32_t actp_bytes;       // bytes of the activation rows of this call
  int umax;                  // most active experts a call of T tokens can have (+ shared)
  const void* x;
  int x_f32;
  uint32_t flags;
  float* out;
  Work w;
  // prefetch by the gate/up waves (pf_issue): the next stack layer's router
  // rows (pf_next_chunks = 0: none) and this call's down slabs
  const void* pf_next;
  uint32_t pf_next_bytes, pf_next_chunk;
  int pf_next_chunks;
  int pf_down;
  uint32_t pf_key;
};

// Active expert u of this call: the experts chosen by any token in ascending
// id order, then the shared expert (id E, every token, weight 1).  Each wave
// finds it on its own, with no workgroup barrier: it marks the chosen ids in
// its own 4096-bit LDS mask (bits), counts the set bits below each 64-bit
// word, and takes the u-th.  Returns false when u is past the last one.
// wt: in lane t < T, token t's routing weight to this expert (0 when not
// routed).  issue() is called once the pair loads are requested (memory
// requests that must not delay them go there).
template <typename F>
__device__ inline bool wave_route(const ExpertArgs& a, int u, uint64_t* bits, int& e_out, uint32_t& mask_out,
                                  int& n_active, float& wt, F&& issue) {
  const int lane = threadIdx.x & 63;
  const int T = a.T, k = a.k, E = a.E, P = T * k, nwords = (E + 63) >> 6;
  // pairs lane and 64 + lane, loaded unconditionally (clamped) so that both
  // loads are in flight together; pairs past 128 (T k > 128) are read later
  int ids[2];
  float ws[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int p = min(lane + 64 * i, P - 1);
    ids[i] = a.w.topk_idx[p];
    ws[i] = a.w.topk_w[p];
  }
  __builtin_amdgcn_sched_barrier(0);
  issue();
  __builtin_amdgcn_sched_barrier(0);
  bits[lane] = 0ull;
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront", "local");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront", "local");
#pragma unroll
  for (int i = 0; i < 2; ++i)
    if (lane + 64 * i < P) atomicOr(&bits[ids[i] >> 6], 1ull << (ids[i] & 63));
  for (int p = lane + 128; p < P; p += 64) {
    const int id = a.w.topk_idx[p];
    atomicOr(&bits[id >> 6], 1ull << (id & 63));
  }
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront", "local");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront", "local");
  uint64_t w = lane < nwords ? bits[lane] : 0ull;
  const int c = __popcll(w);
  int incl = c;                                      // set bits in words 0 .. lane
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(incl, o, 64);
    if (lane >= o) incl += y;
  }
  const int U = __builtin_amdgcn_readlane(incl, 63);
  n_active = U + a.n_shared;
  if (u >= n_active) return false;
  int e = E;                                         // the shared expert past the routed ones
  if (u < U) {
    const bool owner = u >= incl - c && u < incl;    // this lane's word holds the u-th set bit
    int id = 0;
    if (owner) {
      for (int r = u - (incl - c); r > 0; --r) w &= w - 1ull;   // drop the lower set bits
      id = 64 * lane + __builtin_ctzll(w);
    }
    e = __builtin_amdgcn_readlane(id, __builtin_ctzll(__ballot(owner)));
  }
  // tokens routed to e and their weights (the shared expert: every token, weight 1)
  uint32_t m = 0u;
  wt = 0.f;
  if (e < E) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int p = lane + 64 * i;
      const bool hit = p < P && ids[i] == e;
      if (hit) m |= 1u << (p / k);
      // the weight of token lane: its pair with e sits in lane p of register i
      const uint64_t hb = __ballot(hit);
      for (uint64_t b = hb; b; b &= b - 1ull) {
        const int src = __builtin_ctzll(b);
        const float wv = __shfl(ws[i], src, 64);
        if (lane == (src + 64 * i) / k) wt = wv;
      }
    }
    for (int p = lane + 128; p < P; p += 64) {
      if (a.w.topk_idx[p] == e) m |= 1u << (p / k);
    }
    for (int p0 = 128; p0 < P; p0 += 64) {
      const int p = min(p0 + lane, P - 1);
      const bool hit = p0 + lane < P && a.w.topk_idx[p] == e;
      const float wp = a.w.topk_w[p];
      const uint64_t hb = __ballot(hit);
      for (uint64_t b = hb; b; b &= b - 1ull) {
        const int src = __builtin_ctzll(b);
        const float wv = __shfl(wp, src, 64);
        if (lane == (p0 + src) / k) wt = wv;
      }
    }
    // OR over the wave
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) m |= (uint32_t)__shfl_xor((int)m, o, 64);
  } else {
    m = (1u << T) - 1u;
    wt = lane < T ? 1.f : 0.f;
  }
  e_out = __builtin_amdgcn_readfirstlane(e);
  mask_out = (uint32_t)__builtin_amdgcn_readfirstlane((int)m);
  return true;
}

// Prefetch.  While a gate/up wave waits for its routing lookup and its
// weights, it also requests bytes that a later kernel will read, so that
// they come from the caches then instead of HBM: the next stack layer's
// router rows, and the down slabs of its own expert.  A launch's workgroup w
// runs on XCD w % 8 and each XCD has its own L2, so the later kernel's bytes
// are taken as the chunks its workgroups read (chunk c read by its workgroup
// c), and the nwx waves on XCD x (this one: jw) request the chunks x, x + 8,
// ... in 1 KiB pieces, N per lane at most (a hint: what is left over is not
// requested).  Pieces outside the chunks read past the buffer record, which
// fetches nothing.  No result depends on the loaded values: they are folded
// by pf_fold into one word that is stored only if it equals a key
// (a spare meta word, never read), so that the loads are kept.
constexpr int PF_LOADS = 3;
template <int N>
__device__ inline void pf_issue(const void* base, uint32_t bytes, uint32_t chunk, int nchunks, int x, int jw,
                                int nwx, uint4 (&v)[N]) {
  const int lane = threadIdx.x & 63;
  const rsrc_t r = make_rsrc(base, bytes);
  const uint32_t P = (chunk + 1023u) >> 10;                        // pieces per chunk
  const uint32_t mine = nchunks > x ? (uint32_t)(nchunks - x + 7) >> 3 : 0u;
#pragma unroll
  for (int i = 0; i < N; ++i) {
    const uint32_t q = (uint32_t)(jw + i * nwx);
    const uint32_t m = q / P, in = (q - m * P) * 1024u + 16u * (uint32_t)lane;
    const bool ok = q < mine * P && in < chunk;
    v[i] = bload4(r, ok ? ((uint32_t)x + 8u * m) * chunk + in : bytes, 0u);
  }
}
template <int N>
__device__ inline uint32_t pf_fold(const uint4 (&v)[N]) {
  uint32_t h = 0u;
#pragma unroll
  for (int i = 0; i < N; ++i) h ^= v[i].x ^ v[i].y ^ v[i].z ^ v[i].w;
  return h;
}

// gate/up: a workgroup covers G row groups (16G rows i) of one active
// expert; its waves split the H superblocks, each wave G gate + G up slabs
// per superblock (sharing one activation operand); partial sums meet in LDS.
// The workgroup first finds its expert from the top-k ids.  Output:
// silu(g) * u as two fp16 parts, rows (active expert, part, token) of the
// activation buffer.  G = 4 when many experts are active (fewer, larger
// workgroups: all of them resident at once), else 2.

// one superblock of a gate/up wave: 2G slabs and the activation operand
template <int FMT, int G> struct GuStage {
  Codes<FMT> cd[2 * G];
  uint4 sc[2 * G];
};

typedef __attribute__((address_space(3))) void lds_void_t;

// an empty asm that takes and returns every register of a stage: values
// computed from it before cannot be reused after
__device__ inline void opaque(uint4& v) { asm volatile("" : "+v"(v.x), "+v"(v.y), "+v"(v.z), "+v"(v.w)); }
__device__ inline void opaque(uint2& v) { asm volatile("" : "+v"(v.x), "+v"(v.y)); }
__device__ inline void opaque(Codes<2>& c) { opaque(c.lo); }
__device__ inline void opaque(Codes<3>& c) { opaque(c.lo); opaque(c.hi); }
__device__ inline void opaque(Codes<4>& c) { opaque(c.v0); opaque(c.v1); }
__device__ inline void opaque(Codes<5>& c) { opaque(c.v0); opaque(c.v1); }
template <int FMT, int G>
__device__ inline void opaque(GuStage<FMT, G>& st) {
#pragma unroll
  for (int s = 0; s < 2 * G; ++s) { opaque(st.cd[s]); opaque(st.sc[s]); }
}

// The token rows of superblock sb in this wave's LDS region, compact: row
// r = q T + t (part q, token t, T <= 16) holds the superblock's 512 bytes of that row;
// rows 2 i and 2 i + 1 come from one buffer->LDS load (1 KiB, lane j's 16
// bytes land at 16 j) into slot i of the region (slots 1040 bytes apart).
// Row 2 i + h keeps its 16-byte chunk g at 512 h + 16 (g ^ 8 h) of the slot,
// so the 16 rows one operand read touches (a 64-byte block of every row)
// fall into distinct LDS banks for T <= 8.  Slot T holds a row of zeros for
// the A-operand rows of tokens past T.  T loads per superblock instead of 8
// (or 16) for a 16-row operand.
constexpr int GU_SLOT = 1040;
constexpr int GU_MAX_WAVES = 10;   // gate/up waves per workgroup
// dynamic LDS ceiling of the gate/up kernels: the CU's 160 KiB less their
// static arrays (chosen-expert masks, scale exponents)
constexpr size_t GU_DYN_LDS = 160 * 1024 - (GU_MAX_WAVES * 64 * 8 + 16 * 4 + 64);

__device__ inline int gu_region_bytes(int T) { return max(8192, (T + 1) * GU_SLOT); }

// (n row pairs from byte base of the token parts: base 0 and n = T for the
// rows of both parts; base = part 1's plane for its rows alone)
__device__ inline void gu_aload_lds(rsrc_t xr, int n, int H, int sb, int lane, char* region, uint32_t base = 0) {
  const int h = lane >> 5, g = (lane & 31) ^ (8 * h);
  for (int i = 0; i < n; ++i)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(xr, (lds_void_t*)(region + i * GU_SLOT), 16,
                                             base + (uint32_t)((2 * i + h) * 2 * H + 16 * g),
                                             (uint32_t)sb * SB_WEIGHTS * 2, 0, 0);
}

// vector-memory instructions gu_load issues (codes, then the scales, per slab)
template <int FMT, int G>
constexpr int gu_load_count() { return 2 * G * (FMT == 2 ? 2 : 3); }

// LDS address of this lane's A operand of block BB: row arow (i = arow / 2,
// h = arow % 2), chunk 4 BB + ks stored at 16 ((4 BB + ks) ^ 8 h); as BB ^ 2 h
// = BB + 2 h or BB - 2 h by bit 1 of BB, two per-lane bases cover every BB
struct ALane { const char* plus; const char* minus; };
// the lane's A-operand bases for LDS row arow of a wave region, K-slice ks
__device__ inline ALane a_lane(const char* region, int arow, int ks) {
  const char* rbase = region + (arow >> 1) * GU_SLOT + 512 * (arow & 1) + 16 * ks;
  return ALane{rbase + 128 * (arow & 1), rbase - 128 * (arow & 1)};
}
template <int BB>
__device__ inline const uint4* a_operand(const ALane& al) {
  return reinterpret_cast<const uint4*>(((BB >> 1) & 1 ? al.minus : al.plus) + 64 * BB);
}

// The weights of one superblock, requested in the order the compute takes
// them: slab pairs (gate j, up j).
template <int FMT, int G>
__device__ inline void gu_load(rsrc_t wr, uint32_t up_base, int gp, int nsb, int sb, int lane, GuStage<FMT, G>& st) {
  constexpr int SLAB = Fmt<FMT>::slab_codes + 256;
  const int r = lane & 15;
#pragma unroll
  for (int j = 0; j < G; ++j) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int s = h * G + j;
      const uint32_t soff = (h ? up_base : 0u) + (uint32_t)((G * gp + j) * nsb + sb) * SLAB;
      bload_codes<FMT>(wr, soff, lane, st.cd[s]);
      st.sc[s] = bload4(wr, Fmt<FMT>::slab_codes + r * 16, soff);
    }
    __builtin_amdgcn_sched_barrier(0);               // keep the request order
  }
}

// Slab pairs J0 .. J0 + NJ - 1 of one superblock: per block, the activation
// operand from LDS, the offset MFMA, the 2 NJ product MFMAs (independent, so
// their latency overlaps), then their scale FMAs on the first NV of each
// lane's 4 D rows (the rows past the call's tokens hold zeros).
template <int FMT, int G, int J0, int NJ, int NV>
__device__ inline void gu_compute_pairs(const GuStage<FMT, G>& st, const ALane& al, float (&acc)[2 * G][4]) {
#define STRATA_BLOCK(BB)                                                          \
  {                                                                               \
    const f16x8 af = as_f16x8(*a_operand<BB>(al));                                \
    const f32x4 off = block_offset<FMT>(af);                                      \
    f32x4 d[2 * NJ];                                                              \
    _Pragma("unroll") for (int j = 0; j < NJ; ++j) {                              \
      d[2 * j] = block_product<FMT, BB>(af, st.cd[J0 + j], off);                  \
      d[2 * j + 1] = block_product<FMT, BB>(af, st.cd[G + J0 + j], off);          \
    }                                                                             \
    _Pragma("unroll") for (int j = 0; j < NJ; ++j) {                              \
      const float sg = block_scale<FMT, BB>(st.sc[J0 + j]);                       \
      const float su = block_scale<FMT, BB>(st.sc[G + J0 + j]);                   \
      _Pragma("unroll") for (int v = 0; v < NV; ++v) {                            \
        acc[J0 + j][v] = fmaf(sg, d[2 * j][v], acc[J0 + j][v]);                   \
        acc[G + J0 + j][v] = fmaf(su, d[2 * j + 1][v], acc[G + J0 + j][v]);       \
      }                                                                           \
    }                                                                             \
  }
  STRATA_BLOCK(0) STRATA_BLOCK(1) STRATA_BLOCK(2) STRATA_BLOCK(3)
  STRATA_BLOCK(4) STRATA_BLOCK(5) STRATA_BLOCK(6) STRATA_BLOCK(7)
#undef STRATA_BLOCK
}

// One superblock in halves of G/2 slab pairs, each as soon as its weights
// have arrived (the compiler waits on the half's registers; the other half
// stays in flight).
template <int FMT, int G, int NV>
__device__ inline void gu_compute(const GuStage<FMT, G>& st, const ALane& al, float (&acc)[2 * G][4]) {
  // the activation operand was requested by buffer->LDS loads before the
  // gu_load_count() weight loads: once no more than those are outstanding it
  // has landed (the compiler does not track these loads; the memory clobber
  // keeps every LDS read below this point)
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(gu_load_count<FMT, G>()) : "memory");
  gu_compute_pairs<FMT, G, 0, G / 2, NV>(st, al, acc);
  // (the empty memory clobber makes the second half re-read the operands
  // from LDS instead of keeping every block's operand in registers)
  asm volatile("" ::: "memory");
  gu_compute_pairs<FMT, G, G / 2, G / 2, NV>(st, al, acc);
}

// WIDE (9..16 tokens, or fewer when k_down's LDS cannot hold the call): A
// rows = the 16 tokens, the wave region holds the part-0 rows of the
// superblock, and a call with a nonzero second part (flag meta[3], set by
// the router and token-scale kernels) takes a second pass over the same
// weights with the part-1 rows: bf16 tokens rarely have one.  The
// activations are stored [active expert][token][part][I] for k_down16.
// NV: live D rows per lane, min(T, 4) (4 when WIDE).
template <int FMT, int G, bool WIDE, int NV>
__global__ __launch_bounds__(64 * GU_MAX_WAVES) void k_gateup(ExpertArgs a) {
  constexpr int GU_GROUPS = G, GU_SLABS = 2 * G;
  constexpr int WT = WIDE ? WTAB16 : WTAB;
  // per wave gu_region_bytes(T) of LDS: its superblock's token rows, then its
  // partial sums [GU_SLABS][64 lanes] x 4
  extern __shared__ float4 red4[];
  __shared__ uint64_t s_bits[GU_MAX_WAVES][64];      // per wave: the chosen-expert mask
  __shared__ int s_texp[DECODE_MAX_T];               // the tokens' operand scale exponents
  const int u = blockIdx.y, gp = blockIdx.x;
  const int H = a.H, I = a.I, T = a.T, nsb = H / SB_WEIGHTS;
  const int lane = threadIdx.x & 63, nw = blockDim.x >> 6;
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int ks = lane >> 4;                          // K-slice
  const rsrc_t xr = make_rsrc(a.w.xparts, (uint32_t)(NPART * T * H * 2));
  const int npr = WIDE ? (T + 1) / 2 : T;          // row-pair loads per staging
  const int wreg = gu_region_bytes(npr);
  char* region = reinterpret_cast<char*>(red4) + wv * wreg;
  // A row (part, token) of this lane: its token row, the zero row past T
  // (WIDE: row token lane % 16 of the staged part)
  const int tok = WIDE ? (lane & 15) : arow_token(lane);
  const int arow = tok < T ? (WIDE ? 0 : arow_part(lane)) * T + tok : 2 * npr;
  const ALane al = a_lane(region, arow, ks);
  reinterpret_cast<uint2*>(region + npr * GU_SLOT)[lane] = make_uint2(0u, 0u);   // the zero row
  const int part1 = WIDE ? __builtin_amdgcn_readfirstlane(a.w.meta[3]) : 0;
  const int te = a.w.texp[min(lane, T - 1)];         // lane t < T: token t's scale exponent
  // The prefetch costs ~20-35 registers per lane.  It is taken where it was
  // measured to gain: single-token calls of 2- and 3-bit experts with two row
  // groups per workgroup (1 token 20.3 -> 19.9 us, 48-layer Q3 stack 1083 ->
  // 1066 us per step); at 4 tokens it gained nothing and for 4-bit experts
  // the lower occupancy cost a second round of workgroups.
  constexpr bool PF = !WIDE && NV == 1 && FMT <= 3 && G == 2;
  constexpr int NPF = PF ? PF_LOADS : 1;
  // this wave among the waves of its XCD (the next layer's router prefetch)
  const int lw = u * gridDim.x + gp, nwg = gridDim.x * gridDim.y;
  const int xcd = lw & 7;
  uint4 pfr[NPF], pfd[NPF];
  // the first superblock's activation operand and the router prefetch do not
  // depend on the expert: they are requested right behind the routing
  // lookup's loads (wv < nw <= nsb)
  int e, U;
  uint32_t mask;
  float wt;
  if (!wave_route(a, u, s_bits[wv], e, mask, U, wt, [&]() __attribute__((always_inline)) {
        gu_aload_lds(xr, npr, H, wv, lane, region);
        if constexpr (PF)
          pf_issue(a.pf_next, a.pf_next_bytes, a.pf_next_chunk, a.pf_next_chunks, xcd, (lw >> 3) * nw + wv,
                   ((nwg - xcd + 7) >> 3) * nw, pfr);
      })) {
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // no LDS write may land after the exit
    if constexpr (PF)
      if (pf_fold(pfr) == a.pf_key) a.w.meta[8] = 1;
    return;
  }
  if (wv == 0 && lane < T) s_texp[lane] = te;
  if (gp == 0 && wv == 0) {
    // routing of this active expert for the down kernel; the weight of
    // token t also undoes the 2^-2e of its activations (exact)
    if (lane == 0) {
      a.w.udesc[(size_t)u * DESC] = e;
      a.w.udesc[(size_t)u * DESC + 1] = (int)mask;
      if (u == 0) a.w.meta[0] = U;
    }
    if (lane < WT) a.w.wtab[(size_t)u * WT + lane] = wt * pow2i(2 * te);
  }
  const rsrc_t wr = make_rsrc(a.packed + (size_t)e * a.stride, (uint32_t)a.stride);
  const uint32_t up_base = (uint32_t)up_off(FMT, H, I);

  float acc[GU_SLABS][4];
#pragma unroll
  for (int s = 0; s < GU_SLABS; ++s)
#pragma unroll
    for (int v = 0; v < 4; ++v) acc[s][v] = 0.f;
  // the down slabs of this expert that the down kernel's workgroups on this
  // XCD read (group g of 16 rows of H: nsbI slabs, read by workgroup g)
  const int nsbI = I / SB_WEIGHTS;
  const uint32_t dchunk = (uint32_t)nsbI * (Fmt<FMT>::slab_codes + 256);
  const int gdx = gridDim.x, gp0 = (xcd - u * gdx) & 7;             // this XCD's first row group of u
  const int dgroups = a.pf_down ? a.Ho / 16 : 0;
  // One superblock: its activation operand (unless already requested), then
  // the weights, and the compute waits for each part as it needs it; the
  // first superblock with the prefetch also requests the down slabs behind
  // its weights.
  auto superblock = [&](int sb, bool stage_a, auto issue_down) __attribute__((always_inline)) {
    if (stage_a) gu_aload_lds(xr, npr, H, sb, lane, region);
    __builtin_amdgcn_sched_barrier(0);
    GuStage<FMT, G> st;
    gu_load<FMT, G>(wr, up_base, gp, nsb, sb, lane, st);
    if constexpr (decltype(issue_down)::value)
      pf_issue(a.packed + (size_t)e * a.stride + down_off(FMT, H, I), dchunk * (uint32_t)dgroups, dchunk, dgroups,
               xcd, ((gp - gp0) >> 3) * nw + wv, ((gdx - gp0 + 7) >> 3) * nw, pfd);
    __builtin_amdgcn_sched_barrier(0);
    gu_compute<FMT, G, NV>(st, al, acc);
    if (WIDE && part1) {
      // the part-1 rows into the region once the part-0 operand reads are
      // done, then the same weights again (converted afresh: opaque() keeps
      // the compiler from holding every converted operand of the first pass)
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
      gu_aload_lds(xr, npr, H, sb, lane, region, (uint32_t)(T * H * 2));
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      opaque(st);
      gu_compute<FMT, G, NV>(st, al, acc);
    }
  };
  if constexpr (PF) {
    superblock(wv, false, std::true_type{});
    for (int sb = wv + nw; sb < nsb; sb += nw) superblock(sb, true, std::false_type{});
  } else {
    for (int sb = wv; sb < nsb; sb += nw) superblock(sb, sb > wv, std::false_type{});
  }
  if constexpr (PF)
    if ((pf_fold(pfr) ^ pf_fold(pfd)) == a.pf_key) a.w.meta[8] = 1;
  // raw 16x16 results to this wave's LDS region (its operand is consumed)
  float4* dst = reinterpret_cast<float4*>(region) + lane;
#pragma unroll
  for (int s = 0; s < GU_SLABS; ++s) dst[s * 64] = make_float4(acc[s][0], acc[s][1], acc[s][2], acc[s][3]);
  __syncthreads();
  // sums over waves and parts, SwiGLU, fp16 parts of the result
  for (int idx = threadIdx.x; idx < 16 * GU_GROUPS * T; idx += blockDim.x) {
    const int row = idx & 15, gi = (idx >> 4) % GU_GROUPS, t = idx / (16 * GU_GROUPS);
    if (!((mask >> t) & 1u)) continue;
    // D row (part q, token t) sits in lane 16 (2q + t / 4) + row, element
    // t % 4; WIDE: D row t (both parts) in lane 16 (t / 4) + row
    const int l0 = 16 * (t >> 2) + row, l1 = l0 + 32, v = t & 3;
    float g = 0.f, uu = 0.f;
    for (int w = 0; w < nw; ++w) {
      const float* rw = reinterpret_cast<const float*>(reinterpret_cast<const char*>(red4) + w * wreg);
      const float* rg = rw + (size_t)gi * 256 + v;
      const float* ru = rw + (size_t)(GU_GROUPS + gi) * 256 + v;
      if constexpr (WIDE) {
        g += rg[4 * l0];
        uu += ru[4 * l0];
      } else {
        g += rg[4 * l0] + rg[4 * l1];
        uu += ru[4 * l0] + ru[4 * l1];
      }
    }
    // g, uu carry the token's 2^-e: silu of the unscaled gate, and the
    // activation kept at 2^-2e (exact powers of two)
    const int te_t = s_texp[t];
    const float act = silu_f(g * pow2i(te_t)) * uu * pow2i(-te_t);
    _Float16 p[NPART];
    split2(act, p);
    const int i = (GU_GROUPS * gp + gi) * 16 + row;
#pragma unroll
    for (int q = 0; q < NPART; ++q) {
      // [active expert][part][token][I], WIDE: [active expert][token][part][I]
      const size_t row = WIDE ? ((size_t)u * T + t) * NPART + q : ((size_t)u * NPART + q) * T + t;
      a.w.actp[row * I + i] = p[q];
    }
  }
}

// down + weighted combine: one 16-row group of H per workgroup, every active
// expert; waves take (expert, superblock) units in turn, with the loads of
// the next units in flight while one computes.  The routing of all active
// experts sits in LDS.  A unit's activation rows are staged compactly in the
// wave's LDS (as the gate/up token rows: 2 T rows in T buffer->LDS loads);
// lanes of tokens past T or not routed to the unit's expert read the wave's
// zero row.
constexpr int DN_WAVES = 8;
template <int TT> constexpr int dn_depth() { return TT <= 4 ? 3 : 2; }   // units in flight per wave
template <int TT> constexpr int dn_wave_bytes() { return (dn_depth<TT>() * TT + 1) * GU_SLOT; }

template <int FMT> struct DownUnit {
  Codes<FMT> cd;
  uint4 sc;
};

// vector-memory instructions of one unit: TT activation loads, then codes and scales
template <int FMT, int TT>
constexpr int dn_load_count() { return TT + (FMT == 2 ? 2 : 3); }

template <int FMT, int TT>
__device__ inline void down_load(const ExpertArgs& a, const int* ldesc, int unit, int nsb, int g, char* slot,
                                 DownUnit<FMT>& du) {
  const int lane = threadIdx.x & 63, r = lane & 15;
  const int u = unit / nsb, sb = unit - u * nsb;
  const int e = __builtin_amdgcn_readfirstlane(ldesc[2 * u]);
  // activation rows (part, token) of expert u, superblock sb: rows 2 i and
  // 2 i + 1 per load, chunks swizzled as the gate/up token rows
  const rsrc_t ar = make_rsrc(a.w.actp, a.actp_bytes);
  const int h = lane >> 5, gch = (lane & 31) ^ (8 * h);
  const uint32_t asoff = (uint32_t)(((size_t)u * NPART * TT * a.I + (size_t)sb * SB_WEIGHTS) * 2);
#pragma unroll
  for (int i = 0; i < TT; ++i)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(ar, (lds_void_t*)(slot + i * GU_SLOT), 16,
                                             (uint32_t)((2 * i + h) * a.I * 2 + 16 * gch), asoff, 0, 0);
  const rsrc_t wr = make_rsrc(a.packed + (size_t)e * a.stride, (uint32_t)a.stride);
  const uint32_t soff = (uint32_t)(down_off(FMT, a.H, a.I) + ((size_t)g * nsb + sb) * (Fmt<FMT>::slab_codes + 256));
  bload_codes<FMT>(wr, soff, lane, du.cd);
  du.sc = bload4(wr, Fmt<FMT>::slab_codes + r * 16, soff);
}

// out[v] += routing weight of this lane's D-row token v * (this unit's 16x16
// product), for the first NV of the lane's 4 D rows (the others are zero rows)
template <int FMT, int NV>
__device__ inline void down_compute(const DownUnit<FMT>& du, const ALane& al, const float* wt, float* out) {
  f32x4 dd[2];
  float acc[4] = {0.f, 0.f, 0.f, 0.f};
  // the 8 operand reads go out together (their latencies overlap)
  f16x8 afs[8];
  afs[0] = as_f16x8(*a_operand<0>(al)); afs[1] = as_f16x8(*a_operand<1>(al));
  afs[2] = as_f16x8(*a_operand<2>(al)); afs[3] = as_f16x8(*a_operand<3>(al));
  afs[4] = as_f16x8(*a_operand<4>(al)); afs[5] = as_f16x8(*a_operand<5>(al));
  afs[6] = as_f16x8(*a_operand<6>(al)); afs[7] = as_f16x8(*a_operand<7>(al));
  __builtin_amdgcn_sched_barrier(0);
#define STRATA_BLOCK(BB)                                                          \
  {                                                                               \
    const f16x8 af = afs[BB];                                                     \
    dd[BB & 1] = block_product<FMT, BB>(af, du.cd, block_offset<FMT>(af));        \
    if (BB > 0) {                                                                 \
      const float ds = block_scale<FMT, (BB > 0 ? BB - 1 : 0)>(du.sc);            \
      _Pragma("unroll") for (int v = 0; v < NV; ++v)                              \
        acc[v] = fmaf(ds, dd[(BB - 1) & 1][v], acc[v]);                           \
    }                                                                             \
  }
  STRATA_BLOCK(0) STRATA_BLOCK(1) STRATA_BLOCK(2) STRATA_BLOCK(3)
  STRATA_BLOCK(4) STRATA_BLOCK(5) STRATA_BLOCK(6) STRATA_BLOCK(7)
#undef STRATA_BLOCK
  const float ds = block_scale<FMT, 7>(du.sc);
#pragma unroll
  for (int v = 0; v < NV; ++v) {
    acc[v] = fmaf(ds, dd[1][v], acc[v]);
    out[v] = fmaf(wt[v], acc[v], out[v]);
  }
}

// LDS bytes of the down kernel: routing table, partial sums, staging
__host__ __device__ inline size_t dn_table_bytes(int umax) { return ((size_t)umax * (DESC + WTAB) * 4 + 15) & ~(size_t)15; }

// dynamic LDS of the down kernel for T tokens (the routing table, partial
// sums, staged activation rows)
template <int TT>
size_t down_lds(int umax) { return dn_table_bytes(umax) + (size_t)DN_WAVES * 1024 + (size_t)DN_WAVES * dn_wave_bytes<TT>(); }

template <int FMT, int TT>
__global__ __launch_bounds__(64 * DN_WAVES) void k_down(ExpertArgs a) {
  constexpr int DEPTH = dn_depth<TT>();
  extern __shared__ float4 lds_dn4[];
  char* lds = reinterpret_cast<char*>(lds_dn4);
  const int U = a.w.meta[0];
  const int nsb = a.I / SB_WEIGHTS;
  const int lane = threadIdx.x & 63, nw = blockDim.x >> 6, ks = lane >> 4;
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int g = blockIdx.x;
  // the routing of the active experts: all umax entries are copied (the
  // entries past U are stale and unused), so these loads do not wait for U
  int* ldesc = reinterpret_cast<int*>(lds);                     // [umax][2]: expert, token mask
  float* lwt = reinterpret_cast<float*>(ldesc + DESC * a.umax); // [umax][WTAB]
  const size_t tb = dn_table_bytes(a.umax);
  float* red = reinterpret_cast<float*>(lds + tb);              // [nw][64 lanes][4]
  char* stage = lds + tb + (size_t)DN_WAVES * 1024 + (size_t)wv * dn_wave_bytes<TT>();
  char* zrow = stage + DEPTH * TT * GU_SLOT;
  reinterpret_cast<uint2*>(zrow)[lane] = make_uint2(0u, 0u);
  for (int i = threadIdx.x; i < DESC * a.umax; i += blockDim.x) ldesc[i] = a.w.udesc[i];
  for (int i = threadIdx.x; i < a.umax * WTAB; i += blockDim.x) lwt[i] = a.w.wtab[i];
  __syncthreads();

  const int units = U * nsb;
  const int wt_off = 4 * ((lane >> 4) & 1);                     // token of this lane's D element 0
  const int tok = arow_token(lane), part = arow_part(lane);
  float out[4] = {0.f, 0.f, 0.f, 0.f};
  DownUnit<FMT> b[DEPTH];
  // every load unconditional (unit index clamped; a repeated unit is
  // loaded but not computed), so the loads of a step are all in flight
#pragma unroll
  for (int q = 0; q < DEPTH; ++q)
    down_load<FMT, TT>(a, ldesc, min(wv + q * nw, units - 1), nsb, g, stage + q * TT * GU_SLOT, b[q]);
  for (int unit = wv; unit < units; unit += DEPTH * nw) {
#pragma unroll
    for (int q = 0; q < DEPTH; ++q) {
      const int cu = unit + q * nw;
      // this unit's activation rows have landed once no more than the loads
      // issued after them are outstanding (its own weights and the other
      // units' loads); the memory clobber keeps the LDS reads below
      asm volatile("s_waitcnt vmcnt(%0)" ::"n"(dn_load_count<FMT, TT>() - TT + (DEPTH - 1) * dn_load_count<FMT, TT>())
                   : "memory");
      if (cu < units) {
        const int uu = cu / nsb;
        const uint32_t mask = (uint32_t)__builtin_amdgcn_readfirstlane(ldesc[2 * uu + 1]);
        const bool routed = tok < TT && ((mask >> tok) & 1u);
        const int arow = part * TT + tok;
        const char* base = routed ? stage + q * TT * GU_SLOT + (arow >> 1) * GU_SLOT + 512 * (arow & 1) : zrow;
        const int hh = routed ? (arow & 1) : 0;
        const ALane al{base + 16 * ks + 128 * hh, base + 16 * ks - 128 * hh};
        down_compute<FMT, (TT < 4 ? TT : 4)>(b[q], al, lwt + uu * WTAB + wt_off, out);
      }
      // the slot is refilled only once its operand reads have completed: a
      // buffer->LDS load issued while a read of the same bytes is still
      // queued can land first (L2-resident rows return quickly), and the
      // compiler moves the refill up among this unit's MFMAs, so the wait
      // must be a hardware one, not only a compiler barrier
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
      down_load<FMT, TT>(a, ldesc, min(cu + DEPTH * nw, units - 1), nsb, g, stage + q * TT * GU_SLOT, b[q]);
    }
  }
  reinterpret_cast<float4*>(red)[(size_t)wv * 64 + lane] = make_float4(out[0], out[1], out[2], out[3]);
  __syncthreads();                                   // (also drains the last, unused loads)
  for (int idx = threadIdx.x; idx < 16 * TT; idx += blockDim.x) {
    const int row = idx & 15, t = idx >> 4;
    // D row (part q, token t) sits in lane 16 (2q + t / 4) + row, element t % 4
    const int l0 = 16 * (t >> 2) + row, l1 = l0 + 32, v = t & 3;
    float s = 0.f;
    for (int w = 0; w < nw; ++w) {
      const float* r = red + (size_t)w * 256 + v;
      s += r[4 * l0] + r[4 * l1];
    }
    const int h = g * 16 + row;
    const size_t o = (size_t)t * a.Ho + h;
    if (a.flags & 2u) {
      s += a.x_f32 ? reinterpret_cast<const float*>(a.x)[o]
                   : bf16_to_f32(reinterpret_cast<const uint16_t*>(a.x)[o]);
    }
    if (a.flags & 1u) s += a.out[o];
    a.out[o] = s;
  }
}

// down + weighted combine for 9..16 tokens (and for fewer when k_down's LDS
// cannot hold the call): the work split of k_down (one 16-row group of H
// per workgroup, waves taking (active expert, superblock) units two at a
// time).  A row = token lane % 16, one operand per fp16 part.  Only the rows
// of tokens routed to the unit's expert are staged: one buffer->LDS load of
// 1 KiB per token (its two parts are adjacent in the activation buffer,
// [active expert][token][part][I]) into the next free slot; lanes of other
// tokens read the wave's zero row.  A unit stages its first S routed
// tokens with its own loads (always S of them, the unused
// ones past the end of the buffer: a fixed count keeps the waits static);
// an expert with more routed tokens takes further passes over the same
// weights, each staging the next S (the rows of each token are
// fixed, so the passes add up in one accumulator).
constexpr int DN16_DEPTH = 2;
// S = staged token slots per unit: 7 (an expert's routed tokens at 16 tokens
// per call rarely exceed it) where the call's routing table leaves room in
// LDS, else 4
constexpr int DN16_SLOTS_WIDE = 7, DN16_SLOTS_NARROW = 4;
template <int S> constexpr int dn16_wave_bytes() { return (DN16_DEPTH * S + 1) * GU_SLOT; }

template <int FMT> struct DownUnit16 {
  Codes<FMT> cd;
  uint4 sc;
};

// vector-memory instructions of one unit: the token rows, then codes and scales
template <int FMT>
constexpr int dn16_load_count(int S) { return S + (FMT == 2 ? 2 : 3); }

// Token rows of ranks first .. first + S - 1 among the tokens of
// mask (expert u, superblock sb) into the slots at slot; ranks past the
// last routed token load from past the end of the buffer.
template <int S>
__device__ inline void down16_rows(const ExpertArgs& a, int u, int sb, uint32_t mask, int first, char* slot) {
  const int lane = threadIdx.x & 63;
  const int h = lane >> 5, gch = (lane & 31) ^ (8 * h);
  const rsrc_t ar = make_rsrc(a.w.actp, a.actp_bytes);
  uint32_t m = mask;
  for (int r = 0; r < first; ++r) m &= m - 1u;
#pragma unroll
  for (int j = 0; j < S; ++j) {
    const int t = m ? __builtin_ctz(m) : 0;
    // rows (u, t, part 0) and (u, t, part 1): 512 bytes of superblock sb each
    const uint32_t off = m ? (uint32_t)((((size_t)u * a.T + t) * NPART * a.I + (size_t)sb * SB_WEIGHTS) * 2 +
                                        (size_t)h * a.I * 2 + 16 * gch)
                           : OOB;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(ar, (lds_void_t*)(slot + j * GU_SLOT), 16, off, 0, 0, 0);
    m &= m - 1u;
  }
}

template <int FMT, int S>
__device__ inline void down16_load(const ExpertArgs& a, const int* ldesc, int unit, int nsb, int g, char* slot,
                                   DownUnit16<FMT>& du) {
  const int lane = threadIdx.x & 63, r = lane & 15;
  const int u = unit / nsb, sb = unit - u * nsb;
  const int e = __builtin_amdgcn_readfirstlane(ldesc[DESC * u]);
  const uint32_t mask = (uint32_t)__builtin_amdgcn_readfirstlane(ldesc[DESC * u + 1]);
  down16_rows<S>(a, u, sb, mask, 0, slot);
  const rsrc_t wr = make_rsrc(a.packed + (size_t)e * a.stride, (uint32_t)a.stride);
  const uint32_t soff = (uint32_t)(down_off(FMT, a.H, a.I) + ((size_t)g * nsb + sb) * (Fmt<FMT>::slab_codes + 256));
  bload_codes<FMT>(wr, soff, lane, du.cd);
  du.sc = bload4(wr, Fmt<FMT>::slab_codes + r * 16, soff);
}

// acc += this unit's 16x16 product for the tokens staged in the slots (A
// row = token lane % 16, its two parts from al0 / al1)
template <int FMT>
__device__ inline void down16_product(const DownUnit16<FMT>& du, const ALane& al0, const ALane& al1, float* acc) {
  f32x4 dd[2];
  f16x8 a0[8], a1[8];
  a0[0] = as_f16x8(*a_operand<0>(al0)); a0[1] = as_f16x8(*a_operand<1>(al0));
  a0[2] = as_f16x8(*a_operand<2>(al0)); a0[3] = as_f16x8(*a_operand<3>(al0));
  a0[4] = as_f16x8(*a_operand<4>(al0)); a0[5] = as_f16x8(*a_operand<5>(al0));
  a0[6] = as_f16x8(*a_operand<6>(al0)); a0[7] = as_f16x8(*a_operand<7>(al0));
  a1[0] = as_f16x8(*a_operand<0>(al1)); a1[1] = as_f16x8(*a_operand<1>(al1));
  a1[2] = as_f16x8(*a_operand<2>(al1)); a1[3] = as_f16x8(*a_operand<3>(al1));
  a1[4] = as_f16x8(*a_operand<4>(al1)); a1[5] = as_f16x8(*a_operand<5>(al1));
  a1[6] = as_f16x8(*a_operand<6>(al1)); a1[7] = as_f16x8(*a_operand<7>(al1));
  __builtin_amdgcn_sched_barrier(0);
#define STRATA_BLOCK(BB)                                                          \
  {                                                                               \
    f32x4 d = block_offset_acc<FMT>(a1[BB], block_offset<FMT>(a0[BB]));           \
    d = block_product<FMT, BB>(a0[BB], du.cd, d);                                 \
    dd[BB & 1] = block_product<FMT, BB>(a1[BB], du.cd, d);                        \
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

// dynamic LDS of k_down16: the routing table, partial sums, staged rows
template <int S>
inline size_t down16_lds(int umax) {
  return (((size_t)umax * (DESC + WTAB16) * 4 + 15) & ~(size_t)15) + (size_t)DN_WAVES * 1024 +
         (size_t)DN_WAVES * dn16_wave_bytes<S>();
}

template <int FMT, int S>
__global__ __launch_bounds__(64 * DN_WAVES) void k_down16(ExpertArgs a) {
  extern __shared__ float4 lds_dn4[];
  char* lds = reinterpret_cast<char*>(lds_dn4);
  const int U = a.w.meta[0];
  const int nsb = a.I / SB_WEIGHTS, T = a.T;
  const int lane = threadIdx.x & 63, nw = blockDim.x >> 6, ks = lane >> 4;
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int g = blockIdx.x;
  int* ldesc = reinterpret_cast<int*>(lds);                        // [umax][2]: expert, token mask
  float* lwt = reinterpret_cast<float*>(ldesc + DESC * a.umax);    // [umax][WTAB16]
  const size_t tb = ((size_t)a.umax * (DESC + WTAB16) * 4 + 15) & ~(size_t)15;
  float* red = reinterpret_cast<float*>(lds + tb);                 // [nw][64 lanes][4]
  char* stage = lds + tb + (size_t)DN_WAVES * 1024 + (size_t)wv * dn16_wave_bytes<S>();
  char* zrow = stage + DN16_DEPTH * S * GU_SLOT;
  reinterpret_cast<uint2*>(zrow)[lane] = make_uint2(0u, 0u);
  if (g == 0 && threadIdx.x == 0) a.w.meta[3] = 0;                 // the part-1 flag is consumed
  for (int i = threadIdx.x; i < DESC * a.umax; i += blockDim.x) ldesc[i] = a.w.udesc[i];
  for (int i = threadIdx.x; i < a.umax * WTAB16; i += blockDim.x) lwt[i] = a.w.wtab[i];
  __syncthreads();

  const int units = U * nsb;
  const int tok = lane & 15;                                       // this lane's A row
  const int wt_off = 4 * (lane >> 4);                              // token of this lane's D element 0
  const ALane zl = a_lane(zrow, 0, ks);
  float out[4] = {0.f, 0.f, 0.f, 0.f};
  DownUnit16<FMT> b[DN16_DEPTH];
  // every load unconditional (unit index clamped; a repeated unit is loaded
  // but not computed)
#pragma unroll
  for (int q = 0; q < DN16_DEPTH; ++q)
    down16_load<FMT, S>(a, ldesc, min(wv + q * nw, units - 1), nsb, g, stage + q * S * GU_SLOT, b[q]);
  for (int unit = wv; unit < units; unit += DN16_DEPTH * nw) {
#pragma unroll
    for (int q = 0; q < DN16_DEPTH; ++q) {
      const int cu = unit + q * nw;
      char* slots = stage + q * S * GU_SLOT;
      // this unit's token rows have landed once no more than the loads
      // issued after them are outstanding (its weights and the other unit's
      // loads); the memory clobber keeps the LDS reads below
      asm volatile("s_waitcnt vmcnt(%0)" ::"n"(dn16_load_count<FMT>(S) - S +
                                               (DN16_DEPTH - 1) * dn16_load_count<FMT>(S))
                   : "memory");
      if (cu < units) {
        const int uu = cu / nsb, sb = cu - uu * nsb;
        const uint32_t mask = (uint32_t)__builtin_amdgcn_readfirstlane(ldesc[DESC * uu + 1]);
        const int n = __popc(mask);
        const bool routed = tok < T && ((mask >> tok) & 1u);
        const int rank = __popc(mask & ((1u << tok) - 1u));     // among the unit's tokens
        float acc[4] = {0.f, 0.f, 0.f, 0.f};
        for (int first = 0;;) {
          const bool here = routed && rank >= first && rank < first + S;
          const ALane l0 = here ? a_lane(slots, 2 * (rank - first), ks) : zl;
          const ALane l1 = here ? a_lane(slots, 2 * (rank - first) + 1, ks) : zl;
          down16_product<FMT>(b[q], l0, l1, acc);
          first += S;
          if (first >= n) break;
          // an expert with more routed tokens: stage the next ones (after
          // this pass's reads) and wait for them
          asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
          down16_rows<S>(a, uu, sb, mask, first, slots);
          asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        }
        const float* wt = lwt + uu * WTAB16 + wt_off;
#pragma unroll
        for (int v = 0; v < 4; ++v) out[v] = fmaf(wt[v], acc[v], out[v]);
      }
      // the slots are refilled only once their operand reads have completed
      // (see k_down)
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
      down16_load<FMT, S>(a, ldesc, min(cu + DN16_DEPTH * nw, units - 1), nsb, g, slots, b[q]);
    }
  }
  reinterpret_cast<float4*>(red)[(size_t)wv * 64 + lane] = make_float4(out[0], out[1], out[2], out[3]);
  __syncthreads();                                   // (also drains the last, unused loads)
  for (int idx = threadIdx.x; idx < 16 * T; idx += blockDim.x) {
    const int row = idx & 15, t = idx >> 4;
    // D row t sits in lane 16 (t / 4) + row, element t % 4
    const int l0 = 16 * (t >> 2) + row, v = t & 3;
    float s = 0.f;
    for (int w = 0; w < nw; ++w) s += red[(size_t)w * 256 + 4 * l0 + v];
    const int h = g * 16 + row;
    const size_t o = (size_t)t * a.Ho + h;
    if (a.flags & 2u) {
      s += a.x_f32 ? reinterpret_cast<const float*>(a.x)[o]
                   : bf16_to_f32(reinterpret_cast<const uint16_t*>(a.x)[o]);
    }
    if (a.flags & 1u) s += a.out[o];
    a.out[o] = s;
  }
}

// Whether a call's down kernel keeps what it needs in LDS: up to 8 tokens
// the staged kernel (routing table, partial sums, staged activation rows),
// else the register-operand kernel (routing table, partial sums; its
// activation rows must also lie within the 2 GiB a buffer offset
// addresses).  A call of up to 8 tokens that the staged kernel cannot hold
// takes the register-operand kernels.
bool narrow_fits(int T, int umax) {
  size_t need = 0;
  switch (T) {
    case 1: need = down_lds<1>(umax); break;
    case 2: need = down_lds<2>(umax); break;
    case 3: need = down_lds<3>(umax); break;
    case 4: need = down_lds<4>(umax); break;
    case 5: need = down_lds<5>(umax); break;
    case 6: need = down_lds<6>(umax); break;
    case 7: need = down_lds<7>(umax); break;
    default: need = down_lds<8>(umax); break;
  }
  return need <= DECODE_LDS_MAX;
}

bool wide_fits(int T, int umax, int I) {
  return down16_lds<DN16_SLOTS_NARROW>(umax) <= DECODE_LDS_MAX &&
         (size_t)umax * T * NPART * I * 2 < ((size_t)1 << 31);
}

template <int FMT>
hipError_t launch_experts_fmt(const Layer& L, const Work& W, const Call& c, hipStream_t s, Tracer* tr) {
  ExpertArgs a;
  a.packed = L.packed;
  a.stride = L.expert_stride;
  a.H = L.H; a.I = L.I; a.E = L.E; a.k = L.k; a.T = c.T; a.P = c.T * L.k; a.n_shared = L.n_shared;
  a.Ho = L.Ho;
  a.x = c.x; a.x_f32 = c.x_f32; a.flags = c.flags; a.out = c.out; a.w = W;
  const int umax = (a.P < L.E ? a.P : L.E) + L.n_shared;
  a.umax = umax;
  a.actp_bytes = (uint32_t)((size_t)umax * c.T * NPART * L.I * 2);
  // gate/up waves: the largest divisor of the superblock count that is <= 10,
  // so every wave takes the same number of superblocks.  Row groups per
  // workgroup: 4 when 2 would give more workgroups than CUs (one 10-wave
  // workgroup fits a CU at this register count); Q3/Q4 keep 2 (4 would spill).
  // (and whose wave regions fit in LDS: always 10 here, as a wave stages
  // at most 8 row pairs)
  const int nsbH = L.H / SB_WEIGHTS;
  const bool wide_t = c.T > DECODE_NARROW_T || !narrow_fits(c.T, umax);
  const int npr = wide_t ? (c.T + 1) / 2 : c.T;     // row pairs one staging loads
  const size_t wave_lds = (size_t)std::max(8192, (npr + 1) * GU_SLOT);
  // The wide kernels take 2 row groups and at most 5 waves: three such
  // workgroups share a CU, so a call's many active experts spread evenly
  // instead of a second round of 10-wave workgroups on some CUs.
  const int max_waves = wide_t ? GU_MAX_WAVES / 2 : GU_MAX_WAVES;
  int nwg = 1;
  for (int d = 1; d <= max_waves; ++d)
    if (nsbH % d == 0 && d * wave_lds <= GU_DYN_LDS) nwg = d;
  const bool wide = !wide_t && FMT == 2 && (L.I % 64 == 0) && (size_t)(L.I / 32) * umax > 256;
  const int G = wide ? 4 : 2;
  const size_t lds_gu = (size_t)nwg * wave_lds;   // ceiling raised at create

  // prefetch: the next stack layer's router rows (as its router kernel's
  // workgroups read them) and the down slabs
  a.pf_key = 0x9E3779B9u;
  a.pf_down = 1;
  a.pf_next = c.next_router ? (const void*)c.next_router : (const void*)L.packed;
  a.pf_next_bytes = c.next_router ? (uint32_t)((size_t)c.next_E * c.next_Ho * 4) : 0u;
  a.pf_next_chunk = c.next_router ? decode_route_chunk_bytes(c.T, c.next_Ho) : 1024u;
  a.pf_next_chunks = c.next_router ? (int)((a.pf_next_bytes + a.pf_next_chunk - 1) / a.pf_next_chunk) : 0;
  const dim3 ggu(L.I / (16 * G), umax);
#define STRATA_GATEUP(GG)                                                                  \
  if (wide_t) launch(tr, k_gateup<FMT, GG, true, 4>, ggu, dim3(64 * nwg), lds_gu, s, a);    \
  else if (c.T == 1) launch(tr, k_gateup<FMT, GG, false, 1>, ggu, dim3(64 * nwg), lds_gu, s, a); \
  else if (c.T == 2) launch(tr, k_gateup<FMT, GG, false, 2>, ggu, dim3(64 * nwg), lds_gu, s, a); \
  else if (c.T == 3) launch(tr, k_gateup<FMT, GG, false, 3>, ggu, dim3(64 * nwg), lds_gu, s, a); \
  else launch(tr, k_gateup<FMT, GG, false, 4>, ggu, dim3(64 * nwg), lds_gu, s, a);
  if constexpr (FMT == 2) {
    if (wide) { STRATA_GATEUP(4) } else { STRATA_GATEUP(2) }
  } else {
    STRATA_GATEUP(2)
  }
#undef STRATA_GATEUP
  if (wide_t) {
    if (down16_lds<DN16_SLOTS_WIDE>(umax) <= DECODE_LDS_MAX)
      launch(tr, k_down16<FMT, DN16_SLOTS_WIDE>, dim3(L.Ho / 16), dim3(64 * DN_WAVES),
             down16_lds<DN16_SLOTS_WIDE>(umax), s, a);
    else
      launch(tr, k_down16<FMT, DN16_SLOTS_NARROW>, dim3(L.Ho / 16), dim3(64 * DN_WAVES),
             down16_lds<DN16_SLOTS_NARROW>(umax), s, a);
    return hipGetLastError();
  }
  switch (c.T) {
#define STRATA_DOWN(TT)                                                                            \
    case TT:                                                                                       \
      launch(tr, k_down<FMT, TT>, dim3(L.Ho / 16), dim3(64 * DN_WAVES), down_lds<TT>(umax), s, a);   \
      break;
    STRATA_DOWN(1) STRATA_DOWN(2) STRATA_DOWN(3) STRATA_DOWN(4)
    STRATA_DOWN(5) STRATA_DOWN(6) STRATA_DOWN(7) STRATA_DOWN(8)
#undef STRATA_DOWN
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <int FMT, int TT>
hipError_t raise_down_lds() {
  return hipFuncSetAttribute(reinterpret_cast<const void*>(&k_down<FMT, TT>),
                             hipFuncAttributeMaxDynamicSharedMemorySize, (int)DECODE_LDS_MAX);
}

template <int FMT>
hipError_t raise_down_lds_all() {
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&k_down16<FMT, DN16_SLOTS_WIDE>),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)DECODE_LDS_MAX);
  if (e == hipSuccess)
    e = hipFuncSetAttribute(reinterpret_cast<const void*>(&k_down16<FMT, DN16_SLOTS_NARROW>),
                            hipFuncAttributeMaxDynamicSharedMemorySize, (int)DECODE_LDS_MAX);
  if (e == hipSuccess) e = raise_down_lds<FMT, 1>();
  if (e == hipSuccess) e = raise_down_lds<FMT, 2>();
  if (e == hipSuccess) e = raise_down_lds<FMT, 3>();
  if (e == hipSuccess) e = raise_down_lds<FMT, 4>();
  if (e == hipSuccess) e = raise_down_lds<FMT, 5>();
  if (e == hipSuccess) e = raise_down_lds<FMT, 6>();
  if (e == hipSuccess) e = raise_down_lds<FMT, 7>();
  if (e == hipSuccess) e = raise_down_lds<FMT, 8>();
  return e;
}

template <int FMT, int G, bool WIDE, int NV>
hipError_t raise_gateup_lds1() {
  return hipFuncSetAttribute(reinterpret_cast<const void*>(&k_gateup<FMT, G, WIDE, NV>),
                             hipFuncAttributeMaxDynamicSharedMemorySize, (int)GU_DYN_LDS);
}

template <int FMT, int G>
hipError_t raise_gateup_lds_g() {
  hipError_t e = raise_gateup_lds1<FMT, G, true, 4>();
  if (e == hipSuccess) e = raise_gateup_lds1<FMT, G, false, 1>();
  if (e == hipSuccess) e = raise_gateup_lds1<FMT, G, false, 2>();
  if (e == hipSuccess) e = raise_gateup_lds1<FMT, G, false, 3>();
  if (e == hipSuccess) e = raise_gateup_lds1<FMT, G, false, 4>();
  return e;
}

template <int FMT>
hipError_t raise_gateup_lds() {
  hipError_t e = raise_gateup_lds_g<FMT, 2>();
  if constexpr (FMT == 2) {
    if (e == hipSuccess) e = raise_gateup_lds_g<FMT, 4>();
  }
  return e;
}

template <int V1>
hipError_t launch_topk_v1(const TopkArgs& t, hipStream_t s, Tracer* tr) {
  if (t.k <= 16) launch(tr, k_topk<V1, 2>, dim3(t.T), dim3(64 * TOPK_WAVES), 0, s, t);
  else launch(tr, k_topk<V1, 8>, dim3(t.T), dim3(64 * TOPK_WAVES), 0, s, t);
  return hipGetLastError();
}

}  // namespace

// The gate/up kernels always fit (one wave region at the least).
bool decode_fits(int T, int k, int E, int n_shared, int I) {
  if (T < 1 || T > DECODE_MAX_T) return false;
  const int umax = (T * k < E ? T * k : E) + n_shared;
  return (T <= DECODE_NARROW_T && narrow_fits(T, umax)) || wide_fits(T, umax, I);
}

hipError_t prepare_decode_kernels() {
  hipError_t e = raise_gateup_lds<2>();
  if (e == hipSuccess) e = raise_gateup_lds<3>();
  if (e == hipSuccess) e = raise_gateup_lds<4>();
  if (e == hipSuccess) e = raise_gateup_lds<FMT_MXFP4>();
  if (e == hipSuccess) e = raise_down_lds_all<2>();
  if (e == hipSuccess) e = raise_down_lds_all<3>();
  if (e == hipSuccess) e = raise_down_lds_all<4>();
  if (e == hipSuccess) e = raise_down_lds_all<FMT_MXFP4>();
  return e;
}

hipError_t launch_topk_block(const float* rows, size_t stride, const float* bias, int T, int E, int k, int* idx,
                             float* w, hipStream_t s, Tracer* tr) {
  launch(tr, k_topk_block, dim3(T), dim3(1024), 0, s, rows, stride, bias, E, k, idx, w);
  return hipGetLastError();
}

uint32_t decode_route_chunk_bytes(int T, int Ho) {
  return (uint32_t)(route_rows(T <= DECODE_NARROW_T ? T : 16) * Ho * 4);
}

hipError_t launch_decode_route(const Layer& L, const Work& W, const Call& c, hipStream_t s, Tracer* tr,
                               bool permutation) {
  RouteArgs a;
  a.Wr = L.router_w; a.bias = L.router_b; a.x = c.x; a.x_f32 = c.x_f32; a.T = c.T;
  a.H = L.H; a.Ho = L.Ho; a.E = L.E; a.logits = W.logits; a.xparts = W.xparts; a.part1 = W.meta + 3;
  a.texp = W.texp;
  switch (c.T) {
#define STRATA_ROUTE(TT)                                                                 \
    case TT:                                                                               \
      if (c.x_f32)                                                                         \
        launch(tr, k_route_gemv<TT, true>, dim3((L.E + route_rows(TT) - 1) / route_rows(TT)), \
               dim3(64 * ROUTE_WAVES), 0, s, a);                                           \
      else                                                                                 \
        launch(tr, k_route_gemv<TT, false>, dim3((L.E + route_rows(TT) - 1) / route_rows(TT)), \
               dim3(64 * ROUTE_WAVES), 0, s, a);                                           \
      break;
    STRATA_ROUTE(1) STRATA_ROUTE(2) STRATA_ROUTE(3) STRATA_ROUTE(4)
    STRATA_ROUTE(5) STRATA_ROUTE(6) STRATA_ROUTE(7) STRATA_ROUTE(8)
    case 9: case 10: case 11: case 12: case 13: case 14: case 15:
    STRATA_ROUTE(16)
#undef STRATA_ROUTE
    default: return hipErrorInvalidValue;
  }
  TopkArgs t;
  t.T = c.T; t.E = L.E; t.k = L.k; t.n_shared = L.n_shared; t.w = W;
  t.x = c.x; t.x_f32 = c.x_f32; t.H = L.H; t.Ho = L.Ho;
  const int per_wave = (L.E + 64 * TOPK_WAVES - 1) / (64 * TOPK_WAVES);
  hipError_t e = hipSuccess;
  if (L.k > 64) launch(tr, k_topk_block_decode, dim3(c.T), dim3(1024), 0, s, t);
  else if (per_wave <= 1) e = launch_topk_v1<1>(t, s, tr);
  else if (per_wave <= 2) e = launch_topk_v1<2>(t, s, tr);
  else if (per_wave <= 4) e = launch_topk_v1<4>(t, s, tr);
  else e = launch_topk_v1<8>(t, s, tr);
  if (e != hipSuccess) return e;
  if (permutation) launch(tr, k_permute, dim3(1), dim3(512), (size_t)L.E * 8, s, t);
  return hipGetLastError();
}

hipError_t launch_decode_experts(const Layer& L, const Work& W, const Call& c, hipStream_t s, Tracer* tr) {
  switch (L.fmt) {
    case 2: return launch_experts_fmt<2>(L, W, c, s, tr);
    case 3: return launch_experts_fmt<3>(L, W, c, s, tr);
    case 4: return launch_experts_fmt<4>(L, W, c, s, tr);
    default: return launch_experts_fmt<FMT_MXFP4>(L, W, c, s, tr);
  }
}

}  // namespace strata
