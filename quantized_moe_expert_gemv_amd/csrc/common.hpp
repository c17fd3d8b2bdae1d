// Shared definitions of the strata_moe HIP library (gfx950, wave64).
//
// Packed expert layout ("packed"), written once by the create-time repack.
// The bytes are the canonical ones (codes + fp16 scales), regrouped so that
// one 16-B load per lane delivers exactly the operand a lane feeds to a
// 16x16x32 matrix-core instruction:
//
//   A matrix of R rows and reduction length K is cut into 16-row groups and
//   256-weight superblocks (8 quantised blocks).  The bytes of one (group,
//   superblock) form a slab:
//     codes   one 16-B vector per lane (Q4: two vectors, Q3: a 2-bit plane
//             vector plus an 8-B 1-bit plane); lane l holds row l % 16 and,
//             of every block of the superblock, the 8 codes of the K-slice
//             8*(l / 16) .. 8*(l / 16) + 7;
//     scales  16 rows x 8 fp16 (row r at r * 16).
//   Slabs are stored group-major: slab (g, sb) at (g * K/256 + sb) * SLAB.
//   Expert = gate [I x H], up [I x H], down [H x I], back to back.
//
//   Bit order inside a lane (per block, 8 codes for K-offsets e = 0..7):
//     Q2: 16 bits per block (dword w holds blocks 2w | 2w+1 << 16); the code
//         of offset e sits at bit POS2[e] = {0,4,2,6,8,12,10,14}[e], so that
//         masking the dword with 0x33333333 (and after >> 2) yields FP4 nibbles
//         whose byte-wise conversion returns the 8 codes in offset order.
//     Q3: the low two bits as Q2; the third bit of offset e of block 4h + b at
//         bit 4e + b of hi dword h.
//     Q4: 32 bits per block (vector h, dword i holds block 4h + i); byte j
//         holds the codes of offsets j (low nibble) and j + 4 (high nibble),
//         so the dword masked with 0x0F0F0F0F (and after >> 4) is four bytes
//         0000qqqq, each the E4M3 value q 2^-9, whose conversion in byte
//         order returns the codes of offsets 0..3 (4..7).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace strata {

constexpr int WAVE = 64;
constexpr int GROUP_ROWS = 16;
constexpr int SB_WEIGHTS = 256;        // weights per superblock (8 blocks)
constexpr int BLOCK_W = 32;            // weights per quantised block
constexpr int DECODE_MAX_T = 16;      // tokens of one decode call (one pass over the weights)
constexpr int DECODE_NARROW_T = 8;     // up to here the A operand holds 2 parts x 8 tokens

template <int FMT> struct Fmt;
template <> struct Fmt<2> {
  static constexpr int bits = 2, code_bytes = 8, slab_codes = 1024;
  static constexpr float c = 1.5f;
};
template <> struct Fmt<3> {
  static constexpr int bits = 3, code_bytes = 12, slab_codes = 1536;
  static constexpr float c = 3.5f;
};
template <> struct Fmt<4> {
  static constexpr int bits = 4, code_bytes = 16, slab_codes = 2048;
  static constexpr float c = 8.0f;
};
// MXFP4 (OCP Microscaling Formats v1.0): 4-bit E2M1 elements, one E8M0 scale
// per block, no offset
constexpr int FMT_MXFP4 = 5;
template <> struct Fmt<5> {
  static constexpr int bits = 4, code_bytes = 16, slab_codes = 2048;
  static constexpr float c = 0.0f;
};

__host__ __device__ inline int fmt_bits(int fmt) { return fmt == FMT_MXFP4 ? 4 : fmt; }
__host__ __device__ inline int fmt_code_bytes(int fmt) { return 4 * fmt_bits(fmt); }
// canonical block: codes, then the scale (fp16; one E8M0 byte for MXFP4)
__host__ __device__ inline int canon_block_bytes(int fmt) { return fmt_code_bytes(fmt) + (fmt == FMT_MXFP4 ? 1 : 2); }
__host__ __device__ inline int slab_code_bytes(int fmt) { return 16 * 32 * fmt_bits(fmt); }   // 16 rows x 256 codes
// a slab's scales are 16-bit slots (fp16 d, or the E8M0 byte zero-extended)
__host__ __device__ inline int slab_bytes(int fmt) { return slab_code_bytes(fmt) + 256; }
__host__ __device__ inline size_t matrix_bytes(int fmt, int R, int K) {
  return (size_t)(R / GROUP_ROWS) * (K / SB_WEIGHTS) * slab_bytes(fmt);
}
// bytes of one canonical expert record (gate, up, down blocks)
__host__ __device__ inline size_t canon_expert_bytes(int fmt, int H, int I) {
  return (size_t)3 * I * (H / BLOCK_W) * canon_block_bytes(fmt);
}
// bytes of one packed expert (the canonical count, but for MXFP4's 16-bit
// scale slots: one byte more per block)
__host__ __device__ inline size_t packed_expert_bytes(int fmt, int H, int I) {
  return 2 * matrix_bytes(fmt, I, H) + matrix_bytes(fmt, H, I);
}
// byte offsets of the three matrices inside an expert
__host__ __device__ inline size_t gate_off(int, int, int) { return 0; }
__host__ __device__ inline size_t up_off(int fmt, int H, int I) { return matrix_bytes(fmt, I, H); }
__host__ __device__ inline size_t down_off(int fmt, int H, int I) { return 2 * matrix_bytes(fmt, I, H); }
// byte offset of slab (g, sb) inside a matrix with nsb superblocks per row
__host__ __device__ inline size_t slab_off(int fmt, int nsb, int g, int sb) {
  return ((size_t)g * nsb + sb) * slab_bytes(fmt);
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

// Buffer loads: one descriptor (SGPRs) per expert record or workspace
// buffer, a per-lane byte offset (one VGPR) and a wave-uniform byte offset
// (SGPR), so a wave's many slab loads cost no per-slab address registers.
typedef __amdgpu_buffer_rsrc_t rsrc_t;
constexpr int RSRC_WORD3 = 0x00020000;   // raw buffer, 32-bit data format

__device__ inline rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, RSRC_WORD3);
}
__device__ inline uint4 bload4(rsrc_t r, uint32_t voff, uint32_t soff) {
  const auto v = __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0);
  return make_uint4(v[0], v[1], v[2], v[3]);
}
__device__ inline uint2 bload2(rsrc_t r, uint32_t voff, uint32_t soff) {
  const auto v = __builtin_amdgcn_raw_buffer_load_b64(r, voff, soff, 0);
  return make_uint2(v[0], v[1]);
}
__device__ inline uint32_t bload1(rsrc_t r, uint32_t voff, uint32_t soff) {
  return __builtin_amdgcn_raw_buffer_load_b32(r, voff, soff, 0);
}

// DPP lane permutations (gfx9 encodings): xor-1 and xor-2 inside quads,
// mirror inside half-rows of 8 and rows of 16.
constexpr int DPP_QUAD_XOR1 = 0xB1, DPP_QUAD_XOR2 = 0x4E, DPP_ROW_HALF_MIRROR = 0x141,
              DPP_ROW_MIRROR = 0x140;

template <int CTRL>
__device__ inline int dpp_i(int v) {
  return __builtin_amdgcn_update_dpp(0, v, CTRL, 0xF, 0xF, false);
}
template <int CTRL>
__device__ inline float dpp_f(float v) {
  return __int_as_float(dpp_i<CTRL>(__float_as_int(v)));
}

// Sum over the 64 lanes; every lane receives the same (deterministic) result.
__device__ inline float wave_sum(float v) {
  v += dpp_f<DPP_QUAD_XOR1>(v);
  v += dpp_f<DPP_QUAD_XOR2>(v);
  v += dpp_f<DPP_ROW_HALF_MIRROR>(v);
  v += dpp_f<DPP_ROW_MIRROR>(v);          // each row of 16 now holds its row sum
  const float a = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 0));
  const float b = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 16));
  const float c = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 32));
  const float d = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 48));
  return (a + b) + (c + d);
}

__device__ inline void argmax_merge(float& v, int& i, float ov, int oi) {
  if (ov > v || (ov == v && oi < i)) { v = ov; i = oi; }
}

// argmax over the wave of (value, index); ties resolved towards the smaller
// index; every lane receives the result
__device__ inline void wave_argmax(float& v, int& i) {
  argmax_merge(v, i, dpp_f<DPP_QUAD_XOR1>(v), dpp_i<DPP_QUAD_XOR1>(i));
  argmax_merge(v, i, dpp_f<DPP_QUAD_XOR2>(v), dpp_i<DPP_QUAD_XOR2>(i));
  argmax_merge(v, i, dpp_f<DPP_ROW_HALF_MIRROR>(v), dpp_i<DPP_ROW_HALF_MIRROR>(i));
  argmax_merge(v, i, dpp_f<DPP_ROW_MIRROR>(v), dpp_i<DPP_ROW_MIRROR>(i));
  float bv = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 0));
  int bi = __builtin_amdgcn_readlane(i, 0);
#pragma unroll
  for (int r = 16; r < 64; r += 16)
    argmax_merge(bv, bi, __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), r)),
                 __builtin_amdgcn_readlane(i, r));
  v = bv;
  i = bi;
}

__device__ inline float silu_f(float g) { return g / (1.0f + expf(-g)); }

// ------------------------------------------------------------------ token range
// The 16-bit token operands of both paths hold x 2^-e, where e is chosen per
// token from its largest magnitude m (2^(E-1) <= m < 2^E): e = E - 4 when m
// reaches 16 or stays below 2^-4 (either way the scaled token's largest
// magnitude lands in [8, 16)), else 0, and |e| <= 60 (an ordinary token, and
// an all-zero one, is not scaled at all).  The expert sums then come out
// scaled by 2^-e; gate/up takes silu on the unscaled gate and stores
// silu(g) u 2^-2e (the activation goes with the square of the input: a large
// token's would overflow fp16, a tiny token's would sink below fp16's normal
// range and lose its bits), and the combine multiplies that expert output by
// 2^2e.  Every step is a power of two, exact.
constexpr int TOKEN_SCALE_MAX_EXP = 60;
__device__ inline int token_scale_exp(float maxabs) {
  const uint32_t b = __float_as_uint(maxabs);
  const int E = (int)((b >> 23) & 0xffu) - 126;
  const int e = (E > 4 || E < -3) ? E - 4 : 0;
  return b == 0u ? 0 : min(max(e, -TOKEN_SCALE_MAX_EXP), TOKEN_SCALE_MAX_EXP);
}
// 2^n for |n| <= 126, exactly
__device__ inline float pow2i(int n) { return __uint_as_float((uint32_t)(127 + n) << 23); }

// ------------------------------------------------------------------ top-k
// Selection order: value descending, then expert id ascending; NaN ranks
// below every number (-inf included).  Each entry becomes one 64-bit key
// (order-preserving integer image of the float, then the complemented id),
// so "better" is plain unsigned ">" and every comparison below is
// branch-free.  A NaN's image is 0, the image of padding entries (ids past
// E), below -inf's 0x007FFFFF; ties at 0 go to the lower id, so a real
// expert always wins over padding.
__device__ inline uint32_t sortable_bits(float v) {
  const uint32_t b = __float_as_uint(v);
  const uint32_t s = (b & 0x80000000u) ? ~b : (b | 0x80000000u);
  return (v != v) ? 0u : s;
}
__device__ inline float unsortable_bits(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7fffffffu) : ~k);
}

template <int CTRL, int ROWS>
__device__ inline uint64_t dpp_u64(uint64_t v) {
  const uint32_t lo = (uint32_t)v, hi = (uint32_t)(v >> 32);
  const uint32_t l2 = __builtin_amdgcn_update_dpp(lo, lo, CTRL, ROWS, 0xF, false);
  const uint32_t h2 = __builtin_amdgcn_update_dpp(hi, hi, CTRL, ROWS, 0xF, false);
  return ((uint64_t)h2 << 32) | l2;
}
__device__ inline uint64_t umax64(uint64_t a, uint64_t b) { return a > b ? a : b; }

// maximum 64-bit key over the wave; every lane receives it
__device__ inline uint64_t wave_max_u64(uint64_t v) {
  v = umax64(v, dpp_u64<DPP_QUAD_XOR1, 0xF>(v));
  v = umax64(v, dpp_u64<DPP_QUAD_XOR2, 0xF>(v));
  v = umax64(v, dpp_u64<DPP_ROW_HALF_MIRROR, 0xF>(v));
  v = umax64(v, dpp_u64<DPP_ROW_MIRROR, 0xF>(v));       // row maxima
  v = umax64(v, dpp_u64<0x142, 0xA>(v));                 // row_bcast:15 into rows 1, 3
  v = umax64(v, dpp_u64<0x143, 0xC>(v));                 // row_bcast:31 into rows 2, 3
  const uint32_t lo = __builtin_amdgcn_readlane((uint32_t)v, 63);
  const uint32_t hi = __builtin_amdgcn_readlane((uint32_t)(v >> 32), 63);
  return ((uint64_t)hi << 32) | lo;
}

// maximum unsigned 32-bit value over the wave; every lane receives it
__device__ inline uint32_t wave_max_u32(uint32_t v) {
  v = max(v, (uint32_t)dpp_i<DPP_QUAD_XOR1>((int)v));
  v = max(v, (uint32_t)dpp_i<DPP_QUAD_XOR2>((int)v));
  v = max(v, (uint32_t)dpp_i<DPP_ROW_HALF_MIRROR>((int)v));
  v = max(v, (uint32_t)dpp_i<DPP_ROW_MIRROR>((int)v));         // row maxima
  const uint32_t a = __builtin_amdgcn_readlane(v, 0), b = __builtin_amdgcn_readlane(v, 16);
  const uint32_t c = __builtin_amdgcn_readlane(v, 32), d = __builtin_amdgcn_readlane(v, 48);
  return max(max(a, b), max(c, d));
}

__device__ inline uint64_t topk_key(float v, int e) {
  return ((uint64_t)sortable_bits(v) << 32) | (uint32_t)(0xffffffffu - (uint32_t)e);
}

// Finish a selection: lane r < k holds the r-th best key.  Writes the ids in
// ascending order to idx_out[0..k) and the renormalised softmax weights
// (max-shifted exp over the k selected, divided by their sum) to w_out.
__device__ inline void topk_emit(uint64_t my_key, uint64_t top_key, int k, int* idx_out, float* w_out,
                                 int* sel_lds) {
  const int lane = threadIdx.x & (WAVE - 1);
  const int my_id = (int)(0xffffffffu - (uint32_t)my_key);
  const float my_val = unsortable_bits((uint32_t)(my_key >> 32));
  const float top = unsortable_bits((uint32_t)(top_key >> 32));
  const float z = (lane < k) ? expf(my_val - top) : 0.f;
  const float s = wave_sum(z);
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

// Same selection for any E, re-reading the row (plus bias[e] when bias is not
// null) each round.
__device__ inline void wave_topk_loop(const float* row, const float* bias, int E, int k, int* idx_out,
                                      float* w_out, int* sel_lds) {
  const int lane = threadIdx.x & (WAVE - 1);
  uint64_t prev = ~0ull, mine = 0ull, top = 0ull;
  for (int r = 0; r < k; ++r) {
    uint64_t best = 0ull;
    for (int e = lane; e < E; e += WAVE) {
      const uint64_t key = topk_key(row[e] + (bias ? bias[e] : 0.f), e);
      best = umax64(best, (key < prev) ? key : 0ull);
    }
    best = wave_max_u64(best);
    if (r == 0) top = best;
    mine = (lane == r) ? best : mine;
    prev = best;
  }
  topk_emit(mine, top, k, idx_out, w_out, sel_lds);
}

// Radix select over the order-preserving 32-bit images u of the values
// val[i] of ids lane + 64 i (E <= 64*MAXV, one wave): the threshold tau is
// fixed bit by bit from the top (population counts of ballots) and the
// descent stops once exactly k values are >= tau; ties at tau are taken lowest
// id first, and the selected ids come out in ascending order from prefix
// counts of the selection ballots.  Same selection as the rounds above.
template <int MAXV>
__device__ inline void wave_topk_radix(const float (&val)[MAXV], int E, int k, int* idx_out, float* w_out) {
  const int lane = threadIdx.x & (WAVE - 1);
  uint32_t u[MAXV];
#pragma unroll
  for (int i = 0; i < MAXV; ++i) u[i] = (lane + WAVE * i < E) ? sortable_bits(val[i]) : 0u;  // padding ranks lowest
  uint32_t tau = 0;
  for (int b = 31; b >= 0; --b) {
    const uint32_t cand = tau | (1u << b);
    int cnt = 0;
#pragma unroll
    for (int i = 0; i < MAXV; ++i) cnt += __popcll(__ballot(u[i] >= cand));
    if (cnt >= k) {
      tau = cand;
      if (cnt == k) break;                      // {u >= tau} is the selection
    }
  }
  int gt = 0;
#pragma unroll
  for (int i = 0; i < MAXV; ++i) gt += __popcll(__ballot(u[i] > tau));
  const int need = k - gt;                      // ties at tau to take, lowest ids first
  uint32_t umax = 0;
#pragma unroll
  for (int i = 0; i < MAXV; ++i) umax = u[i] > umax ? u[i] : umax;
  umax = (uint32_t)wave_max_u64(umax);
  const float top = unsortable_bits(umax);
  int ties_before = 0, sel_before = 0;
  float zsum = 0.f;
  bool sel[MAXV];
  float z[MAXV];
  int pos[MAXV];
#pragma unroll
  for (int i = 0; i < MAXV; ++i) {
    const bool tie = (u[i] == tau) && (lane + WAVE * i < E);
    const uint64_t tm = __ballot(tie);
    const int trank = ties_before + (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(tm >> 32),
                                          __builtin_amdgcn_mbcnt_lo((uint32_t)tm, 0u));
    ties_before += __popcll(tm);
    sel[i] = (u[i] > tau) || (tie && trank < need);
    const uint64_t sm = __ballot(sel[i]);
    pos[i] = sel_before + (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(sm >> 32),
                                     __builtin_amdgcn_mbcnt_lo((uint32_t)sm, 0u));
    sel_before += __popcll(sm);
    z[i] = sel[i] ? expf(val[i] - top) : 0.f;
    zsum += z[i];
  }
  const float inv = 1.0f / wave_sum(zsum);
#pragma unroll
  for (int i = 0; i < MAXV; ++i) {
    if (sel[i]) {
      idx_out[pos[i]] = lane + WAVE * i;
      w_out[pos[i]] = z[i] * inv;
    }
  }
}

// Sum / maximum over the workgroup (<= 16 waves, blockDim a multiple of 64);
// every thread receives the result.  tmp: >= 16 entries of LDS, reused by
// the next call only after the barrier at the end.
__device__ inline int block_sum_i(int v, int* tmp) {
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6, nw = blockDim.x >> 6;
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  if (lane == 0) tmp[wv] = v;
  __syncthreads();
  int t = 0;
  for (int i = 0; i < nw; ++i) t += tmp[i];
  __syncthreads();
  return t;
}
__device__ inline float block_sum_f(float v, float* tmp) {
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6, nw = blockDim.x >> 6;
  v = wave_sum(v);
  if (lane == 0) tmp[wv] = v;
  __syncthreads();
  float t = 0.f;
  for (int i = 0; i < nw; ++i) t += tmp[i];
  __syncthreads();
  return t;
}
__device__ inline uint32_t block_max_u(uint32_t v, uint32_t* tmp) {
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6, nw = blockDim.x >> 6;
  v = (uint32_t)wave_max_u64(v);
  if (lane == 0) tmp[wv] = v;
  __syncthreads();
  uint32_t t = 0;
  for (int i = 0; i < nw; ++i) t = tmp[i] > t ? tmp[i] : t;
  __syncthreads();
  return t;
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

// Top-k of one row for any k <= E (E <= 4 * blockDim), one workgroup: thread
// i holds the ids 4 i .. 4 i + 3 (so thread order is id order).  The
// threshold key tau is fixed bit by bit from the top (workgroup counts of
// keys >= the candidate) and the descent stops once exactly k keys are >=
// tau; ties at tau are taken lowest id first (ranks from a scan of the tie
// counts in id order), and each selected id's place in the ascending output
// is a scan of the selection counts.  Same selection and weights as the wave
// versions above (values row[e] + bias[e], bias optional).
__device__ inline void block_topk(const float* row, const float* bias, int E, int k, int* idx_out, float* w_out) {
  __shared__ int s_i[16];
  __shared__ float s_f[16];
  __shared__ int2 s_scan[16];
  const int e0 = 4 * threadIdx.x;
  float v[4];
  uint32_t u[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int e = min(e0 + i, E - 1);
    v[i] = row[e] + (bias ? bias[e] : 0.f);
    u[i] = e0 + i < E ? sortable_bits(v[i]) : 0u;   // padding ranks lowest
  }
  uint32_t m = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) m = u[i] > m ? u[i] : m;
  const float top = unsortable_bits(block_max_u(m, reinterpret_cast<uint32_t*>(s_i)));
  uint32_t tau = 0;
  for (int b = 31; b >= 0; --b) {
    const uint32_t cand = tau | (1u << b);
    int c = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) c += u[i] >= cand;
    const int cnt = block_sum_i(c, s_i);
    if (cnt >= k) {
      tau = cand;
      if (cnt == k) break;                  // {u >= tau} is the selection
    }
  }
  int gt = 0, ties = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    gt += u[i] > tau;
    ties += (u[i] == tau) && (e0 + i < E);
  }
  int2 tot;
  const int need = k - block_sum_i(gt, s_i);
  int trank = block_exclusive_scan(make_int2(ties, 0), s_scan, &tot).x;
  bool sel[4];
  int nsel = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const bool tie = (u[i] == tau) && (e0 + i < E);
    sel[i] = (u[i] > tau) || (tie && trank < need);
    trank += tie;
    nsel += sel[i];
  }
  int pos = block_exclusive_scan(make_int2(nsel, 0), s_scan, &tot).x;
  float z[4], zs = 0.f;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    z[i] = sel[i] ? expf(v[i] - top) : 0.f;
    zs += z[i];
  }
  const float inv = 1.0f / block_sum_f(zs, s_f);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    if (sel[i]) {
      idx_out[pos] = e0 + i;
      w_out[pos] = z[i] * inv;
      ++pos;
    }
  }
}

}  // namespace strata
