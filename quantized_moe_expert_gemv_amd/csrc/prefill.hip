// Prefill path (T > 8): the batched regime of the pages, where one prepared
// expert weight serves many tokens of a prefill chunk of up to 8192 tokens
// (devotd.net "Strata memory tiers", section 读取提示与写出回答时;
// blog.5616760.com/0039.html, section 七).  Here every expert is resident in
// HBM, so the chunk is a grouped, genuinely dense contraction and runs on
// the gfx950 matrix cores (fp32 accumulation):
//
//   k_router         x Wr^T, fp32-accurate from bf16 MFMA by splitting Wr
//                    (and an fp32 x) into bf16 high + low parts; split over K
//                    into partial planes when the item grid is small; the
//                    first expert tile also writes the tokens as fp16
//   k_topk_chunks    logits = sum of the planes + b; top-k + renormalised
//                    softmax per token (one wave per token) and, per chunk of
//                    32 tokens, the expert histogram and every pair's rank
//                    inside the chunk; a call of at most 32 tokens (one
//                    chunk) also does the three steps below in the same
//                    workgroup
//   k_colscan        per-expert bases of the chunks (column scan)
//   k_scan           expert counts -> offsets and the flat list of
//                    (expert, 128-row tile) GEMM work items
//   k_scatter        the stable permutation: slot of pair p =
//                    offset[e] + base[e][chunk] + rank  (no atomics, so the
//                    order is (expert, p) on every run)
//   k_gemm_gateup    per work item: gathered fp16 token rows x gate|up
//                    weights dequantised to fp16 in registers -> SwiGLU -> fp16
//   k_gemm_down      per work item: SwiGLU rows x dequantised down weights ->
//                    per-pair output rows (bf16)
//   k_combine        out[t] = sum_j w[t, j] y[slot(t, j)] (+ shared, residual)
//
// The expert GEMMs run on fp16 MFMA (16x16x32, fp32 accumulation): weights
// d (q - c) rounded once to fp16 (11-bit mantissa), activations fp16 (bf16
// inputs exactly, within the fp16 range).
#include <algorithm>
#include <type_traits>

#include "common.hpp"
#include "kernels.hpp"

namespace strata {
namespace {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;

constexpr int BM = PREFILL_BM;      // 128 token rows

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
// 16-byte chunk as a native vector: copies stay in registers (a struct copy can
// become a memcpy through private memory)
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

// two fp32 -> two bf16 (RNE) in one dword, low half first
__device__ inline uint32_t cvt_bf16x2(float a, float b) {
  const f32x2_t v = {a, b};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
}

typedef _Float16 h2_t __attribute__((ext_vector_type(2)));

// 8 bf16 -> 8 fp16 (exact in the fp16 range); 8 fp32 -> 8 fp16 (RNE)
__device__ inline u32x4_t bf16x8_to_f16(u32x4_t v) {
  u32x4_t r;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const f32x2_t f = {__uint_as_float(v[i] << 16), __uint_as_float(v[i] & 0xffff0000u)};
    r[i] = __builtin_bit_cast(uint32_t, __builtin_convertvector(f, h2_t));
  }
  return r;
}
__device__ inline u32x4_t f32x8_to_f16(f32x4_t lo, f32x4_t hi) {
  const f32x2_t p0 = {lo.x, lo.y}, p1 = {lo.z, lo.w}, p2 = {hi.x, hi.y}, p3 = {hi.z, hi.w};
  return u32x4_t{__builtin_bit_cast(uint32_t, __builtin_convertvector(p0, h2_t)),
                 __builtin_bit_cast(uint32_t, __builtin_convertvector(p1, h2_t)),
                 __builtin_bit_cast(uint32_t, __builtin_convertvector(p2, h2_t)),
                 __builtin_bit_cast(uint32_t, __builtin_convertvector(p3, h2_t))};
}

// ------------------------------------------------------------------ routing
struct TopkArgs {
  int T, E, k, nchunks, n_shared;
  int presel;             // 1: the selection is already in topk_idx / topk_w (k > 64)
  int ct;                 // tokens per chunk (prefill_chunk_t)
  int S;                  // router partial planes
  size_t plane;           // elements between planes
  const float* part;      // [S][T][E] partial logits
  const float* bias;      // [E] or null
  const void* x;          // [T][Ho] the tokens (bf16, or fp32 when x_f32)
  int x_f32, H, Ho;
  uint16_t* x16;          // [T][H] their fp16 rows
  const uint32_t* tmax;   // [S][T] each token's largest |x| per router split, or null (read the rows)
  Work w;
};

// The operand scale of token t (one wave): e from the token's largest
// magnitude (token_scale_exp), taken from the router's per-split maxima when
// it wrote them, else from the token row; when e != 0 the wave rewrites the
// token's fp16 row as x 2^-e (the router wrote it unscaled) and marks the
// call scaled (meta[2], cleared by the router kernel, read by the gate/up
// GEMM).
__device__ inline void token_scale(const TopkArgs& a, int t) {
  const int lane = threadIdx.x & 63;
  const int per = a.x_f32 ? 4 : 8;                 // elements per 16-byte load
  const int nch = a.tmax ? 0 : a.Ho / per;
  const char* row = reinterpret_cast<const char*>(a.x) + (size_t)t * a.Ho * (a.x_f32 ? 4 : 2);
  uint32_t m = 0;                                  // largest |x| as bits (non-negative: bit order)
  if (a.tmax && lane < a.S) m = a.tmax[(size_t)lane * a.T + t];
  for (int c0 = 0; c0 < nch; c0 += 4 * 64) {
    uint4 v[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) v[j] = *reinterpret_cast<const uint4*>(row + 16 * (size_t)min(c0 + 64 * j + lane, nch - 1));
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint32_t q[4] = {v[j].x, v[j].y, v[j].z, v[j].w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        if (a.x_f32) {
          m = max(m, q[i] & 0x7fffffffu);
        } else {
          m = max(m, (q[i] & 0x7fffu) << 16);
          m = max(m, q[i] & 0x7fff0000u);
        }
      }
    }
  }
  const int e = token_scale_exp(__uint_as_float((uint32_t)wave_max_u64(m)));
  if (lane == 0) a.w.texp[t] = e;
  if (e == 0) return;
  if (lane == 0) a.w.meta[2] = 1;
  const float sc = pow2i(-e);
  for (int h = 8 * lane; h < a.Ho; h += 8 * 64) {
    float f[8];
#pragma unroll
    for (int i = 0; i < 8; ++i)
      f[i] = a.x_f32 ? reinterpret_cast<const float*>(a.x)[(size_t)t * a.Ho + h + i]
                     : bf16_to_f32(reinterpret_cast<const uint16_t*>(a.x)[(size_t)t * a.Ho + h + i]);
    uint16_t o[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) o[i] = __builtin_bit_cast(uint16_t, (_Float16)(f[i] * sc));
    *reinterpret_cast<uint4*>(a.x16 + (size_t)t * a.H + h) =
        make_uint4(o[0] | (uint32_t)o[1] << 16, o[2] | (uint32_t)o[3] << 16, o[4] | (uint32_t)o[5] << 16,
                   o[6] | (uint32_t)o[7] << 16);
  }
}

// logits of token t for ids lane + 64 i: the partial planes summed in plane
// order, then the bias (ids past E read id E - 1 and are masked by the caller)
template <int MAXV>
__device__ inline void router_row(const TopkArgs& a, int t, float (&val)[MAXV]) {
  const int lane = threadIdx.x & 63;
  int eo[MAXV];
#pragma unroll
  for (int i = 0; i < MAXV; ++i) eo[i] = min(lane + 64 * i, a.E - 1);
  const float* p = a.part + (size_t)t * a.E;
#pragma unroll
  for (int i = 0; i < MAXV; ++i) val[i] = p[eo[i]];
  // the other planes four at a time, every load of a group in flight
  // together; a plane index past the last re-reads the last plane and is not
  // added, so the sum runs over the planes in order
  for (int z0 = 1; z0 < a.S; z0 += 4) {
    float v[4][MAXV];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float* pz = p + (size_t)min(z0 + j, a.S - 1) * a.plane;
#pragma unroll
      for (int i = 0; i < MAXV; ++i) v[j][i] = pz[eo[i]];
    }
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int i = 0; i < MAXV; ++i) val[i] = (z0 + j < a.S) ? val[i] + v[j][i] : val[i];
  }
  if (a.bias) {
    float b[MAXV];
#pragma unroll
    for (int i = 0; i < MAXV; ++i) b[i] = a.bias[eo[i]];
#pragma unroll
    for (int i = 0; i < MAXV; ++i) val[i] += b[i];
  }
}

__device__ inline void token_topk(const TopkArgs& a, int t, int* sel, float* w, int* sel_lds) {
  if (a.E <= 256) {
    float v[4];
    router_row<4>(a, t, v);
    wave_topk_radix<4>(v, a.E, a.k, sel, w);
  } else if (a.E <= 512) {
    float v[8];
    router_row<8>(a, t, v);
    wave_topk_radix<8>(v, a.E, a.k, sel, w);
  } else {
    // one partial plane (the launch guarantees it) re-read per round
    wave_topk_loop(a.part + (size_t)t * a.E, a.bias, a.E, a.k, sel, w, sel_lds);
  }
}

// One chunk of a.ct tokens per workgroup, one wave per token: top-k ids
// (ascending) and renormalised weights; then per expert the bitmask of the
// chunk's tokens that chose it, which gives the chunk's expert histogram and
// each pair's rank among the chunk's earlier tokens with the same expert.
constexpr int TOPK_CHUNK_WAVES = 16;

struct ScanArgs {
  int T, E, k, n_shared, nchunks;
  Work w;
};
__device__ inline void scan_tiles(const ScanArgs& a);
__device__ inline void scatter_pair(const TopkArgs& a, int p);

__global__ __launch_bounds__(64 * TOPK_CHUNK_WAVES) void k_topk_chunks(TopkArgs a) {
  extern __shared__ int lds_i[];
  uint32_t* tmask = reinterpret_cast<uint32_t*>(lds_i);         // [E]
  // the chunk's selections: [ct][k] in LDS after tmask, or (preselected, any
  // k) the chunk's rows of topk_idx
  const int CT = a.ct;
  int* sel = a.presel ? a.w.topk_idx + (size_t)blockIdx.x * CT * a.k : reinterpret_cast<int*>(tmask + a.E);
  __shared__ int s_sel[TOPK_CHUNK_WAVES][64];
  const int wv = threadIdx.x >> 6;
  const int chunk = blockIdx.x, tb = chunk * CT;
  const int k = a.k, E = a.E;
  static_assert(PREFILL_CHUNK_T <= 32, "token masks are 32-bit");
  for (int e = threadIdx.x; e < E; e += blockDim.x) tmask[e] = 0u;
  for (int tl = wv; tl < CT; tl += TOPK_CHUNK_WAVES) {
    const int t = tb + tl;
    if (t >= a.T) continue;
    if (!a.presel) token_topk(a, t, sel + tl * k, a.w.topk_w + (size_t)t * k, s_sel[wv]);
    token_scale(a, t);
  }
  __syncthreads();
  const int nt = min(CT, a.T - tb);
  for (int i = threadIdx.x; i < nt * k; i += blockDim.x) {
    const int e = sel[i];
    if (!a.presel) a.w.topk_idx[(size_t)tb * k + i] = e;
    atomicOr(&tmask[e], 1u << (i / k));
  }
  __syncthreads();
  for (int i = threadIdx.x; i < nt * k; i += blockDim.x)
    a.w.pair_rank[(size_t)tb * k + i] = __popc(tmask[sel[i]] & ((1u << (i / k)) - 1u));
  if (a.nchunks == 1) {
    // a single chunk (T <= CT) is its own column scan: every base is 0 and
    // the chunk's histogram is the expert counts.  This workgroup then holds
    // every pair of the call, so it also takes the scan (offsets, tile list)
    // and the scatter, which would otherwise be two more launches; the
    // barriers order its own global writes for its own reads.
    for (int e = threadIdx.x; e < E; e += blockDim.x) {
      a.w.chunk_base[e] = 0;
      a.w.counts[e] = __popc(tmask[e]);
    }
    __syncthreads();
    ScanArgs sa;
    sa.T = a.T; sa.E = E; sa.k = k; sa.n_shared = a.n_shared; sa.nchunks = 1; sa.w = a.w;
    scan_tiles(sa);
    __syncthreads();
    for (int p = threadIdx.x; p < a.T * k; p += blockDim.x) scatter_pair(a, p);
  } else {
    for (int e = threadIdx.x; e < E; e += blockDim.x) a.w.chunk_base[(size_t)chunk * E + e] = __popc(tmask[e]);
  }
}

// Column scan of the per-chunk expert histograms (chunk-major [nch][E]): each
// count becomes the number of that expert's pairs in earlier chunks, and
// counts[e] the expert's total.  A workgroup takes 64 experts; its 16 waves
// each sum a range of chunks, then rescan it from the ranges' prefix.  Loads
// go in unconditional batches (indices clamped).
constexpr int COLSCAN_GROUPS = 16;

__global__ __launch_bounds__(64 * COLSCAN_GROUPS) void k_colscan(ScanArgs a) {
  __shared__ int part[COLSCAN_GROUPS][64];
  const int E = a.E, nch = a.nchunks;
  const int el = threadIdx.x & 63, g = threadIdx.x >> 6;
  const int e = blockIdx.x * 64 + el, ec = min(e, E - 1);
  const int per = (nch + COLSCAN_GROUPS - 1) / COLSCAN_GROUPS;
  const int c0 = min(nch, g * per), c1 = min(nch, c0 + per);
  int* cb_col = a.w.chunk_base + ec;
  int sum = 0;
  for (int cb = c0; cb < c1; cb += 16) {
    int v[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) v[i] = cb_col[(size_t)min(cb + i, nch - 1) * E];
#pragma unroll
    for (int i = 0; i < 16; ++i) sum += (cb + i < c1) ? v[i] : 0;
  }
  part[g][el] = sum;
  __syncthreads();
  int run = 0;
  for (int q = 0; q < g; ++q) run += part[q][el];
  for (int cb = c0; cb < c1; cb += 16) {
    int v[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) v[i] = cb_col[(size_t)min(cb + i, nch - 1) * E];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      if (cb + i < c1 && e < E) cb_col[(size_t)(cb + i) * E] = run;
      run += (cb + i < c1) ? v[i] : 0;
    }
  }
  if (g == COLSCAN_GROUPS - 1 && e < E) a.w.counts[e] = run;    // the last range ends at the total
}

// row class of a tile: 0 for more than 96 rows, 1 for 65..96, 2 for 33..64,
// 3 for up to 32 (the GEMMs compute 128, 96, 64 and 32 rows for them)
__device__ inline int row_class(int rows) { return rows > 96 ? 0 : rows > 64 ? 1 : rows > 32 ? 2 : 3; }

// Workgroup-wide exclusive scan of an int4 per thread (blockDim a multiple
// of 64, at most 1024); *total gets the sum over the workgroup.
__device__ inline int4 block_exclusive_scan4(int4 v, int4* tmp /* >= 16 */, int4* total) {
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6, nw = blockDim.x >> 6;
  int4 inc = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int ax = __shfl_up(inc.x, o, 64), ay = __shfl_up(inc.y, o, 64);
    const int az = __shfl_up(inc.z, o, 64), aw = __shfl_up(inc.w, o, 64);
    if (lane >= o) { inc.x += ax; inc.y += ay; inc.z += az; inc.w += aw; }
  }
  if (lane == 63) tmp[wv] = inc;
  __syncthreads();
  int4 pre = make_int4(0, 0, 0, 0), tot = make_int4(0, 0, 0, 0);
  for (int i = 0; i < nw; ++i) {
    const int4 t = tmp[i];
    if (i < wv) { pre.x += t.x; pre.y += t.y; pre.z += t.z; pre.w += t.w; }
    tot.x += t.x; tot.y += t.y; tot.z += t.z; tot.w += t.w;
  }
  *total = tot;
  __syncthreads();
  return make_int4(pre.x + inc.x - v.x, pre.y + inc.y - v.y, pre.z + inc.z - v.z, pre.w + inc.w - v.w);
}

__device__ inline int4 class_unit(int c) {
  return make_int4(c == 0, c == 1, c == 2, c == 3);
}
__device__ inline int class_of(const int4& v, int c) { return c == 0 ? v.x : c == 1 ? v.y : c == 2 ? v.z : v.w; }

// Offsets (exclusive scan of the expert counts) and the tile list.  One
// workgroup.  In expert order an entry's tiles are full 128-row tiles and
// then its remainder; that order is cut into 8 contiguous segments of
// ceil(n / 8) tiles (one per XCD in the GEMMs) and each segment is stably
// sorted by row class, so a GEMM workgroup walking its segment in order meets
// the classes in turn.  Each thread places the tiles of its own entries:
// tile j (expert order) of class c in segment x goes to
//   x tp + (segment x's tiles of classes below c) + (class-c tiles in [x tp, j)).
__device__ inline void scan_tiles(const ScanArgs& a) {
  __shared__ int2 tmp[16];
  __shared__ int4 tmp4[16];
  __shared__ int4 bnd[9];          // class counts of the expert-order tiles before each segment start
  const int E = a.E, P = a.T * a.k;
  // exclusive scan over experts (the shared expert is entry E) of (count, tiles)
  // and of the per-class tile counts
  const int n_ent = E + (a.n_shared ? 1 : 0);
  const int per = (n_ent + blockDim.x - 1) / blockDim.x;
  const int e0 = min(n_ent, (int)threadIdx.x * per), e1 = min(n_ent, e0 + per);
  auto cnt_of = [&](int e) { return e < E ? a.w.counts[e] : a.T; };
  int2 loc = make_int2(0, 0);
  int4 cls = make_int4(0, 0, 0, 0);
  for (int e = e0; e < e1; ++e) {
    const int c = cnt_of(e), full = c / BM, rem = c - full * BM;
    loc.x += (e < E) ? c : 0;
    loc.y += full + (rem > 0);
    cls.x += full;
    if (rem > 0) {
      const int4 u = class_unit(row_class(rem));
      cls.x += u.x; cls.y += u.y; cls.z += u.z; cls.w += u.w;
    }
  }
  int2 total;
  int2 base = block_exclusive_scan(loc, tmp, &total);
  int4 ctot;
  const int4 cpre = block_exclusive_scan4(cls, tmp4, &ctot);
  const int n = total.y, tp = (n + 7) / 8;
  // class counts at the segment starts that fall in this thread's tiles
  // (inside an entry only its full tiles precede the start)
  {
    int j = base.y;
    int4 run = cpre;
    for (int e = e0; e < e1; ++e) {
      const int c = cnt_of(e), full = c / BM, rem = c - full * BM, nt = full + (rem > 0);
      for (int x = (j + tp - 1) / tp; x * tp < j + nt; ++x) {
        bnd[x] = make_int4(run.x + (x * tp - j), run.y, run.z, run.w);
      }
      run.x += full;
      if (rem > 0) {
        const int4 u = class_unit(row_class(rem));
        run.x += u.x; run.y += u.y; run.z += u.z; run.w += u.w;
      }
      j += nt;
    }
  }
  if (threadIdx.x == 0) {
    for (int x = (n + tp - 1) / tp; x <= 8; ++x) bnd[x] = ctot;
    a.w.offsets[E] = P;
    a.w.meta[1] = n;
  }
  __syncthreads();
  // Full tiles (class 0) of a segment are placed consecutively from
  // x tp + (class-0 tiles of the segment before them): full tile q of an
  // entry whose tiles start at expert-order index j0, after r0 class-0 tiles,
  // goes to x tp + r0 + q - bnd[x].x with x = (j0 + q) / tp.  A heavy expert
  // has hundreds of them, so each wave writes its lanes' entries' full tiles
  // one entry at a time with all its lanes.  Only an entry's remainder tile
  // needs the lower classes' counts; its own thread places it.
  int4 run = cpre;
  for (int i = 0; i < per; ++i) {
    const int e = e0 + i;
    const bool has = e < e1;
    const int cv = cnt_of(min(e, n_ent - 1));          // (an in-bounds read for every lane)
    const int c = has ? cv : 0, full = c / BM, rem = c - full * BM;
    const int first = (e < E) ? base.x : P;
    if (has && e < E) a.w.offsets[e] = base.x;
    for (uint64_t m = __ballot(full > 0); m; m &= m - 1) {       // the lanes with full tiles
      const int L = __builtin_ctzll(m);
      const int fL = __builtin_amdgcn_readlane(full, L);
      const int eL = __builtin_amdgcn_readlane(e, L), firstL = __builtin_amdgcn_readlane(first, L);
      const int j0 = __builtin_amdgcn_readlane(base.y, L), r0 = __builtin_amdgcn_readlane(run.x, L);
      for (int q = (int)(threadIdx.x & 63); q < fL; q += 64) {
        const int xq = (j0 + q) / tp;
        a.w.tiles[xq * tp + r0 + q - bnd[xq].x] = make_int4(eL, firstL + q * BM, BM, 0);
      }
    }
    base.y += full;
    run.x += full;
    if (has && rem > 0) {
      const int x = base.y / tp;
      const int4 b0 = bnd[x], b1 = bnd[x + 1];
      const int k = row_class(rem);
      int pos = x * tp + class_of(run, k) - class_of(b0, k);
      for (int kk = 0; kk < k; ++kk) pos += class_of(b1, kk) - class_of(b0, kk);
      a.w.tiles[pos] = make_int4(e, first + full * BM, rem, 0);
      const int4 u = class_unit(k);
      run.x += u.x; run.y += u.y; run.z += u.z; run.w += u.w;
      ++base.y;
    }
    if (has && e < E) base.x += c;
  }
}

__global__ __launch_bounds__(1024) void k_scan(ScanArgs a) { scan_tiles(a); }

// slot of pair p: its expert's offset + the pairs of that expert in earlier
// chunks + its rank in its own chunk
__device__ inline void scatter_pair(const TopkArgs& a, int p) {
  const int e = a.w.topk_idx[p];
  const int chunk = (p / a.k) / a.ct;
  const int slot = a.w.offsets[e] + a.w.chunk_base[(size_t)chunk * a.E + e] + a.w.pair_rank[p];
  a.w.perm[slot] = p;
  a.w.inv[p] = slot;
  a.w.slot_tok[slot] = p / a.k;
}

__global__ void k_scatter(TopkArgs a) {
  const int p = blockIdx.x * blockDim.x + threadIdx.x;
  if (p < a.T * a.k) scatter_pair(a, p);
}

// ------------------------------------------------------------------ grouped GEMMs
// fp16 MFMA 16x16x32 with fp32 accumulation.  A work item is one 128-slot
// row tile of an expert (the tile list) times 128 output columns; its four
// waves each take all 128 token rows and 32 columns, so each weight operand is
// dequantised once per work item and feeds up to 8 MFMAs (the dequantisation
// costs VALU time that does not overlap the matrix cores, so it is spread
// over as many token rows as possible).  Subtiles past a short tile's rows
// are skipped 32 rows at a time.  The token rows (A) are staged in LDS as
// fp16, double-buffered, 64 of K per stage, two stages ahead in registers.
// The weights (B) never touch LDS: the slab layout is the B-operand layout
// of this MFMA (lane l holds row l % 16, K-slice 8 (l / 16) of every
// 32-weight block), so each lane dequantises its own operand from the codes
// it loaded half a superblock ahead.
struct GemmArgs {
  const uint8_t* packed;
  size_t stride;
  int H, I, E, k, T, P;
  const uint16_t* x16;     // [T][H] the tokens as fp16 (written by the router GEMM)
  Work w;
};

typedef __attribute__((__vector_size__(8 * sizeof(_Float16)))) _Float16 f16x8;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;

constexpr int XBK = 64;            // K per A stage: two blocks
constexpr int LDA = XBK + 8;       // LDS row pitch in halves (144 B)

// one lane's codes and scales of one slab for two A stages (four blocks)
template <int FMT> struct PairCodes;
template <> struct PairCodes<2> { uint2 w, sc; };
template <> struct PairCodes<3> { uint2 w, sc; uint32_t h; };
template <> struct PairCodes<4> { u32x4_t w; uint2 sc; };
template <> struct PairCodes<5> { u32x4_t w; uint2 sc; };

// blocks 4 hp .. 4 hp + 3 (half hp of the superblock) of a slab for this
// lane: the slab at byte soff of the expert record r
template <int FMT>
__device__ inline void load_pair(rsrc_t r, uint32_t soff, int hp, int lane, PairCodes<FMT>& c) {
  c.sc = bload2(r, Fmt<FMT>::slab_codes + (lane & 15) * 16 + 8 * hp, soff);
  if constexpr (FMT == 4 || FMT == FMT_MXFP4) {
    const uint4 v = bload4(r, hp * 1024 + lane * 16, soff);
    c.w = u32x4_t{v.x, v.y, v.z, v.w};
  } else {
    c.w = bload2(r, lane * 16 + 8 * hp, soff);
    if constexpr (FMT == 3) c.h = bload1(r, 1024 + lane * 8 + 4 * hp, soff);
  }
}

template <int SEL>
__device__ inline h2_t fp4x2_f16(uint32_t src, float scale) {
  return __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(src, scale, SEL);
}

// The B operand of block B (of its superblock) for this lane: its 8 weights
// d (q - c) in K order, as fp16 (one rounding: q d - c d by fused
// multiply-add with c d rounded to fp16 first, exact for Q4's c = 8).
// Codes become fp16 q exactly through the FP4 conversions (nibble 0b00qq at
// scale 2, Q3's third bit 0b000h at scale 8), Q4's through the E4M3
// conversion (byte 0000qqqq is q 2^-9, at scale 2^9).
template <int FMT, int B>
__device__ inline f16x8 dequant_b(const PairCodes<FMT>& c) {
  const uint32_t sw = ((B >> 1) & 1) ? c.sc.y : c.sc.x;
  if constexpr (FMT == FMT_MXFP4) {
    // E2M1 codes times the block's power-of-two scale 2^(e - 127), one
    // conversion per pair (the conversion's scale is exactly that power)
    const uint32_t e = (B & 1) ? (sw >> 16) : (sw & 0xffffu);
    const float s = __uint_as_float(e << 23);
    const uint32_t W = c.w[B & 3];
    const h2_t q0 = fp4x2_f16<0>(W, s), q1 = fp4x2_f16<1>(W, s), q2 = fp4x2_f16<2>(W, s), q3 = fp4x2_f16<3>(W, s);
    f16x8 r;
    r[0] = q0.x; r[1] = q0.y; r[2] = q1.x; r[3] = q1.y;
    r[4] = q2.x; r[5] = q2.y; r[6] = q3.x; r[7] = q3.y;
    return r;
  }
  const _Float16 d = __builtin_bit_cast(_Float16, (uint16_t)((B & 1) ? (sw >> 16) : (sw & 0xffffu)));
  h2_t q[4];
  if constexpr (FMT == 4) {
    const uint32_t W = c.w[B & 3];
    const uint32_t E = W & 0x0F0F0F0Fu, O = (W >> 4) & 0x0F0F0F0Fu;
    q[0] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(E, 512.0f, false);
    q[1] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(E, 512.0f, true);
    q[2] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(O, 512.0f, false);
    q[3] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(O, 512.0f, true);
  } else {
    const uint32_t W = ((B >> 1) & 1) ? c.w.y : c.w.x;
    const uint32_t E = W & 0x33333333u, O = (W >> 2) & 0x33333333u;
    constexpr int b0 = 2 * (B & 1);
    q[0] = fp4x2_f16<b0>(E, 2.0f);
    q[1] = fp4x2_f16<b0>(O, 2.0f);
    q[2] = fp4x2_f16<b0 + 1>(E, 2.0f);
    q[3] = fp4x2_f16<b0 + 1>(O, 2.0f);
    if constexpr (FMT == 3) {
      const uint32_t X = (c.h >> (B & 3)) & 0x11111111u;
      q[0] += fp4x2_f16<0>(X, 8.0f);
      q[1] += fp4x2_f16<1>(X, 8.0f);
      q[2] += fp4x2_f16<2>(X, 8.0f);
      q[3] += fp4x2_f16<3>(X, 8.0f);
    }
  }
  const _Float16 ncd = -((_Float16)Fmt<FMT>::c * d);
  const h2_t d2 = {d, d}, n2 = {ncd, ncd};
#pragma unroll
  for (int k = 0; k < 4; ++k) q[k] = __builtin_elementwise_fma(q[k], d2, n2);
  f16x8 r;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    r[2 * k] = q[k].x;
    r[2 * k + 1] = q[k].y;
  }
  return r;
}

// A stage: 64 of K (two blocks) of the tile's 128 token rows, kept in LDS
// fragment-major: fragment f = 2 m + kb (16-row subtile m, block kb) is the
// 1 KiB A operand of one MFMA; the 16 bytes of its lane p (row 16 m + p % 16,
// columns 32 kb + 8 (p / 16)) sit in 16-byte slot a_slot(p).  Thread (wave
// w, lane l) loads the fragments AF w + i (i < AF) of a stage, four
// neighbouring lanes reading 64 contiguous bytes of one row (one
// address-unit access instead of four): lane l takes row l / 4 of the
// subtile, columns 32 kb + 8 (l % 4), i.e. operand lane l / 4 + 16 (l % 4).
// With the slots XOR 2 (p / 16), both that store and the linear operand
// read are free of LDS bank conflicts (measured on gfx950 with
// SQ_LDS_BANK_CONFLICT).
constexpr int AFRAG = 512;          // halves per fragment
constexpr int ASTAGE = 16 * AFRAG;  // halves per stage (8 subtiles x 2 blocks)
__device__ inline int a_slot(int p) { return p ^ (2 * (p >> 4)); }
constexpr int GEMM_WAVES = 8;
// weight slabs (16 output columns each) per wave: 4 for 2-bit codes; the
// 3- and 4-bit dequantisation needs more registers, so 2 there
template <int FMT> constexpr int nsl() { return FMT == 2 ? 4 : 2; }
constexpr int AF = 16 / GEMM_WAVES;   // fragments of a stage per wave
constexpr int AR = AF / 2;            // token rows per lane
struct AStage { u32x4_t v[AF]; };

// (global address-space loads: a generic pointer's load would also count as
// an LDS access and hold up every LDS read behind it)
typedef __attribute__((address_space(1))) const u32x4_t gu32x4_t;

// Every fragment is loaded and stored, also those of subtiles a short tile
// does not compute (their rows repeat the tile's last row): a load under a
// condition would make the compiler wait for all outstanding loads before
// the next store.  The lane's row is at byte va of the buffer ra; k0 is in
// elements.
__device__ inline void a_load(rsrc_t ra, uint32_t va, int k0, AStage& st) {
#pragma unroll
  for (int i = 0; i < AF; ++i) {
    const uint4 v = bload4(ra, va + 64 * (i & 1), 2 * k0);
    st.v[i] = u32x4_t{v.x, v.y, v.z, v.w};
  }
}

__device__ inline void a_store(const AStage& st, _Float16* buf, int wv, int lane) {
#pragma unroll
  for (int i = 0; i < AF; ++i)
    *reinterpret_cast<u32x4_t*>(buf + (AF * wv + i) * AFRAG + 8 * a_slot((lane >> 2) + 16 * (lane & 3))) = st.v[i];
}

constexpr int MT = BM / 16;        // 16-row subtiles of a tile

// One stage (blocks BB and BB + 1 of the superblock) against the wave's NSL
// slabs: each weight operand is dequantised once and feeds MC MFMAs (one per
// 16-row subtile of the token rows).  The 2 MC token-row operands are read
// from LDS two steps ahead of their MFMAs, so the read latency stays hidden
// behind the MFMAs of the steps in between.
template <int FMT, int BB, int MC, bool TR, int NSL = nsl<FMT>()>
__device__ inline void gemm_stage(const _Float16* buf, const PairCodes<FMT> (&bc)[NSL], int lane,
                                  f32x4 (&acc)[MC][NSL]) {
  constexpr int NS = 2 * MC;                          // steps: (block kb, subtile m), kb-major
  auto rd = [&](int t) __attribute__((always_inline)) {
    const int m = t % MC, kb = t / MC;
    return __builtin_bit_cast(f16x8, *reinterpret_cast<const u32x4_t*>(buf + (2 * m + kb) * AFRAG + 8 * a_slot(lane)));
  };
  f16x8 af[4];
  af[0] = rd(0);
  af[1] = rd(1);
  f16x8 bf[2][NSL];
#pragma unroll
  for (int n = 0; n < NSL; ++n) bf[0][n] = dequant_b<FMT, BB>(bc[n]);
#pragma unroll
  for (int t = 0; t < NS; ++t) {
    if (t + 2 < NS) af[(t + 2) & 3] = rd(t + 2);
    if (t == MC - 1) {
#pragma unroll
      for (int n = 0; n < NSL; ++n) bf[1][n] = dequant_b<FMT, BB + 1>(bc[n]);
    }
    const int m = t % MC, kb = t / MC;
#pragma unroll
    for (int n = 0; n < NSL; ++n)
      acc[m][n] = TR ? __builtin_amdgcn_mfma_f32_16x16x32_f16(bf[kb][n], af[t & 3], acc[m][n], 0, 0, 0)
                     : __builtin_amdgcn_mfma_f32_16x16x32_f16(af[t & 3], bf[kb][n], acc[m][n], 0, 0, 0);
  }
  // keep the reads two steps ahead of the MFMAs that use them
  __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
#pragma unroll
  for (int t = 0; t < NS; ++t) {
    if (t + 2 < NS) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    __builtin_amdgcn_sched_group_barrier(0x008, NSL, 0);
  }
}

// Operand sources of one work item for this lane: its token row (A, byte va
// of buffer ra) and the wave's NSL weight slabs (byte slab[n] of the expert
// record rw; superblock sb of a slab SLAB bytes further per sb).  Buffer
// loads keep the addresses in scalar registers but for one per-lane offset.
static_assert(AR == 1, "one token row per lane");
template <int NSL>
struct ItemSrc {
  rsrc_t ra;
  uint32_t va;
  rsrc_t rw;
  uint32_t slab[NSL];
};

// codes and scales of half h of the K loop (stages 2h, 2h + 1)
template <int FMT, int NSL>
__device__ inline void codes_load(const ItemSrc<NSL>& is, int h, int lane, PairCodes<FMT> (&c)[NSL]) {
  constexpr int SLAB = Fmt<FMT>::slab_codes + 256;
#pragma unroll
  for (int n = 0; n < NSL; ++n) load_pair<FMT>(is.rw, is.slab[n] + (uint32_t)(h >> 1) * SLAB, h & 1, lane, c[n]);
}

// The K loop of one work item, for its first 16 MC token rows.  On entry
// stage 0 of A is in LDS buffer 0, stage 1 in flight in ar[1] and the codes of
// stages 0 and 1 in flight in bc[0].  Stage s + 2 of A is requested while
// stage s is multiplied; stage s + 1 (requested a stage earlier) then goes to
// the other LDS buffer.  Codes run half a superblock (two stages) ahead, in
// two sets.  The last two stages request the next work item's first two A
// stages and first codes (from next(), called only there), which leaves the
// next item's loop the same entry state: the next item's operands are in
// flight while this one's epilogue runs.  K is a multiple of 256, so the
// stage ring positions line up across items.
template <int FMT, int MC, bool TR, int NSL, typename Next>
__device__ inline void gemm_kloop(const ItemSrc<NSL>& cur, Next next, int K, _Float16 (*As)[ASTAGE], int wv,
                                  int lane, AStage (&ar)[4], PairCodes<FMT> (&bc)[2][NSL],
                                  f32x4 (&acc)[MC][NSL]) {
  const int nsb = K / SB_WEIGHTS;
#define STRATA_STAGE(ST, SRC, K0, CODES)                                                \
  {                                                                                     \
    CODES;                                                                              \
    a_load(SRC.ra, SRC.va, K0, ar[(ST + 2) & 3]);                                       \
    __builtin_amdgcn_sched_barrier(0);                                                  \
    gemm_stage<FMT, 2 * ST, MC, TR>(As[ST & 1], bc[(ST / 2) & 1], lane, acc);           \
    a_store(ar[(ST + 1) & 3], As[(ST + 1) & 1], wv, lane);                              \
    __syncthreads();                                                                    \
  }
  for (int sb = 0; sb < nsb - 1; ++sb) {
    const int s = 4 * sb;
    STRATA_STAGE(0, cur, (s + 2) * XBK, codes_load<FMT>(cur, 2 * sb + 1, lane, bc[1]))
    STRATA_STAGE(1, cur, (s + 3) * XBK, (void)0)
    STRATA_STAGE(2, cur, (s + 4) * XBK, codes_load<FMT>(cur, 2 * sb + 2, lane, bc[0]))
    STRATA_STAGE(3, cur, (s + 5) * XBK, (void)0)
  }
  {
    const int sb = nsb - 1, s = 4 * sb;
    STRATA_STAGE(0, cur, (s + 2) * XBK, codes_load<FMT>(cur, 2 * sb + 1, lane, bc[1]))
    STRATA_STAGE(1, cur, (s + 3) * XBK, (void)0)
    const ItemSrc<NSL> nx = next();
    STRATA_STAGE(2, nx, 0, codes_load<FMT>(nx, 0, lane, bc[0]))
    STRATA_STAGE(3, nx, XBK, (void)0)
  }
#undef STRATA_STAGE
}

// first entry state of the K loop (see gemm_kloop)
template <int FMT, int NSL>
__device__ inline void gemm_prologue(const ItemSrc<NSL>& cur, _Float16 (*As)[ASTAGE], int wv, int lane,
                                     AStage (&ar)[4], PairCodes<FMT> (&bc)[2][NSL]) {
  codes_load<FMT>(cur, 0, lane, bc[0]);
  a_load(cur.ra, cur.va, 0, ar[0]);
  a_load(cur.ra, cur.va, XBK, ar[1]);
  a_store(ar[0], As[0], wv, lane);
  __syncthreads();
}

// The work items of a persistent workgroup.  The tile list is cut into 8
// contiguous segments of ceil(n / 8) tiles, one per XCD (the workgroups b
// with b % 8 == x), each sorted by row class; an item is (tile, column tile),
// column tiles of a tile adjacent, and the G = gridDim / 8 workgroups of an
// XCD take every G-th item of its segment.  at(i) is clamped to the
// workgroup's last item, so look-ahead loads past the end stay in bounds.
struct ItemSeq {
  int seg0, n, w0, step, ntn;
  __device__ ItemSeq(int ntiles, int ntn_) {
    const int tp = (ntiles + 7) >> 3;
    seg0 = min(ntiles, (int)(blockIdx.x & 7) * tp);
    n = (min(ntiles, seg0 + tp) - seg0) * ntn_;
    w0 = blockIdx.x >> 3;
    step = gridDim.x >> 3;
    ntn = ntn_;
  }
  __device__ bool valid(int i) const { return w0 + i * step < n; }
  __device__ int at(int i) const { return min(w0 + i * step, w0 + max(0, (n - 1 - w0) / step) * step); }
  __device__ int tile(int i) const { return seg0 + at(i) / ntn; }
  __device__ int col(int i) const { return at(i) % ntn; }
};

// tile entry j, read through the scalar cache (the tile list is read-only
// while the GEMMs run), so the entries and everything derived from them stay
// in scalar registers
typedef const __attribute__((address_space(4))) int* cint_ptr;
__device__ inline int4 tile_entry(const GemmArgs& a, int j) {
  const cint_ptr p = (cint_ptr)(a.w.tiles + j);
  return make_int4(p[0], p[1], p[2], p[3]);
}
__device__ inline int tile_count(const GemmArgs& a) { return *(cint_ptr)(a.w.meta + 1); }

// silu(g) = g / (1 + e^-g) with the hardware exponential and reciprocal
// (relative error a few ulp; the prefill path rounds its result to fp16)
__device__ inline float silu_fast(float g) { return g * __builtin_amdgcn_rcpf(1.0f + __expf(-g)); }

// Column tiles of a work item: GEMM_WAVES waves of nsl() slabs each.
template <int NSL> constexpr int gu_rows() { return GEMM_WAVES * NSL / 2 * 16; }  // rows of I, gate/up
template <int NSL> constexpr int dn_cols() { return GEMM_WAVES * NSL * 16; }      // rows of H, down

// Epilogue staging.  A work item's results are written to an LDS tile of
// [BM rows][NC halves] (16-byte granules of a row XOR-swizzled by row % 8,
// which spreads the 16 rows of one transposed-layout write over the banks)
// and, after a barrier, stored as whole rows: 16 bytes per lane, full
// 128-byte lines.  Stored straight from the MFMA layout, each lane would
// write 8 bytes of 16 different rows per instruction, and the partial-line
// writes cost the expert GEMMs about a third of their time.
__device__ inline void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// 8 bytes (4 halves starting at column c, a multiple of 4) of row `row`
template <int NC>
__device__ inline void stage_put(char* stg, int row, int c, uint2 v) {
  const int g = c >> 3;
  *reinterpret_cast<uint2*>(stg + row * (2 * NC) + ((g ^ (row & 7)) << 4) + ((c & 4) << 1)) = v;
}

// rows [0, rows) of the staged tile to dst (row r at dst + r * pitch halves),
// columns below ncols (a multiple of 8); wave w takes every 8th row group.
// UNR: loop unrolling (a register budget choice of the caller)
template <int NC, int UNR>
__device__ inline void stage_store(const char* stg, int rows, int ncols, _Float16* dst, size_t pitch, int wv,
                                   int lane) {
  constexpr int LPR = NC / 8, RPI = 64 / LPR;         // lanes per row, rows per instruction
  static_assert(LPR <= 64 && 64 % LPR == 0, "staged row width");
  const int gg = lane % LPR, c = 8 * gg;
#pragma unroll UNR
  for (int q = 0; q < BM / (8 * RPI); ++q) {
    const int row = RPI * (wv + 8 * q) + lane / LPR;
    const uint4 v = *reinterpret_cast<const uint4*>(stg + row * (2 * NC) + ((gg ^ (row & 7)) << 4));
    if (row < rows && c < ncols) *reinterpret_cast<uint4*>(dst + (size_t)row * pitch + c) = v;
  }
}

// One gate/up work item with 16 MC computed token rows: K loop, then SwiGLU
// (slabs n < NSL/2 hold gate, n + NSL/2 up, for the same rows i); the lane's
// 4 consecutive i of one token row go out as one 8-byte store.
template <int FMT, int MC, int NSL, typename Next>
__device__ inline void gateup_item(const GemmArgs& a, const ItemSrc<NSL>& cur, Next next, int slot0, int rows,
                                   int col, _Float16 (*As)[ASTAGE], char* stg, int wv, int lane, AStage (&ar)[4],
                                   PairCodes<FMT> (&bc)[2][NSL]) {
  constexpr int NC = gu_rows<NSL>();
  f32x4 acc[MC][NSL];
#pragma unroll
  for (int m = 0; m < MC; ++m)
#pragma unroll
    for (int n = 0; n < NSL; ++n) acc[m][n] = f32x4{0.f, 0.f, 0.f, 0.f};
  gemm_kloop<FMT, MC, true>(cur, next, a.H, As, wv, lane, ar, bc, acc);
  // SwiGLU of this lane's token row 16 m + lane % 16; in a call with scaled
  // tokens (rare) the sums carry the row's 2^-e: silu of the unscaled gate,
  // the activation kept at 2^-2e
  auto swiglu = [&](int m, float sg, float su) __attribute__((always_inline)) {
    const int row = 16 * m + (lane & 15);
#pragma unroll
    for (int n = 0; n < NSL / 2; ++n) {
      h2_t h[2];
#pragma unroll
      for (int v = 0; v < 2; ++v)
        h[v] = h2_t{(_Float16)(silu_fast(acc[m][n][2 * v] * sg) * acc[m][NSL / 2 + n][2 * v] * su),
                    (_Float16)(silu_fast(acc[m][n][2 * v + 1] * sg) * acc[m][NSL / 2 + n][2 * v + 1] * su)};
      stage_put<NC>(stg, row, 16 * (wv * (NSL / 2) + n) + 4 * (lane >> 4),
                    make_uint2(__builtin_bit_cast(uint32_t, h[0]), __builtin_bit_cast(uint32_t, h[1])));
    }
  };
  if (*(cint_ptr)(a.w.meta + 2) == 0) {
#pragma unroll
    for (int m = 0; m < MC; ++m) swiglu(m, 1.f, 1.f);
  } else {
#pragma unroll
    for (int m = 0; m < MC; ++m) {
      const int slot = slot0 + min(16 * m + (lane & 15), rows - 1);
      const int tok = slot < a.P ? a.w.slot_tok[slot] : slot - a.P;
      const int e = a.w.texp[tok];
      swiglu(m, pow2i(e), pow2i(-e));
    }
  }
  lds_barrier();
  stage_store<NC, 2>(stg, rows, NC, reinterpret_cast<_Float16*>(a.w.act) + (size_t)slot0 * a.I + col * NC, a.I, wv,
                  lane);
}

// One down work item with 16 MC computed token rows: K loop (transposed, so
// the lane's 4 results are consecutive h of one token row), then the bf16
// per-pair rows through the staging tile (columns past H, computed by the
// waves past H of the last column tile, are not stored).
template <int FMT, int MC, int NSL, typename Next>
__device__ inline void down_item(const GemmArgs& a, const ItemSrc<NSL>& cur, Next next, int slot0, int rows, int col,
                                 _Float16 (*As)[ASTAGE], char* stg, int wv, int lane, AStage (&ar)[4],
                                 PairCodes<FMT> (&bc)[2][NSL]) {
  constexpr int NC = dn_cols<NSL>();
  f32x4 acc[MC][NSL];
#pragma unroll
  for (int m = 0; m < MC; ++m)
#pragma unroll
    for (int n = 0; n < NSL; ++n) acc[m][n] = f32x4{0.f, 0.f, 0.f, 0.f};
  gemm_kloop<FMT, MC, true>(cur, next, a.I, As, wv, lane, ar, bc, acc);
#pragma unroll
  for (int m = 0; m < MC; ++m) {
    const int row = 16 * m + (lane & 15);
#pragma unroll
    for (int n = 0; n < NSL; ++n)
      stage_put<NC>(stg, row, 16 * (wv * NSL + n) + 4 * (lane >> 4),
                    make_uint2(cvt_bf16x2(acc[m][n][0], acc[m][n][1]), cvt_bf16x2(acc[m][n][2], acc[m][n][3])));
  }
  lds_barrier();
  stage_store<NC, BM>(stg, rows, min(NC, a.H - col * NC),
                  reinterpret_cast<_Float16*>(a.w.ybf) + (size_t)slot0 * a.H + col * NC, a.H, wv, lane);
}

// gate/up: work item = 128 slots x gu_rows() rows of I (gate and up); wave w
// takes NSL/2 row groups of 16 (gate and up slabs) and every token row.
// Persistent: one workgroup per CU walks its items (ItemSeq); the tile entry
// of item i + 2 and the pair of this lane's token row in item i + 1 are
// requested while item i starts, so the next item's operand addresses are
// known by the time its loads are issued (two stages before this item ends).
template <int FMT, int NSL>
__global__ __launch_bounds__(64 * GEMM_WAVES, 1) void k_gemm_gateup(GemmArgs a) {
  __shared__ __attribute__((aligned(16))) _Float16 As[2][ASTAGE];
  __shared__ __attribute__((aligned(16))) char stg[BM * 2 * gu_rows<NSL>()];
  const ItemSeq seq(tile_count(a), a.I / gu_rows<NSL>());
  if (!seq.valid(0)) return;
  const int lane = threadIdx.x & 63, wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int r = 16 * wv + (lane >> 2);                 // this lane's token row of a tile
  const int nsbH = a.H / SB_WEIGHTS;
  // slot of this lane's row (rows past the tile's end repeat its last row);
  // its token (routed slots), read for every slot at an in-bounds index
  auto row_slot = [&](int4 tl) { return tl.y + min(r, tl.z - 1); };
  auto slot_pair = [&](int slot) { return a.w.slot_tok[min(slot, a.P - 1)]; };
  const rsrc_t rx = make_rsrc(a.x16, (uint32_t)((size_t)a.T * a.H * 2));
  auto make_src = [&](int4 tl, int pair, int col) __attribute__((always_inline)) {
    const int slot = row_slot(tl);
    const int tok = slot < a.P ? pair : slot - a.P;
    const int g0 = (col * GEMM_WAVES + wv) * (NSL / 2);
    ItemSrc<NSL> is;
    is.ra = rx;
    is.va = (uint32_t)tok * (uint32_t)(2 * a.H) + 16 * (lane & 3);
    is.rw = make_rsrc(a.packed + (size_t)tl.x * a.stride, (uint32_t)a.stride);
#pragma unroll
    for (int n = 0; n < NSL / 2; ++n) {
      is.slab[n] = (uint32_t)slab_off(FMT, nsbH, g0 + n, 0);
      is.slab[NSL / 2 + n] = (uint32_t)(up_off(FMT, a.H, a.I) + slab_off(FMT, nsbH, g0 + n, 0));
    }
    return is;
  };
  int4 tl0 = tile_entry(a, seq.tile(0));
  int4 tl1 = tile_entry(a, seq.tile(1));
  ItemSrc<NSL> cur = make_src(tl0, slot_pair(row_slot(tl0)), seq.col(0));
  AStage ar[4];
  PairCodes<FMT> bc[2][NSL];
  gemm_prologue<FMT>(cur, As, wv, lane, ar, bc);
  // one loop per row class (the segment is sorted by class): each loop body
  // has a single MC, which keeps the register allocation of each tight
  int i = 0;
#define STRATA_GU_CLASS(MCV, CLS)                                                              \
  for (; seq.valid(i) && row_class(tl0.z) == CLS; ++i) {                                       \
    const int pair1 = slot_pair(row_slot(tl1));                                                \
    const int4 tl2 = tile_entry(a, seq.tile(i + 2));                                           \
    const int c1 = seq.col(i + 1);                                                             \
    auto next = [&]() __attribute__((always_inline)) { return make_src(tl1, pair1, c1); };     \
    gateup_item<FMT, MCV>(a, cur, next, tl0.y, tl0.z, seq.col(i), As, stg, wv, lane, ar, bc);  \
    cur = next();                                                                              \
    tl0 = tl1;                                                                                 \
    tl1 = tl2;                                                                                 \
  }
  STRATA_GU_CLASS(8, 0)
  STRATA_GU_CLASS(6, 1)
  STRATA_GU_CLASS(4, 2)
  STRATA_GU_CLASS(2, 3)
#undef STRATA_GU_CLASS
}

// down: work item = 128 slots x dn_cols() rows of H; wave w takes NSL row
// groups of 16.  Persistent as the gate/up GEMM; its A rows are the slots
// themselves, so only the tile entries are looked up ahead.
template <int FMT, int NSL>
__global__ __launch_bounds__(64 * GEMM_WAVES, 1) void k_gemm_down(GemmArgs a) {
  __shared__ __attribute__((aligned(16))) _Float16 As[2][ASTAGE];
  __shared__ __attribute__((aligned(16))) char stg[BM * 2 * dn_cols<NSL>()];
  const ItemSeq seq(tile_count(a), (a.H + dn_cols<NSL>() - 1) / dn_cols<NSL>());
  if (!seq.valid(0)) return;
  const int lane = threadIdx.x & 63, wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int r = 16 * wv + (lane >> 2);
  const int nsbI = a.I / SB_WEIGHTS;
  // this wave's slabs: H rows 16 g0 .. 16 (g0 + NSL) - 1; waves past H (in
  // the last column tile; whole waves, H being a multiple of 16 NSL) read
  // the first slabs instead and store nothing
  auto wave_g0 = [&](int col) { return (col * GEMM_WAVES + wv) * NSL; };
  auto make_src = [&](int4 tl, int col) __attribute__((always_inline)) {
    const int g0w = wave_g0(col);
    const int g0 = g0w < a.H / GROUP_ROWS ? g0w : 0;
    ItemSrc<NSL> is;
    is.ra = make_rsrc(reinterpret_cast<const char*>(a.w.act) + (size_t)tl.y * a.I * 2, (uint32_t)(BM * a.I * 2));
    is.va = (uint32_t)min(r, tl.z - 1) * (uint32_t)(2 * a.I) + 16 * (lane & 3);
    is.rw = make_rsrc(a.packed + (size_t)tl.x * a.stride, (uint32_t)a.stride);
    const uint32_t dn = (uint32_t)down_off(FMT, a.H, a.I);
#pragma unroll
    for (int n = 0; n < NSL; ++n) is.slab[n] = dn + (uint32_t)slab_off(FMT, nsbI, g0 + n, 0);
    return is;
  };
  int4 tl0 = tile_entry(a, seq.tile(0));
  int4 tl1 = tile_entry(a, seq.tile(1));
  ItemSrc<NSL> cur = make_src(tl0, seq.col(0));
  AStage ar[4];
  PairCodes<FMT> bc[2][NSL];
  gemm_prologue<FMT>(cur, As, wv, lane, ar, bc);
  int i = 0;
#define STRATA_DN_CLASS(MCV, CLS)                                                              \
  for (; seq.valid(i) && row_class(tl0.z) == CLS; ++i) {                                       \
    const int4 tl2 = tile_entry(a, seq.tile(i + 2));                                           \
    const int c1 = seq.col(i + 1);                                                             \
    auto next = [&]() __attribute__((always_inline)) { return make_src(tl1, c1); };            \
    down_item<FMT, MCV>(a, cur, next, tl0.y, tl0.z, seq.col(i), As, stg, wv, lane, ar, bc);   \
    cur = next();                                                                              \
    tl0 = tl1;                                                                                 \
    tl1 = tl2;                                                                                 \
  }
  STRATA_DN_CLASS(8, 0)
  STRATA_DN_CLASS(6, 1)
  STRATA_DN_CLASS(4, 2)
  STRATA_DN_CLASS(2, 3)
#undef STRATA_DN_CLASS
}

// ------------------------------------------------------------------ router GEMM
// Router logits x Wr^T on the 16x16x32 bf16 MFMA with fp32 accumulation,
// fp32-accurate: Wr is held as bf16 high parts and bf16 remainders (together
// Wr to about 2^-16 relative).  bf16 tokens are exact in bf16 (two products
// per weight); fp32 tokens are split the same way (three products: high x
// high, high x low, low x high).
//
// Work item: 128 tokens x 256 experts over a K range; the K range is split
// into partial planes when the item grid is small (the top-k kernel sums the
// planes in plane order, then adds the bias).  8 waves: wave w takes experts
// [32 w, 32 w + 32) of the item and all 128 tokens, computed transposed
// (experts as the A operand), so a lane's 4 results are consecutive experts
// of one token (16-byte stores).
//  - Router weights are laid out at create time in MFMA operand order
//    (1 KiB fragments of 16 experts x 32 of K, lane-major; see
//    k_router_split), so a wave loads its operands straight into registers,
//    one whole fragment per instruction, a stage (64 of K) ahead.  No wave
//    shares them, so they never pass through LDS.
//  - Token rows are staged in LDS fragment-major with coalesced row loads and
//    XOR-swizzled slots (as the expert GEMMs' token rows), two stages ahead in
//    registers; all 8 waves read them.
// Items are XCD-contiguous with token tiles fastest, so each XCD works on one
// (expert tile, K range) slice of the router weights at a time, which its L2
// holds.  The items of the first expert tile also write the tokens as fp16
// for the expert GEMMs (each element once).
constexpr int RT_E = 256;          // experts per work item
constexpr int RT_WAVES = 8;

struct RouterArgs {
  const void* x;          // [T][H] bf16 or fp32
  int T, H, E, S;
  int kper;               // K range of one split, a multiple of 64
  size_t plane;           // elements between partial planes
  const uint16_t* whi;    // Wr high parts, operand order
  const uint16_t* wlo;    // Wr remainders, operand order
  float* part;            // [S][T][E]
  uint16_t* x16;          // [T][H] the tokens as fp16
  uint32_t* tmax;         // [S][T] each token's largest |x| (float bits) over the split's K range
  int* meta;              // meta[2] (the call's scaled-token mark) is cleared here
};

// fp32 pair -> bf16 pair (RNE) in *hi and the bf16 of the remainders in *lo
__device__ inline void split_bf16x2(float a, float b, uint32_t* hi, uint32_t* lo) {
  const uint32_t h = cvt_bf16x2(a, b);
  *hi = h;
  *lo = cvt_bf16x2(a - __uint_as_float(h << 16), b - __uint_as_float(h & 0xffff0000u));
}

__device__ inline bf16x8 rt_frag(const uint16_t* stage, int f, int lane) {
  return __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4_t*>(stage + f * AFRAG + 8 * a_slot(lane)));
}

// One stage (two 32-wide K blocks) of a router work item for one wave:
// token subtiles in pairs, their fragments read from LDS a pair ahead; for a
// pair, the products of the weight high parts, then of the remainders (then
// of the token low parts): the same accumulator comes back every 4th MFMA,
// never back to back.
template <bool XF32>
__device__ inline void router_stage(const uint16_t* buf, const u32x4_t (&b)[2][2][2], int lane,
                                    f32x4 (&acc)[8][2]) {
  constexpr int NP = XF32 ? 2 : 1;                     // token parts
  constexpr int NMF = 4 * (XF32 ? 3 : 2);              // MFMAs per subtile pair
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    bf16x8 af[2][2][NP];                               // [buffer][subtile of the pair][part]
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int p = 0; p < NP; ++p) af[0][i][p] = rt_frag(buf, 16 * p + 2 * i + q, lane);
#pragma unroll
    for (int mp = 0; mp < 4; ++mp) {
      const int cb = mp & 1;
      if (mp < 3) {
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
          for (int p = 0; p < NP; ++p) af[cb ^ 1][i][p] = rt_frag(buf, 16 * p + 2 * (2 * mp + 2 + i) + q, lane);
      }
#pragma unroll
      for (int pass = 0; pass < (XF32 ? 3 : 2); ++pass)
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
          for (int n = 0; n < 2; ++n) {
            // pass 0: W high x token high, 1: W low x token high, 2: W high x token low
            const bf16x8 w = __builtin_bit_cast(bf16x8, b[q][n][pass == 1 ? 1 : 0]);
            const bf16x8 x = af[cb][i][pass == 2 ? NP - 1 : 0];
            acc[2 * mp + i][n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(w, x, acc[2 * mp + i][n], 0, 0, 0);
          }
    }
    // reads a pair ahead of the MFMAs that use them
    __builtin_amdgcn_sched_group_barrier(0x100, 2 * NP, 0);
#pragma unroll
    for (int mp = 0; mp < 4; ++mp) {
      if (mp < 3) __builtin_amdgcn_sched_group_barrier(0x100, 2 * NP, 0);
      __builtin_amdgcn_sched_group_barrier(0x008, NMF, 0);
    }
  }
}

template <bool XF32>
__global__ __launch_bounds__(64 * RT_WAVES, 1) void k_router(RouterArgs a) {
  constexpr int NA = XF32 ? 2 : 1;                    // token parts in LDS: high (and low)
  constexpr int NX = XF32 ? 4 : 2;                    // 16-byte token loads per lane and stage
  __shared__ __attribute__((aligned(16))) uint16_t Ls[2][NA * 16 * AFRAG];
  const int lane = threadIdx.x & 63, wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int ne = (a.E + RT_E - 1) / RT_E, nt = (a.T + BM - 1) / BM, total = ne * nt * a.S;
  const int per = (total + 7) >> 3, idx = blockIdx.x >> 3, w = (blockIdx.x & 7) * per + idx;
  if (idx >= per || w >= total) return;
  if (w == 0 && threadIdx.x == 0) a.meta[2] = 0;        // (the top-k kernel sets it)
  const int ty = w % nt, ex = (w / nt) % ne, kz = w / (nt * ne);
  const int t0 = ty * BM, e0 = ex * RT_E;
  const int kb0 = kz * a.kper, ke = min(a.H, kb0 + a.kper), ns = (ke - kb0) / XBK;
  // The XCD's workgroups share this item's router-weight slice; each starts
  // its K loop at its own stage (wrapping around), so a stage's weights are
  // fetched once by the first workgroup to reach them and found in the L2 by
  // the others, instead of all of them waiting on the same lines at once.
  // (Each workgroup's sum order is fixed, so results are run-to-run exact.)
  const int rot = (int)((long long)idx * ns / per);
  auto rs = [&](int st) { const int r = st + rot; return r >= ns ? r - ns : r; };
  // token loads of this lane: row l/4 of subtile w, 8 elements at column
  // 8 (l % 4) of each 32-wide block (operand lane l / 4 + 16 (l % 4))
  const int r4 = lane >> 2, c4 = 8 * (lane & 3);
  const int trow = min(t0 + 16 * wv + r4, a.T - 1);
  const size_t xoff = (size_t)trow * a.H + c4;
  const int slot = 8 * a_slot(r4 + 16 * (lane & 3));
  // router operands of this wave: expert groups of 16 (clamped to the last)
  const int ng = (a.E + 15) / 16, nkb = a.H / 32;
  const uint16_t* bsrc[2][2];
#pragma unroll
  for (int n = 0; n < 2; ++n) {
    const size_t g = (size_t)min(e0 / 16 + 2 * wv + n, ng - 1);
    bsrc[n][0] = a.whi + g * nkb * AFRAG + 8 * lane;
    bsrc[n][1] = a.wlo + g * nkb * AFRAG + 8 * lane;
  }
  struct BSt { u32x4_t v[2][2][2]; };                 // [block][group][part]
  auto bload = [&](int s, BSt& b) __attribute__((always_inline)) {
    const int kb = kb0 / 32 + 2 * s;
#pragma unroll
    for (int q = 0; q < 2; ++q)
#pragma unroll
      for (int n = 0; n < 2; ++n)
#pragma unroll
        for (int p = 0; p < 2; ++p) b.v[q][n][p] = *(gu32x4_t*)(bsrc[n][p] + (size_t)(kb + q) * AFRAG);
  };
  struct XSt { u32x4_t v[NX]; };
  auto xload = [&](int s, XSt& st) __attribute__((always_inline)) {
    const int k0 = kb0 + s * XBK;
    if constexpr (XF32) {
      const float* p = reinterpret_cast<const float*>(a.x) + xoff + k0;
#pragma unroll
      for (int i = 0; i < 4; ++i)
        st.v[i] = *(gu32x4_t*)(p + 32 * (i >> 1) + 4 * (i & 1));
    } else {
      const uint16_t* p = reinterpret_cast<const uint16_t*>(a.x) + xoff + k0;
      st.v[0] = *(gu32x4_t*)(p);
      st.v[1] = *(gu32x4_t*)(p + 32);
    }
  };
  // this lane's 8 token values of block q as bf16 (high part) and, for fp32
  // tokens, the low parts
  auto xparts = [&](const XSt& st, int q, u32x4_t& hi, u32x4_t& lo) __attribute__((always_inline)) {
    if constexpr (XF32) {
      const u32x4_t f0 = st.v[2 * q], f1 = st.v[2 * q + 1];
      uint32_t h[4], l[4];
      split_bf16x2(__uint_as_float(f0[0]), __uint_as_float(f0[1]), &h[0], &l[0]);
      split_bf16x2(__uint_as_float(f0[2]), __uint_as_float(f0[3]), &h[1], &l[1]);
      split_bf16x2(__uint_as_float(f1[0]), __uint_as_float(f1[1]), &h[2], &l[2]);
      split_bf16x2(__uint_as_float(f1[2]), __uint_as_float(f1[3]), &h[3], &l[3]);
      hi = u32x4_t{h[0], h[1], h[2], h[3]};
      lo = u32x4_t{l[0], l[1], l[2], l[3]};
    } else {
      hi = st.v[q];
    }
  };
  auto xstore = [&](const XSt& st, uint16_t* buf) __attribute__((always_inline)) {
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      u32x4_t hi, lo;
      xparts(st, q, hi, lo);
      *reinterpret_cast<u32x4_t*>(buf + (2 * wv + q) * AFRAG + slot) = hi;
      if constexpr (XF32) *reinterpret_cast<u32x4_t*>(buf + (16 + 2 * wv + q) * AFRAG + slot) = lo;
    }
  };
  const bool write_x16 = ex == 0 && t0 + 16 * wv + r4 < a.T;
  uint32_t xm = 0;          // largest |x| (bits) of this lane's token values, for the operand scale
  auto put_x16 = [&](const XSt& st, int s) __attribute__((always_inline)) {
    if (write_x16) {
      uint16_t* d = a.x16 + xoff + kb0 + s * XBK;
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        u32x4_t h;
        if constexpr (XF32) {
          h = f32x8_to_f16(__builtin_bit_cast(f32x4_t, st.v[2 * q]), __builtin_bit_cast(f32x4_t, st.v[2 * q + 1]));
        } else {
          h = bf16x8_to_f16(st.v[q]);
        }
        *reinterpret_cast<u32x4_t*>(d + 32 * q) = h;
      }
#pragma unroll
      for (int i = 0; i < NX; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const uint32_t w = st.v[i][j];
          if constexpr (XF32) {
            xm = max(xm, w & 0x7fffffffu);
          } else {
            xm = max(xm, max((w & 0x7fffu) << 16, w & 0x7fff0000u));
          }
        }
    }
  };
  f32x4 acc[8][2];
#pragma unroll
  for (int m = 0; m < 8; ++m)
#pragma unroll
    for (int n = 0; n < 2; ++n) acc[m][n] = f32x4{0.f, 0.f, 0.f, 0.f};
  // router operands BD stages ahead (2 for bf16 tokens; the fp32-token
  // kernel has no registers to spare for the second)
  constexpr int BD = XF32 ? 1 : 2, RB = 2 * BD;
  XSt ar[4];
  BSt br[RB];
  bload(rs(0), br[0]);
  if constexpr (BD == 2) bload(rs(min(1, ns - 1)), br[1]);
  xload(rs(0), ar[0]);
  xload(rs(min(1, ns - 1)), ar[1]);
  xstore(ar[0], Ls[0]);
  put_x16(ar[0], rs(0));
  __syncthreads();
  for (int s4 = 0; s4 < ns; s4 += 4) {
#define STRATA_RSTAGE(ST)                                                                    \
    if (s4 + ST < ns) {                                                                      \
      const int s = s4 + ST;                                                                 \
      bload(rs(min(s + BD, ns - 1)), br[(ST + BD) & (RB - 1)]);                              \
      xload(rs(min(s + 2, ns - 1)), ar[(ST + 2) & 3]);                                       \
      __builtin_amdgcn_sched_barrier(0);                                                     \
      router_stage<XF32>(Ls[ST & 1], br[ST & (RB - 1)].v, lane, acc);                        \
      if (s + 1 < ns) {                                                                      \
        xstore(ar[(ST + 1) & 3], Ls[(ST + 1) & 1]);                                          \
        put_x16(ar[(ST + 1) & 3], rs(s + 1));                                                \
      }                                                                                      \
      __syncthreads();                                                                       \
    }
    STRATA_RSTAGE(0) STRATA_RSTAGE(1) STRATA_RSTAGE(2) STRATA_RSTAGE(3)
#undef STRATA_RSTAGE
  }
  // the token's largest magnitude over this K range: its 4 lanes (l / 4 = row)
  if (ex == 0) {
    xm = max(xm, (uint32_t)dpp_i<DPP_QUAD_XOR1>((int)xm));
    xm = max(xm, (uint32_t)dpp_i<DPP_QUAD_XOR2>((int)xm));
    const int t = t0 + 16 * wv + r4;
    if ((lane & 3) == 0 && t < a.T) a.tmax[(size_t)kz * a.T + t] = xm;
  }
  // D[e][t]: lane l holds experts 4 (l / 16) .. + 3 of group n for token 16 m + l % 16
  float* out = a.part + (size_t)kz * a.plane;
#pragma unroll
  for (int n = 0; n < 2; ++n) {
    const int e = e0 + 32 * wv + 16 * n + 4 * (lane >> 4);
#pragma unroll
    for (int m = 0; m < 8; ++m) {
      const int t = t0 + 16 * m + (lane & 15);
      if (t >= a.T) continue;
      if ((a.E & 3) == 0) {
        if (e < a.E) *reinterpret_cast<f32x4*>(out + (size_t)t * a.E + e) = acc[m][n];
      } else {
#pragma unroll
        for (int j = 0; j < 4; ++j)
          if (e + j < a.E) out[(size_t)t * a.E + e + j] = acc[m][n][j];
      }
    }
  }
}

// ------------------------------------------------------------------ one-launch routing
// For calls of at most 64 tokens (E <= 512, k <= 64) the whole routing can
// run in one launch.  Workgroup g computes the complete logits of experts
// 16 g .. 16 g + 15 for every token (the full K, so no partial planes): its
// 16 waves each take a range of 32-wide K blocks on the bf16 MFMA with the
// router's hi/lo split (as the router GEMM; an fp32 token is split too,
// three products), and their partial sums meet in LDS in wave order.  It
// also writes its slice of the fp16 token rows for the expert GEMMs.  Then
// it counts itself done on a counter kept in the layer's packed buffer; the
// last workgroup to finish (it sees every other one counted, after their
// stores) takes the top-k of every token, each expert's token mask (64-bit:
// the expert counts and every pair's rank among the earlier tokens), the
// offsets and tile list and the scatter, and resets the counter.
constexpr int FR_WAVES = 16;
constexpr int FR_MAXT = 64;
constexpr int FR_MAXE = 512;
constexpr int FR_MAXK = 64;

struct FusedRouteArgs {
  const void* x;            // [T][Ho] bf16 or fp32
  int T, H, Ho, E;
  const uint16_t* whi;      // router rows in operand order (k_router_split)
  const uint16_t* wlo;
  uint16_t* x16;            // [T][H] the tokens as fp16, zero past Ho
  int* done;                // completion counter, 0 between calls
  TopkArgs t;               // part = the logits (one plane), bias
};

// the routing of every token of the call, in one workgroup (see above)
__device__ inline void fused_route_tail(const TopkArgs& a) {
  __shared__ int s_sel[FR_MAXT * FR_MAXK];               // [T][k]
  __shared__ unsigned long long s_tm[FR_MAXE];           // tokens of each expert
  const int wv = threadIdx.x >> 6, nw = blockDim.x >> 6;
  const int T = a.T, k = a.k, E = a.E;
  for (int e = threadIdx.x; e < E; e += blockDim.x) s_tm[e] = 0ull;
  if (threadIdx.x == 0) a.w.meta[2] = 0;
  __syncthreads();
  for (int t = wv; t < T; t += nw) {
    token_topk(a, t, s_sel + t * k, a.w.topk_w + (size_t)t * k, nullptr);
    token_scale(a, t);
  }
  __syncthreads();
  for (int i = threadIdx.x; i < T * k; i += blockDim.x) {
    const int e = s_sel[i];
    a.w.topk_idx[i] = e;
    atomicOr(&s_tm[e], 1ull << (i / k));
  }
  __syncthreads();
  for (int i = threadIdx.x; i < T * k; i += blockDim.x)
    a.w.pair_rank[i] = __popcll(s_tm[s_sel[i]] & ((1ull << (i / k)) - 1ull));
  // every pair's rank is among all earlier tokens, so every chunk base is 0
  for (int e = threadIdx.x; e < E; e += blockDim.x) {
    a.w.counts[e] = __popcll(s_tm[e]);
    for (int c = 0; c < a.nchunks; ++c) a.w.chunk_base[(size_t)c * E + e] = 0;
  }
  __syncthreads();
  ScanArgs sa;
  sa.T = T; sa.E = E; sa.k = k; sa.n_shared = a.n_shared; sa.nchunks = a.nchunks; sa.w = a.w;
  scan_tiles(sa);
  __syncthreads();
  for (int p = threadIdx.x; p < T * k; p += blockDim.x) scatter_pair(a, p);
}

template <bool XF32>
__global__ __launch_bounds__(64 * FR_WAVES, 1) void k_route_fused(FusedRouteArgs a) {
  constexpr int INF = XF32 ? 2 : 4;                      // K blocks of loads in flight per wave
  constexpr int NX = XF32 ? 2 : 1;                       // 16-byte token loads per block and subtile
  constexpr uint32_t OOBV = 0x80000000u;                 // buffer offset past the tokens: reads 0
  __shared__ f32x4 red[FR_WAVES][4][64];
  __shared__ int s_last;
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int g = blockIdx.x, ng = gridDim.x;
  const int nkb = a.H / 32;
  const int kb0 = wv * nkb / FR_WAVES, kb1 = (wv + 1) * nkb / FR_WAVES;
  const int esz = XF32 ? 4 : 2;
  const rsrc_t rx = make_rsrc(a.x, (uint32_t)((size_t)a.T * a.Ho * esz));
  // lane l: token 16 m + l % 16 of subtile m, K 32 kb + 8 (l / 16) .. + 7
  uint32_t xrow[4];
#pragma unroll
  for (int m = 0; m < 4; ++m) {
    const int t = 16 * m + (lane & 15);
    xrow[m] = t < a.T ? (uint32_t)((size_t)t * a.Ho * esz) : OOBV;
  }
  const int kl = 8 * (lane >> 4);
  const size_t wbase = (size_t)g * nkb * AFRAG + 8 * lane;
  f32x4 acc[4];
#pragma unroll
  for (int m = 0; m < 4; ++m) acc[m] = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int kb = kb0; kb < kb1; kb += INF) {
    u32x4_t A[INF][2], X[INF][4][NX];
#pragma unroll
    for (int j = 0; j < INF; ++j) {
      const int kbj = min(kb + j, kb1 - 1);
      A[j][0] = *(gu32x4_t*)(a.whi + wbase + (size_t)kbj * AFRAG);
      A[j][1] = *(gu32x4_t*)(a.wlo + wbase + (size_t)kbj * AFRAG);
      const int kk = 32 * kbj + kl;
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        const uint32_t off = (kk < a.Ho && xrow[m] != OOBV) ? xrow[m] + (uint32_t)(kk * esz) : OOBV;
#pragma unroll
        for (int q = 0; q < NX; ++q) {
          const uint4 v = bload4(rx, off == OOBV ? OOBV : off + 16 * q, 0);
          X[j][m][q] = u32x4_t{v.x, v.y, v.z, v.w};
        }
      }
    }
#pragma unroll
    for (int j = 0; j < INF; ++j) {
      if (kb + j >= kb1) break;
      const bf16x8 wh = __builtin_bit_cast(bf16x8, A[j][0]), wl = __builtin_bit_cast(bf16x8, A[j][1]);
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        if constexpr (XF32) {
          const u32x4_t f0 = X[j][m][0], f1 = X[j][m][1];
          uint32_t h[4], l[4];
          split_bf16x2(__uint_as_float(f0[0]), __uint_as_float(f0[1]), &h[0], &l[0]);
          split_bf16x2(__uint_as_float(f0[2]), __uint_as_float(f0[3]), &h[1], &l[1]);
          split_bf16x2(__uint_as_float(f1[0]), __uint_as_float(f1[1]), &h[2], &l[2]);
          split_bf16x2(__uint_as_float(f1[2]), __uint_as_float(f1[3]), &h[3], &l[3]);
          const bf16x8 xh = __builtin_bit_cast(bf16x8, u32x4_t{h[0], h[1], h[2], h[3]});
          const bf16x8 xl = __builtin_bit_cast(bf16x8, u32x4_t{l[0], l[1], l[2], l[3]});
          acc[m] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wh, xh, acc[m], 0, 0, 0);
          acc[m] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wl, xh, acc[m], 0, 0, 0);
          acc[m] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wh, xl, acc[m], 0, 0, 0);
        } else {
          const bf16x8 xh = __builtin_bit_cast(bf16x8, X[j][m][0]);
          acc[m] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wh, xh, acc[m], 0, 0, 0);
          acc[m] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wl, xh, acc[m], 0, 0, 0);
        }
      }
    }
  }
#pragma unroll
  for (int m = 0; m < 4; ++m) red[wv][m][lane] = acc[m];
  // this workgroup's slice of the fp16 token rows [T][H] (zero past Ho)
  {
    const int n = a.T * a.H, chunk = (n + ng - 1) / ng;
    for (int i = g * chunk + (int)threadIdx.x; i < min(n, (g + 1) * chunk); i += blockDim.x) {
      const int t = i / a.H, h = i - t * a.H;
      const size_t src = (size_t)t * a.Ho + min(h, a.Ho - 1);
      float v = XF32 ? reinterpret_cast<const float*>(a.x)[src]
                     : bf16_to_f32(reinterpret_cast<const uint16_t*>(a.x)[src]);
      const _Float16 hv = (_Float16)(h < a.Ho ? v : 0.f);
      a.x16[i] = __builtin_bit_cast(uint16_t, hv);
    }
  }
  __syncthreads();
  // D[e][t] of subtile m: lane l holds experts 4 (l / 16) .. + 3 of the group
  // for token 16 m + l % 16; the waves' partial sums in wave order
  {
    const int m = threadIdx.x >> 8, l = (threadIdx.x >> 2) & 63, v = threadIdx.x & 3;
    float sum = 0.f;
#pragma unroll
    for (int w = 0; w < FR_WAVES; ++w) sum += red[w][m][l][v];
    const int t = 16 * m + (l & 15), e = 16 * g + 4 * (l >> 4) + v;
    if (t < a.T && e < a.E) a.t.w.logits[(size_t)t * a.E + e] = sum;   // (= a.t.part)
  }
  // count this workgroup done once all its stores are visible on the device;
  // the last one routes
  __threadfence();
  __syncthreads();
  if (threadIdx.x == 0) s_last = atomicAdd(a.done, 1) == ng - 1;
  __syncthreads();
  if (!s_last) return;
  __threadfence();                                       // (acquire: the other workgroups' logits)
  fused_route_tail(a.t);
  if (threadIdx.x == 0) *a.done = 0;                     // every other workgroup has counted
}

// The tokens widened to whole superblocks (zero columns past Ho) for the
// router GEMM, in their own type (2 or 4 bytes per element), when the
// layer's width is not a multiple of 256.
__global__ void k_pad_tokens(const void* __restrict__ x, void* __restrict__ xpad, int T, int Ho, int H, int esize) {
  const long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= (long long)T * H) return;
  const int t = (int)(i / H), h = (int)(i - (long long)t * H);
  if (esize == 4) {
    reinterpret_cast<float*>(xpad)[i] = h < Ho ? reinterpret_cast<const float*>(x)[(size_t)t * Ho + h] : 0.f;
  } else {
    reinterpret_cast<uint16_t*>(xpad)[i] = h < Ho ? reinterpret_cast<const uint16_t*>(x)[(size_t)t * Ho + h] : 0;
  }
}

struct CombineArgs {
  int T, H, k, P, n_shared;   // H: the per-pair rows' width (whole superblocks)
  int Ho;                      // the layer's hidden width (x, out)
  const void* x;
  int x_f32;
  uint32_t flags;
  float* out;
  Work w;
};

// out[t] = sum_j w[t][j] * y[slot(t, j)] (+ shared expert row) (+ x) (+ out),
// fixed j order.  One workgroup per token, one thread per 8 columns (a single
// pass over the row); the bf16 per-pair rows are read KB at a time, all KB
// loads in flight together (KB divides k where it can, so no padding rows are
// read; otherwise the last batch reads the last row again with weight 0).
template <int KB>
__global__ __launch_bounds__(512) void k_combine(CombineArgs a) {
  const int t = blockIdx.x;
  const int k = a.k, kp = (k + KB - 1) / KB * KB;
  extern __shared__ int s_cmb[];
  int* s_slot = s_cmb;                                   // [kp]
  float* s_w = reinterpret_cast<float*>(s_cmb + kp);     // [kp]
  // the expert rows of a scaled token carry 2^-2e: the weights undo it
  const float tsc = pow2i(2 * a.w.texp[t]);
  for (int j = threadIdx.x; j < kp; j += blockDim.x) {
    const int jj = min(j, k - 1);
    s_slot[j] = a.w.inv[(size_t)t * k + jj];
    s_w[j] = j < k ? a.w.topk_w[(size_t)t * k + jj] * tsc : 0.f;
  }
  __syncthreads();
  for (int h = threadIdx.x * 8; h < a.Ho; h += blockDim.x * 8) {
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    for (int j0 = 0; j0 < k; j0 += KB) {
      uint4 y[KB];
#pragma unroll
      for (int j = 0; j < KB; ++j)
        y[j] = *reinterpret_cast<const uint4*>(a.w.ybf + (size_t)s_slot[j0 + j] * a.H + h);
#pragma unroll
      for (int j = 0; j < KB; ++j) {
        const float wj = s_w[j0 + j];                          // 0 past k
        const uint32_t q[4] = {y[j].x, y[j].y, y[j].z, y[j].w};
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          acc[2 * c] = fmaf(wj, __uint_as_float(q[c] << 16), acc[2 * c]);
          acc[2 * c + 1] = fmaf(wj, __uint_as_float(q[c] & 0xffff0000u), acc[2 * c + 1]);
        }
      }
    }
    if (a.n_shared) {
      const uint4 ys = *reinterpret_cast<const uint4*>(a.w.ybf + (size_t)(a.P + t) * a.H + h);
      const uint32_t q[4] = {ys.x, ys.y, ys.z, ys.w};
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        acc[2 * c] = fmaf(tsc, __uint_as_float(q[c] << 16), acc[2 * c]);
        acc[2 * c + 1] = fmaf(tsc, __uint_as_float(q[c] & 0xffff0000u), acc[2 * c + 1]);
      }
    }
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      const int hh = h + 4 * half;
      float4 r = make_float4(acc[4 * half], acc[4 * half + 1], acc[4 * half + 2], acc[4 * half + 3]);
      const size_t o = (size_t)t * a.Ho + hh;
      if (a.flags & 2u) {
        if (a.x_f32) {
          const float4 xv = *reinterpret_cast<const float4*>(reinterpret_cast<const float*>(a.x) + o);
          r.x += xv.x; r.y += xv.y; r.z += xv.z; r.w += xv.w;
        } else {
          const uint2 b = *reinterpret_cast<const uint2*>(reinterpret_cast<const uint16_t*>(a.x) + o);
          r.x += __uint_as_float(b.x << 16); r.y += __uint_as_float(b.x & 0xffff0000u);
          r.z += __uint_as_float(b.y << 16); r.w += __uint_as_float(b.y & 0xffff0000u);
        }
      }
      if (a.flags & 1u) {
        const float4 ov = *reinterpret_cast<const float4*>(a.out + o);
        r.x += ov.x; r.y += ov.y; r.z += ov.z; r.w += ov.w;
      }
      *reinterpret_cast<float4*>(a.out + o) = r;
    }
  }
}

// loads per batch of the combine: k itself up to 8, else its largest divisor
// in 4..8, else 8 (with a padded last batch)
int combine_batch(int k) {
  if (k <= 8) return k;
  for (int d = 8; d >= 4; --d)
    if (k % d == 0) return d;
  return 8;
}

// Router split-K plan and the place of the fp16 token rows.  Both live in
// the per-pair output region, dead until the down GEMM: the partial planes
// first, then the token rows (which the gate/up GEMM reads).
size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// calls of up to this many tokens use the narrow expert-GEMM work items
constexpr int SKINNY_T = 64;

// compute units of the current device (cached per device)
int cu_count() {
  static int cache[64] = {};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) dev = 0;
  int* c = &cache[dev & 63];
  if (*c == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n < 8) n = 8;
    *c = n;
  }
  return *c;
}

// persistent GEMM grid: per_cu workgroups per CU (a multiple of 8, one
// group per XCD), fewer when there are fewer items
int persistent_grid(int max_items, int per_cu = 1) {
  return 8 * std::max(1, std::min(per_cu * cu_count() / 8, (max_items + 7) / 8));
}

struct RouterPlan {
  int S, kper;
  size_t plane;
  float* part;
  uint16_t* x16;
};

RouterPlan router_plan(const Layer& L, const Work& W, int T) {
  // split K until the grid has about one workgroup per CU (at most 8 splits,
  // 32 for calls of up to 64 tokens, whose one or two expert tiles would
  // otherwise stream the router through a handful of CUs: top-k reads every
  // plane; one plane past 512 experts, where top-k re-reads its plane)
  RouterPlan r;
  const int slots = cu_count();
  // (a selection past 64 per token runs the block top-k on one plane)
  const int tiles = ((L.E + RT_E - 1) / RT_E) * ((T + BM - 1) / BM);
  const int ksteps = L.H / XBK;
  const size_t x16_bytes = (size_t)T * L.H * 2;       // <= the region (slots >= T)
  r.plane = (size_t)T * L.E;
  int S = 1;
  if (L.E <= 512 && L.k <= 64) {
    S = std::min(std::min(T <= 64 ? 32 : 8, ksteps), std::max(1, (slots + tiles - 1) / tiles));
    while (S > 1 && align256((size_t)S * r.plane * 4) + x16_bytes > W.ybf_bytes) --S;
  }
  r.kper = ((ksteps + S - 1) / S) * XBK;
  r.S = (L.H + r.kper - 1) / r.kper;                   // no empty split
  r.part = r.S > 1 ? reinterpret_cast<float*>(W.ybf) : W.logits;
  r.x16 = reinterpret_cast<uint16_t*>(reinterpret_cast<char*>(W.ybf) +
                                      (r.S > 1 ? align256((size_t)r.S * r.plane * 4) : 0));
  return r;
}

// Whether a call routes in one launch (k_route_fused): asked for with
// STRATA_FUSED_ROUTE, refused with STRATA_SPLIT_ROUTE, else by default for
// calls of at most FUSED_ROUTE_DEFAULT_T tokens; only where its tail holds
// the call (T <= 64, E <= 512, k <= 64).
bool fused_route(const Layer& L, int T, uint32_t flags) {
  if (!fused_route_fits(L.E, L.k, T) || (flags & STRATA_SPLIT_ROUTE_FLAG)) return false;
  return (flags & STRATA_FUSED_ROUTE_FLAG) || T <= FUSED_ROUTE_DEFAULT_T;
}

template <int FMT>
hipError_t launch_gemms_fmt(const Layer& L, const Work& W, const Call& c, hipStream_t s, Tracer* tr) {
  GemmArgs g;
  g.packed = L.packed; g.stride = L.expert_stride; g.H = L.H; g.I = L.I; g.E = L.E; g.k = L.k;
  g.T = c.T; g.P = c.T * L.k; g.w = W;
  g.x16 = fused_route(L, c.T, c.flags) ? reinterpret_cast<uint16_t*>(W.ybf) : router_plan(L, W, c.T).x16;
  const int max_tiles = W.max_tiles;
  // Skinny calls (up to 64 tokens: tiles of a few rows, one or two per
  // touched expert) are bound by streaming each expert's weights through one
  // workgroup; narrower work items (2 slabs per wave for gate/up, 1 for down)
  // spread those streams over 2 and 4 times as many CUs.
  auto gemms = [&](auto gu_nsl, auto dn_nsl) {
    constexpr int GN = decltype(gu_nsl)::value, DN = decltype(dn_nsl)::value;
    launch(tr, k_gemm_gateup<FMT, GN>, dim3(persistent_grid(max_tiles * (L.I / gu_rows<GN>()))),
           dim3(64 * GEMM_WAVES), 0, s, g);
    // (the one-slab down kernel fits two workgroups per CU: under 128 VGPRs,
    // 64 KiB of LDS)
    launch(tr, k_gemm_down<FMT, DN>,
           dim3(persistent_grid(max_tiles * ((L.H + dn_cols<DN>() - 1) / dn_cols<DN>()), DN == 1 ? 2 : 1)),
           dim3(64 * GEMM_WAVES), 0, s, g);
  };
  if (c.T <= SKINNY_T) gemms(std::integral_constant<int, 2>(), std::integral_constant<int, 1>());
  else gemms(std::integral_constant<int, nsl<FMT>()>(), std::integral_constant<int, nsl<FMT>()>());
  return hipGetLastError();
}

}  // namespace

hipError_t launch_prefill_route(const Layer& L, const Work& W, const Call& c, hipStream_t s, Tracer* tr) {
  if (fused_route(L, c.T, c.flags)) {
    FusedRouteArgs f;
    f.x = c.x; f.T = c.T; f.H = L.H; f.Ho = L.Ho; f.E = L.E;
    f.whi = L.router_hi; f.wlo = L.router_lo;
    f.x16 = reinterpret_cast<uint16_t*>(W.ybf);
    f.done = L.route_done;
    TopkArgs& t = f.t;
    t.T = c.T; t.E = L.E; t.k = L.k; t.ct = prefill_chunk_t(c.T); t.nchunks = prefill_chunks(c.T);
    t.n_shared = L.n_shared; t.presel = 0;
    t.x = c.x; t.x_f32 = c.x_f32; t.H = L.H; t.Ho = L.Ho; t.x16 = f.x16; t.tmax = nullptr;
    t.S = 1; t.plane = (size_t)c.T * L.E; t.part = W.logits; t.bias = L.router_b; t.w = W;
    const dim3 grid((L.E + 15) / 16), block(64 * FR_WAVES);
    if (c.x_f32) launch(tr, k_route_fused<true>, grid, block, 0, s, f);
    else launch(tr, k_route_fused<false>, grid, block, 0, s, f);
    return hipGetLastError();
  }
  const RouterPlan rp = router_plan(L, W, c.T);
  const int S = rp.S;
  const size_t plane = rp.plane;
  RouterArgs r;
  r.x = c.x; r.T = c.T; r.H = L.H; r.E = L.E; r.S = S;
  if (L.Ho != L.H) {
    const long long n = (long long)c.T * L.H;
    launch(tr, k_pad_tokens, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, c.x, W.xpad, c.T, L.Ho, L.H,
           c.x_f32 ? 4 : 2);
    r.x = W.xpad;
  }
  r.kper = rp.kper; r.plane = plane;
  r.whi = L.router_hi; r.wlo = L.router_lo;
  r.part = rp.part;
  r.x16 = rp.x16;
  r.tmax = W.tmax;
  r.meta = W.meta;
  const int items = ((L.E + RT_E - 1) / RT_E) * ((c.T + BM - 1) / BM) * S;
  const dim3 grid(8 * ((items + 7) / 8)), block(64 * RT_WAVES);
  if (c.x_f32) launch(tr, k_router<true>, grid, block, 0, s, r);
  else launch(tr, k_router<false>, grid, block, 0, s, r);
  TopkArgs t;
  t.T = c.T; t.E = L.E; t.k = L.k; t.ct = prefill_chunk_t(c.T); t.nchunks = prefill_chunks(c.T); t.w = W;
  t.S = S; t.plane = plane; t.part = r.part; t.bias = L.router_b; t.n_shared = L.n_shared;
  t.presel = L.k > 64;
  t.x = c.x; t.x_f32 = c.x_f32; t.H = L.H; t.Ho = L.Ho; t.x16 = rp.x16; t.tmax = W.tmax;
  if (t.presel) {
    const hipError_t e = launch_topk_block(r.part, L.E, L.router_b, c.T, L.E, L.k, W.topk_idx, W.topk_w, s, tr);
    if (e != hipSuccess) return e;
  }
  const size_t lds = ((t.presel ? 0 : (size_t)t.ct * L.k) + L.E) * 4;
  launch(tr, k_topk_chunks, dim3(t.nchunks), dim3(64 * TOPK_CHUNK_WAVES), lds, s, t);
  if (t.nchunks == 1) return hipGetLastError();   // the one chunk did the scan and the scatter
  ScanArgs sa;
  sa.T = c.T; sa.E = L.E; sa.k = L.k; sa.n_shared = L.n_shared; sa.nchunks = t.nchunks; sa.w = W;
  launch(tr, k_colscan, dim3((L.E + 63) / 64), dim3(64 * COLSCAN_GROUPS), 0, s, sa);
  launch(tr, k_scan, dim3(1), dim3(1024), 0, s, sa);
  const int P = c.T * L.k;
  launch(tr, k_scatter, dim3((P + 255) / 256), dim3(256), 0, s, t);
  return hipGetLastError();
}

hipError_t launch_prefill_experts(const Layer& L, const Work& W, const Call& c, hipStream_t s, Tracer* tr) {
  hipError_t err;
  switch (L.fmt) {
    case 2: err = launch_gemms_fmt<2>(L, W, c, s, tr); break;
    case 3: err = launch_gemms_fmt<3>(L, W, c, s, tr); break;
    case 4: err = launch_gemms_fmt<4>(L, W, c, s, tr); break;
    default: err = launch_gemms_fmt<FMT_MXFP4>(L, W, c, s, tr); break;
  }
  if (err != hipSuccess) return err;
  CombineArgs cb;
  cb.T = c.T; cb.H = L.H; cb.Ho = L.Ho; cb.k = L.k; cb.P = c.T * L.k; cb.n_shared = L.n_shared;
  cb.x = c.x; cb.x_f32 = c.x_f32; cb.flags = c.flags; cb.out = c.out; cb.w = W;
  const int kb = combine_batch(L.k);
  const size_t lds = (size_t)((L.k + kb - 1) / kb * kb) * 8;
  const dim3 cgrid(c.T), cblock(std::min(512, ((L.Ho / 8 + 63) / 64) * 64));
  switch (kb) {
#define STRATA_COMBINE(KB) \
    case KB: launch(tr, k_combine<KB>, cgrid, cblock, lds, s, cb); break;
    STRATA_COMBINE(1) STRATA_COMBINE(2) STRATA_COMBINE(3) STRATA_COMBINE(4)
    STRATA_COMBINE(5) STRATA_COMBINE(6) STRATA_COMBINE(7) STRATA_COMBINE(8)
#undef STRATA_COMBINE
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace strata
