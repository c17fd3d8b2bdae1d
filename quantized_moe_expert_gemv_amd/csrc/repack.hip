// Create-time repack of canonical expert records into the packed layout,
// and the bf16 hi/lo split of the router rows used by the prefill router.
//
// The repack only moves bytes (and, for Q3, reorders the bits of each
// block's codes into a 2-bit plane and a 1-bit plane); the byte count of an
// expert is unchanged.  It follows the one-time re-layout of the expert set
// into a compute-friendly copy that the pages describe for the CPU path
// (devotd.net "Strata memory tiers", section 小模型包不等于合适的模型: a
// one-time ~40 GB copy written for AVX-512 Q2_0) and the contiguous
// per-expert record (lcz.me/topic/2153, section 三 item 4, the per-expert
// blob).
#include "common.hpp"
#include "kernels.hpp"

namespace strata {

namespace {

__device__ inline uint32_t ld_u32_unaligned(const uint8_t* p) {
  return (uint32_t)p[0] | ((uint32_t)p[1] << 8) | ((uint32_t)p[2] << 16) | ((uint32_t)p[3] << 24);
}

__global__ void k_repack(const uint8_t* __restrict__ canon, uint8_t* __restrict__ packed,
                         int fmt, int H, int I, size_t stride, long long n_blocks_total,
                         int first_expert) {
  const long long gid = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  if (gid >= n_blocks_total) return;
  const int cb = fmt_code_bytes(fmt);
  const int bq = cb + 2;
  const int ncv = fmt_ncv(fmt), nv = ncv + 1;
  const long long nGU = (long long)I * (H / BLOCK_W);
  const long long nD = (long long)H * (I / BLOCK_W);
  const long long per = 2 * nGU + nD;
  const int x = (int)(gid / per);
  const long long local = gid % per;

  const uint8_t* src = canon + (size_t)x * stride + (size_t)local * bq;
  uint8_t* ebase = packed + (size_t)(first_expert + x) * stride;

  int row, blk;
  uint8_t* base;
  if (local < 2 * nGU) {
    const int m = (int)(local / nGU);
    const long long l = local % nGU;
    row = (int)(l / (H / BLOCK_W));
    blk = (int)(l % (H / BLOCK_W));
    base = ebase + gu_off(nv, H / SB_WEIGHTS, row / ROWS_PER_TILE, blk / 8, m, 0);
  } else {
    const long long l = local - 2 * nGU;
    row = (int)(l / (I / BLOCK_W));
    blk = (int)(l % (I / BLOCK_W));
    base = ebase + gu_bytes(fmt, H, I) + dn_off(nv, I / SB_WEIGHTS, row / ROWS_PER_TILE, blk / 8, 0);
  }
  base += (row % ROWS_PER_TILE) * 16;
  const int bb = blk % 8;

  if (fmt == 2) {
    uint8_t* dst = base + (bb / 2) * 1024 + (bb % 2) * 8;
    for (int i = 0; i < 8; ++i) dst[i] = src[i];
  } else if (fmt == 4) {
    uint8_t* dst = base + bb * 1024;
    for (int i = 0; i < 16; ++i) dst[i] = src[i];
  } else {
    // 32 three-bit codes, code j at bits [3j, 3j+3) of a 96-bit little-endian string
    uint32_t w[4] = {ld_u32_unaligned(src), ld_u32_unaligned(src + 4), ld_u32_unaligned(src + 8), 0u};
    uint64_t lo = 0;
    uint32_t hi = 0;
    for (int j = 0; j < 32; ++j) {
      const int p = 3 * j, wd = p >> 5, off = p & 31;
      uint32_t v = w[wd] >> off;
      if (off > 29) v |= w[wd + 1] << (32 - off);
      v &= 7u;
      lo |= (uint64_t)(v & 3u) << (2 * j);
      const int ww = j >> 4, i = (j & 15) >> 2, s = j & 3;
      hi |= ((v >> 2) & 1u) << (8 * i + 4 * ww + s);
    }
    uint8_t* dlo = base + (bb / 2) * 1024 + (bb % 2) * 8;
    for (int i = 0; i < 8; ++i) dlo[i] = (uint8_t)(lo >> (8 * i));
    uint8_t* dhi = base + (4 + bb / 4) * 1024 + (bb % 4) * 4;
    for (int i = 0; i < 4; ++i) dhi[i] = (uint8_t)(hi >> (8 * i));
  }
  uint8_t* dsc = base + ncv * 1024 + bb * 2;
  dsc[0] = src[cb];
  dsc[1] = src[cb + 1];
}

__global__ void k_router_split(const float* __restrict__ w, uint16_t* __restrict__ hi,
                               uint16_t* __restrict__ lo, long long n) {
  const long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n) return;
  const float v = w[i];
  const uint16_t h = f32_to_bf16_rne(v);
  hi[i] = h;
  lo[i] = f32_to_bf16_rne(v - bf16_to_f32(h));
}

}  // namespace

hipError_t launch_repack(const Layer& L, const uint8_t* canon, int n_experts_in, int first_expert,
                         hipStream_t s) {
  const long long per = 2LL * L.I * (L.H / BLOCK_W) + (long long)L.H * (L.I / BLOCK_W);
  const long long n = per * n_experts_in;
  if (n == 0) return hipSuccess;
  const int bs = 256;
  const long long grid = (n + bs - 1) / bs;
  hipLaunchKernelGGL(k_repack, dim3((unsigned)grid), dim3(bs), 0, s, canon,
                     const_cast<uint8_t*>(L.packed), L.fmt, L.H, L.I, L.expert_stride, n,
                     first_expert);
  return hipGetLastError();
}

hipError_t launch_router_split(const Layer& L, hipStream_t s) {
  const long long n = (long long)L.E * L.H;
  const int bs = 256;
  hipLaunchKernelGGL(k_router_split, dim3((unsigned)((n + bs - 1) / bs)), dim3(bs), 0, s,
                     L.router_w, const_cast<uint16_t*>(L.router_hi),
                     const_cast<uint16_t*>(L.router_lo), n);
  return hipGetLastError();
}

}  // namespace strata
