// Create-time repack of canonical expert records into the packed slab
// layout, and the bf16 hi/lo split of the router rows used by the prefill
// router.
//
// The repack only moves bits: every code and every scale of the canonical
// record lands in exactly one place, so an expert keeps its byte count (but
// for MXFP4, whose one-byte scales take 16-bit slots, and for widths that are
// not whole 256-weight superblocks, whose padding is written as zero codes
// with zero scales).  It follows the one-time re-layout of the expert set into a
// compute-friendly copy that the pages describe for the CPU path
// (devotd.net "Strata memory tiers", section 小模型包不等于合适的模型: a
// one-time ~40 GB copy written for AVX-512 Q2_0) and the contiguous
// per-expert record (lcz.me/topic/2153, section 三 item 4, the per-expert
// blob).
#include "common.hpp"
#include "kernels.hpp"

namespace strata {

namespace {

__constant__ int POS2[8] = {0, 4, 2, 6, 8, 12, 10, 14};   // Q2/Q3 low-plane bit of offset e
__constant__ int NIB4[8] = {0, 2, 4, 6, 1, 3, 5, 7};      // Q4 nibble of offset e

// code j (0..31) of a canonical block: bits [b*j, b*j + b) of the code bytes
// read as one little-endian bit string
__device__ inline uint32_t canon_code(const uint8_t* blk, int bits, int j) {
  const int p = bits * j;
  uint32_t v = blk[p >> 3] >> (p & 7);
  if ((p & 7) + bits > 8) v |= (uint32_t)blk[(p >> 3) + 1] << (8 - (p & 7));
  return v & ((1u << bits) - 1u);
}

// One thread per (expert, matrix, row, superblock) of the packed geometry
// (H, I: whole superblocks): 8 canonical blocks in, the row's share of one
// slab out (4 lanes' code bits and one scale row).  Ho, Io are the canonical
// widths; rows and blocks past them are written as zero codes with a zero
// scale.
__global__ void k_repack(const uint8_t* __restrict__ canon, uint8_t* __restrict__ packed, int fmt,
                         int H, int I, int Ho, int Io, size_t canon_stride, size_t stride, long long n_items,
                         int first_expert) {
  const long long gid = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  if (gid >= n_items) return;
  const int bq = canon_block_bytes(fmt);
  const long long gu_items = (long long)I * (H / SB_WEIGHTS);     // per gate or up matrix
  const long long dn_items = (long long)H * (I / SB_WEIGHTS);
  const long long per = 2 * gu_items + dn_items;
  const int x = (int)(gid / per);
  long long local = gid % per;

  int m, K, Ko, Ro;
  if (local < 2 * gu_items) {
    m = (int)(local / gu_items);
    local %= gu_items;
    K = H; Ko = Ho; Ro = Io;
  } else {
    m = 2;
    local -= 2 * gu_items;
    K = I; Ko = Io; Ro = Ho;
  }
  const int nsb = K / SB_WEIGHTS;
  const int row = (int)(local / nsb), sb = (int)(local % nsb);
  // canonical: gate blocks [Io][Ho/32], up [Io][Ho/32], down [Ho][Io/32]
  const size_t mat_canon = (m == 0) ? 0 : (m == 1 ? (size_t)Io * (Ho / BLOCK_W) * bq
                                                   : (size_t)2 * Io * (Ho / BLOCK_W) * bq);
  const int rowc = min(row, Ro - 1);                             // (not read when row >= Ro)
  const uint8_t* src = canon + (size_t)x * canon_stride + mat_canon + (size_t)rowc * (Ko / BLOCK_W) * bq;
  // canonical block bb of this superblock, or nullptr past the canonical widths
  auto block = [&](int bb) -> const uint8_t* {
    const int kb = sb * 8 + bb;
    return (row < Ro && kb < Ko / BLOCK_W) ? src + (size_t)kb * bq : nullptr;
  };
  auto code = [&](int bb, int bits, int j) -> uint32_t {
    const uint8_t* b = block(bb);
    return b ? canon_code(b, bits, j) : 0u;
  };
  const size_t mat_packed = (m == 0) ? 0 : (m == 1 ? up_off(fmt, H, I) : down_off(fmt, H, I));
  uint8_t* slab = packed + (size_t)(first_expert + x) * stride + mat_packed +
                  slab_off(fmt, nsb, row / GROUP_ROWS, sb);
  const int r = row % GROUP_ROWS;

  for (int q = 0; q < 4; ++q) {                 // K-slice -> lane q*16 + r
    const int lane = q * 16 + r;
    if (fmt == 4 || fmt == FMT_MXFP4) {
      // Q4: byte j = elements j and j + 4 (low nibble first), so that the
      // masked bytes convert as E4M3 in K order; MXFP4: in K order (byte j =
      // elements 2j, 2j + 1, low nibble first), the order of the FP4 -> fp16
      // conversion
      uint32_t w[8];
      for (int bb = 0; bb < 8; ++bb) {
        uint32_t d = 0;
        for (int e = 0; e < 8; ++e)
          d |= code(bb, 4, 8 * q + e) << (4 * (fmt == 4 ? NIB4[e] : e));
        w[bb] = d;
      }
      uint32_t* v0 = reinterpret_cast<uint32_t*>(slab + lane * 16);
      uint32_t* v1 = reinterpret_cast<uint32_t*>(slab + 1024 + lane * 16);
      for (int i = 0; i < 4; ++i) { v0[i] = w[i]; v1[i] = w[4 + i]; }
    } else {
      uint32_t lo[4] = {0, 0, 0, 0}, hi[2] = {0, 0};
      for (int bb = 0; bb < 8; ++bb) {
        for (int e = 0; e < 8; ++e) {
          const uint32_t c = code(bb, fmt, 8 * q + e);
          lo[bb >> 1] |= (c & 3u) << (16 * (bb & 1) + POS2[e]);
          if (fmt == 3) hi[bb >> 2] |= ((c >> 2) & 1u) << (4 * e + (bb & 3));
        }
      }
      uint32_t* v0 = reinterpret_cast<uint32_t*>(slab + lane * 16);
      for (int i = 0; i < 4; ++i) v0[i] = lo[i];
      if (fmt == 3) {
        uint32_t* vh = reinterpret_cast<uint32_t*>(slab + 1024 + lane * 8);
        vh[0] = hi[0];
        vh[1] = hi[1];
      }
    }
  }
  uint8_t* sc = slab + slab_code_bytes(fmt) + r * 16;
  for (int bb = 0; bb < 8; ++bb) {
    const uint8_t* b = block(bb);
    if (!b) {                                  // padding: zero scale
      sc[2 * bb] = 0;
      sc[2 * bb + 1] = 0;
    } else if (fmt == FMT_MXFP4) {             // the E8M0 byte, zero-extended
      sc[2 * bb] = b[bq - 1];
      sc[2 * bb + 1] = 0;
    } else {
      sc[2 * bb] = b[bq - 2];
      sc[2 * bb + 1] = b[bq - 1];
    }
  }
}

// Router split: Wr (fp32 [E][Ho]) -> bf16 high parts and bf16 remainders,
// each in MFMA operand order for the prefill router: fragment (g, kb) of 16
// experts (group g) x 32 of K (block kb) is 1 KiB at element
// (g * H / 32 + kb) * 512, and its lane l holds the 8 weights of expert
// 16 g + l % 16 at K = 32 kb + 8 (l / 16) + j in element 8 l + j.  Experts
// past E (padding of the last group) and K past Ho are zero.  One thread per
// element of the output.
__global__ void k_router_split(const float* __restrict__ w, uint16_t* __restrict__ hi,
                               uint16_t* __restrict__ lo, int E, int H, int Ho, long long n) {
  const long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n) return;
  const int j = (int)(i & 7), l = (int)((i >> 3) & 63);
  const long long f = i >> 9;
  const int nkb = H / 32, kb = (int)(f % nkb), g = (int)(f / nkb);
  const int e = 16 * g + (l & 15), k = 32 * kb + 8 * (l >> 4) + j;
  const float v = (e < E && k < Ho) ? w[(size_t)e * Ho + k] : 0.0f;
  const uint16_t h = f32_to_bf16_rne(v);
  hi[i] = h;
  lo[i] = f32_to_bf16_rne(v - bf16_to_f32(h));
}

// Scales the kernels cannot carry: every 16-bit weight operand (the prefill
// path's dequantised d (q - c) in fp16, and the products the decode path
// scales in fp32) must stay finite.  fp16 d: NaN or infinite, or above
// 2^15 (Q2), 2^14 (Q3), 2^12 (Q4, whose 8 d is an fp16 operand too);
// MXFP4: e = 255 (NaN) or e > 140 (2^13 and up).  One thread per
// canonical block; bad blocks are counted in *bad.
__global__ void k_check_scales(const uint8_t* __restrict__ canon, long long n_blocks, int fmt, int* bad) {
  const long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n_blocks) return;
  const int bq = canon_block_bytes(fmt);
  const uint8_t* b = canon + (size_t)i * bq;
  bool ok;
  if (fmt == FMT_MXFP4) {
    const int e = b[bq - 1];
    ok = e <= 140;
  } else {
    const uint32_t h = (uint32_t)b[bq - 2] | ((uint32_t)b[bq - 1] << 8);
    const uint32_t mag = h & 0x7fffu;
    const uint32_t lim = fmt == 4 ? 0x6C00u : fmt == 3 ? 0x7400u : 0x7800u;   // 2^12, 2^14, 2^15
    ok = mag <= lim;                             // (NaN and infinity encode above every limit)
  }
  if (!ok) atomicAdd(bad, 1);
}

}  // namespace

hipError_t launch_check_scales(const Layer& L, const uint8_t* canon, int n_records, int* bad, hipStream_t s) {
  const long long n = (long long)n_records * (canon_expert_bytes(L.fmt, L.Ho, L.Io) / canon_block_bytes(L.fmt));
  if (n == 0) return hipSuccess;
  const int bs = 256;
  hipLaunchKernelGGL(k_check_scales, dim3((unsigned)((n + bs - 1) / bs)), dim3(bs), 0, s, canon, n, L.fmt, bad);
  return hipGetLastError();
}

hipError_t launch_repack(const Layer& L, const uint8_t* canon, int n_experts_in, int first_expert,
                         hipStream_t s) {
  const long long per = 2LL * L.I * (L.H / SB_WEIGHTS) + (long long)L.H * (L.I / SB_WEIGHTS);
  const long long n = per * n_experts_in;
  if (n == 0) return hipSuccess;
  const int bs = 256;
  hipLaunchKernelGGL(k_repack, dim3((unsigned)((n + bs - 1) / bs)), dim3(bs), 0, s, canon,
                     const_cast<uint8_t*>(L.packed), L.fmt, L.H, L.I, L.Ho, L.Io,
                     canon_expert_bytes(L.fmt, L.Ho, L.Io), L.expert_stride, n, first_expert);
  return hipGetLastError();
}

hipError_t launch_router_split(const Layer& L, hipStream_t s) {
  const long long n = (long long)((L.E + 15) / 16) * 16 * L.H;
  const int bs = 256;
  hipLaunchKernelGGL(k_router_split, dim3((unsigned)((n + bs - 1) / bs)), dim3(bs), 0, s,
                     L.router_w, const_cast<uint16_t*>(L.router_hi),
                     const_cast<uint16_t*>(L.router_lo), L.E, L.H, L.Ho, n);
  return hipGetLastError();
}

}  // namespace strata
