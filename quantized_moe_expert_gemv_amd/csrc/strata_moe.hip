// C ABI of the strata_moe library: argument checks, buffer layouts and the
// per-call kernel sequence.  The operation each entry point performs is
// specified in include/strata_moe.h.
#include <hip/hip_runtime.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>
#include <string>
#include <mutex>
#include <new>

#include "strata_moe.h"
#include "common.hpp"
#include "kernels.hpp"

using namespace strata;

namespace strata {
}

struct strata_moe {
  strata_moe_config cfg;
  Layer L;
  Work W;          // regions sized for cfg.max_tokens (max_tiles set per call)
  uint8_t* ws;
  size_t ws_bytes;
  int device;                // the device current at create
  uint8_t* scratch;          // device address of that device's static scratch array
  hipEvent_t trace[STRATA_MAX_TRACE_EVENTS];   // armed by strata_moe_trace_next_call
  int n_trace;
};

namespace {

thread_local std::string g_err;

int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return code;
}

int ok() {
  g_err.clear();
  return STRATA_OK;
}

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

size_t pad256(size_t x) { return (x + 255) & ~(size_t)255; }

int check_config(const strata_moe_config* c) {
  if (!c) return fail(STRATA_E_INVALID, "config is NULL");
  if (c->qfmt != STRATA_Q2 && c->qfmt != STRATA_Q3 && c->qfmt != STRATA_Q4 && c->qfmt != STRATA_MXFP4)
    return fail(STRATA_E_INVALID, "qfmt %d is not 2, 3, 4 or 5 (MXFP4)", c->qfmt);
  if (c->hidden <= 0 || c->inter <= 0) return fail(STRATA_E_INVALID, "hidden and inter must be positive");
  if (c->hidden % 32 || c->inter % 32)
    return fail(STRATA_E_INVALID, "hidden (%d) and inter (%d) must be multiples of 32 (one block)", c->hidden,
                c->inter);
  if (c->hidden > 65536 || c->inter > 65536)
    return fail(STRATA_E_UNSUPPORTED, "hidden (%d) and inter (%d) must be at most 65536", c->hidden,
                c->inter);
  if (c->n_experts < 1 || c->n_experts > 4096)
    return fail(STRATA_E_INVALID, "n_experts %d outside [1, 4096]", c->n_experts);
  if (c->top_k < 1 || c->top_k > c->n_experts)
    return fail(STRATA_E_INVALID, "top_k %d outside [1, n_experts = %d]", c->top_k, c->n_experts);
  if (c->n_shared != 0 && c->n_shared != 1) return fail(STRATA_E_INVALID, "n_shared must be 0 or 1");
  if (c->max_tokens < 1) return fail(STRATA_E_INVALID, "max_tokens must be >= 1");
  if ((long long)c->max_tokens * c->top_k > (1LL << 30) / 4)
    return fail(STRATA_E_UNSUPPORTED, "max_tokens * top_k too large");
  if ((long long)c->max_tokens * (long long)pad256(c->hidden) * 2 > 0xFFFFFFFFLL)
    return fail(STRATA_E_UNSUPPORTED, "max_tokens * hidden * 2 bytes of fp16 token rows exceed 4 GiB");
  // the kernels address an expert record and its matrices with 32-bit byte
  // offsets inside one buffer descriptor
  if (packed_expert_bytes(c->qfmt, (int)pad256(c->hidden), (int)pad256(c->inter)) >= (1ull << 31))
    return fail(STRATA_E_UNSUPPORTED, "one packed expert of %d x %d exceeds 2 GiB", c->hidden, c->inter);
  return STRATA_OK;
}

struct WsPlan {
  size_t logits, topk_idx, topk_w, counts, offsets, perm, inv, slot_tok, udesc, wtab, meta,
      chunk_base, pair_rank, texp, tmax, tiles, act, xparts, xpad, y, total;
  int nchunks, max_tiles;
};

int max_tiles_for(const strata_moe_config& c, int T) {
  const long long P = (long long)T * c.top_k;
  const long long t = (P + PREFILL_BM - 1) / PREFILL_BM + (P < c.n_experts ? P : c.n_experts) +
                      (long long)c.n_shared * ((T + PREFILL_BM - 1) / PREFILL_BM);
  return (int)t;
}

WsPlan plan_workspace(const strata_moe_config& c) {
  WsPlan p;
  // H, I: the kernels' widths (whole superblocks)
  const size_t T = c.max_tokens, E = c.n_experts, k = c.top_k, H = pad256(c.hidden), I = pad256(c.inter);
  const size_t P = T * k, slots = P + (size_t)c.n_shared * T;
  p.nchunks = prefill_max_chunks((int)T);
  p.max_tiles = max_tiles_for(c, (int)T);
  size_t o = 0;
  auto take = [&](size_t bytes) { size_t r = o; o = align256(o + bytes); return r; };
  p.logits = take(T * E * 4);
  p.topk_idx = take(P * 4);
  p.topk_w = take(P * 4);
  p.counts = take(E * 4);
  p.offsets = take((E + 1) * 4);
  p.perm = take(P * 4);
  p.inv = take(P * 4);
  p.slot_tok = take(P * 4);
  p.udesc = take((E + 1) * 2 * 4);
  p.wtab = take((E + 1) * 16 * 4);
  p.meta = take(16 * 4);
  p.chunk_base = take(E * (size_t)p.nchunks * 4);
  p.pair_rank = take(P * 4);
  p.texp = take(T * 4);
  p.tmax = take(32 * T * 4);
  p.tiles = take((size_t)p.max_tiles * 16);
  const size_t Td = T < STRATA_DECODE_MAX_T ? T : STRATA_DECODE_MAX_T;
  const size_t act_prefill = slots * I * 2;                                   // bf16 rows
  const size_t umax = (Td * k < E ? Td * k : E) + (size_t)c.n_shared;
  const size_t act_decode = umax * Td * 2 * I * 2;                             // two fp16 parts
  p.act = take(act_prefill > act_decode ? act_prefill : act_decode);
  p.xparts = take(Td * 2 * H * 2);
  p.xpad = take(H != (size_t)c.hidden ? T * H * 4 : 0);
  p.y = take(slots * H * 2);
  p.total = o;
  return p;
}

// The workspace regions of a plan at base ws.
Work layout_work(uint8_t* ws, const WsPlan& p) {
  Work W;
  W.logits = reinterpret_cast<float*>(ws + p.logits);
  W.topk_idx = reinterpret_cast<int*>(ws + p.topk_idx);
  W.topk_w = reinterpret_cast<float*>(ws + p.topk_w);
  W.counts = reinterpret_cast<int*>(ws + p.counts);
  W.offsets = reinterpret_cast<int*>(ws + p.offsets);
  W.perm = reinterpret_cast<int*>(ws + p.perm);
  W.inv = reinterpret_cast<int*>(ws + p.inv);
  W.slot_tok = reinterpret_cast<int*>(ws + p.slot_tok);
  W.udesc = reinterpret_cast<int*>(ws + p.udesc);
  W.meta = reinterpret_cast<int*>(ws + p.meta);
  W.chunk_base = reinterpret_cast<int*>(ws + p.chunk_base);
  W.pair_rank = reinterpret_cast<int*>(ws + p.pair_rank);
  W.texp = reinterpret_cast<int*>(ws + p.texp);
  W.tmax = reinterpret_cast<uint32_t*>(ws + p.tmax);
  W.tiles = reinterpret_cast<int4*>(ws + p.tiles);
  W.act = reinterpret_cast<float*>(ws + p.act);
  W.actp = reinterpret_cast<_Float16*>(ws + p.act);
  W.xparts = reinterpret_cast<_Float16*>(ws + p.xparts);
  W.wtab = reinterpret_cast<float*>(ws + p.wtab);
  W.ybf = reinterpret_cast<uint16_t*>(ws + p.y);
  W.ybf_bytes = p.total - p.y;                 // the last region
  W.xpad = ws + p.xpad;
  W.nchunks = p.nchunks;
  W.max_tiles = p.max_tiles;
  return W;
}

// ------------------------------------------------------------------ static scratch
// The allocation-free entry point keeps its per-call regions in this array
// instead of a caller's workspace.  Each device holds its own copy (at its
// own address) from the first use until the process ends.  In host code the
// array's name is only a stand-in: its device address comes from
// hipGetSymbolAddress, taken once per device with that device current (at
// the first create on the device) and kept in g_scratch.  Nothing in it
// needs to start at zero: every region a call reads is written earlier in
// the same call.
static __device__ __align__(256) uint8_t scratch[STRATA_STATIC_SCRATCH_BYTES];

constexpr int MAX_DEVICES = 64;
std::mutex g_scratch_mu;
uint8_t* g_scratch[MAX_DEVICES] = {};

// the current device's scratch address (looked up on the first call per device)
hipError_t scratch_address(int dev, uint8_t** out) {
  if (dev < 0 || dev >= MAX_DEVICES) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch[dev]) {
    void* ptr = nullptr;
    const hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    g_scratch[dev] = static_cast<uint8_t*>(ptr);
  }
  *out = g_scratch[dev];
  return hipSuccess;
}

// one part (high or low) of the router split: experts padded to groups of 16
size_t router_part_bytes(const strata_moe_config& c) {
  return align256((size_t)((c.n_experts + 15) / 16) * 16 * pad256(c.hidden) * 2);
}

size_t packed_experts_bytes(const strata_moe_config& c) {
  return align256((size_t)(c.n_experts + c.n_shared) *
                  packed_expert_bytes(c.qfmt, (int)pad256(c.hidden), (int)pad256(c.inter)));
}

// after the experts and the router split: 256 bytes of per-layer state
// (the one-launch routing's completion counter), zeroed at create
constexpr size_t STATE_BYTES = 256;

size_t packed_total(const strata_moe_config& c) {
  return packed_experts_bytes(c) + 2 * router_part_bytes(c) + STATE_BYTES;
}

int hip_fail(hipError_t e, const char* what) {
  return fail(STRATA_E_HIP, "%s: %s", what, hipGetErrorString(e));
}

int check_call(strata_moe* h, const void* x, int32_t x_dtype, int32_t T) {
  if (!h) return fail(STRATA_E_INVALID, "handle is NULL");
  if (!x) return fail(STRATA_E_INVALID, "x is NULL");
  if (x_dtype != STRATA_BF16 && x_dtype != STRATA_FP32)
    return fail(STRATA_E_INVALID, "x_dtype %d is not STRATA_BF16 or STRATA_FP32", x_dtype);
  if (T < 1 || T > h->cfg.max_tokens)
    return fail(STRATA_E_INVALID, "T = %d outside [1, max_tokens = %d]", T, h->cfg.max_tokens);
  if (!aligned(x, 16)) return fail(STRATA_E_INVALID, "x must be 16-byte aligned");
  return STRATA_OK;
}

bool fits(const strata_moe_config& c, int T) {
  return decode_fits(T, c.top_k, c.n_experts, c.n_shared, (int)pad256(c.inter));
}

bool use_decode(const strata_moe_config& c, int T, uint32_t flags) {
  if (flags & STRATA_FORCE_PREFILL) return false;
  return fits(c, T);
}

int check_flags(const strata_moe_config& c, int T, uint32_t flags) {
  const uint32_t known = STRATA_ACCUMULATE | STRATA_ADD_INPUT | STRATA_FORCE_DECODE | STRATA_FORCE_PREFILL |
                         STRATA_FUSED_ROUTE | STRATA_SPLIT_ROUTE;
  if (flags & ~known) return fail(STRATA_E_INVALID, "unknown flag bits 0x%x", flags & ~known);
  if ((flags & STRATA_FUSED_ROUTE) && (flags & STRATA_SPLIT_ROUTE))
    return fail(STRATA_E_INVALID, "FUSED_ROUTE and SPLIT_ROUTE are exclusive");
  if ((flags & STRATA_FUSED_ROUTE) && !fused_route_fits(c.n_experts, c.top_k, T))
    return fail(STRATA_E_UNSUPPORTED, "one-launch routing covers T <= 64, n_experts <= 512, top_k <= 64");
  if ((flags & STRATA_FORCE_DECODE) && (flags & STRATA_FORCE_PREFILL))
    return fail(STRATA_E_INVALID, "FORCE_DECODE and FORCE_PREFILL are exclusive");
  if ((flags & STRATA_FORCE_DECODE) && T > STRATA_DECODE_MAX_T)
    return fail(STRATA_E_UNSUPPORTED, "the decode path takes at most %d tokens", STRATA_DECODE_MAX_T);
  if ((flags & STRATA_FORCE_DECODE) && !fits(c, T))
    return fail(STRATA_E_UNSUPPORTED, "the decode path's LDS does not hold %d tokens at top_k %d", T, c.top_k);
  if ((flags & STRATA_ACCUMULATE) && (flags & STRATA_ADD_INPUT))
    return fail(STRATA_E_INVALID, "ACCUMULATE and ADD_INPUT are exclusive");
  return STRATA_OK;
}

int check_forward(strata_moe* h, const void* x, int32_t x_dtype, int32_t T, const float* out, uint32_t flags) {
  int rc = check_call(h, x, x_dtype, T);
  if (rc) return rc;
  if ((rc = check_flags(h->cfg, T, flags))) return rc;
  if (!out) return fail(STRATA_E_INVALID, "out is NULL");
  if (!aligned(out, 16)) return fail(STRATA_E_INVALID, "out must be 16-byte aligned");
  const size_t xb = (size_t)T * h->cfg.hidden * (x_dtype == STRATA_FP32 ? 4 : 2);
  const size_t ob = (size_t)T * h->cfg.hidden * 4;
  const uintptr_t xa = (uintptr_t)x, oa = (uintptr_t)out;
  if (xa < oa + ob && oa < xa + xb) return fail(STRATA_E_INVALID, "x and out overlap");
  return STRATA_OK;
}

Call make_call(const void* x, int32_t x_dtype, int32_t T, float* out, uint32_t flags) {
  Call c;
  c.x = x;
  c.x_f32 = (x_dtype == STRATA_FP32);
  c.T = T;
  c.out = out;
  c.flags = flags;
  return c;
}

// A call consumes the events armed by strata_moe_trace_next_call (one-shot).
struct TraceScope {
  Tracer t;
  Tracer* ptr = nullptr;
  explicit TraceScope(strata_moe* h) {
    if (h->n_trace > 0) {
      t.ev = h->trace;
      t.n = h->n_trace;
      ptr = &t;
      h->n_trace = 0;
    }
  }
};

// permutation: the decode path computes the token->expert permutation only
// when the caller asks for it (route()); its expert kernels do without.
int run_route(strata_moe* h, const Work& W0, const Call& c, bool decode, bool permutation, hipStream_t s,
              Tracer* tr) {
  Work W = W0;
  W.max_tiles = max_tiles_for(h->cfg, c.T);
  hipError_t e = decode ? launch_decode_route(h->L, W, c, s, tr, permutation)
                        : launch_prefill_route(h->L, W, c, s, tr);
  if (e != hipSuccess) return hip_fail(e, "route launch");
  return STRATA_OK;
}

int run_forward(strata_moe* h, const Work& W0, const Call& c, bool decode, hipStream_t s, Tracer* tr) {
  int rc = run_route(h, W0, c, decode, false, s, tr);
  if (rc) return rc;
  Work W = W0;
  W.max_tiles = max_tiles_for(h->cfg, c.T);
  hipError_t e = decode ? launch_decode_experts(h->L, W, c, s, tr) : launch_prefill_experts(h->L, W, c, s, tr);
  if (e != hipSuccess) return hip_fail(e, "expert launch");
  return STRATA_OK;
}

}  // namespace

extern "C" {

size_t strata_moe_expert_bytes(const strata_moe_config* cfg) {
  if (check_config(cfg)) return 0;
  return canon_expert_bytes(cfg->qfmt, cfg->hidden, cfg->inter);
}

size_t strata_moe_packed_bytes(const strata_moe_config* cfg) {
  if (check_config(cfg)) return 0;
  return packed_total(*cfg);
}

size_t strata_moe_workspace_bytes(const strata_moe_config* cfg) {
  if (check_config(cfg)) return 0;
  return plan_workspace(*cfg).total;
}

int strata_moe_create(const strata_moe_config* cfg, const float* router_w, const float* router_bias,
                      const void* experts_canon, const void* shared_canon, void* packed,
                      void* workspace, void* stream, strata_moe** out) {
  int rc = check_config(cfg);
  if (rc) return rc;
  if (!out) return fail(STRATA_E_INVALID, "out is NULL");
  *out = nullptr;
  if (!router_w || !experts_canon || !packed || !workspace)
    return fail(STRATA_E_INVALID, "router_w, experts_canon, packed and workspace must be non-NULL");
  if (cfg->n_shared == 1 && !shared_canon) return fail(STRATA_E_INVALID, "n_shared = 1 needs shared_canon");
  if (cfg->n_shared == 0 && shared_canon) return fail(STRATA_E_INVALID, "shared_canon given but n_shared = 0");
  if (!aligned(packed, 256) || !aligned(workspace, 256))
    return fail(STRATA_E_INVALID, "packed and workspace must be 256-byte aligned");
  if (!aligned(router_w, 16)) return fail(STRATA_E_INVALID, "router_w must be 16-byte aligned");
  if (router_bias && !aligned(router_bias, 4)) return fail(STRATA_E_INVALID, "router_bias must be 4-byte aligned");

  strata_moe* h = new (std::nothrow) strata_moe();
  if (!h) return fail(STRATA_E_INVALID, "out of host memory");
  h->cfg = *cfg;
  const WsPlan p = plan_workspace(*cfg);
  uint8_t* ws = static_cast<uint8_t*>(workspace);
  h->ws = ws;
  h->ws_bytes = p.total;
  Layer& L = h->L;
  L.H = (int)pad256(cfg->hidden); L.I = (int)pad256(cfg->inter); L.Ho = cfg->hidden; L.Io = cfg->inter;
  L.E = cfg->n_experts; L.k = cfg->top_k;
  L.n_shared = cfg->n_shared; L.fmt = cfg->qfmt;
  L.router_w = router_w; L.router_b = router_bias;
  L.packed = static_cast<const uint8_t*>(packed);
  L.expert_stride = packed_expert_bytes(cfg->qfmt, L.H, L.I);
  const size_t rh = packed_experts_bytes(*cfg);
  L.router_hi = reinterpret_cast<const uint16_t*>(L.packed + rh);
  L.router_lo = reinterpret_cast<const uint16_t*>(L.packed + rh + router_part_bytes(*cfg));
  uint8_t* state = static_cast<uint8_t*>(packed) + rh + 2 * router_part_bytes(*cfg);
  L.route_done = reinterpret_cast<int*>(state);
  h->W = layout_work(ws, p);

  hipStream_t s = static_cast<hipStream_t>(stream);
  int* bad_scales = h->W.meta + 4;
  const char* step = "zeroing counters";
  static_assert(STRATA_FUSED_ROUTE == STRATA_FUSED_ROUTE_FLAG && STRATA_SPLIT_ROUTE == STRATA_SPLIT_ROUTE_FLAG,
                "flag bits");
  hipError_t e = hipMemsetAsync(ws + p.meta, 0, 16 * 4, s);
  if (e == hipSuccess) e = hipMemsetAsync(state, 0, STATE_BYTES, s);
  if (e == hipSuccess) {
    step = "scale check";
    e = launch_check_scales(L, static_cast<const uint8_t*>(experts_canon), cfg->n_experts, bad_scales, s);
    if (e == hipSuccess && cfg->n_shared)
      e = launch_check_scales(L, static_cast<const uint8_t*>(shared_canon), 1, bad_scales, s);
  }
  if (e == hipSuccess) {
    step = "expert repack";
    e = launch_repack(L, static_cast<const uint8_t*>(experts_canon), cfg->n_experts, 0, s);
  }
  if (e == hipSuccess && cfg->n_shared) {
    step = "shared expert repack";
    e = launch_repack(L, static_cast<const uint8_t*>(shared_canon), 1, cfg->n_experts, s);
  }
  if (e == hipSuccess) {
    step = "router split";
    e = launch_router_split(L, s);
  }
  if (e == hipSuccess) {
    step = "kernel attributes";
    e = prepare_decode_kernels();
  }
  if (e == hipSuccess) {
    step = "current device";
    e = hipGetDevice(&h->device);
  }
  if (e == hipSuccess) {
    step = "static scratch address";
    e = scratch_address(h->device, &h->scratch);
  }
  if (e == hipSuccess) {
    step = "stream synchronize";
    e = hipStreamSynchronize(s);
  }
  int n_bad = 0;
  if (e == hipSuccess) {
    step = "scale check result";
    e = hipMemcpy(&n_bad, bad_scales, sizeof n_bad, hipMemcpyDeviceToHost);
  }
  if (e != hipSuccess) {
    (void)hipGetLastError();
    delete h;
    char what[64];
    snprintf(what, sizeof what, "create (%s)", step);
    return hip_fail(e, what);
  }
  if (n_bad) {
    delete h;
    return fail(STRATA_E_UNSUPPORTED,
                "%d block scale(s) outside what the 16-bit operands carry (fp16 d NaN, infinite or above "
                "2^15 / 2^14 / 2^12 for Q2 / Q3 / Q4; MXFP4 e = 255 or above 140)", n_bad);
  }
  *out = h;
  return ok();
}

int strata_moe_route(strata_moe* h, const void* x, int32_t x_dtype, int32_t T, int32_t* topk_idx,
                     float* topk_w, int32_t* perm, int32_t* offsets, uint32_t flags, void* stream) {
  int rc = check_call(h, x, x_dtype, T);
  if (rc) return rc;
  if ((rc = check_flags(h->cfg, T, flags))) return rc;
  if (!topk_idx || !topk_w || !perm || !offsets)
    return fail(STRATA_E_INVALID, "route outputs must be non-NULL");
  hipStream_t s = static_cast<hipStream_t>(stream);
  const Call c = make_call(x, x_dtype, T, nullptr, flags);
  TraceScope ts(h);
  if ((rc = run_route(h, h->W, c, use_decode(h->cfg, T, flags), true, s, ts.ptr))) return rc;
  const size_t P = (size_t)T * h->cfg.top_k;
  hipError_t e = hipMemcpyAsync(topk_idx, h->W.topk_idx, P * 4, hipMemcpyDeviceToDevice, s);
  if (e == hipSuccess) e = hipMemcpyAsync(topk_w, h->W.topk_w, P * 4, hipMemcpyDeviceToDevice, s);
  if (e == hipSuccess) e = hipMemcpyAsync(perm, h->W.perm, P * 4, hipMemcpyDeviceToDevice, s);
  if (e == hipSuccess)
    e = hipMemcpyAsync(offsets, h->W.offsets, (size_t)(h->cfg.n_experts + 1) * 4, hipMemcpyDeviceToDevice, s);
  if (e != hipSuccess) return hip_fail(e, "route copy");
  return ok();
}

int strata_moe_forward(strata_moe* h, const void* x, int32_t x_dtype, int32_t T, float* out,
                       uint32_t flags, void* stream) {
  int rc = check_forward(h, x, x_dtype, T, out, flags);
  if (rc) return rc;
  hipStream_t s = static_cast<hipStream_t>(stream);
  TraceScope ts(h);
  if ((rc = run_forward(h, h->W, make_call(x, x_dtype, T, out, flags), use_decode(h->cfg, T, flags), s, ts.ptr)))
    return rc;
  return ok();
}

int strata_moe_forward_static(strata_moe* h, const void* x, int32_t x_dtype, int32_t T, float* out,
                              uint32_t flags, void* stream) {
  int rc = check_forward(h, x, x_dtype, T, out, flags);
  if (rc) return rc;
  strata_moe_config c = h->cfg;
  c.max_tokens = T;
  const WsPlan p = plan_workspace(c);
  if (p.total > STRATA_STATIC_SCRATCH_BYTES)
    return fail(STRATA_E_UNSUPPORTED,
                "a call of %d tokens needs %zu bytes of scratch, more than the static array's %zu", T, p.total,
                (size_t)STRATA_STATIC_SCRATCH_BYTES);
  if (!h->scratch) return fail(STRATA_E_HIP, "the static scratch of device %d was not resolved", h->device);
  const Work W = layout_work(h->scratch, p);
  hipStream_t s = static_cast<hipStream_t>(stream);
  TraceScope ts(h);
  if ((rc = run_forward(h, W, make_call(x, x_dtype, T, out, flags), use_decode(h->cfg, T, flags), s, ts.ptr)))
    return rc;
  return ok();
}

int strata_moe_stack_forward(strata_moe* const* layers, int32_t n_layers, const void* x,
                             int32_t x_dtype, int32_t T, float* out, float* tmp, void* stream) {
  if (!layers || n_layers < 1) return fail(STRATA_E_INVALID, "need at least one layer");
  if (!out || !tmp) return fail(STRATA_E_INVALID, "out and tmp must be non-NULL");
  for (int l = 0; l < n_layers; ++l) {
    if (!layers[l]) return fail(STRATA_E_INVALID, "layer %d is NULL", l);
    if (layers[l]->cfg.hidden != layers[0]->cfg.hidden)
      return fail(STRATA_E_INVALID, "layer %d hidden differs from layer 0", l);
    int rc = check_call(layers[l], x, x_dtype, T);
    if (rc) return rc;
  }
  if (!aligned(out, 16) || !aligned(tmp, 16)) return fail(STRATA_E_INVALID, "out and tmp must be 16-byte aligned");
  const size_t ob = (size_t)T * layers[0]->cfg.hidden * 4;
  const size_t xb = (size_t)T * layers[0]->cfg.hidden * (x_dtype == STRATA_FP32 ? 4 : 2);
  auto overlap = [](uintptr_t a, size_t na, uintptr_t b, size_t nb) { return a < b + nb && b < a + na; };
  if (overlap((uintptr_t)out, ob, (uintptr_t)tmp, ob) || overlap((uintptr_t)x, xb, (uintptr_t)out, ob) ||
      overlap((uintptr_t)x, xb, (uintptr_t)tmp, ob))
    return fail(STRATA_E_INVALID, "x, out and tmp must not overlap");
  hipStream_t s = static_cast<hipStream_t>(stream);
  const void* cur = x;
  int cur_dtype = x_dtype;
  for (int l = 0; l < n_layers; ++l) {
    // the last layer writes `out`; earlier layers alternate so that happens
    float* dst = ((n_layers - 1 - l) % 2 == 0) ? out : tmp;
    Call c = make_call(cur, cur_dtype, T, dst, STRATA_ADD_INPUT);
    const bool decode = use_decode(layers[l]->cfg, T, 0);
    if (decode && l + 1 < n_layers && use_decode(layers[l + 1]->cfg, T, 0)) {
      // this layer's gate/up kernel prefetches the next layer's router rows
      c.next_router = layers[l + 1]->L.router_w;
      c.next_E = layers[l + 1]->L.E;
      c.next_Ho = layers[l + 1]->L.Ho;
    }
    TraceScope ts(layers[l]);
    int rc = run_forward(layers[l], layers[l]->W, c, decode, s, ts.ptr);
    if (rc) return rc;
    cur = dst;
    cur_dtype = STRATA_FP32;
  }
  return ok();
}

int strata_moe_trace_next_call(strata_moe* h, void* const* events, int32_t n_events) {
  if (!h) return fail(STRATA_E_INVALID, "handle is NULL");
  if (n_events < 0 || n_events > STRATA_MAX_TRACE_EVENTS || (n_events & 1))
    return fail(STRATA_E_INVALID, "n_events %d is not even in [0, %d]", n_events, STRATA_MAX_TRACE_EVENTS);
  if (n_events > 0 && !events) return fail(STRATA_E_INVALID, "events is NULL");
  for (int i = 0; i < n_events; ++i) {
    if (!events[i]) return fail(STRATA_E_INVALID, "event %d is NULL", i);
    h->trace[i] = static_cast<hipEvent_t>(events[i]);
  }
  h->n_trace = n_events;
  return ok();
}

void strata_moe_destroy(strata_moe* h) { delete h; }

const char* strata_moe_last_error(void) { return g_err.c_str(); }

}  // extern "C"
