"""Plain fp64 CPU oracle for one routed mixture-of-experts FFN layer.

TEST INFRASTRUCTURE.  Only the test suite, the package smoke check and the
benchmark's CPU-baseline leg may import this module.  It shares no code with
the HIP library: its own unpacking, its own routing, its own expert math.

What it computes (the routing pipeline of blog.5616760.com/0039.html,
section 五 "MoE 的本质", whose flowchart goes router scores -> top-10 ->
softmax-weighted merge; the GPU computing each selected expert and summing
the results, ai-coding.wiselychen.com "Strata two weeks", section
成功思路一; the always-on shared expert of the DeepSeek layer, lcz.me/topic/2153
section 一):

  O1 unpack   w = d * (q - c) per 32-weight block, c = 1.5 / 3.5 / 8;
              MXFP4 (format 5): w = 2^(e - 127) * E2M1(q)
  O2 router   l[t, e] = sum_h x[t, h] * Wr[e, h] + b[e]
  O3 select   S_t = the k largest l[t, .]  (ids returned in ascending order)
  O4 weights  w[t, j] = softmax of l[t, .] restricted to S_t
  O5 expert   y = W_down (silu(W_gate x) * (W_up x)),  silu(z) = z / (1 + e^-z)
  O6 combine  out[t] = sum_j w[t, j] y_j(x_t)  (+ shared y_s(x_t)) (+ residual)
  O7 permute  stable counting sort of pairs p = t*k + j by (expert, p)

The pages fix none of the block layout, the expert FFN form, the
renormalisation or the tie order; the readings used here are:
  * a block is its code bytes, then a little-endian fp16 scale d;
  * code j of a block occupies bits [b*j, b*j + b) of the code bytes read
    as one little-endian bit string (least significant bit first);
  * blocks run along the reduction dimension; gate/up are [I rows][H/32
    blocks], down is [H rows][I/32 blocks]; an expert record is gate, up,
    down back to back;
  * SwiGLU: silu on the gate projection times the up projection, no biases;
  * the softmax is renormalised over the selected k (weights sum to 1);
  * the shared expert enters the sum with weight 1.
Every quantity is fp64; the stored inputs (bf16 x, fp32 router, fp16 d) are
taken exactly.

MXFP4 experts.  The pages name the format (lcz.me/topic/2153, the DeepSeek
suites of section 一) but give no layout; the element and scale encodings are
those of the OCP Microscaling Formats (MX) v1.0 specification: a block of 32
FP4 E2M1 elements (1 sign bit, 2 exponent bits with bias 1, 1 mantissa bit;
exponent field 0 is subnormal: m * 0.5) sharing one E8M0 scale byte e (the
value 2^(e - 127); e = 255 is NaN).  Readings: element j of a block is the
4-bit code j in the block's little-endian bit string (as for the other
formats, so byte j / 2, low nibble first), followed by the scale byte; there
is no offset term.
"""

import numpy as np

# code offset c of each format (w = d * (q - c))
OFFSET = {2: 1.5, 3: 3.5, 4: 8.0}
CODE_BYTES = {2: 8, 3: 12, 4: 16, 5: 16}
CODE_BITS = {2: 2, 3: 3, 4: 4, 5: 4}
SCALE_BYTES = {2: 2, 3: 2, 4: 2, 5: 1}
MXFP4 = 5
BLOCK = 32


def block_bytes(fmt):
    return CODE_BYTES[fmt] + SCALE_BYTES[fmt]


def e2m1_value(q):
    """FP4 E2M1 code(s) -> value: sign bit 3, exponent bits 1-2 (bias 1),
    mantissa bit 0; exponent field 0 is subnormal (m * 2^(1 - 1) * 0.5)."""
    q = np.asarray(q, dtype=np.int64)
    sign = np.where(q & 8, -1.0, 1.0)
    ex = (q >> 1) & 3
    m = (q & 1).astype(np.float64)
    mag = np.where(ex == 0, 0.5 * m, (1.0 + 0.5 * m) * np.exp2(ex.astype(np.float64) - 1.0))
    return sign * mag


def e8m0_value(e):
    """E8M0 scale byte(s) -> 2^(e - 127); 255 is NaN."""
    e = np.asarray(e, dtype=np.int64)
    return np.where(e == 255, np.nan, np.exp2(e.astype(np.float64) - 127.0))


# ---------------------------------------------------------------- O1 unpack
def unpack_codes(code_bytes, bits):
    """Codes of a little-endian bit string: code j = bits [bits*j, bits*j+bits).

    code_bytes: uint8 [..., nbytes]  ->  int16 [..., nbytes*8 // bits]
    """
    stream = np.unpackbits(np.asarray(code_bytes, dtype=np.uint8), axis=-1, bitorder="little")
    n = stream.shape[-1] // bits
    stream = stream[..., : n * bits].reshape(*stream.shape[:-1], n, bits)
    place = (np.uint8(1) << np.arange(bits, dtype=np.uint8))     # bit i of a code weighs 2^i
    return (stream * place).sum(axis=-1, dtype=np.int16)


def dequant_blocks(blocks, fmt):
    """blocks uint8 [..., nblk, Bq] -> fp64 weights [..., nblk*32]."""
    cb = CODE_BYTES[fmt]
    blocks = np.asarray(blocks, dtype=np.uint8)
    q = unpack_codes(blocks[..., :cb], CODE_BITS[fmt])            # [..., nblk, 32]
    if fmt == MXFP4:
        w = e8m0_value(blocks[..., cb])[..., None] * e2m1_value(q)
    else:
        d = np.ascontiguousarray(blocks[..., cb:cb + 2]).view("<f2")[..., 0].astype(np.float64)
        w = d[..., None] * (q.astype(np.float64) - OFFSET[fmt])
    return w.reshape(*w.shape[:-2], w.shape[-2] * BLOCK)


def split_record(record, hidden, inter, fmt):
    """Canonical expert record -> (gate, up, down) block arrays."""
    bq = block_bytes(fmt)
    rec = np.asarray(record, dtype=np.uint8).reshape(-1)
    n_gu = inter * (hidden // BLOCK) * bq
    gate = rec[:n_gu].reshape(inter, hidden // BLOCK, bq)
    up = rec[n_gu:2 * n_gu].reshape(inter, hidden // BLOCK, bq)
    down = rec[2 * n_gu:].reshape(hidden, inter // BLOCK, bq)
    assert down.size == hidden * (inter // BLOCK) * bq
    return gate, up, down


def dequant_expert(record, hidden, inter, fmt):
    """-> W_gate [I, H], W_up [I, H], W_down [H, I] in fp64."""
    g, u, d = split_record(record, hidden, inter, fmt)
    return dequant_blocks(g, fmt), dequant_blocks(u, fmt), dequant_blocks(d, fmt)


# ---------------------------------------------------------------- O2-O4 routing
def router_logits(x, router_w, router_b=None):
    """l[t, e] = sum_h x[t, h] Wr[e, h] + b[e] in fp64."""
    l = np.asarray(x, dtype=np.float64) @ np.asarray(router_w, dtype=np.float64).T
    if router_b is not None:
        l = l + np.asarray(router_b, dtype=np.float64)[None, :]
    return l


def select_topk(logits, k):
    """k largest logits per token.

    Returns (idx [T, k] ascending expert ids, gap [T]) where gap is the
    distance between the k-th and (k+1)-th largest logit (inf when k = E).
    Equal logits rank the lower expert id first.
    """
    logits = np.asarray(logits, dtype=np.float64)
    order = np.argsort(-logits, axis=1, kind="stable")
    idx = np.sort(order[:, :k], axis=1)
    srt = np.take_along_axis(logits, order, axis=1)
    if k < logits.shape[1]:
        gap = srt[:, k - 1] - srt[:, k]
    else:
        gap = np.full(logits.shape[0], np.inf)
    return idx.astype(np.int64), gap


def routing_weights(logits, idx):
    """Softmax of the selected logits (max-subtracted), renormalised over S_t."""
    sel = np.take_along_axis(np.asarray(logits, dtype=np.float64), idx, axis=1)
    z = np.exp(sel - sel.max(axis=1, keepdims=True))
    return z / z.sum(axis=1, keepdims=True)


# ---------------------------------------------------------------- O5 expert
def silu(z):
    return z / (1.0 + np.exp(-z))


def expert_ffn(x, w_gate, w_up, w_down):
    """y = W_down (silu(W_gate x) * (W_up x)) for rows of x [n, H]."""
    x = np.asarray(x, dtype=np.float64)
    g = x @ w_gate.T
    u = x @ w_up.T
    return (silu(g) * u) @ w_down.T


# ---------------------------------------------------------------- O7 permute
def permute(idx, n_experts):
    """Stable counting sort of pairs p = t*k + j by key (expert, p).

    Returns counts [E], offsets [E+1] (exclusive scan), perm [T*k] (sorted
    slot -> p) and inv [T*k] (p -> sorted slot).
    """
    flat = np.asarray(idx, dtype=np.int64).reshape(-1)
    counts = np.bincount(flat, minlength=n_experts).astype(np.int64)
    offsets = np.zeros(n_experts + 1, dtype=np.int64)
    offsets[1:] = np.cumsum(counts)
    perm = np.empty(flat.size, dtype=np.int64)
    inv = np.empty(flat.size, dtype=np.int64)
    fill = offsets[:-1].copy()
    for p, e in enumerate(flat):          # pairs visited in increasing p: stable
        perm[fill[e]] = p
        inv[p] = fill[e]
        fill[e] += 1
    return counts, offsets, perm, inv


# ---------------------------------------------------------------- O6 layer
def route(x, router_w, router_b, k):
    l = router_logits(x, router_w, router_b)
    idx, gap = select_topk(l, k)
    w = routing_weights(l, idx)
    return l, idx, w, gap


def moe_layer(x, router_w, router_b, expert_record, hidden, inter, k, fmt,
              shared_record=None, residual=False):
    """One MoE layer over tokens x [T, H] (fp64 values).

    expert_record(e) returns the canonical record of routed expert e.
    Returns (out [T, H], info) with info holding logits, idx, w and gap.
    """
    x = np.asarray(x, dtype=np.float64)
    T = x.shape[0]
    logits, idx, w, gap = route(x, router_w, router_b, k)
    out = np.zeros((T, hidden), dtype=np.float64)
    for e in np.unique(idx):
        rows, cols = np.nonzero(idx == e)
        wg, wu, wd = dequant_expert(expert_record(int(e)), hidden, inter, fmt)
        y = expert_ffn(x[rows], wg, wu, wd)
        out[rows] += w[rows, cols][:, None] * y
    if shared_record is not None:
        wg, wu, wd = dequant_expert(shared_record, hidden, inter, fmt)
        out += expert_ffn(x, wg, wu, wd)
    if residual:
        out += x
    return out, {"logits": logits, "idx": idx, "w": w, "gap": gap}


def moe_stack(x0, layers, hidden, inter, k, fmt):
    """h <- h + MoE_l(h) over the layers; layers is a list of
    (router_w, router_b, expert_record) tuples.  Returns (h, per-layer info)."""
    h = np.asarray(x0, dtype=np.float64)
    infos = []
    for router_w, router_b, rec in layers:
        h, info = moe_layer(h, router_w, router_b, rec, hidden, inter, k, fmt, residual=True)
        infos.append(info)
    return h, infos
