"""Expected outputs of the 48-layer Q3 stack workload, from the CPU oracle.

    python tests/golden/make_stack48_expected.py

Writes tests/golden/stack48_q3_expected.npz: for each decode step, the
accepted token (bf16 bits; seed, stream, index, attempt of its draw), the
oracle's h_48 (fp64) after h <- h + moe_l(h) over the 48 layers, and the
per-layer logit gap at rank k.  A candidate token is accepted when that gap is
at least 1e-3 at every layer (the stack's relaxed margin; 1e-2 at all 48
layers would keep about 1% of draws).  The stack's expert scales are drawn
with sigma 0.005 (moe_synth.workloads), so the residual stream stays finite.  Inputs come from moe_synth with the
same seed the GPU test uses; every value here is computed by oracle/.
"""

import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import oracle as O                                   # noqa: E402
from moe_synth import WORKLOADS, generate as G       # noqa: E402

SEED = 2026
STREAM = 48
STEPS = 8
MIN_GAP = 1e-3
OUT = os.path.join(os.path.dirname(os.path.abspath(__file__)), "stack48_q3_expected.npz")


def run_stack(x0, w):
    """The oracle stack, one layer at a time; stops at the first layer whose
    gap is below MIN_GAP.  Returns (h, gaps) or (None, gaps)."""
    h = x0.astype(np.float64)
    gaps = []
    for l in range(w.n_layers):
        wr = G.router_weights(SEED, l, w.hidden, w.n_experts)
        b = G.router_bias(SEED, l, w.n_experts, w.zipf_s)
        rec = (lambda e, l=l: G.expert_canonical(SEED, l, int(e), w.hidden, w.inter, w.fmt, w.d_sigma))
        h, info = O.moe_layer(h, wr, b, rec, w.hidden, w.inter, w.top_k, w.fmt, residual=True)
        gaps.append(float(info["gap"][0]))
        if gaps[-1] < MIN_GAP:
            return None, gaps
    return h, gaps


def main():
    w = WORKLOADS["stack48_q3_decode"]
    xs, hs, gaps_all, meta = [], [], [], []
    for step in range(STEPS):
        for attempt in range(50):
            t0 = time.time()
            bits = G.token_candidates(SEED, STREAM, step, w.hidden, attempt)
            x0 = G.bf16_bits_to_f32(bits).astype(np.float64)[None, :]
            h, gaps = run_stack(x0, w)
            print(f"step {step} attempt {attempt}: {len(gaps)} layers, min gap {min(gaps):.2e} "
                  f"({time.time() - t0:.0f} s)", flush=True)
            if h is not None:
                xs.append(bits)
                hs.append(h[0])
                gaps_all.append(gaps)
                meta.append((SEED, STREAM, step, attempt))
                break
        else:
            raise RuntimeError("no token with the required gaps")
    np.savez(OUT, x_bits=np.array(xs, dtype=np.uint16), h48=np.array(hs), gaps=np.array(gaps_all),
             draw=np.array(meta, dtype=np.int64))
    print("wrote", OUT)


if __name__ == "__main__":
    main()
