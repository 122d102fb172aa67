"""Where the bf16 path's score error comes from (CPU, float64, run by hand).

The GPU forward rounds to bf16 at six points: the RMSNorm outputs that feed
the projections (Xn), the Q/K/V projection outputs, q and k after their norm
and rotary embedding, the softmax weights before P.V, the attention output,
and the SwiGLU output (H).  Everything else -- the residual stream, every
accumulation, the head -- is fp32.  This script runs the oracle's forward
(float64 building blocks from oracle/) with those roundings switched on one
at a time, and all together, and reports the score error against the exact
oracle on requests of the headline workload:

    python tests/error_budget.py [n_requests]

It is an analysis aid, not a test: it asserts nothing.
"""
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
sys.path.insert(0, os.path.dirname(os.path.abspath(__file__)))

import synth  # noqa: E402
from oracle import OracleModel, embed_rows, rmsnorm, rope_rotate, score_head, tree_mask  # noqa: E402
from oracle.ranker import mis_positions  # noqa: E402

POINTS = ["xn", "qkv", "qk_rope", "p", "o", "h"]


def bf16(x):
    """Round to the nearest bf16 (ties to even), through float32."""
    f = np.asarray(x, np.float64).astype(np.float32)
    return synth.bf16_bits_to_f32(synth.f32_to_bf16_bits(f)).astype(np.float64)


def forward(model, prefix, cands, rounded):
    R = {p: (bf16 if p in rounded else (lambda a: a)) for p in POINTS}
    cfg = model.cfg
    H, Hkv, hd, eps = cfg.n_heads, cfg.n_kv_heads, cfg.head_dim, cfg.rms_eps
    L, K = len(prefix), len(cands)
    x = embed_rows(model, np.concatenate([prefix, cands]))
    pos = mis_positions(L, K)
    allowed = tree_mask(L, K)
    n = x.shape[0]
    G = H // Hkv
    for W in model.layers:
        a = R["xn"](rmsnorm(x, W["attn_norm"], eps))
        q = R["qkv"](a @ W["wq"].T).reshape(n, H, hd)
        k = R["qkv"](a @ W["wk"].T).reshape(n, Hkv, hd)
        v = R["qkv"](a @ W["wv"].T).reshape(n, Hkv, hd)
        q = R["qk_rope"](rope_rotate(rmsnorm(q, W["q_norm"], eps), pos, cfg.rope_base))
        k = R["qk_rope"](rope_rotate(rmsnorm(k, W["k_norm"], eps), pos, cfg.rope_base))
        o = np.empty((n, H, hd))
        for h in range(H):
            s = q[:, h] @ k[:, h // G].T / np.sqrt(hd)
            s = np.where(allowed, s, -np.inf)
            p = np.exp(s - s.max(axis=1, keepdims=True))
            o[:, h] = (R["p"](p) @ v[:, h // G]) / p.sum(axis=1, keepdims=True)  # weights rounded, fp32 sum
        x = x + R["o"](o.reshape(n, H * hd)) @ W["wo"].T
        b = R["xn"](rmsnorm(x, W["mlp_norm"], eps))
        g = b @ W["w_gate"].T
        u = b @ W["w_up"].T
        x = x + R["h"]((g / (1.0 + np.exp(-g))) * u) @ W["w_down"].T
    return score_head(model, x[L:])


def main():
    n_req = int(sys.argv[1]) if len(sys.argv) > 1 else 4
    from conftest import oracle_item_table
    cfg = synth.QWEN3_0P6B
    w = synth.make_weights(cfg, seed=0)
    model = OracleModel.from_arrays(cfg, w, oracle_item_table(cfg, w, synth.table_encoder_outputs(cfg)))
    reqs = synth.make_requests(3, cfg, n_requests=n_req)
    cases = [()] + [(p,) for p in POINTS] + [tuple(POINTS)]
    errs = {c: [] for c in cases}
    t0 = time.time()
    for r in reqs:
        exact = None
        for c in cases:
            s = forward(model, r.prefix, r.cands, c)
            if exact is None:
                exact = s
                continue
            errs[c].append(np.abs(s - exact))
        print(f"request L={r.L}: {time.time() - t0:.0f} s", flush=True)
    print("| rounded at | max abs score error | RMS score error |")
    print("|---|---|---|")
    for c in cases[1:]:
        e = np.concatenate(errs[c])
        print(f"| {', '.join(c)} | {e.max():.2e} | {np.sqrt(np.mean(e * e)):.2e} |")


if __name__ == "__main__":
    main()
