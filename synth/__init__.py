"""Seeded synthetic inputs for the DuoLM multi-item-scoring (MIS) ranker forward.

This module makes the *inputs* that both the CPU oracle and the HIP library read:
random-init weights of the ranker's shape, the fp16 virtual-token-ID (VID) item
table, and synthetic requests.  It holds none of the ranker's arithmetic: no
normalisation of activations, no attention, no projection, no scoring.  The only
numeric work here is drawing random numbers and rounding them to the storage
formats (bf16 by round-to-nearest-even, fp16 by numpy's own RNE cast).

Sources for the shapes (DuoLM, "Fast and Effective Personalized Recommendation
with Language Models", digest pages):
  * ranker backbone: Qwen3-0.6B, 28 layers (paper.rainbus.top digest, section
    "核心方法" and "复现评估");
  * input template: instruction, then per history item a marker embedding, the
    item vector and its feedback text, then the candidate vector (onedev.kr
    digest, section "어떻게 동작하나");
  * VID ids: item i is virtual id V + iota(i), a row of a GPU-resident FP16
    table appended after the text vocabulary (rainbus digest, "方法步骤详情"
    step 3; onedev.kr, "어떻게 쓰나");
  * evaluation candidates: 1 target + 99 random non-interacted items
    (rainbus digest, "HR@10与NDCG@10").
Real weights, tokenizer and the Amazon Reviews data are not available, so every
input is synthetic; the recipes are listed in the workload table below.
"""
from __future__ import annotations

import dataclasses
from typing import Dict, List, Tuple

import numpy as np

# ----------------------------------------------------------------------------
# model shapes
# ----------------------------------------------------------------------------


@dataclasses.dataclass(frozen=True)
class ModelConfig:
    name: str
    n_layers: int
    d_model: int
    n_heads: int
    n_kv_heads: int
    head_dim: int
    d_ffn: int
    vocab: int
    n_vid: int
    rms_eps: float = 1e-6
    rope_base: float = 1e6


# Tiny ranker: 2 layers, hidden 128, 4 query / 2 KV heads of 32, SwiGLU 384,
# vocab 1000, 500 VID rows.
TINY = ModelConfig("tiny", 2, 128, 4, 2, 32, 384, 1000, 500)
# Qwen3-0.6B-shaped ranker: 28 layers, hidden 1024, 16 query / 8 KV heads of
# 128, SwiGLU 3072, vocab 151936, 200k VID rows.
QWEN3_0P6B = ModelConfig("qwen3-0.6b", 28, 1024, 16, 8, 128, 3072, 151936, 200_000)

INIT_STD = 0.02  # weights, token embedding, head and tiny VID rows ~ N(0, 0.02^2)


def tensor_specs(cfg: ModelConfig) -> List[Tuple[str, Tuple[int, ...], str]]:
    """Canonical tensor order: (name, shape, storage dtype).

    Matrices use the [out_features, in_features] convention (y = x @ W.T).
    'bf16' tensors are stored as uint16 bit patterns, 'f32' as float32.
    """
    d, hq, hk, hd, f = cfg.d_model, cfg.n_heads, cfg.n_kv_heads, cfg.head_dim, cfg.d_ffn
    specs = [("embed", (cfg.vocab, d), "bf16")]
    for l in range(cfg.n_layers):
        p = f"layers.{l}."
        specs += [
            (p + "attn_norm", (d,), "f32"),
            (p + "wq", (hq * hd, d), "bf16"),
            (p + "wk", (hk * hd, d), "bf16"),
            (p + "wv", (hk * hd, d), "bf16"),
            (p + "q_norm", (hd,), "f32"),
            (p + "k_norm", (hd,), "f32"),
            (p + "wo", (d, hq * hd), "bf16"),
            (p + "mlp_norm", (d,), "f32"),
            (p + "w_gate", (f, d), "bf16"),
            (p + "w_up", (f, d), "bf16"),
            (p + "w_down", (d, f), "bf16"),
        ]
    specs += [("final_norm", (d,), "f32"), ("head", (d,), "f32")]
    return specs


# ----------------------------------------------------------------------------
# storage-format rounding (no model arithmetic)
# ----------------------------------------------------------------------------


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (round-to-nearest-even); returns uint16 bits."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    rounding = np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))
    return ((u + rounding) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns to float32."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def f32_to_f16_bits(x: np.ndarray) -> np.ndarray:
    return np.asarray(x, dtype=np.float32).astype(np.float16).view(np.uint16)


# ----------------------------------------------------------------------------
# weights and VID table
# ----------------------------------------------------------------------------


def make_weights(cfg: ModelConfig, seed: int = 0, gain_sigma: float = 0.0) -> Dict[str, np.ndarray]:
    """Random-init ranker weights, one independent PCG64 stream per tensor.

    Matrices, the token embedding and the head vector are N(0, 0.02^2); the
    matrices and the embedding are stored as bf16 (RNE from the fp32 draw),
    the head vector as fp32.  RMSNorm gains are 1, or 1 + N(0, gain_sigma^2)
    when gain_sigma > 0 (used to make a dropped gain visible in tests).
    """
    specs = tensor_specs(cfg)
    children = np.random.SeedSequence(seed).spawn(len(specs))
    out: Dict[str, np.ndarray] = {}
    for (name, shape, dt), ss in zip(specs, children):
        rng = np.random.Generator(np.random.PCG64(ss))
        is_gain = name.endswith("norm")
        if is_gain:
            if gain_sigma > 0:
                v = 1.0 + gain_sigma * rng.standard_normal(shape, dtype=np.float32)
            else:
                v = np.ones(shape, dtype=np.float32)
            out[name] = v.astype(np.float32)
        else:
            v = rng.standard_normal(shape, dtype=np.float32)
            v *= np.float32(INIT_STD)
            out[name] = f32_to_bf16_bits(v) if dt == "bf16" else v.astype(np.float32)
    return out


def make_vid_table(cfg: ModelConfig, seed: int = 1, n_rows: int | None = None) -> np.ndarray:
    """Item table of the tiny ranker: rows ~ N(0, 0.02^2) i.i.d., stored fp16
    (uint16 bits), shape [N, d].

    The 0.6B-shaped ranker's table is made the way the pages make theirs
    instead: encoder outputs (table_encoder_outputs) exported by the
    continuous-input interface, RMS-normalised rows at the reference scale of
    the token embedding (TABLE_GAMMA, TABLE_EPS below).  That export is model
    arithmetic, so it is not done here: the library's export entry point makes
    the GPU table and the oracle's export makes the oracle's.
    """
    n = cfg.n_vid if n_rows is None else n_rows
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence(seed)))
    g = rng.standard_normal((n, cfg.d_model), dtype=np.float32)
    return f32_to_f16_bits(g * np.float32(INIT_STD))


# Export arguments of the 0.6B-shaped ranker's item table: gain e^gamma = 1
# and the ranker's own RMSNorm epsilon; rho is the RMS of the token embedding.
TABLE_GAMMA = 0.0
TABLE_EPS = 1e-6


def table_encoder_outputs(cfg: ModelConfig, seed: int = 1) -> np.ndarray:
    """Encoder outputs a_i, float32 [N, d], whose export is the item table of
    the 0.6B-shaped ranker (one row per VID)."""
    return encoder_outputs(cfg.n_vid, cfg.d_model, seed=seed)


def encoder_outputs(n_rows: int, d: int, seed: int = 11) -> np.ndarray:
    """Synthetic encoder item representations a_i, float32 [n_rows, d].

    They stand in for the last-layer EOS hidden states of the item encoder
    (Qwen3-Embedding-0.6B on the pages), whose scale is unrelated to the
    ranker's embeddings: a_i = r_i * c * g with g ~ N(0, I), a per-row scale
    r_i = exp(N(0, 0.5^2)) and a per-channel scale c = exp(N(0, 1)) shared by
    all rows (a few channels far larger than the rest, as hidden states have).
    """
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence(seed)))
    chan = np.exp(rng.standard_normal(d)).astype(np.float32)
    out = np.empty((n_rows, d), dtype=np.float32)
    step = 65536
    for i in range(0, n_rows, step):
        m = min(step, n_rows - i)
        row = np.exp(0.5 * rng.standard_normal((m, 1))).astype(np.float32)
        out[i:i + m] = rng.standard_normal((m, d), dtype=np.float32) * chan * row
    return out


# ----------------------------------------------------------------------------
# requests
# ----------------------------------------------------------------------------


@dataclasses.dataclass
class Request:
    prefix: np.ndarray      # int32 [L]: instruction, then (marker, VID x m, feedback...) per item
    cands: np.ndarray       # int32 [K*m]: candidate VIDs (V + row), m per candidate, candidate-major
    m: int = 1              # item vectors per item (history and candidates)
    # the same request in the structured form a client sends (ids only, no
    # prefix): history VIDs [n_items, m] and each item's feedback ids
    items: np.ndarray = None
    feedback: List[np.ndarray] = None

    @property
    def L(self) -> int:
        return int(self.prefix.shape[0])

    @property
    def K(self) -> int:
        return int(self.cands.shape[0]) // self.m


@dataclasses.dataclass(frozen=True)
class Workload:
    """Request recipe.  n_items: tuple of allowed history lengths (drawn
    uniformly, or cycled when `cycle_items`); feedback: fixed length, or
    ('poisson', mean, lo, hi) for clip(Poisson(mean), lo, hi) per item."""
    name: str
    n_requests: int
    n_instr: int
    n_items: Tuple[int, ...]
    feedback: object
    n_cand: int
    cycle_items: bool = False
    m: int = 1                          # item vectors per item
    cand_cycle: Tuple[int, ...] = ()    # if set, candidate counts cycled per request


WORKLOADS = {
    1: Workload("tiny-L48-K8", 1, 8, (4,), 8, 8),
    2: Workload("0.6b-C1-L452-K100", 1, 32, (10,), 40, 100),
    3: Workload("0.6b-C64-K100-varlen", 10_000, 32, (1, 3, 5, 10), ("poisson", 40, 5, 120), 100),
    4: Workload("0.6b-C8-K8-rating", 256, 32, (1, 3, 5, 10), 20, 8, cycle_items=True),
    5: Workload("0.6b-C16-L4096-K512", 16, 16, (60,), 66, 512),
    # items spread over m = 8 vectors, candidate counts cycled over {5, 20, 50, 100}:
    # the shape of the pages' FIR m = 8 rating service ([digest] 实验结果)
    6: Workload("0.6b-C8-m8-rating", 256, 32, (1, 3, 5, 10), 20, 100, cycle_items=True, m=8,
                cand_cycle=(5, 20, 50, 100)),
}


def _template(cfg: ModelConfig, seed: int, n_instr: int):
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, 7])))
    marker = int(rng.integers(0, cfg.vocab))
    instr = rng.integers(0, cfg.vocab, size=n_instr).astype(np.int32)
    return marker, instr


def template(config_id: int, cfg: ModelConfig, seed: int | None = None):
    """(marker id, instruction ids) shared by every request of workload config_id."""
    return _template(cfg, config_id if seed is None else seed, WORKLOADS[config_id].n_instr)


def make_requests(config_id: int, cfg: ModelConfig, n_requests: int | None = None,
                  seed: int | None = None, n_cand: int | None = None, m: int | None = None) -> List[Request]:
    """Synthetic requests for workload `config_id` (1..6).

    Shared per run: one marker token id and one instruction of n_instr token ids.
    Per request: n history items, each [marker, m VIDs, f feedback ids] with
    the VIDs drawn without replacement from the table and feedback ids uniform
    in [0, vocab); then K candidates of m VIDs each, drawn without replacement
    from the rows not in the history (target first, then random negatives).
    m = 1 (one vector per item) unless the workload or the caller says
    otherwise.
    """
    wl = WORKLOADS[config_id]
    seed = config_id if seed is None else seed
    n_req = wl.n_requests if n_requests is None else n_requests
    m = wl.m if m is None else m
    marker, instr = _template(cfg, seed, wl.n_instr)
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence(seed)))
    V, N = cfg.vocab, cfg.n_vid
    reqs: List[Request] = []
    for r in range(n_req):
        if n_cand is not None:
            k = n_cand
        elif wl.cand_cycle:
            k = wl.cand_cycle[r % len(wl.cand_cycle)]
        else:
            k = wl.n_cand
        if wl.cycle_items:
            n = wl.n_items[r % len(wl.n_items)]
        else:
            n = int(wl.n_items[int(rng.integers(0, len(wl.n_items)))])
        # history rows and candidate rows: distinct, candidates exclude history
        rows = _distinct(rng, N, (n + k) * m)
        hist, cand = rows[:n * m], rows[n * m:]
        parts = [instr]
        fbs = []
        for i in range(n):
            if isinstance(wl.feedback, tuple):
                _, mean, lo, hi = wl.feedback
                f = int(np.clip(rng.poisson(mean), lo, hi))
            else:
                f = int(wl.feedback)
            fb = rng.integers(0, V, size=f).astype(np.int32)
            fbs.append(fb)
            parts.append(np.concatenate([[marker], V + hist[i * m:(i + 1) * m]]).astype(np.int32))
            parts.append(fb)
        prefix = np.concatenate(parts).astype(np.int32)
        reqs.append(Request(prefix=prefix, cands=(V + cand).astype(np.int32), m=m,
                            items=(V + hist).astype(np.int32).reshape(n, m), feedback=fbs))
    return reqs


def _distinct(rng: np.random.Generator, n_total: int, count: int) -> np.ndarray:
    if count > n_total:
        raise ValueError("not enough table rows for distinct draws")
    if count * 4 < n_total:
        out: List[int] = []
        seen = set()
        while len(out) < count:
            for v in rng.integers(0, n_total, size=count - len(out)):
                v = int(v)
                if v not in seen:
                    seen.add(v)
                    out.append(v)
        return np.array(out, dtype=np.int64)
    return rng.permutation(n_total)[:count].astype(np.int64)


def poisson_arrivals(n: int, rate_per_s: float, seed: int) -> np.ndarray:
    """Seeded Poisson arrival times (seconds) for n requests at the given rate."""
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence(seed)))
    return np.cumsum(rng.exponential(1.0 / rate_per_s, size=n))


def pack_ids(reqs: List[Request]) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
    """Concatenate requests as [prefix_0, cands_0, prefix_1, cands_1, ...].

    Returns (ids int32 [sum(L+K*m)], prefix_len int32 [C], n_cand int32 [C]).
    This is the id layout the library's device entry point consumes (with
    each request's m passed alongside when it is not 1).
    """
    ids = np.concatenate([np.concatenate([r.prefix, r.cands]) for r in reqs]).astype(np.int32)
    return ids, np.array([r.L for r in reqs], np.int32), np.array([r.K for r in reqs], np.int32)
