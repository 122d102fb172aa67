"""Float64 NumPy oracle of the DuoLM ranker forward with multi-item scoring.

TEST INFRASTRUCTURE ONLY (see the package docstring): the product path never
imports this module.

Citation keys used below (page title, then the section):
  [digest]   "DuoLM: Fast and Effective Personalized Recommendation with
             Language Models" (paper.rainbus.top structured digest)
  [onedev]   "DuoLM은 아이템 벡터 재사용과 공유 프리픽스로 LLM 추천 서빙을
             가속한다" (onedev.kr digest)
  [mindverse] "DuoLM verlagert Teile der Empfehlung in die Offline-Verarbeitung"

What is computed.  For a request with prefix ids p_0..p_{L-1} and candidate ids
c_1..c_K the score of candidate j is defined by independent scoring: append c_j
alone to the prefix, run the causal decoder over the L+1 positions 0..L and
read the last row through the shared linear head, s = w^T h ([digest] 核心方法;
[onedev] 어떻게 동작하나).  MIS computes the same numbers in one pass: the K
candidates are packed after the prefix, every candidate sits at logical
position L, and a tree mask lets candidate j see the prefix and itself only
([digest] 核心方法 third innovation and 方法步骤详情 step 4; [mindverse]
"Gemeinsame Nutzerhistorie, getrennte Kandidatenzweige").  In exact arithmetic
the two agree ([digest] 研究动机, the identity s^MIS_{q,j} = s_{q,j}); the
number of prefix query-key pairs MIS drops per layer is (K-1)L(L+1)/2 (same
section).

The decoder is the Qwen3-0.6B backbone named in [digest] 核心方法 and 复现评估.
The pages do not spell out its internals; the readings taken here are:
pre-norm RMSNorm blocks with eps 1e-6, per-head RMSNorm on q and k before the
rotary embedding, rotate-half rotary embedding with inverse frequencies
base^(-2i/hd), attention scale 1/sqrt(hd), query head h reading KV head
h // (H / H_kv), SwiGLU MLP, no projection biases, a final RMSNorm before the
head, and a head vector w with no bias.
"""
from __future__ import annotations

import dataclasses
from typing import Dict, List, Sequence

import numpy as np

F64 = np.float64


# ----------------------------------------------------------------------------
# storage widening (exact)
# ----------------------------------------------------------------------------


def widen_bf16(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns (uint16) -> float64, exactly."""
    u32 = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return u32.view(np.float32).astype(F64)


def widen_f16(bits: np.ndarray) -> np.ndarray:
    """fp16 bit patterns (uint16) -> float64, exactly."""
    return np.asarray(bits, dtype=np.uint16).view(np.float16).astype(F64)


# ----------------------------------------------------------------------------
# model container
# ----------------------------------------------------------------------------


@dataclasses.dataclass
class OracleModel:
    cfg: object                      # has n_layers, d_model, n_heads, ... rope_base
    layers: List[Dict[str, np.ndarray]]
    embed_bits: np.ndarray           # uint16 bf16 [V, d]
    vid_bits: np.ndarray | None      # uint16 fp16 [N, d]
    final_norm: np.ndarray
    head: np.ndarray

    @classmethod
    def from_arrays(cls, cfg, weights: Dict[str, np.ndarray], vid_table: np.ndarray | None):
        def mat(name):
            return widen_bf16(weights[name])

        def vec(name):
            return np.asarray(weights[name], dtype=F64)

        layers = []
        for l in range(cfg.n_layers):
            p = f"layers.{l}."
            layers.append({
                "attn_norm": vec(p + "attn_norm"),
                "wq": mat(p + "wq"), "wk": mat(p + "wk"), "wv": mat(p + "wv"),
                "q_norm": vec(p + "q_norm"), "k_norm": vec(p + "k_norm"),
                "wo": mat(p + "wo"),
                "mlp_norm": vec(p + "mlp_norm"),
                "w_gate": mat(p + "w_gate"), "w_up": mat(p + "w_up"), "w_down": mat(p + "w_down"),
            })
        return cls(cfg=cfg, layers=layers, embed_bits=np.asarray(weights["embed"]),
                   vid_bits=None if vid_table is None else np.asarray(vid_table),
                   final_norm=vec("final_norm"), head=vec("head"))


# ----------------------------------------------------------------------------
# building blocks
# ----------------------------------------------------------------------------


def embed_rows(model: OracleModel, ids: Sequence[int]) -> np.ndarray:
    """Extended-vocabulary lookup: id < V reads the token embedding row; V <= id < V+N
    reads row id-V of the FP16 item table ([digest] 方法步骤详情 step 3; [onedev]
    어떻게 쓰나).  Any other id is an error."""
    V = model.cfg.vocab
    ids = np.asarray(ids, dtype=np.int64)
    n_vid = 0 if model.vid_bits is None else model.vid_bits.shape[0]
    if np.any(ids < 0) or np.any(ids >= V + n_vid):
        raise ValueError("id outside [0, V+N)")
    out = np.empty((ids.shape[0], model.cfg.d_model), dtype=F64)
    tok = ids < V
    if np.any(tok):
        out[tok] = widen_bf16(model.embed_bits[ids[tok]])
    if np.any(~tok):
        out[~tok] = widen_f16(model.vid_bits[ids[~tok] - V])
    return out


def rmsnorm(x: np.ndarray, g: np.ndarray, eps: float) -> np.ndarray:
    """x / sqrt(mean(x^2) + eps) * g over the last axis."""
    ms = np.mean(x * x, axis=-1, keepdims=True)
    return x / np.sqrt(ms + eps) * g


def rope_rotate(x: np.ndarray, pos: np.ndarray, base: float) -> np.ndarray:
    """Rotary embedding, rotate-half layout, on x [n, heads, hd] at positions pos [n].

    Dimension pair (i, i + hd/2) is rotated counter-clockwise by pos * base^(-2i/hd).
    """
    hd = x.shape[-1]
    half = hd // 2
    i = np.arange(half, dtype=F64)
    inv_freq = np.power(F64(base), -2.0 * i / hd)
    ang = np.asarray(pos, dtype=F64)[:, None] * inv_freq[None, :]       # [n, half]
    c = np.cos(ang)[:, None, :]
    s = np.sin(ang)[:, None, :]
    x1, x2 = x[..., :half], x[..., half:]
    return np.concatenate([x1 * c - x2 * s, x2 * c + x1 * s], axis=-1)


def attention(q: np.ndarray, k: np.ndarray, v: np.ndarray, allowed: np.ndarray) -> np.ndarray:
    """Masked softmax attention with grouped KV heads.

    q [n, H, hd], k and v [m, H_kv, hd], allowed [n, m] (True = query may see key).
    Query head h uses KV head h // (H / H_kv).  Scores are q.k / sqrt(hd); masked
    keys get probability 0.
    """
    n, H, hd = q.shape
    Hkv = k.shape[1]
    group = H // Hkv
    out = np.empty_like(q)
    for h in range(H):
        kv = h // group
        s = q[:, h, :] @ k[:, kv, :].T / np.sqrt(F64(hd))
        s = np.where(allowed, s, -np.inf)
        s = s - np.max(s, axis=1, keepdims=True)
        p = np.exp(s)
        p = p / np.sum(p, axis=1, keepdims=True)
        out[:, h, :] = p @ v[:, kv, :]
    return out


def mlp_swiglu(b: np.ndarray, w_gate: np.ndarray, w_up: np.ndarray, w_down: np.ndarray) -> np.ndarray:
    """(silu(b W_gate^T) * (b W_up^T)) W_down^T, silu(g) = g / (1 + exp(-g))."""
    g = b @ w_gate.T
    u = b @ w_up.T
    return ((g / (1.0 + np.exp(-g))) * u) @ w_down.T


def layer_stages(model: OracleModel, layer: int, x: np.ndarray, pos: np.ndarray,
                 allowed: np.ndarray) -> Dict[str, np.ndarray]:
    """One pre-norm decoder layer, returning every intermediate for stage checks."""
    cfg = model.cfg
    W = model.layers[layer]
    n = x.shape[0]
    H, Hkv, hd, eps = cfg.n_heads, cfg.n_kv_heads, cfg.head_dim, cfg.rms_eps
    st: Dict[str, np.ndarray] = {"x_in": x}
    a = rmsnorm(x, W["attn_norm"], eps)
    st["a"] = a
    q = (a @ W["wq"].T).reshape(n, H, hd)
    k = (a @ W["wk"].T).reshape(n, Hkv, hd)
    v = (a @ W["wv"].T).reshape(n, Hkv, hd)
    st["q_proj"], st["k_proj"], st["v"] = q, k, v
    q = rmsnorm(q, W["q_norm"], eps)
    k = rmsnorm(k, W["k_norm"], eps)
    st["q_normed"], st["k_normed"] = q, k
    q = rope_rotate(q, pos, cfg.rope_base)
    k = rope_rotate(k, pos, cfg.rope_base)
    st["q"], st["k"] = q, k
    o = attention(q, k, v, allowed).reshape(n, H * hd)
    st["o"] = o
    x = x + o @ W["wo"].T
    st["x_mid"] = x
    b = rmsnorm(x, W["mlp_norm"], eps)
    st["b"] = b
    g = b @ W["w_gate"].T
    u = b @ W["w_up"].T
    st["h"] = (g / (1.0 + np.exp(-g))) * u
    x = x + mlp_swiglu(b, W["w_gate"], W["w_up"], W["w_down"])
    st["x_out"] = x
    return st


def decoder_forward(model: OracleModel, x: np.ndarray, pos: np.ndarray, allowed: np.ndarray) -> np.ndarray:
    """All decoder layers over rows x [n, d] with an explicit visibility mask."""
    for l in range(model.cfg.n_layers):
        x = layer_stages(model, l, x, pos, allowed)["x_out"]
    return x


def score_head(model: OracleModel, h: np.ndarray) -> np.ndarray:
    """s = w^T RMSNorm_final(h) per row: the shared linear head, no bias ([digest] 核心方法)."""
    return rmsnorm(h, model.final_norm, model.cfg.rms_eps) @ model.head


# ----------------------------------------------------------------------------
# MIS: tree mask, unified positions, packed scoring
# ----------------------------------------------------------------------------


def tree_mask(L: int, K: int, m: int = 1) -> np.ndarray:
    """Visibility over [prefix (L rows); K candidate branches of m rows each].

    Prefix row t sees prefix rows 0..t.  Row i of candidate branch j sees the
    whole prefix and rows 0..i of its own branch, never another candidate
    ([digest] 核心方法; [mindverse] "Gemeinsame Nutzerhistorie, getrennte
    Kandidatenzweige").  m = 1 is the one-vector item of the pages' main
    setting; m > 1 is an item spread over m vectors (the pages' FIR m = 8
    rating service, [digest] 实验结果; [digest] 未来方向 (2)), read here as a
    causal branch.
    """
    n = L + K * m
    allowed = np.zeros((n, n), dtype=bool)
    for t in range(L):
        allowed[t, : t + 1] = True
    for j in range(K):
        b = L + j * m
        for i in range(m):
            allowed[b + i, :L] = True
            allowed[b + i, b:b + i + 1] = True
    return allowed


def mis_positions(L: int, K: int, m: int = 1) -> np.ndarray:
    """Prefix rows at 0..L-1; row i of every candidate branch at logical
    position L + i, where a lone candidate appended to the prefix would sit
    ([digest] 方法步骤详情 step 4)."""
    return np.concatenate([np.arange(L), np.tile(L + np.arange(m), K)]).astype(np.int64)


def oracle_mis(model: OracleModel, prefix: Sequence[int], cands: Sequence[int],
               pos_offset: int = 0, m: int = 1) -> np.ndarray:
    """Scores of the K candidates, in input order, from one packed MIS forward.

    `cands` holds K*m ids, candidate-major; a candidate is scored at the last
    row of its branch ([digest] 核心方法: the last hidden state)."""
    prefix = np.asarray(prefix, dtype=np.int64)
    cands = np.asarray(cands, dtype=np.int64)
    L = prefix.shape[0]
    if L < 1 or m < 1 or cands.shape[0] < m or cands.shape[0] % m:
        raise ValueError("need L >= 1, m >= 1 and K*m candidate ids with K >= 1")
    K = cands.shape[0] // m
    x = embed_rows(model, np.concatenate([prefix, cands]))
    pos = mis_positions(L, K, m) + pos_offset
    h = decoder_forward(model, x, pos, tree_mask(L, K, m))
    return score_head(model, h[L + m - 1::m])


def oracle_mis_packed(model: OracleModel, requests: Sequence[tuple]) -> List[np.ndarray]:
    """Several requests packed one after another in a single forward.

    A request is (prefix, cands) or (prefix, cands, m).  The mask is
    block-diagonal over requests (a request never sees another) with each
    block the request's tree mask; positions restart at 0 per request.
    """
    ids, pos, blocks, spans = [], [], [], []
    row = 0
    for req in requests:
        prefix = np.asarray(req[0], dtype=np.int64)
        cands = np.asarray(req[1], dtype=np.int64)
        m = req[2] if len(req) > 2 else 1
        L, K = prefix.shape[0], cands.shape[0] // m
        ids.append(np.concatenate([prefix, cands]))
        pos.append(mis_positions(L, K, m))
        blocks.append(tree_mask(L, K, m))
        spans.append((row + L + m - 1, row + L + K * m, m))
        row += L + K * m
    allowed = np.zeros((row, row), dtype=bool)
    r = 0
    for b in blocks:
        allowed[r:r + b.shape[0], r:r + b.shape[0]] = b
        r += b.shape[0]
    x = embed_rows(model, np.concatenate(ids))
    h = decoder_forward(model, x, np.concatenate(pos), allowed)
    return [score_head(model, h[a:b:m]) for a, b, m in spans]


def brute_force_independent(model: OracleModel, prefix: Sequence[int], cands: Sequence[int],
                            which: Sequence[int] | None = None, m: int = 1) -> np.ndarray:
    """The definition, literally: for each candidate, a full causal forward over
    [prefix; its m ids] at positions 0..L+m-1, scored at the last row.  `which`
    limits the candidates evaluated (all by default)."""
    prefix = np.asarray(prefix, dtype=np.int64)
    cands = np.asarray(cands, dtype=np.int64)
    L = prefix.shape[0]
    idx = range(cands.shape[0] // m) if which is None else which
    causal = np.tril(np.ones((L + m, L + m), dtype=bool))
    pos = np.arange(L + m)
    out = []
    for j in idx:
        x = embed_rows(model, np.concatenate([prefix, cands[j * m:(j + 1) * m]]))
        h = decoder_forward(model, x, pos, causal)
        out.append(score_head(model, h[-1:])[0])
    return np.array(out, dtype=F64)


def decode_incremental(model: OracleModel, ids: Sequence[int]) -> float:
    """Textbook causal-LM evaluation, one token at a time against a growing KV
    cache; returns the head score of the last token.  It never builds a mask."""
    cfg = model.cfg
    H, Hkv, hd, eps = cfg.n_heads, cfg.n_kv_heads, cfg.head_dim, cfg.rms_eps
    group = H // Hkv
    x_all = embed_rows(model, ids)
    caches = [([], []) for _ in range(cfg.n_layers)]
    h = None
    for t in range(x_all.shape[0]):
        x = x_all[t]
        for l, W in enumerate(model.layers):
            a = rmsnorm(x, W["attn_norm"], eps)
            q = rmsnorm((W["wq"] @ a).reshape(H, hd), W["q_norm"], eps)
            k = rmsnorm((W["wk"] @ a).reshape(Hkv, hd), W["k_norm"], eps)
            v = (W["wv"] @ a).reshape(Hkv, hd)
            q = rope_rotate(q[None], np.array([t]), cfg.rope_base)[0]
            k = rope_rotate(k[None], np.array([t]), cfg.rope_base)[0]
            caches[l][0].append(k)
            caches[l][1].append(v)
            K_ = np.stack(caches[l][0])          # [t+1, Hkv, hd]
            V_ = np.stack(caches[l][1])
            o = np.empty((H, hd))
            for hh in range(H):
                s = K_[:, hh // group, :] @ q[hh] / np.sqrt(F64(hd))
                p = np.exp(s - s.max())
                o[hh] = (p / p.sum()) @ V_[:, hh // group, :]
            x = x + W["wo"] @ o.reshape(-1)
            b = rmsnorm(x, W["mlp_norm"], eps)
            g = W["w_gate"] @ b
            x = x + W["w_down"] @ ((g / (1.0 + np.exp(-g))) * (W["w_up"] @ b))
        h = x
    return float(score_head(model, h[None])[0])


def pair_count(L: int, K: int, m: int = 1) -> Dict[str, int]:
    """Allowed (query, key) pairs per layer: MIS tree mask versus K independent
    causal sequences of L+m rows, counted from the masks themselves."""
    mis = int(tree_mask(L, K, m).sum())
    one = int(np.tril(np.ones((L + m, L + m), dtype=bool)).sum())
    return {"mis": mis, "independent": K * one, "eliminated": K * one - mis}
