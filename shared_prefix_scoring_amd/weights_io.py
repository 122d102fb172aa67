"""Writer of the ranker weights file read by ``duolm_load_ranker``.

Format (little-endian): a 64-byte header -- magic ``DUOLMW01``, int32
n_layers, d_model, n_heads, n_kv_heads, head_dim, d_ffn, vocab, float32
rms_eps, rope_base, 20 reserved bytes -- then the tensors in the order of
:func:`tensor_order`, each starting at a 64-byte aligned offset.  Matrices are
bf16 bit patterns in [out_features, in_features] layout; RMSNorm gains and the
head vector are float32.
"""
from __future__ import annotations

import struct
from typing import Dict, List, Tuple

import numpy as np

MAGIC = b"DUOLMW01"


def tensor_order(cfg) -> List[Tuple[str, Tuple[int, ...], type]]:
    d, hq, hk, hd, f = cfg.d_model, cfg.n_heads, cfg.n_kv_heads, cfg.head_dim, cfg.d_ffn
    out = [("embed", (cfg.vocab, d), np.uint16)]
    for l in range(cfg.n_layers):
        p = f"layers.{l}."
        out += [
            (p + "attn_norm", (d,), np.float32),
            (p + "wq", (hq * hd, d), np.uint16),
            (p + "wk", (hk * hd, d), np.uint16),
            (p + "wv", (hk * hd, d), np.uint16),
            (p + "q_norm", (hd,), np.float32),
            (p + "k_norm", (hd,), np.float32),
            (p + "wo", (d, hq * hd), np.uint16),
            (p + "mlp_norm", (d,), np.float32),
            (p + "w_gate", (f, d), np.uint16),
            (p + "w_up", (f, d), np.uint16),
            (p + "w_down", (d, f), np.uint16),
        ]
    out += [("final_norm", (d,), np.float32), ("head", (d,), np.float32)]
    return out


def _header(cfg) -> bytes:
    h = MAGIC + struct.pack("<7i2f", cfg.n_layers, cfg.d_model, cfg.n_heads, cfg.n_kv_heads, cfg.head_dim,
                            cfg.d_ffn, cfg.vocab, cfg.rms_eps, cfg.rope_base)
    return h + b"\0" * (64 - len(h))


def weights_blob(cfg, tensors: Dict[str, np.ndarray]) -> np.ndarray:
    """The file's bytes as a uint8 array (for duolm_load_ranker_mem)."""
    order = tensor_order(cfg)
    off = 64
    spans = []
    for name, shape, dt in order:
        off = (off + 63) // 64 * 64
        a = np.ascontiguousarray(tensors[name])
        if a.shape != shape or a.dtype != dt:
            raise ValueError(f"{name}: expected {shape} {np.dtype(dt)}, got {a.shape} {a.dtype}")
        spans.append((off, a))
        off += a.nbytes
    blob = np.zeros(off, dtype=np.uint8)
    blob[:64] = np.frombuffer(_header(cfg), dtype=np.uint8)
    for o, a in spans:
        blob[o:o + a.nbytes] = a.reshape(-1).view(np.uint8)
    return blob


def write_weights(path: str, cfg, tensors: Dict[str, np.ndarray]) -> None:
    weights_blob(cfg, tensors).tofile(path)
