"""ctypes binding of libduolm.so: one Python function per C entry point, same
names, argument marshalling only.  All computation happens in the library's
HIP kernels; there is no fallback path.  A missing library raises."""
from __future__ import annotations

import ctypes as C
import os
import weakref
from typing import Iterable, Optional, Sequence, Tuple

import numpy as np

try:  # torch's HIP runtime must be loaded first so the library binds to the same one
    import torch  # noqa: F401
except ImportError:  # pragma: no cover - torch is part of the image
    torch = None

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "lib", "libduolm.so")

DUOLM_MODE_MIS = 0
DUOLM_MODE_INDEPENDENT = 1

KERNEL_CLASSES = ["embed", "rmsnorm", "gemm_qkv", "qk_rope", "attn_prefix", "attn_branch", "gemm_o",
                  "gemm_gateup", "gemm_down", "head"]

STAGES = {"attn_norm": 0, "qkv": 1, "qk_rope": 2, "attn": 3, "attn_resid": 4, "mlp_norm": 5, "swiglu": 6,
          "layer_out": 7, "embed": 8}

EPILOGUES = {"bf16": 0, "resid": 1, "swiglu": 2}

STATUS = {0: "OK", -1: "EINVAL", -2: "ERANGE", -3: "ENOMEM", -4: "EHIP", -5: "EIO", -6: "ESTATE"}


class DuolmError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"{STATUS.get(code, code)}: {msg}")
        self.code = code
        self.status = STATUS.get(code, str(code))


class duolm_dims(C.Structure):
    _fields_ = [("n_layers", C.c_int32), ("d_model", C.c_int32), ("n_heads", C.c_int32),
                ("n_kv_heads", C.c_int32), ("head_dim", C.c_int32), ("d_ffn", C.c_int32), ("vocab", C.c_int32),
                ("rms_eps", C.c_float), ("rope_base", C.c_float), ("n_vid", C.c_int64),
                ("max_prefix", C.c_int32), ("max_rows", C.c_int32)]


class duolm_request(C.Structure):
    _fields_ = [("ids", C.POINTER(C.c_int32)), ("prefix_len", C.c_int32),
                ("cand_ids", C.POINTER(C.c_int32)), ("n_cand", C.c_int32),
                ("inline_vecs", C.c_void_p), ("cand_len", C.c_int32)]


class duolm_opts(C.Structure):
    _fields_ = [("mode", C.c_int32), ("use_graph", C.c_int32), ("hip_stream", C.c_void_p),
                ("max_lanes", C.c_int32), ("reserved", C.c_int32)]


class duolm_template(C.Structure):
    _fields_ = [("instruction", C.c_void_p), ("n_instruction", C.c_int32), ("marker", C.c_int32),
                ("cand_header", C.c_void_p), ("n_cand_header", C.c_int32)]


class duolm_history(C.Structure):
    _fields_ = [("n_items", C.c_int32), ("item_len", C.c_int32), ("item_vids", C.c_void_p),
                ("feedback", C.c_void_p), ("feedback_off", C.c_void_p), ("cand_vids", C.c_void_p),
                ("n_cand", C.c_int32), ("cand_len", C.c_int32)]


class duolm_kernel_stats(C.Structure):
    _fields_ = [("launches", C.c_int64), ("total_ms", C.c_double), ("flops", C.c_double), ("bytes", C.c_double)]


_lib = None

EXPORTS = {
    "duolm_load_ranker": (C.c_int, [C.c_char_p, C.c_int, C.POINTER(C.c_void_p)]),
    "duolm_load_ranker_mem": (C.c_int, [C.c_void_p, C.c_uint64, C.c_int, C.POINTER(C.c_void_p)]),
    "duolm_load_vid_table": (C.c_int, [C.c_void_p, C.c_void_p, C.c_int64]),
    "duolm_get_dims": (C.c_int, [C.c_void_p, C.POINTER(duolm_dims)]),
    "duolm_score_batch": (C.c_int, [C.c_void_p, C.POINTER(duolm_request), C.c_int32, C.c_void_p,
                                    C.POINTER(duolm_opts)]),
    "duolm_score_batch_dev": (C.c_int, [C.c_void_p, C.c_void_p, C.c_void_p, C.c_void_p, C.c_int32, C.c_void_p,
                                        C.c_void_p, C.POINTER(duolm_opts)]),
    "duolm_score_batch_dev_noalloc": (C.c_int, [C.c_void_p, C.c_void_p, C.c_void_p, C.c_void_p, C.c_int32, C.c_void_p,
                                        C.c_void_p, C.POINTER(duolm_opts)]),
    "duolm_set_profiling": (C.c_int, [C.c_void_p, C.c_uint32]),
    "duolm_get_kernel_stats": (C.c_int, [C.c_void_p, C.c_int32, C.POINTER(duolm_kernel_stats)]),
    "duolm_last_error": (C.c_char_p, []),
    "duolm_free_ranker": (None, [C.c_void_p]),
    "duolm_debug_forward": (C.c_int, [C.c_void_p, C.POINTER(duolm_request), C.c_int32, C.c_int32, C.c_int32,
                                      C.c_int32, C.c_void_p, C.c_uint64]),
    "duolm_debug_gemm": (C.c_int, [C.c_int32, C.c_void_p, C.c_void_p, C.c_void_p, C.c_int32, C.c_int32,
                                   C.c_int32, C.c_void_p]),
    "duolm_copy_device": (C.c_int, [C.c_void_p, C.c_void_p, C.c_uint64, C.c_void_p]),
    "duolm_export_item_vectors": (C.c_int, [C.c_void_p, C.c_int32, C.c_int64, C.c_int32, C.c_double, C.c_double,
                                            C.c_double, C.c_void_p, C.c_void_p]),
    "duolm_export_vid_table": (C.c_int, [C.c_void_p, C.c_void_p, C.c_int32, C.c_int64, C.c_double, C.c_double,
                                         C.c_double]),
    "duolm_reference_scale": (C.c_int, [C.c_void_p, C.POINTER(C.c_double)]),
    "duolm_packed_size": (C.c_int, [C.POINTER(duolm_template), C.POINTER(duolm_history), C.c_int32,
                                    C.POINTER(C.c_int64)]),
    "duolm_pack_requests": (C.c_int, [C.POINTER(duolm_template), C.POINTER(duolm_history), C.c_int32, C.c_int32,
                                      C.c_void_p, C.c_int64, C.c_void_p, C.c_void_p, C.c_void_p]),
    "duolm_score_packed": (C.c_int, [C.c_void_p, C.c_void_p, C.c_void_p, C.c_void_p, C.c_int32, C.c_void_p,
                                     C.c_void_p, C.POINTER(duolm_opts)]),
    "duolm_kv_pool_init": (C.c_int, [C.c_void_p, C.c_int64]),
    "duolm_kv_pool_free_pages": (C.c_int, [C.c_void_p, C.POINTER(C.c_int64)]),
    "duolm_session_create": (C.c_int, [C.c_void_p, C.POINTER(C.c_void_p)]),
    "duolm_session_length": (C.c_int, [C.c_void_p, C.POINTER(C.c_int32)]),
    "duolm_session_free": (None, [C.c_void_p]),
    "duolm_session_step": (C.c_int, [C.c_void_p, C.c_void_p, C.c_int32, C.c_void_p, C.c_void_p, C.c_void_p,
                                     C.c_void_p, C.c_void_p, C.POINTER(duolm_opts)]),
}

DUOLM_DTYPE_F32, DUOLM_DTYPE_BF16, DUOLM_DTYPE_F16 = 0, 1, 2


def lib() -> C.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it first (python -m shared_prefix_scoring_amd.build)")
        L = C.CDLL(LIB_PATH, mode=C.RTLD_GLOBAL)
        for name, (res, args) in EXPORTS.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
    return _lib


def _check(rc: int) -> None:
    if rc != 0:
        raise DuolmError(rc, lib().duolm_last_error().decode())


def _i32(a) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(a, dtype=np.int32))


def _cand_lens(n: int, cand_len) -> np.ndarray:
    """Ids per candidate for each of n requests: None (1), one int, or a sequence."""
    if cand_len is None:
        return np.ones(n, dtype=np.int32)
    if np.isscalar(cand_len):
        return np.full(n, int(cand_len), dtype=np.int32)
    m = _i32(cand_len)
    if m.shape != (n,):
        raise ValueError("cand_len must have one entry per request")
    return m


def _requests(reqs: Sequence[Tuple], cand_len=None):
    """Requests as (prefix_ids, cand_ids) or (prefix_ids, cand_ids, inline_vecs),
    inline_vecs an fp16-bits array [number of ids >= V, d_model].  cand_len:
    ids per candidate (None, one int, or one per request); cand_ids then holds
    n_cand * cand_len ids, candidate-major."""
    keep = []
    arr = (duolm_request * len(reqs))()
    ms = _cand_lens(len(reqs), cand_len)
    for i, req in enumerate(reqs):
        p, c = _i32(req[0]), _i32(req[1])
        m = max(int(ms[i]), 1)
        if c.shape[0] % m:
            raise ValueError(f"request {i}: {c.shape[0]} candidate ids is not a multiple of cand_len {m}")
        keep += [p, c]
        arr[i].ids = p.ctypes.data_as(C.POINTER(C.c_int32))
        arr[i].prefix_len = p.shape[0]
        arr[i].cand_ids = c.ctypes.data_as(C.POINTER(C.c_int32))
        arr[i].n_cand = c.shape[0] // m
        arr[i].cand_len = int(ms[i])
        if len(req) > 2 and req[2] is not None:
            v = np.ascontiguousarray(req[2], dtype=np.uint16)
            keep.append(v)
            arr[i].inline_vecs = v.ctypes.data
        else:
            arr[i].inline_vecs = None
    return arr, keep


def _opts(mode: int, use_graph: bool, stream, max_lanes: int = 0) -> duolm_opts:
    return duolm_opts(int(mode), 1 if use_graph else 0, C.c_void_p(stream or 0), int(max_lanes), 0)


# ----------------------------------------------------------------- entry points

def duolm_load_ranker(path: str, hip_device: int = 0) -> C.c_void_p:
    h = C.c_void_p()
    _check(lib().duolm_load_ranker(path.encode(), hip_device, C.byref(h)))
    return h


def duolm_load_ranker_mem(blob: np.ndarray, hip_device: int = 0) -> C.c_void_p:
    b = np.ascontiguousarray(blob, dtype=np.uint8)
    h = C.c_void_p()
    _check(lib().duolm_load_ranker_mem(b.ctypes.data, b.nbytes, hip_device, C.byref(h)))
    return h


def duolm_load_vid_table(r, rows_fp16: np.ndarray) -> None:
    rows = np.ascontiguousarray(rows_fp16, dtype=np.uint16)
    if rows.ndim != 2:
        raise ValueError("rows must be [n_rows, d_model]")
    _check(lib().duolm_load_vid_table(r, rows.ctypes.data, rows.shape[0]))


def duolm_get_dims(r) -> duolm_dims:
    d = duolm_dims()
    _check(lib().duolm_get_dims(r, C.byref(d)))
    return d


def duolm_score_batch(r, reqs, mode: int = DUOLM_MODE_MIS, use_graph: bool = True, stream=None,
                      cand_len=None, max_lanes: int = 0) -> np.ndarray:
    arr, keep = _requests(reqs, cand_len)
    n = sum(int(arr[i].n_cand) for i in range(len(reqs)))
    out = np.empty(n, dtype=np.float32)
    o = _opts(mode, use_graph, stream, max_lanes)
    _check(lib().duolm_score_batch(r, arr, len(reqs), out.ctypes.data, C.byref(o)))
    del keep
    return out


def duolm_score_batch_dev(r, prefix_len, n_cand, d_ids: int, d_scores: int, mode: int = DUOLM_MODE_MIS,
                          use_graph: bool = True, stream=None, cand_len=None, max_lanes: int = 0) -> None:
    L, K = _i32(prefix_len), _i32(n_cand)
    M = None if cand_len is None else _cand_lens(L.shape[0], cand_len)
    o = _opts(mode, use_graph, stream, max_lanes)
    _check(lib().duolm_score_batch_dev(r, L.ctypes.data, K.ctypes.data, None if M is None else M.ctypes.data,
                                       L.shape[0], C.c_void_p(d_ids), C.c_void_p(d_scores), C.byref(o)))


def duolm_score_batch_dev_noalloc(r, prefix_len, n_cand, d_ids: int, d_scores: int, mode: int = DUOLM_MODE_MIS,
                                  stream=None, cand_len=None) -> None:
    L, K = _i32(prefix_len), _i32(n_cand)
    M = None if cand_len is None else _cand_lens(L.shape[0], cand_len)
    o = _opts(mode, False, stream, 1)
    _check(lib().duolm_score_batch_dev_noalloc(r, L.ctypes.data, K.ctypes.data, None if M is None else M.ctypes.data,
                                               L.shape[0], C.c_void_p(d_ids), C.c_void_p(d_scores), C.byref(o)))


def duolm_set_profiling(r, class_mask: int) -> None:
    _check(lib().duolm_set_profiling(r, class_mask))


def duolm_get_kernel_stats(r, kernel_class: int) -> duolm_kernel_stats:
    s = duolm_kernel_stats()
    _check(lib().duolm_get_kernel_stats(r, kernel_class, C.byref(s)))
    return s


def duolm_last_error() -> str:
    return lib().duolm_last_error().decode()


def duolm_free_ranker(r) -> None:
    lib().duolm_free_ranker(r)


def duolm_debug_forward(r, reqs, layer: int, stage: int, out: np.ndarray, mode: int = DUOLM_MODE_MIS,
                        cand_len=None) -> np.ndarray:
    arr, keep = _requests(reqs, cand_len)
    _check(lib().duolm_debug_forward(r, arr, len(reqs), mode, layer, stage, out.ctypes.data, out.nbytes))
    del keep
    return out


def duolm_debug_gemm(epilogue: int, d_A: int, d_W: int, d_C: int, M: int, N: int, K: int, stream=None) -> None:
    _check(lib().duolm_debug_gemm(epilogue, C.c_void_p(d_A), C.c_void_p(d_W), C.c_void_p(d_C), M, N, K,
                                  C.c_void_p(stream or 0)))


def duolm_copy_device(d_dst: int, d_src: int, nbytes: int, stream=None) -> None:
    _check(lib().duolm_copy_device(C.c_void_p(d_dst), C.c_void_p(d_src), nbytes, C.c_void_p(stream or 0)))


def duolm_export_item_vectors(d_a: int, a_dtype: int, n_rows: int, d: int, rho: float, gamma: float, eps: float,
                              d_z: int, stream=None) -> None:
    _check(lib().duolm_export_item_vectors(C.c_void_p(d_a), a_dtype, n_rows, d, rho, gamma, eps, C.c_void_p(d_z),
                                           C.c_void_p(stream or 0)))


def duolm_export_vid_table(r, d_a: int, a_dtype: int, n_rows: int, rho: float, gamma: float, eps: float) -> None:
    _check(lib().duolm_export_vid_table(r, C.c_void_p(d_a), a_dtype, n_rows, rho, gamma, eps))


def duolm_reference_scale(r) -> float:
    v = C.c_double()
    _check(lib().duolm_reference_scale(r, C.byref(v)))
    return v.value


class PackInput:
    """Structured requests marshalled for the packer: keeps the arrays alive.

    instruction, cand_header: id sequences shared by the batch; marker: id.
    histories: per request (item_vids [n_items, m_item] or [n_items*m_item],
    feedbacks: list of id arrays, one per item, cand_vids [K*m_cand],
    item_len, cand_len)."""

    def __init__(self, instruction, marker: int, histories, cand_header=()):
        self._keep = []
        ins = self._arr(instruction)
        hdr = self._arr(cand_header)
        self.tpl = duolm_template(ins.ctypes.data if ins.size else None, ins.size, int(marker),
                                  hdr.ctypes.data if hdr.size else None, hdr.size)
        self.reqs = (duolm_history * len(histories))()
        for i, (vids, fbs, cands, item_len, cand_len) in enumerate(histories):
            v = self._arr(vids)
            fb = self._arr(np.concatenate([np.asarray(f, np.int32) for f in fbs]) if len(fbs) else [])
            fo = self._arr(np.concatenate([[0], np.cumsum([len(f) for f in fbs])]) if len(fbs) else [0])
            c = self._arr(cands)
            self.reqs[i] = duolm_history(len(fbs), int(item_len), v.ctypes.data if v.size else None,
                                         fb.ctypes.data if fb.size else None, fo.ctypes.data, c.ctypes.data,
                                         c.size // max(int(cand_len), 1), int(cand_len))
        self.n = len(histories)

    def _arr(self, a):
        a = np.ascontiguousarray(np.asarray(a, dtype=np.int32).reshape(-1))
        self._keep.append(a)
        return a


def _slice(p: PackInput, start: int, count):
    count = p.n - start if count is None else count
    if start < 0 or count < 1 or start + count > p.n:
        raise ValueError("request range out of bounds")
    ptr = C.cast(C.addressof(p.reqs) + start * C.sizeof(duolm_history), C.POINTER(duolm_history))
    return ptr, count


def duolm_packed_size(p: PackInput, start: int = 0, count: int | None = None) -> int:
    ptr, count = _slice(p, start, count)
    n = C.c_int64()
    _check(lib().duolm_packed_size(C.byref(p.tpl), ptr, count, C.byref(n)))
    return n.value


def duolm_pack_requests(p: PackInput, n_threads: int = 1, ids: np.ndarray | None = None, start: int = 0,
                        count: int | None = None):
    """Pack requests start .. start+count-1 of p.  Returns (ids, prefix_len,
    n_cand, cand_len) as int32 arrays; `ids` may be a caller buffer of at least
    the packed size (the returned ids are then a view of its first part)."""
    ptr, count = _slice(p, start, count)
    if ids is None:
        ids = np.empty(duolm_packed_size(p, start, count), dtype=np.int32)
    L, K, M = (np.empty(count, dtype=np.int32) for _ in range(3))
    _check(lib().duolm_pack_requests(C.byref(p.tpl), ptr, count, n_threads, ids.ctypes.data, ids.size,
                                     L.ctypes.data, K.ctypes.data, M.ctypes.data))
    return ids[:int(L.sum()) + int((K * M).sum())], L, K, M


def duolm_score_packed(r, prefix_len, n_cand, cand_len, ids, mode: int = DUOLM_MODE_MIS, use_graph: bool = True,
                       stream=None, max_lanes: int = 0) -> np.ndarray:
    L, K = _i32(prefix_len), _i32(n_cand)
    M = None if cand_len is None else _i32(cand_len)
    ids = np.ascontiguousarray(ids, dtype=np.int32)
    out = np.empty(int(K.sum()), dtype=np.float32)
    o = _opts(mode, use_graph, stream, max_lanes)
    _check(lib().duolm_score_packed(r, L.ctypes.data, K.ctypes.data, None if M is None else M.ctypes.data,
                                    L.shape[0], ids.ctypes.data, out.ctypes.data, C.byref(o)))
    return out


def duolm_kv_pool_init(r, max_rows: int) -> None:
    _check(lib().duolm_kv_pool_init(r, max_rows))


def duolm_kv_pool_free_pages(r) -> int:
    n = C.c_int64()
    _check(lib().duolm_kv_pool_free_pages(r, C.byref(n)))
    return n.value


def duolm_session_create(r) -> C.c_void_p:
    h = C.c_void_p()
    _check(lib().duolm_session_create(r, C.byref(h)))
    return h


def duolm_session_length(s) -> int:
    n = C.c_int32()
    _check(lib().duolm_session_length(s, C.byref(n)))
    return n.value


def duolm_session_free(s) -> None:
    lib().duolm_session_free(s)


def duolm_session_step(r, sessions, new_ids, cands=None, cand_len=None, mode: int = DUOLM_MODE_MIS,
                       use_graph: bool = True, stream=None, max_lanes: int = 0) -> np.ndarray:
    """sessions: handles; new_ids[i]: ids appended to session i (may be empty);
    cands[i]: its candidate ids (empty or None: none), cand_len as in score()."""
    n = len(sessions)
    cands = [None] * n if cands is None else cands
    M = _cand_lens(n, cand_len)
    m = np.maximum(M, 1)
    new = [np.asarray(x if x is not None else [], dtype=np.int32).reshape(-1) for x in new_ids]
    cc = [np.asarray(x if x is not None else [], dtype=np.int32).reshape(-1) for x in cands]
    n_new = np.array([x.size for x in new], dtype=np.int32)
    n_cand = np.array([c.size // mi for c, mi in zip(cc, m)], dtype=np.int32)
    parts = [a for pair in zip(new, cc) for a in pair]
    ids = np.ascontiguousarray(np.concatenate(parts) if parts else np.zeros(0, np.int32), dtype=np.int32)
    hs = (C.c_void_p * n)(*[s.value if isinstance(s, C.c_void_p) else s for s in sessions])
    out = np.empty(int(n_cand.sum()), dtype=np.float32)
    o = _opts(mode, use_graph, stream, max_lanes)
    _check(lib().duolm_session_step(r, hs, n, n_new.ctypes.data, n_cand.ctypes.data,
                                    None if cand_len is None else M.ctypes.data,
                                    ids.ctypes.data if ids.size else None, out.ctypes.data if out.size else None,
                                    C.byref(o)))
    return out


# ----------------------------------------------------------------- convenience

class Session:
    """Owning wrapper around a session handle (freed with close() or with its ranker)."""

    def __init__(self, ranker: "Ranker"):
        self.ranker = ranker
        self.h = duolm_session_create(ranker.h)
        ranker._sessions.add(self)

    @property
    def length(self) -> int:
        return duolm_session_length(self.h)

    def close(self) -> None:
        if self.h:
            duolm_session_free(self.h)
            self.h = None
            self.ranker._sessions.discard(self)


class Ranker:
    """Owning wrapper around a ranker handle."""

    def __init__(self, handle):
        self.h = handle
        self.dims = duolm_get_dims(handle)
        self._sessions = weakref.WeakSet()

    @classmethod
    def from_file(cls, path: str, device: int = 0) -> "Ranker":
        return cls(duolm_load_ranker(path, device))

    @classmethod
    def from_blob(cls, blob: np.ndarray, device: int = 0) -> "Ranker":
        return cls(duolm_load_ranker_mem(blob, device))

    def load_vid_table(self, rows_fp16: np.ndarray) -> None:
        duolm_load_vid_table(self.h, rows_fp16)
        self.dims = duolm_get_dims(self.h)

    def export_vid_table(self, d_a: int, a_dtype: int, n_rows: int, rho: float, gamma: float = 0.0,
                         eps: float = 0.0) -> None:
        duolm_export_vid_table(self.h, d_a, a_dtype, n_rows, rho, gamma, eps)
        self.dims = duolm_get_dims(self.h)

    def reference_scale(self) -> float:
        return duolm_reference_scale(self.h)

    def score(self, reqs, mode: int = DUOLM_MODE_MIS, use_graph: bool = True, stream=None,
              cand_len=None, max_lanes: int = 0) -> np.ndarray:
        return duolm_score_batch(self.h, reqs, mode, use_graph, stream, cand_len, max_lanes)

    def score_packed(self, prefix_len, n_cand, cand_len, ids, mode: int = DUOLM_MODE_MIS,
                     use_graph: bool = True, stream=None, max_lanes: int = 0) -> np.ndarray:
        return duolm_score_packed(self.h, prefix_len, n_cand, cand_len, ids, mode, use_graph, stream, max_lanes)

    def score_dev(self, prefix_len, n_cand, d_ids: int, d_scores: int, mode: int = DUOLM_MODE_MIS,
                  use_graph: bool = True, stream=None, cand_len=None, max_lanes: int = 0) -> None:
        duolm_score_batch_dev(self.h, prefix_len, n_cand, d_ids, d_scores, mode, use_graph, stream, cand_len,
                              max_lanes)

    def score_dev_noalloc(self, prefix_len, n_cand, d_ids: int, d_scores: int, mode: int = DUOLM_MODE_MIS,
                          stream=None, cand_len=None) -> None:
        duolm_score_batch_dev_noalloc(self.h, prefix_len, n_cand, d_ids, d_scores, mode, stream, cand_len)

    def stage(self, reqs, layer: int, stage: str, mode: int = DUOLM_MODE_MIS, cand_len=None) -> np.ndarray:
        d = self.dims
        ms = [max(int(m), 1) for m in _cand_lens(len(reqs), cand_len)]
        if mode == DUOLM_MODE_MIS:
            T = sum(len(r[0]) + len(r[1]) for r in reqs)
        else:
            T = sum((len(r[0]) + m) * (len(r[1]) // m) for r, m in zip(reqs, ms))
        width, dt = {
            "attn_norm": (d.d_model, np.uint16), "mlp_norm": (d.d_model, np.uint16),
            "qkv": ((d.n_heads + 2 * d.n_kv_heads) * d.head_dim, np.uint16),
            "qk_rope": ((d.n_heads + 2 * d.n_kv_heads) * d.head_dim, np.uint16),
            "attn": (d.n_heads * d.head_dim, np.uint16), "swiglu": (d.d_ffn, np.uint16),
        }.get(stage, (d.d_model, np.float32))
        out = np.empty((T, width), dtype=dt)
        return duolm_debug_forward(self.h, reqs, layer, STAGES[stage], out, mode, cand_len)

    def set_profiling(self, classes: Iterable[str]) -> None:
        mask = 0
        for c in classes:
            mask |= 1 << KERNEL_CLASSES.index(c)
        duolm_set_profiling(self.h, mask)

    def kernel_stats(self, cls: str) -> duolm_kernel_stats:
        return duolm_get_kernel_stats(self.h, KERNEL_CLASSES.index(cls))

    def kv_pool_init(self, max_rows: int) -> None:
        duolm_kv_pool_init(self.h, max_rows)

    def kv_free_pages(self) -> int:
        return duolm_kv_pool_free_pages(self.h)

    def session(self) -> Session:
        return Session(self)

    def step(self, sessions, new_ids, cands=None, cand_len=None, use_graph: bool = True, stream=None,
             mode: int = DUOLM_MODE_MIS, max_lanes: int = 0) -> np.ndarray:
        return duolm_session_step(self.h, [x.h for x in sessions], new_ids, cands, cand_len, mode, use_graph,
                                  stream, max_lanes)

    def close(self) -> None:
        if self.h:
            for x in list(self._sessions):  # the library frees them with the ranker
                x.h = None
            self._sessions = weakref.WeakSet()
            duolm_free_ranker(self.h)
            self.h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass
