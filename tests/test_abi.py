"""Host-only checks of the C ABI: the library loads, exports every function the
public headers declare, and rejects malformed inputs before touching a GPU."""
import os
import re

import numpy as np
import pytest

import synth
from shared_prefix_scoring_amd import _lib, weights_blob, write_weights

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_functions():
    names = set()
    for h in os.listdir(os.path.join(ROOT, "include")):
        if h.endswith(".h"):
            text = open(os.path.join(ROOT, "include", h)).read()
            text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
            names |= set(re.findall(r"\b(duolm_[a-z_0-9]+)\s*\(", text))
    return names


def test_library_exports_every_declared_function():
    lib = _lib.lib()
    names = declared_functions()
    assert {"duolm_load_ranker", "duolm_load_vid_table", "duolm_score_batch"} <= names
    for n in names:
        assert hasattr(lib, n), n
    assert names == set(_lib.EXPORTS), names ^ set(_lib.EXPORTS)


def test_missing_file_is_eio(tmp_path):
    with pytest.raises(_lib.DuolmError) as e:
        _lib.duolm_load_ranker(str(tmp_path / "nope.bin"))
    assert e.value.status == "EIO"


def test_bad_magic_and_short_blob(tmp_path):
    cfg = synth.TINY
    blob = weights_blob(cfg, synth.make_weights(cfg))
    bad = blob.copy()
    bad[:8] = np.frombuffer(b"NOTDUOLM", dtype=np.uint8)
    with pytest.raises(_lib.DuolmError) as e:
        _lib.duolm_load_ranker_mem(bad)
    assert e.value.status == "EIO"
    with pytest.raises(_lib.DuolmError) as e:
        _lib.duolm_load_ranker_mem(blob[: blob.size // 2])
    assert e.value.status == "EIO"
    p = tmp_path / "short.bin"
    blob[:100].tofile(p)
    with pytest.raises(_lib.DuolmError) as e:
        _lib.duolm_load_ranker(str(p))
    assert e.value.status == "EIO"


def test_unsupported_dims_rejected():
    import dataclasses
    for bad in (dict(head_dim=48), dict(n_kv_heads=3), dict(n_kv_heads=4), dict(d_ffn=100)):
        cfg = dataclasses.replace(synth.TINY, **bad)
        try:
            w = synth.make_weights(cfg)
        except Exception:
            continue
        with pytest.raises(_lib.DuolmError) as e:
            _lib.duolm_load_ranker_mem(weights_blob(cfg, w))
        assert e.value.status == "EINVAL"


def test_weights_file_layout(tmp_path):
    cfg = synth.TINY
    w = synth.make_weights(cfg)
    p = tmp_path / "w.bin"
    write_weights(str(p), cfg, w)
    raw = np.fromfile(p, dtype=np.uint8)
    assert bytes(raw[:8]) == b"DUOLMW01"
    hdr = raw[8:44].view(np.int32)[:7]
    assert list(hdr) == [cfg.n_layers, cfg.d_model, cfg.n_heads, cfg.n_kv_heads, cfg.head_dim, cfg.d_ffn,
                         cfg.vocab]
    # first tensor (embedding) starts at byte 64, last (head) ends the file
    np.testing.assert_array_equal(raw[64:64 + 16].view(np.uint16), w["embed"].reshape(-1)[:8])
    np.testing.assert_array_equal(raw[-cfg.d_model * 4:].view(np.float32), w["head"])


def test_null_handle_errors():
    with pytest.raises(_lib.DuolmError) as e:
        _lib.duolm_get_dims(None)
    assert e.value.status == "EINVAL"
    with pytest.raises(_lib.DuolmError) as e:
        _lib.duolm_set_profiling(None, 1)
    assert e.value.status == "EINVAL"
