"""Shared fixtures.  GPU tests are marked ``gpu``; everything else runs on the CPU."""
import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU")
    config.addinivalue_line("markers", "slow: CPU test that takes more than ~10 s")


@pytest.fixture(scope="session")
def tiny():
    import synth
    from oracle import OracleModel
    cfg = synth.TINY
    w = synth.make_weights(cfg, seed=0)
    D = synth.make_vid_table(cfg)
    return cfg, w, D, OracleModel.from_arrays(cfg, w, D)


@pytest.fixture(scope="session")
def tiny_gains():
    """Tiny model whose RMSNorm gains are 1 + N(0, 0.1^2), so a dropped gain shows."""
    import synth
    from oracle import OracleModel
    cfg = synth.TINY
    w = synth.make_weights(cfg, seed=5, gain_sigma=0.1)
    D = synth.make_vid_table(cfg, seed=6)
    return cfg, w, D, OracleModel.from_arrays(cfg, w, D)


def oracle_item_table(cfg, w, a):
    """The oracle's item table: its own float64 export of the encoder outputs a
    (row by row, so exporting in chunks changes nothing), with rho the RMS of
    the token embedding."""
    import numpy as np
    import synth
    from oracle import export_table, reference_scale, widen_bf16
    rho = reference_scale(widen_bf16(w["embed"]))
    D = np.empty(a.shape, np.uint16)
    for i in range(0, a.shape[0], 16384):
        D[i:i + 16384] = export_table(a[i:i + 16384], rho, synth.TABLE_GAMMA, synth.TABLE_EPS)
    return D


@pytest.fixture(scope="session")
def qwen_table_inputs():
    import synth
    return synth.table_encoder_outputs(synth.QWEN3_0P6B)


@pytest.fixture(scope="session")
def qwen(qwen_table_inputs):
    import synth
    from oracle import OracleModel
    cfg = synth.QWEN3_0P6B
    w = synth.make_weights(cfg, seed=0)
    D = oracle_item_table(cfg, w, qwen_table_inputs)
    return cfg, w, D, OracleModel.from_arrays(cfg, w, D)


@pytest.fixture(scope="session")
def gpu_tiny(tiny):
    import shared_prefix_scoring_amd as spa
    cfg, w, D, model = tiny
    r = spa.Ranker.from_blob(spa.weights_blob(cfg, w))
    r.load_vid_table(D)
    yield cfg, w, D, model, r
    r.close()


@pytest.fixture(scope="session")
def gpu_tiny_gains(tiny_gains):
    import shared_prefix_scoring_amd as spa
    cfg, w, D, model = tiny_gains
    r = spa.Ranker.from_blob(spa.weights_blob(cfg, w))
    r.load_vid_table(D)
    yield cfg, w, D, model, r
    r.close()


def export_gpu_item_table(r, a):
    """Fill ranker r's item table through the library's own export entry point
    (encoder outputs on the device, rho from the library's reference scale)."""
    import torch
    import synth
    import shared_prefix_scoring_amd as spa
    da = torch.from_numpy(a).cuda()
    r.export_vid_table(da.data_ptr(), spa.DUOLM_DTYPE_F32, a.shape[0], r.reference_scale(), synth.TABLE_GAMMA,
                       synth.TABLE_EPS)
    del da
    torch.cuda.empty_cache()


@pytest.fixture(scope="session")
def gpu_qwen(qwen, qwen_table_inputs):
    import shared_prefix_scoring_amd as spa
    cfg, w, D, model = qwen
    r = spa.Ranker.from_blob(spa.weights_blob(cfg, w))
    export_gpu_item_table(r, qwen_table_inputs)
    yield cfg, w, D, model, r
    r.close()
