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


@pytest.fixture(scope="session")
def qwen():
    import synth
    from oracle import OracleModel
    cfg = synth.QWEN3_0P6B
    w = synth.make_weights(cfg, seed=0)
    D = synth.make_vid_table(cfg)
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


@pytest.fixture(scope="session")
def gpu_qwen(qwen):
    import shared_prefix_scoring_amd as spa
    cfg, w, D, model = qwen
    r = spa.Ranker.from_blob(spa.weights_blob(cfg, w))
    r.load_vid_table(D)
    yield cfg, w, D, model, r
    r.close()
