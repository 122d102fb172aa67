"""GPU parity of the offline item-vector export and of the reference scale
(z = e^gamma * rho * a / RMS(a) stored as FP16; rho = RMS of the ranker's
native embeddings: "DuoLM: Fast and Effective Personalized Recommendation
with Language Models", 核心方法 and 方法步骤详情 step 3), called through the C
ABI and compared with the float64 oracle.

The FP16 codes must equal the oracle's exactly.  The only admitted difference
is an element whose exact value lies within 1e-12 (relative) of a binary16
rounding midpoint, where two accurate float64 evaluations may round apart; the
GPU must then still return one of the two neighbouring codes.
"""
import math

import numpy as np
import pytest
import torch

import synth
import shared_prefix_scoring_amd as spa
from shared_prefix_scoring_amd import _lib
from oracle import reference_scale, widen_bf16, widen_f16
from oracle.export import interface_vectors, midpoint_distance, to_fp16_bits

pytestmark = pytest.mark.gpu

KNIFE_EDGE = 1e-12


def to_dev(arr: np.ndarray) -> torch.Tensor:
    a = np.ascontiguousarray(arr)
    return torch.from_numpy(a.view(np.uint8).reshape(-1).copy()).cuda()


def run_export(a_host: np.ndarray, dtype: int, rho: float, gamma: float, eps: float, stream=None) -> np.ndarray:
    n, d = a_host.shape
    da = to_dev(a_host)
    dz = torch.empty(n * d * 2, dtype=torch.uint8, device="cuda")
    _lib.duolm_export_item_vectors(da.data_ptr(), dtype, n, d, rho, gamma, eps, dz.data_ptr(), stream)
    torch.cuda.synchronize()
    return dz.cpu().numpy().view(np.uint16).reshape(n, d)


def widen(a_host, dtype):
    if dtype == spa.DUOLM_DTYPE_F32:
        return a_host.astype(np.float64)
    return widen_bf16(a_host) if dtype == spa.DUOLM_DTYPE_BF16 else widen_f16(a_host)


def store(a32, dtype):
    if dtype == spa.DUOLM_DTYPE_F32:
        return a32
    return synth.f32_to_bf16_bits(a32) if dtype == spa.DUOLM_DTYPE_BF16 else synth.f32_to_f16_bits(a32)


def assert_codes(got: np.ndarray, z64: np.ndarray):
    want = to_fp16_bits(z64)
    bad = got != want
    n_edge = int(np.sum(midpoint_distance(z64) < KNIFE_EDGE))
    if bad.any():
        idx = np.argwhere(bad)[:5]
        edge = midpoint_distance(z64[bad]) < KNIFE_EDGE
        assert edge.all(), [(tuple(i), int(got[tuple(i)]), int(want[tuple(i)]), z64[tuple(i)]) for i in idx]
        assert np.all(np.abs(got[bad].astype(np.int32) - want[bad].astype(np.int32)) == 1)
    return int(bad.sum()), n_edge


DTYPES = [spa.DUOLM_DTYPE_F32, spa.DUOLM_DTYPE_BF16, spa.DUOLM_DTYPE_F16]


@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("n,d", [(1, 8), (5, 136), (1001, 1024), (37, 8192), (64, 520)])
def test_export_matches_oracle(dtype, n, d):
    # ragged: row counts off the 4-rows-per-workgroup grid, rows that fill
    # only part of the wave's chunks, the largest supported row
    a32 = synth.encoder_outputs(n, d, seed=100 + n + d)
    if dtype == spa.DUOLM_DTYPE_F16:
        a32 = a32 / np.float32(8.0)  # keep the fp16 storage of the synthetic outputs finite
    a = store(a32, dtype)
    rho, gamma, eps = 0.0211, -0.137, 1e-6
    got = run_export(a, dtype, rho, gamma, eps)
    bad, edge = assert_codes(got, interface_vectors(widen(a, dtype), rho, gamma, eps))
    print(f"n={n} d={d} dtype={dtype}: {bad} knife-edge differences of {edge} knife-edge elements")


def test_fp16_rounding_edges():
    # a row of eight 4.0 (or -4.0) has RMS 4 and exports to exactly +-rho
    # (every step exact in float64), so rho walks the binary16 rounding rule:
    # ties to even, subnormals, the overflow threshold, values near midpoints
    rng = np.random.default_rng(3)
    cells = rng.integers(1, 0x7BFF, size=400).astype(np.uint16).view(np.float16)
    v = cells.astype(np.float64)
    ulp = np.spacing(cells).astype(np.float64)
    vals = np.concatenate([v, v + ulp / 2, v + ulp / 2 + ulp * 2.0 ** -20, v + ulp / 2 - ulp * 2.0 ** -20, [
        1.0 + 2.0 ** -11, 1.0 + 3 * 2.0 ** -11, 65504.0, 65519.0, 65520.0, 65519.99, 70000.0, 2.0 ** -24,
        2.0 ** -25, 3 * 2.0 ** -25, 2.0 ** -25 * 1.0000001, 2.0 ** -26, 2.0 ** -14, 2.0 ** -14 - 2.0 ** -25,
        1e-30]])
    n = len(vals)
    dz = torch.empty(n * 16, dtype=torch.uint8, device="cuda")  # one 8-value fp16 row per value
    for sign in (1.0, -1.0):
        da = to_dev(np.full((1, 8), 4.0 * sign, dtype=np.float32))
        for i, x in enumerate(vals):  # the scale is per call: one call per value
            _lib.duolm_export_item_vectors(da.data_ptr(), spa.DUOLM_DTYPE_F32, 1, 8, float(x), 0.0, 0.0,
                                           dz.data_ptr() + 16 * i)
        torch.cuda.synchronize()
        got = dz.cpu().numpy().view(np.uint16).reshape(n, 8)
        want = to_fp16_bits(sign * vals)
        assert np.all(got == want[:, None]), vals[np.any(got != want[:, None], axis=1)][:5]


def test_zero_rows_and_eps():
    a = np.zeros((6, 64), dtype=np.float32)
    a[1] = 1.0
    a[2, 3] = -2.5
    for eps in (0.0, 1e-6, 3.0):
        got = run_export(a, spa.DUOLM_DTYPE_F32, 0.03, 0.2, eps)
        assert_codes(got, interface_vectors(a, 0.03, 0.2, eps))
        assert np.all(got[0] == 0) and np.all(got[3:] == 0)


def test_stream_and_repeat_determinism():
    a = synth.encoder_outputs(300, 1024, seed=9)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        got1 = run_export(a, spa.DUOLM_DTYPE_F32, 0.02, 0.0, 0.0, stream=s.cuda_stream)
    got2 = run_export(a, spa.DUOLM_DTYPE_F32, 0.02, 0.0, 0.0)
    np.testing.assert_array_equal(got1, got2)


def test_full_table_sampled():
    # the size the item table has at serving time (200,000 rows of 1024), fp32
    # encoder outputs, in the launch configuration the benchmark times:
    # sampled rows against the oracle, every row's RMS against the calibrated
    # scale (each FP16 rounding moves an element by at most 2^-11 relative,
    # or 2^-25 absolute in the subnormal range)
    n, d = 200_000, 1024
    a = synth.encoder_outputs(n, d, seed=11)
    rho, gamma, eps = 0.0198, 0.05, 1e-6
    got = run_export(a, spa.DUOLM_DTYPE_F32, rho, gamma, eps)
    rows = np.random.default_rng(4).choice(n, 2000, replace=False)
    assert_codes(got[rows], interface_vectors(a[rows], rho, gamma, eps))
    target = rho * math.exp(gamma)
    for i in range(0, n, 20000):
        blk = a[i:i + 20000].astype(np.float64)
        ms = np.mean(blk * blk, axis=1)
        want = target * np.sqrt(ms / (ms + eps))
        z = got[i:i + 20000].view(np.float16).astype(np.float64)
        have = np.sqrt(np.mean(z * z, axis=1))
        assert np.all(np.abs(have - want) <= 2.0 ** -11 * want + 2.0 ** -25), i


def test_export_errors():
    da = torch.zeros(4096, dtype=torch.uint8, device="cuda")
    dz = torch.zeros(4096, dtype=torch.uint8, device="cuda")
    ok = dict(d_a=da.data_ptr(), a_dtype=0, n_rows=2, d=64, rho=0.02, gamma=0.0, eps=0.0, d_z=dz.data_ptr())

    def call(**kw):
        args = dict(ok)
        args.update(kw)
        _lib.duolm_export_item_vectors(args["d_a"], args["a_dtype"], args["n_rows"], args["d"], args["rho"],
                                       args["gamma"], args["eps"], args["d_z"])

    call()
    call(n_rows=0, d_a=0, d_z=0)  # no-op
    host = np.zeros(1024, dtype=np.float32)
    for kw in [dict(d=60), dict(d=8200), dict(d=0), dict(a_dtype=3), dict(n_rows=-1), dict(eps=-1.0),
               dict(rho=float("nan")), dict(gamma=float("inf")), dict(d_a=0), dict(d_z=0),
               dict(d_a=host.ctypes.data), dict(d_z=da.data_ptr() + 4), dict(n_rows=1_000_000),
               dict(rho=1e300, gamma=100.0)]:
        with pytest.raises(spa.DuolmError) as ei:
            call(**kw)
        assert ei.value.code == -1, kw


def test_reference_scale_and_table_export(gpu_tiny, qwen):
    # rho from the ranker's own token embedding, against the oracle's RMS of
    # the widened bf16 table (float64 both sides: only summation order differs)
    cfg, w, _, _, r = gpu_tiny
    rho = r.reference_scale()
    assert rho == pytest.approx(reference_scale(widen_bf16(w["embed"])), rel=1e-12)
    assert r.reference_scale() == rho  # fixed-order reduction: same bits every call
    qcfg, qw, _, _ = qwen
    rq = spa.Ranker.from_blob(spa.weights_blob(qcfg, qw))
    try:
        assert rq.reference_scale() == pytest.approx(reference_scale(widen_bf16(qw["embed"])), rel=1e-12)
    finally:
        rq.close()

    # export the tiny ranker's item table from encoder outputs on the device,
    # then score: equal, bit for bit, to scoring with the oracle's exported
    # rows loaded from the host
    a = synth.encoder_outputs(cfg.n_vid, cfg.d_model, seed=21)
    want_rows = to_fp16_bits(interface_vectors(a, rho, 0.1, 1e-6))
    da = to_dev(a)
    r2 = spa.Ranker.from_blob(spa.weights_blob(cfg, w))
    r3 = spa.Ranker.from_blob(spa.weights_blob(cfg, w))
    try:
        r2.export_vid_table(da.data_ptr(), spa.DUOLM_DTYPE_F32, cfg.n_vid, rho, 0.1, 1e-6)
        assert r2.dims.n_vid == cfg.n_vid
        r3.load_vid_table(want_rows)
        reqs = [(q.prefix, q.cands) for q in synth.make_requests(1, cfg)]
        np.testing.assert_array_equal(r2.score(reqs), r3.score(reqs))
        with pytest.raises(spa.DuolmError):
            # far more rows than the input buffer's allocation holds
            r2.export_vid_table(da.data_ptr(), spa.DUOLM_DTYPE_F32, cfg.n_vid + 1_000_000, rho, 0.1, 1e-6)
        np.testing.assert_array_equal(r2.score(reqs), r3.score(reqs))  # failed export left the table alone
    finally:
        r2.close()
        r3.close()
