"""The entry point that allocates nothing (duolm_score_batch_dev_noalloc)
against duolm_score_batch_dev, through the C ABI: two calls in a row, the
second smaller, in MIS and independent mode and with candidates of m ids; a
call over the scratch limit and a call with an out-of-range id are refused
and leave the output untouched."""
import numpy as np
import pytest
import torch

import synth
import shared_prefix_scoring_amd as spa

pytestmark = pytest.mark.gpu


def _dev(reqs):
    ids, L, K = synth.pack_ids(reqs)
    return torch.from_numpy(ids).cuda(), L, K


def _both(r, reqs, mode=0, cand_len=None):
    d_ids, L, K = _dev(reqs)
    n = int(K.sum())
    ref = torch.full((n,), -7.0, device="cuda")
    got = torch.full((n,), -9.0, device="cuda")
    r.score_dev(L, K, d_ids.data_ptr(), ref.data_ptr(), mode=mode, cand_len=cand_len)
    r.score_dev_noalloc(L, K, d_ids.data_ptr(), got.data_ptr(), mode=mode, cand_len=cand_len)
    return got.cpu().numpy(), ref.cpu().numpy()


def test_noalloc_matches_device_entry_point(gpu_qwen):
    cfg, _, _, _, r = gpu_qwen
    big = synth.make_requests(3, cfg, n_requests=12)   # ~4,000 rows
    assert 3000 < sum(q.L + q.K for q in big) < 4600
    small = synth.make_requests(4, cfg, n_requests=3)  # the rating shape: a few hundred rows
    for reqs in (big, small):  # the second call is smaller and reuses the scratch
        got, ref = _both(r, reqs)
        assert np.all(np.isfinite(got))
        np.testing.assert_array_equal(got, ref)
    # independent scoring (one sequence per candidate) and candidates of m ids
    got, ref = _both(r, synth.make_requests(2, cfg, n_requests=1, n_cand=6), mode=spa.DUOLM_MODE_INDEPENDENT)
    np.testing.assert_array_equal(got, ref)
    mv = synth.make_requests(6, cfg, n_requests=2)
    got, ref = _both(r, mv, cand_len=8)
    np.testing.assert_array_equal(got, ref)


def test_noalloc_tiny_and_refusals(gpu_tiny, gpu_qwen):
    tcfg, _, _, _, rt = gpu_tiny
    got, ref = _both(rt, synth.make_requests(1, tcfg))
    np.testing.assert_array_equal(got, ref)
    cfg, _, _, _, r = gpu_qwen
    # over the scratch limit: EINVAL, nothing written
    d_ids, L, K = _dev(synth.make_requests(3, cfg, n_requests=40))
    out = torch.full((int(K.sum()),), -7.0, device="cuda")
    with pytest.raises(spa.DuolmError) as e:
        r.score_dev_noalloc(L, K, d_ids.data_ptr(), out.data_ptr())
    assert e.value.status == "EINVAL"
    assert torch.all(out == -7.0)
    # an out-of-range id: ERANGE, nothing written
    ids, L, K = synth.pack_ids(synth.make_requests(4, cfg, n_requests=2))
    ids[5] = cfg.vocab + cfg.n_vid
    d_bad = torch.from_numpy(ids).cuda()
    out = torch.full((int(K.sum()),), -7.0, device="cuda")
    with pytest.raises(spa.DuolmError) as e:
        r.score_dev_noalloc(L, K, d_bad.data_ptr(), out.data_ptr())
    assert e.value.status == "ERANGE"
    assert torch.all(out == -7.0)
    # and a good call right after works
    got, ref = _both(r, synth.make_requests(4, cfg, n_requests=2))
    np.testing.assert_array_equal(got, ref)
