"""The C host packer (duolm_packed_size / duolm_pack_requests) against the
input-assembly oracle, bit for bit, on the CPU: the packer does no GPU work.
Also: every thread count gives the same output, and malformed requests are
rejected before anything is written."""
import numpy as np
import pytest

import synth
import shared_prefix_scoring_amd as spa
from oracle.packing import assemble_prefix, pack_batch


def pack_input(reqs, marker, instr, header=()):
    hist = [(r.items, r.feedback, r.cands, r.m, r.m) for r in reqs]
    return spa.PackInput(instr, marker, hist, header)


def expected(reqs, marker, instr, header=()):
    return pack_batch([(assemble_prefix(instr, marker, r.items, r.feedback, header), r.cands, r.m) for r in reqs])


@pytest.mark.parametrize("cid,cfg,n", [(1, synth.TINY, 1), (3, synth.QWEN3_0P6B, 200), (6, synth.QWEN3_0P6B, 64),
                                       (5, synth.QWEN3_0P6B, 2)])
def test_packer_matches_oracle(cid, cfg, n):
    reqs = synth.make_requests(cid, cfg, n_requests=n)
    marker, instr = synth.template(cid, cfg)
    for header in ((), (5, 6, 7)):
        p = pack_input(reqs, marker, instr, header)
        want = expected(reqs, marker, instr, header)
        assert spa.duolm_packed_size(p) == want[0].size
        for nt in (0, 1, 3, 8, 64):
            got = spa.duolm_pack_requests(p, n_threads=nt)
            for g, w in zip(got, want):
                np.testing.assert_array_equal(g, w)


def test_packer_many_threads_large_batch():
    # enough ids (about 2.4M) that the work cap allows many threads
    cfg = synth.QWEN3_0P6B
    reqs = synth.make_requests(3, cfg, n_requests=10_000)
    marker, instr = synth.template(3, cfg)
    p = pack_input(reqs, marker, instr)
    want = expected(reqs, marker, instr)
    for nt in (1, 7, 64):
        for g, w in zip(spa.duolm_pack_requests(p, n_threads=nt), want):
            np.testing.assert_array_equal(g, w)


def test_packer_edge_shapes():
    # no history, empty feedback, multi-vector history with single-vector candidates
    reqs = [synth.Request(prefix=None, cands=np.array([900, 901], np.int32), m=1,
                          items=np.zeros((0, 1), np.int32), feedback=[]),
            synth.Request(prefix=None, cands=np.array([902, 903, 904, 905], np.int32), m=2,
                          items=np.array([[800, 801]], np.int32), feedback=[np.zeros(0, np.int32)])]
    hist = [(reqs[0].items, reqs[0].feedback, reqs[0].cands, 1, 1),
            (reqs[1].items, reqs[1].feedback, reqs[1].cands, 2, 2),
            (np.array([[810, 811, 812]], np.int32), [np.array([1, 2], np.int32)], np.array([906], np.int32), 3, 0)]
    p = spa.PackInput([4], 9, hist)
    ids, L, K, M = spa.duolm_pack_requests(p, n_threads=2)
    assert ids.tolist() == [4, 900, 901, 4, 9, 800, 801, 902, 903, 904, 905, 4, 9, 810, 811, 812, 1, 2, 906]
    assert L.tolist() == [1, 4, 7] and K.tolist() == [2, 2, 1] and M.tolist() == [1, 2, 1]


def test_packer_errors():
    good = (np.array([[800]], np.int32), [np.array([1], np.int32)], np.array([900], np.int32), 1, 1)
    cases = [
        ([], 9, [(np.zeros((0, 1), np.int32), [], np.array([900], np.int32), 1, 1)]),  # empty prefix
        ([4], 9, [(good[0], good[1], np.zeros(0, np.int32), 1, 1)]),                   # no candidates
        ([4], 9, [(good[0], good[1], good[2], 1, 65)]),                                   # cand_len too large
        ([4], 9, [(good[0], good[1], good[2], -1, 1)]),                                   # item_len < 0
    ]
    for instr, marker, hist in cases:
        p = spa.PackInput(instr, marker, hist)
        with pytest.raises(spa.DuolmError) as ei:
            spa.duolm_packed_size(p)
        assert ei.value.code == -1
    # a decreasing feedback offset is caught before any output is written
    p = spa.PackInput([4], 9, [good])
    off = (np.array([0, 1], np.int32), np.array([1, 0], np.int32))
    p._keep.extend(off)
    p.reqs[0].feedback_off = off[1].ctypes.data
    buf = np.full(16, -7, np.int32)
    with pytest.raises(spa.DuolmError):
        spa.duolm_pack_requests(p, ids=buf)
    assert np.all(buf == -7)
    # too small an output buffer
    p = spa.PackInput([4], 9, [good])
    with pytest.raises(spa.DuolmError):
        spa.duolm_pack_requests(p, ids=np.empty(2, np.int32))
