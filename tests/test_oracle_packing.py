"""Pins of the input-assembly oracle (oracle/packing.py): the ranker input is
the instruction, then per history item (marker, item vector ids, feedback
ids), then the candidate header, then the candidates ("DuoLM은 아이템 벡터
재사용과 공유 프리픽스로 LLM 추천 서빙을 가속한다", 어떻게 동작하나 and
어떻게 쓰나).  Expected arrays are written out by hand."""
import numpy as np

import synth
from oracle.packing import assemble_prefix, pack_batch


def test_hand_worked_prefix():
    got = assemble_prefix([1, 2], 9, [[100], [101, 102]], [[5], []], cand_header=[7])
    assert got.tolist() == [1, 2, 9, 100, 5, 9, 101, 102, 7]
    # no history: instruction then header
    assert assemble_prefix([1, 2], 9, [], [], [3]).tolist() == [1, 2, 3]
    # no instruction
    assert assemble_prefix([], 9, [[50]], [[4, 4]]).tolist() == [9, 50, 4, 4]


def test_prefix_length_formula():
    rng = np.random.default_rng(0)
    for _ in range(20):
        n, m = int(rng.integers(0, 6)), int(rng.integers(1, 4))
        fb = [list(rng.integers(0, 50, size=int(rng.integers(0, 5)))) for _ in range(n)]
        items = [list(rng.integers(1000, 2000, size=m)) for _ in range(n)]
        ni, nh = int(rng.integers(0, 4)), int(rng.integers(0, 3))
        p = assemble_prefix(list(range(ni)), 9, items, fb, list(range(nh)))
        assert len(p) == ni + sum(1 + m + len(f) for f in fb) + nh
        # every marker is followed by that item's m vector ids
        pos = ni
        for it, f in zip(items, fb):
            assert p[pos] == 9 and p[pos + 1:pos + 1 + m].tolist() == it
            pos += 1 + m + len(f)


def test_pack_batch_hand_worked():
    ids, L, K, M = pack_batch([(np.array([1, 2]), np.array([10, 11, 12]), 1),
                               (np.array([3]), np.array([20, 21, 22, 23]), 2)])
    assert ids.tolist() == [1, 2, 10, 11, 12, 3, 20, 21, 22, 23]
    assert L.tolist() == [2, 1] and K.tolist() == [3, 2] and M.tolist() == [1, 2]


def test_synthetic_requests_follow_the_template():
    for cid, cfg in ((1, synth.TINY), (3, synth.QWEN3_0P6B), (6, synth.QWEN3_0P6B)):
        marker, instr = synth.template(cid, cfg)
        for r in synth.make_requests(cid, cfg, n_requests=20):
            assert np.array_equal(assemble_prefix(instr, marker, r.items, r.feedback), r.prefix)
