"""Sessions: a prefix's K and V kept on the GPU between calls, new history rows
appended without recomputing the old ones (in-session incremental
personalisation, "DuoLM: Fast and Effective Personalized Recommendation with
Language Models", 未来方向 (3)).  With causal attention the old rows do not
depend on the new ones, so by definition a session's scores are those of its
whole prefix scored in one call.  The GPU session path is checked against the
GPU one-call path bit for bit, and against the float64 oracle of the whole
prefix within the score tolerance."""
import numpy as np
import pytest

import synth
import shared_prefix_scoring_amd as spa
from oracle import oracle_mis
from parity import SCORE_TOL, score_err

pytestmark = pytest.mark.gpu


def chunks(prefix, cuts):
    out, o = [], 0
    for c in list(cuts) + [len(prefix)]:
        out.append(prefix[o:c])
        o = c
    return [x for x in out if len(x)]


def test_tiny_session_equals_one_call(gpu_tiny):
    cfg, _, _, model, r = gpu_tiny
    r.kv_pool_init(4096)
    q = synth.make_requests(1, cfg)[0]
    s = r.session()
    try:
        got_len = 0
        for part in chunks(q.prefix, [20, 21]):  # 20, 1 and 27 rows
            scores = r.step([s], [part], [q.cands])
            got_len += len(part)
            assert s.length == got_len
            want = r.score([(q.prefix[:got_len], q.cands)])
            np.testing.assert_array_equal(scores, want)
        ref = oracle_mis(model, q.prefix, q.cands)
        assert score_err(scores, ref) <= SCORE_TOL
        # score-only calls leave the session as it is; graph and eager agree
        again = r.step([s], [[]], [q.cands], use_graph=False)
        np.testing.assert_array_equal(again, scores)
        assert s.length == len(q.prefix)
    finally:
        s.close()


@pytest.mark.parametrize("cid,n", [(3, 6), (6, 4)])
def test_batched_sessions_across_pages(gpu_qwen, cid, n):
    # several users at once, prefixes appended in uneven chunks that straddle
    # the 64-row pages and the 256-row attention tiles; candidates of m rows
    # for the m = 8 workload; every step checked against one-call scoring
    cfg, _, _, model, r = gpu_qwen
    r.kv_pool_init(64 * 1024)
    reqs = synth.make_requests(cid, cfg, n_requests=n)
    rng = np.random.default_rng(cid)
    parts = []
    for q in reqs:
        cuts = sorted(set(int(x) for x in rng.integers(1, q.L, size=3)))
        parts.append(chunks(q.prefix, cuts))
    sess = [r.session() for _ in reqs]
    try:
        done = [0] * n
        for step in range(max(len(p) for p in parts)):
            new = [p[step] if step < len(p) else np.zeros(0, np.int32) for p in parts]
            got = r.step(sess, new, [q.cands for q in reqs], cand_len=[q.m for q in reqs])
            done = [d + len(x) for d, x in zip(done, new)]
            want = r.score([(q.prefix[:d], q.cands) for q, d in zip(reqs, done)], cand_len=[q.m for q in reqs])
            np.testing.assert_array_equal(got, want)
        assert [x.length for x in sess] == [q.L for q in reqs]
        q = reqs[0]
        ref = oracle_mis(model, q.prefix, q.cands, m=q.m)
        assert score_err(got[:q.K], ref) <= SCORE_TOL
    finally:
        for x in sess:
            x.close()


def test_page_aligned_appends(gpu_tiny):
    # appends that end exactly on 64-row page boundaries, then one row into a
    # fresh page; every step's scores equal one-call scoring of the prefix so far
    cfg, _, _, _, r = gpu_tiny
    r.kv_pool_init(64 * 16)
    q = synth.make_requests(1, cfg)[0]
    prefix = np.resize(q.prefix, 129).astype(np.int32)
    s = r.session()
    try:
        done = 0
        for part in chunks(prefix, [64, 128]):  # 64, 64 and 1 rows
            got = r.step([s], [part], [q.cands])
            done += len(part)
            assert s.length == done
            np.testing.assert_array_equal(got, r.score([(prefix[:done], q.cands)]))
        assert r.kv_free_pages() == 16 - 3
    finally:
        s.close()


def test_mixed_step_and_pool_accounting(gpu_tiny):
    cfg, _, _, model, r = gpu_tiny
    r.kv_pool_init(10 * 64)
    assert r.kv_free_pages() == 10
    reqs = synth.make_requests(1, cfg, n_requests=3, seed=40)
    a, b, c = (r.session() for _ in range(3))
    try:
        # a appends only, b appends and scores, c does nothing yet
        out = r.step([a, b], [reqs[0].prefix, reqs[1].prefix], [None, reqs[1].cands])
        np.testing.assert_array_equal(out, r.score([(reqs[1].prefix, reqs[1].cands)]))
        assert r.kv_free_pages() == 10 - 2  # 48 rows each: one page
        # a scores only, c appends and scores, in one call
        out = r.step([a, c], [[], reqs[2].prefix], [reqs[0].cands, reqs[2].cands])
        np.testing.assert_array_equal(out, r.score([(reqs[0].prefix, reqs[0].cands),
                                                    (reqs[2].prefix, reqs[2].cands)]))
        # growth past a page boundary takes one more page
        r.step([a], [reqs[0].prefix[:20]])
        assert a.length == 68 and r.kv_free_pages() == 10 - 4
        # an append that does not fit the pool fails and changes nothing
        big = np.tile(reqs[0].prefix, 20)
        with pytest.raises(spa.DuolmError) as ei:
            r.step([b], [big], [reqs[1].cands])
        assert ei.value.code == -3 and b.length == 48 and r.kv_free_pages() == 6
        # freeing returns the pages
        c.close()
        assert r.kv_free_pages() == 7
    finally:
        for x in (a, b, c):
            x.close()
    assert r.kv_free_pages() == 10


def test_session_errors(gpu_tiny, tiny):
    cfg, w, D, _, r = gpu_tiny
    r.kv_pool_init(1024)
    q = synth.make_requests(1, cfg)[0]
    s = r.session()
    try:
        with pytest.raises(spa.DuolmError) as ei:  # candidates with an empty prefix
            r.step([s], [[]], [q.cands])
        assert ei.value.code == -1
        with pytest.raises(spa.DuolmError):  # the same session twice
            r.step([s, s], [q.prefix[:3], q.prefix[3:6]])
        with pytest.raises(spa.DuolmError):  # independent mode
            r.step([s], [q.prefix], [q.cands], mode=spa.DUOLM_MODE_INDEPENDENT)
        with pytest.raises(spa.DuolmError) as ei:  # an id out of range
            bad = q.prefix.copy()
            bad[2] = cfg.vocab + cfg.n_vid
            r.step([s], [bad], [q.cands])
        assert ei.value.code == -2 and s.length == 0
        with pytest.raises(spa.DuolmError) as ei:  # the pool cannot be replaced under live sessions
            r.kv_pool_init(2048)
        assert ei.value.code == -6
        with pytest.raises(spa.DuolmError):  # nothing to compute
            r.step([s], [[]])
    finally:
        s.close()
    # a ranker without a pool has no sessions
    r2 = spa.Ranker.from_blob(spa.weights_blob(cfg, w))
    try:
        with pytest.raises(spa.DuolmError) as ei:
            r2.session()
        assert ei.value.code == -6
    finally:
        r2.close()


def test_pool_allocation_failure_leaves_ranker_usable(gpu_tiny):
    # A pool larger than any device (2^26 pages of 32 KB: 2 TiB) fails in the
    # device allocation itself: ENOMEM, and the ranker keeps its old pool and
    # scores as before (a failed allocation must not leave HIP's last error
    # behind for the next call's launch check to report).
    cfg, _, _, _, r = gpu_tiny
    q = synth.make_requests(1, cfg)[0]
    want = r.score([(q.prefix, q.cands)])
    r.kv_pool_init(4096)
    with pytest.raises(spa.DuolmError) as ei:
        r.kv_pool_init(64 << 26)
    assert ei.value.code == -3 and "KV pool" in str(ei.value)
    assert r.kv_free_pages() == 64
    np.testing.assert_array_equal(r.score([(q.prefix, q.cands)]), want)
    np.testing.assert_array_equal(r.score([(q.prefix, q.cands)], use_graph=False), want)
    s = r.session()
    try:
        np.testing.assert_array_equal(r.step([s], [q.prefix], [q.cands]), want)
    finally:
        s.close()
    assert r.kv_free_pages() == 64


def test_sessions_in_two_lanes_equal_one(gpu_qwen):
    # a step over many users runs as two concurrent halves; one launch gives
    # the same bits
    cfg, _, _, _, r = gpu_qwen
    r.kv_pool_init(64 * 512)
    reqs = synth.make_requests(3, cfg, n_requests=12, seed=90)
    a = [r.session() for _ in reqs]
    b = [r.session() for _ in reqs]
    try:
        got_a = r.step(a, [q.prefix for q in reqs], [q.cands for q in reqs])
        got_b = r.step(b, [q.prefix for q in reqs], [q.cands for q in reqs], max_lanes=1)
        np.testing.assert_array_equal(got_a, got_b)
    finally:
        for x in a + b:
            x.close()
