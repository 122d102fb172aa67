"""End-to-end parity of the GPU MIS forward with the float64 oracle, at the
workload shapes: tiny (L=48, K=8), one 0.6B request (L=452, K=100), a packed
64-request varlen batch (all 6,400 candidates against stored oracle scores),
the K=8 rating mix, and the L=4096 / K=512 stress shape (sampled candidates
against stored oracle scores and against GPU independent scoring).  Also: GPU MIS versus GPU
independent scoring, graph replay versus eager launch, determinism, batch
and permutation invariance, the error paths, and candidates spanning m rows
(items of m vectors) against the oracle's m-row branches."""
import json
import os

import numpy as np
import pytest
import torch

import synth
from oracle import oracle_mis
import shared_prefix_scoring_amd as spa
from parity import MIS_VS_IND_TOL, SCORE_TOL, score_err, top10_strict_swaps

pytestmark = pytest.mark.gpu

IND = spa.DUOLM_MODE_INDEPENDENT
GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def reqs_of(cfg, cid, n=None, **kw):
    return [(r.prefix, r.cands) for r in synth.make_requests(cid, cfg, n_requests=n, **kw)]


def split(scores, reqs):
    out, o = [], 0
    for _, c in reqs:
        out.append(scores[o:o + len(c)])
        o += len(c)
    return out


def check_against_oracle(model, reqs, gpu_scores, which=None):
    per = split(gpu_scores, reqs)
    errs, swaps = [], 0
    for i in (range(len(reqs)) if which is None else which):
        p, c = reqs[i]
        ref = oracle_mis(model, p, c)
        e = score_err(per[i], ref)
        errs.append(e)
        swaps += top10_strict_swaps(per[i], ref) > 0
        assert e <= SCORE_TOL, (i, e)
    print(f"max rel score err {max(errs):.3e}, requests with a strict top-10 swap: {swaps} of {len(errs)}")
    return max(errs)


@pytest.mark.parametrize("fixture", ["gpu_tiny", "gpu_tiny_gains"])
def test_tiny_workload(fixture, request):
    cfg, _, _, model, r = request.getfixturevalue(fixture)
    reqs = reqs_of(cfg, 1)
    for g in (False, True):
        check_against_oracle(model, reqs, r.score(reqs, use_graph=g))


def test_tiny_many_shapes(gpu_tiny):
    # ragged prefixes and candidate counts across tile boundaries, K up to 300
    cfg, _, _, model, r = gpu_tiny
    rng = np.random.default_rng(11)
    reqs = []
    for L, K in [(1, 1), (2, 3), (63, 1), (64, 129), (65, 128), (130, 7), (200, 300)]:
        reqs.append((rng.integers(0, cfg.vocab + cfg.n_vid, L).astype(np.int32),
                     (cfg.vocab + rng.choice(cfg.n_vid, K, replace=K > cfg.n_vid)).astype(np.int32)))
    check_against_oracle(model, reqs, r.score(reqs))


def test_qwen_single_request(gpu_qwen):
    cfg, _, _, model, r = gpu_qwen
    reqs = reqs_of(cfg, 2)
    assert len(reqs[0][0]) == 452 and len(reqs[0][1]) == 100
    check_against_oracle(model, reqs, r.score(reqs))


def golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def test_qwen_c64_batch_full_sweep(gpu_qwen):
    # every one of the 6,400 candidates of a 64-request headline batch against
    # the oracle's scores (written by tests/golden/make_golden.py from the
    # oracle alone), in the two-lane serving configuration
    cfg, _, _, model, r = gpu_qwen
    reqs = reqs_of(cfg, 3, n=64)
    g = golden("oracle_c64_batch.json")
    assert g["prefix_len"] == [len(p) for p, _ in reqs]
    s = r.score(reqs)
    assert s.shape[0] == 6400 and np.all(np.isfinite(s))
    ref = np.asarray(g["scores"], np.float64)
    per = np.asarray(split(s, reqs), np.float64)
    rel = np.abs(per - ref) / np.maximum(1.0, np.abs(ref))
    strict = sum(top10_strict_swaps(per[i], ref[i]) > 0 for i in range(len(reqs)))
    print(f"c64 sweep: max rel err {rel.max():.3e}, p99 {np.percentile(rel, 99):.3e}, "
          f"median {np.median(rel):.3e}, std of error {np.std(per - ref):.3e}; "
          f"requests with a strict top-10 swap: {strict} of {len(reqs)}")
    assert rel.max() <= SCORE_TOL
    # sampled requests scored alone give bit-identical scores (batch invariance)
    lens = [len(p) for p, _ in reqs]
    for i in [int(np.argmin(lens)), int(np.argmax(lens)), 17]:
        np.testing.assert_array_equal(r.score([reqs[i]]), per[i].astype(np.float32))


def test_qwen_rating_mix(gpu_qwen):
    cfg, _, _, model, r = gpu_qwen
    reqs = reqs_of(cfg, 4, n=8)
    for g in (False, True):
        check_against_oracle(model, reqs, r.score(reqs, use_graph=g))


def test_mis_vs_independent_qwen(gpu_qwen):
    cfg, _, _, model, r = gpu_qwen
    reqs = reqs_of(cfg, 2)
    mis = r.score(reqs)
    ind = r.score(reqs, mode=IND)
    e = score_err(mis, ind)
    print(f"GPU MIS vs GPU independent: max rel diff {e:.3e}")
    assert e <= MIS_VS_IND_TOL


def test_stress_shape_sampled(gpu_qwen):
    # L = 4096, K = 512: all 512 candidates by MIS, sampled ones against the
    # oracle's scores of the same candidates scored on their own (candidates
    # never see each other, so these equal the full-K scores) and against GPU
    # independent scoring
    cfg, _, _, model, r = gpu_qwen
    (p, c), = reqs_of(cfg, 5, n=1)
    assert len(p) == 4096 and len(c) == 512
    mis = r.score([(p, c)])
    g = golden("oracle_stress_subset.json")
    pick = g["candidates"]
    e = score_err(mis[pick], g["scores"])
    print(f"stress shape: GPU MIS vs oracle on {len(pick)} candidates: {e:.3e}")
    assert e <= SCORE_TOL
    ind = r.score([(p, c[pick])], mode=IND)
    e = score_err(mis[pick], ind)
    print(f"stress shape: MIS vs independent on {len(pick)} candidates: {e:.3e}")
    assert e <= MIS_VS_IND_TOL
    # the candidate subset scored by MIS alone matches the full-K scores bit for bit
    np.testing.assert_array_equal(r.score([(p, c[pick])]), mis[pick])


def test_longest_prefix(gpu_qwen):
    # The longest accepted prefix puts its candidates at the rotary table's
    # last position: MIS against independent scoring there, and one more row
    # is refused before anything runs.
    cfg, _, _, _, r = gpu_qwen
    lmax = r.dims.max_prefix
    (p, c), = reqs_of(cfg, 5, n=1)
    prefix = np.resize(p, lmax).astype(np.int32)  # the L = 4096 request's ids, repeated
    cands = c[[0, 255, 511]]
    mis = r.score([(prefix, cands)])
    assert np.all(np.isfinite(mis))
    ind = r.score([(prefix, cands)], mode=IND)
    e = score_err(mis, ind)
    print(f"L = {lmax}: MIS vs independent {e:.3e}")
    assert e <= MIS_VS_IND_TOL
    with pytest.raises(spa.DuolmError) as ei:
        r.score([(np.resize(p, lmax + 1).astype(np.int32), cands)])
    assert ei.value.status == "EINVAL"


def test_launch_row_limit_splits_calls(gpu_qwen, monkeypatch):
    # A ranker whose launches hold at most 4096 rows scores a 64-request batch
    # (about 21k rows) as several launches, request by request, with the same
    # bits as one launch; a single request over the limit is refused.
    cfg, w, D, _, r = gpu_qwen
    monkeypatch.setenv("DUOLM_MAX_ROWS", "4096")
    small = spa.Ranker.from_blob(spa.weights_blob(cfg, w))
    try:
        assert small.dims.max_rows == 4096
        small.load_vid_table(D)
        reqs = reqs_of(cfg, 3, n=64)
        assert sum(len(p) + len(c) for p, c in reqs) > 4 * 4096
        np.testing.assert_array_equal(small.score(reqs), r.score(reqs))
        (p, c), = reqs_of(cfg, 5, n=1)  # 4096 + 512 rows
        with pytest.raises(spa.DuolmError) as ei:
            small.score([(p, c)])
        assert ei.value.status == "EINVAL"
    finally:
        small.close()


def test_graph_matches_eager_and_repeats(gpu_qwen):
    cfg, _, _, _, r = gpu_qwen
    reqs = reqs_of(cfg, 3, n=12)
    eager = r.score(reqs, use_graph=False)
    for _ in range(3):
        np.testing.assert_array_equal(r.score(reqs, use_graph=True), eager)
    # a different batch between replays of the same bucket
    other = reqs_of(cfg, 3, n=12, seed=99)
    r.score(other, use_graph=True)
    np.testing.assert_array_equal(r.score(reqs, use_graph=True), eager)


def test_batch_composition_sweep(gpu_qwen):
    # Random sub-batches of the 64-request headline batch, sized to cross every
    # GEMM tile regime (deep LDS rings below one tile per CU, two-stage and
    # persistent tiles above) and the two-lane threshold, in graph and eager
    # launches and with one or two lanes: each request's scores equal its slice
    # of the full batch bit for bit.
    cfg, _, _, _, r = gpu_qwen
    reqs = reqs_of(cfg, 3, n=64)
    full = split(r.score(reqs), reqs)
    rng = np.random.default_rng(11)
    for n in (1, 2, 5, 13, 40):
        pick = rng.choice(64, size=n, replace=False)
        sub = [reqs[i] for i in pick]
        for graph, lanes in ((True, 0), (False, 0), (True, 1)):
            got = split(r.score(sub, use_graph=graph, max_lanes=lanes), sub)
            for j, i in enumerate(pick):
                np.testing.assert_array_equal(got[j], full[i])


def test_permutation_and_leakage(gpu_tiny):
    cfg, _, _, _, r = gpu_tiny
    (p, c), = reqs_of(cfg, 1)
    base = r.score([(p, c)])
    perm = np.random.default_rng(3).permutation(len(c))
    np.testing.assert_array_equal(r.score([(p, c[perm])]), base[perm])
    c2 = c.copy()
    c2[2] = cfg.vocab + (int(c[2]) - cfg.vocab + 1) % cfg.n_vid
    other = r.score([(p, c2)])
    keep = np.arange(len(c)) != 2
    np.testing.assert_array_equal(other[keep], base[keep])


def test_device_entry_point(gpu_qwen):
    cfg, _, _, _, r = gpu_qwen
    reqs = reqs_of(cfg, 3, n=5)
    ids, L, K = synth.pack_ids([synth.Request(np.asarray(p), np.asarray(c)) for p, c in reqs])
    d_ids = torch.from_numpy(ids).cuda()
    d_s = torch.full((int(K.sum()),), -7.0, device="cuda")
    r.score_dev(L, K, d_ids.data_ptr(), d_s.data_ptr())
    np.testing.assert_array_equal(d_s.cpu().numpy(), r.score(reqs))
    # an out-of-range id: ERANGE and the output left untouched
    bad = ids.copy()
    bad[3] = cfg.vocab + cfg.n_vid
    d_bad = torch.from_numpy(bad).cuda()
    d_s2 = torch.full((int(K.sum()),), -7.0, device="cuda")
    with pytest.raises(spa.DuolmError) as e:
        r.score_dev(L, K, d_bad.data_ptr(), d_s2.data_ptr())
    assert e.value.status == "ERANGE"
    assert torch.all(d_s2 == -7.0)


def test_host_errors(gpu_tiny):
    cfg, _, _, _, r = gpu_tiny
    p = np.arange(5, dtype=np.int32)
    with pytest.raises(spa.DuolmError) as e:
        r.score([(p, np.array([cfg.vocab + cfg.n_vid], np.int32))])
    assert e.value.status == "ERANGE"
    with pytest.raises(spa.DuolmError) as e:
        r.score([(p, np.array([-1], np.int32))])
    assert e.value.status == "ERANGE"
    with pytest.raises(spa.DuolmError) as e:
        r.score([(p, np.array([], np.int32))])
    assert e.value.status == "EINVAL"
    with pytest.raises(spa.DuolmError) as e:
        r.score([(np.array([], np.int32), np.array([cfg.vocab], np.int32))])
    assert e.value.status == "EINVAL"


def test_no_table_is_estate(tiny):
    cfg, w, _, _ = tiny
    r = spa.Ranker.from_blob(spa.weights_blob(cfg, w))
    try:
        with pytest.raises(spa.DuolmError) as e:
            r.score([(np.arange(4, dtype=np.int32), np.array([cfg.vocab], np.int32))])
        assert e.value.status == "ESTATE"
        s = r.score([(np.arange(4, dtype=np.int32), np.array([7, 8], np.int32))])  # text-only ids work
        assert np.all(np.isfinite(s))
    finally:
        r.close()


def test_profiling_counters(gpu_qwen):
    cfg, _, _, _, r = gpu_qwen
    reqs = reqs_of(cfg, 3, n=16)
    base = r.score(reqs)
    r.set_profiling(["gemm_gateup", "attn_branch"])
    for g in (False, True):
        # timing the branch tiles launches them apart from the prefix tiles
        # (the branch-only instantiation of the attention kernel): same bits
        np.testing.assert_array_equal(r.score(reqs, use_graph=g), base)
    st = r.kernel_stats("gemm_gateup")
    # a call this size runs as two concurrent halves (one launch each per layer)
    assert st.launches % (2 * cfg.n_layers) == 0 and st.launches >= 2 * cfg.n_layers and st.total_ms > 0
    assert r.kernel_stats("attn_branch").launches == st.launches
    assert r.kernel_stats("gemm_qkv").launches == 0
    # algorithmic FLOPs: every row in the first n_layers - 1 layers, the
    # candidate rows only in the last one (its prefix rows feed only K and V)
    T = sum(len(p) + len(c) for p, c in reqs)
    TB = sum(len(c) for _, c in reqs)
    per_row = 2 * cfg.d_model * 2 * cfg.d_ffn
    assert st.flops == pytest.approx(2 * per_row * ((cfg.n_layers - 1) * T + TB), rel=1e-12)
    r.set_profiling([])


def _inline_rows(cfg, D, prefix, cands):
    ids = np.concatenate([prefix, cands])
    return D[ids[ids >= cfg.vocab] - cfg.vocab]


def test_inline_vectors_match_table_lookup(gpu_tiny):
    # shipping the item vectors in the request gives the same scores, bit for bit
    cfg, _, D, _, r = gpu_tiny
    reqs = reqs_of(cfg, 1) + reqs_of(cfg, 4, n=3, n_cand=5)
    base = r.score(reqs)
    inl = [(p, c, _inline_rows(cfg, D, p, c)) for p, c in reqs]
    np.testing.assert_array_equal(r.score(inl), base)
    np.testing.assert_array_equal(r.score(inl, use_graph=False), base)
    # mixed batch: one request ships vectors, the others use ids
    mixed = [inl[0]] + reqs[1:]
    np.testing.assert_array_equal(r.score(mixed), base)


def test_inline_vectors_without_table(tiny):
    # a ranker with no table loaded scores requests that carry their vectors,
    # and equals a ranker that holds those vectors in its table
    cfg, w, D, _ = tiny
    D2 = synth.make_vid_table(cfg, seed=77)
    with_table = spa.Ranker.from_blob(spa.weights_blob(cfg, w))
    no_table = spa.Ranker.from_blob(spa.weights_blob(cfg, w))
    try:
        with_table.load_vid_table(D2)
        reqs = reqs_of(cfg, 1)
        inl = [(p, c, _inline_rows(cfg, D2, p, c)) for p, c in reqs]
        np.testing.assert_array_equal(no_table.score(inl), with_table.score(reqs))
    finally:
        with_table.close()
        no_table.close()


def test_inline_rows_not_addressable_by_ids(gpu_tiny):
    # the ids just past the table belong to the call's inline rows only: a
    # request without vectors may not name them
    cfg, _, D, _, r = gpu_tiny
    (p, c), = reqs_of(cfg, 1)
    bad = (np.array([1, 2, cfg.vocab + cfg.n_vid], np.int32), c)
    with pytest.raises(spa.DuolmError) as e:
        r.score([(p, c, _inline_rows(cfg, D, p, c)), bad])
    assert e.value.status == "ERANGE"


def test_graph_replay_after_buffer_growth(gpu_qwen):
    # a bigger call reallocates the id and score buffers: graphs captured
    # before must not be replayed against the freed buffers
    cfg, _, _, _, r = gpu_qwen
    small = reqs_of(cfg, 4, n=2)
    eager = r.score(small, use_graph=False)
    np.testing.assert_array_equal(r.score(small, use_graph=True), eager)
    big = reqs_of(cfg, 3, n=48, seed=5)
    r.score(big, use_graph=True)
    np.testing.assert_array_equal(r.score(small, use_graph=True), eager)


# ---------------------------------------------------------------------------
# candidates of m rows (items spread over m vectors)
# ---------------------------------------------------------------------------


def _mv_check(model, reqs, m, got):
    per, o = [], 0
    for p, c in reqs:
        k = len(c) // m
        per.append(got[o:o + k])
        o += k
    assert o == got.shape[0]
    for (p, c), s in zip(reqs, per):
        ref = oracle_mis(model, p, c, m=m)
        e = score_err(s, ref)
        assert e <= SCORE_TOL, e
    return per


@pytest.mark.parametrize("m,n_cand", [(2, 8), (3, 50), (64, 3)])
def test_multivector_tiny(gpu_tiny, m, n_cand):
    # m = 3 with 50 candidates: 150 branch rows, tiles of 42 whole branches;
    # m = 64, the longest candidate accepted: two whole branches fill a tile
    cfg, _, _, model, r = gpu_tiny
    reqs = [(q.prefix, q.cands) for q in synth.make_requests(1, cfg, m=m, n_cand=n_cand)]
    for g in (False, True):
        _mv_check(model, reqs, m, r.score(reqs, use_graph=g, cand_len=m))


def test_multivector_qwen(gpu_qwen):
    cfg, _, _, model, r = gpu_qwen
    reqs = [(q.prefix, q.cands) for q in synth.make_requests(6, cfg, n_requests=2)]  # m = 8, K = 5 and 20
    _mv_check(model, reqs, 8, r.score(reqs, cand_len=8))


def test_multivector_mis_vs_independent(gpu_qwen):
    cfg, _, _, _, r = gpu_qwen
    reqs = [(q.prefix, q.cands) for q in synth.make_requests(2, cfg, m=4, n_cand=12)]
    mis = r.score(reqs, cand_len=4)
    ind = r.score(reqs, mode=IND, cand_len=4)
    e = score_err(mis, ind)
    print(f"m = 4: GPU MIS vs GPU independent {e:.3e}")
    assert e <= MIS_VS_IND_TOL
    # each candidate's branch rows run the same arithmetic in both modes
    np.testing.assert_array_equal(mis, ind)


def test_multivector_batch_and_defaults(gpu_tiny):
    cfg, _, _, _, r = gpu_tiny
    a = [(q.prefix, q.cands) for q in synth.make_requests(1, cfg, m=3, n_cand=6)]
    b = reqs_of(cfg, 4, n=2, n_cand=5)
    mixed = r.score(a + b, cand_len=[3, 1, 1])
    np.testing.assert_array_equal(mixed[:6], r.score(a, cand_len=3))
    np.testing.assert_array_equal(mixed[6:], r.score(b))
    # cand_len 0 and 1 are the one-row default
    np.testing.assert_array_equal(r.score(b, cand_len=0), r.score(b))
    np.testing.assert_array_equal(r.score(b, cand_len=1), r.score(b))


def test_multivector_device_entry_and_errors(gpu_tiny):
    cfg, _, _, _, r = gpu_tiny
    qs = synth.make_requests(1, cfg, m=2, n_cand=7)
    ids, L, K = synth.pack_ids(qs)
    d_ids = torch.from_numpy(ids).cuda()
    d_s = torch.zeros(int(K.sum()), device="cuda")
    r.score_dev(L, K, d_ids.data_ptr(), d_s.data_ptr(), cand_len=[2])
    np.testing.assert_array_equal(d_s.cpu().numpy(), r.score([(q.prefix, q.cands) for q in qs], cand_len=2))
    p, c = qs[0].prefix, qs[0].cands
    for bad in (-1, 65):
        with pytest.raises(spa.DuolmError) as e:
            r.score([(p, c[:2])], cand_len=[bad]) if bad < 0 else r.score_dev(L, K, d_ids.data_ptr(),
                                                                            d_s.data_ptr(), cand_len=[bad])
        assert e.value.status == "EINVAL"
    with pytest.raises(ValueError):
        r.score([(p, c[:3])], cand_len=2)


def _pack(reqs_full, cid, cfg, header=()):
    marker, instr = synth.template(cid, cfg)
    return spa.PackInput(instr, marker, [(r.items, r.feedback, r.cands, r.m, r.m) for r in reqs_full], header)


def test_packed_host_path_matches_request_path(gpu_qwen, gpu_tiny):
    # structured requests -> host packer -> pinned staging -> scores equal, bit
    # for bit, to scoring the same requests given as flat id arrays
    cfg, _, _, _, r = gpu_qwen
    for cid, n in ((3, 64), (6, 16)):
        full = synth.make_requests(cid, cfg, n_requests=n)
        p = _pack(full, cid, cfg)
        for nt in (1, 4):
            ids, L, K, M = spa.duolm_pack_requests(p, n_threads=nt)
            got = r.score_packed(L, K, M, ids)
            want = r.score([(q.prefix, q.cands) for q in full], cand_len=[q.m for q in full])
            np.testing.assert_array_equal(got, want)
    # staging grows and shrinks across calls; a small call after a large one
    tcfg, _, _, model, rt = gpu_tiny
    small = synth.make_requests(1, tcfg)
    ps = _pack(small, 1, tcfg)
    ids, L, K, M = spa.duolm_pack_requests(ps)
    np.testing.assert_array_equal(rt.score_packed(L, K, M, ids), rt.score([(q.prefix, q.cands) for q in small]))
    check_against_oracle(model, [(q.prefix, q.cands) for q in small], rt.score_packed(L, K, M, ids))
    # a candidate header is just trailing prefix ids
    ph = _pack(small, 1, tcfg, header=(3, 4))
    ids, L, K, M = spa.duolm_pack_requests(ph)
    want = rt.score([(np.concatenate([q.prefix, [3, 4]]).astype(np.int32), q.cands) for q in small])
    np.testing.assert_array_equal(rt.score_packed(L, K, M, ids), want)
    # ids are range-checked on the way into the staging buffer
    bad = ids.copy()
    bad[5] = tcfg.vocab + tcfg.n_vid
    with pytest.raises(spa.DuolmError) as ei:
        rt.score_packed(L, K, M, bad)
    assert ei.value.code == -2


def test_two_lanes_equal_one_launch(gpu_qwen):
    # a large call runs as two concurrent halves on two streams; every row is
    # computed by the same kernels either way, so the scores are the same bits
    cfg, _, _, _, r = gpu_qwen
    reqs = reqs_of(cfg, 3, n=64)
    for g in (True, False):
        two = r.score(reqs, use_graph=g)
        one = r.score(reqs, use_graph=g, max_lanes=1)
        np.testing.assert_array_equal(two, one)
    # independent mode (many short sequences) and the device entry point too
    small = reqs[:3]
    np.testing.assert_array_equal(r.score(small, mode=IND), r.score(small, mode=IND, max_lanes=1))
    with pytest.raises(spa.DuolmError):
        r.score(small, max_lanes=3)


def test_two_lane_out_of_range_id_leaves_scores_untouched(gpu_qwen):
    # a 64-request call runs as two concurrent halves; an out-of-range id in
    # either half must fail the whole call with ERANGE and write no score
    # (the halves' gathers share one device flag, read before any score is
    # handed over), and the next valid call must still be exact
    cfg, _, _, _, r = gpu_qwen
    reqs = reqs_of(cfg, 3, n=64)
    ids, L, K = synth.pack_ids([synth.Request(np.asarray(p), np.asarray(c)) for p, c in reqs])
    want = r.score(reqs)
    n_first = int(L[0] + K[0])                       # first request's ids: first half
    last_off = int((L + K)[:-1].sum())               # last request's first id: second half
    for pos in (n_first - 1, last_off + 1):
        for g in (True, False):
            bad = ids.copy()
            bad[pos] = cfg.vocab + cfg.n_vid
            d_bad = torch.from_numpy(bad).cuda()
            d_s = torch.full((int(K.sum()),), -7.0, device="cuda")
            with pytest.raises(spa.DuolmError) as e:
                r.score_dev(L, K, d_bad.data_ptr(), d_s.data_ptr(), use_graph=g)
            assert e.value.status == "ERANGE"
            assert torch.all(d_s == -7.0)
            bad_reqs = list(reqs)
            p, c = bad_reqs[0 if pos < n_first else -1]
            p = np.array(p, np.int32)
            c = np.array(c, np.int32)
            if pos < n_first:
                c[-1] = cfg.vocab + cfg.n_vid
            else:
                p[1] = cfg.vocab + cfg.n_vid
            bad_reqs[0 if pos < n_first else -1] = (p, c)
            with pytest.raises(spa.DuolmError) as e:
                r.score(bad_reqs, use_graph=g)
            assert e.value.status == "ERANGE"
    d_ids = torch.from_numpy(ids).cuda()
    d_s = torch.empty(int(K.sum()), device="cuda")
    r.score_dev(L, K, d_ids.data_ptr(), d_s.data_ptr())
    np.testing.assert_array_equal(d_s.cpu().numpy(), want)
