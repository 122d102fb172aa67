"""Pins for the oracle's MIS path: the pages' exactness identity against
brute-force independent scoring, the closed-form count of removed pairs, the
K = 1 reduction to textbook causal decoding, and the invariances that rule out
leakage between candidates or requests."""
import json
import os

import numpy as np
import pytest

import synth
from oracle import (brute_force_independent, decode_incremental, embed_rows, oracle_mis,
                    oracle_mis_packed, pair_count, tree_mask)

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def rel_err(a, b):
    a, b = np.asarray(a), np.asarray(b)
    return float(np.max(np.abs(a - b) / np.maximum(1.0, np.abs(b))))


def test_identity_tiny_workload(tiny):
    # s^MIS_{q,j} = s_{q,j}: packed scoring equals appending each candidate alone
    cfg, _, _, model = tiny
    (req,) = synth.make_requests(1, cfg)
    assert req.L == 48 and req.K == 8
    mis = oracle_mis(model, req.prefix, req.cands)
    ind = brute_force_independent(model, req.prefix, req.cands)
    assert rel_err(mis, ind) < 1e-12
    assert np.std(mis) > 1e-3  # scores are not degenerate


def test_identity_with_gains(tiny_gains):
    cfg, _, _, model = tiny_gains
    reqs = synth.make_requests(4, cfg, n_requests=3, n_cand=5)
    for r in reqs:
        assert rel_err(oracle_mis(model, r.prefix, r.cands),
                       brute_force_independent(model, r.prefix, r.cands)) < 1e-12


def test_k1_equals_incremental_decoding(tiny):
    cfg, _, _, model = tiny
    (req,) = synth.make_requests(1, cfg)
    for j in (0, 5):
        s = oracle_mis(model, req.prefix, req.cands[j:j + 1])[0]
        ref = decode_incremental(model, np.concatenate([req.prefix, req.cands[j:j + 1]]))
        assert abs(s - ref) <= 1e-12 * max(1.0, abs(ref))


def test_candidate_permutation_and_no_leakage(tiny):
    cfg, _, _, model = tiny
    (req,) = synth.make_requests(1, cfg)
    base = oracle_mis(model, req.prefix, req.cands)
    perm = np.random.default_rng(0).permutation(req.K)
    np.testing.assert_allclose(oracle_mis(model, req.prefix, req.cands[perm]), base[perm], rtol=1e-12)
    # replacing candidate 3 leaves every other score unchanged
    c2 = req.cands.copy()
    c2[3] = cfg.vocab + 499 if c2[3] != cfg.vocab + 499 else cfg.vocab + 498
    other = oracle_mis(model, req.prefix, c2)
    mask = np.arange(req.K) != 3
    np.testing.assert_allclose(other[mask], base[mask], rtol=1e-12)
    assert abs(other[3] - base[3]) > 1e-6
    # duplicate candidates score identically
    dup = oracle_mis(model, req.prefix, np.array([req.cands[2], req.cands[2]]))
    assert abs(dup[0] - dup[1]) <= 1e-13 * max(1, abs(dup[0]))


def test_packed_batch_equals_per_request(tiny):
    cfg, _, _, model = tiny
    reqs = synth.make_requests(3, cfg, n_requests=3, n_cand=6)
    packed = oracle_mis_packed(model, [(r.prefix, r.cands) for r in reqs])
    for r, s in zip(reqs, packed):
        assert rel_err(s, oracle_mis(model, r.prefix, r.cands)) < 1e-12


def test_position_shift_invariance(tiny):
    # rotary scores depend on position differences only
    cfg, _, _, model = tiny
    (req,) = synth.make_requests(1, cfg)
    a = oracle_mis(model, req.prefix, req.cands)
    b = oracle_mis(model, req.prefix, req.cands, pos_offset=1000)
    assert rel_err(a, b) < 1e-9


def test_positions_matter(tiny):
    # a wrong candidate position (L+1 instead of L) breaks the identity, so the
    # identity test does constrain positions
    cfg, _, _, model = tiny
    from oracle.ranker import decoder_forward, score_head
    (req,) = synth.make_requests(1, cfg)
    L, K = req.L, req.K
    x = embed_rows(model, np.concatenate([req.prefix, req.cands]))
    pos = np.concatenate([np.arange(L), np.full(K, L + 1)])
    wrong = score_head(model, decoder_forward(model, x, pos, tree_mask(L, K))[L:])
    assert rel_err(wrong, brute_force_independent(model, req.prefix, req.cands)) > 1e-6


def test_pair_counts_match_pages_formula():
    with open(os.path.join(GOLDEN, "pair_counts.json")) as f:
        cases = json.load(f)["cases"]
    for c in cases:
        got = pair_count(c["L"], c["K"])
        assert got["eliminated"] == c["eliminated"], c
        L, K = c["L"], c["K"]
        assert got["mis"] == L * (L + 1) // 2 + K * (L + 1)


def test_tree_mask_structure():
    m = tree_mask(4, 3)
    assert m[:4, :4].tolist() == np.tril(np.ones((4, 4), bool)).tolist()
    assert not m[:4, 4:].any()
    assert m[4:, :4].all()
    assert m[4:, 4:].tolist() == np.eye(3, dtype=bool).tolist()


def test_embed_lookup_boundary(tiny):
    cfg, w, D, model = tiny
    V = cfg.vocab
    rows = embed_rows(model, [0, V - 1, V, V + cfg.n_vid - 1])
    np.testing.assert_array_equal(rows[1], synth.bf16_bits_to_f32(w["embed"][V - 1]).astype(np.float64))
    np.testing.assert_array_equal(rows[2], D[0].view(np.float16).astype(np.float64))
    np.testing.assert_array_equal(rows[3], D[-1].view(np.float16).astype(np.float64))
    for bad in (-1, V + cfg.n_vid):
        with pytest.raises(ValueError):
            embed_rows(model, [bad])


@pytest.mark.slow
def test_identity_qwen_shape(qwen):
    # one request of the 0.6B single-request workload (L = 452, K = 100); the
    # brute force is run for three candidates (each is a 453-row forward)
    cfg, _, _, model = qwen
    (req,) = synth.make_requests(2, cfg)
    assert req.L == 452 and req.K == 100
    mis = oracle_mis(model, req.prefix, req.cands)
    which = [0, 41, 99]
    ind = brute_force_independent(model, req.prefix, req.cands, which=which)
    assert rel_err(mis[which], ind) < 1e-10
    assert np.all(np.isfinite(mis)) and np.std(mis) > 1e-2


# ---------------------------------------------------------------------------
# multi-vector items: a candidate spans m rows at positions L..L+m-1, causal
# inside its own branch, scored at its last row
# ---------------------------------------------------------------------------


@pytest.mark.parametrize("m", [2, 3])
def test_multivector_identity_tiny(tiny, m):
    # packed MIS with m-row branches equals appending each candidate's m ids alone
    cfg, _, _, model = tiny
    (req,) = synth.make_requests(1, cfg, m=m)
    assert req.m == m and req.K == 8 and req.cands.shape[0] == 8 * m
    mis = oracle_mis(model, req.prefix, req.cands, m=m)
    ind = brute_force_independent(model, req.prefix, req.cands, m=m)
    assert mis.shape == (8,)
    assert rel_err(mis, ind) < 1e-12
    assert np.std(mis) > 1e-3


def test_multivector_k1_equals_incremental_decoding(tiny):
    # one candidate of m ids: the packed forward is a plain causal LM over L+m tokens
    cfg, _, _, model = tiny
    (req,) = synth.make_requests(1, cfg, m=3, n_cand=1)
    s = oracle_mis(model, req.prefix, req.cands, m=3)[0]
    d = decode_incremental(model, np.concatenate([req.prefix, req.cands]))
    assert abs(s - d) <= 1e-12 * max(1.0, abs(d))


@pytest.mark.parametrize("L,K,m", [(48, 8, 2), (452, 100, 8), (7, 1, 5), (13, 9, 3)])
def test_multivector_pair_counts(L, K, m):
    # per candidate, the independent sequence holds L(L+1)/2 prefix pairs plus the
    # branch's own pairs; MIS keeps one copy of the prefix: (K-1) L (L+1) / 2 removed
    pc = pair_count(L, K, m)
    assert pc["eliminated"] == (K - 1) * L * (L + 1) // 2
    assert pc["mis"] == L * (L + 1) // 2 + K * (m * L + m * (m + 1) // 2)


def test_multivector_mask_and_positions():
    from oracle.ranker import mis_positions
    L, K, m = 5, 3, 4
    mask = tree_mask(L, K, m)
    pos = mis_positions(L, K, m)
    assert list(pos[:L]) == list(range(L))
    for j in range(K):
        for i in range(m):
            r = L + j * m + i
            assert pos[r] == L + i
            assert mask[r, :L].all()
            assert mask[r, L:].sum() == i + 1                      # own branch rows 0..i only
            assert mask[r, L + j * m:L + j * m + i + 1].all()
    assert np.array_equal(tree_mask(L, K, 1), tree_mask(L, K))


def test_multivector_permutation_and_packing(tiny):
    cfg, _, _, model = tiny
    (req,) = synth.make_requests(1, cfg, m=2, n_cand=5)
    base = oracle_mis(model, req.prefix, req.cands, m=2)
    perm = np.array([3, 0, 4, 1, 2])
    blocks = req.cands.reshape(5, 2)[perm].reshape(-1)
    assert np.allclose(oracle_mis(model, req.prefix, blocks, m=2), base[perm], rtol=0, atol=1e-12)
    # a packed batch mixing m = 2 and m = 1 requests equals per-request scoring
    (other,) = synth.make_requests(1, cfg, n_cand=3, seed=5)
    packed = oracle_mis_packed(model, [(req.prefix, req.cands, 2), (other.prefix, other.cands)])
    assert rel_err(packed[0], base) < 1e-12
    assert rel_err(packed[1], oracle_mis(model, other.prefix, other.cands)) < 1e-12
