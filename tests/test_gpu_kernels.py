"""Per-kernel parity on the GPU.

GEMM: the MFMA kernel against float64 products of the same bf16 operands.
Gather: bit-exact against host indexing of the bf16 embedding and the fp16
item table.  Layer stages: every kernel of a decoder layer is checked against
the oracle's building block applied to the GPU's own input for that stage, so
each comparison isolates one kernel.
"""
import numpy as np
import pytest
import torch

import synth
from oracle import attention, rmsnorm, rope_rotate, tree_mask, widen_bf16, widen_f16
from oracle.ranker import mis_positions
import shared_prefix_scoring_amd as spa

pytestmark = pytest.mark.gpu


def bf16_tensor(rng, shape, scale=1.0):
    bits = synth.f32_to_bf16_bits(rng.standard_normal(shape).astype(np.float32) * np.float32(scale))
    return bits, widen_bf16(bits)


def to_dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


GEMM_SHAPES = [
    (1, 64, 64),                                                     # 64x64 tiles of one wave (N % 128 != 0)
    # fewer tiles than CUs: 64x64 tiles of four waves (128x128 for SwiGLU) on
    # an 8-stage LDS ring; K from one slab (64) to 48 slabs, ragged M
    (77, 256, 128), (300, 768, 384), (200, 128, 64), (40, 1024, 3072),
    (513, 4096, 1024),                                               # 128x128 tiles, 4-stage ring
    (4100, 1024, 2048), (1500, 3072, 1024),                          # 128x128 tiles, two stages
    (4096, 4096, 1024), (4133, 6144, 1024),                          # 256x256 tiles, ragged tail
    (16500, 1024, 256), (12000, 2048, 64),                           # 256-row tiles, or 192-row for the residual epilogue
]


@pytest.mark.parametrize("M,N,K", GEMM_SHAPES)
@pytest.mark.parametrize("epi", ["bf16", "resid", "swiglu"])
def test_gemm(M, N, K, epi):
    rng = np.random.default_rng(M * 7 + N + K)
    a_bits, a = bf16_tensor(rng, (M, K))
    w_bits, w = bf16_tensor(rng, (N, K), 0.05)
    dA, dW = to_dev(a_bits.view(np.int16)), to_dev(w_bits.view(np.int16))
    ref = a @ w.T
    bound = np.abs(a) @ np.abs(w).T * (K * 2.0 ** -23)  # fp32 accumulation bound
    if epi == "bf16":
        dC = torch.zeros((M, N), dtype=torch.int16, device="cuda")
        spa.duolm_debug_gemm(0, dA.data_ptr(), dW.data_ptr(), dC.data_ptr(), M, N, K)
        got = widen_bf16(dC.cpu().numpy().view(np.uint16))
        assert np.all(np.abs(got - ref) <= np.abs(ref) * 2.0 ** -8 + bound + 1e-30)
    elif epi == "resid":
        c0 = rng.standard_normal((M, N)).astype(np.float32)
        dC = to_dev(c0)
        spa.duolm_debug_gemm(1, dA.data_ptr(), dW.data_ptr(), dC.data_ptr(), M, N, K)
        got = dC.cpu().numpy().astype(np.float64)
        want = c0.astype(np.float64) + ref
        assert np.all(np.abs(got - want) <= bound + np.abs(want) * 2.0 ** -23 + 1e-30)
    else:
        # interleave gate/up rows in 32-row blocks: gate block p, up block p, ...
        F = N // 2
        g_bits, u_bits = w_bits[:F], w_bits[F:]
        inter = np.empty_like(w_bits)
        for p in range(F // 32):
            inter[64 * p:64 * p + 32] = g_bits[32 * p:32 * p + 32]
            inter[64 * p + 32:64 * p + 64] = u_bits[32 * p:32 * p + 32]
        dW = to_dev(inter.view(np.int16))
        dC = torch.zeros((M, F), dtype=torch.int16, device="cuda")
        spa.duolm_debug_gemm(2, dA.data_ptr(), dW.data_ptr(), dC.data_ptr(), M, N, K)
        got = widen_bf16(dC.cpu().numpy().view(np.uint16))
        g, u = ref[:, :F], ref[:, F:]
        want = g / (1 + np.exp(-g)) * u
        # bf16 output rounding plus the propagated fp32 accumulation error of g and u
        tol = np.abs(want) * 2.0 ** -8 + (np.abs(u) * 1.2 + np.abs(g)) * bound[:, :F] * 2 + 1e-30
        assert np.all(np.abs(got - want) <= tol)


@pytest.mark.parametrize("M,N,K,epi", [(30011, 6144, 1024, "swiglu"), (30011, 4096, 1024, "bf16"),
                                        (30011, 1024, 3072, "resid")])
def test_gemm_many_tiles_sampled(M, N, K, epi):
    # Workgroups walk many tiles each (one workgroup per CU), with a ragged last
    # row tile; rows sampled across the range, including the last one, against
    # float64 products of the same bf16 operands.
    rng = np.random.default_rng(M + N + K)
    a_bits, a = bf16_tensor(rng, (M, K))
    w_bits, w = bf16_tensor(rng, (N, K), 0.05)
    rows = np.unique(np.concatenate([rng.integers(0, M, 40), np.arange(M - 24, M), [0, 255, 256]]))
    ref = a[rows] @ w.T
    bound = np.abs(a[rows]) @ np.abs(w).T * (K * 2.0 ** -23)
    dA = to_dev(a_bits.view(np.int16))
    if epi == "bf16":
        dW = to_dev(w_bits.view(np.int16))
        dC = torch.zeros((M, N), dtype=torch.int16, device="cuda")
        spa.duolm_debug_gemm(0, dA.data_ptr(), dW.data_ptr(), dC.data_ptr(), M, N, K)
        got = widen_bf16(dC.cpu().numpy().view(np.uint16)[rows])
        assert np.all(np.abs(got - ref) <= np.abs(ref) * 2.0 ** -8 + bound + 1e-30)
    elif epi == "resid":
        dW = to_dev(w_bits.view(np.int16))
        c0 = rng.standard_normal((M, N)).astype(np.float32)
        dC = to_dev(c0)
        spa.duolm_debug_gemm(1, dA.data_ptr(), dW.data_ptr(), dC.data_ptr(), M, N, K)
        got = dC.cpu().numpy()[rows].astype(np.float64)
        want = c0[rows].astype(np.float64) + ref
        assert np.all(np.abs(got - want) <= bound + np.abs(want) * 2.0 ** -23 + 1e-30)
    else:
        F = N // 2
        inter = np.empty_like(w_bits)
        for p in range(F // 32):
            inter[64 * p:64 * p + 32] = w_bits[32 * p:32 * p + 32]
            inter[64 * p + 32:64 * p + 64] = w_bits[F + 32 * p:F + 32 * p + 32]
        dW = to_dev(inter.view(np.int16))
        dC = torch.zeros((M, F), dtype=torch.int16, device="cuda")
        spa.duolm_debug_gemm(2, dA.data_ptr(), dW.data_ptr(), dC.data_ptr(), M, N, K)
        got = widen_bf16(dC.cpu().numpy().view(np.uint16)[rows])
        g, u = ref[:, :F], ref[:, F:]
        want = g / (1 + np.exp(-g)) * u
        tol = np.abs(want) * 2.0 ** -8 + (np.abs(u) * 1.2 + np.abs(g)) * bound[:, :F] * 2 + 1e-30
        assert np.all(np.abs(got - want) <= tol)
    # rows are batch invariant: a launch over a slice reproduces them bit for bit
    lo = int(rows[len(rows) // 2])
    n = 300
    sub = torch.zeros((n, dC.shape[1]), dtype=dC.dtype, device="cuda")
    if epi == "resid":
        sub.copy_(to_dev(c0[lo:lo + n]))
    spa.duolm_debug_gemm({"bf16": 0, "resid": 1, "swiglu": 2}[epi], dA[lo:lo + n].data_ptr(), dW.data_ptr(),
                         sub.data_ptr(), n, N, K)
    assert torch.equal(sub, dC[lo:lo + n])


def test_copy_kernel():
    x = torch.randint(-2 ** 31, 2 ** 31 - 1, (1 << 20,), dtype=torch.int32, device="cuda")
    y = torch.zeros_like(x)
    spa.duolm_copy_device(y.data_ptr(), x.data_ptr(), x.numel() * 4)
    torch.cuda.synchronize()
    assert torch.equal(x, y)


def _batch(cfg, cid, n):
    return [(r.prefix, r.cands) for r in synth.make_requests(cid, cfg, n_requests=n)]


@pytest.mark.parametrize("fixture", ["gpu_tiny", "gpu_qwen"])
def test_embed_gather_bit_exact(fixture, request):
    cfg, w, D, model, r = request.getfixturevalue(fixture)
    V, N = cfg.vocab, cfg.n_vid
    reqs = _batch(cfg, 1 if cfg.name == "tiny" else 4, 3)
    # boundary ids: last token, first and last table rows
    reqs.append((np.array([0, V - 1, V, V + N - 1, 5], np.int32), np.array([V + N - 1, V], np.int32)))
    x = r.stage(reqs, 0, "embed")
    ids = np.concatenate([np.concatenate([p, c]) for p, c in reqs])
    want = np.empty((ids.shape[0], cfg.d_model), np.float32)
    tok = ids < V
    want[tok] = synth.bf16_bits_to_f32(w["embed"][ids[tok]])
    want[~tok] = D[ids[~tok] - V].view(np.float16).astype(np.float32)
    np.testing.assert_array_equal(x, want)


def _rel(got, ref):
    return float(np.max(np.abs(got - ref)) / max(np.sqrt(np.mean(ref * ref)), 1e-30))


def _attn_close(got, ref, ref_abs_v):
    """Attention output: the kernel rounds each softmax weight p_k to bf16
    (relative error <= 2^-8) before P.V and normalises by the fp32 sum, so
    |dO| <= 2^-8 sum_k p_k |v_k| / sum_k p_k (the oracle's attention over |V|,
    ref_abs_v), plus one bf16 rounding of the output; checked with a factor 2
    of margin, elementwise."""
    bad = np.abs(got - ref) > 2.0 ** -7 * (ref_abs_v + np.abs(ref)) + 1e-6
    return not bad.any()


def _bf16_close(got, ref, floor=2e-3):
    """Elementwise: one bf16 rounding of the output (2^-8 relative covers it
    with margin) plus a floor of `floor` x RMS(ref) for fp32 accumulation."""
    rms = max(np.sqrt(np.mean(ref * ref)), 1e-30)
    bad = np.abs(got - ref) > 2.0 ** -8 * np.abs(ref) + floor * rms
    return not bad.any()


@pytest.mark.parametrize("fixture,layers", [("gpu_tiny", [0, 1]), ("gpu_tiny_gains", [0, 1]),
                                            ("gpu_qwen", [0, 13, 27])])
def test_layer_stages(fixture, layers, request):
    cfg, w, D, model, r = request.getfixturevalue(fixture)
    reqs = _batch(cfg, 1 if cfg.name == "tiny" else 4, 2)
    H, Hk, hd, d, eps = cfg.n_heads, cfg.n_kv_heads, cfg.head_dim, cfg.d_model, cfg.rms_eps
    pos = np.concatenate([mis_positions(len(p), len(c)) for p, c in reqs])
    T = pos.shape[0]
    allowed = np.zeros((T, T), dtype=bool)
    o = 0
    for p, c in reqs:
        n = len(p) + len(c)
        allowed[o:o + n, o:o + n] = tree_mask(len(p), len(c))
        o += n
    bf = lambda a: widen_bf16(a)
    for l in layers:
        W = model.layers[l]
        x_in = (r.stage(reqs, 0, "embed") if l == 0 else r.stage(reqs, l - 1, "layer_out")).astype(np.float64)
        a = bf(r.stage(reqs, l, "attn_norm"))
        assert _bf16_close(a, rmsnorm(x_in, W["attn_norm"], eps))
        qkv = bf(r.stage(reqs, l, "qkv"))
        wqkv = np.concatenate([W["wq"], W["wk"], W["wv"]])
        assert _bf16_close(qkv, a @ wqkv.T)
        qr = bf(r.stage(reqs, l, "qk_rope"))
        nq, nk = H * hd, Hk * hd
        q_ref = rope_rotate(rmsnorm(qkv[:, :nq].reshape(T, H, hd), W["q_norm"], eps), pos, cfg.rope_base)
        k_ref = rope_rotate(rmsnorm(qkv[:, nq:nq + nk].reshape(T, Hk, hd), W["k_norm"], eps), pos, cfg.rope_base)
        assert _bf16_close(qr[:, :nq], q_ref.reshape(T, nq))
        assert _bf16_close(qr[:, nq:nq + nk], k_ref.reshape(T, nk))
        np.testing.assert_array_equal(qr[:, nq + nk:], qkv[:, nq + nk:])  # v untouched
        att = bf(r.stage(reqs, l, "attn"))
        q_, k_, v_ = qr[:, :nq].reshape(T, H, hd), qr[:, nq:nq + nk].reshape(T, Hk, hd), qr[:, nq + nk:].reshape(T, Hk, hd)
        att_ref = attention(q_, k_, v_, allowed).reshape(T, nq)
        assert _attn_close(att, att_ref, attention(q_, k_, np.abs(v_), allowed).reshape(T, nq))
        xm = r.stage(reqs, l, "attn_resid").astype(np.float64)
        assert _rel(xm, x_in + att @ W["wo"].T) < 1e-5
        b = bf(r.stage(reqs, l, "mlp_norm"))
        assert _bf16_close(b, rmsnorm(xm, W["mlp_norm"], eps))
        h = bf(r.stage(reqs, l, "swiglu"))
        g = b @ W["w_gate"].T
        assert _bf16_close(h, g / (1 + np.exp(-g)) * (b @ W["w_up"].T))
        xo = r.stage(reqs, l, "layer_out").astype(np.float64)
        assert _rel(xo, xm + h @ W["w_down"].T) < 1e-5


def _rope_and_attention_checks(model, cfg, reqs, r, rows, L, K):
    """q/k norm + rotary and attention of layer 0 on the given packed rows of one
    request, each against the oracle's building block applied to the GPU's own
    input for that stage."""
    H, Hk, hd, eps = cfg.n_heads, cfg.n_kv_heads, cfg.head_dim, cfg.rms_eps
    nq, nk = H * hd, Hk * hd
    W = model.layers[0]
    pos = mis_positions(L, K)
    qkv = widen_bf16(r.stage(reqs, 0, "qkv"))
    qr = widen_bf16(r.stage(reqs, 0, "qk_rope"))
    n = rows.shape[0]
    q_ref = rope_rotate(rmsnorm(qkv[rows, :nq].reshape(n, H, hd), W["q_norm"], eps), pos[rows], cfg.rope_base)
    k_ref = rope_rotate(rmsnorm(qkv[rows, nq:nq + nk].reshape(n, Hk, hd), W["k_norm"], eps), pos[rows],
                        cfg.rope_base)
    assert _bf16_close(qr[rows, :nq], q_ref.reshape(n, nq))
    assert _bf16_close(qr[rows, nq:nq + nk], k_ref.reshape(n, nk))
    np.testing.assert_array_equal(qr[:, nq + nk:], qkv[:, nq + nk:])  # v untouched
    att = widen_bf16(r.stage(reqs, 0, "attn"))
    T = L + K
    allowed = tree_mask(L, K)[rows]
    q_, k_, v_ = qr[rows, :nq].reshape(n, H, hd), qr[:, nq:nq + nk].reshape(T, Hk, hd), qr[:, nq + nk:].reshape(T, Hk, hd)
    att_ref = attention(q_, k_, v_, allowed).reshape(n, nq)
    att_abs = attention(q_, k_, np.abs(v_), allowed).reshape(n, nq)
    assert _attn_close(att[rows], att_ref, att_abs)


def test_layer0_stress_shape_against_oracle(gpu_qwen):
    # L = 4096, K = 512 (the stress request): rotary up to position 4096, prefix
    # attention over 32 query tiles x 64 key tiles, branch tiles holding 128 of
    # the 512 candidates, checked on every 7th prefix row and every candidate
    cfg, w, D, model, r = gpu_qwen
    (p, c), = _batch(cfg, 5, 1)
    L, K = len(p), len(c)
    assert (L, K) == (4096, 512)
    rows = np.concatenate([np.arange(0, L, 7), np.arange(L - 64, L), np.arange(L, L + K)])
    _rope_and_attention_checks(model, cfg, [(p, c)], r, np.unique(rows), L, K)


def test_layer0_longest_prefix_against_oracle(gpu_qwen):
    # the longest accepted prefix (L = 32767): the last prefix rows and the
    # candidates, which sit at the rotary table's last position
    cfg, w, D, model, r = gpu_qwen
    (p, c), = _batch(cfg, 5, 1)
    L = r.dims.max_prefix
    prefix = np.resize(p, L).astype(np.int32)
    cands = c[[0, 255, 511]]
    rows = np.concatenate([np.arange(0, 64), np.arange(L - 200, L + 3)])
    _rope_and_attention_checks(model, cfg, [(prefix, cands)], r, rows, L, len(cands))
