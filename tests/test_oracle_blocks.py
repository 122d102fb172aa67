"""Pins for the oracle's building blocks against closed forms, hand-computed
values and independent library routines (torch CPU, float64).

Each test is built so that a plausible slip in the oracle (a dropped gain, a
flipped rotation sign, a transposed projection, a wrong GQA head index, a
missing residual or scale) makes it fail.
"""
import math

import numpy as np
import pytest
import torch
import torch.nn.functional as F

from oracle import attention, layer_stages, mlp_swiglu, rmsnorm, rope_rotate, score_head, widen_bf16, widen_f16

RNG = np.random.default_rng(1234)


# ------------------------------------------------------- storage widening ---


def _special_bits():
    # zeros, smallest and largest subnormals and normals, one, infinities, a NaN,
    # then every pattern of a random draw
    fixed = [0x0000, 0x8000, 0x0001, 0x8001, 0x007F, 0x0080, 0x7F7F, 0xFF7F, 0x3F80, 0xBF80,
             0x7F80, 0xFF80, 0x7FC0, 0x03FF, 0x0400, 0x7BFF, 0x3C00, 0x7C00, 0xFC00, 0x7E00]
    return np.concatenate([np.array(fixed, np.uint16), RNG.integers(0, 1 << 16, 4096).astype(np.uint16)])


def _same_values(got, ref):
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])
    assert np.array_equal(np.signbit(got[~nan]), np.signbit(ref[~nan]))


def test_widen_bf16_matches_torch():
    # torch's own bfloat16 -> float64 conversion of the same bit patterns
    bits = _special_bits()
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    got = widen_bf16(bits)
    assert got.dtype == np.float64
    _same_values(got, ref)
    # hand values: 1.0, -2.0, the largest finite bf16 and the smallest subnormal
    assert widen_bf16(np.array([0x3F80, 0xC000, 0x7F7F, 0x0001], np.uint16)).tolist() == [
        1.0, -2.0, (2 - 2 ** -7) * 2.0 ** 127, 2.0 ** -133]


def test_widen_f16_matches_torch():
    bits = _special_bits()
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.float16).to(torch.float64).numpy()
    got = widen_f16(bits)
    assert got.dtype == np.float64
    _same_values(got, ref)
    assert widen_f16(np.array([0x3C00, 0xC000, 0x7BFF, 0x0001], np.uint16)).tolist() == [
        1.0, -2.0, 65504.0, 2.0 ** -24]


# ---------------------------------------------------------------- RMSNorm ---

def test_rmsnorm_constant_row_gives_gain():
    # x = c * 1 has RMS |c|, so RMSNorm(x) = sign(c) * g (eps = 0)
    g = RNG.standard_normal(64)
    for c in (0.25, 3.0, 1e-3):
        np.testing.assert_allclose(rmsnorm(np.full((2, 64), c), g, 0.0), np.tile(g, (2, 1)), rtol=1e-14)
    np.testing.assert_allclose(rmsnorm(np.full((1, 64), -2.0), g, 0.0)[0], -g, rtol=1e-14)


def test_rmsnorm_hand_value():
    # x = [3, 4]: mean square 12.5, rms = 3.5355339059327378; g = [1, 2]
    out = rmsnorm(np.array([[3.0, 4.0]]), np.array([1.0, 2.0]), 0.0)
    np.testing.assert_allclose(out, [[0.8485281374238570, 2.2627416997969522]], rtol=1e-14)
    # eps enters under the square root: x = [1, 1], eps = 3 -> 1/sqrt(4) = 0.5
    np.testing.assert_allclose(rmsnorm(np.array([[1.0, 1.0]]), np.ones(2), 3.0), [[0.5, 0.5]], rtol=1e-15)


def test_rmsnorm_matches_torch():
    x = RNG.standard_normal((7, 96))
    g = 1 + 0.1 * RNG.standard_normal(96)
    ref = F.rms_norm(torch.from_numpy(x), (96,), torch.from_numpy(g), eps=1e-6).numpy()
    np.testing.assert_allclose(rmsnorm(x, g, 1e-6), ref, rtol=1e-12, atol=1e-14)


# ------------------------------------------------------------------- RoPE ---

def test_rope_position_zero_is_identity():
    x = RNG.standard_normal((3, 2, 32))
    np.testing.assert_array_equal(rope_rotate(x, np.zeros(3), 1e6), x)


def test_rope_hand_values():
    # hd = 2: one pair, inverse frequency base^0 = 1.  e_0 at position 1 rotates
    # counter-clockwise by 1 rad: (cos 1, sin 1); e_1 goes to (-sin 1, cos 1).
    c1, s1 = 0.5403023058681398, 0.8414709848078965
    out = rope_rotate(np.array([[[1.0, 0.0]], [[0.0, 1.0]]]), np.array([1, 1]), 1e6)
    np.testing.assert_allclose(out[0, 0], [c1, s1], rtol=1e-15)
    np.testing.assert_allclose(out[1, 0], [-s1, c1], rtol=1e-15)
    # hd = 4, base = 100: pairs (0, 2) at frequency 1 and (1, 3) at frequency
    # 100^(-2/4) = 0.1.  Position 5: pair 1 rotates by 0.5 rad.
    c05, s05 = 0.8775825618903728, 0.4794255386042030
    out = rope_rotate(np.array([[[0.0, 2.0, 0.0, 0.0]]]), np.array([5]), 100.0)
    np.testing.assert_allclose(out[0, 0], [0.0, 2 * c05, 0.0, 2 * s05], atol=1e-15)


def test_rope_preserves_pair_norms_and_is_relative():
    hd = 32
    q = RNG.standard_normal((1, 1, hd))
    k = RNG.standard_normal((1, 1, hd))
    rq = rope_rotate(q, np.array([11]), 1e6)
    pair = lambda v: v[..., : hd // 2] ** 2 + v[..., hd // 2:] ** 2
    np.testing.assert_allclose(pair(rq), pair(q), rtol=1e-13)
    # <R(m) q, R(n) k> depends on m - n only
    dots = []
    for m, n in ((7, 3), (104, 100), (4, 0)):
        dots.append(float(np.sum(rope_rotate(q, np.array([m]), 1e4) * rope_rotate(k, np.array([n]), 1e4))))
    np.testing.assert_allclose(dots, dots[0], rtol=1e-12)


def test_rope_matches_complex_rotation():
    # Same rotation written as complex multiplication z * exp(i theta) with
    # z = x_i + i x_{i + hd/2}, in torch.
    hd, base = 32, 1e6
    x = RNG.standard_normal((5, 3, hd))
    pos = np.array([0, 1, 17, 450, 4096])
    theta = torch.from_numpy(pos.astype(np.float64))[:, None] * torch.pow(
        torch.tensor(base, dtype=torch.float64), -torch.arange(0, hd, 2, dtype=torch.float64) / hd)[None, :]
    xt = torch.from_numpy(x)
    z = torch.complex(xt[..., : hd // 2], xt[..., hd // 2:]) * torch.polar(torch.ones_like(theta), theta)[:, None, :]
    ref = torch.cat([z.real, z.imag], dim=-1).numpy()
    np.testing.assert_allclose(rope_rotate(x, pos, base), ref, rtol=1e-11, atol=1e-12)


# -------------------------------------------------------------- attention ---

def test_attention_constant_values_and_single_key():
    n, H, Hkv, hd = 6, 4, 2, 16
    q = RNG.standard_normal((n, H, hd))
    k = RNG.standard_normal((n, Hkv, hd))
    vrow = RNG.standard_normal((Hkv, hd))
    v = np.tile(vrow, (n, 1, 1))
    allowed = np.tril(np.ones((n, n), dtype=bool))
    out = attention(q, k, v, allowed)
    for h in range(H):
        np.testing.assert_allclose(out[:, h], np.tile(vrow[h // 2], (n, 1)), rtol=1e-13)
    # one visible key: its value row comes back unchanged
    v2 = RNG.standard_normal((n, Hkv, hd))
    only = np.zeros((n, n), dtype=bool)
    only[:, 3] = True
    out = attention(q, k, v2, only)
    for h in range(H):
        np.testing.assert_allclose(out[:, h], np.tile(v2[3, h // 2], (n, 1)), rtol=1e-13)


def test_attention_two_keys_hand_value():
    # one head, hd = 1 (scale 1): q = 1, keys 0 and ln 3 -> weights 1/4, 3/4
    q = np.array([[[1.0]]])
    k = np.array([[[0.0]], [[math.log(3.0)]]])
    v = np.array([[[2.0]], [[6.0]]])
    out = attention(q, k, v, np.ones((1, 2), dtype=bool))
    np.testing.assert_allclose(out[0, 0, 0], 0.25 * 2 + 0.75 * 6, rtol=1e-14)


def test_attention_gqa_matches_torch_sdpa():
    n, H, Hkv, hd = 9, 8, 2, 16
    q = RNG.standard_normal((n, H, hd))
    k = RNG.standard_normal((n, Hkv, hd))
    v = RNG.standard_normal((n, Hkv, hd))
    allowed = np.tril(np.ones((n, n), dtype=bool))
    allowed[6:, 5] = False  # an irregular mask, not just causal
    ref = F.scaled_dot_product_attention(
        torch.from_numpy(q).transpose(0, 1), torch.from_numpy(k).transpose(0, 1),
        torch.from_numpy(v).transpose(0, 1), attn_mask=torch.from_numpy(allowed),
        enable_gqa=True).transpose(0, 1).numpy()
    np.testing.assert_allclose(attention(q, k, v, allowed), ref, rtol=1e-11, atol=1e-13)


def test_attention_gqa_equals_mha_with_duplicated_kv():
    n, H, hd = 5, 4, 8
    q = RNG.standard_normal((n, H, hd))
    k = RNG.standard_normal((n, 2, hd))
    v = RNG.standard_normal((n, 2, hd))
    allowed = np.tril(np.ones((n, n), dtype=bool))
    kd = np.repeat(k, 2, axis=1)  # head h reads KV head h // 2
    vd = np.repeat(v, 2, axis=1)
    np.testing.assert_allclose(attention(q, k, v, allowed), attention(q, kd, vd, allowed), rtol=1e-14)


# -------------------------------------------------------------- MLP, head ---

def test_swiglu_hand_and_torch():
    # silu(1) = 1/(1+e^-1) = 0.7310585786300049, silu(-1) = -0.2689414213699951
    b = np.array([[1.0, -1.0]])
    eye = np.eye(2)
    out = mlp_swiglu(b, eye, np.full((2, 2), 0.5) * eye, eye)
    np.testing.assert_allclose(out, [[0.5 * 0.7310585786300049, -0.5 * -0.2689414213699951]], rtol=1e-14)
    d, f = 16, 40
    x = RNG.standard_normal((4, d))
    wg, wu, wd = RNG.standard_normal((f, d)), RNG.standard_normal((f, d)), RNG.standard_normal((d, f))
    t = lambda a: torch.from_numpy(a)
    ref = F.linear(F.silu(F.linear(t(x), t(wg))) * F.linear(t(x), t(wu)), t(wd)).numpy()
    np.testing.assert_allclose(mlp_swiglu(x, wg, wu, wd), ref, rtol=1e-12)


def test_score_head_closed_form(tiny_gains):
    cfg, _, _, model = tiny_gains
    # h = c * 1 -> RMSNorm gives g_final * c / sqrt(c^2 + eps), s = that . w
    s = score_head(model, np.full((2, cfg.d_model), 0.7))
    expect = np.sum(model.head * model.final_norm) * 0.7 / np.sqrt(0.49 + cfg.rms_eps)
    np.testing.assert_allclose(s, expect, rtol=1e-12)


# ------------------------------------------------- whole layer vs torch ops ---

def torch_layer(model, layer, x, pos, allowed):
    """One Qwen3-style block assembled from torch library calls (float64)."""
    cfg = model.cfg
    W = {k: torch.from_numpy(v) for k, v in model.layers[layer].items()}
    H, Hkv, hd, eps = cfg.n_heads, cfg.n_kv_heads, cfg.head_dim, cfg.rms_eps
    x = torch.from_numpy(x)
    n = x.shape[0]
    a = F.rms_norm(x, (cfg.d_model,), W["attn_norm"], eps)
    q = F.rms_norm(F.linear(a, W["wq"]).view(n, H, hd), (hd,), W["q_norm"], eps)
    k = F.rms_norm(F.linear(a, W["wk"]).view(n, Hkv, hd), (hd,), W["k_norm"], eps)
    v = F.linear(a, W["wv"]).view(n, Hkv, hd)
    theta = torch.from_numpy(np.asarray(pos, np.float64))[:, None] * torch.pow(
        torch.tensor(cfg.rope_base, dtype=torch.float64),
        -torch.arange(0, hd, 2, dtype=torch.float64) / hd)[None, :]
    rot = torch.polar(torch.ones_like(theta), theta)[:, None, :]

    def rope(t):
        z = torch.complex(t[..., : hd // 2], t[..., hd // 2:]) * rot
        return torch.cat([z.real, z.imag], dim=-1)

    q, k = rope(q), rope(k)
    o = F.scaled_dot_product_attention(q.transpose(0, 1), k.transpose(0, 1), v.transpose(0, 1),
                                       attn_mask=torch.from_numpy(allowed), enable_gqa=True)
    x = x + F.linear(o.transpose(0, 1).reshape(n, H * hd), W["wo"])
    b = F.rms_norm(x, (cfg.d_model,), W["mlp_norm"], eps)
    x = x + F.linear(F.silu(F.linear(b, W["w_gate"])) * F.linear(b, W["w_up"]), W["w_down"])
    return x.numpy()


@pytest.mark.parametrize("fixture", ["tiny", "tiny_gains"])
def test_layer_matches_torch_composition(fixture, request):
    from oracle import tree_mask
    from oracle.ranker import mis_positions
    cfg, _, _, model = request.getfixturevalue(fixture)
    L, K = 20, 5
    x = RNG.standard_normal((L + K, cfg.d_model)) * 0.05
    pos = mis_positions(L, K) + 3
    allowed = tree_mask(L, K)
    for layer in range(cfg.n_layers):
        ours = layer_stages(model, layer, x, pos, allowed)["x_out"]
        np.testing.assert_allclose(ours, torch_layer(model, layer, x, pos, allowed), rtol=1e-10, atol=1e-13)


# ------------------------------------------------- top-10 order criteria ---


def test_top10_strict_swaps():
    from parity import top10_strict_swaps
    ref = np.linspace(10.0, 0.0, 30)
    assert top10_strict_swaps(ref, ref) == 0
    g = ref.copy()
    g[[3, 4]] = g[[4, 3]]                        # adjacent swap inside the top 10
    assert top10_strict_swaps(g, ref) == 1
    g[[0, 7]] = g[[7, 0]]                        # first and eighth trade places as well
    assert top10_strict_swaps(g, ref) > 2
    g3 = ref.copy()
    g3[[20, 21]] = g3[[21, 20]]                  # a swap below the top 10 does not count
    assert top10_strict_swaps(g3, ref) == 0
    g4 = ref.copy()
    g4[[9, 10]] = g4[[10, 9]]                    # 10th and 11th trade places
    assert top10_strict_swaps(g4, ref) == 1
    assert top10_strict_swaps(ref + 0.001 * np.arange(30) / 30, ref) == 0  # shifts that keep the order
