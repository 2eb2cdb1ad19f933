"""Pins of the attention oracle: torch's scaled_dot_product_attention in
float64 on the CPU (an independent library routine), RoPE as complex
rotation, and the invariants of canvas attention."""

import numpy as np
import pytest
import torch
import torch.nn.functional as F

from oracle.attention import attention, rope, CANVAS, CAUSAL


def _rand(rng, *shape):
    return rng.standard_normal(shape)


def test_rope_is_complex_rotation():
    rng = np.random.default_rng(0)
    n, H, dh = 7, 3, 8
    x = _rand(rng, n, H, dh)
    pos = rng.integers(0, 9000, n)
    got = rope(x, pos)
    half = dh // 2
    j = np.arange(half)
    ang = pos[:, None] * 10000.0 ** (-(2 * j) / dh)
    zc = (x[..., :half] + 1j * x[..., half:]) * np.exp(1j * ang)[:, None, :]
    assert np.allclose(got[..., :half], zc.real, atol=1e-12)
    assert np.allclose(got[..., half:], zc.imag, atol=1e-12)
    # norms preserved
    assert np.allclose(np.linalg.norm(got, axis=-1), np.linalg.norm(x, axis=-1))


def test_rope_relative_position():
    rng = np.random.default_rng(1)
    dh = 16
    q = _rand(rng, 1, 1, dh)
    k = _rand(rng, 1, 1, dh)
    for m, n, c in [(3, 10, 100), (0, 5, 4096), (77, 2, 9000)]:
        a = (rope(q, [m]) * rope(k, [n])).sum()
        b = (rope(q, [m + c]) * rope(k, [n + c])).sum()
        assert abs(a - b) < 1e-9


def _sdpa_reference(q, k_new, v_new, k_pre, v_pre, P, mode):
    """Independent path: oracle RoPE (pinned above) + torch SDPA in float64."""
    Lq, Hq, dh = q.shape
    Hkv = k_new.shape[1]
    pos = P + np.arange(Lq)
    qr = torch.from_numpy(rope(q, pos)).permute(1, 0, 2)           # [Hq, Lq, dh]
    kr = torch.from_numpy(rope(k_new, pos)).permute(1, 0, 2)
    K = torch.cat([torch.from_numpy(k_pre), kr], dim=1)            # [Hkv, P+Lq, dh]
    V = torch.cat([torch.from_numpy(v_pre), torch.from_numpy(v_new).permute(1, 0, 2)], dim=1)
    rep = Hq // Hkv
    K = K.repeat_interleave(rep, dim=0)
    V = V.repeat_interleave(rep, dim=0)
    mask = None
    if mode == CAUSAL:
        mask = torch.arange(P + Lq)[None, :] <= torch.from_numpy(pos)[:, None]
    o = F.scaled_dot_product_attention(qr[None], K[None], V[None], attn_mask=mask)
    return o[0].permute(1, 0, 2).numpy()


@pytest.mark.parametrize("mode", [CANVAS, CAUSAL])
@pytest.mark.parametrize("Lq,P,Hq,Hkv,dh", [(4, 5, 4, 2, 8), (6, 0, 2, 2, 4), (3, 9, 8, 2, 16)])
def test_attention_vs_torch_sdpa(mode, Lq, P, Hq, Hkv, dh):
    rng = np.random.default_rng(Lq * 100 + P)
    q = _rand(rng, Lq, Hq, dh)
    kn = _rand(rng, Lq, Hkv, dh)
    vn = _rand(rng, Lq, Hkv, dh)
    kp = _rand(rng, Hkv, P, dh)
    vp = _rand(rng, Hkv, P, dh)
    o, k_rot = attention(q, kn, vn, kp, vp, P, mode)
    ref = _sdpa_reference(q, kn, vn, kp, vp, P, mode)
    assert np.allclose(o, ref, atol=1e-12, rtol=1e-10)
    assert np.allclose(k_rot, rope(kn, P + np.arange(Lq)))


def test_permutation_equivariance_without_rope():
    rng = np.random.default_rng(2)
    Lq, P, Hq, Hkv, dh = 6, 5, 4, 2, 8
    q, kn, vn = _rand(rng, Lq, Hq, dh), _rand(rng, Lq, Hkv, dh), _rand(rng, Lq, Hkv, dh)
    kp, vp = _rand(rng, Hkv, P, dh), _rand(rng, Hkv, P, dh)
    perm = rng.permutation(Lq)
    o, _ = attention(q, kn, vn, kp, vp, P, CANVAS, rope_on=False)
    o2, _ = attention(q[perm], kn[perm], vn[perm], kp, vp, P, CANVAS, rope_on=False)
    assert np.allclose(o2, o[perm], atol=1e-12)


def test_equal_scores_give_mean_of_values():
    rng = np.random.default_rng(3)
    Lq, P, Hq, Hkv, dh = 3, 4, 2, 1, 8
    q = np.zeros((Lq, Hq, dh))
    kn, vn = _rand(rng, Lq, Hkv, dh), _rand(rng, Lq, Hkv, dh)
    kp, vp = _rand(rng, Hkv, P, dh), _rand(rng, Hkv, P, dh)
    o, _ = attention(q, kn, vn, kp, vp, P, CANVAS)
    allv = np.concatenate([vp[0], vn[:, 0]], axis=0)
    assert np.allclose(o[:, 0], allv.mean(axis=0)[None], atol=1e-12)
    oc, _ = attention(q, kn, vn, kp, vp, P, CAUSAL)
    for i in range(Lq):
        assert np.allclose(oc[i, 1], allv[:P + i + 1].mean(axis=0), atol=1e-12)


def test_prompt_rows_do_not_see_the_canvas():
    """Block-diagonal reading: prompt rows (prefilled causally) have the same
    outputs whatever canvas follows, and the canvas rows see the whole
    prefix.  Concatenating prompt+canvas in causal mode reproduces the
    prompt rows exactly."""
    rng = np.random.default_rng(4)
    Pn, Lc, Hq, Hkv, dh = 5, 4, 4, 2, 8
    qp, kp, vp = _rand(rng, Pn, Hq, dh), _rand(rng, Pn, Hkv, dh), _rand(rng, Pn, Hkv, dh)
    empty = np.zeros((Hkv, 0, dh))
    o_prompt, kp_rot = attention(qp, kp, vp, empty, empty, 0, CAUSAL)
    for seed in range(3):
        r2 = np.random.default_rng(100 + seed)
        qc, kc, vc = _rand(r2, Lc, Hq, dh), _rand(r2, Lc, Hkv, dh), _rand(r2, Lc, Hkv, dh)
        o_all, _ = attention(np.concatenate([qp, qc]), np.concatenate([kp, kc]),
                             np.concatenate([vp, vc]), empty, empty, 0, CAUSAL)
        assert np.allclose(o_all[:Pn], o_prompt, atol=1e-12)
    # canvas rows with the prefix in cache see all of it: same as one
    # non-causal pass over [prefix; canvas] restricted to the canvas rows
    oc, _ = attention(qc, kc, vc, kp_rot.transpose(1, 0, 2), vp.transpose(1, 0, 2), Pn, CANVAS)
    ref = _sdpa_reference(qc, kc, vc, kp_rot.transpose(1, 0, 2), vp.transpose(1, 0, 2), Pn, CANVAS)
    assert np.allclose(oc, ref, atol=1e-12)
