"""Pin of the oracle's decoder-layer composition (R17, R18: pre-norm layers,
fused q | k | v rows, attention residual, router and MoE residual; [TR]
"DiffusionGemma의 구성") against a layer composed independently from torch
library calls in float64: F.rms_norm, F.linear, RoPE as a complex rotation,
F.scaled_dot_product_attention with the KV heads repeated per query group,
torch.topk on tie-free router logits, F.gelu (erf form), F.embedding.

Also two structural closed forms: with zero O-projection and zero experts
the layer is the identity; with zero experts it is exactly x + o Wo^T.

Weights are drawn with std 0.3 so that every branch moves the output far
more than the 1e-12 tolerance: a dropped residual, a norm placed after its
sublayer, swapped k / v rows or a transposed operand fails."""

import numpy as np
import pytest
import torch
import torch.nn.functional as F

from oracle import layer_forward, model_forward, TinyModel
from oracle.attention import CANVAS, CAUSAL

# D differs from Hq * dh, and E, k, I are small but not degenerate
D, HQ, HKV, DH, E, K, I, V = 24, 4, 2, 8, 4, 2, 16, 40
THETA = 10000.0
TOL = 1e-12


def _weights(rng, std=0.3):
    return dict(
        wqkv=rng.standard_normal(((HQ + 2 * HKV) * DH, D)) * std,
        wo=rng.standard_normal((D, HQ * DH)) * std,
        wr=rng.standard_normal((E, D)) * std,
        w_gate_up=rng.standard_normal((E, 2 * I, D)) * std,
        w_down=rng.standard_normal((E, D, I)) * std)


def _t(a):
    return torch.from_numpy(np.asarray(a, np.float64))


def _rope_complex(x, pos):
    """x [..., n, dh] rotated at positions pos [n]: the pairs (j, j + dh/2) as
    the complex numbers x_j + i x_{j+dh/2}, times exp(i pos theta^(-2j/dh))."""
    half = x.shape[-1] // 2
    z = torch.complex(x[..., :half], x[..., half:])
    j = torch.arange(half, dtype=torch.float64)
    ang = _t(pos)[:, None] * THETA ** (-2.0 * j / x.shape[-1])
    z = z * torch.polar(torch.ones_like(ang), ang)
    return torch.cat([z.real, z.imag], dim=-1)


def _torch_layer(lw, x, kc, vc, P, mode, router_logits=None):
    """Reference layer; returns (x_out, k_cache, v_cache) as new tensors."""
    x = _t(x)
    kc, vc = _t(kc).clone(), _t(vc).clone()
    B, n, _ = x.shape
    qd, kd = HQ * DH, HKV * DH
    h = F.rms_norm(x, (D,), eps=1e-6)
    qkv = F.linear(h, _t(lw["wqkv"]))
    q = qkv[..., :qd].reshape(B, n, HQ, DH).transpose(1, 2)
    k = qkv[..., qd:qd + kd].reshape(B, n, HKV, DH).transpose(1, 2)
    v = qkv[..., qd + kd:].reshape(B, n, HKV, DH).transpose(1, 2)
    o = torch.zeros(B, HQ, n, DH, dtype=torch.float64)
    for b in range(B):
        p = int(P[b])
        pos = np.arange(p, p + n)
        qr = _rope_complex(q[b], pos)
        kr = _rope_complex(k[b], pos)
        kc[b, :, p:p + n] = kr
        vc[b, :, p:p + n] = v[b]
        keys = kc[b, :, :p + n].repeat_interleave(HQ // HKV, dim=0)
        vals = vc[b, :, :p + n].repeat_interleave(HQ // HKV, dim=0)
        mask = None
        if mode == CAUSAL:
            mask = torch.arange(p + n)[None, :] <= torch.from_numpy(pos)[:, None]
        o[b] = F.scaled_dot_product_attention(qr[None], keys[None], vals[None],
                                              attn_mask=mask)[0]
    x1 = x + F.linear(o.transpose(1, 2).reshape(B, n, qd), _t(lw["wo"]))
    h2 = F.rms_norm(x1, (D,), eps=1e-6).reshape(B * n, D)
    r = F.linear(h2, _t(lw["wr"])) if router_logits is None else _t(router_logits)
    top, ids = torch.topk(r, K, dim=1)
    g = torch.softmax(top, dim=1)
    y = torch.zeros(B * n, D, dtype=torch.float64)
    wgu, wd = _t(lw["w_gate_up"]), _t(lw["w_down"])
    for t in range(B * n):
        for j in range(K):
            e = int(ids[t, j])
            u = h2[t]
            hid = F.gelu(F.linear(u, wgu[e, :I])) * F.linear(u, wgu[e, I:])
            y[t] += g[t, j] * F.linear(hid, wd[e])
    return x1 + y.reshape(B, n, D), kc, vc


def _case(seed, B=2, n=5, Tmax=16):
    rng = np.random.default_rng(seed)
    lw = _weights(rng)
    x = rng.standard_normal((B, n, D))
    P = np.array([3, 6])[:B]
    kc = np.zeros((B, HKV, Tmax, DH))
    vc = np.zeros((B, HKV, Tmax, DH))
    for b in range(B):                      # cached prefix: already rotated keys
        kc[b, :, :P[b]] = rng.standard_normal((HKV, P[b], DH))
        vc[b, :, :P[b]] = rng.standard_normal((HKV, P[b], DH))
    return rng, lw, x, P, kc, vc


def _tie_free(r):
    srt = np.sort(np.asarray(r), axis=1)
    return np.all(np.diff(srt, axis=1) > 1e-9)


@pytest.mark.parametrize("mode", [CANVAS, CAUSAL])
@pytest.mark.parametrize("override", [False, True])
def test_layer_forward_matches_torch_composition(mode, override):
    rng, lw, x, P, kc, vc = _case(1 + mode + 2 * override)
    B, n = x.shape[:2]
    rl = rng.standard_normal((B * n, E)) * 2.0 if override else None
    x_ref, k_ref, v_ref = _torch_layer(lw, x, kc, vc, P, mode, rl)
    kc_o, vc_o = kc.copy(), vc.copy()
    trace = []
    x_o = layer_forward(_model([lw]), lw, x, kc_o, vc_o, P, mode, trace=trace,
                        router_logits=rl)
    assert _tie_free(trace[0]["router_logits"])
    assert np.abs(x_o - x_ref.numpy()).max() < TOL
    assert np.abs(kc_o - k_ref.numpy()).max() < TOL
    assert np.abs(vc_o - v_ref.numpy()).max() < TOL
    # every sublayer moved the stream by far more than the tolerance
    assert np.abs(x_o - x).max() > 1e-2


def _model(layers):
    rng = np.random.default_rng(99)
    m = TinyModel(D=D, Hq=HQ, Hkv=HKV, dh=DH, E=E, k=K, I=I, V=V,
                  emb=rng.standard_normal((V, D)), lm=rng.standard_normal((V, D)) * 0.3)
    m.layers = list(layers)
    return m


@pytest.mark.parametrize("mode", [CANVAS, CAUSAL])
def test_model_forward_matches_torch_composition(mode):
    rng = np.random.default_rng(7 + mode)
    layers = [_weights(rng), _weights(rng)]
    m = _model(layers)
    B, n, Tmax = 2, 4, 16
    P = np.array([2, 5])
    tokens = rng.integers(0, V, size=(B, n))
    kcs = [np.zeros((B, HKV, Tmax, DH)) for _ in layers]
    vcs = [np.zeros((B, HKV, Tmax, DH)) for _ in layers]
    for l in range(len(layers)):
        for b in range(B):
            kcs[l][b, :, :P[b]] = rng.standard_normal((HKV, P[b], DH))
            vcs[l][b, :, :P[b]] = rng.standard_normal((HKV, P[b], DH))
    kcs_ref = [k.copy() for k in kcs]
    vcs_ref = [v.copy() for v in vcs]
    logits = model_forward(m, tokens, kcs, vcs, P, mode)
    x = F.embedding(torch.from_numpy(tokens), _t(m.emb)).numpy()
    for l, lw in enumerate(layers):
        xt, kr, vr = _torch_layer(lw, x, kcs_ref[l], vcs_ref[l], P, mode)
        x = xt.numpy()
        assert np.abs(kcs[l] - kr.numpy()).max() < TOL
        assert np.abs(vcs[l] - vr.numpy()).max() < TOL
    ref = F.linear(F.rms_norm(_t(x), (D,), eps=1e-6), _t(m.lm)).numpy()
    assert np.abs(logits - ref).max() < TOL


def test_zero_sublayers_give_the_identity():
    """wo = 0 and every expert 0: both residual branches add exactly zero."""
    _, lw, x, P, kc, vc = _case(11)
    lw = dict(lw, wo=np.zeros_like(lw["wo"]), w_gate_up=np.zeros_like(lw["w_gate_up"]),
              w_down=np.zeros_like(lw["w_down"]))
    out = layer_forward(_model([lw]), lw, x, kc, vc, P, CANVAS)
    assert np.array_equal(out, x)


def test_zero_experts_give_x_plus_attention_projection():
    """Every expert 0: the layer is exactly x + o Wo^T, with o the attention of
    the normalized stream (torch SDPA on the complex-rotated q and k)."""
    _, lw, x, P, kc, vc = _case(12)
    lw = dict(lw, w_gate_up=np.zeros_like(lw["w_gate_up"]), w_down=np.zeros_like(lw["w_down"]))
    ref, _, _ = _torch_layer(lw, x, kc, vc, P, CANVAS)     # MoE adds 0 here too
    out = layer_forward(_model([lw]), lw, x, kc.copy(), vc.copy(), P, CANVAS)
    assert np.abs(out - ref.numpy()).max() < TOL
    assert np.abs(out - x).max() > 1e-2                      # the attention branch is live
