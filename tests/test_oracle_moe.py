"""Pins of the MoE oracle: brute-force routing, dense masked sum, textbook
gated FFN through torch, fp8 decode through torch's float8_e4m3fn."""

import numpy as np
import pytest
import torch
import torch.nn.functional as F

from oracle.moe import (fp8_e4m3fn_decode, gelu_erf, moe_route, moe_ffn,
                        moe_ffn_dense_masked)


def test_fp8_decode_matches_torch():
    b = torch.arange(256, dtype=torch.uint8)
    ref = b.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = fp8_e4m3fn_decode(b.numpy())
    nan = np.isnan(ref)
    assert np.array_equal(nan, np.isnan(got))
    assert np.array_equal(got[~nan], ref[~nan])
    assert np.nanmax(got) == 448.0 and got[1] == 2.0 ** -9


def test_gelu_matches_torch():
    x = np.linspace(-8, 8, 2001)
    ref = F.gelu(torch.from_numpy(x), approximate="none").numpy()
    assert np.allclose(gelu_erf(x), ref, atol=1e-15, rtol=1e-13)


def test_route_brute_force():
    rng = np.random.default_rng(0)
    T, E, k = 50, 16, 4
    r = rng.standard_normal((T, E)).astype(np.float32).astype(np.float64)
    r[3, :] = 0.5                    # all ties: lowest ids win
    r[7, [2, 9]] = r[7].max() + 1    # a tie at the top
    ids, gates, off, rows = moe_route(r, k)
    assert list(ids[3]) == [0, 1, 2, 3]
    assert list(ids[7][:2]) == [2, 9]
    for t in range(T):
        order = np.lexsort((np.arange(E), -r[t]))    # key: logit desc, then id
        assert list(ids[t]) == list(order[:k])
        full = np.exp(r[t] - r[t].max())
        full /= full.sum()
        sel = full[ids[t]]
        assert np.allclose(gates[t], sel / sel.sum(), atol=1e-15)
        assert abs(gates[t].sum() - 1) < 1e-14
    flat = ids.reshape(-1)
    assert np.array_equal(rows, np.argsort(flat, kind="stable"))
    assert np.array_equal(off, np.concatenate([[0], np.cumsum(np.bincount(flat, minlength=E))]))
    # k = E: gates are the full softmax in id order after sorting
    ids_all, g_all, _, _ = moe_route(r, E)
    full = np.exp(r - r.max(axis=1, keepdims=True))
    full /= full.sum(axis=1, keepdims=True)
    assert np.allclose(np.take_along_axis(full, ids_all, 1), g_all, atol=1e-15)


def _weights(rng, E, I, D, s=0.3):
    return rng.standard_normal((E, 2 * I, D)) * s, rng.standard_normal((E, D, I)) * s


def test_moe_equals_dense_masked_sum():
    rng = np.random.default_rng(1)
    T, D, E, k, I = 37, 12, 6, 2, 10
    u = rng.standard_normal((T, D))
    wgu, wd = _weights(rng, E, I, D)
    ids, gates, _, _ = moe_route(rng.standard_normal((T, E)), k)
    assert np.allclose(moe_ffn(u, wgu, wd, ids, gates),
                       moe_ffn_dense_masked(u, wgu, wd, ids, gates), atol=1e-12)


def test_single_expert_is_textbook_ffn():
    rng = np.random.default_rng(2)
    T, D, I = 9, 8, 16
    u = rng.standard_normal((T, D))
    wgu, wd = _weights(rng, 1, I, D)
    ids, gates, _, _ = moe_route(np.zeros((T, 1)), 1)
    assert np.allclose(gates, 1.0)
    ut, g, up, dn = (torch.from_numpy(a) for a in (u, wgu[0, :I], wgu[0, I:], wd[0]))
    ref = (F.gelu(ut @ g.T) * (ut @ up.T)) @ dn.T
    assert np.allclose(moe_ffn(u, wgu, wd, ids, gates), ref.numpy(), atol=1e-12)


def test_token_permutation_equivariance():
    rng = np.random.default_rng(3)
    T, D, E, k, I = 20, 8, 5, 3, 6
    u = rng.standard_normal((T, D))
    r = rng.standard_normal((T, E))
    wgu, wd = _weights(rng, E, I, D)
    perm = rng.permutation(T)
    ids, gates, _, _ = moe_route(r, k)
    ids2, gates2, _, _ = moe_route(r[perm], k)
    y = moe_ffn(u, wgu, wd, ids, gates)
    y2 = moe_ffn(u[perm], wgu, wd, ids2, gates2)
    assert np.allclose(y2, y[perm], atol=1e-12)
