"""GPU parity of the MXFP4 expert-weight path against the oracle, through the
C ABI: the device quantizer bit-exact against the oracle's OCP conversion,
the tiled pack byte-exact, and the expert FFN with MXFP4 weights within 2e-2
relative per token of the oracle's FFN on the exactly decoded weights (the
kernel decodes the same exact values; activations are bf16 as on the bf16
path)."""

import numpy as np
import pytest
import torch

from block_diffusion_decoding_tok_amd import dg
from block_diffusion_decoding_tok_amd.inputs import moe_case, mxfp4_random, _rngs
from oracle.moe import moe_route, moe_ffn, expert_gate_up
from oracle.mxfp4 import quantize_mxfp4
from tests.util import Mx4ExpertWeights, rel_err_rows, to_f64, pack_mxfp4_tiled

pytestmark = pytest.mark.gpu
DEV = "cuda"
TOL = 2e-2


def _special_rows(K):
    """Rows that hit the quantizer's edge cases: an all-zero block, exact
    round-half-to-even midpoints, saturation, negative zero and values that
    round to a signed zero, a subnormal amax, huge and tiny magnitudes."""
    rows = []
    z = np.zeros(K, np.float32)
    rows.append(z.copy())
    r = z.copy()
    mids = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 7.0, -0.25, -0.75, -5.0, -7.0,
                     6.0, 4.0, -0.0, -0.1], np.float32)
    for b in range(K // 32):
        r[b * 32:b * 32 + 16] = mids * np.float32(2.0 ** (b - 3))
    rows.append(r)
    r = z.copy()
    r[:32] = np.float32(1e-41)                     # subnormal block
    r[32:64] = np.float32(3e38) * np.linspace(-1, 1, 32, dtype=np.float32)
    r[64:96] = np.float32(2.0 ** -123) * np.arange(32, dtype=np.float32)
    rows.append(r)
    return np.stack(rows)


@pytest.mark.parametrize("rows,K", [(300, 2816), (7, 96), (1, 32)])
def test_quantize_mxfp4_matches_oracle(rows, K):
    rng = np.random.default_rng(rows + K)
    w = (rng.standard_normal((rows, K)) * 0.02).astype(np.float32)
    if K >= 96:
        sp = _special_rows(K)
        w[:sp.shape[0]] = sp
    codes, scales = dg.dg_quantize_mxfp4(torch.from_numpy(w).to(DEV))
    torch.cuda.synchronize()
    r_codes, r_scales = quantize_mxfp4(w.astype(np.float64))
    assert np.array_equal(scales.cpu().numpy(), r_scales)
    assert np.array_equal(codes.cpu().numpy(), r_codes)


@pytest.mark.parametrize("G,N,K", [(3, 48, 192), (1, 16, 64), (2, 1408, 2816)])
def test_pack_mxfp4_layout(G, N, K):
    codes, scales = mxfp4_random(np.random.default_rng(G * N + K), (G, N, K), spread=50)
    got = dg.dg_pack_mxfp4(codes.to(DEV), scales.to(DEV)).cpu().numpy()
    assert got.size == dg.mxfp4_tiled_bytes(G, N, K)
    assert np.array_equal(got, pack_mxfp4_tiled(codes.numpy(), scales.numpy()))


def _ffn_case_mx4(case, k, sample=None):
    T, D = case.x.shape
    E = case.w_gate_up.shape[0]
    I = case.w_down.shape[2] * 2
    logits = case.router_logits
    ids, gates, off, rows = dg.dg_moe_route(logits.to(DEV), k)
    torch.cuda.synchronize()
    ids, gates, off, rows = (t.cpu().numpy() for t in (ids, gates, off, rows))
    r_ids, _, r_off, r_rows = moe_route(logits.double().numpy(), k)
    assert np.array_equal(ids, r_ids) and np.array_equal(off, r_off)
    assert np.array_equal(rows, r_rows)
    wgu = dg.dg_pack_mxfp4(case.w_gate_up.to(DEV), case.s_gate_up.to(DEV))
    wd = dg.dg_pack_mxfp4(case.w_down.to(DEV), case.s_down.to(DEV))
    y0 = torch.randn(T, D, generator=torch.Generator().manual_seed(1)) * 0.1
    y = y0.clone().to(DEV)
    dg.dg_moe_ffn(case.x.to(DEV), wgu, wd, None, None, torch.from_numpy(ids).to(DEV),
                  torch.from_numpy(gates).to(DEV), torch.from_numpy(off).to(DEV),
                  torch.from_numpy(rows).to(DEV), y, w_layout=dg.DG_LAYOUT_TILED, E=E, I=I,
                  w_dtype=dg.DG_MXFP4)
    torch.cuda.synchronize()
    got = (y.cpu() - y0).double().numpy()
    sel = np.arange(T) if sample is None else sample
    wg = Mx4ExpertWeights(case.w_gate_up, case.s_gate_up)
    wdn = Mx4ExpertWeights(case.w_down, case.s_down)
    ref = moe_ffn(to_f64(case.x)[sel], wg, wdn, ids[sel], gates[sel].astype(np.float64))
    return rel_err_rows(got[sel], ref), y


def test_moe_ffn_mxfp4_full_size_bs1():
    case = moe_case(T=256, w_dtype="mxfp4", seed=0)
    err, _ = _ffn_case_mx4(case, 8)
    assert err < TOL, err


@pytest.mark.parametrize("T", [512, 1024])
def test_moe_ffn_mxfp4_full_size_sampled(T):
    """bs2 (32-token gate/up tiles) and bs4 (above 40 tokens per expert:
    LDS-staged 64-token tiles for both GEMMs)."""
    case = moe_case(T=T, w_dtype="mxfp4", seed=T)
    sample = np.random.default_rng(T).choice(T, 96, replace=False)
    err, _ = _ffn_case_mx4(case, 8, sample)
    assert err < TOL, err


@pytest.mark.parametrize("T", [1, 3, 8])
def test_moe_ffn_mxfp4_few_tokens(T):
    case = moe_case(T=T, w_dtype="mxfp4", seed=40 + T, skew=False)
    err, _ = _ffn_case_mx4(case, 8)
    assert err < TOL, err


def test_moe_ffn_mxfp4_ragged_small():
    """Few tokens, experts with 0 and > 64 tokens, several row tiles."""
    case = moe_case(T=70, D=256, E=6, k=2, I=128, w_dtype="mxfp4", seed=5, skew=False)
    err, _ = _ffn_case_mx4(case, 2)
    assert err < TOL, err


def test_moe_ffn_mxfp4_many_tokens_per_expert():
    """Above 40 slots per expert (LDS-staged 64-token tiles) at small widths,
    with ragged token tiles per expert."""
    case = moe_case(T=400, D=256, E=6, k=2, I=128, w_dtype="mxfp4", seed=6, skew=False)
    err, _ = _ffn_case_mx4(case, 2)
    assert err < TOL, err


def test_moe_ffn_mxfp4_quantized_normal_weights():
    """N(0, 0.02) weights quantized by the oracle (the value distribution the
    model's experts have), 16 experts, D 512, FFN 256."""
    T, D, E, k, I = 200, 512, 16, 4, 256
    r = _rngs(77, ["x", "router", "wgu", "wd"])
    x = torch.from_numpy(r["x"].standard_normal((T, D), dtype=np.float32)).to(torch.bfloat16)
    logits = torch.from_numpy(r["router"].standard_normal((T, E), dtype=np.float32))
    qgu, sgu = quantize_mxfp4(r["wgu"].standard_normal((E, 2 * I, D)) * 0.02)
    qd, sd = quantize_mxfp4(r["wd"].standard_normal((E, D, I)) * 0.02)

    class Case:
        pass
    case = Case()
    case.x, case.router_logits = x, logits
    case.w_gate_up, case.s_gate_up = torch.from_numpy(qgu), torch.from_numpy(sgu)
    case.w_down, case.s_down = torch.from_numpy(qd), torch.from_numpy(sd)
    err, _ = _ffn_case_mx4(case, k)
    assert err < TOL, err


def test_moe_steps_compose_mxfp4():
    """gate/up -> down -> combine as three calls equals dg_moe_ffn bit for
    bit, and sampled hidden rows match the oracle's expert gate/up."""
    T, k = 256, 8
    case = moe_case(T=T, w_dtype="mxfp4", seed=9)
    D = case.x.shape[1]
    E, I = case.w_gate_up.shape[0], case.w_down.shape[2] * 2
    ids, gates, off, rows = dg.dg_moe_route(case.router_logits.to(DEV), k)
    wgu = dg.dg_pack_mxfp4(case.w_gate_up.to(DEV), case.s_gate_up.to(DEV))
    wd = dg.dg_pack_mxfp4(case.w_down.to(DEV), case.s_down.to(DEV))
    xd = case.x.to(DEV)
    kw = dict(w_layout=dg.DG_LAYOUT_TILED, E=E, I=I, w_dtype=dg.DG_MXFP4)
    y_ffn = torch.zeros((T, D), device=DEV)
    dg.dg_moe_ffn(xd, wgu, wd, None, None, ids, gates, off, rows, y_ffn, **kw)
    h = dg.dg_moe_gate_up(xd, wgu, None, off, rows, k, **kw)
    ys = dg.dg_moe_down(h, wd, None, gates, off, rows, T, D, **kw)
    y3 = dg.dg_moe_combine(ys, k, torch.zeros((T, D), device=DEV))
    torch.cuda.synchronize()
    assert torch.equal(y_ffn, y3)
    off, rows = off.cpu().numpy(), rows.cpu().numpy()
    wg = Mx4ExpertWeights(case.w_gate_up, case.s_gate_up)
    x64, h_got = to_f64(case.x), to_f64(h.cpu())
    sample = np.random.default_rng(3).choice(T * k, 48, replace=False)
    expert_of = np.searchsorted(off, sample, side="right") - 1
    for e in np.unique(expert_of):
        ps = sample[expert_of == e]
        w = wg[e]
        h_ref = expert_gate_up(x64[rows[ps] // k], w[:I], w[I:])
        assert rel_err_rows(h_got[ps], h_ref) < 1e-2
