"""GPU parity of the MoE router and expert FFN against the oracle, through
the C ABI: bit-exact routing tables on identical logits; FFN outputs within
2e-2 (bf16 weights), 5e-2 (fp8 weights) and 1e-5 (f32) relative per token."""

import numpy as np
import pytest
import torch

from block_diffusion_decoding_tok_amd import dg
from block_diffusion_decoding_tok_amd.inputs import moe_case
from oracle.moe import moe_route, moe_ffn, expert_gate_up
from tests.util import ExpertWeights, rel_err_rows, to_f64, pack_tiled

pytestmark = pytest.mark.gpu
DEV = "cuda"
TOL = {"bf16": 2e-2, "fp8": 5e-2, "f32": 1e-5}


def _route_gpu(logits, k):
    ids, gates, off, rows = dg.dg_moe_route(logits.to(DEV), k)
    torch.cuda.synchronize()
    return ids.cpu().numpy(), gates.cpu().numpy(), off.cpu().numpy(), rows.cpu().numpy()


def _check_route(logits, k):
    ids, gates, off, rows = _route_gpu(logits, k)
    r_ids, r_gates, r_off, r_rows = moe_route(logits.double().numpy(), k)
    assert np.array_equal(ids, r_ids)
    assert np.array_equal(off, r_off)
    assert np.array_equal(rows, r_rows)
    assert np.allclose(gates, r_gates, rtol=2e-6, atol=1e-7)
    return ids, gates, off, rows


# up to 64 tokens the top-k and the sort run in one workgroup
# (route_fused_kernel), above that in two launches: both sides of the bound,
# one token (AR decode) and E > 128 on both paths
@pytest.mark.parametrize("T,E,k", [(256, 128, 8), (1024, 128, 8), (37, 5, 2), (300, 256, 16),
                                   (64, 1, 1), (10, 200, 3), (130, 128, 8), (64, 128, 8),
                                   (65, 128, 8), (1, 128, 8), (64, 256, 16), (2, 3, 3)])
def test_route_matches_oracle(T, E, k):
    rng = np.random.default_rng(T + E + k)
    logits = torch.from_numpy(rng.standard_normal((T, E)).astype(np.float32))
    logits[0, :] = 0.25                     # a fully tied row: lowest ids win
    _check_route(logits, k)


def test_route_planted_skew_share():
    case = moe_case(T=256, w_dtype="bf16", seed=0, D=128, I=64, E=128)
    ids, _, off, _ = _check_route(case.router_logits, 8)
    share = np.isin(ids, case.hot).mean()
    assert abs(share - 0.40) <= 0.005
    assert (np.diff(off) > 0).all()          # every expert receives tokens


def _ffn_case(case, k, sample=None, tiled=False):
    T, D = case.x.shape
    ids, gates, off, rows = _check_route(case.router_logits, k)
    y0 = torch.randn(T, D, generator=torch.Generator().manual_seed(1)) * 0.1
    y = y0.clone().to(DEV)
    xd = case.x.to(DEV)
    wgu, wd = case.w_gate_up.to(DEV), case.w_down.to(DEV)
    if tiled:
        wgu, wd = dg.dg_pack_weights(wgu), dg.dg_pack_weights(wd)
    sgu, sd = case.s_gate_up.to(DEV), case.s_down.to(DEV)
    dg.dg_moe_ffn(xd, wgu, wd, sgu, sd, torch.from_numpy(ids).to(DEV),
                  torch.from_numpy(gates).to(DEV), torch.from_numpy(off).to(DEV),
                  torch.from_numpy(rows).to(DEV), y,
                  w_layout=dg.DG_LAYOUT_TILED if tiled else dg.DG_LAYOUT_ROWMAJOR)
    torch.cuda.synchronize()
    got = (y.cpu() - y0).double().numpy()
    sel = np.arange(T) if sample is None else sample
    wg = ExpertWeights(case.w_gate_up, case.s_gate_up)
    wdn = ExpertWeights(case.w_down, case.s_down)
    ref = moe_ffn(to_f64(case.x)[sel], wg, wdn, ids[sel], gates[sel].astype(np.float64))
    return rel_err_rows(got[sel], ref), y


@pytest.mark.parametrize("w_dtype", ["bf16", "fp8"])
@pytest.mark.parametrize("tiled", [False, True])
def test_moe_ffn_full_size_bs1(w_dtype, tiled):
    case = moe_case(T=256, w_dtype=w_dtype, seed=0)
    err, _ = _ffn_case(case, 8, tiled=tiled)
    assert err < TOL[w_dtype], err


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.uint8])
def test_pack_weights_layout(dtype):
    g = torch.Generator().manual_seed(7)
    if dtype == torch.uint8:
        w = torch.randint(0, 256, (3, 48, 192), dtype=torch.uint8, generator=g)
        ref = pack_tiled(w.numpy())
        got = dg.dg_pack_weights(w.to(DEV)).cpu().numpy()
    else:
        w = torch.randn((3, 48, 192), generator=g).to(torch.bfloat16)
        ref = pack_tiled(w.view(torch.int16).numpy())
        got = dg.dg_pack_weights(w.to(DEV)).cpu().view(torch.int16).numpy()
    assert np.array_equal(got, ref)


@pytest.mark.parametrize("w_dtype", ["bf16", "fp8"])
@pytest.mark.parametrize("tiled", [False, True])
def test_moe_ffn_full_size_bs4_sampled(w_dtype, tiled):
    """Batch 4 of the MoE workload (1024 tokens, 128 experts, top-8): above 40
    tokens per expert on average, the LDS-staged 64-token tiles over the
    multi-expert (chunk-column) stack; 96 sampled tokens."""
    case = moe_case(T=1024, w_dtype=w_dtype, seed=1)
    sample = np.random.default_rng(0).choice(1024, 96, replace=False)
    err, _ = _ffn_case(case, 8, sample, tiled=tiled)
    assert err < TOL[w_dtype], err


@pytest.mark.parametrize("T", [1, 3, 8])
@pytest.mark.parametrize("tiled", [False, True])
@pytest.mark.parametrize("w_dtype", ["fp8", "bf16"])
def test_moe_ffn_full_size_few_tokens(T, tiled, w_dtype):
    """A few tokens (AR decode: T * k <= 64 slots): half-size work items."""
    case = moe_case(T=T, w_dtype=w_dtype, seed=20 + T, skew=False)
    err, _ = _ffn_case(case, 8, tiled=tiled)
    assert err < TOL[w_dtype], err



@pytest.mark.parametrize("tiled", [False, True])
def test_moe_ffn_full_size_bs2_fp8_sampled(tiled):
    """Between 20 and 40 tokens per expert on average: one-wave items with
    32-token tiles for gate/up and 16-token tiles for down."""
    case = moe_case(T=512, w_dtype="fp8", seed=4)
    sample = np.random.default_rng(1).choice(512, 96, replace=False)
    err, _ = _ffn_case(case, 8, sample, tiled=tiled)
    assert err < TOL["fp8"], err


@pytest.mark.parametrize("w_dtype", ["bf16", "fp8"])
@pytest.mark.parametrize("tiled", [False, True])
def test_moe_ffn_ragged_small(w_dtype, tiled):
    """Few tokens, experts with 0 and > 64 tokens, several row tiles."""
    case = moe_case(T=70, D=256, E=6, k=2, I=128, w_dtype=w_dtype, seed=5, skew=False)
    err, _ = _ffn_case(case, 2, tiled=tiled)
    assert err < TOL[w_dtype], err


@pytest.mark.parametrize("w_dtype", ["bf16", "fp8"])
@pytest.mark.parametrize("T", [30, 200])
def test_moe_ffn_single_expert_tiled(w_dtype, T):
    """One expert (a stack of one matrix keeps each tile's chunks together,
    unlike a stack of several): one-wave items at 30 slots, LDS-staged tiles
    at 200."""
    case = moe_case(T=T, D=256, E=1, k=1, I=128, w_dtype=w_dtype, seed=70 + T, skew=False)
    err, _ = _ffn_case(case, 1, tiled=True)
    assert err < TOL[w_dtype], err


@pytest.mark.parametrize("tiled", [False, True])
def test_moe_ffn_many_tokens_per_expert(tiled):
    """Above 40 tokens per expert the LDS-staged 64-token tiles take over."""
    case = moe_case(T=512, D=256, E=8, k=2, I=128, w_dtype="fp8", seed=6, skew=False)
    err, _ = _ffn_case(case, 2, tiled=tiled)
    assert err < TOL["fp8"], err


def test_moe_ffn_f32_tiny():
    case = moe_case(T=48, D=64, E=4, k=2, I=128, w_dtype="f32", seed=2, skew=False)
    err, _ = _ffn_case(case, 2)
    assert err < TOL["f32"], err


def test_moe_ffn_deterministic():
    case = moe_case(T=256, D=512, E=16, k=4, I=128, w_dtype="fp8", seed=3)
    _, y1 = _ffn_case(case, 4, sample=np.arange(4))
    _, y2 = _ffn_case(case, 4, sample=np.arange(4))
    assert torch.equal(y1, y2)


@pytest.mark.parametrize("T", [256, 512])
def test_moe_steps_compose_to_ffn(T):
    """gate/up -> down -> combine as three calls equals dg_moe_ffn bit for
    bit; the hidden rows h and the gate-weighted slot rows of a sample of
    sorted positions match the oracle's expert steps."""
    k = 8
    case = moe_case(T=T, w_dtype="fp8", seed=2)
    ids, gates, off, rows = _check_route(case.router_logits, k)
    D, I = case.x.shape[1], case.w_down.shape[2]
    xd = case.x.to(DEV)
    wgu, wd = dg.dg_pack_weights(case.w_gate_up.to(DEV)), dg.dg_pack_weights(case.w_down.to(DEV))
    sgu, sd = case.s_gate_up.to(DEV), case.s_down.to(DEV)
    t_ids, t_gates = torch.from_numpy(ids).to(DEV), torch.from_numpy(gates).to(DEV)
    t_off, t_rows = torch.from_numpy(off).to(DEV), torch.from_numpy(rows).to(DEV)
    kw = dict(w_layout=dg.DG_LAYOUT_TILED, E=case.w_down.shape[0], I=I)
    y_ffn = torch.zeros((T, D), device=DEV)
    dg.dg_moe_ffn(xd, wgu, wd, sgu, sd, t_ids, t_gates, t_off, t_rows, y_ffn, **kw)
    h = dg.dg_moe_gate_up(xd, wgu, sgu, t_off, t_rows, k, **kw)
    ys = dg.dg_moe_down(h, wd, sd, t_gates, t_off, t_rows, T, D, **kw)
    y3 = dg.dg_moe_combine(ys, k, torch.zeros((T, D), device=DEV))
    torch.cuda.synchronize()
    assert torch.equal(y_ffn, y3)

    wg, wdn = ExpertWeights(case.w_gate_up, case.s_gate_up), ExpertWeights(case.w_down, case.s_down)
    x64 = to_f64(case.x)
    h_got = to_f64(h.cpu())
    ys_got = to_f64(ys.cpu())
    sample = np.random.default_rng(3).choice(T * k, 48, replace=False)
    expert_of = np.searchsorted(off, sample, side="right") - 1
    for e in np.unique(expert_of):
        ps = sample[expert_of == e]
        slots = rows[ps]
        w = wg[e]
        h_ref = expert_gate_up(x64[slots // k], w[:I], w[I:])
        assert rel_err_rows(h_got[ps], h_ref) < 1e-2
        y_ref = gates.reshape(-1)[slots][:, None] * (h_ref @ wdn[e].T)
        assert rel_err_rows(ys_got[slots], y_ref) < TOL["fp8"]
