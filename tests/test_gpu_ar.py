"""GPU parity of the autoregressive (AR) decode path (dg_ar_decode: one
token per row per step, causal, greedy) against the oracle's ar_decode,
through the C ABI: the tiny fp32 model end to end (graph and eager), and the
full-width bf16 layers teacher-forced step by step."""

import numpy as np
import pytest
import torch

from block_diffusion_decoding_tok_amd import dg
from block_diffusion_decoding_tok_amd.inputs import (TINY_DIMS, ModelDims, model_weights,
                                                     prompt_ids)
from oracle import prefill, ar_decode, model_forward
from oracle.attention import CAUSAL
from tests.util import oracle_model, empty_caches, rel_err_rows, to_f64

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _caches(dims, B, Tmax, dtype):
    shape = (B, dims.Hkv, Tmax, dims.dh)
    return ([torch.zeros(shape, dtype=dtype, device=DEV) for _ in range(dims.NL)],
            [torch.zeros(shape, dtype=dtype, device=DEV) for _ in range(dims.NL)])


def _tiny_ar(graphs, B=2, P0=20, n=8):
    d = TINY_DIMS
    w = model_weights(d, seed=1)
    m = oracle_model(d, w)
    Tmax = P0 + n + 4
    prompt = prompt_ids(B, P0, d.V, seed=3)
    first = torch.tensor([5, 300][:B], dtype=torch.int32)
    okc, ovc = empty_caches(d, B, Tmax)
    P = prefill(m, prompt.numpy(), okc, ovc)
    o_tok, o_P = ar_decode(m, first.numpy(), okc, ovc, P, n)
    # the oracle's top-2 logit gap of every step (near-ties may legitimately
    # pick the other id)
    seq = np.concatenate([prompt.numpy(), first.numpy()[:, None], o_tok[:, :-1]], axis=1)
    k2, v2 = empty_caches(d, B, Tmax)
    lg = model_forward(m, seq, k2, v2, np.zeros(B, np.int64), CAUSAL)[:, P0:]
    top2 = np.sort(lg, axis=2)[:, :, -2:]
    gap = top2[:, :, 1] - top2[:, :, 0]

    model = dg.DGModel(d, {k: v.to(DEV) for k, v in w.items()}, B, 16, dg.DG_F32, dg.DG_F32)
    model.set_graphs(graphs)
    kc, vc = _caches(d, B, Tmax, torch.float32)
    Pd = torch.zeros(B, dtype=torch.int32, device=DEV)
    stream = torch.cuda.Stream()
    with torch.cuda.stream(stream):
        dg.dg_prefill(model, prompt.to(DEV), kc, vc, Pd)
        tok = dg.dg_ar_decode(model, first.to(DEV), n, kc, vc, Pd)
        stream.synchronize()
    return dict(tok=tok.cpu().numpy(), P=Pd.cpu().numpy(), o_tok=o_tok, o_P=o_P, gap=gap,
                kc=[k.cpu().double().numpy() for k in kc], okc=okc, ovc=ovc,
                vc=[v.cpu().double().numpy() for v in vc])


@pytest.mark.parametrize("graphs", [True, False])
def test_tiny_ar_decode_matches_oracle(graphs):
    r = _tiny_ar(graphs)
    assert np.array_equal(r["P"], r["o_P"])
    # compare up to each row's first near-tie (after it the sequences may part)
    for b in range(r["tok"].shape[0]):
        near = np.nonzero(r["gap"][b] < 1e-5)[0]
        upto = near[0] + 1 if near.size else r["tok"].shape[1]
        assert np.array_equal(r["tok"][b, :upto], r["o_tok"][b, :upto]), b
        if not near.size:
            for l in range(len(r["kc"])):
                assert rel_err_rows(r["kc"][l][b], r["okc"][l][b]) < 1e-5
                assert rel_err_rows(r["vc"][l][b], r["ovc"][l][b]) < 1e-5


def test_tiny_ar_graph_equals_eager():
    a, b = _tiny_ar(True), _tiny_ar(False)
    assert np.array_equal(a["tok"], b["tok"])
    for l in range(len(a["kc"])):
        assert np.array_equal(a["kc"][l], b["kc"][l])


def test_full_width_ar_teacher_forced():
    """2 full-width layers (D 2816, fp8 experts, V 4096), tile-packed weights,
    batch 2 over a 256-token prompt: 4 single steps, each fed the oracle's
    previous token.  The device's greedy token must be a maximal logit of the
    oracle's to within the bf16 error of the logits; the K and V slots each
    step writes (the QKV projection's RoPE epilogue at one token per row)
    must match."""
    d = ModelDims(NL=2, D=2816, Hq=16, Hkv=8, dh=128, E=128, k=8, I=704, V=4096)
    w = model_weights(d, seed=5, expert_dtype="fp8", dense_dtype="bf16")
    m = oracle_model(d, w)
    dw = {}
    for k, v in w.items():
        v = v.to(DEV)
        dw[k] = v if (k == "emb" or k.startswith(("sgu", "sd"))) else dg.dg_pack_weights(v)
    model = dg.DGModel(d, dw, 2, 256, dg.DG_BF16, dg.DG_FP8_E4M3,
                       weight_layout=dg.DG_LAYOUT_TILED)
    B, P0, n = 2, 256, 4
    Tmax = P0 + n
    prompt = prompt_ids(B, P0, d.V, seed=7)
    kc, vc = _caches(d, B, Tmax, torch.bfloat16)
    Pd = torch.zeros(B, dtype=torch.int32, device=DEV)
    dg.dg_prefill(model, prompt.to(DEV), kc, vc, Pd)
    torch.cuda.synchronize()
    tok = np.array([11, 4000])
    for s in range(n):
        okc = [k.cpu().double().numpy() for k in kc]      # the device cache as input
        ovc = [v.cpu().double().numpy() for v in vc]
        P = Pd.cpu().numpy().astype(np.int64)
        logits = model_forward(m, tok[:, None], okc, ovc, P, CAUSAL)[:, 0]
        got = dg.dg_ar_decode(model, torch.from_numpy(tok.astype(np.int32)).to(DEV), 1, kc, vc,
                              Pd)
        torch.cuda.synchronize()
        g = got.cpu().numpy()[:, 0]
        tol = 0.05 * logits.std(axis=1)
        assert np.all(logits[np.arange(B), g] >= logits.max(axis=1) - tol), (s, g)
        assert Pd.cpu().tolist() == list(P + 1)
        for l in range(d.NL):
            slot_k = kc[l].cpu().double().numpy()[:, :, P[0]]
            slot_v = vc[l].cpu().double().numpy()[:, :, P[0]]
            assert rel_err_rows(slot_k, okc[l][:, :, P[0]]) < 3e-2
            assert rel_err_rows(slot_v, ovc[l][:, :, P[0]]) < 3e-2
        tok = np.argmax(logits, axis=1)                    # teacher forcing
