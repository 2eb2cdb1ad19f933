"""GPU parity of the deferred block commit (dg_denoise_block_deferred,
dg_commit_pending) through the C ABI.

A deferred block leaves its commit forward to the next block, whose first
step runs one forward over the pending block followed by the new canvas
with a block-causal mask: the pending block sees the cache before it and
itself (its commit forward), the canvas sees the cache, the pending block
and itself (its first step).

  * the tiny fp32 model: three deferred blocks and the final commit against
    the oracle's three blocks, each denoised and then committed: tokens and
    steps bit-exact (near-ties of the final step excepted, as for one block),
    prefix lengths equal, caches within 1e-5.  With graphs and without.
  * two full-width layers (bf16 dense, fp8 experts, tiled weights), batch 2:
    three deferred blocks and the commit; the caches they leave must equal,
    within the bf16 tolerance, a re-forward of every block's final tokens
    through the plain forward (dg_model_forward over each block at its own
    prefix), and the first block's tokens must equal those of an undeferred
    run bit for bit (both run the same steps).  The routing is a planted
    override that repeats every L rows, so a token routes the same in the
    fused 2L-row forward and in an L-row forward (with the model's own router
    the different kernel shapes' bf16 rounding flips the top-8 of a few
    tokens at near-ties, a few percent of the rows).
  * while a commit is pending every other decoder call fails.
"""

import numpy as np
import pytest
import torch

from block_diffusion_decoding_tok_amd import dg
from block_diffusion_decoding_tok_amd.inputs import (TINY_DIMS, ModelDims, model_weights, prompt_ids,
                                                     router_logits_skewed)
from oracle import SamplerCfg, prefill, denoise_block
from tests.util import oracle_model, empty_caches, rel_err_rows

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _caches(dims, B, Tmax, dtype):
    shape = (B, dims.Hkv, Tmax, dims.dh)
    return ([torch.zeros(shape, dtype=dtype, device=DEV) for _ in range(dims.NL)],
            [torch.zeros(shape, dtype=dtype, device=DEV) for _ in range(dims.NL)])


@pytest.mark.parametrize("graphs", [True, False])
def test_deferred_blocks_tiny_match_oracle(graphs):
    d = TINY_DIMS
    B, L, P0, nb = 2, 16, 32, 3
    w = model_weights(d, seed=0)
    m = oracle_model(d, w)
    Tmax = P0 + nb * L
    prompt = prompt_ids(B, P0, d.V, seed=0)
    okc, ovc = empty_caches(d, B, Tmax)
    P = prefill(m, prompt.numpy(), okc, ovc)
    ocfgs = [SamplerCfg(canvas_len=L, max_steps=8, fixed_steps=3, seed=5 + blk) for blk in range(nb)]
    oracle_blocks = []
    for ocfg in ocfgs:
        o_tok, o_steps, trace, P = denoise_block(m, ocfg, okc, ovc, P)
        oracle_blocks.append((o_tok, o_steps, trace))

    # the fused first step runs 2 L tokens per row: a prefill limit of 2 B L
    model = dg.DGModel(d, {k: v.to(DEV) for k, v in w.items()}, B, L, dg.DG_F32, dg.DG_F32,
                       max_prefill_tokens=2 * B * L)
    model.set_graphs(graphs)
    kc, vc = _caches(d, B, Tmax, torch.float32)
    Pd = torch.zeros(B, dtype=torch.int32, device=DEV)
    stream = torch.cuda.Stream()
    got = []
    with torch.cuda.stream(stream):
        dg.dg_prefill(model, prompt.to(DEV), kc, vc, Pd)
        for blk, ocfg in enumerate(ocfgs):
            gcfg = dg.sampler_cfg(L, ocfg.max_steps, ocfg.fixed_steps, seed=ocfg.seed)
            tok = torch.full((B, L), -1, dtype=torch.int32, device=DEV)
            steps = torch.full((B,), -1, dtype=torch.int32, device=DEV)
            dg.dg_denoise_block_deferred(model, gcfg, B, kc, vc, Pd, tok, steps)
            got.append((tok, steps))
            if blk == 0:
                # a pending commit blocks every other decoder call
                with pytest.raises(RuntimeError, match="pending"):
                    dg.dg_denoise_block(model, gcfg, B, kc, vc, Pd, tok, steps)
        dg.dg_commit_pending(model, B, kc, vc, Pd)
        dg.dg_commit_pending(model, B, kc, vc, Pd)          # nothing pending: no-op
        stream.synchronize()
    assert Pd.cpu().numpy().tolist() == P.tolist() == [P0 + nb * L] * B
    for (tok, steps), (o_tok, o_steps, trace) in zip(got, oracle_blocks):
        assert np.array_equal(steps.cpu().numpy(), o_steps)
        last = trace[-1]
        near = last["gap"] < 1e-6 * np.maximum(1, np.abs(last["top_score"]))
        mism = tok.cpu().numpy() != o_tok
        assert not np.any(mism & ~near), np.argwhere(mism)
    for l in range(d.NL):
        assert rel_err_rows(kc[l].cpu().double().numpy(), okc[l]) < 1e-5
        assert rel_err_rows(vc[l].cpu().double().numpy(), ovc[l]) < 1e-5
    model.close()


def test_deferred_blocks_full_width_commit_equals_reforward():
    d = ModelDims(NL=2, D=2816, Hq=16, Hkv=8, dh=128, E=128, k=8, I=704, V=32768)
    B, L, P0, nb = 2, 256, 512, 3
    w = model_weights(d, seed=5, expert_dtype="fp8", dense_dtype="bf16")
    dw = {}
    for k, v in w.items():
        v = v.to(DEV)
        if k != "emb" and not k.startswith(("sgu", "sd")):
            v = dg.dg_pack_weights(v)
        dw[k] = v
    Tmax = P0 + nb * L
    prompt = prompt_ids(B, P0, d.V, seed=6).to(DEV)
    cfgs = [dg.sampler_cfg(L, 48, 2, seed=11 + blk) for blk in range(nb)]
    # planted routing, row r of every forward taking the logits of r mod L
    override = [torch.from_numpy(np.tile(router_logits_skewed(L, d.E, d.k, seed=40 + l)[0],
                                         (2048 // L, 1))).to(DEV) for l in range(d.NL)]
    stream = torch.cuda.Stream()
    runs = {}
    with torch.cuda.stream(stream):
        for deferred in (False, True):
            model = dg.DGModel(d, dw, B, L, dg.DG_BF16, dg.DG_FP8_E4M3,
                               weight_layout=dg.DG_LAYOUT_TILED, max_prefill_tokens=2048)
            model.set_router_override(override)
            kc, vc = _caches(d, B, Tmax, torch.bfloat16)
            Pd = torch.zeros(B, dtype=torch.int32, device=DEV)
            dg.dg_prefill(model, prompt, kc, vc, Pd)
            pre_k = [k.clone() for k in kc]
            pre_v = [v.clone() for v in vc]
            toks = []
            for cfg in cfgs:
                tok = torch.full((B, L), -1, dtype=torch.int32, device=DEV)
                steps = torch.full((B,), -1, dtype=torch.int32, device=DEV)
                if deferred:
                    dg.dg_denoise_block_deferred(model, cfg, B, kc, vc, Pd, tok, steps)
                else:
                    dg.dg_denoise_block(model, cfg, B, kc, vc, Pd, tok, steps)
                toks.append(tok)
            dg.dg_commit_pending(model, B, kc, vc, Pd)
            model.check_status(stream)
            assert Pd.cpu().tolist() == [P0 + nb * L] * B
            runs[deferred] = dict(model=model, kc=kc, vc=vc, toks=toks, pre_k=pre_k, pre_v=pre_v)

        # the first block runs the same steps either way
        assert torch.equal(runs[False]["toks"][0], runs[True]["toks"][0])

        # re-forward the deferred run's final tokens block by block through
        # the plain forward into a copy of the prompt cache
        r = runs[True]
        model = r["model"]
        kc2, vc2 = r["pre_k"], r["pre_v"]
        x = torch.empty((B * L, d.D), dtype=torch.float32, device=DEV)
        for blk in range(nb):
            Pb = torch.full((B,), P0 + blk * L, dtype=torch.int32, device=DEV)
            dg.dg_model_forward(model, r["toks"][blk], x, B, L, 0, d.NL, kc2, vc2, Pb)
        stream.synchronize()
    for l in range(d.NL):
        got_k = r["kc"][l][:, :, P0:].cpu().double().numpy()
        got_v = r["vc"][l][:, :, P0:].cpu().double().numpy()
        ek = rel_err_rows(got_k, kc2[l][:, :, P0:].cpu().double().numpy())
        ev = rel_err_rows(got_v, vc2[l][:, :, P0:].cpu().double().numpy())
        print(f"layer {l}: deferred-commit K err {ek:.3g}, V err {ev:.3g}")
        assert ek < 2e-2 and ev < 2e-2
    for run in runs.values():
        run["model"].close()
