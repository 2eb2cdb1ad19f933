"""GPU parity of the decoder's block call at full width (dg_denoise_block on
the product configuration: bf16 dense weights and activations, fp8-e4m3
experts, the tiled weight layout, hipGraphs on a non-default stream), through
the C ABI, against the oracle.

The block runs every step's forward, LM head and sampler inside the library.
The test replays the same block step by step: the device forward of the
current tokens (dg_model_forward, the same kernels on the same inputs, run
twice to show it is deterministic) gives that step's logits, and the oracle's
sampler takes them to the next tokens.  The block's final tokens and step
counts must equal the replay's bit for bit (positions the sampler rules
exclude are counted).  The committed K/V of every layer must equal a
re-forward of the final tokens bit for bit and the oracle's layer, teacher
forced on the device's layer inputs, within the bf16 tolerance.

Shapes: 2 layers of the decoder's full width (D 2816, 16/8 heads of 128,
128 experts top-8 of 704), batch 2, a 512-token prompt, canvas 256."""

import numpy as np
import pytest
import torch

from block_diffusion_decoding_tok_amd import dg
from block_diffusion_decoding_tok_amd.inputs import ModelDims, model_weights, prompt_ids
from oracle import SamplerCfg, init_canvas, layer_forward, sampler_step
from oracle.attention import CANVAS
from oracle.host_weights import oracle_model
from tests.util import rel_err_rows, sampler_exclusions

pytestmark = pytest.mark.gpu
DEV = "cuda"
B, P0, L, NL = 2, 512, 256, 2


def _dims(V):
    return ModelDims(NL=NL, D=2816, Hq=16, Hkv=8, dh=128, E=128, k=8, I=704, V=V)


@pytest.fixture(scope="module")
def layer_weights():
    """Host weights of the 2 layers (the same draws at every vocabulary
    size: each tensor has its own seeded stream)."""
    return model_weights(_dims(32768), seed=5, expert_dtype="fp8", dense_dtype="bf16")


def _model(w, V, lm_boost=None):
    d = _dims(V)
    if V != 32768:
        head = model_weights(d, seed=5, dense_dtype="bf16", layers=0)
        w = dict(w, emb=head["emb"], lm=head["lm"])
    dw = {}
    for k, v in w.items():
        v = v.to(DEV)
        if k == "lm" and lm_boost is not None:
            v = v.clone()
            v[:16] = (v[:16].float() * lm_boost).to(v.dtype)   # a planted confident head
        if k != "emb" and not k.startswith(("sgu", "sd")):
            v = dg.dg_pack_weights(v)
        dw[k] = v
    model = dg.DGModel(d, dw, B, L, dg.DG_BF16, dg.DG_FP8_E4M3, weight_layout=dg.DG_LAYOUT_TILED)
    return d, w, model


def _run(w, V, cfg_kw, lm_boost=None):
    d, w, model = _model(w, V, lm_boost)
    Tmax = P0 + L
    shape = (B, d.Hkv, Tmax, d.dh)
    kc = [torch.zeros(shape, dtype=torch.bfloat16, device=DEV) for _ in range(NL)]
    vc = [torch.zeros(shape, dtype=torch.bfloat16, device=DEV) for _ in range(NL)]
    Pd = torch.zeros(B, dtype=torch.int32, device=DEV)
    stream = torch.cuda.Stream()
    ocfg = SamplerCfg(canvas_len=L, seed=11, **cfg_kw)
    gcfg = dg.sampler_cfg(L, ocfg.max_steps, ocfg.fixed_steps, seed=ocfg.seed)
    with torch.cuda.stream(stream):
        dg.dg_prefill(model, prompt_ids(B, P0, V, seed=6).to(DEV), kc, vc, Pd)
        stream.synchronize()
        tok = torch.full((B, L), -1, dtype=torch.int32, device=DEV)
        steps = torch.full((B,), -1, dtype=torch.int32, device=DEV)
        dg.dg_denoise_block(model, gcfg, B, kc, vc, Pd, tok, steps)
        model.check_status(stream)
        assert Pd.cpu().tolist() == [P0 + L] * B
        blk_tok = tok.cpu().numpy()
        blk_steps = steps.cpu().numpy()
        blk_k = [k[:, :, P0:].clone() for k in kc]
        blk_v = [v[:, :, P0:].clone() for v in vc]

        # the replay: device forwards, oracle sampler
        P = np.full(B, P0)
        Pr = torch.full((B,), P0, dtype=torch.int32, device=DEV)
        tokens, committed = init_canvas(ocfg.seed, P, L, V)
        done = np.zeros(B, np.int64)
        state = {}
        r_steps = np.zeros(B, np.int64)
        x = torch.empty((B * L, d.D), dtype=torch.float32, device=DEV)
        lg = torch.empty((B, L, V), dtype=torch.bfloat16, device=DEV)
        lg2 = torch.empty_like(lg)
        n_steps = ocfg.fixed_steps or ocfg.max_steps
        excluded = 0
        for s in range(n_steps):
            t_dev = torch.from_numpy(tokens.astype(np.int32)).to(DEV)
            dg.dg_model_forward(model, t_dev, x, B, L, 0, NL, kc, vc, Pr, logits=lg)
            dg.dg_model_forward(model, t_dev, x, B, L, 0, NL, kc, vc, Pr, logits=lg2)
            stream.synchronize()
            assert torch.equal(lg, lg2), f"step {s}: the forward is not deterministic"
            logits = lg.cpu().double().numpy()
            ref = sampler_step(logits, s, ocfg, P, tokens, committed, done, **state)
            excl, row_excl = sampler_exclusions(ref, ocfg, committed)
            act = done == 0
            n_ex = int(excl[act].sum()) + int(row_excl[act].sum())
            excluded += n_ex
            last = bool(ref["done"].all())
            # a near-threshold decision before the last step would let the two
            # trajectories part: the seeds are chosen so that none occurs
            assert last or n_ex == 0, f"step {s}: {n_ex} excluded decisions"
            r_steps += act
            tokens, committed, done = ref["tokens"], ref["committed"], ref["done"]
            state = dict(renoised=ref["renoised"], maxprob=ref["maxprob"], entropy=ref["entropy"],
                         mean_entropy=ref["mean_entropy"])
            if last:
                break
        print(f"block steps {blk_steps.tolist()}, replay steps {r_steps.tolist()}, "
              f"committed {committed.sum(axis=1).tolist()}, excluded {excluded}")
        assert np.array_equal(blk_steps, r_steps)
        keep = ~excl
        assert np.array_equal(blk_tok[keep], tokens[keep])
        assert excluded <= 2

        # the commit: a re-forward of the block's final tokens writes the same
        # K/V bit for bit; the oracle layer on the device's layer inputs
        # (teacher forced) writes them within the bf16 tolerance
        m = oracle_model(d, dict(w, emb=w["emb"][:1], lm=w["lm"][:1]))
        t_dev = torch.from_numpy(blk_tok).to(DEV)
        dg.dg_model_forward(model, t_dev, x, B, L, 0, 0, kc, vc, Pr)          # embed only
        for l in range(NL):
            stream.synchronize()
            x_in = x.cpu().double().numpy().reshape(B, L, d.D)
            ck = kc[l].cpu().double().numpy()
            cv = vc[l].cpu().double().numpy()
            dg.dg_model_forward(model, None, x, B, L, l, l + 1, kc, vc, Pr)
            stream.synchronize()
            assert torch.equal(kc[l][:, :, P0:], blk_k[l]) and torch.equal(vc[l][:, :, P0:], blk_v[l])
            layer_forward(m, m.layers[l], x_in, ck, cv, P, CANVAS)
            ek = rel_err_rows(blk_k[l].cpu().double().numpy(), ck[:, :, P0:])
            ev = rel_err_rows(blk_v[l].cpu().double().numpy(), cv[:, :, P0:])
            print(f"layer {l}: committed K err {ek:.3g}, V err {ev:.3g}")
            assert ek < 2e-2 and ev < 2e-2
    model.close()
    return blk_steps, committed


def test_block_full_width_full_vocab_fixed_steps(layer_weights):
    """The product call at the full vocabulary (2^18): 2 fixed steps of the
    48-step schedule.  At random weights every position is re-noised at step
    0 (uniform ids) and takes its Gumbel sample at the last step."""
    steps, _ = _run(layer_weights, 262144, dict(max_steps=48, fixed_steps=2))
    assert steps.tolist() == [2, 2]


def test_block_full_width_adaptive_to_the_cap(layer_weights):
    """Adaptive mode (chunks of steps with the done check between them) with
    a cap of 5: random weights never reach the stop threshold, so the block
    runs to the cap and the last step samples without re-noising."""
    steps, _ = _run(layer_weights, 32768, dict(max_steps=5))
    assert steps.tolist() == [5, 5]


def test_block_full_width_planted_head_stops_early(layer_weights):
    """A planted confident head (the first 16 LM-head rows scaled by 400):
    positions commit at once and the mean entropy falls below the threshold,
    so each row stops long before the cap of 48."""
    steps, committed = _run(layer_weights, 32768, dict(max_steps=48), lm_boost=400.0)
    assert (steps < 48).all() and committed.sum() > 0
