"""dg_sampler_step_noalloc (the sampler step on the library's own device
scratch, for callers that cannot allocate) against dg_sampler_step with a
caller workspace, through the C ABI: two calls in a row on one GPU, the
second on a smaller input, every output bit for bit; sizes beyond the
scratch are rejected on the host."""

import pytest
import torch

from block_diffusion_decoding_tok_amd import dg
from block_diffusion_decoding_tok_amd.inputs import sampler_case

pytestmark = pytest.mark.gpu
DEV = "cuda"
OUTS = ("tokens", "committed", "renoised", "maxprob", "entropy", "mean_entropy", "done", "status")


def _state(B, L, V, seed):
    g = torch.Generator().manual_seed(seed)
    return dict(tokens=torch.randint(0, V, (B, L), generator=g, dtype=torch.int32).to(DEV),
                committed=torch.zeros((B, L), dtype=torch.uint8, device=DEV),
                renoised=torch.full((B, L), 7, dtype=torch.uint8, device=DEV),
                maxprob=torch.full((B, L), -1.0, device=DEV),
                entropy=torch.full((B, L), -1.0, device=DEV),
                mean_entropy=torch.full((B,), -1.0, device=DEV),
                done=torch.zeros(B, dtype=torch.int32, device=DEV),
                status=torch.zeros(1, dtype=torch.int32, device=DEV))


@pytest.mark.parametrize("order", ["large_then_small", "small_then_large"])
def test_noalloc_sampler_matches_workspace_call(order):
    cases = [(4, 256, 262144, 0, [0, 47]), (1, 16, 4096, 1, [0, 3, 7])]
    if order == "small_then_large":
        cases = cases[::-1]
    for B, L, V, seed, steps in cases:
        case = sampler_case(B=B, L=L, V=V, seed=seed)
        logits = case.logits.to(DEV)
        cfg = dg.sampler_cfg(L, max(steps) + 1, 0, seed=seed + 5)
        P = torch.arange(B, dtype=torch.int32, device=DEV) * 300 + 17
        a, b = _state(B, L, V, seed), _state(B, L, V, seed)
        n_renoised = 0
        for s in steps:
            dg.dg_sampler_step(logits, s, cfg, P, a["tokens"], a["committed"], a["renoised"],
                               a["maxprob"], a["entropy"], a["mean_entropy"], a["done"],
                               a["status"])
            dg.dg_sampler_step_noalloc(logits, s, cfg, P, b["tokens"], b["committed"],
                                       b["renoised"], b["maxprob"], b["entropy"],
                                       b["mean_entropy"], b["done"], b["status"])
            torch.cuda.synchronize()
            for k in OUTS:
                assert torch.equal(a[k], b[k]), (B, L, V, s, k)
            n_renoised += int(a["renoised"].sum())
        assert n_renoised > 0                 # the update rules were exercised


def test_noalloc_sampler_rejects_sizes_beyond_the_scratch():
    B, L, V = 9, 256, 262144          # 9 * 256 * 16 partials of 32 bytes > 1 MiB
    logits = torch.zeros((1, 8), dtype=torch.bfloat16, device=DEV)   # never read
    st = _state(1, 8, 8, 0)
    cfg = dg.sampler_cfg(L, 48, 0)
    lib = dg.lib()
    p = [logits.data_ptr(), dg.DG_BF16, B, L, V, 0, dg.C.byref(cfg)] + \
        [st[k].data_ptr() for k in ("tokens", "tokens", "committed", "renoised", "maxprob",
                                    "entropy", "mean_entropy", "done", "status")] + [None]
    assert lib.dg_sampler_step_noalloc(*p) == -4
    assert "scratch" in lib.dg_last_error().decode()
