"""GPU parity of canvas attention and the KV commit against the oracle,
through the C ABI (bf16 MFMA path and f32 path)."""

import numpy as np
import pytest
import torch

from block_diffusion_decoding_tok_amd import dg
from block_diffusion_decoding_tok_amd.inputs import attention_case
from oracle.attention import attention, rope, CANVAS, CAUSAL
from tests.util import rel_err_rows

pytestmark = pytest.mark.gpu
DEV = "cuda"
TOL = {torch.bfloat16: 2e-2, torch.float32: 1e-5}


def _run(case, P_list, Tmax, mode, dtype):
    B, Lq, Hq, dh = case.q.shape
    Hkv = case.k_new.shape[2]
    kc = torch.zeros((B, Hkv, Tmax, dh), dtype=dtype)
    vc = torch.zeros((B, Hkv, Tmax, dh), dtype=dtype)
    for b, P in enumerate(P_list):
        kc[b, :, :P] = case.k_prefix[b, :, :P]
        vc[b, :, :P] = case.v_prefix[b, :, :P]
    kc_d, vc_d = kc.to(DEV), vc.to(DEV)
    Pd = torch.tensor(P_list, dtype=torch.int32, device=DEV)
    out = dg.dg_canvas_attention(case.q.to(DEV), case.k_new.to(DEV), case.v_new.to(DEV),
                                 kc_d, vc_d, Pd, mask_mode=mode)
    torch.cuda.synchronize()
    assert torch.equal(Pd.cpu(), torch.tensor(P_list, dtype=torch.int32))   # not advanced
    return out.cpu(), kc_d.cpu(), vc_d.cpu()


def _check(case, P_list, Tmax, mode, dtype):
    out, kc, vc = _run(case, P_list, Tmax, mode, dtype)
    f64 = lambda t: t.to(torch.float64).numpy()
    worst = 0.0
    for b, P in enumerate(P_list):
        o_ref, k_rot = attention(f64(case.q[b]), f64(case.k_new[b]), f64(case.v_new[b]),
                                 f64(case.k_prefix[b, :, :P]), f64(case.v_prefix[b, :, :P]),
                                 P, mode)
        err = rel_err_rows(f64(out[b]), o_ref)
        worst = max(worst, err)
        Lq = case.q.shape[1]
        # cache tail: rotated keys (rounded once to the cache dtype) and values
        tail_k = f64(kc[b, :, P:P + Lq]).transpose(1, 0, 2)
        assert rel_err_rows(tail_k, k_rot) < (8e-3 if dtype == torch.bfloat16 else 1e-6)
        assert torch.equal(vc[b, :, P:P + Lq].transpose(0, 1), case.v_new[b])
        # the prefix is untouched and nothing beyond the block is written
        assert torch.equal(kc[b, :, :P], case.k_prefix[b, :, :P])
        assert not kc[b, :, P + Lq:].any()
    assert worst < TOL[dtype], worst
    return worst


@pytest.mark.parametrize("B", [1, 4])
def test_canvas_attention_bf16_full_size(B):
    """256 canvas queries over 2048 cached prefix tokens + the canvas; 16 query
    heads over 8 KV heads of 128."""
    case = attention_case(B=B, Lq=256, P=2048, seed=B)
    _check(case, [2048] * B, 2304, CANVAS, torch.bfloat16)


@pytest.mark.parametrize("B", [1, 4])
def test_canvas_attention_bf16_canvas_step_size(B):
    """The canvas step's own shape: 256 queries over an 8192-token prefix and
    the canvas (16 query / 8 KV heads of 128) in a cache sized for the prompt
    and four blocks, as bench.py runs it: every workgroup walks up to 9 (batch
    1) or 33 (batch 4) key tiles through the double-buffered LDS copies."""
    case = attention_case(B=B, Lq=256, P=8192, seed=40 + B)
    _check(case, [8192] * B, 8192 + 4 * 256, CANVAS, torch.bfloat16)


def test_canvas_attention_bf16_ragged_rows():
    """Different prefix per row, ragged block and key tiles, spare cache."""
    case = attention_case(B=3, Lq=100, P=700, seed=11)
    _check(case, [77, 700, 0], 1000, CANVAS, torch.bfloat16)


def test_canvas_attention_bf16_spare_cache():
    """A cache sized for far more keys than the rows hold (the splits are
    balanced over each row's own key count on the device): two rows with
    different prefixes in a cache of 8192 slots."""
    case = attention_case(B=2, Lq=256, P=3000, seed=31)
    _check(case, [1500, 3000], 8192, CANVAS, torch.bfloat16)


@pytest.mark.parametrize("Lq", [1, 2, 5, 16])
@pytest.mark.parametrize("mode", [CANVAS, CAUSAL])
def test_attention_bf16_few_queries(Lq, mode):
    """A few query tokens per row (AR decode): up to 4 packed rows per KV head
    take the decode kernel (Lq 1 and 2 here), more take one row tile of the
    MFMA kernel; the cache is split over many workgroups, most of them empty
    past the short row's keys; rows with 8000 and 333 cached keys in 8448
    slots."""
    case = attention_case(B=2, Lq=Lq, P=8000, seed=40 + Lq)
    _check(case, [8000, 333], 8448, mode, torch.bfloat16)


@pytest.mark.parametrize("Hq,Hkv,Lq", [(8, 8, 1), (8, 8, 3), (16, 4, 1), (16, 8, 2)])
@pytest.mark.parametrize("mode", [CANVAS, CAUSAL])
def test_attention_bf16_decode_groups(Hq, Hkv, Lq, mode):
    """The decode kernel at 1, 3 and 4 packed rows per KV head (one, three
    and four query heads per group), ragged prefixes and an empty one."""
    case = attention_case(B=3, Lq=Lq, P=1000, Hq=Hq, Hkv=Hkv, seed=60 + Hq + Hkv + Lq)
    _check(case, [1000, 77, 0], 1100, mode, torch.bfloat16)


def test_attention_bf16_decode_long_prefix():
    """One token over 20000 cached keys: each decode workgroup walks several
    256-key chunks with the online-softmax rescale between them."""
    case = attention_case(B=1, Lq=1, P=20000, seed=70)
    _check(case, [20000], 20480, CAUSAL, torch.bfloat16)


@pytest.mark.parametrize("P", [0, 64, 300])
def test_causal_prefill_bf16(P):
    case = attention_case(B=2, Lq=200, P=max(P, 1), seed=20 + P)
    _check(case, [P, P], P + 256, CAUSAL, torch.bfloat16)


def test_attention_f32_tiny():
    case = attention_case(B=2, Lq=16, P=32, Hq=4, Hkv=2, dh=16, seed=3, dtype=torch.float32)
    _check(case, [32, 32], 64, CANVAS, torch.float32)
    _check(case, [0, 5], 64, CAUSAL, torch.float32)


def test_attention_mha_and_gqa8_f32():
    case = attention_case(B=1, Lq=9, P=13, Hq=8, Hkv=8, dh=64, seed=4, dtype=torch.float32)
    _check(case, [13], 40, CANVAS, torch.float32)
    case = attention_case(B=1, Lq=9, P=13, Hq=8, Hkv=1, dh=128, seed=5, dtype=torch.float32)
    _check(case, [13], 40, CANVAS, torch.float32)


def test_commit_block_writes_and_advances():
    case = attention_case(B=2, Lq=256, P=512, seed=6)
    B, L, Hkv, dh = case.k_new.shape
    Tmax = 1024
    kc = torch.zeros((B, Hkv, Tmax, dh), dtype=torch.bfloat16, device=DEV)
    vc = torch.zeros_like(kc)
    Pd = torch.tensor([512, 100], dtype=torch.int32, device=DEV)
    dg.dg_commit_block(case.k_new.to(DEV), case.v_new.to(DEV), kc, vc, Pd)
    torch.cuda.synchronize()
    assert Pd.cpu().tolist() == [512 + L, 100 + L]
    for b, P in enumerate((512, 100)):
        k_rot = rope(case.k_new[b].double().numpy(), P + np.arange(L))
        got = kc[b, :, P:P + L].cpu().double().numpy().transpose(1, 0, 2)
        assert rel_err_rows(got, k_rot) < 8e-3
        assert torch.equal(vc[b, :, P:P + L].cpu().transpose(0, 1), case.v_new[b])


def test_attention_deterministic():
    case = attention_case(B=1, Lq=256, P=1000, seed=8)
    a, _, _ = _run(case, [1000], 1280, CANVAS, torch.bfloat16)
    b, _, _ = _run(case, [1000], 1280, CANVAS, torch.bfloat16)
    assert torch.equal(a, b)
