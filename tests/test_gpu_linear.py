"""GPU parity of the dense projections and the LM head (dg_linear) against a
float64 matrix product of the same bf16 / f32 values, through the C ABI:
every kernel the decoder uses for them (split-K projections, the narrow
router shape, the vocabulary-sized block GEMM over tile-packed weights, the
generic streaming path), row-major and tile-packed weights, ragged token
counts, the accumulate epilogue."""

import numpy as np
import pytest
import torch

from block_diffusion_decoding_tok_amd import dg
from tests.util import rel_err_rows

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _case(M, N, K, seed, dtype=torch.bfloat16):
    g = torch.Generator().manual_seed(seed)
    x = torch.randn((M, K), generator=g).to(dtype)
    w = (torch.randn((N, K), generator=g) * 0.02).to(dtype)
    return x, w


def _ref(x, w):
    return x.double().numpy() @ w.double().numpy().T


@pytest.mark.parametrize("M,N,K", [(256, 4096, 2816), (256, 2816, 2048), (256, 128, 2816),
                                   (100, 192, 512), (37, 4096, 2816), (1024, 2816, 2048)])
@pytest.mark.parametrize("tiled", [False, True])
def test_linear_projection_shapes(M, N, K, tiled):
    x, w = _case(M, N, K, seed=M + N + K)
    wd = w.to(DEV)
    if tiled:
        wd = dg.dg_pack_weights(wd)
    out = dg.dg_linear(x.to(DEV), wd, out_dtype=torch.float32, N=N,
                       w_layout=dg.DG_LAYOUT_TILED if tiled else dg.DG_LAYOUT_ROWMAJOR)
    torch.cuda.synchronize()
    assert rel_err_rows(out.cpu().double().numpy(), _ref(x, w)) < 1e-5


@pytest.mark.parametrize("M", [256, 37])
@pytest.mark.parametrize("tiled", [False, True])
def test_linear_accumulate_bf16_out(M, tiled):
    N, K = 2816, 2048
    x, w = _case(M, N, K, seed=3 + M)
    wd = dg.dg_pack_weights(w.to(DEV)) if tiled else w.to(DEV)
    lay = dg.DG_LAYOUT_TILED if tiled else dg.DG_LAYOUT_ROWMAJOR
    y0 = torch.randn((M, N), generator=torch.Generator().manual_seed(4 + M))
    y = y0.clone().to(DEV)
    dg.dg_linear(x.to(DEV), wd, out=y, accumulate=True, N=N, w_layout=lay)
    ob = dg.dg_linear(x.to(DEV), wd, out_dtype=torch.bfloat16, N=N, w_layout=lay)
    torch.cuda.synchronize()
    ref = _ref(x, w)
    assert rel_err_rows(y.cpu().double().numpy() - y0.double().numpy(), ref) < 1e-5
    # bf16 output: one rounding of the f32 sum
    assert rel_err_rows(ob.cpu().double().numpy(), ref) < 4e-3


@pytest.mark.parametrize("M", [256, 200, 512])
@pytest.mark.parametrize("tiled", [False, True])
def test_linear_vocab_sized(M, tiled):
    """The LM head shape: N = 2^18 rows (bf16 logits).  Checked on a sample of
    rows and columns of the product (all tokens of 4096 sampled columns)."""
    N, K = 262144, 2816
    g = torch.Generator().manual_seed(11)
    x = torch.randn((M, K), generator=g).to(torch.bfloat16)
    wd = torch.empty((N, K), dtype=torch.bfloat16, device=DEV)
    dg.dg_fill_normal(wd, 0.02, 5, 7)
    cols = np.sort(np.random.default_rng(M).choice(N, 4096, replace=False))
    w_s = wd[torch.from_numpy(cols).to(DEV)].cpu()
    if tiled:
        wd = dg.dg_pack_weights(wd)
    out = dg.dg_linear(x.to(DEV), wd, out_dtype=torch.bfloat16, N=N,
                       w_layout=dg.DG_LAYOUT_TILED if tiled else dg.DG_LAYOUT_ROWMAJOR)
    torch.cuda.synchronize()
    got = out[:, torch.from_numpy(cols).to(DEV)].cpu().double().numpy()
    assert rel_err_rows(got, _ref(x, w_s)) < 4e-3
    del out, wd


def test_linear_f32():
    x, w = _case(48, 200, 64, seed=9, dtype=torch.float32)
    out = dg.dg_linear(x.to(DEV), w.to(DEV))
    torch.cuda.synchronize()
    assert rel_err_rows(out.cpu().double().numpy(), _ref(x, w)) < 1e-6
