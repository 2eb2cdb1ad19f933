"""Float64 views of seeded host weights, in the form the oracle's model
functions take (test infrastructure, see ``oracle/__init__.py``).

The seeded weights arrive as host torch tensors: bf16 or f32 values, or
e4m3fn bytes (uint8) with one f32 scale per row (R21).  Every value is turned
into its exact float64 value; expert stacks are decoded one expert at a time
on indexing, so a full stack never exists in float64."""

import numpy as np
import torch

from .model import TinyModel
from .moe import fp8_e4m3fn_decode

# value of every e4m3fn byte
_FP8_TABLE = fp8_e4m3fn_decode(np.arange(256, dtype=np.uint8))


def to_f64(t):
    """Exact float64 value of a host tensor of bf16 / f32 values."""
    return t.to(torch.float64).numpy()


class ExpertWeights:
    """Per-expert float64 view of host expert weights [E, N, K]: bf16/f32
    values, or e4m3fn bytes times the per-row scales [E, N]."""

    def __init__(self, w, s=None):
        self.w, self.s = w, s
        self.shape = tuple(w.shape)

    def __getitem__(self, e):
        if self.w.dtype == torch.uint8:
            return _FP8_TABLE[self.w[e].numpy()] * self.s[e].to(torch.float64).numpy()[:, None]
        return to_f64(self.w[e])


def oracle_model(dims, weights, layers=None):
    """TinyModel of the first ``layers`` (default all) layers of a weight dict
    with keys emb, lm, wqkv.l, wo.l, wr.l, wgu.l, sgu.l, wd.l, sd.l."""
    nl = dims.NL if layers is None else layers
    m = TinyModel(D=dims.D, Hq=dims.Hq, Hkv=dims.Hkv, dh=dims.dh, E=dims.E,
                  k=dims.k, I=dims.I, V=dims.V, emb=to_f64(weights["emb"]),
                  lm=to_f64(weights["lm"]))
    for l in range(nl):
        m.layers.append(dict(
            wqkv=to_f64(weights[f"wqkv.{l}"]), wo=to_f64(weights[f"wo.{l}"]),
            wr=to_f64(weights[f"wr.{l}"]),
            w_gate_up=ExpertWeights(weights[f"wgu.{l}"], weights[f"sgu.{l}"]),
            w_down=ExpertWeights(weights[f"wd.{l}"], weights[f"sd.{l}"])))
    return m
