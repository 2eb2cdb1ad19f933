"""Helpers shared by the tests: turn the seeded host inputs into the oracle's
float64 model, and the comparison rules used by the parity tests."""

import numpy as np
import torch

from oracle import fp8_e4m3fn_decode, dequantize_mxfp4
from oracle.host_weights import ExpertWeights, oracle_model, to_f64  # noqa: F401


def expert_f64(w, s):
    """Dequantized expert weights: e4m3fn bytes times the per-row scale, or
    the float values as given when the tensor is not uint8."""
    if w.dtype == torch.uint8:
        return fp8_e4m3fn_decode(w.numpy()) * s.to(torch.float64).numpy()[..., None]
    return to_f64(w)


def empty_caches(dims, B, Tmax, layers=None):
    nl = dims.NL if layers is None else layers
    shape = (B, dims.Hkv, Tmax, dims.dh)
    return [np.zeros(shape) for _ in range(nl)], [np.zeros(shape) for _ in range(nl)]


def rel_err_rows(got, ref):
    """Max over rows of ||got - ref|| / ||ref|| (rows = last axis)."""
    got = np.asarray(got, np.float64).reshape(-1, np.shape(ref)[-1])
    ref = np.asarray(ref, np.float64).reshape(-1, np.shape(ref)[-1])
    num = np.linalg.norm(got - ref, axis=1)
    den = np.maximum(np.linalg.norm(ref, axis=1), 1e-30)
    return float((num / den).max())


# ------------------------------------------------------------ sampler rules

TAU_BAND = 1e-6          # |maxprob - threshold| below this: decision excluded
STOP_BAND = 1e-6         # |mean entropy - stop threshold| below this: row excluded


def gumbel_band(top_score):
    """Top-2 perturbed-score gap below which the Gumbel-max id is excluded:
    1e-6 * max(1, |score|) (float32 scores on the device vs float64 here)."""
    return 1e-6 * np.maximum(1.0, np.abs(top_score))


EB_BAND = 1e-5           # entropy-bound sums / rank gaps closer than this: row excluded


def entropy_bound_ambiguous(h, committed, bound):
    """True when the entropy-bound selection of a row could flip between the
    device's and the oracle's entropies: a ranked prefix sum within EB_BAND of
    the bound, or the two positions that straddle the cut within EB_BAND of
    each other."""
    free = sorted((i for i in range(len(h)) if not committed[i]), key=lambda i: (h[i], i))
    if len(free) < 2:
        return False
    hs = np.array([h[i] for i in free])
    csum = np.cumsum(hs)[:-1]
    if np.any(np.abs(csum - bound) < EB_BAND):
        return True
    n_sel = 1 + int(np.sum(csum <= bound))
    return n_sel < len(hs) and hs[n_sel] - hs[n_sel - 1] < EB_BAND


def sampler_exclusions(ref, cfg, committed_before=None):
    """Boolean [B, L] mask of positions whose integer outputs are excluded from
    the bit-exact comparison, and [B] mask of rows whose stop decision is."""
    mp = ref["maxprob"]
    near_tau = (np.abs(mp - cfg.commit_prob) < TAU_BAND) | (np.abs(mp - cfg.renoise_prob) < TAU_BAND)
    if getattr(cfg, "commit_policy", 0) == 1:
        near_tau = np.abs(mp - cfg.renoise_prob) < TAU_BAND
        for b in range(mp.shape[0]):
            if committed_before is not None and entropy_bound_ambiguous(
                    ref["entropy"][b], committed_before[b], cfg.entropy_bound):
                near_tau[b] = True
    near_tie = ref["gap"] < gumbel_band(ref["top_score"])
    row = np.abs(ref["mean_entropy"] - cfg.stop_entropy) < STOP_BAND
    return near_tau | near_tie | row[:, None], row


class Mx4ExpertWeights:
    """Per-expert float64 view of row-major MXFP4 expert weights: codes
    [E, N, K / 2] and E8M0 scales [E, N, K / 32] (uint8 tensors), decoded by
    the oracle one expert at a time."""

    def __init__(self, codes, scales):
        self.codes, self.scales = codes, scales
        self.shape = tuple(codes.shape[:-1]) + (2 * codes.shape[-1],)

    def __getitem__(self, e):
        return dequantize_mxfp4(self.codes[e].numpy(), self.scales[e].numpy())


def pack_mxfp4_tiled(codes, scales):
    """Row-major MXFP4 codes [.., N, K / 2] and scales [.., N, K / 32] -> the
    tiled MXFP4 byte order (flat): per block of 16 rows x 64 k, 512 code
    bytes (lane r + 16 q: row r, bytes 8 q .. 8 q + 7 of the block's 32) then
    32 scale bytes (16 h + r: row r, block half h)."""
    c = np.asarray(codes)
    s = np.asarray(scales)
    N, K = c.shape[-2], 2 * c.shape[-1]
    G = c.size // (N * K // 2)
    cb = c.reshape(G, N // 16, 16, K // 64, 4, 8)           # g, t, r, c, q, byte
    cb = cb.transpose(0, 1, 3, 4, 2, 5).reshape(G, N // 16, K // 64, 512)
    sb = s.reshape(G, N // 16, 16, K // 64, 2)               # g, t, r, c, h
    sb = sb.transpose(0, 1, 3, 4, 2).reshape(G, N // 16, K // 64, 32)
    return np.ascontiguousarray(np.concatenate([cb, sb], axis=-1)).reshape(-1)


def pack_tiled(w):
    """Row-major [.., N, K] -> the DG_LAYOUT_TILED element order (numpy view of
    the same shape): blocks of 16 rows x 64 k in wave-load order; one matrix
    keeps a tile's blocks together (t, c), a stack of G > 1 matrices keeps the
    k chunk c of every matrix's tiles together (c, g, t)."""
    a = np.asarray(w)
    N, K = a.shape[-2], a.shape[-1]
    G = a.size // (N * K)
    x = a.reshape(G, N // 16, 16, K // 64, 4, 16)           # g, t, r, c, q, j
    if a.itemsize == 1:
        out = x.transpose(0, 1, 3, 4, 2, 5)                  # g, t, c, q, r, j
    else:
        x = x.reshape(G, N // 16, 16, K // 64, 4, 2, 8)     # g, t, r, c, q, h, j
        out = x.transpose(0, 1, 3, 5, 4, 2, 6)               # g, t, c, h, q, r, j
    if G > 1:                                                # block order c, g, t
        blocks = np.ascontiguousarray(out).reshape(G, N // 16, K // 64, -1)
        out = blocks.transpose(2, 0, 1, 3)
    return np.ascontiguousarray(out).reshape(a.shape)
