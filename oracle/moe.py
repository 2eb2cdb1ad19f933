"""Oracle of the sparse MoE feed-forward (float64).

Test infrastructure (see ``oracle/__init__.py``).

What the pages fix: the model is a sparse mixture of experts in which only the
selected experts run for each token ([WE0] "26B MoE 설계가 의미하는 것"; [GN]
summary bullets: 26B total, 3.8B active; [TR] "DiffusionGemma의 구성").  They
give neither the router nor the expert shape.

Readings:
  R19 router logits in float32 on the device, float64 here; top-k by logit
      descending with ties to the lower expert id; gates = softmax over the k
      selected logits; the combine sums slots j = 0..k-1; sorted rows are the
      slot entries t*k + j ordered stably by expert.
  R20 expert FFN(u) = (GELU(u Wg^T) * (u Wu^T)) Wd^T with the exact erf GELU.
  R21 fp8 weights are OCP e4m3fn bytes with one float32 scale per output row;
      the dequantized weight is exactly decode(byte) * scale.
Weight layout: w_gate_up [E, 2I, D] (rows 0..I-1 gate, I..2I-1 up),
w_down [E, D, I].
"""

import numpy as np
from scipy.special import erf


def fp8_e4m3fn_decode(b):
    """Value of OCP FP8 E4M3FN bytes: 1 sign, 4 exponent (bias 7), 3 mantissa
    bits; exponent 0 is subnormal (m * 2^-9); S.1111.111 is NaN; no
    infinities."""
    b = np.asarray(b, dtype=np.uint8).astype(np.int64)
    sign = np.where(b >> 7, -1.0, 1.0)
    e = (b >> 3) & 0xF
    m = b & 0x7
    normal = (1.0 + m / 8.0) * np.exp2(e.astype(np.float64) - 7.0)
    sub = m * 2.0 ** -9
    val = sign * np.where(e == 0, sub, normal)
    return np.where((e == 15) & (m == 7), np.nan, val)


def gelu_erf(x):
    """Exact GELU: x * Phi(x) = 0.5 x (1 + erf(x / sqrt 2))."""
    x = np.asarray(x, np.float64)
    return 0.5 * x * (1.0 + erf(x / np.sqrt(2.0)))


def moe_route(router_logits, k):
    """Top-k routing of T tokens over E experts (R19).

    Returns topk_ids [T, k] int64, gates [T, k] float64,
    expert_offsets [E + 1] int64, sorted_rows [T * k] int64."""
    r = np.asarray(router_logits, np.float64)
    T, E = r.shape
    ids = np.zeros((T, k), np.int64)
    gates = np.zeros((T, k))
    for t in range(T):
        order = sorted(range(E), key=lambda e: (-r[t, e], e))
        ids[t] = order[:k]
        sel = r[t, ids[t]]
        w = np.exp(sel - sel.max())
        gates[t] = w / w.sum()
    counts = np.bincount(ids.reshape(-1), minlength=E)
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int64)
    slots = np.arange(T * k)
    sorted_rows = np.array(sorted(slots, key=lambda s: (ids.reshape(-1)[s], s)),
                           dtype=np.int64)
    return ids, gates, offsets, sorted_rows


def expert_gate_up(u, wg, wu):
    """The gated hidden activation of one expert for the rows of u [n, D]:
    GELU(u Wg^T) * (u Wu^T), [n, I]."""
    return gelu_erf(u @ wg.T) * (u @ wu.T)


def expert_ffn(u, wg, wu, wd):
    """One expert applied to the rows of u [n, D]."""
    return expert_gate_up(u, wg, wu) @ wd.T


def moe_ffn(u, w_gate_up, w_down, topk_ids, gates):
    """y [T, D] = sum_j gates[t, j] * FFN_{topk_ids[t, j]}(u_t).

    u [T, D]; w_gate_up [E, 2I, D]; w_down [E, D, I] (float64 values, already
    dequantized for fp8).  Experts are evaluated on the rows routed to them;
    the combine adds slots in order j = 0..k-1."""
    u = np.asarray(u, np.float64)
    T, D = u.shape
    E, I2, _ = w_gate_up.shape
    I = I2 // 2
    k = topk_ids.shape[1]
    out = np.zeros((T, k, D))
    for e in range(E):
        rows, slots = np.nonzero(topk_ids == e)
        if rows.size == 0:
            continue
        w = np.asarray(w_gate_up[e], np.float64)
        o = expert_ffn(u[rows], w[:I], w[I:], np.asarray(w_down[e], np.float64))
        out[rows, slots] = o
    y = np.zeros((T, D))
    for j in range(k):
        y += gates[:, j:j + 1] * out[:, j]
    return y


def moe_ffn_dense_masked(u, w_gate_up, w_down, topk_ids, gates):
    """Every expert on every token, weighted by its gate if selected else 0.
    Mathematically equal to ``moe_ffn``; used as its brute-force pin."""
    u = np.asarray(u, np.float64)
    T, D = u.shape
    E, I2, _ = w_gate_up.shape
    I = I2 // 2
    y = np.zeros((T, D))
    for e in range(E):
        w = np.asarray(w_gate_up[e], np.float64)
        o = expert_ffn(u, w[:I], w[I:], np.asarray(w_down[e], np.float64))
        g = np.where(topk_ids == e, gates, 0.0).sum(axis=1)
        y += g[:, None] * o
    return y
