"""Oracle of canvas attention (float64).

Test infrastructure (see ``oracle/__init__.py``).

What the pages fix: every canvas position attends to every other canvas
position in one forward pass ([GN] "핵심 트레이드오프"; [WE0] "양방향 어텐션과
자기 수정의 역할"; [GUIDE] "Prefill과 Denoising의 이중 어텐션"); the prompt and
earlier blocks are read from the KV cache ([GUIDE] "Block Autoregressive
Diffusion"; [TR] "DiffusionGemma의 구성", flowchart); the block-diagonal mask
keeps the prompt as cache and makes attention bidirectional only inside the
current block ([TR] "DiffusionGemma의 구성", SFT paragraph), so prompt rows
never see canvas keys.

Readings (R15, R27): scores q.k / sqrt(dh), softmax over the visible keys;
query head h reads KV head floor(h * Hkv / Hq) (grouped-query attention);
RoPE rotates the pairs (j, j + dh/2) by angle pos * theta^(-2j/dh) at absolute
positions, theta = 10000, and the cache stores rotated keys.  Mode "canvas":
a query at slot i sees keys [0, P + Lq).  Mode "causal" (prompt prefill):
it sees keys [0, P + i].
"""

import numpy as np

CANVAS = 0
CAUSAL = 1


def rope(x, pos, theta=10000.0):
    """Rotate x [n, H, dh] at absolute positions pos [n] (rotate-half)."""
    x = np.asarray(x, dtype=np.float64)
    dh = x.shape[-1]
    half = dh // 2
    j = np.arange(half, dtype=np.float64)
    inv = theta ** (-2.0 * j / dh)
    ang = np.asarray(pos, dtype=np.float64)[:, None] * inv[None, :]   # [n, half]
    cos = np.cos(ang)[:, None, :]
    sin = np.sin(ang)[:, None, :]
    x1, x2 = x[..., :half], x[..., half:]
    return np.concatenate([x1 * cos - x2 * sin, x2 * cos + x1 * sin], axis=-1)


def attention(q, k_new, v_new, k_prefix, v_prefix, P, mode=CANVAS,
              theta=10000.0, rope_on=True):
    """Attention of one batch row.

    q          [Lq, Hq, dh]   un-rotated queries of the block
    k_new      [Lq, Hkv, dh]  un-rotated keys of the block
    v_new      [Lq, Hkv, dh]
    k_prefix   [Hkv, P, dh]   cached keys of positions [0, P), already rotated
    v_prefix   [Hkv, P, dh]
    Returns (o [Lq, Hq, dh], k_rot [Lq, Hkv, dh]) where k_rot is what the
    block writes to cache slots [P, P + Lq).
    """
    q = np.asarray(q, np.float64)
    k_new = np.asarray(k_new, np.float64)
    v_new = np.asarray(v_new, np.float64)
    Lq, Hq, dh = q.shape
    Hkv = k_new.shape[1]
    pos = P + np.arange(Lq)
    if rope_on:
        q_r = rope(q, pos, theta)
        k_r = rope(k_new, pos, theta)
    else:
        q_r, k_r = q, k_new
    keys = np.concatenate([np.asarray(k_prefix, np.float64).reshape(Hkv, P, dh),
                           k_r.transpose(1, 0, 2)], axis=1)       # [Hkv, P+Lq, dh]
    vals = np.concatenate([np.asarray(v_prefix, np.float64).reshape(Hkv, P, dh),
                           v_new.transpose(1, 0, 2)], axis=1)
    n_keys = P + Lq
    o = np.zeros((Lq, Hq, dh))
    for h in range(Hq):
        g = (h * Hkv) // Hq
        s = q_r[:, h, :] @ keys[g].T / np.sqrt(dh)                 # [Lq, n_keys]
        if mode == CAUSAL:
            visible = np.arange(n_keys)[None, :] <= pos[:, None]
            s = np.where(visible, s, -np.inf)
        s = s - s.max(axis=1, keepdims=True)
        p = np.exp(s)
        p /= p.sum(axis=1, keepdims=True)
        o[:, h, :] = p @ vals[g]
    return o, k_r
