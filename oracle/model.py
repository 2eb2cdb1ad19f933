"""Oracle of the decoder forward and of one block-autoregressive block
(float64).

Test infrastructure (see ``oracle/__init__.py``).

Control flow ([TR] "DiffusionGemma의 구성", flowchart; [GUIDE] "Block
Autoregressive Diffusion"; [WE0] "DiffusionGemma가 다르게 하는 점"): the prompt
is encoded into the KV cache; a canvas of random tokens is denoised one
bidirectional forward per step until the adaptive stop; the finished block is
committed to the KV cache; the next canvas starts.

Readings:
  R17 pre-norm layers, RMSNorm(x) = x / sqrt(mean(x^2) + 1e-6) with unit gain;
      no embedding scale, QK-norm, soft-cap or sliding window; untied LM head.
  R18 residual width D; attention inner width Hq*dh (Wq: D -> Hq*dh,
      Wk, Wv: D -> Hkv*dh, Wo: Hq*dh -> D); fused weight rows are [q | k | v].
  R27 the prompt is prefilled with a causal mask.
  R28 a finished block is committed by one more forward of its final tokens,
      whose rotated keys and values of every layer go to cache slots
      [P, P + L); then P += L.
  R29 autoregressive (AR) decoding on the same model -- the left-to-right
      baseline the pages compare the canvas with ([JPH] "좌→우 순차 처리와의
      대비"; [TR] "수치") -- is a causal forward of one token per row at
      position P (its K/V to slot P), the final norm and LM head, then the
      greedy choice argmax_v logits (ties to the lowest id); P += 1.  The
      pages fix no AR sampling rule; greedy is the plainest.
  R32 EOS-terminated multi-block decode ([TR] "DiffusionGemma의 구성",
      flowchart: after a block is committed, the loop ends if EOS was reached,
      else a new canvas starts): a row ends after the first committed block
      that holds the EOS id anywhere, or after max_blocks blocks.  Rows run as
      one batch; a row that has ended rides along in later blocks with its
      prefix length frozen (its canvas and cache slots past the prefix are
      scratch), and its later output blocks are -1.
"""

from dataclasses import dataclass, field
from typing import List

import numpy as np

from .attention import attention, CANVAS, CAUSAL
from .moe import moe_route, moe_ffn
from .sampler import sampler_step, init_canvas


def rmsnorm(x, eps=1e-6):
    x = np.asarray(x, np.float64)
    return x / np.sqrt((x * x).mean(axis=-1, keepdims=True) + eps)


@dataclass
class TinyModel:
    """Weights as float64 arrays (fp8 experts already dequantized)."""
    D: int
    Hq: int
    Hkv: int
    dh: int
    E: int
    k: int
    I: int
    V: int
    emb: np.ndarray                      # [V, D]
    lm: np.ndarray                       # [V, D]
    layers: List[dict] = field(default_factory=list)
    # each layer: wqkv [(Hq+2Hkv)*dh, D], wo [D, Hq*dh], wr [E, D],
    #             w_gate_up [E, 2I, D], w_down [E, D, I]
    theta: float = 10000.0


def layer_forward(m, lw, x, k_cache, v_cache, P, mode, trace=None, router_logits=None):
    """One decoder layer over x [B, n, D] at cache positions [P_b, P_b + n).

    k_cache, v_cache [B, Hkv, Tmax, dh] are updated in place with the block's
    rotated keys and values.  ``router_logits`` [B * n, E], when given, replace
    the router projection's output (a stated routing distribution for a
    random-init model).  Returns the new residual stream."""
    B, n, D = x.shape
    qd, kd = m.Hq * m.dh, m.Hkv * m.dh
    h = rmsnorm(x)
    qkv = h @ np.asarray(lw["wqkv"], np.float64).T
    o = np.zeros((B, n, qd))
    for b in range(B):
        p = int(P[b])
        q = qkv[b, :, :qd].reshape(n, m.Hq, m.dh)
        kn = qkv[b, :, qd:qd + kd].reshape(n, m.Hkv, m.dh)
        vn = qkv[b, :, qd + kd:].reshape(n, m.Hkv, m.dh)
        ob, k_rot = attention(q, kn, vn, k_cache[b, :, :p], v_cache[b, :, :p],
                              p, mode, m.theta)
        k_cache[b, :, p:p + n] = k_rot.transpose(1, 0, 2)
        v_cache[b, :, p:p + n] = vn.transpose(1, 0, 2)
        o[b] = ob.reshape(n, qd)
    x = x + o @ np.asarray(lw["wo"], np.float64).T
    h2 = rmsnorm(x).reshape(B * n, D)
    r = h2 @ np.asarray(lw["wr"], np.float64).T
    if router_logits is not None:
        r = np.asarray(router_logits, np.float64)
    ids, gates, _, _ = moe_route(r, m.k)
    y = moe_ffn(h2, lw["w_gate_up"], lw["w_down"], ids, gates)
    if trace is not None:
        trace.append(dict(router_logits=r, topk_ids=ids, gates=gates))
    return x + y.reshape(B, n, D)


def model_forward(m, tokens, k_caches, v_caches, P, mode=CANVAS,
                  lm_head=True):
    """Embed, run every layer, and (optionally) the final norm + LM head.
    Returns logits [B, n, V] or None."""
    x = np.asarray(m.emb, np.float64)[np.asarray(tokens)]
    for li, lw in enumerate(m.layers):
        x = layer_forward(m, lw, x, k_caches[li], v_caches[li], P, mode)
    if not lm_head:
        return None
    return rmsnorm(x) @ np.asarray(m.lm, np.float64).T


def prefill(m, prompt, k_caches, v_caches):
    """R27: causal forward of the prompt [B, Pn] from position 0; fills cache
    slots [0, Pn).  Returns the new prefix lengths [B]."""
    B, Pn = prompt.shape
    P = np.zeros(B, np.int64)
    model_forward(m, prompt, k_caches, v_caches, P, CAUSAL, lm_head=False)
    return P + Pn


def denoise_block(m, cfg, k_caches, v_caches, P):
    """One block: init canvas, denoise until every row is done, commit.

    Returns (tokens [B, L], steps_taken [B], trace, new P).  ``trace`` holds
    per step the logits and the sampler's outputs (with its exclusion
    diagnostics)."""
    B = len(P)
    L = cfg.canvas_len
    tokens, committed = init_canvas(cfg.seed, P, L, m.V)
    done = np.zeros(B, np.int64)
    steps = np.zeros(B, np.int64)
    trace = []
    n_steps = cfg.fixed_steps if cfg.fixed_steps > 0 else cfg.max_steps
    state = dict(renoised=None, maxprob=None, entropy=None, mean_entropy=None)
    for s in range(n_steps):
        logits = model_forward(m, tokens, k_caches, v_caches, P, CANVAS)
        res = sampler_step(logits, s, cfg, P, tokens, committed, done, **state)
        steps += 1 - done
        trace.append(dict(step=s, tokens_in=tokens, logits=logits, **res))
        tokens, committed, done = res["tokens"], res["committed"], res["done"]
        state = dict(renoised=res["renoised"], maxprob=res["maxprob"],
                     entropy=res["entropy"], mean_entropy=res["mean_entropy"])
        if done.all():
            break
    model_forward(m, tokens, k_caches, v_caches, P, CANVAS, lm_head=False)
    return tokens, steps, trace, np.asarray(P) + L


def ar_decode(m, tokens_in, k_caches, v_caches, P, n_steps):
    """R29: n_steps greedy AR steps from tokens_in [B] at positions P [B].

    Returns (tokens [B, n_steps], new P).  Each step's token is the input of
    the next; the caches receive one slot per step."""
    tok = np.asarray(tokens_in, np.int64).copy()
    P = np.asarray(P, np.int64).copy()
    out = []
    for _ in range(n_steps):
        logits = model_forward(m, tok[:, None], k_caches, v_caches, P, CAUSAL)
        tok = np.argmax(logits[:, 0], axis=1)          # first maximum: lowest id
        out.append(tok)
        P = P + 1
    return np.stack(out, axis=1), P


def generate(m, cfg, k_caches, v_caches, P, eos_id, max_blocks):
    """R32: blocks until every row has produced a block holding eos_id, or
    max_blocks blocks.  Returns (tokens [B, max_blocks, L] with -1 after a
    row's last block, n_blocks [B], final P [B])."""
    P = np.array(P, np.int64)
    B, L = len(P), cfg.canvas_len
    out = np.full((B, max_blocks, L), -1, np.int64)
    n_blocks = np.zeros(B, np.int64)
    active = np.ones(B, bool)
    for blk in range(max_blocks):
        if not active.any():
            break
        tokens, _, _, P_next = denoise_block(m, cfg, k_caches, v_caches, P)
        for b in range(B):
            if not active[b]:
                continue
            out[b, blk] = tokens[b]
            n_blocks[b] = blk + 1
            P[b] = P_next[b]
            if np.any(tokens[b] == eos_id):
                active[b] = False
    return out, n_blocks, P
