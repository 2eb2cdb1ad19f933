"""Oracle of one sampler step of the canvas denoiser (float64).

Test infrastructure (see ``oracle/__init__.py``).

What the pages fix ([TR] "DiffusionGemma의 구성", sampler-settings paragraph):
canvas length 256, at most 48 denoising steps, temperature decaying linearly
from 0.8 to 0.4, adaptive stop threshold 0.005.  Confident positions are kept
as anchors ([GN] "텍스트 확산의 작동 방식"; [WE0] "DiffusionGemma가 다르게 하는
점") and low-confidence positions are re-randomized ([GUIDE] "Uniform State
Diffusion"; [JPH] "좌→우 순차 처리와의 대비").

Readings where the pages are silent (numbering as in the design notes):
  R1  T_s = T0 + (T1 - T0) * s / (S - 1), over the step cap S (T0 when S = 1).
  R2  z = logits / T_s; p = softmax(z); maxprob = max p = 1 / sum exp(z - max z).
  R3  entropy H = -sum p ln p in nats = ln Z - sum p (z - m).
  R4  stop statistic: mean of H over all L positions of the row (committed
      ones included); stop when it is strictly below the threshold.
  R5  the step's update is applied first; done = stop or last step.
  R6  commit: uncommitted position with maxprob >= commit_prob takes the
      Gumbel sample and is frozen for the rest of the block.
  R7  re-noise: otherwise, maxprob < renoise_prob -> a fresh uniform id.
  R8  the step that ends the block never re-noises.
  R9  otherwise the position takes the Gumbel sample.
  R10 sample = argmax_v (z_v + g_v), ties to the lowest v.
  R14 fixed_steps > 0 disables the adaptive stop; the schedule stays over S.
  R31 the entropy-bound commit policy (the serving configuration's
      "entropy_bound" sampler with bound 0.1: a confidence-based early exit;
      developer guide, "vLLM으로 서빙하기"), read as entropy-bounded
      unmasking (Ben-Hamu et al., "Accelerated Sampling from Masked Diffusion
      Models via Entropy Bounded Unmasking", 2025) carried over to the
      uniform-state canvas: at each step the uncommitted positions are ranked
      by entropy (ties to the lower position) and the longest prefix U of that
      ranking with sum_U H - max_U H <= bound is committed with its samples
      (at least one position per step); the rest follow R7 and R9.  In the
      adaptive mode the block also ends once every position is committed.
Rows already done on entry are left untouched.
"""

from dataclasses import dataclass

import numpy as np

from .philox import (gumbel_row, renoise_id, canvas_id)


@dataclass
class SamplerCfg:
    canvas_len: int = 256
    max_steps: int = 48
    fixed_steps: int = 0          # 0 -> adaptive stop
    temp_start: float = 0.8
    temp_end: float = 0.4
    stop_entropy: float = 0.005
    commit_prob: float = 0.9
    renoise_prob: float = 0.1
    seed: int = 0
    commit_policy: int = 0        # 0: maxprob >= commit_prob (R6); 1: entropy bound (R31)
    entropy_bound: float = 0.1


COMMIT_MAXPROB = 0
COMMIT_ENTROPY_BOUND = 1


def entropy_bound_select(entropy, committed, bound):
    """R31: the positions to commit this step.  Candidates are the
    uncommitted positions ranked by (entropy, position); the longest prefix
    whose entropies sum, minus their maximum (the last one), to at most
    ``bound`` is selected.  Returns a boolean mask."""
    order = sorted((i for i in range(len(entropy)) if not committed[i]),
                   key=lambda i: (entropy[i], i))
    sel = np.zeros(len(entropy), bool)
    total = 0.0                    # sum of the prefix before the candidate
    for i in order:
        if total > bound:
            break
        sel[i] = True
        total += entropy[i]
    return sel


def temperature(step, max_steps, t0=0.8, t1=0.4):
    """R1: linear decay from t0 (step 0) to t1 (step max_steps - 1)."""
    if max_steps <= 1:
        return float(t0)
    return t0 + (t1 - t0) * step / (max_steps - 1)


def position_stats(logits, T):
    """Softmax statistics of one position's logits at temperature T.

    Returns (maxprob, entropy, z) with z = logits / T (float64)."""
    z = np.asarray(logits, dtype=np.float64) / T
    m = z.max()
    e = np.exp(z - m)
    Z = e.sum()
    maxprob = 1.0 / Z
    entropy = np.log(Z) - (e * (z - m)).sum() / Z
    return maxprob, entropy, z


def sampler_step(logits, step, cfg, prefix_pos, tokens, committed, done,
                 renoised=None, maxprob=None, entropy=None, mean_entropy=None):
    """One sampler step over a batch of canvases.

    logits      [B, L, V] (any float dtype; upcast to float64 exactly)
    prefix_pos  [B] absolute position of canvas slot 0 (Philox counter c1)
    tokens      [B, L] int, committed [B, L] 0/1, done [B] 0/1 (inputs)
    renoised, maxprob, entropy, mean_entropy: previous contents of the output
        buffers, returned unchanged for rows that are done on entry.

    Returns a dict with the new state and outputs plus diagnostics used by
    the exclusion rules: ``sample`` (Gumbel-max id), ``gap`` (top-1 minus
    top-2 perturbed score), ``top_score``, ``ends`` (this step ended the row).
    """
    logits = np.asarray(logits)
    B, L, V = logits.shape
    S = cfg.max_steps
    T = temperature(step, S, cfg.temp_start, cfg.temp_end)

    tok = np.array(tokens, dtype=np.int64, copy=True)
    com = np.array(committed, dtype=np.int64, copy=True)
    dn = np.array(done, dtype=np.int64, copy=True)
    ren = (np.zeros((B, L), np.int64) if renoised is None
           else np.array(renoised, dtype=np.int64, copy=True))
    mp = (np.zeros((B, L)) if maxprob is None
          else np.array(maxprob, dtype=np.float64, copy=True))
    ent = (np.zeros((B, L)) if entropy is None
           else np.array(entropy, dtype=np.float64, copy=True))
    ment = (np.zeros(B) if mean_entropy is None
            else np.array(mean_entropy, dtype=np.float64, copy=True))
    sample = np.full((B, L), -1, np.int64)
    gap = np.full((B, L), np.inf)
    top_score = np.zeros((B, L))
    ends = np.zeros(B, np.int64)

    for b in range(B):
        if done[b]:
            continue
        for i in range(L):
            pos = int(prefix_pos[b]) + i
            p_max, h, z = position_stats(logits[b, i].astype(np.float64), T)
            mp[b, i] = p_max
            ent[b, i] = h
            score = z + gumbel_row(cfg.seed, pos, step, b, V)
            v = int(np.argmax(score))             # first maximum = lowest id
            sample[b, i] = v
            top_score[b, i] = score[v]
            rest = np.delete(score, v)
            gap[b, i] = score[v] - rest.max() if rest.size else np.inf
        ment[b] = ent[b].mean()
        if cfg.commit_policy == COMMIT_ENTROPY_BOUND:
            commit = entropy_bound_select(ent[b], com[b], cfg.entropy_bound)
        else:
            commit = mp[b] >= cfg.commit_prob
        if cfg.fixed_steps > 0:
            end = step == cfg.fixed_steps - 1
        else:
            end = (ment[b] < cfg.stop_entropy) or (step == S - 1)
            if cfg.commit_policy == COMMIT_ENTROPY_BOUND:
                end = end or bool(np.all(com[b] | commit))
        ends[b] = int(end)
        for i in range(L):
            ren[b, i] = 0
            if com[b, i]:
                continue
            if commit[i]:
                tok[b, i] = sample[b, i]
                com[b, i] = 1
            elif mp[b, i] < cfg.renoise_prob and not end:
                tok[b, i] = renoise_id(cfg.seed, int(prefix_pos[b]) + i,
                                       step, b, V)
                ren[b, i] = 1
            else:
                tok[b, i] = sample[b, i]
        dn[b] = int(end)

    return dict(tokens=tok, committed=com, renoised=ren, maxprob=mp,
                entropy=ent, mean_entropy=ment, done=dn, sample=sample,
                gap=gap, top_score=top_score, ends=ends, temperature=T)


def init_canvas(seed, prefix_pos, L, V):
    """R13: the initial canvas holds uniform-random ids (stream 2); nothing is
    committed.  ``prefix_pos`` [B] gives the absolute position of slot 0."""
    B = len(prefix_pos)
    tok = np.zeros((B, L), np.int64)
    for b in range(B):
        for i in range(L):
            tok[b, i] = canvas_id(seed, int(prefix_pos[b]) + i, b, V)
    return tok, np.zeros((B, L), np.int64)
