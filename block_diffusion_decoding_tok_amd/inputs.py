"""Seeded synthetic inputs shared by the GPU path's tests/bench and the oracle.

This module holds input recipes only: random draws and dtype casts.  It
computes none of the method's arithmetic (no softmax, no attention, no
routing, no sampling); it imports neither the oracle nor the HIP library.

Every tensor is drawn from NumPy's PCG64 through ``SeedSequence(seed)``
spawned once per named tensor, so adding a tensor never changes another.
"N(0, s)" is read as standard deviation s.  bf16 and fp8 casts use torch's
round-to-nearest-even conversions on the CPU.

Workloads (sizes are those of the pages' canvas: 256 tokens per block, a
vocabulary of 2^18, 30-layer MoE decoder with 128 experts, top-8):
  tiny_model      the tiny full loop (fp32): canvas 16 over a 32-token prompt,
                  1 layer, D 64, 4 query / 2 KV heads of 16, 4 experts top-2,
                  FFN 128, vocab 512, weights N(0, 0.02).
  attention_case  canvas attention alone (bf16): 256 queries over 2048 cached
                  prefix tokens + 256 canvas tokens, 16 query / 8 KV heads of
                  128, all N(0, 1)/sqrt(128).
  moe_case        MoE FFN on 256*B tokens, D 2816, 128 experts top-8, FFN 704,
                  hidden N(0, 1), router logits N(0, 1) plus a planted skew so
                  that 10% of experts (13) receive 40% of the assignments,
                  weights N(0, 0.02) in bf16 or fp8-e4m3 with per-row scales,
                  or random MXFP4 codes (see mxfp4_random).
  sampler_case    logits [B, 256, 2^18] N(0, 2) in bf16 with a +12 peak at a
                  random id on 60% of positions (154 of 256).
"""

import os
from dataclasses import dataclass

import numpy as np
import torch

FP8_MAX = 448.0


def _rngs(seed, names):
    ss = np.random.SeedSequence(seed)
    kids = ss.spawn(len(names))
    return {n: np.random.Generator(np.random.PCG64(k)) for n, k in zip(names, kids)}


def to_bf16(a):
    """float array -> torch.bfloat16 CPU tensor (RNE)."""
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(torch.bfloat16)


def bf16_to_f64(t):
    return t.to(torch.float64).numpy()


def quantize_fp8_rows(w):
    """Per-output-row e4m3fn quantization of w [..., N, K] (float32):
    scale = max|row| / 448, byte = RNE(w / scale) saturated to +-448.
    Returns (uint8 bytes as torch tensor, float32 scales as torch tensor)."""
    w = torch.from_numpy(np.ascontiguousarray(w, dtype=np.float32))
    amax = w.abs().amax(dim=-1, keepdim=True)
    scale = torch.where(amax > 0, amax / FP8_MAX, torch.ones_like(amax))
    q = (w / scale).clamp(-FP8_MAX, FP8_MAX).to(torch.float8_e4m3fn)
    return q.view(torch.uint8), scale.squeeze(-1).contiguous()


# ---------------------------------------------------------------- sampler

@dataclass
class SamplerCase:
    logits: torch.Tensor        # [B, L, V] bfloat16 (or float32)
    peak_ids: np.ndarray        # [B, L] planted id or -1


def sampler_case(B=1, L=256, V=262144, seed=0, sigma=2.0, peak=12.0,
                 peak_frac=0.6, dtype=torch.bfloat16):
    r = _rngs(seed, ["logits", "which", "ids"])
    x = r["logits"].standard_normal((B, L, V), dtype=np.float32) * np.float32(sigma)
    n_peak = int(round(peak_frac * L))
    peak_ids = np.full((B, L), -1, np.int64)
    for b in range(B):
        pos = r["which"].permutation(L)[:n_peak]
        ids = r["ids"].integers(0, V, size=n_peak)
        x[b, pos, ids] += np.float32(peak)
        peak_ids[b, pos] = ids
    t = torch.from_numpy(x)
    t = t.to(dtype) if dtype != torch.float32 else t
    return SamplerCase(logits=t, peak_ids=peak_ids)


# ---------------------------------------------------------------- attention

@dataclass
class AttentionCase:
    q: torch.Tensor          # [B, Lq, Hq, dh]
    k_new: torch.Tensor      # [B, Lq, Hkv, dh]  (un-rotated)
    v_new: torch.Tensor
    k_prefix: torch.Tensor   # [B, Hkv, P, dh]   (treated as already rotated)
    v_prefix: torch.Tensor
    P: int


def attention_case(B=1, Lq=256, P=2048, Hq=16, Hkv=8, dh=128, seed=0,
                   dtype=torch.bfloat16):
    r = _rngs(seed, ["q", "k", "v", "kp", "vp"])
    s = np.float32(1.0 / np.sqrt(dh))

    def draw(name, shape):
        a = r[name].standard_normal(shape, dtype=np.float32) * s
        t = torch.from_numpy(a)
        return t.to(dtype) if dtype != torch.float32 else t

    return AttentionCase(q=draw("q", (B, Lq, Hq, dh)),
                         k_new=draw("k", (B, Lq, Hkv, dh)),
                         v_new=draw("v", (B, Lq, Hkv, dh)),
                         k_prefix=draw("kp", (B, Hkv, P, dh)),
                         v_prefix=draw("vp", (B, Hkv, P, dh)), P=P)


# ---------------------------------------------------------------- MoE

@dataclass
class MoECase:
    x: torch.Tensor              # [T, D] bf16 (or f32)
    router_logits: torch.Tensor  # [T, E] float32
    w_gate_up: torch.Tensor      # [E, 2I, D] bf16 / f32, or uint8 e4m3fn bytes
    w_down: torch.Tensor         # [E, D, I]
    s_gate_up: torch.Tensor      # [E, 2I] float32 (ones unless fp8)
    s_down: torch.Tensor         # [E, D]
    hot: np.ndarray              # the planted hot experts
    beta: float                  # planted logit offset
    w_dtype: str                 # "bf16" | "fp8" | "f32"


def _hot_share(r, hot, k):
    top = np.argpartition(-r, k - 1, axis=1)[:, :k]
    return np.isin(top, hot).mean()


def router_logits_skewed(T, E, k, seed, hot_frac=0.1, share=0.40):
    """N(0,1) router logits plus +beta on round(hot_frac*E) seeded experts,
    beta found by bisection so the hot experts take ``share`` of the top-k
    assignments (to within +-0.005)."""
    r = _rngs(seed, ["logits", "hot"])
    base = r["logits"].standard_normal((T, E), dtype=np.float32)
    hot = np.sort(r["hot"].permutation(E)[:int(round(hot_frac * E))])
    lo, hi = 0.0, 6.0
    beta = 0.0
    for _ in range(60):
        beta = 0.5 * (lo + hi)
        x = base.copy()
        x[:, hot] += np.float32(beta)
        s = _hot_share(x, hot, k)
        if abs(s - share) <= 0.001:
            break
        if s < share:
            lo = beta
        else:
            hi = beta
    x = base.copy()
    x[:, hot] += np.float32(beta)
    return x, hot, beta


def _normal_f32(rng, shape, std, chunk=1 << 24):
    """std * N(0, 1) float32 array.  Chunks of 2^24 values each take their own
    child generator (seeded from ``rng``), so the result does not depend on
    how many threads fill it."""
    n = int(np.prod(shape))
    out = np.empty(n, np.float32)
    nchunks = (n + chunk - 1) // chunk
    seeds = rng.integers(0, 2**63, size=nchunks, dtype=np.int64)

    def fill(c):
        g = np.random.Generator(np.random.PCG64(int(seeds[c])))
        lo = c * chunk
        hi = min(n, lo + chunk)
        out[lo:hi] = g.standard_normal(hi - lo, dtype=np.float32)
        out[lo:hi] *= np.float32(std)

    if nchunks == 1:
        fill(0)
    else:
        import concurrent.futures as cf
        with cf.ThreadPoolExecutor(min(16, os.cpu_count() or 4)) as ex:
            list(ex.map(fill, range(nchunks)))
    return out.reshape(shape)


def mxfp4_random(rng, shape, scale_byte=120, spread=1):
    """Random OCP MXFP4 weights of logical shape [..., N, K]: code bytes
    uniform over 0..255 (two E2M1 elements each), E8M0 scale bytes uniform in
    scale_byte +- spread (2^-7, the scale that N(0, 0.02) weights take).
    Returns (codes [..., N, K / 2], scales [..., N, K / 32]) uint8 tensors."""
    *lead, K = shape
    codes = rng.integers(0, 256, tuple(lead) + (K // 2,), dtype=np.uint8)
    scales = rng.integers(scale_byte - spread, scale_byte + spread + 1,
                          tuple(lead) + (K // 32,), dtype=np.uint8)
    return torch.from_numpy(codes), torch.from_numpy(scales)


def moe_case(T=256, D=2816, E=128, k=8, I=704, w_dtype="bf16", seed=0,
             w_std=0.02, skew=True):
    r = _rngs(seed, ["x", "router", "wgu", "wd"])
    x = r["x"].standard_normal((T, D), dtype=np.float32)
    if skew:
        logits, hot, beta = router_logits_skewed(T, E, k, seed + 1)
    else:
        logits = r["router"].standard_normal((T, E), dtype=np.float32)
        hot, beta = np.zeros(0, np.int64), 0.0
    if w_dtype == "mxfp4":
        qgu, sgu = mxfp4_random(r["wgu"], (E, 2 * I, D))
        qd, sd = mxfp4_random(r["wd"], (E, D, I))
        return MoECase(to_bf16(x), torch.from_numpy(logits), qgu, qd, sgu, sd, hot, beta,
                       "mxfp4")
    wgu = _normal_f32(r["wgu"], (E, 2 * I, D), w_std)
    wd = _normal_f32(r["wd"], (E, D, I), w_std)
    if w_dtype == "fp8":
        qgu, sgu = quantize_fp8_rows(wgu)
        qd, sd = quantize_fp8_rows(wd)
        return MoECase(to_bf16(x), torch.from_numpy(logits), qgu, qd, sgu, sd,
                       hot, beta, "fp8")
    if w_dtype == "bf16":
        return MoECase(to_bf16(x), torch.from_numpy(logits), to_bf16(wgu),
                       to_bf16(wd), torch.ones(E, 2 * I), torch.ones(E, D),
                       hot, beta, "bf16")
    return MoECase(torch.from_numpy(x), torch.from_numpy(logits),
                   torch.from_numpy(wgu), torch.from_numpy(wd),
                   torch.ones(E, 2 * I), torch.ones(E, D), hot, beta, "f32")


# ---------------------------------------------------------------- models

@dataclass
class ModelDims:
    NL: int
    D: int
    Hq: int
    Hkv: int
    dh: int
    E: int
    k: int
    I: int
    V: int


TINY_DIMS = ModelDims(NL=1, D=64, Hq=4, Hkv=2, dh=16, E=4, k=2, I=128, V=512)
FULL_DIMS = ModelDims(NL=30, D=2816, Hq=16, Hkv=8, dh=128, E=128, k=8, I=704,
                      V=262144)


def model_weights(dims, seed=0, std=0.02, expert_dtype="f32",
                  dense_dtype="f32", lm_boost_rows=0, lm_boost=1.0,
                  layers=None):
    """Host weights of a random-init decoder: dict of torch tensors.

    Keys: emb [V, D], lm [V, D], and per layer l: wqkv.l [(Hq+2Hkv)dh, D],
    wo.l [D, Hq dh], wr.l [E, D], wgu.l [E, 2I, D], wd.l [E, D, I],
    sgu.l [E, 2I], sd.l [E, D].  ``lm_boost_rows`` > 0 multiplies the first
    that many LM-head rows by ``lm_boost`` (a planted variant whose positions
    become confident)."""
    d = dims
    nl = d.NL if layers is None else layers
    names = ["emb", "lm"] + [f"{n}.{l}" for l in range(nl)
                             for n in ("wqkv", "wo", "wr", "wgu", "wd")]
    r = _rngs(seed, names)
    dense = (lambda a: to_bf16(a)) if dense_dtype == "bf16" else torch.from_numpy
    out = {}
    out["emb"] = dense(_normal_f32(r["emb"], (d.V, d.D), std))
    lm = _normal_f32(r["lm"], (d.V, d.D), std)
    if lm_boost_rows:
        lm[:lm_boost_rows] *= np.float32(lm_boost)
    out["lm"] = dense(lm)
    for l in range(nl):
        out[f"wqkv.{l}"] = dense(_normal_f32(r[f"wqkv.{l}"], ((d.Hq + 2 * d.Hkv) * d.dh, d.D), std))
        out[f"wo.{l}"] = dense(_normal_f32(r[f"wo.{l}"], (d.D, d.Hq * d.dh), std))
        out[f"wr.{l}"] = dense(_normal_f32(r[f"wr.{l}"], (d.E, d.D), std))
        wgu = _normal_f32(r[f"wgu.{l}"], (d.E, 2 * d.I, d.D), std)
        wd = _normal_f32(r[f"wd.{l}"], (d.E, d.D, d.I), std)
        if expert_dtype == "fp8":
            out[f"wgu.{l}"], out[f"sgu.{l}"] = quantize_fp8_rows(wgu)
            out[f"wd.{l}"], out[f"sd.{l}"] = quantize_fp8_rows(wd)
        else:
            cast = to_bf16 if expert_dtype == "bf16" else torch.from_numpy
            out[f"wgu.{l}"] = cast(wgu)
            out[f"wd.{l}"] = cast(wd)
            out[f"sgu.{l}"] = torch.ones(d.E, 2 * d.I)
            out[f"sd.{l}"] = torch.ones(d.E, d.D)
    return out


def prompt_ids(B, n, V, seed=0):
    """Uniform prompt token ids [B, n] (int32)."""
    r = _rngs(seed, ["prompt"])
    return torch.from_numpy(r["prompt"].integers(0, V, size=(B, n)).astype(np.int32))
