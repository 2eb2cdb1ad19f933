"""Benchmark of the canvas denoising hot path on one MI355X.

Workload (the end-to-end block-autoregressive decode): a random-init decoder
of 30 layers (D 2816; 16 query / 8 KV heads of 128; MoE of 128 experts, top-8,
FFN 704, fp8-e4m3 experts with per-row scales, bf16 dense weights), vocabulary
2^18, an 8192-token prompt prefilled into the KV cache (untimed), then blocks
of 256 canvas tokens, each run for a fixed number of denoise steps (default 12;
the random weights do not converge) and committed to the KV cache.

A "step" is one canvas denoise step: the forward over the canvas (all 30
layers, canvas attention over the cache, MoE), the LM head and the sampler.
``--steps K`` steps are timed as consecutive fixed-step blocks: K // block_steps
blocks of block_steps steps, then one block of the remaining K % block_steps
steps, bracketed by device synchronization.  Each block is one hipGraph
replay of dg_denoise_block_deferred: a block's commit forward (the K/V of its
final tokens) runs fused into the next block's first step, and the last
block's by dg_commit_pending, inside the timed region.  ``--warmup W`` steps
run the same way, untimed, before, and then the timed sequence once more, so
no graph capture falls inside the timed region.

Printed: one JSON line with steps/s (value), canvas tok/s, ms per step,
tok/s at 12 steps per block, the roofline of the dominant kernel (the experts'
gate/up GEMM), and the oracle's throughput on the host cores for a bounded
sample.
"""

import argparse
import json
import os
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

from block_diffusion_decoding_tok_amd import dg  # noqa: E402
from block_diffusion_decoding_tok_amd.inputs import (FULL_DIMS, ModelDims, prompt_ids,  # noqa: E402
                                                     router_logits_skewed)

METRIC = "canvas denoise steps/s & canvas tok/s (256-tok, bs1); % of MFMA/HBM roofline"
HBM_PEAK_GBS = 8000.0
CANVAS = 256
PROMPT = 8192
PREFILL_CHUNK = 2048          # prompt tokens per row in one prefill forward
AR_STEPS = 64


def make_weights(d, seed=0):
    """Device weights N(0, 0.02): bf16 dense, fp8 experts (quantized per row
    from a float32 draw); every weight but the embedding is repacked into the
    tiled layout the streaming kernels read contiguously."""
    dev = "cuda"
    w = {}

    def bf16(shape, sid, pack=True):
        t = torch.empty(shape, dtype=torch.bfloat16, device=dev)
        dg.dg_fill_normal(t, 0.02, seed, sid)
        return dg.dg_pack_weights(t) if pack else t

    w["emb"] = bf16((d.V, d.D), 1, pack=False)
    w["lm"] = bf16((d.V, d.D), 2)
    tmp = torch.empty((d.E, 2 * d.I, d.D), dtype=torch.float32, device=dev)
    for l in range(d.NL):
        base = 16 + 16 * l
        w[f"wqkv.{l}"] = bf16(((d.Hq + 2 * d.Hkv) * d.dh, d.D), base)
        w[f"wo.{l}"] = bf16((d.D, d.Hq * d.dh), base + 1)
        w[f"wr.{l}"] = bf16((d.E, d.D), base + 2)
        for name, shape, sid in (("gu", (d.E, 2 * d.I, d.D), base + 3), ("d", (d.E, d.D, d.I), base + 4)):
            src = tmp.view(-1)[: int(np.prod(shape))].view(shape)
            dg.dg_fill_normal(src, 0.02, seed, sid)
            q = torch.empty(shape, dtype=torch.uint8, device=dev)
            s = torch.empty(shape[:-1], dtype=torch.float32, device=dev)
            dg.dg_quantize_fp8_rows(src, q, s)
            w[f"w{name}.{l}"] = dg.dg_pack_weights(q)
            w[f"s{name}.{l}"] = s
            del q
    torch.cuda.synchronize()
    del tmp
    return w


def make_mxfp4_experts(d, w, seed=0):
    """The same model with MXFP4 experts: the experts' float32 draws (same
    Philox streams as the fp8 experts) quantized on the device to OCP MXFP4
    and tile-packed; the dense weights are shared with w."""
    dev = "cuda"
    out = {k: v for k, v in w.items() if not k.startswith(("wgu.", "wd.", "sgu.", "sd."))}
    tmp = torch.empty((d.E, 2 * d.I, d.D), dtype=torch.float32, device=dev)
    for l in range(d.NL):
        base = 16 + 16 * l
        for name, shape, sid in (("gu", (d.E, 2 * d.I, d.D), base + 3), ("d", (d.E, d.D, d.I), base + 4)):
            src = tmp.view(-1)[: int(np.prod(shape))].view(shape)
            dg.dg_fill_normal(src, 0.02, seed, sid)
            codes, scales = dg.dg_quantize_mxfp4(src)
            out[f"w{name}.{l}"] = dg.dg_pack_mxfp4(codes, scales)
            del codes, scales
    torch.cuda.synchronize()
    del tmp
    return out


def entropy_bound_timing(d, w, model, B, kc, vc, Pd, stream):
    """The entropy-bound commit policy (bound 0.1, adaptive mode):
      * one block on the random-init model, whose positions stay uncertain
        (entropy about 12 nats): one commit per step, so it runs to the cap
        of 48 steps in chunks of 4 with a host check of the done flags between
        chunks -- set against the same 48 steps as one graph (fixed mode);
      * dg_generate with EOS on a copy of the model whose first 16 LM-head
        rows are scaled by 400 (a planted confident head): every position
        fits the bound at once, so a block ends after one step; 4 blocks
        without EOS, then with the EOS id set to a token of the first block.
    The prompt cache is reused; the prefix is rewound after each run."""
    eb_cfg = dg.sampler_cfg(CANVAS, 48, 0, seed=0, commit_policy=dg.DG_COMMIT_ENTROPY_BOUND,
                            entropy_bound=0.1)
    fixed = dg.sampler_cfg(CANVAS, 48, 48, seed=0)
    tok = torch.empty((B, CANVAS), dtype=torch.int32, device="cuda")
    steps = torch.empty(B, dtype=torch.int32, device="cuda")

    def one_block(m, c):
        Pd.fill_(PROMPT)
        dg.dg_denoise_block(m, c, B, kc, vc, Pd, tok, steps)      # capture + warm
        stream.synchronize()
        Pd.fill_(PROMPT)
        stream.synchronize()
        t0 = time.perf_counter()
        dg.dg_denoise_block(m, c, B, kc, vc, Pd, tok, steps)
        stream.synchronize()
        return 1e3 * (time.perf_counter() - t0), steps.cpu().tolist()
    ms_eb, st_eb = one_block(model, eb_cfg)
    ms_fx, _ = one_block(model, fixed)
    out = {"bound": 0.1,
           "random_init_block": {"steps": st_eb, "ms": round(ms_eb, 2),
                                 "fixed_48_step_graph_ms": round(ms_fx, 2),
                                 "adaptive_overhead_frac": round(ms_eb / ms_fx - 1, 4)}}
    lm = w["lm"].clone()
    lm[: (d.D // 64) * 1024] *= 400.0                        # tile 0: LM rows 0..15
    w_pl = dict(w)
    w_pl["lm"] = lm
    m_pl = dg.DGModel(d, w_pl, B, CANVAS, dg.DG_BF16, dg.DG_FP8_E4M3,
                      weight_layout=dg.DG_LAYOUT_TILED)
    m_pl.set_router_override(planted_router_logits(d, CANVAS * B))

    def gen(eos):
        Pd.fill_(PROMPT)
        dg.dg_generate(m_pl, eb_cfg, B, kc, vc, Pd, eos, 4)       # capture + warm
        stream.synchronize()
        Pd.fill_(PROMPT)
        stream.synchronize()
        t0 = time.perf_counter()
        toks, nb, st = dg.dg_generate(m_pl, eb_cfg, B, kc, vc, Pd, eos, 4)
        stream.synchronize()
        el = time.perf_counter() - t0
        n_tok = int(nb.sum().item()) * CANVAS
        return dict(ms=round(1e3 * el, 2), n_blocks=nb.cpu().tolist(),
                    steps=st.cpu().tolist(), tok_per_s=round(n_tok / el, 1)), toks
    g_noeos, toks = gen(-1)
    eos = int(toks[0, 0, 0].item())
    g_eos, _ = gen(eos)
    g_eos["eos_id"] = eos
    # what the blocks would take with no step beyond each block's end: the
    # steps taken at the fixed-graph step time, plus one commit per block
    # (step and commit times from the 48-step and 12-step fixed blocks)
    fixed12 = dg.sampler_cfg(CANVAS, 48, 12, seed=0)
    ms_12, _ = one_block(model, fixed12)
    step_ms = (ms_fx - ms_12) / 36
    commit_ms = ms_12 - 12 * step_ms
    for g in (g_noeos, g_eos):
        n_steps = sum(sum(r) for r in g["steps"])
        n_blk = sum(g["n_blocks"])
        g["steps_plus_commits_ms"] = round(n_steps * step_ms + n_blk * commit_ms, 2)
    out["step_ms"] = round(step_ms, 3)
    out["commit_ms"] = round(commit_ms, 3)
    out["planted_confident_generate"] = {"no_eos": g_noeos, "eos": g_eos}
    m_pl.close()
    del lm, w_pl
    Pd.fill_(PROMPT)
    stream.synchronize()
    return out


def block_plan(n_steps, block_steps):
    """Fixed step counts of the consecutive blocks that make up n_steps
    denoise steps: whole blocks of block_steps, then one shorter block with
    the remainder (each block is committed, as a finished block is)."""
    plan = [block_steps] * (n_steps // block_steps)
    if n_steps % block_steps:
        plan.append(n_steps % block_steps)
    return plan


def planted_router_logits(d, T, seed=100):
    """Per-layer router logits with the stated MoE routing: N(0, 1) plus a
    planted skew so that 13 of 128 experts take 40% of the top-8 assignments
    (a random-init router instead sends most canvas tokens to a few experts
    after the first layer)."""
    return [torch.from_numpy(router_logits_skewed(T, d.E, d.k, seed=seed + l)[0]).to("cuda")
            for l in range(d.NL)]


def _graph_ms(fn, reps):
    """Average device time of fn over reps calls captured into one graph and
    replayed between two HIP events on the replay stream (host launch cost is
    not counted)."""
    for _ in range(3):
        fn()
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for _ in range(reps):
            fn()
    graph.replay()
    torch.cuda.synchronize()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record()
    graph.replay()
    end.record()
    torch.cuda.synchronize()
    return start.elapsed_time(end) / reps


def moe_roofline(model_w, d, B, reps=20, mxfp4=False):
    """The dominant kernel of the step, the experts' gate/up GEMM
    (dg_moe_gate_up), timed on a middle layer's experts for the canvas tokens
    with that layer's planted routing (every expert active).  Algorithmic
    bytes: every expert's fp8 gate/up rows and their scales read once, the
    token rows read once, the hidden rows written once, the routing tables.
    The whole expert FFN (gate/up + down + combine) is timed beside it."""
    T = CANVAS * B
    dev = "cuda"
    layer = d.NL // 2
    slots = T * d.k
    g = torch.Generator(device=dev).manual_seed(5)
    logits = torch.from_numpy(router_logits_skewed(T, d.E, d.k, seed=100 + layer)[0]).to(dev)
    x = (torch.randn((T, d.D), device=dev, generator=g)).to(torch.bfloat16)
    y = torch.zeros((T, d.D), device=dev)
    ids, gates, off, rows = dg.dg_moe_route(logits, d.k)
    h = torch.empty((slots, d.I), dtype=torch.bfloat16, device=dev)
    ws = torch.empty(dg.lib().dg_moe_ffn_workspace_size(T, d.D, d.I, d.E, d.k, dg.DG_BF16),
                     dtype=torch.uint8, device=dev)
    wgu, wd = model_w[f"wgu.{layer}"], model_w[f"wd.{layer}"]
    sgu, sd = model_w.get(f"sgu.{layer}"), model_w.get(f"sd.{layer}")
    kw = dict(w_layout=dg.DG_LAYOUT_TILED, E=d.E, I=d.I)
    if mxfp4:
        kw["w_dtype"] = dg.DG_MXFP4
    ms_gu = _graph_ms(lambda: dg.dg_moe_gate_up(x, wgu, sgu, off, rows, d.k, h=h, **kw), reps)
    ms_ffn = _graph_ms(lambda: dg.dg_moe_ffn(x, wgu, wd, sgu, sd, ids, gates, off, rows, y,
                                             ws=ws, **kw), reps)
    route_bytes = (d.E + 1) * 4 + slots * 4

    def wbytes(rows, K):                       # weight rows with their scales
        return rows * K // 2 + rows * K // 32 if mxfp4 else rows * K + 4 * rows
    gu_bytes = (wbytes(d.E * 2 * d.I, d.D)     # gate/up rows + scales
                + T * d.D * 2                  # token rows (bf16)
                + slots * d.I * 2              # hidden rows written (bf16)
                + route_bytes)
    # whole FFN: + down rows and scales, h read, gate-weighted slot rows
    # written + read (bf16), y read + written (f32)
    ffn_bytes = (gu_bytes + wbytes(d.E * d.D, d.I) + slots * d.I * 2
                 + slots * d.D * 2 * 2 + T * d.D * 4 * 2 + slots * 4)
    fmt = "MXFP4" if mxfp4 else "fp8"
    # the library's dispatch: one-wave items up to 40 slots per expert on
    # average, LDS-staged 64-token tiles above
    kname = "gemm_wave_kernel" if slots <= 40 * d.E else "gemm_stream_kernel"
    return dict(kernel=(f"{kname} (dg_moe_gate_up): experts of layer {layer}, {T} "
                        f"tokens, {fmt} tiled weights, planted routing (all 128 experts active)"),
                ms=ms_gu, algo_bytes=gu_bytes, gbs=gu_bytes / (ms_gu * 1e-3) / 1e9,
                ffn_ms=ms_ffn, ffn_bytes=ffn_bytes, ffn_gbs=ffn_bytes / (ms_ffn * 1e-3) / 1e9)


MFMA_BF16_PEAK_TFLOPS = 2500.0


def attention_fraction(d, B, P, reps=20):
    """dg_canvas_attention (RoPE + split-KV MFMA kernel + merge) on one
    layer's shapes: 256 canvas queries over P cached keys + the canvas.
    FLOPs = 4 * Hq * L * (P + L) * dh (QK^T and PV)."""
    dev = "cuda"
    g = torch.Generator(device=dev).manual_seed(9)
    L = CANVAS
    Tmax = P + L
    q = (torch.randn((B, L, d.Hq, d.dh), device=dev, generator=g) / d.dh ** 0.5).to(torch.bfloat16)
    kn = (torch.randn((B, L, d.Hkv, d.dh), device=dev, generator=g) / d.dh ** 0.5).to(torch.bfloat16)
    vn = torch.randn((B, L, d.Hkv, d.dh), device=dev, generator=g).to(torch.bfloat16)
    kc = (torch.randn((B, d.Hkv, Tmax, d.dh), device=dev, generator=g) / d.dh ** 0.5).to(torch.bfloat16)
    vc = torch.randn((B, d.Hkv, Tmax, d.dh), device=dev, generator=g).to(torch.bfloat16)
    Pd = torch.full((B,), P, dtype=torch.int32, device=dev)
    out = torch.empty_like(q)
    ws = torch.empty(dg.lib().dg_attention_workspace_size(B, L, d.Hq, d.Hkv, d.dh, Tmax, dg.DG_BF16),
                     dtype=torch.uint8, device=dev)
    ms = _graph_ms(lambda: dg.dg_canvas_attention(q, kn, vn, kc, vc, Pd, out=out, ws=ws), reps)
    flops = 4.0 * B * d.Hq * L * (P + L) * d.dh
    tf = flops / (ms * 1e-3) / 1e12
    return {"op": f"dg_canvas_attention bf16, batch {B}, 256 queries over {P} + 256 keys, 16/8 "
                  "heads of 128 (RoPE + MFMA kernel + split merge)",
            "ms_per_call": round(ms, 4), "tflops": round(tf, 1), "bound": "mfma",
            "peak_tflops": MFMA_BF16_PEAK_TFLOPS, "frac": round(tf / MFMA_BF16_PEAK_TFLOPS, 4)}


def sampler_fraction(d, B, reps=20):
    """dg_sampler_step on bf16 logits [B, 256, V] (step 0): HBM bytes = the
    logits read once; also the Gumbel draws per second (VALU-bound: a quarter
    Philox-10 call and two logarithms per logit)."""
    dev = "cuda"
    L = CANVAS
    logits = torch.empty((B, L, d.V), dtype=torch.bfloat16, device=dev)
    dg.dg_fill_normal(logits, 2.0, 3, 11)
    cfg = dg.sampler_cfg(L, 48, 0, seed=0)
    Pd = torch.full((B,), PROMPT, dtype=torch.int32, device=dev)
    tok = torch.zeros((B, L), dtype=torch.int32, device=dev)
    com = torch.zeros((B, L), dtype=torch.uint8, device=dev)
    ren = torch.zeros_like(com)
    mp = torch.zeros((B, L), dtype=torch.float32, device=dev)
    en = torch.zeros_like(mp)
    me = torch.zeros(B, dtype=torch.float32, device=dev)
    done = torch.zeros(B, dtype=torch.int32, device=dev)
    ws = torch.empty(dg.lib().dg_sampler_workspace_size(B, L, d.V), dtype=torch.uint8, device=dev)
    ms = _graph_ms(lambda: dg.dg_sampler_step(logits, 0, cfg, Pd, tok, com, ren, mp, en, me, done,
                                              ws=ws), reps)
    gbs = B * L * d.V * 2 / (ms * 1e-3) / 1e9
    # the entropy-bound commit policy on the same logits (its ranked
    # selection runs in the per-row finishing kernel)
    cfg_eb = dg.sampler_cfg(L, 48, 0, seed=0, commit_policy=dg.DG_COMMIT_ENTROPY_BOUND,
                            entropy_bound=0.1)
    com.zero_()
    ms_eb = _graph_ms(lambda: dg.dg_sampler_step(logits, 0, cfg_eb, Pd, tok, com, ren, mp, en, me,
                                                 done, ws=ws), reps)
    return {"op": f"dg_sampler_step, bf16 logits [{B}, 256, {d.V}], step 0",
            "ms_per_call": round(ms, 4), "ms_per_call_entropy_bound": round(ms_eb, 4),
            "gbs": round(gbs, 1), "bound": "alu (Philox + 2 ln per logit)",
            "hbm_frac": round(gbs / HBM_PEAK_GBS, 4),
            "gumbel_draws_per_s": float(f"{B * L * d.V / (ms * 1e-3):.4g}")}


# Sources of the gate/up kernel: a traffic figure taken with byte counters
# is used only while these files are unchanged.
_KERNEL_SOURCES = ["block_diffusion_decoding_tok_amd/csrc/gemm_mfma.h",
                   "block_diffusion_decoding_tok_amd/csrc/moe.hip",
                   "block_diffusion_decoding_tok_amd/csrc/common.h"]
_COUNTER_FILE = os.path.join(ROOT, "profiles", "moe_gate_up_counters_canvas256.md")


def forward_floor_bytes(d, B, n, P, experts_touched):
    """Bytes one forward of n tokens per row (B rows, P cached keys per row)
    has to move at the least: every layer's dense weights, the fp8 rows and
    scales of the experts its tokens touch, the K/V cache it attends over
    (read) and the new keys' K/V (written); the LM head's weights and the
    logits (written, then read by the sampler or argmax).  Activations are
    left out (a few MB per layer)."""
    dense = ((d.Hq + 2 * d.Hkv) * d.dh * d.D + d.D * d.Hq * d.dh + d.E * d.D) * 2
    experts = experts_touched * ((2 * d.I * d.D + d.D * d.I) + (2 * d.I + d.D) * 4)
    kv = B * 2 * d.Hkv * d.dh * 2 * ((P + n) + n)
    head = d.V * d.D * 2 + 2 * B * n * d.V * 2
    return d.NL * (dense + experts + kv) + head


def kernel_source_hash():
    import hashlib
    hsh = hashlib.sha256()
    for f in _KERNEL_SOURCES:
        with open(os.path.join(ROOT, f), "rb") as fh:
            hsh.update(fh.read())
    return hsh.hexdigest()[:16]


def measured_traffic():
    """HBM bytes per launch of the gate/up kernel from the committed counter
    summary (FETCH_SIZE and WRITE_SIZE, scaled by a plain copy), or None when
    there is none or the kernel's sources changed since it was taken."""
    if not os.path.exists(_COUNTER_FILE):
        return None
    vals = {}
    with open(_COUNTER_FILE) as fh:
        for line in fh:
            if line.startswith("- ") and ":" in line:
                key, _, val = line[2:].partition(":")
                vals[key.strip()] = val.strip().strip("`")
    if vals.get("source_hash") != kernel_source_hash() or "traffic_bytes_per_launch" not in vals:
        return None
    return int(float(vals["traffic_bytes_per_launch"]))


def copy_calibration(nbytes=1 << 28):
    """One plain device copy of a known size, so FETCH_SIZE / WRITE_SIZE
    counters taken over this run can be scaled to bytes (the copy reads and
    writes exactly ``nbytes``)."""
    src = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    src.fill_(1)
    torch.cuda.synchronize()
    dst.copy_(src)
    torch.cuda.synchronize()
    return nbytes


def cpu_baseline(d, B, P, seed=0):
    """The oracle (float64 NumPy) on the host cores for a bounded sample of one
    denoise step: one decoder layer's weights applied 4 times over the whole
    canvas of one row, plus the LM head and sampler for 32 of its 256
    positions; scaled to one full step (30 layers, 256 positions) of B rows."""
    from oracle import SamplerCfg, layer_forward, position_stats, sampler_step, rmsnorm
    from oracle.attention import CANVAS as MASK_CANVAS
    from oracle.host_weights import oracle_model
    from block_diffusion_decoding_tok_amd.inputs import model_weights

    d1 = ModelDims(NL=1, D=d.D, Hq=d.Hq, Hkv=d.Hkv, dh=d.dh, E=d.E, k=d.k, I=d.I, V=d.V)
    w = model_weights(d1, seed=seed, expert_dtype="fp8", dense_dtype="bf16")
    m = oracle_model(d1, w)
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((1, CANVAS, d.D)) * 0.02
    kc = rng.standard_normal((1, d.Hkv, P + CANVAS, d.dh)) / np.sqrt(d.dh)
    vc = rng.standard_normal((1, d.Hkv, P + CANVAS, d.dh)) / np.sqrt(d.dh)
    n_pass = 4                   # the layer is applied n_pass times in a row
    t0 = time.perf_counter()
    for _ in range(n_pass):
        x = layer_forward(m, m.layers[0], x, kc, vc, np.array([P]), MASK_CANVAS)
    t_layer = (time.perf_counter() - t0) / n_pass
    n_pos = 32
    lm = w["lm"].to(torch.float64).numpy()
    t0 = time.perf_counter()
    logits = rmsnorm(x[0, :n_pos]) @ lm.T
    cfg = SamplerCfg(canvas_len=n_pos)
    sampler_step(logits[None], 0, cfg, np.array([P]), np.zeros((1, n_pos), np.int64),
                 np.zeros((1, n_pos), np.int64), np.zeros(1, np.int64))
    t_head = time.perf_counter() - t0
    t_step = B * (d.NL * t_layer + t_head * CANVAS / n_pos)
    cores = len(os.sched_getaffinity(0))
    omp = os.environ.get("OMP_NUM_THREADS")
    if omp and omp.isdigit():
        cores = min(cores, int(omp))
    return dict(value=1.0 / t_step, unit="steps/s", cores=cores, kind="oracle",
                sample=(f"one decoder layer over the 256-token canvas, {n_pass} passes "
                        f"({t_layer:.2f} s each) + LM head and sampler on {n_pos} of 256 positions "
                        f"({t_head:.2f} s), prefix {P}, scaled to one full step ({d.NL} layers, "
                        f"256 positions) of batch {B}"),
                measured_s=n_pass * t_layer + t_head)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=48)
    ap.add_argument("--warmup", type=int, default=12)
    ap.add_argument("--batch", type=int, default=1)
    ap.add_argument("--block-steps", type=int, default=12)
    ap.add_argument("--layers", type=int, default=FULL_DIMS.NL)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-roofline", action="store_true")
    ap.add_argument("--no-natural", action="store_true",
                    help="skip the secondary timing with the random router's own routing")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="run one 256 MiB device copy (scale for byte counters)")
    ap.add_argument("--no-ar", action="store_true", help="skip the AR-mode decode timing")
    ap.add_argument("--no-prefill-timing", action="store_true",
                    help="skip the timed re-encoding of the prompt")
    ap.add_argument("--no-mxfp4", action="store_true",
                    help="skip the timing of the same model with MXFP4 experts")
    ap.add_argument("--no-eb", action="store_true",
                    help="skip the entropy-bound policy / EOS generate timings")
    ap.add_argument("--steps48", action="store_true",
                    help="also time 4 blocks at 48 fixed steps each")
    a = ap.parse_args()
    if a.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: there is no multi-GPU path (the canvas "
              "path would shard by batch rows, one model replica per GPU, with no "
              "collective on the step).", file=sys.stderr)
        sys.exit(2)
    if a.steps < 1 or a.warmup < 0 or not 1 <= a.block_steps <= 48:
        sys.exit("need --steps >= 1, --warmup >= 0 and 1 <= --block-steps <= 48")
    d = ModelDims(NL=a.layers, D=FULL_DIMS.D, Hq=FULL_DIMS.Hq, Hkv=FULL_DIMS.Hkv,
                  dh=FULL_DIMS.dh, E=FULL_DIMS.E, k=FULL_DIMS.k, I=FULL_DIMS.I, V=FULL_DIMS.V)
    B = a.batch
    torch.cuda.set_device(0)
    plan = block_plan(a.steps, a.block_steps)          # timed blocks
    warm_plan = block_plan(a.warmup, a.block_steps) if a.warmup else []
    warm_plan += [f for f in sorted(set(plan)) if f not in warm_plan]
    n_blocks = len(plan)
    # the cache holds the prompt plus the longest run of consecutive blocks
    # (the timed blocks, the warmup blocks, the 4 blocks of --steps48 and of
    # the EOS generate timing); the prefix is rewound before each run
    Tmax = PROMPT + CANVAS * max(n_blocks, len(warm_plan), 4)
    t_setup = time.perf_counter()
    w = make_weights(d)
    model = dg.DGModel(d, w, B, CANVAS, dg.DG_BF16, dg.DG_FP8_E4M3,
                       weight_layout=dg.DG_LAYOUT_TILED, max_prefill_tokens=PREFILL_CHUNK * B)
    kc = [torch.zeros((B, d.Hkv, Tmax, d.dh), dtype=torch.bfloat16, device="cuda") for _ in range(d.NL)]
    vc = [torch.zeros_like(kc[0]) for _ in range(d.NL)]
    Pd = torch.zeros(B, dtype=torch.int32, device="cuda")
    stream = torch.cuda.Stream()
    tok = torch.empty((B, CANVAS), dtype=torch.int32, device="cuda")
    steps_taken = torch.empty(B, dtype=torch.int32, device="cuda")
    with torch.cuda.stream(stream):
        dg.dg_prefill(model, prompt_ids(B, PROMPT, d.V, seed=0).to("cuda"), kc, vc, Pd)
        stream.synchronize()
        assert Pd.cpu().tolist() == [PROMPT] * B
        cfgs = {}

        def cfg_of(f):
            # a fixed-step block of f steps; the schedule stays over the cap 48
            if f not in cfgs:
                cfgs[f] = dg.sampler_cfg(CANVAS, 48, f, seed=0)
            return cfgs[f]

        block_ms = []     # device time of each block of the last timed() call

        def run_blocks(m, blocks, ev=None):
            # consecutive blocks, each block's commit forward fused into the
            # next block's first step (dg_denoise_block_deferred); the last
            # block's commit by dg_commit_pending
            for i, f in enumerate(blocks):
                dg.dg_denoise_block_deferred(m, cfg_of(f), B, kc, vc, Pd, tok, steps_taken)
                if ev is not None and i + 1 < len(blocks):
                    ev[i + 1].record(stream)
            dg.dg_commit_pending(m, B, kc, vc, Pd)
            if ev is not None:
                ev[len(blocks)].record(stream)

        def timed(blocks, warm, m=model):
            """Run the warm blocks and then the timed sequence once, untimed
            (they capture every graph the timed run replays), rewinding the
            prefix after each; then time the blocks (host clock around all of
            them; HIP events on the bench stream between blocks give each
            block's device time, the last block's with the final commit).
            blocks, warm: fixed step counts per block."""
            for seq in (warm, blocks):
                if seq:
                    run_blocks(m, seq)
                stream.synchronize()
                Pd.fill_(PROMPT)
                stream.synchronize()
            torch.cuda.synchronize()
            nb = len(blocks)
            ev = [torch.cuda.Event(enable_timing=True) for _ in range(nb + 1)]
            t0 = time.perf_counter()
            ev[0].record(stream)
            run_blocks(m, blocks, ev)
            stream.synchronize()
            torch.cuda.synchronize()
            el = time.perf_counter() - t0
            block_ms[:] = [ev[i].elapsed_time(ev[i + 1]) for i in range(nb)]
            assert Pd.cpu().tolist() == [PROMPT + CANVAS * nb] * B
            assert steps_taken.cpu().tolist() == [blocks[-1]] * B
            Pd.fill_(PROMPT)
            stream.synchronize()
            return el

        print(f"[bench] setup {time.perf_counter() - t_setup:.1f} s; timing {a.steps} steps as "
              f"blocks {plan} (warmup blocks {warm_plan}), batch {B}", file=sys.stderr,
              flush=True)
        # the model's own routing (random router: few experts after layer 0)
        elapsed_natural = None if a.no_natural else timed(plan, warm_plan)
        # the stated routing: N(0,1) + planted skew, every expert active
        model.set_router_override(planted_router_logits(d, max(CANVAS, PREFILL_CHUNK) * B))
        elapsed = timed(plan, warm_plan)
        print(f"[bench] timed {a.steps} steps: {1e3 * elapsed:.1f} ms", file=sys.stderr,
              flush=True)
        planted_block_ms = list(block_ms)
        # the prompt prefill itself (causal, all 30 layers, the planted
        # routing): re-encode the same prompt from position 0, timed, in
        # chunks of PREFILL_CHUNK tokens per row, and for comparison in
        # canvas-sized chunks (a context without the prefill limit)
        prefill_s = prefill_small_s = None
        if not a.no_prefill_timing:
            prompt = prompt_ids(B, PROMPT, d.V, seed=0).to("cuda")

            def time_prefill(m):
                dg.dg_prefill(m, prompt[:, :PREFILL_CHUNK].contiguous(), kc, vc, Pd.zero_())  # warm
                Pd.zero_()
                stream.synchronize()
                torch.cuda.synchronize()
                t0 = time.perf_counter()
                dg.dg_prefill(m, prompt, kc, vc, Pd)
                stream.synchronize()
                el = time.perf_counter() - t0
                assert Pd.cpu().tolist() == [PROMPT] * B
                return el
            prefill_s = time_prefill(model)
            m_small = dg.DGModel(d, w, B, CANVAS, dg.DG_BF16, dg.DG_FP8_E4M3,
                                 weight_layout=dg.DG_LAYOUT_TILED)
            m_small.set_router_override(planted_router_logits(d, CANVAS * B))
            prefill_small_s = time_prefill(m_small)
            m_small.close()
            # the cache again holds the prompt encoded by the main context
            prefill_s = min(prefill_s, time_prefill(model))
        # AR-mode decode on the same model: greedy single-token causal steps
        # from the prompt (one hipGraph of AR_STEPS steps; the cache slots
        # after the prompt are rewritten)
        ar_s = None
        if not a.no_ar:
            first = torch.zeros(B, dtype=torch.int32, device="cuda")
            ar_out = torch.empty((B, AR_STEPS), dtype=torch.int32, device="cuda")
            Pd.fill_(PROMPT)
            dg.dg_ar_decode(model, first, AR_STEPS, kc, vc, Pd, ar_out)   # capture + warm
            stream.synchronize()
            Pd.fill_(PROMPT)
            stream.synchronize()
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            dg.dg_ar_decode(model, first, AR_STEPS, kc, vc, Pd, ar_out)
            stream.synchronize()
            ar_s = time.perf_counter() - t0
            assert Pd.cpu().tolist() == [PROMPT + AR_STEPS] * B
            Pd.fill_(PROMPT)
            stream.synchronize()
        t48 = None
        if a.steps48:
            t48 = timed([48] * 4, [48])
        # entropy-bound commit policy (adaptive blocks, early exit) and
        # EOS-terminated generate
        eb = None
        if not a.no_eb:
            eb = entropy_bound_timing(d, w, model, B, kc, vc, Pd, stream)
        # the same step with MXFP4 experts (same draws, quantized on the
        # device), planted routing, same prompt cache
        mx = None
        if not a.no_mxfp4:
            w_mx = make_mxfp4_experts(d, w)
            # (the fused first step of a deferred block runs 2 canvases per
            # row: the context's prefill limit and the override hold them)
            model_mx = dg.DGModel(d, w_mx, B, CANVAS, dg.DG_BF16, dg.DG_MXFP4,
                                  weight_layout=dg.DG_LAYOUT_TILED,
                                  max_prefill_tokens=2 * CANVAS * B)
            model_mx.set_router_override(planted_router_logits(d, 2 * CANVAS * B))
            el_mx = timed(plan, warm_plan, model_mx)
            mx = {"steps_per_s": round(a.steps / el_mx, 3),
                  "ms_per_step": round(1e3 * el_mx / a.steps, 3),
                  "canvas_tok_per_s": round(CANVAS * B * a.steps / el_mx, 1)}
            if not a.no_roofline:
                r = moe_roofline(w_mx, d, B, mxfp4=True)
                mx["gate_up"] = {"kernel": r["kernel"], "ms": round(r["ms"], 4),
                                 "algo_bytes": r["algo_bytes"], "gbs": round(r["gbs"], 1),
                                 "hbm_frac": round(r["gbs"] / HBM_PEAK_GBS, 4)}
                mx["ffn"] = {"ms": round(r["ffn_ms"], 4), "algo_bytes": r["ffn_bytes"],
                             "gbs": round(r["ffn_gbs"], 1),
                             "hbm_frac": round(r["ffn_gbs"] / HBM_PEAK_GBS, 4)}
            model_mx.close()
            del w_mx
        if a.copy_calibration:
            copy_calibration()
        roof = None
        extra = {}
        if not a.no_roofline:
            roof = moe_roofline(w, d, B)
            extra["attention"] = attention_fraction(d, B, PROMPT)
            extra["sampler"] = sampler_fraction(d, B)
            # the canvas forward alone (30 layers + LM head, no sampler),
            # 10 forwards captured in one graph on the bench stream
            fw_tok = prompt_ids(B, CANVAS, d.V, seed=42).to("cuda")
            fw_x = torch.empty((B * CANVAS, d.D), dtype=torch.float32, device="cuda")
            fw_logits = torch.empty((B, CANVAS, d.V), dtype=torch.bfloat16, device="cuda")
            Pd.fill_(PROMPT)
            stream.synchronize()
            extra["ms_per_canvas_forward"] = round(_graph_ms(
                lambda: dg.dg_model_forward(model, fw_tok, fw_x, B, CANVAS, 0, d.NL, kc, vc, Pd,
                                            logits=fw_logits), 10), 3)
    steps_per_s = a.steps / elapsed
    out = {
        "metric": METRIC,
        "value": round(steps_per_s, 3),
        "unit": "steps/s",
        "n_gpus": 1,
        "steps": a.steps,
        "warmup": a.warmup,
        "ms_per_step": round(1e3 * elapsed / a.steps, 3),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16 activations, fp8-e4m3 expert weights (W8A16), f32 accumulation",
        "data": "synthetic",
        "config": {"workload": (f"block-autoregressive canvas decode: {d.NL}-layer MoE decoder "
                                f"(D 2816, 16/8 heads x 128, 128 experts top-8 FFN 704 fp8-e4m3, "
                                f"bf16 dense), vocab 262144, prompt {PROMPT} prefilled, "
                                f"{n_blocks} consecutive 256-token canvases of {plan} "
                                f"fixed steps, each committed; MoE routing N(0,1) + planted "
                                f"skew (13 hot experts take 40%)"),
                   "batch": B, "canvas": CANVAS, "prefix": PROMPT, "layers": d.NL,
                   "block_steps": a.block_steps, "blocks": plan, "warmup_blocks": warm_plan,
                   "parallelism": "single GPU"},
        "canvas_tok_per_s": round(steps_per_s * CANVAS * B, 1),
        # committed tokens per second over the timed blocks (host clock)
        "tok_per_s_timed_blocks": round(n_blocks * CANVAS * B / elapsed, 1),
        # each timed block's device time (HIP events on the bench stream; the
        # block's steps and its commit), over the n blocks of the run
        "block_ms": {"n": len(planted_block_ms), "steps": plan,
                     "ms": [round(x, 3) for x in planted_block_ms]},
    }
    # committed tokens per second at a fixed 12 steps per block, from the
    # device time of the timed 12-step blocks (commit included)
    ms12 = [x for f, x in zip(plan, planted_block_ms) if f == 12]
    if ms12:
        out["tok_per_s_at_12"] = round(CANVAS * B / (float(np.median(ms12)) * 1e-3), 1)
    if elapsed_natural is not None:
        out["natural_routing"] = {
            "steps_per_s": round(a.steps / elapsed_natural, 3),
            "ms_per_step": round(1e3 * elapsed_natural / a.steps, 3),
            "note": "the random-init router's own top-8 (concentrated on a few experts after "
                    "layer 0, so fewer expert bytes move)"}
    if t48 is not None:
        out["tok_per_s_at_48"] = round(4 * CANVAS * B / t48, 1)
    if eb is not None:
        out["entropy_bound"] = eb
    if mx is not None:
        mx["note"] = ("the same step with OCP MXFP4 experts (E2M1, one E8M0 scale per 32 k) "
                      "quantized on the device from the same draws, planted routing")
        out["mxfp4_experts"] = mx
    if roof is not None:
        out["ms_per_canvas_forward"] = extra["ms_per_canvas_forward"]
        out["kernel_fractions"] = {"moe_gate_up": {"frac_hbm": round(roof["gbs"] / HBM_PEAK_GBS, 4)},
                                   "attention": extra["attention"], "sampler": extra["sampler"]}
    # HBM floors (forward_floor_bytes at 8 TB/s): the canvas forward touches
    # every expert (planted routing), an AR token at most B * k of them
    canvas_floor_ms = forward_floor_bytes(d, B, CANVAS, PROMPT, d.E) / (HBM_PEAK_GBS * 1e6)
    out["step_hbm_floor"] = {"ms": round(canvas_floor_ms, 3),
                             "frac_of_step": round(canvas_floor_ms / (1e3 * elapsed / a.steps), 3),
                             "note": "weights, K/V cache and logits one canvas forward must move, "
                                     "at 8 TB/s, against the measured ms per step"}
    if ar_s is not None:
        ar_ms = 1e3 * ar_s / AR_STEPS
        ar_floor_ms = forward_floor_bytes(d, B, 1, PROMPT + AR_STEPS // 2,
                                          min(d.E, B * d.k)) / (HBM_PEAK_GBS * 1e6)
        out["ar_decode"] = {"steps": AR_STEPS, "ms_per_token": round(ar_ms, 3),
                            "tok_per_s": round(AR_STEPS * B / ar_s, 1),
                            "hbm_floor_ms_per_token": round(ar_floor_ms, 3),
                            "frac_of_floor": round(ar_floor_ms / ar_ms, 3),
                            "canvas_forward_vs_ar_forward": round(
                                (1e3 * elapsed / a.steps) / ar_ms, 2),
                            "canvas_forward_vs_ar_forward_at_floors": round(
                                canvas_floor_ms / ar_floor_ms, 2),
                            "note": "greedy single-token causal steps after the prompt, "
                                    "one hipGraph, same weights and routing override; the "
                                    "ratios compare one canvas step with one AR token, measured "
                                    "and at the two HBM floors"}
    if prefill_s is not None:
        out["prefill"] = {"tokens": PROMPT * B, "ms": round(1e3 * prefill_s, 2),
                          "tok_per_s": round(PROMPT * B / prefill_s, 1),
                          "chunk_tokens_per_row": PREFILL_CHUNK,
                          "canvas_chunks_ms": round(1e3 * prefill_small_s, 2),
                          "canvas_chunks_tok_per_s": round(PROMPT * B / prefill_small_s, 1),
                          "note": f"causal prefill of the prompt in chunks of {PREFILL_CHUNK} "
                                  f"tokens per row (and, for comparison, of {CANVAS}), planted "
                                  f"routing, eager launches, host clock around the call"}
    if roof is not None:
        out["roofline"] = {"bound": "hbm", "achieved": round(roof["gbs"], 1), "peak": HBM_PEAK_GBS,
                           "unit": "GB/s", "frac": round(roof["gbs"] / HBM_PEAK_GBS, 4),
                           "traffic": measured_traffic(), "kernel": roof["kernel"],
                           "ms_per_launch": round(roof["ms"], 4),
                           "algorithmic_bytes": int(roof["algo_bytes"]),
                           "kernel_source_hash": kernel_source_hash(),
                           "moe_ffn": {"ms_per_launch": round(roof["ffn_ms"], 4),
                                       "algorithmic_bytes": int(roof["ffn_bytes"]),
                                       "achieved_gbs": round(roof["ffn_gbs"], 1)}}
    if not a.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(d, B, PROMPT)
        out["cpu_baseline"]["value"] = float(f"{out['cpu_baseline']['value']:.4g}")
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
