"""CPU oracle for the canvas denoising step of a block-autoregressive,
uniform-state text-diffusion decoder (DiffusionGemma-style).

THIS PACKAGE IS TEST INFRASTRUCTURE.  Only ``tests/``, ``__graft_entry__.smoke()``
and the ``cpu_baseline`` leg of ``bench.py`` may import or call it.  The GPU
product path (``block_diffusion_decoding_tok_amd``) never imports it, and this
package imports nothing from the product path: the two share no kernels,
helpers, tables or constants.  Only the seeded input generators
(``block_diffusion_decoding_tok_amd.inputs``) feed both sides.

Everything here is plain NumPy in float64 (integers in uint64/int64), written
for a reader to check by eye against the pages.  No blocking, fusion or
reordering beyond what the definitions state.

Pages cited (by title; section names are the pages' own headings):

  [TR]    "[AI] DiffusionGemma: 256토큰 블록을 병렬 정제하는 확산 LLM"
          (a summary of the DiffusionGemma technical report)
  [GUIDE] "diffusion-gemma tutorial / developer guide" (aisparkup wiki):
          sections "256토큰 Canvas 병렬 생성", "Uniform State Diffusion",
          "Block Autoregressive Diffusion", "vLLM으로 서빙하기"
  [GN]    "DiffusionGemma: 4배 빠른 텍스트 생성" (GeekNews summary of the
          Google blog): sections "핵심 트레이드오프", "텍스트 확산의 작동 방식"
  [WE0]   the test.we0.ai article on DiffusionGemma: sections
          "DiffusionGemma가 다르게 하는 점", "양방향 어텐션과 자기 수정의 역할",
          "26B MoE 설계가 의미하는 것"
  [JPH]   "구글, 순차 처리 탈피한 확산 기반 AI 모델 디퓨전젬마 공개":
          section "좌→우 순차 처리와의 대비"

Where the pages leave a step open, the module docstrings state the reading
taken (R1..R32 in the design notes).

Parity pins: every function has at least one pin in ``tests/test_oracle_*.py``
that checks it against something other than itself (closed forms, brute
force, an independent library routine, invariants).  Functions without such a
pin say "parity unpinned" in their docstring.  Current status:

  philox4x32_10   pinned: rocRAND's independent Philox4x32-10 (host build),
                  statistical uniformity.
  sampler_step    pinned: closed-form two-level softmax values, uniform-logit
                  entropy, temperature schedule closed form, Gumbel-max
                  frequencies vs softmax (chi-square), planted commit/re-noise/
                  stop scenarios; the entropy-bound selection against a
                  brute-force search over all subsets, planted entropy-bound
                  steps (two-level closed form), bound 0 and unbounded cases.
  attention       pinned: torch scaled_dot_product_attention (fp64, CPU),
                  prompt-row independence, permutation equivariance, RoPE
                  shift invariance, equal-score mean.
  moe_route       pinned: brute-force stable sort, gate sums, k = E dense mix.
  moe_ffn         pinned: dense masked every-expert sum, E = k = 1 textbook FFN,
                  token permutation equivariance, torch float8_e4m3fn decode.
  model forward   pinned: an independently composed float64 torch layer
                  (rms_norm, SDPA with repeated KV heads, complex-rotation
                  RoPE, topk, erf GELU) at 1e-12; zero-sublayer closed forms
                  (identity; x + o Wo^T).  The tiny-loop scenario is pinned by
                  its own invariants (re-noise every step at random weights;
                  planted commits; adaptive stop).
  mxfp4           pinned: torch's e4m3fn and e8m0 decoders on the same bit
                  fields, worked round-to-nearest-even and saturation cases,
                  brute-force nearest value, exact round trips, error bound.
  generate        pinned: no EOS reproduces consecutive single blocks; an EOS
                  first produced in a row's second block stops that row
                  there (prefix frozen) and leaves the other row unchanged.
  ar_decode       pinned: the incremental (KV-cache) greedy tokens equal the
                  argmax of one causal pass over the whole sequence from an
                  empty cache; equal logits (zero LM head) give id 0.
"""

from .philox import (philox4x32_10, uniform24, gumbel_from_word,
                     uniform_id, STREAM_GUMBEL, STREAM_RENOISE, STREAM_CANVAS)
from .sampler import (SamplerCfg, temperature, position_stats, sampler_step,
                      init_canvas, entropy_bound_select)
from .attention import rope, attention
from .moe import (fp8_e4m3fn_decode, moe_route, moe_ffn, moe_ffn_dense_masked,
                  expert_gate_up, gelu_erf)
from .mxfp4 import e2m1_decode, e8m0_decode, quantize_mxfp4, dequantize_mxfp4
from .model import (rmsnorm, TinyModel, layer_forward, model_forward,
                    prefill, denoise_block, ar_decode, generate)

__all__ = [
    "philox4x32_10", "uniform24", "gumbel_from_word", "uniform_id",
    "STREAM_GUMBEL", "STREAM_RENOISE", "STREAM_CANVAS",
    "SamplerCfg", "temperature", "position_stats", "sampler_step",
    "init_canvas", "rope", "attention", "fp8_e4m3fn_decode", "moe_route",
    "moe_ffn", "moe_ffn_dense_masked", "expert_gate_up", "gelu_erf", "rmsnorm", "TinyModel",
    "layer_forward", "model_forward", "prefill", "denoise_block", "ar_decode",
    "e2m1_decode", "e8m0_decode", "quantize_mxfp4", "dequantize_mxfp4",
    "entropy_bound_select", "generate",
]
