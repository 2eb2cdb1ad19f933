"""MI355X (gfx950) canvas denoising for block-autoregressive, uniform-state
text diffusion: hand-written HIP kernels behind the C ABI of ``libdg.so``.

The binding lives in ``block_diffusion_decoding_tok_amd.dg``; importing this
package does not load the library.
"""

__version__ = "0.1.0"
