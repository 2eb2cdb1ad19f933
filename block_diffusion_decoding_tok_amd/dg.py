"""ctypes binding of libdg.so: one Python function per C entry point, same
names.  Argument marshalling only -- torch supplies device memory and the
current stream; every computation runs in the library's HIP kernels.

The library is loaded on first use; if it is missing (not built) or no GPU is
visible, calls raise instead of falling back to anything else.
"""

import ctypes as C
import os

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libdg.so")

DG_F32, DG_BF16, DG_FP8_E4M3, DG_MXFP4 = 0, 1, 2, 3
DG_MASK_CANVAS, DG_MASK_CAUSAL = 0, 1
DG_LAYOUT_ROWMAJOR, DG_LAYOUT_TILED = 0, 1
STATUS_NONFINITE_LOGITS = 1

_STATUS = {0: "DG_OK", -1: "DG_ERR_INVALID_ARG", -2: "DG_ERR_SHAPE",
           -3: "DG_ERR_UNSUPPORTED", -4: "DG_ERR_WORKSPACE", -5: "DG_ERR_HIP",
           -6: "DG_ERR_NONFINITE"}


class DGError(RuntimeError):
    def __init__(self, code, msg):
        super().__init__(f"{_STATUS.get(code, code)}: {msg}")
        self.code = code


class dg_sampler_cfg(C.Structure):
    _fields_ = [("canvas_len", C.c_int32), ("max_steps", C.c_int32),
                ("fixed_steps", C.c_int32), ("temp_start", C.c_float),
                ("temp_end", C.c_float), ("stop_entropy", C.c_float),
                ("commit_prob", C.c_float), ("renoise_prob", C.c_float),
                ("seed", C.c_uint64), ("commit_policy", C.c_int32),
                ("entropy_bound", C.c_float)]


DG_COMMIT_MAXPROB, DG_COMMIT_ENTROPY_BOUND = 0, 1


def sampler_cfg(canvas_len=256, max_steps=48, fixed_steps=0, temp_start=0.8,
                temp_end=0.4, stop_entropy=0.005, commit_prob=0.9,
                renoise_prob=0.1, seed=0, commit_policy=DG_COMMIT_MAXPROB,
                entropy_bound=0.1):
    return dg_sampler_cfg(canvas_len, max_steps, fixed_steps, temp_start,
                          temp_end, stop_entropy, commit_prob, renoise_prob,
                          seed, commit_policy, entropy_bound)


class dg_model_dims(C.Structure):
    _fields_ = [("n_layers", C.c_int32), ("d_model", C.c_int32),
                ("n_heads", C.c_int32), ("n_kv_heads", C.c_int32),
                ("head_dim", C.c_int32), ("n_experts", C.c_int32),
                ("top_k", C.c_int32), ("d_ff", C.c_int32), ("vocab", C.c_int32),
                ("rope_theta", C.c_float), ("act_dtype", C.c_int32),
                ("expert_dtype", C.c_int32), ("weight_layout", C.c_int32)]


class dg_model_weights(C.Structure):
    _fields_ = [("emb", C.c_void_p), ("lm_head", C.c_void_p),
                ("wqkv", C.POINTER(C.c_void_p)), ("wo", C.POINTER(C.c_void_p)),
                ("wr", C.POINTER(C.c_void_p)), ("w_gate_up", C.POINTER(C.c_void_p)),
                ("w_down", C.POINTER(C.c_void_p)), ("s_gate_up", C.POINTER(C.c_void_p)),
                ("s_down", C.POINTER(C.c_void_p))]


_lib = None

# name -> (restype, argtypes)
_VP, _SZ, _I, _I64, _U64, _F = C.c_void_p, C.c_size_t, C.c_int, C.c_int64, C.c_uint64, C.c_float
_SIGS = {
    "dg_version": (C.c_int, []),
    "dg_last_error": (C.c_char_p, []),
    "dg_sampler_workspace_size": (_SZ, [_I, _I, _I]),
    "dg_sampler_step": (_I, [_VP, _I, _I, _I, _I, _I, C.POINTER(dg_sampler_cfg), _VP, _VP,
                             _VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _SZ, _VP]),
    "dg_sampler_step_noalloc": (_I, [_VP, _I, _I, _I, _I, _I, C.POINTER(dg_sampler_cfg), _VP,
                                     _VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP]),
    "dg_init_canvas": (_I, [_VP, _I, _I, _I, _U64, _VP, _VP, _VP, _VP]),
    "dg_attention_workspace_size": (_SZ, [_I, _I, _I, _I, _I, _I, _I]),
    "dg_canvas_attention": (_I, [_VP, _VP, _VP, _VP, _VP, _VP, _I, _I, _I, _I, _I, _I, _I,
                                 _F, _I, _VP, _VP, _SZ, _VP]),
    "dg_commit_block": (_I, [_VP, _VP, _VP, _VP, _VP, _I, _I, _I, _I, _I, _F, _I, _VP]),
    "dg_moe_route_workspace_size": (_SZ, [_I, _I, _I]),
    "dg_moe_route": (_I, [_VP, _I, _I, _I, _VP, _VP, _VP, _VP, _VP, _SZ, _VP]),
    "dg_moe_ffn_workspace_size": (_SZ, [_I, _I, _I, _I, _I, _I]),
    "dg_moe_ffn": (_I, [_VP, _I, _VP, _VP, _I, _I, _VP, _VP, _VP, _VP, _VP, _VP, _I, _I, _I,
                        _I, _I, _VP, _VP, _SZ, _VP]),
    "dg_moe_gate_up": (_I, [_VP, _I, _VP, _I, _I, _VP, _VP, _VP, _I, _I, _I, _I, _I, _VP, _VP]),
    "dg_moe_down": (_I, [_VP, _I, _VP, _I, _I, _VP, _VP, _VP, _VP, _I, _I, _I, _I, _I, _VP,
                         _VP]),
    "dg_moe_combine": (_I, [_VP, _I, _I, _I, _I, _VP, _VP]),
    "dg_linear": (_I, [_VP, _VP, _VP, _I, _I, _I, _I, _I, _I, _I, _VP]),
    "dg_ar_decode": (_I, [_VP, _I, _I, _VP, C.POINTER(_VP), C.POINTER(_VP), _I, _VP, _VP, _VP]),
    "dg_ctx_workspace_size": (_SZ, [C.POINTER(dg_model_dims), _I, _I, _I]),
    "dg_ctx_create": (_I, [C.POINTER(_VP), C.POINTER(dg_model_dims),
                           C.POINTER(dg_model_weights), _I, _I, _I, _VP, _SZ]),
    "dg_ctx_destroy": (_I, [_VP]),
    "dg_ctx_set_graphs": (_I, [_VP, _I]),
    "dg_ctx_check_status": (_I, [_VP, _VP]),
    "dg_ctx_set_router_override": (_I, [_VP, C.POINTER(_VP), _I]),
    "dg_model_forward": (_I, [_VP, _VP, _VP, _I, _I, _I, _I, C.POINTER(_VP), C.POINTER(_VP),
                              _I, _VP, _I, _VP, _VP]),
    "dg_prefill": (_I, [_VP, _VP, _I, _I, C.POINTER(_VP), C.POINTER(_VP), _I, _VP, _VP]),
    "dg_denoise_block": (_I, [_VP, C.POINTER(dg_sampler_cfg), _I, C.POINTER(_VP),
                              C.POINTER(_VP), _I, _VP, _VP, _VP, _VP]),
    "dg_generate": (_I, [_VP, C.POINTER(dg_sampler_cfg), _I, C.POINTER(_VP), C.POINTER(_VP),
                         _I, _VP, C.c_int32, _I, _VP, _VP, _VP, _VP]),
    "dg_denoise_block_deferred": (_I, [_VP, C.POINTER(dg_sampler_cfg), _I, C.POINTER(_VP),
                                       C.POINTER(_VP), _I, _VP, _VP, _VP, _VP]),
    "dg_commit_pending": (_I, [_VP, _I, C.POINTER(_VP), C.POINTER(_VP), _I, _VP, _VP]),
    "dg_fill_normal": (_I, [_VP, _I, _SZ, _F, _U64, C.c_uint32, _VP]),
    "dg_quantize_fp8_rows": (_I, [_VP, _VP, _VP, _I64, _I, _VP]),
    "dg_pack_weights": (_I, [_VP, _VP, _I64, _I, _I, _I, _VP]),
    "dg_quantize_mxfp4": (_I, [_VP, _VP, _VP, _I64, _I, _VP]),
    "dg_pack_mxfp4": (_I, [_VP, _VP, _VP, _I64, _I, _I, _VP]),
    "dg_philox": (_I, [_VP, _I64, _U64, _VP, _VP]),
    "dg_gumbel": (_I, [_VP, _I64, _VP, _VP]),
}
EXPORTED = tuple(_SIGS)


def lib():
    """Load libdg.so (once).  Raises if it is not built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: run "
                               "`python -m block_diffusion_decoding_tok_amd.build`")
        l = C.CDLL(LIB_PATH, mode=C.RTLD_GLOBAL)
        for name, (res, args) in _SIGS.items():
            fn = getattr(l, name, None)
            if fn is None:          # reported by missing_symbols()
                continue
            fn.restype = res
            fn.argtypes = args
        _lib = l
    return _lib


def missing_symbols():
    """Entry points of the binding that the loaded library does not export."""
    l = lib()
    return [n for n in _SIGS if getattr(l, n, None) is None]


def _check(code):
    if code != 0:
        raise DGError(code, lib().dg_last_error().decode())


def _dev(t, name, dtypes=None):
    if t is None:
        return None
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name}: expected a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name}: must be a device tensor (got {t.device})")
    if not t.is_contiguous():
        raise ValueError(f"{name}: must be contiguous")
    if dtypes is not None and t.dtype not in dtypes:
        raise ValueError(f"{name}: dtype {t.dtype} not in {dtypes}")
    return t.data_ptr()


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream


def _dtype_code(t):
    if t.dtype == torch.bfloat16:
        return DG_BF16
    if t.dtype == torch.float32:
        return DG_F32
    if t.dtype in (torch.uint8, torch.float8_e4m3fn):
        return DG_FP8_E4M3
    raise ValueError(f"unsupported dtype {t.dtype}")


def _workspace(nbytes, device):
    return torch.empty(max(int(nbytes), 1), dtype=torch.uint8, device=device)


def _ptr_array(tensors):
    arr = (C.c_void_p * len(tensors))()
    for i, t in enumerate(tensors):
        arr[i] = None if t is None else t.data_ptr()
    return arr


# ------------------------------------------------------------------ sampler

def dg_sampler_step(logits, step, cfg, prefix_len, tokens, committed, renoised,
                    maxprob, entropy, mean_entropy, done, status=None, ws=None,
                    stream=None):
    B, L, V = logits.shape
    if ws is None:
        ws = _workspace(lib().dg_sampler_workspace_size(B, L, V), logits.device)
    _check(lib().dg_sampler_step(
        _dev(logits, "logits", (torch.bfloat16, torch.float32)), _dtype_code(logits),
        B, L, V, int(step), C.byref(cfg), _dev(prefix_len, "prefix_len", (torch.int32,)),
        _dev(tokens, "tokens", (torch.int32,)), _dev(committed, "committed", (torch.uint8,)),
        _dev(renoised, "renoised", (torch.uint8,)), _dev(maxprob, "maxprob", (torch.float32,)),
        _dev(entropy, "entropy", (torch.float32,)),
        _dev(mean_entropy, "mean_entropy", (torch.float32,)),
        _dev(done, "done", (torch.int32,)), _dev(status, "status", (torch.int32,)),
        ws.data_ptr(), ws.numel(), _stream(stream)))


def dg_sampler_step_noalloc(logits, step, cfg, prefix_len, tokens, committed, renoised,
                            maxprob, entropy, mean_entropy, done, status=None, stream=None):
    """dg_sampler_step on the library's own scratch (no workspace argument)."""
    B, L, V = logits.shape
    _check(lib().dg_sampler_step_noalloc(
        _dev(logits, "logits", (torch.bfloat16, torch.float32)), _dtype_code(logits),
        B, L, V, int(step), C.byref(cfg), _dev(prefix_len, "prefix_len", (torch.int32,)),
        _dev(tokens, "tokens", (torch.int32,)), _dev(committed, "committed", (torch.uint8,)),
        _dev(renoised, "renoised", (torch.uint8,)), _dev(maxprob, "maxprob", (torch.float32,)),
        _dev(entropy, "entropy", (torch.float32,)),
        _dev(mean_entropy, "mean_entropy", (torch.float32,)),
        _dev(done, "done", (torch.int32,)), _dev(status, "status", (torch.int32,)),
        _stream(stream)))


def dg_init_canvas(prefix_len, L, V, seed, tokens, committed, done, stream=None):
    B = prefix_len.numel()
    _check(lib().dg_init_canvas(_dev(prefix_len, "prefix_len", (torch.int32,)), B, L, V,
                                int(seed), _dev(tokens, "tokens", (torch.int32,)),
                                _dev(committed, "committed", (torch.uint8,)),
                                _dev(done, "done", (torch.int32,)), _stream(stream)))


def dg_philox(counters, seed, out=None, stream=None):
    """counters: uint32-valued int32/int64 tensor [n, 4] on the device."""
    n = counters.shape[0]
    if out is None:
        out = torch.empty((n, 4), dtype=torch.int32, device=counters.device)
    _check(lib().dg_philox(_dev(counters, "counters", (torch.int32,)), n, int(seed),
                           _dev(out, "out", (torch.int32,)), _stream(stream)))
    return out


def dg_gumbel(words, out=None, stream=None):
    n = words.numel()
    if out is None:
        out = torch.empty(n, dtype=torch.float32, device=words.device)
    _check(lib().dg_gumbel(_dev(words, "words", (torch.int32,)), n,
                           _dev(out, "out", (torch.float32,)), _stream(stream)))
    return out


# ---------------------------------------------------------------- attention

def dg_canvas_attention(q, k_new, v_new, k_cache, v_cache, prefix_len, mask_mode=0,
                        rope_theta=10000.0, out=None, ws=None, stream=None):
    B, Lq, Hq, dh = q.shape
    Hkv = k_new.shape[2]
    Tmax = k_cache.shape[2]
    dt = _dtype_code(q)
    if out is None:
        out = torch.empty_like(q)
    if ws is None:
        ws = _workspace(lib().dg_attention_workspace_size(B, Lq, Hq, Hkv, dh, Tmax, dt),
                        q.device)
    _check(lib().dg_canvas_attention(
        _dev(q, "q"), _dev(k_new, "k_new"), _dev(v_new, "v_new"), _dev(k_cache, "k_cache"),
        _dev(v_cache, "v_cache"), _dev(prefix_len, "prefix_len", (torch.int32,)),
        B, Lq, Hq, Hkv, dh, Tmax, int(mask_mode), float(rope_theta), dt, _dev(out, "out"),
        ws.data_ptr(), ws.numel(), _stream(stream)))
    return out


def dg_commit_block(k_new, v_new, k_cache, v_cache, prefix_len, rope_theta=10000.0,
                    stream=None):
    B, L, Hkv, dh = k_new.shape
    _check(lib().dg_commit_block(
        _dev(k_new, "k_new"), _dev(v_new, "v_new"), _dev(k_cache, "k_cache"),
        _dev(v_cache, "v_cache"), _dev(prefix_len, "prefix_len", (torch.int32,)),
        B, L, Hkv, dh, k_cache.shape[2], float(rope_theta), _dtype_code(k_new),
        _stream(stream)))


# ---------------------------------------------------------------------- MoE

def dg_moe_route(router_logits, k, topk_ids=None, gates=None, expert_offsets=None,
                 sorted_rows=None, ws=None, stream=None):
    T, E = router_logits.shape
    dev = router_logits.device
    topk_ids = topk_ids if topk_ids is not None else torch.empty((T, k), dtype=torch.int32, device=dev)
    gates = gates if gates is not None else torch.empty((T, k), dtype=torch.float32, device=dev)
    expert_offsets = (expert_offsets if expert_offsets is not None
                      else torch.empty(E + 1, dtype=torch.int32, device=dev))
    sorted_rows = (sorted_rows if sorted_rows is not None
                   else torch.empty(T * k, dtype=torch.int32, device=dev))
    if ws is None:
        ws = _workspace(lib().dg_moe_route_workspace_size(T, E, k), dev)
    _check(lib().dg_moe_route(
        _dev(router_logits, "router_logits", (torch.float32,)), T, E, k,
        _dev(topk_ids, "topk_ids", (torch.int32,)), _dev(gates, "gates", (torch.float32,)),
        _dev(expert_offsets, "expert_offsets", (torch.int32,)),
        _dev(sorted_rows, "sorted_rows", (torch.int32,)), ws.data_ptr(), ws.numel(),
        _stream(stream)))
    return topk_ids, gates, expert_offsets, sorted_rows


def dg_moe_ffn(x, w_gate_up, w_down, s_gate_up, s_down, topk_ids, gates, expert_offsets,
               sorted_rows, y, ws=None, stream=None, w_layout=DG_LAYOUT_ROWMAJOR, E=None, I=None,
               w_dtype=None):
    """w_gate_up / w_down: [E, 2I, D] / [E, D, I] row-major, or the same bytes
    in DG_LAYOUT_TILED (then pass E and I, or keep the logical shape).  MXFP4
    weights (from dg_pack_mxfp4) need w_dtype=DG_MXFP4, the tiled layout, E
    and I."""
    T, D = x.shape
    if E is None:
        E, I2 = w_gate_up.shape[0], w_gate_up.shape[1]
        I = I2 // 2
    k = topk_ids.shape[1]
    xd = _dtype_code(x)
    wd = _dtype_code(w_gate_up) if w_dtype is None else int(w_dtype)
    if ws is None:
        ws = _workspace(lib().dg_moe_ffn_workspace_size(T, D, I, E, k, xd), x.device)
    _check(lib().dg_moe_ffn(
        _dev(x, "x"), xd, _dev(w_gate_up, "w_gate_up"), _dev(w_down, "w_down"), wd, int(w_layout),
        _dev(s_gate_up, "s_gate_up", (torch.float32,)), _dev(s_down, "s_down", (torch.float32,)),
        _dev(topk_ids, "topk_ids", (torch.int32,)), _dev(gates, "gates", (torch.float32,)),
        _dev(expert_offsets, "expert_offsets", (torch.int32,)),
        _dev(sorted_rows, "sorted_rows", (torch.int32,)), T, D, I, E, k,
        _dev(y, "y", (torch.float32,)), ws.data_ptr(), ws.numel(), _stream(stream)))
    return y


def _expert_dims(w, E, I, gate_up):
    if E is None:
        E = w.shape[0]
        I = w.shape[1] // 2 if gate_up else w.shape[2]
    return E, I


def dg_moe_gate_up(x, w_gate_up, s_gate_up, expert_offsets, sorted_rows, k, h=None, stream=None,
                   w_layout=DG_LAYOUT_ROWMAJOR, E=None, I=None, w_dtype=None):
    """h [T * k, I] (x's dtype), one row per sorted position."""
    T, D = x.shape
    E, I = _expert_dims(w_gate_up, E, I, True)
    if h is None:
        h = torch.empty((T * k, I), dtype=x.dtype, device=x.device)
    _check(lib().dg_moe_gate_up(
        _dev(x, "x"), _dtype_code(x), _dev(w_gate_up, "w_gate_up"),
        _dtype_code(w_gate_up) if w_dtype is None else int(w_dtype),
        int(w_layout), _dev(s_gate_up, "s_gate_up", (torch.float32,)),
        _dev(expert_offsets, "expert_offsets", (torch.int32,)),
        _dev(sorted_rows, "sorted_rows", (torch.int32,)), T, D, I, E, k,
        _dev(h, "h", (x.dtype,)), _stream(stream)))
    return h


def dg_moe_down(h, w_down, s_down, gates, expert_offsets, sorted_rows, T, D, y_slot=None,
                stream=None, w_layout=DG_LAYOUT_ROWMAJOR, E=None, I=None, w_dtype=None):
    """y_slot [T * k, D] (h's dtype), one gate-weighted row per slot."""
    E, I = _expert_dims(w_down, E, I, False)
    k = h.shape[0] // T
    if y_slot is None:
        y_slot = torch.empty((T * k, D), dtype=h.dtype, device=h.device)
    _check(lib().dg_moe_down(
        _dev(h, "h"), _dtype_code(h), _dev(w_down, "w_down"),
        _dtype_code(w_down) if w_dtype is None else int(w_dtype), int(w_layout),
        _dev(s_down, "s_down", (torch.float32,)), _dev(gates, "gates", (torch.float32,)),
        _dev(expert_offsets, "expert_offsets", (torch.int32,)),
        _dev(sorted_rows, "sorted_rows", (torch.int32,)), T, D, I, E, k,
        _dev(y_slot, "y_slot", (h.dtype,)), _stream(stream)))
    return y_slot


def dg_moe_combine(y_slot, k, y, stream=None):
    """y [T, D] f32 += sum over each token's k slot rows."""
    T, D = y.shape
    _check(lib().dg_moe_combine(_dev(y_slot, "y_slot"), _dtype_code(y_slot), T, D, k,
                                _dev(y, "y", (torch.float32,)), _stream(stream)))
    return y


def dg_linear(x, w, out=None, out_dtype=None, accumulate=False, stream=None,
              w_layout=DG_LAYOUT_ROWMAJOR, N=None):
    """out [M, N] (=|+=) x [M, K] @ w[N, K]^T; w may be tile-packed (pass N
    or keep w's logical shape)."""
    M, K = x.shape
    N = w.shape[0] if N is None else N
    if out is None:
        od = out_dtype if out_dtype is not None else x.dtype
        out = torch.zeros((M, N), dtype=od, device=x.device)
    _check(lib().dg_linear(_dev(x, "x"), _dev(w, "w"), _dev(out, "out"), M, N, K,
                           _dtype_code(x), int(w_layout), _dtype_code(out), int(bool(accumulate)),
                           _stream(stream)))
    return out


# ---------------------------------------------------------- whole decoder

class DGModel:
    """A dg_ctx over device weights (a dict of torch tensors with the keys of
    ``inputs.model_weights``).  Holds references so the weights and the
    workspace outlive the context."""

    def __init__(self, dims, weights, max_batch, max_tokens, act_dtype, expert_dtype,
                 rope_theta=10000.0, device="cuda", weight_layout=DG_LAYOUT_ROWMAJOR,
                 max_prefill_tokens=0):
        self.dims = dims
        self.weights = weights
        nl = dims.NL
        self.cdims = dg_model_dims(nl, dims.D, dims.Hq, dims.Hkv, dims.dh, dims.E, dims.k,
                                   dims.I, dims.V, rope_theta, act_dtype, expert_dtype,
                                   weight_layout)
        self._override = None
        self._arrays = {n: _ptr_array([weights.get(f"{n}.{l}") for l in range(nl)])
                        for n in ("wqkv", "wo", "wr", "wgu", "wd", "sgu", "sd")}
        a = self._arrays
        self.cw = dg_model_weights(weights["emb"].data_ptr(), weights["lm"].data_ptr(),
                                   a["wqkv"], a["wo"], a["wr"], a["wgu"], a["wd"], a["sgu"],
                                   a["sd"])
        nbytes = lib().dg_ctx_workspace_size(C.byref(self.cdims), max_batch, max_tokens,
                                             max_prefill_tokens)
        self.ws = _workspace(nbytes, device)
        h = C.c_void_p()
        _check(lib().dg_ctx_create(C.byref(h), C.byref(self.cdims), C.byref(self.cw),
                                   max_batch, max_tokens, max_prefill_tokens,
                                   self.ws.data_ptr(), self.ws.numel()))
        self.ctx = h

    def close(self):
        if self.ctx:
            lib().dg_ctx_destroy(self.ctx)
            self.ctx = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def set_graphs(self, on):
        _check(lib().dg_ctx_set_graphs(self.ctx, int(bool(on))))

    def check_status(self, stream=None):
        """dg_ctx_check_status: wait for the stream; raise DGError
        (DG_ERR_NONFINITE) if a finished decoder call met NaN/Inf logits."""
        _check(lib().dg_ctx_check_status(self.ctx, _stream(stream)))

    def set_router_override(self, logits_per_layer):
        """Route with the given per-layer f32 [n_tokens, E] logits (None: the
        model's own routing)."""
        if logits_per_layer is None:
            self._override = None
            _check(lib().dg_ctx_set_router_override(self.ctx, None, 0))
            return
        self._override = (list(logits_per_layer), _ptr_array(logits_per_layer))
        _check(lib().dg_ctx_set_router_override(self.ctx, self._override[1],
                                                logits_per_layer[0].shape[0]))


def dg_model_forward(model, tokens, x, B, n, layer_begin, layer_end, k_caches, v_caches,
                     prefix_len, mask_mode=0, logits=None, stream=None):
    kc, vc = _ptr_array(k_caches), _ptr_array(v_caches)
    _check(lib().dg_model_forward(
        model.ctx, None if tokens is None else _dev(tokens, "tokens", (torch.int32,)),
        _dev(x, "x", (torch.float32,)), B, n, layer_begin, layer_end, kc, vc,
        k_caches[0].shape[2], _dev(prefix_len, "prefix_len", (torch.int32,)), int(mask_mode),
        None if logits is None else _dev(logits, "logits"), _stream(stream)))


def dg_ar_decode(model, tokens_in, n_steps, k_caches, v_caches, prefix_len, tokens_out=None,
                 stream=None):
    """Greedy AR decoding: tokens_out [B, n_steps] (prefix_len advances by n_steps)."""
    B = tokens_in.shape[0]
    if tokens_out is None:
        tokens_out = torch.empty((B, n_steps), dtype=torch.int32, device=tokens_in.device)
    kc, vc = _ptr_array(k_caches), _ptr_array(v_caches)
    _check(lib().dg_ar_decode(
        model.ctx, B, n_steps, _dev(tokens_in, "tokens_in", (torch.int32,)), kc, vc,
        k_caches[0].shape[2], _dev(prefix_len, "prefix_len", (torch.int32,)),
        _dev(tokens_out, "tokens_out", (torch.int32,)), _stream(stream)))
    return tokens_out


def dg_prefill(model, prompt, k_caches, v_caches, prefix_len, stream=None):
    B, n = prompt.shape
    kc, vc = _ptr_array(k_caches), _ptr_array(v_caches)
    _check(lib().dg_prefill(model.ctx, _dev(prompt, "prompt", (torch.int32,)), B, n, kc, vc,
                            k_caches[0].shape[2],
                            _dev(prefix_len, "prefix_len", (torch.int32,)), _stream(stream)))


def dg_denoise_block(model, cfg, B, k_caches, v_caches, prefix_len, tokens_out, steps_taken,
                     stream=None):
    kc, vc = _ptr_array(k_caches), _ptr_array(v_caches)
    _check(lib().dg_denoise_block(
        model.ctx, C.byref(cfg), B, kc, vc, k_caches[0].shape[2],
        _dev(prefix_len, "prefix_len", (torch.int32,)),
        _dev(tokens_out, "tokens_out", (torch.int32,)),
        _dev(steps_taken, "steps_taken", (torch.int32,)), _stream(stream)))


def dg_denoise_block_deferred(model, cfg, B, k_caches, v_caches, prefix_len, tokens_out,
                              steps_taken, stream=None):
    kc, vc = _ptr_array(k_caches), _ptr_array(v_caches)
    _check(lib().dg_denoise_block_deferred(
        model.ctx, C.byref(cfg), B, kc, vc, k_caches[0].shape[2],
        _dev(prefix_len, "prefix_len", (torch.int32,)),
        _dev(tokens_out, "tokens_out", (torch.int32,)),
        _dev(steps_taken, "steps_taken", (torch.int32,)), _stream(stream)))


def dg_commit_pending(model, B, k_caches, v_caches, prefix_len, stream=None):
    kc, vc = _ptr_array(k_caches), _ptr_array(v_caches)
    _check(lib().dg_commit_pending(
        model.ctx, B, kc, vc, k_caches[0].shape[2],
        _dev(prefix_len, "prefix_len", (torch.int32,)), _stream(stream)))


def dg_generate(model, cfg, B, k_caches, v_caches, prefix_len, eos_id, max_blocks,
                tokens_out=None, n_blocks=None, steps_taken=None, stream=None):
    """EOS-terminated multi-block decode; returns (tokens_out [B, max_blocks,
    L], n_blocks [B], steps_taken [B, max_blocks])."""
    dev = prefix_len.device
    L = cfg.canvas_len
    if tokens_out is None:
        tokens_out = torch.empty((B, max_blocks, L), dtype=torch.int32, device=dev)
    if n_blocks is None:
        n_blocks = torch.empty(B, dtype=torch.int32, device=dev)
    if steps_taken is None:
        steps_taken = torch.empty((B, max_blocks), dtype=torch.int32, device=dev)
    kc, vc = _ptr_array(k_caches), _ptr_array(v_caches)
    _check(lib().dg_generate(
        model.ctx, C.byref(cfg), B, kc, vc, k_caches[0].shape[2],
        _dev(prefix_len, "prefix_len", (torch.int32,)), int(eos_id), int(max_blocks),
        _dev(tokens_out, "tokens_out", (torch.int32,)),
        _dev(n_blocks, "n_blocks", (torch.int32,)),
        _dev(steps_taken, "steps_taken", (torch.int32,)), _stream(stream)))
    return tokens_out, n_blocks, steps_taken


# ------------------------------------------------------------ utilities

def dg_fill_normal(dst, std, seed, stream_id, stream=None):
    _check(lib().dg_fill_normal(_dev(dst, "dst", (torch.float32, torch.bfloat16)),
                                _dtype_code(dst), dst.numel(), float(std), int(seed),
                                int(stream_id), _stream(stream)))


def dg_pack_weights(src, dst=None, stream=None):
    """Row-major [.., N, K] (bf16 or 1-byte) -> DG_LAYOUT_TILED, same shape."""
    if dst is None:
        dst = torch.empty_like(src)
    N, K = src.shape[-2], src.shape[-1]
    groups = src.numel() // (N * K)
    code = DG_BF16 if src.dtype == torch.bfloat16 else DG_FP8_E4M3
    _check(lib().dg_pack_weights(_dev(src, "src", (torch.bfloat16, torch.uint8)),
                                 _dev(dst, "dst", (torch.bfloat16, torch.uint8)), groups, N, K,
                                 code, _stream(stream)))
    return dst


def dg_quantize_mxfp4(src, codes=None, scales=None, stream=None):
    """OCP MXFP4 of f32 src [..., K] (K % 32 == 0): codes [..., K / 2] and
    E8M0 scales [..., K / 32], both uint8, row-major."""
    K = src.shape[-1]
    rows = src.numel() // K
    if codes is None:
        codes = torch.empty(src.shape[:-1] + (K // 2,), dtype=torch.uint8, device=src.device)
    if scales is None:
        scales = torch.empty(src.shape[:-1] + (K // 32,), dtype=torch.uint8, device=src.device)
    _check(lib().dg_quantize_mxfp4(_dev(src, "src", (torch.float32,)),
                                   _dev(codes, "codes", (torch.uint8,)),
                                   _dev(scales, "scales", (torch.uint8,)), rows, K,
                                   _stream(stream)))
    return codes, scales


def mxfp4_tiled_bytes(groups, N, K):
    return groups * N * K * 17 // 32


def dg_pack_mxfp4(codes, scales, dst=None, stream=None):
    """Row-major MXFP4 codes [.., N, K / 2] + scales [.., N, K / 32] -> the
    tiled MXFP4 layout (flat uint8, groups * N * K * 17 / 32 bytes)."""
    N, K = codes.shape[-2], 2 * codes.shape[-1]
    groups = codes.numel() // (N * K // 2)
    if tuple(scales.shape[:-1]) != tuple(codes.shape[:-1]) or scales.shape[-1] * 32 != K:
        raise ValueError("dg_pack_mxfp4: codes and scales shapes disagree")
    if dst is None:
        dst = torch.empty(mxfp4_tiled_bytes(groups, N, K), dtype=torch.uint8, device=codes.device)
    _check(lib().dg_pack_mxfp4(_dev(codes, "codes", (torch.uint8,)),
                               _dev(scales, "scales", (torch.uint8,)),
                               _dev(dst, "dst", (torch.uint8,)), groups, N, K, _stream(stream)))
    return dst


def dg_quantize_fp8_rows(src, q, scale, stream=None):
    rows, cols = src.shape[:-1].numel(), src.shape[-1]
    _check(lib().dg_quantize_fp8_rows(_dev(src, "src", (torch.float32,)),
                                      _dev(q, "q", (torch.uint8,)),
                                      _dev(scale, "scale", (torch.float32,)), rows, cols,
                                      _stream(stream)))
