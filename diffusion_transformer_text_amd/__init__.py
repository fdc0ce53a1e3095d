"""Python binding of libmoss_dit.so, the MI355X (gfx950) MOSS-Image DiT denoising step.

Argument marshalling only: every step of the path runs in the library's HIP kernels. Functions keep
the C ABI's names (include/moss_dit.h, include/moss_dit_ops.h). Device tensors are torch tensors on
the current HIP device; the stream defaults to torch's current stream. Importing this package fails
loudly when the library has not been built (``python diffusion_transformer_text_amd/build.py``).
"""
from __future__ import annotations

import ctypes as C
import os
from typing import Dict, List, Optional, Sequence

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmoss_dit.so")

if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is missing: build it with `python diffusion_transformer_text_amd/build.py`")
# torch ships its own HIP runtime with the same soname (libamdhip64.so.7) as ROCm's. Loading torch
# first makes the library's dependency resolve to that already-loaded runtime, so the process has a
# single HIP runtime and torch's device memory and streams are valid handles for the library.
import torch  # noqa: E402,F401
_lib = C.CDLL(LIB_PATH)

MOSS_OK, MOSS_ERR_INVALID_ARGUMENT, MOSS_ERR_NOT_SUPPORTED, MOSS_ERR_OUT_OF_MEMORY, MOSS_ERR_DEVICE, \
    MOSS_ERR_ABI_MISMATCH = range(6)
ABI_VERSION = 1


class MossError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"[{status}: {moss_status_string(status)}] {message}")
        self.status = status


# ---- structs (same field order and types as the C header) ----
class moss_dit_config(C.Structure):
    _fields_ = [("struct_size", C.c_uint32), ("num_layers", C.c_int32), ("hidden", C.c_int32),
                ("num_heads", C.c_int32), ("head_dim", C.c_int32), ("ffn_hidden", C.c_int32),
                ("latent_channels", C.c_int32), ("patch", C.c_int32), ("temb_dim", C.c_int32),
                ("qk_norm", C.c_int32), ("rope_theta", C.c_float), ("norm_eps", C.c_float),
                ("flow_multiplier", C.c_float), ("text_dim", C.c_int32), ("refiner_layers", C.c_int32),
                ("gemm_precision", C.c_int32), ("attention_mode", C.c_int32)]


class moss_dit_weights(C.Structure):
    _fields_ = [("struct_size", C.c_uint32), ("t_w1", C.c_void_p), ("t_w2", C.c_void_p), ("x_embed_w", C.c_void_p),
                ("mod_w", C.POINTER(C.c_void_p)), ("qkv_w", C.POINTER(C.c_void_p)), ("out_w", C.POINTER(C.c_void_p)),
                ("gate_up_w", C.POINTER(C.c_void_p)), ("down_w", C.POINTER(C.c_void_p)),
                ("q_norm_w", C.POINTER(C.c_void_p)), ("k_norm_w", C.POINTER(C.c_void_p)),
                ("final_mod_w", C.c_void_p), ("final_w", C.c_void_p), ("text_proj_w", C.c_void_p),
                ("refiner_qkv_w", C.POINTER(C.c_void_p)), ("refiner_out_w", C.POINTER(C.c_void_p)),
                ("refiner_gate_up_w", C.POINTER(C.c_void_p)), ("refiner_down_w", C.POINTER(C.c_void_p))]


class moss_forward_args(C.Structure):
    _fields_ = [("struct_size", C.c_uint32), ("batch", C.c_int32), ("latent_h", C.c_int32), ("latent_w", C.c_int32),
                ("text_len", C.c_int32), ("latents", C.c_void_p), ("text", C.c_void_p),
                ("sigma", C.POINTER(C.c_float)), ("skip_mask", C.POINTER(C.c_uint64)), ("velocity", C.c_void_p),
                ("residual_dump", C.c_void_p)]


class moss_step_args(C.Structure):
    _fields_ = [("struct_size", C.c_uint32), ("latent_h", C.c_int32), ("latent_w", C.c_int32),
                ("text_len", C.c_int32), ("num_steps", C.c_int32), ("step", C.c_int32), ("x", C.c_void_p),
                ("text_cond", C.c_void_p), ("text_uncond", C.c_void_p), ("sigmas", C.POINTER(C.c_float)),
                ("cfg_scale", C.c_float), ("slg_start", C.c_float), ("slg_stop", C.c_float),
                ("uncond_skip_layers", C.POINTER(C.c_int32)), ("n_skip", C.c_int32), ("slg_scale", C.c_float),
                ("cfg_truncation", C.c_float), ("step_cache", C.c_int32), ("step_cache_threshold", C.c_float)]


class moss_block_taps(C.Structure):
    _fields_ = [("struct_size", C.c_uint32), ("a", C.c_void_p), ("qkv", C.c_void_p), ("o", C.c_void_p),
                ("attn", C.c_void_p), ("x1", C.c_void_p), ("a2", C.c_void_p), ("h", C.c_void_p), ("ffn", C.c_void_p)]


def _sig(name, res, *args):
    f = getattr(_lib, name)
    f.restype = res
    f.argtypes = list(args)
    return f


_P = C.c_void_p
_sig("moss_dit_abi_version", C.c_int)
_sig("moss_status_string", C.c_char_p, C.c_int)
_sig("moss_dit_last_error", C.c_char_p, _P)
_sig("moss_dit_config_init", None, C.POINTER(moss_dit_config), C.c_uint32)
_sig("moss_dit_weights_init", None, C.POINTER(moss_dit_weights), C.c_uint32)
_sig("moss_forward_args_init", None, C.POINTER(moss_forward_args), C.c_uint32)
_sig("moss_step_args_init", None, C.POINTER(moss_step_args), C.c_uint32)
_sig("moss_block_taps_init", None, C.POINTER(moss_block_taps), C.c_uint32)
_sig("moss_dit_create", C.c_int, C.POINTER(moss_dit_config), C.POINTER(moss_dit_weights), C.c_int, _P, C.POINTER(_P))
_sig("moss_dit_destroy", None, _P)
_sig("moss_dit_forward", C.c_int, _P, C.POINTER(moss_forward_args), _P)
_sig("moss_validate_forward_args", C.c_int, C.POINTER(moss_dit_config), C.POINTER(moss_forward_args), C.c_char_p, C.c_int32)
_sig("moss_sigmas", C.c_int, C.c_int32, C.c_float, C.POINTER(C.c_float))
_sig("moss_sample_step", C.c_int, _P, C.POINTER(moss_step_args), _P)
_sig("moss_validate_step_args", C.c_int, C.POINTER(moss_dit_config), C.POINTER(moss_step_args), C.c_char_p, C.c_int32)
_sig("moss_cfg_euler", C.c_int, _P, _P, _P, C.c_int64, C.c_float, C.c_float, C.c_float, _P)
_sig("moss_guidance_euler", C.c_int, _P, _P, _P, _P, C.c_int64, C.c_float, C.c_float, C.c_float, C.c_float, _P)
_sig("moss_dit_modulation", C.c_int, _P, C.POINTER(C.c_float), C.c_int32, _P, _P)
_sig("moss_dit_block", C.c_int, _P, C.c_int32, _P, C.c_int32, C.c_int32, C.c_int32, C.c_int32, _P, C.c_int64,
     C.POINTER(moss_block_taps), _P)
_sig("moss_step_cache_stats", C.c_int, _P, C.POINTER(C.c_int32), C.POINTER(C.c_int32), C.POINTER(C.c_float))
_sig("moss_text_refine", C.c_int, _P, C.c_int32, C.c_int32, _P, _P, _P)
_sig("moss_attention", C.c_int, _P, _P, C.c_int32, C.c_int32, C.c_int32, C.c_int32, C.c_int32, C.c_int32, _P)
_sig("moss_attention_noalloc", C.c_int, _P, _P, C.c_int32, C.c_int32, C.c_int32, C.c_int32, C.c_int32, C.c_int32, _P)
_sig("moss_gemm_bf16", C.c_int, _P, _P, _P, C.c_int32, C.c_int32, C.c_int32, _P)
_sig("moss_mx_quantize", C.c_int, _P, C.c_int32, C.c_int32, _P, _P, C.c_int64, _P)
_sig("moss_attention_q8_workspace", C.c_int64, C.c_int32, C.c_int32, C.c_int32)
_sig("moss_attention_q8", C.c_int, _P, _P, C.c_int32, C.c_int32, C.c_int32, _P, C.c_int64, _P)
_sig("moss_gemm_mxfp8", C.c_int, _P, _P, C.c_int64, _P, _P, C.c_int64, _P, C.c_int32, C.c_int32, C.c_int32, _P)
_sig("moss_dit_profile_enable", C.c_int, _P, C.c_int32)
_sig("moss_dit_profile_read", C.c_int, _P, C.POINTER(C.c_double), C.POINTER(C.c_int64))

PROF_CLASSES = ["modulation", "embed", "ln_mod", "gemm_qkv_rope", "attention", "gemm_out_residual",
                "gemm_gate_up_swiglu", "gemm_down_residual", "final_layer", "cfg_euler"]

# every symbol the headers declare (checked by the CPU test-suite)
EXPORTED = ["moss_dit_abi_version", "moss_status_string", "moss_dit_last_error", "moss_dit_config_init",
            "moss_dit_weights_init", "moss_dit_create", "moss_dit_destroy", "moss_forward_args_init",
            "moss_dit_forward", "moss_validate_forward_args", "moss_sigmas", "moss_step_args_init",
            "moss_sample_step", "moss_validate_step_args", "moss_cfg_euler", "moss_guidance_euler",
            "moss_text_refine", "moss_step_cache_stats", "moss_dit_modulation",
            "moss_block_taps_init", "moss_dit_block", "moss_attention", "moss_attention_noalloc", "moss_gemm_bf16",
            "moss_mx_quantize", "moss_gemm_mxfp8", "moss_attention_q8_workspace", "moss_attention_q8",
            "moss_dit_profile_enable", "moss_dit_profile_read"]


# ---- host-only calls ----
def moss_dit_abi_version() -> int:
    return _lib.moss_dit_abi_version()


def moss_status_string(status: int) -> str:
    return _lib.moss_status_string(status).decode()


def moss_dit_last_error(handle=None) -> str:
    return _lib.moss_dit_last_error(handle).decode()


def moss_dit_config_init(**overrides) -> moss_dit_config:
    c = moss_dit_config()
    _lib.moss_dit_config_init(C.byref(c), C.sizeof(c))
    for k, v in overrides.items():
        setattr(c, k, v)
    return c


def moss_forward_args_init() -> moss_forward_args:
    a = moss_forward_args()
    _lib.moss_forward_args_init(C.byref(a), C.sizeof(a))
    return a


def moss_step_args_init() -> moss_step_args:
    a = moss_step_args()
    _lib.moss_step_args_init(C.byref(a), C.sizeof(a))
    return a


def moss_sigmas(num_steps: int, shift: float = 5.0) -> np.ndarray:
    out = np.zeros(num_steps + 1, dtype=np.float32)
    st = _lib.moss_sigmas(num_steps, shift, out.ctypes.data_as(C.POINTER(C.c_float)))
    if st != MOSS_OK:
        raise MossError(st, moss_dit_last_error())
    return out


def moss_validate_step_args(cfg: moss_dit_config, args: moss_step_args):
    buf = C.create_string_buffer(512)
    st = _lib.moss_validate_step_args(C.byref(cfg), C.byref(args), buf, 512)
    return st, buf.value.decode()


def moss_validate_forward_args(cfg: moss_dit_config, args: moss_forward_args):
    buf = C.create_string_buffer(512)
    st = _lib.moss_validate_forward_args(C.byref(cfg), C.byref(args), buf, 512)
    return st, buf.value.decode()


# ---- device calls ----
def _stream(stream):
    if stream is not None:
        return C.c_void_p(stream)
    import torch
    return C.c_void_p(torch.cuda.current_stream().cuda_stream)


def _ptr(t) -> Optional[int]:
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _check_dev(t, dtype, name):
    import torch
    if not (t.is_cuda and t.is_contiguous() and t.dtype == dtype):
        raise ValueError(f"{name} must be a contiguous {dtype} tensor on the GPU")


def _check(st: int, handle=None):
    if st != MOSS_OK:
        raise MossError(st, moss_dit_last_error(handle))


def moss_cfg_euler(v_cond, v_uncond, x, cfg: float, sigma: float, sigma_next: float, stream=None):
    import torch
    for t, n in ((v_cond, "v_cond"), (x, "x")):
        _check_dev(t, torch.float32, n)
    if v_uncond is not None:
        _check_dev(v_uncond, torch.float32, "v_uncond")
    _check(_lib.moss_cfg_euler(_ptr(v_cond), _ptr(v_uncond), _ptr(x), x.numel(), cfg, sigma, sigma_next,
                               _stream(stream)))


def moss_guidance_euler(v_cond, v_uncond, v_skip, x, cfg: float, slg: float, sigma: float, sigma_next: float,
                        stream=None):
    import torch
    for t, n in ((v_cond, "v_cond"), (x, "x")):
        _check_dev(t, torch.float32, n)
    for t, n in ((v_uncond, "v_uncond"), (v_skip, "v_skip")):
        if t is not None:
            _check_dev(t, torch.float32, n)
    _check(_lib.moss_guidance_euler(_ptr(v_cond), _ptr(v_uncond), _ptr(v_skip), _ptr(x), x.numel(), cfg, slg, sigma,
                                    sigma_next, _stream(stream)))


def moss_attention(qkv, out, batch: int, seq: int, heads: int, text_len: int, grid_w: int, rope: bool = True,
                   stream=None):
    import torch
    _check_dev(qkv, torch.bfloat16, "qkv")
    _check_dev(out, torch.bfloat16, "out")
    if qkv.numel() != batch * seq * 3 * heads * 128 or out.numel() != batch * seq * heads * 128:
        raise ValueError("qkv / out sizes do not match batch, seq, heads")
    _check(_lib.moss_attention(_ptr(qkv), _ptr(out), batch, seq, heads, text_len, grid_w, int(rope), _stream(stream)))


def moss_attention_noalloc(qkv, out, batch: int, seq: int, heads: int, text_len: int, grid_w: int, rope: bool = True,
                           stream=None):
    """moss_attention on the library's static per-GPU scratch: no device allocation, no synchronisation."""
    import torch
    _check_dev(qkv, torch.bfloat16, "qkv")
    _check_dev(out, torch.bfloat16, "out")
    if qkv.numel() != batch * seq * 3 * heads * 128 or out.numel() != batch * seq * heads * 128:
        raise ValueError("qkv / out sizes do not match batch, seq, heads")
    _check(_lib.moss_attention_noalloc(_ptr(qkv), _ptr(out), batch, seq, heads, text_len, grid_w, int(rope),
                                       _stream(stream)))


def moss_gemm_bf16(A, W, out, stream=None):
    import torch
    _check_dev(A, torch.bfloat16, "A")
    _check_dev(W, torch.bfloat16, "W")
    _check_dev(out, torch.float32, "out")
    M, K = A.shape
    N = W.shape[0]
    if W.shape[1] != K or tuple(out.shape) != (M, N):
        raise ValueError("shape mismatch")
    _check(_lib.moss_gemm_bf16(_ptr(A), _ptr(W), _ptr(out), M, N, K, _stream(stream)))


def moss_attention_q8_workspace(batch: int, seq: int, heads: int) -> int:
    return int(_lib.moss_attention_q8_workspace(batch, seq, heads))


def moss_attention_q8(qkv, out, batch: int, seq: int, heads: int, ws=None, stream=None):
    """8-bit attention of qkv bf16 [B, S, 3 H 128] into out bf16 [B, S, H 128]; ws: uint8 device tensor of
    at least moss_attention_q8_workspace bytes (allocated here when None). Returns the workspace."""
    import torch
    _check_dev(qkv, torch.bfloat16, "qkv")
    _check_dev(out, torch.bfloat16, "out")
    if qkv.numel() != batch * seq * 3 * heads * 128 or out.numel() != batch * seq * heads * 128:
        raise ValueError("qkv / out sizes do not match batch, seq, heads")
    need = moss_attention_q8_workspace(batch, seq, heads)
    if ws is None:
        ws = torch.empty(need + 256, dtype=torch.uint8, device=qkv.device)
    _check_dev(ws, torch.uint8, "ws")
    off = (-ws.data_ptr()) % 256
    if ws.numel() - off < need:
        raise ValueError("workspace too small")
    _check(_lib.moss_attention_q8(_ptr(qkv), _ptr(out), batch, seq, heads, C.c_void_p(ws.data_ptr() + off),
                                  ws.numel() - off, _stream(stream)))
    return ws


def mx_scale_words(rows: int, K: int) -> int:
    """Words of MXFP8 scale storage for `rows` rows (ld = rows) of reduction length K."""
    return K // 128 * rows


def moss_mx_quantize(x, codes, scales, ld_scale=None, stream=None):
    """x bf16 [rows, K] -> codes uint8 [rows, K] and scale words int32 [K / 128 * ld_scale]."""
    import torch
    _check_dev(x, torch.bfloat16, "x")
    _check_dev(codes, torch.uint8, "codes")
    _check_dev(scales, torch.int32, "scales")
    rows, K = x.shape
    ld = rows if ld_scale is None else int(ld_scale)
    if tuple(codes.shape) != (rows, K) or scales.numel() < K // 128 * ld:
        raise ValueError("codes / scales sizes do not match x")
    _check(_lib.moss_mx_quantize(_ptr(x), rows, K, _ptr(codes), _ptr(scales), ld, _stream(stream)))


def moss_gemm_mxfp8(A, A_scales, lds_a, W, W_scales, lds_w, out, stream=None):
    """out fp32 [M, N] = MXFP8(A) MXFP8(W)^T from codes (uint8 [M, K], [N, K]) and scale words (int32)."""
    import torch
    for t, name in ((A, "A"), (W, "W")):
        _check_dev(t, torch.uint8, name)
    for t, name in ((A_scales, "A_scales"), (W_scales, "W_scales")):
        _check_dev(t, torch.int32, name)
    _check_dev(out, torch.float32, "out")
    M, K = A.shape
    N = W.shape[0]
    if W.shape[1] != K or tuple(out.shape) != (M, N):
        raise ValueError("shape mismatch")
    if A_scales.numel() < K // 128 * lds_a or W_scales.numel() < K // 128 * lds_w:
        raise ValueError("scale words too short for lds_a / lds_w")
    _check(_lib.moss_gemm_mxfp8(_ptr(A), _ptr(A_scales), int(lds_a), _ptr(W), _ptr(W_scales), int(lds_w), _ptr(out),
                                M, N, K, _stream(stream)))


class MossDiT:
    """Owns a moss_dit handle (weights copied into the library at creation)."""

    def __init__(self, cfg: moss_dit_config, weights: Dict, stream=None):
        """weights: dict with the C struct's field names; values are bf16 torch tensors on the GPU
        (per-block entries are lists), or uint16 numpy arrays (host copies)."""
        on_device = not isinstance(weights["t_w1"], np.ndarray)
        keep = []

        def p(t):
            if isinstance(t, np.ndarray):
                a = np.ascontiguousarray(t, dtype=np.uint16)
                keep.append(a)
                return a.ctypes.data
            if not t.is_contiguous():
                raise ValueError("weights must be contiguous")
            return t.data_ptr()

        w = moss_dit_weights()
        _lib.moss_dit_weights_init(C.byref(w), C.sizeof(w))
        for k in ("t_w1", "t_w2", "x_embed_w", "final_mod_w", "final_w"):
            setattr(w, k, p(weights[k]))
        arrays = {}
        per_block = ["mod_w", "qkv_w", "out_w", "gate_up_w", "down_w"]
        if weights.get("text_proj_w") is not None:           # optional text refiner
            w.text_proj_w = p(weights["text_proj_w"])
            per_block += ["refiner_qkv_w", "refiner_out_w", "refiner_gate_up_w", "refiner_down_w"]
        for k in per_block:
            lst = weights[k]
            arr = (C.c_void_p * max(1, len(lst)))(*[p(t) for t in lst])
            arrays[k] = arr
            setattr(w, k, C.cast(arr, C.POINTER(C.c_void_p)))
        self.cfg = cfg
        self.handle = C.c_void_p()
        st = _lib.moss_dit_create(C.byref(cfg), C.byref(w), int(on_device), _stream(stream), C.byref(self.handle))
        _check(st)
        del keep, arrays

    @property
    def mod_stride(self) -> int:
        return self.cfg.num_layers * 6 * self.cfg.hidden + 2 * self.cfg.hidden

    def close(self):
        if self.handle:
            _lib.moss_dit_destroy(self.handle)
            self.handle = C.c_void_p()

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def last_error(self) -> str:
        return moss_dit_last_error(self.handle)

    def moss_dit_profile_enable(self, enable: bool = True):
        _check(_lib.moss_dit_profile_enable(self.handle, int(enable)), self.handle)

    def moss_dit_profile_read(self) -> Dict[str, tuple]:
        ms = (C.c_double * len(PROF_CLASSES))()
        n = (C.c_int64 * len(PROF_CLASSES))()
        _check(_lib.moss_dit_profile_read(self.handle, ms, n), self.handle)
        return {k: (ms[i], n[i]) for i, k in enumerate(PROF_CLASSES)}

    def moss_dit_forward(self, latents, text, sigma: Sequence[float], velocity, skip_mask: Optional[Sequence[int]] = None,
                         residual_dump=None, stream=None):
        import torch
        _check_dev(latents, torch.float32, "latents")
        _check_dev(text, torch.float32, "text")
        _check_dev(velocity, torch.float32, "velocity")
        B, Cc, h, w = latents.shape
        a = moss_forward_args_init()
        a.batch, a.latent_h, a.latent_w, a.text_len = B, h, w, text.shape[1]
        a.latents, a.text, a.velocity = _ptr(latents), _ptr(text), _ptr(velocity)
        sig = (C.c_float * B)(*[float(s) for s in sigma])
        a.sigma = C.cast(sig, C.POINTER(C.c_float))
        if skip_mask is not None:
            sm = (C.c_uint64 * B)(*[int(s) for s in skip_mask])
            a.skip_mask = C.cast(sm, C.POINTER(C.c_uint64))
        if residual_dump is not None:
            _check_dev(residual_dump, torch.bfloat16, "residual_dump")
            a.residual_dump = _ptr(residual_dump)
        _check(_lib.moss_dit_forward(self.handle, C.byref(a), _stream(stream)), self.handle)

    def moss_sample_step(self, x, text_cond, text_uncond, sigmas: np.ndarray, step: int, cfg_scale: float = 3.0,
                         uncond_skip_layers: Sequence[int] = (22,), slg_start: float = 0.01, slg_stop: float = 1.0,
                         slg_scale: float = 0.0, cfg_truncation: float = 1.0, step_cache: bool = False,
                         step_cache_threshold: float = 0.0, stream=None):
        import torch
        _check_dev(x, torch.float32, "x")
        _check_dev(text_cond, torch.float32, "text_cond")
        if text_uncond is not None:
            _check_dev(text_uncond, torch.float32, "text_uncond")
        a = moss_step_args_init()
        _, _, h, w = x.shape
        a.latent_h, a.latent_w, a.text_len = h, w, text_cond.shape[1]
        a.num_steps, a.step = len(sigmas) - 1, step
        a.x, a.text_cond, a.text_uncond = _ptr(x), _ptr(text_cond), _ptr(text_uncond)
        sg = np.ascontiguousarray(sigmas, dtype=np.float32)
        a.sigmas = sg.ctypes.data_as(C.POINTER(C.c_float))
        a.cfg_scale, a.slg_start, a.slg_stop = cfg_scale, slg_start, slg_stop
        sk = (C.c_int32 * max(1, len(uncond_skip_layers)))(*[int(l) for l in uncond_skip_layers])
        a.uncond_skip_layers = C.cast(sk, C.POINTER(C.c_int32))
        a.n_skip = len(uncond_skip_layers)
        a.slg_scale, a.cfg_truncation = slg_scale, cfg_truncation
        a.step_cache, a.step_cache_threshold = int(step_cache), step_cache_threshold
        _check(_lib.moss_sample_step(self.handle, C.byref(a), _stream(stream)), self.handle)

    def moss_step_cache_stats(self):
        """(full_calls, reused_calls, last_change) of the current sampling run's step cache."""
        f, r, c = C.c_int32(), C.c_int32(), C.c_float()
        _check(_lib.moss_step_cache_stats(self.handle, C.byref(f), C.byref(r), C.byref(c)), self.handle)
        return f.value, r.value, c.value

    def moss_text_refine(self, enc, out, stream=None):
        """enc: fp32 [batch, text_len, text_dim] on the GPU -> out: fp32 [batch, text_len, hidden]."""
        import torch
        _check_dev(enc, torch.float32, "enc")
        _check_dev(out, torch.float32, "out")
        B, T, E = enc.shape
        if E != self.cfg.text_dim or tuple(out.shape) != (B, T, self.cfg.hidden):
            raise ValueError("enc must be [B, T, text_dim] and out [B, T, hidden]")
        _check(_lib.moss_text_refine(self.handle, B, T, _ptr(enc), _ptr(out), _stream(stream)), self.handle)

    def moss_dit_modulation(self, sigma: Sequence[float], mod, stream=None):
        import torch
        _check_dev(mod, torch.bfloat16, "mod")
        B = len(sigma)
        sig = (C.c_float * B)(*[float(s) for s in sigma])
        _check(_lib.moss_dit_modulation(self.handle, sig, B, _ptr(mod), _stream(stream)), self.handle)

    def moss_dit_block(self, layer: int, x, text_len: int, grid_h: int, grid_w: int, mod,
                       taps: Optional[Dict[str, object]] = None, stream=None):
        import torch
        _check_dev(x, torch.bfloat16, "x")
        _check_dev(mod, torch.bfloat16, "mod")
        B = x.shape[0]
        t = None
        if taps:
            t = moss_block_taps()
            _lib.moss_block_taps_init(C.byref(t), C.sizeof(t))
            for k, v in taps.items():
                setattr(t, k, _ptr(v))
        _check(_lib.moss_dit_block(self.handle, layer, _ptr(x), B, text_len, grid_h, grid_w, _ptr(mod),
                                   mod.shape[-1], C.byref(t) if t is not None else None, _stream(stream)),
               self.handle)
