"""ctypes binding of libmmdit.so: the C ABI of include/mmdit.h, same names.

Argument marshalling only. Tensors may be passed as integers (device
addresses) or as objects with ``data_ptr()`` (torch tensors); a stream may be
an integer handle, None (the null stream) or an object with ``cuda_stream``.
Every call returns the library's integer status; ``check`` raises on a
non-zero status. There is no fallback: if the built library is missing,
importing this module raises.
"""
from __future__ import annotations

import ctypes
import os
import re
from ctypes import POINTER, Structure, c_char_p, c_float, c_int, c_int32, c_int64, c_size_t, c_void_p

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libmmdit.so")
HEADER_PATH = os.path.join(os.path.dirname(_PKG), "include", "mmdit.h")

if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is not built; run python -m diffusion_transformer_image_mm_amd.build")

# One HIP runtime per process. The library resolves libamdhip64.so.7 by
# SONAME, so it binds to whichever HIP runtime the process loaded first.
# PyTorch (the allocator and stream provider here) ships its own HIP and HSA
# runtimes; if this library were loaded first, the process would end up with
# the system HIP runtime next to PyTorch's HSA runtime, two runtimes driving
# one device. Loading PyTorch first makes the library share its runtime.
try:
    import torch  # noqa: F401
except ImportError:  # a process without PyTorch uses the system runtime
    pass
lib = ctypes.CDLL(LIB_PATH)

# ---------------------------------------------------------------- constants
MMDIT_ABI_VERSION = 3
MMDIT_OK, MMDIT_E_NULL, MMDIT_E_ALIGN, MMDIT_E_SHAPE = 0, 1, 2, 3
MMDIT_E_DTYPE, MMDIT_E_WORKSPACE, MMDIT_E_HIP, MMDIT_E_ARG = 4, 5, 6, 7
MMDIT_E_SCRATCH = 8
MMDIT_NOALLOC_SCRATCH_BYTES = 4 << 20
MMDIT_BF16, MMDIT_INT8, MMDIT_F16, MMDIT_FP8 = 0, 1, 2, 3
MMDIT_WS_DOUBLE, MMDIT_WS_SINGLE, MMDIT_WS_STEP = 0, 1, 2
(MMDIT_EPI_BIAS, MMDIT_EPI_BIAS_GELU, MMDIT_EPI_GATE_RESID, MMDIT_EPI_SPLIT_GELU,
 MMDIT_EPI_BIAS_F32, MMDIT_EPI_EULER, MMDIT_EPI_SWIGLU, MMDIT_EPI_SPLIT_SWIGLU) = range(8)
MMDIT_ACT_GELU_TANH, MMDIT_ACT_SWIGLU = 0, 1


# ---------------------------------------------------------------- structs
class mmdit_dims(Structure):
    _fields_ = [("txt_len", c_int32), ("img_len", c_int32), ("hidden", c_int32), ("heads", c_int32),
                ("head_dim", c_int32), ("mlp_hidden", c_int32), ("in_channels", c_int32),
                ("rope_axes", c_int32 * 3), ("rope_theta", c_float), ("ln_eps", c_float),
                ("rms_eps", c_float), ("weight_dtype", c_int32), ("n_double", c_int32),
                ("n_single", c_int32), ("mlp_act", c_int32), ("guidance_embed", c_int32),
                ("ref_len", c_int32)]


class mmdit_linear(Structure):
    _fields_ = [("w", c_void_p), ("scale", c_void_p), ("bias", c_void_p)]


class mmdit_stream_weights(Structure):
    _fields_ = [("mod", mmdit_linear), ("qkv", mmdit_linear), ("proj", mmdit_linear),
                ("fc1", mmdit_linear), ("fc2", mmdit_linear), ("q_norm", c_void_p), ("k_norm", c_void_p)]


class mmdit_double_weights(Structure):
    _fields_ = [("txt", mmdit_stream_weights), ("img", mmdit_stream_weights)]


class mmdit_single_weights(Structure):
    _fields_ = [("mod", mmdit_linear), ("linear1", mmdit_linear), ("linear2", mmdit_linear),
                ("q_norm", c_void_p), ("k_norm", c_void_p)]


class mmdit_model(Structure):
    _fields_ = [("img_in", mmdit_linear), ("time_in", mmdit_linear * 2), ("guid_in", mmdit_linear * 2),
                ("final_mod", mmdit_linear), ("final_out", mmdit_linear),
                ("doubles", POINTER(mmdit_double_weights)), ("singles", POINTER(mmdit_single_weights))]


class mmdit_gemm(Structure):
    _fields_ = [("m", c_int32), ("n", c_int32), ("k", c_int32), ("weight_dtype", c_int32),
                ("a", c_void_p), ("lda", c_int32), ("w", mmdit_linear), ("epilogue", c_int32),
                ("out", c_void_p), ("ldo", c_int32), ("gate", c_void_p), ("resid", c_void_p),
                ("ldr", c_int32), ("split_n", c_int32), ("out2", c_void_p), ("ldo2", c_int32),
                ("out2_col", c_int32), ("alpha", c_float), ("a_scale", c_void_p)]


# ---------------------------------------------------------------- marshalling
def ptr(x) -> int:
    """Device address of a tensor-like object (or an int / None)."""
    if x is None:
        return 0
    if isinstance(x, int):
        return x
    return int(x.data_ptr())


def stream_handle(s) -> int:
    if s is None:
        return 0
    if isinstance(s, int):
        return s
    return int(s.cuda_stream)


_P = c_void_p
_SIGS = {
    "mmdit_abi_version": (c_int, []),
    "mmdit_status_string": (c_char_p, [c_int]),
    "mmdit_workspace_bytes": (c_size_t, [POINTER(mmdit_dims), c_int]),
    "mmdit_block_forward": (c_int, [POINTER(mmdit_dims), POINTER(mmdit_double_weights), _P, _P, _P, _P,
                                    _P, c_size_t, _P]),
    "mmdit_single_block_forward": (c_int, [POINTER(mmdit_dims), POINTER(mmdit_single_weights), _P, _P,
                                           _P, _P, _P, c_size_t, _P]),
    "mmdit_denoise_step": (c_int, [POINTER(mmdit_dims), POINTER(mmdit_model), _P, _P, _P, c_float,
                                   c_float, c_float, _P, c_size_t, _P]),
    "mmdit_rope_table": (c_int, [POINTER(mmdit_dims), _P, _P, _P]),
    "mmdit_quantize_fp8_rows": (c_int, [_P, c_int, c_int, c_int, c_int, _P, c_int, _P, _P]),
    "mmdit_modulation_floats": (c_size_t, [POINTER(mmdit_dims)]),
    "mmdit_modulation_workspace_bytes": (c_size_t, [POINTER(mmdit_dims), c_int]),
    "mmdit_modulation_batch": (c_int, [POINTER(mmdit_dims), POINTER(mmdit_model), POINTER(c_float), c_int, c_float,
                                       _P, _P, c_size_t, _P]),
    "mmdit_modulation_batch_noalloc": (c_int, [POINTER(mmdit_dims), POINTER(mmdit_model), POINTER(c_float), c_int,
                                               c_float, _P, _P]),
    "mmdit_denoise_step_premod": (c_int, [POINTER(mmdit_dims), POINTER(mmdit_model), _P, _P, _P, _P, c_float,
                                          c_float, _P, c_size_t, _P]),
    "mmdit_k_ln_modulate": (c_int, [_P, c_int, c_int, c_int, _P, _P, _P, _P, c_float, _P, _P]),
    "mmdit_k_qknorm_rope": (c_int, [_P, c_int, c_int, c_int, c_int, c_int, _P, _P, _P, _P, _P, c_float,
                                    c_int, _P, _P, _P, _P]),
    "mmdit_k_attention": (c_int, [_P, _P, _P, c_int, c_int, c_int, c_int, _P, c_int, _P]),
    "mmdit_k_quantize_attention_fp8": (c_int, [_P, _P, _P, c_int, c_int, c_int, _P, _P, _P, _P, _P, _P, _P, _P,
                                               _P, _P]),
    "mmdit_k_attention_fp8": (c_int, [_P, _P, _P, _P, _P, c_int, c_int, c_int, c_int, _P, c_int, _P]),
    "mmdit_k_gemm": (c_int, [POINTER(mmdit_gemm), _P]),
    "mmdit_k_gemv": (c_int, [_P, c_int, POINTER(mmdit_linear), c_int, c_int, c_int, c_int, _P, _P]),
    "mmdit_k_time_embed": (c_int, [POINTER(mmdit_dims), POINTER(mmdit_model), c_float, c_float, _P, _P,
                                   c_size_t, _P]),
    "mmdit_k_euler": (c_int, [_P, _P, c_int64, c_float, _P]),
    "mmdit_weights_to_f16": (c_int, [_P, _P, c_size_t, _P]),
}
for _name, (_res, _args) in _SIGS.items():
    _f = getattr(lib, _name)
    _f.restype = _res
    _f.argtypes = _args


def header_functions() -> list:
    """Names of the functions declared in include/mmdit.h."""
    with open(HEADER_PATH) as f:
        text = f.read()
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[\w ]+?\*?\s*\b(mmdit_\w+)\s*\(", text, re.M)))


class MMDiTError(RuntimeError):
    def __init__(self, status: int, where: str):
        super().__init__(f"{where}: {mmdit_status_string(status)} (status {status})")
        self.status = status


def check(status: int, where: str = "mmdit") -> None:
    if status != MMDIT_OK:
        raise MMDiTError(status, where)


# ---------------------------------------------------------------- functions
def mmdit_abi_version() -> int:
    return lib.mmdit_abi_version()


def mmdit_status_string(status: int) -> str:
    return lib.mmdit_status_string(status).decode()


def mmdit_workspace_bytes(dims: mmdit_dims, kind: int) -> int:
    return lib.mmdit_workspace_bytes(ctypes.byref(dims), kind)


def mmdit_block_forward(dims, w, vec, rope, x_in, x_out, ws, ws_bytes, stream=None) -> int:
    return lib.mmdit_block_forward(ctypes.byref(dims), ctypes.byref(w), ptr(vec), ptr(rope), ptr(x_in),
                                   ptr(x_out), ptr(ws), ws_bytes, stream_handle(stream))


def mmdit_single_block_forward(dims, w, vec, rope, x_in, x_out, ws, ws_bytes, stream=None) -> int:
    return lib.mmdit_single_block_forward(ctypes.byref(dims), ctypes.byref(w), ptr(vec), ptr(rope),
                                          ptr(x_in), ptr(x_out), ptr(ws), ws_bytes, stream_handle(stream))


def mmdit_quantize_fp8_rows(x, x_dtype, rows, cols, ldx, codes, ldc, scales, stream=None) -> int:
    return lib.mmdit_quantize_fp8_rows(ptr(x), x_dtype, rows, cols, ldx, ptr(codes), ldc, ptr(scales),
                                       stream_handle(stream))


def mmdit_modulation_floats(dims) -> int:
    return lib.mmdit_modulation_floats(ctypes.byref(dims))


def mmdit_modulation_workspace_bytes(dims, n_steps: int) -> int:
    return lib.mmdit_modulation_workspace_bytes(ctypes.byref(dims), n_steps)


def mmdit_modulation_batch(dims, model, t, guidance, mod, ws, ws_bytes, stream=None) -> int:
    """t: a sequence of step times (host); marshalled to a float32 array."""
    n = len(t)
    arr = (c_float * max(n, 1))(*[float(v) for v in t])
    return lib.mmdit_modulation_batch(ctypes.byref(dims), ctypes.byref(model), arr, n, guidance, ptr(mod),
                                      ptr(ws), ws_bytes, stream_handle(stream))


def mmdit_modulation_batch_noalloc(dims, model, t, guidance, mod, stream=None) -> int:
    """t: a sequence of step times (host); marshalled to a float32 array."""
    n = len(t)
    arr = (c_float * max(n, 1))(*[float(v) for v in t])
    return lib.mmdit_modulation_batch_noalloc(ctypes.byref(dims), ctypes.byref(model), arr, n, guidance, ptr(mod),
                                              stream_handle(stream))


def mmdit_denoise_step_premod(dims, model, mod, latent, txt, rope, t_cur, t_next, ws, ws_bytes,
                              stream=None) -> int:
    return lib.mmdit_denoise_step_premod(ctypes.byref(dims), ctypes.byref(model), ptr(mod), ptr(latent), ptr(txt),
                                         ptr(rope), t_cur, t_next, ptr(ws), ws_bytes, stream_handle(stream))


def mmdit_denoise_step(dims, model, latent, txt, rope, t_cur, t_next, guidance, ws, ws_bytes,
                       stream=None) -> int:
    return lib.mmdit_denoise_step(ctypes.byref(dims), ctypes.byref(model), ptr(latent), ptr(txt), ptr(rope),
                                  t_cur, t_next, guidance, ptr(ws), ws_bytes, stream_handle(stream))


def mmdit_rope_table(dims, ids, rope, stream=None) -> int:
    return lib.mmdit_rope_table(ctypes.byref(dims), ptr(ids), ptr(rope), stream_handle(stream))


def mmdit_k_ln_modulate(x, rows, hidden, split, shift0, scale0, shift1, scale1, eps, out,
                        stream=None) -> int:
    return lib.mmdit_k_ln_modulate(ptr(x), rows, hidden, split, ptr(shift0), ptr(scale0), ptr(shift1),
                                   ptr(scale1), eps, ptr(out), stream_handle(stream))


def mmdit_k_qknorm_rope(qkv, ld, seq_len, heads, head_dim, split, qn0, kn0, qn1, kn1, rope, eps, l_pad,
                        q_out, k_out, vt_out, stream=None) -> int:
    return lib.mmdit_k_qknorm_rope(ptr(qkv), ld, seq_len, heads, head_dim, split, ptr(qn0), ptr(kn0),
                                   ptr(qn1), ptr(kn1), ptr(rope), eps, l_pad, ptr(q_out), ptr(k_out),
                                   ptr(vt_out), stream_handle(stream))


def mmdit_k_attention(q, k, vt, heads, seq_len, head_dim, l_pad, out, ldo, stream=None) -> int:
    return lib.mmdit_k_attention(ptr(q), ptr(k), ptr(vt), heads, seq_len, head_dim, l_pad, ptr(out), ldo,
                                 stream_handle(stream))


def mmdit_k_quantize_attention_fp8(q, k, vt, heads, head_dim, l_pad, q_norm0, q_norm1, k_norm0, k_norm1,
                                   q8, k8, vt8, v_scale, exps, stream=None) -> int:
    return lib.mmdit_k_quantize_attention_fp8(ptr(q), ptr(k), ptr(vt), heads, head_dim, l_pad, ptr(q_norm0),
                                              ptr(q_norm1), ptr(k_norm0), ptr(k_norm1), ptr(q8), ptr(k8), ptr(vt8),
                                              ptr(v_scale), ptr(exps), stream_handle(stream))


def mmdit_k_attention_fp8(q8, k8, vt8, v_scale, exps, heads, seq_len, head_dim, l_pad, out, ldo, stream=None) -> int:
    return lib.mmdit_k_attention_fp8(ptr(q8), ptr(k8), ptr(vt8), ptr(v_scale), ptr(exps), heads, seq_len, head_dim,
                                     l_pad, ptr(out), ldo, stream_handle(stream))


def mmdit_k_gemm(g: mmdit_gemm, stream=None) -> int:
    return lib.mmdit_k_gemm(ctypes.byref(g), stream_handle(stream))


def mmdit_k_gemv(x, k, w: mmdit_linear, n, weight_dtype, silu_input, accumulate, out, stream=None) -> int:
    return lib.mmdit_k_gemv(ptr(x), k, ctypes.byref(w), n, weight_dtype, silu_input, accumulate, ptr(out),
                            stream_handle(stream))


def mmdit_k_time_embed(dims, model, t, guidance, vec, ws, ws_bytes, stream=None) -> int:
    return lib.mmdit_k_time_embed(ctypes.byref(dims), ctypes.byref(model), t, guidance, ptr(vec), ptr(ws),
                                  ws_bytes, stream_handle(stream))


def mmdit_k_euler(z, v, n, dt, stream=None) -> int:
    return lib.mmdit_k_euler(ptr(z), ptr(v), n, dt, stream_handle(stream))


def mmdit_weights_to_f16(src, dst, count, stream=None) -> int:
    return lib.mmdit_weights_to_f16(ptr(src), ptr(dst), count, stream_handle(stream))
