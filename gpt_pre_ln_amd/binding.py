"""ctypes binding of libgpt2.so: the C ABI of include/gpt2.h under the same names.

Argument marshalling only -- every step of the forward runs in the HIP
kernels behind the library.  PyTorch is used for device memory and streams;
device pointers are passed as integers (``tensor.data_ptr()``) and the stream
as ``torch.cuda.current_stream().cuda_stream``.

If the library has not been built, loading fails loudly: there is no CPU
fallback.
"""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libgpt2.so")

GPT2_OK = 0
GPT2_ERR_INVALID_ARG = 1
GPT2_ERR_SHAPE = 2
GPT2_ERR_CAPACITY = 3
GPT2_ERR_WORKSPACE = 4
GPT2_ERR_UNSUPPORTED = 5
GPT2_ERR_HIP = 6

GPT2_F32 = 0
GPT2_BF16 = 1

KERNEL_CLASSES = {"embed": 0, "layernorm": 1, "qkv_gemm": 2, "attention": 3, "attn_proj_gemm": 4,
                  "fc_gemm": 5, "mlp_proj_gemm": 6, "lm_head_gemm": 7}


class gpt2_config(ctypes.Structure):
    _fields_ = [("vocab_size", ctypes.c_int32), ("n_positions", ctypes.c_int32),
                ("d_model", ctypes.c_int32), ("n_head", ctypes.c_int32),
                ("n_layer", ctypes.c_int32), ("d_ff", ctypes.c_int32),
                ("ln_eps", ctypes.c_float), ("dtype", ctypes.c_int32), ("logits_dtype", ctypes.c_int32),
                ("activation", ctypes.c_int32), ("scale_attn_by_inverse_layer_idx", ctypes.c_int32),
                ("post_ln", ctypes.c_int32), ("separate_head", ctypes.c_int32)]


class gpt2_kv_view(ctypes.Structure):
    _fields_ = [("d_kv", ctypes.c_void_p), ("B", ctypes.c_int32), ("max_T", ctypes.c_int32),
                ("past_len", ctypes.c_int32)]


class gpt2_param_info(ctypes.Structure):
    _fields_ = [("blob_offset", ctypes.c_int64), ("rows", ctypes.c_int32), ("cols", ctypes.c_int32),
                ("dev_dtype", ctypes.c_int32), ("transposed", ctypes.c_int32), ("dev_offset", ctypes.c_int64),
                ("dev_ld", ctypes.c_int64), ("dev_rows", ctypes.c_int64)]


class GPT2Error(RuntimeError):
    def __init__(self, status: int, where: str):
        lib = load()
        msg = lib.gpt2_status_string(status).decode()
        detail = lib.gpt2_last_error().decode()
        super().__init__(f"{where}: {msg}" + (f" ({detail})" if detail and status == GPT2_ERR_HIP else ""))
        self.status = status


_lib = None

_P = ctypes.c_void_p
_SIG = {
    "gpt2_param_blob_floats": (ctypes.c_int, [ctypes.POINTER(gpt2_config), ctypes.POINTER(ctypes.c_size_t)]),
    "gpt2_param_bytes": (ctypes.c_int, [ctypes.POINTER(gpt2_config), ctypes.POINTER(ctypes.c_size_t)]),
    "gpt2_param_tensor_count": (ctypes.c_int, [ctypes.POINTER(gpt2_config), ctypes.POINTER(ctypes.c_int32)]),
    "gpt2_param_tensor": (ctypes.c_int, [ctypes.POINTER(gpt2_config), ctypes.c_int32,
                                         ctypes.POINTER(gpt2_param_info)]),
    "gpt2_kv_stride": (ctypes.c_int, [ctypes.POINTER(gpt2_config), ctypes.c_int32, ctypes.POINTER(ctypes.c_int32)]),
    "gpt2_set_id_check": (ctypes.c_int, [_P, _P]),
    "gpt2_decode_step_noalloc": (ctypes.c_int, [_P, ctypes.POINTER(gpt2_kv_view), _P, _P, _P]),
    "gpt2_decode_scratch_bytes": (ctypes.c_int, [ctypes.POINTER(gpt2_config), ctypes.c_int32,
                                                 ctypes.POINTER(ctypes.c_size_t), ctypes.POINTER(ctypes.c_size_t)]),
    "gpt2_source_hash": (ctypes.c_char_p, []),
    "gpt2_workspace_bytes": (ctypes.c_int, [ctypes.POINTER(gpt2_config), ctypes.c_int32, ctypes.c_int32,
                                            ctypes.POINTER(ctypes.c_size_t)]),
    "gpt2_kv_cache_bytes": (ctypes.c_int, [ctypes.POINTER(gpt2_config), ctypes.c_int32, ctypes.c_int32,
                                           ctypes.POINTER(ctypes.c_size_t)]),
    "gpt2_create": (ctypes.c_int, [ctypes.POINTER(gpt2_config), _P, ctypes.c_size_t, _P, ctypes.c_size_t,
                                   ctypes.POINTER(_P)]),
    "gpt2_destroy": (None, [_P]),
    "gpt2_init_params": (ctypes.c_int, [_P, _P, ctypes.c_size_t, _P]),
    "gpt2_forward": (ctypes.c_int, [_P, _P, ctypes.c_int32, ctypes.c_int32, _P, _P,
                                    ctypes.POINTER(gpt2_kv_view), _P]),
    "gpt2_logits_padded_ld": (ctypes.c_int, [ctypes.POINTER(gpt2_config), ctypes.POINTER(ctypes.c_int64)]),
    "gpt2_forward_strided": (ctypes.c_int, [_P, _P, ctypes.c_int32, ctypes.c_int32, _P, ctypes.c_int64, _P,
                                            ctypes.POINTER(gpt2_kv_view), _P]),
    "gpt2_forward_loss": (ctypes.c_int, [_P, _P, _P, ctypes.c_int32, ctypes.c_int32, _P, _P, _P]),
    "gpt2_decode_step": (ctypes.c_int, [_P, ctypes.POINTER(gpt2_kv_view), _P, _P, _P]),
    "gpt2_generate": (ctypes.c_int, [_P, ctypes.POINTER(gpt2_kv_view), _P, ctypes.c_int32, _P, _P]),
    "gpt2_generate_sample": (ctypes.c_int, [_P, ctypes.POINTER(gpt2_kv_view), _P, ctypes.c_int32, ctypes.c_float,
                                            ctypes.c_uint64, _P, _P]),
    "gpt2_block_backward_workspace_bytes": (ctypes.c_int, [ctypes.POINTER(gpt2_config), ctypes.c_int32,
                                                           ctypes.c_int32, ctypes.POINTER(ctypes.c_size_t)]),
    "gpt2_block_backward": (ctypes.c_int, [_P, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, _P, _P, _P, _P, _P,
                                           ctypes.c_size_t, _P]),
    "gpt2_set_trace": (ctypes.c_int, [_P, _P, ctypes.c_size_t]),
    "gpt2_timing_enable": (ctypes.c_int, [_P, ctypes.c_int32, ctypes.c_int32]),
    "gpt2_timing_read": (ctypes.c_int, [_P, ctypes.POINTER(ctypes.c_double), ctypes.POINTER(ctypes.c_int32)]),
    "gpt2_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "gpt2_last_error": (ctypes.c_char_p, []),
}


def load(path: str = LIB_PATH):
    """Load libgpt2.so (raises if it is missing: build it with gpt_pre_ln_amd/build.py).

    The library carries the digest of the sources it was built from; loading
    refuses a binary whose digest differs from that of the sources beside it
    (a stale build), unless GPT2_ALLOW_STALE_LIB=1."""
    global _lib
    if _lib is None:
        if not os.path.exists(path):
            raise RuntimeError(f"{path} is missing: the HIP library must be built "
                               "(python gpt_pre_ln_amd/build.py); there is no fallback")
        lib = ctypes.CDLL(path)
        lib.gpt2_source_hash.restype = ctypes.c_char_p
        lib.gpt2_source_hash.argtypes = []
        built = lib.gpt2_source_hash().decode()
        from gpt_pre_ln_amd.build import source_hash
        want = source_hash()
        if built != want and os.environ.get("GPT2_ALLOW_STALE_LIB") != "1":
            raise RuntimeError(f"{path} was built from sources {built}, but the sources here hash to {want}: "
                               "rebuild it (python gpt_pre_ln_amd/build.py)")
        for name, (res, args) in _SIG.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        _lib = lib
    return _lib


def _check(status: int, where: str):
    if status != GPT2_OK:
        raise GPT2Error(status, where)


def _dtype_code(dtype) -> int:
    return {"f32": GPT2_F32, "bf16": GPT2_BF16}[dtype] if isinstance(dtype, str) else int(dtype)


def make_config(vocab_size, n_positions, d_model, n_head, n_layer, d_ff, ln_eps=1e-5, dtype="bf16",
                logits_dtype=None, activation="gelu_new", scale_attn_by_inverse_layer_idx=False, post_ln=False,
                tie_word_embeddings=True):
    """logits_dtype defaults to the arithmetic dtype (bf16 logits for a bf16 model).
    activation: "gelu_new" (tanh form) or "gelu" (erf form)."""
    dt = _dtype_code(dtype)
    ldt = dt if logits_dtype is None else _dtype_code(logits_dtype)
    if activation not in ("gelu_new", "gelu"):
        raise ValueError(f"activation {activation!r}")
    return gpt2_config(vocab_size, n_positions, d_model, n_head, n_layer, d_ff, ln_eps, dt, ldt,
                       int(activation == "gelu"), int(bool(scale_attn_by_inverse_layer_idx)), int(bool(post_ln)),
                       int(not tie_word_embeddings))


# ------------------------------------------------------------ thin wrappers


def gpt2_param_blob_floats(cfg) -> int:
    n = ctypes.c_size_t()
    _check(load().gpt2_param_blob_floats(ctypes.byref(cfg), ctypes.byref(n)), "gpt2_param_blob_floats")
    return n.value


def gpt2_param_bytes(cfg) -> int:
    n = ctypes.c_size_t()
    _check(load().gpt2_param_bytes(ctypes.byref(cfg), ctypes.byref(n)), "gpt2_param_bytes")
    return n.value


def gpt2_workspace_bytes(cfg, B: int, T: int) -> int:
    n = ctypes.c_size_t()
    _check(load().gpt2_workspace_bytes(ctypes.byref(cfg), B, T, ctypes.byref(n)), "gpt2_workspace_bytes")
    return n.value


def gpt2_kv_cache_bytes(cfg, B: int, max_T: int) -> int:
    n = ctypes.c_size_t()
    _check(load().gpt2_kv_cache_bytes(ctypes.byref(cfg), B, max_T, ctypes.byref(n)), "gpt2_kv_cache_bytes")
    return n.value


def gpt2_create(cfg, d_params: int, param_bytes: int, d_workspace: int, ws_bytes: int):
    h = ctypes.c_void_p()
    _check(load().gpt2_create(ctypes.byref(cfg), d_params, param_bytes, d_workspace, ws_bytes, ctypes.byref(h)),
           "gpt2_create")
    return h


def gpt2_destroy(handle):
    load().gpt2_destroy(handle)


def gpt2_init_params(handle, d_blob: int, n_floats: int, stream: int):
    _check(load().gpt2_init_params(handle, d_blob, n_floats, stream), "gpt2_init_params")


def gpt2_forward(handle, d_tokens: int, B: int, T: int, d_logits, d_hidden, kv, stream: int):
    _check(load().gpt2_forward(handle, d_tokens, B, T, d_logits, d_hidden,
                               ctypes.byref(kv) if kv is not None else None, stream), "gpt2_forward")


def gpt2_logits_padded_ld(cfg) -> int:
    ld = ctypes.c_int64()
    _check(load().gpt2_logits_padded_ld(ctypes.byref(cfg), ctypes.byref(ld)), "gpt2_logits_padded_ld")
    return ld.value


def gpt2_forward_strided(handle, d_tokens: int, B: int, T: int, d_logits, logits_ld: int, d_hidden, kv,
                         stream: int):
    _check(load().gpt2_forward_strided(handle, d_tokens, B, T, d_logits, logits_ld, d_hidden,
                                       ctypes.byref(kv) if kv is not None else None, stream),
           "gpt2_forward_strided")


def gpt2_forward_loss(handle, d_tokens: int, d_labels, B: int, T: int, d_token_loss, d_mean_loss, stream: int):
    _check(load().gpt2_forward_loss(handle, d_tokens, d_labels, B, T, d_token_loss, d_mean_loss, stream),
           "gpt2_forward_loss")


def gpt2_decode_step(handle, kv, d_new_tokens: int, d_logits: int, stream: int):
    _check(load().gpt2_decode_step(handle, ctypes.byref(kv), d_new_tokens, d_logits, stream), "gpt2_decode_step")


def gpt2_generate(handle, kv, d_tokens: int, n_steps: int, d_out_tokens: int, stream: int):
    _check(load().gpt2_generate(handle, ctypes.byref(kv), d_tokens, n_steps, d_out_tokens, stream), "gpt2_generate")


def gpt2_generate_sample(handle, kv, d_tokens: int, n_steps: int, temperature: float, seed: int, d_out_tokens: int,
                         stream: int):
    _check(load().gpt2_generate_sample(handle, ctypes.byref(kv), d_tokens, n_steps, temperature, seed, d_out_tokens,
                                       stream), "gpt2_generate_sample")


def gpt2_block_backward_workspace_bytes(cfg, B: int, T: int) -> int:
    n = ctypes.c_size_t()
    _check(load().gpt2_block_backward_workspace_bytes(ctypes.byref(cfg), B, T, ctypes.byref(n)),
           "gpt2_block_backward_workspace_bytes")
    return n.value


def gpt2_block_backward(handle, layer: int, B: int, T: int, d_x: int, d_dy: int, d_dx: int, d_grads: int,
                        d_ws: int, ws_bytes: int, stream: int):
    _check(load().gpt2_block_backward(handle, layer, B, T, d_x, d_dy, d_dx, d_grads, d_ws, ws_bytes, stream),
           "gpt2_block_backward")


def gpt2_set_trace(handle, d_trace, n_floats: int):
    _check(load().gpt2_set_trace(handle, d_trace, n_floats), "gpt2_set_trace")


def gpt2_timing_enable(handle, which, on: bool):
    w = KERNEL_CLASSES[which] if isinstance(which, str) else int(which)
    _check(load().gpt2_timing_enable(handle, w, 1 if on else 0), "gpt2_timing_enable")


def gpt2_timing_read(handle):
    ms = ctypes.c_double()
    n = ctypes.c_int32()
    _check(load().gpt2_timing_read(handle, ctypes.byref(ms), ctypes.byref(n)), "gpt2_timing_read")
    return ms.value, n.value


def gpt2_param_tensor_count(cfg) -> int:
    n = ctypes.c_int32()
    _check(load().gpt2_param_tensor_count(ctypes.byref(cfg), ctypes.byref(n)), "gpt2_param_tensor_count")
    return n.value


def gpt2_param_tensor(cfg, index: int) -> gpt2_param_info:
    info = gpt2_param_info()
    _check(load().gpt2_param_tensor(ctypes.byref(cfg), index, ctypes.byref(info)), "gpt2_param_tensor")
    return info


def gpt2_kv_stride(cfg, max_T: int) -> int:
    n = ctypes.c_int32()
    _check(load().gpt2_kv_stride(ctypes.byref(cfg), max_T, ctypes.byref(n)), "gpt2_kv_stride")
    return n.value


def gpt2_set_id_check(handle, d_flag):
    _check(load().gpt2_set_id_check(handle, d_flag), "gpt2_set_id_check")


def gpt2_source_hash() -> str:
    return load().gpt2_source_hash().decode()


def gpt2_decode_step_noalloc(handle, kv, d_new_tokens: int, d_logits: int, stream: int):
    _check(load().gpt2_decode_step_noalloc(handle, ctypes.byref(kv), d_new_tokens, d_logits, stream),
           "gpt2_decode_step_noalloc")


def gpt2_decode_scratch_bytes(cfg, B: int):
    """(bytes the allocation-free decode step needs at batch B, the library's per-device limit)."""
    n, lim = ctypes.c_size_t(), ctypes.c_size_t()
    _check(load().gpt2_decode_scratch_bytes(ctypes.byref(cfg), B, ctypes.byref(n), ctypes.byref(lim)),
           "gpt2_decode_scratch_bytes")
    return n.value, lim.value
