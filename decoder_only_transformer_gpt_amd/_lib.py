"""ctypes binding of ``libgpt_amd.so`` (the C ABI in ``include/gpt.h``).

Argument marshalling only: every step of the training step runs in the HIP
library. PyTorch supplies device memory (tensors' ``data_ptr()``) and the
stream (``torch.cuda.current_stream().cuda_stream``). If the library has not
been built this module raises; there is no fallback path.
"""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libgpt_amd.so")

GPT_OK = 0
GPT_E_INVALID_ARG = -1
GPT_E_UNSUPPORTED = -2
GPT_E_WORKSPACE = -3
GPT_E_STATE = -4
GPT_E_HIP = -5
GPT_E_DEVICE = -6
GPT_F32 = 0
GPT_BF16 = 1
GPT_FP8_E4M3 = 2
GPT_OPT_GEMM_TILE = 1
GPT_OPT_DKV_HSPLIT = 2
GPT_OPT_RESID_GRAD = 3


class gpt_config(ctypes.Structure):
    _fields_ = [
        ("n_layer", ctypes.c_int32), ("model_dim", ctypes.c_int32), ("n_head", ctypes.c_int32),
        ("n_kv_head", ctypes.c_int32), ("head_dim", ctypes.c_int32), ("mlp_dim", ctypes.c_int32),
        ("vocab_size", ctypes.c_int32), ("max_seq_len", ctypes.c_int32),
        ("rope_theta", ctypes.c_float), ("logit_softcap", ctypes.c_float), ("norm_eps", ctypes.c_float),
        ("dtype", ctypes.c_int32), ("window_short", ctypes.c_int32), ("window_pattern", ctypes.c_char * 8),
        ("x0_lambdas", ctypes.c_int32), ("value_embeds", ctypes.c_int32),
    ]

    def as_dict(self) -> dict:
        d = {k: getattr(self, k) for k, _ in self._fields_}
        d["window_pattern"] = d["window_pattern"].decode()
        return d


class gpt_optim_config(ctypes.Structure):
    _fields_ = [(k, ctypes.c_float) for k in ("lr_muon", "lr_embed", "lr_unembed", "lr_scalar", "momentum", "beta1",
                                              "beta2", "eps", "wd_muon", "wd_adamw")] + [
        ("ns_steps", ctypes.c_int32), ("ns_a", ctypes.c_float), ("ns_b", ctypes.c_float), ("ns_c", ctypes.c_float)]

    def as_dict(self) -> dict:
        return {k: getattr(self, k) for k, _ in self._fields_}


class gpt_tensor_desc(ctypes.Structure):
    _fields_ = [("name", ctypes.c_char * 32), ("offset", ctypes.c_int64), ("rows", ctypes.c_int64),
                ("cols", ctypes.c_int64)]


class GptError(RuntimeError):
    def __init__(self, status: int, where: str, detail: str):
        super().__init__(f"{where}: {status_string(status)} ({status}): {detail}")
        self.status = status


_lib = None

# name -> (restype, argtypes), exactly the functions include/gpt.h declares
_P = ctypes.c_void_p
_SIGS = {
    "gpt_status_string": (ctypes.c_char_p, [ctypes.c_int32]),
    "gpt_last_error_message": (ctypes.c_char_p, []),
    "gpt_config_from_depth": (ctypes.c_int32, [ctypes.c_int32, ctypes.c_int32, ctypes.POINTER(gpt_config)]),
    "gpt_config_validate": (ctypes.c_int32, [ctypes.POINTER(gpt_config)]),
    "gpt_param_count": (ctypes.c_int64, [ctypes.POINTER(gpt_config)]),
    "gpt_param_layout": (ctypes.c_int32, [ctypes.POINTER(gpt_config), ctypes.POINTER(gpt_tensor_desc),
                                          ctypes.POINTER(ctypes.c_int32)]),
    "gpt_workspace_bytes": (ctypes.c_int32, [ctypes.POINTER(gpt_config), ctypes.c_int32, ctypes.c_int32,
                                             ctypes.POINTER(ctypes.c_size_t)]),
    "gpt_init": (ctypes.c_int32, [ctypes.POINTER(gpt_config), _P, _P, _P, ctypes.c_size_t, ctypes.c_int32,
                                  ctypes.c_int32, _P, ctypes.POINTER(_P)]),
    "gpt_forward_loss": (ctypes.c_int32, [_P, _P, _P, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, _P, _P, _P]),
    "gpt_backward": (ctypes.c_int32, [_P, ctypes.c_float, ctypes.c_int32, _P]),
    "gpt_sync_status": (ctypes.c_int32, [_P, _P]),
    "gpt_destroy": (ctypes.c_int32, [_P]),
    "gpt_profile_begin": (ctypes.c_int32, [_P, ctypes.c_int32]),
    "gpt_profile_end": (ctypes.c_int32, [_P, ctypes.POINTER(ctypes.c_double), ctypes.POINTER(ctypes.c_int64)]),
    "gpt_kernel_tag_name": (ctypes.c_char_p, [ctypes.c_int32]),
    "gpt_set_option": (ctypes.c_int32, [_P, ctypes.c_int32, ctypes.c_int32]),
    "gpt_debug_buffer": (ctypes.c_int32, [_P, ctypes.c_char_p, ctypes.c_int32, ctypes.POINTER(_P),
                                          ctypes.POINTER(ctypes.c_size_t)]),
    "gpt_fp8_quantize": (ctypes.c_int32, [_P, ctypes.c_int64, ctypes.c_int64, _P, _P, ctypes.c_int64, _P, _P]),
    "gpt_optimizer_state_elems": (ctypes.c_int32, [ctypes.POINTER(gpt_config), ctypes.POINTER(ctypes.c_int64)]),
    "gpt_optimizer_step": (ctypes.c_int32, [_P, ctypes.POINTER(gpt_optim_config), _P, _P, ctypes.c_int32, _P]),
    "gpt_fp8_matmul": (ctypes.c_int32, [_P, ctypes.c_int64, _P, _P, ctypes.c_int64, _P, ctypes.c_int32, ctypes.c_int32,
                                        ctypes.c_int32, ctypes.c_int32, _P, ctypes.c_int64, ctypes.c_int32,
                                        ctypes.c_int32, _P, _P]),
    "gpt_fp8_matmul_noalloc": (ctypes.c_int32, [_P, ctypes.c_int64, _P, _P, ctypes.c_int64, _P, ctypes.c_int32,
                                                ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, _P, ctypes.c_int64,
                                                ctypes.c_int32, ctypes.c_int32, _P]),
}


def lib():
    """Loads the built library (raises if it is missing)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built; run decoder_only_transformer_gpt_amd.build.build()")
        # torch ships its own HIP runtime: load it first, so that the
        # library's libamdhip64 dependency resolves to that same runtime (one
        # runtime and one device context per process, whichever module the
        # caller imports first)
        try:
            import torch  # noqa: F401
        except ImportError:
            pass
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGS.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
    return _lib


def status_string(s: int) -> str:
    return lib().gpt_status_string(s).decode()


def _check(status: int, where: str):
    if status != GPT_OK:
        raise GptError(status, where, lib().gpt_last_error_message().decode())


# ------------------------------------------------------------------ host --

def gpt_config_from_depth(depth: int, dtype: int = GPT_BF16) -> gpt_config:
    c = gpt_config()
    _check(lib().gpt_config_from_depth(depth, dtype, ctypes.byref(c)), "gpt_config_from_depth")
    return c


def make_config(**fields) -> gpt_config:
    c = gpt_config()
    for k, v in fields.items():
        setattr(c, k, v)
    return c


def gpt_config_validate(cfg: gpt_config) -> int:
    return lib().gpt_config_validate(ctypes.byref(cfg))


def gpt_param_count(cfg: gpt_config) -> int:
    return lib().gpt_param_count(ctypes.byref(cfg))


def gpt_param_layout(cfg: gpt_config):
    n = ctypes.c_int32(0)
    _check(lib().gpt_param_layout(ctypes.byref(cfg), None, ctypes.byref(n)), "gpt_param_layout")
    arr = (gpt_tensor_desc * n.value)()
    _check(lib().gpt_param_layout(ctypes.byref(cfg), arr, ctypes.byref(n)), "gpt_param_layout")
    return [(d.name.decode(), d.offset, d.rows, d.cols) for d in arr]


def gpt_workspace_bytes(cfg: gpt_config, max_B: int, max_T: int) -> int:
    b = ctypes.c_size_t(0)
    _check(lib().gpt_workspace_bytes(ctypes.byref(cfg), max_B, max_T, ctypes.byref(b)), "gpt_workspace_bytes")
    return b.value


def gpt_kernel_tag_names():
    out, t = [], 0
    while True:
        s = lib().gpt_kernel_tag_name(t)
        if s is None:
            return out
        out.append(s.decode())
        t += 1


# ---------------------------------------------------------------- device --

def gpt_init(cfg: gpt_config, params_ptr: int, grads_ptr: int, ws_ptr: int, ws_bytes: int, max_B: int, max_T: int,
             stream: int):
    h = ctypes.c_void_p()
    _check(lib().gpt_init(ctypes.byref(cfg), params_ptr, grads_ptr, ws_ptr, ws_bytes, max_B, max_T, stream,
                          ctypes.byref(h)), "gpt_init")
    return h


def gpt_forward_loss(h, idx_ptr: int, tgt_ptr: int, B: int, T: int, need_grad: int, loss_ptr: int,
                     row_loss_ptr: int | None, stream: int):
    _check(lib().gpt_forward_loss(h, idx_ptr, tgt_ptr, B, T, need_grad, loss_ptr, row_loss_ptr, stream),
           "gpt_forward_loss")


def gpt_backward(h, dloss: float, accumulate: int, stream: int):
    _check(lib().gpt_backward(h, dloss, accumulate, stream), "gpt_backward")


def gpt_sync_status(h, stream: int) -> int:
    return lib().gpt_sync_status(h, stream)


def gpt_destroy(h):
    _check(lib().gpt_destroy(h), "gpt_destroy")


def gpt_profile_begin(h, tag: int):
    _check(lib().gpt_profile_begin(h, tag), "gpt_profile_begin")


def gpt_profile_end(h):
    ms, n = ctypes.c_double(0), ctypes.c_int64(0)
    _check(lib().gpt_profile_end(h, ctypes.byref(ms), ctypes.byref(n)), "gpt_profile_end")
    return ms.value, n.value


def gpt_set_option(h, option: int, value: int):
    _check(lib().gpt_set_option(h, option, value), "gpt_set_option")


def gpt_debug_buffer(h, name: str, layer: int = 0):
    p, b = ctypes.c_void_p(), ctypes.c_size_t(0)
    _check(lib().gpt_debug_buffer(h, name.encode(), layer, ctypes.byref(p), ctypes.byref(b)), "gpt_debug_buffer")
    return p.value, b.value


def gpt_fp8_quantize(x_ptr: int, rows: int, cols: int, q_ptr, qT_ptr, ldT: int, amax_ptr: int, stream: int):
    _check(lib().gpt_fp8_quantize(x_ptr, rows, cols, q_ptr, qT_ptr, ldT, amax_ptr, stream), "gpt_fp8_quantize")


def gpt_fp8_matmul(a_ptr, lda, amax_a_ptr, b_ptr, ldb, amax_b_ptr, M, N, K, out_dtype, out_ptr, ldo, tile=0,
                   splits=1, partials_ptr=None, stream=0):
    _check(lib().gpt_fp8_matmul(a_ptr, lda, amax_a_ptr, b_ptr, ldb, amax_b_ptr, M, N, K, out_dtype, out_ptr, ldo,
                                tile, splits, partials_ptr, stream), "gpt_fp8_matmul")


def gpt_fp8_matmul_noalloc(a_ptr, lda, amax_a_ptr, b_ptr, ldb, amax_b_ptr, M, N, K, out_dtype, out_ptr, ldo, tile=0,
                           splits=1, stream=0):
    _check(lib().gpt_fp8_matmul_noalloc(a_ptr, lda, amax_a_ptr, b_ptr, ldb, amax_b_ptr, M, N, K, out_dtype, out_ptr,
                                        ldo, tile, splits, stream), "gpt_fp8_matmul_noalloc")


def gpt_optimizer_state_elems(cfg: gpt_config) -> int:
    n = ctypes.c_int64(0)
    _check(lib().gpt_optimizer_state_elems(ctypes.byref(cfg), ctypes.byref(n)), "gpt_optimizer_state_elems")
    return n.value


def gpt_optimizer_step(h, oc: gpt_optim_config, master_ptr: int, state_ptr: int, t: int, stream: int):
    _check(lib().gpt_optimizer_step(h, ctypes.byref(oc), master_ptr, state_ptr, t, stream), "gpt_optimizer_step")
