"""ctypes binding of libmoe_sel.so: the C ABI of include/moe_sel.h, same names.

Argument marshalling only. Host arrays are NumPy arrays; device arrays are any
object with ``data_ptr()`` (torch tensors on the GPU) or a raw integer address.
Streams are ``hipStream_t`` handles as integers (``torch.cuda.current_stream()
.cuda_stream``); ``None`` means the current torch stream when torch is on a GPU,
else the default stream.

The library must have been built (``python -m activation_sparse_expert_amd.build``);
importing this module without it raises immediately: there is no fallback.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libmoe_sel.so")

MOE_SEL_OK, MOE_SEL_EINVAL, MOE_SEL_EUNSUPPORTED, MOE_SEL_ENOMEM, MOE_SEL_EDEVICE, MOE_SEL_EIO = range(6)

EXPORTED = (
    "moe_sel_abi_version", "moe_sel_status_str", "moe_sel_last_error",
    "moe_sel_prepare_expert_host", "moe_sel_prepare", "moe_sel_forward",
    "moe_sel_forward_dense", "moe_sel_forward_threshold", "moe_sel_debug_selection", "moe_sel_export_expert",
    "moe_sel_get_config", "moe_sel_device_bytes", "moe_sel_destroy", "moe_sel_check_device",
    "moe_sel_set_path", "moe_sel_last_path", "moe_sel_set_score", "moe_sel_router_logits", "moe_sel_residual_rmsnorm",
    "moe_sel_residual_rmsnorm_router", "moe_sel_save", "moe_sel_load", "moe_sel_set_wait_limit",
    "moe_sel_debug_silu", "moe_sel_debug_score", "moe_sel_read_stream", "moe_sel_debug_fail_alloc",
    "moe_sel_forward_noalloc",
)

MOE_SEL_PATH_AUTO, MOE_SEL_PATH_MULTI_KERNEL, MOE_SEL_PATH_SINGLE_LAUNCH = range(3)
MOE_SEL_SCORE_FULL, MOE_SEL_SCORE_GATE_ONLY, MOE_SEL_SCORE_NO_DOWN_NORM, MOE_SEL_SCORE_X_INT16 = range(4)


class moe_sel_config(ctypes.Structure):
    _fields_ = [
        ("struct_size", ctypes.c_uint32),
        ("d", ctypes.c_int32),
        ("n_experts", ctypes.c_int32),
        ("m", ctypes.c_int32),
        ("rank", ctypes.c_int32),
        ("max_top_e", ctypes.c_int32),
        ("max_batch", ctypes.c_int32),
        ("tern_ratio", ctypes.c_double),
    ]


class MoeSelError(RuntimeError):
    def __init__(self, status: int, func: str, detail: str):
        super().__init__(f"{func}: {_status_name(status)} ({status}): {detail}")
        self.status = status


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with `python -m activation_sparse_expert_amd.build`")
    # One HIP runtime per process: torch ships its own libamdhip64 (same soname).
    # Loading torch first makes the library bind to that runtime, so torch's
    # device pointers and stream handles are valid inside the library.
    try:
        import torch  # noqa: F401
    except ImportError:
        pass
    lib = ctypes.CDLL(LIB_PATH)
    vp, i32, f32p = ctypes.c_void_p, ctypes.c_int32, ctypes.c_void_p
    sig = {
        "moe_sel_abi_version": (i32, []),
        "moe_sel_status_str": (ctypes.c_char_p, [ctypes.c_int]),
        "moe_sel_last_error": (ctypes.c_char_p, []),
        "moe_sel_prepare_expert_host": (ctypes.c_int, [ctypes.POINTER(moe_sel_config), vp, vp, vp,
                                                       vp, vp, f32p, f32p, f32p, vp, vp, vp, vp]),
        "moe_sel_prepare": (ctypes.c_int, [ctypes.POINTER(moe_sel_config), vp, vp, vp, vp,
                                           ctypes.POINTER(vp)]),
        "moe_sel_forward": (ctypes.c_int, [vp, vp, vp, i32, i32, i32, vp, vp]),
        "moe_sel_forward_noalloc": (ctypes.c_int, [vp, vp, vp, i32, i32, i32, vp, vp]),
        "moe_sel_forward_dense": (ctypes.c_int, [vp, vp, vp, i32, i32, vp, vp]),
        "moe_sel_forward_threshold": (ctypes.c_int, [vp, vp, vp, i32, i32, ctypes.c_float, vp, vp]),
        "moe_sel_debug_selection": (ctypes.c_int, [vp, vp, vp, vp, vp, vp, vp]),
        "moe_sel_export_expert": (ctypes.c_int, [vp, i32, vp, vp, vp, vp, vp, vp, vp, vp, vp]),
        "moe_sel_get_config": (ctypes.c_int, [vp, ctypes.POINTER(moe_sel_config)]),
        "moe_sel_device_bytes": (ctypes.c_uint64, [vp]),
        "moe_sel_destroy": (None, [vp]),
        "moe_sel_check_device": (ctypes.c_int, [vp]),
        "moe_sel_set_path": (ctypes.c_int, [vp, ctypes.c_int]),
        "moe_sel_last_path": (i32, [vp]),
        "moe_sel_set_score": (ctypes.c_int, [vp, ctypes.c_int]),
        "moe_sel_router_logits": (ctypes.c_int, [vp, vp, i32, i32, i32, vp, vp]),
        "moe_sel_residual_rmsnorm": (ctypes.c_int, [vp, vp, i32, i32, ctypes.c_float, vp, vp]),
        "moe_sel_residual_rmsnorm_router": (ctypes.c_int, [vp, vp, vp, i32, i32, i32, ctypes.c_float, vp, vp, vp]),
        "moe_sel_save": (ctypes.c_int, [vp, ctypes.c_char_p]),
        "moe_sel_load": (ctypes.c_int, [ctypes.c_char_p, vp, ctypes.POINTER(vp)]),
        "moe_sel_set_wait_limit": (ctypes.c_int, [vp, i32]),
        "moe_sel_debug_silu": (ctypes.c_int, [vp, vp, ctypes.c_int64, vp]),
        "moe_sel_debug_score": (ctypes.c_int, [vp, vp, vp, vp, ctypes.c_int, vp, vp, ctypes.c_int64, vp]),
        "moe_sel_read_stream": (ctypes.c_int, [vp, ctypes.c_uint64, vp, vp]),
        "moe_sel_debug_fail_alloc": (ctypes.c_int, [i32]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    return lib


_lib = _load()


def _status_name(status: int) -> str:
    return _lib.moe_sel_status_str(int(status)).decode()


def _check(status: int, func: str):
    if status != MOE_SEL_OK:
        raise MoeSelError(status, func, _lib.moe_sel_last_error().decode())


def _host_ptr(a, dtype):
    if a is None:
        return None
    assert isinstance(a, np.ndarray) and a.dtype == dtype and a.flags.c_contiguous, (a.dtype, dtype)
    return a.ctypes.data


def _dev_ptr(a):
    if a is None:
        return None
    if isinstance(a, int):
        return a
    return a.data_ptr()


def _stream(stream):
    if stream is not None:
        return int(stream)
    try:
        import torch
        if torch.cuda.is_available():
            return torch.cuda.current_stream().cuda_stream
    except ImportError:
        pass
    return None


def make_config(d, n_experts, m, rank, max_top_e, max_batch=1, tern_ratio=0.7) -> moe_sel_config:
    return moe_sel_config(ctypes.sizeof(moe_sel_config), d, n_experts, m, rank, max_top_e, max_batch,
                          float(tern_ratio))


def moe_sel_abi_version() -> int:
    return _lib.moe_sel_abi_version()


def moe_sel_prepare_expert_host(cfg: moe_sel_config, w_gate, w_up, w_down, *, sketch=True, lowrank=True):
    """Host-only preparation of one expert; returns a dict of NumPy arrays."""
    m, d, r = cfg.m, cfg.d, cfg.rank
    out = dict(alpha_gate=np.zeros(m, np.float32), alpha_up=np.zeros(m, np.float32),
               down_norm=np.zeros(m, np.float32), nnz_gate=np.zeros(m, np.int32), nnz_up=np.zeros(m, np.int32))
    if sketch:
        out["tern_gate"] = np.zeros((m, d), np.int8)
        out["tern_up"] = np.zeros((m, d), np.int8)
    if lowrank and r > 0:
        out["p_bf16"] = np.zeros((r, d), np.uint16)
        out["q_bf16"] = np.zeros((m, r), np.uint16)
    st = _lib.moe_sel_prepare_expert_host(
        ctypes.byref(cfg), _host_ptr(w_gate, np.uint16), _host_ptr(w_up, np.uint16), _host_ptr(w_down, np.uint16),
        _host_ptr(out.get("tern_gate"), np.int8), _host_ptr(out.get("tern_up"), np.int8),
        _host_ptr(out["alpha_gate"], np.float32), _host_ptr(out["alpha_up"], np.float32),
        _host_ptr(out["down_norm"], np.float32), _host_ptr(out["nnz_gate"], np.int32),
        _host_ptr(out["nnz_up"], np.int32), _host_ptr(out.get("p_bf16"), np.uint16),
        _host_ptr(out.get("q_bf16"), np.uint16))
    _check(st, "moe_sel_prepare_expert_host")
    return out


def moe_sel_prepare(cfg: moe_sel_config, w_gate, w_up, w_down, stream=None) -> int:
    """Build a context from host bf16 weights [E][m][d], [E][m][d], [E][d][m]; returns its handle."""
    ctx = ctypes.c_void_p()
    st = _lib.moe_sel_prepare(ctypes.byref(cfg), _host_ptr(w_gate, np.uint16), _host_ptr(w_up, np.uint16),
                              _host_ptr(w_down, np.uint16), _stream(stream), ctypes.byref(ctx))
    _check(st, "moe_sel_prepare")
    return ctx.value


def moe_sel_save(ctx, path):
    """Write the prepared layer of ctx to path."""
    _check(_lib.moe_sel_save(ctx, os.fsencode(path)), "moe_sel_save")


def moe_sel_load(path, stream=None) -> int:
    """Build a context from a file written by moe_sel_save; returns its handle."""
    ctx = ctypes.c_void_p()
    _check(_lib.moe_sel_load(os.fsencode(path), _stream(stream), ctypes.byref(ctx)), "moe_sel_load")
    return ctx.value


def moe_sel_forward(ctx, x, logits, batch, top_e, k_budget, out, stream=None):
    st = _lib.moe_sel_forward(ctx, _dev_ptr(x), _dev_ptr(logits), int(batch), int(top_e), int(k_budget),
                              _dev_ptr(out), _stream(stream))
    _check(st, "moe_sel_forward")


def moe_sel_forward_noalloc(ctx, x, logits, batch, top_e, k_budget, out, stream=None):
    st = _lib.moe_sel_forward_noalloc(ctx, _dev_ptr(x), _dev_ptr(logits), int(batch), int(top_e), int(k_budget),
                                      _dev_ptr(out), _stream(stream))
    _check(st, "moe_sel_forward_noalloc")


def moe_sel_forward_threshold(ctx, x, logits, batch, top_e, threshold, out, stream=None):
    _check(_lib.moe_sel_forward_threshold(ctx, _dev_ptr(x), _dev_ptr(logits), int(batch), int(top_e),
                                          float(threshold), _dev_ptr(out), _stream(stream)),
           "moe_sel_forward_threshold")


def moe_sel_forward_dense(ctx, x, logits, batch, top_e, out, stream=None):
    st = _lib.moe_sel_forward_dense(ctx, _dev_ptr(x), _dev_ptr(logits), int(batch), int(top_e), _dev_ptr(out),
                                    _stream(stream))
    _check(st, "moe_sel_forward_dense")


def moe_sel_debug_selection(ctx, batch, top_e, k, m, with_scores=True):
    out = dict(expert_ids=np.zeros((batch, top_e), np.int32), gate_w=np.zeros((batch, top_e), np.float32),
               chan_idx=np.zeros((batch, top_e, k), np.int32), chan_count=np.zeros((batch, top_e), np.int32))
    if with_scores:
        out["h_hat"] = np.zeros((batch, top_e, m), np.float32)
        out["score"] = np.zeros((batch, top_e, m), np.float32)
    st = _lib.moe_sel_debug_selection(ctx, out["expert_ids"].ctypes.data, out["gate_w"].ctypes.data,
                                      out["chan_idx"].ctypes.data, out["chan_count"].ctypes.data,
                                      _host_ptr(out.get("h_hat"), np.float32), _host_ptr(out.get("score"), np.float32))
    _check(st, "moe_sel_debug_selection")
    return out


def moe_sel_export_expert(ctx, expert, cfg: moe_sel_config):
    m, d, r = cfg.m, cfg.d, cfg.rank
    out = dict(tern_gate=np.zeros((m, d), np.int8), tern_up=np.zeros((m, d), np.int8),
               alpha_gate=np.zeros(m, np.float32), alpha_up=np.zeros(m, np.float32),
               down_norm=np.zeros(m, np.float32), nnz_gate=np.zeros(m, np.int32), nnz_up=np.zeros(m, np.int32))
    if r > 0:
        out["p_bf16"] = np.zeros((r, d), np.uint16)
        out["q_bf16"] = np.zeros((m, r), np.uint16)
    st = _lib.moe_sel_export_expert(ctx, int(expert), out["tern_gate"].ctypes.data, out["tern_up"].ctypes.data,
                                    out["alpha_gate"].ctypes.data, out["alpha_up"].ctypes.data,
                                    out["down_norm"].ctypes.data, out["nnz_gate"].ctypes.data,
                                    out["nnz_up"].ctypes.data, _host_ptr(out.get("p_bf16"), np.uint16),
                                    _host_ptr(out.get("q_bf16"), np.uint16))
    _check(st, "moe_sel_export_expert")
    return out


def moe_sel_get_config(ctx) -> moe_sel_config:
    cfg = moe_sel_config()
    _check(_lib.moe_sel_get_config(ctx, ctypes.byref(cfg)), "moe_sel_get_config")
    return cfg


def moe_sel_device_bytes(ctx) -> int:
    return int(_lib.moe_sel_device_bytes(ctx))


def moe_sel_check_device(ctx):
    _check(_lib.moe_sel_check_device(ctx), "moe_sel_check_device")


def moe_sel_set_wait_limit(ctx, polls: int):
    _check(_lib.moe_sel_set_wait_limit(ctx, int(polls)), "moe_sel_set_wait_limit")


def moe_sel_debug_silu(z, out, n, stream=None):
    """out[i] = the pinned binary32 silu of z[i] (device fp32 arrays)."""
    _check(_lib.moe_sel_debug_silu(_dev_ptr(z), _dev_ptr(out), int(n), _stream(stream)), "moe_sel_debug_silu")


def moe_sel_debug_score(dot_gate, dot_up, xexp, stats, kind, h_hat, score, n, stream=None):
    """Pinned score of n channels from their integer sketch dots (device arrays)."""
    _check(_lib.moe_sel_debug_score(_dev_ptr(dot_gate), _dev_ptr(dot_up), _dev_ptr(xexp), _dev_ptr(stats), int(kind),
                                    _dev_ptr(h_hat), _dev_ptr(score), int(n), _stream(stream)), "moe_sel_debug_score")


def moe_sel_read_stream(buf, nbytes, sink, stream=None):
    """Read every byte of a device buffer once (the measured read ceiling)."""
    _check(_lib.moe_sel_read_stream(_dev_ptr(buf), int(nbytes), _dev_ptr(sink), _stream(stream)),
           "moe_sel_read_stream")


def moe_sel_debug_fail_alloc(nth: int):
    """Make the nth allocation the library attempts from now on fail (0 disarms)."""
    _check(_lib.moe_sel_debug_fail_alloc(int(nth)), "moe_sel_debug_fail_alloc")


def moe_sel_set_path(ctx, path: int):
    _check(_lib.moe_sel_set_path(ctx, int(path)), "moe_sel_set_path")


def moe_sel_set_score(ctx, kind: int):
    _check(_lib.moe_sel_set_score(ctx, int(kind)), "moe_sel_set_score")


def moe_sel_last_path(ctx) -> int:
    return int(_lib.moe_sel_last_path(ctx))


def moe_sel_destroy(ctx):
    _lib.moe_sel_destroy(ctx)


def moe_sel_status_str(status: int) -> str:
    return _status_name(status)


def moe_sel_last_error() -> str:
    return _lib.moe_sel_last_error().decode()


def moe_sel_router_logits(x, w_router, batch, d, n_experts, logits, stream=None):
    _check(_lib.moe_sel_router_logits(_dev_ptr(x), _dev_ptr(w_router), int(batch), int(d), int(n_experts),
                                      _dev_ptr(logits), _stream(stream)), "moe_sel_router_logits")


def moe_sel_residual_rmsnorm(x, y, batch, d, eps, out, stream=None):
    _check(_lib.moe_sel_residual_rmsnorm(_dev_ptr(x), _dev_ptr(y), int(batch), int(d), float(eps),
                                         _dev_ptr(out), _stream(stream)), "moe_sel_residual_rmsnorm")


def moe_sel_residual_rmsnorm_router(x, y, w_router, batch, d, n_experts, eps, x_out, logits, stream=None):
    _check(_lib.moe_sel_residual_rmsnorm_router(_dev_ptr(x), _dev_ptr(y), _dev_ptr(w_router), int(batch), int(d),
                                                int(n_experts), float(eps), _dev_ptr(x_out), _dev_ptr(logits),
                                                _stream(stream)), "moe_sel_residual_rmsnorm_router")
