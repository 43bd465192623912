"""Python binding of librecsa (the RecSA hot path on one MI355X).

Argument marshalling only: every step of tree build, append, descent and the
mixed softmax runs in the HIP kernels behind the C ABI declared in
``include/recsa.h``.  PyTorch supplies device memory and the stream.  There
is no fallback: if the library is not built, importing the binding's entry
points raises.
"""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "librecsa.so")

RECSA_OK, RECSA_ERR_INVALID_ARG, RECSA_ERR_UNSUPPORTED, RECSA_ERR_CAPACITY, RECSA_ERR_HIP = range(5)
RECSA_FP32, RECSA_BF16 = 0, 1
RECSA_PATH_AUTO, RECSA_PATH_ROWWISE, RECSA_PATH_PARENT_MAJOR = 0, 1, 2
PATHS = {"auto": RECSA_PATH_AUTO, "rowwise": RECSA_PATH_ROWWISE, "parent_major": RECSA_PATH_PARENT_MAJOR}

EXPORTED = (
    "recsa_num_levels", "recsa_tree_bytes", "recsa_tree_layout", "recsa_max_candidates",
    "recsa_workspace_bytes", "recsa_build_tree", "recsa_append", "recsa_decode",
    "recsa_prefill", "recsa_status_string", "recsa_last_error", "recsa_multi_workspace_bytes",
    "recsa_decode_multi", "recsa_decode_grouped", "recsa_backward_workspace_bytes",
    "recsa_backward", "recsa_dense_workspace_bytes", "recsa_dense_decode",
    "recsa_distill_workspace_bytes", "recsa_distill_step", "recsa_decode_multi_noalloc",
    "recsa_backward_bf16_workspace_bytes", "recsa_backward_bf16",
)


class recsa_params(ctypes.Structure):
    _fields_ = [
        ("n_kv_heads", ctypes.c_int32), ("n_q_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32), ("fanout_b", ctypes.c_int32),
        ("budget_k", ctypes.c_int32), ("store_dtype", ctypes.c_int32),
        ("out_dtype", ctypes.c_int32), ("path", ctypes.c_int32),
        ("rope_base", ctypes.c_double), ("softmax_scale", ctypes.c_float),
        ("pool_scale", ctypes.c_float), ("capacity", ctypes.c_int64),
    ]


class recsa_tree_desc(ctypes.Structure):
    _fields_ = [
        ("k_cache", ctypes.c_void_p), ("v_cache", ctypes.c_void_p), ("tree", ctypes.c_void_p),
        ("pool_w", ctypes.c_void_p), ("length", ctypes.c_int64),
    ]


class recsa_debug(ctypes.Structure):
    _fields_ = [("selected", ctypes.c_void_p), ("kth_gap", ctypes.c_void_p),
                ("n_keys", ctypes.c_void_p)]


class RecsaError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(message)
        self.status = status


_lib = None


def load_library():
    """dlopen librecsa.so (after torch, so the process keeps one HIP runtime)."""
    global _lib
    if _lib is not None:
        return _lib
    import torch  # noqa: F401  -- loads torch's libamdhip64 first; librecsa binds to it
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built: run `python -m long_context_recsa_amd.build`")
    lib = ctypes.CDLL(LIB_PATH)
    P = ctypes.POINTER(recsa_params)
    D = ctypes.POINTER(recsa_tree_desc)
    G = ctypes.POINTER(recsa_debug)
    v, i64, i32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32
    sig = {
        "recsa_num_levels": (i32, [P]),
        "recsa_tree_bytes": (ctypes.c_size_t, [P]),
        "recsa_tree_layout": (i32, [P, i32, ctypes.POINTER(ctypes.c_size_t),
                                    ctypes.POINTER(ctypes.c_size_t), ctypes.POINTER(i64)]),
        "recsa_max_candidates": (i64, [P]),
        "recsa_workspace_bytes": (ctypes.c_size_t, [P, i64]),
        "recsa_build_tree": (i32, [P, D, i64, v]),
        "recsa_append": (i32, [P, D, v, v, i64, v]),
        "recsa_decode": (i32, [P, D, v, i32, v, G, v, v]),
        "recsa_prefill": (i32, [P, D, v, i64, v, G, v, v]),
        "recsa_status_string": (ctypes.c_char_p, [i32]),
        "recsa_last_error": (ctypes.c_char_p, []),
        "recsa_multi_workspace_bytes": (ctypes.c_size_t, [i32]),
        "recsa_decode_multi": (i32, [P, D, i32, v, v, G, v, v]),
        "recsa_decode_multi_noalloc": (i32, [P, D, i32, v, v, G, v]),
        "recsa_decode_grouped": (i32, [P, D, v, i32, v, G, v, v]),
        "recsa_backward_workspace_bytes": (ctypes.c_size_t, [P, i64]),
        "recsa_backward": (i32, [P, D, v, i64, i32, v, v, v, v, v, G, v, v]),
        "recsa_backward_bf16_workspace_bytes": (ctypes.c_size_t, [P, i64]),
        "recsa_backward_bf16": (i32, [P, D, v, i64, i32, v, v, v, v, v, G, v, v]),
        "recsa_dense_workspace_bytes": (ctypes.c_size_t, [P, i32]),
        "recsa_dense_decode": (i32, [P, D, v, i32, v, v, v]),
        "recsa_distill_workspace_bytes": (ctypes.c_size_t, [P, i32]),
        "recsa_distill_step": (i32, [P, D, v, v, i32, v, ctypes.c_float, ctypes.c_float, v, v, v, v]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def _check(status: int) -> None:
    if status != RECSA_OK:
        lib = load_library()
        raise RecsaError(status, f"{lib.recsa_status_string(status).decode()}: "
                                 f"{lib.recsa_last_error().decode()}")


# ---- the C entry points, same names ------------------------------------------
def recsa_num_levels(p: recsa_params) -> int:
    return load_library().recsa_num_levels(ctypes.byref(p))


def recsa_tree_bytes(p: recsa_params) -> int:
    return load_library().recsa_tree_bytes(ctypes.byref(p))


def recsa_max_candidates(p: recsa_params) -> int:
    return load_library().recsa_max_candidates(ctypes.byref(p))


def recsa_workspace_bytes(p: recsa_params, max_rows: int) -> int:
    return load_library().recsa_workspace_bytes(ctypes.byref(p), max_rows)


def recsa_tree_layout(p: recsa_params, level: int):
    ko, vo, nc = ctypes.c_size_t(), ctypes.c_size_t(), ctypes.c_int64()
    _check(load_library().recsa_tree_layout(ctypes.byref(p), level, ctypes.byref(ko),
                                            ctypes.byref(vo), ctypes.byref(nc)))
    return ko.value, vo.value, nc.value


def recsa_build_tree(p, desc, length, stream=None) -> None:
    _check(load_library().recsa_build_tree(ctypes.byref(p), ctypes.byref(desc), length, stream))


def recsa_append(p, desc, k_new_ptr, v_new_ptr, n_new, stream=None) -> None:
    _check(load_library().recsa_append(ctypes.byref(p), ctypes.byref(desc), k_new_ptr,
                                       v_new_ptr, n_new, stream))


def recsa_decode(p, desc, q_ptr, batch, out_ptr, dbg=None, ws=None, stream=None) -> None:
    _check(load_library().recsa_decode(ctypes.byref(p), ctypes.byref(desc), q_ptr, batch,
                                       out_ptr, ctypes.byref(dbg) if dbg is not None else None,
                                       ws, stream))


def recsa_decode_grouped(p, desc, q_ptr, batch, out_ptr, dbg=None, ws=None, stream=None) -> None:
    _check(load_library().recsa_decode_grouped(ctypes.byref(p), ctypes.byref(desc), q_ptr, batch,
                                               out_ptr, ctypes.byref(dbg) if dbg is not None else None,
                                               ws, stream))


def recsa_prefill(p, desc, q_ptr, n_q, out_ptr, dbg=None, ws=None, stream=None) -> None:
    _check(load_library().recsa_prefill(ctypes.byref(p), ctypes.byref(desc), q_ptr, n_q,
                                        out_ptr, ctypes.byref(dbg) if dbg is not None else None,
                                        ws, stream))


def recsa_backward_workspace_bytes(p, max_rows: int) -> int:
    return load_library().recsa_backward_workspace_bytes(ctypes.byref(p), max_rows)


def recsa_backward(p, desc, q_ptr, n_q, causal, dout_ptr, dq_ptr, dk_ptr, dv_ptr, dw_ptr, dbg=None,
                   ws=None, stream=None) -> None:
    _check(load_library().recsa_backward(ctypes.byref(p), ctypes.byref(desc), q_ptr, n_q, int(causal),
                                         dout_ptr, dq_ptr, dk_ptr, dv_ptr, dw_ptr,
                                         ctypes.byref(dbg) if dbg is not None else None, ws, stream))


def recsa_backward_bf16_workspace_bytes(p, max_rows: int) -> int:
    return load_library().recsa_backward_bf16_workspace_bytes(ctypes.byref(p), max_rows)


def recsa_backward_bf16(p, desc, q_ptr, n_q, causal, dout_ptr, dq_ptr, dk_ptr, dv_ptr, dw_ptr, dbg=None,
                        ws=None, stream=None) -> None:
    _check(load_library().recsa_backward_bf16(ctypes.byref(p), ctypes.byref(desc), q_ptr, n_q, int(causal),
                                              dout_ptr, dq_ptr, dk_ptr, dv_ptr, dw_ptr,
                                              ctypes.byref(dbg) if dbg is not None else None, ws, stream))


def recsa_dense_workspace_bytes(p, batch: int) -> int:
    return load_library().recsa_dense_workspace_bytes(ctypes.byref(p), batch)


def recsa_dense_decode(p, desc, q_ptr, batch, out_ptr, ws, stream=None) -> None:
    _check(load_library().recsa_dense_decode(ctypes.byref(p), ctypes.byref(desc), q_ptr, batch, out_ptr,
                                             ws, stream))


def recsa_distill_workspace_bytes(p, batch: int) -> int:
    return load_library().recsa_distill_workspace_bytes(ctypes.byref(p), batch)


def recsa_distill_step(p, desc, w_ptr, q_ptr, batch, teacher_ptr, lr, momentum, vel_ptr, loss_ptr, ws,
                       stream=None) -> None:
    _check(load_library().recsa_distill_step(ctypes.byref(p), ctypes.byref(desc), w_ptr, q_ptr, batch,
                                             teacher_ptr, lr, momentum, vel_ptr, loss_ptr, ws, stream))


def recsa_multi_workspace_bytes(n_seq: int) -> int:
    return load_library().recsa_multi_workspace_bytes(n_seq)


def recsa_decode_multi(p, descs, n_seq, q_ptr, out_ptr, dbg=None, ws=None, stream=None) -> None:
    """descs: a ctypes array of n_seq recsa_tree_desc."""
    _check(load_library().recsa_decode_multi(ctypes.byref(p), descs, n_seq, q_ptr, out_ptr,
                                             ctypes.byref(dbg) if dbg is not None else None,
                                             ws, stream))


def recsa_decode_multi_noalloc(p, descs, n_seq, q_ptr, out_ptr, dbg=None, stream=None) -> None:
    """As recsa_decode_multi, with the sequence table in the library's fixed device table
    (no workspace; at most 4096 sequences)."""
    _check(load_library().recsa_decode_multi_noalloc(ctypes.byref(p), descs, n_seq, q_ptr, out_ptr,
                                                     ctypes.byref(dbg) if dbg is not None else None,
                                                     stream))


def make_params(n_kv_heads, n_q_heads, head_dim, fanout_b, budget_k, capacity,
                store="bf16", out="f32", rope_base=1e6, softmax_scale=None,
                pool_scale=None, path="auto") -> recsa_params:
    """path: "auto", "rowwise" or "parent_major" (recsa_path: the layout of prefill and
    backward work)."""
    dt = {"f32": RECSA_FP32, "bf16": RECSA_BF16}
    s = 1.0 / head_dim ** 0.5
    return recsa_params(n_kv_heads, n_q_heads, head_dim, fanout_b, budget_k, dt[store], dt[out],
                        PATHS[path], rope_base, s if softmax_scale is None else softmax_scale,
                        s if pool_scale is None else pool_scale, capacity)


from .layer import RecsaLayer  # noqa: E402,F401
