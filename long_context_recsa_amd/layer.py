"""Owner of one attention layer's RecSA state in device memory (torch tensors)
and thin wrappers of the C calls.  Marshalling only: no arithmetic here."""
from __future__ import annotations

import ctypes

import torch

from . import (PATHS, RECSA_BF16, recsa_append, recsa_backward, recsa_backward_bf16,
               recsa_backward_bf16_workspace_bytes, recsa_backward_workspace_bytes,
               recsa_build_tree, recsa_dense_decode, recsa_dense_workspace_bytes, recsa_distill_step,
               recsa_distill_workspace_bytes, recsa_debug, recsa_decode, recsa_decode_grouped, recsa_decode_multi, recsa_decode_multi_noalloc, recsa_max_candidates, recsa_multi_workspace_bytes,
               recsa_num_levels, recsa_params, recsa_prefill, recsa_tree_bytes, recsa_tree_desc,
               recsa_tree_layout, recsa_workspace_bytes)


def _ptr(t: torch.Tensor | None):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


class RecsaLayer:
    """K/V cache, tree buffer and pooler vectors of one layer on one GPU."""

    def __init__(self, params: recsa_params, device: str | torch.device = "cuda"):
        self.p = params
        self.device = torch.device(device)
        if self.device.type == "cuda" and self.device.index is None:
            self.device = torch.device("cuda", torch.cuda.current_device())
        self.store = torch.bfloat16 if params.store_dtype == RECSA_BF16 else torch.float32
        self.out_dtype = torch.bfloat16 if params.out_dtype == RECSA_BF16 else torch.float32
        Hkv, D, cap = params.n_kv_heads, params.head_dim, params.capacity
        nbytes = recsa_tree_bytes(params)
        if nbytes == 0:
            raise ValueError("invalid recsa_params")
        self.k_cache = torch.zeros((Hkv, cap, D), dtype=self.store, device=self.device)
        self.v_cache = torch.zeros((Hkv, cap, D), dtype=self.store, device=self.device)
        self.tree = torch.zeros(nbytes, dtype=torch.uint8, device=self.device)
        self.pool_w = torch.zeros((Hkv, D), dtype=torch.float32, device=self.device)
        self.n_levels = recsa_num_levels(params)
        self.max_candidates = recsa_max_candidates(params)
        self.desc = recsa_tree_desc(self.k_cache.data_ptr(), self.v_cache.data_ptr(),
                                    self.tree.data_ptr(), self.pool_w.data_ptr(), 0)
        self._ws = None
        self._bws = None

    def workspace(self, rows: int):
        """Device scratch for a call over `rows` rows, as the library sizes it (kept and
        grown across calls; None when the call needs none)."""
        nbytes = recsa_workspace_bytes(self.p, rows)
        if nbytes == 0:
            return None
        if self._ws is None or self._ws.numel() < nbytes:
            self._ws = None
            self._ws = torch.empty(nbytes, dtype=torch.uint8, device=self.device)
        return _ptr(self._ws)

    def set_path(self, path: str) -> None:
        """Layout of prefill and backward work: "auto", "rowwise" or "parent_major"
        (the recsa_params.path field; sizing and running calls read the same field)."""
        self.p.path = PATHS[path]

    @property
    def length(self) -> int:
        return int(self.desc.length)

    @staticmethod
    def stream():
        return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)

    def _check_dev(self, t: torch.Tensor, shape, dtype):
        if t.device != self.device or not t.is_contiguous() or t.dtype != dtype or tuple(t.shape) != tuple(shape):
            raise ValueError(f"expected contiguous {dtype} {tuple(shape)} on {self.device}, got "
                             f"{t.dtype} {tuple(t.shape)} on {t.device}")

    # ---- calls ----------------------------------------------------------------
    def build(self, length: int) -> None:
        recsa_build_tree(self.p, self.desc, length, self.stream())

    def append(self, k_new: torch.Tensor, v_new: torch.Tensor) -> None:
        n = k_new.shape[0]
        shape = (n, self.p.n_kv_heads, self.p.head_dim)
        self._check_dev(k_new, shape, self.store)
        self._check_dev(v_new, shape, self.store)
        recsa_append(self.p, self.desc, _ptr(k_new), _ptr(v_new), n, self.stream())

    def _debug(self, rows: int, debug: bool):
        if not debug:
            return None, None
        d = {
            "selected": torch.full((rows, self.n_levels, self.p.budget_k), -7, dtype=torch.int32,
                                   device=self.device),
            "kth_gap": torch.zeros((rows, self.n_levels), dtype=torch.float32, device=self.device),
            "n_keys": torch.zeros((rows,), dtype=torch.int32, device=self.device),
        }
        return d, recsa_debug(d["selected"].data_ptr(), d["kth_gap"].data_ptr(),
                              d["n_keys"].data_ptr())

    def decode(self, q: torch.Tensor, debug: bool = False, out: torch.Tensor | None = None):
        B = q.shape[0]
        shape = (B, self.p.n_q_heads, self.p.head_dim)
        self._check_dev(q, shape, self.store)
        if out is None:
            out = torch.empty(shape, dtype=self.out_dtype, device=self.device)
        d, dbg = self._debug(B * self.p.n_q_heads, debug)
        recsa_decode(self.p, self.desc, _ptr(q), B, _ptr(out), dbg, None, self.stream())
        return (out, d) if debug else out

    def decode_grouped(self, q: torch.Tensor, debug: bool = False, out: torch.Tensor | None = None):
        """Decode with one selection per (query, KV group); debug rows are i * n_kv + g."""
        B = q.shape[0]
        shape = (B, self.p.n_q_heads, self.p.head_dim)
        self._check_dev(q, shape, self.store)
        if out is None:
            out = torch.empty(shape, dtype=self.out_dtype, device=self.device)
        d, dbg = self._debug(B * self.p.n_kv_heads, debug)
        recsa_decode_grouped(self.p, self.desc, _ptr(q), B, _ptr(out), dbg, None, self.stream())
        return (out, d) if debug else out

    def prefill(self, q: torch.Tensor, debug: bool = False, out: torch.Tensor | None = None):
        n = q.shape[0]
        shape = (n, self.p.n_q_heads, self.p.head_dim)
        self._check_dev(q, shape, self.store)
        if out is None:
            out = torch.empty(shape, dtype=self.out_dtype, device=self.device)
        d, dbg = self._debug(n * self.p.n_q_heads, debug)
        ws = self.workspace(n * self.p.n_q_heads)
        recsa_prefill(self.p, self.desc, _ptr(q), n, _ptr(out), dbg, ws, self.stream())
        return (out, d) if debug else out

    def backward(self, q: torch.Tensor, dout: torch.Tensor, causal: bool = False, debug: bool = False,
                 grads: dict | None = None, grad_dtype: str = "f32"):
        """Gradients of <dout, out> with the selection held fixed, for the rows of
        decode(q) (causal=False) or prefill(q) (causal=True).  Returns a dict with
        dq [n][Hq][D] and dk, dv [Hkv][capacity][D], dw [Hkv][D] (fp32; dk and dv in
        bf16 with grad_dtype="bf16", through recsa_backward_bf16); pass `grads` (such a
        dict) to have dk, dv, dw written into existing tensors (dk, dv rows from the
        cache's length on are left as they are)."""
        if grad_dtype not in ("f32", "bf16"):
            raise ValueError(f"grad_dtype must be 'f32' or 'bf16', not {grad_dtype!r}")
        n = q.shape[0]
        shape = (n, self.p.n_q_heads, self.p.head_dim)
        self._check_dev(q, shape, self.store)
        self._check_dev(dout, shape, torch.float32)
        Hkv, D, cap = self.p.n_kv_heads, self.p.head_dim, self.p.capacity
        tdt = torch.bfloat16 if grad_dtype == "bf16" else torch.float32
        if grads is None:
            grads = {"dk": torch.zeros((Hkv, cap, D), dtype=tdt, device=self.device),
                     "dv": torch.zeros((Hkv, cap, D), dtype=tdt, device=self.device),
                     "dw": torch.zeros((Hkv, D), dtype=torch.float32, device=self.device)}
        for name in ("dk", "dv"):
            self._check_dev(grads[name], (Hkv, cap, D), tdt)
        self._check_dev(grads["dw"], (Hkv, D), torch.float32)
        grads["dq"] = torch.empty(shape, dtype=torch.float32, device=self.device)
        rows = n * self.p.n_q_heads
        sizing = recsa_backward_bf16_workspace_bytes if grad_dtype == "bf16" else recsa_backward_workspace_bytes
        call = recsa_backward_bf16 if grad_dtype == "bf16" else recsa_backward
        nbytes = sizing(self.p, rows)
        if nbytes and (self._bws is None or self._bws.numel() < nbytes):
            self._bws = None
            self._bws = torch.empty(nbytes, dtype=torch.uint8, device=self.device)
        d, dbg = self._debug(rows, debug)
        call(self.p, self.desc, _ptr(q), n, causal, _ptr(dout), _ptr(grads["dq"]),
             _ptr(grads["dk"]), _ptr(grads["dv"]), _ptr(grads["dw"]), dbg,
             _ptr(self._bws) if nbytes else None, self.stream())
        return (grads, d) if debug else grads

    def dense_decode(self, q: torch.Tensor, out: torch.Tensor | None = None):
        """Dense causal attention of decode queries at the cache's length (no tree)."""
        B = q.shape[0]
        shape = (B, self.p.n_q_heads, self.p.head_dim)
        self._check_dev(q, shape, self.store)
        if out is None:
            out = torch.empty(shape, dtype=self.out_dtype, device=self.device)
        ws = torch.empty(recsa_dense_workspace_bytes(self.p, B), dtype=torch.uint8, device=self.device)
        recsa_dense_decode(self.p, self.desc, _ptr(q), B, _ptr(out), _ptr(ws), self.stream())
        return out

    def distill_step(self, q: torch.Tensor, teacher: torch.Tensor, lr: float, momentum: float,
                     velocity: torch.Tensor, loss: torch.Tensor, ws: torch.Tensor | None = None):
        """One pooler distillation step (updates pool_w and velocity, rebuilds the tree);
        the loss before the step goes to `loss` (one fp32 element on the device)."""
        B = q.shape[0]
        shape = (B, self.p.n_q_heads, self.p.head_dim)
        self._check_dev(q, shape, self.store)
        self._check_dev(teacher, shape, torch.float32)
        self._check_dev(velocity, (self.p.n_kv_heads, self.p.head_dim), torch.float32)
        if ws is None:
            ws = torch.empty(recsa_distill_workspace_bytes(self.p, B), dtype=torch.uint8, device=self.device)
        recsa_distill_step(self.p, self.desc, _ptr(self.pool_w), _ptr(q), B, _ptr(teacher), lr, momentum,
                           _ptr(velocity), _ptr(loss), _ptr(ws), self.stream())
        return loss

    # ---- inspection -------------------------------------------------------------
    def level(self, l: int):
        """(keys, values) of level l as views [n_kv][node_capacity][head_dim] of the tree."""
        ko, vo, nc = recsa_tree_layout(self.p, l)
        esz = 2 if self.store == torch.bfloat16 else 4
        n = self.p.n_kv_heads * nc * self.p.head_dim
        shape = (self.p.n_kv_heads, nc, self.p.head_dim)
        keys = self.tree[ko:ko + n * esz].view(self.store).view(shape)
        vals = self.tree[vo:vo + n * esz].view(self.store).view(shape)
        return keys, vals


def decode_multi(layers, q: torch.Tensor, debug: bool = False, out: torch.Tensor | None = None,
                 ws: torch.Tensor | None = None, noalloc: bool = False):
    """One decode step for a batch of sequences: layers[i] (same params, own cache and
    tree) answers query q[i] at its own length.  q: [n][n_q_heads][head_dim].
    noalloc: call recsa_decode_multi_noalloc (no workspace; pass `out`, and no debug,
    for a call that allocates nothing)."""
    first = layers[0]
    n = len(layers)
    # the kernel addresses every sequence's cache and tree with the first one's layout
    key = [f for f, _ in recsa_params._fields_ if f != "path"]
    for i, l in enumerate(layers[1:], 1):
        if l.device != first.device or any(getattr(l.p, f) != getattr(first.p, f) for f in key):
            raise ValueError(f"decode_multi: layer {i} differs from layer 0 in its params or device; "
                             "every sequence must share one layout")
    shape = (n, first.p.n_q_heads, first.p.head_dim)
    first._check_dev(q, shape, first.store)
    if out is None:
        out = torch.empty(shape, dtype=first.out_dtype, device=first.device)
    descs = (recsa_tree_desc * n)(*[l.desc for l in layers])
    if noalloc:
        d, dbg = first._debug(n * first.p.n_q_heads, debug)
        recsa_decode_multi_noalloc(first.p, descs, n, _ptr(q), _ptr(out), dbg, first.stream())
        return (out, d) if debug else out
    nbytes = recsa_multi_workspace_bytes(n)
    if nbytes and (ws is None or ws.numel() < nbytes):
        ws = torch.empty(nbytes, dtype=torch.uint8, device=first.device)
    d, dbg = first._debug(n * first.p.n_q_heads, debug)
    recsa_decode_multi(first.p, descs, n, _ptr(q), _ptr(out), dbg, _ptr(ws) if nbytes else None,
                       first.stream())
    return (out, d) if debug else out
