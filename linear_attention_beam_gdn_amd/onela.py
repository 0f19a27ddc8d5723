"""Thin ctypes binding of libonela.so (the C ABI declared in include/onela.h).

Argument marshalling only: torch tensors supply device memory and the HIP
stream, every step of the decode path runs in the library's kernels. If the
library is missing this module raises; there is no fallback.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libonela.so")

ONELA_OK = 0
STATUS_NAMES = {
    0: "ONELA_OK",
    -1: "ONELA_E_INVALID_ARG",
    -2: "ONELA_E_BAD_STATE",
    -3: "ONELA_E_CAPACITY",
    -4: "ONELA_E_PARENT_RANGE",
    -5: "ONELA_E_HIP",
    -6: "ONELA_E_OOM",
    -7: "ONELA_E_UNSUPPORTED",
}
EXPORTED = (
    "onela_create", "onela_destroy", "onela_init_request", "onela_step", "onela_reset",
    "onela_sync", "onela_set_beams_per_block", "onela_get_step", "onela_get_ancestry",
    "onela_get_records", "onela_get_memory", "onela_status_string", "onela_last_error",
    "onela_fs_create", "onela_fs_destroy", "onela_fs_init_request", "onela_fs_step", "onela_fs_reset",
    "onela_fs_sync", "onela_fs_get_memory",
    "onela_rs_create", "onela_rs_destroy", "onela_rs_init_request", "onela_rs_step", "onela_rs_reset",
    "onela_rs_sync", "onela_rs_get_memory",
    "onela_init_requests_from_prompts", "onela_prefill", "onela_create_sharing_index", "onela_set_graph_mode",
    "onela_step_raw", "onela_set_beam_order",
)


class OnelaError(RuntimeError):
    def __init__(self, status: int, where: str, detail: str = ""):
        self.status = status
        name = STATUS_NAMES.get(status, str(status))
        super().__init__(f"{where}: {name}" + (f" ({detail})" if detail else ""))


class _Config(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in
                ("max_requests", "num_heads", "d_k", "d_v", "beam_width", "max_steps")]


class _Gates(ctypes.Structure):
    _fields_ = [("A_log", ctypes.c_void_p), ("dt_bias", ctypes.c_void_p), ("norm_eps", ctypes.c_float)]


_lib = None


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libonela.so once; raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise ImportError(f"{path} is missing: build it with `python -m linear_attention_beam_gdn_amd.build`")
    lib = ctypes.CDLL(path)
    vp, i32, p_i32 = ctypes.c_void_p, ctypes.c_int32, ctypes.POINTER(ctypes.c_int32)
    sigs = {
        "onela_create": (i32, [ctypes.POINTER(_Config), vp, ctypes.POINTER(vp)]),
        "onela_destroy": (i32, [vp]),
        "onela_init_request": (i32, [vp, i32, vp]),
        "onela_step": (i32, [vp, i32, p_i32, vp, vp, vp, vp, vp, vp, vp, vp]),
        "onela_reset": (i32, [vp, i32]),
        "onela_sync": (i32, [vp]),
        "onela_set_beams_per_block": (i32, [vp, i32]),
        "onela_set_beam_order": (i32, [vp, i32]),
        "onela_get_step": (i32, [vp, i32, p_i32]),
        "onela_get_ancestry": (i32, [vp, i32, vp]),
        "onela_get_records": (i32, [vp, i32, i32, i32, vp, vp, vp]),
        "onela_get_memory": (i32, [vp, vp, vp, vp]),
        "onela_status_string": (ctypes.c_char_p, [i32]),
        "onela_fs_create": (i32, [ctypes.POINTER(_Config), vp, ctypes.POINTER(vp)]),
        "onela_fs_destroy": (i32, [vp]),
        "onela_fs_init_request": (i32, [vp, i32, vp]),
        "onela_fs_step": (i32, [vp, i32, p_i32, vp, vp, vp, vp, vp, vp, vp, vp]),
        "onela_fs_reset": (i32, [vp, i32]),
        "onela_fs_sync": (i32, [vp]),
        "onela_fs_get_memory": (i32, [vp, vp]),
        "onela_rs_create": (i32, [ctypes.POINTER(_Config), vp, ctypes.POINTER(vp)]),
        "onela_rs_destroy": (i32, [vp]),
        "onela_rs_init_request": (i32, [vp, i32, vp]),
        "onela_rs_step": (i32, [vp, i32, p_i32, vp, vp, vp, vp, vp, vp, vp, vp]),
        "onela_rs_reset": (i32, [vp, i32]),
        "onela_rs_sync": (i32, [vp]),
        "onela_rs_get_memory": (i32, [vp, vp]),
        "onela_last_error": (ctypes.c_char_p, [vp]),
        "onela_init_requests_from_prompts": (i32, [vp, i32, p_i32, i32, vp, vp, vp, vp]),
        "onela_prefill": (i32, [i32, i32, i32, i32, i32, vp, vp, vp, vp, vp, vp, vp]),
        "onela_create_sharing_index": (i32, [ctypes.POINTER(_Config), vp, vp, ctypes.POINTER(vp)]),
        "onela_set_graph_mode": (i32, [vp, i32]),
        "onela_step_raw": (i32, [vp, i32, p_i32, vp, vp, vp, vp, vp, ctypes.POINTER(_Gates), vp, vp, vp]),
    }
    for name, (res, args) in sigs.items():
        fn = getattr(lib, name)
        fn.restype, fn.argtypes = res, args
    _lib = lib
    return lib


def _ptr(t, name, dtype=None, shape=None, optional=False):
    """Device pointer of a contiguous CUDA/HIP tensor after checking it."""
    if t is None:
        if optional:
            return None
        raise ValueError(f"{name} is required")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype not in dtype:
        raise ValueError(f"{name} has dtype {t.dtype}, expected one of {dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    return ctypes.c_void_p(t.data_ptr())


class Onela:
    """One GDN layer's OneLA decode state on the current HIP device."""

    def __init__(self, max_requests, num_heads, d_k, d_v, beam_width, max_steps, stream=None, share_index_of=None):
        """share_index_of: another Onela (a layer of the same requests) whose
        ancestry index this layer reads instead of keeping its own."""
        import torch

        self._torch = torch
        self.lib = load_library()
        self.cfg = _Config(max_requests, num_heads, d_k, d_v, beam_width, max_steps)
        self.stream = stream if stream is not None else torch.cuda.current_stream()
        self._ctx = ctypes.c_void_p()
        self.index_owner = share_index_of
        s = ctypes.c_void_p(self.stream.cuda_stream)
        if share_index_of is None:
            st = self.lib.onela_create(ctypes.byref(self.cfg), s, ctypes.byref(self._ctx))
        else:
            st = self.lib.onela_create_sharing_index(ctypes.byref(self.cfg), s, share_index_of._ctx,
                                                     ctypes.byref(self._ctx))
        self._check(st, "onela_create")

    # -- helpers --------------------------------------------------------------
    def _check(self, status, where):
        if status != ONELA_OK:
            detail = ""
            if self._ctx:
                detail = (self.lib.onela_last_error(self._ctx) or b"").decode()
            raise OnelaError(status, where, detail)

    def close(self):
        if self._ctx:
            self._check(self.lib.onela_destroy(self._ctx), "onela_destroy")
            self._ctx = ctypes.c_void_p()

    def __enter__(self):
        return self

    def __exit__(self, *exc):
        self.close()

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    # -- API -----------------------------------------------------------------
    def init_request(self, req: int, S0):
        c = self.cfg
        p = _ptr(S0, "S0", (self._torch.float32,), (c.num_heads, c.d_v, c.d_k))
        self._check(self.lib.onela_init_request(self._ctx, req, p), "onela_init_request")

    def init_requests_from_prompts(self, reqs, k, v, alpha, beta):
        """S0 of each listed request folded from its prompt on the GPU: k [n][L][H][d_k],
        v [n][L][H][d_v] (bf16 bits), alpha, beta [n][L][H] float32."""
        torch = self._torch
        c = self.cfg
        n, L = len(reqs), int(k.shape[1])
        bf = (torch.bfloat16, torch.int16, torch.uint16)
        arr = (ctypes.c_int32 * n)(*[int(r) for r in reqs])
        st = self.lib.onela_init_requests_from_prompts(
            self._ctx, n, arr, L,
            _ptr(k, "k", bf, (n, L, c.num_heads, c.d_k)), _ptr(v, "v", bf, (n, L, c.num_heads, c.d_v)),
            _ptr(alpha, "alpha", (torch.float32,), (n, L, c.num_heads)),
            _ptr(beta, "beta", (torch.float32,), (n, L, c.num_heads)))
        self._check(st, "onela_init_requests_from_prompts")

    def step(self, reqs, q, k, v, alpha, beta, parent_idx, o, delta_out=None):
        """Advance the given requests one step. q, k, v: bf16 (or int16/uint16 bits)."""
        torch = self._torch
        c = self.cfg
        n = len(reqs)
        rows = n * c.beam_width
        bf = (torch.bfloat16, torch.int16, torch.uint16)
        f32 = (torch.float32,)
        arr = (ctypes.c_int32 * n)(*[int(r) for r in reqs])
        st = self.lib.onela_step(
            self._ctx, n, arr,
            _ptr(q, "q", bf, (rows, c.num_heads, c.d_k)),
            _ptr(k, "k", bf, (rows, c.num_heads, c.d_k)),
            _ptr(v, "v", bf, (rows, c.num_heads, c.d_v)),
            _ptr(alpha, "alpha", f32, (rows, c.num_heads)),
            _ptr(beta, "beta", f32, (rows, c.num_heads)),
            _ptr(parent_idx, "parent_idx", (torch.int32,), (n, c.beam_width), optional=True),
            _ptr(o, "o", f32, (rows, c.num_heads, c.d_v)),
            _ptr(delta_out, "delta_out", f32, (rows, c.num_heads, c.d_v), optional=True),
        )
        self._check(st, "onela_step")

    def step_raw(self, reqs, q_raw, k_raw, v, a_raw, b_raw, A_log, dt_bias, parent_idx, o_bf16, delta_out=None,
                 norm_eps=1e-6):
        """onela_step from raw projections (q, k normalised, gates computed in the launch), o in bf16."""
        torch = self._torch
        c = self.cfg
        n = len(reqs)
        rows = n * c.beam_width
        bf = (torch.bfloat16, torch.int16, torch.uint16)
        f32 = (torch.float32,)
        arr = (ctypes.c_int32 * n)(*[int(r) for r in reqs])
        gates = _Gates(_ptr(A_log, "A_log", f32, (c.num_heads,)), _ptr(dt_bias, "dt_bias", f32, (c.num_heads,)),
                       float(norm_eps))
        st = self.lib.onela_step_raw(
            self._ctx, n, arr,
            _ptr(q_raw, "q_raw", bf, (rows, c.num_heads, c.d_k)),
            _ptr(k_raw, "k_raw", bf, (rows, c.num_heads, c.d_k)),
            _ptr(v, "v", bf, (rows, c.num_heads, c.d_v)),
            _ptr(a_raw, "a_raw", f32, (rows, c.num_heads)),
            _ptr(b_raw, "b_raw", f32, (rows, c.num_heads)),
            ctypes.byref(gates),
            _ptr(parent_idx, "parent_idx", (torch.int32,), (n, c.beam_width), optional=True),
            _ptr(o_bf16, "o_bf16", bf, (rows, c.num_heads, c.d_v)),
            _ptr(delta_out, "delta_out", f32, (rows, c.num_heads, c.d_v), optional=True),
        )
        self._check(st, "onela_step_raw")

    def reset(self, req: int):
        self._check(self.lib.onela_reset(self._ctx, req), "onela_reset")

    def sync(self):
        self._check(self.lib.onela_sync(self._ctx), "onela_sync")

    def set_graph_mode(self, on: bool):
        """Step counters on the device, so captured onela_step launches replay correctly."""
        self._check(self.lib.onela_set_graph_mode(self._ctx, int(bool(on))), "onela_set_graph_mode")

    def set_beams_per_block(self, beams: int):
        self._check(self.lib.onela_set_beams_per_block(self._ctx, beams), "onela_set_beams_per_block")

    def set_beam_order(self, mode: int):
        """-1 automatic, 0 beam-index order, 1 ancestry order (onela_set_beam_order)."""
        self._check(self.lib.onela_set_beam_order(self._ctx, mode), "onela_set_beam_order")

    def get_step(self, req: int) -> int:
        t = ctypes.c_int32()
        self._check(self.lib.onela_get_step(self._ctx, req, ctypes.byref(t)), "onela_get_step")
        return t.value

    def get_ancestry(self, req: int) -> np.ndarray:
        c = self.cfg
        out = np.empty((c.beam_width, c.max_steps), dtype=np.int32)
        self._check(self.lib.onela_get_ancestry(self._ctx, req, out.ctypes.data_as(ctypes.c_void_p)),
                    "onela_get_ancestry")
        return out

    def get_records(self, req: int, head: int, n_rec: int):
        c = self.cfg
        a = np.empty(n_rec, dtype=np.float32)
        d = np.empty((n_rec, c.d_v), dtype=np.float32)
        kk = np.empty((n_rec, c.d_k), dtype=np.uint16)
        self._check(self.lib.onela_get_records(self._ctx, req, head, n_rec,
                                               a.ctypes.data_as(ctypes.c_void_p),
                                               d.ctypes.data_as(ctypes.c_void_p),
                                               kk.ctypes.data_as(ctypes.c_void_p)), "onela_get_records")
        return a, d, kk

    def memory(self) -> dict:
        s0, rec, idx = ctypes.c_uint64(), ctypes.c_uint64(), ctypes.c_uint64()
        self._check(self.lib.onela_get_memory(self._ctx, ctypes.byref(s0), ctypes.byref(rec), ctypes.byref(idx)),
                    "onela_get_memory")
        return {"s0_bytes": s0.value, "record_bytes": rec.value, "index_bytes": idx.value}


class _Comparator:
    """A comparator context: same calls as Onela, C functions named by PREFIX."""

    PREFIX = ""

    def __init__(self, max_requests, num_heads, d_k, d_v, beam_width, max_steps, stream=None):
        import torch

        self._torch = torch
        self.lib = load_library()
        self.cfg = _Config(max_requests, num_heads, d_k, d_v, beam_width, max_steps)
        self.stream = stream if stream is not None else torch.cuda.current_stream()
        self._ctx = ctypes.c_void_p()
        st = self._fn("create")(ctypes.byref(self.cfg), ctypes.c_void_p(self.stream.cuda_stream),
                                ctypes.byref(self._ctx))
        if st != ONELA_OK:
            raise OnelaError(st, f"{self.PREFIX}_create")

    def _fn(self, name):
        return getattr(self.lib, f"{self.PREFIX}_{name}")

    def _check(self, status, where):
        if status != ONELA_OK:
            raise OnelaError(status, f"{self.PREFIX}_{where}")

    def close(self):
        if self._ctx:
            self._fn("destroy")(self._ctx)
            self._ctx = ctypes.c_void_p()

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def init_request(self, req: int, S0):
        c = self.cfg
        p = _ptr(S0, "S0", (self._torch.float32,), (c.num_heads, c.d_v, c.d_k))
        self._check(self._fn("init_request")(self._ctx, req, p), "init_request")

    def step(self, reqs, q, k, v, alpha, beta, parent_idx, o, delta_out=None):
        torch = self._torch
        c = self.cfg
        n = len(reqs)
        rows = n * c.beam_width
        bf = (torch.bfloat16, torch.int16, torch.uint16)
        f32 = (torch.float32,)
        arr = (ctypes.c_int32 * n)(*[int(r) for r in reqs])
        st = self._fn("step")(
            self._ctx, n, arr,
            _ptr(q, "q", bf, (rows, c.num_heads, c.d_k)),
            _ptr(k, "k", bf, (rows, c.num_heads, c.d_k)),
            _ptr(v, "v", bf, (rows, c.num_heads, c.d_v)),
            _ptr(alpha, "alpha", f32, (rows, c.num_heads)),
            _ptr(beta, "beta", f32, (rows, c.num_heads)),
            _ptr(parent_idx, "parent_idx", (torch.int32,), (n, c.beam_width), optional=True),
            _ptr(o, "o", f32, (rows, c.num_heads, c.d_v)),
            _ptr(delta_out, "delta_out", f32, (rows, c.num_heads, c.d_v), optional=True),
        )
        self._check(st, "step")

    def reset(self, req: int):
        self._check(self._fn("reset")(self._ctx, req), "reset")

    def sync(self):
        self._check(self._fn("sync")(self._ctx), "sync")

    def memory(self) -> int:
        b = ctypes.c_uint64()
        self._check(self._fn("get_memory")(self._ctx, ctypes.byref(b)), "get_memory")
        return b.value


class FullState(_Comparator):
    """The comparator that keeps a full d_v x d_k state per beam (onela_fs_*)."""

    PREFIX = "onela_fs"


class ReplayState(_Comparator):
    """The comparator in which every beam rebuilds its state from S0 and its own
    ancestral records at every step (onela_rs_*)."""

    PREFIX = "onela_rs"


def prefill(k, v, alpha, beta, S_init=None, out=None, stream=None):
    """Fold prompts into float32 states on the GPU (onela_prefill).

    k: [n][L][H][d_k] and v: [n][L][H][d_v] bf16 (or int16/uint16 bits); alpha,
    beta: [n][L][H] float32; S_init: optional [n][H][d_v][d_k] float32. Returns
    `out` (allocated if None), [n][H][d_v][d_k] float32; out may be S_init.
    """
    import torch

    lib = load_library()
    n, L, H, dk = (int(x) for x in k.shape)
    dv = int(v.shape[3])
    bf = (torch.bfloat16, torch.int16, torch.uint16)
    f32 = (torch.float32,)
    if out is None:
        out = torch.empty((n, H, dv, dk), dtype=torch.float32, device=k.device)
    stream = stream if stream is not None else torch.cuda.current_stream()
    st = lib.onela_prefill(
        n, H, dk, dv, L,
        _ptr(k, "k", bf, (n, L, H, dk)), _ptr(v, "v", bf, (n, L, H, dv)),
        _ptr(alpha, "alpha", f32, (n, L, H)), _ptr(beta, "beta", f32, (n, L, H)),
        _ptr(S_init, "S_init", f32, (n, H, dv, dk), optional=True),
        _ptr(out, "out", f32, (n, H, dv, dk)), ctypes.c_void_p(stream.cuda_stream))
    if st != ONELA_OK:
        raise OnelaError(st, "onela_prefill")
    return out
