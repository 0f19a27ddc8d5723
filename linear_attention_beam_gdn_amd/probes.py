"""ctypes binding of libonela_probes.so (onela_probes.h): the bench's
measurement probes, a plain device copy, a register-only MFMA loop and the
shared-state projection on its own. Not part of the decode path."""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
PROBE_LIB_PATH = os.path.join(_HERE, "libonela_probes.so")
EXPORTED = ("onela_probe_copy", "onela_probe_mfma", "onela_probe_planes", "onela_probe_projection")

_lib = None


def load(path: str = PROBE_LIB_PATH) -> ctypes.CDLL:
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise ImportError(f"{path} is missing: build it with `python -m linear_attention_beam_gdn_amd.build`")
    lib = ctypes.CDLL(path)
    vp, i32 = ctypes.c_void_p, ctypes.c_int32
    lib.onela_probe_copy.restype, lib.onela_probe_copy.argtypes = i32, [vp, vp, ctypes.c_size_t, vp]
    lib.onela_probe_mfma.restype, lib.onela_probe_mfma.argtypes = i32, [vp, i32, i32, vp]
    lib.onela_probe_planes.restype, lib.onela_probe_planes.argtypes = i32, [vp, vp, i32, vp]
    lib.onela_probe_projection.restype = i32
    lib.onela_probe_projection.argtypes = [vp, vp, vp, i32, i32, i32, i32, vp, vp]
    _lib = lib
    return lib


def _stream(stream):
    import torch

    return ctypes.c_void_p((stream if stream is not None else torch.cuda.current_stream()).cuda_stream)


def _ok(status, what):
    if status != 0:
        raise RuntimeError(f"{what} failed with status {status}")


def copy(src, dst, stream=None):
    """dst <- src (contiguous device tensors of the same byte size, a multiple of 16)."""
    nbytes = src.numel() * src.element_size()
    if nbytes % 16 or dst.numel() * dst.element_size() != nbytes or not (src.is_contiguous() and dst.is_contiguous()):
        raise ValueError("copy: equal contiguous sizes, a multiple of 16 bytes")
    _ok(load().onela_probe_copy(ctypes.c_void_p(src.data_ptr()), ctypes.c_void_p(dst.data_ptr()), nbytes // 16,
                                _stream(stream)), "onela_probe_copy")


def mfma_loop(out, n_wg: int, iters: int, stream=None):
    """n_wg workgroups x 8 waves x iters x 8 MFMAs (16x16x32 bf16); out float32 [n_wg*512]."""
    if out.numel() < n_wg * 512 or not out.is_contiguous():
        raise ValueError("mfma_loop: out needs n_wg*512 floats")
    _ok(load().onela_probe_mfma(ctypes.c_void_p(out.data_ptr()), n_wg, iters, _stream(stream)), "onela_probe_mfma")


def planes(S0, stream=None):
    """S0 float32 [R][H][128][128] -> the bf16 hi/lo planes [R][H][2][128*128]
    (int16 bits, A-fragment order) that `projection` reads."""
    import torch

    R, H = int(S0.shape[0]), int(S0.shape[1])
    if tuple(S0.shape) != (R, H, 128, 128) or S0.dtype != torch.float32 or not S0.is_contiguous():
        raise ValueError("planes: S0 float32 [R][H][128][128], contiguous")
    out = torch.empty((R, H, 2, 128 * 128), dtype=torch.int16, device=S0.device)
    _ok(load().onela_probe_planes(ctypes.c_void_p(S0.data_ptr()), ctypes.c_void_p(out.data_ptr()), R * H,
                                  _stream(stream)), "onela_probe_planes")
    return out


def projection(pl, k, q, W: int, colsum, resident_pairs: int = 0, stream=None):
    """colsum[p][i] = sum_b (S0_s k_b + S0_s q_b)[i] for pair p = r*H + h, with s = p, or
    p mod resident_pairs when that is set; pl the planes of S0 [R][H][128][128] from
    `planes`, k, q [R*W][H][128] bf16 bits, colsum [R*H][128] float32."""
    R, H = int(pl.shape[0]), int(pl.shape[1])
    if tuple(pl.shape) != (R, H, 2, 128 * 128) or not pl.is_contiguous():
        raise ValueError("projection: planes [R][H][2][128*128]")
    if tuple(k.shape) != (R * W, H, 128) or tuple(q.shape) != (R * W, H, 128) or colsum.numel() != R * H * 128:
        raise ValueError("projection: shapes")
    _ok(load().onela_probe_projection(ctypes.c_void_p(pl.data_ptr()), ctypes.c_void_p(k.data_ptr()),
                                      ctypes.c_void_p(q.data_ptr()), R, H, W, int(resident_pairs),
                                      ctypes.c_void_p(colsum.data_ptr()),
                                      _stream(stream)), "onela_probe_projection")
