"""TEST INFRASTRUCTURE ONLY: the CPU fp64 oracle for paged GQA decode attention.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package. It is independent of the HIP library in
``paged_kv_split_amd/``: the two share no code and neither imports the other.

``decode`` wraps the C oracle (``ref_decode.c``), which evaluates the plain
definition ``softmax(scale * q K^T) V`` over the pages that ``block_table``
names, in double precision (see that file's header for the passages it
follows). ``brute`` is a second, independent numpy implementation used to pin
the C oracle on small inputs.
"""
import ctypes
import os

import numpy as np
import torch

from . import build as _build

__all__ = ["decode", "e4m3fn_to_float64", "available_threads", "OracleError"]

KV_BF16 = 0
KV_FP8_E4M3 = 1

_ERRORS = {
    1: "bad shape or argument",
    2: "context length beyond the block table",
    3: "block_table entry outside [0, num_pages)",
    4: "out of memory",
}


class OracleError(RuntimeError):
    pass


class _Problem(ctypes.Structure):
    _fields_ = [
        ("batch", ctypes.c_int32),
        ("num_q_heads", ctypes.c_int32),
        ("num_kv_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("page_size", ctypes.c_int32),
        ("max_pages_per_seq", ctypes.c_int32),
        ("num_pages", ctypes.c_int32),
        ("kv_kind", ctypes.c_int32),
        ("scale", ctypes.c_double),
    ]


_lib = None


def load_library(path):
    """Open an oracle build at ``path`` (the tests also open deliberately
    broken builds this way, to show that the pins catch them)."""
    lib = ctypes.CDLL(path)
    lib.oracle_decode.restype = ctypes.c_int
    lib.oracle_decode.argtypes = [ctypes.POINTER(_Problem)] + [ctypes.c_void_p] * 9 + [
        ctypes.c_int, ctypes.POINTER(ctypes.c_int)]
    lib.oracle_e4m3fn_to_double.restype = ctypes.c_double
    lib.oracle_e4m3fn_to_double.argtypes = [ctypes.c_uint8]
    lib.oracle_available_threads.restype = ctypes.c_int
    lib.oracle_available_threads.argtypes = []
    return lib


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_build.LIBRARY):
            _build.build()
        _lib = load_library(_build.LIBRARY)
    return _lib


def available_threads() -> int:
    return int(_load().oracle_available_threads())


def e4m3fn_to_float64(code: int, library=None) -> float:
    """The oracle's own decoding of one OCP E4M3FN code."""
    lib = library if library is not None else _load()
    return float(lib.oracle_e4m3fn_to_double(ctypes.c_uint8(code)))


def _bits(t: torch.Tensor, dtype) -> np.ndarray:
    t = t.detach().cpu().contiguous()
    return np.ascontiguousarray(t.view(dtype).numpy())


def decode(q, k_pages, v_pages, block_table, context_lens, *, scale=None,
           k_scale=None, v_scale=None, threads=0, return_threads=False, library=None):
    """Oracle output for one decode step.

    q: bf16 [B, Hq, d]. k_pages / v_pages: bf16 or float8_e4m3fn
    [num_pages, P, Hkv, d]. k_scale / v_scale: fp32 [num_pages, P, Hkv] for
    fp8 pools. block_table: int32 [B, max_pages]. context_lens: int32 [B].
    scale: softmax scale, default 1/sqrt(d).
    Returns (out float64 [B, Hq, d], lse float64 [B, Hq]) as torch tensors.
    """
    if q.dtype != torch.bfloat16:
        raise TypeError("q must be bfloat16")
    B, Hq, D = q.shape
    num_pages, P, Hkv, D2 = k_pages.shape
    if D2 != D or tuple(v_pages.shape) != tuple(k_pages.shape):
        raise ValueError("pool shape mismatch")
    if k_pages.dtype == torch.bfloat16:
        kind = KV_BF16
        kb, vb = _bits(k_pages, torch.int16), _bits(v_pages, torch.int16)
        ks = vs = None
    elif k_pages.dtype == torch.float8_e4m3fn:
        kind = KV_FP8_E4M3
        kb, vb = _bits(k_pages, torch.uint8), _bits(v_pages, torch.uint8)
        if k_scale is None or v_scale is None:
            raise ValueError("fp8 pools need k_scale and v_scale")
        ks = np.ascontiguousarray(k_scale.detach().cpu().to(torch.float32).numpy())
        vs = np.ascontiguousarray(v_scale.detach().cpu().to(torch.float32).numpy())
        if ks.shape != (num_pages, P, Hkv) or vs.shape != (num_pages, P, Hkv):
            raise ValueError("scale shape mismatch")
    else:
        raise TypeError("pools must be bfloat16 or float8_e4m3fn")
    qb = _bits(q, torch.int16)
    bt = np.ascontiguousarray(block_table.detach().cpu().to(torch.int32).numpy())
    lens = np.ascontiguousarray(context_lens.detach().cpu().to(torch.int32).numpy())
    if bt.ndim != 2 or bt.shape[0] != B or lens.shape != (B,):
        raise ValueError("block_table / context_lens shape mismatch")
    prob = _Problem(B, Hq, Hkv, D, P, bt.shape[1], num_pages, kind,
                    float(1.0 / np.sqrt(D)) if scale is None else float(scale))
    out = np.zeros((B, Hq, D), dtype=np.float64)
    lse = np.zeros((B, Hq), dtype=np.float64)
    used = ctypes.c_int(0)

    def ptr(a):
        return None if a is None else a.ctypes.data_as(ctypes.c_void_p)

    lib = library if library is not None else _load()
    rc = lib.oracle_decode(ctypes.byref(prob), ptr(qb), ptr(kb), ptr(vb), ptr(ks), ptr(vs),
                               ptr(bt), ptr(lens), ptr(out), ptr(lse), int(threads),
                               ctypes.byref(used))
    if rc != 0:
        raise OracleError(_ERRORS.get(rc, f"oracle error {rc}"))
    res = (torch.from_numpy(out), torch.from_numpy(lse))
    if return_threads:
        return res + (int(used.value),)
    return res
