"""Seeded synthetic inputs for the CSA2 FP4-KV decode path.

This module is shared by the two independent sides of the parity checks: the
oracle (host) and the HIP library (device).  It contains no step of the method
itself -- no quantisation, scoring, selection or attention -- only:

* a counter-based integer generator: element ``i`` of tensor ``tid`` is the
  ``(i+1)``-th output of Vigna's splitmix64 generator (public definition:
  state += 0x9E3779B97F4A7C15, then the xor-shift/multiply output mix) whose
  state starts at ``mix((seed << 32) ^ tid)``;
* two value maps applied to that 64-bit output ``h``:
  - ``INT9``:   ``(h mod 9) - 4``, an integer in [-4, 4] stored exactly as bf16
    (the indexer query and key workload of the pages: small integers, so the
    indexer scores are exact);
  - ``NORMAL``: ``NTAB[h >> 48]``, a 65,536-entry table of standard-normal
    quantiles ``bf16(float32(Phi^-1((j + 0.5) / 65536)))`` (the N(0,1) bf16
    workload of the pages' latent rows, main queries and SWA rows).

The same generator runs on the device (``synth/fill.hip`` built into
``synth/libcsa2_synth.so``); the table is built here and uploaded, so both
sides produce identical bits.

Row-structured tensors use the flat index ``((b << 24) + row) * dim + d``
(sequence ``b``, row ``row``, column ``d``), so a row's values do not depend
on the capacity or batch size of the buffer it is written into.
"""
from __future__ import annotations

import ctypes
import os
from functools import lru_cache

import numpy as np

__all__ = [
    "INT9", "NORMAL", "tensor_id", "ntab", "gen_rows", "gen_flat",
    "splitmix64_outputs", "device_lib",
]

INT9 = 0
NORMAL = 1

_GAMMA = np.uint64(0x9E3779B97F4A7C15)
_M1 = np.uint64(0xBF58476D1CE4E5B9)
_M2 = np.uint64(0x94D049BB133111EB)
_MASK = (1 << 64) - 1

# Tensor kinds, used to build tensor ids (kind << 24 | a << 12 | b).
KIND_KV_SRC = 1      # main-KV latent source rows; a = kv tensor id
KIND_IDX_K = 2       # indexer K per position
KIND_BLK_K = 3       # hierarchical block keys per block of 8 positions
KIND_IDX_Q = 4       # indexer Q; a = layer, b = step
KIND_MAIN_Q = 5      # main Q; a = layer, b = step
KIND_SWA = 6         # SWA rows; a = layer, b = step (0 = initial window)
KIND_NEW_ROW = 7     # appended latent row; a = kv tensor id, b = step
KIND_IDX_W = 8       # optional indexer head weights; a = layer, b = step
KIND_NEW_IDX_K = 9   # indexer key of an appended position; b = step


def tensor_id(kind: int, a: int = 0, b: int = 0) -> int:
    """Tensor id of a synthetic stream (32-bit)."""
    assert 0 <= kind < 256 and 0 <= a < 4096 and 0 <= b < 4096
    return (kind << 24) | (a << 12) | b


def _mix(z: np.ndarray) -> np.ndarray:
    """splitmix64 output function (Vigna), on uint64 arrays (wrapping)."""
    z = (z ^ (z >> np.uint64(30))) * _M1
    z = (z ^ (z >> np.uint64(27))) * _M2
    return z ^ (z >> np.uint64(31))


def _mix_int(z: int) -> int:
    z &= _MASK
    z = ((z ^ (z >> 30)) * 0xBF58476D1CE4E5B9) & _MASK
    z = ((z ^ (z >> 27)) * 0x94D049BB133111EB) & _MASK
    return z ^ (z >> 31)


def stream_key(seed: int, tid: int) -> int:
    assert 0 <= seed < (1 << 32) and 0 <= tid < (1 << 32)
    return _mix_int((seed << 32) ^ tid)


def splitmix64_outputs(seed: int, tid: int, idx: np.ndarray) -> np.ndarray:
    """64-bit generator outputs at flat indices ``idx`` (uint64 array)."""
    key = np.uint64(stream_key(seed, tid))
    idx = np.asarray(idx, dtype=np.uint64)
    with np.errstate(over="ignore"):
        state = key + (idx + np.uint64(1)) * _GAMMA
        return _mix(state)


def _f32_to_bf16_rne(x: np.ndarray) -> np.ndarray:
    u = np.asarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    rounded = (u + np.uint64(0x7FFF) + ((u >> np.uint64(16)) & np.uint64(1))) >> np.uint64(16)
    return rounded.astype(np.uint16)


@lru_cache(maxsize=1)
def ntab() -> np.ndarray:
    """The 65,536-entry normal-quantile table as bf16 bit patterns (uint16)."""
    from scipy.special import ndtri

    p = (np.arange(65536, dtype=np.float64) + 0.5) / 65536.0
    return _f32_to_bf16_rne(ndtri(p).astype(np.float32))


_INT_BF16 = np.array([0xC080, 0xC040, 0xC000, 0xBF80, 0x0000,
                      0x3F80, 0x4000, 0x4040, 0x4080], dtype=np.uint16)  # -4..4


def _values(h: np.ndarray, kind: int) -> np.ndarray:
    if kind == INT9:
        return _INT_BF16[(h % np.uint64(9)).astype(np.int64)]
    if kind == NORMAL:
        return ntab()[(h >> np.uint64(48)).astype(np.int64)]
    raise ValueError(f"unknown value kind {kind}")


def gen_rows_numpy(seed: int, tid: int, kind: int, b, rows, dim: int) -> np.ndarray:
    """Definition of :func:`gen_rows` in numpy (slow for large tensors)."""
    b = np.asarray(b, dtype=np.uint64).reshape(-1, 1, 1)
    rows = np.asarray(rows, dtype=np.uint64).reshape(1, -1, 1)
    d = np.arange(dim, dtype=np.uint64).reshape(1, 1, -1)
    idx = ((b << np.uint64(24)) + rows) * np.uint64(dim) + d
    return _values(splitmix64_outputs(seed, tid, idx), kind)


_HOST_SRC = os.path.join(os.path.dirname(os.path.abspath(__file__)), "gen_host.c")
_HOST_LIB = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libcsa2_synth_host.so")


def build_host(force: bool = False) -> str:
    """Compile the host generator (plain C, gcc)."""
    import subprocess

    if force or not os.path.exists(_HOST_LIB) or os.path.getmtime(_HOST_LIB) < os.path.getmtime(_HOST_SRC):
        tmp = _HOST_LIB + f".tmp{os.getpid()}"
        subprocess.check_call(["gcc", "-O2", "-std=c11", "-shared", "-fPIC", "-o", tmp, _HOST_SRC])
        os.replace(tmp, _HOST_LIB)
    return _HOST_LIB


@lru_cache(maxsize=1)
def _host_lib():
    lib = ctypes.CDLL(build_host())
    P = ctypes.c_void_p
    lib.synth_gen_rows_host.argtypes = [ctypes.c_uint64, ctypes.c_int32, P, ctypes.c_int64, P,
                                        ctypes.c_int64, ctypes.c_int32, P, P]
    lib.synth_gen_rows_host.restype = None
    return lib


def gen_rows(seed: int, tid: int, kind: int, b, rows, dim: int) -> np.ndarray:
    """bf16 bit patterns [len(b)][len(rows)][dim] of row-structured tensor ``tid``.

    ``b`` and ``rows`` are integer sequences (sequence ids and row ids).
    Computed by the C generator; equal to :func:`gen_rows_numpy`."""
    bs = np.ascontiguousarray(np.asarray(b, dtype=np.int64).reshape(-1))
    rs = np.ascontiguousarray(np.asarray(rows, dtype=np.int64).reshape(-1))
    out = np.empty((len(bs), len(rs), dim), np.uint16)
    tab = ntab()
    _host_lib().synth_gen_rows_host(stream_key(seed, tid), kind, bs.ctypes.data, len(bs), rs.ctypes.data,
                                    len(rs), dim, tab.ctypes.data, out.ctypes.data)
    return out


def gen_flat(seed: int, tid: int, kind: int, n: int) -> np.ndarray:
    """bf16 bit patterns of the first ``n`` elements of a flat tensor."""
    return _values(splitmix64_outputs(seed, tid, np.arange(n, dtype=np.uint64)), kind)


def bf16_to_f32(u16: np.ndarray) -> np.ndarray:
    return (np.asarray(u16, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


# --------------------------------------------------------------------------
# Device side: the same generator as a HIP fill kernel (synth/fill.hip).
# --------------------------------------------------------------------------
_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libcsa2_synth.so")


@lru_cache(maxsize=1)
def device_lib() -> ctypes.CDLL:
    """Load the device generator library (built by ``__graft_entry__.build``)."""
    if not os.path.exists(_LIB_PATH):
        raise RuntimeError(f"{_LIB_PATH} is missing: run __graft_entry__.build() first")
    lib = ctypes.CDLL(_LIB_PATH)
    lib.synth_fill_rows.argtypes = [
        ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64,   # dst, batch stride, row stride (elements)
        ctypes.c_int32, ctypes.c_int64, ctypes.c_int32,    # nb, n_rows, dim
        ctypes.c_int32, ctypes.c_int64,                    # b0, row0
        ctypes.c_uint64, ctypes.c_uint32, ctypes.c_int32,  # seed, tid, kind
        ctypes.c_void_p, ctypes.c_void_p,                  # ntab (device), stream
    ]
    lib.synth_fill_rows.restype = ctypes.c_int32
    return lib


def fill_rows_device(dst, seed: int, tid: int, kind: int, b0: int = 0, row0: int = 0,
                     ntab_dev=None, stream=None) -> None:
    """Fill a device tensor ``dst`` of shape [nb][n_rows][dim] (bf16 / int16 /
    uint16 storage, last dim contiguous) with rows ``row0..`` of sequences
    ``b0..`` of tensor ``tid``; identical bits to :func:`gen_rows`."""
    import torch

    assert dst.dim() == 3 and dst.element_size() == 2 and dst.stride(2) == 1
    nb, n_rows, dim = dst.shape
    if ntab_dev is None:
        ntab_dev = _ntab_device(dst.device)
    if stream is None:
        stream = torch.cuda.current_stream(dst.device).cuda_stream
    rc = device_lib().synth_fill_rows(
        dst.data_ptr(), dst.stride(0), dst.stride(1), nb, n_rows, dim, b0, row0,
        seed, tid, kind, ntab_dev.data_ptr(), stream)
    if rc != 0:
        raise RuntimeError(f"synth_fill_rows failed with code {rc}")


_NTAB_DEV = {}


def _ntab_device(device):
    import torch

    key = str(device)
    if key not in _NTAB_DEV:
        _NTAB_DEV[key] = torch.from_numpy(ntab().view(np.int16).copy()).to(device)
    return _NTAB_DEV[key]
