"""Python binding of libcsa2, the CSA2 FP4-KV decode path for MI355X (gfx950).

Argument marshalling only: every step runs in the HIP kernels of libcsa2.so.
PyTorch provides device memory and the current HIP stream.  The functions
mirror the C entry points of include/csa2.h (same names without the
``csa2_`` prefix); tensors must already be on the GPU with the documented
shapes and dtypes (bf16 data may be passed as torch.bfloat16 or int16).
There is no fallback: if the library is missing, importing raises.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence

import torch

__all__ = [
    "LIB_PATH", "Csa2Error", "FP4KV", "quant_rows", "quant_append", "index_score", "topk", "topk_workspace_size",
    "sparse_attn", "sparse_attn_workspace_size", "sparse_attn_noalloc", "sparse_attn_partial", "attn_merge", "pool_select", "pool_select_workspace_size", "flat_select", "flat_select_workspace_size", "Sched", "Layer", "FULL", "REINDEX", "REUSE",
    "prefill_index_score", "Prefill", "quant_fp8_rows", "block_keys", "append_index_keys",
    "LATENT", "CODE_BYTES", "SCALE_BYTES", "HEADS", "IDX_HEADS", "IDX_DIM",
]

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libcsa2.so")
LATENT, CODE_BYTES, SCALE_BYTES = 512, 256, 32
HEADS, IDX_HEADS, IDX_DIM = 16, 8, 64
FULL, REINDEX, REUSE = 0, 1, 2

if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is missing; build it with `python fp4_kv_cache_quant_amd/build.py`")
_lib = ctypes.CDLL(LIB_PATH)

_P, _I32, _I64, _F32, _SZ = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_float, ctypes.c_size_t


class _FP4KV(ctypes.Structure):
    _fields_ = [("codes", _P), ("scales", _P), ("cap", _I64), ("n_seq", _I32)]


class _Layer(ctypes.Structure):
    _fields_ = [("mode", _I32), ("kv_id", _I32), ("hierarchical", _I32)]


class _SchedDesc(ctypes.Structure):
    _fields_ = [("n_seq", _I32), ("n_layers", _I32), ("layers", _P), ("key_cap", _I64),
                ("blk_cap", _I64), ("topk", _I32), ("pool_blocks", _I32), ("blk", _I32),
                ("swa_max", _I32), ("sm_scale", _F32), ("swa_fp8", _I32)]


class _StepIO(ctypes.Structure):
    _fields_ = [("n_kv", _I32), ("kv", _P), ("lens", _P), ("new_row", _P), ("append_kv", _I32),
                ("idx_k", _P), ("blk_k", _P), ("idx_q", _P), ("idx_w", _P), ("main_q", _P),
                ("swa", _P), ("swa_len", _P), ("out", _P), ("new_idx_k", _P), ("layer_idx_k", _P),
                ("new_swa_row", _P)]


class _PrefillDesc(ctypes.Structure):
    _fields_ = [("n_layers", _I32), ("layers", _P), ("n_entries", _I64), ("ratio", _I32), ("n_q", _I32),
                ("t0", _I64), ("topk", _I32), ("swa", _I32), ("sm_scale", _F32)]


class _PrefillIO(ctypes.Structure):
    _fields_ = [("n_kv", _I32), ("kv", _P), ("entry_k", _P), ("idx_q", _P), ("idx_w", _P), ("main_q", _P),
                ("swa", _P), ("out", _P), ("idx", _P)]


def _sig(name, res, *args):
    f = getattr(_lib, name)
    f.restype = res
    f.argtypes = list(args)
    return f


_last_error = _sig("csa2_last_error", ctypes.c_char_p)
abi_version = _sig("csa2_abi_version", _I32)
_quant_rows = _sig("csa2_quant_rows", _I32, _P, _I64, _P, _P, _P)
_quant_append = _sig("csa2_quant_append", _I32, _P, _FP4KV, _P, _P, _P)
_index_score = _sig("csa2_index_score", _I32, _P, _P, _P, _I64, _P, _I32, _P, _I32, _I32, _P, _I64, _I32, _P)
_topk_ws = _sig("csa2_topk_workspace_size", _SZ, _I64, _I32)
_topk = _sig("csa2_topk", _I32, _P, _I64, _P, _I32, _I32, _P, _I32, _I32, _P, _P, _SZ, _I32, _P)
_flat_ws = _sig("csa2_flat_select_workspace_size", _SZ, _I64, _I32, _I32)
_flat_select = _sig("csa2_flat_select", _I32, _P, _P, _P, _I64, _P, _I32, _P, _P, _SZ, _I32, _P)
_pool_ws = _sig("csa2_pool_select_workspace_size", _SZ, _I32, _I32, _I32)
_pool_select = _sig("csa2_pool_select", _I32, _P, _P, _P, _I64, _P, _P, _I32, _I32, _I32, _P, _P, _SZ, _I32, _P)
_attn_ws = _sig("csa2_sparse_attn_workspace_size", _SZ, _I32, _I32, _I32)
_attn_f8w = _sig("csa2_sparse_attn_f8w", _I32, _P, _I32, ctypes.POINTER(_FP4KV), _I32, _P, _I32, _P, _I64, _P,
                 _I32, _F32, _P, _P, _SZ, _P)
_quant_fp8 = _sig("csa2_quant_fp8_rows", _I32, _P, _I64, _P, _P)
_block_keys = _sig("csa2_block_keys", _I32, _P, _I64, _P, _I32, _P, _I64, _I32, _P)
_append_keys = _sig("csa2_append_index_keys", _I32, _P, _P, _I64, _P, _I64, _I32, _P, _P, _I32, _P)
_attn = _sig("csa2_sparse_attn", _I32, _P, _I32, ctypes.POINTER(_FP4KV), _I32, _P, _I32, _P, _I64, _P,
             _I32, _F32, _P, _P, _SZ, _P)
_attn_partial = _sig("csa2_sparse_attn_partial", _I32, _P, _I32, ctypes.POINTER(_FP4KV), _I32, _P, _I32, _P, _I64,
                     _P, _I32, _F32, _P, _P, _P, _SZ, _P)
_attn_merge = _sig("csa2_attn_merge", _I32, _P, _P, _I32, _I32, _P, _P)
_attn_noalloc = _sig("csa2_sparse_attn_noalloc", _I32, _P, _I32, ctypes.POINTER(_FP4KV), _I32, _P, _I32, _P, _I64,
                     _P, _I32, _F32, _P, _P)
_sched_create = _sig("csa2_sched_create", _I32, ctypes.POINTER(_SchedDesc), ctypes.POINTER(_P))
_sched_step = _sig("csa2_sched_decode_step", _I32, _P, ctypes.POINTER(_StepIO), _P)
_sched_indices = _sig("csa2_sched_indices", _P, _P, _I32)
_sched_pool = _sig("csa2_sched_pool", _P, _P)
_sched_check = _sig("csa2_sched_check", _I32, _P, ctypes.POINTER(_I32), _P)
_sched_destroy = _sig("csa2_sched_destroy", None, _P)
_prefill_score = _sig("csa2_prefill_index_score", _I32, _P, _P, _P, _I64, _I64, _I32, _I32, _P, _P, _P)
_prefill_ws = _sig("csa2_prefill_workspace_size", _SZ, ctypes.POINTER(_PrefillDesc))
_prefill_select_ws = _sig("csa2_prefill_select_workspace_size", _SZ, _I64, _I32, _I32)
_prefill_select = _sig("csa2_prefill_select", _I32, _P, _P, _P, _I64, _I64, _I32, _I32, _I32, _P, _P, _P, _SZ, _P)
_prefill_chunk = _sig("csa2_prefill_chunk", _I32, ctypes.POINTER(_PrefillDesc), ctypes.POINTER(_PrefillIO),
                      _P, _SZ, _P)


class Csa2Error(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"csa2 error {code}: {msg}")
        self.code = code


def _check(rc: int) -> None:
    if rc != 0:
        raise Csa2Error(rc, _last_error().decode(errors="replace"))


def _ptr(t: Optional[torch.Tensor]):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("tensor must be on the GPU")
    if not t.is_contiguous():
        raise ValueError("tensor must be contiguous")
    return t.data_ptr()


def _stream(stream):
    return (stream if stream is not None else torch.cuda.current_stream()).cuda_stream


class FP4KV:
    """An FP4 main-KV tensor: codes [n_seq][cap][256] u8 + scales [n_seq][cap][32] u8."""

    def __init__(self, codes: torch.Tensor, scales: torch.Tensor):
        assert codes.dtype == torch.uint8 and scales.dtype == torch.uint8
        assert codes.dim() == 3 and codes.shape[2] == CODE_BYTES
        assert scales.shape == (*codes.shape[:2], SCALE_BYTES)
        self.codes, self.scales = codes, scales

    @classmethod
    def empty(cls, n_seq: int, cap: int, device="cuda"):
        return cls(torch.zeros(n_seq, cap, CODE_BYTES, dtype=torch.uint8, device=device),
                   torch.zeros(n_seq, cap, SCALE_BYTES, dtype=torch.uint8, device=device))

    @property
    def n_seq(self):
        return self.codes.shape[0]

    @property
    def cap(self):
        return self.codes.shape[1]

    def c(self) -> _FP4KV:
        return _FP4KV(_ptr(self.codes), _ptr(self.scales), self.cap, self.n_seq)


def quant_rows(src: torch.Tensor, codes: torch.Tensor, scales: torch.Tensor, stream=None) -> None:
    """src [n][512] bf16 -> codes [n][256], scales [n][32] (views of a cache are fine if contiguous)."""
    n = src.numel() // LATENT
    assert codes.numel() >= n * CODE_BYTES and scales.numel() >= n * SCALE_BYTES
    _check(_quant_rows(_ptr(src), n, _ptr(codes), _ptr(scales), _stream(stream)))


def quant_fp8_rows(src: torch.Tensor, dst: torch.Tensor, stream=None) -> None:
    """Window rows src [n][512] bf16 -> dst [n][512] uint8 E4M3 codes."""
    n = src.numel() // LATENT
    assert dst.dtype == torch.uint8 and dst.numel() >= n * LATENT
    _check(_quant_fp8(_ptr(src), n, _ptr(dst), _stream(stream)))


def block_keys(idx_k: torch.Tensor, lens: torch.Tensor, blk_k: torch.Tensor, blk: int = 8, stream=None) -> None:
    """idx_k [n_seq][key_cap][64] -> blk_k [n_seq][blk_cap][64]: sums of the blocks' keys (bf16)."""
    n_seq, key_cap = idx_k.shape[0], idx_k.shape[1]
    _check(_block_keys(_ptr(idx_k), key_cap, _ptr(lens), blk, _ptr(blk_k), blk_k.shape[1], n_seq, _stream(stream)))


def append_index_keys(new_k: torch.Tensor, idx_k: torch.Tensor, lens: torch.Tensor,
                      blk_k: Optional[torch.Tensor] = None, blk: int = 8, err_flag: Optional[torch.Tensor] = None,
                      stream=None) -> None:
    """Write new_k [n_seq][64] at row lens[b] of idx_k and add it to its block's key."""
    n_seq, key_cap = idx_k.shape[0], idx_k.shape[1]
    _check(_append_keys(_ptr(new_k), _ptr(idx_k), key_cap, _ptr(blk_k), blk_k.shape[1] if blk_k is not None else 0,
                        blk, _ptr(lens), _ptr(err_flag), n_seq, _stream(stream)))


def quant_append(src: torch.Tensor, kv: FP4KV, lens: torch.Tensor, err_flag: Optional[torch.Tensor] = None,
                 stream=None) -> None:
    assert src.numel() == kv.n_seq * LATENT and lens.dtype == torch.int32 and lens.numel() == kv.n_seq
    _check(_quant_append(_ptr(src), kv.c(), _ptr(lens), _ptr(err_flag), _stream(stream)))


def index_score(q: torch.Tensor, keys: torch.Tensor, lens: torch.Tensor, scores: torch.Tensor,
                w: Optional[torch.Tensor] = None, len_div: int = 1, pool: Optional[torch.Tensor] = None,
                blk: int = 8, stream=None) -> None:
    """q [n_seq][8][64], keys [n_seq][key_cap][64], scores [n_seq][n_out] f32."""
    n_seq, key_cap = keys.shape[0], keys.shape[1]
    n_out = scores.shape[1]
    n_pool = pool.shape[1] if pool is not None else 0
    _check(_index_score(_ptr(q), _ptr(w), _ptr(keys), key_cap, _ptr(lens), len_div, _ptr(pool), n_pool,
                        blk, _ptr(scores), n_out, n_seq, _stream(stream)))


def topk_workspace_size(n: int, n_seq: int) -> int:
    return int(_topk_ws(n, n_seq))


def topk(scores: torch.Tensor, k: int, out: torch.Tensor, lens: Optional[torch.Tensor] = None,
         len_div: int = 1, pool: Optional[torch.Tensor] = None, blk: int = 8,
         ws: Optional[torch.Tensor] = None, stream=None) -> None:
    """scores [n_seq][n] f32 -> out [n_seq][k] int32 ascending ids, -1 padded.
    ws: a zero-filled workspace reused across calls (a fresh one if None)."""
    n_seq, n = scores.shape
    n_pool = pool.shape[1] if pool is not None else 0
    if ws is None:
        ws = torch.zeros(max(topk_workspace_size(n, n_seq), 1), dtype=torch.uint8, device=scores.device)
    _check(_topk(_ptr(scores), n, _ptr(lens), len_div, k, _ptr(pool), n_pool, blk, _ptr(out), _ptr(ws),
                 ws.numel(), n_seq, _stream(stream)))


def flat_select_workspace_size(key_cap: int, k: int, n_seq: int) -> int:
    return int(_flat_ws(key_cap, k, n_seq))


def flat_select(q: torch.Tensor, keys: torch.Tensor, lens: torch.Tensor, k: int, out: torch.Tensor,
                w: Optional[torch.Tensor] = None, ws: Optional[torch.Tensor] = None, stream=None) -> None:
    """q [n_seq][8][64], keys [n_seq][key_cap][64] bf16 -> out [n_seq][k] int32: the Top-k positions by
    indexer score over all positions (csa2_flat_select).  ws: a zero-filled workspace reused across calls
    (a fresh one if None)."""
    n_seq, key_cap = keys.shape[0], keys.shape[1]
    if ws is None:
        ws = torch.zeros(max(flat_select_workspace_size(key_cap, k, n_seq), 1), dtype=torch.uint8,
                         device=keys.device)
    _check(_flat_select(_ptr(q), _ptr(w), _ptr(keys), key_cap, _ptr(lens), k, _ptr(out), _ptr(ws), ws.numel(),
                        n_seq, _stream(stream)))


def pool_select_workspace_size(n_pool: int, blk: int, n_seq: int) -> int:
    return int(_pool_ws(n_pool, blk, n_seq))


def pool_select(q: torch.Tensor, keys: torch.Tensor, lens: torch.Tensor, pool: torch.Tensor, k: int,
                out: torch.Tensor, blk: int = 8, w: Optional[torch.Tensor] = None, ws: Optional[torch.Tensor] = None,
                stream=None) -> None:
    """q [n_seq][8][64], keys [n_seq][key_cap][64] bf16, pool [n_seq][n_pool] int32 -> out [n_seq][k] int32:
    the Top-k positions of the pool's blocks by indexer score (csa2_pool_select).  ws: a zero-filled
    workspace reused across calls (a fresh one if None)."""
    n_seq, key_cap = keys.shape[0], keys.shape[1]
    n_pool = pool.shape[1]
    if ws is None:
        ws = torch.zeros(max(pool_select_workspace_size(n_pool, blk, n_seq), 1), dtype=torch.uint8,
                         device=keys.device)
    _check(_pool_select(_ptr(q), _ptr(w), _ptr(keys), key_cap, _ptr(lens), _ptr(pool), n_pool, blk, k, _ptr(out),
                        _ptr(ws), ws.numel(), n_seq, _stream(stream)))


def sparse_attn_workspace_size(n_q: int, k_idx: int, swa_max: int) -> int:
    return int(_attn_ws(n_q, k_idx, swa_max))


def sparse_attn_noalloc(q: torch.Tensor, kv: FP4KV, idx: torch.Tensor, swa: torch.Tensor, swa_len: torch.Tensor,
                        sm_scale: float, out: torch.Tensor, q_per_seq: int = 1,
                        swa_q_stride_rows: Optional[int] = None, swa_max: Optional[int] = None, stream=None) -> None:
    """csa2_sparse_attn_noalloc: sparse_attn (bf16 window rows) with its split partials in the library's
    static scratch instead of a workspace; allocates nothing."""
    n_q = q.shape[0]
    k_idx = idx.shape[1] if idx is not None and idx.dim() == 2 else 0
    if swa_max is None:
        swa_max = swa.shape[1] if swa.dim() == 3 else 0
    if swa_q_stride_rows is None:
        swa_q_stride_rows = swa_max
    kvc = kv.c()
    _check(_attn_noalloc(_ptr(q), n_q, ctypes.byref(kvc), q_per_seq, _ptr(idx), k_idx, _ptr(swa), swa_q_stride_rows,
                         _ptr(swa_len), swa_max, sm_scale, _ptr(out), _stream(stream)))


def sparse_attn_partial(q: torch.Tensor, kv: FP4KV, idx: Optional[torch.Tensor], swa: Optional[torch.Tensor],
                        swa_len: torch.Tensor, sm_scale: float, out_o: torch.Tensor, out_ml: torch.Tensor,
                        ws: Optional[torch.Tensor] = None, q_per_seq: int = 1,
                        swa_q_stride_rows: Optional[int] = None, swa_max: Optional[int] = None, stream=None) -> None:
    """csa2_sparse_attn_partial: a rank's share of a context-parallel split -- out_o [n_q][16][512] f32
    (unnormalised), out_ml [n_q][16][2] f32 (base-2 max, sum).  swa None: no window rows (swa_max 0)."""
    n_q = q.shape[0]
    k_idx = idx.shape[1] if idx is not None and idx.dim() == 2 else 0
    if swa_max is None:
        swa_max = swa.shape[1] if swa is not None and swa.dim() == 3 else 0
    if swa_q_stride_rows is None:
        swa_q_stride_rows = swa_max
    need = sparse_attn_workspace_size(n_q, k_idx, swa_max)
    if ws is None:
        ws = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    kvc = kv.c()
    _check(_attn_partial(_ptr(q), n_q, ctypes.byref(kvc), q_per_seq, _ptr(idx), k_idx, _ptr(swa), swa_q_stride_rows,
                         _ptr(swa_len), swa_max, sm_scale, _ptr(out_o), _ptr(out_ml), _ptr(ws), ws.numel(),
                         _stream(stream)))


def attn_merge(parts_o: torch.Tensor, parts_ml: torch.Tensor, out: torch.Tensor, stream=None) -> None:
    """csa2_attn_merge: parts_o [S][n_q][16][512] f32, parts_ml [S][n_q][16][2] f32 -> out [n_q][16][512]."""
    n_parts, n_q = parts_o.shape[0], parts_o.shape[1]
    _check(_attn_merge(_ptr(parts_o), _ptr(parts_ml), n_parts, n_q, _ptr(out), _stream(stream)))


def sparse_attn(q: torch.Tensor, kv: FP4KV, idx: torch.Tensor, swa: torch.Tensor, swa_len: torch.Tensor,
                sm_scale: float, out: torch.Tensor, ws: Optional[torch.Tensor] = None, q_per_seq: int = 1,
                swa_q_stride_rows: Optional[int] = None, swa_max: Optional[int] = None, stream=None) -> None:
    """q [n_q][16][512] bf16; idx [n_q][k_idx] int32; swa rows [..][512] bf16, or uint8 E4M3 codes
    (the FP8 window, csa2_sparse_attn_f8w); out [n_q][16][512] f32."""
    n_q = q.shape[0]
    k_idx = idx.shape[1] if idx is not None and idx.dim() == 2 else 0
    if swa_max is None:
        swa_max = swa.shape[1] if swa.dim() == 3 else 0
    if swa_q_stride_rows is None:
        swa_q_stride_rows = swa_max
    need = sparse_attn_workspace_size(n_q, k_idx, swa_max)
    if ws is None:
        ws = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    kvc = kv.c()
    fn = _attn_f8w if (swa is not None and swa.dtype == torch.uint8) else _attn  # E4M3 window rows
    _check(fn(_ptr(q), n_q, ctypes.byref(kvc), q_per_seq, _ptr(idx), k_idx, _ptr(swa), swa_q_stride_rows,
              _ptr(swa_len), swa_max, sm_scale, _ptr(out), _ptr(ws), ws.numel(), _stream(stream)))


class Layer:
    def __init__(self, mode: int, kv_id: int = 0, hierarchical: bool = False):
        self.mode, self.kv_id, self.hierarchical = mode, kv_id, hierarchical


class Sched:
    """The native layer-group scheduler (csa2_sched_*)."""

    def __init__(self, layers: Sequence[Layer], n_seq: int, key_cap: int, blk_cap: int = 0, topk: int = 512,
                 pool_blocks: int = 2048, blk: int = 8, swa_max: int = 128, sm_scale: float = 512 ** -0.5,
                 swa_fp8: bool = False):
        arr = (_Layer * len(layers))(*[_Layer(l.mode, l.kv_id, int(l.hierarchical)) for l in layers])
        desc = _SchedDesc(n_seq, len(layers), ctypes.cast(arr, _P), key_cap, blk_cap, topk, pool_blocks, blk,
                          swa_max, sm_scale, int(swa_fp8))
        h = _P()
        _check(_sched_create(ctypes.byref(desc), ctypes.byref(h)))
        self._h = h
        self.layers, self.n_seq, self.topk, self.pool_blocks = list(layers), n_seq, topk, pool_blocks
        self._keep = None

    def close(self):
        if getattr(self, "_h", None):
            _sched_destroy(self._h)
            self._h = None

    def __del__(self):
        self.close()

    def prepare(self, kv: Sequence[FP4KV], lens, idx_k, main_q, swa, swa_len, out, idx_q, blk_k=None,
                new_row=None, append_kv: int = 0, idx_w=None, new_idx_k=None, layer_idx_k=None,
                new_swa_row=None) -> "_StepIO":
        """Build (and keep alive) the step descriptor for a fixed set of tensors.
        layer_idx_k: None, or per layer the own indexer K of a flat Full layer
        (None entries: idx_k).  new_swa_row: None, or per layer the step token's
        window rows [n_seq][512], stored into window slot (lens[b] - 1) % swa_max
        as the layer runs."""
        nl = len(self.layers)
        kvs = (_FP4KV * len(kv))(*[k.c() for k in kv])
        P = _P * nl
        iq = P(*[_ptr(t) if t is not None else None for t in idx_q])
        iw = P(*[_ptr(t) for t in idx_w]) if idx_w is not None else None
        mq, sw, ou = P(*[_ptr(t) for t in main_q]), P(*[_ptr(t) for t in swa]), P(*[_ptr(t) for t in out])
        lk = P(*[_ptr(t) if t is not None else None for t in layer_idx_k]) if layer_idx_k is not None else None
        nw = P(*[_ptr(t) for t in new_swa_row]) if new_swa_row is not None else None
        io = _StepIO(len(kv), ctypes.cast(kvs, _P), _ptr(lens), _ptr(new_row), append_kv, _ptr(idx_k),
                     _ptr(blk_k), ctypes.cast(iq, _P), ctypes.cast(iw, _P) if iw is not None else None,
                     ctypes.cast(mq, _P), ctypes.cast(sw, _P), _ptr(swa_len), ctypes.cast(ou, _P),
                     _ptr(new_idx_k), ctypes.cast(lk, _P) if lk is not None else None,
                     ctypes.cast(nw, _P) if nw is not None else None)
        io._keep = (kvs, iq, iw, mq, sw, ou, lk, nw, kv, lens, idx_k, main_q, swa, swa_len, out, idx_q, blk_k,
                    new_row, idx_w, new_idx_k, layer_idx_k, new_swa_row)
        return io

    def decode_step(self, io: "_StepIO", stream=None) -> None:
        _check(_sched_step(self._h, ctypes.byref(io), _stream(stream)))

    def indices(self, layer: int) -> torch.Tensor:
        """Copy of the indices [n_seq][topk] a layer attended with in the last step."""
        p = _sched_indices(self._h, layer)
        return _device_copy_int32(p, self.n_seq * self.topk).view(self.n_seq, self.topk)

    def pool(self) -> Optional[torch.Tensor]:
        p = _sched_pool(self._h)
        if not p:
            return None
        return _device_copy_int32(p, self.n_seq * self.pool_blocks).view(self.n_seq, self.pool_blocks)

    def check(self, stream=None) -> int:
        """Read and clear the device flags on `stream` (default: the current stream), after
        the steps enqueued there."""
        f = _I32()
        _check(_sched_check(self._h, ctypes.byref(f), _stream(stream)))
        return f.value


def prefill_index_score(q: torch.Tensor, keys: torch.Tensor, t0: int, ratio: int, scores: torch.Tensor,
                        n_vis: torch.Tensor, w: Optional[torch.Tensor] = None, stream=None) -> None:
    """q [n_q][8][64] bf16, keys [n_entries][64] bf16 -> scores [n_q][n_entries] f32, n_vis [n_q] int32."""
    n_q, n_entries = scores.shape
    assert q.numel() == n_q * IDX_HEADS * IDX_DIM and keys.numel() == n_entries * IDX_DIM
    assert scores.dtype == torch.float32 and n_vis.dtype == torch.int32 and n_vis.numel() >= n_q
    _check(_prefill_score(_ptr(q), _ptr(w), _ptr(keys), n_entries, t0, ratio, n_q, _ptr(scores), _ptr(n_vis),
                          _stream(stream)))


def prefill_select_workspace_size(n_entries: int, n_q: int, k: int) -> int:
    n = int(_prefill_select_ws(n_entries, n_q, k))
    if n == 0:
        raise Csa2Error(-2, _last_error().decode(errors="replace"))
    return n


def prefill_select(q: torch.Tensor, keys: torch.Tensor, t0: int, ratio: int, idx: torch.Tensor, n_vis: torch.Tensor,
                   ws: torch.Tensor, w: Optional[torch.Tensor] = None, stream=None) -> None:
    """q [n_q][8][64] bf16, keys [n_entries][64] bf16 -> idx [n_q][k] int32 (each query's Top-k of its visible
    entries), n_vis [n_q] int32; ws: prefill_select_workspace_size bytes, zero-filled before its first use."""
    n_q, k = idx.shape
    n_entries = keys.numel() // IDX_DIM
    assert q.numel() == n_q * IDX_HEADS * IDX_DIM and idx.dtype == torch.int32
    assert n_vis.dtype == torch.int32 and n_vis.numel() >= n_q
    _check(_prefill_select(_ptr(q), _ptr(w), _ptr(keys), n_entries, t0, ratio, n_q, k, _ptr(idx), _ptr(n_vis),
                           _ptr(ws), ws.numel() * ws.element_size(), _stream(stream)))


class Prefill:
    """A causal prefill chunk of a layer group (csa2_prefill_chunk) with its
    workspace (zero-filled once here, as the entry point requires)."""

    def __init__(self, layers: Sequence[Layer], n_entries: int, ratio: int, n_q: int, t0: int, topk: int = 512,
                 swa: int = 128, sm_scale: float = 512 ** -0.5):
        self._arr = (_Layer * len(layers))(*[_Layer(l.mode, l.kv_id, int(l.hierarchical)) for l in layers])
        self.desc = _PrefillDesc(len(layers), ctypes.cast(self._arr, _P), n_entries, ratio, n_q, t0, topk, swa,
                                 sm_scale)
        self.ws_bytes = int(_prefill_ws(ctypes.byref(self.desc)))
        if self.ws_bytes == 0:
            raise Csa2Error(-2, _last_error().decode(errors="replace"))
        self.ws = torch.zeros(self.ws_bytes, dtype=torch.uint8, device="cuda")
        self.layers, self.n_q, self.topk = list(layers), n_q, topk

    def prepare(self, kv: Sequence[FP4KV], entry_k, idx_q, main_q, swa, out, idx, idx_w=None) -> "_PrefillIO":
        nl = len(self.layers)
        kvs = (_FP4KV * len(kv))(*[k.c() for k in kv])
        P = _P * nl

        def arr(ts):
            return P(*[_ptr(t) if t is not None else None for t in ts])

        iq, mq, sw, ou, ix = arr(idx_q), arr(main_q), arr(swa), arr(out), arr(idx)
        iw = arr(idx_w) if idx_w is not None else None
        io = _PrefillIO(len(kv), ctypes.cast(kvs, _P), _ptr(entry_k), ctypes.cast(iq, _P),
                        ctypes.cast(iw, _P) if iw is not None else None, ctypes.cast(mq, _P), ctypes.cast(sw, _P),
                        ctypes.cast(ou, _P), ctypes.cast(ix, _P))
        io._keep = (kvs, iq, mq, sw, ou, ix, iw, kv, entry_k, idx_q, main_q, swa, out, idx, idx_w)
        return io

    def run(self, io: "_PrefillIO", stream=None) -> None:
        _check(_prefill_chunk(ctypes.byref(self.desc), ctypes.byref(io), _ptr(self.ws), self.ws_bytes,
                              _stream(stream)))


_hip = None


def _device_copy_int32(ptr: int, n: int) -> torch.Tensor:
    """Copy n int32 from a library-owned device buffer into a new tensor (on the current stream)."""
    global _hip
    if _hip is None:
        _hip = ctypes.CDLL("libamdhip64.so")
        _hip.hipMemcpyAsync.argtypes = [_P, _P, _SZ, ctypes.c_int, _P]
        _hip.hipMemcpyAsync.restype = ctypes.c_int
    out = torch.empty(n, dtype=torch.int32, device="cuda")
    rc = _hip.hipMemcpyAsync(out.data_ptr(), ptr, 4 * n, 3, torch.cuda.current_stream().cuda_stream)
    if rc != 0:
        raise RuntimeError(f"hipMemcpyAsync failed ({rc})")
    return out
