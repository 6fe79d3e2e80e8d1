"""TEST INFRASTRUCTURE: the CPU oracle of the CSA2 FP4-KV decode path.

Only ``tests/``, ``__graft_entry__.smoke()`` and ``bench.py``'s CPU-baseline
leg may import this package.  The product library never loads it and shares
no code with it; inputs come from :mod:`synth`.

The arithmetic lives in ``csa2_oracle.c`` (plain scalar C, double precision,
exact comparisons for the quantiser); this module is a ctypes binding plus the
layer walk of a decode step and of a prefill chunk, written as plain loops.

Citations name the page and its section:
  [P1] "DeepSeek AI Released DeepSeek-V4.1-Flash with 1M Context, FP4 KV
       Cache, and Cross-Layer Attention Reuse" (thecryptopost.io)
  [P3] "DeepSeek-V4.1 Flash: Pushing the Limits of KV Cache Compression"
       (tldrocket.com)

Parity status of each function is listed in ``PINS`` below.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from dataclasses import dataclass, field
from typing import List, Optional, Sequence

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "csa2_oracle.c")
_LIB = os.path.join(_HERE, "libcsa2_oracle.so")

D = 512
GROUP = 16
CODE_BYTES = 256
SCALE_BYTES = 32
IDX_HEADS = 8
IDX_DIM = 64
HEADS = 16
TOPK = 512            # [P1 "Compressed Sparse Attention 2 (CSA2)"]: fresh Top-512
POOL_BLOCKS = 2048    # [P1 "Compressed Sparse Attention 2 (CSA2)"]: 2,048 blocks of 8
BLK = 8
SWA = 128             # [P1 "Causal Encoder-Decoder: Half the Prefill"]: 128-token window

FULL, REINDEX, REUSE = 0, 1, 2

# What pins each oracle function to something other than itself (tests/test_oracle_pins.py).
PINS = {
    "orc_e4m3_value": "OCP E4M3FN landmark values (golden file) + monotone, 127 distinct finite",
    "orc_e2m1_value": "E2M1 grid {0,.5,1,1.5,2,3,4,6} (golden file)",
    "orc_scale_code": "all 65,536 bf16 amax vs exact-rational nearest-even by Fraction bisection",
    "orc_e2m1_code": "all bf16 magnitudes x all 126 nonzero scales vs float64 quotient + numpy half-even",
    "orc_quant_row": "byte layout golden row; dequant(quant(grid*s)) == grid*s; every reachable (bf16 magnitude, "
                     "scale) pair in both signs and every bf16 amax vs numpy/torch (tests/quant_sweep.py)",
    "orc_index_score_one": "one-hot closed forms, sign/ReLU cases, numpy int64 matmul on integer inputs, "
                           "weighted sums against exact rational (Fraction) arithmetic rounded once",
    "orc_select": "brute force via numpy lexsort; tie-heavy inputs; -1 padding; NaN/-inf never selected, -0 == +0",
    "orc_pool_blocks/orc_pool_select": "hierarchical == flat when blocks <= pool; subset/size invariants",
    "orc_sparse_attn": "k >= L equals torch CPU float64 dense softmax attention; 1 key, equal keys, q = 0",
    "decode_step": "Reuse reproduces the latest Full/Reindex indices; Reindex with Full's Q == Full",
    "orc_sparse_attn_partial": "o / l equals orc_sparse_attn on the same rows; m is the largest base-2 logit "
                               "(numpy float64); l >= 1; empty share m = -inf, l = 0, o = 0",
    "orc_attn_merge": "merge of shares over random splits of a query's rows (window on one share, empty "
                      "shares) equals orc_sparse_attn over all of them; one share gives o / l",
    "orc_fp8_code": "all 65,536 bf16 patterns vs torch's float8_e4m3fn cast in range, saturation and NaN beyond; golden ties",
    "orc_sparse_attn_fp8w": "equals orc_sparse_attn on window rows that FP8 represents exactly (bf16 of E4M3 values)",
    "orc_block_key": "numpy int64 sums of integer keys per block, partial last block; one-hot closed forms",
}


def build(force: bool = False) -> str:
    """Compile the oracle with gcc (no fast-math, no FMA contraction)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + f".tmp{os.getpid()}"
        subprocess.check_call([
            "gcc", "-O2", "-std=c11", "-Wall", "-ffp-contract=off", "-fno-fast-math",
            "-shared", "-fPIC", "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


_lib = None


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        L = ctypes.CDLL(build())
        P = ctypes.c_void_p
        i64 = ctypes.c_int64
        L.orc_bf16_value.argtypes = [ctypes.c_uint16]
        L.orc_bf16_value.restype = ctypes.c_double
        L.orc_e4m3_value.argtypes = [ctypes.c_uint8]
        L.orc_e4m3_value.restype = ctypes.c_double
        L.orc_e2m1_value.argtypes = [ctypes.c_uint8]
        L.orc_e2m1_value.restype = ctypes.c_double
        L.orc_scale_code.argtypes = [ctypes.c_double]
        L.orc_scale_code.restype = ctypes.c_uint8
        L.orc_e2m1_code.argtypes = [ctypes.c_double, ctypes.c_int, ctypes.c_double]
        L.orc_e2m1_code.restype = ctypes.c_uint8
        L.orc_quant_rows.argtypes = [P, i64, P, P]
        L.orc_quant_rows.restype = None
        L.orc_dequant_row.argtypes = [P, P, P]
        L.orc_dequant_row.restype = None
        L.orc_index_score.argtypes = [P, P, P, P, i64, P]
        L.orc_index_score.restype = None
        L.orc_select.argtypes = [P, P, i64, i64, P]
        L.orc_select.restype = i64
        L.orc_flat_select.argtypes = [P, P, P, i64, i64, P]
        L.orc_flat_select.restype = i64
        L.orc_pool_blocks.argtypes = [P, P, P, i64, i64, i64, P]
        L.orc_pool_blocks.restype = i64
        L.orc_pool_select.argtypes = [P, P, P, i64, P, i64, i64, i64, P]
        L.orc_pool_select.restype = i64
        L.orc_sparse_attn.argtypes = [P, P, P, P, i64, P, i64, ctypes.c_double, P]
        L.orc_sparse_attn.restype = None
        L.orc_sparse_attn_partial.argtypes = [P, P, P, P, i64, P, i64, ctypes.c_double, P, P]
        L.orc_sparse_attn_partial.restype = None
        L.orc_attn_merge.argtypes = [P, P, i64, P]
        L.orc_attn_merge.restype = None
        L.orc_fp8_code.argtypes = [ctypes.c_uint16]
        L.orc_fp8_code.restype = ctypes.c_uint8
        L.orc_fp8_rows.argtypes = [P, i64, P]
        L.orc_fp8_rows.restype = None
        L.orc_sparse_attn_fp8w.argtypes = [P, P, P, P, i64, P, i64, ctypes.c_double, P]
        L.orc_sparse_attn_fp8w.restype = None
        L.orc_block_key.argtypes = [P, i64, i64, i64, P]
        L.orc_block_key.restype = None
        _lib = L
    return _lib


def _p(a: Optional[np.ndarray]):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _u16(a) -> np.ndarray:
    return np.ascontiguousarray(a, dtype=np.uint16)


# ------------------------------------------------------------------ formats
def e4m3_value(c: int) -> float:
    return lib().orc_e4m3_value(c)


def e2m1_value(c: int) -> float:
    return lib().orc_e2m1_value(c)


def scale_code(amax: float) -> int:
    return lib().orc_scale_code(amax)


def e2m1_code(absx: float, neg: int, s: float) -> int:
    return lib().orc_e2m1_code(absx, neg, s)


def quant_rows(x_bf16: np.ndarray):
    """bf16 rows [n][512] -> (codes [n][256] u8, scales [n][32] u8)."""
    x = _u16(x_bf16).reshape(-1, D)
    n = x.shape[0]
    codes = np.zeros((n, CODE_BYTES), np.uint8)
    scales = np.zeros((n, SCALE_BYTES), np.uint8)
    lib().orc_quant_rows(_p(x), n, _p(codes), _p(scales))
    return codes, scales


def dequant_row(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    out = np.zeros(D, np.float64)
    lib().orc_dequant_row(_p(np.ascontiguousarray(codes, np.uint8)),
                          _p(np.ascontiguousarray(scales, np.uint8)), _p(out))
    return out


# ------------------------------------------------------------------ scoring
def _w(w):
    return None if w is None else np.ascontiguousarray(w, dtype=np.float32).reshape(IDX_HEADS)


def index_score(q: np.ndarray, keys: np.ndarray, ids: Sequence[int], w=None) -> np.ndarray:
    """Scores of keys[ids] against indexer Q [8][64] (bf16 bits)."""
    q = _u16(q).reshape(IDX_HEADS, IDX_DIM)
    keys = _u16(keys).reshape(-1, IDX_DIM)
    ids = np.ascontiguousarray(ids, dtype=np.int64)
    out = np.zeros(len(ids), np.float32)
    lib().orc_index_score(_p(q), _p(_w(w)), _p(keys), _p(ids), len(ids), _p(out))
    return out


def select(scores: np.ndarray, ids: Sequence[int], k: int) -> np.ndarray:
    scores = np.ascontiguousarray(scores, dtype=np.float32)
    ids = np.ascontiguousarray(ids, dtype=np.int64)
    out = np.zeros(k, np.int64)
    lib().orc_select(_p(scores), _p(ids), len(ids), k, _p(out))
    return out


def flat_select(q, tok_keys, L: int, k: int = TOPK, w=None) -> np.ndarray:
    out = np.zeros(k, np.int64)
    lib().orc_flat_select(_p(_u16(q)), _p(_w(w)), _p(_u16(tok_keys)), L, k, _p(out))
    return out


def pool_blocks(q, blk_keys, L: int, n_pool: int = POOL_BLOCKS, blk: int = BLK, w=None) -> np.ndarray:
    out = np.zeros(n_pool, np.int64)
    lib().orc_pool_blocks(_p(_u16(q)), _p(_w(w)), _p(_u16(blk_keys)), L, blk, n_pool, _p(out))
    return out


def pool_select(q, tok_keys, L: int, pool: np.ndarray, k: int = TOPK, blk: int = BLK, w=None) -> np.ndarray:
    pool = np.ascontiguousarray(pool, dtype=np.int64)
    out = np.zeros(k, np.int64)
    lib().orc_pool_select(_p(_u16(q)), _p(_w(w)), _p(_u16(tok_keys)), L, _p(pool), len(pool), blk,
                          k, _p(out))
    return out


# ---------------------------------------------------------------- attention
def sparse_attn(q, codes, scales, idx, swa, swa_len: int, sm_scale: float) -> np.ndarray:
    """One (query, layer): q [16][512] bf16 bits; codes/scales: the FP4 rows
    addressed by idx (an index < 0 is skipped); swa [>=swa_len][512] bf16."""
    q = _u16(q).reshape(HEADS, D)
    codes = np.ascontiguousarray(codes, np.uint8).reshape(-1, CODE_BYTES)
    scales = np.ascontiguousarray(scales, np.uint8).reshape(-1, SCALE_BYTES)
    idx = np.ascontiguousarray(idx, dtype=np.int64)
    assert idx.max(initial=-1) < codes.shape[0]
    swa = _u16(swa).reshape(-1, D)
    assert swa_len <= swa.shape[0]
    out = np.zeros((HEADS, D), np.float32)
    lib().orc_sparse_attn(_p(q), _p(codes), _p(scales), _p(idx), len(idx), _p(swa), swa_len,
                          float(sm_scale), _p(out))
    return out


def sparse_attn_gathered(q, rows_codes, rows_scales, idx, swa, swa_len, sm_scale, swa8=None):
    """Like :func:`sparse_attn` for a compact cache: ``rows_*[i]`` holds the
    row of position ``idx[i]`` (used when the full cache is not on the host).
    With ``swa8`` the window rows are those FP8 codes (``swa`` is ignored)."""
    idx = np.asarray(idx, dtype=np.int64)
    local = np.where(idx >= 0, np.arange(len(idx)), -1)
    if swa8 is not None:
        return sparse_attn_fp8w(q, rows_codes, rows_scales, local, swa8, swa_len, sm_scale)
    return sparse_attn(q, rows_codes, rows_scales, local, swa, swa_len, sm_scale)


def sparse_attn_partial(q, codes, scales, idx, swa, swa_len: int, sm_scale: float):
    """One rank's share (the rows of :func:`sparse_attn`): o [16][512] and
    ml [16][2] = (m, l), float64, base-2 units (see orc_sparse_attn_partial)."""
    q = _u16(q).reshape(HEADS, D)
    codes = np.ascontiguousarray(codes, np.uint8).reshape(-1, CODE_BYTES)
    scales = np.ascontiguousarray(scales, np.uint8).reshape(-1, SCALE_BYTES)
    idx = np.ascontiguousarray(idx, dtype=np.int64)
    assert idx.max(initial=-1) < codes.shape[0]
    swa = _u16(swa).reshape(-1, D)
    assert swa_len <= swa.shape[0]
    o = np.zeros((HEADS, D), np.float64)
    ml = np.zeros((HEADS, 2), np.float64)
    lib().orc_sparse_attn_partial(_p(q), _p(codes), _p(scales), _p(idx), len(idx), _p(swa), swa_len,
                                  float(sm_scale), _p(o), _p(ml))
    return o, ml


def attn_merge(o_parts, ml_parts) -> np.ndarray:
    """Softmax over the union of shares: o_parts [S][16][512], ml_parts [S][16][2] -> [16][512] f32."""
    o_parts = np.ascontiguousarray(o_parts, np.float64).reshape(-1, HEADS, D)
    ml_parts = np.ascontiguousarray(ml_parts, np.float64).reshape(-1, HEADS, 2)
    assert o_parts.shape[0] == ml_parts.shape[0]
    out = np.zeros((HEADS, D), np.float32)
    lib().orc_attn_merge(_p(o_parts), _p(ml_parts), o_parts.shape[0], _p(out))
    return out


# ------------------------------------------------- block-key maintenance
def block_keys(tok_keys: np.ndarray, L: int, blk: int = BLK) -> np.ndarray:
    """Block keys [ceil(L/blk)][64] (bf16 bits) of the first L positions."""
    tok = _u16(tok_keys).reshape(-1, IDX_DIM)
    nb = -(-L // blk)
    out = np.zeros((nb, IDX_DIM), np.uint16)
    for b in range(nb):
        lib().orc_block_key(_p(tok), L, blk, b, _p(out[b]))
    return out


# ------------------------------------------------------------ FP8 window
def fp8_code(b: int) -> int:
    """E4M3 code of one bf16 bit pattern (round to nearest even, saturating)."""
    return int(lib().orc_fp8_code(int(b) & 0xFFFF))


def fp8_rows(x_bf16: np.ndarray) -> np.ndarray:
    """bf16 rows [n][512] -> E4M3 codes [n][512] (uint8)."""
    x = _u16(x_bf16).reshape(-1, D)
    out = np.zeros(x.shape, np.uint8)
    lib().orc_fp8_rows(_p(x), x.shape[0], _p(out))
    return out


def sparse_attn_fp8w(q, codes, scales, idx, swa8, swa_len: int, sm_scale: float) -> np.ndarray:
    """:func:`sparse_attn` with the window rows given as E4M3 codes [>= swa_len][512]."""
    q = _u16(q).reshape(HEADS, D)
    codes = np.ascontiguousarray(codes, np.uint8).reshape(-1, CODE_BYTES)
    scales = np.ascontiguousarray(scales, np.uint8).reshape(-1, SCALE_BYTES)
    idx = np.ascontiguousarray(idx, dtype=np.int64)
    assert idx.max(initial=-1) < codes.shape[0]
    swa8 = np.ascontiguousarray(swa8, np.uint8).reshape(-1, D)
    assert swa_len <= swa8.shape[0]
    out = np.zeros((HEADS, D), np.float32)
    lib().orc_sparse_attn_fp8w(_p(q), _p(codes), _p(scales), _p(idx), len(idx), _p(swa8), swa_len,
                               float(sm_scale), _p(out))
    return out


# ------------------------------------------------------------- layer walk
@dataclass
class Layer:
    mode: int            # FULL, REINDEX or REUSE
    kv_id: int = 0       # which FP4 main-KV tensor this layer's group attends over
    hierarchical: bool = False


def check_table(layers: Sequence[Layer]) -> None:
    """[P1 "Compressed Sparse Attention 2 (CSA2)"]: Reindex reuses the last
    Full layer's keys, Reuse the latest Top-K; so layer 0 must be Full."""
    seen_full = seen_sel = False
    for l in layers:
        if l.mode == FULL:
            seen_full = seen_sel = True
        elif l.mode == REINDEX:
            if not seen_full:
                raise ValueError("Reindex layer without an earlier Full layer")
            seen_sel = True
        elif l.mode == REUSE:
            if not seen_sel:
                raise ValueError("Reuse layer without an earlier Full/Reindex layer")
        else:
            raise ValueError("unknown mode")


@dataclass
class SeqState:
    """Host view of one sequence as the oracle needs it."""
    L: int                                  # positions in the main KV
    tok_keys: np.ndarray                    # indexer K rows [>= L][64] bf16 bits
    blk_keys: Optional[np.ndarray] = None   # block keys [>= ceil(L/8)][64]
    kv_rows: Optional[callable] = None      # kv_rows(kv_id, ids) -> (codes, scales) of those rows
    layer_keys: Optional[dict] = None       # Full layer -> its own indexer K rows (else tok_keys)


@dataclass
class LayerInputs:
    idx_q: Optional[np.ndarray]   # [8][64] for Full/Reindex layers
    main_q: np.ndarray            # [16][512]
    swa: np.ndarray               # [>= swa_len][512] bf16 bits
    swa_len: int
    w: Optional[np.ndarray] = None
    swa8: Optional[np.ndarray] = None  # the window as E4M3 codes instead of swa


@dataclass
class LayerResult:
    idx: np.ndarray
    pool: Optional[np.ndarray]
    out: np.ndarray


def decode_layers(layers: Sequence[Layer], seq: SeqState, inputs: Sequence[LayerInputs],
                  sm_scale: float, k: int = TOPK, n_pool: int = POOL_BLOCKS,
                  attend: bool = True) -> List[LayerResult]:
    """Walk a static layer table for one sequence after the append.

    [P1 "Compressed Sparse Attention 2 (CSA2)"]: Full selects a fresh Top-K
    (through the block pool when hierarchical); Reindex rescores the last Full
    layer's pool (or all L positions when that Full layer is flat) with its
    own indexer Q; Reuse reuses the latest indices; every layer attends with
    its own main Q and SWA window.  A Full layer scores its own indexer K when
    seq.layer_keys holds one for it (each Full layer projects its keys), and
    the Reindex layers after it rescore those."""
    check_table(layers)
    res: List[LayerResult] = []
    idx = pool = None
    last_full_pool = None
    keys = seq.tok_keys
    for l, (layer, inp) in enumerate(zip(layers, inputs)):
        if layer.mode == FULL:
            keys = seq.tok_keys
            if seq.layer_keys is not None and l in seq.layer_keys:
                keys = seq.layer_keys[l]
            if layer.hierarchical:
                pool = pool_blocks(inp.idx_q, seq.blk_keys, seq.L, n_pool, BLK, inp.w)
                idx = pool_select(inp.idx_q, keys, seq.L, pool, k, BLK, inp.w)
            else:
                pool = None
                idx = flat_select(inp.idx_q, keys, seq.L, k, inp.w)
            last_full_pool = pool
        elif layer.mode == REINDEX:
            if last_full_pool is not None:
                idx = pool_select(inp.idx_q, keys, seq.L, last_full_pool, k, BLK, inp.w)
            else:
                idx = flat_select(inp.idx_q, keys, seq.L, k, inp.w)
            pool = last_full_pool
        # REUSE: idx and pool stay as they are.
        out = None
        if attend:
            codes, scales = seq.kv_rows(layer.kv_id, idx)
            out = sparse_attn_gathered(inp.main_q, codes, scales, idx, inp.swa, inp.swa_len, sm_scale, inp.swa8)
        res.append(LayerResult(idx=idx.copy(), pool=None if pool is None else pool.copy(), out=out))
    return res


# ---------------------------------------------------------------- prefill
def prefill_visible_entries(t: int, ratio: int, n_entries: Optional[int] = None) -> int:
    """READING: compressed entry e merges tokens ratio*e .. ratio*e+ratio-1
    ([P3]: encoder-side merging of adjacent positions; [P1 "Compressed Sparse
    Attention 2 (CSA2)"]: encoder ratio 2) and is visible to the query at
    token t once its last token is <= t; a cache of n_entries entries holds
    no more than those."""
    v = (t + 1) // ratio
    return v if n_entries is None else min(v, n_entries)


def prefill_window(t: int, swa: int = SWA):
    """READING: the query at token t attends to the window tokens
    max(0, t-swa+1) .. t ([P1 "Causal Encoder-Decoder: Half the Prefill"]:
    a 128-token sliding window in every layer); returns (first token, count)."""
    lo = max(0, t - swa + 1)
    return lo, t - lo + 1


def prefill_query(layers: Sequence[Layer], t: int, ratio: int, entry_keys: np.ndarray,
                  kv_rows, inputs: Sequence[LayerInputs], sm_scale: float, k: int = TOPK):
    """All layers of one prefill query at token t over compressed entries.
    Each query selects independently; Reuse layers reuse that query's
    indices.  ``inputs[l].swa`` holds the window tokens of prefill_window(t)."""
    n_vis = prefill_visible_entries(t, ratio, entry_keys.shape[0])
    seq = SeqState(L=n_vis, tok_keys=entry_keys, kv_rows=kv_rows)
    return decode_layers(layers, seq, inputs, sm_scale, k)
