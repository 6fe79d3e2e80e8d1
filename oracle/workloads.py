"""TEST INFRASTRUCTURE: oracle results of a decode or prefill workload (synth/configs.py).

Regenerates on the host, from the same seeds as the device builder, exactly
the inputs one decode step of one sequence reads, and runs the oracle's
layer walk on them.  Only tests, the smoke check and the benchmark's CPU
baseline use it.
"""
from __future__ import annotations

import numpy as np

import synth
from synth.configs import REUSE, DecodeConfig, PrefillConfig

from . import (Layer, LayerInputs, SeqState, block_keys, decode_layers, fp8_rows, prefill_query,
               prefill_visible_entries, prefill_window, quant_rows)

SM_SCALE = 512 ** -0.5


def _gen(cfg: DecodeConfig, tid_kind, b: int, rows, dim: int) -> np.ndarray:
    tid, kind = tid_kind
    return synth.gen_rows(cfg.seed, tid, kind, [b], np.asarray(rows, dtype=np.int64), dim)[0]


def kv_source_rows(cfg: DecodeConfig, kv_id: int, b: int, ids: np.ndarray) -> np.ndarray:
    """bf16 latent rows at positions ids (all >= 0) of tensor kv_id, sequence b:
    the pre-filled source row, or for an appended position the row appended by
    the step that wrote it."""
    ids = np.asarray(ids, dtype=np.int64)
    out = _gen(cfg, cfg.kv_src(kv_id), b, ids, 512)
    if cfg.append and kv_id == cfg.append_kv:
        for i, p in enumerate(ids):
            if p >= cfg.L0:
                out[i] = _gen(cfg, cfg.new_row(int(p - cfg.L0)), b, [0], 512)[0]
    return out


def index_key_rows(cfg: DecodeConfig, b: int, L: int) -> np.ndarray:
    """Indexer K of positions 0..L-1 of sequence b: the pre-filled rows, and
    with maintained keys the appended positions' own keys."""
    if not (cfg.maintain_keys and cfg.append) or L <= cfg.L0:
        return _gen(cfg, cfg.idx_k(), b, np.arange(L), 64)
    tok = _gen(cfg, cfg.idx_k(), b, np.arange(cfg.L0), 64)
    new = [_gen(cfg, cfg.new_idx_k(p - cfg.L0), b, [0], 64) for p in range(cfg.L0, L)]
    return np.concatenate([tok] + new)


def seq_state(cfg: DecodeConfig, b: int, step: int) -> SeqState:
    L = cfg.lens_at(step)
    tok = index_key_rows(cfg, b, L)
    blk = None
    if cfg.hierarchical:
        blk = (block_keys(tok, L, cfg.blk) if cfg.maintain_keys
               else _gen(cfg, cfg.blk_k(), b, np.arange(-(-L // cfg.blk)), 64))

    def kv_rows(kv_id, ids):
        ids = np.asarray(ids, dtype=np.int64)
        src = np.zeros((len(ids), 512), np.uint16)
        ok = ids >= 0
        if ok.any():
            src[ok] = kv_source_rows(cfg, kv_id, b, ids[ok])
        return quant_rows(src)

    own = {l: _gen(cfg, cfg.layer_idx_k(l), b, np.arange(L), 64)
           for l in range(len(cfg.layers)) if cfg.own_keys(l)}
    return SeqState(L=L, tok_keys=tok, blk_keys=blk, kv_rows=kv_rows, layer_keys=own or None)


def window_rows(cfg: DecodeConfig, l: int, b: int, step: int) -> np.ndarray:
    """Layer l's window of sequence b as decode step `step` attends over it:
    the initial rows, with every step s <= step having written its token's
    row into that token's ring slot (when the workload writes windows)."""
    sw = _gen(cfg, cfg.swa_rows(l), b, np.arange(cfg.swa), 512)
    if cfg.window_writes:
        for s in range(step + 1):
            sw[cfg.swa_slot(s)] = _gen(cfg, cfg.new_swa_row(l, s), b, [0], 512)[0]
    return sw


def layer_inputs(cfg: DecodeConfig, b: int, step: int):
    ins = []
    for l, (mode, _, _) in enumerate(cfg.layers):
        iq = None if mode == REUSE else _gen(cfg, cfg.idx_q(l, step), b, np.arange(8), 64)
        mq = _gen(cfg, cfg.main_q(l, step), b, np.arange(16), 512)
        sw = window_rows(cfg, l, b, step)
        sw8 = fp8_rows(sw) if cfg.swa_fp8 else None
        ins.append(LayerInputs(idx_q=iq, main_q=mq, swa=sw, swa_len=cfg.swa, swa8=sw8))
    return ins


def reference_step(cfg: DecodeConfig, step: int, b: int, attend=True):
    """Oracle LayerResults of decode step `step` (0-based) for sequence b."""
    layers = [Layer(m, k, bool(h)) for m, k, h in cfg.layers]
    return decode_layers(layers, seq_state(cfg, b, step), layer_inputs(cfg, b, step), SM_SCALE,
                         k=cfg.topk, n_pool=cfg.pool_blocks, attend=attend)


# ---------------------------------------------------------------- prefill
def prefill_entry_keys(cfg: PrefillConfig) -> np.ndarray:
    """Indexer K of every entry, [n_entries][64] bf16 bits."""
    return _gen(cfg, cfg.entry_k(), 0, np.arange(cfg.n_entries), 64)


def prefill_kv_rows(cfg: PrefillConfig):
    def kv_rows(kv_id, ids):
        ids = np.asarray(ids, dtype=np.int64)
        src = np.zeros((len(ids), 512), np.uint16)
        ok = ids >= 0
        if ok.any():
            src[ok] = _gen(cfg, cfg.entry_src(), 0, ids[ok], 512)
        return quant_rows(src)
    return kv_rows


def prefill_layer_inputs(cfg: PrefillConfig, i: int):
    """Per-layer inputs of query i (token t0 + i)."""
    t = cfg.t0 + i
    lo, cnt = prefill_window(t, cfg.swa)
    ins = []
    for l, (mode, _, _) in enumerate(cfg.layers):
        iq = None if mode == REUSE else _gen(cfg, cfg.idx_q(l), i, np.arange(8), 64)
        mq = _gen(cfg, cfg.main_q(l), i, np.arange(16), 512)
        sw = _gen(cfg, cfg.swa_tok(l), 0, np.arange(lo, lo + cnt), 512)
        ins.append(LayerInputs(idx_q=iq, main_q=mq, swa=sw, swa_len=cnt))
    return ins


def prefill_reference(cfg: PrefillConfig, i: int, entry_keys=None, attend=True):
    """Oracle LayerResults of query i of the prefill chunk."""
    layers = [Layer(m, k, bool(h)) for m, k, h in cfg.layers]
    keys = prefill_entry_keys(cfg) if entry_keys is None else entry_keys
    ins = prefill_layer_inputs(cfg, i)
    if not attend:
        n_vis = prefill_visible_entries(cfg.t0 + i, cfg.ratio, cfg.n_entries)
        return decode_layers(layers, SeqState(L=n_vis, tok_keys=keys), ins, SM_SCALE, k=cfg.topk, attend=False)
    return prefill_query(layers, cfg.t0 + i, cfg.ratio, keys, prefill_kv_rows(cfg), ins, SM_SCALE, k=cfg.topk)
