"""Device-resident inputs of a decode or prefill workload (see synth/configs.py).

Every tensor is generated on the GPU by the seeded generator (synth's fill
kernel) and the FP4 caches are quantised on the GPU with csa2_quant_rows,
so a 1M-position, 16-sequence, 5-tensor cache (24 GB) is built in seconds
without host traffic.  The oracle side regenerates any row on the host from
the same seeds.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import List, Optional

import torch

import synth
from synth.configs import DecodeConfig, PrefillConfig

from . import FP4KV, LATENT, Layer, Prefill, Sched, block_keys, quant_fp8_rows, quant_rows


def fill_tensor(shape, tid_kind, seed=0):
    """A new bf16 tensor [n_seq][rows][dim] holding rows 0.. of each sequence."""
    tid, kind = tid_kind
    t = torch.empty(shape, dtype=torch.int16, device="cuda")
    synth.fill_rows_device(t, seed, tid, kind)
    return t


def fill_kv_rows(kv: FP4KV, b: int, row0: int, n_rows: int, tid_kind, seed: int, chunk: int = 1 << 19,
                 staging: Optional[torch.Tensor] = None):
    """Generate bf16 source rows row0.. of sequence b and quantise them into kv."""
    tid, kind = tid_kind
    if staging is None:
        staging = torch.empty(min(chunk, n_rows), LATENT, dtype=torch.int16, device="cuda")
    done = 0
    while done < n_rows:
        m = min(staging.shape[0], n_rows - done)
        st = staging[:m]
        synth.fill_rows_device(st.view(1, m, LATENT), seed, tid, kind, b0=b, row0=row0 + done)
        quant_rows(st, kv.codes[b, row0 + done:row0 + done + m], kv.scales[b, row0 + done:row0 + done + m])
        done += m


@dataclass
class DecodeInputs:
    cfg: DecodeConfig
    steps: int
    kv: List[FP4KV]
    lens: torch.Tensor
    idx_k: torch.Tensor
    blk_k: Optional[torch.Tensor]
    swa: List[torch.Tensor]
    swa_len: torch.Tensor
    out: List[torch.Tensor]
    idx_q: List[List[Optional[torch.Tensor]]] = field(default_factory=list)   # [set][layer]
    main_q: List[List[torch.Tensor]] = field(default_factory=list)            # [set][layer]
    new_row: List[Optional[torch.Tensor]] = field(default_factory=list)       # [set]
    new_idx_k: List[Optional[torch.Tensor]] = field(default_factory=list)     # [set], maintained keys
    new_swa_row: List[Optional[List[torch.Tensor]]] = field(default_factory=list)  # [set][layer], window rows
    layer_idx_k: Optional[List[Optional[torch.Tensor]]] = None                 # [layer]: own indexer K

    @property
    def cap(self):
        return self.cfg.cap(self.steps)

    def reset_lens(self):
        self.lens.fill_(self.cfg.L0)


def build_decode_inputs(cfg: DecodeConfig, steps: int) -> DecodeInputs:
    """Allocate and fill every input of `steps` decode steps of cfg."""
    n, seed = cfg.n_seq, cfg.seed
    cap, nl = cfg.cap(steps), len(cfg.layers)
    kv = []
    staging = torch.empty(min(1 << 19, cap), LATENT, dtype=torch.int16, device="cuda")
    for k in range(cfg.n_kv):
        t = FP4KV.empty(n, cap)
        rows = cfg.L0 if (cfg.append and k == cfg.append_kv) else cap
        for b in range(n):
            fill_kv_rows(t, b, 0, rows, cfg.kv_src(k), seed, staging=staging)
        kv.append(t)
    del staging
    idx_k = fill_tensor((n, cap, 64), cfg.idx_k(), seed=seed)
    blk_k = fill_tensor((n, cfg.blk_cap(steps), 64), cfg.blk_k(), seed=seed) if cfg.hierarchical else None
    swa = [fill_tensor((n, cfg.swa, LATENT), cfg.swa_rows(l), seed=seed) for l in range(nl)]
    if cfg.swa_fp8:  # the window rows as E4M3 codes
        swa8 = []
        for t in swa:
            t8 = torch.empty(t.shape, dtype=torch.uint8, device="cuda")
            quant_fp8_rows(t, t8)
            swa8.append(t8)
        swa = swa8
    inp = DecodeInputs(cfg=cfg, steps=steps, kv=kv,
                       lens=torch.full((n,), cfg.L0, dtype=torch.int32, device="cuda"),
                       idx_k=idx_k, blk_k=blk_k, swa=swa,
                       swa_len=torch.full((n,), cfg.swa, dtype=torch.int32, device="cuda"),
                       out=[torch.empty(n, 16, LATENT, dtype=torch.float32, device="cuda") for _ in range(nl)])
    for s in range(cfg.q_sets):
        inp.idx_q.append([fill_tensor((n, 8, 64), cfg.idx_q(l, s), seed=seed) if cfg.layers[l][0] != 2 else None
                          for l in range(nl)])
        inp.main_q.append([fill_tensor((n, 16, LATENT), cfg.main_q(l, s), seed=seed) for l in range(nl)])
        inp.new_row.append(fill_tensor((n, 1, LATENT), cfg.new_row(s), seed=seed) if cfg.append else None)
        inp.new_idx_k.append(fill_tensor((n, 1, 64), cfg.new_idx_k(s), seed=seed)
                             if (cfg.maintain_keys and cfg.append) else None)
        rows = None
        if cfg.window_writes:
            rows = [fill_tensor((n, 1, LATENT), cfg.new_swa_row(l, s), seed=seed) for l in range(nl)]
            if cfg.swa_fp8:
                rows8 = []
                for t in rows:
                    t8 = torch.empty(t.shape, dtype=torch.uint8, device="cuda")
                    quant_fp8_rows(t.view(n, LATENT), t8.view(n, LATENT))
                    rows8.append(t8)
                rows = rows8
        inp.new_swa_row.append(rows)
    if cfg.layer_keys:
        inp.layer_idx_k = [fill_tensor((n, cap, 64), cfg.layer_idx_k(l), seed=seed) if cfg.own_keys(l) else None
                           for l in range(nl)]
    if cfg.maintain_keys and blk_k is not None:  # keys of the prefilled blocks, from indexer K
        block_keys(idx_k, inp.lens, blk_k, cfg.blk)
    torch.cuda.synchronize()
    return inp


def make_sched(inp: DecodeInputs) -> Sched:
    cfg = inp.cfg
    layers = [Layer(m, k, bool(h)) for m, k, h in cfg.layers]
    return Sched(layers, n_seq=cfg.n_seq, key_cap=inp.cap,
                 blk_cap=cfg.blk_cap(inp.steps) if cfg.hierarchical else 0, topk=cfg.topk,
                 pool_blocks=cfg.pool_blocks, blk=cfg.blk, swa_max=cfg.swa, swa_fp8=cfg.swa_fp8)


def step_ios(sched: Sched, inp: DecodeInputs):
    """One prepared step descriptor per query set (step s uses ios[s % q_sets])."""
    return [sched.prepare(kv=inp.kv, lens=inp.lens, idx_k=inp.idx_k, main_q=inp.main_q[s], swa=inp.swa,
                          swa_len=inp.swa_len, out=inp.out, idx_q=inp.idx_q[s], blk_k=inp.blk_k,
                          new_row=inp.new_row[s], append_kv=inp.cfg.append_kv,
                          new_idx_k=inp.new_idx_k[s] if inp.new_idx_k else None,
                          layer_idx_k=inp.layer_idx_k,
                          new_swa_row=inp.new_swa_row[s] if inp.new_swa_row else None)
            for s in range(inp.cfg.q_sets)]


# ---------------------------------------------------------------- prefill
@dataclass
class PrefillInputs:
    cfg: PrefillConfig
    kv: List[FP4KV]                       # one tensor, n_seq 1, cap n_entries
    entry_k: torch.Tensor                 # [n_entries][64]
    idx_q: List[Optional[torch.Tensor]]   # [layer]: [n_q][8][64] (Reuse: None)
    main_q: List[torch.Tensor]            # [layer]: [n_q][16][512]
    swa: List[torch.Tensor]               # [layer]: [n_q + swa - 1][512], row j = token t0 - swa + 1 + j
    out: List[torch.Tensor]               # [layer]: [n_q][16][512] f32
    idx: List[Optional[torch.Tensor]]     # [layer]: [n_q][topk] int32 (Reuse: None)


def build_prefill_inputs(cfg: PrefillConfig) -> PrefillInputs:
    """Allocate and fill every input of one prefill chunk of cfg."""
    seed, nq, nl = cfg.seed, cfg.n_q, len(cfg.layers)
    kv = FP4KV.empty(1, cfg.n_entries)
    fill_kv_rows(kv, 0, 0, cfg.n_entries, cfg.entry_src(), seed)
    entry_k = fill_tensor((1, cfg.n_entries, 64), cfg.entry_k(), seed=seed)[0]
    idx_q = [fill_tensor((nq, 8, 64), cfg.idx_q(l), seed=seed) if m != 2 else None
             for l, (m, _, _) in enumerate(cfg.layers)]
    main_q = [fill_tensor((nq, 16, LATENT), cfg.main_q(l), seed=seed) for l in range(nl)]
    swa = []
    for l in range(nl):
        t = torch.empty(cfg.swa_rows_total, LATENT, dtype=torch.int16, device="cuda")
        tid, kind = cfg.swa_tok(l)
        synth.fill_rows_device(t.view(1, cfg.swa_rows_total, LATENT), seed, tid, kind, b0=0, row0=cfg.swa_row0)
        swa.append(t)
    out = [torch.empty(nq, 16, LATENT, dtype=torch.float32, device="cuda") for _ in range(nl)]
    idx = [torch.empty(nq, cfg.topk, dtype=torch.int32, device="cuda") if m != 2 else None
           for m, _, _ in cfg.layers]
    torch.cuda.synchronize()
    return PrefillInputs(cfg=cfg, kv=[kv], entry_k=entry_k, idx_q=idx_q, main_q=main_q, swa=swa, out=out, idx=idx)


def make_prefill(inp: PrefillInputs):
    """The chunk runner and its prepared descriptor."""
    cfg = inp.cfg
    layers = [Layer(m, k, bool(h)) for m, k, h in cfg.layers]
    pf = Prefill(layers, n_entries=cfg.n_entries, ratio=cfg.ratio, n_q=cfg.n_q, t0=cfg.t0, topk=cfg.topk,
                 swa=cfg.swa)
    io = pf.prepare(kv=inp.kv, entry_k=inp.entry_k, idx_q=inp.idx_q, main_q=inp.main_q, swa=inp.swa,
                    out=inp.out, idx=inp.idx)
    return pf, io
