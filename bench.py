"""Benchmark of the CSA2 FP4-KV decode step on one MI355X.

Workload (the headline): the 20-layer decoder schedule at 1M positions,
batch 16 (group 1 = hierarchical Full + 3 Reuse, groups 2-5 = Reindex + 3
Reuse, five FP4 main-KV tensors, one FP4 append per sequence per step),
seeded synthetic inputs resident in HBM.  A step is one pass of the whole
path: append, indexer scoring, Top-512 with the 2,048 x 8 pool, gather +
dequant, sparse + SWA attention for all 20 layers.  Every step has its own
main Q, indexer Q, appended row and window rows (each layer writes its
token's window row as it runs), so no step replays another's selections out
of the caches.

Prints one JSON line: (seq.layer)-steps/s, ms per step, the step's
algorithmic HBM bytes as GB/s and fraction of the 8 TB/s peak, the roofline
of the dominant op (HIP events; the kernel-trace time beside it when the
sources match a committed trace), the CPU oracle on a bounded sample of the
same workload (all host cores, plus one core), parity of step 0 and of the
last timed step against that sample and of every appended row; the other
decode workloads (key "configs": one Full layer at 4K positions, the Full +
3 Reuse group at 64K x 32, hierarchical Full + Reindex at 1M x 8) measured
and checked the same way; and (keys "fp8_window", "maintained_keys",
"encoder_decode", "prefill") the step with E4M3 window rows, with block keys
maintained on append, the encoder's ratio-2 decode and the ratio-2 causal
prefill chunk; and (key "context_parallel") a rank's attention share and
the merge of eight shares when a sequence is split over GPUs by positions.

usage: python bench.py [--gpus 1] [--steps 100] [--warmup 10] [--no-graph] [--no-cpu]
                       [--config NAME] [--no-configs] [--no-prefill] [--prefill-reps 5]
                       [--no-fp8-window] [--no-keys] [--no-encoder] [--calibrate]
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

METRIC = "CSA2 decode (seq·layer)-steps/s at 1M ctx + achieved HBM GB/s as % of peak"
PEAK_HBM_GBPS = 8000.0

# HBM bytes per call measured with the FETCH_SIZE and WRITE_SIZE counters
# (scaled by a 1 GiB copy; see profiles/), keyed by op, with the SHA-256 of
# the kernel sources they were taken on: a figure is reported only while
# those sources are unchanged.
MEASURED_TRAFFIC = {
    "decoder20_1m/sparse_attn": {
        "bytes": 12728378, "profile": "profiles/decode20_1m_b16_hbm_traffic.md",
        "sources": {"fp4_kv_cache_quant_amd/csrc/sparse_attn.hip":
                    "28d5635347045cc57ac37e31a076065f6ec85c5949fc68aeb6e2d5b0294b7de4",
                    "fp4_kv_cache_quant_amd/csrc/attn_dev.hpp":
                    "f661423ba3cb7510492a0ac6c0be9cc00bcf54af70b4fc72973da1614caddf09",
                    "fp4_kv_cache_quant_amd/csrc/common.hpp":
                    "16bbfd324bed22718b51c5dce1bdb40ab694408572eaf2f6e359577fa431688e"}},
    "decoder20_1m/block_scan": {
        "bytes": 209850117, "profile": "profiles/decode20_1m_b16_hbm_traffic.md",
        "sources": {"fp4_kv_cache_quant_amd/csrc/index_score.hip":
                    "709a8fb0d0eacbead763334c820a7bdb0967657ff5e4fa7119f473c2273fdcc9",
                    "fp4_kv_cache_quant_amd/csrc/common.hpp":
                    "16bbfd324bed22718b51c5dce1bdb40ab694408572eaf2f6e359577fa431688e",
                    "fp4_kv_cache_quant_amd/csrc/topk_ws.hpp":
                    "851d1bdbabfc69fc98ad3b94960d99fe8e200dd9c6fcf1a619231b9c52f11f07",
                    "fp4_kv_cache_quant_amd/csrc/select_dev.hpp":
                    "1a346e416aaaf92b6758b0632876d1ca8b0891d0c26c9feeba822aca9d06e9d9"}},
    "decoder20_1m/pool_select": {
        "bytes": 36533672, "profile": "profiles/decode20_1m_b16_hbm_traffic.md",
        "sources": {"fp4_kv_cache_quant_amd/csrc/index_score.hip":
                    "709a8fb0d0eacbead763334c820a7bdb0967657ff5e4fa7119f473c2273fdcc9",
                    "fp4_kv_cache_quant_amd/csrc/topk.hip":
                    "5f39e3a7ddddb62d4e1f18f6853b3f8b6a101be74815adc89d5c3061bec1fc70",
                    "fp4_kv_cache_quant_amd/csrc/common.hpp":
                    "16bbfd324bed22718b51c5dce1bdb40ab694408572eaf2f6e359577fa431688e",
                    "fp4_kv_cache_quant_amd/csrc/topk_ws.hpp":
                    "851d1bdbabfc69fc98ad3b94960d99fe8e200dd9c6fcf1a619231b9c52f11f07",
                    "fp4_kv_cache_quant_amd/csrc/select_dev.hpp":
                    "1a346e416aaaf92b6758b0632876d1ca8b0891d0c26c9feeba822aca9d06e9d9"}},
    "encoder_1m/flat_select": {
        "bytes": 1092364722, "profile": "profiles/encoder_decode_1m_b16_kernels.md",
        "sources": {"fp4_kv_cache_quant_amd/csrc/index_score.hip":
                    "709a8fb0d0eacbead763334c820a7bdb0967657ff5e4fa7119f473c2273fdcc9",
                    "fp4_kv_cache_quant_amd/csrc/topk.hip":
                    "5f39e3a7ddddb62d4e1f18f6853b3f8b6a101be74815adc89d5c3061bec1fc70",
                    "fp4_kv_cache_quant_amd/csrc/common.hpp":
                    "16bbfd324bed22718b51c5dce1bdb40ab694408572eaf2f6e359577fa431688e",
                    "fp4_kv_cache_quant_amd/csrc/topk_ws.hpp":
                    "851d1bdbabfc69fc98ad3b94960d99fe8e200dd9c6fcf1a619231b9c52f11f07",
                    "fp4_kv_cache_quant_amd/csrc/select_dev.hpp":
                    "1a346e416aaaf92b6758b0632876d1ca8b0891d0c26c9feeba822aca9d06e9d9"}},
}


def config_key(cfg):
    """The DECODE_CONFIGS key of cfg (matched by name), or None."""
    from synth.configs import DECODE_CONFIGS

    return next((k for k, c in DECODE_CONFIGS.items() if c.name == cfg.name), None)


def measured_traffic(op_key: str):
    """Counter-measured HBM bytes per call of op_key ("workload/op"), or None
    when unmeasured or when its kernel sources changed since the counters
    were taken."""
    import hashlib

    rec = MEASURED_TRAFFIC.get(op_key)
    if rec is None:
        return None
    root = os.path.dirname(os.path.abspath(__file__))
    for rel, digest in rec["sources"].items():
        try:
            with open(os.path.join(root, rel), "rb") as fh:
                if hashlib.sha256(fh.read()).hexdigest() != digest:
                    return None
        except OSError:
            return None
    return rec["bytes"]


# Average kernel time per call of an op in a rocprofv3 kernel trace of the
# same workload (the kernels of one call summed), with the SHA-256 of the
# sources it was taken on: reported next to the HIP-event time while those
# sources are unchanged.
KERNEL_TRACE = {
    "decoder20_1m/sparse_attn": {
        "us": 12.74, "profile": "profiles/decode20_1m_b16_kernels.md",
        "sources": {"fp4_kv_cache_quant_amd/csrc/sparse_attn.hip":
                    "28d5635347045cc57ac37e31a076065f6ec85c5949fc68aeb6e2d5b0294b7de4",
                    "fp4_kv_cache_quant_amd/csrc/attn_dev.hpp":
                    "f661423ba3cb7510492a0ac6c0be9cc00bcf54af70b4fc72973da1614caddf09",
                    "fp4_kv_cache_quant_amd/csrc/common.hpp":
                    "16bbfd324bed22718b51c5dce1bdb40ab694408572eaf2f6e359577fa431688e"}},
    "decoder20_1m/pool_select": {
        "us": 21.13, "profile": "profiles/decode20_1m_b16_kernels.md",
        "sources": {"fp4_kv_cache_quant_amd/csrc/index_score.hip":
                    "709a8fb0d0eacbead763334c820a7bdb0967657ff5e4fa7119f473c2273fdcc9",
                    "fp4_kv_cache_quant_amd/csrc/topk.hip":
                    "5f39e3a7ddddb62d4e1f18f6853b3f8b6a101be74815adc89d5c3061bec1fc70",
                    "fp4_kv_cache_quant_amd/csrc/common.hpp":
                    "16bbfd324bed22718b51c5dce1bdb40ab694408572eaf2f6e359577fa431688e",
                    "fp4_kv_cache_quant_amd/csrc/topk_ws.hpp":
                    "851d1bdbabfc69fc98ad3b94960d99fe8e200dd9c6fcf1a619231b9c52f11f07",
                    "fp4_kv_cache_quant_amd/csrc/select_dev.hpp":
                    "1a346e416aaaf92b6758b0632876d1ca8b0891d0c26c9feeba822aca9d06e9d9"}},
    "encoder_1m/flat_select": {
        "us": 215.05, "profile": "profiles/encoder_decode_1m_b16_kernels.md",
        "sources": {"fp4_kv_cache_quant_amd/csrc/index_score.hip":
                    "709a8fb0d0eacbead763334c820a7bdb0967657ff5e4fa7119f473c2273fdcc9",
                    "fp4_kv_cache_quant_amd/csrc/topk.hip":
                    "5f39e3a7ddddb62d4e1f18f6853b3f8b6a101be74815adc89d5c3061bec1fc70",
                    "fp4_kv_cache_quant_amd/csrc/common.hpp":
                    "16bbfd324bed22718b51c5dce1bdb40ab694408572eaf2f6e359577fa431688e",
                    "fp4_kv_cache_quant_amd/csrc/topk_ws.hpp":
                    "851d1bdbabfc69fc98ad3b94960d99fe8e200dd9c6fcf1a619231b9c52f11f07",
                    "fp4_kv_cache_quant_amd/csrc/select_dev.hpp":
                    "1a346e416aaaf92b6758b0632876d1ca8b0891d0c26c9feeba822aca9d06e9d9"}},
}


def kernel_trace_us(op_key: str):
    """Kernel-trace microseconds per call of op_key, or None (unmeasured, or
    the sources changed since the trace was taken)."""
    import hashlib

    rec = KERNEL_TRACE.get(op_key)
    if rec is None:
        return None
    root = os.path.dirname(os.path.abspath(__file__))
    for rel, digest in rec["sources"].items():
        try:
            with open(os.path.join(root, rel), "rb") as fh:
                if hashlib.sha256(fh.read()).hexdigest() != digest:
                    return None
        except OSError:
            return None
    return rec["us"]


def algorithmic_bytes(cfg, L: int) -> dict:
    """Bytes the method must move in one decode step (each distinct byte once).

    Per sequence: the block keys of all ceil(L/8) blocks (128 B each), the
    indexer keys of the pool's positions (128 B each; shared by the Full and
    Reindex layers; once more for every Full layer with its own keys), the selected FP4 rows of each main-KV tensor (512 x 288
    B), every layer's SWA window (128 x 1 KiB, or 512 B rows in FP8), main Q (16 KiB) and f32
    output (32 KiB), each selecting layer's indexer Q (1 KiB) and indices
    (2 KiB), and the append (1 KiB read, 288 B written)."""
    n = cfg.n_seq
    nl = len(cfg.layers)
    sel_layers = sum(1 for m, _, _ in cfg.layers if m != 2)
    groups = len({k for _, k, _ in cfg.layers})
    key_sets = 1 + sum(1 for l in range(nl) if cfg.own_keys(l))
    nblk = -(-L // cfg.blk)
    pool_pos = min(L, cfg.pool_blocks * cfg.blk) if cfg.hierarchical else L
    parts = {
        "block_keys": n * nblk * 128 if cfg.hierarchical else 0,
        "indexer_keys": n * pool_pos * 128 * key_sets,
        "fp4_rows": n * groups * cfg.topk * 288,
        "swa": n * nl * cfg.swa * (512 if cfg.swa_fp8 else 1024),
        "main_q": n * nl * 16 * 1024,
        "out": n * nl * 16 * 512 * 4,
        "indexer_q_and_indices": n * sel_layers * (1024 + cfg.topk * 4),
        "append": n * (1024 + 288) if cfg.append else 0,
    }
    parts["total"] = sum(parts.values())
    return parts


def cpu_baseline(cfg, step: int, seqs, threads: int, reps: int = 1):
    """Oracle (as it stands) on one full decode step of `seqs`: inputs are
    regenerated first (not timed), then the oracle's layer walk over all of
    them is timed `reps` times (dt is the total)."""
    from concurrent.futures import ThreadPoolExecutor

    from oracle import workloads as ow
    import oracle

    prep = {}

    def prepare(b):
        prep[b] = (ow.seq_state(cfg, b, step), ow.layer_inputs(cfg, b, step))

    with ThreadPoolExecutor(threads) as ex:
        list(ex.map(prepare, seqs))
    layers = [oracle.Layer(m, k, bool(h)) for m, k, h in cfg.layers]

    def run(b):
        st, ins = prep[b]
        return b, oracle.decode_layers(layers, st, ins, ow.SM_SCALE, k=cfg.topk, n_pool=cfg.pool_blocks)

    t0 = time.perf_counter()
    with ThreadPoolExecutor(threads) as ex:
        for _ in range(reps):
            res = dict(ex.map(run, seqs))
    dt = time.perf_counter() - t0
    return res, dt


def _graph_time_us(fn, per_graph: int = 20, replays: int = 10, graph: bool = True) -> float:
    """Average GPU time of fn() (a sequence of launches on the current
    stream): per_graph calls captured in one HIP graph, replayed, timed with
    HIP events on the stream (graph=False: the same calls launched eagerly)."""
    import torch

    fn()
    torch.cuda.synchronize()
    if not graph:
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(per_graph * replays):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1000.0 / (replays * per_graph)
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        with torch.cuda.graph(g, stream=side):
            for _ in range(per_graph):
                fn()
    torch.cuda.current_stream().wait_stream(side)
    g.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(replays):
        g.replay()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) * 1000.0 / (replays * per_graph)


def op_rooflines(cfg, inp, total_steps, graph: bool = True):
    """Algorithmic bytes per call, time and GB/s of every op of the step, each
    called through the C ABI on the step's own buffers (the scheduler fuses
    the Top-k histogram into the score kernel; a standalone Top-k builds it
    itself, so its figure here includes that pass).

    Bytes per call (n = sequences): block scan n*ceil(L/8)*(128+4) (block
    keys read, scores written); block Top-k n*slots*4 (scores read once);
    pool select n*16384*(128+4) (indexer keys of the pool positions, scores
    written and read back once: counted once);
    attention n*(512*4 + 512*288 + 128*1024 + 16*1024 + 16*512*4) (indices,
    selected FP4 rows, SWA window, main Q, f32 output)."""
    import torch

    import fp4_kv_cache_quant_amd as csa2
    from synth.configs import DECODE_CONFIGS

    n = cfg.n_seq
    L = int(inp.lens[0].item())
    nblk = -(-L // cfg.blk)
    blk_cap = cfg.blk_cap(total_steps)
    pool_slots = cfg.pool_blocks * cfg.blk
    q0 = inp.idx_q[0][0]
    bscores = torch.empty(n, blk_cap, dtype=torch.float32, device="cuda")
    pool = torch.empty(n, cfg.pool_blocks, dtype=torch.int32, device="cuda")
    idx = torch.empty(n, cfg.topk, dtype=torch.int32, device="cuda")
    out = torch.empty(n, 16, 512, dtype=torch.float32, device="cuda")
    tws = torch.zeros(csa2.topk_workspace_size(blk_cap, n), dtype=torch.uint8, device="cuda")
    pws = torch.zeros(csa2.pool_select_workspace_size(cfg.pool_blocks, cfg.blk, n), dtype=torch.uint8, device="cuda")
    aws = torch.empty(csa2.sparse_attn_workspace_size(n, cfg.topk, cfg.swa), dtype=torch.uint8, device="cuda")
    csa2.index_score(q0, inp.blk_k, inp.lens, bscores, len_div=cfg.blk)
    csa2.topk(bscores, cfg.pool_blocks, pool, lens=inp.lens, len_div=cfg.blk, ws=tws)
    csa2.pool_select(q0, inp.idx_k, inp.lens, pool, cfg.topk, idx, blk=cfg.blk, ws=pws)
    sel_layers = sum(1 for m, _, _ in cfg.layers if m != 2)
    ops = [
        ("block_scan", "block scan (index_score, block keys)", 1, n * nblk * 132,
         lambda: csa2.index_score(q0, inp.blk_k, inp.lens, bscores, len_div=cfg.blk)),
        ("block_topk", "block Top-2048 (topk)", 1, n * nblk * 4,
         lambda: csa2.topk(bscores, cfg.pool_blocks, pool, lens=inp.lens, len_div=cfg.blk, ws=tws)),
        ("pool_select", "pool score + Top-512 (pool_select)", sel_layers, n * pool_slots * (128 + 4),
         lambda: csa2.pool_select(q0, inp.idx_k, inp.lens, pool, cfg.topk, idx, blk=cfg.blk, ws=pws)),
        ("sparse_attn", "sparse+SWA attention (sparse_attn: chunk + combine kernels)", len(cfg.layers),
         n * (cfg.topk * 4 + cfg.topk * 288 + cfg.swa * (512 if cfg.swa_fp8 else 1024) + 16 * 1024 + 16 * 512 * 4),
         lambda: csa2.sparse_attn(inp.main_q[0][0], inp.kv[0], idx, inp.swa[0], inp.swa_len, 512 ** -0.5, out,
                                  ws=aws)),
    ]
    res = []
    for key, name, per_step, nbytes, fn in ops:
        us = _graph_time_us(fn, graph=graph)
        res.append({"key": key, "op": name, "launches_per_step": per_step, "bytes_per_launch": nbytes,
                    "avg_us": round(us, 2), "us_per_step": round(us * per_step, 1),
                    "GBps": round(nbytes / (us * 1e-6) / 1e9, 1),
                    "frac_of_peak": round(nbytes / (us * 1e-6) / 1e9 / PEAK_HBM_GBPS, 4),
                    "traffic_bytes": measured_traffic(f"{config_key(cfg)}/{key}"),
                    "kernel_trace_us": kernel_trace_us(f"{config_key(cfg)}/{key}")})
    return res


def context_parallel_ops(cfg, inp, total_steps, graph: bool = True, ranks: int = 8) -> dict:
    """The attention of the step when one sequence is split over `ranks`
    GPUs by positions (context parallelism), at the workload's batch: one
    rank's share (csa2_sparse_attn_partial) over all 512 selected rows and
    the window -- the largest share a rank can hold, every selected row on
    it -- and the merge of `ranks` shares (csa2_attn_merge).  Each rank's
    selection is the single-GPU selection over its positions, and the
    exchange between the ranks (RCCL over xGMI) is not on one GPU: neither is
    timed here.  Bytes per call (n = sequences): the share as the attention
    plus (m, l) written, n*(512*4 + 512*288 + 128*1024 + 16*1024 + 16*512*4
    + 16*8); the merge reads every share and writes the output,
    n*(ranks*(16*512*4 + 16*8) + 16*512*4)."""
    import torch

    import fp4_kv_cache_quant_amd as csa2

    n = cfg.n_seq
    L = int(inp.lens[0].item())
    blk_cap = cfg.blk_cap(total_steps)
    q0 = inp.idx_q[0][0]
    bscores = torch.empty(n, blk_cap, dtype=torch.float32, device="cuda")
    pool = torch.empty(n, cfg.pool_blocks, dtype=torch.int32, device="cuda")
    idx = torch.empty(n, cfg.topk, dtype=torch.int32, device="cuda")
    csa2.index_score(q0, inp.blk_k, inp.lens, bscores, len_div=cfg.blk)
    csa2.topk(bscores, cfg.pool_blocks, pool, lens=inp.lens, len_div=cfg.blk)
    csa2.pool_select(q0, inp.idx_k, inp.lens, pool, cfg.topk, idx, blk=cfg.blk)
    aws = torch.empty(max(1, csa2.sparse_attn_workspace_size(n, cfg.topk, cfg.swa)), dtype=torch.uint8,
                      device="cuda")
    parts_o = torch.empty(ranks, n, 16, 512, dtype=torch.float32, device="cuda")
    parts_ml = torch.empty(ranks, n, 16, 2, dtype=torch.float32, device="cuda")
    out = torch.empty(n, 16, 512, dtype=torch.float32, device="cuda")
    q, kv, swa = inp.main_q[0][0], inp.kv[0], inp.swa[0]

    def share(r=0):
        csa2.sparse_attn_partial(q, kv, idx, swa, inp.swa_len, 512 ** -0.5, parts_o[r], parts_ml[r], ws=aws)

    for r in range(ranks):  # valid shares for the merge to read
        share(r)
    ops = [("attn_share", "a rank's attention share (sparse_attn_partial: all 512 selected rows + window)",
            n * (cfg.topk * 4 + cfg.topk * 288 + cfg.swa * 1024 + 16 * 1024 + 16 * 512 * 4 + 16 * 8), share),
           ("attn_merge", f"merge of {ranks} shares (attn_merge)",
            n * (ranks * (16 * 512 * 4 + 16 * 8) + 16 * 512 * 4), lambda: csa2.attn_merge(parts_o, parts_ml, out))]
    res = []
    for key, name, nbytes, fn in ops:
        us = _graph_time_us(fn, graph=graph)
        res.append({"key": key, "op": name, "bytes_per_launch": nbytes, "avg_us": round(us, 2),
                    "GBps": round(nbytes / (us * 1e-6) / 1e9, 1),
                    "frac_of_peak": round(nbytes / (us * 1e-6) / 1e9 / PEAK_HBM_GBPS, 4)})
    return {"ranks": ranks, "positions_per_rank": -(-L // ranks), "ops": res,
            "not_timed": "the per-rank selection (the single-GPU kernels over L / ranks positions) and the "
                         "exchange of (score, id) pairs and of the shares between ranks"}


def flat_op_rooflines(cfg, inp, graph: bool = True):
    """The ops of a flat-selection step (every selecting layer takes a fresh
    Top-k over all L positions), as op_rooflines does for the hierarchical
    one.  Bytes per call: flat select n*(L*128 + 1024 + k*4) (every indexer
    key read once, indexer Q, indices written; csa2_flat_select keeps
    per-workgroup candidates instead of writing the scores); attention as in
    op_rooflines."""
    import torch

    import fp4_kv_cache_quant_amd as csa2

    n = cfg.n_seq
    L = int(inp.lens[0].item())
    q0 = inp.idx_q[0][0]
    idx = torch.empty(n, cfg.topk, dtype=torch.int32, device="cuda")
    out = torch.empty(n, 16, 512, dtype=torch.float32, device="cuda")
    fws = torch.zeros(csa2.flat_select_workspace_size(inp.cap, cfg.topk, n), dtype=torch.uint8, device="cuda")
    aws = torch.empty(csa2.sparse_attn_workspace_size(n, cfg.topk, cfg.swa), dtype=torch.uint8, device="cuda")
    csa2.flat_select(q0, inp.idx_k, inp.lens, cfg.topk, idx, ws=fws)
    sel_layers = sum(1 for m, _, _ in cfg.layers if m != 2)
    ops = [
        ("flat_select", "flat select (flat_select: scores + Top-k of all positions)", sel_layers,
         n * (L * 128 + 1024 + cfg.topk * 4),
         lambda: csa2.flat_select(q0, inp.idx_k, inp.lens, cfg.topk, idx, ws=fws)),
        ("sparse_attn", "sparse+SWA attention (sparse_attn: chunk + combine kernels)", len(cfg.layers),
         n * (cfg.topk * 4 + cfg.topk * 288 + cfg.swa * (512 if cfg.swa_fp8 else 1024) + 16 * 1024 + 16 * 512 * 4),
         lambda: csa2.sparse_attn(inp.main_q[0][0], inp.kv[0], idx, inp.swa[0], inp.swa_len, 512 ** -0.5, out,
                                  ws=aws)),
    ]
    res = []
    for key, name, per_step, nbytes, fn in ops:
        us = _graph_time_us(fn, graph=graph)
        res.append({"key": key, "op": name, "launches_per_step": per_step, "bytes_per_launch": nbytes,
                    "avg_us": round(us, 2), "us_per_step": round(us * per_step, 1),
                    "GBps": round(nbytes / (us * 1e-6) / 1e9, 1),
                    "frac_of_peak": round(nbytes / (us * 1e-6) / 1e9 / PEAK_HBM_GBPS, 4),
                    "traffic_bytes": measured_traffic(f"{config_key(cfg)}/{key}"),
                    "kernel_trace_us": kernel_trace_us(f"{config_key(cfg)}/{key}")})
    return res


def calibration_copy(nbytes: int = 1 << 30):
    """A plain device copy of known size, for scaling the HBM-traffic
    counters of a profile of this run (the copy reads and writes nbytes)."""
    import torch

    a = torch.empty(nbytes // 4, dtype=torch.float32, device="cuda")
    b = torch.empty_like(a)
    b.copy_(a)
    torch.cuda.synchronize()


PEAK_MFMA_BF16_TFLOPS = 2500.0


def prefill_bench(args) -> dict:
    """The causal prefill chunk of the encoder group (ratio 2, 64K entries,
    4,096 queries, Full + 5 Reuse): time per chunk, MFMA rate of the scoring
    and attention kernels against the dense bf16 peak, parity of sampled
    queries against the oracle, and the oracle's own rate on them."""
    import numpy as np
    import torch

    import fp4_kv_cache_quant_amd as csa2
    from fp4_kv_cache_quant_amd import workloads as wl
    from synth.configs import PREFILL_CONFIGS

    cfg = PREFILL_CONFIGS["encoder_prefill_128k"]
    nq, E, nl = cfg.n_q, cfg.n_entries, len(cfg.layers)
    inp = wl.build_prefill_inputs(cfg)
    pf, io = wl.make_prefill(inp)
    pf.run(io)
    torch.cuda.synchronize()
    idx0 = inp.idx[0].cpu().numpy()
    outs_sample = {}
    sample = [0, nq // 2 + 1, nq - 1]
    for i in sample:
        outs_sample[i] = [inp.out[l][i].cpu().numpy() for l in range(nl)]
    reps = max(1, args.prefill_reps)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        pf.run(io)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps

    # The chunk's two ops on their own, launched as the chunk launches them
    # (its selection, filtered while scoring, and the attention of one
    # layer), and the unfused public calls beside them: every score written
    # (csa2_prefill_index_score), then selected from memory (csa2_topk).
    q0 = inp.idx_q[0]
    sws = torch.zeros(csa2.prefill_select_workspace_size(E, nq, cfg.topk), dtype=torch.uint8, device="cuda")
    sidx = torch.empty(nq, cfg.topk, dtype=torch.int32, device="cuda")
    n_vis_sel = torch.empty(nq, dtype=torch.int32, device="cuda")
    csa2.prefill_select(q0, inp.entry_k, cfg.t0, cfg.ratio, sidx, n_vis_sel, sws)
    select_matches_chunk = bool(np.array_equal(sidx.cpu().numpy(), idx0))
    scores = torch.empty(nq, E, dtype=torch.float32, device="cuda")
    n_vis = torch.empty(nq, dtype=torch.int32, device="cuda")
    idx = torch.empty(nq, cfg.topk, dtype=torch.int32, device="cuda")
    out = torch.empty(nq, 16, 512, dtype=torch.float32, device="cuda")
    tws = torch.zeros(csa2.topk_workspace_size(E, nq), dtype=torch.uint8, device="cuda")
    win = torch.full((nq,), cfg.swa, dtype=torch.int32, device="cuda")
    csa2.prefill_index_score(q0, inp.entry_k, cfg.t0, cfg.ratio, scores, n_vis)
    csa2.topk(scores, cfg.topk, idx, lens=n_vis, ws=tws)
    ops = [
        ("prefill_select", lambda: csa2.prefill_select(q0, inp.entry_k, cfg.t0, cfg.ratio, sidx, n_vis_sel, sws),
         2.0 * nq * 8 * 64 * E, E * 128 + nq * 1024 + nq * cfg.topk * 4),
        ("prefill_score", lambda: csa2.prefill_index_score(q0, inp.entry_k, cfg.t0, cfg.ratio, scores, n_vis),
         2.0 * nq * 8 * 64 * E, nq * E * 4 + E * 128 + nq * 1024),
        ("prefill_topk", lambda: csa2.topk(scores, cfg.topk, idx, lens=n_vis, ws=tws), 0.0, nq * E * 4),
        ("prefill_attn", lambda: csa2.sparse_attn(inp.main_q[0], inp.kv[0], idx, inp.swa[0], win, 512 ** -0.5, out,
                                                  q_per_seq=nq, swa_q_stride_rows=1, swa_max=cfg.swa),
         2.0 * 2 * nq * 16 * (cfg.topk + cfg.swa) * 512,
         nq * (16 * 1024 + 16 * 512 * 4 + cfg.topk * 4) + E * 288 + cfg.swa_rows_total * 1024),
    ]
    op_res = []
    for key, fn, flops, nbytes in ops:
        us = _graph_time_us(fn, per_graph=2, replays=3, graph=not args.no_graph)
        r = {"key": key, "avg_us": round(us, 1), "bytes": int(nbytes), "GBps": round(nbytes / (us * 1e-6) / 1e9, 1)}
        if flops:
            tf = flops / (us * 1e-6) / 1e12
            r.update({"flops": flops, "TFLOPs": round(tf, 1), "mfma_frac_of_bf16_peak": round(tf / PEAK_MFMA_BF16_TFLOPS, 4)})
        op_res.append(r)

    # Parity and the oracle's rate on the sampled queries.
    from oracle import workloads as ow

    keys = ow.prefill_entry_keys(cfg)
    t0 = time.perf_counter()
    refs = {i: ow.prefill_reference(cfg, i, entry_keys=keys) for i in sample}
    cpu_s = time.perf_counter() - t0
    ok_idx = all(np.array_equal(idx0[i], refs[i][0].idx) for i in sample)
    worst_rel = worst_abs = 0.0
    for i in sample:
        for l in range(nl):
            o, r = outs_sample[i][l].astype(np.float64), refs[i][l].out.astype(np.float64)
            err = np.linalg.norm(o - r, axis=1) / np.maximum(np.linalg.norm(r, axis=1), 1e-30)
            worst_rel = max(worst_rel, float(err.max()))
            worst_abs = max(worst_abs, float(np.abs(o - r).max()))
    return {
        "workload": cfg.name, "n_entries": E, "ratio": cfg.ratio, "n_q": nq, "t0": cfg.t0, "layers": nl,
        "ms_per_chunk": round(ms, 3), "query_layers_per_s": round(nq * nl / (ms * 1e-3), 1),
        "reps": reps, "ops": op_res,
        "select_matches_chunk": select_matches_chunk,
        "parity_sample": {"queries": sample, "indices_bit_exact": bool(ok_idx), "attn_max_rel_l2": worst_rel,
                          "attn_max_abs": worst_abs,
                          "ok": bool(ok_idx and worst_rel <= 1e-3 and worst_abs <= 5e-3)},
        "cpu_baseline": {"value": round(len(sample) * nl / cpu_s, 2), "unit": "(query·layer)/s", "cores": 1,
                         "kind": "oracle",
                         "sample": f"{len(sample)} queries x {nl} layers of the chunk, {cpu_s:.1f} s"},
    }


def _capture_steps(sched, ios, steps, graph: bool):
    """One captured HIP graph per step (each step has its own inputs)."""
    import torch

    if not graph:
        return None
    stream = torch.cuda.current_stream()
    side = torch.cuda.Stream()
    side.wait_stream(stream)
    graphs = {}
    with torch.cuda.stream(side):
        for s_ in steps:
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=side):
                sched.decode_step(ios[s_])
            graphs[s_] = g
    stream.wait_stream(side)
    return graphs


def _time_steps(c, inp, K: int, W: int, graph: bool) -> dict:
    """Time K steps (after W warm-up steps) of workload c on the inputs inp,
    with a scheduler of its own; lengths are reset first so that the appends
    rewrite the same rows (step s uses query set s, so inp must hold
    1 + W + K of them)."""
    import torch

    from fp4_kv_cache_quant_amd import workloads as wl

    assert c.q_sets >= 1 + W + K
    inp.reset_lens()
    sched = wl.make_sched(inp)
    ios = wl.step_ios(sched, inp)
    sched.decode_step(ios[0])
    graphs = _capture_steps(sched, ios, range(1, 1 + W + K), graph)

    def run_step(s_):
        if graphs:
            graphs[s_].replay()
        else:
            sched.decode_step(ios[s_])

    for s_ in range(1, 1 + W):
        run_step(s_)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for s_ in range(1 + W, 1 + W + K):
        run_step(s_)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / K
    flag = sched.check()
    sched.close()
    ab = algorithmic_bytes(c, c.lens_at(1 + W + K // 2))
    return {"workload": c.name, "ms_per_step": round(ms, 4),
            "value": round(c.n_seq * len(c.layers) / (ms * 1e-3), 1), "unit": "(seq·layer)-steps/s",
            "algorithmic_bytes_per_step": ab["total"], "GBps": round(ab["total"] / (ms * 1e-3) / 1e9, 1),
            "device_flags": int(flag)}


def fp8_window_leg(cfg, inp, K: int, W: int, graph: bool) -> dict:
    """The same step with the window rows stored as E4M3 (FP8): the window
    tensors are quantised from the bf16 ones, every other input is shared."""
    import torch

    import fp4_kv_cache_quant_amd as csa2
    from fp4_kv_cache_quant_amd import workloads as wl

    c8 = cfg.with_(swa_fp8=True, name=cfg.name + ", FP8 window rows")

    def fp8(t):
        t8 = torch.empty(t.shape, dtype=torch.uint8, device="cuda")
        csa2.quant_fp8_rows(t.view(-1, 512), t8.view(-1, 512))
        return t8

    swa8 = [fp8(t) for t in inp.swa]
    new8 = [[fp8(t) for t in rows] if rows is not None else None for rows in inp.new_swa_row]
    inp8 = wl.DecodeInputs(cfg=c8, steps=inp.steps, kv=inp.kv, lens=inp.lens, idx_k=inp.idx_k, blk_k=inp.blk_k,
                           swa=swa8, swa_len=inp.swa_len, out=inp.out, idx_q=inp.idx_q, main_q=inp.main_q,
                           new_row=inp.new_row, new_swa_row=new8)
    r = _time_steps(c8, inp8, K, W, graph)
    del swa8, new8, inp8
    return r


def maintained_keys_leg(cfg, inp, K: int, W: int, graph: bool) -> dict:
    """The same step with block keys maintained on append: the block keys
    are re-formed as sums of the prefilled indexer keys, and every step
    appends its position's indexer key and updates its block's key.
    Overwrites the block keys and appended indexer-key rows of inp."""
    import fp4_kv_cache_quant_amd as csa2
    from fp4_kv_cache_quant_amd import workloads as wl

    ck = cfg.with_(maintain_keys=True, name=cfg.name + ", block keys maintained on append")
    inp.reset_lens()
    csa2.block_keys(inp.idx_k, inp.lens, inp.blk_k, ck.blk)
    new_k = [wl.fill_tensor((ck.n_seq, 1, 64), ck.new_idx_k(s_), seed=ck.seed) for s_ in range(ck.q_sets)]
    inpk = wl.DecodeInputs(cfg=ck, steps=inp.steps, kv=inp.kv, lens=inp.lens, idx_k=inp.idx_k, blk_k=inp.blk_k,
                           swa=inp.swa, swa_len=inp.swa_len, out=inp.out, idx_q=inp.idx_q, main_q=inp.main_q,
                           new_row=inp.new_row, new_idx_k=new_k, new_swa_row=inp.new_swa_row)
    return _time_steps(ck, inpk, K, W, graph)


def encoder_decode_leg(K: int, W: int, graph: bool, cpu_seqs: int) -> dict:
    """The encoder's 18 layers at ratio 2 in decode (3 groups of Full + 5
    Reuse over 512K entries, batch 16, each Full layer with its own indexer
    K): step time, the flat ops' rooflines, and step 0 of a few sequences
    against the oracle (also timed as its CPU rate)."""
    import torch

    from fp4_kv_cache_quant_amd import workloads as wl
    from synth.configs import DECODE_CONFIGS

    cfg = DECODE_CONFIGS["encoder_1m"].with_(q_sets=1 + W + K)
    nl = len(cfg.layers)
    inp = wl.build_decode_inputs(cfg, 1 + W + K)
    sched = wl.make_sched(inp)
    sched.decode_step(wl.step_ios(sched, inp)[0])
    torch.cuda.synchronize()
    gpu0 = {"idx": [sched.indices(l).cpu().numpy() for l in range(nl)], "pool": None,
            "out": [o.cpu().numpy() for o in inp.out]}
    sched.close()
    r = _time_steps(cfg, inp, K, W, graph)
    r["ops"] = flat_op_rooflines(cfg, inp, graph=graph)
    dom = max(r["ops"], key=lambda o: o["us_per_step"])
    r["roofline"] = {"op": dom["key"], "bound": "hbm", "achieved": dom["GBps"], "peak": PEAK_HBM_GBPS,
                     "unit": "GB/s", "frac": round(dom["GBps"] / PEAK_HBM_GBPS, 4),
                     "traffic": dom["traffic_bytes"]}
    if cpu_seqs > 0:
        seqs = sorted({0, cfg.n_seq - 1} if cpu_seqs > 1 else {0})
        threads = max(1, len(os.sched_getaffinity(0)))
        res, dt = cpu_baseline(cfg, 0, seqs, threads)
        r["parity_step0"] = compare_step(cfg, gpu0, res)
        r["cpu_baseline"] = {"value": round(len(seqs) * nl / dt, 2), "unit": "(seq·layer)-steps/s",
                             "cores": threads, "kind": "oracle",
                             "sample": f"decode step 0 of sequences {seqs}, all {nl} layers, {dt:.1f} s"}
    del inp
    torch.cuda.empty_cache()
    return r


def compare_step(cfg, gpu, ref) -> dict:
    """GPU step-0 results against the oracle sample: indices and pool
    bit-exact, attention rel. L2 <= 1e-3 and max abs <= 5e-3 per (seq, head)."""
    import numpy as np

    idx_ok = pool_ok = True
    worst_rel = worst_abs = 0.0
    for b, layers in ref.items():
        for l, r in enumerate(layers):
            idx_ok &= bool(np.array_equal(gpu["idx"][l][b], r.idx))
            if r.pool is not None and gpu["pool"] is not None and cfg.layers[l][0] == 0:
                pool_ok &= bool(np.array_equal(gpu["pool"][b], r.pool))
            o = gpu["out"][l][b].astype(np.float64)
            e = o - r.out.astype(np.float64)
            rel = np.linalg.norm(e, axis=1) / np.maximum(np.linalg.norm(r.out, axis=1), 1e-30)
            worst_rel = max(worst_rel, float(rel.max()))
            worst_abs = max(worst_abs, float(np.abs(e).max()))
    ok = idx_ok and pool_ok and worst_rel <= 1e-3 and worst_abs <= 5e-3
    return {"ok": ok, "indices_bit_exact": idx_ok, "pool_bit_exact": pool_ok,
            "attn_max_rel_l2": worst_rel, "attn_max_abs": worst_abs, "seqs": len(ref)}


def _snapshot(sched, inp, nl: int, hierarchical: bool) -> dict:
    """Indices, pool and outputs of the step that ran last (host copies)."""
    import torch

    torch.cuda.synchronize()
    return {"idx": [sched.indices(l).cpu().numpy() for l in range(nl)],
            "pool": sched.pool().cpu().numpy() if hierarchical else None,
            "out": [o.cpu().numpy().copy() for o in inp.out]}


def appended_rows_exact(cfg, inp, n_steps: int) -> bool:
    """Every row appended by the n_steps steps, every sequence: the device's
    FP4 bytes equal the oracle's quantisation of the appended source rows."""
    import numpy as np

    import oracle
    from oracle import workloads as ow

    if not cfg.append:
        return True
    kv = inp.kv[cfg.append_kv]
    pos = np.arange(cfg.L0, cfg.L0 + n_steps)
    codes = kv.codes[:, cfg.L0:cfg.L0 + n_steps].cpu().numpy()
    scales = kv.scales[:, cfg.L0:cfg.L0 + n_steps].cpu().numpy()
    ok = True
    for b in range(cfg.n_seq):
        rc, rs = oracle.quant_rows(ow.kv_source_rows(cfg, cfg.append_kv, b, pos))
        ok &= bool(np.array_equal(codes[b], rc) and np.array_equal(scales[b], rs))
    return ok


def roofline_of(ops, op_key_prefix: str) -> dict:
    """The roofline entry of the op with the largest share of the step."""
    dom = max(ops, key=lambda o: o["us_per_step"])
    r = {"op": dom["key"], "bound": "hbm", "achieved": dom["GBps"], "peak": PEAK_HBM_GBPS, "unit": "GB/s",
         "frac": round(dom["GBps"] / PEAK_HBM_GBPS, 4), "traffic": dom["traffic_bytes"],
         "timing": "HIP events around graph replays of the op on its stream"}
    kt = kernel_trace_us(f"{op_key_prefix}/{dom['key']}")
    if kt is not None:
        r["kernel_trace_us"] = kt
        r["achieved_kernel_trace"] = round(dom["bytes_per_launch"] / (kt * 1e-6) / 1e9, 1)
    return r, dom


def decode_leg(cfg, K: int, W: int, graph: bool, parity_seqs, cpu: bool, single_core: bool = False,
               keep_inputs: bool = False):
    """One decode workload: step 0 eagerly, then W warm-up and K timed steps
    replayed from one captured graph per step -- every step has its own main
    Q, indexer Q, appended row and window rows, so no step repeats another's
    selections -- timed with HIP events on the stream.  Step 0 and the last
    timed step are checked against the oracle on parity_seqs (all appended
    rows of all sequences bit-exact), and the oracle's time on that sample
    is the CPU baseline (host threads = the cores this process may use)."""
    import torch

    from fp4_kv_cache_quant_amd import workloads as wl

    total = 1 + W + K
    c = cfg.with_(q_sets=total)
    nl = len(c.layers)
    t_build = time.perf_counter()
    inp = wl.build_decode_inputs(c, total)
    sched = wl.make_sched(inp)
    ios = wl.step_ios(sched, inp)
    build_s = time.perf_counter() - t_build
    sched.decode_step(ios[0])
    gpu0 = _snapshot(sched, inp, nl, c.hierarchical)
    graphs = _capture_steps(sched, ios, range(1, total), graph)

    def run_step(s_):
        if graphs:
            graphs[s_].replay()
        else:
            sched.decode_step(ios[s_])

    for s_ in range(1, 1 + W):
        run_step(s_)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record()
    for s_ in range(1 + W, total):
        run_step(s_)
    e1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = e0.elapsed_time(e1) / K
    gpu_last = _snapshot(sched, inp, nl, c.hierarchical)
    flags = sched.check()
    sched.close()
    del graphs
    ab = algorithmic_bytes(c, c.lens_at(1 + W + K // 2))
    r = {"workload": c.name, "n_seq": c.n_seq, "positions": c.L0, "layers": nl,
         "ms_per_step": round(ms, 4), "value": round(c.n_seq * nl / (ms * 1e-3), 1),
         "unit": "(seq·layer)-steps/s", "algorithmic_bytes_per_step": ab["total"],
         "GBps": round(ab["total"] / (ms * 1e-3) / 1e9, 1),
         "frac_of_peak": round(ab["total"] / (ms * 1e-3) / 1e9 / PEAK_HBM_GBPS, 4), "parts": ab,
         "device_flags": int(flags), "wall_s_timed": round(wall, 3), "build_s": round(build_s, 1),
         "appended_rows_bit_exact": appended_rows_exact(c, inp, total)}
    ops = (op_rooflines(c, inp, total, graph=graph) if c.hierarchical else flat_op_rooflines(c, inp, graph=graph))
    r["roofline"], r["dominant_op"] = roofline_of(ops, config_key(cfg) or c.name)
    r["ops"] = ops
    if c.hierarchical and config_key(cfg) == "decoder20_1m":
        r["context_parallel"] = context_parallel_ops(c, inp, total, graph=graph)
    if cpu:
        threads = max(1, len(os.sched_getaffinity(0)))
        seqs = list(parity_seqs)
        res0, dt0 = cpu_baseline(c, 0, seqs, threads)
        resl, dtl = cpu_baseline(c, total - 1, seqs, threads)
        r["parity"] = {"step_0": compare_step(c, gpu0, res0), f"step_{total - 1}": compare_step(c, gpu_last, resl),
                       "appended_rows_bit_exact": r["appended_rows_bit_exact"]}
        r["parity"]["ok"] = bool(r["parity"]["step_0"]["ok"] and r["parity"][f"step_{total - 1}"]["ok"]
                                 and r["appended_rows_bit_exact"])
        r["cpu_baseline"] = {"value": round(2 * len(seqs) * nl / (dt0 + dtl), 2), "unit": "(seq·layer)-steps/s",
                             "cores": threads, "kind": "oracle",
                             "sample": f"decode steps 0 and {total - 1} of sequences {seqs[0]}..{seqs[-1]} "
                                       f"({len(seqs)} of {c.n_seq}), all {nl} layers, {threads} threads: "
                                       f"{dt0 + dtl:.1f} s"}
        if single_core:
            _, dt1 = cpu_baseline(c, 0, seqs[:1], 1)
            r["cpu_baseline"]["single_core"] = {"value": round(nl / dt1, 2), "unit": "(seq·layer)-steps/s",
                                                "sample": f"decode step 0 of sequence {seqs[0]}, all {nl} layers, "
                                                          f"1 thread: {dt1:.1f} s"}
    if keep_inputs:
        return r, c, inp
    del inp
    torch.cuda.empty_cache()
    return r, c, None


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--no-graph", action="store_true", help="launch each step eagerly")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle (parity and baseline)")
    ap.add_argument("--config", default="decoder20_1m")
    ap.add_argument("--no-configs", action="store_true", help="skip the other decode workloads (C1, C2, C4)")
    ap.add_argument("--no-prefill", action="store_true", help="skip the prefill-chunk measurement")
    ap.add_argument("--no-fp8-window", action="store_true", help="skip the FP8-window variant of the step")
    ap.add_argument("--no-keys", action="store_true", help="skip the maintained-block-keys variant of the step")
    ap.add_argument("--no-encoder", action="store_true", help="skip the encoder ratio-2 decode leg")
    ap.add_argument("--prefill-reps", type=int, default=5, help="timed prefill chunks")
    ap.add_argument("--calibrate", action="store_true",
                    help="also run a 1 GiB device copy (for scaling profiler traffic counters)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the multi-GPU split of this path is designed but "
              "not built, so only --gpus 1 is supported", file=sys.stderr)
        return 2

    import torch

    from synth.configs import DECODE_CONFIGS

    cfg = DECODE_CONFIGS[args.config]
    K, W = args.steps, args.warmup
    graph = not args.no_graph
    torch.cuda.init()
    if args.calibrate:
        calibration_copy()
    progress = lambda msg: print(f"[bench] {msg}", file=sys.stderr, flush=True)

    progress(f"headline {cfg.name}")
    head, c, inp = decode_leg(cfg, K, W, graph, range(cfg.n_seq), cpu=not args.no_cpu, single_core=True,
                              keep_inputs=True)
    if head["device_flags"] != 0:
        print("an append found a full cache during the timed steps", file=sys.stderr)
        return 1

    fp8w = keys = None
    if not args.no_fp8_window and not c.swa_fp8:
        progress("FP8 window leg")
        fp8w = fp8_window_leg(c, inp, K, W, graph)
    if not args.no_keys and c.hierarchical and c.append and not c.maintain_keys:
        progress("maintained keys leg")
        keys = maintained_keys_leg(c, inp, K, W, graph)
    del inp
    torch.cuda.empty_cache()

    configs = {}
    if not args.no_configs and args.config == "decoder20_1m":
        for key, seqs in (("single_4k", [0]), ("group_64k", [0, 31]), ("hier_1m", [0, 7])):
            progress(f"config {key}")
            r, _, _ = decode_leg(DECODE_CONFIGS[key], K, W, graph, seqs, cpu=not args.no_cpu)
            configs[key] = r

    encoder = None
    if not args.no_encoder and args.config != "encoder_1m":
        progress("encoder decode leg")
        encoder = encoder_decode_leg(K, W, graph=graph, cpu_seqs=0 if args.no_cpu else 2)

    prefill = None
    if not args.no_prefill:
        progress("prefill chunk")
        prefill = prefill_bench(args)

    line = {
        "metric": METRIC, "value": head["value"], "unit": "(seq·layer)-steps/s", "n_gpus": 1,
        "steps": K, "warmup": W, "ms_per_step": head["ms_per_step"], "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (seeded; FP4 E2M1 + E4M3/16 main KV, integer indexer Q/K, N(0,1) bf16 latents; "
                "every step its own main Q, indexer Q, appended row and window rows)",
        "config": {"workload": c.name, "n_seq": c.n_seq, "positions": c.L0, "layers": len(c.layers),
                   "fp4_kv_tensors": c.n_kv, "topk": c.topk, "pool": f"{c.pool_blocks}x{c.blk}",
                   "swa": c.swa, "graph": graph},
        "hbm": {"algorithmic_bytes_per_step": head["algorithmic_bytes_per_step"], "GBps": head["GBps"],
                "frac_of_peak": head["frac_of_peak"], "parts": head["parts"]},
        "roofline": head["roofline"], "dominant_op": head["dominant_op"], "ops": head["ops"],
        "cpu_baseline": head.get("cpu_baseline"), "parity": head.get("parity"),
        "appended_rows_bit_exact": head["appended_rows_bit_exact"],
        "configs": configs, "fp8_window": fp8w, "maintained_keys": keys, "encoder_decode": encoder,
        "prefill": prefill, "context_parallel": head.get("context_parallel"),
        "wall_s_timed": head["wall_s_timed"], "build_s": head["build_s"],
    }
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
