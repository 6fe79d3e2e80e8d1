"""Workload descriptions of the CSA2 decode path: shapes, layer-mode tables
and the synthetic tensor behind every input.  Pure data, shared by the device
input builder and the oracle side; no step of the method lives here.

Layer modes use the ABI's numbering: 0 = Full, 1 = Reindex, 2 = Reuse.
"""
from __future__ import annotations

from dataclasses import dataclass, replace
from typing import Tuple

from . import (INT9, NORMAL, KIND_BLK_K, KIND_IDX_K, KIND_IDX_Q, KIND_KV_SRC, KIND_MAIN_Q,
               KIND_NEW_IDX_K, KIND_NEW_ROW, KIND_SWA, tensor_id)

FULL, REINDEX, REUSE = 0, 1, 2


@dataclass(frozen=True)
class DecodeConfig:
    name: str
    n_seq: int
    L0: int                                   # positions before the first step
    layers: Tuple[Tuple[int, int, int], ...]  # (mode, kv_id, hierarchical)
    n_kv: int = 1
    append: bool = False                      # one appended row per sequence per step
    append_kv: int = 0
    topk: int = 512
    pool_blocks: int = 2048
    blk: int = 8
    swa: int = 128
    q_sets: int = 4                           # step s uses query set s % q_sets
    seed: int = 0
    swa_fp8: bool = False                     # window rows stored as E4M3 (FP8) codes
    maintain_keys: bool = False               # block keys = sums of indexer keys, kept current on append
    layer_keys: bool = False                  # every flat Full layer after layer 0 has its own indexer K
    window_writes: bool = True                # every step writes its token's window row in every layer

    def cap(self, steps: int) -> int:
        """Rows per sequence of every main-KV tensor and of indexer K."""
        return self.L0 + (steps if self.append else 0)

    def blk_cap(self, steps: int) -> int:
        return -(-self.cap(steps) // self.blk)

    @property
    def hierarchical(self) -> bool:
        return any(m == FULL and h for m, _, h in self.layers)

    def lens_at(self, step: int) -> int:
        """Positions seen by the layers of step `step` (after its append)."""
        return self.L0 + (step + 1 if self.append else 0)

    def with_(self, **kw) -> "DecodeConfig":
        return replace(self, **kw)

    # ---- synthetic tensors (tensor id, value kind)
    def kv_src(self, kv_id: int):
        return tensor_id(KIND_KV_SRC, kv_id), NORMAL

    def new_row(self, step: int):
        return tensor_id(KIND_NEW_ROW, self.append_kv, step % self.q_sets), NORMAL

    def idx_k(self):
        return tensor_id(KIND_IDX_K), INT9

    def own_keys(self, layer: int) -> bool:
        """Whether Full layer `layer` scores its own indexer K (else idx_k)."""
        mode, _, hier = self.layers[layer]
        return self.layer_keys and layer > 0 and mode == FULL and not hier

    def layer_idx_k(self, layer: int):
        return tensor_id(KIND_IDX_K, layer, 0), INT9

    def new_idx_k(self, step: int):
        return tensor_id(KIND_NEW_IDX_K, 0, step % self.q_sets), INT9

    def blk_k(self):
        return tensor_id(KIND_BLK_K), INT9

    def idx_q(self, layer: int, step: int):
        return tensor_id(KIND_IDX_Q, layer, step % self.q_sets), INT9

    def main_q(self, layer: int, step: int):
        return tensor_id(KIND_MAIN_Q, layer, step % self.q_sets), NORMAL

    def swa_rows(self, layer: int):
        return tensor_id(KIND_SWA, layer, 0), NORMAL

    def new_swa_row(self, layer: int, step: int):
        """The window row of step `step`'s token in layer `layer`."""
        return tensor_id(KIND_SWA, layer, 1 + step % self.q_sets), NORMAL

    def swa_slot(self, step: int) -> int:
        """Window slot of step `step`'s token: windows are rings of `swa` rows,
        position p in slot p % swa, and the token is the last position."""
        return (self.lens_at(step) - 1) % self.swa


def _group(mode0: int, kv: int, hier: int, n_reuse: int):
    return ((mode0, kv, hier),) + ((REUSE, kv, 0),) * n_reuse


# One Full CSA2 layer over 4,096 cached positions, one decode query.
SINGLE_LAYER_4K = DecodeConfig(name="single Full layer, 4K positions, batch 1", n_seq=1, L0=4096,
                               layers=((FULL, 0, 0),), q_sets=1)

# Decoder group at ratio 1: Full + 3 Reuse over 64K positions, batch 32, one append per step.
GROUP_64K = DecodeConfig(name="decoder group Full+3 Reuse, 64K positions, batch 32", n_seq=32,
                         L0=65536, layers=_group(FULL, 0, 0, 3), append=True)

# Hierarchical Full + Reindex over 1M positions, batch 8.
HIER_1M = DecodeConfig(name="hierarchical Full + Reindex, 1M positions, batch 8", n_seq=8,
                       L0=1 << 20, layers=((FULL, 0, 1), (REINDEX, 0, 0)))

# 20-layer decoder schedule at 1M, batch 16: group 1 = Full + 3 Reuse, groups
# 2-5 = Reindex + 3 Reuse, one FP4 main-KV tensor per group, one append per
# sequence per step into the Full group's tensor.
DECODER_20L_1M = DecodeConfig(
    name="20-layer decoder schedule, 1M positions, batch 16", n_seq=16, L0=1 << 20,
    layers=_group(FULL, 0, 1, 3) + sum((_group(REINDEX, g, 0, 3) for g in range(1, 5)), ()),
    n_kv=5, append=True)

# The same schedule with the block keys maintained on append (sums of the
# blocks' indexer keys; appended positions bring their own indexer key).
DECODER_20L_1M_KEYS = DECODER_20L_1M.with_(
    name="20-layer decoder schedule, 1M positions, batch 16, block keys maintained on append",
    maintain_keys=True)

# The same schedule with FP8 window rows.
DECODER_20L_1M_FP8_WINDOW = DECODER_20L_1M.with_(
    name="20-layer decoder schedule, 1M positions, batch 16, FP8 window rows", swa_fp8=True)

# The encoder's 18 CSA2 layers at ratio 2 in decode: three groups of Full +
# 5 Reuse, each group with its own FP4 main-KV tensor and its Full layer with
# its own indexer K, over 524,288 compressed entries (1M tokens), batch 16.
# Every entry is complete; the token being decoded is in the windows.
ENCODER_DECODE_1M = DecodeConfig(
    name="encoder schedule at ratio 2 (3 groups of Full + 5 Reuse), 512K entries (1M tokens), batch 16",
    n_seq=16, L0=1 << 19, layers=sum((_group(FULL, g, 0, 5) for g in range(3)), ()), n_kv=3,
    layer_keys=True)

DECODE_CONFIGS = {"single_4k": SINGLE_LAYER_4K, "group_64k": GROUP_64K, "hier_1m": HIER_1M,
                  "decoder20_1m": DECODER_20L_1M, "decoder20_1m_fp8win": DECODER_20L_1M_FP8_WINDOW,
                  "decoder20_1m_keys": DECODER_20L_1M_KEYS, "encoder_1m": ENCODER_DECODE_1M}


@dataclass(frozen=True)
class PrefillConfig:
    """A causal prefill chunk of an encoder layer group over compressed
    entries: entry e merges tokens ratio*e .. ratio*e+ratio-1; the chunk's
    query i sits at token t0 + i.  One FP4 main-KV tensor and one indexer K
    (one row per entry) are shared by the group; every layer has its own
    main Q and its own token-level SWA rows."""
    name: str
    n_entries: int
    ratio: int
    n_q: int
    t0: int
    layers: Tuple[Tuple[int, int, int], ...]
    topk: int = 512
    swa: int = 128
    seed: int = 0

    def with_(self, **kw) -> "PrefillConfig":
        return replace(self, **kw)

    @property
    def swa_row0(self) -> int:
        """Token of the first SWA row held: the window of query 0 starts here."""
        return self.t0 - self.swa + 1

    @property
    def swa_rows_total(self) -> int:
        return self.n_q + self.swa - 1

    # ---- synthetic tensors (tensor id, value kind); entry and SWA rows use
    # sequence 0 and the entry / token index as the row, query tensors use
    # the query index as the sequence.
    def entry_src(self):
        return tensor_id(KIND_KV_SRC, 0, 1), NORMAL

    def entry_k(self):
        return tensor_id(KIND_IDX_K, 0, 1), INT9

    def idx_q(self, layer: int):
        return tensor_id(KIND_IDX_Q, layer, 1), INT9

    def main_q(self, layer: int):
        return tensor_id(KIND_MAIN_Q, layer, 1), NORMAL

    def swa_tok(self, layer: int):
        return tensor_id(KIND_SWA, layer, 1), NORMAL


# Encoder group at ratio 2: Full + 5 Reuse over 128K tokens held as 64K
# compressed entries, a 4,096-query causal prefill chunk at the end of the
# context (queries at tokens 126,976 .. 131,071).
ENCODER_PREFILL_128K = PrefillConfig(
    name="encoder group Full+5 Reuse at ratio 2, 64K entries (128K tokens), 4,096-query prefill chunk",
    n_entries=1 << 16, ratio=2, n_q=4096, t0=(1 << 17) - 4096, layers=_group(FULL, 0, 0, 5))

PREFILL_CONFIGS = {"encoder_prefill_128k": ENCODER_PREFILL_128K}
