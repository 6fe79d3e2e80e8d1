"""Helpers for the GPU parity tests: seeded inputs for both sides, the
attention tolerance, and launch-shape checks done on the host."""
import numpy as np
import torch

import synth

SEED = 0
SM_SCALE = 512 ** -0.5
# Attention bar: per (query, head) relative L2 error and max abs error, fp32.
REL_L2 = 1e-3
MAX_ABS = 5e-3


def dev(a: np.ndarray) -> torch.Tensor:
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    return torch.from_numpy(a).cuda()


def host_u16(t: torch.Tensor) -> np.ndarray:
    return t.cpu().numpy().view(np.uint16)


def rows(kind_tid, kind, b, r, dim, seed=SEED):
    return synth.gen_rows(seed, kind_tid, kind, b, r, dim)


def kv_source(kv_id, n_seq, n_rows, seed=SEED):
    """bf16 latent source rows [n_seq][n_rows][512] of main-KV tensor kv_id."""
    return synth.gen_rows(seed, synth.tensor_id(synth.KIND_KV_SRC, kv_id), synth.NORMAL,
                          range(n_seq), np.arange(n_rows), 512)


def assert_attention_close(out: np.ndarray, ref: np.ndarray, what: str = ""):
    """out/ref [..][16][512]: per (query, head) rel L2 <= 1e-3 and max abs <= 5e-3."""
    out = out.reshape(-1, 512).astype(np.float64)
    ref = ref.reshape(-1, 512).astype(np.float64)
    assert np.all(np.isfinite(out)), what
    err = np.linalg.norm(out - ref, axis=1)
    nrm = np.linalg.norm(ref, axis=1)
    rel = np.where(nrm > 0, err / np.maximum(nrm, 1e-30), err)
    mx = np.abs(out - ref).max(axis=1)
    assert rel.max() <= REL_L2 and mx.max() <= MAX_ABS, f"{what}: rel L2 {rel.max():.3e}, max abs {mx.max():.3e}"
    return rel.max(), mx.max()


def print_case(msg: str):
    print(f"[gpu case] {msg}", flush=True)
