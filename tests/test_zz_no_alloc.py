"""csa2_sparse_attn_noalloc (the allocation-free entry point) against
csa2_sparse_attn with a caller workspace: the same kernels over the same
inputs give bit-identical outputs, on two calls in a row (the second with
fewer queries and rows, so that the static scratch holds the previous
call's partials); a call needing more than the scratch is rejected before
anything is enqueued."""
import numpy as np
import pytest
import torch

import synth
from gpu_helpers import SEED, SM_SCALE, dev, kv_source, print_case

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def csa2():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import fp4_kv_cache_quant_amd as m
    return m


def _case(csa2, n_q, cap, k_idx, swa_max, seed):
    src = kv_source(7, n_q, cap, seed=seed)
    kv = csa2.FP4KV.empty(n_q, cap)
    csa2.quant_rows(dev(src.reshape(-1, 512)), kv.codes, kv.scales)
    rng = np.random.default_rng(seed)
    idx = np.stack([np.sort(rng.choice(cap, k_idx, replace=False)) for _ in range(n_q)]).astype(np.int32)
    idx[0, k_idx // 3:] = -1
    q = synth.gen_rows(SEED + seed, synth.tensor_id(synth.KIND_MAIN_Q, 7), synth.NORMAL, range(n_q), np.arange(16), 512)
    swa = synth.gen_rows(SEED + seed, synth.tensor_id(synth.KIND_SWA, 7), synth.NORMAL, range(n_q),
                         np.arange(swa_max), 512)
    swa_len = rng.integers(0, swa_max + 1, size=n_q).astype(np.int32)
    swa_len[-1] = swa_max
    return kv, dev(idx), dev(q), dev(swa), dev(swa_len)


@pytest.mark.parametrize("order", ["large_then_small"])
def test_noalloc_matches_workspace_entry_point(csa2, order):
    for n_q, cap, k_idx, swa_max, seed in ((24, 3000, 512, 128, 1), (5, 900, 200, 64, 2)):
        print_case(f"sparse_attn_noalloc n_q={n_q} k_idx={k_idx} swa={swa_max}")
        kv, idx, q, swa, swa_len = _case(csa2, n_q, cap, k_idx, swa_max, seed)
        need = csa2.sparse_attn_workspace_size(n_q, k_idx, swa_max)
        assert 0 < need <= 16 << 20
        ref = torch.full((n_q, 16, 512), float("nan"), dtype=torch.float32, device="cuda")
        ws = torch.zeros(need, dtype=torch.uint8, device="cuda")
        csa2.sparse_attn(q, kv, idx, swa, swa_len, SM_SCALE, ref, ws=ws)
        got = torch.full((n_q, 16, 512), float("nan"), dtype=torch.float32, device="cuda")
        csa2.sparse_attn_noalloc(q, kv, idx, swa, swa_len, SM_SCALE, got)
        torch.cuda.synchronize()
        r, g = ref.cpu().numpy(), got.cpu().numpy()
        assert np.all(np.isfinite(r))
        assert np.array_equal(g, r), (n_q, float(np.abs(g - r).max()))


def test_noalloc_rejects_calls_beyond_the_scratch(csa2):
    n_q, k_idx, swa_max = 600, 512, 128
    assert csa2.sparse_attn_workspace_size(n_q, k_idx, swa_max) > 16 << 20
    kv = csa2.FP4KV.empty(n_q, 8)
    q = torch.zeros(n_q, 16, 512, dtype=torch.int16, device="cuda")
    idx = torch.full((n_q, k_idx), -1, dtype=torch.int32, device="cuda")
    swa = torch.zeros(n_q, swa_max, 512, dtype=torch.int16, device="cuda")
    swa_len = torch.zeros(n_q, dtype=torch.int32, device="cuda")
    out = torch.zeros(n_q, 16, 512, dtype=torch.float32, device="cuda")
    print_case("sparse_attn_noalloc beyond the scratch")
    with pytest.raises(csa2.Csa2Error, match="static scratch"):
        csa2.sparse_attn_noalloc(q, kv, idx, swa, swa_len, SM_SCALE, out)
    torch.cuda.synchronize()
    assert not out.any()  # nothing ran
